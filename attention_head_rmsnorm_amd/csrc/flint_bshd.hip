// BSHD input with document ids and arbitrary padding, turned into the THD
// description the attention kernels take.
//
// flint.layers page, FlintAttention.forward: an attention_mask [B, S] marks
// valid tokens (padded queries and keys leave attention, the sink stays
// valid); TE's BSHD path takes trailing padding and arbitrary padding goes
// through THD packing; integer document_ids [B, S] give a block-diagonal mask.
// Documents are the maximal runs of equal id among a row's valid tokens.
//
// The plan kernel reads the mask and the ids once and writes one of two THD
// descriptions of the same layer:
//  * in place (no document has a padded token inside it): the B*S tokens as
//    they lie in memory are the THD stream. A sequence starts at each
//    document's first token and runs up to the next document's first token;
//    its valid length is the document's length, so padding after a document
//    (up to the next one, across row ends) is that sequence's trailing
//    padding. Padding before the first document of row 0 is one more sequence
//    of valid length 0. Positions default to the index in the sequence, which
//    is the index in the document.
//  * packed (some document has a hole): the valid tokens in order are the
//    stream, one sequence per document. The caller gathers q, k, v and the
//    positions with `pack` and scatters the output back with `unpack`.

#include <hip/hip_runtime.h>

#include <algorithm>

#include "flint_common.h"

namespace flint {

namespace {

constexpr int kPlanThreads = 1024;

struct PlanPtrs {
  int* info;
  int* cu;
  int* seqused;
  int* pack;
  int* unpack;
  int* tstream;  // stream position of each sequence's first token (index d + lead)
  int* tpack;    // packed index of each document's first token (index d + lead)
};

__host__ __device__ inline PlanPtrs plan_ptrs(int* base, int64_t N) {
  PlanPtrs p;
  p.info = base;
  p.cu = base + 8;
  p.seqused = p.cu + N + 1;
  p.pack = p.seqused + N;
  p.unpack = p.pack + N;
  p.tstream = p.unpack + N;
  p.tpack = p.tstream + N + 1;
  return p;
}

// One workgroup walks the B*S tokens in chunks of 1024: packed index of every
// valid token (a prefix count), its predecessor among the valid tokens
// (through `pack` of the packed index before it), document starts (first
// valid token of a row, or an id different from the predecessor's) and holes
// (a valid token whose predecessor in the same document is not the token
// just before it).
__global__ __launch_bounds__(kPlanThreads) void bshd_plan_kernel(const uint8_t* __restrict__ mask,
                                                                 const int* __restrict__ ids,
                                                                 int batch, int seqlen,
                                                                 int* __restrict__ plan) {
  __shared__ int tmp[16];
  __shared__ int s_holes, s_max;
  const int64_t N = (int64_t)batch * seqlen;
  const PlanPtrs P = plan_ptrs(plan, N);
  const int tid = threadIdx.x;
  if (tid == 0) {
    s_holes = 0;
    s_max = 0;
  }
  __syncthreads();
  if (N == 0) {
    if (tid == 0) {
      P.info[0] = 0; P.info[1] = 0; P.info[2] = 0; P.info[3] = 0;
      P.info[4] = 0; P.info[5] = 0; P.info[6] = 0; P.info[7] = 0;
      P.cu[0] = 0;
    }
    return;
  }
  const int lead = (mask && mask[0] == 0) ? 1 : 0;
  int nvalid = 0, ndocs = 0;
  for (int64_t c0 = 0; c0 < N; c0 += kPlanThreads) {
    const int64_t i = c0 + tid;
    const bool in = i < N;
    const bool v = in && (!mask || mask[i] != 0);
    int tot;
    const int ci = nvalid + block_excl_scan(v ? 1 : 0, tmp, &tot);
    if (v) P.pack[ci] = (int)i;
    if (in) P.unpack[i] = v ? ci : -1;
    __syncthreads();  // the predecessors' pack entries of this chunk are written
    bool start = false, hole = false;
    if (v) {
      const int64_t row0 = (i / seqlen) * seqlen;
      const int prev = ci > 0 ? P.pack[ci - 1] : -1;
      start = prev < row0 || (ids && ids[prev] != ids[i]);
      hole = !start && prev != i - 1;
    }
    int dtot;
    const int d = ndocs + block_excl_scan(start ? 1 : 0, tmp, &dtot);
    if (start) {
      P.tstream[d + lead] = (int)i;
      P.tpack[d + lead] = ci;
    }
    if (hole) atomicOr(&s_holes, 1);
    nvalid += tot;
    ndocs += dtot;
  }
  __syncthreads();
  const bool packed = s_holes != 0;
  const int n = packed ? ndocs : ndocs + lead;
  const int off = packed ? lead : 0;
  int mx = 0;
  for (int k = tid; k < n; k += kPlanThreads) {
    if (packed) {
      const int a = P.tpack[k + off];
      const int e = k + 1 < n ? P.tpack[k + 1 + off] : nvalid;
      P.cu[k] = a;
      P.seqused[k] = e - a;
      mx = max(mx, e - a);
    } else {
      const int a = k < lead ? 0 : P.tstream[k];
      const int e = k + 1 < n ? P.tstream[k + 1] : (int)N;
      const int u = k < lead ? 0 : (k + 1 < n ? P.tpack[k + 1] : nvalid) - P.tpack[k];
      P.cu[k] = a;
      P.seqused[k] = u;
      mx = max(mx, e - a);
    }
  }
  atomicMax(&s_max, mx);
  __syncthreads();
  if (tid == 0) {
    P.cu[n] = packed ? nvalid : (int)N;
    P.info[0] = n;
    P.info[1] = s_max;
    P.info[2] = packed ? nvalid : (int)N;
    P.info[3] = packed ? 1 : 0;
    P.info[4] = nvalid;
    P.info[5] = ndocs;
    P.info[6] = 0;
    P.info[7] = 0;
  }
}

// dst row r = src row index[r], or `fill` words where index[r] < 0. Rows are
// `row_words` units of W bytes (16 or 4); grid-stride over (row, unit).
template <typename U>
__global__ __launch_bounds__(256) void copy_rows_kernel(const U* __restrict__ src,
                                                        const int* __restrict__ index,
                                                        int64_t n_rows, int64_t row_units, U fill,
                                                        U* __restrict__ dst) {
  const int64_t total = n_rows * row_units;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total;
       e += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = e / row_units, w = e - r * row_units;
    const int s = index[r];
    dst[e] = s >= 0 ? src[(int64_t)s * row_units + w] : fill;
  }
}

}  // namespace

}  // namespace flint

using namespace flint;

extern "C" size_t flint_attn_bshd_plan_bytes(int32_t batch, int32_t seqlen) {
  if (batch < 0 || seqlen < 0) return 0;
  const int64_t N = (int64_t)batch * seqlen;
  return (size_t)(8 + 6 * N + 3) * sizeof(int32_t);
}

extern "C" int flint_attn_bshd_plan(const uint8_t* attention_mask, const int32_t* document_ids,
                                    int32_t batch, int32_t seqlen, void* plan, size_t plan_bytes,
                                    void* stream) {
  if (batch < 0 || seqlen < 0) return FLINT_ERR_SHAPE;
  const int64_t N = (int64_t)batch * seqlen;
  if (N >= (int64_t)1 << 30) return FLINT_ERR_SHAPE;
  if (!plan) return FLINT_ERR_NULL;
  if (!aligned(plan, 4) || (document_ids && !aligned(document_ids, 4))) return FLINT_ERR_ALIGN;
  if (plan_bytes < flint_attn_bshd_plan_bytes(batch, seqlen)) return FLINT_ERR_WORKSPACE;
  (void)hipGetLastError();
  bshd_plan_kernel<<<1, kPlanThreads, 0, reinterpret_cast<hipStream_t>(stream)>>>(
      N > 0 ? attention_mask : nullptr, N > 0 ? document_ids : nullptr, batch, seqlen,
      static_cast<int*>(plan));
  if (hipGetLastError() != hipSuccess) return FLINT_ERR_HIP;
  return FLINT_OK;
}

extern "C" int flint_attn_copy_rows(const void* src, const int32_t* index, int32_t n_rows,
                                    int32_t row_bytes, uint32_t fill, void* dst, void* stream) {
  if (n_rows < 0 || row_bytes <= 0 || (row_bytes & 3)) return FLINT_ERR_SHAPE;
  if (n_rows == 0) return FLINT_OK;
  if (!src || !index || !dst) return FLINT_ERR_NULL;
  const bool wide = (row_bytes & 15) == 0 && aligned(src, 16) && aligned(dst, 16);
  if (!aligned(src, 4) || !aligned(dst, 4) || !aligned(index, 4)) return FLINT_ERR_ALIGN;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const int64_t units = wide ? row_bytes / 16 : row_bytes / 4;
  const int64_t total = (int64_t)n_rows * units;
  const unsigned grid = (unsigned)std::min<int64_t>((total + 255) / 256, 8192);
  (void)hipGetLastError();
  if (wide)
    copy_rows_kernel<uint4><<<grid, 256, 0, st>>>(static_cast<const uint4*>(src), index, n_rows,
                                                  units, make_uint4(fill, fill, fill, fill),
                                                  static_cast<uint4*>(dst));
  else
    copy_rows_kernel<uint32_t><<<grid, 256, 0, st>>>(static_cast<const uint32_t*>(src), index,
                                                     n_rows, units, fill,
                                                     static_cast<uint32_t*>(dst));
  if (hipGetLastError() != hipSuccess) return FLINT_ERR_HIP;
  return FLINT_OK;
}
