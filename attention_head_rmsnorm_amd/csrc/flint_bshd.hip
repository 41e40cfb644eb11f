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

constexpr int kPlanThreads = 1024;  // one token per thread, one block per 1024 tokens

struct PlanPtrs {
  int* info;
  int* cu;
  int* seqused;
  int* pack;
  int* unpack;
  int* tstream;   // stream position of each sequence's first token (index d + lead)
  int* tpack;     // packed index of each document's first token (index d + lead)
  int* agg_valid;  // per block of tokens: valid tokens
  int* agg_last;   // per block: largest valid token index, -1 if none
  int* agg_docs;   // per block: document starts
};

__host__ __device__ inline int64_t plan_blocks(int64_t N) { return (N + kPlanThreads - 1) / kPlanThreads; }

__host__ __device__ inline PlanPtrs plan_ptrs(int* base, int64_t N) {
  PlanPtrs p;
  const int64_t nb = plan_blocks(N);
  p.info = base;
  p.cu = base + 8;
  p.seqused = p.cu + N + 1;
  p.pack = p.seqused + N;
  p.unpack = p.pack + N;
  p.tstream = p.unpack + N;
  p.tpack = p.tstream + N + 1;
  p.agg_valid = p.tpack + N + 1;
  p.agg_last = p.agg_valid + nb;
  p.agg_docs = p.agg_last + nb;
  return p;
}

// Exclusive max-scan over the 1024 threads of a block (identity -1).
__device__ int block_excl_max(int v, int* tmp) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off);
    if (lane >= off) x = max(x, y);
  }
  int ex = __shfl_up(x, 1);
  if (lane == 0) ex = -1;
  if (lane == 63) tmp[wave] = x;
  __syncthreads();
  int before = -1;
  for (int w = 0; w < wave; ++w) before = max(before, tmp[w]);
  __syncthreads();
  return max(before, ex);
}

// Sum (or max) of a per-block array over blocks [0, b), by the whole block.
__device__ int prefix_over_blocks(const int* agg, int b, bool take_max, int* tmp) {
  int x = take_max ? -1 : 0;
  for (int j = threadIdx.x; j < b; j += kPlanThreads) x = take_max ? max(x, agg[j]) : x + agg[j];
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const int y = __shfl_xor(x, off);
    x = take_max ? max(x, y) : x + y;
  }
  if ((threadIdx.x & 63) == 0) tmp[threadIdx.x >> 6] = x;
  __syncthreads();
  int r = take_max ? -1 : 0;
  for (int w = 0; w < kPlanThreads / 64; ++w) r = take_max ? max(r, tmp[w]) : r + tmp[w];
  __syncthreads();
  return r;
}

__device__ __forceinline__ bool token_valid(const uint8_t* mask, int64_t i, int64_t N) {
  return i < N && (!mask || mask[i] != 0);
}

// Phase 1: per block, its valid tokens and its last valid token.
__global__ __launch_bounds__(kPlanThreads) void plan_count_kernel(const uint8_t* __restrict__ mask,
                                                                  int64_t N, int* __restrict__ plan) {
  __shared__ int tmp[16];
  const PlanPtrs P = plan_ptrs(plan, N);
  const int b = blockIdx.x;
  const int64_t i = (int64_t)b * kPlanThreads + threadIdx.x;
  const bool v = token_valid(mask, i, N);
  int tot;
  (void)block_excl_scan(v ? 1 : 0, tmp, &tot);
  int last = v ? (int)i : -1;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) last = max(last, __shfl_xor(last, off));
  if ((threadIdx.x & 63) == 0) tmp[threadIdx.x >> 6] = last;
  __syncthreads();
  if (threadIdx.x == 0) {
    int m = -1;
    for (int w = 0; w < 16; ++w) m = max(m, tmp[w]);
    P.agg_valid[b] = tot;
    P.agg_last[b] = m;
    if (b == 0) {
      P.info[1] = 0;  // max_seqlen, raised by the last phase
      P.info[6] = 0;  // holes
    }
  }
}

// A token's place: packed index ci, whether it starts a document (first valid
// token of its row, or an id different from the previous valid token's) and
// whether it follows a hole (the previous valid token of its document is not
// the token just before it).
struct TokenPlace {
  bool v, start, hole;
  int ci;
};

__device__ TokenPlace token_place(const uint8_t* mask, const int* ids, int seqlen, int64_t N,
                                  const PlanPtrs& P, int* tmp) {
  const int b = blockIdx.x;
  const int64_t i = (int64_t)b * kPlanThreads + threadIdx.x;
  TokenPlace t;
  t.v = token_valid(mask, i, N);
  const int valid_before = prefix_over_blocks(P.agg_valid, b, false, tmp);
  const int last_before = prefix_over_blocks(P.agg_last, b, true, tmp);
  int tot;
  t.ci = valid_before + block_excl_scan(t.v ? 1 : 0, tmp, &tot);
  const int prev = max(last_before, block_excl_max(t.v ? (int)i : -1, tmp));
  t.start = t.hole = false;
  if (t.v) {
    const int64_t row0 = (i / seqlen) * seqlen;
    t.start = prev < row0 || (ids && ids[prev] != ids[i]);
    t.hole = !t.start && prev != i - 1;
  }
  return t;
}

// Phase 2: per block, its document starts; any hole sets the packed flag.
__global__ __launch_bounds__(kPlanThreads) void plan_docs_kernel(const uint8_t* __restrict__ mask,
                                                                 const int* __restrict__ ids,
                                                                 int seqlen, int64_t N,
                                                                 int* __restrict__ plan) {
  __shared__ int tmp[16];
  const PlanPtrs P = plan_ptrs(plan, N);
  const TokenPlace t = token_place(mask, ids, seqlen, N, P, tmp);
  int tot;
  (void)block_excl_scan(t.start ? 1 : 0, tmp, &tot);
  const bool hole = __syncthreads_or(t.hole);
  if (threadIdx.x == 0) {
    P.agg_docs[blockIdx.x] = tot;
    if (hole) atomicOr(&P.info[6], 1);
  }
}

// Phase 3: pack / unpack of every token, first token of every document.
__global__ __launch_bounds__(kPlanThreads) void plan_place_kernel(const uint8_t* __restrict__ mask,
                                                                  const int* __restrict__ ids,
                                                                  int seqlen, int64_t N,
                                                                  int* __restrict__ plan) {
  __shared__ int tmp[16];
  const PlanPtrs P = plan_ptrs(plan, N);
  const TokenPlace t = token_place(mask, ids, seqlen, N, P, tmp);
  const int docs_before = prefix_over_blocks(P.agg_docs, blockIdx.x, false, tmp);
  int tot;
  const int d = docs_before + block_excl_scan(t.start ? 1 : 0, tmp, &tot);
  const int64_t i = (int64_t)blockIdx.x * kPlanThreads + threadIdx.x;
  const int lead = (mask && mask[0] == 0) ? 1 : 0;
  if (t.v) P.pack[t.ci] = (int)i;
  if (i < N) P.unpack[i] = t.v ? t.ci : -1;
  if (t.start) {
    P.tstream[d + lead] = (int)i;
    P.tpack[d + lead] = t.ci;
  }
}

// Phase 4: the sequences (one per document, plus the leading padding when the
// stream starts with it and is used in place): cu_seqlens, valid lengths, the
// longest sequence and the counts.
__global__ __launch_bounds__(kPlanThreads) void plan_seqs_kernel(const uint8_t* __restrict__ mask,
                                                                 int64_t N, int* __restrict__ plan) {
  __shared__ int tmp[16];
  const PlanPtrs P = plan_ptrs(plan, N);
  const int nb = (int)plan_blocks(N);
  const int nvalid = prefix_over_blocks(P.agg_valid, nb, false, tmp);
  const int ndocs = prefix_over_blocks(P.agg_docs, nb, false, tmp);
  const bool packed = P.info[6] != 0;
  const int lead = (mask && mask[0] == 0) ? 1 : 0;
  const int n = packed ? ndocs : ndocs + lead;
  const int off = packed ? lead : 0;
  const int k = blockIdx.x * kPlanThreads + threadIdx.x;
  int len = 0;
  if (k < n) {
    if (packed) {
      const int a = P.tpack[k + off];
      const int e = k + 1 < n ? P.tpack[k + 1 + off] : nvalid;
      P.cu[k] = a;
      P.seqused[k] = e - a;
      len = e - a;
    } else {
      const int a = k < lead ? 0 : P.tstream[k];
      const int e = k + 1 < n ? P.tstream[k + 1] : (int)N;
      P.cu[k] = a;
      P.seqused[k] = k < lead ? 0 : (k + 1 < n ? P.tpack[k + 1] : nvalid) - P.tpack[k];
      len = e - a;
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) len = max(len, __shfl_xor(len, o));
  if ((threadIdx.x & 63) == 0 && len > 0) atomicMax(&P.info[1], len);
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    P.cu[n] = packed ? nvalid : (int)N;
    P.info[0] = n;
    P.info[2] = packed ? nvalid : (int)N;
    P.info[3] = packed ? 1 : 0;
    P.info[4] = nvalid;
    P.info[5] = ndocs;
    P.info[7] = 0;
  }
}

__global__ void fill_kernel(int* __restrict__ p, int n, int value) {
  for (int i = threadIdx.x; i < n; i += blockDim.x) p[i] = value;
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
  return (size_t)(8 + 6 * N + 3 + 3 * plan_blocks(N)) * sizeof(int32_t);
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
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  int* p = static_cast<int*>(plan);
  (void)hipGetLastError();
  if (N == 0) {
    fill_kernel<<<1, 64, 0, st>>>(p, 9, 0);  // info and cu[0]
  } else {
    const unsigned nb = (unsigned)plan_blocks(N);
    plan_count_kernel<<<nb, kPlanThreads, 0, st>>>(attention_mask, N, p);
    plan_docs_kernel<<<nb, kPlanThreads, 0, st>>>(attention_mask, document_ids, seqlen, N, p);
    plan_place_kernel<<<nb, kPlanThreads, 0, st>>>(attention_mask, document_ids, seqlen, N, p);
    // sequences: at most one per valid token plus the leading padding
    plan_seqs_kernel<<<nb, kPlanThreads, 0, st>>>(attention_mask, N, p);
  }
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
