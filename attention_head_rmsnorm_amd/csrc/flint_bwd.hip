// Flint sink-aware attention backward for AMD Instinct MI355X (gfx950).
//
// Gradients of the layer of flint_attn.hip (NeMo AutoModel "flint" page,
// "Model Architecture"; flint.layers API page, FlintAttention; Hugging Face
// discussion #26 on RecursiveSI/flint, "What was unusually easy", and "Where
// other stacks fail" for the sink in backward). With Z = Q'K'^T / sqrt(d),
// W the sink softmax and O = W V, an upstream dO gives
//   Dr = rowsum(dO * O),  dZ = W * (dO V^T - Dr),
//   dV = W^T dO,  dQ' = dZ K' / sqrt(d),  dK' = dZ^T Q' / sqrt(d),
//   d sink_h = -sum_t p_sink(t, h) Dr(t, h)   (the sink has value 0),
// then the adjoint of the RoPE rotation (the opposite turn) and of the
// weight-form RMSNorm, which also yields the two norm-weight gradients.
// W is recomputed from the forward's per-row normalizer lse: W = exp(Z - lse).
//
// Kernels, in order on the caller's stream:
//   schedule_kernel (forward)  sequence table, key tiles, query blocks.
//   bwd_schedule_kernel   one workgroup: cuts the query range seen by each
//                         256-key block at fixed chunk boundaries and orders
//                         the chunks by query position, so the workgroups on
//                         one L2 share the query tiles they stream.
//   bwd_kv_prep_kernel    per (64-key tile, kv head): K' = RoPE(RMSNorm(k)) in
//                         bf16 as a K' operand tile, V as a V operand tile, and
//                         K'^T in the key-slot order of the dQ product; zero dq
//                         rows of padded tokens.
//   bwd_q_prep_kernel     per (32-query block, kv head), its 8 query heads in
//                         turn: Q' (with the softmax scale in log2 units, the
//                         bits the forward forms) as a swizzled operand tile,
//                         the row terms lse (log2 units) and Dr, the block's
//                         share of the sink adjoint.
//   bwd_dq_kernel         query-major: per (query block, the 8 heads of a kv head),
//                         over the key tiles in the window: S^T = K'Q'^T,
//                         dP^T = V dO^T, dS^T, dQ'^T += K'^T dS^T; then RoPE and
//                         RMSNorm adjoints, dq, and the block's q-norm-weight
//                         terms.
//   bwd_dkdv_kernel       key-major: per (256 keys, kv head, query chunk), over
//                         the chunk's query blocks x 8 heads: S = Q'K'^T,
//                         dP = dO V^T, dS, dV^T += dO^T P, dK'^T += Q'^T dS, as
//                         FP32 partial sums of the chunk.
//   bwd_kv_reduce_kernel  per (64-key tile, kv head): sums the chunks in a fixed
//                         order, RoPE and RMSNorm adjoints, dk, dv, and the
//                         tile's k-norm-weight terms.
//   bwd_finalize_kernel   sums the norm-weight terms and the sink shares in a
//                         fixed order (the result does not depend on timing).
// Every product runs on v_mfma_f32_32x32x16_bf16 with FP32 accumulation.

#include <hip/hip_runtime.h>

#include "flint_common.h"

namespace flint {

constexpr int kKvbPart = kBN * kD * 2;       // 16 KiB: one 64-key operand part
constexpr int kKvbBytes = 3 * kKvbPart;      // K' | V | K'^T (key-slot order)
constexpr int kQtPart = kBM * kD * 2;        // 8 KiB: one 32-query operand part
constexpr int kQtStats = 2 * kBM * 4;        // lse (log2 units) [32], Dr [32]
constexpr int kQtBytes = kQtPart + kQtStats;  // Q' in swizzled operand order | stats
constexpr int kBwdStages = 3;
constexpr int kKBTiles = 4;                  // key tiles per dK/dV item
constexpr int kKB = kKBTiles * kBN;          // keys per dK/dV item (one wave per 32)
constexpr int kTargetChunks = 1024;          // about this many key-major items per kv head
constexpr int kMinChunkQB = 8;               // query blocks per chunk, at least (sliding layers)
constexpr int kMinChunkQBFull = 16;          // the same for full attention
constexpr int kXcds = 8;                     // L2 domains; workgroups reach them round robin
constexpr int kHdrNC = 8;                    // header: key-major items
constexpr int kHdrCH = 9;                    // header: query blocks per chunk
constexpr float kInvSqrtD = 0.08838834764831845f;
constexpr int kPartFloats = 2 * kKB * kD;    // dK' and dV of one chunk

struct BwdWs {
  Ws f;            // the forward schedule's regions
  char* kvb;       // [kG][ntmax][kKvbBytes]
  char* qt;        // [nqmax][kH][kQtBytes]
  float* sinkpart; // [kH][nqmax]: sum over the block's rows of p_sink * Dr
  float* wq;       // [kD][nqmax * kG]: q-norm-weight terms per (query block, kv head)
  float* wk;       // [kD][ntmax * kG]: k-norm-weight terms per (tile, kv head)
  int* cb;         // [ntmax] first chunk slot of the key block starting at tile e
  int* nc;         // [ntmax] its chunks
  int2* kitems;    // [ncmax] {tile, chunk}, by the chunk's global query position
  float* part;     // [ncmax][kG][kPartFloats]
  int nqmax, ncmax, n;
};

struct BwdLayout {
  Layout f;
  size_t kvb, qt, sinkpart, wq, wk, cb, nc, kitems, part, total;
  int64_t ncmax;
};

static BwdLayout make_bwd_layout(int64_t T, int64_t n) {
  BwdLayout L;
  L.f = make_layout(T, n, false);
  // chunks of a key block: at most work / CH + 2; key blocks: at most (ntmax + 3n) / 4
  L.ncmax = kTargetChunks + L.f.ntmax + n;
  size_t o = L.f.total;
  L.kvb = o;      o = align_up(o + (size_t)kG * L.f.ntmax * kKvbBytes, 256);
  L.qt = o;       o = align_up(o + (size_t)L.f.nqmax * kH * kQtBytes, 256);
  L.sinkpart = o; o = align_up(o + (size_t)kH * L.f.nqmax * 4, 256);
  L.wq = o;       o = align_up(o + (size_t)kD * L.f.nqmax * kG * 4, 256);
  L.wk = o;       o = align_up(o + (size_t)kD * L.f.ntmax * kG * 4, 256);
  L.cb = o;       o = align_up(o + (size_t)L.f.ntmax * 4, 256);
  L.nc = o;       o = align_up(o + (size_t)L.f.ntmax * 4, 256);
  L.kitems = o;   o = align_up(o + (size_t)L.ncmax * 8, 256);
  L.part = o;     o = align_up(o + (size_t)L.ncmax * kG * kPartFloats * 4, 256);
  L.total = o;
  return L;
}

// ----------------------------------------------------------------- helpers

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_of(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, kBufferWord3);
}

// One 16-byte vector per lane from global memory straight into LDS: lane L's
// vector lands at `lds` + 16 L.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, int voff, int soff, void* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16,
                                           voff, soff, 0, 0);
}

__device__ __forceinline__ void dma4(__amdgpu_buffer_rsrc_t r, int voff, int soff, void* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 4,
                                           voff, soff, 0, 0);
}

__device__ __forceinline__ bf16x8 ld_frag(const uint4* p) { return __builtin_bit_cast(bf16x8, *p); }

// Swizzled operand order of the 32-query tiles (Q' and dO): row r's channels
// 16kk + 8half .. + 8 sit at 16-byte unit 64kk + 32half + (r ^ 8half). A
// 16-byte operand read of k-step kk is a permutation of one 1 KiB unit run,
// conflict free; lane `lane` reads unit 64kk + swz(lane).
__device__ __forceinline__ int swz(int lane) { return lane ^ ((lane >> 5) << 3); }


__device__ __forceinline__ bf16x8 pack_frag(const float* x) { return __builtin_bit_cast(bf16x8, pack8(x)); }

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Query blocks [*lo, *hi) that see some key of the 256-key block starting at
// key k0 of a sequence with valid length u (none when k0 >= u).
__device__ __forceinline__ void kb_queries(int k0, int u, int window, int* lo, int* hi) {
  if (k0 >= u) {
    *lo = *hi = 0;
    return;
  }
  const int last_key = min(k0 + kKB, u) - 1;
  const int q_end = window > 0 ? min(u, last_key + window) : u;
  *lo = k0 / kBM;
  *hi = (q_end + kBM - 1) / kBM;
}

// Query blocks [*lo, *hi) seen by the key block that starts at tile e; empty
// for tiles inside a key block (one is kKBTiles tiles) and for key blocks of
// padding.
// Returns the tile's sequence.
__device__ __forceinline__ int kb_range(const BwdWs& ws, int e, int window, int* lo, int* hi) {
  const int2 te = ws.f.tiles[e];
  *lo = *hi = 0;
  if (te.y % kKBTiles) return te.x;
  kb_queries(te.y * kBN, ws.f.seq[te.x].z, window, lo, hi);
  return te.x;
}

// ----------------------------------------------------------------- schedule

// Key-major work items. The query range seen by a 256-key block is cut at
// fixed query-block positions, multiples of CH: chunk c of a sequence covers
// its query blocks [c CH, (c + 1) CH). Every key block overlapping chunk c
// reads the same Q'/dO tiles, so the item list is sorted by the chunk's
// global position, and each of the kXcds L2 domains takes one contiguous
// stretch of it (per kv head): the workgroups running together on one L2
// stream the same tiles at about the same time. CH grows with the total work
// so there are about kTargetChunks chunks per kv head.
__global__ __launch_bounds__(1024) void bwd_schedule_kernel(int window, BwdWs ws) {
  __shared__ int tmp[1024];
  __shared__ int hist[kBuckets];
  const int tid = threadIdx.x;
  const int NT = ws.f.hdr[1];
  int lo, hi;
  int local = 0;
  for (int e = tid; e < NT; e += 1024) {
    kb_range(ws, e, window, &lo, &hi);
    local += hi - lo;
  }
  int total;
  (void)block_excl_scan(local, tmp, &total);
  // Full layers take longer chunks: half the FP32 partials to write and sum
  // (measured 2-4% faster at 8,192 tokens). A 513-key window spans too few
  // query blocks for that (7% slower on 8 x 8,192 sliding).
  const int CH = max(window > 0 ? kMinChunkQB : kMinChunkQBFull,
                     (total + kTargetChunks - 1) / kTargetChunks);

  int carry = 0;
  for (int base = 0; base < NT; base += 1024) {
    const int e = base + tid;
    int c = 0;
    if (e < NT) {
      kb_range(ws, e, window, &lo, &hi);
      c = hi > lo ? (hi + CH - 1) / CH - lo / CH : 0;
    }
    int tot;
    const int ex = block_excl_scan(c, tmp, &tot);
    if (e < NT) {
      ws.cb[e] = carry + ex;
      ws.nc[e] = c;
    }
    carry += tot;
  }
  // counting sort by the chunk's global query position (qbase + c CH) / CH
  for (int i = tid; i < kBuckets; i += 1024) hist[i] = 0;
  __syncthreads();
  for (int e = tid; e < NT; e += 1024) {
    const int sq = kb_range(ws, e, window, &lo, &hi);
    const int qb = ws.f.qbase[sq];
    for (int c = lo / CH; c * CH < hi; ++c) atomicAdd(&hist[min((qb + c * CH) / CH, kBuckets - 1)], 1);
  }
  __syncthreads();
  int local4[4], sum = 0;
  for (int j = 0; j < 4; ++j) {
    local4[j] = hist[4 * tid + j];
    sum += local4[j];
  }
  int tot;
  int run = block_excl_scan(sum, tmp, &tot);
  for (int j = 0; j < 4; ++j) {
    hist[4 * tid + j] = run;
    run += local4[j];
  }
  __syncthreads();
  for (int e = tid; e < NT; e += 1024) {
    const int sq = kb_range(ws, e, window, &lo, &hi);
    const int qb = ws.f.qbase[sq];
    for (int c = lo / CH; c * CH < hi; ++c) {
      const int pos = atomicAdd(&hist[min((qb + c * CH) / CH, kBuckets - 1)], 1);
      ws.kitems[pos] = make_int2(e, c);
    }
  }
  if (tid == 0) {
    ws.f.hdr[kHdrNC] = carry;
    ws.f.hdr[kHdrCH] = CH;
  }
}

// ----------------------------------------------------------------- K/V prep

__global__ __launch_bounds__(256) void bwd_kv_prep_kernel(const uint16_t* __restrict__ k,
                                                          const uint16_t* __restrict__ v,
                                                          const float* __restrict__ k_norm_w,
                                                          const int* __restrict__ positions,
                                                          float eps, int use_rope, BwdWs ws,
                                                          uint16_t* __restrict__ dq) {
  __shared__ __attribute__((aligned(16))) uint16_t kt[kD * kBN];
  const int e = blockIdx.x, g = blockIdx.y;
  if (e >= ws.f.hdr[1]) return;
  const int2 te = ws.f.tiles[e];
  const int4 meta = ws.f.seq[te.x];
  const int start = meta.x, len = meta.y, u = meta.z;
  const int tid = threadIdx.x, r = tid >> 2, p = tid & 3;
  const int ell = te.y * kBN + r;
  const bool valid = ell < u;
  const size_t t = (size_t)start + ell;
  char* tile = ws.kvb + ((size_t)g * ws.f.ntmax + e) * kKvbBytes;
  const int b = r >> 5, col = r & 31;

  // K': channels [16p, 16p+16) and their RoPE partners +64.
  float x[32];
  if (valid) {
    const uint4* src = reinterpret_cast<const uint4*>(k + (t * kG + g) * kD);
    unpack8(src[2 * p], x);
    unpack8(src[2 * p + 1], x + 8);
    unpack8(src[8 + 2 * p], x + 16);
    unpack8(src[9 + 2 * p], x + 24);
  } else {
#pragma unroll
    for (int i = 0; i < 32; ++i) x[i] = 0.f;
  }
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) ss += x[i] * x[i];
  ss += __shfl_xor(ss, 1);
  ss += __shfl_xor(ss, 2);
  const float rstd = 1.0f / sqrtf(ss * (1.0f / kD) + eps);
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    x[i] *= rstd * k_norm_w[16 * p + i];
    x[16 + i] *= rstd * k_norm_w[64 + 16 * p + i];
  }
  if (use_rope && valid) {
    const int pos = positions ? positions[t] : ell;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float c, s;
      rope_cos_sin(pos, ws.f.rope[16 * p + i], &c, &s);
      rope_turn(x[i], x[16 + i], c, s);
    }
  }
  {
    uint4* kfrag = reinterpret_cast<uint4*>(tile);
    const uint4 w[4] = {pack8(x), pack8(x + 8), pack8(x + 16), pack8(x + 24)};
    kfrag[frag_index(b, 8, p, 0, col)] = w[0];
    kfrag[frag_index(b, 8, p, 1, col)] = w[1];
    kfrag[frag_index(b, 8, 4 + p, 0, col)] = w[2];
    kfrag[frag_index(b, 8, 4 + p, 1, col)] = w[3];
    // K'^T in key-slot order, through LDS
    const int slot = vt_slot(r);
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const uint32_t w4[4] = {w[q4].x, w[q4].y, w[q4].z, w[q4].w};
      const int d0 = (q4 < 2 ? 16 * p + 8 * q4 : 64 + 16 * p + 8 * (q4 - 2));
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        kt[(d0 + 2 * j) * kBN + slot] = (uint16_t)(w4[j] & 0xffff);
        kt[(d0 + 2 * j + 1) * kBN + slot] = (uint16_t)(w4[j] >> 16);
      }
    }
  }
  // V operand tile: key rows, channels [32p, 32p+32)
  {
    uint4* vfrag = reinterpret_cast<uint4*>(tile + kKvbPart);
    const uint4* src = reinterpret_cast<const uint4*>(v + (t * kG + g) * kD);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      vfrag[frag_index(b, 8, 2 * p + (i >> 1), i & 1, col)] = valid ? src[4 * p + i] : make_uint4(0, 0, 0, 0);
  }
  __syncthreads();
  {
    uint4* ktile = reinterpret_cast<uint4*>(tile + 2 * kKvbPart);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int qv = tid + 256 * i;
      const int d = qv >> 3, c = qv & 7;
      ktile[frag_index(d >> 5, 4, c >> 1, c & 1, d & 31)] =
          *reinterpret_cast<const uint4*>(&kt[d * kBN + c * 8]);
    }
  }
  // Padded query rows of this kv head's 8 query heads get zero gradients.
  if (ell >= u && ell < len) {
    uint4* dst = reinterpret_cast<uint4*>(dq + (t * kH + (size_t)g * kHpg) * kD);
    const uint4 z = make_uint4(0, 0, 0, 0);
#pragma unroll 4
    for (int i = 0; i < 32; ++i) dst[p * 32 + i] = z;
  }
}

// ----------------------------------------------------------------- Q / dO prep

// cos and sin of the RoPE angles of a thread's 8 channel pairs (8p + i) at
// position pos.
template <bool kMixed>
__device__ __forceinline__ void rope_table8(int pos, const RopeFreq* fr, float* cs, float* sn) {
  const float pf = (float)pos;
#pragma unroll
  for (int i = 0; i < 8; ++i) rope_cos_sin<kMixed>(pos, pf, fr[i], &cs[i], &sn[i]);
}

// DPP moves: row_shl:n (0x100 + n) gives lane L the value of lane L + n within
// its 16-lane row; the quad permutation [1,0,3,2] (0xB1) the value of lane ^ 1.
__device__ __forceinline__ float dpp_xor1(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));
}

template <int kCtrl>
__device__ __forceinline__ uint4 dpp_u4(const uint4& x) {
  return make_uint4((unsigned)__builtin_amdgcn_update_dpp(0, (int)x.x, kCtrl, 0xF, 0xF, false),
                    (unsigned)__builtin_amdgcn_update_dpp(0, (int)x.y, kCtrl, 0xF, 0xF, false),
                    (unsigned)__builtin_amdgcn_update_dpp(0, (int)x.z, kCtrl, 0xF, 0xF, false),
                    (unsigned)__builtin_amdgcn_update_dpp(0, (int)x.w, kCtrl, 0xF, 0xF, false));
}

// Per (32-query block, kv head): the block's rows of the kv head's 8 query
// heads in turn. Thread (row r, part p) holds channels [8p, 8p+8) (16-byte
// unit p of the row) and their RoPE partners +64 (unit 8 + p). The RoPE angles
// and the norm weights depend on the row and the channels only, so they are
// formed once for the 8 heads. Q' is formed with the attention kernel's own
// operations in its order, so its bits are the forward's: the sum of squares
// of each half-row (units 2kk + half, kk = 0..7, by v_dot2 in turn) is formed
// by thread p = half from units gathered from its 8-thread group, the two
// halves are added, then the norm weight times the softmax scale and the RoPE
// turn.
__global__ __launch_bounds__(256) void bwd_q_prep_kernel(const uint16_t* __restrict__ q,
                                                         const uint16_t* __restrict__ o,
                                                         const uint16_t* __restrict__ dout,
                                                         const float* __restrict__ lse,
                                                         const float* __restrict__ q_norm_w,
                                                         const float* __restrict__ sink,
                                                         const int* __restrict__ positions,
                                                         float eps, int use_rope, BwdWs ws) {
  __shared__ float red[4][kHpg];
  const int qg = blockIdx.x, g = blockIdx.y;
  if (qg >= ws.f.hdr[2]) return;
  const int s = find_seq(ws.f.qbase, ws.n, qg);
  const int qb = qg - ws.f.qbase[s];
  const int4 meta = ws.f.seq[s];
  const int start = meta.x, u = meta.z;
  const int tid = threadIdx.x, lane = tid & 63, r = tid >> 3, p = tid & 7;
  const int ell = qb * kBM + r;
  const bool valid = ell < u;
  const size_t t = (size_t)start + ell;

  float wlo[8], whi[8];  // q_norm weights times the softmax scale, as the forward holds them
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    wlo[i] = q_norm_w[8 * p + i] * kQScale;
    whi[i] = q_norm_w[64 + 8 * p + i] * kQScale;
  }
  float cs[8], sn[8];
  const bool rot = use_rope && valid;
  if (rot) {
    const int pos = positions ? positions[t] : ell;
    if (!rope_wave_mixed(pos)) rope_table8<false>(pos, ws.f.rope + 8 * p, cs, sn);
    else rope_table8<true>(pos, ws.f.rope + 8 * p, cs, sn);
  }
  // channels 8p.. are k-step p>>1, half p&1; channels 64+8p.. are k-step
  // 4+(p>>1); swizzled operand order (unit 64kk + 32half + (r ^ 8half))
  const int su = 32 * (p & 1) + (r ^ (8 * (p & 1)));
  const uint4 z4 = make_uint4(0, 0, 0, 0);

#pragma unroll 1
  for (int hl = 0; hl < kHpg; ++hl) {
    const int h = g * kHpg + hl;
    char* tile = ws.qt + ((size_t)qg * kH + h) * kQtBytes;
    const size_t row = (t * kH + h) * kD;
    const uint4 qa = valid ? *reinterpret_cast<const uint4*>(q + row + 8 * p) : z4;
    const uint4 qc = valid ? *reinterpret_cast<const uint4*>(q + row + 64 + 8 * p) : z4;
    const uint4 da = valid ? *reinterpret_cast<const uint4*>(dout + row + 8 * p) : z4;
    const uint4 dc = valid ? *reinterpret_cast<const uint4*>(dout + row + 64 + 8 * p) : z4;
    const uint4 oa = valid ? *reinterpret_cast<const uint4*>(o + row + 8 * p) : z4;
    const uint4 oc = valid ? *reinterpret_cast<const uint4*>(o + row + 64 + 8 * p) : z4;
    const float lv = valid ? lse[t * kH + h] : 0.f;
    // sum of squares of the half-row of thread p = half (p < 2): units
    // p, p + 2, p + 4, p + 6 (its own and its group's qa) then the same of qc
    float ss;
    {
      const uint4 a2 = dpp_u4<0x102>(qa), a4 = dpp_u4<0x104>(qa), a6 = dpp_u4<0x106>(qa);
      const uint4 c2 = dpp_u4<0x102>(qc), c4 = dpp_u4<0x104>(qc), c6 = dpp_u4<0x106>(qc);
      float sh = sumsq8_dot(qa, 0.f);
      sh = sumsq8_dot(a2, sh);
      sh = sumsq8_dot(a4, sh);
      sh = sumsq8_dot(a6, sh);
      sh = sumsq8_dot(qc, sh);
      sh = sumsq8_dot(c2, sh);
      sh = sumsq8_dot(c4, sh);
      sh = sumsq8_dot(c6, sh);
      ss = sh + dpp_xor1(sh);   // thread 0 of the group: half 0's sum plus half 1's
      ss = __shfl(ss, lane & ~7);         // to the group's 8 threads
    }
    float x[16], dy[16], y[16];
    unpack8(qa, x);
    unpack8(qc, x + 8);
    unpack8(da, dy);
    unpack8(dc, dy + 8);
    unpack8(oa, y);
    unpack8(oc, y + 8);
    float dr = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) dr += dy[i] * y[i];
#pragma unroll
    for (int off = 1; off < 8; off <<= 1) dr += __shfl_xor(dr, off);
    const float rstd = 1.0f / sqrtf(ss * (1.0f / kD) + eps);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      x[i] *= rstd * wlo[i];
      x[8 + i] *= rstd * whi[i];
      if (rot) rope_turn(x[i], x[8 + i], cs[i], sn[i]);
    }
    uint4* qf = reinterpret_cast<uint4*>(tile);
    qf[64 * (p >> 1) + su] = pack8(x);
    qf[64 * (4 + (p >> 1)) + su] = pack8(x + 8);
    // row terms and the block's share of the sink adjoint
    float* stats = reinterpret_cast<float*>(tile + kQtPart);
    const float l2 = valid ? lv * kLog2e : INFINITY;
    float share = 0.f;
    if (p == 0) {
      stats[r] = l2;
      stats[kBM + r] = valid ? dr : 0.f;
      const float sk2 = sink[h] * kLog2e;
      share = valid ? __builtin_amdgcn_exp2f(sk2 - l2) * dr : 0.f;
    }
#pragma unroll
    for (int off = 8; off < 64; off <<= 1) share += __shfl_xor(share, off);
    if (lane == 0) red[tid >> 6][hl] = share;
  }
  __syncthreads();
  if (tid < kHpg)
    ws.sinkpart[(size_t)(g * kHpg + tid) * ws.nqmax + qg] = (red[0][tid] + red[1][tid]) + (red[2][tid] + red[3][tid]);
}

// ----------------------------------------------------------------- dQ

constexpr int kDqAhead = 4;  // operand fragments read ahead of their product

constexpr int kDqThreads = 64 * kHpg;   // one wave per query head of a kv head
constexpr int kDqVecPerWave = kKvbBytes / (16 * kDqThreads);  // 6

// One 64-key tile of the query-major kernel for the wave's head, as one
// straight block, a 32-key block b at a time: S^T = K'Q'^T and dP^T = V dO^T
// (A operands from LDS, read kDqAhead products ahead; lane (col, half) gets
// query col and keys k0 + 32b + 8(i>>2) + 4half + (i&3)), then
// dS^T = P^T (dP^T - Dr) with P^T = exp2(S^T - lse), then the block's share
// of dQ'^T += K'^T dS^T (key steps 2b, 2b + 1). The lane's query sees keys
// klo .. klo + krange (causal, window and length limits), applied on every
// tile. One block at a time keeps the wave within 256 registers, so two waves
// share each SIMD.
__device__ __forceinline__ void dq_tile(const uint4* st, int lane, int half, const bf16x8* qf,
                                       const bf16x8* df, float l2, float dr, int klo,
                                       unsigned krange, int k0, f32x16* acc) {
  const int d0 = k0 + 4 * half - klo;
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    f32x16 sc = {}, dp = {};
    {
      // fragment i: channel step i >> 1, K' (even) or V (odd)
      auto frag = [&](int i) {
        return ld_frag(st + (i & 1) * (kKvbPart / 16) + frag_index(b, 8, i >> 1, 0, 0) + lane);
      };
      bf16x8 f[16];
#pragma unroll
      for (int i = 0; i < kDqAhead; ++i) f[i] = frag(i);
      __builtin_amdgcn_sched_group_barrier(0x100, kDqAhead, 0);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if (i + kDqAhead < 16) f[i + kDqAhead] = frag(i + kDqAhead);
        if (i & 1) dp = mfma(f[i], df[i >> 1], dp);
        else sc = mfma(f[i], qf[i >> 1], sc);
        if (i + kDqAhead < 16) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      }
    }
    bf16x8 ds[2];
    {
      float g[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float pv = __builtin_amdgcn_exp2f(sc[i] - l2);
        pv = (unsigned)(d0 + 32 * b + 8 * (i >> 2) + (i & 3)) <= krange ? pv : 0.f;
        g[i] = pv * (dp[i] - dr);
      }
      ds[0] = pack_frag(g);
      ds[1] = pack_frag(g + 8);
    }
    {
      // fragment i: K'^T channel block i >> 1, key step 2b + (i & 1)
      auto frag = [&](int i) {
        return ld_frag(st + 2 * (kKvbPart / 16) + frag_index(i >> 1, 4, 2 * b + (i & 1), 0, 0) + lane);
      };
      bf16x8 f[8];
#pragma unroll
      for (int i = 0; i < kDqAhead; ++i) f[i] = frag(i);
      __builtin_amdgcn_sched_group_barrier(0x100, kDqAhead, 0);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if (i + kDqAhead < 8) f[i + kDqAhead] = frag(i + kDqAhead);
        acc[i >> 1] = mfma(f[i], ds[i & 1], acc[i >> 1]);
        if (i + kDqAhead < 8) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      }
    }
  }
}

// Reduce-scatter over the 32 lanes of each half-wave: v[0..N) of every lane
// in, and out in v[0..N/2) of the lane the sums of the values its partner
// kept. The partner is lane ^ 16 (kLevel 0), or the mirror image within 16
// lanes, within 8 lanes, lane ^ 2 and lane ^ 1 (kLevel 1 to 4); a lane whose
// level bit is set keeps the upper half of v. After the five levels lane L of a
// half holds in v[0], v[1] the sums of entries 2 (L & 31) and 2 (L & 31) + 1.
template <int kLevel, int N>
__device__ __forceinline__ void reduce_scatter_step(float* v, int lane) {
  constexpr int kBit = 4 - kLevel;
  const bool up = (lane >> kBit) & 1;
#pragma unroll
  for (int k = 0; k < N / 2; ++k) {
    const float keep = up ? v[k + N / 2] : v[k];
    const float send = up ? v[k] : v[k + N / 2];
    float recv;
    if constexpr (kLevel == 0) {
      // rows 0/1 and 2/3 trade places: even rows find the odd row's value in
      // the second result, odd rows the even row's in the first
      const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(send), __float_as_uint(send), false, false);
      recv = __uint_as_float(up ? r[0] : r[1]);
    } else {
      constexpr int kCtrl = kLevel == 1 ? 0x140 : kLevel == 2 ? 0x141 : kLevel == 3 ? 0x4E : 0xB1;
      recv = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(send), kCtrl, 0xF, 0xF, false));
    }
    v[k] = keep + recv;
  }
}

__device__ __forceinline__ void reduce_scatter32(float* v, int lane) {
  reduce_scatter_step<0, 64>(v, lane);
  reduce_scatter_step<1, 32>(v, lane);
  reduce_scatter_step<2, 16>(v, lane);
  reduce_scatter_step<3, 8>(v, lane);
  reduce_scatter_step<4, 4>(v, lane);
}

// Adjoint of the RoPE rotation on the dQ'^T accumulators of the lane's query:
// channels c = 32db + 8(i>>2) + 4half + (i&3) (db < 2) pair with c + 64.
template <bool kMixed>
__device__ __forceinline__ void rope_adjoint_dq(int pos, const RopeFreq* rope, int half, f32x16* acc) {
  const float pf = (float)pos;
#pragma unroll
  for (int db = 0; db < 2; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float cs, sn;
      rope_cos_sin<kMixed>(pos, pf, rope[32 * db + 8 * (i >> 2) + 4 * half + (i & 3)], &cs, &sn);
      const float a = acc[db][i], b = acc[db + 2][i];
      acc[db][i] = a * cs + b * sn;
      acc[db + 2][i] = b * cs - a * sn;
    }
}

__global__ __launch_bounds__(kDqThreads) void bwd_dq_kernel(const uint16_t* __restrict__ q,
                                                            const uint16_t* __restrict__ dout,
                                                            const float* __restrict__ q_norm_w,
                                                            const int* __restrict__ positions,
                                                            int window, int use_rope, float eps,
                                                            BwdWs ws, uint16_t* __restrict__ dq) {
  __shared__ uint4 smem[kBwdStages][kKvbBytes / 16];
  const int bid = blockIdx.x;
  const int i_item = bid >> 2, g = bid & (kG - 1);
  if (i_item >= ws.f.hdr[2]) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, half = lane >> 5;
  const int h = g * kHpg + wave;
  const int2 itm = ws.f.items[i_item];
  const int4 meta = ws.f.seq[itm.x];
  const int start = __builtin_amdgcn_readfirstlane(meta.x);
  const int u = __builtin_amdgcn_readfirstlane(meta.z);
  const int t0 = itm.y * kBM;
  int klo, khi;
  block_keys(u, itm.y, window, &klo, &khi);
  const int tile_lo = klo / kBN;
  const int ntiles = (khi + kBN - 1) / kBN - tile_lo;
  const int qg = ws.f.qbase[itm.x] + itm.y;
  const int voff = lane * 16 + wave * 1024;

  // Q' and dO of this head as B operands (query col, channels 16kk + 8half..),
  // Q' from its prepared tile, dO straight from the caller's tensor (rows past
  // the valid length read as zeros), and the row terms of query col.
  const char* qtile = ws.qt + ((size_t)qg * kH + h) * kQtBytes;
  const uint4* qfp = reinterpret_cast<const uint4*>(qtile);
  const int rows = min(u - t0, kBM);
  const __amdgpu_buffer_rsrc_t dor = rsrc_of(dout + ((size_t)(start + t0) * kH + h) * kD, rows * (kH * kD * 2));
  bf16x8 qf[8], df[8];
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) {
    qf[kk] = ld_frag(qfp + kk * 64 + swz(lane));
    df[kk] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(
                                            dor, col * (kH * kD * 2) + (16 * kk + 8 * half) * 2, 0, 0));
  }
  const float* stats = reinterpret_cast<const float*>(qtile + kQtPart);
  const float l2 = stats[col];
  const float dr = stats[kBM + col];

  const char* tiles = ws.kvb + ((size_t)g * ws.f.ntmax + meta.w + tile_lo) * kKvbBytes;
  const __amdgpu_buffer_rsrc_t trs = rsrc_of(tiles, ntiles * kKvbBytes);
  auto load_tile = [&](int k, int stage) {
#pragma unroll
    for (int i = 0; i < kDqVecPerWave; ++i)
      dma16(trs, voff, k * kKvbBytes + i * 8192,
            reinterpret_cast<char*>(smem[stage]) + i * 8192 + wave * 1024);
  };
  load_tile(0, 0);
  if (ntiles > 1) load_tile(1, 1);

  f32x16 acc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[db][i] = 0.f;
  // keys this lane's query sees: max(0, q - window + 1) .. min(q, u - 1);
  // none for a padded row (an empty range: krange wraps past 2^31)
  const int qrow = t0 + col;
  const int kfirst = window > 0 ? max(0, qrow - (window - 1)) : 0;
  const unsigned krange = qrow < u ? (unsigned)(qrow - kfirst) : 0xffffffffu;

  for (int kt = 0; kt < ntiles; ++kt) {
    if (kt + 1 < ntiles) ring_barrier_n<kDqVecPerWave>();
    else ring_barrier_n<0>();
    if (kt + 2 < ntiles) load_tile(kt + 2, (kt + 2) % kBwdStages);
    dq_tile(smem[kt % kBwdStages], lane, half, qf, df, l2, dr, kfirst, krange,
            (tile_lo + kt) * kBN, acc);
  }

  // Epilogue. Lane (col, half) holds dQ'^T for query t0 + col, channels
  // c = 32db + 8rg + 4half + j at acc[db][4rg + j]; c and c + 64 are db and
  // db + 2 at the same index.
  const bool valid = col < rows;
  float xq[4][16];
  const __amdgpu_buffer_rsrc_t qr = rsrc_of(q + ((size_t)(start + t0) * kH + h) * kD, rows * (kH * kD * 2));
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      const uint2 w = __builtin_bit_cast(
          uint2, __builtin_amdgcn_raw_buffer_load_b64(qr, col * (kH * kD * 2) + (32 * db + 8 * rg + 4 * half) * 2, 0, 0));
      xq[db][4 * rg + 0] = bf16_lo(w.x);
      xq[db][4 * rg + 1] = bf16_hi(w.x);
      xq[db][4 * rg + 2] = bf16_lo(w.y);
      xq[db][4 * rg + 3] = bf16_hi(w.y);
    }
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[db][i] *= kInvSqrtD;
  if (use_rope) {  // adjoint of the rotation: the opposite turn
    const int pos = positions ? (valid ? positions[(size_t)start + t0 + col] : 0) : t0 + col;
    if (!rope_wave_mixed(pos)) rope_adjoint_dq<false>(pos, ws.f.rope, half, acc);
    else rope_adjoint_dq<true>(pos, ws.f.rope, half, acc);
  }
  // RMSNorm adjoint: dq = rstd (dy w - xn mean(xn dy w)), xn = q rstd
  float ss = 0.f;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) ss += xq[db][i] * xq[db][i];
  ss += __shfl_xor(ss, 32);
  const float rstd = 1.0f / sqrtf(ss * (1.0f / kD) + eps);
  float dot = 0.f;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      xq[db][i] *= rstd;
      dot += xq[db][i] * acc[db][i] * q_norm_w[32 * db + 8 * (i >> 2) + 4 * half + (i & 3)];
    }
  dot += __shfl_xor(dot, 32);
  dot *= 1.0f / kD;
  const __amdgpu_buffer_rsrc_t dqr = rsrc_of(dq + ((size_t)(start + t0) * kH + h) * kD, rows * (kH * kD * 2));
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      float y[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int i = 4 * rg + j;
        const float w = q_norm_w[32 * db + 8 * rg + 4 * half + j];
        y[j] = rstd * (acc[db][i] * w - xq[db][i] * dot);
      }
      const uint2 pk = make_uint2(pack2(y[0], y[1]), pack2(y[2], y[3]));
      __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(__attribute__((ext_vector_type(2))) unsigned, pk),
                                            dqr, col * (kH * kD * 2) + (32 * db + 8 * rg + 4 * half) * 2, 0, 0);
    }
  // q-norm-weight terms dy * xn: each wave sums its 32 rows per channel across
  // its lanes (a reduce-scatter on the VALU), then the 8 waves' sums are added
  // in wave order through a ring stage that no wave reads any more (the last
  // tile uses stage (ntiles - 1) % 3, and no loads are pending).
  {
    float v[64];
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) v[16 * db + i] = acc[db][i] * xq[db][i];
    reduce_scatter32(v, lane);
    float* wsum = reinterpret_cast<float*>(smem[ntiles % kBwdStages]);  // [8 waves][128]
#pragma unroll
    for (int e2 = 0; e2 < 2; ++e2) {
      const int vi = 2 * col + e2;  // entry 16db + 4rg + j: channel 32db + 8rg + 4half + j
      wsum[wave * kD + 32 * (vi >> 4) + 8 * ((vi >> 2) & 3) + 4 * half + (vi & 3)] = v[e2];
    }
    __syncthreads();
    if (tid < kD) {
      float sum = 0.f;
#pragma unroll
      for (int w = 0; w < kHpg; ++w) sum += wsum[w * kD + tid];
      // indexed by the query block's place in the sequences, not by the
      // workgroup: the schedule's order of equal-cost items varies from call
      // to call, and the finalize sums these terms in index order
      ws.wq[(size_t)tid * (ws.nqmax * kG) + qg * kG + g] = sum;
    }
  }
}

// ----------------------------------------------------------------- dK, dV

constexpr int kDkdvThreads = 512;  // eight waves, one per 32 keys
constexpr int kDkdvStages = 2;     // the step in use and the next one loading
constexpr int kDkdvAhead = 3;      // operand fragments read ahead of their product
constexpr int kStepBytes = 2 * kQtPart + kQtStats;  // a step in LDS: Q' | dO | stats

// A operand of the 32x32x16 MFMA holding X^T, from X (32 rows x 128
// channels, bf16, swizzled operand order) in LDS: A[c][j] = X[row(j)][c] for
// channel c = 32db + (lane & 31), rows 16kk + 8s + 4(lane >> 5) + m for k
// index 8(lane >> 5) + 4s + m. Two transposing LDS reads (ds_read_b64_tr_b16)
// give the two halves: within each group of 16 lanes, lane i's m-th value is
// value i & 3 of the 8 bytes that lane 4m + (i >> 2) addresses, so lane
// 16G + 4m + q addresses row 16kk + 8s + 4(G >> 1) + m, channels
// 32db + 16(G & 1) + 4q .. + 4. tr_lane_offset(lane, s) is that byte address
// for db = kk = 0; the swizzle makes the 16 units of each read fall on
// distinct banks.
__device__ __forceinline__ unsigned tr_lane_offset(int lane, int s) {
  const int G = lane >> 4, m = (lane >> 2) & 3, q = lane & 3, hf = q >> 1;
  const int row = 8 * s + 4 * (G >> 1) + m;
  return (unsigned)(((G & 1) * 64 + hf * 32 + (row ^ (8 * hf))) * 16 + (q & 1) * 8);
}

__device__ __forceinline__ bf16x8 ld_frag_tr(const uint4* x, unsigned off0, unsigned off1, int db, int kk) {
  typedef short v4i16 __attribute__((ext_vector_type(4)));
  typedef short v8i16 __attribute__((ext_vector_type(8)));
  __attribute__((address_space(3))) char* b = (__attribute__((address_space(3))) char*)x + db * 2048 + kk * 256;
  const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)(b + off0));
  const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)(b + off1));
  const v8i16 r = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, r);
}

// Row terms lse (log2 units) and Dr of queries 8rg + 4half + [0, 4) for the
// lanes of `half` (the step's terms, which arrive in LDS with its operands).
__device__ __forceinline__ void read_stats4(const float* stats, int half, int rg, float* lv, float* rv) {
  const float4 a = *reinterpret_cast<const float4*>(stats + 4 * half + 8 * rg);
  const float4 b = *reinterpret_cast<const float4*>(stats + kBM + 4 * half + 8 * rg);
  lv[0] = a.x; lv[1] = a.y; lv[2] = a.z; lv[3] = a.w;
  rv[0] = b.x; rv[1] = b.y; rv[2] = b.z; rv[3] = b.w;
}

// One step of the key-major kernel for the wave's 32 keys, as one straight
// block: S = Q'K'^T and dP = dO V^T (A operands from the step's stage, V's B
// operand from the item's V tiles in LDS, K' in registers; fragments read
// kDkdvAhead products ahead), P = exp2(S - lse) and dS = P (dP - Dr), then
// dV^T += dO^T P and dK'^T += Q'^T dS with dO^T and Q'^T read transposed from
// the same stage. P and dS sit in the B operand with their query rows in the
// order the transposed reads deliver (k index 8half + 4s + m is query
// 16kk + 8s + 4half + m, the S accumulator's own row order). The lane's key is seen by queries
// qlo .. qlo + qrange (causal, window and length limits); the mask is applied
// on every step, so the loop body has no branch.
__device__ __forceinline__ void dkdv_step(const uint4* st, const uint4* vt, int lane, int half,
                                          unsigned tr0, unsigned tr1, const bf16x8* kf,
                                          f32x16* dk, f32x16* dv, int qlo, unsigned qrange, int t0) {
  f32x16 s = {}, dp = {};
  {
    // fragment i: Q' (i even, A of S at channel step i >> 1) or, for odd i,
    // dO (A of dP) and V (its B), at channel step i >> 1
    bf16x8 f[16], fv[8];
    const int sl = swz(lane);
    auto frag = [&](int i) { return ld_frag(st + (i & 1) * (kQtPart / 16) + (i >> 1) * 64 + sl); };
#pragma unroll
    for (int i = 0; i < kDkdvAhead; ++i) {
      f[i] = frag(i);
      if (i & 1) fv[i >> 1] = ld_frag(vt + (i >> 1) * 64 + lane);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (i + kDkdvAhead < 16) {
        const int n = i + kDkdvAhead;
        f[n] = frag(n);
        if (n & 1) fv[n >> 1] = ld_frag(vt + (n >> 1) * 64 + lane);
      }
      if (i & 1) dp = mfma(f[i], fv[i >> 1], dp);
      else s = mfma(f[i], kf[i >> 1], s);
    }
  }
  bf16x8 pb[2], gb[2];
  {
    const float* stats = reinterpret_cast<const float*>(st + 2 * kQtPart / 16);
    // S rows are queries t0 + 8rg + 4half + j; this lane's key allows rows
    // qlo .. qlo + qrange
    const int d0 = t0 + 4 * half - qlo;
    float pr[16], gr[16];
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      float lv[4], rv[4];
      read_stats4(stats, half, rg, lv, rv);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int e = 4 * rg + j;
        float pv = __builtin_amdgcn_exp2f(s[e] - lv[j]);
        pv = (unsigned)(d0 + 8 * rg + j) <= qrange ? pv : 0.f;
        pr[e] = pv;
        gr[e] = pv * (dp[e] - rv[j]);
      }
    }
    pb[0] = pack_frag(pr);
    pb[1] = pack_frag(pr + 8);
    gb[0] = pack_frag(gr);
    gb[1] = pack_frag(gr + 8);
  }
  {
    // fragment i: dO^T (even) or Q'^T (odd) of channel block i >> 2, query step (i >> 1) & 1
    auto frag = [&](int i) {
      return ld_frag_tr(st + ((i & 1) ? 0 : kQtPart / 16), tr0, tr1, i >> 2, (i >> 1) & 1);
    };
    bf16x8 f[16];
#pragma unroll
    for (int i = 0; i < kDkdvAhead; ++i) f[i] = frag(i);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (i + kDkdvAhead < 16) f[i + kDkdvAhead] = frag(i + kDkdvAhead);
      const int db = i >> 2, kk = (i >> 1) & 1;
      if (i & 1) dk[db] = mfma(f[i], gb[kk], dk[db]);
      else dv[db] = mfma(f[i], pb[kk], dv[db]);
    }
  }
}

__global__ __launch_bounds__(kDkdvThreads) void bwd_dkdv_kernel(const uint16_t* __restrict__ dout,
                                                                int window, BwdWs ws) {
  __shared__ uint4 smem[kDkdvStages][kStepBytes / 16];
  __shared__ uint4 vlds[kKBTiles][kKvbPart / 16];  // the item's V operand tiles
  // Workgroup b runs on L2 domain b % kXcds; domain x takes ranks
  // [x per, (x + 1) per) of the kv-head-major item list.
  const int NC = ws.f.hdr[kHdrNC];
  const int per = (NC * kG + kXcds - 1) / kXcds;
  const int rank = (int)(blockIdx.x % kXcds) * per + (int)(blockIdx.x / kXcds);
  if ((int)(blockIdx.x / kXcds) >= per || rank >= NC * kG) return;
  const int g = rank / NC, ii = rank - g * NC;
  const int CH = ws.f.hdr[kHdrCH];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, half = lane >> 5;
  const int2 kit = ws.kitems[ii];
  const int e = kit.x, chunk = kit.y;
  const int2 te = ws.f.tiles[e];
  const int4 meta = ws.f.seq[te.x];
  const int u = __builtin_amdgcn_readfirstlane(meta.z);
  const int start = __builtin_amdgcn_readfirstlane(meta.x);
  const int len = meta.y;
  const int k0 = te.y * kBN;
  int qlo, qhi;
  kb_queries(k0, u, window, &qlo, &qhi);
  const int qb0 = max(qlo, chunk * CH);
  const int qb1 = min(qhi, (chunk + 1) * CH);
  const int nsteps = (qb1 - qb0) * kHpg;
  const int qgbase = ws.f.qbase[te.x];
  const int voff = lane * 16 + wave * 1024;

  // The item's key tiles e .. e + 3 (those inside the sequence; reads past
  // them return zeros and their keys are masked). Wave w owns keys
  // 32 (w & 1) .. + 32 of tile w >> 1: K' as B operands in registers, V's
  // operand tiles in LDS.
  const int kt = wave >> 1, bb = wave & 1;
  const int kbase = k0 + kt * kBN + bb * 32;
  const int ntiles = min(kKBTiles, (len + kBN - 1) / kBN - te.y);
  const char* tiles = ws.kvb + ((size_t)g * ws.f.ntmax + e) * kKvbBytes;
  const __amdgpu_buffer_rsrc_t krs = rsrc_of(tiles, ntiles * kKvbBytes);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int ci = i * 8 + wave;  // 1 KiB chunk ci of the 64 KiB of V tiles
    dma16(krs, lane * 16, (ci >> 4) * kKvbBytes + kKvbPart + (ci & 15) * 1024,
          reinterpret_cast<char*>(vlds[ci >> 4]) + (ci & 15) * 1024);
  }
  bf16x8 kf[8];
#pragma unroll
  for (int kk = 0; kk < 8; ++kk)
    kf[kk] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(
                                            krs, kt * kKvbBytes + frag_index(bb, 8, kk, half, col) * 16, 0, 0));

  // step j: query block qb0 + j / 8, head 8g + j % 8. Each wave moves one
  // 1 KiB operand unit of Q' (from its prepared tile) and one of dO, gathered
  // from the caller's tensor (rows past the valid length read as zeros), and
  // the step's row terms (every wave loads the same 256 bytes).
  auto load_step = [&](int j, int stage) {
    const int qb = qb0 + j / kHpg, hh = g * kHpg + j % kHpg;
    const char* src = ws.qt + ((size_t)(qgbase + qb) * kH + hh) * kQtBytes;
    const __amdgpu_buffer_rsrc_t r = rsrc_of(src, kQtBytes);
    const __amdgpu_buffer_rsrc_t dr = rsrc_of(dout + ((size_t)(start + qb * kBM) * kH + hh) * kD,
                                              min(u - qb * kBM, kBM) * (kH * kD * 2));
    char* dst = reinterpret_cast<char*>(smem[stage]);
    dma16(r, voff, 0, dst + wave * 1024);
    // the lane at unit position `lane` carries row (col ^ 8half): the swizzle
    dma16(dr, (col ^ (8 * half)) * (kH * kD * 2) + (16 * wave + 8 * half) * 2, 0, dst + kQtPart + wave * 1024);
    dma4(r, lane * 4, kQtPart, dst + 2 * kQtPart);
  };
  load_step(0, 0);
  // Everything loaded so far (V tiles, K' operands, step 0) is waited for here,
  // where the compiler sees it: the first ring barrier would wait for it anyway,
  // and loads still pending at the loop's entry would make the compiler wait for
  // every load in flight (the next step's) before the LDS reads of every step.
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);

  f32x16 dk[4], dv[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      dk[db][i] = 0.f;
      dv[db][i] = 0.f;
    }
  // queries that see this lane's key: key .. min(key + window - 1, u - 1);
  // none for a padding key (an empty range: qrange wraps past 2^31)
  const int key = kbase + col;
  const int qlast = window > 0 ? min(key + window - 1, u - 1) : u - 1;
  const unsigned qrange = key < u ? (unsigned)(qlast - key) : 0xffffffffu;
  const int qfirst = key < u ? key : 0x40000000;
  const uint4* vt = vlds[kt] + frag_index(bb, 8, 0, 0, 0);
  const unsigned tr0 = tr_lane_offset(lane, 0), tr1 = tr_lane_offset(lane, 1);
  // Queries that see some key of the wave: kbase .. min(kbase + 31 + window
  // - 1, u - 1). A step whose 32 queries miss that range is skipped (its P is
  // zero); with two waves per SIMD the other wave takes the matrix cores.
  const int wq_lo = kbase, wq_hi = window > 0 ? min(kbase + 31 + window - 1, u - 1) : u - 1;
  for (int j = 0; j < nsteps; ++j) {
    // step j's operands (and, at j = 0, the V tiles) are in LDS once this
    // wave's loads are done; after the barrier every wave has finished step
    // j - 1, so its stage takes step j + 1
    ring_barrier_n<0>();
    if (j + 1 < nsteps) load_step(j + 1, (j + 1) % kDkdvStages);
    const int t0 = (qb0 + j / kHpg) * kBM;
    if (t0 + kBM - 1 < wq_lo || t0 > wq_hi) continue;
    dkdv_step(smem[j % kDkdvStages], vt, lane, half, tr0, tr1, kf, dk, dv, qfirst, qrange, t0);
  }

  // FP32 partial sums of this chunk: [dK' | dV][256 keys][128 channels];
  // lane (col, half) holds key col of the wave's block, channels
  // 32db + 8rg + 4half + [0, 4) at index 4rg + [0, 4). Q' carries the
  // softmax scale log2(e)/sqrt(d), so dK' = dS^T Q' ln 2.
  float* part = ws.part + ((size_t)(ws.cb[e] + chunk - qlo / CH) * kG + g) * kPartFloats;
  const int krow = kt * kBN + bb * 32 + col;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      const int c = 32 * db + 8 * rg + 4 * half;
      *reinterpret_cast<float4*>(part + krow * kD + c) =
          make_float4(dk[db][4 * rg] * kLn2, dk[db][4 * rg + 1] * kLn2,
                      dk[db][4 * rg + 2] * kLn2, dk[db][4 * rg + 3] * kLn2);
      *reinterpret_cast<float4*>(part + kKB * kD + krow * kD + c) =
          make_float4(dv[db][4 * rg], dv[db][4 * rg + 1], dv[db][4 * rg + 2], dv[db][4 * rg + 3]);
    }
}

// ----------------------------------------------------------------- K/V reduce

// Adjoint of the RoPE rotation on a thread's 16 channel pairs (g[i] with
// g[16 + i]) at position pos.
template <bool kMixed>
__device__ __forceinline__ void rope_adjoint16(int pos, const RopeFreq* fr, float* g) {
  const float pf = (float)pos;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    float cs, sn;
    rope_cos_sin<kMixed>(pos, pf, fr[i], &cs, &sn);
    const float a = g[i], b = g[16 + i];
    g[i] = a * cs + b * sn;
    g[16 + i] = b * cs - a * sn;
  }
}

__global__ __launch_bounds__(256) void bwd_kv_reduce_kernel(const uint16_t* __restrict__ k,
                                                            const float* __restrict__ k_norm_w,
                                                            const int* __restrict__ positions,
                                                            float eps, int use_rope, BwdWs ws,
                                                            uint16_t* __restrict__ dk,
                                                            uint16_t* __restrict__ dv) {
  __shared__ float red[kBN * kD + 2 * kD];
  const int e = blockIdx.x, g = blockIdx.y;
  if (e >= ws.f.hdr[1]) return;
  const int2 te = ws.f.tiles[e];
  const int4 meta = ws.f.seq[te.x];
  const int start = meta.x, len = meta.y, u = meta.z;
  const int tid = threadIdx.x, r = tid >> 2, p = tid & 3;
  const int ell = te.y * kBN + r;
  const bool valid = ell < u;
  const size_t t = (size_t)start + ell;
  const int eb = e - te.y % kKBTiles;
  const int row = te.y % kKBTiles * kBN + r;
  // channels [16p, 16p+16) and [64+16p, 64+16p+16)
  float gk[32], gv[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) gk[i] = gv[i] = 0.f;
  const int nch = valid ? ws.nc[eb] : 0;
  const float* part = ws.part + ((size_t)ws.cb[eb] * kG + g) * kPartFloats;
  for (int ch = 0; ch < nch; ++ch) {
    const float* pk = part + (size_t)ch * kG * kPartFloats + row * kD;
    const float* pv = pk + kKB * kD;
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float4 a = *reinterpret_cast<const float4*>(pk + 64 * h2 + 16 * p + 4 * i);
        const float4 b = *reinterpret_cast<const float4*>(pv + 64 * h2 + 16 * p + 4 * i);
        float* x = gk + 16 * h2 + 4 * i;
        float* y = gv + 16 * h2 + 4 * i;
        x[0] += a.x; x[1] += a.y; x[2] += a.z; x[3] += a.w;
        y[0] += b.x; y[1] += b.y; y[2] += b.z; y[3] += b.w;
      }
  }
  float xk[32];
  if (valid) {
    const uint4* src = reinterpret_cast<const uint4*>(k + (t * kG + g) * kD);
    unpack8(src[2 * p], xk);
    unpack8(src[2 * p + 1], xk + 8);
    unpack8(src[8 + 2 * p], xk + 16);
    unpack8(src[9 + 2 * p], xk + 24);
  } else {
#pragma unroll
    for (int i = 0; i < 32; ++i) xk[i] = 0.f;
  }
  if (use_rope && valid) {  // adjoint of the rotation
    const int pos = positions ? positions[t] : ell;
    if (!rope_wave_mixed(pos)) rope_adjoint16<false>(pos, ws.f.rope + 16 * p, gk);
    else rope_adjoint16<true>(pos, ws.f.rope + 16 * p, gk);
  }
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) ss += xk[i] * xk[i];
  ss += __shfl_xor(ss, 1);
  ss += __shfl_xor(ss, 2);
  const float rstd = 1.0f / sqrtf(ss * (1.0f / kD) + eps);
  float dot = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    xk[i] *= rstd;
    dot += xk[i] * gk[i] * k_norm_w[(i < 16 ? 16 * p : 64 + 16 * p) + (i & 15)];
  }
  dot += __shfl_xor(dot, 1);
  dot += __shfl_xor(dot, 2);
  dot *= 1.0f / kD;
  if (ell < len) {
    float y[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const float w = k_norm_w[(i < 16 ? 16 * p : 64 + 16 * p) + (i & 15)];
      y[i] = rstd * (gk[i] * w - xk[i] * dot);
    }
    uint4* dkr = reinterpret_cast<uint4*>(dk + (t * kG + g) * kD);
    uint4* dvr = reinterpret_cast<uint4*>(dv + (t * kG + g) * kD);
    dkr[2 * p] = pack8(y);
    dkr[2 * p + 1] = pack8(y + 8);
    dkr[8 + 2 * p] = pack8(y + 16);
    dkr[9 + 2 * p] = pack8(y + 24);
    dvr[2 * p] = pack8(gv);
    dvr[2 * p + 1] = pack8(gv + 8);
    dvr[8 + 2 * p] = pack8(gv + 16);
    dvr[9 + 2 * p] = pack8(gv + 24);
  }
  // k-norm-weight terms dy * xn of the tile's 64 keys, summed in key order
#pragma unroll
  for (int i = 0; i < 32; ++i) red[r * kD + (i < 16 ? 16 * p : 64 + 16 * p) + (i & 15)] = gk[i] * xk[i];
  __syncthreads();
  {
    const int c = tid & (kD - 1), half2 = tid >> 7;
    float sum = 0.f;
    for (int rr = 32 * half2; rr < 32 * half2 + 32; ++rr) sum += red[rr * kD + c];
    red[kBN * kD + half2 * kD + c] = sum;
    __syncthreads();
    if (half2 == 0)
      ws.wk[(size_t)c * (ws.f.ntmax * kG) + (size_t)e * kG + g] = red[kBN * kD + c] + red[kBN * kD + kD + c];
  }
}

// ----------------------------------------------------------------- finalize

// Block sum of 256 values in a fixed order.
__device__ float block_sum256(float v, float* sh) {
  const int tid = threadIdx.x;
  sh[tid] = v;
  __syncthreads();
  for (int off = 128; off > 0; off >>= 1) {
    if (tid < off) sh[tid] += sh[tid + off];
    __syncthreads();
  }
  return sh[0];
}

// With `empty` (no tokens) nothing was scheduled and the sums are zero.
__global__ __launch_bounds__(256) void bwd_finalize_kernel(BwdWs ws, int empty,
                                                           float* __restrict__ dq_norm_w,
                                                           float* __restrict__ dk_norm_w,
                                                           float* __restrict__ dsink) {
  __shared__ float sh[256];
  const int b = blockIdx.x, tid = threadIdx.x;
  const int NQ = empty ? 0 : ws.f.hdr[2], NT = empty ? 0 : ws.f.hdr[1];
  float v = 0.f;
  if (b < kD) {
    const float* src = ws.wq + (size_t)b * (ws.nqmax * kG);
    for (int j = tid; j < NQ * kG; j += 256) v += src[j];
    v = block_sum256(v, sh);
    if (tid == 0) dq_norm_w[b] = v;
  } else if (b < 2 * kD) {
    const float* src = ws.wk + (size_t)(b - kD) * (ws.f.ntmax * kG);
    for (int j = tid; j < NT * kG; j += 256) v += src[j];
    v = block_sum256(v, sh);
    if (tid == 0) dk_norm_w[b - kD] = v;
  } else {
    const int h = b - 2 * kD;
    const float* src = ws.sinkpart + (size_t)h * ws.nqmax;
    for (int j = tid; j < NQ; j += 256) v += src[j];
    v = block_sum256(v, sh);
    if (tid == 0) dsink[h] = -v;
  }
}

}  // namespace flint

// ===================================================================== C ABI

using namespace flint;

extern "C" size_t flint_attn_bwd_workspace_bytes(int32_t total_tokens, int32_t n_seqs,
                                                 int32_t max_seqlen, int32_t num_kv_heads,
                                                 int32_t head_dim) {
  if (total_tokens < 0 || n_seqs < 0 || max_seqlen < 0 || max_seqlen > kMaxSeqLen) return 0;
  if (num_kv_heads != kG || head_dim != kD) return 0;
  return make_bwd_layout(total_tokens, n_seqs).total;
}

extern "C" int flint_attn_bwd(const void* q, const void* k, const void* v, const float* q_norm_w,
                              const float* k_norm_w, const float* sink, const int32_t* positions,
                              const int32_t* cu_seqlens, const int32_t* seqused, int32_t n_seqs,
                              int32_t max_seqlen, int32_t total_tokens, int32_t num_q_heads,
                              int32_t num_kv_heads, int32_t head_dim, int32_t window,
                              int32_t use_rope, float rope_theta, float eps, const void* out,
                              const float* lse, const void* dout, void* workspace,
                              size_t workspace_bytes, void* dq, void* dk, void* dv,
                              float* dq_norm_w, float* dk_norm_w, float* dsink, void* stream) {
  if (total_tokens < 0 || n_seqs < 0 || max_seqlen < 0) return FLINT_ERR_SHAPE;
  if (num_q_heads != kH || num_kv_heads != kG || head_dim != kD || max_seqlen > kMaxSeqLen)
    return FLINT_ERR_UNSUPPORTED;
  if (window < 0 || !(eps > 0.f) || !isfinite(eps)) return FLINT_ERR_VALUE;
  if (use_rope && (!(rope_theta > 0.f) || !isfinite(rope_theta))) return FLINT_ERR_VALUE;
  if (!dq_norm_w || !dk_norm_w || !dsink) return FLINT_ERR_NULL;
  if (total_tokens > 0 && n_seqs < 1) return FLINT_ERR_SHAPE;
  if (total_tokens > 0 && (!q || !k || !v || !q_norm_w || !k_norm_w || !sink || !cu_seqlens ||
                           !out || !lse || !dout || !dq || !dk || !dv))
    return FLINT_ERR_NULL;
  if (!workspace) return FLINT_ERR_WORKSPACE;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) ||
      !aligned(dout, 16) || !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16) ||
      !aligned(lse, 16) || !aligned(workspace, 256) || !aligned(q_norm_w, 4) ||
      !aligned(k_norm_w, 4) || !aligned(sink, 4) || !aligned(cu_seqlens, 4) ||
      !aligned(dq_norm_w, 4) || !aligned(dk_norm_w, 4) || !aligned(dsink, 4) ||
      (positions && !aligned(positions, 4)) || (seqused && !aligned(seqused, 4)))
    return FLINT_ERR_ALIGN;
  const BwdLayout L = make_bwd_layout(total_tokens, n_seqs);
  if (workspace_bytes < L.total) return FLINT_ERR_WORKSPACE;

  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  BwdWs ws;
  ws.f = ws_at(workspace, L.f);
  char* base = static_cast<char*>(workspace);
  ws.kvb = base + L.kvb;
  ws.qt = base + L.qt;
  ws.sinkpart = reinterpret_cast<float*>(base + L.sinkpart);
  ws.wq = reinterpret_cast<float*>(base + L.wq);
  ws.wk = reinterpret_cast<float*>(base + L.wk);
  ws.cb = reinterpret_cast<int*>(base + L.cb);
  ws.nc = reinterpret_cast<int*>(base + L.nc);
  ws.kitems = reinterpret_cast<int2*>(base + L.kitems);
  ws.part = reinterpret_cast<float*>(base + L.part);
  ws.nqmax = (int)L.f.nqmax;
  ws.ncmax = (int)L.ncmax;
  ws.n = n_seqs;

  const uint16_t* qh = static_cast<const uint16_t*>(q);
  const uint16_t* kh = static_cast<const uint16_t*>(k);
  const uint16_t* vh = static_cast<const uint16_t*>(v);
  const int rope = use_rope ? 1 : 0;
  const int* pos = rope ? positions : nullptr;

  (void)hipGetLastError();
  if (total_tokens == 0) {
    // no rows: the parameter gradients are zero
    bwd_finalize_kernel<<<2 * kD + kH, 256, 0, st>>>(ws, 1, dq_norm_w, dk_norm_w, dsink);
  } else {
    launch_schedule(cu_seqlens, seqused, n_seqs, total_tokens, max_seqlen, window,
                    (double)rope_theta, ws.f, st);
    bwd_schedule_kernel<<<1, 1024, 0, st>>>(window, ws);
    bwd_kv_prep_kernel<<<dim3((unsigned)L.f.ntmax, kG), 256, 0, st>>>(
        kh, vh, k_norm_w, pos, eps, rope, ws, static_cast<uint16_t*>(dq));
    bwd_q_prep_kernel<<<dim3((unsigned)L.f.nqmax, kG), 256, 0, st>>>(
        qh, static_cast<const uint16_t*>(out), static_cast<const uint16_t*>(dout), lse, q_norm_w,
        sink, pos, eps, rope, ws);
    bwd_dq_kernel<<<(unsigned)(L.f.nqmax * kG), kDqThreads, 0, st>>>(
        qh, static_cast<const uint16_t*>(dout), q_norm_w, pos, window, rope, eps, ws, static_cast<uint16_t*>(dq));
    bwd_dkdv_kernel<<<(unsigned)((L.ncmax * kG + kXcds - 1) / kXcds * kXcds), kDkdvThreads, 0, st>>>(
        static_cast<const uint16_t*>(dout), window, ws);
    bwd_kv_reduce_kernel<<<dim3((unsigned)L.f.ntmax, kG), 256, 0, st>>>(
        kh, k_norm_w, pos, eps, rope, ws, static_cast<uint16_t*>(dk), static_cast<uint16_t*>(dv));
    bwd_finalize_kernel<<<2 * kD + kH, 256, 0, st>>>(ws, 0, dq_norm_w, dk_norm_w, dsink);
  }
  if (hipGetLastError() != hipSuccess) return FLINT_ERR_HIP;
  if (debug_sync()) {
    int32_t flags = 0;
    return flint_attn_device_status(workspace, stream, &flags);
  }
  return FLINT_OK;
}
