// Flint sink-aware attention forward (prefill) for AMD Instinct MI355X (gfx950).
//
// The layer (NeMo AutoModel "flint" page, section "Model Architecture";
// flint.layers API page, FlintAttention; Hugging Face discussion #26 on
// RecursiveSI/flint, "What was unusually easy" and "Configuration oddities"):
// per-head weight-form RMSNorm of q and k, NeoX RoPE (channel c with c+64) on
// sliding layers only, grouped-query attention of 32 query heads over 4
// key/value heads with head dimension 128, a causal window of 513 keys that
// counts the current token (or full causal attention), and one FP32 sink
// logit per query head that joins the softmax max and denominator with zero
// value and no 1/sqrt(d) scaling.
//
// Two launches run in order on the caller's stream:
//   prep_kernel       block 0 runs the schedule: checks cu_seqlens/seqused,
//                     lays out the 32-token query blocks, orders them by
//                     decreasing work and lists the 64-row units that hold
//                     padded rows; the other blocks, at the same time, one
//                     per (64-key tile, kv head): RMSNorm + RoPE of K in
//                     FP32, one bf16 rounding, stored as an MFMA-ready tile
//                     in operand-fragment order; V transposed and
//                     key-permuted into the PV operand order; zeros for
//                     padded keys. A tile finds its sequence from cu_seqlens
//                     alone (sequence s owns the tiles from cu[s] / 64 + s
//                     on), so it does not wait for the schedule.
//   attn_kernel       persistent: one workgroup per CU, each running a list
//                     of work items (32 query tokens x the 8 query heads of one
//                     kv head). Its 8 waves, one per query head, share each
//                     K/V tile, which arrives in a 4-stage LDS ring by direct
//                     global->LDS loads; the ring runs across item boundaries,
//                     and the next item's query rows are fetched during the
//                     current one. The query prologue (RMSNorm, RoPE, softmax
//                     scale in log2 units, bf16) is fused in. S^T = K Q^T and
//                     O^T += V^T P^T run on v_mfma_f32_32x32x16_bf16 with FP32
//                     accumulation, over the tiles inside the causal window
//                     only. It then writes the padded rows of `out` as
//                     zeros. Problems with fewer work items than CUs run on
//                     attn_half_kernel instead: two 4-wave workgroups per item,
//                     4 query heads each, so twice the CUs take part.
//
// Softmax shift. The QK RMSNorm bounds every logit: by Cauchy-Schwarz
// |s| = |q'.k'| <= |q'| max|k'| = B for the rounded operands the MFMA
// multiplies (s in log2 units). A wave whose rows all have B <= kStaticBound
// (and whose sink stays within it too) needs no shift at all: P = exp2(s)
// stays within [2^-B, 2^B], far from FP32 and bf16 overflow and underflow,
// the sink adds exp2(sink) to the denominator, and O = sum P v / l is the
// same ratio as with any shift. The MFMA accumulators start at zero and
// P = exp2(acc) needs no running max, no per-tile max reduction and no
// rescaling; max |k'| is bounded from the key-norm weights (key_norm_bound),
// so no pass over the keys has to run first. Waves with a larger bound take
// the streaming path: a running max
// that starts at the sink (m = sink, l = 1), subtracted before exp2 and
// raised lazily with rescaling. The start is never below -B, the least logit
// possible: a sink far below every logit (or -INF) then adds ~0 to l without
// moving the shift away from the logits, where s - m would lose their bits.

#include <hip/hip_runtime.h>

#include <mutex>

#include "flint_common.h"

namespace flint {

// ----------------------------------------------------------------- operand type

// The attention products take bf16 operands, or fp16 ones in the FP16
// attention-compute variant ([flint page] Numerical comparison: normalized,
// rotated Q/K/V cast to FP16 at the attention boundary). Operands travel as
// 16-bit containers either way; F16 picks the element type.
typedef _Float16 f16x8 __attribute__((__vector_size__(8 * sizeof(_Float16))));
typedef _Float16 f16x2_t __attribute__((__vector_size__(2 * sizeof(_Float16))));

template <bool F16>
__device__ __forceinline__ f32x16 mma(bf16x8 a, bf16x8 b, f32x16 c) {
  if constexpr (F16)
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c,
                                                  0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

template <bool F16>
__device__ __forceinline__ uint32_t pack2t(float a, float b) {
  if constexpr (F16) {
    f16x2_t h = {(_Float16)a, (_Float16)b};
    return __builtin_bit_cast(uint32_t, h);
  } else {
    return pack2(a, b);
  }
}

template <bool F16>
__device__ __forceinline__ uint4 pack8t(const float* x) {
  return make_uint4(pack2t<F16>(x[0], x[1]), pack2t<F16>(x[2], x[3]), pack2t<F16>(x[4], x[5]),
                    pack2t<F16>(x[6], x[7]));
}

// acc + sum of the eight packed values in c
template <bool F16>
__device__ __forceinline__ float dot2_sumt(const uint4& c, float acc) {
  if constexpr (F16) {
    const f16x2_t ones = {(_Float16)1.0f, (_Float16)1.0f};
    acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, c.x), ones, acc, false);
    acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, c.y), ones, acc, false);
    acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, c.z), ones, acc, false);
    acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, c.w), ones, acc, false);
    return acc;
  } else {
    return dot2_sum(c, __builtin_bit_cast(bf16x2_t, 0x3f803f80u), acc);
  }
}

// Sum of squares of eight packed values.
template <bool F16>
__device__ __forceinline__ float sumsq8t(const uint4& c) {
  if constexpr (F16) {
    const uint32_t w[4] = {c.x, c.y, c.z, c.w};
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f16x2_t h = __builtin_bit_cast(f16x2_t, w[i]);
      const float a = (float)h[0], b = (float)h[1];
      s += a * a + b * b;
    }
    return s;
  } else {
    return sumsq8(c);
  }
}

// ----------------------------------------------------------------- schedule

// Shared memory of schedule_body with NT threads.
template <int NT>
struct SchedLds {
  int tmp[NT / 64];
  int hist[kBuckets];
  int flags;
};

// The schedule, run by one block of NT threads: checks cu_seqlens / seqused,
// writes the sequence table, the query-block bases and the work items sorted
// by decreasing number of key tiles, and the RoPE frequencies. `fwd` selects
// the forward layout: key tiles from tile_base (no tile list) and the bases of
// the padded 64-row units (rows at or past a sequence's valid length, which
// the attention kernel zeroes); otherwise the packed layout the backward uses,
// tiles numbered back to back with a tile list.
template <int NT>
__device__ void schedule_body(const int* __restrict__ cu, const int* __restrict__ seqused, int n,
                              int T, int max_seqlen, int window, double theta, Ws ws, bool fwd,
                              SchedLds<NT>& sh) {
  const int tid = threadIdx.x;
  if (tid == 0) sh.flags = 0;
  if (tid < 64) ws.rope[tid] = rope_freq(theta, tid);
  __syncthreads();

  int flags = 0;
  int carry_t = 0, carry_q = 0, carry_p = 0;
  for (int base = 0; base < n; base += NT) {
    const int s = base + tid;
    int nt = 0, nq = 0, np = 0, a = 0, len = 0, u = 0;
    if (s < n) {
      a = cu[s];
      const int b = cu[s + 1];
      if (s == 0 && a != 0) flags |= FLINT_DEV_CU_START;
      if (b < a) flags |= FLINT_DEV_CU_ORDER;
      if (s == n - 1 && b != T) flags |= FLINT_DEV_CU_END;
      len = b >= a ? b - a : 0;
      if (len > max_seqlen) flags |= FLINT_DEV_MAX_SEQLEN;
      u = seqused ? seqused[s] : len;
      if (u < 0 || u > len) {
        flags |= FLINT_DEV_SEQUSED;
        u = max(0, min(u, len));
      }
      nt = (len + kBN - 1) / kBN;
      nq = (u + kBM - 1) / kBM;
      np = u < len ? nt - u / kBN : 0;
    }
    int tot_t, tot_q, tot_p;
    const int ex_t = block_excl_scan_t<NT>(nt, sh.tmp, &tot_t);
    const int ex_q = block_excl_scan_t<NT>(nq, sh.tmp, &tot_q);
    const int ex_p = block_excl_scan_t<NT>(np, sh.tmp, &tot_p);
    if (s < n) {
      const int tb = fwd ? tile_base(a, s) : carry_t + ex_t;
      ws.seq[s] = make_int4(a, len, u, tb);
      ws.tbase[s] = tb;
      ws.qbase[s] = carry_q + ex_q;
      ws.pbase[s] = carry_p + ex_p;
    }
    carry_t += tot_t;
    carry_q += tot_q;
    carry_p += tot_p;
  }
  if (flags) atomicOr(&sh.flags, flags);
  __syncthreads();
  const int f = sh.flags;
  if (f) {  // invalid device data: schedule nothing
    if (tid == 0) {
      ws.hdr[0] = f;
      ws.hdr[1] = 0;
      ws.hdr[2] = 0;
      ws.hdr[3] = 0;
    }
    return;
  }
  if (tid == 0) {
    ws.tbase[n] = carry_t;
    ws.qbase[n] = carry_q;
    ws.pbase[n] = carry_p;
  }
  const int NTL = carry_t, NQ = carry_q;
  for (int i = tid; i < kBuckets; i += NT) sh.hist[i] = 0;
  __syncthreads();

  if (!fwd) {
    for (int e = tid; e < NTL; e += NT) {
      const int s = find_seq(ws.tbase, n, e);
      ws.tiles[e] = make_int2(s, e - ws.tbase[s]);
    }
  }
  for (int e = tid; e < NQ; e += NT) {
    const int s = find_seq(ws.qbase, n, e);
    const int c = min(block_cost(ws.seq[s].z, e - ws.qbase[s], window), kBuckets - 1);
    atomicAdd(&sh.hist[c], 1);
  }
  __syncthreads();
  // bucket starts in order of decreasing cost; thread tid owns kBuckets / NT buckets
  constexpr int kPer = kBuckets / NT;
  int local[kPer], sum = 0;
  for (int j = 0; j < kPer; ++j) {
    local[j] = sh.hist[kBuckets - 1 - (kPer * tid + j)];
    sum += local[j];
  }
  int tot;
  int run = block_excl_scan_t<NT>(sum, sh.tmp, &tot);
  for (int j = 0; j < kPer; ++j) {
    sh.hist[kBuckets - 1 - (kPer * tid + j)] = run;
    run += local[j];
  }
  __syncthreads();
  // Items of equal cost keep runs of consecutive query blocks together: the
  // lanes of a wave take their places in lane order.
  for (int e = tid; e < NQ; e += NT) {
    const int s = find_seq(ws.qbase, n, e);
    const int qb = e - ws.qbase[s];
    const int c = min(block_cost(ws.seq[s].z, qb, window), kBuckets - 1);
    const int pos = atomicAdd(&sh.hist[c], 1);
    ws.items[pos] = make_int2(s, qb);
  }
  if (tid == 0) {
    ws.hdr[0] = 0;
    ws.hdr[1] = fwd ? 0 : NTL;
    ws.hdr[2] = NQ;
    ws.hdr[3] = fwd ? carry_p : 0;
  }
}

__global__ __launch_bounds__(1024) void schedule_kernel(const int* __restrict__ cu,
                                                        const int* __restrict__ seqused, int n,
                                                        int T, int max_seqlen, int window,
                                                        double theta, Ws ws) {
  __shared__ SchedLds<1024> sh;
  schedule_body<1024>(cu, seqused, n, T, max_seqlen, window, theta, ws, false, sh);
}

void launch_schedule(const int* cu, const int* seqused, int n, int T, int max_seqlen, int window,
                     double theta, const Ws& ws, hipStream_t st) {
  schedule_kernel<<<1, 1024, 0, st>>>(cu, seqused, n, T, max_seqlen, window, theta, ws);
}

// ----------------------------------------------------------------- K/V prologue

// The sequence of forward key tile e and its index in the sequence, from
// cu_seqlens alone (tile_base layout); false for a tile slot no sequence owns
// and for entries that cannot be valid (then nothing is read or written; the
// schedule reports the error).
struct TileOf {
  int start, len, u, j;
};

__device__ __forceinline__ bool tile_of(const int* __restrict__ cu, const int* __restrict__ seqused,
                                        int n, int T, int e, TileOf& r) {
  const int s = tile_seq(cu, n, e);
  const int a = cu[s], b = cu[s + 1];
  if (a < 0 || b > T || b < a) return false;
  r.start = a;
  r.len = b - a;
  r.j = e - tile_base(a, s);
  if (r.j < 0 || r.j >= (r.len + kBN - 1) / kBN) return false;
  const int u = seqused ? seqused[s] : r.len;
  r.u = max(0, min(u, r.len));
  return true;
}

// Shared memory of kv_tile.
// Channel pairs (x[i], x[16 + i]), i < 16, turned by the RoPE angles of
// frequencies f[i] at position pos.
template <bool kMixed>
__device__ __forceinline__ void rope16(float* x, int pos, const RopeFreq* f) {
  const float pf = (float)pos;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    float c, s;
    rope_cos_sin<kMixed>(pos, pf, f[i], &c, &s);
    rope_turn(x[i], x[16 + i], c, s);
  }
}

struct KvLds {
  __attribute__((aligned(16))) uint16_t vt[kD * kBN];
  RopeFreq rope[kD / 2];
};

// One key tile e of kv head g, by 256 threads: RMSNorm + RoPE of K in FP32,
// one rounding, stored as an MFMA-ready tile in operand-fragment order; V
// transposed and key-permuted into the PV operand order; zeros for padded
// keys. F16: k and v are FP32 and the tiles fp16 (the FP16 attention-compute
// variant); otherwise k and v are bf16.
template <bool F16>
__device__ void kv_tile(int e, int g, const void* __restrict__ kp, const void* __restrict__ vp,
                        const float* __restrict__ k_norm_w, const int* __restrict__ positions,
                        const int* __restrict__ cu, const int* __restrict__ seqused, int n, int T,
                        float eps, int use_rope, double theta, Ws ws, KvLds& sh) {
  const uint16_t* k = static_cast<const uint16_t*>(kp);
  const uint16_t* v = static_cast<const uint16_t*>(vp);
  uint16_t* vt = sh.vt;
  TileOf to;
  if (!tile_of(cu, seqused, n, T, e, to)) return;
  const int start = to.start, u = to.u;
  const int tid = threadIdx.x, r = tid >> 2, p = tid & 3;
  if (use_rope && tid < kD / 2) sh.rope[tid] = rope_freq(theta, tid);
  const int ell = to.j * kBN + r;
  const bool valid = ell < u;
  const size_t t = (size_t)start + ell;
  char* tile = ws.kv + ((size_t)g * ws.ntmax + e) * kTileBytes;
  __syncthreads();

  // K: this thread owns channels [16p, 16p+16) and their RoPE partners +64.
  float x[32];
  if (valid && F16) {
    const float4* src = reinterpret_cast<const float4*>(static_cast<const float*>(kp) + (t * kG + g) * kD);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float4 a = src[4 * p + i], b = src[16 + 4 * p + i];
      x[4 * i] = a.x; x[4 * i + 1] = a.y; x[4 * i + 2] = a.z; x[4 * i + 3] = a.w;
      x[16 + 4 * i] = b.x; x[16 + 4 * i + 1] = b.y; x[16 + 4 * i + 2] = b.z; x[16 + 4 * i + 3] = b.w;
    }
  } else if (valid) {
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
    if (rope_wave_mixed(pos)) rope16<true>(x, pos, sh.rope + 16 * p);
    else rope16<false>(x, pos, sh.rope + 16 * p);
  }
  {
    uint4* kfrag = reinterpret_cast<uint4*>(tile);
    const int b = r >> 5, col = r & 31;
    kfrag[frag_index(b, 8, p, 0, col)] = pack8t<F16>(x);           // channels 16p .. 16p+7
    kfrag[frag_index(b, 8, p, 1, col)] = pack8t<F16>(x + 8);       // 16p+8 .. 16p+15
    kfrag[frag_index(b, 8, 4 + p, 0, col)] = pack8t<F16>(x + 16);  // 64+16p .. 64+16p+7
    kfrag[frag_index(b, 8, 4 + p, 1, col)] = pack8t<F16>(x + 24);  // 64+16p+8 .. 64+16p+15
  }

  // V: transpose through LDS; this thread owns channels [32p, 32p+32) of key r.
  {
    uint4 c4[4];
    if (valid && F16) {
      const float4* src = reinterpret_cast<const float4*>(static_cast<const float*>(vp) + (t * kG + g) * kD);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float4 a = src[8 * p + 2 * i], b = src[8 * p + 2 * i + 1];
        const float y[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
        c4[i] = pack8t<true>(y);
      }
    } else if (valid) {
      const uint4* src = reinterpret_cast<const uint4*>(v + (t * kG + g) * kD);
#pragma unroll
      for (int i = 0; i < 4; ++i) c4[i] = src[4 * p + i];
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) c4[i] = make_uint4(0, 0, 0, 0);
    }
    const int slot = vt_slot(r);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t w4[4] = {c4[i].x, c4[i].y, c4[i].z, c4[i].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int d = 32 * p + 8 * i + 2 * j;
        vt[d * kBN + slot] = (uint16_t)(w4[j] & 0xffff);
        vt[(d + 1) * kBN + slot] = (uint16_t)(w4[j] >> 16);
      }
    }
  }
  __syncthreads();
  {
    uint4* vtile = reinterpret_cast<uint4*>(tile + kHalfTile);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int qv = tid + 256 * i;
      const int d = qv >> 3, c = qv & 7;
      vtile[frag_index(d >> 5, 4, c >> 1, c & 1, d & 31)] =
          *reinterpret_cast<const uint4*>(&vt[d * kBN + c * 8]);
    }
  }
}

// What prep_kernel runs.
constexpr int kPrepSchedule = 1;
constexpr int kPrepKv = 2;

// The forward's preparation in one launch of 256-thread blocks: block 0 runs
// the schedule (kPrepSchedule), blocks 1.. the K/V tiles (kPrepKv), tile
// (b - 1) / 4 of kv head (b - 1) % 4 for block b. The tiles do not depend on
// the schedule (tile_base layout), so both run at once; the attention kernel
// reads both. Tile slots that no sequence owns are skipped.
template <bool F16>
__global__ __launch_bounds__(256) void prep_kernel(const void* __restrict__ kp, const void* __restrict__ vp,
                                                   const float* __restrict__ k_norm_w,
                                                   const int* __restrict__ positions,
                                                   const int* __restrict__ cu,
                                                   const int* __restrict__ seqused, int n, int T,
                                                   int max_seqlen, int window, double theta,
                                                   float eps, int use_rope, Ws ws, int parts) {
  __shared__ union {
    SchedLds<256> sched;
    KvLds kv;
  } sh;
  int b = blockIdx.x;
  if (parts & kPrepSchedule) {
    if (b == 0) {
      schedule_body<256>(cu, seqused, n, T, max_seqlen, window, theta, ws, true, sh.sched);
      return;
    }
    --b;
  }
  kv_tile<F16>(b >> 2, b & 3, kp, vp, k_norm_w, positions, cu, seqused, n, T, eps, use_rope, theta, ws,
               sh.kv);
}

// ----------------------------------------------------------------- FP16 query prep

// The FP16 attention-compute variant's query rows: RMSNorm, RoPE and the
// softmax scale in log2 units on the FP32 projection, one fp16 rounding, into
// q16 [T][32][128] (the layout the attention kernel reads raw bf16 rows from).
// Per (64-token tile, kv head): thread (token r, quarter p) forms channels
// [16p, 16p+16) and their RoPE partners +64 of the kv head's 8 query heads.
// Padded rows are not written; the attention kernel never reads them.
__global__ __launch_bounds__(256) void q16_prep_kernel(const float* __restrict__ q,
                                                       const float* __restrict__ q_norm_w,
                                                       const int* __restrict__ positions,
                                                       const int* __restrict__ cu,
                                                       const int* __restrict__ seqused, int n, int T,
                                                       float eps, int use_rope, Ws ws,
                                                       uint16_t* __restrict__ q16) {
  const int e = blockIdx.x, g = blockIdx.y;
  TileOf to;
  if (!tile_of(cu, seqused, n, T, e, to)) return;
  const int tid = threadIdx.x, r = tid >> 2, p = tid & 3;
  const int ell = to.j * kBN + r;
  if (ell >= to.u) return;  // padding; the shuffles below stay within valid quads
  const size_t t = (size_t)to.start + ell;
  float cs[16], sn[16];
  if (use_rope) {
    const int pos = positions ? positions[t] : ell;
    const float pf = (float)pos;
    if (rope_wave_mixed(pos)) {
#pragma unroll
      for (int i = 0; i < 16; ++i) rope_cos_sin<true>(pos, pf, ws.rope[16 * p + i], &cs[i], &sn[i]);
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) rope_cos_sin<false>(pos, pf, ws.rope[16 * p + i], &cs[i], &sn[i]);
    }
  }
  const float scale = kLog2e * 0.08838834764831845f;
  for (int hl = 0; hl < kHpg; ++hl) {
    const size_t row = (t * kH + g * kHpg + hl) * kD;
    const float4* src = reinterpret_cast<const float4*>(q + row);
    float x[32];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float4 a = src[4 * p + i], b = src[16 + 4 * p + i];
      x[4 * i] = a.x; x[4 * i + 1] = a.y; x[4 * i + 2] = a.z; x[4 * i + 3] = a.w;
      x[16 + 4 * i] = b.x; x[16 + 4 * i + 1] = b.y; x[16 + 4 * i + 2] = b.z; x[16 + 4 * i + 3] = b.w;
    }
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) ss += x[i] * x[i];
    ss += __shfl_xor(ss, 1);
    ss += __shfl_xor(ss, 2);
    const float rstd = 1.0f / sqrtf(ss * (1.0f / kD) + eps);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      x[i] *= rstd * q_norm_w[16 * p + i];
      x[16 + i] *= rstd * q_norm_w[64 + 16 * p + i];
    }
    if (use_rope) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float a = x[i], b = x[16 + i];
        x[i] = a * cs[i] - b * sn[i];
        x[16 + i] = b * cs[i] + a * sn[i];
      }
    }
#pragma unroll
    for (int i = 0; i < 32; ++i) x[i] *= scale;
    uint4* dst = reinterpret_cast<uint4*>(q16 + row);
    dst[2 * p] = pack8t<true>(x);
    dst[2 * p + 1] = pack8t<true>(x + 8);
    dst[8 + 2 * p] = pack8t<true>(x + 16);
    dst[9 + 2 * p] = pack8t<true>(x + 24);
  }
}

// ----------------------------------------------------------------- attention

// Direct global->LDS copy of a 32 KiB tile into an LDS stage by four waves
// (w = 0..3): each lane moves eight 16-byte vectors with buffer_load ... lds,
// which writes lane L's vector at the wave-uniform LDS base (M0) + 16 L, so the
// tile lands in LDS with the byte order it has in the workspace. `rsrc` covers
// one item's tiles only (reads past it return zeros), `soff` is the tile's
// byte offset in it, `voff` = 16 lane + 1024 w, and vector i of the lane is
// byte 4096 i + voff of the tile.
__device__ __forceinline__ void load_vec_async4(__amdgpu_buffer_rsrc_t rsrc, int voff, int soff,
                                                uint4* stage, int i, int wave) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      rsrc,
      (__attribute__((address_space(3))) void*)(reinterpret_cast<char*>(stage) + i * 4096 + wave * 1024),
      16, voff, soff + i * 4096, 0, 0);
}

__device__ __forceinline__ void load_tile_async4(__amdgpu_buffer_rsrc_t rsrc, int voff, int tile_off,
                                                 uint4* stage, int wave) {
#pragma unroll
  for (int i = 0; i < 8; ++i) load_vec_async4(rsrc, voff, tile_off, stage, i, wave);
}

// Group A (waves 0-3) moves every tile into LDS, 8 loads per wave and slot,
// issued after its logits of the slot two earlier (before any later vector-
// memory operation);
// group B issues none, and reaches LDS data only through the barrier, after
// group A has waited for it. For a wave of group A, inside an item and from
// its third slot on, the only newer operations are the next slot's loads (8)
// or none. An item's first two slots were loaded before the item's query rows;
// loads complete in issue order, so waiting for those rows (n = the
// operations issued since: output stores, 8, the normalizer store when it is
// written, 1, and for group A the third slot's loads, 8) waits for the slots
// as well. The FP32 output of the FP16 variant takes 16 stores (and writes no
// normalizer).
template <bool F16>
__device__ __forceinline__ void ring_barrier(int n) {
  if constexpr (F16) {
    switch (n) {
      case 8: ring_barrier_n<8>(); break;
      case 16: ring_barrier_n<16>(); break;
      case 24: ring_barrier_n<24>(); break;
      default: ring_barrier_n<0>(); break;
    }
  } else {
    switch (n) {
      case 8: ring_barrier_n<8>(); break;
      case 9: ring_barrier_n<9>(); break;
      case 16: ring_barrier_n<16>(); break;
      case 17: ring_barrier_n<17>(); break;
      default: ring_barrier_n<0>(); break;
    }
  }
}

struct RowState {
  f32x16 acc[4];  // O^T accumulators: channels 32db + ..., query col
  float m;        // streaming path: running max (log2 units), may be -INF
  float l0, l1;   // partial denominators (this lane's keys)
  bool online;    // streaming path for this wave
};

// S^T for the 64 keys of a tile: two 32x32 logit blocks, accumulators from
// zero. Operand fragments are read kFragAhead MFMAs ahead of their use.
template <bool F16>
__device__ __forceinline__ void tile_logits(const uint4* kt, int lane, const bf16x8* qf,
                                            f32x16& s0, f32x16& s1) {
  bf16x8 f[16];
#pragma unroll
  for (int i = 0; i < kFragAhead; ++i)
    f[i] = __builtin_bit_cast(bf16x8, kt[((i & 1) * 8 + (i >> 1)) * 64 + lane]);
  __builtin_amdgcn_sched_group_barrier(0x100, kFragAhead, 0);  // the first reads
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    if (i + kFragAhead < 16) {
      const int j = i + kFragAhead;
      f[j] = __builtin_bit_cast(bf16x8, kt[((j & 1) * 8 + (j >> 1)) * 64 + lane]);
    }
    const int kk = i >> 1;
    if (i & 1) {
      s1 = kk == 0 ? mma<F16>(f[i], qf[kk], f32x16{}) : mma<F16>(f[i], qf[kk], s1);
    } else {
      s0 = kk == 0 ? mma<F16>(f[i], qf[kk], f32x16{}) : mma<F16>(f[i], qf[kk], s0);
    }
    if (i + kFragAhead < 16) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // the next read
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                           // this MFMA
  }
}

// Mask, (streaming path) running max, and P = exp2(S - m) as the bf16 B
// operand of the PV product; the denominators sum the same rounded values.
template <bool F16>
__device__ __forceinline__ void tile_softmax(f32x16& s0, f32x16& s1, RowState& st, bf16x8* pk,
                                             int k0, int t0, int qrow, int u, int window, int half) {
  const bool need_mask =
      (k0 + kBN - 1 > t0) || (k0 + kBN > u) || (window > 0 && t0 + kBM - 1 - k0 > window - 1);
  if (need_mask) {
    // allowed keys of this query: [lo, hi]; element i of block b holds key
    // k0 + 32b + 4half + c_i with c_i = 8(i>>2) + (i&3)
    const int hi = min(qrow, u - 1);
    const int lo = window > 0 ? max(0, qrow - (window - 1)) : 0;
    const int kb = k0 + 4 * half;
    const bool empty = hi < lo;
    const int a = empty ? (1 << 30) : lo - kb;
    const unsigned range = empty ? 0u : (unsigned)(hi - lo);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int c = 8 * (i >> 2) + (i & 3);
      s0[i] = (unsigned)(c - a) <= range ? s0[i] : -INFINITY;
      s1[i] = (unsigned)(c + 32 - a) <= range ? s1[i] : -INFINITY;
    }
  }
  if (st.online) {
    // s - m relative to the current (finite) shift; a -INF max means no
    // shift yet, and the first finite tile max becomes the shift.
    const float mref = st.m == -INFINITY ? 0.f : st.m;
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      s0[i] -= mref;
      s1[i] -= mref;
      mx = fmaxf(mx, fmaxf(s0[i], s1[i]));
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const bool need = (st.m == -INFINITY) ? (mx > -INFINITY) : (mx > kRescaleSlack);
    if (__any(need)) {
      const float delta = need ? mx : 0.f;
      const float alpha = need ? (st.m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(-delta)) : 1.f;
      st.m = need ? mref + delta : st.m;
      st.l0 *= alpha;
      st.l1 *= alpha;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) st.acc[db][i] *= alpha;
#pragma unroll
      for (int i = 0; i < 16; ++i) { s0[i] -= delta; s1[i] -= delta; }
    }
  }
  float p[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) p[i] = __builtin_amdgcn_exp2f(s0[i]);
  const uint4 w0 = pack8t<F16>(p), w1 = pack8t<F16>(p + 8);
#pragma unroll
  for (int i = 0; i < 16; ++i) p[i] = __builtin_amdgcn_exp2f(s1[i]);
  const uint4 w2 = pack8t<F16>(p), w3 = pack8t<F16>(p + 8);
  pk[0] = __builtin_bit_cast(bf16x8, w0);
  pk[1] = __builtin_bit_cast(bf16x8, w1);
  pk[2] = __builtin_bit_cast(bf16x8, w2);
  pk[3] = __builtin_bit_cast(bf16x8, w3);
  st.l0 = dot2_sumt<F16>(w0, st.l0);
  st.l1 = dot2_sumt<F16>(w1, st.l1);
  st.l0 = dot2_sumt<F16>(w2, st.l0);
  st.l1 = dot2_sumt<F16>(w3, st.l1);
}

// O^T[d, query] += V^T[d, keys] P^T[keys, query]; fragments read
// kFragAhead MFMAs ahead.
template <bool F16>
__device__ __forceinline__ void tile_pv(const uint4* vt, int lane, const bf16x8* pk, RowState& st) {
  bf16x8 f[16];
#pragma unroll
  for (int i = 0; i < kFragAhead; ++i) f[i] = __builtin_bit_cast(bf16x8, vt[i * 64 + lane]);
  __builtin_amdgcn_sched_group_barrier(0x100, kFragAhead, 0);
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    if (i + kFragAhead < 16)
      f[i + kFragAhead] = __builtin_bit_cast(bf16x8, vt[(i + kFragAhead) * 64 + lane]);
    const int db = i >> 2, kk = i & 3;
    st.acc[db] = mma<F16>(f[i], pk[kk], st.acc[db]);
    if (i + kFragAhead < 16) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
  }
}

// Largest |k'| any key can have, from the key-norm weights: RMSNorm gives a
// head vector of norm sqrt(128 ms / (ms + eps)) <= sqrt(128), the weight scales
// each channel by at most max |w|, RoPE turns channel pairs without changing
// their norm, and one rounding to bf16 or fp16 adds at most 2^-8 relatively.
// Every wave reads the 128 weights itself (two per lane).
__device__ __forceinline__ float key_norm_bound(const float* __restrict__ k_norm_w, int lane) {
  float w = fmaxf(fabsf(k_norm_w[lane]), fabsf(k_norm_w[lane + 64]));
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) w = fmaxf(w, __shfl_xor(w, off));
  w = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(w)));
  return 11.313708498984761f * w * 1.00390625f;
}

// Padded rows (index in the sequence at or past the valid length) of `out`
// are exact zeros and their normalizer -INF (an empty softmax). The schedule
// lists them in nu 64-row units (ws.pbase; the caller passes nu = 0 when the
// schedule found invalid device data, so nothing is written then); unit i goes
// to workgroup i % nw of the ones serving kv head g, which zeroes its `heads`
// query heads from h0 = g * 8 + hoff on, with its NT threads.
template <bool F16, int NT>
__device__ void zero_padded_rows(const Ws& ws, int n, int nu, int g, int hoff, int heads, int w, int nw,
                                 void* __restrict__ outp, float* __restrict__ lse) {
  constexpr int kElem = F16 ? 4 : 2;
  const int row_vec = heads * kD * kElem / 16;  // 16-byte vectors of one token's rows
  const int h0 = g * kHpg + hoff;
  const int tid = threadIdx.x;
  for (int i = w; i < nu; i += nw) {
    const int s = find_seq(ws.pbase, n, i);
    const int4 meta = ws.seq[s];  // start, length, valid length
    const int j = meta.z / kBN + (i - ws.pbase[s]);
    const int r0 = max(j * kBN, meta.z), r1 = min(j * kBN + kBN, meta.y);
    for (int idx = tid; idx < (r1 - r0) * row_vec; idx += NT) {
      const int rr = r0 + idx / row_vec, c = idx - (idx / row_vec) * row_vec;
      uint4* dst = reinterpret_cast<uint4*>(static_cast<char*>(outp) +
                                            ((size_t)(meta.x + rr) * kH + h0) * kD * kElem) + c;
      *dst = make_uint4(0, 0, 0, 0);
    }
    if (lse)
      for (int idx = tid; idx < (r1 - r0) * heads; idx += NT) {
        const int rr = r0 + idx / heads;
        lse[(size_t)(meta.x + rr) * kH + h0 + idx % heads] = -INFINITY;
      }
  }
}

// One work item = 32 query tokens x the 8 query heads of one kv head. A
// workgroup keeps the list of its items in LDS as {sequence start, valid
// length, first query, first tile of the sequence}; the rest follows. The
// list's size is what the LDS left beside the tile ring and the RoPE table
// holds.
constexpr int kMaxItemsPerGroup = 896;

// RoPE cos / sin of an item's 32 query rows, formed once per workgroup for
// its 8 heads (every head of a row turns by the same angles). Lane (col,
// half) of the query prologue turns channel pairs c = 16kk + 8half + jj; its
// logical chunk i = 4kk + (jj >> 1) holds {cos, sin} of pairs c0 and c0 + 1,
// c0 = 16 (i >> 2) + 8 half + 2 (i & 3), and sits at float4 index
// (2 col + half) * 16 + (i ^ (col & 15)), so 16 consecutive lanes reading
// their chunk i meet 16 distinct 16-byte bank groups.
constexpr int kCsChunks = kBM * 2 * 16;  // 1024 float4 = 16 KiB

// Thread tid (of 512) forms logical chunks 2m and 2m + 1 (m = tid & 7), i.e.
// pairs 16 (m >> 1) + 8 half + 4 (m & 1) + 0..3, of row tid >> 4, half
// (tid >> 3) & 1, at position pos, with the function every RoPE step uses
// (kMixed when a lane of the wave needs the exact angle reduction; a lane's
// values do not depend on the choice).
template <bool kMixed>
__device__ __forceinline__ void cs_table_part(float4* s_cs, int tid, int pos, const RopeFreq* s_rope) {
  const int col = tid >> 4, half = (tid >> 3) & 1, m = tid & 7;
  const int c0 = 16 * (m >> 1) + 8 * half + 4 * (m & 1);
  const float pf = (float)pos;
  float cs[4], sn[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) rope_cos_sin<kMixed>(pos, pf, s_rope[c0 + i], &cs[i], &sn[i]);
  const int base = (2 * col + half) * 16, sw = col & 15;
  s_cs[base + ((2 * m) ^ sw)] = make_float4(cs[0], sn[0], cs[1], sn[1]);
  s_cs[base + ((2 * m + 1) ^ sw)] = make_float4(cs[2], sn[2], cs[3], sn[3]);
}

// s_waitcnt lgkmcnt(0) and a workgroup barrier: LDS writes made before it are
// seen by every wave after it; vector-memory loads stay in flight.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ void cs_table(float4* s_cs, int tid, int pos, const RopeFreq* s_rope) {
  if (rope_wave_mixed(pos)) cs_table_part<true>(s_cs, tid, pos, s_rope);
  else cs_table_part<false>(s_cs, tid, pos, s_rope);
}

struct Item {
  int start;    // first token of the sequence
  int u;        // valid length of the sequence
  int t0;       // first query of the block (index in the sequence)
  int tile_lo;  // first key tile visited (index in the sequence)
  int ntiles;   // key tiles visited
  int tfirst;   // workspace tile index of tile tile_lo
};

__device__ __forceinline__ Item item_from(int4 e, int window) {
  Item r;
  r.start = __builtin_amdgcn_readfirstlane(e.x);
  r.u = __builtin_amdgcn_readfirstlane(e.y);
  r.t0 = __builtin_amdgcn_readfirstlane(e.z);
  int klo, khi;
  block_keys(r.u, r.t0 / kBM, window, &klo, &khi);
  r.tile_lo = klo / kBN;
  r.ntiles = (khi + kBN - 1) / kBN - r.tile_lo;
  r.tfirst = __builtin_amdgcn_readfirstlane(e.w) + r.tile_lo;
  return r;
}

// Item j of workgroup w among nw (per kv head): a snake over the list sorted
// by decreasing work, ranks w, 2nw-1-w, 2nw+w, ..., so the workgroups' totals
// stay close.
__device__ __forceinline__ int item_rank(int j, int w, int nw) {
  return j * nw + ((j & 1) ? nw - 1 - w : w);
}

// Place of workgroup wg (of nwg serving one kv head) in the snake. Workgroup
// b = 4 wg + g of attn_kernel runs on XCD b % 8 = g + 4 (wg & 1), so the even
// workgroups take the first half of each round and the odd ones the second:
// consecutive ranks, which for equal costs are neighbouring query blocks of a
// sequence sharing most of their key tiles, then share an XCD and its L2.
__device__ __forceinline__ int snake_pos(int wg, int nwg) {
  return (wg & 1) ? (nwg + 1) / 2 + (wg >> 1) : (wg >> 1);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t tiles_rsrc(const Ws& ws, int g, int tfirst, int ntiles) {
  const char* base = ws.kv + ((size_t)g * ws.ntmax + tfirst) * kTileBytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base), 0, ntiles * kTileBytes, kBufferWord3);
}

// The query rows of an item for head h, lane (col, half): channels
// 16kk + 8half + [0, 8) of token t0 + col, and its RoPE position. Rows at or
// past the valid length read as zeros (buffer range check), so the number of
// vector-memory operations is fixed: 8, plus 1 when positions are read.
struct QRaw {
  uint4 x[8];
  int pos;
};

__device__ __forceinline__ void load_q(const uint16_t* q, const int* positions, bool qpos,
                                       const Item& it, int h, int col, int half, QRaw& r) {
  const int rows = min(it.u - it.t0, kBM);
  const __amdgpu_buffer_rsrc_t qr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(q + ((size_t)(it.start + it.t0) * kH + h) * kD), 0,
      rows * (kH * kD * 2), kBufferWord3);
#pragma unroll
  for (int kk = 0; kk < 8; ++kk)
    r.x[kk] = __builtin_bit_cast(
        uint4, __builtin_amdgcn_raw_buffer_load_b128(qr, col * (kH * kD * 2) + (2 * kk + half) * 16, 0, 0));
  r.pos = it.t0 + col;
  if (qpos) {
    const __amdgpu_buffer_rsrc_t pr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<int*>(positions + it.start + it.t0), 0, rows * 4, kBufferWord3);
    r.pos = (int)__builtin_amdgcn_raw_buffer_load_b32(pr, col * 4, 0, 0);
  }
}

// The RoPE position of row `row` of item `it` for the cos / sin table: the
// same value load_q gives the query lane of that row (rows at or past the
// valid length read 0 when positions are given). One vector-memory operation
// when positions are read (none otherwise); an absent item (`valid` false)
// reads nothing in range.
__device__ __forceinline__ int table_pos_load(const int* positions, bool qpos, const Item& it, bool valid,
                                              int row) {
  if (!qpos) return it.t0 + row;
  const int rows = valid ? min(it.u - it.t0, kBM) : 0;
  const __amdgpu_buffer_rsrc_t pr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<int*>(positions + (valid ? it.start + it.t0 : 0)), 0, rows * 4, kBufferWord3);
  return (int)__builtin_amdgcn_raw_buffer_load_b32(pr, row * 4, 0, 0);
}

// Norm weight, RoPE and one bf16 rounding of a wave's query rows, into the
// MFMA B-operand layout of Q^T; n2 accumulates the lane's sum of squares of
// the rounded values. s_qw holds the query norm weights times the softmax
// scale; channel c pairs with c + 64 under RoPE.
// kTab: the cos / sin come from the workgroup's table s_cs (lane col =
// lane & 31) instead of being formed here.
template <bool kRope, bool kMixed, bool kTab = false>
__device__ __forceinline__ void q_scale_rope(const QRaw& qraw, const float* s_qw, const RopeFreq* s_rope,
                                             float rstd, int half, bf16x8* qf, float& n2,
                                             const float4* s_cs = nullptr) {
  const float pf = (float)qraw.pos;
  const int tcol = __lane_id() & 31;
  const int tbase = (2 * tcol + half) * 16;
  if constexpr (kRope) {
    // channels 16kk + 8half + j pair with 16(kk+4) + 8half + j
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      float a[8], b[8];
      unpack8(qraw.x[kk], a);
      unpack8(qraw.x[kk + 4], b);
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const int c = 16 * kk + 8 * half + jj;
        float cs, sn;
        if constexpr (kTab) {
          const float4 t4 = s_cs[tbase + ((4 * kk + (jj >> 1)) ^ (tcol & 15))];
          cs = (jj & 1) ? t4.z : t4.x;
          sn = (jj & 1) ? t4.w : t4.y;
        } else {
          rope_cos_sin<kMixed>(qraw.pos, pf, s_rope[c], &cs, &sn);
        }
        a[jj] *= rstd * s_qw[c];
        b[jj] *= rstd * s_qw[c + 64];
        rope_turn(a[jj], b[jj], cs, sn);
      }
      const uint4 wa = pack8(a), wb = pack8(b);
      n2 = sumsq8_dot(wb, sumsq8_dot(wa, n2));
      qf[kk] = __builtin_bit_cast(bf16x8, wa);
      qf[kk + 4] = __builtin_bit_cast(bf16x8, wb);
    }
  } else {
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      float a[8];
      unpack8(qraw.x[kk], a);
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) a[jj] *= rstd * s_qw[16 * kk + 8 * half + jj];
      const uint4 wa = pack8(a);
      n2 = sumsq8_dot(wa, n2);
      qf[kk] = __builtin_bit_cast(bf16x8, wa);
    }
  }
}

// Query prologue: RMSNorm, RoPE, softmax scale in log2 units and one bf16
// rounding, in the MFMA B-operand layout of Q^T; qmax = max |q'| over the
// wave's 32 queries. With F16 the rows arrive prepared (q16_prep_kernel) and
// only qmax is formed. kTab: the RoPE cos / sin come from the table s_cs.
template <bool F16, bool kTab = false>
__device__ __forceinline__ void q_prologue(const QRaw& qraw, const float* s_qw, const RopeFreq* s_rope,
                                           bool rope, float eps, int half, bf16x8* qf, float& qmax,
                                           const float4* s_cs = nullptr) {
  float n2 = 0.f;
  if constexpr (F16) {
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      qf[kk] = __builtin_bit_cast(bf16x8, qraw.x[kk]);
      n2 += sumsq8t<true>(qraw.x[kk]);
    }
  } else {
    // The weight and frequency tables are re-read from LDS for every item; the
    // empty asm hides that the offset is zero, so the reads are not hoisted and
    // held in registers across the tile loop.
    int z = 0;
    asm volatile("" : "+s"(z));
    s_qw = static_cast<const float*>(__builtin_assume_aligned(s_qw + z, 16));
    s_rope += z;
    float ss = 0.f;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) ss = sumsq8_dot(qraw.x[kk], ss);
    ss += __shfl_xor(ss, 32);
    const float rstd = 1.0f / sqrtf(ss * (1.0f / kD) + eps);
    if (!rope) q_scale_rope<false, false>(qraw, s_qw, s_rope, rstd, half, qf, n2);
    else if (kTab) q_scale_rope<true, false, true>(qraw, s_qw, s_rope, rstd, half, qf, n2, s_cs);
    else if (!rope_wave_mixed(qraw.pos)) q_scale_rope<true, false>(qraw, s_qw, s_rope, rstd, half, qf, n2);
    else q_scale_rope<true, true>(qraw, s_qw, s_rope, rstd, half, qf, n2);
  }
  n2 += __shfl_xor(n2, 32);
  qmax = sqrtf(n2);
#pragma unroll
  for (int off = 1; off < 32; off <<= 1) qmax = fmaxf(qmax, __shfl_xor(qmax, off));
  qmax = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(qmax)));
}

// Persistent attention kernel: one workgroup per CU and kv head group, each
// running its items back to back. The 8 waves (one per query head) run in two
// groups, waves 0-3 (A) and 4-7 (B); the hardware places waves w and w+4 on
// the same SIMD. Group B runs half a tile behind group A, so on each SIMD one
// wave feeds the matrix cores while the other runs its softmax. Key tiles
// flow through a 4-stage LDS ring that does not stop at item boundaries: the
// tile two slots ahead streams in meanwhile, copied by group A alone (group A
// waits at the ring barrier for group B, which is the critical path), and the
// next item's query rows are fetched while the current item runs.
//
// F16 (the FP16 attention-compute variant): q holds the prepared fp16 rows,
// the tiles are fp16, the products v_mfma_f32_32x32x16_f16, and `out` is FP32
// holding the fp16-rounded output (the kernel-output boundary restored to
// FP32). The unshifted path then needs every weight below fp16's largest
// finite value, so its bound is 15 (log2 units) instead of kStaticBound.
//
// kTab (bf16 RoPE layers): the query prologue takes its RoPE cos / sin from
// the table s_cs. The table of item j + 1 is formed at item j's first tile
// (after its ring barrier, so every wave has read item j's table) from
// positions loaded with item j's query rows, and read at item j's end (after
// its second barrier, or an extra one when the item has one tile).
template <bool F16, bool kTab = false>
__global__ __launch_bounds__(kAttnThreads) void attn_kernel(const uint16_t* __restrict__ q,
                                                            const float* __restrict__ q_norm_w,
                                                            const float* __restrict__ k_norm_w,
                                                            const float* __restrict__ sink,
                                                            const int* __restrict__ positions,
                                                            int window, int use_rope, float eps,
                                                            Ws ws, int n, void* __restrict__ outp,
                                                            float* __restrict__ lse) {
  constexpr float kBound = F16 ? 15.0f : kStaticBound;
  __shared__ uint4 smem[kStages][kTileVec];
  __shared__ __attribute__((aligned(16))) float s_qw[kD];  // q_norm weights times the softmax scale
  __shared__ RopeFreq s_rope[kD / 2];           // RoPE frequencies
  __shared__ int4 s_items[kMaxItemsPerGroup];
  __shared__ float4 s_cs[kCsChunks];  // RoPE cos / sin of the next item's query rows
  const int g = blockIdx.x & (kG - 1);
  const int wg = blockIdx.x / kG, nwg = gridDim.x / kG;
  // schedule header, read once at entry: query blocks, 64-row units holding
  // padded rows (none after a device-data error)
  const int4 hdr = *reinterpret_cast<const int4*>(ws.hdr);
  const int nitems = hdr.z;
  const int npad = hdr.x != 0 ? 0 : hdr.w;
  // Items of this workgroup: the snake's ranks grow with j, so they are the
  // first nj; the last, partial round holds ranks below nitems only. The
  // launch keeps nj within kMaxItemsPerGroup.
  const int rounds = nitems / nwg, rem = nitems - rounds * nwg;
  const int sp = snake_pos(wg, nwg);
  const int nj = min(rounds + (((rounds & 1) ? nwg - 1 - sp : sp) < rem ? 1 : 0), kMaxItemsPerGroup);
  if (nj > 0) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave
  const int col = lane & 31, half = lane >> 5;
  const int h = g * kHpg + wave;
  const bool group_b = wave >= 4;
  const int voff = lane * 16 + (wave & 3) * 1024;  // group A's tile copies
  const bool rope = use_rope != 0;
  const bool qpos = rope && positions;
  static_assert(!(F16 && kTab), "the FP16 variant takes prepared query rows");
  const bool tab = kTab && rope;
  const int q_ops = (qpos ? 9 : 8) + (kTab && qpos ? 1 : 0);  // query rows, position, table position
  const int slot_ops = group_b ? 0 : 8;  // tile loads per slot
  const float sk = sink[h] * kLog2e;
  const float kmax = key_norm_bound(k_norm_w, lane);  // |k'| of every key is at most this
  if (tid < kD) s_qw[tid] = q_norm_w[tid] * kQScale;
  if (tid < kD / 2) s_rope[tid] = ws.rope[tid];
  for (int jj = tid; jj < nj; jj += kAttnThreads) {
    const int2 it = ws.items[item_rank(jj, sp, nwg)];
    const int4 meta = ws.seq[it.x];
    s_items[jj] = make_int4(meta.x, meta.z, it.y * kBM, meta.w);
  }
  __syncthreads();
  if (tab) {  // the first item's table
    const Item i0 = item_from(s_items[0], window);
    cs_table(s_cs, tid, table_pos_load(positions, qpos, i0, true, tid >> 4), s_rope);
    lds_barrier();
  }

  // Tile cursor: the next slot to load is tile ck of item cj (cn tiles from
  // workspace tile ctf). Slot s of the ring lives in stage s % kStages; the
  // tile in slot s + 2 is loaded while slot s is processed. `ops` counts this
  // wave's vector-memory operations; end0 / end1 are its value after the loads
  // of slots s / s + 1.
  int cj = 0, ck = 0, cn, ctf;
  {
    const Item c = item_from(s_items[0], window);
    cn = c.ntiles;
    ctf = c.tfirst;
  }
  int ops = 0, end0 = 0, end1 = 0;
  int slot = 0;

#define FLINT_NEXT_SLOT(LOAD, RSRC, LOFF)                       \
  {                                                             \
    LOAD = cj < nj;                                             \
    if (LOAD) {                                                 \
      RSRC = tiles_rsrc(ws, g, ctf, cn);                        \
      LOFF = ck * kTileBytes;                                   \
      ops += slot_ops;                                          \
      if (++ck == cn) {                                         \
        ck = 0;                                                 \
        if (++cj < nj) {                                        \
          const Item c = item_from(s_items[cj], window);        \
          cn = c.ntiles;                                        \
          ctf = c.tfirst;                                       \
        }                                                       \
      }                                                         \
    }                                                           \
  }

  // Slots 0 and 1, then the first item's query rows.
  Item it = item_from(s_items[0], window);
  {
    bool ld;
    __amdgpu_buffer_rsrc_t r;
    int lo = 0;
    FLINT_NEXT_SLOT(ld, r, lo);
    if (!group_b) load_tile_async4(r, voff, lo, smem[0], wave);
    end0 = ops;
    FLINT_NEXT_SLOT(ld, r, lo);
    if (ld && !group_b) load_tile_async4(r, voff, lo, smem[1], wave);
    end1 = ops;
  }
  QRaw qraw;
  load_q(q, positions, qpos, it, h, col, half, qraw);
  int pnext = 0;  // this thread's table row position of the item after the current one
  if (kTab && tab) pnext = table_pos_load(positions, qpos, item_from(s_items[min(1, nj - 1)], window), nj > 1, tid >> 4);
  ops += q_ops;
  int endq = ops;  // `ops` after the current item's query loads
  // group A's pending copies of the tile two slots ahead
  bool pend = false;
  __amdgpu_buffer_rsrc_t pr = __builtin_amdgcn_make_buffer_rsrc(nullptr, 0, 0, kBufferWord3);
  int plo = 0;
  uint4* pst = smem[0];
  bf16x8 qf[8];
  float qmax;
  q_prologue<F16, kTab>(qraw, s_qw, s_rope, rope, eps, half, qf, qmax, s_cs);

  for (int j = 0; j < nj; ++j) {
    // Softmax shift: none when the logit bound |q'| max|k'| and the sink stay
    // within kStaticBound; otherwise the streaming path.
    RowState st;
    const float bnd = qmax * kmax * 1.0001f;
    st.online = !(sk <= kBound) || !(bnd <= kBound);
    // Every logit is at least -bnd: a sink far below that (or -INF) leaves
    // the shift at -bnd, so s - m keeps the precision of the logits.
    st.m = st.online ? fmaxf(sk, -bnd) : 0.f;
    st.l0 = (half == 0 && sk != -INFINITY) ? __builtin_amdgcn_exp2f(sk - st.m) : 0.f;
    st.l1 = 0.f;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) st.acc[db][i] = 0.f;

    // Both groups run the same pipelined body - softmax and PV of tile k-1,
    // then the logits of tile k - but group A passes the ring barrier just
    // before the logits and group B at the top of the body.
    const int qrow = it.t0 + col;
    f32x16 s0, s1;
    bf16x8 pk[4];
    for (int k = 0; k < it.ntiles; ++k, ++slot) {
      if (group_b) ring_barrier<F16>(k < 2 ? ops - endq : ops - end0);
      if (k > 0) {
        if (pend) {  // group A's copies of the tile two slots ahead (see below)
          load_tile_async4(pr, voff, plo, pst, wave);
          pend = false;
        }
        tile_softmax<F16>(s0, s1, st, pk, (it.tile_lo + k - 1) * kBN, it.t0, qrow, it.u, window, half);
        tile_pv<F16>(smem[(slot - 1) % kStages] + kTileVec / 2, lane, pk, st);
      }
      if (!group_b) ring_barrier<F16>(k < 2 ? ops - endq : ops - end0);  // slot is in LDS; stage (slot+2)%4 is free
      bool ld;
      __amdgpu_buffer_rsrc_t r;
      int lo = 0;
      FLINT_NEXT_SLOT(ld, r, lo);
      tile_logits<F16>(smem[slot % kStages], lane, qf, s0, s1);
      if (kTab && tab && k == 0 && j + 1 < nj) cs_table(s_cs, tid, pnext, s_rope);
      // Group A copies the tile of slot + 2 into the stage the barrier freed,
      // in one burst after its logits, at the top of the next body (or before
      // the next item's query loads): measured faster than spreading the
      // copies over the logits or the PV products, than the same burst in the
      // block of the logits, and than issuing them from group B (which runs
      // half a tile behind and is the critical path: group A waits for it at
      // the barrier).
      pend = ld && !group_b;
      pr = r;
      plo = lo;
      pst = smem[(slot + 2) % kStages];
      end0 = end1;
      end1 = ops;
    }
    // The next item's query rows stream in during this item's last tile's
    // softmax and PV.
    const bool more = j + 1 < nj;
    Item nx = it;
    if (pend) {  // before the next item's query rows, as the accounting assumes
      load_tile_async4(pr, voff, plo, pst, wave);
      pend = false;
    }
    if (more) {
      nx = item_from(s_items[j + 1], window);
      load_q(q, positions, qpos, nx, h, col, half, qraw);
      if (kTab && tab)
        pnext = table_pos_load(positions, qpos, item_from(s_items[min(j + 2, nj - 1)], window), j + 2 < nj,
                               tid >> 4);
      ops += q_ops;
      endq = ops;
    }
    tile_softmax<F16>(s0, s1, st, pk, (it.tile_lo + it.ntiles - 1) * kBN, it.t0, qrow, it.u, window, half);
    tile_pv<F16>(smem[(slot - 1) % kStages] + kTileVec / 2, lane, pk, st);
    // Epilogue: O = acc / l in bf16. Lane (col, half) holds channels
    // 32db + 8rg + 4half + [0, 4) of query t0 + col; one swap with the
    // partner lane (col, 1 - half) gives it channels 32db + 16r2 + 8half +
    // [0, 8) instead, 16 contiguous bytes per store.
    const float lsum = st.l0 + st.l1;
    const float lt = lsum + __shfl_xor(lsum, 32);
    const float inv = lt > 0.f ? 1.0f / lt : 0.f;
    uint4 ow[8];
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int r2 = 0; r2 < 2; ++r2) {
        const f32x16& c = st.acc[db];
        const int o = 8 * r2;
        const unsigned a0 = pack2t<F16>(c[o] * inv, c[o + 1] * inv), a1 = pack2t<F16>(c[o + 2] * inv, c[o + 3] * inv);
        const unsigned b0 = pack2t<F16>(c[o + 4] * inv, c[o + 5] * inv), b1 = pack2t<F16>(c[o + 6] * inv, c[o + 7] * inv);
        // lanes 32-63 of the first operand trade places with lanes 0-31 of the second
        const auto x0 = __builtin_amdgcn_permlane32_swap(a0, b0, false, false);
        const auto x1 = __builtin_amdgcn_permlane32_swap(a1, b1, false, false);
        ow[2 * db + r2] = make_uint4(x0[0], x1[0], x0[1], x1[1]);
      }
    // The next item's query prologue runs before this item's output stores,
    // so its query loads are the newest vector-memory operations it waits on.
    if (more) {
      if (kTab && tab && it.ntiles == 1) lds_barrier();  // the table written at this item's only tile
      q_prologue<F16, kTab>(qraw, s_qw, s_rope, rope, eps, half, qf, qmax, s_cs);
    }
    // Rows past the valid length fall outside the store range and are dropped.
    constexpr int kOutElem = F16 ? 4 : 2;  // FP32 restored from fp16, or bf16
    const __amdgpu_buffer_rsrc_t orsrc = __builtin_amdgcn_make_buffer_rsrc(
        static_cast<char*>(outp) + ((size_t)(it.start + it.t0) * kH + h) * kD * kOutElem, 0,
        min(it.u - it.t0, kBM) * (kH * kD * kOutElem), kBufferWord3);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int ob = col * (kH * kD * kOutElem) + (32 * (i >> 1) + 16 * (i & 1) + 8 * half) * kOutElem;
      if constexpr (F16) {
        const uint32_t w[4] = {ow[i].x, ow[i].y, ow[i].z, ow[i].w};
        float y[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const f16x2_t hv = __builtin_bit_cast(f16x2_t, w[e]);
          y[2 * e] = (float)hv[0];
          y[2 * e + 1] = (float)hv[1];
        }
        typedef float f32x4_t __attribute__((ext_vector_type(4)));
        __builtin_amdgcn_raw_buffer_store_b128(
            __builtin_bit_cast(__attribute__((ext_vector_type(4))) unsigned, f32x4_t{y[0], y[1], y[2], y[3]}), orsrc,
            ob, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b128(
            __builtin_bit_cast(__attribute__((ext_vector_type(4))) unsigned, f32x4_t{y[4], y[5], y[6], y[7]}), orsrc,
            ob + 16, 0, 0);
      } else {
        __builtin_amdgcn_raw_buffer_store_b128(
            __builtin_bit_cast(__attribute__((ext_vector_type(4))) unsigned, ow[i]), orsrc, ob, 0, 0);
      }
    }
    ops += F16 ? 16 : 8;
    if (lse) {
      // natural-log normalizer of the row: (m + log2 l) ln 2 with m = 0 on the unshifted path
      const float m = st.online ? st.m : 0.f;
      const float lv = lt > 0.f ? (m + __builtin_amdgcn_logf(lt)) * kLn2 : -INFINITY;
      const __amdgpu_buffer_rsrc_t lr = __builtin_amdgcn_make_buffer_rsrc(
          lse + (size_t)(it.start + it.t0) * kH + h, 0, min(it.u - it.t0, kBM) * (kH * 4), kBufferWord3);
      if (half == 0) __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(lv), lr, col * (kH * 4), 0, 0);
      ops += 1;
    }

    it = nx;
  }
#undef FLINT_NEXT_SLOT
  }  // nj > 0
  zero_padded_rows<F16, kAttnThreads>(ws, n, npad, g, 0, kHpg, wg, nwg, outp, lse);
}

// ----------------------------------------------------------------- mask helper

__global__ __launch_bounds__(1024) void mask_kernel(const uint8_t* __restrict__ mask, int batch,
                                                    int seqlen, int* __restrict__ seqused,
                                                    int* __restrict__ n_bad) {
  __shared__ int s_cnt, s_first, s_bad;
  const int tid = threadIdx.x;
  if (tid == 0) s_bad = 0;
  for (int b = 0; b < batch; ++b) {
    if (tid == 0) {
      s_cnt = 0;
      s_first = seqlen;
    }
    __syncthreads();
    int cnt = 0, first = seqlen;
    const uint8_t* row = mask + (size_t)b * seqlen;
    for (int i = tid; i < seqlen; i += 1024) {
      if (row[i]) ++cnt;
      else first = min(first, i);
    }
    atomicAdd(&s_cnt, cnt);
    atomicMin(&s_first, first);
    __syncthreads();
    if (tid == 0) {
      // a row that is not ones followed by zeros gets the invalid length -1,
      // which the forward reports as a device-data error
      const bool bad = s_cnt != s_first;
      seqused[b] = bad ? -1 : s_cnt;
      if (bad) ++s_bad;
    }
    __syncthreads();
  }
  if (tid == 0) *n_bad = s_bad;
}

}  // namespace flint

// ===================================================================== C ABI

using namespace flint;

extern "C" size_t flint_attn_workspace_bytes(int32_t total_tokens, int32_t n_seqs,
                                             int32_t max_seqlen, int32_t num_kv_heads,
                                             int32_t head_dim) {
  if (total_tokens < 0 || n_seqs < 0 || max_seqlen < 0 || max_seqlen > kMaxSeqLen) return 0;
  if (num_kv_heads != kG || head_dim != kD) return 0;
  return make_layout(total_tokens, n_seqs).total;
}

extern "C" const char* flint_attn_strerror(int status) {
  switch (status) {
    case FLINT_OK: return "ok";
    case FLINT_ERR_NULL: return "a required pointer is NULL";
    case FLINT_ERR_SHAPE: return "invalid sizes (negative or inconsistent)";
    case FLINT_ERR_UNSUPPORTED: return "unsupported head layout (need 32 query heads, 4 kv heads, head_dim 128)";
    case FLINT_ERR_VALUE: return "invalid value (window < 0, eps <= 0, rope_theta <= 0 with RoPE, or NaN)";
    case FLINT_ERR_WORKSPACE: return "workspace missing or smaller than flint_attn_workspace_bytes()";
    case FLINT_ERR_ALIGN: return "misaligned pointer (tensors need 16 bytes, workspace 256, int32 arrays 4)";
    case FLINT_ERR_HIP: return "HIP runtime error";
    case FLINT_ERR_DEVICE_DATA: return "invalid device data (cu_seqlens, seqused or mask)";
    case FLINT_ERR_TOO_LARGE: return "the call needs more workspace than flint_attn_fwd_static's static scratch holds";
    default: return "unknown flint_attn status";
  }
}

// Workgroups per kv head of the persistent attention kernel: one per CU in
// all (the LDS ring admits one workgroup per CU), more only when a
// workgroup's item list would outgrow its LDS table, never more than the
// query blocks.
static int64_t attn_groups(int64_t nqmax) {
  static int cus[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = 0;
  int n = (dev >= 0 && dev < 64) ? cus[dev] : 0;
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    if (dev >= 0 && dev < 64) cus[dev] = n;
  }
  int64_t per_head = n / kG > 0 ? n / kG : 1;
  // FLINT_ATTN_WORKGROUPS=<n> sets the workgroups per kv head (clamped as
  // below): the results do not depend on it, which the tests check
  if (const char* e = getenv("FLINT_ATTN_WORKGROUPS")) {
    const long v = strtol(e, nullptr, 10);
    if (v > 0) per_head = v;
  }
  // each workgroup's item list fits its LDS table
  const int64_t need = (nqmax + kMaxItemsPerGroup - 1) / kMaxItemsPerGroup;
  if (per_head < need) per_head = need;
  return nqmax < per_head ? nqmax : per_head;
}

// ----------------------------------------------------------------- small problems

// When there are fewer work items than CUs, each item runs on two workgroups
// of 4 waves, one per query head of its half of the kv head's 8 heads, so the
// small grid covers twice as many CUs and each workgroup's MFMA work per key
// tile halves. A workgroup has its own 2-stage LDS ring (64 KiB), fills it with
// the same direct-to-LDS tile copies, and runs the same logits, softmax and PV
// steps per 64-key tile as attn_kernel, without the two-group stagger.
constexpr int kHalfThreads = 256;
constexpr int kHStages = 2;
constexpr int kMaxItemsHalf = 512;

// tile_logits for 4-wave workgroups: eight tile loads per wave, one after
// every second MFMA.
__device__ __forceinline__ void tile_logits_h(const uint4* kt, int lane, const bf16x8* qf, f32x16& s0,
                                              f32x16& s1, bool load, __amdgpu_buffer_rsrc_t rsrc,
                                              int voff, int loff, uint4* lstage, int wave) {
  bf16x8 f[16];
#pragma unroll
  for (int i = 0; i < kFragAhead; ++i)
    f[i] = __builtin_bit_cast(bf16x8, kt[((i & 1) * 8 + (i >> 1)) * 64 + lane]);
  __builtin_amdgcn_sched_group_barrier(0x100, kFragAhead, 0);
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    if (i + kFragAhead < 16) {
      const int j = i + kFragAhead;
      f[j] = __builtin_bit_cast(bf16x8, kt[((j & 1) * 8 + (j >> 1)) * 64 + lane]);
    }
    const int kk = i >> 1;
    if (i & 1) {
      s1 = kk == 0 ? mma<false>(f[i], qf[kk], f32x16{}) : mma<false>(f[i], qf[kk], s1);
    } else {
      s0 = kk == 0 ? mma<false>(f[i], qf[kk], f32x16{}) : mma<false>(f[i], qf[kk], s0);
    }
    if (i + kFragAhead < 16) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if ((i & 1) == 1 && load) load_vec_async4(rsrc, voff, loff, lstage, i >> 1, wave);
  }
}

// Grid: 8 consecutive workgroups per group of items, bits 0-1 the kv head and
// bit 2 which half of its query heads; items are dealt to the groups as in
// attn_kernel.
__global__ __launch_bounds__(kHalfThreads, 2) void attn_half_kernel(const uint16_t* __restrict__ q,
                                                                     const float* __restrict__ q_norm_w,
                                                                     const float* __restrict__ k_norm_w,
                                                                     const float* __restrict__ sink,
                                                                     const int* __restrict__ positions,
                                                                     int window, int use_rope, float eps,
                                                                     Ws ws, int n, void* __restrict__ outp,
                                                                     float* __restrict__ lse) {
  __shared__ uint4 smem[kHStages][kTileVec];
  __shared__ __attribute__((aligned(16))) float s_qw[kD];
  __shared__ RopeFreq s_rope[kD / 2];
  __shared__ int4 s_items[kMaxItemsHalf];
  const int g = blockIdx.x & (kG - 1);
  const int hh = (blockIdx.x >> 2) & 1;
  const int wg = blockIdx.x >> 3, nwg = gridDim.x >> 3;
  // schedule header, read once at entry: query blocks, 64-row units holding
  // padded rows (none after a device-data error)
  const int4 hdr = *reinterpret_cast<const int4*>(ws.hdr);
  const int nitems = hdr.z;
  const int npad = hdr.x != 0 ? 0 : hdr.w;
  const int rounds = nitems / nwg, rem = nitems - rounds * nwg;
  const int nj = min(rounds + (((rounds & 1) ? nwg - 1 - wg : wg) < rem ? 1 : 0), kMaxItemsHalf);
  if (nj > 0) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, half = lane >> 5;
  const int h = g * kHpg + hh * 4 + wave;
  const int voff = lane * 16 + wave * 1024;
  const bool rope = use_rope != 0;
  const bool qpos = rope && positions;
  const float sk = sink[h] * kLog2e;
  const float kmax = key_norm_bound(k_norm_w, lane);
  if (tid < kD) s_qw[tid] = q_norm_w[tid] * kQScale;
  if (tid < kD / 2) s_rope[tid] = ws.rope[tid];
  for (int jj = tid; jj < nj; jj += kHalfThreads) {
    const int2 it = ws.items[item_rank(jj, wg, nwg)];
    const int4 meta = ws.seq[it.x];
    s_items[jj] = make_int4(meta.x, meta.z, it.y * kBM, meta.w);
  }
  __syncthreads();

  int cj = 0, ck = 0, cn, ctf;
  {
    const Item c = item_from(s_items[0], window);
    cn = c.ntiles;
    ctf = c.tfirst;
  }
  int slot = 0;
#define FLINT_NEXT_SLOT_H(LOAD, RSRC, LOFF)                     \
  {                                                             \
    LOAD = cj < nj;                                             \
    if (LOAD) {                                                 \
      RSRC = tiles_rsrc(ws, g, ctf, cn);                        \
      LOFF = ck * kTileBytes;                                   \
      if (++ck == cn) {                                         \
        ck = 0;                                                 \
        if (++cj < nj) {                                        \
          const Item c = item_from(s_items[cj], window);        \
          cn = c.ntiles;                                        \
          ctf = c.tfirst;                                       \
        }                                                       \
      }                                                         \
    }                                                           \
  }
  Item it = item_from(s_items[0], window);
  {
    bool ld;
    __amdgpu_buffer_rsrc_t r;
    int lo = 0;
    FLINT_NEXT_SLOT_H(ld, r, lo);
#pragma unroll
    for (int i = 0; i < 8; ++i) load_vec_async4(r, voff, lo, smem[0], i, wave);
  }
  QRaw qraw;
  load_q(q, positions, qpos, it, h, col, half, qraw);
  bf16x8 qf[8];
  float qmax;
  q_prologue<false>(qraw, s_qw, s_rope, rope, eps, half, qf, qmax);

  for (int j = 0; j < nj; ++j) {
    RowState st;
    const float bnd = qmax * kmax * 1.0001f;
    st.online = !(sk <= kStaticBound) || !(bnd <= kStaticBound);
    st.m = st.online ? fmaxf(sk, -bnd) : 0.f;  // as in attn_kernel
    st.l0 = (half == 0 && sk != -INFINITY) ? __builtin_amdgcn_exp2f(sk - st.m) : 0.f;
    st.l1 = 0.f;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) st.acc[db][i] = 0.f;
    const int qrow = it.t0 + col;
    f32x16 s0, s1;
    bf16x8 pk[4];
    for (int k = 0; k < it.ntiles; ++k, ++slot) {
      // this slot is in LDS, and every wave is done with the other stage,
      // which the loads below refill
      ring_barrier_n<0>();
      bool ld;
      __amdgpu_buffer_rsrc_t r;
      int lo = 0;
      FLINT_NEXT_SLOT_H(ld, r, lo);
      tile_logits_h(smem[slot % kHStages], lane, qf, s0, s1, ld, r, voff, lo, smem[(slot + 1) % kHStages], wave);
      tile_softmax<false>(s0, s1, st, pk, (it.tile_lo + k) * kBN, it.t0, qrow, it.u, window, half);
      tile_pv<false>(smem[slot % kHStages] + kTileVec / 2, lane, pk, st);
    }
    const bool more = j + 1 < nj;
    Item nx = it;
    if (more) {
      nx = item_from(s_items[j + 1], window);
      load_q(q, positions, qpos, nx, h, col, half, qraw);
    }
    const float lsum = st.l0 + st.l1;
    const float lt = lsum + __shfl_xor(lsum, 32);
    const float inv = lt > 0.f ? 1.0f / lt : 0.f;
    uint4 ow[8];
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int r2 = 0; r2 < 2; ++r2) {
        const f32x16& c = st.acc[db];
        const int o = 8 * r2;
        const unsigned a0 = pack2(c[o] * inv, c[o + 1] * inv), a1 = pack2(c[o + 2] * inv, c[o + 3] * inv);
        const unsigned b0 = pack2(c[o + 4] * inv, c[o + 5] * inv), b1 = pack2(c[o + 6] * inv, c[o + 7] * inv);
        const auto x0 = __builtin_amdgcn_permlane32_swap(a0, b0, false, false);
        const auto x1 = __builtin_amdgcn_permlane32_swap(a1, b1, false, false);
        ow[2 * db + r2] = make_uint4(x0[0], x1[0], x0[1], x1[1]);
      }
    if (more) q_prologue<false>(qraw, s_qw, s_rope, rope, eps, half, qf, qmax);
    const __amdgpu_buffer_rsrc_t orsrc = __builtin_amdgcn_make_buffer_rsrc(
        static_cast<char*>(outp) + ((size_t)(it.start + it.t0) * kH + h) * kD * 2, 0,
        min(it.u - it.t0, kBM) * (kH * kD * 2), kBufferWord3);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int ob = col * (kH * kD * 2) + (32 * (i >> 1) + 16 * (i & 1) + 8 * half) * 2;
      __builtin_amdgcn_raw_buffer_store_b128(
          __builtin_bit_cast(__attribute__((ext_vector_type(4))) unsigned, ow[i]), orsrc, ob, 0, 0);
    }
    if (lse) {
      const float m = st.online ? st.m : 0.f;
      const float lv = lt > 0.f ? (m + __builtin_amdgcn_logf(lt)) * kLn2 : -INFINITY;
      const __amdgpu_buffer_rsrc_t lr = __builtin_amdgcn_make_buffer_rsrc(
          lse + (size_t)(it.start + it.t0) * kH + h, 0, min(it.u - it.t0, kBM) * (kH * 4), kBufferWord3);
      if (half == 0) __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(lv), lr, col * (kH * 4), 0, 0);
    }
    it = nx;
  }
#undef FLINT_NEXT_SLOT_H
  }  // nj > 0
  zero_padded_rows<false, kHalfThreads>(ws, n, npad, g, 4 * ((blockIdx.x >> 2) & 1), 4, wg, nwg, outp, lse);
}

// Query blocks per kv head up to which the forward runs on attn_half_kernel:
// half the CUs per kv head, so every item still gets its two workgroups.
static int64_t small_limit() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
  return n / kG;
}

// The attention kernel of a bf16 forward over these sizes: the split 4-wave
// kernel when the query blocks per kv head are at most half the CUs per kv
// head, else the 8-wave one.
static bool use_split_kernel(int64_t nqmax) { return nqmax * 2 <= small_limit(); }

extern "C" int flint_attn_fwd_kernel(int32_t total_tokens, int32_t n_seqs) {
  if (total_tokens < 0 || n_seqs < 0) return FLINT_ERR_SHAPE;
  if (total_tokens == 0) return 0;
  if (n_seqs < 1) return FLINT_ERR_SHAPE;
  return use_split_kernel(make_layout(total_tokens, n_seqs, false).nqmax) ? FLINT_KERNEL_SPLIT
                                                                           : FLINT_KERNEL_WIDE;
}

// Workgroup pairs per kv head of attn_half_kernel.
static int64_t attn_groups_half(int64_t nqmax) {
  int64_t per_head = attn_groups(nqmax);
  const int64_t need = (nqmax + kMaxItemsHalf - 1) / kMaxItemsHalf;
  if (per_head < need) per_head = need;
  return nqmax < per_head ? nqmax : per_head;
}

extern "C" int flint_attn_device_status(const void* workspace, void* stream, int32_t* flags) {
  if (!workspace || !flags) return FLINT_ERR_NULL;
  if (!aligned(workspace, 256)) return FLINT_ERR_ALIGN;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  int32_t host = 0;
  if (hipMemcpyAsync(&host, workspace, sizeof(int32_t), hipMemcpyDeviceToHost, st) != hipSuccess)
    return FLINT_ERR_HIP;
  if (hipStreamSynchronize(st) != hipSuccess) return FLINT_ERR_HIP;
  *flags = host;
  return host ? FLINT_ERR_DEVICE_DATA : FLINT_OK;
}

static int fwd_impl(const void* q, const void* k, const void* v, const float* q_norm_w,
                    const float* k_norm_w, const float* sink, const int32_t* positions,
                    const int32_t* cu_seqlens, const int32_t* seqused, int32_t n_seqs,
                    int32_t max_seqlen, int32_t total_tokens, int32_t num_q_heads,
                    int32_t num_kv_heads, int32_t head_dim, int32_t window, int32_t use_rope,
                    float rope_theta, float eps, void* workspace, size_t workspace_bytes, void* out,
                    float* lse, void* stream, int32_t phases, bool f16 = false) {
  if (phases <= 0 || (phases & ~FLINT_PHASE_ALL)) return FLINT_ERR_VALUE;
  if (total_tokens < 0 || n_seqs < 0 || max_seqlen < 0) return FLINT_ERR_SHAPE;
  if (num_q_heads != kH || num_kv_heads != kG || head_dim != kD || max_seqlen > kMaxSeqLen)
    return FLINT_ERR_UNSUPPORTED;
  if (window < 0 || !(eps > 0.f) || !isfinite(eps)) return FLINT_ERR_VALUE;
  if (use_rope && (!(rope_theta > 0.f) || !isfinite(rope_theta))) return FLINT_ERR_VALUE;
  if (total_tokens == 0) return FLINT_OK;
  if (n_seqs < 1) return FLINT_ERR_SHAPE;
  if (!q || !k || !v || !q_norm_w || !k_norm_w || !sink || !cu_seqlens || !out)
    return FLINT_ERR_NULL;
  if (!workspace) return FLINT_ERR_WORKSPACE;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) ||
      !aligned(workspace, 256) || !aligned(q_norm_w, 4) || !aligned(k_norm_w, 4) ||
      !aligned(sink, 4) || !aligned(cu_seqlens, 4) || (positions && !aligned(positions, 4)) ||
      (seqused && !aligned(seqused, 4)) || (lse && !aligned(lse, 16)))
    return FLINT_ERR_ALIGN;
  const Layout L = make_layout(total_tokens, n_seqs, true, f16);
  if (workspace_bytes < L.total) return FLINT_ERR_WORKSPACE;

  const Ws ws = ws_at(workspace, L);

  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const uint16_t* qh = static_cast<const uint16_t*>(q);
  const uint16_t* kh = static_cast<const uint16_t*>(k);
  const uint16_t* vh = static_cast<const uint16_t*>(v);
  uint16_t* oh = static_cast<uint16_t*>(out);
  const int rope = use_rope ? 1 : 0;
  const int* pos = rope ? positions : nullptr;

  (void)hipGetLastError();
  // The schedule and the K/V tiles in one launch (prep_kernel), then the
  // attention kernel, which also zeroes the padded rows of `out`.
  const int parts = ((phases & FLINT_PHASE_SCHEDULE) ? kPrepSchedule : 0) |
                    ((phases & FLINT_PHASE_KV) ? kPrepKv : 0);
  const double theta = (double)rope_theta;
  if (parts) {
    const unsigned grid = (unsigned)((parts & kPrepKv) ? L.ntmax * kG : 0) + ((parts & kPrepSchedule) ? 1u : 0u);
    if (f16)
      prep_kernel<true><<<grid, 256, 0, st>>>(k, v, k_norm_w, pos, cu_seqlens, seqused, n_seqs, total_tokens,
                                              max_seqlen, window, theta, eps, rope, ws, parts);
    else
      prep_kernel<false><<<grid, 256, 0, st>>>(kh, vh, k_norm_w, pos, cu_seqlens, seqused, n_seqs,
                                               total_tokens, max_seqlen, window, theta, eps, rope, ws,
                                               parts);
  }
  uint16_t* q16 = reinterpret_cast<uint16_t*>(static_cast<char*>(workspace) + L.q16);
  if (f16 && (phases & FLINT_PHASE_KV))  // reads the RoPE table the schedule wrote
    q16_prep_kernel<<<dim3((unsigned)L.ntmax, kG), 256, 0, st>>>(
        static_cast<const float*>(q), q_norm_w, pos, cu_seqlens, seqused, n_seqs, total_tokens, eps, rope,
        ws, q16);
  if (phases & FLINT_PHASE_ATTEND) {
    const unsigned grid = (unsigned)(attn_groups(L.nqmax) * kG);
    if (f16)
      attn_kernel<true><<<grid, kAttnThreads, 0, st>>>(q16, q_norm_w, k_norm_w, sink, pos, window, rope,
                                                       eps, ws, n_seqs, out, nullptr);
    else if (use_split_kernel(L.nqmax))
      attn_half_kernel<<<(unsigned)(attn_groups_half(L.nqmax) * kG * 2), kHalfThreads, 0, st>>>(
          qh, q_norm_w, k_norm_w, sink, pos, window, rope, eps, ws, n_seqs, oh, lse);
    else if (rope)
      attn_kernel<false, true><<<grid, kAttnThreads, 0, st>>>(qh, q_norm_w, k_norm_w, sink, pos, window,
                                                              rope, eps, ws, n_seqs, oh, lse);
    else
      attn_kernel<false><<<grid, kAttnThreads, 0, st>>>(qh, q_norm_w, k_norm_w, sink, pos, window, rope,
                                                        eps, ws, n_seqs, oh, lse);
  }
  if (hipGetLastError() != hipSuccess) return FLINT_ERR_HIP;
  if (debug_sync()) {
    int32_t flags = 0;
    return flint_attn_device_status(workspace, stream, &flags);
  }
  return FLINT_OK;
}

extern "C" int flint_attn_fwd_phases(const void* q, const void* k, const void* v,
                                     const float* q_norm_w, const float* k_norm_w,
                                     const float* sink, const int32_t* positions,
                                     const int32_t* cu_seqlens, const int32_t* seqused,
                                     int32_t n_seqs, int32_t max_seqlen, int32_t total_tokens,
                                     int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                     int32_t window, int32_t use_rope, float rope_theta, float eps,
                                     void* workspace, size_t workspace_bytes, void* out,
                                     void* stream, int32_t phases) {
  return fwd_impl(q, k, v, q_norm_w, k_norm_w, sink, positions, cu_seqlens, seqused, n_seqs,
                  max_seqlen, total_tokens, num_q_heads, num_kv_heads, head_dim, window, use_rope,
                  rope_theta, eps, workspace, workspace_bytes, out, nullptr, stream, phases);
}

extern "C" int flint_attn_fwd_lse(const void* q, const void* k, const void* v,
                                  const float* q_norm_w, const float* k_norm_w, const float* sink,
                                  const int32_t* positions, const int32_t* cu_seqlens,
                                  const int32_t* seqused, int32_t n_seqs, int32_t max_seqlen,
                                  int32_t total_tokens, int32_t num_q_heads, int32_t num_kv_heads,
                                  int32_t head_dim, int32_t window, int32_t use_rope,
                                  float rope_theta, float eps, void* workspace,
                                  size_t workspace_bytes, void* out, float* lse, void* stream) {
  if (!lse && total_tokens > 0) return FLINT_ERR_NULL;
  return fwd_impl(q, k, v, q_norm_w, k_norm_w, sink, positions, cu_seqlens, seqused, n_seqs,
                  max_seqlen, total_tokens, num_q_heads, num_kv_heads, head_dim, window, use_rope,
                  rope_theta, eps, workspace, workspace_bytes, out, lse, stream, FLINT_PHASE_ALL);
}

extern "C" size_t flint_attn_f16_workspace_bytes(int32_t total_tokens, int32_t n_seqs,
                                                 int32_t max_seqlen, int32_t num_kv_heads,
                                                 int32_t head_dim) {
  if (total_tokens < 0 || n_seqs < 0 || max_seqlen < 0 || max_seqlen > kMaxSeqLen) return 0;
  if (num_kv_heads != kG || head_dim != kD) return 0;
  return make_layout(total_tokens, n_seqs, true, true).total;
}

extern "C" int flint_attn_fwd_f16(const float* q, const float* k, const float* v,
                                  const float* q_norm_w, const float* k_norm_w, const float* sink,
                                  const int32_t* positions, const int32_t* cu_seqlens,
                                  const int32_t* seqused, int32_t n_seqs, int32_t max_seqlen,
                                  int32_t total_tokens, int32_t num_q_heads, int32_t num_kv_heads,
                                  int32_t head_dim, int32_t window, int32_t use_rope,
                                  float rope_theta, float eps, void* workspace,
                                  size_t workspace_bytes, float* out, void* stream) {
  return fwd_impl(q, k, v, q_norm_w, k_norm_w, sink, positions, cu_seqlens, seqused, n_seqs,
                  max_seqlen, total_tokens, num_q_heads, num_kv_heads, head_dim, window, use_rope,
                  rope_theta, eps, workspace, workspace_bytes, out, nullptr, stream, FLINT_PHASE_ALL,
                  true);
}

extern "C" int flint_attn_fwd(const void* q, const void* k, const void* v, const float* q_norm_w,
                              const float* k_norm_w, const float* sink, const int32_t* positions,
                              const int32_t* cu_seqlens, const int32_t* seqused, int32_t n_seqs,
                              int32_t max_seqlen, int32_t total_tokens, int32_t num_q_heads,
                              int32_t num_kv_heads, int32_t head_dim, int32_t window,
                              int32_t use_rope, float rope_theta, float eps, void* workspace,
                              size_t workspace_bytes, void* out, void* stream) {
  return flint_attn_fwd_phases(q, k, v, q_norm_w, k_norm_w, sink, positions, cu_seqlens, seqused,
                               n_seqs, max_seqlen, total_tokens, num_q_heads, num_kv_heads,
                               head_dim, window, use_rope, rope_theta, eps, workspace,
                               workspace_bytes, out, stream, FLINT_PHASE_ALL);
}

// ----------------------------------------------------------------- forward without allocation

// The workspace of flint_attn_fwd_static: one array per GPU in the code
// object's device memory, held until the process ends. Host code never passes
// its name to a kernel (in host code it is only a stand-in for the device
// symbol); it uses the device address that hipGetSymbolAddress returns,
// looked up once per device.
constexpr size_t kStaticScratchBytes = FLINT_ATTN_STATIC_SCRATCH_BYTES;
static __device__ __align__(256) char scratch[kStaticScratchBytes];

static std::mutex g_scratch_mu;
static void* g_scratch_ptr[64];

// Device address of this device's scratch array, or NULL when the lookup fails.
static void* static_scratch() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
      (void)hipGetLastError();
      return nullptr;
    }
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

extern "C" int flint_attn_fwd_static(const void* q, const void* k, const void* v,
                                     const float* q_norm_w, const float* k_norm_w,
                                     const float* sink, const int32_t* positions,
                                     const int32_t* cu_seqlens, const int32_t* seqused,
                                     int32_t n_seqs, int32_t max_seqlen, int32_t total_tokens,
                                     int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                     int32_t window, int32_t use_rope, float rope_theta, float eps,
                                     void* out, void* stream) {
  if (total_tokens < 0 || n_seqs < 0 || max_seqlen < 0) return FLINT_ERR_SHAPE;
  if (num_q_heads != kH || num_kv_heads != kG || head_dim != kD || max_seqlen > kMaxSeqLen)
    return FLINT_ERR_UNSUPPORTED;
  if (total_tokens == 0) return FLINT_OK;
  if (make_layout(total_tokens, n_seqs).total > kStaticScratchBytes) return FLINT_ERR_TOO_LARGE;
  void* ws = static_scratch();
  if (!ws) return FLINT_ERR_HIP;
  return fwd_impl(q, k, v, q_norm_w, k_norm_w, sink, positions, cu_seqlens, seqused, n_seqs,
                  max_seqlen, total_tokens, num_q_heads, num_kv_heads, head_dim, window, use_rope,
                  rope_theta, eps, ws, kStaticScratchBytes, out, nullptr, stream, FLINT_PHASE_ALL);
}

extern "C" int flint_attn_seqused_from_mask(const uint8_t* mask, int32_t batch, int32_t seqlen,
                                            int32_t* seqused, int32_t* n_bad, void* stream) {
  if (batch < 0 || seqlen < 0) return FLINT_ERR_SHAPE;
  if (!seqused || !n_bad || (!mask && batch > 0 && seqlen > 0)) return FLINT_ERR_NULL;
  if (!aligned(seqused, 4) || !aligned(n_bad, 4)) return FLINT_ERR_ALIGN;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  mask_kernel<<<1, 1024, 0, st>>>(mask, batch, seqlen, seqused, n_bad);
  if (hipGetLastError() != hipSuccess) return FLINT_ERR_HIP;
  return FLINT_OK;
}
