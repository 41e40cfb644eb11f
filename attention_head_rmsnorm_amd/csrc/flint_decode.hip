// Decode with a per-layer KV cache for the Flint sink attention (one new
// token per sequence attending over its cache), gfx950.
//
// Hugging Face discussion #26 on RecursiveSI/flint ("Minor asks") asks for a
// hybrid KV cache that honours each layer's window: sliding layers keep the
// window, full layers every token. The NeMo implementation leaves KV caching
// out of scope (flint page, "Parallelism and backends"), so the cache layout
// is this library's own; its result for token t is row t of the prefill over
// tokens 0..t.

#include <hip/hip_runtime.h>

#include "flint_common.h"

namespace flint {
// ----------------------------------------------------------------- decode with a KV cache

// Per-layer cache, head-major so that each (sequence, kv head) streams one
// contiguous region, in blocks of 32 slots: the K' block [2][4][64][8] and the
// V block [8][64][8] hold the decode products' operand fragments lane by lane
// (dec_k_index and dec_v_index give an element's place), so every load of a
// block reads 1 KiB in order. Token t of a sequence sits in slot t (full
// layers) or t % cap (sliding layers, cap >= window: a ring holding the
// window). cap is a multiple of kDecBlock, so an aligned block of 32 tokens
// occupies 32 consecutive slots.
constexpr int kDecBlock = 32;         // tokens per step of the decode attention
constexpr int kDecMinSplitBlocks = 2;  // smallest split (64 tokens), sizes the workspace
constexpr int kDecMaxSplitBlocks = 16;  // largest split (512 tokens)
constexpr int kDecMergeLanes = 32;     // splits merged in parallel per (sequence, head)
constexpr int kDecBlockElems = kDecBlock * kD;  // bf16 elements of one K' or V cache block

// Position in its cache block of channel c of the key in slot kb of the block:
// K' fragment 4kh + ds of lane 16qd + col holds key 16kh + col, channels
// 32ds + 8qd .. +8; V fragment db of lane 16qd + col holds channel 16db + col
// of keys 4qd .. +4 (elements 0-3) and 16 + 4qd .. +4 (elements 4-7).
__device__ __forceinline__ int dec_k_index(int kb, int c) {
  const int kh = kb >> 4, col = kb & 15, ds = c >> 5, qd = (c >> 3) & 3, e = c & 7;
  return (((4 * kh + ds) * 64) + 16 * qd + col) * 8 + e;
}
__device__ __forceinline__ int dec_v_index(int kb, int c) {
  const int db = c >> 4, col = c & 15, hi = kb >> 4, qd = (kb >> 2) & 3, e = 4 * hi + (kb & 3);
  return ((db * 64) + 16 * qd + col) * 8 + e;
}

struct DecWs {
  int* hdr;        // [0] device-data error bits
  uint16_t* q;     // [B][32][128] bf16 query rows, normalized, rotated, scaled to log2 units
  float* ml;       // [B][4][nsplit][8][2] running max and denominator of each split
  float* part;     // [B][4][nsplit][8][128] unnormalized output of each split
  int nsplit;      // split slots per (sequence, kv head) in ml / part
  int bps;         // blocks per split of this call
};

struct DecLayout {
  size_t hdr, q, ml, part, total;
  int nsplit;
};

static DecLayout make_dec_layout(int64_t batch, int64_t cap) {
  DecLayout L;
  L.nsplit = (int)((cap / kDecBlock + 1 + kDecMinSplitBlocks - 1) / kDecMinSplitBlocks);
  size_t o = 0;
  L.hdr = o;  o = align_up(o + 64 * sizeof(int), 256);
  L.q = o;    o = align_up(o + (size_t)batch * kH * kD * 2, 256);
  L.ml = o;   o = align_up(o + (size_t)batch * kG * L.nsplit * kHpg * 2 * sizeof(float), 256);
  L.part = o; o = align_up(o + (size_t)batch * kG * L.nsplit * kHpg * kD * sizeof(float), 256);
  L.total = o;
  return L;
}

// One row of 128 channels per wave, lane c holding channels c and c + 64 (a
// RoPE pair): RMSNorm with weight w, RoPE at `pos`, then `scale`.
__device__ __forceinline__ void norm_rope_row(const uint16_t* src, const float* w, float eps,
                                              bool rope, int pos, const RopeFreq& f, float scale,
                                              int lane, float& a, float& b) {
  a = __uint_as_float((uint32_t)src[lane] << 16);
  b = __uint_as_float((uint32_t)src[lane + 64] << 16);
  float ss = a * a + b * b;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) ss += __shfl_xor(ss, off);
  const float rstd = 1.0f / sqrtf(ss * (1.0f / kD) + eps);
  a *= rstd * w[lane];
  b *= rstd * w[lane + 64];
  if (rope) {
    float c, sn;
    rope_cos_sin(pos, f, &c, &sn);
    const float x = a, y = b;
    a = x * c - y * sn;
    b = y * c + x * sn;
  }
  a *= scale;
  b *= scale;
}

__device__ __forceinline__ uint16_t bf16_bits(float x) { return (uint16_t)(pack2(x, 0.f) & 0xffff); }

// Slot of token t, or -1 when a full layer's cache cannot hold it.
__device__ __forceinline__ int dec_slot(int t, int cap, int window) {
  if (window > 0) return t % cap;
  return t < cap ? t : -1;
}

// Appends tokens cache_len[b] + i (i < n_new) of every sequence: K' and V^T
// into the cache (wave 0), and, when q is given (n_new = 1), the query rows
// of the kv head's 8 query heads into the workspace (waves 1-8).
__global__ __launch_bounds__(64 * (1 + kHpg)) void decode_append_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const float* __restrict__ q_norm_w, const float* __restrict__ k_norm_w,
    const int* __restrict__ positions, const int* __restrict__ cache_len, int n_new, int cap,
    int window, int use_rope, double theta, float eps, uint16_t* __restrict__ k_cache,
    uint16_t* __restrict__ vt_cache, DecWs ws) {
  const int i = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if ((i | g | b) == 0) {
    // The call's device-data flags, written whole by this one block (so no
    // reset launch is needed): a sequence whose length is negative or whose
    // new tokens overflow a full layer's cache is skipped everywhere.
    int bad = 0;
    for (int s = threadIdx.x; s < gridDim.z; s += blockDim.x) {
      const int l = cache_len[s];
      bad |= (l < 0 || (window == 0 && l > cap - n_new)) ? 1 : 0;
    }
    bad = __syncthreads_or(bad);
    if (threadIdx.x == 0) ws.hdr[0] = bad ? FLINT_DEV_CACHE : 0;
  }
  const int len = cache_len[b];
  const int t = len + i;
  const int slot = len >= 0 ? dec_slot(t, cap, window) : -1;
  if (slot < 0) return;
  const bool rope = use_rope != 0;
  const int pos = positions ? positions[(size_t)b * n_new + i] : t;
  const RopeFreq f = rope ? rope_freq(theta, lane) : RopeFreq{0ull, 0.f, 0.f};
  const size_t tok = (size_t)b * n_new + i;
  float a, c;
  if (wave == 0) {
    norm_rope_row(k + (tok * kG + g) * kD, k_norm_w, eps, rope, pos, f, 1.0f, lane, a, c);
    // block of 32 slots in the decode operand order (see DecFrags)
    const size_t blk = ((size_t)b * kG + g) * (cap / kDecBlock) + slot / kDecBlock;
    const int kb = slot % kDecBlock;
    uint16_t* kblk = k_cache + blk * kDecBlockElems;
    kblk[dec_k_index(kb, lane)] = bf16_bits(a);
    kblk[dec_k_index(kb, lane + 64)] = bf16_bits(c);
    const uint16_t* vr = v + (tok * kG + g) * kD;
    uint16_t* vblk = vt_cache + blk * kDecBlockElems;
    vblk[dec_v_index(kb, lane)] = vr[lane];
    vblk[dec_v_index(kb, lane + 64)] = vr[lane + 64];
  } else if (q) {
    const int h = g * kHpg + wave - 1;
    norm_rope_row(q + ((size_t)b * kH + h) * kD, q_norm_w, eps, rope, pos, f,
                  kLog2e * 0.08838834764831845f, lane, a, c);
    uint16_t* qr = ws.q + ((size_t)b * kH + h) * kD;
    qr[lane] = bf16_bits(a);
    qr[lane + 64] = bf16_bits(c);
  }
}

typedef __bf16 bf16x8_t __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef float f32x4 __attribute__((__vector_size__(4 * sizeof(float))));

// Keys of the new token of sequence b: tokens [t_lo, t_hi] with t_hi =
// cache_len[b] (the appended token) and the window's first token for
// sliding layers; in aligned 32-token blocks [blk_lo, blk_hi].
__device__ __forceinline__ void dec_range(int len, int window, int* t_lo, int* t_hi, int* blk_lo,
                                          int* nblk) {
  *t_hi = len;
  *t_lo = window > 0 ? max(0, len - window + 1) : 0;
  *blk_lo = *t_lo / kDecBlock;
  *nblk = *t_hi / kDecBlock - *blk_lo + 1;
}

// Split s of the decode attention of (sequence b, kv head g): one wave runs
// ws.bps blocks of 32 keys with v_mfma_f32_16x16x32_bf16, the 8 query heads
// as the columns 0-7 of S^T = K' Q'^T (columns 8-15 zero) and
// O^T += V^T P^T, with a streaming softmax (running max per head; the sink
// joins in the merge). Lane l holds column l % 16 and rows 4(l / 16) + [0, 4)
// of each 16-row result block. The next block's K' and V^T fragments load
// while the current one is computed.
struct DecFrags {
  bf16x8_t k[2][4];  // K' key 16kh + col, channels 32ds + 8qd .. +8
  bf16x8_t v[8];     // V channel 16db + col, keys 4qd .. +4 and 16 + 4qd .. +4
};

// A cache block holds these fragments lane by lane (K: fragment 4kh + ds,
// V: fragment db; 16 bytes per lane), so each load reads 1 KiB in order.
__device__ __forceinline__ void dec_load(const uint16_t* kblk, const uint16_t* vblk, int lane,
                                         DecFrags& f) {
  const uint4* kp = reinterpret_cast<const uint4*>(kblk) + lane;
  const uint4* vp = reinterpret_cast<const uint4*>(vblk) + lane;
#pragma unroll
  for (int kh = 0; kh < 2; ++kh)
#pragma unroll
    for (int ds = 0; ds < 4; ++ds) f.k[kh][ds] = __builtin_bit_cast(bf16x8_t, kp[(4 * kh + ds) * 64]);
#pragma unroll
  for (int db = 0; db < 8; ++db) f.v[db] = __builtin_bit_cast(bf16x8_t, vp[db * 64]);
}

// Blocks [b0, b1) of the keys [t_lo, t_hi] of one (sequence, kv head) for one
// wave: streaming softmax (running max per head) and the unnormalized output.
// qf: the query fragments (columns 0-7 the kv head's 8 query heads, 8-15 zero);
// cblk(blk): the cache block of token block blk. Returns m and l per column
// (reduced over the lane's rows) and acc.
template <typename CBlk>
__device__ __forceinline__ void dec_split(const uint16_t* __restrict__ k_cache,
                                          const uint16_t* __restrict__ vt_cache, CBlk cblk, int b0,
                                          int b1, int t_lo, int t_hi, int lane, const bf16x8_t* qf,
                                          float& m, float& l, f32x4* acc) {
  const int qd = lane >> 4;
  m = -INFINITY;
  l = 0.f;
#pragma unroll
  for (int db = 0; db < 8; ++db) acc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (b0 >= b1) return;
  DecFrags cur, nxt;
  dec_load(k_cache + cblk(b0) * kDecBlockElems, vt_cache + cblk(b0) * kDecBlockElems, lane, cur);
  for (int blk = b0; blk < b1; ++blk) {
    if (blk + 1 < b1)
      dec_load(k_cache + cblk(blk + 1) * kDecBlockElems, vt_cache + cblk(blk + 1) * kDecBlockElems, lane,
               nxt);
    f32x4 sc[2];
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
      sc[kh] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ds = 0; ds < 4; ++ds)
        sc[kh] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cur.k[kh][ds], qf[ds], sc[kh], 0, 0, 0);
    }
    // mask keys outside [t_lo, t_hi]; key of sc[kh][i] is blk*32 + 16kh + 4qd + i
    float mx = -INFINITY;
#pragma unroll
    for (int kh = 0; kh < 2; ++kh)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = blk * kDecBlock + 16 * kh + 4 * qd + i;
        if (t < t_lo || t > t_hi) sc[kh][i] = -INFINITY;
        mx = fmaxf(mx, sc[kh][i]);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mn = fmaxf(m, mx);
    const float alpha = mn == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m - mn);
    float p[8];
#pragma unroll
    for (int kh = 0; kh < 2; ++kh)
#pragma unroll
      for (int i = 0; i < 4; ++i) p[4 * kh + i] = mn == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(sc[kh][i] - mn);
    const uint4 pw = pack8(p);
    float x[8];
    unpack8(pw, x);
    float ps = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) ps += x[i];
    l = l * alpha + ps;
    m = mn;
    const bf16x8_t pf = __builtin_bit_cast(bf16x8_t, pw);
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      acc[db] *= alpha;
      acc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cur.v[db], pf, acc[db], 0, 0, 0);
    }
    cur = nxt;
  }
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
}

__global__ __launch_bounds__(64) void decode_attn_kernel(const int* __restrict__ cache_len, int cap,
                                                         int window,
                                                         const uint16_t* __restrict__ k_cache,
                                                         const uint16_t* __restrict__ vt_cache,
                                                         DecWs ws) {
  const int s = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x, col = lane & 15, qd = lane >> 4;
  const int len = cache_len[b];
  if (len < 0 || (window == 0 && len >= cap)) return;
  int t_lo, t_hi, blk_lo, nblk;
  dec_range(len, window, &t_lo, &t_hi, &blk_lo, &nblk);
  const int bs = s * ws.bps;
  if (bs >= nblk) return;
  const int be = min(bs + ws.bps, nblk);

  bf16x8_t qf[4];
#pragma unroll
  for (int ds = 0; ds < 4; ++ds) {
    uint4 w = make_uint4(0, 0, 0, 0);
    if (col < kHpg)
      w = *reinterpret_cast<const uint4*>(ws.q + ((size_t)b * kH + g * kHpg + col) * kD + 32 * ds + 8 * qd);
    qf[ds] = __builtin_bit_cast(bf16x8_t, w);
  }
  const size_t blk0 = ((size_t)b * kG + g) * (cap / kDecBlock);
  // cache block of token block blk (a ring of cap / 32 blocks on sliding layers)
  auto cblk = [&](int blk) { return blk0 + (window > 0 ? blk % (cap / kDecBlock) : blk); };

  float m, l;
  f32x4 acc[8];
  dec_split(k_cache, vt_cache, cblk, blk_lo + bs, blk_lo + be, t_lo, t_hi, lane, qf, m, l, acc);
  if (col < kHpg) {
    const size_t base = (((size_t)b * kG + g) * ws.nsplit + s) * kHpg + col;
    float* pr = ws.part + base * kD;
#pragma unroll
    for (int db = 0; db < 8; ++db)
      *reinterpret_cast<f32x4*>(pr + 16 * db + 4 * qd) = acc[db];
    if (qd == 0) *reinterpret_cast<float2*>(ws.ml + base * 2) = make_float2(m, l);
  }
}

// The whole decode step of a small cache in one launch, one workgroup of 8
// waves per (sequence, kv head): wave 0 appends the new key (as
// decode_append_kernel does), every wave forms one query head's row into LDS;
// after a barrier (which also makes wave 0's cache writes visible to the
// workgroup) the 8 waves split the key blocks among themselves as the
// split-K kernel splits them among workgroups, and the partial results merge
// through LDS with the sink joining once, as in decode_merge_kernel. The
// launch count is what bounds the step at these sizes.
constexpr int kDecFusedWaves = 8;
// Which step a call takes, from measurements (us per step, fused against
// split-K): short caches, such as the sliding layers' 544-slot rings, take
// the fused step at any batch (batch 1: 9.1 against 12.8; batch 64: 17.1
// against 28.8); longer caches take it when the batch gives at least 128
// workgroups (64 x 8,192 slots: 178 against 212; 64 x 32,768: 709 against
// 827), and otherwise keep the split-K kernel, which spreads a few long
// sequences over many waves (1 x 4,000: 22.7 against 12.2; 16 x 32,768: 329
// against 212).
constexpr int kDecFusedMaxBlocks = 32;         // 1,024 slots
constexpr int kDecFusedMaxBlocksWide = 1056;   // 33,792 slots: 32,768 tokens and the next ones
constexpr int kDecFusedWideGroups = 128;

__global__ __launch_bounds__(64 * kDecFusedWaves) void decode_fused_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const float* __restrict__ q_norm_w, const float* __restrict__ k_norm_w, const float* __restrict__ sink,
    const int* __restrict__ positions, const int* __restrict__ cache_len, int cap, int window, int use_rope,
    double theta, float eps, uint16_t* __restrict__ k_cache, uint16_t* __restrict__ vt_cache, DecWs ws,
    uint16_t* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) uint16_t s_q[kHpg][kD];
  __shared__ __attribute__((aligned(16))) float s_part[kDecFusedWaves][kHpg][kD];
  __shared__ float s_ml[kDecFusedWaves][kHpg][2];
  const int g = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if ((g | b) == 0) {
    // the call's device-data flags, written whole by this one workgroup
    int bad = 0;
    for (int s2 = tid; s2 < gridDim.y; s2 += blockDim.x) {
      const int l2 = cache_len[s2];
      bad |= (l2 < 0 || (window == 0 && l2 > cap - 1)) ? 1 : 0;
    }
    bad = __syncthreads_or(bad);
    if (tid == 0) ws.hdr[0] = bad ? FLINT_DEV_CACHE : 0;
  }
  const int len = cache_len[b];
  uint16_t* o = out + ((size_t)b * kH + g * kHpg) * kD;
  const int slot = len >= 0 ? dec_slot(len, cap, window) : -1;
  if (slot < 0) {  // skipped sequence: zero output, as the merge writes it
    for (int i = tid; i < kHpg * kD; i += blockDim.x) o[i] = 0;
    return;
  }
  const bool rope = use_rope != 0;
  const int pos = positions ? positions[b] : len;
  const RopeFreq f = rope ? rope_freq(theta, lane) : RopeFreq{0ull, 0.f, 0.f};
  float a, c;
  if (wave == 0) {
    norm_rope_row(k + ((size_t)b * kG + g) * kD, k_norm_w, eps, rope, pos, f, 1.0f, lane, a, c);
    const size_t blk = ((size_t)b * kG + g) * (cap / kDecBlock) + slot / kDecBlock;
    const int kb = slot % kDecBlock;
    uint16_t* kblk = k_cache + blk * kDecBlockElems;
    kblk[dec_k_index(kb, lane)] = bf16_bits(a);
    kblk[dec_k_index(kb, lane + 64)] = bf16_bits(c);
    const uint16_t* vr = v + ((size_t)b * kG + g) * kD;
    uint16_t* vblk = vt_cache + blk * kDecBlockElems;
    vblk[dec_v_index(kb, lane)] = vr[lane];
    vblk[dec_v_index(kb, lane + 64)] = vr[lane + 64];
  }
  norm_rope_row(q + ((size_t)b * kH + g * kHpg + wave) * kD, q_norm_w, eps, rope, pos, f,
                kLog2e * 0.08838834764831845f, lane, a, c);
  s_q[wave][lane] = bf16_bits(a);
  s_q[wave][lane + 64] = bf16_bits(c);
  __syncthreads();

  int t_lo, t_hi, blk_lo, nblk;
  dec_range(len, window, &t_lo, &t_hi, &blk_lo, &nblk);
  const int col = lane & 15, qd = lane >> 4;
  bf16x8_t qf[4];
#pragma unroll
  for (int ds = 0; ds < 4; ++ds) {
    uint4 w = make_uint4(0, 0, 0, 0);
    if (col < kHpg) w = *reinterpret_cast<const uint4*>(&s_q[col][32 * ds + 8 * qd]);
    qf[ds] = __builtin_bit_cast(bf16x8_t, w);
  }
  const size_t blk0 = ((size_t)b * kG + g) * (cap / kDecBlock);
  auto cblk = [&](int blk) { return blk0 + (window > 0 ? blk % (cap / kDecBlock) : blk); };
  const int per = (nblk + kDecFusedWaves - 1) / kDecFusedWaves;
  const int b0 = blk_lo + min(nblk, wave * per), b1 = blk_lo + min(nblk, (wave + 1) * per);
  float m, l;
  f32x4 acc[8];
  dec_split(k_cache, vt_cache, cblk, b0, b1, t_lo, t_hi, lane, qf, m, l, acc);
  if (col < kHpg) {
#pragma unroll
    for (int db = 0; db < 8; ++db) *reinterpret_cast<f32x4*>(&s_part[wave][col][16 * db + 4 * qd]) = acc[db];
    if (qd == 0) {
      s_ml[wave][col][0] = m;
      s_ml[wave][col][1] = l;
    }
  }
  __syncthreads();
  // merge: output (head hh, channel ch) over the waves' partial results
  for (int e = tid; e < kHpg * kD; e += blockDim.x) {
    const int hh = e / kD, ch = e % kD;
    const float sk = sink[g * kHpg + hh] * kLog2e;
    float mt = sk;
#pragma unroll
    for (int w = 0; w < kDecFusedWaves; ++w) mt = fmaxf(mt, s_ml[w][hh][0]);
    float lsum = (mt == -INFINITY || sk == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(sk - mt);
    float acc2 = 0.f;
#pragma unroll
    for (int w = 0; w < kDecFusedWaves; ++w) {
      const float mw = s_ml[w][hh][0];
      const float sc = mw == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mw - mt);
      lsum += s_ml[w][hh][1] * sc;
      acc2 += s_part[w][hh][ch] * sc;
    }
    o[hh * kD + ch] = bf16_bits(lsum > 0.f ? acc2 / lsum : 0.f);
  }
}

// out[b][h] = (sum_s acc_s 2^(m_s - m)) / (2^(sink - m) + sum_s l_s 2^(m_s - m)),
// m = max(sink, max_s m_s): the sink joins the softmax once. Thread (sl, dc)
// of the 256 merges splits sl, sl + 32, ... for channels 16dc .. +16; the 32
// partial merges then combine through LDS.
__global__ __launch_bounds__(256) void decode_merge_kernel(const int* __restrict__ cache_len, int cap,
                                                           int window, const float* __restrict__ sink,
                                                           DecWs ws, uint16_t* __restrict__ out) {
  __shared__ float s_m[kDecMergeLanes], s_l[kDecMergeLanes];
  __shared__ float s_acc[kDecMergeLanes][kD];
  const int h = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int sl = tid & (kDecMergeLanes - 1), dc = tid / kDecMergeLanes;  // dc: 16-channel chunk
  const int g = h / kHpg, col = h % kHpg;
  uint16_t* o = out + ((size_t)b * kH + h) * kD;
  const int len = cache_len[b];
  if (len < 0 || (window == 0 && len >= cap)) {
    if (tid < kD) o[tid] = 0;
    return;
  }
  int t_lo, t_hi, blk_lo, nblk;
  dec_range(len, window, &t_lo, &t_hi, &blk_lo, &nblk);
  const int ns = (nblk + ws.bps - 1) / ws.bps;
  const size_t base = ((size_t)b * kG + g) * ws.nsplit * kHpg + col;
  float m = -INFINITY, l = 0.f, acc[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.f;
  for (int sidx = sl; sidx < ns; sidx += kDecMergeLanes) {
    const size_t e = base + (size_t)sidx * kHpg;
    const float2 ml = *reinterpret_cast<const float2*>(ws.ml + e * 2);
    const float mn = fmaxf(m, ml.x);
    const float a0 = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m - mn);
    const float a1 = ml.x == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ml.x - mn);
    const float4* pr = reinterpret_cast<const float4*>(ws.part + e * kD + 16 * dc);
    l = l * a0 + ml.y * a1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float4 v = pr[i];
      acc[4 * i] = acc[4 * i] * a0 + v.x * a1;
      acc[4 * i + 1] = acc[4 * i + 1] * a0 + v.y * a1;
      acc[4 * i + 2] = acc[4 * i + 2] * a0 + v.z * a1;
      acc[4 * i + 3] = acc[4 * i + 3] * a0 + v.w * a1;
    }
    m = mn;
  }
  if (dc == 0) {
    s_m[sl] = m;
    s_l[sl] = l;
  }
  __syncthreads();
  float mt = sink[h] * kLog2e;
  const float sk = mt;
#pragma unroll 4
  for (int i = 0; i < kDecMergeLanes; ++i) mt = fmaxf(mt, s_m[i]);
  const float w = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m - mt);
#pragma unroll
  for (int i = 0; i < 16; ++i) s_acc[sl][16 * dc + i] = acc[i] * w;
  __syncthreads();
  if (tid < kD) {
    float lsum = (mt == -INFINITY || sk == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(sk - mt);
    float a = 0.f;
    for (int i = 0; i < kDecMergeLanes; ++i) {
      const float mi = s_m[i];
      lsum += mi == -INFINITY ? 0.f : s_l[i] * __builtin_amdgcn_exp2f(mi - mt);
      a += s_acc[i][tid];
    }
    o[tid] = bf16_bits(lsum > 0.f ? a / lsum : 0.f);
  }
}

}  // namespace flint

// ----------------------------------------------------------------- decode host side

namespace flint {

static DecWs dec_ws(void* workspace, const DecLayout& L) {
  char* base = static_cast<char*>(workspace);
  DecWs ws;
  ws.hdr = reinterpret_cast<int*>(base + L.hdr);
  ws.q = reinterpret_cast<uint16_t*>(base + L.q);
  ws.ml = reinterpret_cast<float*>(base + L.ml);
  ws.part = reinterpret_cast<float*>(base + L.part);
  ws.nsplit = L.nsplit;
  ws.bps = kDecMaxSplitBlocks;
  return ws;
}

// Host checks shared by the decode entry points.
static int dec_check(int32_t batch, int32_t cache_cap, int32_t num_kv_heads, int32_t head_dim,
                     int32_t window, int32_t use_rope, float rope_theta, float eps,
                     const void* k_cache, const void* vt_cache, const void* workspace,
                     size_t workspace_bytes, const void* cache_len) {
  if (batch < 1 || cache_cap <= 0 || cache_cap % kDecBlock) return FLINT_ERR_SHAPE;
  if (num_kv_heads != kG || head_dim != kD) return FLINT_ERR_UNSUPPORTED;
  if (window < 0 || !(eps > 0.f) || !isfinite(eps)) return FLINT_ERR_VALUE;
  if (use_rope && (!(rope_theta > 0.f) || !isfinite(rope_theta))) return FLINT_ERR_VALUE;
  if (window > 0 && cache_cap < window) return FLINT_ERR_SHAPE;
  if (!k_cache || !vt_cache || !cache_len) return FLINT_ERR_NULL;
  if (!workspace) return FLINT_ERR_WORKSPACE;
  if (!aligned(k_cache, 16) || !aligned(vt_cache, 16) || !aligned(workspace, 256) ||
      !aligned(cache_len, 4))
    return FLINT_ERR_ALIGN;
  if (workspace_bytes < make_dec_layout(batch, cache_cap).total) return FLINT_ERR_WORKSPACE;
  return FLINT_OK;
}

}  // namespace flint

using namespace flint;

extern "C" size_t flint_attn_decode_workspace_bytes(int32_t batch, int32_t cache_cap) {
  if (batch < 1 || cache_cap <= 0) return 0;
  return make_dec_layout(batch, cache_cap).total;
}

extern "C" int flint_attn_kv_append(const void* k, const void* v, const float* k_norm_w,
                                    const int32_t* positions, const int32_t* cache_len,
                                    int32_t batch, int32_t n_new, void* k_cache, void* vt_cache,
                                    int32_t cache_cap, int32_t num_kv_heads, int32_t head_dim,
                                    int32_t window, int32_t use_rope, float rope_theta, float eps,
                                    void* workspace, size_t workspace_bytes, void* stream) {
  int st0 = dec_check(batch, cache_cap, num_kv_heads, head_dim, window, use_rope, rope_theta, eps,
                      k_cache, vt_cache, workspace, workspace_bytes, cache_len);
  if (st0 != FLINT_OK) return st0;
  if (n_new < 1 || (window > 0 && n_new > cache_cap)) return FLINT_ERR_SHAPE;
  if (!k || !v || !k_norm_w) return FLINT_ERR_NULL;
  if (!aligned(k, 16) || !aligned(v, 16) || !aligned(k_norm_w, 4) ||
      (positions && !aligned(positions, 4)))
    return FLINT_ERR_ALIGN;
  const DecWs ws = dec_ws(workspace, make_dec_layout(batch, cache_cap));
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const int rope = use_rope ? 1 : 0;
  (void)hipGetLastError();
  decode_append_kernel<<<dim3((unsigned)n_new, kG, (unsigned)batch), 64, 0, st>>>(
      nullptr, static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), nullptr, k_norm_w,
      rope ? positions : nullptr, cache_len, n_new, cache_cap, window, rope, (double)rope_theta, eps,
      static_cast<uint16_t*>(k_cache), static_cast<uint16_t*>(vt_cache), ws);
  if (hipGetLastError() != hipSuccess) return FLINT_ERR_HIP;
  if (debug_sync()) {
    int32_t flags = 0;
    return flint_attn_device_status(workspace, stream, &flags);
  }
  return FLINT_OK;
}

extern "C" int flint_attn_decode(const void* q, const void* k, const void* v, const float* q_norm_w,
                                 const float* k_norm_w, const float* sink, const int32_t* positions,
                                 const int32_t* cache_len, int32_t batch, void* k_cache,
                                 void* vt_cache, int32_t cache_cap, int32_t num_q_heads,
                                 int32_t num_kv_heads, int32_t head_dim, int32_t window,
                                 int32_t use_rope, float rope_theta, float eps, void* workspace,
                                 size_t workspace_bytes, void* out, void* stream) {
  if (num_q_heads != kH) return FLINT_ERR_UNSUPPORTED;
  int st0 = dec_check(batch, cache_cap, num_kv_heads, head_dim, window, use_rope, rope_theta, eps,
                      k_cache, vt_cache, workspace, workspace_bytes, cache_len);
  if (st0 != FLINT_OK) return st0;
  if (!q || !k || !v || !q_norm_w || !k_norm_w || !sink || !out) return FLINT_ERR_NULL;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) ||
      !aligned(q_norm_w, 4) || !aligned(k_norm_w, 4) || !aligned(sink, 4) ||
      (positions && !aligned(positions, 4)))
    return FLINT_ERR_ALIGN;
  const DecLayout L = make_dec_layout(batch, cache_cap);
  DecWs ws = dec_ws(workspace, L);
  // Split size: the largest that still gives about 2048 waves (2 per SIMD,
  // the occupancy of the attention kernel) over the cache's blocks, at least
  // kDecMinSplitBlocks; larger splits leave less for the merge.
  const int64_t blocks = (int64_t)batch * kG * (cache_cap / kDecBlock + 1);
  int bps = kDecMaxSplitBlocks;
  while (bps > kDecMinSplitBlocks && blocks / bps < 2048) bps /= 2;
  ws.bps = bps;
  const int nsplit = (int)((cache_cap / kDecBlock + 1 + bps - 1) / bps);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const int rope = use_rope ? 1 : 0;
  const uint16_t* kc = static_cast<const uint16_t*>(k_cache);
  const uint16_t* vc = static_cast<const uint16_t*>(vt_cache);
  (void)hipGetLastError();
  const int cblocks = cache_cap / kDecBlock;
  if (cblocks <= kDecFusedMaxBlocks ||
      (cblocks <= kDecFusedMaxBlocksWide && (int64_t)batch * kG >= kDecFusedWideGroups)) {
    // the whole step in one launch
    decode_fused_kernel<<<dim3(kG, (unsigned)batch), 64 * kDecFusedWaves, 0, st>>>(
        static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v),
        q_norm_w, k_norm_w, sink, rope ? positions : nullptr, cache_len, cache_cap, window, rope,
        (double)rope_theta, eps, static_cast<uint16_t*>(k_cache), static_cast<uint16_t*>(vt_cache), ws,
        static_cast<uint16_t*>(out));
    if (hipGetLastError() != hipSuccess) return FLINT_ERR_HIP;
    if (debug_sync()) {
      int32_t flags = 0;
      return flint_attn_device_status(workspace, stream, &flags);
    }
    return FLINT_OK;
  }
  decode_append_kernel<<<dim3(1, kG, (unsigned)batch), 64 * (1 + kHpg), 0, st>>>(
      static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v),
      q_norm_w, k_norm_w, rope ? positions : nullptr, cache_len, 1, cache_cap, window, rope,
      (double)rope_theta, eps, static_cast<uint16_t*>(k_cache), static_cast<uint16_t*>(vt_cache), ws);
  decode_attn_kernel<<<dim3((unsigned)nsplit, kG, (unsigned)batch), 64, 0, st>>>(cache_len, cache_cap,
                                                                                 window, kc, vc, ws);
  decode_merge_kernel<<<dim3(kH, (unsigned)batch), 256, 0, st>>>(cache_len, cache_cap, window, sink,
                                                                  ws, static_cast<uint16_t*>(out));
  if (hipGetLastError() != hipSuccess) return FLINT_ERR_HIP;
  if (debug_sync()) {
    int32_t flags = 0;
    return flint_attn_device_status(workspace, stream, &flags);
  }
  return FLINT_OK;
}

