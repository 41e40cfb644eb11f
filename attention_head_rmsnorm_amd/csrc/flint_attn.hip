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
// Three kernels run in order on the caller's stream:
//   schedule_kernel   one workgroup; checks cu_seqlens/seqused, lays out the
//                     64-token key tiles of every sequence and the 32-token
//                     query blocks, and orders the blocks by decreasing work.
//   kv_prologue_kernel  per (key tile, kv head): RMSNorm + RoPE of K in FP32,
//                     one bf16 rounding, stored as an MFMA-ready swizzled tile;
//                     V transposed and key-permuted into the PV operand order;
//                     zeros for padded keys; zero rows of `out` for padded
//                     queries.
//   attn_kernel       per (query block, kv head): 8 waves, one per query head
//                     of the group, share each K/V tile, which arrives in a
//                     3-stage LDS ring by direct global->LDS loads. The query
//                     prologue (RMSNorm, RoPE, softmax scale in log2 units,
//                     bf16) is fused in. S^T = K Q^T and O^T += V^T P^T run on
//                     v_mfma_f32_32x32x16_bf16 with FP32 accumulation, over
//                     the tiles inside the causal window only.
//
// Softmax shift. The QK RMSNorm bounds every logit: by Cauchy-Schwarz
// |s| = |q'.k'| <= |q'| max|k'| = B for the rounded operands the MFMA
// multiplies (s in log2 units). A wave whose rows all have B <= kStaticBound
// needs no shift at all: P = exp2(s) stays within [2^-B, 2^B], far from FP32
// and bf16 overflow and underflow, the sink adds exp2(sink) to the
// denominator, and O = sum P v / l is the same ratio as with any shift. The
// MFMA accumulators start at zero and P = exp2(acc) needs no running max, no
// per-tile max reduction and no rescaling. Waves with a larger bound take the
// streaming path: a running max that starts at the sink (m = sink, l = 1),
// subtracted before exp2 and raised lazily with rescaling.

#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include "flint_attn.h"

namespace flint {

constexpr int kH = 32;        // query heads
constexpr int kG = 4;         // key/value heads
constexpr int kD = 128;       // head dimension
constexpr int kHpg = kH / kG; // query heads per key/value head
constexpr int kBM = 32;       // query tokens per work item
constexpr int kBN = 64;       // keys per tile
constexpr int kHalfTile = kBN * kD * 2;     // bytes of one K' tile or one V^T tile
constexpr int kTileBytes = 2 * kHalfTile;   // K' tile followed by V^T tile
constexpr int kTileVec = kTileBytes / 16;   // 16-byte vectors per tile
constexpr int kBuckets = 4096;              // cost buckets of the schedule sort
constexpr int kAttnThreads = 64 * kHpg;     // one wave per query head of a group
constexpr float kLog2e = 1.4426950408889634f;
// Keep a stale running max until a tile's max exceeds it by this much (log2
// units): exp2 values then stay below 2^8, and the final O / l is unchanged.
constexpr float kRescaleSlack = 8.0f;
// Largest logit bound (log2 units) that takes the unshifted path: P <= 2^56
// and l <= 2^56 * 2^18 keys leave FP32 headroom for |v| up to ~2^50.
constexpr float kStaticBound = 56.0f;
constexpr int kStages = 4;  // LDS ring depth of the attention kernel

typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef float f32x16 __attribute__((__vector_size__(16 * sizeof(float))));
typedef __bf16 bf16x2_t __attribute__((__vector_size__(2 * sizeof(__bf16))));

struct Ws {
  int* hdr;       // [0] device-data error bits, [1] key tiles, [2] query blocks
  unsigned long long* rope_r;  // [64] theta^(-c/64) / (2 pi) as a 0.64 fixed-point fraction
  int4* seq;      // [n] {start, length, valid length, first tile}
  float* tmax;    // [kG][ntmax] max |k'| over the keys of each tile
  int* tbase;     // [n+1] first key tile of each sequence
  int* qbase;     // [n+1] first query block of each sequence
  int2* tiles;    // [ntmax] {sequence, tile in sequence}
  int2* items;    // [nqmax] {sequence, query block}, most work first
  char* kv;       // [kG][ntmax][kTileBytes]
  int ntmax;
};

struct Layout {
  size_t hdr, rope_r, seq, tmax, tbase, qbase, tiles, items, kv, total;
  int64_t ntmax, nqmax;
};

static inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

static Layout make_layout(int64_t T, int64_t n) {
  Layout L;
  L.ntmax = (T + kBN - 1) / kBN + n;
  L.nqmax = (T + kBM - 1) / kBM + n;
  size_t o = 0;
  L.hdr = o;   o = align_up(o + 64 * sizeof(int), 256);
  L.rope_r = o; o = align_up(o + 64 * sizeof(unsigned long long), 256);
  L.seq = o;   o = align_up(o + (size_t)n * sizeof(int4), 256);
  L.tmax = o;  o = align_up(o + (size_t)kG * L.ntmax * sizeof(float), 256);
  L.tbase = o; o = align_up(o + (size_t)(n + 1) * sizeof(int), 256);
  L.qbase = o; o = align_up(o + (size_t)(n + 1) * sizeof(int), 256);
  L.tiles = o; o = align_up(o + (size_t)L.ntmax * sizeof(int2), 256);
  L.items = o; o = align_up(o + (size_t)L.nqmax * sizeof(int2), 256);
  L.kv = o;    o = align_up(o + (size_t)kG * (size_t)L.ntmax * kTileBytes, 256);
  L.total = o;
  return L;
}

// ----------------------------------------------------------------- helpers

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ void unpack8(const uint4& c, float* x) {
  x[0] = bf16_lo(c.x); x[1] = bf16_hi(c.x);
  x[2] = bf16_lo(c.y); x[3] = bf16_hi(c.y);
  x[4] = bf16_lo(c.z); x[5] = bf16_hi(c.z);
  x[6] = bf16_lo(c.w); x[7] = bf16_hi(c.w);
}

// Round to bf16 (nearest even) and pack two values into one word.
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  typedef __bf16 bf16x2 __attribute__((__vector_size__(2 * sizeof(__bf16))));
  bf16x2 p = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, p);
}

__device__ __forceinline__ uint4 pack8(const float* x) {
  return make_uint4(pack2(x[0], x[1]), pack2(x[2], x[3]), pack2(x[4], x[5]), pack2(x[6], x[7]));
}

// cos and sin of the RoPE angle pos * omega_c. The angle in revolutions,
// pos * omega_c / (2 pi), is reduced exactly: with R = omega_c / (2 pi) as a
// 0.64 fixed-point fraction, pos * R mod 2^64 is the fractional revolution,
// whose top 32 bits (as a signed value in [-1/2, 1/2)) feed the hardware
// sine and cosine, which take revolutions and are accurate to ~1.3e-7.
__device__ __forceinline__ void rope_cos_sin(int pos, unsigned long long r, float* c, float* s) {
  const unsigned long long prod = (unsigned long long)(long long)pos * r;
  const float rev = (float)(int)(unsigned)(prod >> 32) * 2.3283064365386963e-10f;  // 2^-32
  *s = __builtin_amdgcn_sinf(rev);
  *c = __builtin_amdgcn_cosf(rev);
}

// acc + sum of the eight packed bf16 values in c (v_dot2 with (1, 1)).
__device__ __forceinline__ float dot2_sum(const uint4& c, bf16x2_t ones, float acc) {
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, c.x), ones, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, c.y), ones, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, c.z), ones, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, c.w), ones, acc, false);
  return acc;
}

// Sum of squares of eight packed bf16 values.
__device__ __forceinline__ float sumsq8(const uint4& c) {
  float x[8];
  unpack8(c, x);
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) s += x[i] * x[i];
  return s;
}

// Tile layout (workspace and LDS alike), in 16-byte vectors, "fragment
// order": every MFMA operand fragment of the attention kernel is one run of
// 64 vectors, vector `lane` being what MFMA lane `lane` = 32 half + col
// supplies, so each operand read is one contiguous, conflict-free 1 KiB.
//   K' part  [2 key blocks b][8 channel steps kk][64 lanes]:
//            K'[32b + col][16kk + 8half .. +8)
//   V^T part [4 channel blocks db][4 key steps kk][64 lanes]:
//            V^T[32db + col][slots 16kk + 8half .. +8), slot s holding key vt_slot(s)
__device__ __forceinline__ int frag_index(int blk, int steps, int kk, int half, int col) {
  return (blk * steps + kk) * 64 + half * 32 + col;
}

// Swizzle of the 32-row x 256-byte output staging area (16-byte chunks).
__device__ __forceinline__ int o_swizzle(int r) { return (r & 15) ^ ((r >> 4) & 1); }

// Exclusive scan over the 1024 threads of a block; *total gets the sum.
// Wave-level shuffle scans, then a scan of the 16 wave totals.
__device__ int block_excl_scan(int v, int* tmp, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == 63) tmp[wave] = x;
  __syncthreads();
  if (wave == 0) {
    int w = lane < 16 ? tmp[lane] : 0;
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) {
      const int y = __shfl_up(w, off);
      if (lane >= off) w += y;
    }
    if (lane < 16) tmp[lane] = w;
  }
  __syncthreads();
  const int base = wave > 0 ? tmp[wave - 1] : 0;
  *total = tmp[15];
  __syncthreads();
  return base + x - v;
}

// Largest s in [0, n) with base[s] <= e (base non-decreasing, base[0] = 0).
__device__ __forceinline__ int find_seq(const int* base, int n, int e) {
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (base[mid] <= e) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Key range of query block qb: [lo, hi) in sequence positions.
__device__ __forceinline__ void block_keys(int u, int qb, int window, int* lo, int* hi) {
  const int t0 = qb * kBM;
  *hi = min(t0 + kBM, u);
  *lo = window > 0 ? max(0, t0 - (window - 1)) : 0;
}

__device__ __forceinline__ int block_cost(int u, int qb, int window) {
  int lo, hi;
  block_keys(u, qb, window, &lo, &hi);
  return ((hi + kBN - 1) / kBN) - lo / kBN;
}

// ----------------------------------------------------------------- schedule

__global__ __launch_bounds__(1024) void schedule_kernel(const int* __restrict__ cu,
                                                        const int* __restrict__ seqused, int n,
                                                        int T, int max_seqlen, int window,
                                                        double theta, Ws ws) {
  __shared__ int tmp[1024];
  __shared__ int hist[kBuckets];
  __shared__ int sflags;
  const int tid = threadIdx.x;
  if (tid == 0) sflags = 0;
  if (tid < 64) {
    // theta^(-c/64) / (2 pi) < 1/(2 pi): scaled by 2^64 it fits an unsigned 64-bit integer
    const double r = pow(theta, -(double)tid / 64.0) * 0.15915494309189533577;
    ws.rope_r[tid] = (unsigned long long)(r * 18446744073709551616.0);
  }
  __syncthreads();

  int flags = 0;
  int carry_t = 0, carry_q = 0;
  for (int base = 0; base < n; base += 1024) {
    const int s = base + tid;
    int nt = 0, nq = 0, a = 0, len = 0, u = 0;
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
    }
    int tot_t, tot_q;
    const int ex_t = block_excl_scan(nt, tmp, &tot_t);
    const int ex_q = block_excl_scan(nq, tmp, &tot_q);
    if (s < n) {
      ws.seq[s] = make_int4(a, len, u, carry_t + ex_t);
      ws.tbase[s] = carry_t + ex_t;
      ws.qbase[s] = carry_q + ex_q;
    }
    carry_t += tot_t;
    carry_q += tot_q;
  }
  if (flags) atomicOr(&sflags, flags);
  __syncthreads();
  const int f = sflags;
  if (f) {  // invalid device data: schedule nothing
    if (tid == 0) {
      ws.hdr[0] = f;
      ws.hdr[1] = 0;
      ws.hdr[2] = 0;
    }
    return;
  }
  if (tid == 0) {
    ws.tbase[n] = carry_t;
    ws.qbase[n] = carry_q;
  }
  const int NT = carry_t, NQ = carry_q;
  for (int i = tid; i < kBuckets; i += 1024) hist[i] = 0;
  __syncthreads();

  for (int e = tid; e < NT; e += 1024) {
    const int s = find_seq(ws.tbase, n, e);
    ws.tiles[e] = make_int2(s, e - ws.tbase[s]);
  }
  for (int e = tid; e < NQ; e += 1024) {
    const int s = find_seq(ws.qbase, n, e);
    const int c = min(block_cost(ws.seq[s].z, e - ws.qbase[s], window), kBuckets - 1);
    atomicAdd(&hist[c], 1);
  }
  __syncthreads();
  // bucket starts in order of decreasing cost; thread tid owns 4 buckets
  int local[4], sum = 0;
  for (int j = 0; j < 4; ++j) {
    local[j] = hist[kBuckets - 1 - (4 * tid + j)];
    sum += local[j];
  }
  int tot;
  int run = block_excl_scan(sum, tmp, &tot);
  for (int j = 0; j < 4; ++j) {
    hist[kBuckets - 1 - (4 * tid + j)] = run;
    run += local[j];
  }
  __syncthreads();
  for (int e = tid; e < NQ; e += 1024) {
    const int s = find_seq(ws.qbase, n, e);
    const int qb = e - ws.qbase[s];
    const int c = min(block_cost(ws.seq[s].z, qb, window), kBuckets - 1);
    const int pos = atomicAdd(&hist[c], 1);
    ws.items[pos] = make_int2(s, qb);
  }
  if (tid == 0) {
    ws.hdr[0] = 0;
    ws.hdr[1] = NT;
    ws.hdr[2] = NQ;
  }
}

// ----------------------------------------------------------------- K/V prologue

// Slot of key r (0..63) inside a V^T row: bits 2 and 3 swapped, which is the
// order in which the softmax output P^T sits in the MFMA B operand.
__device__ __forceinline__ int vt_slot(int r) { return r ^ ((((r >> 2) ^ (r >> 3)) & 1) * 12); }

__global__ __launch_bounds__(256) void kv_prologue_kernel(const uint16_t* __restrict__ k,
                                                          const uint16_t* __restrict__ v,
                                                          const float* __restrict__ k_norm_w,
                                                          const int* __restrict__ positions,
                                                          float eps, int use_rope, Ws ws,
                                                          uint16_t* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) uint16_t vt[kD * kBN];
  __shared__ float red[4];
  const int e = blockIdx.x, g = blockIdx.y;
  if (e >= ws.hdr[1]) return;
  const int2 te = ws.tiles[e];
  const int4 meta = ws.seq[te.x];
  const int start = meta.x, len = meta.y, u = meta.z;
  const int tid = threadIdx.x, r = tid >> 2, p = tid & 3;
  const int ell = te.y * kBN + r;
  const bool valid = ell < u;
  const size_t t = (size_t)start + ell;
  char* tile = ws.kv + ((size_t)g * ws.ntmax + meta.w + te.y) * kTileBytes;

  // K: this thread owns channels [16p, 16p+16) and their RoPE partners +64.
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
      rope_cos_sin(pos, ws.rope_r[16 * p + i], &c, &s);
      const float a = x[i], b = x[16 + i];
      x[i] = a * c - b * s;
      x[16 + i] = b * c + a * s;
    }
  }
  {
    uint4* kfrag = reinterpret_cast<uint4*>(tile);
    const int b = r >> 5, col = r & 31;
    const uint4 w0 = pack8(x), w1 = pack8(x + 8), w2 = pack8(x + 16), w3 = pack8(x + 24);
    kfrag[frag_index(b, 8, p, 0, col)] = w0;      // channels 16p .. 16p+7
    kfrag[frag_index(b, 8, p, 1, col)] = w1;      // 16p+8 .. 16p+15
    kfrag[frag_index(b, 8, 4 + p, 0, col)] = w2;  // 64+16p .. 64+16p+7
    kfrag[frag_index(b, 8, 4 + p, 1, col)] = w3;  // 64+16p+8 .. 64+16p+15
    // |k'| of the rounded key, for the logit bound of the attention kernel
    float n2 = sumsq8(w0) + sumsq8(w1) + sumsq8(w2) + sumsq8(w3);
    n2 += __shfl_xor(n2, 1);
    n2 += __shfl_xor(n2, 2);
    // tile max of |k'|: wave max, then across the four waves
    float kn = sqrtf(n2);
#pragma unroll
    for (int off = 4; off < 64; off <<= 1) kn = fmaxf(kn, __shfl_xor(kn, off));
    if ((tid & 63) == 0) red[tid >> 6] = kn;
  }

  // V: transpose through LDS; this thread owns channels [32p, 32p+32) of key r.
  {
    uint4 c4[4];
    if (valid) {
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
  if (tid == 0)
    ws.tmax[(size_t)g * ws.ntmax + meta.w + te.y] = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
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

  // Padded query rows of this kv head's 8 query heads are exact zeros.
  if (ell >= u && ell < len) {
    uint4* dst = reinterpret_cast<uint4*>(out + (t * kH + (size_t)g * kHpg) * kD);
    const uint4 z = make_uint4(0, 0, 0, 0);
#pragma unroll 4
    for (int i = 0; i < 32; ++i) dst[p * 32 + i] = z;
  }
}

// ----------------------------------------------------------------- attention

// Direct global->LDS copy of one 32 KiB tile into an LDS stage: each of the
// 512 threads moves four 16-byte vectors; global_load_lds writes lane L's
// vector at the wave-uniform LDS base (M0) + 16 L, so the tile lands in LDS
// with the byte order it has in the workspace. `src` and `stage` are uniform
// and `wave` is a scalar, so the addresses are a scalar base plus a constant
// per-lane offset.
__device__ __forceinline__ void load_tile_async(const char* src, uint4* stage, int lane, int wave) {
#pragma unroll
  for (int i = 0; i < kTileVec / kAttnThreads; ++i) {
    const int v0 = i * kAttnThreads + wave * 64;
    __builtin_amdgcn_global_load_lds(
        reinterpret_cast<const uint4*>(src + (size_t)v0 * 16) + lane,
        (__attribute__((address_space(3))) void*)(stage + v0), 16, 0, 0);
  }
}

// Workgroup barrier for the tile ring. Each wave first waits until at most
// one tile of its direct-to-LDS loads (4 per thread) is still in flight, or
// none, and its LDS reads are done. Unlike __syncthreads() it does not wait
// for the newest tile's loads.
__device__ __forceinline__ void ring_barrier(bool keep_one_tile) {
  if (keep_one_tile) asm volatile("s_waitcnt vmcnt(4) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  else asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

struct RowState {
  f32x16 acc[4];  // O^T accumulators: channels 32db + ..., query col
  float m;        // streaming path: running max (log2 units), may be -INF
  float l0, l1;   // partial denominators (this lane's keys)
  bool online;    // streaming path for this wave
};

// S^T for the 64 keys of a tile: two 32x32 logit blocks, accumulators from
// zero. Operand fragments are read four MFMAs ahead of their use. When
// `lsrc` is set, this wave's four direct-to-LDS loads of a later tile (into
// `lstage`) are spread over the MFMAs, one after every fourth, so the loads
// of all waves do not reach the texture unit in one burst.
__device__ __forceinline__ void tile_logits(const uint4* kt, int lane, const bf16x8* qf,
                                            f32x16& s0, f32x16& s1, const char* lsrc, uint4* lstage, int wave) {
  bf16x8 f[16];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    f[i] = __builtin_bit_cast(bf16x8, kt[((i & 1) * 8 + (i >> 1)) * 64 + lane]);
  __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);  // the first four reads
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    if (i + 4 < 16) {
      const int j = i + 4;
      f[j] = __builtin_bit_cast(bf16x8, kt[((j & 1) * 8 + (j >> 1)) * 64 + lane]);
    }
    const int kk = i >> 1;
    if (i & 1) {
      s1 = kk == 0 ? __builtin_amdgcn_mfma_f32_32x32x16_bf16(f[i], qf[kk], f32x16{}, 0, 0, 0)
                   : __builtin_amdgcn_mfma_f32_32x32x16_bf16(f[i], qf[kk], s1, 0, 0, 0);
    } else {
      s0 = kk == 0 ? __builtin_amdgcn_mfma_f32_32x32x16_bf16(f[i], qf[kk], f32x16{}, 0, 0, 0)
                   : __builtin_amdgcn_mfma_f32_32x32x16_bf16(f[i], qf[kk], s0, 0, 0, 0);
    }
    if (i + 4 < 16) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // the next read
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                  // this MFMA
    if ((i & 3) == 3 && lsrc) {
      const int v0 = (i >> 2) * kAttnThreads + wave * 64;
      __builtin_amdgcn_global_load_lds(
          reinterpret_cast<const uint4*>(lsrc + (size_t)v0 * 16) + lane,
          (__attribute__((address_space(3))) void*)(lstage + v0), 16, 0, 0);
    }
  }
}

// Mask, (streaming path) running max, and P = exp2(S - m) as the bf16 B
// operand of the PV product; the denominators sum the same rounded values.
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
  const bf16x2_t ones = __builtin_bit_cast(bf16x2_t, 0x3f803f80u);
  float p[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) p[i] = __builtin_amdgcn_exp2f(s0[i]);
  const uint4 w0 = pack8(p), w1 = pack8(p + 8);
#pragma unroll
  for (int i = 0; i < 16; ++i) p[i] = __builtin_amdgcn_exp2f(s1[i]);
  const uint4 w2 = pack8(p), w3 = pack8(p + 8);
  pk[0] = __builtin_bit_cast(bf16x8, w0);
  pk[1] = __builtin_bit_cast(bf16x8, w1);
  pk[2] = __builtin_bit_cast(bf16x8, w2);
  pk[3] = __builtin_bit_cast(bf16x8, w3);
  st.l0 = dot2_sum(w0, ones, st.l0);
  st.l1 = dot2_sum(w1, ones, st.l1);
  st.l0 = dot2_sum(w2, ones, st.l0);
  st.l1 = dot2_sum(w3, ones, st.l1);
}

// O^T[d, query] += V^T[d, keys] P^T[keys, query]; fragments read four
// MFMAs ahead.
__device__ __forceinline__ void tile_pv(const uint4* vt, int lane, const bf16x8* pk, RowState& st) {
  bf16x8 f[16];
#pragma unroll
  for (int i = 0; i < 4; ++i) f[i] = __builtin_bit_cast(bf16x8, vt[i * 64 + lane]);
  __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    if (i + 4 < 16) f[i + 4] = __builtin_bit_cast(bf16x8, vt[(i + 4) * 64 + lane]);
    const int db = i >> 2, kk = i & 3;
    st.acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f[i], pk[kk], st.acc[db], 0, 0, 0);
    if (i + 4 < 16) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
  }
}

// One work item = 32 query tokens x the 8 query heads of one kv head. The 8
// waves (one per head) run in two groups, waves 0-3 (A) and 4-7 (B); the
// hardware places waves w and w+4 on the same SIMD. Group B runs half a
// tile behind group A, so on each SIMD one wave feeds the matrix cores while
// the other runs its softmax. Tile k+2 streams into the 4-stage LDS ring
// meanwhile.
__global__ __launch_bounds__(kAttnThreads) void attn_kernel(const uint16_t* __restrict__ q,
                                                            const float* __restrict__ q_norm_w,
                                                            const float* __restrict__ sink,
                                                            const int* __restrict__ positions,
                                                            int window, int use_rope, float eps,
                                                            Ws ws, uint16_t* __restrict__ out) {
  __shared__ uint4 smem[kStages][kTileVec];
  const int g = blockIdx.x & (kG - 1);
  const int e = blockIdx.x / kG;
  if (e >= ws.hdr[2]) return;
  const int2 item = ws.items[e];
  const int4 meta = ws.seq[item.x];
  const int start = meta.x, u = meta.z;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave
  const int col = lane & 31, half = lane >> 5;
  const int h = g * kHpg + wave;
  const bool group_b = wave >= 4;
  const int t0 = item.y * kBM;
  int klo, khi;
  block_keys(u, item.y, window, &klo, &khi);
  const int tile_lo = klo / kBN;
  const int ntiles = (khi + kBN - 1) / kBN - tile_lo;
  const char* kvbase = ws.kv + ((size_t)g * ws.ntmax + meta.w + tile_lo) * kTileBytes;

  load_tile_async(kvbase, smem[0], lane, wave);
  if (ntiles > 1) load_tile_async(kvbase + kTileBytes, smem[1], lane, wave);

  // Query prologue: lane (col, half) holds channels 16kk + 8half + [0,8) of
  // token t0 + col, which is the MFMA B-operand layout of Q^T.
  const int qrow = t0 + col;
  const bool qvalid = qrow < u;
  const size_t tq = (size_t)start + qrow;
  bf16x8 qf[8];
  float qnorm;
  {
    float x[64];
    if (qvalid) {
      const uint4* src = reinterpret_cast<const uint4*>(q + (tq * kH + h) * kD);
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) unpack8(src[2 * kk + half], x + 8 * kk);
    } else {
#pragma unroll
      for (int i = 0; i < 64; ++i) x[i] = 0.f;
    }
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < 64; ++i) ss += x[i] * x[i];
    ss += __shfl_xor(ss, 32);
    const float rstd = 1.0f / sqrtf(ss * (1.0f / kD) + eps);
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
#pragma unroll
      for (int j = 0; j < 8; ++j) x[8 * kk + j] *= rstd * q_norm_w[16 * kk + 8 * half + j];
    if (use_rope && qvalid) {
      const int pos = positions ? positions[tq] : qrow;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          float c, s;
          rope_cos_sin(pos, ws.rope_r[16 * kk + 8 * half + j], &c, &s);
          const float a = x[8 * kk + j], b = x[8 * (kk + 4) + j];
          x[8 * kk + j] = a * c - b * s;
          x[8 * (kk + 4) + j] = b * c + a * s;
        }
    }
    // logits in log2 units: q . k / sqrt(128) * log2(e)
    const float scale = kLog2e * 0.08838834764831845f;
    float n2 = 0.f;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
#pragma unroll
      for (int j = 0; j < 8; ++j) x[8 * kk + j] *= scale;
      const uint4 w = pack8(x + 8 * kk);
      n2 += sumsq8(w);
      qf[kk] = __builtin_bit_cast(bf16x8, w);
    }
    n2 += __shfl_xor(n2, 32);
    qnorm = sqrtf(n2);
  }

  // max |k'| over the tiles this item visits (a block-wide max)
  __shared__ float kred[kAttnThreads / 64];
  {
    const float* tm = ws.tmax + (size_t)g * ws.ntmax + meta.w + tile_lo;
    float km = 0.f;
    for (int i = tid; i < ntiles; i += kAttnThreads) km = fmaxf(km, tm[i]);
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) km = fmaxf(km, __shfl_xor(km, off));
    if (lane == 0) kred[wave] = km;
  }
  __syncthreads();
  float kmax = kred[0];
#pragma unroll
  for (int w = 1; w < kAttnThreads / 64; ++w) kmax = fmaxf(kmax, kred[w]);

  // Softmax shift (see the file header): none when the logit bound allows.
  RowState st;
  {
    const float sk = sink[h] * kLog2e;
    const float bound = qnorm * kmax * 1.0001f;
    st.online = __any(!(bound <= kStaticBound));
    // the sink's share of the denominator, counted once per query (lane half 0)
    st.m = st.online ? sk : 0.f;
    st.l0 = (half == 0 && sk != -INFINITY) ? __builtin_amdgcn_exp2f(sk - st.m) : 0.f;
    st.l1 = 0.f;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) st.acc[db][i] = 0.f;
  }

  // Both groups run the same pipelined body - softmax and PV of tile k-1,
  // then the logits of tile k - but group A passes the ring barrier just
  // before the logits and group B at the top of the body. Between barriers k
  // and k+1 group A therefore computes logits, softmax and PV of tile k while
  // group B computes softmax and PV of tile k-1 and the logits of tile k.
  f32x16 s0, s1;
  bf16x8 pk[4];
  for (int k = 0; k < ntiles; ++k) {
    if (group_b) ring_barrier(k + 1 < ntiles);
    if (k > 0) {
      tile_softmax(s0, s1, st, pk, (tile_lo + k - 1) * kBN, t0, qrow, u, window, half);
      tile_pv(smem[(k - 1) % kStages] + kTileVec / 2, lane, pk, st);
    }
    if (!group_b) ring_barrier(k + 1 < ntiles);  // tile k is in LDS; stage (k+2)%4 is free
    tile_logits(smem[k % kStages], lane, qf, s0, s1,
                k + 2 < ntiles ? kvbase + (size_t)(k + 2) * kTileBytes : nullptr,
                smem[(k + 2) % kStages], wave);
  }
  tile_softmax(s0, s1, st, pk, (tile_lo + ntiles - 1) * kBN, t0, qrow, u, window, half);
  tile_pv(smem[(ntiles - 1) % kStages] + kTileVec / 2, lane, pk, st);
  __syncthreads();

  // Epilogue: O = acc / l, staged through LDS so each token row (256 bytes of
  // one head) leaves in full 16-byte vectors.
  const float lsum = st.l0 + st.l1;
  const float lt = lsum + __shfl_xor(lsum, 32);
  const float inv = lt > 0.f ? 1.0f / lt : 0.f;
  uint2* orow = reinterpret_cast<uint2*>(reinterpret_cast<char*>(&smem[0][0]) + wave * (kBM * kD * 2));
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      const int chunk = (4 * db + rg) ^ o_swizzle(col);
      const uint2 w = make_uint2(pack2(st.acc[db][4 * rg] * inv, st.acc[db][4 * rg + 1] * inv),
                                 pack2(st.acc[db][4 * rg + 2] * inv, st.acc[db][4 * rg + 3] * inv));
      orow[col * 32 + chunk * 2 + half] = w;
    }
  __syncthreads();
  const uint4* ostage = reinterpret_cast<const uint4*>(orow);
#pragma unroll
  for (int i = 0; i < kBM * 16 / 64; ++i) {
    const int idx = i * 64 + lane;
    const int r = idx >> 4, c = idx & 15;
    if (t0 + r < u) {
      const uint4 w = ostage[r * 16 + (c ^ o_swizzle(r))];
      reinterpret_cast<uint4*>(out + (((size_t)start + t0 + r) * kH + h) * kD)[c] = w;
    }
  }
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
      seqused[b] = s_cnt;
      if (s_cnt != s_first) ++s_bad;
    }
    __syncthreads();
  }
  if (tid == 0) *n_bad = s_bad;
}

}  // namespace flint

// ===================================================================== C ABI

using namespace flint;

static bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

extern "C" size_t flint_attn_workspace_bytes(int32_t total_tokens, int32_t n_seqs,
                                             int32_t max_seqlen, int32_t num_kv_heads,
                                             int32_t head_dim) {
  if (total_tokens < 0 || n_seqs < 0 || max_seqlen < 0) return 0;
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
    default: return "unknown flint_attn status";
  }
}

static bool debug_sync() {
  const char* e = getenv("FLINT_ATTN_DEBUG");
  return e && e[0] == '1';
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

extern "C" int flint_attn_fwd_phases(const void* q, const void* k, const void* v,
                                     const float* q_norm_w, const float* k_norm_w,
                                     const float* sink, const int32_t* positions,
                                     const int32_t* cu_seqlens, const int32_t* seqused,
                                     int32_t n_seqs, int32_t max_seqlen, int32_t total_tokens,
                                     int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                     int32_t window, int32_t use_rope, float rope_theta, float eps,
                                     void* workspace, size_t workspace_bytes, void* out,
                                     void* stream, int32_t phases) {
  if (phases <= 0 || (phases & ~FLINT_PHASE_ALL)) return FLINT_ERR_VALUE;
  if (total_tokens < 0 || n_seqs < 0 || max_seqlen < 0) return FLINT_ERR_SHAPE;
  if (num_q_heads != kH || num_kv_heads != kG || head_dim != kD) return FLINT_ERR_UNSUPPORTED;
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
      (seqused && !aligned(seqused, 4)))
    return FLINT_ERR_ALIGN;
  const Layout L = make_layout(total_tokens, n_seqs);
  if (workspace_bytes < L.total) return FLINT_ERR_WORKSPACE;

  char* base = static_cast<char*>(workspace);
  Ws ws;
  ws.hdr = reinterpret_cast<int*>(base + L.hdr);
  ws.rope_r = reinterpret_cast<unsigned long long*>(base + L.rope_r);
  ws.seq = reinterpret_cast<int4*>(base + L.seq);
  ws.tmax = reinterpret_cast<float*>(base + L.tmax);
  ws.tbase = reinterpret_cast<int*>(base + L.tbase);
  ws.qbase = reinterpret_cast<int*>(base + L.qbase);
  ws.tiles = reinterpret_cast<int2*>(base + L.tiles);
  ws.items = reinterpret_cast<int2*>(base + L.items);
  ws.kv = base + L.kv;
  ws.ntmax = (int)L.ntmax;

  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const uint16_t* qh = static_cast<const uint16_t*>(q);
  const uint16_t* kh = static_cast<const uint16_t*>(k);
  const uint16_t* vh = static_cast<const uint16_t*>(v);
  uint16_t* oh = static_cast<uint16_t*>(out);
  const int rope = use_rope ? 1 : 0;
  const int* pos = rope ? positions : nullptr;

  (void)hipGetLastError();
  if (phases & FLINT_PHASE_SCHEDULE)
    schedule_kernel<<<1, 1024, 0, st>>>(cu_seqlens, seqused, n_seqs, total_tokens, max_seqlen,
                                        window, (double)rope_theta, ws);
  if (phases & FLINT_PHASE_KV)
    kv_prologue_kernel<<<dim3((unsigned)L.ntmax, kG), 256, 0, st>>>(kh, vh, k_norm_w, pos, eps,
                                                                    rope, ws, oh);
  if (phases & FLINT_PHASE_ATTEND)
    attn_kernel<<<(unsigned)(L.nqmax * kG), kAttnThreads, 0, st>>>(qh, q_norm_w, sink, pos,
                                                                   window, rope, eps, ws, oh);
  if (hipGetLastError() != hipSuccess) return FLINT_ERR_HIP;
  if (debug_sync()) {
    int32_t flags = 0;
    return flint_attn_device_status(workspace, stream, &flags);
  }
  return FLINT_OK;
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
