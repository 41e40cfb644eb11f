// Shared definitions of the Flint attention kernels (forward, decode and
// backward): head layout constants, the workspace layout of the forward
// schedule, bf16 packing, RoPE angles, MFMA operand-fragment tile order and
// small block-wide helpers. Included by every HIP source of the library.
#pragma once

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
// softmax scale of the query rows in log2 units: log2(e) / sqrt(128)
constexpr float kQScale = kLog2e * 0.08838834764831845f;
constexpr float kLn2 = 0.6931471805599453f;
// Keep a stale running max until a tile's max exceeds it by this much (log2
// units): exp2 values then stay below 2^8, and the final O / l is unchanged.
constexpr float kRescaleSlack = 8.0f;
// Largest logit bound (log2 units) that takes the unshifted path: P <= 2^56
// and l <= 2^56 * 2^18 keys leave FP32 headroom for |v| up to ~2^50.
constexpr float kStaticBound = 56.0f;
constexpr int kStages = 4;  // LDS ring depth of the attention kernel
// Longest sequence the kernels take (FLINT_MAX_SEQLEN): a buffer resource
// covering one sequence's key tiles (32 KiB per 64 keys forward, 48 KiB
// backward) then stays within its 32-bit byte count.
constexpr int kMaxSeqLen = FLINT_MAX_SEQLEN;
constexpr int kFragAhead = 4;  // MFMA operand fragments read ahead of their use
// Word 3 of a raw (stride 0) buffer resource on gfx9-family GPUs: 32-bit
// data format, no swizzle, byte-granular range check against num_records.
constexpr int kBufferWord3 = 0x00020000;

typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef float f32x16 __attribute__((__vector_size__(16 * sizeof(float))));
typedef __bf16 bf16x2_t __attribute__((__vector_size__(2 * sizeof(__bf16))));

// RoPE frequency of channel pair c, omega_c / (2 pi) = theta^(-c/64) / (2 pi)
// revolutions per position, held twice: as a 0.64 fixed-point fraction `r`
// (an exact angle reduction for every int32 position) and as the unevaluated
// float sum hi + lo of the same value (~48 significant bits; a reduction in
// full-rate FP32 arithmetic for positions of magnitude below 2^24).
struct RopeFreq {
  unsigned long long r;
  float hi, lo;
};

struct Ws {
  int* hdr;       // [0] device-data error bits, [1] key tiles (packed layout), [2] query
                  // blocks, [3] 64-row units holding padded rows (forward layout)
  RopeFreq* rope;  // [64] RoPE frequencies (rope_freq)
  int4* seq;      // [n] {start, length, valid length, first tile}
  int* tbase;     // [n+1] first key tile of each sequence
  int* qbase;     // [n+1] first query block of each sequence
  int* pbase;     // [n+1] first padded 64-row unit of each sequence (forward layout)
  int2* tiles;    // [ntmax] {sequence, tile in sequence} (packed layout)
  int2* items;    // [nqmax] {sequence, query block}, most work first
  char* kv;       // [kG][ntmax][kTileBytes]
  int ntmax;
};

struct Layout {
  size_t hdr, rope, seq, tbase, qbase, pbase, tiles, items, kv, q16, total;
  int64_t ntmax, nqmax;
};

static inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Workspace regions of the forward; the key-tile region only `with_kv`, the
// fp16 query rows of the FP16 variant only `with_q16`.
static inline Layout make_layout(int64_t T, int64_t n, bool with_kv = true, bool with_q16 = false) {
  Layout L;
  L.ntmax = (T + kBN - 1) / kBN + n;
  L.nqmax = (T + kBM - 1) / kBM + n;
  size_t o = 0;
  L.hdr = o;   o = align_up(o + 64 * sizeof(int), 256);
  L.rope = o; o = align_up(o + 64 * sizeof(RopeFreq), 256);
  L.seq = o;   o = align_up(o + (size_t)n * sizeof(int4), 256);
  L.tbase = o; o = align_up(o + (size_t)(n + 1) * sizeof(int), 256);
  L.qbase = o; o = align_up(o + (size_t)(n + 1) * sizeof(int), 256);
  L.pbase = o; o = align_up(o + (size_t)(n + 1) * sizeof(int), 256);
  L.tiles = o; o = align_up(o + (size_t)L.ntmax * sizeof(int2), 256);
  L.items = o; o = align_up(o + (size_t)L.nqmax * sizeof(int2), 256);
  L.kv = o;
  if (with_kv) o = align_up(o + (size_t)kG * (size_t)L.ntmax * kTileBytes, 256);
  L.q16 = o;
  if (with_q16) o = align_up(o + (size_t)T * kH * kD * 2, 256);
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

__device__ __forceinline__ RopeFreq rope_freq(double theta, int c) {
  RopeFreq f;
  const double x = pow(theta, -(double)c / 64.0) * 0.15915494309189533577;
  f.r = (unsigned long long)(x * 18446744073709551616.0);
  const double R = (double)f.r * 5.421010862427522170e-20;  // r / 2^64
  f.hi = (float)R;
  f.lo = (float)(R - (double)f.hi);
  return f;
}

// |pos| < 2^24: the position is exact as a float.
constexpr int kRopeFastPos = 1 << 24;
__device__ __forceinline__ bool rope_pos_fast(int pos) {
  return (unsigned)pos + (unsigned)(kRopeFastPos - 1) < (unsigned)(2 * kRopeFastPos - 1);
}

// Fractional revolutions of pos * r / 2^64, exactly up to the float rounding
// of the top 32 bits: pos * r mod 2^64 taken as a signed value in [-1/2, 1/2)
// (three 32-bit integer multiplies, quarter rate).
__device__ __forceinline__ float rope_rev_exact(int pos, unsigned long long r) {
  const unsigned long long prod = (unsigned long long)(long long)pos * r;
  return (float)(int)(unsigned)(prod >> 32) * 2.3283064365386963e-10f;  // 2^-32
}

// The same for |pos| < 2^24 (p = (float)pos exact), in FP32: p * hi splits
// exactly into its rounded value xh and the FMA residual; the integer part of
// xh is dropped exactly (fract) and the residual plus p * lo is added. The
// residual and p * lo are each below 1/8 in magnitude, so the result lies in
// (-1/4, 5/4) within ~2^-24 revolutions of the exact reduction.
__device__ __forceinline__ float rope_rev_fast(float p, const RopeFreq& f) {
  const float xh = p * f.hi;
  const float e = fmaf(p, f.hi, -xh);
  const float xl = fmaf(p, f.lo, e);
  return __builtin_amdgcn_fractf(xh) + xl;
}

// cos and sin of the RoPE angle pos * omega_c from its revolutions; the
// hardware sine and cosine take revolutions and are accurate to ~1.3e-7.
// kMixed: the wave holds a position of magnitude >= 2^24 somewhere, so each
// lane picks the exact reduction for its own such position (a lane's result
// never depends on the other lanes' positions). Callers pick kMixed once per
// wave with rope_wave_mixed.
template <bool kMixed>
__device__ __forceinline__ void rope_cos_sin(int pos, float pf, const RopeFreq& f, float* c, float* s) {
  float rev = rope_rev_fast(pf, f);
  if constexpr (kMixed) rev = rope_pos_fast(pos) ? rev : rope_rev_exact(pos, f.r);
  *s = __builtin_amdgcn_sinf(rev);
  *c = __builtin_amdgcn_cosf(rev);
}

// The RoPE turn of a channel pair (x: channel c, y: channel c + 64) by the
// angle's cos and sin, with its products and roundings spelled out, so that
// every kernel that forms q' or k' forms the same bits.
__device__ __forceinline__ void rope_turn(float& x, float& y, float cs, float sn) {
  const float a = fmaf(x, cs, -(y * sn));
  const float b = fmaf(x, sn, y * cs);
  x = a;
  y = b;
}

__device__ __forceinline__ bool rope_wave_mixed(int pos) {
  return __builtin_amdgcn_ballot_w64(!rope_pos_fast(pos)) != 0;
}

// One-off form (both reductions evaluated, the lane's own one kept).
__device__ __forceinline__ void rope_cos_sin(int pos, const RopeFreq& f, float* c, float* s) {
  rope_cos_sin<true>(pos, (float)pos, f, c, s);
}

// Sum of squares of eight packed bf16 values plus acc (v_dot2 of c with itself).
__device__ __forceinline__ float sumsq8_dot(const uint4& c, float acc) {
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, c.x), __builtin_bit_cast(bf16x2_t, c.x), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, c.y), __builtin_bit_cast(bf16x2_t, c.y), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, c.z), __builtin_bit_cast(bf16x2_t, c.z), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, c.w), __builtin_bit_cast(bf16x2_t, c.w), acc, false);
  return acc;
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

// Exclusive scan over the NT threads of a block; *total gets the sum.
// Wave-level shuffle scans, then a scan of the NT / 64 wave totals (tmp holds
// at least that many ints).
template <int NT>
__device__ int block_excl_scan_t(int v, int* tmp, int* total) {
  constexpr int W = NT / 64;
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
    int w = lane < W ? tmp[lane] : 0;
#pragma unroll
    for (int off = 1; off < W; off <<= 1) {
      const int y = __shfl_up(w, off);
      if (lane >= off) w += y;
    }
    if (lane < W) tmp[lane] = w;
  }
  __syncthreads();
  const int base = wave > 0 ? tmp[wave - 1] : 0;
  *total = tmp[W - 1];
  __syncthreads();
  return base + x - v;
}

// The same over the 1024 threads of a block.
__device__ __forceinline__ int block_excl_scan(int v, int* tmp, int* total) {
  return block_excl_scan_t<1024>(v, tmp, total);
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

// Key tiles of the forward layout: sequence s owns the tiles from
// cu[s] / 64 + s on, one per 64 keys. These ranges never overlap (cu[s+1] / 64
// + s + 1 >= cu[s] / 64 + s + ceil(len / 64)) and stay below T / 64 + n, and
// a tile's sequence follows from cu_seqlens alone: the largest s with
// cu[s] / 64 + s <= e (for valid cu_seqlens; any s in [0, n) otherwise).
__device__ __forceinline__ int tile_base(int cu_s, int s) { return (cu_s >> 6) + s; }

__device__ __forceinline__ int tile_seq(const int* cu, int n, int e) {
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (tile_base(cu[mid], mid) <= e) lo = mid; else hi = mid - 1;
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

// Slot of key r (0..63) inside a V^T row: bits 2 and 3 swapped, which is the
// order in which the softmax output P^T sits in the MFMA B operand.
__device__ __forceinline__ int vt_slot(int r) { return r ^ ((((r >> 2) ^ (r >> 3)) & 1) * 12); }

// s_waitcnt immediate: vmcnt(0), expcnt and lgkmcnt not waited on.
constexpr int kWaitVmcnt0 = 0x0F70;

// Workgroup barrier for the tile ring. Vector-memory operations complete in
// issue order, so a wave whose tile loads were followed by exactly `n` more
// vector-memory operations has that tile in LDS once at most `n` remain in
// flight; the wave also finishes its LDS reads, then joins the barrier.
// Unlike __syncthreads() this leaves the newer loads in flight.
template <int N>
__device__ __forceinline__ void ring_barrier_n() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// Host-side helpers shared by the entry points.
static inline bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

static inline bool debug_sync() {
  const char* e = getenv("FLINT_ATTN_DEBUG");
  return e && e[0] == '1';
}

// Workspace view of the forward schedule's regions at `base`.
static inline Ws ws_at(void* workspace, const Layout& L) {
  char* base = static_cast<char*>(workspace);
  Ws ws;
  ws.hdr = reinterpret_cast<int*>(base + L.hdr);
  ws.rope = reinterpret_cast<RopeFreq*>(base + L.rope);
  ws.seq = reinterpret_cast<int4*>(base + L.seq);
  ws.tbase = reinterpret_cast<int*>(base + L.tbase);
  ws.qbase = reinterpret_cast<int*>(base + L.qbase);
  ws.pbase = reinterpret_cast<int*>(base + L.pbase);
  ws.tiles = reinterpret_cast<int2*>(base + L.tiles);
  ws.items = reinterpret_cast<int2*>(base + L.items);
  ws.kv = base + L.kv;
  ws.ntmax = (int)L.ntmax;
  return ws;
}

// Enqueues the schedule kernel (sequence table, key tiles in the packed
// layout, query blocks sorted by work, RoPE frequencies) on `st`; the
// backward's layout.
void launch_schedule(const int* cu, const int* seqused, int n, int T, int max_seqlen, int window,
                     double theta, const Ws& ws, hipStream_t st);

}  // namespace flint
