// Projections around the attention layer: q, k, v from the hidden states and
// the output projection (flint.layers page, FlintAttention: separate q_proj,
// k_proj, v_proj and o_proj, nn.Linear without bias, y = x W^T with W
// [out, in]; FlintConfig page: hidden 2048, 32 query heads and 4 key/value
// heads of 128 channels).
//
// One GEMM kernel serves both: C = X W^T for X [M tokens][K] and W [N][K],
// both K-contiguous, bf16 in, FP32 accumulation, bf16 out. The output channel
// axis may be split into up to three regions, each with its own weight and
// output tensor, so q, k and v come out of one launch over the concatenated
// channels (4096 + 512 + 512) into their own [T, heads, 128] tensors.
//
// Tiling for gfx950: a workgroup of 8 waves owns 256 channels x 256 tokens.
// The product runs as C^T = W X^T on v_mfma_f32_32x32x16_bf16, so a lane
// holds one token and 16 channels of each 32x32 block: the epilogue swaps
// halves with the partner lane and stores 16 contiguous bytes of a token's
// row. Wave w covers channels 128 (w & 1) + [0, 128) (one head) and tokens
// 64 (w >> 1) + [0, 64): 4 x 2 blocks, 128 FP32 accumulators, two waves per
// SIMD. k advances 64 at a time through a 2-stage LDS ring (2 x 64 KiB) filled
// by direct global-to-LDS loads one stage ahead; inside a stage the operands of
// the next 16-wide k step are read while the MFMAs of this one run. Rows are
// 128 bytes in LDS; 16-byte chunk c of row r sits at chunk c ^ ((r >> 1) & 7),
// so the 16 lanes of an operand read hit 16 different bank groups. Token rows
// past M read as zero and their stores are dropped (buffer range checks).

#include <hip/hip_runtime.h>

#include "flint_common.h"

namespace flint {

namespace {

constexpr int kPN = 256;          // output channels per tile
constexpr int kProjKAlign = 64;   // K is a multiple of every tile configuration's k step
constexpr int kProjMaxTM = 256;   // largest token tile (buffer offsets stay 32-bit)

struct ProjRegions {
  const uint16_t* w[3];  // [n][K] per region
  uint16_t* out[3];      // [M][n] per region
  int n[3];              // channels per region, multiples of kPN
};

__device__ __forceinline__ f32x16 mma_bf16(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Tile shape: TM tokens x 256 channels, k advancing PK per stage through a
// ring of STAGES stages with loads AHEAD stages ahead, WAVES waves of which
// each covers 128 channels (one head) and TM / (WAVES / 2) tokens.
template <int PK, int STAGES, int AHEAD, int WAVES, int TM>
struct ProjCfg {
  static constexpr int kChunks = PK / 8;              // 16-byte chunks per LDS row
  static constexpr int kRowB = PK * 2;                // bytes per LDS row
  static constexpr int kRowsPerLoad = 1024 / kRowB;   // rows one wave-wide load fills
  static constexpr int kWLoads = kPN / kRowsPerLoad;  // loads of the W part of a stage
  static constexpr int kXLoads = TM / kRowsPerLoad;   // loads of the X part
  static constexpr int kLoadsPerWave = (kWLoads + kXLoads) / WAVES;
  static constexpr int kWBytes = kPN * kRowB;
  static constexpr int kStageBytes = (kPN + TM) * kRowB;
  static constexpr int kWaveTok = TM / (WAVES / 2);   // tokens per wave
  static constexpr int kI = kWaveTok / 32;            // 32-token blocks per wave
  static_assert((kWLoads + kXLoads) % WAVES == 0, "loads split evenly over the waves");
  static_assert(AHEAD < STAGES, "a stage is reloaded only after it was read");
  static_assert(STAGES * kStageBytes <= 160 * 1024, "LDS");
};

// 16-byte chunk c of LDS row r sits at chunk position c ^ swz(r): the 16
// lanes of an operand read (16 consecutive rows, one chunk) then cover all 64
// banks. 64-byte rows pack 4 rows per 256 bytes, 128-byte rows 2.
template <int kChunks>
__device__ __forceinline__ int swz(int r) {
  return kChunks == 4 ? ((r >> 2) & 3) : ((r >> 1) & 7);
}

// This wave's loads of one stage. Load q of the stage fills rows
// q * kRowsPerLoad + [0, kRowsPerLoad) of the W part (q < kWLoads) or the X
// part; lane L lands at LDS byte 16 L of it: row L / kChunks, chunk position
// L % kChunks, so it reads source chunk (L % kChunks) ^ swz(row).
#define WAVES_OF(C) ((C::kWLoads + C::kXLoads) / C::kLoadsPerWave)

template <class C>
__device__ __forceinline__ void load_stage(__amdgpu_buffer_rsrc_t wr, __amdgpu_buffer_rsrc_t xr,
                                           int row_bytes, int kbyte, char* stage, int wave,
                                           int lane) {
#pragma unroll
  for (int n = 0; n < C::kLoadsPerWave; ++n) {
    const int q = wave + n * WAVES_OF(C);
    const bool isw = q < C::kWLoads;
    const int row0 = (isw ? q : q - C::kWLoads) * C::kRowsPerLoad;
    const int row = row0 + lane / C::kChunks;
    const int c = (lane % C::kChunks) ^ swz<C::kChunks>(row);
    char* base = stage + (isw ? 0 : C::kWBytes) + row0 * C::kRowB;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(isw ? wr : xr,
                                             (__attribute__((address_space(3))) void*)base, 16,
                                             row * row_bytes + c * 16, kbyte, 0, 0);
  }
}

// Operand fragment of 32 rows starting at `row0` (a multiple of 16) for
// k-step kk: lane reads row row0 + lane % 32, chunk 2 kk + lane / 32.
template <class C>
__device__ __forceinline__ bf16x8 ld_operand(const char* part, int row0, int kk, int lane) {
  const int r = row0 + (lane & 31);
  const int c = (2 * kk + (lane >> 5)) ^ swz<C::kChunks>(r);
  return *reinterpret_cast<const bf16x8*>(part + r * C::kRowB + c * 16);
}

template <int N>
__device__ __forceinline__ void proj_barrier_upto(int newer) {
  if constexpr (N <= 0) {
    ring_barrier_n<0>();
  } else {
    if (newer == N) ring_barrier_n<(N > 0 ? N : 0)>();
    else proj_barrier_upto<N - 1>(newer);
  }
}

template <class C, int PK, int STAGES, int AHEAD, int WAVES, int TM, int MINB>
__global__ __launch_bounds__(64 * WAVES, MINB) void proj_gemm_kernel(const uint16_t* __restrict__ x,
                                                                   int M, int K, ProjRegions R) {
  __shared__ __attribute__((aligned(16))) char smem[STAGES][C::kStageBytes];
  const int nt_n = (R.n[0] + R.n[1] + R.n[2]) / kPN;
  const int nt_m = (M + TM - 1) / TM;
  const int b = blockIdx.x;
  int tm, tn;
  if (nt_m % 32 == 0) {
    // Workgroup b runs on XCD b % 8. Each XCD owns nt_m / 8 token tiles and
    // runs them in groups of 4, taking the channel tiles in order for all 4
    // together: the 32 workgroups an XCD runs at once are 4 token tiles x 8
    // channel tiles, so each k slice it fetches is used 4 or 8 times from its
    // L2.
    const int per = nt_m / 8, r = b / 8;
    const int g = r / (4 * nt_n), w = r % (4 * nt_n);
    tn = w / 4;
    tm = (b % 8) * per + 4 * g + w % 4;
  } else {
    // few token tiles: consecutive workgroups walk the channel tiles of one
    tm = b / nt_n;
    tn = b % nt_n;
  }
  // the region of this channel tile (selects, not an indexed argument array)
  int c0 = tn * kPN;
  const int reg = c0 < R.n[0] ? 0 : (c0 < R.n[0] + R.n[1] ? 1 : 2);
  c0 -= reg == 0 ? 0 : (reg == 1 ? R.n[0] : R.n[0] + R.n[1]);
  const int n_out = reg == 0 ? R.n[0] : (reg == 1 ? R.n[1] : R.n[2]);
  const uint16_t* wreg = reg == 0 ? R.w[0] : (reg == 1 ? R.w[1] : R.w[2]);
  uint16_t* oreg = reg == 0 ? R.out[0] : (reg == 1 ? R.out[1] : R.out[2]);
  const int m0 = tm * TM;
  const int rows = min(M - m0, TM);
  const int row_bytes = K * 2;
  const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(wreg + (size_t)c0 * K), 0, kPN * row_bytes, kBufferWord3);
  const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(x + (size_t)m0 * K), 0, rows * row_bytes, kBufferWord3);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wc = wave & 1, wt = wave >> 1;
  const int nk = K / PK;

  f32x16 acc[C::kI][4];
#pragma unroll
  for (int i = 0; i < C::kI; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  for (int s = 0; s < AHEAD && s < nk; ++s)
    load_stage<C>(wr, xr, row_bytes, s * PK * 2, smem[s], wave, lane);
  for (int s = 0; s < nk; ++s) {
    // stage s is in LDS once only the loads of the later stages already
    // issued remain in flight; every wave has also finished reading stage s - 1
    proj_barrier_upto<C::kLoadsPerWave * (AHEAD - 1)>(C::kLoadsPerWave * min(AHEAD - 1, nk - 1 - s));
    if (s + AHEAD < nk)
      load_stage<C>(wr, xr, row_bytes, (s + AHEAD) * PK * 2, smem[(s + AHEAD) % STAGES], wave, lane);
    const char* wp = smem[s % STAGES];
    const char* xp = wp + C::kWBytes;
    // the operands of k-step kk + 1 are read while the MFMAs of kk run
    constexpr int kF = C::kI + 4;  // fragments per k-step
    bf16x8 f[2][kF];
    auto read = [&](int kk, bf16x8* dst) {
#pragma unroll
      for (int i = 0; i < C::kI; ++i) dst[i] = ld_operand<C>(xp, C::kWaveTok * wt + 32 * i, kk, lane);
#pragma unroll
      for (int j = 0; j < 4; ++j) dst[C::kI + j] = ld_operand<C>(wp, 128 * wc + 32 * j, kk, lane);
    };
    read(0, f[0]);
    __builtin_amdgcn_sched_group_barrier(0x100, kF, 0);
#pragma unroll
    for (int kk = 0; kk < PK / 16; ++kk) {
      if (kk + 1 < PK / 16) read(kk + 1, f[(kk + 1) & 1]);
      const bf16x8* g = f[kk & 1];
#pragma unroll
      for (int i = 0; i < C::kI; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mma_bf16(g[C::kI + j], g[i], acc[i][j]);
#pragma unroll
      for (int m = 0; m < 4 * C::kI; ++m) {
        if (kk + 1 < PK / 16 && m < kF) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      }
    }
  }

  // Epilogue: lane (col, half) holds channels 32j + 8g + 4half + [0, 4) of
  // token kWaveTok wt + 32i + col; a swap with the partner lane gives it
  // channels 32j + 16r2 + 8half + [0, 8), 16 contiguous bytes per store.
  const int col = lane & 31, half = lane >> 5;
  const __amdgpu_buffer_rsrc_t orsrc = __builtin_amdgcn_make_buffer_rsrc(
      oreg + (size_t)m0 * n_out, 0, rows * n_out * 2, kBufferWord3);
#pragma unroll
  for (int i = 0; i < C::kI; ++i) {
    const int tok = C::kWaveTok * wt + 32 * i + col;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r2 = 0; r2 < 2; ++r2) {
        const f32x16& c = acc[i][j];
        const int o = 8 * r2;
        const unsigned a0 = pack2(c[o], c[o + 1]), a1 = pack2(c[o + 2], c[o + 3]);
        const unsigned b0 = pack2(c[o + 4], c[o + 5]), b1 = pack2(c[o + 6], c[o + 7]);
        const auto x0 = __builtin_amdgcn_permlane32_swap(a0, b0, false, false);
        const auto x1 = __builtin_amdgcn_permlane32_swap(a1, b1, false, false);
        const uint4 w = make_uint4(x0[0], x1[0], x0[1], x1[1]);
        const int ch = c0 + 128 * wc + 32 * j + 16 * r2 + 8 * half;  // channel in the region
        __builtin_amdgcn_raw_buffer_store_b128(
            __builtin_bit_cast(__attribute__((ext_vector_type(4))) unsigned, w), orsrc,
            (tok * n_out + ch) * 2, 0, 0);
      }
  }
}

// Tile configuration (k step, ring stages, stages loaded ahead, waves, tokens
// per tile, workgroups per CU). 64-wide k steps in a two-stage ring measured
// fastest on gfx950: fewer barriers per MFMA than 32-wide steps in four stages.
#ifndef FLINT_PROJ_CFG
#define FLINT_PROJ_CFG 64, 2, 1, 8, 256, 1
#endif

template <int PK, int STAGES, int AHEAD, int WAVES, int TM, int MINB>
int launch_proj_cfg(const void* x, int M, int K, const ProjRegions& R, hipStream_t st) {
  using C = ProjCfg<PK, STAGES, AHEAD, WAVES, TM>;
  const int n = R.n[0] + R.n[1] + R.n[2];
  const int64_t total = (int64_t)((M + TM - 1) / TM) * (n / kPN);
  if (total == 0) return FLINT_OK;
  if (K % PK != 0) return FLINT_ERR_UNSUPPORTED;
  (void)hipGetLastError();
  proj_gemm_kernel<C, PK, STAGES, AHEAD, WAVES, TM, MINB>
      <<<(unsigned)total, 64 * WAVES, 0, st>>>(static_cast<const uint16_t*>(x), M, K, R);
  if (hipGetLastError() != hipSuccess) return FLINT_ERR_HIP;
  return FLINT_OK;
}

int launch_proj(const void* x, int M, int K, const ProjRegions& R, hipStream_t st) {
  return launch_proj_cfg<FLINT_PROJ_CFG>(x, M, K, R, st);
}

}  // namespace

}  // namespace flint

using namespace flint;

extern "C" int flint_proj_qkv(const void* x, const void* w_q, const void* w_k, const void* w_v,
                              int32_t total_tokens, int32_t hidden, int32_t num_q_heads,
                              int32_t num_kv_heads, int32_t head_dim, void* q, void* k, void* v,
                              void* stream) {
  if (total_tokens < 0 || hidden <= 0) return FLINT_ERR_SHAPE;
  if (num_q_heads != kH || num_kv_heads != kG || head_dim != kD) return FLINT_ERR_UNSUPPORTED;
  if (hidden % kProjKAlign != 0 || (int64_t)hidden * 2 * kPN >= ((int64_t)1 << 31))
    return FLINT_ERR_UNSUPPORTED;
  if (total_tokens == 0) return FLINT_OK;
  if (!x || !w_q || !w_k || !w_v || !q || !k || !v) return FLINT_ERR_NULL;
  if (!aligned(x, 16) || !aligned(w_q, 16) || !aligned(w_k, 16) || !aligned(w_v, 16) ||
      !aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16))
    return FLINT_ERR_ALIGN;
  ProjRegions R;
  R.w[0] = static_cast<const uint16_t*>(w_q);
  R.w[1] = static_cast<const uint16_t*>(w_k);
  R.w[2] = static_cast<const uint16_t*>(w_v);
  R.out[0] = static_cast<uint16_t*>(q);
  R.out[1] = static_cast<uint16_t*>(k);
  R.out[2] = static_cast<uint16_t*>(v);
  R.n[0] = kH * kD;
  R.n[1] = kG * kD;
  R.n[2] = kG * kD;
  return launch_proj(x, total_tokens, hidden, R, reinterpret_cast<hipStream_t>(stream));
}

extern "C" int flint_proj_out(const void* o, const void* w_o, int32_t total_tokens, int32_t hidden,
                              int32_t num_q_heads, int32_t head_dim, void* y, void* stream) {
  if (total_tokens < 0 || hidden <= 0) return FLINT_ERR_SHAPE;
  if (num_q_heads != kH || head_dim != kD) return FLINT_ERR_UNSUPPORTED;
  if (hidden % kPN != 0 || (int64_t)kProjMaxTM * hidden * 2 >= ((int64_t)1 << 31))
    return FLINT_ERR_UNSUPPORTED;
  if (total_tokens == 0) return FLINT_OK;
  if (!o || !w_o || !y) return FLINT_ERR_NULL;
  if (!aligned(o, 16) || !aligned(w_o, 16) || !aligned(y, 16)) return FLINT_ERR_ALIGN;
  ProjRegions R;
  R.w[0] = static_cast<const uint16_t*>(w_o);
  R.out[0] = static_cast<uint16_t*>(y);
  R.n[0] = hidden;
  R.w[1] = R.w[2] = nullptr;
  R.out[1] = R.out[2] = nullptr;
  R.n[1] = R.n[2] = 0;
  return launch_proj(o, total_tokens, kH * kD, R, reinterpret_cast<hipStream_t>(stream));
}
