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
// SIMD. k advances 32 at a time through a 4-stage LDS ring filled by direct
// global-to-LDS loads, three stages ahead. Rows are 64 bytes in LDS; 16-byte
// chunk c of row r sits at chunk c ^ ((r >> 2) & 3), so the 16 lanes of an
// operand read hit 16 different bank groups. Token rows past M read as zero
// and their stores are dropped (buffer range checks).

#include <hip/hip_runtime.h>

#include "flint_common.h"

namespace flint {

namespace {

constexpr int kPM = 256;                      // tokens per tile
constexpr int kPN = 256;                      // output channels per tile
constexpr int kPK = 32;                       // k per stage
constexpr int kPStages = 4;                   // LDS ring depth
constexpr int kPThreads = 512;                // 8 waves
constexpr int kPHalf = kPN * kPK * 2;         // bytes of the W part of a stage (16 KiB)
constexpr int kPStageBytes = 2 * kPHalf;      // W part, then X part (32 KiB)
constexpr int kPStageVec = kPStageBytes / 16;

struct ProjRegions {
  const uint16_t* w[3];  // [n][K] per region
  uint16_t* out[3];      // [M][n] per region
  int n[3];              // channels per region, multiples of kPN
};

__device__ __forceinline__ f32x16 mma_bf16(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// This wave's share of one stage: W rows 32 wave + [0, 32) and X rows
// 32 wave + [0, 32), 16 rows (1 KiB) per load. Lane L of a load lands at
// LDS byte 16 L of its 1 KiB: row L / 4, chunk position L % 4, which holds
// source chunk (L % 4) ^ ((row >> 2) & 3) = (L % 4) ^ ((L >> 4) & 3).
__device__ __forceinline__ void load_stage(__amdgpu_buffer_rsrc_t wr, __amdgpu_buffer_rsrc_t xr,
                                           int row_bytes, int kbyte, uint4* stage, int wave,
                                           int lane) {
  const int c = (lane & 3) ^ ((lane >> 4) & 3);
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int row = 32 * wave + 16 * i + (lane >> 2);
    const int voff = row * row_bytes + c * 16;
    char* base = reinterpret_cast<char*>(stage) + (32 * wave + 16 * i) * 64;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        wr, (__attribute__((address_space(3))) void*)base, 16, voff, kbyte, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        xr, (__attribute__((address_space(3))) void*)(base + kPHalf), 16, voff, kbyte, 0, 0);
  }
}

// Operand fragment of 32 rows starting at `row0` (a multiple of 16) for
// k-step kk: lane reads row row0 + lane % 32, chunk 2 kk + lane / 32.
__device__ __forceinline__ bf16x8 ld_operand(const uint4* part, int row0, int kk, int lane) {
  const int r = lane & 31;
  const int c = (2 * kk + (lane >> 5)) ^ ((r >> 2) & 3);
  return __builtin_bit_cast(bf16x8, part[(row0 + r) * 4 + c]);
}

__device__ __forceinline__ void proj_barrier(int newer) {
  switch (newer) {
    case 8: ring_barrier_n<8>(); break;
    case 4: ring_barrier_n<4>(); break;
    default: ring_barrier_n<0>(); break;
  }
}

__global__ __launch_bounds__(kPThreads, 1) void proj_gemm_kernel(const uint16_t* __restrict__ x,
                                                                  int M, int K, ProjRegions R) {
  __shared__ uint4 smem[kPStages][kPStageVec];
  const int nt_n = (R.n[0] + R.n[1] + R.n[2]) / kPN;
  const int nt_m = (M + kPM - 1) / kPM;
  const int total = nt_m * nt_n;
  // Consecutive ranks go to one XCD (workgroup b runs on XCD b % 8); a rank
  // walks the channel tiles of one token tile, which stays in that L2.
  const int b = blockIdx.x;
  const int rank = (total % 8 == 0) ? (b % 8) * (total / 8) + b / 8 : b;
  const int tm = rank / nt_n, tn = rank % nt_n;
  // the region of this channel tile (selects, not an indexed argument array)
  int c0 = tn * kPN;
  const int reg = c0 < R.n[0] ? 0 : (c0 < R.n[0] + R.n[1] ? 1 : 2);
  c0 -= reg == 0 ? 0 : (reg == 1 ? R.n[0] : R.n[0] + R.n[1]);
  const int n_out = reg == 0 ? R.n[0] : (reg == 1 ? R.n[1] : R.n[2]);
  const uint16_t* wreg = reg == 0 ? R.w[0] : (reg == 1 ? R.w[1] : R.w[2]);
  uint16_t* oreg = reg == 0 ? R.out[0] : (reg == 1 ? R.out[1] : R.out[2]);
  const int m0 = tm * kPM;
  const int rows = min(M - m0, kPM);
  const int row_bytes = K * 2;
  const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(wreg + (size_t)c0 * K), 0, kPN * row_bytes, kBufferWord3);
  const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(x + (size_t)m0 * K), 0, rows * row_bytes, kBufferWord3);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wc = wave & 1, wt = wave >> 1;
  const int nk = K / kPK;

  f32x16 acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  for (int s = 0; s < 3 && s < nk; ++s) load_stage(wr, xr, row_bytes, s * kPK * 2, smem[s], wave, lane);
  for (int s = 0; s < nk; ++s) {
    // stage s is in LDS once only the loads of the (up to two) later stages
    // remain in flight; every wave has also finished reading stage s - 1
    proj_barrier(4 * min(2, nk - 1 - s));
    if (s + 3 < nk) load_stage(wr, xr, row_bytes, (s + 3) * kPK * 2, smem[(s + 3) % kPStages], wave, lane);
    const uint4* wp = smem[s % kPStages];
    const uint4* xp = wp + kPHalf / 16;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      bf16x8 fw[4], fx[2];
#pragma unroll
      for (int j = 0; j < 4; ++j) fw[j] = ld_operand(wp, 128 * wc + 32 * j, kk, lane);
#pragma unroll
      for (int i = 0; i < 2; ++i) fx[i] = ld_operand(xp, 64 * wt + 32 * i, kk, lane);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mma_bf16(fw[j], fx[i], acc[i][j]);
    }
  }

  // Epilogue: lane (col, half) holds channels 32j + 8g + 4half + [0, 4) of
  // token 64wt + 32i + col; a swap with the partner lane gives it channels
  // 32j + 16r2 + 8half + [0, 8), 16 contiguous bytes per store.
  const int col = lane & 31, half = lane >> 5;
  const __amdgpu_buffer_rsrc_t orsrc = __builtin_amdgcn_make_buffer_rsrc(
      oreg + (size_t)m0 * n_out, 0, rows * n_out * 2, kBufferWord3);
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int tok = 64 * wt + 32 * i + col;
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

int launch_proj(const void* x, int M, int K, const ProjRegions& R, hipStream_t st) {
  const int n = R.n[0] + R.n[1] + R.n[2];
  const int64_t total = (int64_t)((M + kPM - 1) / kPM) * (n / kPN);
  if (total == 0) return FLINT_OK;
  (void)hipGetLastError();
  proj_gemm_kernel<<<(unsigned)total, kPThreads, 0, st>>>(static_cast<const uint16_t*>(x), M, K, R);
  if (hipGetLastError() != hipSuccess) return FLINT_ERR_HIP;
  return FLINT_OK;
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
  if (hidden % kPK != 0 || (int64_t)hidden * 2 * kPN >= ((int64_t)1 << 31)) return FLINT_ERR_UNSUPPORTED;
  if (total_tokens == 0) return FLINT_OK;
  if (!x || !w_q || !w_k || !w_v || !q || !k || !v) return FLINT_ERR_NULL;
  if (!aligned(x, 16) || !aligned(w_q, 16) || !aligned(w_k, 16) || !aligned(w_v, 16) ||
      !aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16))
    return FLINT_ERR_ALIGN;
  if ((int64_t)kPM * kH * kD * 2 >= ((int64_t)1 << 31)) return FLINT_ERR_SHAPE;
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
  if (hidden % kPN != 0 || (int64_t)kPM * hidden * 2 >= ((int64_t)1 << 31)) return FLINT_ERR_UNSUPPORTED;
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
