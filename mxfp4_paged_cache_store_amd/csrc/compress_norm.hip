// compress_norm.hip -- the compress-ratio-1 case of the DeepSeek-V4.1
// save/compress/norm step, for gfx950.
//
// At compress ratio 1 each token is a group of its own: no ring state, no
// pooling, and the slot mapping only says which tokens are valid ("vllm.
// models.deepseek_v41.common.ops.fused_compress_quant_cache",
// `fused_save_compress_norm`, description and parameters).  What remains is
// an RMSNorm of the token's fp32 row of 512 values with a bf16 weight,
// written as bf16 for tokens whose slot is >= 0:
//   y[d] = bf16_rn((x[d] * r) * w[d]),  r = 1 / sqrt(sum(x^2) / 512 + eps),
// all in fp32 with correctly rounded sqrt and division.  Rows of invalid
// tokens are not written.
//
// One wave per token, two tokens per wave.  Lane l holds values 4l..4l+3
// and 256+4l..256+4l+3 (two 16-byte loads, each 1 KiB contiguous across
// the wave), so loads and the 8-byte bf16 stores are fully coalesced.  The
// sum of squares is reduced with DPP within rows of 16 lanes, then across
// rows with two lane shuffles; every step adds a value to its exact mirror,
// so all 64 lanes end with the same bits.  HBM-bound: 2048 B in, 1024 B out;
// the output rows are written through to memory (NT + SC1).
#include "kernels.hpp"

namespace mxs {
namespace {

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kTokensPerWave = 2;
constexpr int kWavesPerBlock = 4;
constexpr int kWidth = 512;
constexpr int kRowMirror = 0x140;      // lane i reads lane 15-i of its row of 16
constexpr int kRowHalfMirror = 0x141;  // lane i reads lane 7-i of its half-row

__device__ __forceinline__ float wave_sum(float v) {
  v += as_f32(dpp<kQuadSwap1>(as_u32(v)));
  v += as_f32(dpp<kQuadSwap2>(as_u32(v)));
  v += as_f32(dpp<kRowHalfMirror>(as_u32(v)));
  v += as_f32(dpp<kRowMirror>(as_u32(v)));
  v += __shfl_xor(v, 16);
  v += __shfl_xor(v, 32);
  return v;
}

// fp32 -> bf16, round to nearest even; NaN stays a (quiet) NaN.
__device__ __forceinline__ uint32_t bf16_rn(float f) {
  const uint32_t u = as_u32(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__global__ __launch_bounds__(kWave * kWavesPerBlock) void compress_norm_cr1_kernel(const NormArgs a) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t first = ((int64_t)xcd_contiguous_block() * kWavesPerBlock + wave) * kTokensPerWave;

  const __amdgpu_buffer_rsrc_t wbuf = buffer_at(a.weight, kWidth * 2);
  u32x2 w[2];
#pragma unroll
  for (int c = 0; c < 2; ++c)
    w[c] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(wbuf, (c * 64 + lane) * 8, 0, 0));

  __amdgpu_buffer_rsrc_t src[kTokensPerWave], dst[kTokensPerWave];
#pragma unroll
  for (int p = 0; p < kTokensPerWave; ++p) {
    const int64_t t = first + p;
    const bool ok = t < a.num_tokens && a.slots[t] >= 0;
    src[p] = buffer_at(a.kv + (ok ? t * a.kv_row_stride : 0), ok ? kWidth * 4u : 0u);
    dst[p] = buffer_at(a.out + (ok ? t * a.out_row_stride : 0), ok ? kWidth * 2u : 0u);
  }
  u32x4 x[kTokensPerWave][2];
#pragma unroll
  for (int p = 0; p < kTokensPerWave; ++p)
#pragma unroll
    for (int c = 0; c < 2; ++c)
      x[p][c] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(src[p], (c * 64 + lane) * 16, 0, 0));

#pragma unroll
  for (int p = 0; p < kTokensPerWave; ++p) {
    float ss = 0.0f;
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float v = as_f32(x[p][c][k]);
        ss += v * v;
      }
    ss = wave_sum(ss);
    const float r = __fdiv_rn(1.0f, __fsqrt_rn(ss / (float)kWidth + a.eps));
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      uint32_t h[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t wb = k & 1 ? (w[c][k >> 1] & 0xFFFF0000u) : (w[c][k >> 1] << 16);
        h[k] = bf16_rn((as_f32(x[p][c][k]) * r) * as_f32(wb));
      }
      const u32x2 o = {h[0] | (h[1] << 16), h[2] | (h[3] << 16)};
      // Whole output rows: streamed to memory (NT + SC1).
      __builtin_amdgcn_raw_buffer_store_b64(o, dst[p], (c * 64 + lane) * 8, 0, kBufNTDevice);
    }
  }
}

}  // namespace

hipError_t launch_compress_norm_cr1(const NormArgs& a, hipStream_t stream) {
  constexpr int64_t kPerBlock = (int64_t)kWavesPerBlock * kTokensPerWave;
  const int64_t blocks = (a.num_tokens + kPerBlock - 1) / kPerBlock;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(compress_norm_cr1_kernel, dim3((unsigned)blocks), dim3(kWave * kWavesPerBlock), 0,
                     stream, a);
  return hipGetLastError();
}

}  // namespace mxs
