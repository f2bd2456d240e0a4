// rope_insert.hip -- GPT-J RoPE followed by MXFP8 (528-byte), NVFP4
// (288-byte) or V4 (584-byte) quantization of a 512-wide bf16 latent into a
// paged compressed KV cache, for gfx950.
//
// What is computed follows the DeepSeek-V4.1 insert page ("vllm.models.
// deepseek_v41.common.ops.fused_compress_quant_cache":
// `_rope_quant_insert_mxfp8_kernel`, `_rope_quant_insert_nvfp4_kernel`,
// `rope_quant_insert`):
//   gate   a token is written only for a valid slot and when (position + 1)
//          is a multiple of the compress ratio;
//   RoPE   pairs (2p, 2p+1) for p >= 224 (dims 448..511) rotate by the cos/sin
//          row of the group's first position, (position / CR) * CR; the NoPE
//          pairs go through the same arithmetic with (cos, sin) = (1, 0), so
//          signed zeros and NaNs behave alike; each multiply and add rounds
//          once (this file is built without contraction);
//   sanitize  NaN -> +0 after the rotation;
//   MXFP8  per 32 values: amax floored at 1e-4, E = ceil(log2(amax/448)) read
//          exactly from the fp32 bit pattern of fp32(amax * fl(1/448)),
//          values e4m3(clamp(r * 2^-E, +-448)), scale byte clamp(E+127);
//   NVFP4  per 16 values: S8 = e4m3(clamp(amax * fl(1/6), 2^-9, 448)),
//          y = r / S8 correctly rounded, nearest-even E2M1 codes saturating
//          at 6, sign bit only below zero, NaN (possible only without
//          sanitising) coded 0;
//   V4     (the page gives the record's widths, not its kernel) the 448 NoPE
//          values as E4M3 in 7 groups of 64 under the MXFP8 rule, then the 64
//          rotated RoPE values as bf16 (nearest-even, NaN -> 0x7FC0), then
//          7 UE8M0 bytes and one zero padding byte in the page's scale area.
//
// Layout on CDNA4: one wave per token; lane l holds values 8l..8l+7 (pairs
// 4l..4l+3), so the RoPE pairs live in lanes 56..63, an MXFP8 group is a DPP
// quad, a V4 group a half-row of 8 lanes and an NVFP4 tile a lane pair.
// E4M3 and E2M1 conversions use gfx950's v_cvt_scalef32_pk_fp8_f32 /
// v_cvt_scalef32_pk_fp4_f32 with scale 1.0.
#include "kernels.hpp"

namespace mxs {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short i16x2 __attribute__((ext_vector_type(2)));

constexpr int kTokensPerWave = 1;  // measured: more waves beat a per-wave token loop
constexpr int kWavesPerBlock = 4;

// Gate + rotation for one token.  Returns false (uniformly) when the token is
// not written.  On success r[0..7] hold the lane's rotated values.
__device__ __forceinline__ bool rope_token(const RopeArgs& a, int64_t t, int lane,
                                           float r[8], int64_t& page_off, uint32_t& in_page) {
  const int64_t s = a.slots[t];
  if (s < 0 || s >= (int64_t)a.num_slots) return false;
  const int64_t pos = a.positions[t];
  int64_t base;
  if ((uint64_t)pos < 0x7FFFFFFFull) {
    const uint32_t p32 = (uint32_t)pos, cr = (uint32_t)a.cr;
    if ((p32 + 1u) % cr != 0u) return false;
    base = (int64_t)(p32 / cr * cr);
  } else {
    if ((pos + 1) % a.cr != 0) return false;
    base = pos / a.cr * a.cr;
  }
  if (base < 0 || base >= a.cos_rows) return false;

  const u32x4 w = *reinterpret_cast<const u32x4*>(a.latent + t * 512 + lane * 8);
  float c[4] = {1.0f, 1.0f, 1.0f, 1.0f};
  float sn[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  if (lane >= 56) {
    const float* cs = a.cos_sin + base * a.cos_stride + (lane - 56) * 4;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      c[i] = cs[i];
      sn[i] = cs[32 + i];
    }
  }
  const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float even = as_f32(wd[i] << 16);
    const float odd = as_f32(wd[i] & 0xFFFF0000u);
    const float ec = even * c[i];
    const float os = odd * sn[i];
    const float oc = odd * c[i];
    const float es = even * sn[i];
    r[2 * i] = ec - os;
    r[2 * i + 1] = oc + es;
  }
  if (a.sanitize) {
#pragma unroll
    for (int i = 0; i < 8; ++i) r[i] = (r[i] == r[i]) ? r[i] : 0.0f;
  }
  const uint32_t s32 = (uint32_t)s;
  uint32_t page;
  if (a.block_shift >= 0) {
    page = s32 >> a.block_shift;
    in_page = s32 & (a.block - 1u);
  } else {
    page = s32 / a.block;
    in_page = s32 - page * a.block;
  }
  page_off = (int64_t)page * a.page_stride;
  return true;
}

__device__ __forceinline__ float max_abs8(const float r[8]) {
  float m = fabsf(r[0]);
#pragma unroll
  for (int i = 1; i < 8; ++i) m = fmaxf(m, fabsf(r[i]));
  return m;
}

// Two fp32 -> two OCP E4M3 bytes (RNE, sign kept), low byte from `lo`.
__device__ __forceinline__ uint32_t e4m3x2(float lo, float hi) {
  i16x2 z = {0, 0};
  i16x2 p = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(z, lo, hi, 1.0f, false);
  return __builtin_bit_cast(uint32_t, p) & 0xFFFFu;
}

__global__ __launch_bounds__(kWave * kWavesPerBlock) void mxfp8_rope_kernel(const RopeArgs a) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t first = ((int64_t)blockIdx.x * kWavesPerBlock + wave) * kTokensPerWave;
  const float inv448 = (float)(1.0 / 448.0);

  for (int p = 0; p < kTokensPerWave; ++p) {
    const int64_t t = first + p;
    if (t >= a.num_tokens) break;
    float r[8];
    int64_t page_off;
    uint32_t in_page;
    if (!rope_token(a, t, lane, r, page_off, in_page)) continue;

    float amax = max_abs8(r);
    amax = fmaxf(amax, as_f32(dpp<kQuadSwap1>(as_u32(amax))));
    amax = fmaxf(amax, as_f32(dpp<kQuadSwap2>(as_u32(amax))));
    amax = fmaxf(amax, 1e-4f);
    const uint32_t vb = as_u32(amax * inv448);
    // v >= fl(1e-4) * fl(1/448) is normal; +inf reads as exponent 128.
    const int E = (int)((vb >> 23) & 0xFFu) - 127 + ((vb & 0x7FFFFFu) != 0u ? 1 : 0);
    const float mul = E <= 126 ? as_f32((uint32_t)(127 - E) << 23)
                               : as_f32(0x00400000u >> (E - 127));
    float y[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) y[i] = fminf(fmaxf(r[i] * mul, -448.0f), 448.0f);
    const uint32_t lo = e4m3x2(y[0], y[1]) | (e4m3x2(y[2], y[3]) << 16);
    const uint32_t hi = e4m3x2(y[4], y[5]) | (e4m3x2(y[6], y[7]) << 16);

    int enc = E + 127;
    enc = max(enc, 0);
    enc = min(enc, a.sanitize ? 254 : 255);
    const uint32_t sb = (uint32_t)enc;
    const uint32_t sdw =
        dpp<kRowShr12>(sb) | (dpp<kRowShr8>(sb) << 8) | (dpp<kRowShr4>(sb) << 16) | (sb << 24);

    uint8_t* page = a.cache + page_off;
    uint8_t* values = page + (int64_t)in_page * 512;
    uint8_t* scales = page + (int64_t)a.block * 512 + (int64_t)in_page * 16;
    *reinterpret_cast<u32x2*>(values + lane * 8) = u32x2{lo, hi};
    if ((lane & 15) == 12) reinterpret_cast<uint32_t*>(scales)[lane >> 4] = sdw;
  }
}

__global__ __launch_bounds__(kWave * kWavesPerBlock) void nvfp4_rope_kernel(const RopeArgs a) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t first = ((int64_t)blockIdx.x * kWavesPerBlock + wave) * kTokensPerWave;
  const float inv6 = (float)(1.0 / 6.0);

  for (int p = 0; p < kTokensPerWave; ++p) {
    const int64_t t = first + p;
    if (t >= a.num_tokens) break;
    float r[8];
    int64_t page_off;
    uint32_t in_page;
    if (!rope_token(a, t, lane, r, page_off, in_page)) continue;

    float amax = max_abs8(r);
    amax = fmaxf(amax, as_f32(dpp<kQuadSwap1>(as_u32(amax))));  // tile = lane pair
    float sf = amax * inv6;
    sf = fminf(fmaxf(sf, 0.001953125f), 448.0f);
    const uint32_t s8 = e4m3x2(sf, sf) & 0xFFu;
    // E4M3 value of s8 (positive): exponent field 0 is m * 2^-9.
    const uint32_t ef = s8 >> 3, mf = s8 & 7u;
    const float S = ef == 0u ? (float)mf * 0.001953125f : as_f32(((ef + 120u) << 23) | (mf << 20));

    float y[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float q = __fdiv_rn(r[i], S);
      q = (q == q) ? q : 0.0f;           // NaN (only without sanitising) -> code 0
      q = fminf(fmaxf(q, -6.0f), 6.0f);  // saturate; leaves [-6, 6] unchanged
      y[i] = q + 0.0f;                   // -0.0 -> +0.0: sign only below zero
    }
    uint32_t codes = 0;
    codes = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(codes, y[0], y[1], 1.0f, 0);
    codes = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(codes, y[2], y[3], 1.0f, 1);
    codes = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(codes, y[4], y[5], 1.0f, 2);
    codes = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(codes, y[6], y[7], 1.0f, 3);

    // Scale dword j = tiles 4j..4j+3 = lanes 8j, 8j+2, 8j+4, 8j+6.
    const uint32_t sdw =
        dpp<kRowShr6>(s8) | (dpp<kRowShr4>(s8) << 8) | (dpp<kRowShr2>(s8) << 16) | (s8 << 24);

    uint8_t* page = a.cache + page_off;
    uint8_t* values = page + (int64_t)in_page * 256;
    uint8_t* scales = page + (int64_t)a.block * 256 + (int64_t)in_page * 32;
    reinterpret_cast<uint32_t*>(values)[lane] = codes;
    if ((lane & 7) == 6) reinterpret_cast<uint32_t*>(scales)[lane >> 3] = sdw;
  }
}

constexpr int kRowHalfMirror = 0x141;  // lane i reads lane 7-i of its half-row

// fp32 -> bf16, nearest-even; NaN -> 0x7FC0.
__device__ __forceinline__ uint32_t bf16_rn(float f) {
  const uint32_t u = as_u32(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__global__ __launch_bounds__(kWave * kWavesPerBlock) void v4_rope_kernel(const RopeArgs a) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t first = ((int64_t)blockIdx.x * kWavesPerBlock + wave) * kTokensPerWave;
  const float inv448 = (float)(1.0 / 448.0);

  for (int p = 0; p < kTokensPerWave; ++p) {
    const int64_t t = first + p;
    if (t >= a.num_tokens) break;
    float r[8];
    int64_t page_off;
    uint32_t in_page;
    if (!rope_token(a, t, lane, r, page_off, in_page)) continue;

    // Group of 64 = lanes 8g..8g+7 (lanes 56..63, the RoPE dims, form their
    // own half-row and their scale is not used).
    float amax = max_abs8(r);
    amax = fmaxf(amax, as_f32(dpp<kQuadSwap1>(as_u32(amax))));
    amax = fmaxf(amax, as_f32(dpp<kQuadSwap2>(as_u32(amax))));
    amax = fmaxf(amax, as_f32(dpp<kRowHalfMirror>(as_u32(amax))));
    amax = fmaxf(amax, 1e-4f);
    const uint32_t vb = as_u32(amax * inv448);
    const int E = (int)((vb >> 23) & 0xFFu) - 127 + ((vb & 0x7FFFFFu) != 0u ? 1 : 0);
    const float mul = E <= 126 ? as_f32((uint32_t)(127 - E) << 23)
                               : as_f32(0x00400000u >> (E - 127));
    int enc = E + 127;
    enc = max(enc, 0);
    enc = min(enc, a.sanitize ? 254 : 255);

    uint8_t* page = a.cache + page_off;
    uint8_t* values = page + (int64_t)in_page * 576;
    uint8_t* scales = page + (int64_t)a.block * 576 + (int64_t)in_page * 8;
    if (lane < 56) {
      float y[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) y[i] = fminf(fmaxf(r[i] * mul, -448.0f), 448.0f);
      const uint32_t lo = e4m3x2(y[0], y[1]) | (e4m3x2(y[2], y[3]) << 16);
      const uint32_t hi = e4m3x2(y[4], y[5]) | (e4m3x2(y[6], y[7]) << 16);
      *reinterpret_cast<u32x2*>(values + lane * 8) = u32x2{lo, hi};
    } else {
      const u32x4 h = {bf16_rn(r[0]) | (bf16_rn(r[1]) << 16), bf16_rn(r[2]) | (bf16_rn(r[3]) << 16),
                       bf16_rn(r[4]) | (bf16_rn(r[5]) << 16), bf16_rn(r[6]) | (bf16_rn(r[7]) << 16)};
      *reinterpret_cast<u32x4*>(values + 448 + (lane - 56) * 16) = h;
    }
    uint32_t s[7];
#pragma unroll
    for (int g = 0; g < 7; ++g) s[g] = (uint32_t)__builtin_amdgcn_readlane(enc, 8 * g);
    if (lane == 0)
      *reinterpret_cast<u32x2*>(scales) =
          u32x2{s[0] | (s[1] << 8) | (s[2] << 16) | (s[3] << 24), s[4] | (s[5] << 8) | (s[6] << 16)};
  }
}

hipError_t launch_rope(void (*kernel)(const RopeArgs), const RopeArgs& a, hipStream_t stream) {
  constexpr int64_t kToksPerBlock = (int64_t)kWavesPerBlock * kTokensPerWave;
  const int64_t blocks = (a.num_tokens + kToksPerBlock - 1) / kToksPerBlock;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(kernel, dim3((unsigned)blocks), dim3(kWave * kWavesPerBlock), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_mxfp8_rope(const RopeArgs& a, hipStream_t stream) {
  return launch_rope(mxfp8_rope_kernel, a, stream);
}

hipError_t launch_nvfp4_rope(const RopeArgs& a, hipStream_t stream) {
  return launch_rope(nvfp4_rope_kernel, a, stream);
}

hipError_t launch_v4_rope(const RopeArgs& a, hipStream_t stream) {
  return launch_rope(v4_rope_kernel, a, stream);
}

}  // namespace mxs
