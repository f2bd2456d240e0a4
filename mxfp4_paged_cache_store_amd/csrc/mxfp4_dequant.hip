// mxfp4_dequant.hip -- gather packed MXFP4 rows of a paged KV cache by slot
// and unpack them to bf16, for gfx950.
//
// What is computed follows the pull request adding the mxfp4_mla cache
// (Details, read path: every E2M1 code times its group's E8M0 scale, as
// bf16; Claims: equal to the dequantized values stored as bf16).  The
// product of a 2-significant-bit E2M1 value and a power of two is exact in
// bf16 unless it reaches 2^128 (then +-Inf); scale byte 0xFF is the E8M0
// NaN and gives the quiet NaN 0x7FC0.
//
// Lane l of a wave reads code dword l of a row (values 8l..8l+7) and the
// scale dword holding its group's byte, and gfx950's
// v_cvt_scalef32_pk_bf16_fp4 expands one code byte into two bf16 values
// scaled by 2^(byte-127) (the scale operand carries the E8M0 byte in an fp32
// exponent field).  Four conversions give the lane's 16 output bytes, stored
// with one non-temporal dwordx4 store.
#include "kernels.hpp"

namespace mxs {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kWavesPerBlock = 4;

__device__ __forceinline__ u32x4 dequant8(uint32_t codes, uint32_t scale_byte) {
  const float scale = as_f32(scale_byte << 23);
  u32x4 r;
  r.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 0));
  r.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 1));
  r.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 2));
  r.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 3));
  if (scale_byte == 0xFFu) r = u32x4{0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u};
  return r;
}

// kSlotsPerWave: passes per wave, 1 for small lists and 2 otherwise (chosen
// at launch from measurements).
template <int LATENT, bool kPow2, int kSlotsPerWave>
__global__ __launch_bounds__(kWave * kWavesPerBlock) void mxfp4_dequant_kernel(const DequantArgs a) {
  constexpr int kLanesPerTok = LATENT >= 512 ? 64 : LATENT / 8;
  constexpr int kToksPerPass = kWave / kLanesPerTok;
  constexpr int kSub = LATENT >= 512 ? LATENT / 512 : 1;
  constexpr int64_t kPitch = LATENT / 2 + LATENT / 32;
  constexpr int kToks = kSlotsPerWave * kToksPerPass;

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int tok_in_pass = lane / kLanesPerTok;
  const int lane_in_tok = lane % kLanesPerTok;
  const int64_t wave_first = ((int64_t)xcd_contiguous_block() * kWavesPerBlock + wave) * kToks;

  uint32_t codes[kSlotsPerWave][kSub];
  uint32_t sdw[kSlotsPerWave][kSub];
  bool ok[kSlotsPerWave];

  int64_t slot[kSlotsPerWave];
  if (wave_first + kToks <= a.n) {
#pragma unroll
    for (int p = 0; p < kSlotsPerWave; ++p)
      slot[p] = a.slots[wave_first + p * kToksPerPass + tok_in_pass];
  } else {
#pragma unroll
    for (int p = 0; p < kSlotsPerWave; ++p) {
      const int64_t i = wave_first + p * kToksPerPass + tok_in_pass;
      slot[p] = i < a.n ? a.slots[i] : -1;
    }
  }

#pragma unroll
  for (int p = 0; p < kSlotsPerWave; ++p) {
    const int64_t s = slot[p];
    ok[p] = s >= 0 && s < (int64_t)a.map.num_slots;
    const uint8_t* row = a.cache + (ok[p] ? a.map.row<kPow2>((uint32_t)s) * kPitch : 0);
    if constexpr (kToksPerPass == 1) {
      // Raw buffer over the row (empty when skipped): branch-free loads.
      // Plain (not non-temporal) loads: measured 3-4% faster from 1M slots
      // and no slower below.
      const __amdgpu_buffer_rsrc_t rs = buffer_at(row, ok[p] ? (uint32_t)kPitch : 0u);
#pragma unroll
      for (int sub = 0; sub < kSub; ++sub) {
        codes[p][sub] = __builtin_amdgcn_raw_buffer_load_b32(rs, sub * 256 + lane_in_tok * 4, 0, 0);
        sdw[p][sub] = __builtin_amdgcn_raw_buffer_load_b32(
            rs, LATENT / 2 + sub * 16 + (lane_in_tok >> 4) * 4, 0, 0);
      }
    } else {
      if (ok[p]) {
        codes[p][0] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(row) + lane_in_tok);
        sdw[p][0] = __builtin_nontemporal_load(
            reinterpret_cast<const uint32_t*>(row + LATENT / 2) + (lane_in_tok >> 4));
      } else {
        codes[p][0] = 0u;
        sdw[p][0] = 0u;
      }
    }
  }

#pragma unroll
  for (int p = 0; p < kSlotsPerWave; ++p) {
    if (!ok[p]) continue;
    const int64_t i = wave_first + (int64_t)p * kToksPerPass + tok_in_pass;
#pragma unroll
    for (int sub = 0; sub < kSub; ++sub) {
      const uint32_t sb = (sdw[p][sub] >> (8 * ((lane_in_tok >> 2) & 3))) & 0xFFu;
      const u32x4 r = dequant8(codes[p][sub], sb);
      __builtin_nontemporal_store(
          r, reinterpret_cast<u32x4*>(a.out + i * a.out_stride + sub * 512 + lane_in_tok * 8));
    }
  }
}

template <int LATENT, int SPW>
hipError_t launch_spw(const DequantArgs& a, hipStream_t stream) {
  constexpr int kLanesPerTok = LATENT >= 512 ? 64 : LATENT / 8;
  constexpr int64_t kToksPerBlock = (int64_t)kWavesPerBlock * SPW * (kWave / kLanesPerTok);
  const int64_t blocks = (a.n + kToksPerBlock - 1) / kToksPerBlock;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  if (a.map.pow2)
    hipLaunchKernelGGL((mxfp4_dequant_kernel<LATENT, true, SPW>), dim3((unsigned)blocks),
                       dim3(kWave * kWavesPerBlock), 0, stream, a);
  else
    hipLaunchKernelGGL((mxfp4_dequant_kernel<LATENT, false, SPW>), dim3((unsigned)blocks),
                       dim3(kWave * kWavesPerBlock), 0, stream, a);
  return hipGetLastError();
}

// Slots per wave (latent 512, random slots; HIP-graph replays and single
// launches after a cache flush): 1 up to 4,096 slots (256 slots 1.92 vs 2.79
// us with 8), 2 above (16,384 slots 4.1 vs 5.1 us, 4.5M slots 1074 vs
// 1139 us); 1 is slower from 65,536 slots on when the rows come from HBM.
template <int LATENT>
hipError_t launch_latent(const DequantArgs& a, hipStream_t stream) {
  if (a.n <= 4096) return launch_spw<LATENT, 1>(a, stream);
  return launch_spw<LATENT, 2>(a, stream);
}

}  // namespace

hipError_t launch_mxfp4_dequant(const DequantArgs& a, int latent, hipStream_t stream) {
  switch (latent) {
    case 128: return launch_latent<128>(a, stream);
    case 256: return launch_latent<256>(a, stream);
    case 512: return launch_latent<512>(a, stream);
    case 1024: return launch_latent<1024>(a, stream);
    case 2048: return launch_latent<2048>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace mxs
