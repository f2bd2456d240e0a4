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
// Layout on CDNA4: a wave quantizes one token at a time (at ratio 1 and from
// 2^16 tokens up, 2 or 4 tokens per wave with every load issued up front);
// lane l holds values 8l..8l+7 (pairs 4l..4l+3), so the RoPE pairs live in
// lanes 56..63, an MXFP8 group is a DPP quad, a V4 group a half-row of 8
// lanes and an NVFP4 tile a lane pair.  E4M3 and E2M1 conversions use
// gfx950's v_cvt_scalef32_pk_fp8_f32 / v_cvt_scalef32_pk_fp4_f32 with scale
// 1.0; the NVFP4 quotient r / S is a product with an fp64 reciprocal that
// leads to the same E2M1 code as the correctly rounded fp32 quotient.  A
// token's value bytes are written through to memory (NT + SC1 buffer
// stores: a page's value area is whole contiguous lines); its scale words go
// through the caches, which merge them.
#include "kernels.hpp"

namespace mxs {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short i16x2 __attribute__((ext_vector_type(2)));

constexpr int kWavesPerBlock = 4;

__device__ __forceinline__ void load_cs(const RopeArgs& a, int64_t base, int lane, float c[4], float sn[4]);
__device__ __forceinline__ void rotate_cs(const RopeArgs& a, const u32x4 w, const float c[4], const float sn[4],
                                          float r[8]);
__device__ __forceinline__ void page_of(const RopeArgs& a, int64_t s, int64_t& page_off, uint32_t& in_page);

// Gate + rotation for one token.  Returns false (uniformly) when the token is
// not written.  On success r[0..7] hold the lane's rotated values.
__device__ __forceinline__ bool rope_token(const RopeArgs& a, int64_t t, int lane,
                                           float r[8], int64_t& page_off, uint32_t& in_page) {
  int64_t s = a.slots[t];
  int64_t pos = a.positions[t];
  // both loads in flight before either is waited for (one round trip)
  asm volatile("" : "+s"(s), "+s"(pos));
  if (s < 0 || s >= (int64_t)a.num_slots) return false;
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
  float c[4], sn[4];
  load_cs(a, base, lane, c, sn);
  rotate_cs(a, w, c, sn, r);
  page_of(a, s, page_off, in_page);
  return true;
}

// cos/sin of the lane's 4 pairs from row `base` (lanes 56..63, the RoPE
// pairs); (1, 0) for the NoPE lanes.  Every lane loads (from a row of the
// table), so the loads need no branch.
__device__ __forceinline__ void load_cs(const RopeArgs& a, int64_t base, int lane, float c[4], float sn[4]) {
  const float* cs = a.cos_sin + base * a.cos_stride + (lane & 7) * 4;
  const bool rope = lane >= 56;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float ci = cs[i], si = cs[32 + i];
    c[i] = rope ? ci : 1.0f;
    sn[i] = rope ? si : 0.0f;
  }
}

// The lane's 8 values of a token after the rotation, NaN -> +0 when
// sanitising.
__device__ __forceinline__ void rotate_cs(const RopeArgs& a, const u32x4 w, const float c[4], const float sn[4],
                                          float r[8]) {
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
    // A NaN among the lane's values makes their sum NaN (so can Inf - Inf,
    // which only costs the replacement pass); waves with no such lane skip
    // the per-value replacement.
    const float sum = ((r[0] + r[1]) + (r[2] + r[3])) + ((r[4] + r[5]) + (r[6] + r[7]));
    if (__builtin_amdgcn_ballot_w64(sum != sum)) {
#pragma unroll
      for (int i = 0; i < 8; ++i) r[i] = (r[i] == r[i]) ? r[i] : 0.0f;
    }
  }
}

// Page byte offset and row within the page of a valid slot.
__device__ __forceinline__ void page_of(const RopeArgs& a, int64_t s, int64_t& page_off, uint32_t& in_page) {
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

// Four fp32 -> four E4M3 bytes in one dword, a first: the second convert
// writes the upper half-word of the first one's result.
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
  i16x2 p = {0, 0};
  p = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(p, a, b, 1.0f, false);
  p = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(p, c, d, 1.0f, true);
  return __builtin_bit_cast(uint32_t, p);
}

// MXFP8 record of one token (r: the lane's rotated values).
struct Mxfp8 {
  static constexpr int kTpw = 2;  // tokens per wave at ratio 1 (measured)
  static __device__ __forceinline__ void finish(const RopeArgs& a, int lane, const float r[8],
                                                int64_t page_off, uint32_t in_page) {
    const float inv448 = (float)(1.0 / 448.0);
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
    const uint32_t lo = e4m3x4(y[0], y[1], y[2], y[3]);
    const uint32_t hi = e4m3x4(y[4], y[5], y[6], y[7]);

    int enc = E + 127;
    enc = max(enc, 0);
    enc = min(enc, a.sanitize ? 254 : 255);
    const uint32_t sb = (uint32_t)enc;
    const uint32_t sdw =
        dpp<kRowShr12>(sb) | (dpp<kRowShr8>(sb) << 8) | (dpp<kRowShr4>(sb) << 16) | (sb << 24);

    uint8_t* page = a.cache + page_off;
    uint8_t* values = page + (int64_t)in_page * 512;
    uint8_t* scales = page + (int64_t)a.block * 512 + (int64_t)in_page * 16;
    // Value areas of a page are contiguous whole lines: streamed to memory
    // (NT + SC1); the scattered 4-byte scale words go through the caches.
    __builtin_amdgcn_raw_buffer_store_b64(u32x2{lo, hi}, buffer_at(values, 512), lane * 8, 0, kBufNTDevice);
    if ((lane & 15) == 12) reinterpret_cast<uint32_t*>(scales)[lane >> 4] = sdw;
  }
};

// NVFP4 record of one token.
struct Nvfp4 {
  static constexpr int kTpw = 4;
  // With sanitising on, r holds no NaN, and neither can the quotient (S is
  // finite and positive), so its NaN check is left out of that branch.
  static __device__ __forceinline__ void finish(const RopeArgs& a, int lane, const float r[8],
                                                int64_t page_off, uint32_t in_page) {
    if (a.sanitize)
      finish_impl<false>(a, lane, r, page_off, in_page);
    else
      finish_impl<true>(a, lane, r, page_off, in_page);
  }

  template <bool kNaN>
  static __device__ __forceinline__ void finish_impl(const RopeArgs& a, int lane, const float r[8],
                                                     int64_t page_off, uint32_t in_page) {
    const float inv6 = (float)(1.0 / 6.0);
    float amax = max_abs8(r);
    amax = fmaxf(amax, as_f32(dpp<kQuadSwap1>(as_u32(amax))));  // tile = lane pair
    float sf = amax * inv6;
    sf = fminf(fmaxf(sf, 0.001953125f), 448.0f);
    const uint32_t s8 = e4m3x2(sf, sf) & 0xFFu;
    // E4M3 value of s8 (positive): exponent field 0 is m * 2^-9.
    const uint32_t ef = s8 >> 3, mf = s8 & 7u;
    const float S = ef == 0u ? (float)mf * 0.001953125f : as_f32(((ef + 120u) << 23) | (mf << 20));

    // r / S without a division.  S has at most 4 significant bits, so in the
    // fp32 normal range r / S is never halfway between two floats and lies
    // at least 2^-30 (relative) from every such halfway point.  In fp32:
    // q0 = r * y0 (y0 the 1-ulp hardware reciprocal), the residual
    // e = r - q0 * S in one fma (exact: it has at most 6 significant bits
    // unless it underflows), then q = q0 + e * y0 in one fma, within 2^-45
    // of r / S: it rounds to the same float.  Where q is not a normal float
    // (a zero, subnormal, infinite or NaN quotient, or a residual that
    // underflowed) the lane redoes its 8 values as r * (1/S) in fp64 with
    // 1/S known to within 2^-43 and taken low by 2^-51..2^-43, so that the
    // product is always smaller in magnitude than r / S; then in the
    // subnormal range, where only the sign reaches the code, a quotient of
    // exactly half the smallest subnormal rounds to zero as
    // round-to-nearest-even does.  (1/S there: one Newton step in fp64 from
    // y0; the step's residual is exact and leaves the estimate low by its
    // error squared.)  A host check restates both and compares the codes
    // with those of the correctly rounded quotient.
    const float y0 = __builtin_amdgcn_rcpf(S);
    float y[8];
    bool slow = false;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float q0 = r[i] * y0;
      const float e = __builtin_fmaf(-q0, S, r[i]);
      y[i] = __builtin_fmaf(e, y0, q0);
      slow |= !__builtin_isnormal(y[i]);
    }
    if (slow) {
      const double sd = S, yd = y0;
      const double inv_s = __builtin_fma(yd, __builtin_fma(-sd, yd, 1.0), yd) * (1.0 - 0x1p-50);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        float q = (float)((double)r[i] * inv_s);
        if (kNaN) q = (q == q) ? q : 0.0f;  // NaN -> code 0 (the converter gives 7)
        y[i] = q + 0.0f;                    // -0.0 -> +0.0: sign only below zero
      }
    }
    // The converter saturates: magnitudes above 6, up to +-Inf, give code 7
    // with the sign (checked on the device), as the E2M1 rule asks.
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
    __builtin_amdgcn_raw_buffer_store_b32(codes, buffer_at(values, 256), lane * 4, 0, kBufNTDevice);
    if ((lane & 7) == 6) reinterpret_cast<uint32_t*>(scales)[lane >> 3] = sdw;
  }
};

constexpr int kRowHalfMirror = 0x141;  // lane i reads lane 7-i of its half-row

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Two fp32 -> a bf16 pair (lo in the low half), nearest-even, by the
// hardware converter; not for NaN (whose payload it may keep).
__device__ __forceinline__ uint32_t bf16x2_hw(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

// fp32 -> bf16, nearest-even; NaN -> 0x7FC0.
__device__ __forceinline__ uint32_t bf16_rn(float f) {
  const uint32_t u = as_u32(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// V4 record of one token.
struct V4 {
  static constexpr int kTpw = 2;
  // With sanitising on, r holds no NaN and the RoPE values take gfx950's
  // bf16 pack (v_cvt_pk_bf16_f32), which rounds every non-NaN fp32 exactly
  // as bf16_rn does (checked on the device over all 2^32 bit patterns);
  // otherwise bf16_rn keeps NaN at 0x7FC0.
  static __device__ __forceinline__ void finish(const RopeArgs& a, int lane, const float r[8],
                                                int64_t page_off, uint32_t in_page) {
    if (a.sanitize)
      finish_impl<true>(a, lane, r, page_off, in_page);
    else
      finish_impl<false>(a, lane, r, page_off, in_page);
  }

  template <bool kNoNaN>
  static __device__ __forceinline__ void finish_impl(const RopeArgs& a, int lane, const float r[8],
                                                     int64_t page_off, uint32_t in_page) {
    const float inv448 = (float)(1.0 / 448.0);
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
      const uint32_t lo = e4m3x4(y[0], y[1], y[2], y[3]);
      const uint32_t hi = e4m3x4(y[4], y[5], y[6], y[7]);
      __builtin_amdgcn_raw_buffer_store_b64(u32x2{lo, hi}, buffer_at(values, 576), lane * 8, 0, kBufNTDevice);
    } else {
      u32x4 h;
      if (kNoNaN) {
        h = u32x4{bf16x2_hw(r[0], r[1]), bf16x2_hw(r[2], r[3]), bf16x2_hw(r[4], r[5]), bf16x2_hw(r[6], r[7])};
      } else {
        h = u32x4{bf16_rn(r[0]) | (bf16_rn(r[1]) << 16), bf16_rn(r[2]) | (bf16_rn(r[3]) << 16),
                  bf16_rn(r[4]) | (bf16_rn(r[5]) << 16), bf16_rn(r[6]) | (bf16_rn(r[7]) << 16)};
      }
      __builtin_amdgcn_raw_buffer_store_b128(h, buffer_at(values, 576), 448 + (lane - 56) * 16, 0, kBufNTDevice);
    }
    uint32_t s[7];
#pragma unroll
    for (int g = 0; g < 7; ++g) s[g] = (uint32_t)__builtin_amdgcn_readlane(enc, 8 * g);
    if (lane == 0)
      *reinterpret_cast<u32x2*>(scales) =
          u32x2{s[0] | (s[1] << 8) | (s[2] << 16) | (s[3] << 24), s[4] | (s[5] << 8) | (s[6] << 16)};
  }
};

// One wave per token; TPW tokens per wave.  kCr1 (compress ratio 1: every
// token with a valid slot is written): the wave's latent rows are loaded
// before, and independent of, its slots and positions, which come in one
// vector load each (lane p holds token p's; vector loads return in order, so
// waiting for them leaves the rows in flight), and all cos/sin loads are
// issued before any rotation.  Otherwise (a ratio that writes one token in
// cr) a token's row is loaded only once its gate has passed.
template <class F, int TPW, bool kCr1>
__global__ __launch_bounds__(kWave * kWavesPerBlock) void rope_kernel(const RopeArgs a) {
  static_assert(TPW >= 1 && TPW <= kWave && (TPW & (TPW - 1)) == 0, "lane p holds token p's slot");
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t first = ((int64_t)blockIdx.x * kWavesPerBlock + wave) * TPW;
  if constexpr (kCr1) {
    const int64_t last = a.num_tokens - 1;
    u32x4 w[TPW];
#pragma unroll
    for (int p = 0; p < TPW; ++p) {
      const int64_t t = first + p;
      w[p] = *reinterpret_cast<const u32x4*>(a.latent + (t < last ? t : last) * 512 + lane * 8);
    }
    const int64_t tl = first + (lane & (TPW - 1));
    int64_t vs = a.slots[tl < last ? tl : last];
    int64_t vp = a.positions[tl < last ? tl : last];
    // keeps the row loads above the slot arithmetic and its wait
    asm volatile("" : "+v"(vs), "+v"(vp) : : "memory");
    int64_t slot[TPW];
    bool ok[TPW];
    float c[TPW][4], sn[TPW][4];
#pragma unroll
    for (int p = 0; p < TPW; ++p) {
      slot[p] = (int64_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readlane((uint32_t)((uint64_t)vs >> 32), p) << 32) |
                          (uint32_t)__builtin_amdgcn_readlane((uint32_t)vs, p));
      const int64_t pos =
          (int64_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readlane((uint32_t)((uint64_t)vp >> 32), p) << 32) |
                    (uint32_t)__builtin_amdgcn_readlane((uint32_t)vp, p));
      ok[p] = first + p < a.num_tokens && slot[p] >= 0 && slot[p] < (int64_t)a.num_slots && pos >= 0 &&
              pos < a.cos_rows;
      load_cs(a, ok[p] ? pos : 0, lane, c[p], sn[p]);
    }
#pragma unroll
    for (int p = 0; p < TPW; ++p) {
      if (!ok[p]) continue;
      float r[8];
      rotate_cs(a, w[p], c[p], sn[p], r);
      int64_t page_off;
      uint32_t in_page;
      page_of(a, slot[p], page_off, in_page);
      F::finish(a, lane, r, page_off, in_page);
    }
  } else {
    for (int p = 0; p < TPW; ++p) {
      const int64_t t = first + p;
      if (t >= a.num_tokens) break;
      float r[8];
      int64_t page_off;
      uint32_t in_page;
      if (!rope_token(a, t, lane, r, page_off, in_page)) continue;
      F::finish(a, lane, r, page_off, in_page);
    }
  }
}

template <class F>
hipError_t launch_rope(const RopeArgs& a, hipStream_t stream) {
  // Ratio 1 with a table: F::kTpw tokens per wave from 2^16 tokens up, else
  // one (small batches are latency-bound: more, shorter waves finish sooner).
  const bool cr1 = a.cr == 1 && a.cos_rows >= 1;
  const int tpw = cr1 && a.num_tokens >= (int64_t(1) << 16) ? F::kTpw : 1;
  const int64_t per_block = (int64_t)kWavesPerBlock * tpw;
  const int64_t blocks = (a.num_tokens + per_block - 1) / per_block;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)blocks), block(kWave * kWavesPerBlock);
  if (!cr1)
    hipLaunchKernelGGL((rope_kernel<F, 1, false>), grid, block, 0, stream, a);
  else if (tpw > 1)
    hipLaunchKernelGGL((rope_kernel<F, F::kTpw, true>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((rope_kernel<F, 1, true>), grid, block, 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_mxfp8_rope(const RopeArgs& a, hipStream_t stream) { return launch_rope<Mxfp8>(a, stream); }

hipError_t launch_nvfp4_rope(const RopeArgs& a, hipStream_t stream) { return launch_rope<Nvfp4>(a, stream); }

hipError_t launch_v4_rope(const RopeArgs& a, hipStream_t stream) { return launch_rope<V4>(a, stream); }

}  // namespace mxs
