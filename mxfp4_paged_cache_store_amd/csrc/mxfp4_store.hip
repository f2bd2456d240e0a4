// mxfp4_store.hip -- MXFP4 quantize-and-scatter of a bf16 MLA latent into a
// paged KV cache, for gfx950.
//
// What is computed follows the store page ("vllm.v1.attention.ops.mxfp4_mla.
// store": `_ceil_pow2_exponent`, `_quantize_e2m1`, `store_mxfp4_mla`) and the
// pull request adding the mxfp4_mla cache (Overview, Details); how it is
// computed is specific to CDNA4:
//
//   * One wavefront owns one 512-value slice of a token per pass: lane l
//     loads 16 bytes (values 8l..8l+7) with a non-temporal dwordx4 load, so a
//     pass reads one whole 1024-byte latent row, fully coalesced.  A wave
//     issues the loads of TOKENS_PER_WAVE tokens before it computes any, to
//     keep enough bytes in flight for HBM.
//   * A 32-value group is exactly the 4 lanes of a DPP quad: the group amax
//     is a packed-u16 max over the lane's |bf16| bit patterns followed by two
//     quad_perm DPP maxes.  |bf16| bit patterns order like the magnitudes.
//   * The scale exponent comes straight from the amax bit pattern with
//     integer ops.  For a bf16 amax = 2^(E-127) * (1 + m/128), the smallest
//     e with 2^e >= amax/6 is E - 129 when m <= 64 and E - 128 when m > 64
//     (1 + m/128 > 1.5 exactly when m > 64, and amax/6 never rounds onto a
//     power of two from above in fp32); it is floored at -126 as the fp32 bit
//     pattern of a subnormal amax/6 reads.
//   * Each value is multiplied by 2^-e in fp32 (the same single rounding as a
//     division by 2^e, with gradual underflow), +0.0 is added so that a zero
//     quotient carries no sign, and gfx950's v_cvt_scalef32_pk_fp4_f32 (scale
//     1.0) rounds two quotients to E2M1 codes, nearest-even, sign kept:
//     four conversions give the lane's 8 codes as one dword, which is code
//     dword l of the row (low nibble = lower index).  For e <= 16 (every
//     group below 6 * 2^16) the quotient never underflows, and the packed
//     bf16 values go straight to v_cvt_scalef32_pk_fp4_bf16 with scale 2^e,
//     zeros' signs cleared first: the same codes (encode8_bf16).
//   * The scatter form with one token per pass writes a row as 64 code
//     dwords and one byte store of the 16 scale bytes (each lane stores its
//     group's byte; the four lanes of a group write the same byte).  Where a
//     pass holds several tokens, and in the slot-order form, the scale bytes
//     are gathered with row_shr DPP moves into four dwords held by lanes 12,
//     28, 44 and 60, and the row is written as whole dwords.  When a wave's tokens fill
//     consecutive slots, or the whole batch's rows fit in the Infinity
//     Cache, the stores are plain (L2 and that cache merge neighbouring rows
//     into whole lines); other scattered rows use non-temporal stores.
//   * A wave's slots come in one vector load issued ahead of its rows.  In
//     batches of up to 16,384 tokens (bound by latency) the rows do not wait
//     for them: a pad or out-of-range slot skips the token's store (its row
//     is read and dropped).  Larger batches wait for the slots and read the
//     rows of written tokens only, so pads cost no row traffic.  Loads and stores go
//     through raw buffer descriptors whose range is the token's row / the
//     slot's row, empty past the batch or for a skipped slot (the hardware
//     range check returns zeros or drops the access without touching
//     memory).  Latents below 512 put several tokens in a pass and skip a
//     pad token's load too.  All addressing is 64-bit.
//   * The slot-order form, for dense scattered batches larger than the
//     Infinity Cache, turns the scatter into a gather: an inverse map
//     (slot -> token, built by a fill and one scattered int32 write per
//     token) lets each wave walk 4 consecutive slots, load their tokens' rows,
//     quantize them, assemble the 4 rows in LDS and write them as 16-byte
//     chunks of one contiguous span, written through to memory (NT + SC1).
#include <mutex>

#include "kernels.hpp"

namespace mxs {

// Inverse map of the allocation-free slot-order store, one int32 per slot.
// Every GPU the library runs on holds its own copy until the process ends.
// In host code this name is only a stand-in for the symbol: the device
// address comes from hipGetSymbolAddress (scratch_of_current_device).
static __device__ __align__(256) int32_t scratch[kNoAllocScratchBytes / 4];

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kWavesPerBlock = 4;

__device__ __forceinline__ uint32_t pk_max_u16(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2, a),
                                                                __builtin_bit_cast(u16x2, b)));
}

// Largest |bf16| bit pattern over the lane's 8 values and its quad (32 values).
__device__ __forceinline__ uint32_t group_amax_bits(const u32x4 w) {
  const uint32_t m = 0x7FFF7FFFu;
  uint32_t x = pk_max_u16(pk_max_u16(w.x & m, w.y & m), pk_max_u16(w.z & m, w.w & m));
  x = pk_max_u16(x, __builtin_amdgcn_alignbit(x, x, 16)) & 0xFFFFu;
  x = max(x, dpp<kQuadSwap1>(x));
  x = max(x, dpp<kQuadSwap2>(x));
  return x;
}

// 8 E2M1 codes of the lane's values divided by 2^e, where mul = 2^-e.
__device__ __forceinline__ uint32_t encode8(const u32x4 w, float mul) {
  float l0 = as_f32(w.x << 16) * mul, h0 = as_f32(w.x & 0xFFFF0000u) * mul;
  float l1 = as_f32(w.y << 16) * mul, h1 = as_f32(w.y & 0xFFFF0000u) * mul;
  float l2 = as_f32(w.z << 16) * mul, h2 = as_f32(w.z & 0xFFFF0000u) * mul;
  float l3 = as_f32(w.w << 16) * mul, h3 = as_f32(w.w & 0xFFFF0000u) * mul;
  // A quotient that is -0.0 (from -0.0 or from underflow) does not compare
  // below zero and must encode as code 0; x + 0.0 maps -0.0 to +0.0 and
  // leaves every other value unchanged.
  l0 += 0.0f; h0 += 0.0f; l1 += 0.0f; h1 += 0.0f;
  l2 += 0.0f; h2 += 0.0f; l3 += 0.0f; h3 += 0.0f;
  uint32_t c = 0;
  c = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c, l0, h0, 1.0f, 0);
  c = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c, l1, h1, 1.0f, 1);
  c = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c, l2, h2, 1.0f, 2);
  c = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c, l3, h3, 1.0f, 3);
  return c;
}

// The same codes for groups with e <= kBf16MaxE, from the packed bf16
// values: gfx950's v_cvt_scalef32_pk_fp4_bf16 with scale 2^e rounds the
// exact quotient x / 2^e to E2M1.  For those e the fp32 quotient x * 2^-e
// is exact too (|x| >= 2^-133, a multiple of 2^-133, so x * 2^-e is a
// multiple of 2^-149 and never underflows), so the two round the same value;
// a device sweep of every bf16 value against encode8 for every e in [-126,
// 126] found no difference up to 16 and, from 17 on, only negatives whose
// fp32 quotient underflows to -0.0 (code 0 there, 8 from the converter).  A
// zero's sign is cleared first (-0.0 encodes as code 0): for each half,
// (|h| + 0x7FFF) has bit 15 set exactly when |h| is not 0.
constexpr int kBf16MaxE = 16;
__device__ __forceinline__ uint32_t encode8_bf16(const u32x4 w, float scale) {
  uint32_t c = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t m = w[k] & 0x7FFF7FFFu;
    const uint32_t z = ((m + 0x7FFF7FFFu) & w[k]) | m;
    switch (k) {
      case 0: c = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(c, __builtin_bit_cast(bf16x2, z), scale, 0); break;
      case 1: c = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(c, __builtin_bit_cast(bf16x2, z), scale, 1); break;
      case 2: c = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(c, __builtin_bit_cast(bf16x2, z), scale, 2); break;
      default: c = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(c, __builtin_bit_cast(bf16x2, z), scale, 3); break;
    }
  }
  return c;
}

// Quantizes the 512-value slice held by the wave (16 bytes per lane):
// returns the lane's code dword (codes of its 8 values) and, in
// `scale_byte`, the scale byte of the lane's group (lanes 4g .. 4g+3 hold
// group g).
__device__ __forceinline__ uint32_t quantize_slice_sb(const u32x4 w, uint32_t& scale_byte) {
  const uint32_t amax = group_amax_bits(w);
  const bool nonfinite = amax >= 0x7F80u;
  int e = (int)(amax >> 7) - 129 + ((amax & 0x7Fu) > 64u ? 1 : 0);
  e = max(e, -126);
  if (amax == 0u || nonfinite) e = 0;
  scale_byte = nonfinite ? 0xFFu : (uint32_t)(e + 127);
  uint32_t codes;
  if (e <= kBf16MaxE) {
    codes = encode8_bf16(w, as_f32((uint32_t)(127 + e) << 23));  // 2^e
  } else {
    codes = encode8(w, as_f32((uint32_t)(127 - e) << 23));  // 2^-e, e in [17, 126]
  }
  if (nonfinite) codes = 0u;
  return codes;
}

// As quantize_slice_sb, with the scale bytes gathered into the scale dword
// that the lanes 12 mod 16 store: dword k = groups 4k..4k+3 = lanes 16k,
// 16k+4, 16k+8, 16k+12.
__device__ __forceinline__ uint32_t quantize_slice(const u32x4 w, uint32_t& sdw) {
  uint32_t scale_byte;
  const uint32_t codes = quantize_slice_sb(w, scale_byte);
  sdw = dpp<kRowShr12>(scale_byte) | (dpp<kRowShr8>(scale_byte) << 8) |
        (dpp<kRowShr4>(scale_byte) << 16) | (scale_byte << 24);
  return codes;
}

// LATENT: values per token (power of two, 128..2048).  A token occupies
// min(LATENT/8, 64) lanes per pass; LATENT > 512 takes LATENT/512 passes.
// kPow2: slot -> row by shift/mask (else a 32-bit division).
// kTokensPerWave: passes per wave (1, 2 or 4 by batch size: measured).
// kSlotFirst (one token per pass): request a token's row only once its slot
// is known, so pads cost no row read; otherwise the rows are requested
// before the slots arrive (and a pad's row is read and dropped).
template <int LATENT, bool kPow2, int kTokensPerWave, bool kSlotFirst>
__global__ __launch_bounds__(kWave * kWavesPerBlock) void mxfp4_store_kernel(const StoreArgs a) {
  constexpr int kLanesPerTok = LATENT >= 512 ? 64 : LATENT / 8;
  constexpr int kToksPerPass = kWave / kLanesPerTok;
  constexpr int kSub = LATENT >= 512 ? LATENT / 512 : 1;
  constexpr int64_t kPitch = LATENT / 2 + LATENT / 32;
  constexpr int kToks = kTokensPerWave * kToksPerPass;  // tokens per wave

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int tok_in_pass = lane / kLanesPerTok;
  const int lane_in_tok = lane % kLanesPerTok;
  const int64_t wave_first = ((int64_t)xcd_contiguous_block() * kWavesPerBlock + wave) * kToks;

  int64_t slot[kTokensPerWave];
  u32x4 v[kTokensPerWave][kSub];
  if constexpr (kToksPerPass == 1) {
    // Whole wave on one token per pass.  The wave's slots come in one
    // vector load (lane p & (kTokensPerWave-1) reads pass p's), issued
    // before the rows: vector loads return in order, so waiting for the
    // slots leaves the row loads in flight, where a scalar load would be
    // waited for together with every other scalar load.
    const int64_t last = a.num_tokens - 1;
    const int64_t tl = wave_first + (lane & (kTokensPerWave - 1));
    const int64_t vs = a.slots[tl < last ? tl : last];
    // kSlotFirst: wait for the slots and request only the rows of tokens
    // that are written (a pad's row is never read).
    bool want[kTokensPerWave];
#pragma unroll
    for (int p = 0; p < kTokensPerWave; ++p) {
      if constexpr (kSlotFirst) {
        const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)vs, p);
        const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)((uint64_t)vs >> 32), p);
        const int64_t s = (int64_t)(((uint64_t)hi << 32) | lo);
        want[p] = s >= 0 && s < (int64_t)a.map.num_slots;
      } else {
        want[p] = true;
      }
    }
#pragma unroll
    for (int p = 0; p < kTokensPerWave; ++p) {
      // Raw buffer over the token's row, empty past the batch or for a
      // skipped token: no branch.
      const int64_t t = wave_first + p;
      const bool have = t < a.num_tokens && want[p];
      const __amdgpu_buffer_rsrc_t rs =
          buffer_at(a.src + (have ? t * a.src_stride : 0), have ? LATENT * 2 : 0);
#pragma unroll
      for (int sub = 0; sub < kSub; ++sub)
        v[p][sub] = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, (sub * 64 + lane_in_tok) * 16, 0, kBufNT));
    }
    // Keeps the row loads above this point (the compiler would otherwise
    // sink them below the slot arithmetic and its wait).
    int64_t vs_ready = vs;
    asm volatile("" : "+v"(vs_ready) : : "memory");
#pragma unroll
    for (int p = 0; p < kTokensPerWave; ++p) {
      const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)vs_ready, p);
      const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)((uint64_t)vs_ready >> 32), p);
      slot[p] = wave_first + p < a.num_tokens ? (int64_t)(((uint64_t)hi << 32) | lo) : -1;
    }
  } else {
    // Several tokens per pass: one merged load of the slots when the wave
    // is whole; rows of skipped tokens are not read.
    if (wave_first + kToks <= a.num_tokens) {
#pragma unroll
      for (int p = 0; p < kTokensPerWave; ++p)
        slot[p] = a.slots[wave_first + p * kToksPerPass + tok_in_pass];
    } else {
#pragma unroll
      for (int p = 0; p < kTokensPerWave; ++p) {
        const int64_t t = wave_first + p * kToksPerPass + tok_in_pass;
        slot[p] = t < a.num_tokens ? a.slots[t] : -1;
      }
    }
#pragma unroll
    for (int p = 0; p < kTokensPerWave; ++p) {
      const int64_t t = wave_first + p * kToksPerPass + tok_in_pass;
      if (slot[p] >= 0 && slot[p] < (int64_t)a.map.num_slots) {
        const u32x4* src = reinterpret_cast<const u32x4*>(a.src + t * a.src_stride + lane_in_tok * 8);
        v[p][0] = __builtin_nontemporal_load(src);
      } else {
        v[p][0] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  }

  int64_t row_off[kTokensPerWave];
#pragma unroll
  for (int p = 0; p < kTokensPerWave; ++p) {
    const bool ok = slot[p] >= 0 && slot[p] < (int64_t)a.map.num_slots;
    row_off[p] = ok ? a.map.row<kPow2>((uint32_t)slot[p]) * kPitch : -1;
  }

  // A wave whose tokens fill consecutive slots writes adjacent rows: plain
  // stores let L2 assemble whole lines from them.  Scattered rows are
  // streamed with non-temporal stores instead (measured faster for rows
  // whose neighbours are written at unrelated times), unless the whole
  // batch fits in the Infinity Cache (plain_stores), where the partial lines
  // of neighbouring rows merge before they are written back.
  bool run = true;
#pragma unroll
  for (int p = 1; p < kTokensPerWave; ++p) run = run && slot[p] == slot[p - 1] + kToksPerPass;
  run = (run && row_off[0] >= 0 && row_off[kTokensPerWave - 1] >= 0) || a.plain_stores;

#pragma unroll
  for (int p = 0; p < kTokensPerWave; ++p) {
    if constexpr (kToksPerPass == 1) {
      // Raw buffer over the token's row (empty when skipped): the hardware
      // range check drops the stores of a skipped token.  Every lane stores
      // its group's scale byte (the four lanes of a group the same byte at
      // the same offset), one byte store per slice.  The two cache policies
      // are distinct instructions, so they stay separate.
      const bool ok = row_off[p] >= 0;
      const __amdgpu_buffer_rsrc_t rs =
          buffer_at(a.cache + (ok ? row_off[p] : 0), ok ? (uint32_t)kPitch : 0u);
#pragma unroll
      for (int sub = 0; sub < kSub; ++sub) {
        uint32_t sb;
        const uint32_t codes = quantize_slice_sb(v[p][sub], sb);
        const uint32_t code_off = sub * 256 + lane_in_tok * 4;
        const uint32_t scale_off = LATENT / 2 + sub * 16 + (lane_in_tok >> 2);
        if (run) {
          __builtin_amdgcn_raw_buffer_store_b32(codes, rs, code_off, 0, 0);
          __builtin_amdgcn_raw_buffer_store_b8((uint8_t)sb, rs, scale_off, 0, 0);
        } else {
          __builtin_amdgcn_raw_buffer_store_b32(codes, rs, code_off, 0, kBufNT);
          __builtin_amdgcn_raw_buffer_store_b8((uint8_t)sb, rs, scale_off, 0, kBufNT);
        }
      }
    } else {
      uint32_t sdw;
      const uint32_t codes = quantize_slice(v[p][0], sdw);
      if (row_off[p] < 0) continue;
      uint32_t* code_dst = reinterpret_cast<uint32_t*>(a.cache + row_off[p]) + lane_in_tok;
      if (run) *code_dst = codes; else __builtin_nontemporal_store(codes, code_dst);
      if ((lane_in_tok & 15) == 12) {
        uint32_t* scale_dst = reinterpret_cast<uint32_t*>(a.cache + row_off[p] + LATENT / 2) + (lane_in_tok >> 4);
        if (run) *scale_dst = sdw; else __builtin_nontemporal_store(sdw, scale_dst);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Slot-order form.  For a batch that fills most of the cache's slots in a
// scattered order (e.g. a random permutation), scattered 272-byte row writes
// are the bottleneck: DRAM serves random 1 KiB reads at nearly full speed but
// random sub-line writes at well under half.  So the scatter is inverted:
// inv[s] = t is built once per slot mapping (it serves every layer that
// stores with that mapping), then waves walk slots in order, gather the token
// row inv[s] (or nothing) and write rows sequentially.  For distinct slots the
// bytes written are identical to the scatter form's.  A slot named by several
// tokens races in both: here the whole row of the token whose inverse entry
// won lands, while the scatter form may mix one token's code dwords with
// another's scale dwords.

constexpr int kSlotsPerWave = 4;

__global__ __launch_bounds__(256) void fill_inverse(int32_t* __restrict__ inv, int64_t n) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i + 4 <= n) {
    *reinterpret_cast<u32x4*>(inv + i) = u32x4{0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu};
  } else {
    for (int64_t k = i; k < n; ++k) inv[k] = -1;
  }
}

__global__ __launch_bounds__(256) void invert_slots(const int64_t* __restrict__ slots, int64_t n,
                                                    int32_t* __restrict__ inv, uint32_t num_slots) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= n) return;
  const int64_t s = slots[t];
  if (s >= 0 && s < (int64_t)num_slots) inv[s] = (int32_t)t;
}

// kStaged: the wave's kSlotsPerWave slots are consecutive rows of the cache (a
// flat cache, or a block size that is a multiple of kSlotsPerWave; 16-byte
// aligned), so its rows form one contiguous span; they are assembled in LDS and written as 16-byte chunks
// (row pitches are multiples of 16, so a chunk never straddles two rows and a
// skipped row's chunks are simply dropped).  Otherwise each row is written
// with dword stores.
template <int LATENT, bool kPow2, bool kStaged>
__global__ __launch_bounds__(kWave * kWavesPerBlock) void mxfp4_store_by_slot_kernel(
    const StoreArgs a, const int32_t* __restrict__ inv) {
  static_assert(LATENT >= 512, "slot order is used for latents of 512 and more");
  constexpr int kSub = LATENT / 512;
  constexpr int64_t kPitch = LATENT / 2 + LATENT / 32;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t s0 = ((int64_t)xcd_contiguous_block() * kWavesPerBlock + wave) * kSlotsPerWave;
  const int64_t num_slots = a.map.num_slots;

  int32_t tok[kSlotsPerWave];
  if (s0 + kSlotsPerWave <= num_slots) {
#pragma unroll
    for (int p = 0; p < kSlotsPerWave; ++p) tok[p] = inv[s0 + p];
  } else {
#pragma unroll
    for (int p = 0; p < kSlotsPerWave; ++p) tok[p] = s0 + p < num_slots ? inv[s0 + p] : -1;
  }
  // An entry is a token of this batch or -1; anything else is skipped.
#pragma unroll
  for (int p = 0; p < kSlotsPerWave; ++p)
    if ((int64_t)tok[p] >= a.num_tokens) tok[p] = -1;

  u32x4 v[kSlotsPerWave][kSub];
#pragma unroll
  for (int p = 0; p < kSlotsPerWave; ++p) {
    const bool ok = tok[p] >= 0;
    const __amdgpu_buffer_rsrc_t rs =
        buffer_at(a.src + (ok ? (int64_t)tok[p] * a.src_stride : 0), ok ? LATENT * 2 : 0);
#pragma unroll
    for (int sub = 0; sub < kSub; ++sub)
      v[p][sub] = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, (sub * 64 + lane) * 16, 0, kBufNT));
  }

  constexpr uint32_t kDrop = 0x7FFFFFF0u;
  if constexpr (kStaged) {
    constexpr int kSpan = kSlotsPerWave * (int)kPitch;  // bytes of the wave's rows
    __shared__ uint32_t stage[kWavesPerBlock][kSpan / 4];
    uint32_t* st = stage[wave];
    uint32_t valid = 0;
#pragma unroll
    for (int p = 0; p < kSlotsPerWave; ++p) {
      valid |= (tok[p] >= 0 ? 1u : 0u) << p;
#pragma unroll
      for (int sub = 0; sub < kSub; ++sub) {
        uint32_t sdw;
        const uint32_t codes = quantize_slice(v[p][sub], sdw);
        st[(p * (int)kPitch + sub * 256) / 4 + lane] = codes;
        if ((lane & 15) == 12) st[(p * (int)kPitch + LATENT / 2 + sub * 16) / 4 + (lane >> 4)] = sdw;
      }
    }
    // Each lane reads back chunks written by other lanes of the wave: the
    // fences order the LDS writes before the barrier and the reads after it
    // for the compiler (the hardware keeps one wave's LDS accesses in order).
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // Rows go out in slot order as whole 16-byte chunks of a contiguous span,
    // streamed through to memory (NT + SC1): measured on the 4.5M-token
    // batch, 1136 -> 1074 us per step back to back (the previous step's
    // dirty lines no longer drain during this one), 1121 -> 1082 us after a
    // cache flush, and 1062 -> 958 us for prefill-style runs of slots.
    const __amdgpu_buffer_rsrc_t rs =
        buffer_at(a.cache + a.map.row<kPow2>((uint32_t)s0) * kPitch, (uint32_t)kSpan);
#pragma unroll
    for (int c0 = 0; c0 < kSpan / 16; c0 += kWave) {
      const int c = c0 + lane;
      if (c0 + kWave <= kSpan / 16 || c < kSpan / 16) {
        const u32x4 d = *reinterpret_cast<const u32x4*>(&st[4 * c]);
        const uint32_t off = (valid >> (c / ((int)kPitch / 16))) & 1u ? (uint32_t)(16 * c) : kDrop;
        __builtin_amdgcn_raw_buffer_store_b128(d, rs, off, 0, kBufNTDevice);
      }
    }
  } else {
#pragma unroll
    for (int p = 0; p < kSlotsPerWave; ++p) {
      const bool ok = tok[p] >= 0;
      const int64_t row_off = ok ? a.map.row<kPow2>((uint32_t)(s0 + p)) * kPitch : 0;
      const __amdgpu_buffer_rsrc_t rs = buffer_at(a.cache + row_off, ok ? (uint32_t)kPitch : 0u);
#pragma unroll
      for (int sub = 0; sub < kSub; ++sub) {
        uint32_t sdw;
        const uint32_t codes = quantize_slice(v[p][sub], sdw);
        const uint32_t scale_off = (lane & 15) == 12 ? LATENT / 2 + sub * 16 + (lane >> 4) * 4 : kDrop;
        // Rows go out in slot order, so plain stores let L2 merge neighbours.
        __builtin_amdgcn_raw_buffer_store_b32(codes, rs, sub * 256 + lane * 4, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b32(sdw, rs, scale_off, 0, 0);
      }
    }
  }
}

template <int LATENT, bool kPow2>
void launch_by_slot_pow2(const StoreArgs& a, const int32_t* inv, unsigned blocks, hipStream_t stream) {
  // consecutive slots are consecutive rows within a block (the flat form has
  // a single block); a wave's slots share a block when the block size is a
  // multiple of kSlotsPerWave
  const bool flat = a.map.pow2 && a.map.block_shift == 32;
  const bool staged = (flat || a.map.block_size % kSlotsPerWave == 0) &&
                      (reinterpret_cast<uintptr_t>(a.cache) & 15u) == 0;
  if (staged)
    hipLaunchKernelGGL((mxfp4_store_by_slot_kernel<LATENT, kPow2, true>), dim3(blocks),
                       dim3(kWave * kWavesPerBlock), 0, stream, a, inv);
  else
    hipLaunchKernelGGL((mxfp4_store_by_slot_kernel<LATENT, kPow2, false>), dim3(blocks),
                       dim3(kWave * kWavesPerBlock), 0, stream, a, inv);
}

template <int LATENT>
hipError_t launch_by_slot(const StoreArgs& a, const int32_t* inv, hipStream_t stream) {
  constexpr int64_t kPerBlock = (int64_t)kWavesPerBlock * kSlotsPerWave;
  const unsigned blocks = (unsigned)(((int64_t)a.map.num_slots + kPerBlock - 1) / kPerBlock);
  if (a.map.pow2)
    launch_by_slot_pow2<LATENT, true>(a, inv, blocks, stream);
  else
    launch_by_slot_pow2<LATENT, false>(a, inv, blocks, stream);
  return hipGetLastError();
}

// Four passes per wave (batches above 16,384 tokens) wait for the slots
// before the rows: measured against rows-first on MI355X, dense batches of
// 65,536 to 4.5M tokens within -1..+2.5%, and 262,144 tokens with half or
// nine tenths pads 17-25% faster (their rows are not read).  Smaller
// batches are bound by latency, where rows-first is 4-6% faster and a pad's
// row costs little.
template <int LATENT, int TPW>
hipError_t launch_tpw(const StoreArgs& a, hipStream_t stream) {
  constexpr int kLanesPerTok = LATENT >= 512 ? 64 : LATENT / 8;
  constexpr int64_t kToksPerBlock = (int64_t)kWavesPerBlock * TPW * (kWave / kLanesPerTok);
  constexpr bool kSlotFirst = TPW == 4;
  const int64_t blocks = (a.num_tokens + kToksPerBlock - 1) / kToksPerBlock;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  if (a.map.pow2)
    hipLaunchKernelGGL((mxfp4_store_kernel<LATENT, true, TPW, kSlotFirst>), dim3((unsigned)blocks),
                       dim3(kWave * kWavesPerBlock), 0, stream, a);
  else
    hipLaunchKernelGGL((mxfp4_store_kernel<LATENT, false, TPW, kSlotFirst>), dim3((unsigned)blocks),
                       dim3(kWave * kWavesPerBlock), 0, stream, a);
  return hipGetLastError();
}

template <int LATENT>
hipError_t launch_latent(const StoreArgs& args, hipStream_t stream) {
  StoreArgs a = args;
  a.plain_stores = a.num_tokens <= kPlainStoreBytes / (LATENT / 2 + LATENT / 32);
  // Passes per wave by batch size, from HIP-graph timings of back-to-back
  // launches (random slots, latent 512): one up to 8,192 tokens (shorter
  // waves finish sooner: 256 tokens 1.97 vs 2.22 us with two), two up to
  // 16,384 (4.9 vs 5.3 us), four above (32,768 tokens 8.3 vs 8.8 us,
  // 262,143 tokens 59 vs 65 us).
  if (a.num_tokens <= 8192) return launch_tpw<LATENT, 1>(a, stream);
  if (a.num_tokens <= 16384) return launch_tpw<LATENT, 2>(a, stream);
  return launch_tpw<LATENT, 4>(a, stream);
}

}  // namespace

hipError_t launch_build_inverse(const int64_t* slots, int64_t num_tokens, uint32_t num_slots,
                                int32_t* inverse, hipStream_t stream) {
  hipLaunchKernelGGL(fill_inverse, dim3((unsigned)(((int64_t)num_slots + 1023) / 1024)), dim3(256), 0,
                     stream, inverse, (int64_t)num_slots);
  if (num_tokens > 0)
    hipLaunchKernelGGL(invert_slots, dim3((unsigned)((num_tokens + 255) / 256)), dim3(256), 0, stream,
                       slots, num_tokens, inverse, num_slots);
  return hipGetLastError();
}

hipError_t launch_mxfp4_store_by_slot(const StoreArgs& a, int latent, const int32_t* inverse,
                                      hipStream_t stream) {
  switch (latent) {
    case 512: return launch_by_slot<512>(a, inverse, stream);
    case 1024: return launch_by_slot<1024>(a, inverse, stream);
    case 2048: return launch_by_slot<2048>(a, inverse, stream);
    default: return hipErrorInvalidValue;
  }
}

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
int32_t* g_scratch[kMaxDevices] = {};

// Device address of `scratch` on the current device, looked up on the first
// call there and kept (each GPU holds the array at its own address).
hipError_t scratch_of_current_device(int32_t** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch[dev] = static_cast<int32_t*>(p);
  }
  *out = g_scratch[dev];
  return hipSuccess;
}

}  // namespace

hipError_t launch_mxfp4_store_slot_order_noalloc(const StoreArgs& a, int latent,
                                                 hipStream_t stream) {
  if ((int64_t)a.map.num_slots * 4 > kNoAllocScratchBytes) return hipErrorInvalidValue;
  int32_t* inv = nullptr;
  hipError_t e = scratch_of_current_device(&inv);
  if (e != hipSuccess) return e;
  // The map is refilled on every call (fill kernel, then the tokens'
  // entries), so nothing a previous call left in the array is read.
  e = launch_build_inverse(a.slots, a.num_tokens, a.map.num_slots, inv, stream);
  if (e != hipSuccess) return e;
  return launch_mxfp4_store_by_slot(a, latent, inv, stream);
}

hipError_t launch_mxfp4_store(const StoreArgs& a, int latent, hipStream_t stream) {
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
