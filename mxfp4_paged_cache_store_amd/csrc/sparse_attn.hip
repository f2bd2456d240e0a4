// sparse_attn.hip -- sparse MLA attention straight from the MXFP4 cache, for
// gfx950 (the read side of the format).
//
// What is computed ("[ROCm][Attention] Add an mxfp4_mla KV cache for
// rope-free sparse MLA", Claims and Details / read path): for a query token
// and head, softmax attention over the token's listed cache slots, keys and
// values both being the slot's dequantized 512-wide latent (rope-free MLA in
// its absorbed form), optionally with a per-head sink logit in the
// denominator.  Invalid slots (negative, or past the cache) are skipped.
//
// Work split.  One workgroup of 4 waves per (query token, block of HB = 16
// or 32 heads); the token's slots are walked in tiles of 64, 16 per wave.
//   gather   lane (key = l%16, quarter = l/16) loads 64 code bytes + 1 scale
//            dword of its key's row through a raw buffer whose range is the
//            row, or empty for an invalid slot (the loads return zeros);
//   unpack   gfx950's v_cvt_scalef32_pk_bf16_fp4 turns each code dword into
//            8 exact bf16 values -- already the B operand of a
//            16x16x32 bf16 MFMA for the scores (the reduction order over the
//            512 dims is permuted identically in the query fragments);
//   scores   S[16 heads x 16 keys] per head tile, fp32 accumulate;
//   V^T      the same bf16 values are written transposed to LDS ([dim][key])
//            so the PV MFMA can read 8 consecutive keys of one dim as 16 B;
//   softmax  base-2 online softmax: per-head tile maxima are exchanged
//            through LDS so every wave rescales with the same running max;
//            each wave keeps its own partial row sums;
//   PV       wave w owns output dims 128w..128w+127 for all HB heads:
//            O[16 x 16] += P[16 heads x 32 keys] . V[32 keys x 16 dims].
// The next tile's slot indices and code rows are loaded while the current
// tile is computed.  At the end the sink is folded in, the 4 partial sums are
// added, and O / l is rounded to bf16.
#include "kernels.hpp"

namespace mxs {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr int kTile = 64;       // keys per tile, 16 per wave
constexpr int kLatent = 512;
constexpr int kRowBytes = 272;
constexpr int kPitch = 72;      // bf16 per LDS row of 64 keys (+8: 16-byte aligned rows)
constexpr int kRowMirror = 0x140;
constexpr int kRowHalfMirror = 0x141;
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, as_f32(dpp<kQuadSwap1>(as_u32(v))));
  v = fmaxf(v, as_f32(dpp<kQuadSwap2>(as_u32(v))));
  v = fmaxf(v, as_f32(dpp<kRowHalfMirror>(as_u32(v))));
  v = fmaxf(v, as_f32(dpp<kRowMirror>(as_u32(v))));
  return v;
}

__device__ __forceinline__ float row16_sum(float v) {
  v += as_f32(dpp<kQuadSwap1>(as_u32(v)));
  v += as_f32(dpp<kQuadSwap2>(as_u32(v)));
  v += as_f32(dpp<kRowHalfMirror>(as_u32(v)));
  v += as_f32(dpp<kRowMirror>(as_u32(v)));
  return v;
}

__device__ __forceinline__ uint16_t bf16_rn(float f) {
  const uint32_t u = as_u32(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

template <int HB>
struct AttnSmem {
  uint16_t vt[kLatent * kPitch];  // V^T of the tile: [dim][key]
  uint16_t p[HB * kPitch];        // P of the tile (bf16): [head][key]
  float red[kWaves][HB];          // per-wave tile maxima, then partial sums
};

template <int HB, bool kPow2>
__global__ __launch_bounds__(kWave * kWaves) void sparse_mla_attn_kernel(const AttnArgs a) {
  constexpr int HT = HB / 16;
  __shared__ AttnSmem<HB> sm;
  const int lane = threadIdx.x & (kWave - 1);
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int li = lane & 15, lq = lane >> 4;
  const uint32_t nhb = (uint32_t)(a.num_heads / HB);
  const uint32_t blk = xcd_contiguous_block();
  const int64_t t = blk / nhb;
  const int h0 = (int)(blk % nhb) * HB;

  // Query fragments (A operand): lane (head li, quarter lq) holds dims
  // 128*lq + 8*ks .. +8 at k-step ks.
  bf16x8 qf[HT][16];
#pragma unroll
  for (int ht = 0; ht < HT; ++ht) {
    const uint16_t* qh = a.q + t * a.q_token_stride + (int64_t)(h0 + 16 * ht + li) * a.q_head_stride + 128 * lq;
#pragma unroll
    for (int ks = 0; ks < 16; ++ks)
      qf[ht][ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(qh + 8 * ks));
  }

  f32x4 o[HT][8];
  float m[HT][4], lpart[HT][4];
#pragma unroll
  for (int ht = 0; ht < HT; ++ht) {
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) o[ht][nt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      m[ht][r] = -INFINITY;
      lpart[ht][r] = 0.0f;
    }
  }

  const int key = 16 * w + li;
  const int32_t* idx_row = a.indices + t * a.idx_stride;
  const int64_t ntile = (a.topk + kTile - 1) / kTile;
  auto load_index = [&](int64_t tile) -> int32_t {
    const int64_t j = tile * kTile + key;
    return (tile < ntile && j < a.topk) ? idx_row[j] : -1;
  };
  auto row_of = [&](int32_t s, bool& valid) -> __amdgpu_buffer_rsrc_t {
    valid = s >= 0 && (uint32_t)s < a.map.num_slots;
    const int64_t row = valid ? a.map.template row<kPow2>((uint32_t)s) : 0;
    return buffer_at(a.cache + row * kRowBytes, valid ? (uint32_t)kRowBytes : 0u);
  };

  bool valid;
  __amdgpu_buffer_rsrc_t rs = row_of(load_index(0), valid);
  u32x4 cw[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    cw[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, 64 * lq + 16 * i, 0, 0));
  uint32_t sdw = __builtin_amdgcn_raw_buffer_load_b32(rs, 256 + 4 * lq, 0, 0);
  int32_t idx_next = load_index(1);

  for (int64_t tile = 0; tile < ntile; ++tile) {
    // ---- unpack + scores; V^T to LDS
    f32x4 s[HT];
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) s[ht] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) {
      const uint32_t codes = cw[ks >> 2][ks & 3];
      const float scale = as_f32(((sdw >> (8 * (ks >> 2))) & 0xFFu) << 23);
      uint32_t x[4];
      x[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 0));
      x[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 1));
      x[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 2));
      x[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 3));
      const bf16x8 kf = __builtin_bit_cast(bf16x8, u32x4{x[0], x[1], x[2], x[3]});
#pragma unroll
      for (int ht = 0; ht < HT; ++ht) s[ht] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qf[ht][ks], kf, s[ht], 0, 0, 0);
      const int d0 = 128 * lq + 8 * ks;
#pragma unroll
      for (int i = 0; i < 8; ++i)
        sm.vt[(d0 + i) * kPitch + key] = (uint16_t)(x[i >> 1] >> (16 * (i & 1)));
    }
    const bool key_valid = valid;

    // ---- next tile's gather, in flight during softmax and PV
    if (tile + 1 < ntile) {
      rs = row_of(idx_next, valid);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        cw[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, 64 * lq + 16 * i, 0, 0));
      sdw = __builtin_amdgcn_raw_buffer_load_b32(rs, 256 + 4 * lq, 0, 0);
      idx_next = load_index(tile + 2);
    }

    // ---- softmax (base 2).  Lane (key li, quarter lq) holds S[head 4lq + r][key].
    float x2[HT][4];
#pragma unroll
    for (int ht = 0; ht < HT; ++ht)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        x2[ht][r] = key_valid ? s[ht][r] * a.c : -INFINITY;
        const float mx = row16_max(x2[ht][r]);
        if (li == 0) sm.red[w][16 * ht + 4 * lq + r] = mx;
      }
    __syncthreads();
    float alpha[HT][4];
#pragma unroll
    for (int ht = 0; ht < HT; ++ht)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int h = 16 * ht + 4 * lq + r;
        const float mt = fmaxf(fmaxf(sm.red[0][h], sm.red[1][h]), fmaxf(sm.red[2][h], sm.red[3][h]));
        const float mnew = fmaxf(m[ht][r], mt);
        const bool none = mnew == -INFINITY;
        alpha[ht][r] = none ? 1.0f : exp2f(m[ht][r] - mnew);
        const float p = none ? 0.0f : exp2f(x2[ht][r] - mnew);
        lpart[ht][r] = lpart[ht][r] * alpha[ht][r] + row16_sum(p);
        m[ht][r] = mnew;
        sm.p[h * kPitch + key] = bf16_rn(p);
      }
#pragma unroll
    for (int ht = 0; ht < HT; ++ht)
#pragma unroll
      for (int nt = 0; nt < 8; ++nt)
#pragma unroll
        for (int r = 0; r < 4; ++r) o[ht][nt][r] *= alpha[ht][r];
    __syncthreads();

    // ---- PV: wave w owns dims 128w .. 128w + 127
#pragma unroll
    for (int ks2 = 0; ks2 < 2; ++ks2) {
      bf16x8 pf[HT];
#pragma unroll
      for (int ht = 0; ht < HT; ++ht)
        pf[ht] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(&sm.p[(16 * ht + li) * kPitch + 32 * ks2 + 8 * lq]));
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) {
        const int d = 128 * w + 16 * nt + li;
        const bf16x8 vf = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(&sm.vt[d * kPitch + 32 * ks2 + 8 * lq]));
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) o[ht][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pf[ht], vf, o[ht][nt], 0, 0, 0);
      }
    }
    __syncthreads();
  }

  // ---- sink, partial sums, normalisation
#pragma unroll
  for (int ht = 0; ht < HT; ++ht)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int h = 16 * ht + 4 * lq + r;
      float l = lpart[ht][r];
      if (a.sink) {
        const float s2 = a.sink[h0 + h] * kLog2e;
        const float mf = fmaxf(m[ht][r], s2);
        const float sc = m[ht][r] == -INFINITY ? 0.0f : exp2f(m[ht][r] - mf);
        l *= sc;
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) o[ht][nt][r] *= sc;
        if (w == 0) l += exp2f(s2 - mf);
      }
      if (li == 0) sm.red[w][h] = l;
    }
  __syncthreads();
#pragma unroll
  for (int ht = 0; ht < HT; ++ht)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int h = 16 * ht + 4 * lq + r;
      const float l = (sm.red[0][h] + sm.red[1][h]) + (sm.red[2][h] + sm.red[3][h]);
      uint16_t* orow = a.out + t * a.out_token_stride + (int64_t)(h0 + h) * a.out_head_stride + 128 * w + li;
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) orow[16 * nt] = bf16_rn(l > 0.0f ? o[ht][nt][r] / l : 0.0f);
    }
}

template <int HB>
hipError_t launch_hb(const AttnArgs& a, hipStream_t stream) {
  const int64_t blocks = a.num_tokens * (a.num_heads / HB);
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  if (a.map.pow2)
    hipLaunchKernelGGL((sparse_mla_attn_kernel<HB, true>), dim3((unsigned)blocks), dim3(kWave * kWaves), 0,
                       stream, a);
  else
    hipLaunchKernelGGL((sparse_mla_attn_kernel<HB, false>), dim3((unsigned)blocks), dim3(kWave * kWaves), 0,
                       stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_sparse_mla_attn(const AttnArgs& a, hipStream_t stream) {
  if (a.num_tokens == 0) return hipSuccess;
  if (a.num_heads % 32 == 0) return launch_hb<32>(a, stream);
  return launch_hb<16>(a, stream);
}

}  // namespace mxs
