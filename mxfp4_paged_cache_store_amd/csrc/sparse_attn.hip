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
// Work split: one workgroup of 8 waves per (query token, block of HB = 32 or
// 16 heads = HT head tiles of 16); the token's slots are walked in tiles of
// 16 * 8 / HT keys (64 or 128).
//   scores   wave w computes S for head tile w % HT and the 16 keys of key
//            group w / HT.  Lane (key l%16, quarter l/16) loads 64 code bytes
//            and one scale dword of its key's row (prefetched a tile
//            ahead);
//            gfx950's v_cvt_scalef32_pk_bf16_fp4 turns each code dword into
//            8 exact bf16 values -- the B operand of a 16x16x32 bf16 MFMA
//            (the 512-dim reduction order is permuted identically in the
//            query fragments, which stay in registers).  The waves of head
//            tile 0 also copy the packed rows into LDS (272 B per key).
//   softmax  base-2 online softmax in fp32: per-head maxima of each key
//            group go through LDS, so every wave rescales with the same
//            running maximum; each scores wave keeps partial row sums of its
//            keys; the weights go to LDS as bf16.
//   PV       wave w owns dims 128*(w%4) .. +127 and half of the tile's keys
//            (w / 4), all HB heads.  The B operand needs 8 consecutive keys
//            of one dim (a transpose of the cache layout): lane (j = l%16,
//            q = l/16) reads from the packed LDS copy the code dword of dims
//            128*(w%4) + 8j .. +7 for keys 8q .. 8q+7 of a 32-key step and
//            their scale bytes, converts each (bf16 pairs along dims), and
//            re-pairs the halves along keys with v_perm_b32: 8 B operands,
//            for 8 MFMAs whose output column j is dim 128*(w%4) + 8j + n.
// LDS buffers alternate between tiles, so a tile costs two barriers.  At the
// end the sink is folded in, the two key halves of O and the partial sums are
// added, and O / l is rounded to bf16.
#include "kernels.hpp"

namespace mxs {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 8;
constexpr int kRowBytes = 272;
constexpr int kRowMirror = 0x140;
constexpr int kRowHalfMirror = 0x141;
constexpr float kLog2e = 1.4426950408889634f;
constexpr uint32_t kPermLo = 0x05040100u;  // (src1.lo, src0.lo)
constexpr uint32_t kPermHi = 0x07060302u;  // (src1.hi, src0.hi)

__device__ __forceinline__ float max2(float a, float b) { return a > b ? a : b; }

__device__ __forceinline__ float row16_max(float v) {
  v = max2(v, as_f32(dpp<kQuadSwap1>(as_u32(v))));
  v = max2(v, as_f32(dpp<kQuadSwap2>(as_u32(v))));
  v = max2(v, as_f32(dpp<kRowHalfMirror>(as_u32(v))));
  v = max2(v, as_f32(dpp<kRowMirror>(as_u32(v))));
  return v;
}

__device__ __forceinline__ float row16_sum(float v) {
  v += as_f32(dpp<kQuadSwap1>(as_u32(v)));
  v += as_f32(dpp<kQuadSwap2>(as_u32(v)));
  v += as_f32(dpp<kRowHalfMirror>(as_u32(v)));
  v += as_f32(dpp<kRowMirror>(as_u32(v)));
  return v;
}

__device__ __forceinline__ uint32_t bf16_rn(float f) {
  const uint32_t u = as_u32(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ u32x4 unpack8(uint32_t codes, uint32_t scale_byte) {
  const float scale = as_f32(scale_byte << 23);
  return u32x4{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 0)),
               __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 1)),
               __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 2)),
               __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 3))};
}

// Byte `sel` of a code dword -> bf16 pair (the selector must be a constant;
// after unrolling the switch folds away).
__device__ __forceinline__ uint32_t cvt_byte(uint32_t codes, float scale, int sel) {
  switch (sel) {
    case 0: return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 0));
    case 1: return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 1));
    case 2: return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 2));
    default: return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 3));
  }
}

template <int HB>
struct Cfg {
  static constexpr int HT = HB / 16;           // head tiles
  static constexpr int NKG = kWaves / HT;      // key groups of 16 in the scores phase
  static constexpr int TILE = 16 * NKG;        // keys per tile
  static constexpr int KH = TILE / 2;          // keys per PV half
  static constexpr int KS2 = KH / 32;          // PV k-steps per wave and tile
  static constexpr int PITCH = TILE + 8;       // bf16 per LDS weight row (rows stay 16-B aligned)
};

// Packed rows in LDS are 280 bytes apart (272 + 8): rows 8 apart then start
// 16 banks apart, so the PV reads of keys 8q + k (q = 0..3) do not collide.
constexpr int kKvPitch = 280;
// The running maximum is raised only when a tile's maximum exceeds it by more
// than this (base-2 units): weights stay below 2^8, far from fp32 / bf16
// overflow, and most tiles need no rescaling of O.
constexpr float kMaxSlack = 8.0f;

template <int HB>
struct AttnSmem {
  using C = Cfg<HB>;
  union {
    struct {
      uint8_t kv[2][C::TILE][kKvPitch];       // packed rows of the tile
      uint16_t p[2][HB * C::PITCH];           // the tile's weights (bf16): [head][key]
      float red[2][HB][C::NKG];               // per-key-group maxima
    } loop;
    struct {
      f32x4 o[4][C::HT * 8][kWave];           // second key half of O, per dim group
      float l[C::NKG][HB];                    // partial sums
    } fin;
  };
};

template <int NKG>
__device__ __forceinline__ float group_max(const float* red) {
  float mt = red[0];
#pragma unroll
  for (int g = 1; g < NKG; ++g) mt = fmaxf(mt, red[g]);
  return mt;
}

template <int HB, bool kPow2>
__global__ __launch_bounds__(kWave * kWaves) void sparse_mla_attn_kernel(const AttnArgs a) {
  using C = Cfg<HB>;
  constexpr int HT = C::HT, TILE = C::TILE, KH = C::KH, KS2 = C::KS2, PITCH = C::PITCH, NKG = C::NKG;
  __shared__ AttnSmem<HB> sm;
  const int lane = threadIdx.x & (kWave - 1);
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int li = lane & 15, lq = lane >> 4;
  const int hw = w % HT, kg = w / HT;   // scores role
  const int dg = w & 3, kh = w >> 2;    // PV role
  const uint32_t nhb = (uint32_t)(a.num_heads / HB);
  const uint32_t blk = xcd_contiguous_block();
  const int64_t t = blk / nhb;
  const int h0 = (int)(blk % nhb) * HB;

  // Query fragments of head tile hw: lane (head li, quarter lq) holds dims
  // 128*lq + 8*ks .. +8 at k-step ks.  They are the B operand of S^T = K Q^T.
  bf16x8 qf[16];
  {
    const uint16_t* qh = a.q + t * a.q_token_stride + (int64_t)(h0 + 16 * hw + li) * a.q_head_stride + 128 * lq;
#pragma unroll
    for (int ks = 0; ks < 16; ++ks)
      qf[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(qh + 8 * ks));
  }

  f32x4 o[HT][8];
  float m_pv[HT][4];  // running maxima of the O rows, heads 16ht + 4lq + r
  float m_qk = -INFINITY;  // running maximum of head 16hw + li (scores role)
  float lsum = 0.0f;       // this lane's share of the sum for head 16hw + li
#pragma unroll
  for (int ht = 0; ht < HT; ++ht) {
#pragma unroll
    for (int n = 0; n < 8; ++n) o[ht][n] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int r = 0; r < 4; ++r) m_pv[ht][r] = -INFINITY;
  }

  const int key = 16 * kg + li;  // this lane's key in the scores gather
  const int32_t* idx_row = a.indices + t * a.idx_stride;
  const int64_t ntile = (a.topk + TILE - 1) / TILE;
  // Loads are unconditional (addresses clamped, results masked), so the
  // compiler can count outstanding loads precisely instead of draining them
  // at every branch join; the loop below only runs when topk >= 1.
  auto load_index = [&](int64_t tile) -> int32_t {
    const int64_t j = tile * TILE + key;
    const int32_t v = idx_row[j < a.topk ? j : a.topk - 1];
    return j < a.topk ? v : -1;
  };
  auto row_index = [&](int32_t s) -> int32_t {
    const bool ok = s >= 0 && (uint32_t)s < a.map.num_slots;
    return ok ? (int32_t)a.map.template row<kPow2>((uint32_t)s) : -1;
  };
  auto gather_k = [&](int32_t row, u32x4 (&c)[4], uint32_t& sd) {
    const uint8_t* rp = a.cache + (int64_t)(row < 0 ? 0 : row) * kRowBytes;
    const u32x4* cp = reinterpret_cast<const u32x4*>(rp + 64 * lq);
#pragma unroll
    for (int i = 0; i < 4; ++i) c[i] = cp[i];
    sd = *reinterpret_cast<const uint32_t*>(rp + 256 + 4 * lq);
  };

  // The gather of a tile is issued right after the previous tile's scores
  // (one tile ahead, into the same registers); slot indices are loaded one
  // tile earlier still.
  struct Stage {
    int32_t row;
    u32x4 cw[4];
    uint32_t sd;
    int32_t idx;
  };
  Stage g;
  if (ntile > 0) {
    g.row = row_index(load_index(0));
    gather_k(g.row, g.cw, g.sd);
    g.idx = load_index(1);
  }

  for (int64_t tile = 0; tile < ntile; ++tile) {
    const int buf = (int)(tile & 1);
    // ---- scores S^T[key][head] for key group kg, head tile hw; head tile 0
    // stages the packed rows
    const bool key_valid = g.row >= 0;
    const uint32_t vmask = (uint32_t)__ballot(key_valid) & 0xFFFFu;  // keys 0..15 of the group
    if (!key_valid) {
#pragma unroll
      for (int i = 0; i < 4; ++i) g.cw[i] = u32x4{0u, 0u, 0u, 0u};
      g.sd = 0x7F7F7F7Fu;
    }
    if (hw == 0) {
      uint8_t* dst = sm.loop.kv[buf][key] + 64 * lq;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        *reinterpret_cast<uint64_t*>(dst + 16 * i) = (uint64_t)g.cw[i][0] | ((uint64_t)g.cw[i][1] << 32);
        *reinterpret_cast<uint64_t*>(dst + 16 * i + 8) = (uint64_t)g.cw[i][2] | ((uint64_t)g.cw[i][3] << 32);
      }
      *reinterpret_cast<uint32_t*>(sm.loop.kv[buf][key] + 256 + 4 * lq) = g.sd;
    }
    f32x4 s0 = f32x4{0.0f, 0.0f, 0.0f, 0.0f}, s1 = s0;
#pragma unroll
    for (int ks = 0; ks < 16; ks += 2) {
      const uint32_t sb = (g.sd >> (8 * (ks >> 2))) & 0xFFu;
      const bf16x8 k0 = __builtin_bit_cast(bf16x8, unpack8(g.cw[ks >> 2][ks & 3], sb));
      const bf16x8 k1 = __builtin_bit_cast(bf16x8, unpack8(g.cw[ks >> 2][(ks & 3) + 1], sb));
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0, qf[ks], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1, qf[ks + 1], s1, 0, 0, 0);
    }

    // ---- gather of the next tile (the index load goes first: waiting for
    // it later must not wait for the gather, as loads complete in order)
    const int32_t nxt = g.idx;
    g.idx = load_index(tile + 2);
    g.row = row_index(nxt);
    gather_k(g.row, g.cw, g.sd);

    // ---- softmax (base 2).  Lane (head li, quarter lq) holds S[head][key
    // 4lq + r] of the group; invalid keys become -inf.
    const uint32_t vbits = vmask >> (4 * lq);
    float x[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) x[r] = ((vbits >> r) & 1u) ? (s0[r] + s1[r]) * a.c : -INFINITY;
    float mx = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    if (lq == 0) sm.loop.red[buf][16 * hw + li][kg] = mx;
    __syncthreads();
    {
      const float mt = group_max<NKG>(sm.loop.red[buf][16 * hw + li]);
      const float mnew = mt > m_qk + kMaxSlack ? mt : m_qk;
      const float alpha = mnew == m_qk ? 1.0f : __builtin_amdgcn_exp2f(m_qk - mnew);
      m_qk = mnew;
      uint32_t pb[4];
      float ps = 0.0f;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float p = mnew == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(x[r] - mnew);
        ps += p;
        pb[r] = bf16_rn(p);
      }
      lsum = lsum * alpha + ps;
      *reinterpret_cast<uint64_t*>(&sm.loop.p[buf][(16 * hw + li) * PITCH + 16 * kg + 4 * lq]) =
          (uint64_t)(pb[0] | (pb[1] << 16)) | ((uint64_t)(pb[2] | (pb[3] << 16)) << 32);
    }
    bool changed = false;
    float alpha_pv[HT][4];
#pragma unroll
    for (int ht = 0; ht < HT; ++ht)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float mt = group_max<NKG>(sm.loop.red[buf][16 * ht + 4 * lq + r]);
        const float mold = m_pv[ht][r];
        const float mnew = mt > mold + kMaxSlack ? mt : mold;
        alpha_pv[ht][r] = mnew == mold ? 1.0f : __builtin_amdgcn_exp2f(mold - mnew);
        changed |= mnew != mold;
        m_pv[ht][r] = mnew;
      }
    if (__any(changed)) {
#pragma unroll
      for (int ht = 0; ht < HT; ++ht)
#pragma unroll
        for (int n = 0; n < 8; ++n)
#pragma unroll
          for (int r = 0; r < 4; ++r) o[ht][n][r] *= alpha_pv[ht][r];
    }
    __syncthreads();

    // ---- PV: dims 128dg .. +127, keys KH*kh .. +KH of the tile
#pragma unroll
    for (int ks2 = 0; ks2 < KS2; ++ks2) {
      const int kb = KH * kh + 32 * ks2;
      bf16x8 pf[HT];
#pragma unroll
      for (int ht = 0; ht < HT; ++ht)
        pf[ht] = __builtin_bit_cast(bf16x8,
                                    *reinterpret_cast<const u32x4*>(&sm.loop.p[buf][(16 * ht + li) * PITCH + kb + 8 * lq]));
      uint32_t vc[8];
      float vs[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const uint8_t* row = sm.loop.kv[buf][kb + 8 * lq + k];
        vc[k] = *reinterpret_cast<const uint32_t*>(row + 64 * dg + 4 * li);
        vs[k] = as_f32((uint32_t)row[256 + 4 * dg + (li >> 2)] << 23);
      }
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) {
        uint32_t xv[8];  // key k: bf16 pair of dims 8li + 2s4, +1
#pragma unroll
        for (int k = 0; k < 8; ++k)
          xv[k] = cvt_byte(vc[k], vs[k], s4);
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int n = 2 * s4 + e;
          const uint32_t sel = e ? kPermHi : kPermLo;
          const u32x4 vb = {__builtin_amdgcn_perm(xv[1], xv[0], sel), __builtin_amdgcn_perm(xv[3], xv[2], sel),
                            __builtin_amdgcn_perm(xv[5], xv[4], sel), __builtin_amdgcn_perm(xv[7], xv[6], sel)};
          const bf16x8 vf = __builtin_bit_cast(bf16x8, vb);
#pragma unroll
          for (int ht = 0; ht < HT; ++ht) o[ht][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pf[ht], vf, o[ht][n], 0, 0, 0);
        }
      }
    }
  }

  // ---- sink, partial sums, the two key halves, normalisation
  lsum += __shfl_xor(lsum, 16);
  lsum += __shfl_xor(lsum, 32);
  float sc[HT][4];
#pragma unroll
  for (int ht = 0; ht < HT; ++ht)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      sc[ht][r] = 1.0f;
      if (a.sink) {
        const float s2 = a.sink[h0 + 16 * ht + 4 * lq + r] * kLog2e;
        const float mf = fmaxf(m_pv[ht][r], s2);
        sc[ht][r] = m_pv[ht][r] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m_pv[ht][r] - mf);
      }
    }
  float l = lsum;
  if (a.sink) {
    const float s2 = a.sink[h0 + 16 * hw + li] * kLog2e;
    const float mf = fmaxf(m_qk, s2);
    l = m_qk == -INFINITY ? 0.0f : l * __builtin_amdgcn_exp2f(m_qk - mf);
    if (kg == 0) l += __builtin_amdgcn_exp2f(s2 - mf);
  }
  __syncthreads();  // the loop's LDS is reused below
  if (lq == 0) sm.fin.l[kg][16 * hw + li] = l;
#pragma unroll
  for (int ht = 0; ht < HT; ++ht)
#pragma unroll
    for (int n = 0; n < 8; ++n)
#pragma unroll
      for (int r = 0; r < 4; ++r) o[ht][n][r] *= sc[ht][r];
  if (kh == 1) {
#pragma unroll
    for (int ht = 0; ht < HT; ++ht)
#pragma unroll
      for (int n = 0; n < 8; ++n) sm.fin.o[dg][ht * 8 + n][lane] = o[ht][n];
  }
  __syncthreads();
  if (kh == 0) {
#pragma unroll
    for (int ht = 0; ht < HT; ++ht)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int h = 16 * ht + 4 * lq + r;
        float lt = sm.fin.l[0][h];
#pragma unroll
        for (int g = 1; g < NKG; ++g) lt += sm.fin.l[g][h];
        uint32_t b[8];
#pragma unroll
        for (int n = 0; n < 8; ++n) {
          const float v = o[ht][n][r] + sm.fin.o[dg][ht * 8 + n][lane][r];
          b[n] = bf16_rn(lt > 0.0f ? v / lt : 0.0f);
        }
        uint16_t* orow = a.out + t * a.out_token_stride + (int64_t)(h0 + h) * a.out_head_stride + 128 * dg + 8 * li;
        if (a.out_aligned) {
          *reinterpret_cast<u32x4*>(orow) =
              u32x4{b[0] | (b[1] << 16), b[2] | (b[3] << 16), b[4] | (b[5] << 16), b[6] | (b[7] << 16)};
        } else {
#pragma unroll
          for (int n = 0; n < 8; ++n) orow[n] = (uint16_t)b[n];
        }
      }
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
