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
// 64 keys.  The waves specialise, and the two halves overlap on every SIMD:
//   producers (waves 0..3, 16 keys each) compute S^T = K Q^T for tile s.
//            Lane (key l%16, quarter l/16) loads 64 code bytes and one scale
//            dword of its key's row (one tile ahead); gfx950's
//            v_cvt_scalef32_pk_bf16_fp4 turns each code dword into 8 exact
//            bf16 values -- the A operand of a 16x16x32 bf16 MFMA -- and the
//            query fragments of all HB heads (the B operand, same permuted
//            512-dim order) stay in registers, so each key is unpacked once.
//            The packed rows are copied to LDS (280 B apart).  Softmax in
//            base 2: tile maxima of the 4 producers meet in LDS; the running
//            maximum moves only past a slack, and when it moves the new
//            maxima are published with a flag; weights go to LDS as bf16.
//   consumers (waves 4..7) own output dims 128*(w-4) .. +127 of all HB
//            heads and compute O += P V for tile s - 1.  The B operand needs
//            8 consecutive keys of one dim (a transpose of the cache layout):
//            lane (j = l%16, q = l/16) reads from the packed LDS copy the
//            code dword of dims 8j .. 8j+7 of its slab for keys 8q .. 8q+7
//            of a 32-key step and their scale bytes, converts each (bf16
//            pairs along dims) and re-pairs the halves along keys with
//            v_perm_b32: 8 B operands for 8 MFMAs whose output column j is
//            dim 8j + n of the slab.
// LDS buffers alternate between tiles; a step costs two barriers.  At the
// end the sink is folded in, the producers' partial sums are added, and
// O / l is rounded to bf16.
#include "kernels.hpp"

namespace mxs {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int kWaves = 8;
constexpr int kRowBytes = 272;
constexpr float kLog2e = 1.4426950408889634f;
constexpr uint32_t kPermLo = 0x05040100u;  // (src1.lo, src0.lo)
constexpr uint32_t kPermHi = 0x07060302u;  // (src1.hi, src0.hi)

// Two fp32 -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t bf16x2_rn(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

// Maximum over lanes l, l^16, l^32, l^48 (gfx950 permlane swaps: the pair
// returned for lane l is (x[l & ~16], x[l | 16]), resp. with 32).
__device__ __forceinline__ float max_over_quarters(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(as_u32(v), as_u32(v), false, false);
  v = fmaxf(as_f32(a[0]), as_f32(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(as_u32(v), as_u32(v), false, false);
  return fmaxf(as_f32(b[0]), as_f32(b[1]));
}

__device__ __forceinline__ float sum_over_quarters(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(as_u32(v), as_u32(v), false, false);
  v = as_f32(a[0]) + as_f32(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(as_u32(v), as_u32(v), false, false);
  return as_f32(b[0]) + as_f32(b[1]);
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

// Waves 0..3 produce (scores, softmax) and waves 4..7 consume (weighted
// sum); a tile has 64 keys, 16 per producer and all 64 for each consumer,
// which owns 128 output dims.
constexpr int kTile = 64;
constexpr int kProducers = 4;
constexpr int kPitch = kTile + 8;  // bf16 per LDS weight row (rows stay 16-B aligned)
// Packed rows in LDS are 280 bytes apart (272 + 8): rows 8 apart then start
// 16 banks apart, so the consumers' reads of keys 8q + k (q = 0..3) do not
// collide.
constexpr int kKvPitch = 280;
// The running maximum is raised only when a tile's maximum exceeds it by more
// than this (base-2 units): weights stay below 2^8, far from fp32 / bf16
// overflow, and most tiles need no rescaling of O.
constexpr float kMaxSlack = 8.0f;

template <int HB>
struct AttnSmem {
  static constexpr int HT = HB / 16;
  union {
    struct {
      uint8_t kv[2][kTile][kKvPitch];        // packed rows of a tile
      uint16_t p[2][HB * kPitch];            // a tile's weights (bf16): [head][key]
      float red[2][HB][kProducers];          // per-producer tile maxima
      float mpub[2][HB];                     // running maxima after a tile
      uint32_t moved[2];                     // some head's running maximum moved
    } loop;
    struct {
      float l[kProducers][HB];               // partial sums
    } fin;
  };
};

template <int HB, bool kPow2>
__global__ __launch_bounds__(kWave * kWaves) void sparse_mla_attn_kernel(const AttnArgs a) {
  constexpr int HT = HB / 16;
  __shared__ AttnSmem<HB> sm;
  const int lane = threadIdx.x & (kWave - 1);
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int li = lane & 15, lq = lane >> 4;
  const bool producer = w < kProducers;
  const int kg = w;                  // producer: key group (keys 16kg .. +15 of a tile)
  const int dg = w - kProducers;     // consumer: dims 128dg .. +127
  const uint32_t nhb = (uint32_t)(a.num_heads / HB);
  const uint32_t blk = xcd_contiguous_block();
  const int64_t t = blk / nhb;
  const int h0 = (int)(blk % nhb) * HB;
  const int64_t ntile = (a.topk + kTile - 1) / kTile;

  const int key = 16 * kg + li;  // a producer lane's key within the tile
  const int32_t* idx_row = a.indices + t * a.idx_stride;
  if (threadIdx.x < 2) sm.loop.moved[threadIdx.x] = 0u;  // ordered by the first barrier

  // Producers and consumers run separate loops (so their registers are not
  // live at the same time) with the same barriers: two per step, step s
  // producing tile s and consuming tile s - 1, then two in the epilogue.
  if (producer) {
    // Query fragments of all HB heads (B operand of S^T = K Q^T: lane (head
    // li, quarter lq) holds dims 128lq + 8ks .. +8 at k-step ks); running
    // maxima and partial sums of heads 16ht + li.
    bf16x8 qf[HT][16];
    float m_qk[HT], lsum[HT];
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
      m_qk[ht] = -INFINITY;
      lsum[ht] = 0.0f;
      const uint16_t* qh = a.q + t * a.q_token_stride + (int64_t)(h0 + 16 * ht + li) * a.q_head_stride + 128 * lq;
#pragma unroll
      for (int ks = 0; ks < 16; ++ks)
        qf[ht][ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(qh + 8 * ks));
    }
    // Loads are unconditional (addresses clamped, results masked), so the
    // compiler can count outstanding loads precisely instead of draining
    // them at every branch join; they run only when topk >= 1.
    auto load_index = [&](int64_t tile) -> int32_t {
      const int64_t j = tile * kTile + key;
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
    // (one tile ahead); slot indices are loaded one tile earlier still.
    int32_t g_row = -1, g_idx = -1;
    u32x4 g_cw[4];
    uint32_t g_sd = 0;
    if (ntile > 0) {
      g_row = row_index(load_index(0));
      gather_k(g_row, g_cw, g_sd);
      g_idx = load_index(1);
    }

    for (int64_t step = 0; step <= ntile; ++step) {
      const int pb = (int)(step & 1), cb = pb ^ 1;
      float x[HT][4];
      if (step < ntile) {
        // ---- scores S^T[key][head]; the packed rows go to LDS for the consumers
        const bool key_valid = g_row >= 0;
        const uint32_t vbits = ((uint32_t)__ballot(key_valid) >> (4 * lq)) & 0xFu;  // keys 4lq + r
        if (!key_valid) {
#pragma unroll
          for (int i = 0; i < 4; ++i) g_cw[i] = u32x4{0u, 0u, 0u, 0u};
          g_sd = 0x7F7F7F7Fu;
        }
        {
          uint8_t* dst = sm.loop.kv[pb][key];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            *reinterpret_cast<uint64_t*>(dst + 64 * lq + 16 * i) = (uint64_t)g_cw[i][0] | ((uint64_t)g_cw[i][1] << 32);
            *reinterpret_cast<uint64_t*>(dst + 64 * lq + 16 * i + 8) = (uint64_t)g_cw[i][2] | ((uint64_t)g_cw[i][3] << 32);
          }
          *reinterpret_cast<uint32_t*>(dst + 256 + 4 * lq) = g_sd;
        }
        f32x4 s[HT][2];
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) s[ht][0] = s[ht][1] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int ks = 0; ks < 16; ++ks) {
          const bf16x8 kf =
              __builtin_bit_cast(bf16x8, unpack8(g_cw[ks >> 2][ks & 3], (g_sd >> (8 * (ks >> 2))) & 0xFFu));
#pragma unroll
          for (int ht = 0; ht < HT; ++ht)
            s[ht][ks & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[ht][ks], s[ht][ks & 1], 0, 0, 0);
        }
        // ---- next tile's gather (the index load goes first: waiting for it
        // later must not wait for the gather, as loads complete in order)
        const int32_t nxt = g_idx;
        g_idx = load_index(step + 2);
        g_row = row_index(nxt);
        gather_k(g_row, g_cw, g_sd);
        // ---- tile maxima (base 2).  Lane (head li, quarter lq) holds
        // S[head 16ht + li][key 16kg + 4lq + r]; invalid keys become -inf.
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) {
#pragma unroll
          for (int r = 0; r < 4; ++r) x[ht][r] = ((vbits >> r) & 1u) ? (s[ht][0][r] + s[ht][1][r]) * a.c : -INFINITY;
          const float mx = max_over_quarters(fmaxf(fmaxf(x[ht][0], x[ht][1]), fmaxf(x[ht][2], x[ht][3])));
          if (lq == 0) sm.loop.red[pb][16 * ht + li][kg] = mx;
        }
      }
      __syncthreads();
      if (step < ntile) {
        // ---- running maxima, weights, partial sums; publish
        if (threadIdx.x == 0) sm.loop.moved[cb] = 0u;  // the consumers read it before this barrier
        bool moved = false;
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) {
          const float* red = sm.loop.red[pb][16 * ht + li];
          const float mt = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
          const float mnew = mt > m_qk[ht] + kMaxSlack ? mt : m_qk[ht];
          const float alpha = mnew != m_qk[ht] ? __builtin_amdgcn_exp2f(m_qk[ht] - mnew) : 1.0f;
          moved |= mnew != m_qk[ht];
          m_qk[ht] = mnew;
          float p[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) p[r] = mnew == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(x[ht][r] - mnew);
          lsum[ht] = lsum[ht] * alpha + ((p[0] + p[1]) + (p[2] + p[3]));
          *reinterpret_cast<uint64_t*>(&sm.loop.p[pb][(16 * ht + li) * kPitch + 16 * kg + 4 * lq]) =
              (uint64_t)bf16x2_rn(p[0], p[1]) | ((uint64_t)bf16x2_rn(p[2], p[3]) << 32);
          if (kg == 0 && lq == 0) sm.loop.mpub[pb][16 * ht + li] = mnew;
        }
        if (__any(moved) && lane == 0) sm.loop.moved[pb] = 1u;
      }
      __syncthreads();
    }

    // ---- sink and partial sums
    float l[HT];
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
      l[ht] = sum_over_quarters(lsum[ht]);
      if (a.sink) {
        const float s2 = a.sink[h0 + 16 * ht + li] * kLog2e;
        const float mf = fmaxf(m_qk[ht], s2);
        l[ht] = m_qk[ht] == -INFINITY ? 0.0f : l[ht] * __builtin_amdgcn_exp2f(m_qk[ht] - mf);
        if (kg == 0) l[ht] += __builtin_amdgcn_exp2f(s2 - mf);
      }
    }
    __syncthreads();  // the loop's LDS is reused
#pragma unroll
    for (int ht = 0; ht < HT; ++ht)
      if (lq == 0) sm.fin.l[kg][16 * ht + li] = l[ht];
    __syncthreads();
  } else {
    // O rows heads 16ht + 4lq + r, columns dims 128dg + 8li + n, and the
    // running maxima of those rows.
    f32x4 o[HT][8];
    float m_pv[HT][4];
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
#pragma unroll
      for (int n = 0; n < 8; ++n) o[ht][n] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int r = 0; r < 4; ++r) m_pv[ht][r] = -INFINITY;
    }
    // O += P V for one 32-key step of the tile in buffer cb
    auto pv_step = [&](int cb, int ks2) {
      const int kb = 32 * ks2;
      bf16x8 pf[HT];
#pragma unroll
      for (int ht = 0; ht < HT; ++ht)
        pf[ht] = __builtin_bit_cast(
            bf16x8, *reinterpret_cast<const u32x4*>(&sm.loop.p[cb][(16 * ht + li) * kPitch + kb + 8 * lq]));
      uint32_t vc[8];
      float vs[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const uint8_t* row = sm.loop.kv[cb][kb + 8 * lq + k];
        vc[k] = *reinterpret_cast<const uint32_t*>(row + 64 * dg + 4 * li);
        vs[k] = as_f32((uint32_t)row[256 + 4 * dg + (li >> 2)] << 23);
      }
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) {
        uint32_t xv[8];  // key k: bf16 pair of dims 8li + 2s4, +1
#pragma unroll
        for (int k = 0; k < 8; ++k) xv[k] = cvt_byte(vc[k], vs[k], s4);
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
    };
    // Tile step - 1 is consumed across the first barrier, overlapping the
    // producers' softmax between the two barriers (its buffers are not
    // rewritten before the next step).
    for (int64_t step = 0; step <= ntile; ++step) {
      const int cb = (int)(step & 1) ^ 1;
      if (step > 0) {
        // ---- O rows follow the running maxima (re-read only when a
        // producer flagged a move)
        if (sm.loop.moved[cb]) {
#pragma unroll
          for (int ht = 0; ht < HT; ++ht)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const float mnew = sm.loop.mpub[cb][16 * ht + 4 * lq + r];
              const float alpha = mnew == m_pv[ht][r] ? 1.0f : __builtin_amdgcn_exp2f(m_pv[ht][r] - mnew);
              m_pv[ht][r] = mnew;
#pragma unroll
              for (int n = 0; n < 8; ++n) o[ht][n][r] *= alpha;
            }
        }
        pv_step(cb, 0);
      }
      __syncthreads();
      if (step > 0) pv_step(cb, 1);
      __syncthreads();
    }

    // ---- sink, normalisation
    __syncthreads();
    __syncthreads();
#pragma unroll
    for (int ht = 0; ht < HT; ++ht)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int h = 16 * ht + 4 * lq + r;
        float sc = 1.0f;
        if (a.sink) {
          const float s2 = a.sink[h0 + h] * kLog2e;
          const float mf = fmaxf(m_pv[ht][r], s2);
          sc = m_pv[ht][r] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m_pv[ht][r] - mf);
        }
        const float lt = (sm.fin.l[0][h] + sm.fin.l[1][h]) + (sm.fin.l[2][h] + sm.fin.l[3][h]);
        float v[8];
#pragma unroll
        for (int n = 0; n < 8; ++n) v[n] = lt > 0.0f ? (o[ht][n][r] * sc) / lt : 0.0f;
        const u32x4 b = {bf16x2_rn(v[0], v[1]), bf16x2_rn(v[2], v[3]), bf16x2_rn(v[4], v[5]), bf16x2_rn(v[6], v[7])};
        uint16_t* orow = a.out + t * a.out_token_stride + (int64_t)(h0 + h) * a.out_head_stride + 128 * dg + 8 * li;
        if (a.out_aligned) {
          *reinterpret_cast<u32x4*>(orow) = b;
        } else {
#pragma unroll
          for (int n = 0; n < 8; ++n) orow[n] = (uint16_t)(b[n >> 1] >> (16 * (n & 1)));
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
