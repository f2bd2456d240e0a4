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
// 64 keys.  The waves specialise by role and by a 128-dim slice of the
// latent, and two workgroups share a CU (both roles fit in 128 registers):
//   producers (waves pd = 0..3) compute partial scores S^T = K Q^T over
//            dims 128pd .. +127 for all 64 keys of tile s.  Lane (li, lq)
//            loads, one tile ahead, the 16 code bytes of dims 128pd + 32lq
//            .. +31 of keys 16kt + li (kt = 0..3) and their scale bytes;
//            gfx950's v_cvt_scalef32_pk_bf16_fp4 turns each code dword into
//            8 exact bf16 values -- the A operand of a 16x16x32 bf16 MFMA --
//            against query fragments of the same dims (B operand, all HB
//            heads, in registers), so every key is unpacked once.  Each
//            producer copies its slice of the packed rows to LDS for the
//            consumer of that slice and writes its partial scores to LDS
//            (a skipped key's partial is -inf in producer pd for key tile pd
//            and an exact 0 elsewhere).  After a barrier producer pd owns
//            heads HB/4*pd .. +HB/4-1 over all 64 keys: it adds the four
//            partials of its (head, key) pairs in a fixed order and runs the
//            softmax in base 2 on those sums, scaled only in the weights'
//            exponent -- the tile maximum of a head is reduced among the
//            head's consecutive lanes, the running maximum moves only past a
//            slack, and when it moves the new maxima are published with a
//            flag; weights go to LDS as bf16.
//   consumers (waves 4..7) own output dims 128*(w-4) .. +127 of all HB
//            heads and compute O += P V for tile s - 1.  The B operand needs
//            8 consecutive keys of one dim (a transpose of the cache layout):
//            lane (j = l%16, q = l/16) reads from the packed LDS copy the
//            code dword of dims 8j .. 8j+7 of its slab for keys 8q .. 8q+7
//            of a 32-key step and their scale bytes, converts each (bf16
//            pairs along dims) and re-pairs the halves along keys with
//            v_perm_b32: 8 B operands for 8 MFMAs whose output column j is
//            dim 8j + n of the slab.
// The packed-row buffers alternate between tiles; a step costs two barriers
// (partial scores, weights), and the consumers do all their work before the
// first.  At the end each owner folds the sink into its heads' weight sums,
// and O / l is rounded to bf16.
#include <type_traits>
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
// bf16 per LDS weight row: 160 bytes, 8 dwords past a multiple of 32, at
// which rows read or written 16 bytes each at one column meet no bank
// conflict (measured).
constexpr int kPitch = kTile + 16;
// A key's row in LDS: its 256 code bytes, then the 16 group scales as fp32
// (E8M0 byte in the exponent field, the form the converter takes), 8 bytes
// of padding: rows 328 bytes apart, so rows 8 apart start 16 banks apart and
// the consumers' reads of keys 8q + k (q = 0..3) do not collide.
constexpr int kKvPitch = 328;
constexpr int kKvScales = 256;
// The running maximum is raised only when a tile's maximum exceeds it by more
// than this (base-2 units): weights stay below 2^8, far from fp32 / bf16
// overflow, and most tiles need no rescaling of O.
constexpr float kMaxSlack = 8.0f;
// Row index standing for a skipped key in views gathered through a raw
// buffer: every byte of its row lies at an offset at or past the largest
// such view and below 2^32, so its loads read zeros with no test, and no row
// of such a view (fewer than kAttnBufBytes / 272 rows) has this index.
constexpr uint32_t kRowSkip = 0xF0F0EFu;
static_assert((uint64_t)kRowSkip * kRowBytes >= kAttnBufBytes &&
              (uint64_t)kRowSkip * kRowBytes + kRowBytes <= 0x100000000ull &&
              kRowSkip < (1u << 24) && kAttnBufBytes / kRowBytes < kRowSkip,
              "skip row must read past every buffered view");

template <int HB>
struct AttnSmem {
  static constexpr int HT = HB / 16;
  union {
    struct {
      uint8_t kv[2][kTile][kKvPitch];        // packed rows of a tile
      uint16_t p[HB * kPitch];               // the latest tile's weights (bf16): [head][key]
      // partial scores, 16 bytes (4 keys of one head) each: row (producer,
      // head tile, sub-block q, head li) holds the head's key blocks kk, at
      // column kk ^ li (see the producer); an owner's 8 lanes of one head
      // read one 128-byte row, and 8 writing lanes hit 8 distinct columns
      f32x4 sp[kProducers * kProducers * HT * kWave];
      float mpub[HB];                        // running maxima after the latest tile
      uint32_t moved[2];                     // some head's running maximum moved at that tile
    } loop;
    struct {
      float l[HB];                           // weight sums (the sink folded in)
    } fin;
  };
};

// Reductions over aligned groups of 8 or 16 consecutive lanes, in DPP
// steps: swap neighbours, swap pairs, mirror within 8 lanes, mirror within
// 16.  Every lane ends with the same value (each step combines two values
// the same way in both lanes).  The maximum is written as v_max_f32 with a
// DPP operand directly: through fmaxf the compiler would add NaN-quieting
// moves on the moved value (scores are never NaN).  A DPP read of a VGPR
// written by the previous VALU instruction needs two wait states.
template <int N>
__device__ __forceinline__ float max_lanes(float v) {
  asm("s_nop 1\n\tv_max_f32_dpp %0, %1, %1 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf" : "=v"(v) : "v"(v));
  asm("s_nop 1\n\tv_max_f32_dpp %0, %1, %1 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf" : "=v"(v) : "v"(v));
  asm("s_nop 1\n\tv_max_f32_dpp %0, %1, %1 row_half_mirror row_mask:0xf bank_mask:0xf" : "=v"(v) : "v"(v));
  if constexpr (N == 16)
    asm("s_nop 1\n\tv_max_f32_dpp %0, %1, %1 row_mirror row_mask:0xf bank_mask:0xf" : "=v"(v) : "v"(v));
  return v;
}
template <int N>
__device__ __forceinline__ float sum_lanes(float v) {
  v += as_f32((uint32_t)__builtin_amdgcn_mov_dpp((int)as_u32(v), 0xB1, 0xF, 0xF, true));   // quad_perm [1,0,3,2]
  v += as_f32((uint32_t)__builtin_amdgcn_mov_dpp((int)as_u32(v), 0x4E, 0xF, 0xF, true));   // quad_perm [2,3,0,1]
  v += as_f32((uint32_t)__builtin_amdgcn_mov_dpp((int)as_u32(v), 0x141, 0xF, 0xF, true));  // row_half_mirror
  if constexpr (N == 16) v += as_f32((uint32_t)__builtin_amdgcn_mov_dpp((int)as_u32(v), 0x140, 0xF, 0xF, true));  // row_mirror
  return v;
}

// Two workgroups per CU: at most 128 registers per lane (4 waves per SIMD).
template <int HB, bool kPow2, bool kBuf, bool kSplit>
__global__ __launch_bounds__(kWave * kWaves) __attribute__((amdgpu_waves_per_eu(4)))
void sparse_mla_attn_kernel(const AttnArgs a) {
  constexpr int HT = HB / 16;
  __shared__ AttnSmem<HB> sm;
  const int lane = threadIdx.x & (kWave - 1);
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int li = lane & 15, lq = lane >> 4;
  const bool producer = w < kProducers;
  const int dg = w - kProducers;     // consumer: dims 128dg .. +127
  const uint32_t nhb = (uint32_t)(a.num_heads / HB);
  // Split form: consecutive blocks take consecutive key ranges (whole tiles)
  // of one (token, head block).
  const uint32_t nsplit = kSplit ? (uint32_t)a.splits : 1u;
  const uint32_t blk_all = xcd_contiguous_block();
  const uint32_t split = kSplit ? blk_all % nsplit : 0u;
  const uint32_t blk = kSplit ? blk_all / nsplit : blk_all;
  const int64_t t = blk / nhb;
  const int h0 = (int)(blk % nhb) * HB;
  // topk <= 2^24: tile counts fit in 32 bits (and compare in scalar registers)
  const int32_t ntile_all = (int32_t)((a.topk + kTile - 1) / kTile);
  const int32_t per_split = (ntile_all + (int32_t)nsplit - 1) / (int32_t)nsplit;
  const int32_t tile0 = (int32_t)split * per_split;
  const int32_t ntile = kSplit ? (tile0 < ntile_all ? min(per_split, ntile_all - tile0) : 0) : ntile_all;

  const int32_t* idx_row = a.indices + t * a.idx_stride;
  if (threadIdx.x < 2) sm.loop.moved[threadIdx.x] = 0u;  // ordered by the first barrier

  // Producers and consumers run separate loops (so their registers are not
  // live at the same time) with the same barriers: two per step, step s
  // producing tile s and consuming tile s - 1, then two in the epilogue.
  // The producer body is instantiated per slice (pd a constant: its LDS
  // offsets and own-tile choice fold away).
  if (producer) {
    auto produce = [&](auto pdc) {
      // Producer pd = w owns dims 128pd .. +127 of every key of a tile: lane
      // (li, lq) holds, for key tile kt = 0..3, the 16 code bytes of dims
      // 128pd + 32lq .. +31 of key 16kt + li and their scale byte, and the
      // query fragments of those dims for all HB heads (B operand: head li,
      // dims 128pd + 32lq + 8ks .. +7 at k-step ks).  Its MFMAs give partial
      // scores over its 128 dims for all 64 keys; the four partials meet in
      // LDS, where each producer sums those of the heads it owns.
      constexpr int pd = decltype(pdc)::value;
      bf16x8 qf[HT][4];
      // After the first barrier of a step producer pd owns heads HPO*pd ..
      // +HPO-1 over all 64 keys: lane (hh, kk) = hh*LPH + kk holds head
      // HPO*pd + hh and keys KPL*kk .. +KPL-1 (a head's lanes are LPH
      // consecutive ones), whose scores it reads from NQ slots of each
      // producer's partial-score tiles.
      constexpr int HPO = HB / kProducers, KPL = kTile * HPO / kWave, NQ = KPL / 4, LPH = kWave / HPO;
      const int kk = lane % LPH, hh = lane / LPH;
      const int oh = HPO * pd + hh, oht = oh >> 4, oli = oh & 15;
      // Partial-score slot of (producer v, head tile ht, sub-block q, head
      // li, key block kk): keys KPL*kk + 4q .. +3 of head 16ht + li.
      auto sp_at = [](int v, int ht, int q, int li, int kk) {
        return (((v * HT + ht) * NQ + q) * 16 + li) * LPH + (kk ^ (li & (LPH - 1)));
      };
      float m_own = -INFINITY, lsum = 0.0f;
#pragma unroll
      for (int ht = 0; ht < HT; ++ht) {
        const uint16_t* qh = a.q + t * a.q_token_stride + (int64_t)(h0 + 16 * ht + li) * a.q_head_stride +
                             128 * pd + 32 * lq;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
          qf[ht][ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(qh + 8 * ks));
      }
      if (a.q_xor != 0u || a.q_and != ~0u) {  // a negative or zero scale
#pragma unroll
        for (int ht = 0; ht < HT; ++ht)
#pragma unroll
          for (int ks = 0; ks < 4; ++ks)
            qf[ht][ks] = __builtin_bit_cast(bf16x8, (__builtin_bit_cast(u32x4, qf[ht][ks]) ^ a.q_xor) & a.q_and);
      }
      // Slot index of key 16lq + li (one load per lane covers the tile),
      // through a raw buffer over the tile's listed entries (topk <= 2^24):
      // unconditional (lanes past the list read 0 and return -1) so the
      // compiler's wait counts stay exact.  Loads run only when topk >= 1.
      auto load_index = [&](int32_t tile) -> int32_t {
        const int64_t j0 = (int64_t)(tile0 + tile) * kTile, rem = a.topk - j0;
        const uint32_t n = rem <= 0 ? 0u : rem >= kTile ? (uint32_t)kTile : (uint32_t)rem;
        const int32_t v = (int32_t)__builtin_amdgcn_raw_buffer_load_b32(buffer_at(idx_row + j0, 4u * n), 4 * lane, 0, 0);
        return (uint32_t)lane < n ? v : -1;
      };
      // Below 4 GiB a view has fewer than 2^24 rows, so a listed slot's row
      // and its byte offset come from 24-bit products (full-rate multiplies):
      // block index and stride are both below 2^24 unless there is a single
      // block, whose index is 0.  A skipped key's row is kRowSkip there, -1
      // otherwise.
      auto row_index = [&](int32_t s) -> int32_t {
        const bool ok = (uint32_t)s < a.map.num_slots;  // fewer than 2^31 slots
        if constexpr (kBuf) {
          uint32_t q, r;
          if constexpr (kPow2) {
            q = (uint32_t)((uint64_t)(uint32_t)s >> a.map.block_shift);
            r = (uint32_t)s & a.map.block_mask;
          } else {
            q = (uint32_t)s / a.map.block_size;
            r = (uint32_t)s - q * a.map.block_size;
          }
          return ok ? (int32_t)(__umul24(q, (uint32_t)a.map.block_stride_rows) + r) : (int32_t)kRowSkip;
        } else {
          return ok ? (int32_t)a.map.template row<kPow2>((uint32_t)s) : -1;
        }
      };
      // Rows of keys 16kt + li, kt = 0..3, from the lanes (li, kt) that hold
      // them (permlane swaps: lane (li, lq) ends with the value of lane (li, kt)).
      auto spread_rows = [&](int32_t x, int32_t (&rows)[4]) {
        const auto ab = __builtin_amdgcn_permlane32_swap((uint32_t)x, (uint32_t)x, false, false);
        const auto c0 = __builtin_amdgcn_permlane16_swap(ab[0], ab[0], false, false);
        const auto c1 = __builtin_amdgcn_permlane16_swap(ab[1], ab[1], false, false);
        rows[0] = (int32_t)c0[0];
        rows[1] = (int32_t)c0[1];
        rows[2] = (int32_t)c1[0];
        rows[3] = (int32_t)c1[1];
      };
      // Through a raw buffer over the cache view when it spans less than
      // kAttnBufBytes: a skipped key's row kRowSkip lies past the view, so its
      // codes and scale read as zeros (zero values); otherwise global loads
      // of row 0, masked where they are used.  Lane (li, lq) loads the scale
      // byte of its own 32 dims.
      const __amdgpu_buffer_rsrc_t crs = buffer_at(a.cache, kBuf ? a.cache_bytes : 0u);
      auto gather = [&](const int32_t (&rows)[4], u32x4 (&c)[4], uint32_t (&sb)[4]) {
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
          if constexpr (kBuf) {
            const uint32_t base = __umul24((uint32_t)rows[kt], kRowBytes);
            c[kt] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(crs, base + 64 * pd + 16 * lq, 0, 0));
            sb[kt] = __builtin_amdgcn_raw_buffer_load_b8(crs, base + 256 + 4 * pd + lq, 0, 0);
          } else {
            const uint8_t* rp = a.cache + (int64_t)(rows[kt] < 0 ? 0 : rows[kt]) * kRowBytes;
            c[kt] = *reinterpret_cast<const u32x4*>(rp + 64 * pd + 16 * lq);
            sb[kt] = rp[256 + 4 * pd + lq];
          }
        }
      };
      // The gather of a tile is issued right after the previous tile's scores
      // (one tile ahead); slot indices are loaded one tile earlier still.
      int32_t g_own = -1, g_idx = -1;  // row of key 16lq + li; next tile's index
      u32x4 g_cw[4];
      uint32_t g_sb[4];  // scale byte of the lane's 32 dims, per key tile
      if (ntile > 0) {
        g_own = row_index(load_index(0));
        int32_t rows[4];
        spread_rows(g_own, rows);
        gather(rows, g_cw, g_sb);
        g_idx = load_index(1);
      }

      for (int32_t step = 0; step <= ntile; ++step) {
        const int pb = (int)(step & 1), cb = pb ^ 1;
        uint64_t valid = 0;  // bit k: key k of the tile is listed
        if (step < ntile) {
          // ---- the packed slice to LDS for consumer pd; partial scores
          valid = __ballot(kBuf ? g_own != (int32_t)kRowSkip : g_own >= 0);
#pragma unroll
          for (int kt = 0; kt < 4; ++kt) {
            if (!kBuf && !((valid >> (16 * kt + li)) & 1u)) {
              g_cw[kt] = u32x4{0u, 0u, 0u, 0u};
              g_sb[kt] = 0u;
            }
            uint8_t* dst = sm.loop.kv[pb][16 * kt + li];
            *reinterpret_cast<uint64_t*>(dst + 64 * pd + 16 * lq) = (uint64_t)g_cw[kt][0] | ((uint64_t)g_cw[kt][1] << 32);
            *reinterpret_cast<uint64_t*>(dst + 64 * pd + 16 * lq + 8) = (uint64_t)g_cw[kt][2] | ((uint64_t)g_cw[kt][3] << 32);
            *reinterpret_cast<float*>(dst + kKvScales + 4 * (4 * pd + lq)) = as_f32(g_sb[kt] << 23);
          }
          // Key tile by key tile: partial scores over the 128 dims, to LDS
          // for the owners of their heads.  The accumulators start at 0,
          // except that in key tile pd those of skipped keys (rows 4lq + r)
          // start at -inf: a skipped key's codes are zeros, so its partials
          // are exact zeros but for this one, and its score sum is -inf.
          f32x4 bias;
          {
            const uint32_t skip = (uint32_t)(~valid >> (16 * pd)) >> (4 * lq);
#pragma unroll
            for (int r = 0; r < 4; ++r) bias[r] = as_f32((0u - ((skip >> r) & 1u)) & 0xFF800000u);
          }
#pragma unroll
          for (int kt = 0; kt < 4; ++kt) {
            f32x4 s[HT];
#pragma unroll
            for (int ht = 0; ht < HT; ++ht) s[ht] = kt == pd ? bias : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
            const uint32_t sbyte = g_sb[kt];
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
              const bf16x8 kf = __builtin_bit_cast(bf16x8, unpack8(g_cw[kt][ks], sbyte));
#pragma unroll
              for (int ht = 0; ht < HT; ++ht)
                s[ht] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[ht][ks], s[ht], 0, 0, 0);
            }
#pragma unroll
            for (int ht = 0; ht < HT; ++ht)
              sm.loop.sp[sp_at(pd, ht, ((16 * kt + 4 * lq) % KPL) / 4, li, (16 * kt + 4 * lq) / KPL)] = s[ht];
          }
          // ---- next tile's gather (the index load goes first: waiting for it
          // later must not wait for the gather, as loads complete in order)
          const int32_t nxt = g_idx;
          g_idx = load_index(step + 2);
          g_own = row_index(nxt);
          int32_t rows[4];
          spread_rows(g_own, rows);
          gather(rows, g_cw, g_sb);
        }
        __syncthreads();
        if (step < ntile) {
          // ---- owned heads: score sums (the four producers' partials in a
          // fixed order; -inf for skipped keys), the tile maximum over the
          // head's lanes, running maximum, weights, partial sum; publish.
          // The sums are scaled by c > 0 only in the weights' exponent (one
          // fma): max_j fl(c x_j) = fl(c max_j x_j), as rounding is monotonic.
          if (threadIdx.x == 0) sm.loop.moved[cb] = 0u;  // read as tile step - 1's flag before the first barrier
          float x[KPL];
#pragma unroll
          for (int q = 0; q < NQ; ++q) {
            f32x4 part[kProducers];
#pragma unroll
            for (int v = 0; v < kProducers; ++v)
              part[v] = sm.loop.sp[sp_at(v, oht, q, oli, kk)];
#pragma unroll
            for (int r = 0; r < 4; ++r) x[4 * q + r] = (part[0][r] + part[1][r]) + (part[2][r] + part[3][r]);
          }
          float mt = x[0];
#pragma unroll
          for (int j = 1; j < KPL; ++j) mt = fmaxf(mt, x[j]);
          mt = max_lanes<LPH>(mt) * a.c;
          const float mnew = mt > m_own + kMaxSlack ? mt : m_own;
          const bool mv = mnew != m_own;
          // mnew is -inf only while every key so far was skipped (x = -inf);
          // alpha is exactly 1 when the maximum did not move, and 0 while
          // m_own is -inf
          const float mref = mnew == -INFINITY ? 0.0f : mnew;
          const float alpha = __builtin_amdgcn_exp2f(m_own - mref);
          float pw[KPL];
#pragma unroll
          for (int j = 0; j < KPL; ++j) pw[j] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[j], a.c, -mref));
          float ps = (pw[0] + pw[1]) + (pw[2] + pw[3]);
#pragma unroll
          for (int q = 1; q < NQ; ++q) ps += (pw[4 * q] + pw[4 * q + 1]) + (pw[4 * q + 2] + pw[4 * q + 3]);
          lsum = __builtin_fmaf(lsum, alpha, ps);
          m_own = mnew;
          uint16_t* prow = &sm.loop.p[oh * kPitch + KPL * kk];
          if constexpr (KPL == 8) {
            *reinterpret_cast<u32x4*>(prow) = u32x4{bf16x2_rn(pw[0], pw[1]), bf16x2_rn(pw[2], pw[3]),
                                                    bf16x2_rn(pw[4], pw[5]), bf16x2_rn(pw[6], pw[7])};
          } else {
            *reinterpret_cast<uint64_t*>(prow) =
                (uint64_t)bf16x2_rn(pw[0], pw[1]) | ((uint64_t)bf16x2_rn(pw[2], pw[3]) << 32);
          }
          if (kk == 0) sm.loop.mpub[oh] = mnew;
          if (__any(mv) && lane == 0) sm.loop.moved[pb] = 1u;
        }
        __syncthreads();
      }

      // ---- weight sum of the owned head over its lanes (fixed order), sink
      float l = sum_lanes<LPH>(lsum);
      if (a.sink && !kSplit) {  // the split form folds the sink in when merging
        const float s2 = a.sink[h0 + oh] * kLog2e;
        const float mf = fmaxf(m_own, s2);
        l = (m_own == -INFINITY ? 0.0f : l * __builtin_amdgcn_exp2f(m_own - mf)) + __builtin_amdgcn_exp2f(s2 - mf);
      }
      __syncthreads();  // the loop's LDS is reused
      if (kk == 0) sm.fin.l[oh] = l;
      __syncthreads();
    };
    switch (w) {
      case 0: produce(std::integral_constant<int, 0>{}); break;
      case 1: produce(std::integral_constant<int, 1>{}); break;
      case 2: produce(std::integral_constant<int, 2>{}); break;
      default: produce(std::integral_constant<int, 3>{}); break;
    }
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
            bf16x8, *reinterpret_cast<const u32x4*>(&sm.loop.p[(16 * ht + li) * kPitch + kb + 8 * lq]));
      uint32_t vc[8];
      float vs[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const uint8_t* row = sm.loop.kv[cb][kb + 8 * lq + k];
        vc[k] = *reinterpret_cast<const uint32_t*>(row + 64 * dg + 4 * li);
        vs[k] = *reinterpret_cast<const float*>(row + kKvScales + 4 * (4 * dg + (li >> 2)));
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
    // Tile step - 1 is consumed before the first barrier, beside the
    // producers' scores of tile step (its buffers are rewritten only in the
    // next step).
    for (int32_t step = 0; step <= ntile; ++step) {
      const int cb = (int)(step & 1) ^ 1;
      if (step > 0) {
        // ---- O rows follow the running maxima (re-read only when a
        // producer flagged a move)
        if (sm.loop.moved[cb]) {
#pragma unroll
          for (int ht = 0; ht < HT; ++ht)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const float mnew = sm.loop.mpub[16 * ht + 4 * lq + r];
              const float alpha = mnew == m_pv[ht][r] ? 1.0f : __builtin_amdgcn_exp2f(m_pv[ht][r] - mnew);
              m_pv[ht][r] = mnew;
#pragma unroll
              for (int n = 0; n < 8; ++n) o[ht][n][r] *= alpha;
            }
        }
        pv_step(cb, 0);
        pv_step(cb, 1);
      }
      __syncthreads();
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
        const float lt = sm.fin.l[h];
        if constexpr (kSplit) {
          // Unnormalised partial output and (running maximum, weight sum)
          // of this key range, merged by attn_merge_kernel.
          const int64_t prow = ((t * a.num_heads + h0 + h) * nsplit + split);
          f32x4* po = reinterpret_cast<f32x4*>(a.ws + prow * 512 + 128 * dg + 8 * li);
          po[0] = f32x4{o[ht][0][r], o[ht][1][r], o[ht][2][r], o[ht][3][r]};
          po[1] = f32x4{o[ht][4][r], o[ht][5][r], o[ht][6][r], o[ht][7][r]};
          if (dg == 0 && li == 0) {
            float* pml = a.ws + a.num_tokens * a.num_heads * nsplit * 512 + prow * 2;
            pml[0] = m_pv[ht][r];
            pml[1] = lt;
          }
          continue;
        }
        float sc = 1.0f;
        if (a.sink) {
          const float s2 = a.sink[h0 + h] * kLog2e;
          const float mf = fmaxf(m_pv[ht][r], s2);
          sc = m_pv[ht][r] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m_pv[ht][r] - mf);
        }
        // One division per row, then products (within an fp32 ulp of
        // dividing each value; the bf16 rounding that follows dominates).
        const float inv = lt > 0.0f ? sc / lt : 0.0f;
        float v[8];
#pragma unroll
        for (int n = 0; n < 8; ++n) v[n] = lt > 0.0f ? o[ht][n][r] * inv : 0.0f;
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

// Merge of the split form.  With M the largest running maximum of the key
// ranges (and the sink logit, base 2), out = sum_i 2^(m_i - M) O_i /
// (sum_i 2^(m_i - M) l_i + 2^(sink - M)): the same value as one pass over
// all keys; zeros when no range saw a valid key.  A (token, head) row is
// merged by wpr = 1, 2, 4 or 8 waves (ceil(ranges / 8), at most 64 ranges):
// lane i reads range i's (m, l); wave sub of the row adds the outputs of
// ranges sub, sub + wpr, ... (lane l: dims 8l .. +7, all loads issued at
// once) and the row's waves meet in LDS.  A workgroup of 8 waves holds
// 8 / wpr rows.
constexpr int kMergeWaves = 8;

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

__device__ __forceinline__ float wave_add(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__global__ __launch_bounds__(kWave * kMergeWaves) void attn_merge_kernel(const AttnArgs a, int wpr) {
  __shared__ f32x4 part[kMergeWaves][kWave][2];
  const int lane = threadIdx.x & (kWave - 1);
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int sub = w % wpr;
  const int64_t row = (int64_t)blockIdx.x * (kMergeWaves / wpr) + w / wpr;  // t * num_heads + h
  const bool live = row < a.num_tokens * a.num_heads;
  const int ns = a.splits;
  f32x4 acc0 = {0.0f, 0.0f, 0.0f, 0.0f}, acc1 = acc0;
  float mx = -INFINITY, lt = 0.0f;
  if (live) {
    const float* ml = a.ws + a.num_tokens * a.num_heads * ns * 512 + row * ns * 2;
    float mi = -INFINITY, li_ = 0.0f;
    if (lane < ns) {
      mi = ml[2 * lane];
      li_ = ml[2 * lane + 1];
    }
    mx = wave_max(mi);
    float mf = mx, sink_w = 0.0f;
    if (a.sink && mx != -INFINITY) {
      const float s2 = a.sink[row % a.num_heads] * kLog2e;
      mf = fmaxf(mx, s2);
      sink_w = __builtin_amdgcn_exp2f(s2 - mf);
    }
    const float wi = mi == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mi - mf);
    lt = wave_add(li_ * wi) + sink_w;
    f32x4 p[8][2];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int i = sub + wpr * k;
      if (i < ns) {
        const f32x4* po = reinterpret_cast<const f32x4*>(a.ws + (row * ns + i) * 512 + 8 * lane);
        p[k][0] = po[0];
        p[k][1] = po[1];
      }
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int i = sub + wpr * k;
      if (i < ns) {
        const float wk = __shfl(wi, i);
        acc0 += p[k][0] * wk;
        acc1 += p[k][1] * wk;
      }
    }
  }
  if (wpr > 1) {
    part[w][lane][0] = acc0;
    part[w][lane][1] = acc1;
    __syncthreads();
    if (sub != 0) return;
#pragma unroll
    for (int k = 1; k < kMergeWaves; ++k) {
      if (k < wpr) {
        acc0 += part[w + k][lane][0];
        acc1 += part[w + k][lane][1];
      }
    }
  }
  if (!live) return;
  float v[8];
#pragma unroll
  for (int n = 0; n < 4; ++n) {
    v[n] = mx != -INFINITY && lt > 0.0f ? acc0[n] / lt : 0.0f;
    v[4 + n] = mx != -INFINITY && lt > 0.0f ? acc1[n] / lt : 0.0f;
  }
  const u32x4 b = {bf16x2_rn(v[0], v[1]), bf16x2_rn(v[2], v[3]), bf16x2_rn(v[4], v[5]), bf16x2_rn(v[6], v[7])};
  const int64_t t = row / a.num_heads;
  uint16_t* orow = a.out + t * a.out_token_stride + (row % a.num_heads) * a.out_head_stride + 8 * lane;
  if (a.out_aligned) {
    *reinterpret_cast<u32x4*>(orow) = b;
  } else {
#pragma unroll
    for (int n = 0; n < 8; ++n) orow[n] = (uint16_t)(b[n >> 1] >> (16 * (n & 1)));
  }
}

template <int HB, bool kPow2, bool kSplit>
hipError_t launch_map(const AttnArgs& a, unsigned blocks, hipStream_t stream) {
  if (a.cache_bytes != 0u)
    hipLaunchKernelGGL((sparse_mla_attn_kernel<HB, kPow2, true, kSplit>), dim3(blocks), dim3(kWave * kWaves), 0,
                       stream, a);
  else
    hipLaunchKernelGGL((sparse_mla_attn_kernel<HB, kPow2, false, kSplit>), dim3(blocks), dim3(kWave * kWaves), 0,
                       stream, a);
  return hipGetLastError();
}

template <int HB>
hipError_t launch_hb(const AttnArgs& a, hipStream_t stream) {
  const int64_t blocks = a.num_tokens * (a.num_heads / HB) * a.splits;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  hipError_t e;
  if (a.splits > 1) {
    e = a.map.pow2 ? launch_map<HB, true, true>(a, (unsigned)blocks, stream)
                   : launch_map<HB, false, true>(a, (unsigned)blocks, stream);
    if (e != hipSuccess) return e;
    const int64_t rows = a.num_tokens * a.num_heads;
    const int wpr = a.splits <= 8 ? 1 : a.splits <= 16 ? 2 : a.splits <= 32 ? 4 : 8;
    const int64_t mblocks = (rows * wpr + kMergeWaves - 1) / kMergeWaves;
    if (mblocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(attn_merge_kernel, dim3((unsigned)mblocks), dim3(kWave * kMergeWaves), 0, stream, a, wpr);
    return hipGetLastError();
  }
  return a.map.pow2 ? launch_map<HB, true, false>(a, (unsigned)blocks, stream)
                    : launch_map<HB, false, false>(a, (unsigned)blocks, stream);
}

}  // namespace

hipError_t launch_sparse_mla_attn(const AttnArgs& a, hipStream_t stream) {
  if (a.num_tokens == 0) return hipSuccess;
  if (a.num_heads % 32 == 0) return launch_hb<32>(a, stream);
  return launch_hb<16>(a, stream);
}

}  // namespace mxs
