// device_common.hpp -- small gfx950 device helpers shared by the kernels of
// libmxstore (cross-lane DPP moves, bit casts, paged slot addressing).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxs {

constexpr int kWave = 64;

// DPP control words (GFX9 encoding).
constexpr int kQuadSwap1 = 0xB1;  // quad_perm(1,0,3,2): partner lane ^ 1
constexpr int kQuadSwap2 = 0x4E;  // quad_perm(2,3,0,1): partner lane ^ 2
constexpr int kRowShr2 = 0x112;   // row_shr:2  (lane i reads lane i-2 in its row of 16)
constexpr int kRowShr4 = 0x114;
constexpr int kRowShr6 = 0x116;
constexpr int kRowShr8 = 0x118;
constexpr int kRowShr12 = 0x11C;

template <int Ctrl>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
  // row_mask/bank_mask 0xF: every lane; bound_ctrl: lanes with no source read 0.
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, Ctrl, 0xF, 0xF, true);
}

// Cache-policy bits of buffer instructions on gfx94x/gfx950: bit 1 = NT,
// bit 4 = SC1 (device scope).
constexpr int kBufNT = 2;
// NT + SC1: a store that goes through L2 to memory without staying dirty in
// L2 or the Infinity Cache.  For streams of whole-line writes this avoids
// the write-back of one launch's dirty lines during the next.  Scattered
// sub-line stores need the caches to merge them and must not use it.
constexpr int kBufNTDevice = kBufNT | 16;
// Buffer descriptor word 3 for GFX9 raw (untyped) buffers.
constexpr int kBufWord3 = 0x00020000;

// A raw buffer of `bytes` bytes at `base`.  Accesses at offsets >= bytes
// return zero (loads) or are dropped (stores) by the hardware range check,
// so bytes = 0 turns every access into a no-op without a branch.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_at(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kBufWord3);
}

// Workgroups are dispatched round-robin over the 8 XCDs of an MI355X, so
// consecutive blockIdx values land on different XCDs (and L2s).  This remap
// gives each XCD a contiguous range of logical blocks (all but the last
// gridDim % 8 blocks, which keep their index), so each XCD streams through
// its own region of the data; measured 4% faster for sequential row writes.
__device__ __forceinline__ uint32_t xcd_contiguous_block() {
  const uint32_t nb = gridDim.x, full = nb & ~7u, b = blockIdx.x;
  return b < full ? (b & 7u) * (full >> 3) + (b >> 3) : b;
}

__device__ __forceinline__ float as_f32(uint32_t u) { return __uint_as_float(u); }
__device__ __forceinline__ uint32_t as_u32(float f) { return __float_as_uint(f); }

// Row index of a slot in a paged layer view: blocks of block_size rows, block
// b starting block_stride_rows rows after block b-1.  Two forms, chosen on the
// host and passed as a template flag to the kernels: a power-of-two block
// size (shift/mask; a flat cache is the special case shift = 32, mask = all
// ones, so the block index is always 0) or a generic 32-bit division.  The
// caller has already checked 0 <= slot < num_slots < 2^32.
struct SlotMap {
  uint32_t num_slots;
  uint32_t block_size;
  uint32_t block_shift;  // pow2 form: log2(block_size), or 32 for a flat cache
  uint32_t block_mask;   // pow2 form: block_size - 1, or 0xFFFFFFFF for flat
  int64_t block_stride_rows;
  bool pow2;  // host-side: which form the launch instantiates

  template <bool kPow2>
  __device__ __forceinline__ int64_t row(uint32_t s) const {
    uint64_t q;
    uint32_t r;
    if (kPow2) {
      q = (uint64_t)s >> block_shift;
      r = s & block_mask;
    } else {
      const uint32_t q32 = s / block_size;
      q = q32;
      r = s - q32 * block_size;
    }
    return (int64_t)q * block_stride_rows + (int64_t)r;
  }
};

}  // namespace mxs
