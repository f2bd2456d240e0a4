// kernels.hpp -- argument blocks and launchers of the libmxstore kernels.
// Host code (the C ABI) fills these after validating the caller's arguments.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.hpp"

namespace mxs {

struct StoreArgs {
  const uint16_t* src;   // bf16 [num_tokens, latent], row stride src_stride
  int64_t src_stride;    // elements, multiple of 8
  const int64_t* slots;  // [num_tokens]
  int64_t num_tokens;
  uint8_t* cache;
  SlotMap map;
  bool plain_stores;     // scatter form: plain stores for scattered rows too
};

// Rows written by one store launch that fit in MI355X's 256 MiB Infinity
// Cache: scattered rows of such a batch are written with plain stores (their
// partial 128-byte lines merge in that cache before they reach HBM); larger
// scattered batches stream with non-temporal stores, or take the slot-order
// form when they are dense.
constexpr int64_t kPlainStoreBytes = int64_t(256) << 20;

struct DequantArgs {
  const uint8_t* cache;
  SlotMap map;
  const int64_t* slots;  // [n]
  int64_t n;
  uint16_t* out;         // bf16 [n, latent], row stride out_stride
  int64_t out_stride;    // elements, multiple of 8
};

struct RopeArgs {
  const uint16_t* latent;  // bf16 [num_tokens, 512] contiguous
  const int64_t* positions;
  const float* cos_sin;
  int64_t cos_stride;  // elements
  int64_t cos_rows;
  uint8_t* cache;
  int64_t page_stride;  // bytes between pages of `block` tokens
  uint32_t block;
  int32_t block_shift;  // log2(block) or -1
  uint32_t num_slots;   // num_blocks * block
  const int64_t* slots;
  int64_t num_tokens;
  int32_t cr;
  int32_t sanitize;
};

struct RingArgs {
  const float* rows;  // [num_rows, width], row stride row_stride (elements)
  int64_t num_rows;
  int64_t width;      // multiple of 4
  int64_t row_stride;
  const int64_t* slots;
  float* state;       // ring: block stride state_stride, row stride state_row_stride
  uint32_t num_slots; // num_blocks * capacity
  uint32_t capacity;
  int64_t state_stride;
  int64_t state_row_stride;
};

struct NormArgs {
  const float* kv;        // [num_tokens, 512] fp32, row stride kv_row_stride (elements)
  int64_t num_tokens;
  int64_t kv_row_stride;
  const int64_t* slots;   // < 0: token not written
  const uint16_t* weight; // [512] bf16
  float eps;
  uint16_t* out;          // [num_tokens, 512] bf16, row stride out_row_stride (elements)
  int64_t out_row_stride;
};

struct AttnArgs {
  const uint16_t* q;          // bf16 [num_tokens, num_heads, 512] (strides in elements)
  int64_t q_token_stride;
  int64_t q_head_stride;
  const uint8_t* cache;       // MXFP4 rows of 272 bytes
  uint32_t cache_bytes;       // byte extent of the cache view if at most kAttnBufBytes (gathers
                              // through a raw buffer), else 0
  SlotMap map;
  const int32_t* indices;     // [num_tokens, topk], row stride idx_stride
  int64_t topk;
  int64_t idx_stride;
  float c;                    // |softmax scale| * log2(e) (> 0), or 1 when that is 0
  uint32_t q_xor, q_and;      // applied to each bf16 pair of q: 0x80008000 / ~0 for a
                              // negative scale (scores from -q times |scale|, exactly the
                              // same), 0 / 0 for a zero one (all scores 0), else 0 / ~0
  const float* sink;          // [num_heads] natural-log logits, or null
  uint16_t* out;              // bf16 [num_tokens, num_heads, 512]
  int64_t out_token_stride;
  int64_t out_head_stride;
  bool out_aligned;           // out 16-byte aligned, strides multiples of 8
  int32_t num_heads;          // multiple of 16
  int64_t num_tokens;
  int32_t splits;             // key ranges per (token, head block); > 1: partials to ws
  float* ws;                  // splits > 1: fp32 [T*H*splits][512] unnormalised outputs, then
                              // [T*H*splits][2] (running maximum in base 2, weight sum)
};

// Largest cache view the attention gathers through a raw buffer (32-bit
// offsets; offsets from here up read as zeros).
constexpr uint32_t kAttnBufBytes = 0xFFFF0000u;

// Each returns the hipError_t of the launch.
hipError_t launch_ring_rows(const RingArgs& a, hipStream_t stream);
hipError_t launch_compress_norm_cr1(const NormArgs& a, hipStream_t stream);
hipError_t launch_sparse_mla_attn(const AttnArgs& a, hipStream_t stream);
hipError_t launch_mxfp4_store(const StoreArgs& a, int latent, hipStream_t stream);
// Slot-order form: inverse[s] = token of slot s or -1 (num_slots int32,
// 16-byte aligned), then the gather-store over all slots.
hipError_t launch_build_inverse(const int64_t* slots, int64_t num_tokens, uint32_t num_slots,
                                int32_t* inverse, hipStream_t stream);
hipError_t launch_mxfp4_store_by_slot(const StoreArgs& a, int latent, const int32_t* inverse,
                                      hipStream_t stream);
// The slot-order store with its inverse map in the library's static device
// array (kNoAllocScratchBytes per GPU, looked up once per device): no
// allocation, no workspace.  The caller has checked that the map fits.
constexpr int64_t kNoAllocScratchBytes = int64_t(32) << 20;
hipError_t launch_mxfp4_store_slot_order_noalloc(const StoreArgs& a, int latent,
                                                 hipStream_t stream);
hipError_t launch_mxfp4_dequant(const DequantArgs& a, int latent, hipStream_t stream);
hipError_t launch_mxfp8_rope(const RopeArgs& a, hipStream_t stream);
hipError_t launch_nvfp4_rope(const RopeArgs& a, hipStream_t stream);
hipError_t launch_v4_rope(const RopeArgs& a, hipStream_t stream);

}  // namespace mxs
