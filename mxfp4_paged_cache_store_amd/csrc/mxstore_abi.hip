// mxstore_abi.hip -- the extern "C" boundary of libmxstore.so: argument
// validation (mirroring the checks of the pages' Python wrappers, plus the
// alignment and range rules the gfx950 kernels rely on) and the launch on the
// caller's stream.  No allocation, no synchronisation.  Declarations and the
// full contract are in include/mxstore.h.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include "mxstore.h"
#include "kernels.hpp"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = '\0';
  return MX_OK;
}

bool is_pow2(int64_t v) { return v > 0 && (v & (v - 1)) == 0; }

int log2_exact(int64_t v) {
  int k = 0;
  while ((int64_t(1) << k) < v) ++k;
  return k;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Shared checks of the paged MXFP4 layer view [store page, `store_mxfp4_mla`:
// whole rows per block; block stride may exceed the block].
int check_paged(int64_t latent, int32_t group, int64_t num_blocks, int64_t block_size,
                int64_t block_stride_rows, mxs::SlotMap* map) {
  if (group != 32) return fail(MX_E_SHAPE, "group must be 32 (one E8M0 scale per 32 values), got %d", group);
  if (!is_pow2(latent) || latent < 128 || latent > 2048)
    return fail(MX_E_SHAPE, "latent must be a power of two in [128, 2048], got %lld", (long long)latent);
  if (num_blocks < 1 || block_size < 1)
    return fail(MX_E_RANGE, "num_blocks (%lld) and block_size (%lld) must be >= 1",
                (long long)num_blocks, (long long)block_size);
  if (block_stride_rows < block_size)
    return fail(MX_E_STRIDE, "block_stride_rows (%lld) is smaller than block_size (%lld)",
                (long long)block_stride_rows, (long long)block_size);
  if (num_blocks > (int64_t(0xFFFFFFFF) / block_size))
    return fail(MX_E_RANGE, "num_blocks * block_size must stay below 2^32");
  map->num_slots = (uint32_t)(num_blocks * block_size);
  map->block_size = (uint32_t)block_size;
  map->block_stride_rows = block_stride_rows;
  if (num_blocks == 1 || block_stride_rows == block_size) {
    // Contiguous blocks: the row is the slot itself.
    map->block_shift = 32;
    map->block_mask = 0xFFFFFFFFu;
    map->pow2 = true;
  } else if (is_pow2(block_size)) {
    map->block_shift = (uint32_t)log2_exact(block_size);
    map->block_mask = (uint32_t)block_size - 1u;
    map->pow2 = true;
  } else {
    map->block_shift = 0;
    map->block_mask = 0;
    map->pow2 = false;
  }
  return MX_OK;
}

int launched(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(MX_E_LAUNCH, "%s launch failed: %s", what, hipGetErrorString(e));
  return ok();
}

int check_rope(const uint16_t* latent, const int64_t* positions, const float* cos_sin,
               int64_t cos_stride, int64_t cos_rows, uint8_t* cache, int64_t page_stride,
               int64_t block, int64_t num_blocks, const int64_t* slots, int64_t num_tokens,
               int32_t cr, int64_t record, mxs::RopeArgs* a) {
  if (num_tokens < 0) return fail(MX_E_RANGE, "num_tokens must be >= 0");
  if (cr < 1) return fail(MX_E_ARG, "compress_ratio must be >= 1, got %d", cr);
  if (block < 1 || num_blocks < 1) return fail(MX_E_RANGE, "cache_block and num_blocks must be >= 1");
  if (num_blocks > (int64_t(0xFFFFFFFF) / block)) return fail(MX_E_RANGE, "num_blocks * cache_block must stay below 2^32");
  if (page_stride < block * record || page_stride % 16)
    return fail(MX_E_STRIDE, "cache_block_stride (%lld) must be a multiple of 16 and >= cache_block * %lld",
                (long long)page_stride, (long long)record);
  if (cos_stride < 64) return fail(MX_E_STRIDE, "cos_stride must be >= 64, got %lld", (long long)cos_stride);
  if (cos_rows < 0) return fail(MX_E_RANGE, "cos_rows must be >= 0");
  if (num_tokens > 0 && (!latent || !positions || !cos_sin || !cache || !slots))
    return fail(MX_E_NULL, "null device pointer");
  if (!aligned(latent, 16) || !aligned(cache, 16) || !aligned(cos_sin, 4))
    return fail(MX_E_ALIGN, "latent and cache must be 16-byte aligned, cos_sin 4-byte aligned");
  a->latent = latent;
  a->positions = positions;
  a->cos_sin = cos_sin;
  a->cos_stride = cos_stride;
  a->cos_rows = cos_rows;
  a->cache = cache;
  a->page_stride = page_stride;
  a->block = (uint32_t)block;
  a->block_shift = is_pow2(block) ? log2_exact(block) : -1;
  a->num_slots = (uint32_t)(num_blocks * block);
  a->slots = slots;
  a->num_tokens = num_tokens;
  a->cr = cr;
  return MX_OK;
}


// Argument checks shared by mxfp4_store and mxfp4_store_by_slot; `index` is
// the slot list or the inverse map (only checked for NULL here).  Returns
// MX_OK with `a` filled (a->slots left unset), or an error status; *empty is
// set for num_tokens == 0.
int check_store(const uint16_t* src_bf16, int64_t num_tokens, int64_t latent,
                int64_t src_row_stride, const void* index, uint8_t* cache,
                int64_t num_blocks, int64_t block_size, int64_t block_stride_rows,
                int32_t group, mxs::StoreArgs* a, bool* empty) {
  int rc = check_paged(latent, group, num_blocks, block_size, block_stride_rows, &a->map);
  if (rc) return rc;
  if (num_tokens < 0) return fail(MX_E_RANGE, "num_tokens must be >= 0");
  if (src_row_stride < latent)
    return fail(MX_E_STRIDE, "src_row_stride (%lld) is smaller than latent (%lld)",
                (long long)src_row_stride, (long long)latent);
  *empty = num_tokens == 0;
  if (*empty) return MX_OK;
  if (!src_bf16 || !index || !cache) return fail(MX_E_NULL, "null device pointer");
  if (!aligned(src_bf16, 16) || src_row_stride % 8)
    return fail(MX_E_ALIGN, "latent rows must be 16-byte aligned (base %% 16 == 0, row stride %% 8 == 0)");
  if (!aligned(cache, 4)) return fail(MX_E_ALIGN, "cache must be 4-byte aligned");
  a->src = src_bf16;
  a->src_stride = src_row_stride;
  a->num_tokens = num_tokens;
  a->cache = cache;
  return MX_OK;
}

}  // namespace

extern "C" {

int64_t mx_row_bytes(int64_t latent, int32_t group) {
  if (group <= 0 || latent <= 0 || latent % group) return MX_E_SHAPE;
  return latent / 2 + latent / group;
}

int mxfp4_store(const uint16_t* src_bf16, int64_t num_tokens, int64_t latent,
                int64_t src_row_stride, const int64_t* slot_mapping, uint8_t* cache,
                int64_t num_blocks, int64_t block_size, int64_t block_stride_rows,
                int32_t group, void* stream) {
  mxs::StoreArgs a{};
  bool empty = false;
  int rc = check_store(src_bf16, num_tokens, latent, src_row_stride, slot_mapping, cache,
                       num_blocks, block_size, block_stride_rows, group, &a, &empty);
  if (rc) return rc;
  if (empty) return ok();
  a.slots = slot_mapping;
  return launched(mxs::launch_mxfp4_store(a, (int)latent, (hipStream_t)stream), "mxfp4_store");
}

int64_t mxfp4_inverse_bytes(int64_t num_blocks, int64_t block_size) {
  if (num_blocks < 1 || block_size < 1 || num_blocks > (int64_t(0xFFFFFFFF) / block_size))
    return MX_E_RANGE;
  return ((num_blocks * block_size * 4 + 15) / 16) * 16;
}

int mxfp4_slot_order_advised(int64_t num_tokens, int64_t latent, int64_t num_blocks,
                             int64_t block_size) {
  if (latent < 512 || latent > 2048 || !is_pow2(latent)) return 0;
  if (mxfp4_inverse_bytes(num_blocks, block_size) < 0) return 0;
  // The slot order pays for its inverse once a batch covers at least half
  // of the slots and its rows no longer fit in the Infinity Cache (below
  // that the scatter form's plain stores merge partial lines there).
  const int64_t num_slots = num_blocks * block_size;
  const int64_t row = latent / 2 + latent / 32;
  return num_tokens > mxs::kPlainStoreBytes / row && num_tokens <= 0x7FFFFFFF &&
         2 * num_tokens >= num_slots;
}

int mxfp4_build_inverse(const int64_t* slot_mapping, int64_t num_tokens, int64_t num_blocks,
                        int64_t block_size, int32_t* inverse, int64_t inverse_bytes, void* stream) {
  const int64_t need = mxfp4_inverse_bytes(num_blocks, block_size);
  if (need < 0) return fail(MX_E_RANGE, "num_blocks and block_size must be >= 1 with fewer than 2^32 slots");
  if (num_tokens < 0 || num_tokens > 0x7FFFFFFF)
    return fail(MX_E_RANGE, "num_tokens must be in [0, 2^31)");
  if (inverse_bytes < need)
    return fail(MX_E_RANGE, "inverse holds %lld bytes, needs %lld", (long long)inverse_bytes, (long long)need);
  if (!inverse || (num_tokens > 0 && !slot_mapping)) return fail(MX_E_NULL, "null device pointer");
  if (!aligned(inverse, 16)) return fail(MX_E_ALIGN, "inverse must be 16-byte aligned");
  return launched(mxs::launch_build_inverse(slot_mapping, num_tokens,
                                            (uint32_t)(num_blocks * block_size), inverse,
                                            (hipStream_t)stream),
                  "mxfp4_build_inverse");
}

int mxfp4_store_by_slot(const uint16_t* src_bf16, int64_t num_tokens, int64_t latent,
                        int64_t src_row_stride, const int32_t* inverse, int64_t inverse_bytes,
                        uint8_t* cache, int64_t num_blocks, int64_t block_size,
                        int64_t block_stride_rows, int32_t group, void* stream) {
  mxs::StoreArgs a{};
  bool empty = false;
  int rc = check_store(src_bf16, num_tokens, latent, src_row_stride, inverse, cache, num_blocks,
                       block_size, block_stride_rows, group, &a, &empty);
  if (rc) return rc;
  if (latent < 512)
    return fail(MX_E_SHAPE, "the slot-order store needs latent >= 512, got %lld", (long long)latent);
  if (empty) return ok();
  const int64_t need = mxfp4_inverse_bytes(num_blocks, block_size);
  if (inverse_bytes < need)
    return fail(MX_E_RANGE, "inverse holds %lld bytes, %lld slots need %lld",
                (long long)inverse_bytes, (long long)(num_blocks * block_size), (long long)need);
  if (!aligned(inverse, 16)) return fail(MX_E_ALIGN, "inverse must be 16-byte aligned");
  return launched(mxs::launch_mxfp4_store_by_slot(a, (int)latent, inverse, (hipStream_t)stream),
                  "mxfp4_store_by_slot");
}

static_assert(MX_NOALLOC_SCRATCH_BYTES == mxs::kNoAllocScratchBytes,
              "the header's scratch size is the array's");

int mxfp4_store_slot_order_noalloc(const uint16_t* src_bf16, int64_t num_tokens, int64_t latent,
                                   int64_t src_row_stride, const int64_t* slot_mapping,
                                   uint8_t* cache, int64_t num_blocks, int64_t block_size,
                                   int64_t block_stride_rows, int32_t group, void* stream) {
  mxs::StoreArgs a{};
  bool empty = false;
  int rc = check_store(src_bf16, num_tokens, latent, src_row_stride, slot_mapping, cache,
                       num_blocks, block_size, block_stride_rows, group, &a, &empty);
  if (rc) return rc;
  if (latent < 512)
    return fail(MX_E_SHAPE, "the slot-order store needs latent >= 512, got %lld", (long long)latent);
  const int64_t need = mxfp4_inverse_bytes(num_blocks, block_size);
  if (need > MX_NOALLOC_SCRATCH_BYTES)
    return fail(MX_E_RANGE, "%lld slots need a %lld-byte inverse map; the static one holds %lld",
                (long long)(num_blocks * block_size), (long long)need,
                (long long)MX_NOALLOC_SCRATCH_BYTES);
  if (num_tokens > 0x7FFFFFFF) return fail(MX_E_RANGE, "num_tokens must be in [0, 2^31)");
  if (empty) return ok();
  a.slots = slot_mapping;
  return launched(mxs::launch_mxfp4_store_slot_order_noalloc(a, (int)latent, (hipStream_t)stream),
                  "mxfp4_store_slot_order_noalloc");
}

int mxfp4_gather_dequant(const uint8_t* cache, int64_t num_blocks, int64_t block_size,
                         int64_t block_stride_rows, int64_t latent, int32_t group,
                         const int64_t* slots, int64_t num_slots_in_list, uint16_t* out_bf16,
                         int64_t out_row_stride, void* stream) {
  mxs::DequantArgs a{};
  int rc = check_paged(latent, group, num_blocks, block_size, block_stride_rows, &a.map);
  if (rc) return rc;
  if (num_slots_in_list < 0) return fail(MX_E_RANGE, "num_slots_in_list must be >= 0");
  if (out_row_stride < latent)
    return fail(MX_E_STRIDE, "out_row_stride (%lld) is smaller than latent (%lld)",
                (long long)out_row_stride, (long long)latent);
  if (num_slots_in_list == 0) return ok();
  if (!cache || !slots || !out_bf16) return fail(MX_E_NULL, "null device pointer");
  if (!aligned(out_bf16, 16) || out_row_stride % 8)
    return fail(MX_E_ALIGN, "output rows must be 16-byte aligned (base %% 16 == 0, row stride %% 8 == 0)");
  if (!aligned(cache, 4)) return fail(MX_E_ALIGN, "cache must be 4-byte aligned");
  a.cache = cache;
  a.slots = slots;
  a.n = num_slots_in_list;
  a.out = out_bf16;
  a.out_stride = out_row_stride;
  return launched(mxs::launch_mxfp4_dequant(a, (int)latent, (hipStream_t)stream),
                  "mxfp4_gather_dequant");
}

int mxfp8_rope_store(const uint16_t* latent_bf16, const int64_t* positions, const float* cos_sin,
                     int64_t cos_stride, int64_t cos_rows, uint8_t* cache,
                     int64_t cache_block_stride, int64_t cache_block, int64_t num_blocks,
                     const int64_t* slot_mapping, int64_t num_tokens, int32_t compress_ratio,
                     int32_t sanitize_nans, void* stream) {
  mxs::RopeArgs a{};
  int rc = check_rope(latent_bf16, positions, cos_sin, cos_stride, cos_rows, cache,
                      cache_block_stride, cache_block, num_blocks, slot_mapping, num_tokens,
                      compress_ratio, 528, &a);
  if (rc) return rc;
  if (num_tokens == 0) return ok();
  a.sanitize = sanitize_nans ? 1 : 0;
  return launched(mxs::launch_mxfp8_rope(a, (hipStream_t)stream), "mxfp8_rope_store");
}

int nvfp4_rope_store(const uint16_t* latent_bf16, const int64_t* positions, const float* cos_sin,
                     int64_t cos_stride, int64_t cos_rows, uint8_t* cache,
                     int64_t cache_block_stride, int64_t cache_block, int64_t num_blocks,
                     const int64_t* slot_mapping, int64_t num_tokens, int32_t compress_ratio,
                     int32_t sanitize_nans, void* stream) {
  mxs::RopeArgs a{};
  int rc = check_rope(latent_bf16, positions, cos_sin, cos_stride, cos_rows, cache,
                      cache_block_stride, cache_block, num_blocks, slot_mapping, num_tokens,
                      compress_ratio, 288, &a);
  if (rc) return rc;
  if (num_tokens == 0) return ok();
  a.sanitize = sanitize_nans ? 1 : 0;
  return launched(mxs::launch_nvfp4_rope(a, (hipStream_t)stream), "nvfp4_rope_store");
}

int v4_rope_store(const uint16_t* latent_bf16, const int64_t* positions, const float* cos_sin,
                  int64_t cos_stride, int64_t cos_rows, uint8_t* cache,
                  int64_t cache_block_stride, int64_t cache_block, int64_t num_blocks,
                  const int64_t* slot_mapping, int64_t num_tokens, int32_t compress_ratio,
                  int32_t sanitize_nans, void* stream) {
  mxs::RopeArgs a{};
  int rc = check_rope(latent_bf16, positions, cos_sin, cos_stride, cos_rows, cache,
                      cache_block_stride, cache_block, num_blocks, slot_mapping, num_tokens,
                      compress_ratio, 584, &a);
  if (rc) return rc;
  if (num_tokens == 0) return ok();
  a.sanitize = sanitize_nans ? 1 : 0;
  return launched(mxs::launch_v4_rope(a, (hipStream_t)stream), "v4_rope_store");
}

int save_ring_rows(const float* rows, int64_t num_rows, int64_t width, int64_t row_stride,
                   const int64_t* slot_mapping, float* state, int64_t num_blocks, int64_t capacity,
                   int64_t state_stride, int64_t state_row_stride, void* stream) {
  if (num_rows < 0) return fail(MX_E_RANGE, "num_rows must be >= 0");
  if (width < 4 || width % 4 || width > (int64_t(1) << 20))
    return fail(MX_E_SHAPE, "width must be a multiple of 4 in [4, 2^20], got %lld", (long long)width);
  if (num_blocks < 1 || capacity < 1 || num_blocks > (int64_t(0xFFFFFFFF) / capacity))
    return fail(MX_E_RANGE, "num_blocks and capacity must be >= 1 with fewer than 2^32 ring rows");
  if (row_stride < width || state_row_stride < width || state_stride < capacity * state_row_stride)
    return fail(MX_E_STRIDE, "row strides must cover a row and the block stride a whole ring");
  if (row_stride % 4 || state_row_stride % 4 || state_stride % 4)
    return fail(MX_E_ALIGN, "strides must be multiples of 4 elements (16 bytes)");
  if (num_rows == 0) return ok();
  if (!rows || !slot_mapping || !state) return fail(MX_E_NULL, "null device pointer");
  if (!aligned(rows, 16) || !aligned(state, 16))
    return fail(MX_E_ALIGN, "rows and state must be 16-byte aligned");
  mxs::RingArgs a{};
  a.rows = rows;
  a.num_rows = num_rows;
  a.width = width;
  a.row_stride = row_stride;
  a.slots = slot_mapping;
  a.state = state;
  a.num_slots = (uint32_t)(num_blocks * capacity);
  a.capacity = (uint32_t)capacity;
  a.state_stride = state_stride;
  a.state_row_stride = state_row_stride;
  return launched(mxs::launch_ring_rows(a, (hipStream_t)stream), "save_ring_rows");
}

int fused_save_compress_norm_cr1(const float* kv_score, int64_t num_tokens, int64_t width,
                                 int64_t kv_row_stride, const int64_t* slot_mapping,
                                 const uint16_t* rms_norm_weight, float rms_norm_eps, uint16_t* latent_out,
                                 int64_t out_row_stride, void* stream) {
  if (num_tokens < 0 || num_tokens > (int64_t(1) << 33)) return fail(MX_E_RANGE, "num_tokens must be in [0, 2^33]");
  if (width != 512) return fail(MX_E_SHAPE, "width must be 512 at compress ratio 1, got %lld", (long long)width);
  if (!(rms_norm_eps >= 0.0f) || rms_norm_eps > 3.0e38f)
    return fail(MX_E_ARG, "rms_norm_eps must be finite and >= 0");
  if (kv_row_stride < width || out_row_stride < width)
    return fail(MX_E_STRIDE, "row strides must cover a row of 512 values");
  if (kv_row_stride % 4 || out_row_stride % 4)
    return fail(MX_E_ALIGN, "row strides must be multiples of 4 elements");
  if (num_tokens == 0) return ok();
  if (!kv_score || !slot_mapping || !rms_norm_weight || !latent_out) return fail(MX_E_NULL, "null device pointer");
  if (!aligned(kv_score, 16) || !aligned(rms_norm_weight, 8) || !aligned(latent_out, 8))
    return fail(MX_E_ALIGN, "kv_score must be 16-byte and weight / latent_out 8-byte aligned");
  mxs::NormArgs a{};
  a.kv = kv_score;
  a.num_tokens = num_tokens;
  a.kv_row_stride = kv_row_stride;
  a.slots = slot_mapping;
  a.weight = rms_norm_weight;
  a.eps = rms_norm_eps;
  a.out = latent_out;
  a.out_row_stride = out_row_stride;
  return launched(mxs::launch_compress_norm_cr1(a, (hipStream_t)stream), "fused_save_compress_norm_cr1");
}

constexpr int kMaxAttnSplits = 64;

static int attention(const uint16_t* q_bf16, int64_t num_tokens, int64_t num_heads, int64_t latent,
                         int64_t q_token_stride, int64_t q_head_stride, const uint8_t* cache,
                         int64_t num_blocks, int64_t block_size, int64_t block_stride_rows,
                         const int32_t* indices, int64_t topk, int64_t indices_stride, float scale,
                         const float* sink, uint16_t* out_bf16, int64_t out_token_stride,
                         int64_t out_head_stride, int32_t splits, void* workspace, int64_t workspace_bytes,
                         void* stream, const char* name) {
  mxs::AttnArgs a{};
  if (latent != 512) return fail(MX_E_SHAPE, "latent must be 512, got %lld", (long long)latent);
  int rc = check_paged(latent, 32, num_blocks, block_size, block_stride_rows, &a.map);
  if (rc) return rc;
  if (num_blocks * block_size > 0x7FFFFFFF) return fail(MX_E_RANGE, "the cache must hold fewer than 2^31 slots (int32 indices)");
  if (num_tokens < 0 || num_tokens > 0x7FFFFFFF) return fail(MX_E_RANGE, "num_tokens must be in [0, 2^31)");
  if (num_heads < 16 || num_heads > 1024 || num_heads % 16)
    return fail(MX_E_SHAPE, "num_heads must be a multiple of 16 in [16, 1024], got %lld", (long long)num_heads);
  if (topk < 0 || topk > (int64_t(1) << 24)) return fail(MX_E_RANGE, "topk must be in [0, 2^24]");
  if (!(scale == scale) || scale > 3.0e38f || scale < -3.0e38f) return fail(MX_E_ARG, "scale must be finite");
  if (q_head_stride < latent || q_token_stride < num_heads * q_head_stride || out_head_stride < latent ||
      out_token_stride < num_heads * out_head_stride || indices_stride < topk)
    return fail(MX_E_STRIDE, "strides must cover a head row, a token's heads and a token's topk indices");
  if (q_head_stride % 8 || q_token_stride % 8)
    return fail(MX_E_ALIGN, "query strides must be multiples of 8 elements (16-byte rows)");
  if (splits < 1 || splits > kMaxAttnSplits)
    return fail(MX_E_RANGE, "splits must be in [1, %d], got %d", kMaxAttnSplits, splits);
  if (splits > 1) {
    if (num_tokens * num_heads * splits > 0x7FFFFFFF)
      return fail(MX_E_RANGE, "num_tokens * num_heads * splits must stay below 2^31");
    const int64_t need = sparse_mla_attention_workspace_bytes(num_tokens, num_heads, splits);
    if (workspace_bytes < need)
      return fail(MX_E_RANGE, "workspace holds %lld bytes, needs %lld", (long long)workspace_bytes, (long long)need);
  }
  if (num_tokens == 0) return ok();
  if (splits > 1 && !workspace) return fail(MX_E_NULL, "null workspace");
  if (splits > 1 && !aligned(workspace, 16)) return fail(MX_E_ALIGN, "workspace must be 16-byte aligned");
  if (!q_bf16 || !cache || (!indices && topk > 0) || !out_bf16) return fail(MX_E_NULL, "null device pointer");
  if (!aligned(q_bf16, 16) || !aligned(cache, 16) || !aligned(indices, 4) || !aligned(out_bf16, 2) ||
      (sink && !aligned(sink, 4)))
    return fail(MX_E_ALIGN, "q and cache must be 16-byte aligned, indices and sink 4-byte, out 2-byte");
  a.q = q_bf16;
  a.q_token_stride = q_token_stride;
  a.q_head_stride = q_head_stride;
  a.cache = cache;
  {
    const __int128 extent = ((__int128)(num_blocks - 1) * block_stride_rows + block_size) * 272;
    a.cache_bytes = extent <= (__int128)mxs::kAttnBufBytes ? (uint32_t)extent : 0u;
  }
  a.indices = indices;
  a.topk = topk;
  a.idx_stride = indices_stride;
  {
    // The kernel scales scores by a positive c: a negative scale negates q
    // instead (exact), and a zero one (or one that rounds to 0) zeroes it.
    const float c = (float)((double)scale * 1.4426950408889634);
    a.c = c == 0.0f ? 1.0f : fabsf(c);
    a.q_xor = c < 0.0f ? 0x80008000u : 0u;
    a.q_and = c == 0.0f ? 0u : ~0u;
  }
  a.sink = sink;
  a.out = out_bf16;
  a.out_token_stride = out_token_stride;
  a.out_head_stride = out_head_stride;
  a.out_aligned = aligned(out_bf16, 16) && out_token_stride % 8 == 0 && out_head_stride % 8 == 0;
  a.num_heads = (int32_t)num_heads;
  a.num_tokens = num_tokens;
  a.splits = splits;
  a.ws = static_cast<float*>(workspace);
  return launched(mxs::launch_sparse_mla_attn(a, (hipStream_t)stream), name);
}

int sparse_mla_attention(const uint16_t* q_bf16, int64_t num_tokens, int64_t num_heads, int64_t latent,
                         int64_t q_token_stride, int64_t q_head_stride, const uint8_t* cache,
                         int64_t num_blocks, int64_t block_size, int64_t block_stride_rows,
                         const int32_t* indices, int64_t topk, int64_t indices_stride, float scale,
                         const float* sink, uint16_t* out_bf16, int64_t out_token_stride,
                         int64_t out_head_stride, void* stream) {
  return attention(q_bf16, num_tokens, num_heads, latent, q_token_stride, q_head_stride, cache, num_blocks,
                   block_size, block_stride_rows, indices, topk, indices_stride, scale, sink, out_bf16,
                   out_token_stride, out_head_stride, 1, nullptr, 0, stream, "sparse_mla_attention");
}

int64_t sparse_mla_attention_workspace_bytes(int64_t num_tokens, int64_t num_heads, int64_t splits) {
  if (num_tokens < 0 || num_tokens > 0x7FFFFFFF || num_heads < 1 || num_heads > 1024 || splits < 1 ||
      splits > kMaxAttnSplits)
    return MX_E_RANGE;
  if (splits == 1) return 0;
  return ((num_tokens * num_heads * splits * (512 + 2) * 4 + 255) / 256) * 256;
}

int32_t sparse_mla_attention_splits_advised(int64_t num_tokens, int64_t num_heads, int64_t topk) {
  if (num_tokens < 1 || num_heads < 16 || num_heads % 16 || topk < 1) return 1;
  // One workgroup per CU on 256 CUs (measured: at 64 queries 4 ranges beat
  // 8 by 2-4%, at 256 queries one pass beats 2 ranges); each key range keeps
  // at least two 64-key tiles so that its gathers overlap its scores.
  const int64_t blocks = num_tokens * (num_heads / (num_heads % 32 == 0 ? 32 : 16));
  const int64_t tiles = (topk + 63) / 64;
  int64_t s = (256 + blocks - 1) / blocks;
  if (s > tiles / 2) s = tiles / 2;
  if (s > kMaxAttnSplits) s = kMaxAttnSplits;
  return s < 2 ? 1 : (int32_t)s;
}

int sparse_mla_attention_split(const uint16_t* q_bf16, int64_t num_tokens, int64_t num_heads, int64_t latent,
                               int64_t q_token_stride, int64_t q_head_stride, const uint8_t* cache,
                               int64_t num_blocks, int64_t block_size, int64_t block_stride_rows,
                               const int32_t* indices, int64_t topk, int64_t indices_stride, float scale,
                               const float* sink, uint16_t* out_bf16, int64_t out_token_stride,
                               int64_t out_head_stride, int32_t splits, void* workspace,
                               int64_t workspace_bytes, void* stream) {
  return attention(q_bf16, num_tokens, num_heads, latent, q_token_stride, q_head_stride, cache, num_blocks,
                   block_size, block_stride_rows, indices, topk, indices_stride, scale, sink, out_bf16,
                   out_token_stride, out_head_stride, splits, workspace, workspace_bytes, stream,
                   "sparse_mla_attention_split");
}

const char* mx_last_error(void) { return g_err; }

}  // extern "C"
