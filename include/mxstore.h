/*
 * mxstore.h -- C ABI of libmxstore.so: MXFP4 quantize-and-scatter store of
 * an MLA latent into a paged KV cache, its gather-dequant companion, and the
 * MXFP8 / NVFP4 RoPE+quant record inserts, as hand-written HIP kernels for
 * gfx950 (MI355X).
 *
 * Sources (web pages; sections named):
 *   [P1] docs page "vllm.v1.attention.ops.mxfp4_mla.store"
 *   [P2] docs page "vllm.models.deepseek_v41.common.ops.fused_compress_quant_cache"
 *   [P3] pull request "[ROCm][Attention] Add an mxfp4_mla KV cache for
 *        rope-free sparse MLA (read/write path)"
 *
 * Conventions shared by every entry point
 *   - Every data pointer is a DEVICE pointer owned by the caller; the library
 *     never allocates, frees or synchronises.  Work is enqueued on `stream`
 *     (a hipStream_t passed as void*; NULL is the default stream) and runs
 *     asynchronously: the caller keeps every buffer alive until the stream
 *     has passed the call.
 *   - bf16 data is passed as its raw 16-bit patterns (uint16_t).
 *   - Return value: MX_OK, or a negative MX_E_* code when an argument breaks
 *     the contract stated below; nothing is launched then, and
 *     mx_last_error() describes the first violated rule.  Data errors on the
 *     device are never reported: a slot that is negative (PAD_SLOT_ID) or
 *     past the last slot is skipped.
 *   - num_tokens == 0 (or an empty slot list) launches nothing and returns
 *     MX_OK [P1 `store_mxfp4_mla`; P2 `rope_quant_insert`].
 *   - Two tokens mapping to the same slot race: the row's contents are then
 *     unspecified and may mix bytes of both tokens.
 */
#ifndef MXSTORE_H
#define MXSTORE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MX_OK 0
#define MX_E_NULL (-1)   /* a required pointer is NULL                       */
#define MX_E_SHAPE (-2)  /* latent / group / record width not supported      */
#define MX_E_STRIDE (-3) /* a stride is inconsistent with the layout         */
#define MX_E_ALIGN (-4)  /* a pointer or stride breaks the alignment rule    */
#define MX_E_RANGE (-5)  /* a count is negative or too large                 */
#define MX_E_ARG (-6)    /* another argument is invalid (compress ratio ...) */
#define MX_E_LAUNCH (-7) /* the HIP launch itself failed                     */

/*
 * Bytes of one packed MXFP4 row: latent/2 code bytes + latent/group E8M0
 * scale bytes [P1 module docstring `row_bytes`; P3 Overview: 272 for 512].
 * Returns a negative MX_E_SHAPE when latent is not a positive multiple of
 * group (group > 0).  Host-only, no device work.
 */
int64_t mx_row_bytes(int64_t latent, int32_t group);

/*
 * MXFP4 store [P1 `store_mxfp4_mla` and its helpers `_ceil_pow2_exponent`,
 * `_quantize_e2m1`; P3 Details].  For each token t < num_tokens with slot
 * s = slot_mapping[t] in [0, num_blocks * block_size):
 *   per group of 32 latent values: amax in fp32; scale exponent e = smallest
 *   integer with 2^e >= amax/6 (bit-pattern reading: floored at -126); an
 *   all-zero group uses e = 0; a group holding NaN/Inf writes scale 0xFF and
 *   zero codes; every value is divided by 2^e in fp32 and rounded to the
 *   nearest E2M1 code (ties to even), sign bit set when the quotient is
 *   below zero.
 *   Row = [latent/2 code bytes (element 2i in the low nibble of byte i) |
 *   latent/32 scale bytes (e + 127)], written at byte offset
 *   ((s / block_size) * block_stride_rows + s % block_size) * row_bytes.
 *
 * src_bf16        [num_tokens, latent] bf16, row stride src_row_stride
 *                 elements (>= latent), unit inner stride.  The base address
 *                 must be 16-byte aligned and src_row_stride a multiple of 8.
 * slot_mapping    int64 [num_tokens].
 * cache           uint8, 4-byte aligned, holding at least
 *                 ((num_blocks-1) * block_stride_rows + block_size) rows of
 *                 row_bytes bytes.  A flat cache is num_blocks = 1,
 *                 block_size = block_stride_rows = number of slots.
 * latent          power of two in [128, 2048]; group must be 32 [P3 review:
 *                 kv_lora_rank is a power of two >= 128; OCP block 32].
 * block_stride_rows >= block_size; num_blocks * block_size < 2^32.
 */
int mxfp4_store(const uint16_t* src_bf16, int64_t num_tokens, int64_t latent,
                int64_t src_row_stride, const int64_t* slot_mapping,
                uint8_t* cache, int64_t num_blocks, int64_t block_size,
                int64_t block_stride_rows, int32_t group, void* stream);

/*
 * Slot-order form of the MXFP4 store, in two calls.  For a batch that fills
 * most of the cache's slots in scattered order (e.g. a random permutation),
 * scattered 272-byte row writes are what limits mxfp4_store: DRAM serves
 * scattered 1 KiB reads at nearly full speed but scattered sub-line writes at
 * well under half.  The slot-order form inverts the scatter: an inverse map
 * inverse[s] = token of slot s (or -1) is built once per slot mapping -- it
 * serves every layer that stores with that mapping in the step -- and the
 * store then walks the slots in order, gathers each slot's latent row and
 * writes the rows sequentially.  For distinct slots it writes exactly the
 * bytes mxfp4_store writes.  A slot named by several tokens is a race in
 * both forms: the slot-order form writes the whole row of the token whose
 * inverse entry won, while the scatter form may leave a row that mixes one
 * token's code bytes with another's scale bytes.
 */

/* Bytes of the inverse map: one int32 per slot (num_blocks * block_size),
 * rounded up to 16.  MX_E_RANGE if num_blocks or block_size < 1 or the slot
 * count reaches 2^32.  Host-only. */
int64_t mxfp4_inverse_bytes(int64_t num_blocks, int64_t block_size);

/* 1 when the slot-order form is expected to beat mxfp4_store for this shape:
 * latent in {512, 1024, 2048}, num_tokens < 2^31, num_tokens >= half the
 * slots, and the batch's rows (num_tokens * row bytes) exceed 256 MiB, the
 * size of MI355X's Infinity Cache (smaller batches merge their scattered
 * rows there); else 0.  Host-only heuristic (measured on MI355X), no device
 * work. */
int mxfp4_slot_order_advised(int64_t num_tokens, int64_t latent,
                             int64_t num_blocks, int64_t block_size);

/*
 * Build the inverse map of a slot mapping: inverse[s] = -1 for every slot,
 * then inverse[slot_mapping[t]] = t for every t < num_tokens whose slot is in
 * [0, num_blocks * block_size).  inverse: device int32 buffer of at least
 * mxfp4_inverse_bytes(num_blocks, block_size) bytes, 16-byte aligned,
 * overwritten.  num_tokens < 2^31.  Two launches on `stream`.
 */
int mxfp4_build_inverse(const int64_t* slot_mapping, int64_t num_tokens,
                        int64_t num_blocks, int64_t block_size, int32_t* inverse,
                        int64_t inverse_bytes, void* stream);

/*
 * MXFP4 store in slot order: same arguments and result as mxfp4_store, with
 * the slot mapping replaced by its inverse map (built by mxfp4_build_inverse
 * for the same num_blocks and block_size; entries outside [0, num_tokens) are
 * skipped).  latent must be 512, 1024 or 2048; inverse 16-byte aligned and
 * inverse_bytes (its size) at least mxfp4_inverse_bytes(num_blocks,
 * block_size), else MX_E_RANGE.  The library cannot tell whether the inverse
 * belongs to the slot mapping of this batch: a map built from another
 * mapping writes the rows its own entries name, and the call still returns
 * MX_OK.  Rebuild it whenever the mapping changes.  One launch over all
 * num_blocks * block_size slots, so it is meant for batches that cover a
 * large share of them (mxfp4_slot_order_advised).
 */
int mxfp4_store_by_slot(const uint16_t* src_bf16, int64_t num_tokens, int64_t latent,
                        int64_t src_row_stride, const int32_t* inverse, int64_t inverse_bytes,
                        uint8_t* cache, int64_t num_blocks, int64_t block_size,
                        int64_t block_stride_rows, int32_t group, void* stream);

/*
 * Allocation-free slot-order store, for callers that cannot allocate device
 * memory or pass a workspace (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation).  Same arguments, checks and
 * result as mxfp4_store (and as mxfp4_build_inverse + mxfp4_store_by_slot on
 * the same mapping): it builds the inverse map in a static device array of
 * MX_NOALLOC_SCRATCH_BYTES that the library holds on each GPU it runs on
 * until the process ends, then stores in slot order.  Three launches on
 * `stream`, no allocation, no workspace argument.
 *   - The array of the CURRENT device is used (looked up on the first call
 *     there); `stream` must belong to that device.
 *   - num_blocks * block_size slots need mxfp4_inverse_bytes(num_blocks,
 *     block_size) <= MX_NOALLOC_SCRATCH_BYTES (8,388,608 slots), else
 *     MX_E_RANGE with nothing launched.  latent 512, 1024 or 2048;
 *     num_tokens < 2^31.
 *   - Every call on a GPU shares that GPU's array, and the map is rebuilt by
 *     each call: calls that overlap on one GPU (on different streams without
 *     ordering between them) race and may write wrong rows.
 */
#define MX_NOALLOC_SCRATCH_BYTES ((int64_t)32 << 20)
int mxfp4_store_slot_order_noalloc(const uint16_t* src_bf16, int64_t num_tokens, int64_t latent,
                                   int64_t src_row_stride, const int64_t* slot_mapping,
                                   uint8_t* cache, int64_t num_blocks, int64_t block_size,
                                   int64_t block_stride_rows, int32_t group, void* stream);

/*
 * MXFP4 gather-dequant [P3 Details, read path: unpack to bf16; Claims: the
 * result equals the dequantized values stored as bf16].  For each i <
 * num_slots_in_list with slot s = slots[i] in range, writes
 * out[i, d] = bf16(E2M1(code_d) * 2^(scale_byte - 127)) for d < latent:
 * exact, except that a product >= 2^128 gives +-Inf and scale byte 0xFF gives
 * the quiet NaN 0x7FC0.  A slot out of range leaves row i of out untouched.
 *
 * cache           same layout and arguments as mxfp4_store (read only).
 * slots           int64 [num_slots_in_list].
 * out_bf16        [num_slots_in_list, latent] bf16, row stride
 *                 out_row_stride elements (>= latent, multiple of 8),
 *                 16-byte aligned base.
 */
int mxfp4_gather_dequant(const uint8_t* cache, int64_t num_blocks,
                         int64_t block_size, int64_t block_stride_rows,
                         int64_t latent, int32_t group, const int64_t* slots,
                         int64_t num_slots_in_list, uint16_t* out_bf16,
                         int64_t out_row_stride, void* stream);

/*
 * MXFP8 RoPE+quant insert, 528-byte record [P2
 * `_rope_quant_insert_mxfp8_kernel`, `rope_quant_insert`].  Token t is
 * written when s = slot_mapping[t] is in [0, num_blocks * cache_block) and
 * (positions[t] + 1) % compress_ratio == 0.  Its 512 bf16 values are rotated
 * GPT-J style on pairs (448+2i, 449+2i), i < 32, with cos/sin row
 * r = (positions[t] / compress_ratio) * compress_ratio of cos_sin (cos in
 * columns 0..31, sin in 32..63; a row outside [0, cos_rows) skips the
 * token); with sanitize_nans, NaN becomes +0.  Per group of 32:
 * amax = max(max|r|, 1e-4f); E = ceil(log2(fp32(amax * (1/448)))) taken
 * exactly; values = E4M3(clamp(r * 2^-E, +-448)); scale = clamp(E + 127, 0,
 * sanitize ? 254 : 255).  Page layout (page = s / cache_block, base
 * cache + page * cache_block_stride):
 *   [cache_block x 512 value bytes | cache_block x 16 scale bytes].
 *
 * latent_bf16     [>= num_tokens, 512] bf16, contiguous, 16-byte aligned.
 * positions       int64 [num_tokens].
 * cos_sin         fp32 [cos_rows, cos_stride >= 64] table.
 * cache           uint8, 16-byte aligned; cache_block_stride (bytes) is a
 *                 multiple of 16 and >= cache_block * 528.
 * compress_ratio  >= 1 (the pages' wrapper allows 1 or 2; the kernel math
 *                 holds for any ratio).
 */
int mxfp8_rope_store(const uint16_t* latent_bf16, const int64_t* positions,
                     const float* cos_sin, int64_t cos_stride, int64_t cos_rows,
                     uint8_t* cache, int64_t cache_block_stride,
                     int64_t cache_block, int64_t num_blocks,
                     const int64_t* slot_mapping, int64_t num_tokens,
                     int32_t compress_ratio, int32_t sanitize_nans,
                     void* stream);

/*
 * NVFP4 RoPE+quant insert, 288-byte record [P2
 * `_rope_quant_insert_nvfp4_kernel`, `rope_quant_insert`].  Same gate,
 * rotation and sanitising as mxfp8_rope_store.  Per tile of 16:
 * S8 = E4M3(clamp(fp32(amax * (1/6)), 2^-9, 448)); y = fp32(r / S8) with a
 * correctly rounded division; code = nearest E2M1 (ties to even, |y| > 6
 * saturates to 6, sign bit when y < 0); byte i = code(2i) | code(2i+1) << 4.
 * Page layout: [cache_block x 256 value bytes | cache_block x 32 scale bytes].
 * cache_block_stride (bytes) is a multiple of 16 and >= cache_block * 288.
 */
int nvfp4_rope_store(const uint16_t* latent_bf16, const int64_t* positions,
                     const float* cos_sin, int64_t cos_stride, int64_t cos_rows,
                     uint8_t* cache, int64_t cache_block_stride,
                     int64_t cache_block, int64_t num_blocks,
                     const int64_t* slot_mapping, int64_t num_tokens,
                     int32_t compress_ratio, int32_t sanitize_nans,
                     void* stream);

/*
 * V4 RoPE+quant insert, 584-byte record [P2 `rope_quant_insert`: the V4
 * record is 576 value bytes and eight UE8M0 scale bytes, one of them zero
 * padding; the kernel body is not printed].  Same gate, rotation and
 * sanitising as mxfp8_rope_store.  Reading of the record: the 448 NoPE
 * values as E4M3 in 7 groups of 64 under the MXFP8 scale rule, then the 64
 * rotated RoPE values as bf16 (nearest-even, little-endian; NaN, possible
 * only without sanitising, as 0x7FC0).  Page layout:
 *   [cache_block x 576 value bytes | cache_block x 8 scale bytes],
 * scale bytes 0..6 for the groups, byte 7 = 0.  cache_block_stride (bytes) is
 * a multiple of 16 and >= cache_block * 584.
 */
int v4_rope_store(const uint16_t* latent_bf16, const int64_t* positions,
                  const float* cos_sin, int64_t cos_stride, int64_t cos_rows,
                  uint8_t* cache, int64_t cache_block_stride,
                  int64_t cache_block, int64_t num_blocks,
                  const int64_t* slot_mapping, int64_t num_tokens,
                  int32_t compress_ratio, int32_t sanitize_nans,
                  void* stream);

/*
 * Ring-state save [P2 `save_ring_rows`; ring rule from the
 * `fused_save_compress_norm` docstring]: for each i < num_rows with
 * s = slot_mapping[i] in [0, num_blocks * capacity), copy the fp32 row
 * rows[i, 0:width] bit for bit to
 *   state + (s / capacity) * state_stride + (s % capacity) * state_row_stride
 * (all strides in elements).  Slot -1 -- and any other negative slot or one
 * past the last ring row -- is skipped.  The pages' rows are the [kv, score]
 * states, width 1024.
 *
 * rows            fp32 [num_rows, width], row stride row_stride >= width.
 * state           fp32 ring [num_blocks, capacity, width]-shaped view with
 *                 state_row_stride >= width, state_stride >= capacity *
 *                 state_row_stride.
 * width           multiple of 4 in [4, 2^20]; rows and state 16-byte aligned
 *                 and every stride a multiple of 4 elements.
 */
int save_ring_rows(const float* rows, int64_t num_rows, int64_t width, int64_t row_stride,
                   const int64_t* slot_mapping, float* state, int64_t num_blocks,
                   int64_t capacity, int64_t state_stride, int64_t state_row_stride,
                   void* stream);

/*
 * Compress-ratio-1 case of the save/compress/norm step [P2
 * `fused_save_compress_norm`: ratio 1 keeps no ring and the slot mapping
 * only marks valid tokens; weight bf16 [512], output bf16 [tokens, 512]
 * written only where valid].  For each t < num_tokens with
 * slot_mapping[t] >= 0:
 *   r = 1 / sqrt(sum_d kv[t, d]^2 / 512 + rms_norm_eps)
 *   latent_out[t, d] = bf16_rn((kv[t, d] * r) * w[d])
 * in fp32 with correctly rounded sqrt and division; the order of the sum is
 * the kernel's own (the pages do not fix it).  Rows of other tokens are not
 * written.
 *
 * kv_score         fp32 [num_tokens, 512], row stride kv_row_stride >= 512,
 *                  a multiple of 4; 16-byte aligned.
 * width            must be 512.
 * rms_norm_weight  bf16 [512], 8-byte aligned.
 * rms_norm_eps     finite, >= 0.
 * latent_out       bf16 [num_tokens, 512], row stride out_row_stride >= 512,
 *                  a multiple of 4; 8-byte aligned.
 * num_tokens       [0, 2^33]; 0 is a no-op.
 */
int fused_save_compress_norm_cr1(const float* kv_score, int64_t num_tokens, int64_t width,
                                 int64_t kv_row_stride, const int64_t* slot_mapping,
                                 const uint16_t* rms_norm_weight, float rms_norm_eps,
                                 uint16_t* latent_out, int64_t out_row_stride, void* stream);

/*
 * Sparse MLA attention over the MXFP4 cache -- the read side of the format
 * [P3: Claims -- attention over the packed cache equals attention over the
 * same values dequantized to bf16; Details, read path -- the ragged sparse
 * kernel unpacks each gathered tile once and feeds both products].  Rope-free
 * MLA in absorbed form: keys and values are both the cached 512-wide latent.
 * For each query token t and head h, over the listed slots
 * s = indices[t * indices_stride + j], j < topk, that are valid (0 <= s <
 * num_blocks * block_size; others are skipped):
 *   score_j = scale * dot(q[t, h, :], v_s)            (v_s: the row as bf16)
 *   out[t, h, :] = sum_j e^(score_j - m) v_s / (sum_j e^(score_j - m)
 *                                                + e^(sink[h] - m))
 * with m the running maximum and the sink term only when `sink` is given
 * (natural-log logits, one per head).  A token with no valid slot gets zeros.
 * Scores accumulate in fp32 on bf16 MFMAs; the softmax runs in base 2 in
 * fp32; the weights are rounded to bf16 for the weighted sum (fp32
 * accumulate); the result is rounded to bf16.
 *
 * q_bf16        bf16 [num_tokens, num_heads, 512]; strides in elements,
 *               multiples of 8; 16-byte aligned.
 * cache         the paged MXFP4 cache as for mxfp4_store (latent 512, 272-byte
 *               rows, fewer than 2^31 slots); 16-byte aligned.
 * indices       int32 [num_tokens, indices_stride >= topk]; may be null when
 *               topk is 0 (every output is then zero).
 * num_heads     a multiple of 16 in [16, 1024].
 * scale         finite softmax scale (e.g. 1/sqrt(qk head dim)).
 * out_bf16      bf16 [num_tokens, num_heads, 512]; strides in elements.
 */
int sparse_mla_attention(const uint16_t* q_bf16, int64_t num_tokens, int64_t num_heads,
                         int64_t latent, int64_t q_token_stride, int64_t q_head_stride,
                         const uint8_t* cache, int64_t num_blocks, int64_t block_size,
                         int64_t block_stride_rows, const int32_t* indices, int64_t topk,
                         int64_t indices_stride, float scale, const float* sink,
                         uint16_t* out_bf16, int64_t out_token_stride, int64_t out_head_stride,
                         void* stream);

/*
 * Split-key form of sparse_mla_attention for few query tokens (decode), where
 * one workgroup per (token, head block) leaves most of the GPU idle [P3
 * Details, follow-ups: split-K decode over the mxfp4_mla cache -- named, not
 * described; the merge below is the usual log-sum-exp combination, so the
 * result is the same attention].  Each (token, head block) is walked by
 * `splits` workgroups over consecutive ranges of whole 64-key tiles; each
 * writes its unnormalised output, running maximum and weight sum to
 * `workspace`, and a second launch merges them (sink folded in there) and
 * rounds to bf16.  Same arguments and result as sparse_mla_attention (up to
 * fp32 rounding order), plus:
 * splits           1 .. 64 (1: exactly sparse_mla_attention, no workspace).
 * workspace        device buffer of >= sparse_mla_attention_workspace_bytes
 *                  bytes, 16-byte aligned, overwritten; owned by the caller.
 * Two launches on `stream` (one when splits is 1).
 */
int sparse_mla_attention_split(const uint16_t* q_bf16, int64_t num_tokens, int64_t num_heads,
                               int64_t latent, int64_t q_token_stride, int64_t q_head_stride,
                               const uint8_t* cache, int64_t num_blocks, int64_t block_size,
                               int64_t block_stride_rows, const int32_t* indices, int64_t topk,
                               int64_t indices_stride, float scale, const float* sink,
                               uint16_t* out_bf16, int64_t out_token_stride,
                               int64_t out_head_stride, int32_t splits, void* workspace,
                               int64_t workspace_bytes, void* stream);

/* Workspace bytes of sparse_mla_attention_split: num_tokens * num_heads *
 * splits * 514 fp32 values, rounded up to 256 (0 for splits == 1).
 * MX_E_RANGE for counts out of range.  Host-only. */
int64_t sparse_mla_attention_workspace_bytes(int64_t num_tokens, int64_t num_heads,
                                             int64_t splits);

/* Split count expected to be fastest on MI355X: enough workgroups for one per
 * CU on 256 CUs, at least two 64-key tiles per split, at most 64; 1 when
 * the batch already fills the GPU.  Host-only heuristic, no device work. */
int32_t sparse_mla_attention_splits_advised(int64_t num_tokens, int64_t num_heads, int64_t topk);

/* Message for the last nonzero status returned on this thread ("" if none).
 * The pointer stays valid until the next call on the same thread. */
const char* mx_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MXSTORE_H */
