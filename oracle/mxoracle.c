/*
 * mxoracle.c -- plain, slow, scalar CPU reference for the MXFP4 paged-cache
 * store, its gather-dequant companion and the MXFP8 / NVFP4 RoPE+quant
 * inserts.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the checker the GPU library is
 * compared against.  Only the test suite, the smoke entry point and the CPU
 * baseline leg of the benchmark may load it.  It shares no source, header,
 * table or constant generator with the HIP library, and it imports nothing
 * from it.
 *
 * Sources (web pages; sections named, no line numbers):
 *   [P1] docs page "vllm.v1.attention.ops.mxfp4_mla.store": module docstring
 *        (row = packed data then scales, row_bytes), `_ceil_pow2_exponent`,
 *        `_quantize_e2m1`, `store_mxfp4_mla` (argument meaning, paged view,
 *        pad slots).
 *   [P2] docs page "vllm.models.deepseek_v41.common.ops.
 *        fused_compress_quant_cache": `_rope_quant_insert_mxfp8_kernel`,
 *        `_rope_quant_insert_nvfp4_kernel`, `rope_quant_insert`.
 *   [P3] pull request "[ROCm][Attention] Add an mxfp4_mla KV cache for
 *        rope-free sparse MLA (read/write path)": Overview (272-byte row),
 *        Details (nibble order, round-up exponent), review threads (zero
 *        group scale byte 127, E2M1 midpoints, kv_lora_rank rule).
 *
 * Arithmetic: IEEE binary32 with round-to-nearest-even and gradual underflow
 * wherever the pages compute in fp32 (they convert the latent to fp32 and
 * read the fp32 bit pattern), exact double arithmetic elsewhere.  Build with
 * -O2 -ffp-contract=off and no fast-math so that every operation rounds once
 * and subnormals are kept.
 *
 * Readings where the pages leave a step open are marked "Reading R<n>"; the
 * list is kept in the design notes of the repository.
 *
 * Parity status: every function below is pinned by the CPU tests against
 * exact rational brute force, closed forms or torch's float8 conversion,
 * except where a comment says "parity unpinned".
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_OK 0
#define ORC_EINVAL (-1)

/* ------------------------------------------------------------------ */
/* Scalar helpers                                                      */
/* ------------------------------------------------------------------ */

static float f32_from_bits(uint32_t u) {
  float f;
  memcpy(&f, &u, sizeof f);
  return f;
}

static uint32_t bits_from_f32(float f) {
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  return u;
}

/* bf16 is the top half of an fp32 word, so widening is exact. */
static float bf16_to_f32(uint16_t h) { return f32_from_bits((uint32_t)h << 16); }

/* Row size of one packed MXFP4 token: one nibble per element plus one E8M0
 * byte per group of elements [P1 module docstring; P3 Overview]. */
int64_t orc_row_bytes(int64_t latent, int32_t group) {
  if (latent <= 0 || group <= 0 || latent % group) return ORC_EINVAL;
  return latent / 2 + latent / group;
}

/*
 * Smallest integer e with 2^e >= v, for a positive fp32 v [P1
 * `_ceil_pow2_exponent`].  Written from the definition: frexp gives
 * v = m * 2^k with m in [0.5, 1); v is a power of two exactly when m == 0.5,
 * and then e = k - 1, otherwise e = k.
 *
 * The pages compute this on the fp32 bit pattern, which reads a subnormal v
 * as biased exponent 0 with a nonzero mantissa, i.e. -126.  The exact ceiling
 * would go lower than any E8M0 code can express, so e is floored at -126 to
 * agree with that bit-pattern reading (Reading R3).  +inf is read through the
 * same bit-pattern convention as exponent field 255 with a zero mantissa,
 * i.e. 128 (Reading R11, only reachable from the RoPE variants).
 */
int orc_ceil_pow2_exponent(float v) {
  if (isinf(v)) return 128;
  int k = 0;
  float m = frexpf(v, &k);
  int e = (m == 0.5f) ? k - 1 : k;
  return e < -126 ? -126 : e;
}

/*
 * Round a non-negative magnitude to the nearest point of the E2M1 magnitude
 * grid {0, 0.5, 1, 1.5, 2, 3, 4, 6}, ties to the even grid index [P1
 * `_quantize_e2m1`: the midpoint count with alternating strict and non-strict
 * comparisons is exactly this rule].  At or above 6 the nearest point is 6,
 * index 7 (the midpoint count also stops at 7), +inf included; this is
 * decided before the distance search because a - 0.5 in double is no longer
 * exact once a is about 2^53 or larger, and every distance would then tie.
 * Below 6 the search by distance in double orders the candidates exactly for
 * every fp32 input.
 */
static int e2m1_nearest_index(double a) {
  static const double grid[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
  if (a >= 6.0) return 7;
  int best = 0;
  double best_d = fabs(a - grid[0]);
  for (int i = 1; i < 8; ++i) {
    double d = fabs(a - grid[i]);
    if (d < best_d || (d == best_d && (i % 2 == 0) && (best % 2 == 1))) {
      best = i;
      best_d = d;
    }
  }
  return best;
}

/*
 * 4-bit E2M1 code of an fp32 value already divided by its scale [P1
 * `_quantize_e2m1`].  The sign bit (bit 3) is set exactly when the value
 * compares below zero, so a negative value whose magnitude rounds to zero
 * still gives code 8, while -0.0 (which does not compare below zero) gives 0.
 * NaN gives 0 (Reading R16; unreachable from the MXFP4 store).
 */
int orc_e2m1_code(float q) {
  if (isnan(q)) return 0;
  int idx = e2m1_nearest_index(fabs((double)q));
  return idx | ((q < 0.0f) ? 8 : 0);
}

/* Value of an E2M1 code (sign bit 3, magnitude index in bits 0..2). */
static double e2m1_value(int code) {
  static const double grid[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
  double v = grid[code & 7];
  return (code & 8) ? -v : v;
}

/* OCP E4M3FN value of a byte (bias 7, no infinities, 0x7F/0xFF NaN). */
static double e4m3_value(uint8_t b) {
  int expf = (b >> 3) & 0xF, man = b & 7;
  double v;
  if (expf == 0xF && man == 7) return NAN;
  if (expf == 0)
    v = ldexp((double)man / 8.0, -6);
  else
    v = ldexp(1.0 + (double)man / 8.0, expf - 7);
  return (b & 0x80) ? -v : v;
}

/*
 * fp32 -> OCP E4M3FN byte, round to nearest, ties to the even code
 * (Reading R14).  The magnitude is compared against all 127 finite
 * non-negative codes in ascending order; the sign is copied, so -0.0 and
 * negative values that round to zero give 0x80.  Magnitudes beyond 448
 * saturate to 0x7E (both callers clamp to +-448 first); NaN gives 0x7F.
 */
uint8_t orc_e4m3_encode(float v) {
  if (isnan(v)) return 0x7F;
  uint8_t sign = signbit(v) ? 0x80 : 0x00;
  double a = fabs((double)v);
  if (a >= 448.0) return (uint8_t)(sign | 0x7E);
  int best = 0;
  double best_d = a; /* distance to code 0 (value 0) */
  for (int c = 1; c <= 0x7E; ++c) {
    double d = fabs(a - e4m3_value((uint8_t)c));
    if (d < best_d || (d == best_d && (c % 2 == 0) && (best % 2 == 1))) {
      best = c;
      best_d = d;
    }
  }
  return (uint8_t)(sign | best);
}

double orc_e4m3_value(uint8_t b) { return e4m3_value(b); }

void orc_e4m3_encode_array(const float* v, int64_t n, uint8_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_e4m3_encode(v[i]);
}

/* ------------------------------------------------------------------ */
/* Paged addressing [P1 `store_mxfp4_mla`]                             */
/* ------------------------------------------------------------------ */

/*
 * Row index of a slot in the paged cache: blocks of block_size rows, block b
 * starting block_stride_rows rows after block b-1 (other layers' pages may sit
 * in between).  Returns -1 for a slot that must not be written: negative
 * (PAD_SLOT_ID) or at/after num_blocks * block_size (Reading R7).
 */
static int64_t slot_row(int64_t slot, int64_t num_blocks, int64_t block_size,
                        int64_t block_stride_rows) {
  if (slot < 0 || slot >= num_blocks * block_size) return -1;
  return (slot / block_size) * block_stride_rows + slot % block_size;
}

/* ------------------------------------------------------------------ */
/* MXFP4 store                                                         */
/* ------------------------------------------------------------------ */

/*
 * Quantize one latent row of `latent` bf16 values to a packed MXFP4 row of
 * latent/2 code bytes followed by latent/32 E8M0 scale bytes.
 *
 * Per group of 32 elements, in the order the pages describe:
 *   1. amax = largest |x| over the group, in fp32 (exact from bf16).
 *   2. v = amax / 6 in fp32 (6 is the largest E2M1 magnitude); the scale
 *      exponent e is the smallest integer with 2^e >= v [P1
 *      `_ceil_pow2_exponent`; P3 Details: round-up exponent, so nothing
 *      clamps].  Reading R1: the division is an fp32 divide; every
 *      formulation agrees on bf16 inputs.
 *   3. An all-zero group (amax == 0, either sign) takes e = 0, scale byte
 *      127 [P3 review thread on the zero-group byte] (Reading R2).
 *   4. Scale byte = e + 127 (E8M0 bias).
 *   5. Each element is divided by 2^e in fp32 (one IEEE rounding, which only
 *      matters on underflow; Reading R4) and rounded to its E2M1 code [P1
 *      `_quantize_e2m1`].
 *   6. Codes are packed two per byte, the lower element index in the low
 *      nibble [P3 Details].
 *
 * A group holding a NaN or an infinity gets scale byte 0xFF and zero code
 * bytes (Reading R6: the pages do not say; this is the OCP MX NaN scale).
 */
void orc_mxfp4_quantize_row(const uint16_t* x, int64_t latent, uint8_t* row) {
  const int64_t group = 32;
  const int64_t ngroups = latent / group;
  uint8_t* codes = row;
  uint8_t* scales = row + latent / 2;

  for (int64_t g = 0; g < ngroups; ++g) {
    const uint16_t* xg = x + g * group;
    float amax = 0.0f;
    int nonfinite = 0;
    for (int64_t j = 0; j < group; ++j) {
      float v = bf16_to_f32(xg[j]);
      if (!isfinite(v))
        nonfinite = 1;
      else if (fabsf(v) > amax)
        amax = fabsf(v);
    }

    uint8_t* cg = codes + g * group / 2;
    if (nonfinite) {
      scales[g] = 0xFF;
      for (int64_t j = 0; j < group / 2; ++j) cg[j] = 0;
      continue;
    }

    int e = 0;
    if (amax > 0.0f) e = orc_ceil_pow2_exponent(amax / 6.0f);
    scales[g] = (uint8_t)(e + 127);

    const float scale = ldexpf(1.0f, e); /* e in [-126, 126]: exact normal */
    for (int64_t j = 0; j < group; j += 2) {
      float q0 = bf16_to_f32(xg[j]) / scale;
      float q1 = bf16_to_f32(xg[j + 1]) / scale;
      int c0 = orc_e2m1_code(q0);
      int c1 = orc_e2m1_code(q1);
      cg[j / 2] = (uint8_t)(c0 | (c1 << 4));
    }
  }
}

/*
 * Store num_tokens latent rows into the paged cache [P1 `store_mxfp4_mla`].
 * src is bf16 [num_tokens, latent] with row stride src_row_stride elements
 * and unit inner stride.  Tokens whose slot is negative or out of range
 * write nothing.  Returns 0, or -1 for arguments outside the contract.
 */
int orc_mxfp4_store(const uint16_t* src, int64_t num_tokens, int64_t latent,
                    int64_t src_row_stride, const int64_t* slot_mapping,
                    uint8_t* cache, int64_t num_blocks, int64_t block_size,
                    int64_t block_stride_rows) {
  const int64_t pitch = orc_row_bytes(latent, 32);
  if (pitch <= 0 || num_tokens < 0 || src_row_stride < latent) return ORC_EINVAL;
  if (num_blocks < 1 || block_size < 1 || block_stride_rows < block_size)
    return ORC_EINVAL;
  for (int64_t t = 0; t < num_tokens; ++t) {
    int64_t r = slot_row(slot_mapping[t], num_blocks, block_size, block_stride_rows);
    if (r < 0) continue;
    orc_mxfp4_quantize_row(src + t * src_row_stride, latent, cache + r * pitch);
  }
  return ORC_OK;
}

/* ------------------------------------------------------------------ */
/* MXFP4 gather-dequant                                                */
/* ------------------------------------------------------------------ */

/*
 * bf16 bits of one dequantized element: E2M1 value times 2^(byte - 127)
 * [P3 Details and Claims: the read path unpacks to bf16 and equals the
 * dequantized values], Reading R10.  The product is exact in double; it is
 * representable in bf16 unless it reaches 2^128, where it rounds to
 * infinity.  Scale byte 0xFF is the E8M0 NaN and gives the bf16 quiet NaN
 * 0x7FC0.
 */
uint16_t orc_mxfp4_dequant_bf16(int code, int scale_byte) {
  if (scale_byte == 0xFF) return 0x7FC0;
  double v = ldexp(e2m1_value(code), scale_byte - 127);
  if (fabs(v) >= ldexp(1.0, 128)) return (v < 0) ? 0xFF80 : 0x7F80;
  uint32_t u = bits_from_f32((float)v); /* exact: v has <= 2 significant bits */
  return (uint16_t)(u >> 16);
}

/*
 * Gather `n` slots from the paged cache and dequantize each row to bf16
 * [num, latent] with row stride out_row_stride elements.  A slot that is
 * negative or out of range leaves its output row untouched (Reading R10).
 */
int orc_mxfp4_gather_dequant(const uint8_t* cache, int64_t num_blocks,
                             int64_t block_size, int64_t block_stride_rows,
                             int64_t latent, const int64_t* slots, int64_t n,
                             uint16_t* out, int64_t out_row_stride) {
  const int64_t pitch = orc_row_bytes(latent, 32);
  if (pitch <= 0 || n < 0 || out_row_stride < latent) return ORC_EINVAL;
  if (num_blocks < 1 || block_size < 1 || block_stride_rows < block_size)
    return ORC_EINVAL;
  for (int64_t i = 0; i < n; ++i) {
    int64_t r = slot_row(slots[i], num_blocks, block_size, block_stride_rows);
    if (r < 0) continue;
    const uint8_t* row = cache + r * pitch;
    uint16_t* o = out + i * out_row_stride;
    for (int64_t d = 0; d < latent; ++d) {
      int byte = row[d / 2];
      int code = (d % 2 == 0) ? (byte & 0xF) : (byte >> 4);
      o[d] = orc_mxfp4_dequant_bf16(code, row[latent / 2 + d / 32]);
    }
  }
  return ORC_OK;
}

/*
 * Sparse MLA attention over the MXFP4 cache, the read side of the format [P3:
 * Claims -- attention over the packed cache equals attention over the same
 * values dequantized to bf16; Details, read path -- the ragged sparse kernel
 * unpacks each gathered tile once and feeds both products].  Rope-free MLA
 * in its absorbed form: keys and values are both the cached latent row.  For
 * query token t and head h, over the listed slots j = indices[t, 0..topk)
 * that are valid (>= 0 and inside the cache; others are skipped, as pads are
 * by the store):
 *   s_j = scale * sum_d q[t, h, d] * v_j[d]         (v_j: the row as bf16)
 *   m   = max(max_j s_j, sink[h] when given)
 *   out[t, h, :] = sum_j e^(s_j - m) v_j / (sum_j e^(s_j - m) + e^(sink[h] - m))
 * (the sink term only when sinks are given); no valid slot gives zeros.  A
 * slot listed twice counts twice.  Computed in double from the bf16 query
 * and the bf16 dequantized rows (finite inputs assumed).
 */
int orc_sparse_mla_attention(const uint16_t* q, int64_t num_tokens, int64_t num_heads,
                             int64_t latent, const uint8_t* cache, int64_t num_blocks,
                             int64_t block_size, int64_t block_stride_rows,
                             const int32_t* indices, int64_t topk, double scale,
                             const float* sink, double* out) {
  const int64_t pitch = orc_row_bytes(latent, 32);
  if (pitch <= 0 || num_tokens < 0 || num_heads < 1 || topk < 0) return ORC_EINVAL;
  if (num_blocks < 1 || block_size < 1 || block_stride_rows < block_size) return ORC_EINVAL;
  double* v = (double*)malloc((size_t)(topk > 0 ? topk : 1) * (size_t)latent * sizeof(double));
  double* sc = (double*)malloc((size_t)(topk > 0 ? topk : 1) * sizeof(double));
  int* ok = (int*)malloc((size_t)(topk > 0 ? topk : 1) * sizeof(int));
  if (!v || !sc || !ok) {
    free(v);
    free(sc);
    free(ok);
    return ORC_EINVAL;
  }
  for (int64_t t = 0; t < num_tokens; ++t) {
    for (int64_t j = 0; j < topk; ++j) {
      int64_t r = slot_row((int64_t)indices[t * topk + j], num_blocks, block_size, block_stride_rows);
      ok[j] = r >= 0;
      if (!ok[j]) continue;
      const uint8_t* row = cache + r * pitch;
      for (int64_t d = 0; d < latent; ++d) {
        int byte = row[d / 2];
        int code = (d % 2 == 0) ? (byte & 0xF) : (byte >> 4);
        v[j * latent + d] = (double)bf16_to_f32(orc_mxfp4_dequant_bf16(code, row[latent / 2 + d / 32]));
      }
    }
    for (int64_t h = 0; h < num_heads; ++h) {
      const uint16_t* qh = q + (t * num_heads + h) * latent;
      double* o = out + (t * num_heads + h) * latent;
      double m = -INFINITY;
      int any = 0;
      for (int64_t j = 0; j < topk; ++j) {
        if (!ok[j]) continue;
        double dot = 0.0;
        for (int64_t d = 0; d < latent; ++d) dot += (double)bf16_to_f32(qh[d]) * v[j * latent + d];
        sc[j] = scale * dot;
        if (sc[j] > m) m = sc[j];
        any = 1;
      }
      for (int64_t d = 0; d < latent; ++d) o[d] = 0.0;
      if (!any) continue;
      if (sink && (double)sink[h] > m) m = (double)sink[h];
      double den = sink ? exp((double)sink[h] - m) : 0.0;
      for (int64_t j = 0; j < topk; ++j) {
        if (!ok[j]) continue;
        double w = exp(sc[j] - m);
        den += w;
        for (int64_t d = 0; d < latent; ++d) o[d] += w * v[j * latent + d];
      }
      for (int64_t d = 0; d < latent; ++d) o[d] /= den;
    }
  }
  free(v);
  free(sc);
  free(ok);
  return ORC_OK;
}

/* ------------------------------------------------------------------ */
/* RoPE + quantized insert variants [P2]                               */
/* ------------------------------------------------------------------ */

#define ROPE_LATENT 512
#define ROPE_PAIRS 256
#define ROPE_FIRST_PAIR 224 /* pairs 224..255 are dims 448..511 */

/*
 * Decide whether token t is written, and if so produce its rotated fp32
 * latent [P2 `_rope_quant_insert_mxfp8_kernel` / `_nvfp4_kernel`, shared
 * preamble]:
 *   - skip a negative slot, or one at/after num_blocks * B (Reading R7);
 *   - skip unless (position + 1) is a multiple of the compress ratio;
 *   - the cos/sin row is the first position of the token's compress group,
 *     (position / CR) * CR, with cos in columns 0..31 and sin in 32..63;
 *     a row outside [0, cos_rows) skips the token (our bounds reading);
 *   - GPT-J rotation of the interleaved pairs (2p, 2p+1): for p >= 224 the
 *     table gives (c, s); for the NoPE pairs (c, s) = (1, 0), computed with
 *     the same arithmetic so signed zeros behave as the pages' kernel does;
 *     one rounding per multiply and per add, no fusion (Reading R12);
 *   - with sanitize, NaN becomes +0.
 * Returns 1 when the token is written.
 */
static int rope_token(const uint16_t* latent_row, int64_t position,
                      const float* cos_sin, int64_t cos_stride, int64_t cos_rows,
                      int64_t slot, int64_t num_blocks, int64_t block,
                      int32_t cr, int32_t sanitize, float* r) {
  if (slot < 0 || slot >= num_blocks * block) return 0;
  if ((position + 1) % cr != 0) return 0;
  int64_t base = position / cr * cr;
  if (base < 0 || base >= cos_rows) return 0;
  const float* cs = cos_sin + base * cos_stride;
  for (int p = 0; p < ROPE_PAIRS; ++p) {
    float even = bf16_to_f32(latent_row[2 * p]);
    float odd = bf16_to_f32(latent_row[2 * p + 1]);
    float c = 1.0f, s = 0.0f;
    if (p >= ROPE_FIRST_PAIR) {
      c = cs[p - ROPE_FIRST_PAIR];
      s = cs[32 + p - ROPE_FIRST_PAIR];
    }
    float ec = even * c;
    float os = odd * s;
    float oc = odd * c;
    float es = even * s;
    r[2 * p] = ec - os;
    r[2 * p + 1] = oc + es;
  }
  if (sanitize)
    for (int d = 0; d < ROPE_LATENT; ++d)
      if (isnan(r[d])) r[d] = 0.0f;
  return 1;
}

/*
 * The rotated fp32 latent of each token, as the three inserts below see it
 * (their shared preamble above, with the slot gate left open): out[t, :] is
 * written and written[t] = 1 when the compress-ratio gate and the table row
 * admit token t, else written[t] = 0 and out[t, :] is left as it is.  Exposed
 * so that the rotation itself can be checked value by value.
 */
int orc_rope_rotate(const uint16_t* latent, const int64_t* positions,
                    const float* cos_sin, int64_t cos_stride, int64_t cos_rows,
                    int64_t num_tokens, int32_t cr, int32_t sanitize, float* out,
                    uint8_t* written) {
  if (num_tokens < 0 || cr < 1) return ORC_EINVAL;
  for (int64_t t = 0; t < num_tokens; ++t)
    written[t] = (uint8_t)rope_token(latent + t * ROPE_LATENT, positions[t], cos_sin,
                                     cos_stride, cos_rows, 0, 1, 1, cr, sanitize,
                                     out + t * ROPE_LATENT);
  return ORC_OK;
}

/*
 * MXFP8 record insert [P2 `_rope_quant_insert_mxfp8_kernel`].  Page of B
 * tokens = [B x 512 E4M3 values | B x 16 UE8M0 scales]; page p starts at
 * byte p * cache_block_stride.  Per group of 32 rotated values:
 *   amax = max(max |r|, fl32(1e-4));
 *   E    = smallest integer with 2^E >= fl32(amax * fl32(1/448)) (Reading R11:
 *          the exact ceil of log2 of that fp32 value);
 *   value byte = E4M3(clamp(fl32(r * 2^-E), -448, 448));
 *   scale byte = min(max(E + 127, 0), 254 with sanitize else 255).
 */
int orc_mxfp8_rope_store(const uint16_t* latent, const int64_t* positions,
                         const float* cos_sin, int64_t cos_stride, int64_t cos_rows,
                         uint8_t* cache, int64_t cache_block_stride, int64_t block,
                         int64_t num_blocks, const int64_t* slot_mapping,
                         int64_t num_tokens, int32_t cr, int32_t sanitize) {
  if (num_tokens < 0 || cr < 1 || block < 1 || num_blocks < 1) return ORC_EINVAL;
  if (cache_block_stride < block * 528) return ORC_EINVAL;
  const float floor_amax = 1e-4f;
  const float inv448 = (float)(1.0 / 448.0);
  float r[ROPE_LATENT];
  for (int64_t t = 0; t < num_tokens; ++t) {
    int64_t slot = slot_mapping[t];
    if (!rope_token(latent + t * ROPE_LATENT, positions[t], cos_sin, cos_stride,
                    cos_rows, slot, num_blocks, block, cr, sanitize, r))
      continue;
    uint8_t* page = cache + (slot / block) * cache_block_stride;
    uint8_t* values = page + (slot % block) * 512;
    uint8_t* scales = page + block * 512 + (slot % block) * 16;
    for (int g = 0; g < 16; ++g) {
      float amax = 0.0f;
      for (int j = 0; j < 32; ++j) amax = fmaxf(amax, fabsf(r[32 * g + j]));
      amax = fmaxf(amax, floor_amax);
      float v = amax * inv448;
      int E = orc_ceil_pow2_exponent(v); /* v >= ~2^-22: never floored */
      float mult = ldexpf(1.0f, -E);      /* exact, 2^-128 is a subnormal */
      for (int j = 0; j < 32; ++j) {
        float y = r[32 * g + j] * mult;
        y = fminf(fmaxf(y, -448.0f), 448.0f);
        values[32 * g + j] = orc_e4m3_encode(y);
      }
      int enc = E + 127;
      int max_enc = sanitize ? 254 : 255;
      if (enc < 0) enc = 0;
      if (enc > max_enc) enc = max_enc;
      scales[g] = (uint8_t)enc;
    }
  }
  return ORC_OK;
}

/*
 * NVFP4 record insert [P2 `_rope_quant_insert_nvfp4_kernel`].  Page of B
 * tokens = [B x 256 bytes of E2M1 pairs | B x 32 E4M3 scales].  Per tile of 16
 * rotated values:
 *   S8 = E4M3(clamp(fl32(amax * fl32(1/6)), 2^-9, 448))   (Reading R15)
 *   y  = fl32(r / value(S8))                              (IEEE division)
 *   code(y): nearest E2M1 point, ties to even, saturating at 6, sign bit when
 *   y < 0 (Reading R16); byte i = code(2i) | code(2i+1) << 4.
 */
int orc_nvfp4_rope_store(const uint16_t* latent, const int64_t* positions,
                         const float* cos_sin, int64_t cos_stride, int64_t cos_rows,
                         uint8_t* cache, int64_t cache_block_stride, int64_t block,
                         int64_t num_blocks, const int64_t* slot_mapping,
                         int64_t num_tokens, int32_t cr, int32_t sanitize) {
  if (num_tokens < 0 || cr < 1 || block < 1 || num_blocks < 1) return ORC_EINVAL;
  if (cache_block_stride < block * 288) return ORC_EINVAL;
  const float inv6 = (float)(1.0 / 6.0);
  const float lo_clamp = 0.001953125f; /* 2^-9 */
  float r[ROPE_LATENT];
  for (int64_t t = 0; t < num_tokens; ++t) {
    int64_t slot = slot_mapping[t];
    if (!rope_token(latent + t * ROPE_LATENT, positions[t], cos_sin, cos_stride,
                    cos_rows, slot, num_blocks, block, cr, sanitize, r))
      continue;
    uint8_t* page = cache + (slot / block) * cache_block_stride;
    uint8_t* values = page + (slot % block) * 256;
    uint8_t* scales = page + block * 256 + (slot % block) * 32;
    for (int k = 0; k < 32; ++k) {
      float amax = 0.0f;
      for (int j = 0; j < 16; ++j) amax = fmaxf(amax, fabsf(r[16 * k + j]));
      float sf = amax * inv6;
      sf = fminf(fmaxf(sf, lo_clamp), 448.0f);
      uint8_t s8 = orc_e4m3_encode(sf);
      float S = (float)e4m3_value(s8);
      for (int j = 0; j < 16; j += 2) {
        float y0 = r[16 * k + j] / S;
        float y1 = r[16 * k + j + 1] / S;
        values[(16 * k + j) / 2] =
            (uint8_t)(orc_e2m1_code(y0) | (orc_e2m1_code(y1) << 4));
      }
      scales[k] = s8;
    }
  }
  return ORC_OK;
}

/* ------------------------------------------------------------------ */
/* Ring-state save [P2 `save_ring_rows`]                               */
/* ------------------------------------------------------------------ */

/*
 * Copy fp32 rows of `width` values (the [kv, score] state, 1024 wide on the
 * page) to their ring slots.  A slot s encodes block * capacity + row, row =
 * the position modulo the ring capacity [P2 `fused_save_compress_norm`
 * docstring], so the destination is state + (s / capacity) * state_stride +
 * (s % capacity) * state_row_stride (strides in elements).  Slot -1 (and, by
 * our reading, any negative slot or one past the last ring row) is skipped.
 * The copy is bit-for-bit (NaN payloads included).
 */
int orc_save_ring_rows(const float* rows, int64_t num_rows, int64_t width, int64_t row_stride,
                       const int64_t* slot_mapping, float* state, int64_t num_blocks,
                       int64_t capacity, int64_t state_stride, int64_t state_row_stride) {
  if (num_rows < 0 || width < 1 || row_stride < width || num_blocks < 1 || capacity < 1)
    return ORC_EINVAL;
  if (state_row_stride < width || state_stride < capacity * state_row_stride) return ORC_EINVAL;
  for (int64_t i = 0; i < num_rows; ++i) {
    int64_t s = slot_mapping[i];
    if (s < 0 || s >= num_blocks * capacity) continue;
    float* dst = state + (s / capacity) * state_stride + (s % capacity) * state_row_stride;
    memcpy(dst, rows + i * row_stride, (size_t)width * sizeof(float));
  }
  return ORC_OK;
}

/*
 * fp32 -> bf16, round to nearest, ties to even, by comparing the distances to
 * the two bf16 neighbours of |x| in double (exact).  NaN -> 0x7FC0 (the
 * canonical quiet NaN); +-0 and +-Inf keep their sign.  A magnitude at or
 * above the midpoint between the largest finite bf16 and 2^128 becomes Inf.
 */
uint16_t orc_f32_to_bf16(float x) {
  const uint32_t u = bits_from_f32(x);
  if (isnan(x)) return 0x7FC0;
  const uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
  if (isinf(x) || x == 0.0f) return (uint16_t)(u >> 16);
  const uint32_t mag = u & 0x7FFFFFFFu;
  const uint16_t lo = (uint16_t)(mag >> 16); /* toward zero */
  const uint16_t hi = (uint16_t)(lo + 1);    /* next magnitude up (0x7F80 = Inf) */
  const double a = fabs((double)x);
  const double vlo = (double)bf16_to_f32(lo);
  const double vhi = hi == 0x7F80 ? ldexp(1.0, 128) : (double)bf16_to_f32(hi);
  const double dlo = a - vlo, dhi = vhi - a;
  uint16_t pick;
  if (dlo < dhi) pick = lo;
  else if (dhi < dlo) pick = hi;
  else pick = (lo & 1u) ? hi : lo;
  return (uint16_t)(sign | pick);
}

/*
 * V4 record insert: the 584-byte paged record of DeepSeek-V4 [P2
 * `rope_quant_insert`, its description of the record widths: 576 value bytes
 * followed by eight UE8M0 scale bytes, the last of them zero padding; the V4
 * kernel's body is not printed].  Readings (parity against the pages
 * unpinned beyond the layout): the 576 value bytes are the 448 NoPE dims as
 * E4M3 followed by the 64 rotated RoPE dims as bf16 (448 + 128 = 576); the
 * seven real scales cover the NoPE dims in groups of 64 (448 / 7) and follow
 * the MXFP8 kernel's rule on the same page (amax floored at 1e-4, exact
 * ceil-log2 exponent of fp32(amax / 448), clamp to +-448, byte clamped to
 * [0, 254 or 255]); the gate, RoPE and sanitising are those of the other two
 * inserts; the records are segregated as in the other two:
 *   page = [B x 576 value bytes | B x 8 scale bytes].
 */
int orc_v4_rope_store(const uint16_t* latent, const int64_t* positions,
                      const float* cos_sin, int64_t cos_stride, int64_t cos_rows,
                      uint8_t* cache, int64_t cache_block_stride, int64_t block,
                      int64_t num_blocks, const int64_t* slot_mapping,
                      int64_t num_tokens, int32_t cr, int32_t sanitize) {
  if (num_tokens < 0 || cr < 1 || block < 1 || num_blocks < 1) return ORC_EINVAL;
  if (cache_block_stride < block * 584) return ORC_EINVAL;
  const float floor_amax = 1e-4f;
  const float inv448 = (float)(1.0 / 448.0);
  float r[ROPE_LATENT];
  for (int64_t t = 0; t < num_tokens; ++t) {
    int64_t slot = slot_mapping[t];
    if (!rope_token(latent + t * ROPE_LATENT, positions[t], cos_sin, cos_stride,
                    cos_rows, slot, num_blocks, block, cr, sanitize, r))
      continue;
    uint8_t* page = cache + (slot / block) * cache_block_stride;
    uint8_t* values = page + (slot % block) * 576;
    uint8_t* scales = page + block * 576 + (slot % block) * 8;
    for (int g = 0; g < 7; ++g) {
      float amax = 0.0f;
      for (int j = 0; j < 64; ++j) amax = fmaxf(amax, fabsf(r[64 * g + j]));
      amax = fmaxf(amax, floor_amax);
      int E = orc_ceil_pow2_exponent(amax * inv448);
      float mult = ldexpf(1.0f, -E);
      for (int j = 0; j < 64; ++j) {
        float y = fminf(fmaxf(r[64 * g + j] * mult, -448.0f), 448.0f);
        values[64 * g + j] = orc_e4m3_encode(y);
      }
      int enc = E + 127;
      int max_enc = sanitize ? 254 : 255;
      if (enc < 0) enc = 0;
      if (enc > max_enc) enc = max_enc;
      scales[g] = (uint8_t)enc;
    }
    scales[7] = 0;
    for (int d = 448; d < ROPE_LATENT; ++d) {
      uint16_t h = orc_f32_to_bf16(r[d]);
      values[448 + 2 * (d - 448)] = (uint8_t)(h & 0xFF);
      values[448 + 2 * (d - 448) + 1] = (uint8_t)(h >> 8);
    }
  }
  return ORC_OK;
}

/* ------------------------------------------------------------------ */
/* Compress-ratio-1 normalisation [P2 `fused_save_compress_norm`]      */
/* ------------------------------------------------------------------ */

/*
 * With compress ratio 1 each token is a group of its own: there is no ring
 * state and nothing to pool, and the slot mapping serves only to say which
 * tokens are valid (a negative slot: not written) [P2
 * `fused_save_compress_norm`, its description and parameter list].  The
 * step is then an RMSNorm of the token's fp32 row (`width` values, 512 on
 * the page) with a bf16 weight:
 *   y[d] = x[d] / sqrt(mean(x^2) + eps) * w[d].
 * Computed here in double (the pages do not fix the reduction order), so the
 * result is the exact value up to double rounding; out[t] is written only
 * for slot_mapping[t] >= 0.  Parity against the GPU is a tolerance derived
 * from fp32 arithmetic and the final bf16 rounding.
 */
int orc_rmsnorm_cr1(const float* kv, int64_t num_tokens, int64_t width, int64_t row_stride,
                    const int64_t* slot_mapping, const uint16_t* weight_bf16, float eps,
                    double* out, int64_t out_row_stride) {
  if (num_tokens < 0 || width < 1 || row_stride < width || out_row_stride < width) return ORC_EINVAL;
  for (int64_t t = 0; t < num_tokens; ++t) {
    if (slot_mapping[t] < 0) continue;
    const float* x = kv + t * row_stride;
    double ss = 0.0;
    for (int64_t d = 0; d < width; ++d) ss += (double)x[d] * (double)x[d];
    const double r = 1.0 / sqrt(ss / (double)width + (double)eps);
    double* y = out + t * out_row_stride;
    for (int64_t d = 0; d < width; ++d) y[d] = (double)x[d] * r * (double)bf16_to_f32(weight_bf16[d]);
  }
  return ORC_OK;
}
