"""The pins are discriminating: each plausible mistake planted in a copy of
the oracle's C source (on the CPU, in a temporary directory) makes at least
one pin of tests/test_oracle_pins.py fail.  The real oracle is untouched."""

import pytest

import oracle
from tests import test_oracle_pins as pins

# (pin, keyword arguments), cheapest first; a mutant stops at its first failure.
CHECKS = [
    (pins.test_format_constants, {}),
    (pins.test_negative_zero_small_negatives_and_nibble_order, {}),
    (pins.test_all_zero_groups_and_nonfinite, {}),
    (pins.test_powers_of_two, {"j": 0}),
    (pins.test_powers_of_two, {"j": -124}),
    (pins.test_powers_of_two, {"j": 126}),
    (pins.test_ties_to_even, {"k": 0}),
    (pins.test_paged_addressing_pads_and_canaries, {}),
    (pins.test_strided_source_rows, {}),
    (pins.test_dequant_table_exhaustive, {}),
    (pins.test_dequant_skips_bad_slots, {}),
    (pins.test_e2m1_saturates_for_huge_quotients, {}),
    (pins.test_mxfp8_zero_group_byte_105, {}),
    (pins.test_mxfp8_exponent_just_above_powers_of_two, {}),
    (pins.test_rope_nan_sanitised, {}),
    (pins.test_save_ring_rows_placement, {}),
    (pins.test_rmsnorm_cr1_closed_forms, {}),
    (pins.test_f32_to_bf16_matches_torch, {}),
    (pins.test_v4_record_values_scales_and_pad, {}),
    (pins.test_attention_single_key_pads_and_sink, {}),
    (pins.test_attention_uniform_when_query_is_zero, {}),
    (pins.test_attention_temperature, {}),
    (pins.test_attention_hard_limit_and_order, {}),
    (pins.test_rope_gate_and_canaries, {}),
    (pins.test_rope_exact_angles_pin_pairing_and_row, {}),
    (pins.test_rope_strided_table_and_pages, {}),
    (pins.test_rope_rotation_general_angles_against_numpy, {}),
    (pins.test_rope_inserts_at_general_angles, {}),
    (pins.test_nvfp4_huge_tiles_saturate, {}),
    (pins.test_e4m3_encode_matches_torch, {}),
    (pins.test_nvfp4_scales_and_codes, {}),
    (pins.test_round_trip_within_half_gap, {}),
    (pins.test_invariants_on_random_rows, {}),
    (pins.test_anchored_sweep, {"k": 0}),
    (pins.test_anchored_sweep, {"k": 125}),
    (pins.test_anchored_sweep, {"k": -126}),
    (pins.test_mxfp8_exponent_exhaustive_and_values, {}),
    (lambda orc: pins.test_solo_codes_exhaustive(pins.make_solo_sweep(orc), orc=orc), {}),
    (lambda orc: pins.test_scale_exponent_exhaustive(pins.make_solo_sweep(orc), orc=orc), {}),
]

# name -> (text in mxoracle.c, replacement)
MUTANTS = {
    "exponent via ceil(log2)": (
        "int e = (m == 0.5f) ? k - 1 : k;", "int e = (int)ceilf(log2f(v)); (void)m;"),
    "no -126 floor": ("return e < -126 ? -126 : e;", "return e;"),
    "E2M1 ties away from zero": (
        "if (d < best_d || (d == best_d && (i % 2 == 0) && (best % 2 == 1))) {\n      best = i;\n      best_d = d;\n    }\n  }\n  return best;\n}\n\n/*\n * 4-bit",
        "if (d <= best_d) {\n      best = i;\n      best_d = d;\n    }\n  }\n  return best;\n}\n\n/*\n * 4-bit"),
    "sign bit from signbit()": ("return idx | ((q < 0.0f) ? 8 : 0);", "return idx | (signbit(q) ? 8 : 0);"),
    "nibbles swapped": ("cg[j / 2] = (uint8_t)(c0 | (c1 << 4));", "cg[j / 2] = (uint8_t)(c1 | (c0 << 4));"),
    "zero group scale byte 0": ("scales[g] = (uint8_t)(e + 127);", "scales[g] = (uint8_t)(amax > 0.0f ? e + 127 : 0);"),
    "scale one step too small": ("const float scale = ldexpf(1.0f, e);", "const float scale = ldexpf(1.0f, e - 1);"),
    "block stride ignored": (
        "return (slot / block_size) * block_stride_rows + slot % block_size;",
        "return (slot / block_size) * block_size + slot % block_size;"),
    "dequant bias 128": ("ldexp(e2m1_value(code), scale_byte - 127)", "ldexp(e2m1_value(code), scale_byte - 128)"),
    "E4M3 ties away from zero": (
        "if (d < best_d || (d == best_d && (c % 2 == 0) && (best % 2 == 1))) {",
        "if (d <= best_d) {"),
    "MXFP8 amax floor dropped": ("amax = fmaxf(amax, floor_amax);", "(void)floor_amax;"),
    "MXFP8 exponent of amax, not amax/448": ("float v = amax * inv448;", "float v = amax; (void)inv448;"),
    "RoPE row = position": ("int64_t base = position / cr * cr;", "int64_t base = position;"),
    "RoPE gate off by one": ("if ((position + 1) % cr != 0) return 0;", "if (position % cr != 0) return 0;"),
    "RoPE cos/sin swapped": (
        "c = cs[p - ROPE_FIRST_PAIR];\n      s = cs[32 + p - ROPE_FIRST_PAIR];",
        "s = cs[p - ROPE_FIRST_PAIR];\n      c = cs[32 + p - ROPE_FIRST_PAIR];"),
    "RoPE rotation sign": ("r[2 * p] = ec - os;", "r[2 * p] = ec + os;"),
    "RoPE rotation fused (fmaf)": ("r[2 * p] = ec - os;", "r[2 * p] = fmaf(even, c, -os); (void)ec;"),
    "RoPE rotation in double": (
        "r[2 * p] = ec - os;\n    r[2 * p + 1] = oc + es;",
        "r[2 * p] = (float)((double)even * c - (double)odd * s);\n"
        "    r[2 * p + 1] = (float)((double)odd * c + (double)even * s); (void)ec; (void)os; (void)oc; (void)es;"),
    "RoPE table stride ignored": ("const float* cs = cos_sin + base * cos_stride;",
                                  "const float* cs = cos_sin + base * 64; (void)cos_stride;"),
    "insert page stride ignored": ("uint8_t* page = cache + (slot / block) * cache_block_stride;",
                                   "uint8_t* page = cache + (slot / block) * block * 528;"),
    "no NaN sanitising": ("if (isnan(r[d])) r[d] = 0.0f;", "(void)r;"),
    "NVFP4 scale not rounded to E4M3": ("float S = (float)e4m3_value(s8);", "float S = sf;"),
    "ring row from block stride": (
        "(s / capacity) * state_stride + (s % capacity) * state_row_stride;",
        "(s / capacity) * state_stride + (s % capacity) * width;"),
    "ring keeps slots past the end": ("if (s < 0 || s >= num_blocks * capacity) continue;", "if (s < 0) continue;"),
    "RMSNorm without eps": ("sqrt(ss / (double)width + (double)eps)", "sqrt(ss / (double)width)"),
    "RMSNorm mean over width-1": ("sqrt(ss / (double)width + (double)eps)", "sqrt(ss / (double)(width - 1) + (double)eps)"),
    "RMSNorm writes invalid tokens": ("    if (slot_mapping[t] < 0) continue;\n    const float* x = kv", "    const float* x = kv"),
    "bf16 ties away from zero": ("else pick = (lo & 1u) ? hi : lo;", "else pick = hi;"),
    "V4 groups of 32": ("for (int j = 0; j < 64; ++j) amax = fmaxf(amax, fabsf(r[64 * g + j]));",
                        "for (int j = 0; j < 32; ++j) amax = fmaxf(amax, fabsf(r[64 * g + j]));"),
    "V4 pad scale not zero": ("    scales[7] = 0;\n", "    scales[7] = scales[6];\n"),
    "V4 RoPE bf16 big-endian": ("values[448 + 2 * (d - 448)] = (uint8_t)(h & 0xFF);",
                                "values[448 + 2 * (d - 448)] = (uint8_t)(h >> 8); continue;"),
    "attention without scale": ("sc[j] = scale * dot;", "sc[j] = dot; (void)scale;"),
    "attention sink ignored": ("double den = sink ? exp((double)sink[h] - m) : 0.0;", "double den = 0.0;"),
    "attention without max shift": ("double w = exp(sc[j] - m);", "double w = exp(sc[j]);"),
    "attention normalised by count": ("for (int64_t d = 0; d < latent; ++d) o[d] /= den;",
                                      "for (int64_t d = 0; d < latent; ++d) o[d] /= (double)topk;"),
    "attention scores negated": ("sc[j] = scale * dot;", "sc[j] = -scale * dot;"),
    "attention query of head 0": ("const uint16_t* qh = q + (t * num_heads + h) * latent;",
                                  "const uint16_t* qh = q + (t * num_heads) * latent;"),
    "NVFP4 sign of -0.0 kept": ("return idx | ((q < 0.0f) ? 8 : 0);", "return idx | ((q < 0.0f || signbit(q)) ? 8 : 0);"),
}


def test_unmutated_copy_passes_every_check(tmp_path):
    """Control: a verbatim copy built the same way passes all checks, so a
    failure below is the mutation's doing."""
    src = tmp_path / "copy.c"
    src.write_text(open(oracle.SRC).read())
    orc = oracle.Oracle(oracle.build(str(src), str(tmp_path / "libcopy.so")))
    for check, kwargs in CHECKS:
        check(orc=orc, **kwargs)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, tmp_path):
    old, new = MUTANTS[name]
    text = open(oracle.SRC).read()
    assert text.count(old) >= 1, f"mutation anchor not found: {name}"
    src = tmp_path / "mutant.c"
    src.write_text(text.replace(old, new, 1))
    orc = oracle.Oracle(oracle.build(str(src), str(tmp_path / "libmutant.so")))
    for check, kwargs in CHECKS:
        try:
            check(orc=orc, **kwargs)
        except (AssertionError, ValueError):
            return
    pytest.fail(f"no pin catches the mutant '{name}'")
