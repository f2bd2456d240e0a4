"""Pins of the CPU oracle against what the pages and the mathematics fix.

Nothing here compares the oracle with itself: expected values come from
exact rational arithmetic (Python fractions), the pages' own rules and
constants (tests/golden/format_constants.json, each entry cited), closed
forms, or torch's float8_e4m3fn conversion.  A mistake in the oracle's
exponent rule, rounding, tie handling, sign rule, nibble order, layout,
paged addressing, gating or RoPE indexing fails at least one test below.

Sources: [P1] docs page "vllm.v1.attention.ops.mxfp4_mla.store";
[P2] docs page "vllm.models.deepseek_v41.common.ops.fused_compress_quant_cache";
[P3] pull request "Add an mxfp4_mla KV cache for rope-free sparse MLA".
"""

from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from tests.exact_ref import (
    bf16_bits_of_fraction,
    bf16_fraction,
    ceil_log2,
    f32_bits,
    fp32_quotient_is_zero,
    golden,
    midpoint_index,
)

G = golden()
MIDS = G["e2m1_midpoints"]
STRICT = G["e2m1_midpoint_strict"]
GRID = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2),
        Fraction(3), Fraction(4), Fraction(6)]
TWO = Fraction(2)


def expected_mxfp4_code(x: Fraction, xbits: int, e: int) -> int:
    """Code of one element under scale 2^e: the pages' midpoint count on the
    exact quotient, sign bit when the fp32 quotient is below zero."""
    q = x / TWO ** e
    if fp32_quotient_is_zero(x, e):
        return 0
    idx = midpoint_index(abs(q), MIDS, STRICT)
    return idx | (8 if (xbits & 0x8000) else 0)


def expected_scale_exponent(amax: Fraction) -> int:
    """Smallest e with 2^e >= amax/6, floored at -126 (bit-pattern reading of a
    subnormal amax/6)."""
    return max(ceil_log2(amax / 6), -126)


def flat_store(src: np.ndarray, orc=oracle) -> np.ndarray:
    n = src.shape[0]
    cache = np.full(n * 272, 0xA5, dtype=np.uint8)
    orc.mxfp4_store(src, np.arange(n, dtype=np.int64), cache, 1, n, n)
    return cache.reshape(n, 272)


def nibble(rows: np.ndarray, token: int, elem: int) -> int:
    b = int(rows[token, elem // 2])
    return (b & 0xF) if elem % 2 == 0 else (b >> 4)


# ---------------------------------------------------------------- constants

def test_format_constants(orc=oracle):
    assert orc.row_bytes(512) == G["row_bytes_512"] == 512 // 2 + 512 // 32
    assert round(G["bf16_row_bytes_512"] / G["row_bytes_512"], 2) == float(G["capacity_ratio"])
    assert orc.row_bytes(128) == 68 and orc.row_bytes(1024) == 544
    assert orc.row_bytes(100) < 0  # not a multiple of the group
    # E2M1 grid: midpoints are exactly halfway between consecutive magnitudes.
    assert [float((GRID[i] + GRID[i + 1]) / 2) for i in range(7)] == MIDS
    assert float(GRID[-1]) == G["e2m1_max"]
    # E4M3 extremes used by the variants.
    assert orc.e4m3_value(0x7E) == G["e4m3_max"]
    assert orc.e4m3_value(0x01) == G["nvfp4_scale_min"]  # 2^-9: least subnormal
    assert orc.e4m3_value(0x08) == 2.0 ** -6              # least normal


# ---------------------------------------------------------------- exponent + codes

def make_solo_sweep(orc=oracle):
    """All 65,536 bf16 patterns, each alone in its group (rest +0)."""
    pats = np.arange(65536, dtype=np.uint32).reshape(4096, 16)
    src = np.zeros((4096, 512), dtype=np.uint16)
    src[:, ::32] = pats.astype(np.uint16)
    return pats, flat_store(src, orc)


@pytest.fixture(scope="module")
def solo_sweep():
    return make_solo_sweep()


def test_scale_exponent_exhaustive(solo_sweep, orc=oracle):
    pats, rows = solo_sweep
    for t in range(4096):
        for g in range(16):
            p = int(pats[t, g])
            x = bf16_fraction(p)
            got = int(rows[t, 256 + g])
            if x is None:
                assert got == 0xFF, hex(p)  # reading R6
            elif x == 0:
                assert got == G["zero_group_scale_byte"], hex(p)
            else:
                assert got == expected_scale_exponent(abs(x)) + G["e8m0_bias"], hex(p)


def test_bit_pattern_rule_agrees_with_definition(orc=oracle):
    """The store page computes the exponent on the fp32 bit pattern of
    amax/6; for every positive finite bf16 amax it equals the exact
    definition (floored at -126), so the reading of how amax/6 is formed
    does not matter."""
    for p in range(1, 0x7F80):
        a = np.float32(float(bf16_fraction(p)))
        bits = f32_bits(np.float32(a) / np.float32(6.0))
        exp_field, mant = (bits >> 23) & 0xFF, bits & 0x7FFFFF
        rule = exp_field - 127 + (1 if mant else 0)
        assert rule == expected_scale_exponent(Fraction(float(a))), hex(p)
        assert orc.ceil_pow2_exponent(float(np.float32(a) / np.float32(6.0))) == rule


def test_solo_codes_exhaustive(solo_sweep, orc=oracle):
    pats, rows = solo_sweep
    for t in range(4096):
        for g in range(16):
            p = int(pats[t, g])
            x = bf16_fraction(p)
            got = nibble(rows, t, 32 * g)
            if x is None or x == 0:
                assert got == 0, hex(p)
                continue
            e = expected_scale_exponent(abs(x))
            assert got == expected_mxfp4_code(x, p, e), hex(p)
            # the amax element's magnitude lands in (3, 6] unless the floor hit
            if abs(x) / 6 >= TWO ** -126:
                assert got & 7 >= 5, hex(p)
            # the other 31 elements are +0
            assert all(nibble(rows, t, 32 * g + j) == 0 for j in range(1, 32))


@pytest.mark.parametrize("k", [0, 125, -126, 17, -100])
def test_anchored_sweep(k, orc=oracle):
    """Groups [6*2^k, x, ...] fix e = k; every finite bf16 x with
    |x| <= 6*2^k is swept (k = 125 reaches the fp32 underflow region of the
    quotient, k = -126 the subnormal inputs)."""
    anchor = Fraction(6) * TWO ** k
    abits = bf16_bits_of_fraction(anchor)
    cands = [p for p in range(65536)
             if bf16_fraction(p) is not None and abs(bf16_fraction(p)) <= anchor]
    per = 31
    ngroups = -(-len(cands) // per)
    ntok = -(-ngroups // 16)
    src = np.zeros((ntok, 512), dtype=np.uint16)
    flat = src.reshape(-1, 32)
    flat[:ngroups, 0] = abits
    for i, p in enumerate(cands):
        flat[i // per, 1 + i % per] = p
    rows = flat_store(src, orc)
    for gi in range(ngroups):
        t, g = divmod(gi, 16)
        assert int(rows[t, 256 + g]) == k + 127
        assert nibble(rows, t, 32 * g) == 7  # 6 * 2^k / 2^k = 6
    for i, p in enumerate(cands):
        gi = i // per
        t, g = divmod(gi, 16)
        elem = 32 * g + 1 + i % per
        assert nibble(rows, t, elem) == expected_mxfp4_code(bf16_fraction(p), p, k), (hex(p), k)


@pytest.mark.parametrize("j", [-124, -60, -3, 0, 1, 7, 64, 126])
def test_powers_of_two(j, orc=oracle):
    """A power-of-two amax costs no exponent step: amax = 2^j encodes as
    4.0 (code 6) with byte j-2+127; amax = 3*2^j as 6.0 (code 7) with byte
    j-1+127 (a log2-based ceiling would give byte +1 and code 5)."""
    src = np.zeros((1, 512), dtype=np.uint16)
    src[0, 0] = bf16_bits_of_fraction(TWO ** j)
    src[0, 32] = bf16_bits_of_fraction(-TWO ** j)
    src[0, 64] = bf16_bits_of_fraction(3 * TWO ** j)
    rows = flat_store(src, orc)
    assert rows[0, 256] == j - 2 + 127 and nibble(rows, 0, 0) == 6
    assert rows[0, 257] == j - 2 + 127 and nibble(rows, 0, 32) == 6 | 8
    assert rows[0, 258] == j - 1 + 127 and nibble(rows, 0, 64) == 7


@pytest.mark.parametrize("k", [-120, -5, 0, 3, 100])
def test_ties_to_even(k, orc=oracle):
    """Exact midpoints m*2^k (anchor 6*2^k) go to the even index of their
    two neighbours: indices 0, 2, 2, 4, 4, 6, 6 for the seven midpoints."""
    src = np.zeros((1, 512), dtype=np.uint16)
    src[0, 0] = bf16_bits_of_fraction(6 * TWO ** k)
    for i, m in enumerate(MIDS):
        src[0, 1 + i] = bf16_bits_of_fraction(Fraction(m) * TWO ** k)
        src[0, 9 + i] = bf16_bits_of_fraction(-Fraction(m) * TWO ** k)
    rows = flat_store(src, orc)
    expect = [0, 2, 2, 4, 4, 6, 6]
    for i in range(7):
        assert nibble(rows, 0, 1 + i) == expect[i]
        assert nibble(rows, 0, 9 + i) == expect[i] | 8


def test_negative_zero_small_negatives_and_nibble_order(orc=oracle):
    """bf16 -0.0 gives code 0; a small negative gives code 8 [P1
    `_quantize_e2m1`]; element 2i sits in the low nibble of byte i [P3
    Details]."""
    src = np.zeros((1, 512), dtype=np.uint16)
    src[0, 0] = bf16_bits_of_fraction(Fraction(6))     # code 7, e = 0
    src[0, 1] = bf16_bits_of_fraction(Fraction(1, 2))  # code 1
    src[0, 2] = 0x8000                                 # -0.0 -> 0
    src[0, 3] = 0xBC24                                 # about -0.01 -> 8
    rows = flat_store(src, orc)
    assert rows[0, 0] == 0x17
    assert rows[0, 1] == 0x80
    assert rows[0, 256] == 127


def test_all_zero_groups_and_nonfinite(orc=oracle):
    src = np.zeros((1, 512), dtype=np.uint16)
    src[0, 32:64] = 0x8000           # all -0.0
    src[0, 64] = 0x7F80              # +Inf with finite neighbours
    src[0, 65] = 0x4000
    src[0, 96] = 0x7FC1              # NaN
    rows = flat_store(src, orc)
    assert rows[0, 256] == 127 and rows[0, 257] == 127
    assert (rows[0, 16:32] == 0).all()
    assert rows[0, 258] == 0xFF and (rows[0, 32:48] == 0).all()
    assert rows[0, 259] == 0xFF and (rows[0, 48:64] == 0).all()


def test_invariants_on_random_rows(orc=oracle):
    """On varied random rows: decoded magnitude never exceeds 6, the scale is
    minimal (the amax element decodes to >= 3 times the scale unless the
    -126 floor applies), scale bytes lie in [1, 253], and the error is at most
    half the local E2M1 gap times the scale."""
    rng = np.random.default_rng(7)
    x = rng.standard_t(2, size=(64, 512)) * np.exp2(rng.uniform(-130, 120, size=(64, 1)))
    with np.errstate(over="ignore", under="ignore"):
        xf = x.astype(np.float32)
    bits = ((xf.view(np.uint32).astype(np.uint64) + 0x7FFF + ((xf.view(np.uint32) >> 16) & 1)) >> 16)
    src = bits.astype(np.uint16)
    src[(src & 0x7F80) == 0x7F80] = 0x3F80  # keep the rows finite
    rows = flat_store(src, orc)
    for t in range(64):
        for g in range(16):
            byte = int(rows[t, 256 + g])
            vals = [bf16_fraction(int(src[t, 32 * g + j])) for j in range(32)]
            amax = max(abs(v) for v in vals)
            if amax == 0:
                assert byte == 127
                continue
            assert 1 <= byte <= 253
            e = byte - 127
            for j, v in enumerate(vals):
                c = nibble(rows, t, 32 * g + j)
                dq = GRID[c & 7] * (-1 if c & 8 else 1)
                q = v / TWO ** e
                assert abs(dq) <= 6
                gap = Fraction(1, 2) if abs(q) <= 2 else (Fraction(1) if abs(q) <= 4 else Fraction(2))
                assert abs(q - dq) <= gap / 2
            top = max(range(32), key=lambda j: abs(vals[j]))
            if amax / 6 >= TWO ** -126:
                assert nibble(rows, t, 32 * g + top) & 7 >= 5


# ---------------------------------------------------------------- layout

def test_paged_addressing_pads_and_canaries(orc=oracle):
    """Row of slot s at ((s // B) * stride_rows + s % B) * 272 [P1
    `store_mxfp4_mla`]; pads (-1) and slots past the last one write nothing;
    every byte outside written rows keeps its canary."""
    rng = np.random.default_rng(3)
    nb, bs, stride = 5, 8, 24
    src = (rng.integers(0, 0x7F00, size=(12, 512)) | (rng.integers(0, 2, size=(12, 512)) << 15)).astype(np.uint16)
    slots = np.array([0, 7, 8, 15, 39, -1, 17, 40, 1000, 33, -5, 3], dtype=np.int64)
    cache = np.full(((nb - 1) * stride + bs) * 272, 0xA5, dtype=np.uint8)
    orc.mxfp4_store(src, slots, cache, nb, bs, stride)
    touched = np.zeros(cache.size, dtype=bool)
    for t, s in enumerate(slots):
        if s < 0 or s >= nb * bs:
            continue
        off = ((s // bs) * stride + s % bs) * 272
        assert (cache[off:off + 272] == orc.quantize_row(src[t])).all()
        touched[off:off + 272] = True
    assert (cache[~touched] == 0xA5).all()


def test_strided_source_rows(orc=oracle):
    """The latent may be a row-strided view (e.g. the first 512 columns of a
    [T, 576] tensor); only rows are strided."""
    rng = np.random.default_rng(4)
    wide = rng.integers(0, 0x7F00, size=(6, 576)).astype(np.uint16)
    view = wide[:, :512]
    cache = np.zeros(6 * 272, dtype=np.uint8)
    orc.mxfp4_store(view, np.arange(6, dtype=np.int64), cache, 1, 6, 6)
    for t in range(6):
        assert (cache[t * 272:(t + 1) * 272] == orc.quantize_row(np.ascontiguousarray(view[t]))).all()


# ---------------------------------------------------------------- dequant

def test_dequant_table_exhaustive(orc=oracle):
    """All 16 codes x 256 scale bytes against the exact product
    E2M1(code) * 2^(byte - 127) (+-Inf from 2^128, NaN for byte 0xFF)."""
    for b in range(256):
        for c in range(16):
            got = orc.dequant_bf16(c, b)
            if b == 0xFF:
                assert got == 0x7FC0
                continue
            v = GRID[c & 7] * (-1 if c & 8 else 1) * TWO ** (b - 127)
            if c == 8:
                assert got == 0x8000  # -0.0
            else:
                assert got == bf16_bits_of_fraction(v), (c, b)


def test_round_trip_within_half_gap(orc=oracle):
    rng = np.random.default_rng(5)
    src = (rng.standard_normal((16, 512)) * np.exp2(rng.uniform(-30, 30, (16, 1)))).astype(np.float32)
    bits = (src.view(np.uint32) >> 16).astype(np.uint16)  # truncation is fine for test data
    rows = flat_store(bits, orc)
    cache = rows.reshape(-1).copy()
    out = orc.mxfp4_gather_dequant(cache, 1, 16, 16, 512, np.arange(16, dtype=np.int64))
    for t in range(16):
        for g in range(16):
            e = int(rows[t, 256 + g]) - 127
            for j in range(32):
                x = bf16_fraction(int(bits[t, 32 * g + j]))
                d = bf16_fraction(int(out[t, 32 * g + j]))
                q = abs(x) / TWO ** e
                gap = Fraction(1, 2) if q <= 2 else (Fraction(1) if q <= 4 else Fraction(2))
                assert abs(x - d) <= gap / 2 * TWO ** e


def test_dequant_skips_bad_slots(orc=oracle):
    cache = np.zeros(4 * 272, dtype=np.uint8)
    out = np.full((3, 512), 0x1234, dtype=np.uint16)
    orc.mxfp4_gather_dequant(cache, 1, 4, 4, 512, np.array([-1, 4, 2], dtype=np.int64), out)
    assert (out[0] == 0x1234).all() and (out[1] == 0x1234).all() and (out[2] == 0).all()


# ---------------------------------------------------------------- e4m3

def _torch_e4m3(v: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32)).to(torch.float8_e4m3fn) \
        .view(torch.uint8).numpy()


def test_e4m3_encode_matches_torch(orc=oracle):
    """fp32 -> E4M3FN with round-to-nearest-even, subnormals and the sign of
    zero, against torch's float8_e4m3fn over every bf16 value in [-448, 448],
    every grid midpoint +-1 ulp, and random fp32 values."""
    vals = []
    h = np.arange(65536, dtype=np.uint32)
    f = (h << 16).view(np.float32)
    vals.append(f[np.isfinite(f) & (np.abs(f) <= 448)])
    grid = np.array([orc.e4m3_value(c) for c in range(0x7F)], dtype=np.float64)
    mids = ((grid[:-1] + grid[1:]) / 2).astype(np.float32)
    vals += [mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(1000))]
    rng = np.random.default_rng(6)
    vals.append((rng.uniform(-1, 1, 200000) * np.exp2(rng.uniform(-14, 9, 200000))).astype(np.float32))
    v = np.concatenate(vals).astype(np.float32)
    v = np.concatenate([v, -v])
    v = v[np.abs(v) <= 448]
    assert (orc.e4m3_encode_array(v) == _torch_e4m3(v)).all()
    assert orc.e4m3_encode(-0.0) == 0x80 and orc.e4m3_encode(0.0) == 0x00


# ---------------------------------------------------------------- RoPE variants

def _identity_table(rows=8):
    t = np.zeros((rows, 64), dtype=np.float32)
    t[:, :32] = 1.0
    return t


def _run_rope(fn, latent, positions, table, slots, block=4, nb=None, cr=4, width=528):
    nb = nb or max(1, -(-int(max(slots.max(), 0) + 1) // block))
    cache = np.full(nb * block * width, 0xA5, dtype=np.uint8)
    fn(latent, positions, table, cache, block, nb, slots, cr)
    return cache, nb


def test_mxfp8_exponent_exhaustive_and_values(orc=oracle):
    """Every positive finite bf16 value as a group's only nonzero element,
    through an identity rotation: scale byte = min(max(E + 127, 0), 254) with
    E the exact ceiling of log2 of fp32(max(amax, fl(1e-4)) * fl(1/448))
    (the fp32 product taken with numpy), value byte = torch's E4M3 of
    fp32(amax * 2^-E)."""
    pats = np.arange(1, 0x7F80, dtype=np.uint16)
    n = -(-pats.size // 16)
    latent = np.zeros((n, 512), dtype=np.uint16)
    flat = latent.reshape(-1, 32)
    flat[: pats.size, 0] = pats
    positions = np.full(n, 3, dtype=np.int64)
    slots = np.arange(n, dtype=np.int64)
    block = 16
    nb = -(-n // block)
    cache = np.full(nb * block * 528, 0xA5, dtype=np.uint8)
    orc.mxfp8_rope_store(latent, positions, _identity_table(), cache, block, nb, slots, 4)
    pages = cache.reshape(nb, block * 528)
    inv448 = np.float32(1.0 / 448.0)
    floor = np.float32(1e-4)
    amax = np.maximum((pats.astype(np.uint32) << 16).view(np.float32), floor)
    v = (amax * inv448).astype(np.float32)
    E = np.array([ceil_log2(Fraction(float(x))) for x in v])
    y = np.array([np.float32(float(bf16_fraction(int(p)) / TWO ** int(k))) for p, k in zip(pats, E)])
    want_val = _torch_e4m3(y)
    for i, p in enumerate(pats):
        t, g = divmod(i, 16)
        page, r = divmod(t, block)
        sbyte = pages[page, block * 512 + r * 16 + g]
        assert sbyte == min(max(int(E[i]) + 127, 0), 254), hex(p)
        assert pages[page, r * 512 + 32 * g] == want_val[i], hex(p)


def test_mxfp8_zero_group_byte_105(orc=oracle):
    latent = np.zeros((1, 512), dtype=np.uint16)
    cache, _ = _run_rope(orc.mxfp8_rope_store, latent, np.array([3], dtype=np.int64),
                         _identity_table(), np.array([0], dtype=np.int64))
    assert (cache[4 * 512: 4 * 512 + 16] == 105).all()
    assert (cache[:512] == 0).all()


def test_rope_exact_angles_pin_pairing_and_row(orc=oracle):
    """Rotations by exactly 90 and 180 degrees are permutations/negations of
    the RoPE pairs: (e, o) -> (-o, e) and (-e, -o) on dims 448..511 only.
    The table row is (position // CR) * CR: rows 41..43 and 61..63 hold NaN and
    must not be read, while the comparison tokens sit on identity rows 80..83,
    so only the right row makes the pairs agree."""
    rng = np.random.default_rng(8)
    a = rng.standard_normal((1, 512)).astype(np.float32)
    a[a == 0] = 1.0
    ab = (a.view(np.uint32) >> 16).astype(np.uint16)
    af = (ab.astype(np.uint32) << 16).view(np.float32)
    table = np.full((96, 64), np.nan, dtype=np.float32)
    table[40, :32], table[40, 32:] = 0.0, 1.0    # 90 degrees at row 40
    table[60, :32], table[60, 32:] = -1.0, 0.0   # 180 degrees at row 60
    table[80:84, :32], table[80:84, 32:] = 1.0, 0.0  # identity at rows 80..83
    b90 = af.copy()
    b90[0, 448::2], b90[0, 449::2] = -af[0, 449::2], af[0, 448::2]
    b180 = af.copy()
    b180[0, 448:] = -af[0, 448:]
    to_bits = lambda x: (x.view(np.uint32) >> 16).astype(np.uint16)
    latent = np.concatenate([ab, to_bits(b90), ab, to_bits(b180)])
    positions = np.array([43, 83, 63, 83], dtype=np.int64)  # bases 40, 80, 60, 80
    slots = np.arange(4, dtype=np.int64)
    for fn, width in ((orc.mxfp8_rope_store, 528), (orc.nvfp4_rope_store, 288),
                      (orc.v4_rope_store, 584)):
        cache = np.full(4 * width, 0xA5, dtype=np.uint8)
        fn(latent, positions, table, cache, 4, 1, slots, 4)
        vb = {528: 512, 288: 256, 584: 576}[width]
        sb = width - vb
        vals = cache[: 4 * vb].reshape(4, vb)
        scales = cache[4 * vb:].reshape(4, sb)
        assert (vals[0] == vals[1]).all() and (scales[0] == scales[1]).all()
        assert (vals[2] == vals[3]).all() and (scales[2] == scales[3]).all()


def test_rope_gate_and_canaries(orc=oracle):
    """Only tokens with a valid slot and (position + 1) % CR == 0 are written;
    everything else keeps its canary."""
    rng = np.random.default_rng(9)
    latent = (rng.standard_normal((8, 512)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    positions = np.array([3, 4, 7, 8, 11, 15, 1, 2], dtype=np.int64)
    slots = np.array([0, 1, 2, 3, -1, 5, 6, 7], dtype=np.int64)
    table = _identity_table(16)
    for fn, width in ((orc.mxfp8_rope_store, 528), (orc.nvfp4_rope_store, 288),
                      (orc.v4_rope_store, 584)):
        cache = np.full(2 * 4 * width, 0xA5, dtype=np.uint8)
        fn(latent, positions, table, cache, 4, 2, slots, 4)
        vb = {528: 512, 288: 256, 584: 576}[width]
        sb = width - vb
        written = {0, 2, 5}  # positions 3, 7, 15 with valid slots
        for s in range(8):
            page, r = divmod(s, 4)
            base = page * 4 * width
            v = cache[base + r * vb: base + (r + 1) * vb]
            sc = cache[base + 4 * vb + r * sb: base + 4 * vb + (r + 1) * sb]
            if s in written:
                assert not (v == 0xA5).all()
            else:
                assert (v == 0xA5).all() and (sc == 0xA5).all(), s


def _rope_table():
    from workloads import rope_cos_sin_table

    return rope_cos_sin_table()


def _rope_latents(n, seed):
    """bf16 N(0,1) rows, some scaled by 2^-130 (subnormal products) or
    2^125 (sums near the top of the range), with signed zeros and
    infinities in a few NoPE and RoPE dims."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, 512)).astype(np.float32)
    x[n // 8: n // 4] *= np.float32(2.0 ** -130)
    x[n // 4: 3 * n // 8] *= np.float32(2.0 ** 125)
    bits = (x.view(np.uint32) >> 16).astype(np.uint16)
    picks = rng.integers(0, 512, (n, 6))
    rows = np.arange(n)[:, None]
    bits[rows, picks[:, :2]] = 0x0000
    bits[rows, picks[:, 2:4]] = 0x8000
    bits[n - 4:, 448:452] = [0x7F80, 0xFF80, 0x7F80, 0x3F80]
    return bits


def _numpy_rope(bits, positions, table, cr):
    """The pages' GPT-J rotation [P2 `_rope_quant_insert_mxfp8_kernel`: even*c
    - odd*s, odd*c + even*s on the interleaved pairs] in numpy float32
    element-wise operations (each product and each sum rounds once; numpy
    does not fuse), over all 256 pairs with (c, s) = (1, 0) for the NoPE
    pairs, using table row (position // cr) * cr."""
    x = (bits.astype(np.uint32) << 16).view(np.float32)
    n = x.shape[0]
    base = positions // cr * cr
    c = np.ones((n, 256), dtype=np.float32)
    s = np.zeros((n, 256), dtype=np.float32)
    c[:, 224:] = table[base, :32]
    s[:, 224:] = table[base, 32:64]
    e, o = x[:, 0::2], x[:, 1::2]
    r = np.empty_like(x)
    with np.errstate(invalid="ignore", over="ignore"):
        r[:, 0::2] = e * c - o * s
        r[:, 1::2] = o * c + e * s
    return r


def _same_f32(a, b):
    """Bitwise equality, NaN matching NaN whatever its payload."""
    return (a.view(np.uint32) == b.view(np.uint32)) | (np.isnan(a) & np.isnan(b))


def _e2m1_codes(y):
    """The pages' midpoint count [P1 `_quantize_e2m1`] on fp32 quotients,
    vectorised: index = number of midpoints below |y| (strict at 0.25, 1.25,
    2.5, 5; inclusive at 0.75, 1.75, 3.5), sign bit when y < 0, NaN -> 0."""
    a = np.abs(y)
    idx = sum((a > m) if st else (a >= m) for m, st in zip(MIDS, STRICT))
    code = idx.astype(np.uint8) | np.where(y < 0, 8, 0).astype(np.uint8)
    return np.where(np.isnan(y), 0, code).astype(np.uint8)


def _exact_ceil_log2_f32(v):
    """Exact ceil(log2 v) of positive finite fp32 values (frexp of the exact
    double: v = m * 2^k, m in [0.5, 1), ceil is k - 1 at m = 0.5, else k)."""
    m, k = np.frexp(v.astype(np.float64))
    return np.where(m == 0.5, k - 1, k).astype(np.int64)


def _mxfp8_expected(r, group=32, sanitize=True):
    """MXFP8 values and scale bytes of rotated rows r [n, D] in groups of
    `group` [P2 `_rope_quant_insert_mxfp8_kernel`; readings R11, R14]."""
    n, d = r.shape
    g = r.reshape(n, d // group, group)
    amax = np.maximum(np.abs(g).max(axis=2), np.float32(1e-4))
    v = (amax * np.float32(1.0 / 448.0)).astype(np.float32)
    fin = np.isfinite(v)
    E = np.where(fin, _exact_ceil_log2_f32(np.where(fin, v, 1.0)), 128)
    mult = np.ldexp(np.float32(1.0), -E).astype(np.float32)
    with np.errstate(invalid="ignore"):
        y = np.clip((g * mult[:, :, None]).astype(np.float32), -448, 448)
    vals = _torch_e4m3(y.reshape(n, d))
    scales = np.clip(E + 127, 0, 254 if sanitize else 255).astype(np.uint8)
    return vals, scales


def _nvfp4_expected(r):
    """NVFP4 code bytes and E4M3 scales of rotated rows r [n, 512] [P2
    `_rope_quant_insert_nvfp4_kernel`; readings R15, R16]: the quotient is
    numpy's correctly rounded fp32 division."""
    n = r.shape[0]
    t = r.reshape(n, 32, 16)
    sf = np.clip((np.abs(t).max(axis=2) * np.float32(1.0 / 6.0)).astype(np.float32),
                 np.float32(2.0 ** -9), np.float32(448))
    s8 = _torch_e4m3(sf)
    S = torch.from_numpy(s8).view(torch.float8_e4m3fn).float().numpy()
    codes = _e2m1_codes((t / S[:, :, None]).astype(np.float32)).reshape(n, 512)
    return (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8), s8


def test_rope_rotation_general_angles_against_numpy(orc=oracle):
    """Reading R12 pinned at general angles: the oracle's rotated latent
    equals numpy's float32 element-wise rotation bit for bit, on the real
    65,536-row GPT-J table (theta 10^4) at random positions, for ratios 1 and
    4, with and without sanitising.  An FMA in the rotation, or the rotation
    evaluated in double and rounded once, changes the last bit of many
    values and fails here."""
    table = _rope_table()
    rng = np.random.default_rng(41)
    n = 4096
    bits = _rope_latents(n, 42)
    for cr in (1, 4):
        positions = rng.integers(0, 65536, n).astype(np.int64)
        if cr > 1:
            positions[: n // 2] = positions[: n // 2] // cr * cr + cr - 1  # half pass the gate
        want = _numpy_rope(bits, positions, table, cr)
        gate = (positions + 1) % cr == 0
        for sanitize in (True, False):
            got, written = orc.rope_rotate(bits, positions, table, cr, sanitize)
            assert (written == gate).all()
            w = want[gate].copy()
            if sanitize:
                w[np.isnan(w)] = 0.0
            ok = _same_f32(got[gate], w)
            assert ok.all(), f"cr={cr} sanitize={sanitize}: {np.count_nonzero(~ok)} values differ"
            assert np.isnan(got[~gate]).all()


def test_rope_inserts_at_general_angles(orc=oracle):
    """The three records built from numpy's rotation (above) through encoders
    restated from the pages' rules: V4's RoPE dims are torch's bf16
    (nearest-even) of the rotated values byte for byte, its NoPE dims and
    the MXFP8 record follow the E8M0/E4M3 rule, NVFP4 the E4M3 tile scale and
    the midpoint count of the fp32 quotient.  Real table, random positions,
    ratio 1, every record compared."""
    table = _rope_table()
    rng = np.random.default_rng(43)
    n = 2048
    bits = _rope_latents(n, 44)
    positions = rng.integers(0, 65536, n).astype(np.int64)
    slots = rng.permutation(n).astype(np.int64)
    r = _numpy_rope(bits, positions, table, 1)
    r[np.isnan(r)] = 0.0
    block = 64
    nb = n // block
    inv = np.argsort(slots)  # token of each slot

    cache = np.full(nb * block * 528, 0xA5, dtype=np.uint8)
    orc.mxfp8_rope_store(bits, positions, table, cache, block, nb, slots, 1)
    pages = cache.reshape(nb, block * 528)
    vals = pages[:, : block * 512].reshape(n, 512)
    scales = pages[:, block * 512:].reshape(n, 16)
    wv, ws = _mxfp8_expected(r[inv])
    assert (vals == wv).all() and (scales == ws).all()

    cache = np.full(nb * block * 288, 0xA5, dtype=np.uint8)
    orc.nvfp4_rope_store(bits, positions, table, cache, block, nb, slots, 1)
    pages = cache.reshape(nb, block * 288)
    vals = pages[:, : block * 256].reshape(n, 256)
    scales = pages[:, block * 256:].reshape(n, 32)
    wv, ws = _nvfp4_expected(r[inv])
    assert (scales == ws).all() and (vals == wv).all()

    cache = np.full(nb * block * 584, 0xA5, dtype=np.uint8)
    orc.v4_rope_store(bits, positions, table, cache, block, nb, slots, 1)
    pages = cache.reshape(nb, block * 584)
    vals = pages[:, : block * 576].reshape(n, 576)
    scales = pages[:, block * 576:].reshape(n, 8)
    rs = r[inv]
    rope_bf16 = torch.from_numpy(np.ascontiguousarray(rs[:, 448:])).to(torch.bfloat16) \
        .view(torch.int16).numpy().view(np.uint16)
    assert (vals[:, 448:].copy().view(np.uint16) == rope_bf16).all()
    wv, ws = _mxfp8_expected(np.ascontiguousarray(rs[:, :448]), group=64)
    assert (vals[:, :448] == wv).all()
    assert (scales[:, :7] == ws).all() and (scales[:, 7] == 0).all()


def test_rope_strided_table_and_pages(orc=oracle):
    """The table may be a column slice of a wider one (row stride > 64) and
    pages may sit further apart than one block of records [P2
    `rope_quant_insert` passes `cos_sin_cache.stride(0)` and
    `kv_cache.stride(0)`].  Hand-placed: the wider table's extra columns and
    the rows the gate never selects are NaN; pages are 48 bytes apart beyond
    their records, the gaps (and a spare page past the last) hold canaries.
    The result page by page equals the dense one, and every gap byte is
    still 0xA5."""
    table = _rope_table()[:512]
    rng = np.random.default_rng(45)
    n, block, nb = 96, 8, 16
    bits = _rope_latents(n, 46)
    positions = rng.integers(0, 512, n).astype(np.int64)
    slots = rng.permutation(nb * block)[:n].astype(np.int64)
    slots[::7] = -1
    wide = np.full((512, 80), np.nan, dtype=np.float32)
    wide[:, :64] = table
    for fn, width in ((orc.mxfp8_rope_store, 528), (orc.nvfp4_rope_store, 288),
                      (orc.v4_rope_store, 584)):
        for cr in (1, 4):
            dense = np.full(nb * block * width, 0xA5, dtype=np.uint8)
            fn(bits, positions, table, dense, block, nb, slots, cr)
            stride = block * width + 48
            strided = np.full((nb + 1) * stride, 0xA5, dtype=np.uint8)
            fn(bits, positions, wide[:, :64], strided, block, nb, slots, cr,
               cache_block_stride=stride)
            pages = strided.reshape(nb + 1, stride)
            assert (pages[:nb, : block * width].reshape(-1) == dense).all(), (width, cr)
            assert (pages[:nb, block * width:] == 0xA5).all() and (pages[nb] == 0xA5).all()


def test_nvfp4_scales_and_codes(orc=oracle):
    """NVFP4 tile scale = torch E4M3 of clamp(fp32(amax * fl(1/6)), 2^-9, 448);
    codes = the pages' midpoint count on the numpy fp32 quotient r / scale,
    saturating at index 7, sign bit below zero."""
    rng = np.random.default_rng(10)
    n = 64
    x = (rng.standard_normal((n, 512)) * np.exp2(rng.uniform(-16, 12, (n, 32)).repeat(16, 1)))
    x = x.astype(np.float32)
    x[0, :16] = 0.0
    x[1, :16] = -0.0
    bits = (x.view(np.uint32) >> 16).astype(np.uint16)
    xf = (bits.astype(np.uint32) << 16).view(np.float32)
    positions = np.full(n, 3, dtype=np.int64)
    slots = np.arange(n, dtype=np.int64)
    cache = np.full(n * 288, 0xA5, dtype=np.uint8)
    orc.nvfp4_rope_store(bits, positions, _identity_table(), cache, n, 1, slots, 4)
    vals = cache[: n * 256].reshape(n, 256)
    scales = cache[n * 256:].reshape(n, 32)
    tiles = xf.reshape(n, 32, 16)
    amax = np.abs(tiles).max(axis=2)
    sf = np.clip((amax * np.float32(1.0 / 6.0)).astype(np.float32), np.float32(2.0 ** -9), np.float32(448))
    s8 = _torch_e4m3(sf)
    assert (scales == s8).all()
    S = torch.from_numpy(s8).view(torch.float8_e4m3fn).float().numpy()
    for t in range(n):
        for k in range(32):
            for j in range(16):
                y = np.float32(tiles[t, k, j]) / np.float32(S[t, k])
                yq = Fraction(float(y))
                code = midpoint_index(abs(yq), MIDS, STRICT) | (8 if y < 0 else 0)
                d = 16 * k + j
                got = (vals[t, d // 2] >> (4 * (d % 2))) & 0xF
                assert got == code, (t, k, j, float(y))


def test_e2m1_saturates_for_huge_quotients(orc=oracle):
    """The pages' midpoint count gives index 7 to every magnitude above 5, so
    huge quotients (an NVFP4 tile whose scale clamped at 448) saturate to
    +-6, whatever their size; NaN codes 0 (reading R16)."""
    for v in [5.0000005, 6.0, 6.5, 7.0, 1e6, 2.0 ** 60, 3.4e38, float("inf")]:
        for s in (1.0, -1.0):
            q = np.float32(s * v)
            want = midpoint_index(abs(Fraction(float(q))) if np.isfinite(q) else Fraction(10 ** 40),
                                  MIDS, STRICT) | (8 if q < 0 else 0)
            assert orc.e2m1_code(float(q)) == want == (7 | (8 if s < 0 else 0)), v
    assert orc.e2m1_code(float("nan")) == 0


def test_nvfp4_huge_tiles_saturate(orc=oracle):
    """Tiles with amax far above 6 * 448: scale byte 0x7E (448) and every
    element above 5 * 448 in magnitude codes +-6."""
    latent = np.zeros((1, 512), dtype=np.uint16)
    latent[0, :16] = 0x7F00      # 2^127
    latent[0, 1] = 0xFF00        # -2^127
    latent[0, 2] = 0x4500        # 2048 -> 2048 / 448 = 4.57 -> code 6
    cache = np.full(288, 0xA5, dtype=np.uint8)
    orc.nvfp4_rope_store(latent, np.array([3], dtype=np.int64), _identity_table(), cache, 1, 1,
                            np.array([0], dtype=np.int64), 4)
    assert cache[256] == 0x7E
    assert cache[0] == 0x7 | (0xF << 4)
    assert cache[1] == 0x6 | (0x7 << 4)


def test_rope_nan_sanitised(orc=oracle):
    """With sanitising, NaN becomes +0 before the scales are picked.  NoPE
    pairs go through the same rotation arithmetic with (cos, sin) = (1, 0), so
    a NaN also turns its pair partner into NaN (odd*1 + NaN*0) and both become
    0.  Latent [NaN, 0, 1.0, 0, ...] through an identity rotation:
    MXFP8 group 0: amax 1 -> v = fl(1/448) in (2^-9, 2^-8] -> E = -8, scale
    byte 119; 1.0 * 2^8 = 256 -> E4M3 0x78 at element 2; elements 0, 1 -> 0x00.
    NVFP4 tile 0: sf = fl(1/6) = 0.16667 lies above the E4M3 midpoint 0.1640625
    of 0.15625 and 0.171875 -> scale 0x23; 1 / 0.171875 = 5.82 -> code 7 at
    element 2, so byte 0 = 0x00 and byte 1 = 0x07."""
    latent = np.zeros((1, 512), dtype=np.uint16)
    latent[0, 0] = 0x7FC0  # NaN
    latent[0, 1] = 0x0000  # its pair partner
    latent[0, 2] = 0x3F80  # 1.0, next pair
    pos, slot = np.array([3], dtype=np.int64), np.array([0], dtype=np.int64)
    c8 = np.full(528, 0xA5, dtype=np.uint8)
    orc.mxfp8_rope_store(latent, pos, _identity_table(), c8, 1, 1, slot, 4)
    assert c8[0] == 0x00 and c8[1] == 0x00 and c8[2] == 0x78 and c8[512] == 119
    c4 = np.full(288, 0xA5, dtype=np.uint8)
    orc.nvfp4_rope_store(latent, pos, _identity_table(), c4, 1, 1, slot, 4)
    assert c4[0] == 0x00 and c4[1] == 0x07 and c4[256] == 0x23


def test_mxfp8_exponent_just_above_powers_of_two(orc=oracle):
    """R11: the exponent is the exact ceiling of log2(v).  RoPE output is full
    fp32, so with a table entry c and input 1.0 the group amax is exactly c;
    c is chosen so that v = fl(c * fl(1/448)) is the fp32 just above 2^k.
    There an fp32 log2 rounds down to k (|k| >= 4), while the exact ceiling,
    computed here in rationals, is k + 1."""
    inv448 = np.float32(1.0 / 448.0)
    for k in (-20, -9, -5, 4, 10, 60):
        target = np.nextafter(np.float32(2.0 ** k), np.float32(np.inf))
        c = np.float32(float(target) * 448.0)
        for _ in range(64):  # walk c until the fp32 product is the target
            v = np.float32(c * inv448)
            if v == target:
                break
            c = np.nextafter(c, np.float32(np.inf) if v < target else np.float32(0))
        assert np.float32(c * inv448) == target
        table = np.zeros((4, 64), dtype=np.float32)
        table[:, :32] = c
        latent = np.zeros((1, 512), dtype=np.uint16)
        latent[0, 448] = 0x3F80  # 1.0 -> rotated to exactly c
        cache = np.full(528, 0xA5, dtype=np.uint8)
        orc.mxfp8_rope_store(latent, np.array([3], dtype=np.int64), table, cache, 1, 1,
                             np.array([0], dtype=np.int64), 4)
        E = ceil_log2(Fraction(float(target)))
        assert E == k + 1
        assert cache[512 + 14] == min(max(E + 127, 0), 254), k


def test_save_ring_rows_placement(orc=oracle):
    """[P2 `save_ring_rows`] with the ring rule of `fused_save_compress_norm`:
    slot s lands in block s // capacity, ring row s % capacity.  Hand-placed
    case (capacity 3, 3 blocks, padded strides): slots 0, 4, -1, 5, 8, 9, -7
    -> (0,0), (1,1), skip, (1,2), (2,2), skip (past the last row), skip.
    Rows are bit patterns, NaN payloads and -0.0 included."""
    rng = np.random.default_rng(30)
    bits = rng.integers(0, 2**32, size=(7, 6), dtype=np.uint64).astype(np.uint32)
    bits[0, 0] = 0x7FC01234  # NaN with payload
    bits[1, 1] = 0x80000000  # -0.0
    rows_wide = np.zeros((7, 8), dtype=np.float32)
    rows_wide[:, :6] = bits.view(np.float32)
    rows = rows_wide[:, :6]
    # a fourth block of canaries sits where slot 9 would land if kept
    backing = np.full((4, 4, 7), np.float32(1.5), dtype=np.float32)
    state = backing[:3, :3, :6]
    slots = np.array([0, 4, -1, 5, 8, 9, -7], dtype=np.int64)
    orc.save_ring_rows(rows, slots, state)
    placed = {(0, 0): 0, (1, 1): 1, (1, 2): 3, (2, 2): 4}
    for b in range(4):
        for r in range(4):
            for c in range(7):
                got = np.array(backing[b, r, c]).view(np.uint32)
                if r < 3 and c < 6 and (b, r) in placed:
                    assert got == bits[placed[(b, r)], c], (b, r, c)
                else:
                    assert got == np.array(np.float32(1.5)).view(np.uint32), (b, r, c)


def test_rmsnorm_cr1_closed_forms(orc=oracle):
    """Compress ratio 1 [P2 `fused_save_compress_norm`]: y = x / rms(x) * w.
    Closed forms: a constant row c with eps = 0 gives sign(c) * w exactly;
    x = (3, 4, 0, ...) over 512 dims has rms 5 / sqrt(512); scaling x by 2^k
    leaves y unchanged when eps = 0; eps enters under the root; tokens with a
    negative slot are not written."""
    w = np.full(512, 0x3F80, dtype=np.uint16)          # 1.0
    w[7] = 0xC000                                       # -2.0
    kv = np.zeros((5, 512), dtype=np.float32)
    kv[0] = 0.75
    kv[1] = -3.0
    kv[2, 0], kv[2, 1] = 3.0, 4.0
    kv[3] = kv[2] * np.float32(2.0 ** 40)
    kv[4] = 1.0
    slots = np.array([0, 1, 2, 3, -1], dtype=np.int64)
    y = orc.rmsnorm_cr1(kv, slots, w, 0.0)
    assert (y[0] == np.where(np.arange(512) == 7, -2.0, 1.0)).all()
    assert (y[1] == np.where(np.arange(512) == 7, 2.0, -1.0)).all()
    s = np.sqrt(512.0) / 5.0
    assert abs(y[2, 0] - 3 * s) < 1e-12 and abs(y[2, 1] - 4 * s) < 1e-12 and (y[2, 2:] == 0).all()
    assert np.allclose(y[3], y[2], rtol=1e-15, atol=0)
    assert np.isnan(y[4]).all()                         # not written
    eps = 0.25
    y_eps = orc.rmsnorm_cr1(kv[:1], slots[:1], w, eps)
    assert abs(y_eps[0, 0] - 0.75 / np.sqrt(0.75 ** 2 + eps)) < 1e-15


def test_bf16_rounding_checker_matches_torch():
    """The parity checker used for bf16 outputs reproduces torch's fp32 ->
    bf16 round-to-nearest-even on values exact in fp32 (normal, subnormal,
    midpoints, signed zeros), and rejects a value one ulp off."""
    from tests.exact_ref import check_bf16_rounding
    rng = np.random.default_rng(7)
    v = (rng.standard_normal(20000) * np.exp2(rng.uniform(-140, 120, 20000))).astype(np.float32)
    mids = (rng.integers(0, 2**16, 2000).astype(np.uint32) << 16) | 0x8000   # exact midpoints
    v = np.concatenate([v, mids.view(np.float32), np.float32([0.0, -0.0, 1e-45, -3e-39])])
    v = v[np.isfinite(v)]
    bits = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    check_bf16_rounding(bits, v.astype(np.float64), band=0.0)
    bad = bits.copy()
    i = int(np.flatnonzero(np.abs(v) > 1e-30)[0])
    bad[i] ^= 1
    with pytest.raises(AssertionError):
        check_bf16_rounding(bad, v.astype(np.float64), band=0.0)


def test_f32_to_bf16_matches_torch(orc=oracle):
    """The oracle's fp32 -> bf16 rounding equals torch's (nearest, ties to
    even) on random values over the whole exponent range, exact midpoints,
    subnormals, the overflow boundary, signed zeros and infinities; NaN gives
    0x7FC0."""
    rng = np.random.default_rng(12)
    bits = rng.integers(0, 2**32, 3000, dtype=np.uint64).astype(np.uint32)
    mids = (rng.integers(0, 2**16, 1000).astype(np.uint32) << 16) | 0x8000
    edge = np.array([0x7F7F7FFF, 0x7F7F8000, 0x7F7FC000, 0x7F7F8001, 0x00008000, 0x00018000,
                     0x80000000, 0x00000000, 0x7F800000, 0xFF800000, 0x00000001], dtype=np.uint32)
    v = np.concatenate([bits, mids, edge]).view(np.float32)
    v = v[~np.isnan(v)]
    want = torch.from_numpy(v.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([orc.f32_to_bf16(x) for x in v], dtype=np.uint16)
    assert (got == want).all(), [(hex(int(v.view(np.uint32)[i])), hex(got[i]), hex(want[i]))
                                 for i in np.flatnonzero(got != want)[:5]]
    assert orc.f32_to_bf16(float("nan")) == 0x7FC0


def test_v4_record_values_scales_and_pad(orc=oracle):
    """V4 record (584 B): group g (64 NoPE dims) anchored at 448 * 2^k_g has
    scale byte k_g + 127 and values torch-E4M3 of x / 2^k_g; the eighth scale
    byte is 0; through an identity rotation the RoPE dims come back as the
    input's bf16 bits (little-endian, after the 448 E4M3 bytes).  A zero
    latent gives the 1e-4 floor's byte 105 and zero values."""
    rng = np.random.default_rng(13)
    ks = [0, -7, 5, -20, 60, -13, 100]   # 448 * 2^k above the 1e-4 floor
    lat = np.zeros((2, 512), dtype=np.float32)
    for g, k in enumerate(ks):
        x = rng.uniform(-0.5, 0.5, 64) * 448.0 * 2.0 ** k
        x[32 + 4 * g] = 448.0 * 2.0 ** k   # the anchor sits in the group's second half
        lat[0, 64 * g: 64 * g + 64] = x
    lat[0, 448:] = rng.standard_normal(64)
    lb = (lat.view(np.uint32) >> 16).astype(np.uint16)   # truncate: bf16 values
    lb[1] = 0
    lf = (lb.astype(np.uint32) << 16).view(np.float32)
    cache, _ = _run_rope(orc.v4_rope_store, lb, np.array([3, 7], dtype=np.int64),
                         _identity_table(), np.array([0, 1], dtype=np.int64), width=584)
    vals = cache[:4 * 576].reshape(4, 576)
    scales = cache[4 * 576: 4 * 584].reshape(4, 8)
    assert list(scales[0]) == [k + 127 for k in ks] + [0]
    for g, k in enumerate(ks):
        q = torch.from_numpy((lf[0, 64 * g: 64 * g + 64].astype(np.float64) * 2.0 ** -k).astype(np.float32))
        want = q.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert (vals[0, 64 * g: 64 * g + 64] == want).all(), g
    assert (vals[0, 448:].view(np.uint16) == lb[0, 448:]).all()
    assert list(scales[1]) == [105] * 7 + [0]
    assert (vals[1] == 0).all()
    assert (cache[2 * 576: 4 * 576] == 0xA5).all() and (scales[2:] == 0xA5).all()


# ---------------------------------------------------------------- attention (read side)

def _attn_cache(rows_f32: np.ndarray, orc=oracle):
    """Store fp32 rows (rounded to bf16) as an MXFP4 flat cache; return the
    cache and the rows' dequantized values (the pinned store and dequant)."""
    n = rows_f32.shape[0]
    bits = (np.ascontiguousarray(rows_f32, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)
    cache = np.zeros(n * 272, dtype=np.uint8)
    orc.mxfp4_store(bits, np.arange(n, dtype=np.int64), cache, 1, n, n)
    deq = orc.mxfp4_gather_dequant(cache, 1, n, n, 512, np.arange(n, dtype=np.int64))
    return cache, (deq.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _bf16_bits(x: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(x, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def test_attention_single_key_pads_and_sink(orc=oracle):
    """[P3 read path] One valid key among pads (-1, a negative, a slot past
    the cache) returns that row exactly for any query; no valid key returns
    zeros; with q = 0 the score is 0, so a sink of 0 halves the row, a sink
    of -inf changes nothing and a huge sink drives the output to 0."""
    rng = np.random.default_rng(40)
    cache, v = _attn_cache(rng.standard_normal((8, 512)).astype(np.float32), orc)
    q = _bf16_bits(rng.standard_normal((4, 2, 512)))
    q[2:] = 0
    idx = np.array([[5, -1, 99999, -7], [-1, -1, 8, -3], [5, -1, -1, -1], [5, -1, -1, -1]],
                   dtype=np.int32)
    out = orc.sparse_mla_attention(q, cache, 1, 8, 8, idx, 0.04)
    assert (out[0] == v[5]).all() and (out[1] == 0).all() and (out[2] == v[5]).all()
    out = orc.sparse_mla_attention(q, cache, 1, 8, 8, idx, 0.04,
                                   sink=np.array([0.0, -np.inf], dtype=np.float32))
    assert (out[2, 0] == v[5] / 2).all() and (out[2, 1] == v[5]).all()
    out = orc.sparse_mla_attention(q, cache, 1, 8, 8, idx, 0.04,
                                   sink=np.array([1e4, 1e4], dtype=np.float32))
    assert np.abs(out[2:]).max() < 1e-300 and (out[0] == v[5] * 0).all()


def test_attention_uniform_when_query_is_zero(orc=oracle):
    """q = 0 gives equal weights: the mean of the listed valid rows, a row
    listed twice counting twice."""
    rng = np.random.default_rng(41)
    cache, v = _attn_cache(rng.standard_normal((6, 512)).astype(np.float32), orc)
    q = np.zeros((2, 3, 512), dtype=np.uint16)
    idx = np.array([[0, 1, 2, 3, -1], [4, 4, 1, -1, -1]], dtype=np.int32)
    out = orc.sparse_mla_attention(q, cache, 1, 6, 6, idx, 1.0)
    assert np.allclose(out[0], v[:4].mean(axis=0), rtol=1e-14, atol=1e-300)
    assert np.allclose(out[1], (2 * v[4] + v[1]) / 3, rtol=1e-14, atol=1e-300)


def test_attention_temperature(orc=oracle):
    """Rows 0 (zeros) and 1 (one-hot 1.0) with a one-hot query give scores 0
    and `scale`; scale = ln 3 weighs them 1 : 3, so output dim 0 is 3/4."""
    rows = np.zeros((2, 512), dtype=np.float32)
    rows[1, 0] = 1.0
    cache, v = _attn_cache(rows, orc)
    assert v[1, 0] == 1.0 and (v[1, 1:] == 0).all() and (v[0] == 0).all()
    q = np.zeros((1, 1, 512), dtype=np.float32)
    q[0, 0, 0] = 1.0
    out = orc.sparse_mla_attention(_bf16_bits(q), cache, 1, 2, 2,
                                   np.array([[0, 1]], dtype=np.int32), np.log(3.0))
    assert abs(out[0, 0, 0] - 0.75) < 1e-15 and (out[0, 0, 1:] == 0).all()


def test_attention_hard_limit_and_order(orc=oracle):
    """A very large scale turns softmax into argmax: the output is the row
    with the largest exact dot product (found by brute force); listing the
    slots in another order gives the same output."""
    rng = np.random.default_rng(42)
    cache, v = _attn_cache(rng.standard_normal((32, 512)).astype(np.float32), orc)
    qf = rng.standard_normal((3, 2, 512)).astype(np.float32)
    q = _bf16_bits(qf)
    qd = (q.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    idx = np.stack([rng.permutation(32)[:20] for _ in range(3)]).astype(np.int32)
    for t in range(3):
        for h in range(2):
            dots = sorted(((float(qd[t, h] @ v[j]), j) for j in idx[t]), reverse=True)
            assert dots[0][0] - dots[1][0] > 1e-3
    out = orc.sparse_mla_attention(q, cache, 1, 32, 32, idx, 1e6)
    for t in range(3):
        for h in range(2):
            best = max(idx[t], key=lambda j: float(qd[t, h] @ v[j]))
            assert np.allclose(out[t, h], v[best], rtol=0, atol=1e-12)
    out1 = orc.sparse_mla_attention(q, cache, 1, 32, 32, idx, 0.05)
    out2 = orc.sparse_mla_attention(q, cache, 1, 32, 32, idx[:, ::-1].copy(), 0.05)
    assert np.allclose(out1, out2, rtol=0, atol=1e-12)   # values are O(1)
    assert not np.allclose(out1[0, 0], out1[0, 1])   # heads see their own queries
