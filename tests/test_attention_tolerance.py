"""The attention parity tolerance (tests/attn_tolerance.py) checked on the
CPU: an emulation of the kernel's roundings stays within it on the GPU
tests' inputs, and a rounding coarser than the kernel's does not.

The emulation follows the one-pass kernel's arithmetic: fp32 scores summed
over 32-dim chunks; c = |scale| * log2 e rounded to fp32 (1 for a zero
scale, the query negated for a negative one); the scaled maximum fl(c m);
each weight 2^fma(x, c, -fl(c m)) in fp32, with results below 2^-126
flushed to zero as the hardware exp2 does; the sink folded into the fp32
weight sum; bf16 weights in the fp32 weighted sum over 32-key chunks; one
division per row; the bf16 output.  It does not model the running
maximum's slack or the order of the MFMA's additions, which the
tolerance's terms bound separately."""

import numpy as np
import pytest

import oracle
import workloads
from tests.attn_tolerance import dequant_rows, tolerance

LOG2E = np.float32(1.4426950408889634)
TINY = np.float32(2.0 ** -126)


def f32(x):
    return np.asarray(x, dtype=np.float32)


def bf16_round(x: np.ndarray, mantissa_bits: int = 7) -> np.ndarray:
    """Round fp32 to `mantissa_bits` stored bits (7 = bf16), nearest-even."""
    u = f32(x).view(np.uint32).astype(np.uint64)
    drop = 23 - mantissa_bits
    u = ((u + (1 << (drop - 1)) - 1 + ((u >> drop) & 1)) >> drop) << drop
    return u.astype(np.uint32).view(np.float32)


def exp2_flushed(x: np.ndarray) -> np.ndarray:
    p = f32(np.exp2(np.asarray(x, dtype=np.float64)))
    return np.where(p < TINY, np.float32(0.0), p)


def emulate(case: workloads.AttnCase, weight_bits: int = 7) -> np.ndarray:
    q = workloads.bf16_bits_to_f32(case.q)                               # [T, H, D]
    c = np.float32(case.scale * 1.4426950408889634)
    if c == 0.0:
        q, c = np.zeros_like(q), np.float32(1.0)
    elif c < 0.0:
        q, c = -q, -c
    t_n, h_n, d_n = q.shape
    out = np.zeros((t_n, h_n, d_n), dtype=np.float64)
    for t in range(t_n):
        idx = case.indices[t]
        good = (idx >= 0) & (idx < case.num_blocks * case.block_size)
        if not good.any():
            continue
        v = f32(dequant_rows(case.cache, case.num_blocks, case.block_size, case.block_stride_rows, idx[good]))
        s = np.zeros((h_n, v.shape[0]), dtype=np.float32)
        for b in range(0, d_n, 32):
            s = f32(s + f32(q[t][:, b:b + 32] @ v[:, b:b + 32].T))
        mref = f32(s.max(axis=1) * c)
        arg = f32(s.astype(np.float64) * np.float64(c) - mref[:, None].astype(np.float64))
        p = exp2_flushed(arg)
        lsum = np.zeros(h_n, dtype=np.float32)
        for j in range(p.shape[1]):
            lsum = f32(lsum + p[:, j])
        sc = np.ones(h_n, dtype=np.float32)
        if case.sink is not None:
            s2 = f32(f32(case.sink) * LOG2E)
            mf = np.maximum(mref, s2)
            sc = exp2_flushed(f32(mref - mf))
            lsum = f32(f32(lsum * sc) + exp2_flushed(f32(s2 - mf)))
        pb = bf16_round(p, weight_bits)
        o = np.zeros((h_n, d_n), dtype=np.float32)
        for k in range(0, p.shape[1], 32):
            o = f32(o + f32(pb[:, k:k + 32] @ v[k:k + 32]))
        inv = f32(sc / lsum)
        out[t] = bf16_round(f32(o * inv[:, None]))
    return out


def wide_range_case() -> workloads.AttnCase:
    """The GPU tests' wide-range query: values times 2^k, k in [-30, 6], a
    block of bf16 subnormals and a zero head."""
    case = workloads.attention_case(4, 32, 200, 31, sink=True)
    rng = np.random.default_rng(131)
    qf = workloads.bf16_bits_to_f32(case.q)
    qf = qf * np.exp2(rng.integers(-30, 7, size=qf.shape)).astype(np.float32)
    qf[:, 3, 64:96] = rng.standard_normal((4, 32)).astype(np.float32) * np.float32(2.0 ** -130)
    qf[:, 5, :] = 0.0
    case.q = workloads.f32_to_bf16_bits(qf.astype(np.float32))
    return case


def cases():
    yield "one tile", workloads.attention_case(4, 16, 64, 1)
    yield "ragged, sinks", workloads.attention_case(5, 32, 200, 3, sink=True)
    yield "sharp, paged", workloads.attention_case(4, 32, 300, 6, num_blocks=40, block_size=48,
                                                   block_stride_rows=80, score_std=12.0, sink=True)
    neg = workloads.attention_case(5, 32, 200, 21, sink=True)
    neg.scale = -neg.scale
    yield "negative scale", neg
    zero = workloads.attention_case(5, 32, 200, 21, sink=True)
    zero.scale = 0.0
    yield "zero scale", zero
    yield "wide-range query", wide_range_case()


def worst_ratio(case, weight_bits=7):
    want = oracle.sparse_mla_attention(case.q, case.cache, case.num_blocks, case.block_size,
                                       case.block_stride_rows, case.indices, case.scale, case.sink)
    got = emulate(case, weight_bits)
    tol = tolerance(case.q, case.cache, case.num_blocks, case.block_size, case.block_stride_rows,
                    case.indices, case.scale, case.sink, want)
    return float((np.abs(got - want) / np.maximum(tol, 1e-300)).max()), float(np.abs(got - want).max())


@pytest.mark.parametrize("name,case", list(cases()), ids=[n for n, _ in cases()])
def test_emulated_kernel_within_tolerance(name, case):
    ratio, err = worst_ratio(case)
    assert err > 0.0 or name == "zero scale", "the emulation should differ from the exact result"
    assert ratio < 1.0, (name, ratio)


def test_coarser_weights_exceed_tolerance():
    """The tolerance has teeth: weights rounded to 3 stored bits (a relative
    2^-4) instead of bf16's 7 leave it."""
    ratio, _ = worst_ratio(workloads.attention_case(5, 32, 200, 3, sink=True), weight_bits=3)
    assert ratio > 1.0, ratio
