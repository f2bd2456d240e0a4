"""The norm's GPU criterion (each output the nearest-even bf16 of the exact
value, either neighbour within 2^-10 ulp of a midpoint:
tests/exact_ref.check_bf16_rounding) checked on the CPU against an emulation
of the kernel's fp32 arithmetic, and shown to reject a coarser one.

The emulation follows fused_save_compress_norm_cr1's kernel: squares in
fp32, each lane's 8 values (4l..4l+3 and 256+4l..256+4l+3) summed in
order, the 64 lane sums reduced by mirror adds, the divide by 512, + eps, a
correctly rounded sqrt and reciprocal, then (x * r) * w rounded to bf16."""

import numpy as np
import pytest

import oracle
import workloads
from tests.exact_ref import check_bf16_rounding

LANE_VALUES = np.concatenate([np.arange(4)[None, :] + 4 * np.arange(64)[:, None],
                              256 + np.arange(4)[None, :] + 4 * np.arange(64)[:, None]], axis=1)


def f32(x):
    return np.asarray(x, dtype=np.float32)


def round_bits(x: np.ndarray, mantissa_bits: int) -> np.ndarray:
    """fp32 rounded to `mantissa_bits` stored bits, nearest-even (23: as is)."""
    if mantissa_bits >= 23:
        return f32(x)
    u = f32(x).view(np.uint32).astype(np.uint64)
    drop = 23 - mantissa_bits
    u = ((u + (1 << (drop - 1)) - 1 + ((u >> drop) & 1)) >> drop) << drop
    return u.astype(np.uint32).view(np.float32)


def emulate(kv: np.ndarray, w_bits: np.ndarray, eps: float, r_bits: int = 23) -> np.ndarray:
    x = f32(kv)
    w = workloads.bf16_bits_to_f32(w_bits)
    sq = f32(x * x)
    part = sq[:, LANE_VALUES[:, 0]]
    for k in range(1, 8):
        part = f32(part + sq[:, LANE_VALUES[:, k]])
    while part.shape[1] > 1:
        half = part.shape[1] // 2
        part = f32(part[:, :half] + part[:, half:][:, ::-1])
    mean = f32(part[:, 0] / np.float32(512.0))
    rms = np.sqrt(f32(mean + np.float32(eps)))
    r = round_bits(f32(np.float32(1.0) / rms), r_bits)
    y = f32(f32(x * r[:, None]) * w[None, :])
    return workloads.f32_to_bf16_bits(y)


def rows(seed: int, n: int) -> np.ndarray:
    rng = np.random.default_rng(seed)
    kv = (rng.standard_normal((n, 512)) * np.exp2(rng.uniform(-20, 20, (n, 1)))).astype(np.float32)
    kv[0] = 0.0                                                  # a zero row: eps alone
    kv[1] = np.float32(2.0 ** -60) * rng.standard_normal(512).astype(np.float32)
    kv[2, ::2] = 0.0                                             # half the row zero
    return kv


def weights(seed: int) -> np.ndarray:
    rng = np.random.default_rng(seed)
    w = (0.8 + 0.5 * rng.standard_normal(512)).astype(np.float32)
    return workloads.f32_to_bf16_bits(w)


@pytest.mark.parametrize("n,eps,seed", [(1000, 1e-6, 1), (777, 0.0, 4), (500, 1e-5, 7)])
def test_emulated_kernel_meets_the_criterion(n, eps, seed):
    kv, w = rows(seed, n), weights(seed)
    if eps == 0.0:
        kv[0] = 1.0                                              # no zero row without eps
    slots = np.arange(n, dtype=np.int64)
    want = oracle.rmsnorm_cr1(kv, slots, w, eps)
    near = check_bf16_rounding(emulate(kv, w, eps), want)
    assert near <= max(16, kv.size // 100), near


def test_coarser_arithmetic_fails_the_criterion():
    """The criterion has teeth: the reciprocal rounded to 15 bits instead of
    fp32's 23 (a relative 2^-16) breaks it."""
    kv, w = rows(1, 1000), weights(1)
    slots = np.arange(1000, dtype=np.int64)
    want = oracle.rmsnorm_cr1(kv, slots, w, 1e-6)
    with pytest.raises(AssertionError):
        check_bf16_rounding(emulate(kv, w, 1e-6, r_bits=15), want)
