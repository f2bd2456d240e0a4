"""GPU parity of fused_save_compress_norm_cr1 (compress ratio 1: RMSNorm of
each valid fp32 row with a bf16 weight) against the oracle's double-precision
result.

Tolerance, derived from the arithmetic: the kernel works in fp32 (squares, a
sum of 512 terms in 8 sequential steps and 6 tree levels, a divide by 512, +eps,
a correctly rounded sqrt and division, two products), a relative error below
about 14 + 0.5 + 7.5 + 1 + 2 = 25 units of 2^-24, i.e. under 2^-19.  Before the
final bf16 rounding that is under 256 * 2^-19 = 2^-11 of a bf16 ulp, so each
output must be the round-to-nearest-even of the exact value, except within
2^-10 ulp of a midpoint, where either neighbour is accepted.  Rows of tokens
with a negative slot must stay untouched (bit-for-bit canaries)."""

import numpy as np
import pytest
import torch

import oracle
from mxfp4_paged_cache_store_amd import ops
from tests.exact_ref import check_bf16_rounding
from tests.gpu_util import bf16_dev, i64_dev, log

pytestmark = pytest.mark.gpu

CANARY = 0x7FA5  # a NaN pattern the kernel never writes


def f32_dev(a, device):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int32)).to(device).view(torch.float32)


def weight_bits(rng) -> np.ndarray:
    w = (0.8 + 0.5 * rng.standard_normal(512)).astype(np.float32)
    return torch.from_numpy(w).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def run_case(device, kv_backing, slots, w_bits, eps, out_pad=0):
    """Launch on the first 512 columns of the fp32 rows ``kv_backing``; the
    output rows are ``out_pad`` bf16 wider than 512, all canaries first."""
    n = slots.size
    kv_dev = f32_dev(kv_backing, device)[:, :512]
    out_backing = torch.full((n, 512 + out_pad), CANARY, dtype=torch.int16, device=device)
    out_dev = out_backing.view(torch.bfloat16)[:, :512]
    log(f"compress_norm_cr1 n={n} eps={eps} kv_stride={kv_dev.stride(0)} out_stride={out_dev.stride(0)}")
    ops.fused_save_compress_norm_cr1(kv_dev, i64_dev(slots, device), bf16_dev(w_bits, device), eps, out_dev)
    torch.cuda.synchronize()
    got = out_backing.cpu().numpy().view(np.uint16)
    return got


def check(got, kv_host, slots, w_bits, eps, out_pad=0):
    want = oracle.rmsnorm_cr1(kv_host, slots, w_bits, eps)
    valid = slots >= 0
    assert (got[~valid] == CANARY).all(), "row of an invalid token was written"
    if out_pad:
        assert (got[:, 512:] == CANARY).all(), "padding was written"
    if valid.any():
        return check_bf16_rounding(got[valid, :512], want[valid])
    return 0


@pytest.mark.parametrize("n,kv_pad,out_pad,eps,seed", [
    (1, 0, 0, 1e-6, 0),
    (1000, 0, 0, 1e-6, 1),          # ragged: 1000 = 125 blocks of 8 tokens
    (16384, 0, 0, 1e-6, 2),         # the insert workload's batch
    (3001, 16, 8, 1e-5, 3),         # strided rows in and out
    (777, 4, 4, 0.0, 4),
])
def test_compress_norm_parity(device, n, kv_pad, out_pad, eps, seed):
    rng = np.random.default_rng(seed)
    backing = (rng.standard_normal((n, 512 + kv_pad)) *
               np.exp2(rng.uniform(-20, 20, (n, 1)))).astype(np.float32)
    kv_host = backing[:, :512]
    slots = np.arange(n, dtype=np.int64)
    slots[rng.random(n) < 0.1] = -1
    w = weight_bits(rng)
    got = run_case(device, backing, slots, w, eps, out_pad)
    near = check(got, kv_host, slots, w, eps, out_pad)
    assert near <= max(16, got.size // 100)


def test_compress_norm_special_rows(device):
    """Zero rows (with and without eps), constant rows, huge and tiny
    scales, an infinity and a NaN in a row, and the sign of zero."""
    rng = np.random.default_rng(11)
    kv = rng.standard_normal((12, 512)).astype(np.float32)
    kv[0] = 0.0
    kv[1] = -0.0
    kv[2] = 0.75
    kv[3] = -3.0
    kv[4] *= np.float32(2.0 ** 55)
    kv[5] *= np.float32(2.0 ** -55)
    kv[6, 100] = np.inf
    kv[7, 3] = np.nan
    kv[8, ::2] = 0.0
    kv[8, 1::2] = -1.0
    w = weight_bits(rng)
    w[5] = 0x8000   # -0.0 weight
    w[6] = 0x0000
    slots = np.arange(12, dtype=np.int64)
    slots[11] = -5
    for eps in (1e-6, 0.0):
        got = run_case(device, kv, slots, w, eps)
        check(got, kv, slots, w, eps)


def test_compress_norm_empty(device):
    kv = torch.zeros((4, 512), dtype=torch.float32, device=device)
    out = torch.full((4, 512), 1.0, dtype=torch.bfloat16, device=device)
    w = torch.ones(512, dtype=torch.bfloat16, device=device)
    ops.fused_save_compress_norm_cr1(kv, torch.empty(0, dtype=torch.int64, device=device), w, 1e-6, out)
    torch.cuda.synchronize()
    assert (out == 1.0).all()


def test_compress_norm_large_sampled(device):
    """2,097,152 tokens (4 GiB of fp32 rows; the launch the benchmark
    times), 1% invalid: 4,096 sampled rows checked against the oracle, and
    every invalid row checked for its canary."""
    n = 1 << 21
    g = torch.Generator(device=device)
    g.manual_seed(21)
    kv = torch.randn((n, 512), generator=g, device=device, dtype=torch.float32)
    kv *= torch.exp2(torch.empty((n, 1), device=device).uniform_(-20, 20, generator=g))
    slots = torch.arange(n, dtype=torch.int64, device=device)
    slots[torch.rand(n, generator=g, device=device) < 0.01] = -1
    w = weight_bits(np.random.default_rng(21))
    out = torch.full((n, 512), CANARY, dtype=torch.int16, device=device)
    log(f"compress_norm_cr1 large n={n}")
    ops.fused_save_compress_norm_cr1(kv, slots, bf16_dev(w, device), 1e-6, out.view(torch.bfloat16))
    torch.cuda.synchronize()
    invalid = slots < 0
    assert (out[invalid] == CANARY).all()
    rng = np.random.default_rng(22)
    pick = np.sort(rng.choice(n, 4096, replace=False))
    pick_dev = torch.from_numpy(pick).to(device)
    kv_s = kv[pick_dev].cpu().numpy()
    slots_s = slots[pick_dev].cpu().numpy()
    got = out[pick_dev].cpu().numpy().view(np.uint16)
    want = oracle.rmsnorm_cr1(kv_s, slots_s, w, 1e-6)
    valid = slots_s >= 0
    check_bf16_rounding(got[valid], want[valid])
    assert (got[~valid] == CANARY).all()


@pytest.mark.parametrize("seed", range(24))
def test_compress_norm_random_geometry(device, seed):
    """Seeded random batches: token counts (0-20,000, ragged), row padding of
    the fp32 input and the bf16 output, epsilon, the share of invalid tokens
    (negative slots), row magnitudes over 2^+-50, and rows that are all
    zeros.  (Rows whose fp32 sum of squares overflows, from magnitudes of
    about 2^59 up, are outside the fp32 arithmetic this kernel shares with the
    pages' and outside the derived tolerance.)"""
    rng = np.random.default_rng(6000 + seed)
    n = int(rng.choice([0, 1, 7, 8, 9, 513, 4096, 20_000]))
    kv_pad, out_pad = int(rng.choice([0, 4, 12])), int(rng.choice([0, 8]))
    eps = float(rng.choice([0.0, 1e-6, 1e-5, 1e-2]))
    backing = (rng.standard_normal((n, 512 + kv_pad)) *
               np.exp2(rng.uniform(-50, 50, (n, 1)))).astype(np.float32)
    if n:
        backing[rng.random(n) < 0.05] = 0.0
    slots = np.arange(n, dtype=np.int64)
    slots[rng.random(n) < float(rng.choice([0.0, 0.1, 0.9]))] = -1
    w = weight_bits(rng)
    log(f"random norm seed={seed}: n={n} kv_pad={kv_pad} out_pad={out_pad} eps={eps}")
    got = run_case(device, backing, slots, w, eps, out_pad)
    near = check(got, backing[:, :512], slots, w, eps, out_pad)
    assert near <= max(16, got.size // 100)
