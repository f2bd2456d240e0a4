"""GPU parity of save_ring_rows against the oracle (bit-for-bit copies)."""

import numpy as np
import pytest
import torch

import oracle
from mxfp4_paged_cache_store_amd import ops
from tests.gpu_util import i64_dev, log

pytestmark = pytest.mark.gpu


def f32_dev(a, device):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int32)).to(device).view(torch.float32)


@pytest.mark.parametrize("n,nb,cap,width,pad", [
    (1, 1, 1, 1024, 0),
    (999, 200, 8, 1024, 0),         # the pages' width
    (5000, 300, 20, 1024, 64),      # padded ring rows and blocks (strided views)
    (200_000, 8192, 32, 1024, 0),   # a large batch
    (777, 150, 7, 260, 4),          # another width (generic path)
])
def test_save_ring_rows(device, n, nb, cap, width, pad):
    rng = np.random.default_rng(n + width)
    bits = rng.integers(0, 2**32, size=(n, width + pad), dtype=np.uint64).astype(np.uint32)
    bits[::11, 0] = 0x7FC0BEEF  # NaN payloads survive
    bits[::13, 1] = 0x80000000  # -0.0
    rows_host = bits.view(np.float32)[:, :width]
    slots = rng.choice(nb * cap, n, replace=False).astype(np.int64)
    slots[rng.random(n) < 0.1] = -1
    if n > 3:
        slots[:3] = [nb * cap, nb * cap + 5, -(2**40)]
    canary = np.frombuffer(np.uint32(0x3FC00000).tobytes(), dtype=np.float32)[0]  # 1.5
    backing = np.full((nb, cap + 1, width + pad), canary, dtype=np.float32)
    state_host = backing[:, :cap, :width]
    rows_dev = f32_dev(bits.view(np.float32), device)[:, :width]
    backing_dev = f32_dev(backing, device)
    state_dev = backing_dev[:, :cap, :width]
    log(f"save_ring_rows n={n} blocks={nb} capacity={cap} width={width}")
    ops.save_ring_rows(rows_dev, i64_dev(slots, device), state_dev)
    torch.cuda.synchronize()
    oracle.save_ring_rows(rows_host, slots, state_host)
    got = backing_dev.cpu().numpy().view(np.uint32)
    want = backing.view(np.uint32)
    assert (got == want).all(), np.argwhere(got != want)[:5]


@pytest.mark.parametrize("seed", range(24))
def test_save_ring_rows_random_geometry(device, seed):
    """Seeded random geometries: widths (multiples of 4 up to 2048), ring
    capacity and blocks, padded rows and blocks, row count, the share of
    skipped slots and slots in runs or scattered; every state byte against
    the oracle."""
    rng = np.random.default_rng(5000 + seed)
    width = 4 * int(rng.integers(1, 513))
    cap = int(rng.choice([1, 3, 8, 32, 100]))
    nb = int(rng.integers(1, 400))
    n = int(rng.integers(0, min(nb * cap, 20_000) + 1))
    rpad, bpad = int(rng.choice([0, 4, 16])), int(rng.choice([0, 1]))
    bits = rng.integers(0, 2**32, size=(n, width + rpad), dtype=np.uint64).astype(np.uint32)
    if rng.random() < 0.5:
        start = int(rng.integers(0, nb * cap - n + 1))
        slots = np.arange(start, start + n, dtype=np.int64)
    else:
        slots = rng.choice(nb * cap, n, replace=False).astype(np.int64)
    slots[rng.random(n) < float(rng.choice([0.0, 0.1, 0.7]))] = -1
    canary = np.frombuffer(np.uint32(0x3FC00000).tobytes(), dtype=np.float32)[0]
    backing = np.full((nb, cap + bpad, width + rpad), canary, dtype=np.float32)
    state_host = backing[:, :cap, :width]
    rows_dev = f32_dev(bits.view(np.float32), device)[:, :width]
    backing_dev = f32_dev(backing, device)
    state_dev = backing_dev[:, :cap, :width]
    log(f"random ring seed={seed}: n={n} blocks={nb} capacity={cap} width={width} pads={rpad},{bpad}")
    ops.save_ring_rows(rows_dev, i64_dev(slots, device), state_dev)
    torch.cuda.synchronize()
    oracle.save_ring_rows(bits.view(np.float32)[:, :width], slots, state_host)
    got = backing_dev.cpu().numpy().view(np.uint32)
    want = backing.view(np.uint32)
    assert (got == want).all(), np.argwhere(got != want)[:5]
