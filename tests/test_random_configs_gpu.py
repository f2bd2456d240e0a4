"""GPU parity over seeded random geometries: latent width, token count, block
size, block stride, pad share, slot pattern, source row stride and cache
alignment for the MXFP4 store (scatter and slot-order forms) and its
gather-dequant; compress ratio, block, page stride, table stride, positions
and sanitising for the three RoPE inserts.  Every cache byte and every
dequantized value is compared with the oracle's."""

import numpy as np
import pytest
import torch

import oracle
import workloads
from mxfp4_paged_cache_store_amd import ops
from tests.gpu_util import bf16_dev, bf16_host, first_mismatch, i64_dev, log, oracle_threads, u8_dev

pytestmark = pytest.mark.gpu


def _latent_rows(rng, n, width):
    x = rng.standard_normal((n, width)) * np.exp2(rng.uniform(-30, 30, size=(n, 1)))
    bits = (x.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    # a few exact zeros of both signs and tiny values in every batch
    k = max(1, bits.size // 500)
    flat = bits.reshape(-1)
    flat[rng.integers(0, flat.size, k)] = 0x8000
    flat[rng.integers(0, flat.size, k)] = 0x0000
    flat[rng.integers(0, flat.size, k)] = 0x8001
    return bits


@pytest.mark.parametrize("seed", range(96))
def test_store_and_dequant_random_geometry(device, seed):
    rng = np.random.default_rng(1000 + seed)
    latent = int(rng.choice([128, 256, 512, 512, 1024, 2048]))
    pitch = latent // 2 + latent // 32
    n = int(rng.choice([1, 63, 700, 5000, 9000, 17000, 40000]))
    bs = int(rng.choice([1, 16, 48, 64, 100, 128]))
    nb = max(1, -(-int(n * rng.uniform(1.0, 3.0)) // bs))
    stride = bs + int(rng.choice([0, 0, 1, 7, bs]))
    pad = float(rng.choice([0.0, 0.05, 0.5, 0.95]))
    pattern = rng.choice(["random", "runs"])
    if pattern == "runs" and nb * bs >= n:
        start = int(rng.integers(0, nb * bs - n + 1))
        slots = np.arange(start, start + n, dtype=np.int64)
    else:
        slots = rng.choice(nb * bs, n, replace=False).astype(np.int64)
    bad = rng.random(n) < pad
    slots[bad] = rng.choice(np.array([-1, -3, nb * bs, nb * bs + 5], dtype=np.int64), int(bad.sum()))
    extra = int(rng.choice([0, 8, 64]))
    src_wide = _latent_rows(rng, n, latent + extra)
    cache_bytes = ((nb - 1) * stride + bs) * pitch
    offset = int(rng.choice([0, 16]))  # cache base 16 B past an allocation boundary
    host = np.full(cache_bytes + offset, 0xA5, dtype=np.uint8)
    log(f"random store seed={seed}: latent={latent} n={n} nb={nb} bs={bs} stride={stride} pad={pad} "
        f"{pattern} extra={extra} offset={offset}")
    dev = u8_dev(host, device)
    view = dev[offset:]
    src_dev = bf16_dev(src_wide, device)[:, :latent]
    ops.mxfp4_store(src_dev, i64_dev(slots, device), view, nb, bs, stride)
    torch.cuda.synchronize()
    want = host.copy()
    sub = np.ascontiguousarray(want[offset:])
    oracle.mxfp4_store(src_wide[:, :latent], slots, sub, nb, bs, stride, threads=oracle_threads())
    want[offset:] = sub
    got = dev.cpu().numpy()
    assert (got == want).all(), first_mismatch(got, want, pitch)

    # the slot-order form on the same batch writes the same bytes
    if latent >= 512 and offset == 0:
        dev2 = u8_dev(host, device)
        inv = ops.mxfp4_inverse_workspace(nb, bs, device)
        ops.mxfp4_build_inverse(i64_dev(slots, device), nb, bs, inv)
        ops.mxfp4_store_by_slot(src_dev, n, inv, dev2, nb, bs, stride)
        torch.cuda.synchronize()
        got2 = dev2.cpu().numpy()
        assert (got2 == want).all(), first_mismatch(got2, want, pitch)

    # gather-dequant of the written slots and a few bad ones
    listed = np.concatenate([slots[:3000], np.array([-1, nb * bs], dtype=np.int64)])
    out_host = np.full((listed.size, latent + 8), 0x5555, dtype=np.uint16)
    out_dev = bf16_dev(out_host, device)
    ops.mxfp4_gather_dequant(view, nb, bs, stride, latent, i64_dev(listed, device), out_dev[:, :latent])
    torch.cuda.synchronize()
    want_dq = out_host.copy()
    part = np.ascontiguousarray(want_dq[:, :latent])
    oracle.mxfp4_gather_dequant(sub, nb, bs, stride, latent, listed, part)
    want_dq[:, :latent] = part
    got_dq = bf16_host(out_dev)
    assert (got_dq == want_dq).all(), first_mismatch(got_dq, want_dq, latent + 8)


VARIANTS = {
    "mxfp8": (ops.mxfp8_rope_store, oracle.mxfp8_rope_store, 528),
    "nvfp4": (ops.nvfp4_rope_store, oracle.nvfp4_rope_store, 288),
    "v4": (ops.v4_rope_store, oracle.v4_rope_store, 584),
}


@pytest.mark.parametrize("seed", range(60))
def test_rope_inserts_random_geometry(device, seed):
    rng = np.random.default_rng(2000 + seed)
    variant = ["mxfp8", "nvfp4", "v4"][seed % 3]
    gpu_fn, orc_fn, width = VARIANTS[variant]
    cr = int(rng.choice([1, 1, 2, 3, 4]))
    n = int(rng.choice([1, 300, 5000, 70000]))
    block = int(rng.choice([1, 16, 48, 64]))
    nb = max(1, -(-int(n * rng.uniform(1.0, 2.0)) // block))
    page_stride = -(-block * width // 16) * 16 + 16 * int(rng.choice([0, 1, 3]))  # a multiple of 16
    rows = int(rng.choice([4096, 65536]))
    cos_stride = int(rng.choice([64, 80]))
    sanitize = bool(rng.random() < 0.7)
    latent = _latent_rows(rng, n, 512)
    if not sanitize:
        latent[rng.integers(0, n, 3), rng.integers(0, 512, 3)] = 0x7FC0  # NaN
    positions = rng.integers(-2, rows + 2, n).astype(np.int64)
    slots = rng.choice(nb * block, n, replace=False).astype(np.int64)
    slots[rng.random(n) < 0.05] = -1
    table = np.full((rows, cos_stride), np.nan, dtype=np.float32)
    table[:, :64] = workloads.rope_cos_sin_table(rows=rows)
    host = np.full((nb + 1) * page_stride, 0xA5, dtype=np.uint8)
    log(f"random rope seed={seed}: {variant} cr={cr} n={n} block={block} nb={nb} page_stride={page_stride} "
        f"rows={rows} cos_stride={cos_stride} sanitize={sanitize}")
    backing = u8_dev(host, device)
    view = torch.as_strided(backing, (nb, block, width), (page_stride, width, 1))
    tdev = torch.from_numpy(table).to(device)[:, :64]
    gpu_fn(bf16_dev(latent, device), i64_dev(positions, device), tdev, view, i64_dev(slots, device), cr,
           sanitize)
    torch.cuda.synchronize()
    got = backing.cpu().numpy()
    orc_fn(latent, positions, table[:, :64], host, block, nb, slots, cr, sanitize,
           cache_block_stride=page_stride, threads=oracle_threads())
    assert (got == host).all(), first_mismatch(got, host)
