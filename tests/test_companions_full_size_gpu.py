"""GPU parity of the companion kernels at the sizes and in the launch
configuration the benchmark times them: the RoPE inserts over 1,048,576
tokens at compress ratio 1, gather-dequant of 4,500,000 slots, and the ring
save of 262,144 rows.  Where the oracle cannot redo the whole batch in
seconds, sampled outputs are recomputed one by one from the same inputs."""

import numpy as np
import pytest
import torch

import oracle
import workloads
from mxfp4_paged_cache_store_amd import ops
from tests.gpu_util import bf16_host, first_mismatch, log

pytestmark = pytest.mark.gpu

# value bytes and scale bytes per record, by format
RECORDS = {
    "mxfp8": (ops.mxfp8_rope_store, oracle.mxfp8_rope_store, 528, 512, 16),
    "nvfp4": (ops.nvfp4_rope_store, oracle.nvfp4_rope_store, 288, 256, 32),
    "v4": (ops.v4_rope_store, oracle.v4_rope_store, 584, 576, 8),
}


def record_bytes(pages: np.ndarray, slots: np.ndarray, block: int, vw: int, sw: int) -> np.ndarray:
    """[len(slots), vw + sw]: each slot's value bytes then its scale bytes,
    from pages [num_blocks, block * (vw + sw)]."""
    page, row = slots // block, slots % block
    v = pages[page[:, None], row[:, None] * vw + np.arange(vw)[None, :]]
    s = pages[page[:, None], block * vw + row[:, None] * sw + np.arange(sw)[None, :]]
    return np.concatenate([v, s], axis=1)


@pytest.mark.parametrize("variant", ["mxfp8", "nvfp4", "v4"])
def test_rope_insert_bandwidth_scale_sampled(device, variant):
    """Every token written (ratio 1) into a permutation of the slots; 4096
    sampled tokens, the first and the last included, against the oracle run
    on those tokens alone."""
    gpu_fn, orc_fn, width, vw, sw = RECORDS[variant]
    latent, positions, table, slots = workloads.rope_large_device()
    n = latent.shape[0]
    kv = torch.full((n // 64, 64, width), 0xA5, dtype=torch.uint8, device=device)
    log(f"rope {variant}: {n} tokens at ratio 1")
    gpu_fn(latent, positions, table, kv, slots, 1)
    torch.cuda.synchronize()
    rng = np.random.default_rng(8)
    idx = np.unique(np.concatenate([rng.choice(n, 4094, replace=False), [0, n - 1]]))
    idx_dev = torch.from_numpy(idx).to(device)
    lat_s = latent.index_select(0, idx_dev).view(torch.int16).cpu().numpy().view(np.uint16)
    pos_s = positions.index_select(0, idx_dev).cpu().numpy()
    slot_s = slots.index_select(0, idx_dev).cpu().numpy()
    k = idx.size
    nbc = -(-k // 64)
    host = np.full(nbc * 64 * width, 0xA5, dtype=np.uint8)
    orc_fn(lat_s, pos_s, table.cpu().numpy(), host, 64, nbc, np.arange(k, dtype=np.int64), 1)
    want = record_bytes(host.reshape(nbc, 64 * width), np.arange(k), 64, vw, sw)
    got = record_bytes(kv.view(n // 64, 64 * width).cpu().numpy(), slot_s, 64, vw, sw)
    assert (got == want).all(), first_mismatch(got, want, vw + sw)


def test_gather_dequant_bandwidth_scale_sampled(device):
    """All 4.5M slots of a flat cache of random bytes (2.3e9 output values,
    past 2^31) dequantized in one launch; 4096 sampled rows, the last ones
    included, against the oracle."""
    n = workloads.LARGE_TOKENS
    cache = workloads.random_cache_device(n)
    slots = torch.arange(n, dtype=torch.int64, device=device)
    out = torch.empty((n, 512), dtype=torch.bfloat16, device=device)
    log(f"gather-dequant: {n} slots")
    ops.mxfp4_gather_dequant(cache, 1, n, n, 512, slots, out)
    torch.cuda.synchronize()
    rng = np.random.default_rng(9)
    idx = np.unique(np.concatenate([rng.choice(n, 4090, replace=False), np.arange(n - 6, n)]))
    idx_dev = torch.from_numpy(idx).to(device)
    rows = cache.view(n, 272).index_select(0, idx_dev).cpu().numpy().reshape(-1)
    got = bf16_host(out.index_select(0, idx_dev))
    k = idx.size
    want = oracle.mxfp4_gather_dequant(rows, 1, k, k, 512, np.arange(k, dtype=np.int64))
    assert (got == want).all(), first_mismatch(got, want, 512)


def test_ring_save_bandwidth_scale(device):
    """262,144 rows of 1024 fp32 to distinct random slots of an 8192 x 32
    ring (1 GiB each side), the whole ring compared bit for bit; untouched
    ring rows keep their canary."""
    rows, slots, shape = workloads.ring_large_device()
    canary = 1.5
    ring = torch.full(shape, canary, dtype=torch.float32, device=device)
    log(f"save_ring_rows: {rows.shape[0]} rows into {shape}")
    ops.save_ring_rows(rows, slots, ring)
    torch.cuda.synchronize()
    got = ring.cpu().numpy()
    del ring
    rows_host = rows.cpu().numpy()
    slots_host = slots.cpu().numpy()
    want = np.full(shape, canary, dtype=np.float32)
    oracle.save_ring_rows(rows_host, slots_host, want)
    assert (got.view(np.uint32) == want.view(np.uint32)).all(), np.argwhere(got != want)[:5]
