"""GPU parity of mxfp4_gather_dequant against the oracle (bit-exact bf16)."""

import numpy as np
import pytest
import torch

import oracle
import workloads
from mxfp4_paged_cache_store_amd import ops
from tests.gpu_util import bf16_dev, bf16_host, first_mismatch, i64_dev, log, oracle_threads, u8_dev

pytestmark = pytest.mark.gpu


def test_all_code_scale_pairs(device):
    """Every (code, scale byte) pair: 256 rows, row b holds scale byte b in
    every group and the 16 codes repeated, so all 4,096 products appear."""
    rows = np.zeros((256, 272), dtype=np.uint8)
    codes = np.arange(16, dtype=np.uint8)
    pairs = (codes[0::2] | (codes[1::2] << 4)).astype(np.uint8)  # 8 bytes = 16 codes
    rows[:, :256] = np.tile(pairs, 32)
    rows[:, 256:] = np.arange(256, dtype=np.uint8)[:, None]
    cache = rows.reshape(-1)
    slots = np.arange(256, dtype=np.int64)
    out = torch.full((256, 512), 0x1234, dtype=torch.int16, device=device).view(torch.bfloat16)
    log("dequant: all code x scale pairs")
    ops.mxfp4_gather_dequant(u8_dev(cache, device), 1, 256, 256, 512, i64_dev(slots, device), out)
    torch.cuda.synchronize()
    got = bf16_host(out)
    want = oracle.mxfp4_gather_dequant(cache, 1, 256, 256, 512, slots)
    assert (got == want).all(), first_mismatch(got, want, 512)


def test_prefill_round_trip(device):
    """Store the prefill chunk, then gather every valid slot back to bf16."""
    case = workloads.prefill_case()
    dev_cache = u8_dev(case.fresh_cache(), device)
    log("dequant: prefill store + gather")
    ops.mxfp4_store(bf16_dev(case.src, device), i64_dev(case.slots, device), dev_cache,
                    case.num_blocks, case.block_size, case.block_stride_rows)
    n = case.gather_slots.size
    out = torch.empty((n, 512), dtype=torch.bfloat16, device=device)
    ops.mxfp4_gather_dequant(dev_cache, case.num_blocks, case.block_size, case.block_stride_rows,
                             512, i64_dev(case.gather_slots, device), out)
    torch.cuda.synchronize()
    got = bf16_host(out)
    host = case.fresh_cache()
    oracle.mxfp4_store(case.src, case.slots, host, case.num_blocks, case.block_size,
                       case.block_stride_rows, threads=oracle_threads())
    want = oracle.mxfp4_gather_dequant(host, case.num_blocks, case.block_size,
                                       case.block_stride_rows, 512, case.gather_slots)
    assert (got == want).all(), first_mismatch(got, want, 512)


@pytest.mark.parametrize("latent", [128, 256, 512, 1024, 2048])
@pytest.mark.parametrize("n", [333, 5001])
def test_latents_paged_bad_slots_strided_out(device, latent, n):
    """Every latent, paged with interleaved blocks, random slots with bad
    ones, a strided output; 5,001 slots run the two-slots-per-wave kernel."""
    rng = np.random.default_rng(latent + n)
    pitch = latent // 2 + latent // 32
    nb, bs, stride = 20, 48, 70
    cache = rng.integers(0, 256, size=((nb - 1) * stride + bs) * pitch, dtype=np.uint8)
    slots = rng.integers(-3, nb * bs + 3, size=n).astype(np.int64)
    out_host = np.full((n, latent + 16), 0x5555, dtype=np.uint16)
    out_dev = bf16_dev(out_host, device)
    log(f"dequant latent={latent} n={n}")
    ops.mxfp4_gather_dequant(u8_dev(cache, device), nb, bs, stride, latent, i64_dev(slots, device),
                             out_dev[:, :latent])
    torch.cuda.synchronize()
    got = bf16_host(out_dev)
    want = out_host.copy()
    sub = np.ascontiguousarray(want[:, :latent])
    oracle.mxfp4_gather_dequant(cache, nb, bs, stride, latent, slots, sub)
    want[:, :latent] = sub
    assert (got == want).all(), first_mismatch(got, want, latent + 16)
