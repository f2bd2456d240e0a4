"""GPU parity of the MXFP4 store (mxfp4_store through the C ABI) against the
CPU oracle: every byte of the cache buffer, canaries included, must match."""

import numpy as np
import pytest
import torch

import oracle
from mxfp4_paged_cache_store_amd import ops, workloads
from tests.gpu_util import bf16_dev, first_mismatch, i64_dev, log, oracle_threads, u8_dev

pytestmark = pytest.mark.gpu


def run_both(device, src_bits, slots, num_blocks, block_size, stride_rows, cache_bytes):
    """Store on the GPU and in the oracle from the same canary-filled buffer;
    return (gpu bytes, oracle bytes)."""
    host = np.full(cache_bytes, 0xA5, dtype=np.uint8)
    dev_cache = u8_dev(host, device)
    ops.mxfp4_store(bf16_dev(src_bits, device), i64_dev(slots, device), dev_cache,
                    num_blocks, block_size, stride_rows)
    torch.cuda.synchronize()
    got = dev_cache.cpu().numpy()
    oracle.mxfp4_store(src_bits, slots, host, num_blocks, block_size, stride_rows,
                       threads=oracle_threads())
    return got, host


def check_case(device, case: workloads.StoreCase):
    log(f"store {case.name}: {case.src.shape[0]} tokens, blocks={case.num_blocks} "
        f"B={case.block_size} stride={case.block_stride_rows}")
    got, want = run_both(device, case.src, case.slots, case.num_blocks, case.block_size,
                         case.block_stride_rows, case.cache_bytes)
    assert (got == want).all(), first_mismatch(got, want, 272)
    return got


def test_tiny(device):
    check_case(device, workloads.tiny_case())


def test_decode_paged_interleaved(device):
    check_case(device, workloads.decode_case())


def test_prefill_runs(device):
    check_case(device, workloads.prefill_case())


def test_solo_sweep_exhaustive(device):
    """All 65,536 bf16 patterns alone in a group."""
    src = np.zeros((4096, 512), dtype=np.uint16)
    src[:, ::32] = np.arange(65536, dtype=np.uint32).reshape(4096, 16).astype(np.uint16)
    slots = np.arange(4096, dtype=np.int64)
    log("store solo sweep")
    got, want = run_both(device, src, slots, 1, 4096, 4096, 4096 * 272)
    assert (got == want).all(), first_mismatch(got, want, 272)


@pytest.mark.parametrize("k", [0, 125, -126, 17, -100, 60])
def test_anchored_sweep(device, k):
    """Groups [6*2^k, x...] over every finite bf16 x with |x| <= 6*2^k, with
    the anchor at a varying lane position."""
    f = (np.arange(65536, dtype=np.uint32) << 16).view(np.float32)
    anchor = np.float32(6.0 * 2.0 ** k)  # exact
    cands = np.flatnonzero(np.isfinite(f) & (np.abs(f.astype(np.float64)) <= 6.0 * 2.0 ** k)).astype(np.uint16)
    abits = np.uint16(np.array([anchor], dtype=np.float32).view(np.uint32)[0] >> 16)
    per = 31
    ngroups = -(-cands.size // per)
    groups = np.zeros((ngroups, 32), dtype=np.uint16)
    body = np.zeros(ngroups * per, dtype=np.uint16)
    body[: cands.size] = cands
    body = body.reshape(ngroups, per)
    for gi in range(ngroups):
        pos = gi % 32
        row = np.insert(body[gi], pos, abits)
        groups[gi] = row
    ntok = -(-ngroups // 16)
    src = np.zeros((ntok * 16, 32), dtype=np.uint16)
    src[:ngroups] = groups
    src = src.reshape(ntok, 512)
    slots = np.arange(ntok, dtype=np.int64)
    log(f"store anchored sweep k={k}: {ntok} tokens")
    got, want = run_both(device, src, slots, 1, ntok, ntok, ntok * 272)
    assert (got == want).all(), first_mismatch(got, want, 272)


def test_extreme_scale_rows(device):
    rng = np.random.default_rng(11)
    x = rng.standard_t(2, size=(1000, 512)) * np.exp2(rng.uniform(-140, 126, size=(1000, 1)))
    with np.errstate(over="ignore", under="ignore"):
        xf = x.astype(np.float32)
    src = (xf.view(np.uint32) >> 16).astype(np.uint16)
    # sprinkle signed zeros, NaN and Inf into some groups
    src[::7, 5] = 0x8000
    src[3, 40] = 0x7F80
    src[5, 100] = 0xFF80
    src[9, 300] = 0x7FC0
    slots = rng.permutation(1000).astype(np.int64)
    log("store extreme-scale rows")
    got, want = run_both(device, src, slots, 1, 1000, 1000, 1000 * 272)
    assert (got == want).all(), first_mismatch(got, want, 272)


@pytest.mark.parametrize("latent", [128, 256, 1024, 2048])
@pytest.mark.parametrize("ntok", [1, 37, 1001])
def test_other_latents_ragged(device, latent, ntok):
    """Power-of-two latents other than 512, ragged token counts (partial
    waves and blocks), a non-power-of-two block with interleaved blocks, and
    a row-strided source (the first `latent` columns of a wider tensor)."""
    rng = np.random.default_rng(latent + ntok)
    wide = latent + 64
    x = rng.standard_normal((ntok, wide)) * np.exp2(rng.uniform(-10, 10, size=(ntok, 1)))
    src_wide = (x.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    nb, bs, stride = 50, 48, 100
    slots = rng.choice(nb * bs, ntok, replace=False).astype(np.int64)
    slots[rng.random(ntok) < 0.1] = -1
    pitch = latent // 2 + latent // 32
    cache_bytes = ((nb - 1) * stride + bs) * pitch
    host = np.full(cache_bytes, 0xA5, dtype=np.uint8)
    dev_cache = u8_dev(host, device)
    src_dev = bf16_dev(src_wide, device)[:, :latent]
    log(f"store latent={latent} ntok={ntok}")
    ops.mxfp4_store(src_dev, i64_dev(slots, device), dev_cache, nb, bs, stride)
    torch.cuda.synchronize()
    got = dev_cache.cpu().numpy()
    oracle.mxfp4_store(src_wide[:, :latent], slots, host, nb, bs, stride)
    assert (got == host).all(), first_mismatch(got, host, pitch)


def test_strided_source_and_pow2_paged(device):
    rng = np.random.default_rng(12)
    ntok = 3000
    src_wide = (rng.standard_normal((ntok, 576)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    nb, bs, stride = 64, 64, 160
    slots = rng.choice(nb * bs, ntok, replace=False).astype(np.int64)
    host = np.full(((nb - 1) * stride + bs) * 272, 0xA5, dtype=np.uint8)
    dev_cache = u8_dev(host, device)
    log("store strided source, pow2 paged")
    ops.mxfp4_store(bf16_dev(src_wide, device)[:, :512], i64_dev(slots, device), dev_cache, nb, bs, stride)
    torch.cuda.synchronize()
    got = dev_cache.cpu().numpy()
    oracle.mxfp4_store(src_wide[:, :512], slots, host, nb, bs, stride)
    assert (got == host).all(), first_mismatch(got, host, 272)


def test_bad_slots_write_nothing(device):
    rng = np.random.default_rng(13)
    src = (rng.standard_normal((64, 512)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    slots = np.array([-1, -7, 100, 101, 10**12, -(2**62)] + list(range(58)), dtype=np.int64)
    log("store bad slots")
    got, want = run_both(device, src, slots, 1, 100, 100, 100 * 272)
    assert (got == want).all(), first_mismatch(got, want, 272)
    assert (got.reshape(100, 272)[58:] == 0xA5).all()


def test_empty_batch_launches_nothing(device):
    cache = torch.full((10 * 272,), 0xA5, dtype=torch.uint8, device=device)
    src = torch.zeros((0, 512), dtype=torch.bfloat16, device=device)
    ops.mxfp4_store(src, torch.zeros(0, dtype=torch.int64, device=device), cache, 1, 10, 10)
    torch.cuda.synchronize()
    assert (cache == 0xA5).all()


def test_page_api_views(device):
    """store_mxfp4_mla resolves a 3-D paged view (block stride > block) and a
    flat view exactly as the store page's wrapper does."""
    rng = np.random.default_rng(14)
    src = (rng.standard_normal((40, 512)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    slots = rng.choice(6 * 16, 40, replace=False).astype(np.int64)
    backing = torch.full((6 * 48 * 272,), 0xA5, dtype=torch.uint8, device=device)
    view = backing.view(6, 48, 272)[:, 16:32, :]  # [6, 16, 272], block stride 48 rows
    log("store page API views")
    ops.store_mxfp4_mla(bf16_dev(src, device), i64_dev(slots, device), view)
    torch.cuda.synchronize()
    got = backing.cpu().numpy()
    host = np.full(6 * 48 * 272, 0xA5, dtype=np.uint8)
    oracle.mxfp4_store(src, slots, host[16 * 272:], 6, 16, 48)
    assert (got == host).all(), first_mismatch(got, host, 272)

    flat = torch.full((96 * 272,), 0xA5, dtype=torch.uint8, device=device)
    ops.store_mxfp4_mla(bf16_dev(src, device), i64_dev(slots, device), flat)
    torch.cuda.synchronize()
    host = np.full(96 * 272, 0xA5, dtype=np.uint8)
    oracle.mxfp4_store(src, slots, host, 1, 96, 96)
    assert (flat.cpu().numpy() == host).all()


def test_large_int64_addressing(device):
    """4.5M tokens x 512 (2.3e9 values, past 2^31), random-permutation slots
    into a flat 1.224 GB cache, compared byte for byte with the oracle; run
    in the launch configuration the benchmark times."""
    n = workloads.LARGE_TOKENS
    log(f"store large: {n} tokens (generating on device)")
    src, slots = workloads.large_case_device(n)
    cache = torch.full((n * 272,), 0xA5, dtype=torch.uint8, device=device)
    ops.mxfp4_store(src, slots, cache, 1, n, n)
    torch.cuda.synchronize()
    log("store large: copying back and running the oracle")
    got = cache.cpu().numpy()
    del cache
    src_host = src.view(torch.int16).cpu().numpy().view(np.uint16)
    slots_host = slots.cpu().numpy()
    del src, slots
    torch.cuda.empty_cache()
    want = np.full(n * 272, 0xA5, dtype=np.uint8)
    oracle.mxfp4_store(src_host, slots_host, want, 1, n, n, threads=oracle_threads())
    assert (got == want).all(), first_mismatch(got, want, 272)
    # tokens past 2^31 / 512 really were written (the permutation covers every slot)
    tail = slots_host[(1 << 31) // 512:]
    assert not (got.reshape(n, 272)[tail[:1000]] == 0xA5).all(axis=1).any()
