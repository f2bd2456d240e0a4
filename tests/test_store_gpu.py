"""GPU parity of the MXFP4 store (mxfp4_store through the C ABI) against the
CPU oracle: every byte of the cache buffer, canaries included, must match."""

import numpy as np
import pytest
import torch

import oracle
import workloads
from mxfp4_paged_cache_store_amd import ops
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


def anchored_groups(k):
    """Groups of 32 bf16 patterns [6*2^k, x...] over every finite bf16 x with
    |x| <= 6*2^k (scale exponent k), the anchor at a varying lane position."""
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
        groups[gi] = np.insert(body[gi], gi % 32, abits)
    return groups


@pytest.mark.parametrize("k", [16, 17])
def test_mixed_scale_exponents_in_a_wave(device, k):
    """Tokens whose groups alternate between scale exponents k - 16 .. k and
    k + 1 (every finite bf16 below each anchor): a wave's groups take both
    encodings (up to e = 16 from the packed bf16 values, above from fp32
    quotients), including the boundary e = 16 / 17."""
    lo, hi = anchored_groups(k - 16), anchored_groups(k + 1)
    mid = anchored_groups(k)
    n = min(lo.shape[0], hi.shape[0], mid.shape[0]) // 8 * 8
    groups = np.empty((3 * n, 32), dtype=np.uint16)
    groups[0::3], groups[1::3], groups[2::3] = lo[:n], hi[:n], mid[:n]
    ntok = groups.shape[0] // 16
    src = groups[: ntok * 16].reshape(ntok, 512)
    slots = np.random.default_rng(k).permutation(ntok).astype(np.int64)
    log(f"store mixed exponents k={k}: {ntok} tokens")
    got, want = run_both(device, src, slots, 1, ntok, ntok, ntok * 272)
    assert (got == want).all(), first_mismatch(got, want, 272)
    # the slot-order form quantizes the same way
    inv = ops.mxfp4_inverse_workspace(1, ntok, device)
    ops.mxfp4_build_inverse(i64_dev(slots, device), 1, ntok, inv)
    dev_cache = u8_dev(np.full(ntok * 272, 0xA5, dtype=np.uint8), device)
    ops.mxfp4_store_by_slot(bf16_dev(src, device), ntok, inv, dev_cache, 1, ntok, ntok)
    torch.cuda.synchronize()
    got = dev_cache.cpu().numpy()
    assert (got == want).all(), first_mismatch(got, want, 272)


@pytest.mark.parametrize("k", [0, 125, -126, 16, 17, -100, 60])
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
@pytest.mark.parametrize("ntok", [1, 37, 1001, 9001, 20001])
def test_other_latents_ragged(device, latent, ntok):
    """Power-of-two latents other than 512, ragged token counts (partial
    waves and blocks; 9,001 and 20,001 tokens run the two- and four-pass
    kernels), a non-power-of-two block with interleaved blocks, and a
    row-strided source (the first `latent` columns of a wider tensor)."""
    rng = np.random.default_rng(latent + ntok)
    wide = latent + 64
    x = rng.standard_normal((ntok, wide)) * np.exp2(rng.uniform(-10, 10, size=(ntok, 1)))
    src_wide = (x.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    nb, bs, stride = max(50, ntok // 40 + 10), 48, 100
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
    into a flat 1.224 GB cache, in both the scatter form and the slot-order
    form (the one the benchmark times), each compared byte for byte with the
    oracle."""
    n = workloads.LARGE_TOKENS
    log(f"store large: {n} tokens (generating on device)")
    src, slots = workloads.large_case_device(n)
    cache = torch.full((n * 272,), 0xA5, dtype=torch.uint8, device=device)
    ops.mxfp4_store(src, slots, cache, 1, n, n)
    torch.cuda.synchronize()
    got_scatter = cache.cpu().numpy()
    assert ops.mxfp4_slot_order_advised(n, 512, 1, n)
    inv = ops.mxfp4_inverse_workspace(1, n, device)
    cache.fill_(0xA5)
    log("store large: slot-order form")
    ops.mxfp4_build_inverse(slots, 1, n, inv)
    ops.mxfp4_store_by_slot(src, n, inv, cache, 1, n, n)
    torch.cuda.synchronize()
    got_slot_order = cache.cpu().numpy()
    del cache, inv
    log("store large: copying back and running the oracle")
    src_host = src.view(torch.int16).cpu().numpy().view(np.uint16)
    slots_host = slots.cpu().numpy()
    del src, slots
    torch.cuda.empty_cache()
    want = np.full(n * 272, 0xA5, dtype=np.uint8)
    oracle.mxfp4_store(src_host, slots_host, want, 1, n, n, threads=oracle_threads())
    assert (got_scatter == want).all(), first_mismatch(got_scatter, want, 272)
    assert (got_slot_order == want).all(), first_mismatch(got_slot_order, want, 272)
    # tokens past 2^31 / 512 really were written (the permutation covers every slot)
    tail = slots_host[(1 << 31) // 512:]
    assert not (want.reshape(n, 272)[tail[:1000]] == 0xA5).all(axis=1).any()


@pytest.mark.parametrize("latent,nb,bs,stride,ntok", [
    (512, 1000, 150, 200, 140_000),    # non-power-of-two block, interleaved blocks
    (512, 4096, 64, 64, 200_000),      # contiguous power-of-two blocks
    (512, 2048, 64, 96, 131_072),      # power-of-two block, interleaved
    (1024, 1100, 128, 128, 140_000),
])
def test_slot_order_form(device, latent, nb, bs, stride, ntok):
    """build_inverse + store_by_slot over dense scattered batches (with pads
    and out-of-range slots) writes the same bytes as the oracle; one inverse
    serves two layers that share the slot mapping.  (The library advises this
    form only for batches past 256 MiB of rows; it is correct at any size.)"""
    rng = np.random.default_rng(ntok + latent)
    num_slots = nb * bs
    slots = rng.choice(num_slots, ntok, replace=False).astype(np.int64)
    slots[rng.random(ntok) < 0.03] = -1
    slots[:5] = [num_slots, num_slots + 7, 10**13, -2, -(2**40)]
    pitch = latent // 2 + latent // 32
    inv = ops.mxfp4_inverse_workspace(nb, bs, device)
    log(f"store slot order latent={latent} nb={nb} bs={bs} stride={stride} ntok={ntok}")
    ops.mxfp4_build_inverse(i64_dev(slots, device), nb, bs, inv)
    for layer in range(2):
        x = rng.standard_normal((ntok, latent)) * np.exp2(rng.uniform(-12, 12, size=(ntok, 1)))
        src = (x.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
        host = np.full(((nb - 1) * stride + bs) * pitch, 0xA5, dtype=np.uint8)
        dev_cache = u8_dev(host, device)
        ops.mxfp4_store_by_slot(bf16_dev(src, device), ntok, inv, dev_cache, nb, bs, stride)
        torch.cuda.synchronize()
        got = dev_cache.cpu().numpy()
        oracle.mxfp4_store(src, slots, host, nb, bs, stride, threads=oracle_threads())
        assert (got == host).all(), (layer, first_mismatch(got, host, pitch))


def test_slot_order_row_writes(device):
    """The slot-order store assembles a wave's rows (4 slots) in LDS and writes
    them as 16-byte chunks when they are consecutive in a 16-byte-aligned
    cache; with a cache that is only 4-byte aligned, or a block of 10 slots (a
    wave's slots may straddle two blocks), it writes row by row.  All forms
    give the oracle's bytes, including skipped slots' canaries inside a chunk
    span."""
    rng = np.random.default_rng(77)
    for nb, bs, stride, base in ((200, 128, 128, 4), (900, 10, 14, 0), (300, 64, 64, 0), (700, 12, 20, 0)):
        num_slots = nb * bs
        ntok = num_slots * 3 // 4
        slots = rng.choice(num_slots, ntok, replace=False).astype(np.int64)
        slots[rng.random(ntok) < 0.05] = -1
        x = rng.standard_normal((ntok, 512)) * np.exp2(rng.uniform(-10, 10, size=(ntok, 1)))
        src = (x.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
        nbytes = ((nb - 1) * stride + bs) * 272
        host = np.full(nbytes, 0xA5, dtype=np.uint8)
        backing = u8_dev(np.full(nbytes + 16, 0xA5, dtype=np.uint8), device)
        dev_cache = backing[base: base + nbytes]
        inv = ops.mxfp4_inverse_workspace(nb, bs, device)
        log(f"store slot order rows: nb={nb} bs={bs} stride={stride} cache offset {base}")
        ops.mxfp4_build_inverse(i64_dev(slots, device), nb, bs, inv)
        ops.mxfp4_store_by_slot(bf16_dev(src, device), ntok, inv, dev_cache, nb, bs, stride)
        torch.cuda.synchronize()
        got = backing.cpu().numpy()
        oracle.mxfp4_store(src, slots, host, nb, bs, stride, threads=oracle_threads())
        assert (got[base: base + nbytes] == host).all(), first_mismatch(got[base: base + nbytes], host, 272)
        assert (got[:base] == 0xA5).all() and (got[base + nbytes:] == 0xA5).all()


def test_page_api_with_inverse(device):
    """store_mxfp4_mla with an inverse buffer: slot order for a dense batch
    past 256 MiB of rows, the scatter form (plain stores: the rows fit in the
    Infinity Cache) for a smaller one and for a sparse one; all match the
    oracle."""
    rng = np.random.default_rng(22)
    for ntok, nslots in ((1 << 20, 1 << 20), (1 << 17, 1 << 17), (140_000, 1 << 20)):
        # finite bf16 patterns of both signs, magnitudes 2^-31 .. 2^8
        src = rng.integers(0x3000, 0x4380, size=(ntok, 512), dtype=np.uint16)
        src |= (rng.integers(0, 2, size=(ntok, 512), dtype=np.uint16) << 15)
        slots = rng.choice(nslots, ntok, replace=False).astype(np.int64)
        assert ops.mxfp4_slot_order_advised(ntok, 512, 1, nslots) == (ntok == 1 << 20)
        inv = ops.mxfp4_inverse_workspace(1, nslots, device)
        cache = torch.full((nslots * 272,), 0xA5, dtype=torch.uint8, device=device)
        log(f"store page API with inverse: {ntok} tokens, {nslots} slots")
        ops.store_mxfp4_mla(bf16_dev(src, device), i64_dev(slots, device), cache, inverse=inv)
        torch.cuda.synchronize()
        host = np.full(nslots * 272, 0xA5, dtype=np.uint8)
        oracle.mxfp4_store(src, slots, host, 1, nslots, nslots, threads=oracle_threads())
        assert (cache.cpu().numpy() == host).all()


def test_inverse_map_contents(device):
    """The inverse map itself: -1 everywhere except at the batch's valid
    slots, which hold their token index; the map is the workspace's first
    num_slots int32 entries and nothing past it is written."""
    rng = np.random.default_rng(23)
    nb, bs, n = 37, 33, 900
    slots = rng.choice(nb * bs, n, replace=False).astype(np.int64)
    slots[::17] = -1
    slots[5] = nb * bs
    words = ops.mxfp4_inverse_bytes(nb, bs) // 4
    inv = torch.full((words + 4,), 12345, dtype=torch.int32, device=device)
    ops.mxfp4_build_inverse(i64_dev(slots, device), nb, bs, inv)
    torch.cuda.synchronize()
    want = np.full(nb * bs, -1, dtype=np.int32)
    ok = (slots >= 0) & (slots < nb * bs)
    want[slots[ok]] = np.flatnonzero(ok)
    got = inv.cpu().numpy()
    assert (got[: nb * bs] == want).all()
    assert (got[words:] == 12345).all()  # nothing past the map


def _check_map_with_duplicates(got, slots, num_slots):
    """Each slot named by some tokens holds one of them; the others hold -1."""
    ok = (slots >= 0) & (slots < num_slots)
    owners = {}
    for t in np.flatnonzero(ok):
        owners.setdefault(int(slots[t]), set()).add(int(t))
    named = np.zeros(num_slots, dtype=bool)
    named[list(owners)] = True
    assert (got[~named] == -1).all()
    for s_, toks in owners.items():
        assert int(got[s_]) in toks, (s_, int(got[s_]))


@pytest.mark.parametrize("case", ["one_range_full", "crowded", "more_tokens_than_slots"])
def test_inverse_map_ranges_and_duplicates(device, case):
    """A batch that fills one contiguous range of slots exactly; one whose
    700 tokens crowd onto 40 slots; and a batch with more tokens than slots
    (pads, duplicates, slots past the end): every named slot holds one of
    its tokens, every other slot -1."""
    rng = np.random.default_rng(24)
    nb, bs = 50, 40  # 2,000 slots
    ns = nb * bs
    if case == "one_range_full":
        slots = rng.permutation(np.arange(500, 750)).astype(np.int64)
    elif case == "crowded":
        slots = rng.integers(750, 790, size=700).astype(np.int64)
        slots[::50] = rng.integers(0, ns, size=14)
    else:
        slots = rng.integers(-2, ns + 3, size=5000).astype(np.int64)
    inv = ops.mxfp4_inverse_workspace(nb, bs, device)
    log(f"inverse map, {case}: {slots.size} tokens, {ns} slots")
    ops.mxfp4_build_inverse(i64_dev(slots, device), nb, bs, inv)
    torch.cuda.synchronize()
    got = inv[:ns].cpu().numpy()
    _check_map_with_duplicates(got, slots, ns)
    if case == "one_range_full":
        want = np.full(ns, -1, dtype=np.int32)
        want[slots] = np.arange(slots.size)
        assert (got == want).all()


def test_cache_extent_checked(device):
    """The C ABI gets only the cache pointer, so the binding refuses a paged
    geometry that reaches past the tensor (nothing is launched)."""
    nb, bs, stride = 4, 16, 24
    need = ((nb - 1) * stride + bs) * 272
    src = torch.zeros((8, 512), dtype=torch.bfloat16, device=device)
    slots = torch.arange(8, dtype=torch.int64, device=device)
    inv = ops.mxfp4_inverse_workspace(nb, bs, device)
    out = torch.empty((8, 512), dtype=torch.bfloat16, device=device)
    short = torch.full((need - 1,), 0xA5, dtype=torch.uint8, device=device)
    with pytest.raises(ValueError, match="cache holds"):
        ops.mxfp4_store(src, slots, short, nb, bs, stride)
    with pytest.raises(ValueError, match="cache holds"):
        ops.mxfp4_store_by_slot(src, 8, inv, short, nb, bs, stride)
    with pytest.raises(ValueError, match="cache holds"):
        ops.mxfp4_gather_dequant(short, nb, bs, stride, 512, slots, out)
    torch.cuda.synchronize()
    assert (short.cpu().numpy() == 0xA5).all()
    # exactly enough, also as the strided paged view of interleaved layers
    backing = torch.full((nb * stride * 272,), 0xA5, dtype=torch.uint8, device=device)
    view = backing.view(nb, stride, 272)[:, :bs, :]
    ops.mxfp4_store(src, slots, backing[:need], nb, bs, stride)
    ops.mxfp4_store(src, slots, view, nb, bs, stride)
    torch.cuda.synchronize()


def test_large_batch_ragged_generic_paging(device):
    """A batch past the 16,384-token switch (4 tokens per wave) with a ragged
    tail, a non-power-of-two block, interleaved blocks and scattered slots."""
    rng = np.random.default_rng(24)
    n, nb, bs, stride = 300_001, 3100, 100, 150
    x = rng.standard_normal((n, 512)) * np.exp2(rng.uniform(-30, 30, size=(n, 1)))
    src = (x.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    slots = rng.choice(nb * bs, n, replace=False).astype(np.int64)
    slots[rng.random(n) < 0.02] = -1
    log(f"store {n} tokens, B={bs}, stride={stride}")
    got, want = run_both(device, src, slots, nb, bs, stride, ((nb - 1) * stride + bs) * 272)
    assert (got == want).all(), first_mismatch(got, want, 272)


@pytest.mark.parametrize("pad", [0.5, 0.9, 1.0])
def test_pad_heavy_large_batch(device, pad):
    """Batches above 16,384 tokens request a token's row only once its slot
    is known: 70,001 tokens with half, nine tenths or all of them pads
    (negative, past the cache, -2^62), scattered into an interleaved paged
    cache -- every cache byte as the oracle's."""
    rng = np.random.default_rng(int(pad * 100) + 7)
    n, nb, bs, stride = 70_001, 1200, 64, 80
    x = rng.standard_normal((n, 512)) * np.exp2(rng.uniform(-20, 20, size=(n, 1)))
    src = (x.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    slots = rng.choice(nb * bs, n, replace=False).astype(np.int64)
    bad = rng.random(n) < pad
    slots[bad] = rng.choice(np.array([-1, -7, nb * bs, -(1 << 62)], dtype=np.int64), int(bad.sum()))
    log(f"store {n} tokens, pad fraction {pad}")
    got, want = run_both(device, src, slots, nb, bs, stride, ((nb - 1) * stride + bs) * 272)
    assert (got == want).all(), first_mismatch(got, want, 272)
