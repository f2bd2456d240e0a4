"""GPU parity of the MXFP8 / NVFP4 / V4 RoPE+quant inserts against the oracle:
every byte of the paged compressed cache, canaries included."""

import numpy as np
import pytest
import torch

import oracle
import workloads
from mxfp4_paged_cache_store_amd import ops
from tests.gpu_util import bf16_dev, first_mismatch, i64_dev, log, u8_dev

pytestmark = pytest.mark.gpu

VARIANTS = {
    "mxfp8": (ops.mxfp8_rope_store, oracle.mxfp8_rope_store, 528),
    "nvfp4": (ops.nvfp4_rope_store, oracle.nvfp4_rope_store, 288),
    "v4": (ops.v4_rope_store, oracle.v4_rope_store, 584),
}


def run_both(device, variant, latent, positions, table, slots, block, num_blocks, cr,
             sanitize=True):
    gpu_fn, orc_fn, width = VARIANTS[variant]
    host = np.full(num_blocks * block * width, 0xA5, dtype=np.uint8)
    dev_cache = u8_dev(host, device).view(num_blocks, block, width)
    gpu_fn(bf16_dev(latent, device), i64_dev(positions, device),
           torch.from_numpy(np.ascontiguousarray(table)).to(device), dev_cache,
           i64_dev(slots, device), cr, sanitize)
    torch.cuda.synchronize()
    got = dev_cache.cpu().numpy().reshape(-1)
    orc_fn(latent, positions, np.ascontiguousarray(table), host, block, num_blocks, slots, cr,
           sanitize)
    return got, host


@pytest.mark.parametrize("variant", ["mxfp8", "nvfp4", "v4"])
def test_rope_insert_workload(device, variant):
    """16384 tokens, positions in [0, 65536), compress ratio 4, cache block
    64: only tokens with (pos + 1) % 4 == 0 are written."""
    case = workloads.rope_case()
    log(f"rope {variant}: {case.latent.shape[0]} tokens")
    got, want = run_both(device, variant, case.latent, case.positions, case.cos_sin, case.slots,
                         case.block, case.num_blocks, case.compress_ratio)
    assert (got == want).all(), first_mismatch(got, want)


@pytest.mark.parametrize("variant", ["mxfp8", "nvfp4", "v4"])
@pytest.mark.parametrize("cr", [1, 2, 3])
def test_rope_ratios_extremes(device, variant, cr):
    """Compress ratios 1..3, a non-power-of-two block, wide value ranges
    (down to subnormal quotients and up to overflowing rotations), signed
    zeros, NaN (sanitised) and +-Inf, bad slots and out-of-table rows."""
    rng = np.random.default_rng(100 + cr)
    n = 2000
    x = rng.standard_normal((n, 512)) * np.exp2(rng.uniform(-140, 127, size=(n, 1)))
    with np.errstate(over="ignore", under="ignore"):
        xf = x.astype(np.float32)
    latent = (xf.view(np.uint32) >> 16).astype(np.uint16)
    latent[(latent & 0x7F80) == 0x7F80] = 0x3F80
    latent[::5, 3] = 0x8000
    latent[::9, 100:140] = 0
    latent[::9, 100:140:3] = 0x8000
    latent[7, 10] = 0x7FC0
    latent[11, 460] = 0xFFC1
    latent[13, 20] = 0x7F80
    latent[17, 501] = 0xFF80
    latent[19, 449] = 0x7F7F
    latent[19, 448] = 0xFF7F
    table = workloads.rope_cos_sin_table(rows=5000)
    positions = rng.integers(0, 5200, size=n).astype(np.int64)  # some rows off the table
    block, nb = 48, 45
    slots = rng.permutation(nb * block)[:n].astype(np.int64)
    slots[rng.random(n) < 0.05] = -1
    slots[:3] = [nb * block, nb * block + 5, 10**11]
    log(f"rope {variant} cr={cr} extremes")
    got, want = run_both(device, variant, latent, positions, table, slots, block, nb, cr)
    assert (got == want).all(), first_mismatch(got, want)


@pytest.mark.parametrize("sanitize", [True, False])
@pytest.mark.parametrize("variant", ["mxfp8", "nvfp4", "v4"])
def test_rope_ratio_one_many_tokens(device, variant, sanitize):
    """Compress ratio 1 at 70001 tokens, the size at which a wave takes
    several tokens: a ragged last wave, negative and out-of-table positions,
    pad and out-of-range slots, wide value ranges and specials.  Most slots
    are pads (the oracle's cost is per written token); the first 4096
    tokens are all valid, so whole waves of written tokens are covered."""
    rng = np.random.default_rng(31)
    n = 70001
    x = rng.standard_normal((n, 512)) * np.exp2(rng.uniform(-130, 120, size=(n, 1)))
    with np.errstate(over="ignore", under="ignore"):
        xf = x.astype(np.float32)
    latent = (xf.view(np.uint32) >> 16).astype(np.uint16)
    latent[(latent & 0x7F80) == 0x7F80] = 0x3F80
    latent[::97, 5] = 0x7FC0
    latent[::89, 470] = 0xFF80
    latent[::83, 30:40] = 0x8000
    table = workloads.rope_cos_sin_table(rows=5000)
    positions = rng.integers(0, 5200, size=n).astype(np.int64)
    positions[::101] = -1
    positions[::103] = -(2**40)
    block, nb = 64, 1100
    slots = rng.permutation(nb * block)[:n].astype(np.int64)
    pad = rng.random(n) < 0.85
    pad[:4096] = False
    slots[pad] = -1
    slots[1::997] = nb * block + 3
    slots[-1] = 0 if slots[-1] < 0 else slots[-1]
    log(f"rope {variant} cr=1, {n} tokens, {int((slots >= 0).sum())} with a slot, sanitize={sanitize}")
    got, want = run_both(device, variant, latent, positions, table, slots, block, nb, 1, sanitize=sanitize)
    assert (got == want).all(), first_mismatch(got, want)


@pytest.mark.parametrize("variant", ["mxfp8", "nvfp4", "v4"])
def test_rope_exponent_sweep(device, variant):
    """Every positive finite bf16 value as the only nonzero in its group or
    tile, positive and negative, through the real table."""
    pats = np.arange(1, 0x7F80, dtype=np.uint16)
    pats = np.concatenate([pats, pats | 0x8000])
    per = {"mxfp8": 16, "nvfp4": 32, "v4": 8}[variant]
    step = 512 // per
    n = -(-pats.size // per)
    latent = np.zeros((n, 512), dtype=np.uint16)
    flat = latent.reshape(-1, step)
    flat[: pats.size, 1] = pats
    positions = (np.arange(n, dtype=np.int64) * 4 + 3) % 60000
    table = workloads.rope_cos_sin_table(rows=60000)
    block = 64
    nb = -(-n // block)
    slots = np.arange(n, dtype=np.int64)
    log(f"rope {variant} exponent sweep: {n} tokens")
    got, want = run_both(device, variant, latent, positions, table, slots, block, nb, 4)
    assert (got == want).all(), first_mismatch(got, want)


def test_rope_quant_insert_dispatch(device):
    case = workloads.rope_case(tokens=1024)
    for width, variant in ((528, "mxfp8"), (288, "nvfp4"), (584, "v4")):
        kv = torch.full((16, 64, width), 0xA5, dtype=torch.uint8, device=device)
        ops.rope_quant_insert(bf16_dev(case.latent, device), i64_dev(case.positions, device),
                              torch.from_numpy(case.cos_sin).to(device), kv,
                              i64_dev(case.slots, device), 4)
        torch.cuda.synchronize()
        host = np.full(16 * 64 * width, 0xA5, dtype=np.uint8)
        VARIANTS[variant][1](case.latent, case.positions, case.cos_sin, host, 64, 16, case.slots, 4)
        assert (kv.cpu().numpy().reshape(-1) == host).all(), variant
    with pytest.raises(ValueError):
        ops.rope_quant_insert(bf16_dev(case.latent, device), i64_dev(case.positions, device),
                              torch.from_numpy(case.cos_sin).to(device),
                              torch.zeros((4, 64, 600), dtype=torch.uint8, device=device),
                              i64_dev(case.slots, device), 4)


@pytest.mark.parametrize("variant", ["mxfp8", "nvfp4", "v4"])
def test_rope_without_sanitising(device, variant):
    """sanitize_nans = 0: NaN reaches the quantizer (MXFP8 scale bytes may
    reach 255); both sides follow the same IEEE max/clamp rules."""
    rng = np.random.default_rng(77)
    n = 512
    latent = (rng.standard_normal((n, 512)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    latent[::3, rng.integers(0, 512, size=4)] = 0x7FC0
    latent[1::7, 450] = 0xFFC0
    latent[5, 0:32] = 0x7F80
    latent[9, 480] = 0x7F80
    table = workloads.rope_cos_sin_table(rows=4096)
    positions = (np.arange(n, dtype=np.int64) * 4 + 3) % 4096
    slots = rng.permutation(n).astype(np.int64)
    log(f"rope {variant} without sanitising")
    got, want = run_both(device, variant, latent, positions, table, slots, 64, n // 64, 4,
                         sanitize=False)
    assert (got == want).all(), first_mismatch(got, want)


def test_mxfp8_exponent_just_above_powers_of_two(device):
    """fp32 group maxima whose fp32(amax * fl(1/448)) is the float just above
    2^k: the kernel's exponent must be the exact ceiling (k + 1)."""
    inv448 = np.float32(1.0 / 448.0)
    tables, ks = [], (-20, -9, -5, 4, 10, 60)
    for k in ks:
        target = np.nextafter(np.float32(2.0 ** k), np.float32(np.inf))
        c = np.float32(float(target) * 448.0)
        for _ in range(64):
            v = np.float32(c * inv448)
            if v == target:
                break
            c = np.nextafter(c, np.float32(np.inf) if v < target else np.float32(0))
        assert np.float32(c * inv448) == target
        tables.append(c)
    n = len(ks)
    table = np.zeros((4 * n, 64), dtype=np.float32)
    for i, c in enumerate(tables):
        table[4 * i:4 * i + 4, :32] = c
    latent = np.zeros((n, 512), dtype=np.uint16)
    latent[:, 448] = 0x3F80
    positions = np.arange(n, dtype=np.int64) * 4 + 3
    slots = np.arange(n, dtype=np.int64)
    got, want = run_both(device, "mxfp8", latent, positions, table, slots, n, 1, 4)
    assert (got == want).all(), first_mismatch(got, want)
    scales = want[n * 512:].reshape(n, 16)[:, 14]
    assert [int(b) - 127 for b in scales] == [k + 1 for k in ks]


@pytest.mark.parametrize("variant", ["mxfp8", "nvfp4", "v4"])
@pytest.mark.parametrize("cr,n", [(1, 70_001), (4, 16_384)])
def test_rope_strided_table_and_interleaved_pages(device, variant, cr, n):
    """The table as a column slice of a wider one (row stride 96 floats, the
    extra columns NaN) and pages 48 bytes further apart than one block of
    records (the gaps, and a spare page past the last, hold canaries)
    [P2 `rope_quant_insert` passes the table's and the cache's row strides].
    Ratio 1 at 70,001 tokens runs the several-tokens-per-wave kernels with a
    ragged tail; ratio 4 the gated one.  Every byte of the backing buffer is
    compared with the oracle's."""
    from tests.gpu_util import oracle_threads

    gpu_fn, orc_fn, width = VARIANTS[variant]
    rng = np.random.default_rng(300 + cr)
    x = rng.standard_normal((n, 512)) * np.exp2(rng.uniform(-20, 20, size=(n, 1)))
    latent = (x.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    positions = rng.integers(0, 65536, n).astype(np.int64)
    block = 64
    nb = -(-n * 21 // 20 // block)
    slots = rng.permutation(nb * block)[:n].astype(np.int64)
    slots[rng.random(n) < 0.05] = -1
    wide = np.full((65536, 96), np.nan, dtype=np.float32)
    wide[:, :64] = workloads.rope_cos_sin_table()
    stride = block * width + 48
    host = np.full((nb + 1) * stride, 0xA5, dtype=np.uint8)
    backing = u8_dev(host, device)
    view = torch.as_strided(backing, (nb, block, width), (stride, width, 1))
    table_dev = torch.from_numpy(wide).to(device)[:, :64]
    assert table_dev.stride(0) == 96 and view.stride(0) == stride
    log(f"rope {variant}: {n} tokens, cr={cr}, table stride 96, page stride {stride}")
    gpu_fn(bf16_dev(latent, device), i64_dev(positions, device), table_dev, view,
           i64_dev(slots, device), cr)
    torch.cuda.synchronize()
    got = backing.cpu().numpy()
    orc_fn(latent, positions, wide[:, :64], host, block, nb, slots, cr,
           cache_block_stride=stride, threads=oracle_threads())
    assert (got == host).all(), first_mismatch(got, host)
