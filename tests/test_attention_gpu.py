"""GPU parity of sparse_mla_attention against the oracle's double-precision
attention over the bf16 dequantized cache, within the tolerance derived in
tests/attn_tolerance.py.  A token whose only valid slot is listed once must
reproduce that row exactly; a token with no valid slot gives zeros."""

import numpy as np
import pytest
import torch

import oracle
import workloads
from mxfp4_paged_cache_store_amd import ops
from tests.attn_tolerance import dequant_rows, tolerance
from tests.gpu_util import bf16_dev, log, u8_dev

pytestmark = pytest.mark.gpu

def run_gpu(device, case: workloads.AttnCase, out_pad: int = 0, splits: int = 1):
    t, h, _ = case.q.shape
    cache = u8_dev(case.cache, device)
    if case.block_stride_rows != case.block_size or case.num_blocks > 1:
        cache = cache.view(case.num_blocks, case.block_stride_rows, 272)[:, :case.block_size]
    q = bf16_dev(case.q, device)
    idx = torch.from_numpy(np.ascontiguousarray(case.indices)).to(device)
    sink = None if case.sink is None else torch.from_numpy(case.sink).to(device)
    backing = torch.full((t, h, 512 + out_pad), -7.0, dtype=torch.bfloat16, device=device)
    out = backing[:, :, :512]
    log(f"attention T={t} H={h} topk={case.indices.shape[1]} sink={case.sink is not None} splits={splits}")
    ops.sparse_mla_attention(q, cache, idx, case.scale, sink=sink, out=out, splits=splits)
    torch.cuda.synchronize()
    if out_pad:
        assert (backing[:, :, 512:] == -7.0).all(), "padding written"
    return out.float().cpu().numpy().astype(np.float64)


def check_case(device, case: workloads.AttnCase, out_pad: int = 0, splits: int = 1):
    got = run_gpu(device, case, out_pad, splits)
    want = oracle.sparse_mla_attention(case.q, case.cache, case.num_blocks, case.block_size,
                                       case.block_stride_rows, case.indices, case.scale, case.sink)
    tol = tolerance(case.q, case.cache, case.num_blocks, case.block_size, case.block_stride_rows,
                    case.indices, case.scale, case.sink, want)
    err = np.abs(got - want)
    worst = float((err / np.maximum(tol, 1e-300)).max()) if err.size else 0.0
    bad = np.argwhere(err > tol)
    assert bad.size == 0, (worst, [(tuple(i), got[tuple(i)], want[tuple(i)], tol[tuple(i)]) for i in bad[:5]])
    return worst


@pytest.mark.parametrize("tokens,heads,topk,sink,seed", [
    (4, 16, 64, False, 1),       # one tile
    (6, 16, 256, False, 2),      # four tiles
    (5, 32, 200, True, 3),       # ragged last tile, sinks, 32-head blocks
    (3, 48, 130, False, 4),      # three 16-head blocks
    (2, 64, 512, True, 5),       # two 32-head blocks
])
def test_attention_parity(device, tokens, heads, topk, sink, seed):
    case = workloads.attention_case(tokens, heads, topk, seed, sink=sink)
    worst = check_case(device, case)
    log(f"worst error / tolerance = {worst:.3f}")


@pytest.mark.parametrize("sign", [-1.0, 0.0])
@pytest.mark.parametrize("splits", [1, 3])
def test_attention_negative_and_zero_scale(device, sign, splits):
    """A negative softmax scale (the kernel scores -q against |scale|,
    which gives exactly the same scores) and a zero one (every score 0: the
    weights are uniform over the valid slots, beside the sink), with skipped
    slots and a ragged tile, in the one-pass and split forms."""
    case = workloads.attention_case(5, 32, 200, 21, sink=True)
    case.scale = sign * case.scale
    check_case(device, case, splits=splits)


def test_attention_query_dynamic_range(device):
    """Query blocks whose values span many binades (each value times 2^k, k
    uniform in [-30, 6]), a head with bf16 subnormals in one block and a zero
    head; one pass and split.  Scores here span ~160, so some outputs come
    from weights below the fp32 normal range (the tolerance's absolute
    terms)."""
    case = workloads.attention_case(4, 32, 200, 31, sink=True)
    rng = np.random.default_rng(131)
    qf = (case.q.astype(np.uint32) << 16).view(np.float32)
    qf = qf * np.exp2(rng.integers(-30, 7, size=qf.shape)).astype(np.float32)
    qf[:, 3, 64:96] = rng.standard_normal((4, 32)).astype(np.float32) * np.float32(2.0 ** -130)
    qf[:, 5, :] = 0.0
    case.q = workloads.f32_to_bf16_bits(qf.astype(np.float32))
    assert ((case.q[:, 3, 64:96] & 0x7F80) == 0).all() and (case.q[:, 3, 64:96] != 0).any()
    for splits in (1, 2):
        check_case(device, case, splits=splits)


def test_attention_sharp_scores_and_paged_cache(device):
    """Peaked softmax (score std ~12), a non-power-of-two block (48) with
    other layers' rows interleaved (stride 80), and a padded output."""
    case = workloads.attention_case(4, 32, 300, 6, num_blocks=40, block_size=48,
                                    block_stride_rows=80, score_std=12.0, sink=True)
    check_case(device, case, out_pad=8)


def test_attention_degenerate_tokens(device):
    """Token 0: no valid slot -> zeros (with sinks too); token 1: one valid
    slot -> exactly that row; token 2: a slot listed 40 times among pads;
    token 3: topk entries all past the cache."""
    case = workloads.attention_case(4, 16, 96, 7, sink=False)
    idx = np.full((4, 96), -1, dtype=np.int32)
    idx[1, 50] = 17
    idx[2, ::2][:40] = 33
    idx[3, :] = case.num_blocks * case.block_size + 3
    case.indices = idx
    got = run_gpu(device, case)
    assert (got[0] == 0).all() and (got[3] == 0).all()
    row = dequant_rows(case.cache, case.num_blocks, case.block_size, case.block_stride_rows,
                       np.array([17]))[0]
    assert (got[1] == row[None, :]).all()
    assert (got[2] == dequant_rows(case.cache, case.num_blocks, case.block_size,
                                   case.block_stride_rows, np.array([33]))[0][None, :]).all()
    case.sink = np.linspace(-2, 2, 16).astype(np.float32)
    got = run_gpu(device, case)
    assert (got[0] == 0).all() and (got[3] == 0).all()
    check_case(device, case)


def test_attention_topk_zero(device):
    case = workloads.attention_case(3, 16, 0, 8)
    got = run_gpu(device, case)
    assert (got == 0).all()


def test_attention_workload_sampled(device):
    """The benchmark's workload (the last 4,096 queries of a 16,384-token
    prefill, 32 heads, top-2048 causal slots) in the launch the benchmark
    times; 6 sampled tokens (first, last and random) checked against the
    oracle, all heads."""
    q, cache, idx, scale = workloads.attention_workload_device()
    log(f"attention workload T={q.shape[0]} H={q.shape[1]} topk={idx.shape[1]}")
    out = ops.sparse_mla_attention(q, cache, idx, scale, splits=1)
    torch.cuda.synchronize()
    rng = np.random.default_rng(9)
    pick = np.unique(np.concatenate([[0, q.shape[0] - 1], rng.choice(q.shape[0], 4, replace=False)]))
    pick_dev = torch.from_numpy(pick).to(q.device)
    q_s = q[pick_dev].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    idx_s = idx[pick_dev].cpu().numpy()
    cache_h = cache.cpu().numpy().reshape(-1)
    n = cache.shape[0]
    got = out[pick_dev].float().cpu().numpy().astype(np.float64)
    want = oracle.sparse_mla_attention(q_s, cache_h, 1, n, n, idx_s, scale)
    tol = tolerance(q_s, cache_h, 1, n, n, idx_s, scale, None, want)
    err = np.abs(got - want)
    assert (err <= tol).all(), float((err / tol).max())


def test_attention_cache_past_4gib(device):
    """A paged view spanning more than 4 GiB (two blocks 16M rows apart):
    the kernel gathers with 64-bit addresses there (below that, through a
    raw buffer whose range check zeroes skipped keys).  Same result as the
    oracle on the compact copy of the two blocks."""
    case = workloads.attention_case(3, 32, 100, 11, num_blocks=2, block_size=64, sink=True)
    far = 16_000_000
    backing = torch.empty(((far + 64) * 272,), dtype=torch.uint8, device=device)
    view = backing.view(far + 64, 272)
    rows = torch.from_numpy(case.cache.reshape(2 * 64, 272)).to(device)
    view[:64] = rows[:64]
    view[far:far + 64] = rows[64:]
    q = bf16_dev(case.q, device)
    idx = torch.from_numpy(np.ascontiguousarray(case.indices)).to(device)
    sink = torch.from_numpy(case.sink).to(device)
    log(f"attention over a {backing.numel() / 2**30:.2f} GiB paged view")
    paged = backing.as_strided((2, 64, 272), (far * 272, 272, 1))
    out = ops.sparse_mla_attention(q, paged, idx, case.scale, sink=sink, splits=1)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy().astype(np.float64)
    want = oracle.sparse_mla_attention(case.q, case.cache, 2, 64, 64, case.indices, case.scale, case.sink)
    tol = tolerance(case.q, case.cache, 2, 64, 64, case.indices, case.scale, case.sink, want)
    assert (np.abs(got - want) <= tol).all()


@pytest.mark.parametrize("tokens,heads,topk,sink,seed,splits", [
    (4, 16, 256, True, 21, 2),     # two ranges of two tiles
    (5, 32, 200, True, 22, 3),     # ragged last tile; the third range is empty
    (3, 48, 130, False, 23, 5),    # three tiles over five ranges (two empty)
    (2, 64, 512, True, 24, 8),     # one tile per range
    (3, 32, 1000, False, 25, 64),  # the largest split count
])
def test_attention_split_parity(device, tokens, heads, topk, sink, seed, splits):
    """The split-key form (partials per key range, merged by log-sum-exp)
    against the oracle, within the same tolerance as one pass."""
    case = workloads.attention_case(tokens, heads, topk, seed, sink=sink)
    worst = check_case(device, case, splits=splits)
    log(f"split {splits}: worst error / tolerance = {worst:.3f}")


def test_attention_split_degenerate_tokens(device):
    """Split form: a token with no valid slot gives zeros (with sinks too);
    a token with one valid slot listed once reproduces that row exactly."""
    case = workloads.attention_case(3, 16, 320, 26, sink=False)
    idx = np.full((3, 320), -1, dtype=np.int32)
    idx[1, 250] = 17
    idx[2, ::3] = np.arange(107) % 64
    case.indices = idx
    for sink in (None, np.linspace(-2, 2, 16).astype(np.float32)):
        case.sink = sink
        got = run_gpu(device, case, splits=4)
        assert (got[0] == 0).all()
        if sink is None:
            row = dequant_rows(case.cache, case.num_blocks, case.block_size, case.block_stride_rows,
                               np.array([17]))[0]
            assert (got[1] == row[None, :]).all()
        check_case(device, case, splits=4)


def test_attention_split_workspace_reuse(device):
    """A workspace full of arbitrary bytes, reused across calls with different
    token counts and split counts (and each call made twice), gives the
    oracle's result every time: the split form keeps no state in it between
    calls."""
    ws = torch.full((1 << 22,), 0xFF, dtype=torch.uint8, device=device)
    for tokens, splits, seed in ((3, 4, 31), (5, 2, 32), (2, 8, 33), (3, 4, 34)):
        case = workloads.attention_case(tokens, 32, 300, seed, sink=True)
        q = bf16_dev(case.q, device)
        idx = torch.from_numpy(np.ascontiguousarray(case.indices)).to(device)
        sink = torch.from_numpy(case.sink).to(device)
        log(f"attention split workspace reuse T={tokens} splits={splits}")
        for _ in range(2):
            out = ops.sparse_mla_attention(q, u8_dev(case.cache, device), idx, case.scale, sink=sink,
                                           splits=splits, workspace=ws)
            torch.cuda.synchronize()
            got = out.float().cpu().numpy().astype(np.float64)
            want = oracle.sparse_mla_attention(case.q, case.cache, case.num_blocks, case.block_size,
                                               case.block_stride_rows, case.indices, case.scale, case.sink)
            tol = tolerance(case.q, case.cache, case.num_blocks, case.block_size, case.block_stride_rows,
                            case.indices, case.scale, case.sink, want)
            assert (np.abs(got - want) <= tol).all()


def test_attention_decode_workload_split(device):
    """64 decode queries (the last 64 of a 16,384-token context, top-2048
    slots each) in the advised split form and in one pass: 8 sampled tokens
    of both against the oracle."""
    q, cache, idx, scale = workloads.attention_workload_device(tokens=64)
    splits = ops.sparse_mla_attention_splits_advised(64, q.shape[1], idx.shape[1])
    assert splits > 1
    log(f"attention decode workload T=64 splits={splits}")
    out = ops.sparse_mla_attention(q, cache, idx, scale)
    one = ops.sparse_mla_attention(q, cache, idx, scale, splits=1)
    torch.cuda.synchronize()
    rng = np.random.default_rng(10)
    pick = np.sort(rng.choice(64, 8, replace=False))
    pick_dev = torch.from_numpy(pick).to(q.device)
    q_s = q[pick_dev].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    idx_s = idx[pick_dev].cpu().numpy()
    cache_h = cache.cpu().numpy().reshape(-1)
    n = cache.shape[0]
    want = oracle.sparse_mla_attention(q_s, cache_h, 1, n, n, idx_s, scale)
    tol = tolerance(q_s, cache_h, 1, n, n, idx_s, scale, None, want)
    for form in (out, one):
        got = form[pick_dev].float().cpu().numpy().astype(np.float64)
        assert (np.abs(got - want) <= tol).all(), float((np.abs(got - want) / tol).max())


def test_attention_most_heads(device):
    """The largest head count (1024 = 32 blocks of 32 heads), one pass and
    split, against the oracle."""
    case = workloads.attention_case(2, 1024, 100, 41, sink=True)
    check_case(device, case)
    check_case(device, case, splits=2)


def test_attention_long_sparse_list(device):
    """A listed-slot row of 1,048,576 entries of which 300 are valid, spread
    over the whole row (16,384 tiles, most of them empty): one pass and 16
    key ranges, against the oracle; the index loads reach past 2^20
    entries."""
    case = workloads.attention_case(2, 16, 0, 42, sink=True)
    topk = 1 << 20
    rng = np.random.default_rng(43)
    idx = np.full((2, topk), -1, dtype=np.int32)
    for t in range(2):
        pos = rng.choice(topk, 300, replace=False)
        idx[t, pos] = rng.integers(0, case.num_blocks * case.block_size, size=300)
    idx[1, -1] = 5   # the very last entry
    case.indices = idx
    check_case(device, case)
    check_case(device, case, splits=16)


def test_attention_strided_query(device):
    """The query as the first 512 of 576 values per head (the rope-free part
    of a [T, H, 576] MLA query), one pass and split; same result as the
    contiguous query."""
    case = workloads.attention_case(3, 32, 200, 44, sink=True)
    t, h, _ = case.q.shape
    wide = torch.zeros((t, h, 576), dtype=torch.bfloat16, device=device)
    wide[:, :, :512] = bf16_dev(case.q, device)
    wide[:, :, 512:] = 1e4  # must not be read
    q = wide[:, :, :512]
    cache = u8_dev(case.cache, device)
    idx = torch.from_numpy(np.ascontiguousarray(case.indices)).to(device)
    sink = torch.from_numpy(case.sink).to(device)
    want = oracle.sparse_mla_attention(case.q, case.cache, case.num_blocks, case.block_size,
                                       case.block_stride_rows, case.indices, case.scale, case.sink)
    tol = tolerance(case.q, case.cache, case.num_blocks, case.block_size, case.block_stride_rows,
                    case.indices, case.scale, case.sink, want)
    for splits in (1, 3):
        log(f"attention strided query splits={splits}")
        out = ops.sparse_mla_attention(q, cache, idx, case.scale, sink=sink, splits=splits)
        torch.cuda.synchronize()
        got = out.float().cpu().numpy().astype(np.float64)
        assert (np.abs(got - want) <= tol).all()


@pytest.mark.parametrize("seed", range(16))
def test_attention_random_geometry(device, seed):
    """Seeded random geometries: heads (16-80), tokens, top-k (0-700, ragged
    last tiles), block size and interleaved blocks, share of invalid slots,
    sinks, score sharpness, and the one-pass or split-key form (1-8 ranges,
    some of them empty)."""
    rng = np.random.default_rng(3000 + seed)
    heads = int(rng.choice([16, 32, 48, 64, 80]))
    tokens = int(rng.integers(1, 7))
    topk = int(rng.choice([0, 1, 17, 64, 100, 256, 333, 700]))
    bs = int(rng.choice([16, 48, 64, 100]))
    nb = int(rng.integers(2, 60))
    bsr = bs + int(rng.choice([0, 0, 8, bs]))
    invalid = float(rng.choice([0.0, 0.1, 0.5, 0.95]))
    sink = bool(rng.random() < 0.5)
    std = float(rng.choice([0.5, 2.0, 8.0]))
    splits = int(rng.choice([1, 1, 2, 3, 8]))
    log(f"random attention seed={seed}: T={tokens} H={heads} topk={topk} blocks={nb}x{bs} stride={bsr} "
        f"invalid={invalid} sink={sink} std={std} splits={splits}")
    case = workloads.attention_case(tokens, heads, topk, 4000 + seed, num_blocks=nb, block_size=bs,
                                    block_stride_rows=bsr, invalid_frac=invalid, sink=sink, score_std=std)
    check_case(device, case, splits=splits)
