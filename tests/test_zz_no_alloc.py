"""The allocation-free slot-order store (mxfp4_store_slot_order_noalloc:
inverse map in the library's static per-GPU array) against the existing
entry points on the same inputs, byte for byte: two calls in a row on one
stream, the second with fewer tokens and fewer slots, each compared with
mxfp4_build_inverse + mxfp4_store_by_slot (the same store with a caller's
workspace) and with the scatter-form mxfp4_store."""

import numpy as np
import pytest
import torch

from mxfp4_paged_cache_store_amd import _abi, ops
from tests.gpu_util import bf16_dev, first_mismatch, i64_dev, log

pytestmark = pytest.mark.gpu


def _case(rng, ntok, nb, bs, stride, pad):
    x = rng.standard_normal((ntok, 512)) * np.exp2(rng.uniform(-20, 20, size=(ntok, 1)))
    src = (x.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    slots = rng.permutation(nb * bs)[:ntok].astype(np.int64)
    slots[rng.random(ntok) < pad] = -1
    return src, slots, ((nb - 1) * stride + bs) * 272


def test_noalloc_matches_workspace_form_twice(device):
    rng = np.random.default_rng(77)
    cases = [
        # 300,000 tokens over 4,800 blocks of 64 slots, blocks 80 rows apart
        (300_000, 4800, 64, 80, 0.03),
        # then fewer tokens and slots: 1,000 tokens, 20 blocks of 62 (62 % 4 != 0:
        # rows written one by one instead of staged in LDS)
        (1_000, 20, 62, 70, 0.1),
    ]
    runs = []
    stream = torch.cuda.current_stream()
    for ntok, nb, bs, stride, pad in cases:
        src, slots, nbytes = _case(rng, ntok, nb, bs, stride, pad)
        s_dev, sl_dev = bf16_dev(src, device), i64_dev(slots, device)
        noalloc = torch.full((nbytes,), 0xA5, dtype=torch.uint8, device=device)
        log(f"noalloc store: {ntok} tokens, {nb} x {bs} slots, stride {stride}")
        ops.mxfp4_store_slot_order_noalloc(s_dev, sl_dev, noalloc, nb, bs, stride, stream=stream)
        runs.append((s_dev, sl_dev, noalloc, ntok, nb, bs, stride, nbytes))
    torch.cuda.synchronize()
    for s_dev, sl_dev, noalloc, ntok, nb, bs, stride, nbytes in runs:
        inv = ops.mxfp4_inverse_workspace(nb, bs, device)
        ws = torch.full((nbytes,), 0xA5, dtype=torch.uint8, device=device)
        scatter = torch.full((nbytes,), 0xA5, dtype=torch.uint8, device=device)
        log(f"workspace and scatter forms: {ntok} tokens")
        ops.mxfp4_build_inverse(sl_dev, nb, bs, inv)
        ops.mxfp4_store_by_slot(s_dev, ntok, inv, ws, nb, bs, stride)
        ops.mxfp4_store(s_dev, sl_dev, scatter, nb, bs, stride)
        torch.cuda.synchronize()
        got, want, sc = noalloc.cpu().numpy(), ws.cpu().numpy(), scatter.cpu().numpy()
        assert (got == want).all(), first_mismatch(got, want, 272)
        assert (got == sc).all(), first_mismatch(got, sc, 272)


def test_noalloc_refuses_maps_past_the_array(device):
    """A geometry whose inverse map exceeds the static array is refused on
    the host with nothing launched; the largest that fits is accepted."""
    src = torch.zeros((4, 512), dtype=torch.bfloat16, device=device)
    slots = torch.arange(4, dtype=torch.int64, device=device)
    fits = _abi.NOALLOC_SCRATCH_BYTES // 4
    big = torch.full((272 * 8,), 0xA5, dtype=torch.uint8, device=device)
    with pytest.raises(_abi.MxError) as err:
        _abi.check(_abi.lib().mxfp4_store_slot_order_noalloc(
            src.data_ptr(), 4, 512, 512, slots.data_ptr(), big.data_ptr(), 1, fits + 1, fits + 1,
            32, None))
    assert err.value.status == _abi.MX_E_RANGE
    cache = torch.full((fits * 272,), 0xA5, dtype=torch.uint8, device=device)
    log(f"noalloc store: 4 tokens into {fits} slots")
    ops.mxfp4_store_slot_order_noalloc(src, slots, cache, 1, fits, fits)
    torch.cuda.synchronize()
    head = cache[: 8 * 272].cpu().numpy()
    assert (head[: 4 * 272].reshape(4, 272)[:, 256:] == 127).all()  # zero rows: scale byte 127
    assert (head[4 * 272:] == 0xA5).all()
    del cache


def test_noalloc_graph_replays(device):
    """Captured in a HIP graph (the use the entry point is for: nothing to
    allocate, no memset recorded), every replay writes the bytes of the
    workspace form, also when an eager call with another slot mapping has
    left its own map in the shared array just before."""
    rng = np.random.default_rng(78)
    ntok, nb, bs, stride = 50_000, 900, 64, 72
    src, slots, nbytes = _case(rng, ntok, nb, bs, stride, 0.05)
    s_dev, sl_dev = bf16_dev(src, device), i64_dev(slots, device)
    inv = ops.mxfp4_inverse_workspace(nb, bs, device)
    want = torch.full((nbytes,), 0xA5, dtype=torch.uint8, device=device)
    ops.mxfp4_build_inverse(sl_dev, nb, bs, inv)
    ops.mxfp4_store_by_slot(s_dev, ntok, inv, want, nb, bs, stride)
    # another batch, stored eagerly between replays
    o_src, o_slots, o_nbytes = _case(rng, 3_000, 60, 64, 64, 0.0)
    o_src_dev, o_slots_dev = bf16_dev(o_src, device), i64_dev(o_slots, device)
    o_cache = torch.empty((o_nbytes,), dtype=torch.uint8, device=device)

    cache = torch.empty((nbytes,), dtype=torch.uint8, device=device)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up outside the capture
        cache.fill_(0xA5)
        ops.mxfp4_store_slot_order_noalloc(s_dev, sl_dev, cache, nb, bs, stride)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    assert torch.equal(cache, want), "eager call"

    graph = torch.cuda.CUDAGraph()
    log(f"capturing the noalloc store: {ntok} tokens, {nb} x {bs} slots")
    with torch.cuda.graph(graph):
        ops.mxfp4_store_slot_order_noalloc(s_dev, sl_dev, cache, nb, bs, stride)
    for rep in range(3):
        log(f"noalloc graph replay {rep}")
        cache.fill_(0xA5)
        ops.mxfp4_store_slot_order_noalloc(o_src_dev, o_slots_dev, o_cache, 60, 64, 64)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got, exp = cache.cpu().numpy(), want.cpu().numpy()
        assert (got == exp).all(), (rep, first_mismatch(got, exp, 272))
