"""The entry points can be captured in a HIP graph: every replay, with eager
work and synchronisations in between, writes the same bytes as eager calls.
(No entry point records a memset: the inverse map is cleared by a kernel,
and the split attention keeps nothing in its workspace between calls.)"""

import numpy as np
import pytest
import torch

import workloads
from mxfp4_paged_cache_store_amd import ops
from tests.gpu_util import bf16_dev, i64_dev, log

pytestmark = pytest.mark.gpu


def test_graph_replays_match_eager(device):
    n = 1 << 17  # a dense scattered batch through the slot-order form
    g_src = torch.empty((n, 512), dtype=torch.bfloat16, device=device)
    g_slots = torch.randperm(n, device=device)
    inv = ops.mxfp4_inverse_workspace(1, n, device)
    g_cache = torch.empty(n * 272, dtype=torch.uint8, device=device)
    p_src = torch.empty((4096, 512), dtype=torch.bfloat16, device=device)
    p_slots = torch.randperm(1 << 16, device=device)[:4096]
    p_cache = torch.empty((1 << 16) * 272, dtype=torch.uint8, device=device)
    dq_out = torch.empty((4096, 512), dtype=torch.bfloat16, device=device)
    rc = workloads.rope_case(tokens=1024)
    r_lat = bf16_dev(rc.latent, device)
    r_pos, r_cs, r_slots = i64_dev(rc.positions, device), torch.from_numpy(rc.cos_sin).to(device), i64_dev(rc.slots, device)
    r_kv = torch.empty((16, 64, 528), dtype=torch.uint8, device=device)
    # compress ratio 1 at 70,000 tokens: the path where a wave takes several tokens
    r1_lat = torch.empty((70_000, 512), dtype=torch.bfloat16, device=device)
    r1_pos = torch.randint(0, r_cs.shape[0], (70_000,), device=device)
    r1_slots = torch.randperm(1094 * 64, device=device)[:70_000].contiguous()
    r1_kv = torch.empty((1094, 64, 288), dtype=torch.uint8, device=device)
    # a decode step's read side over the cache the scatter store just wrote:
    # one pass and the split-key form (its workspace allocated up front)
    a_q = torch.empty((8, 32, 512), dtype=torch.bfloat16, device=device)
    a_idx = torch.randint(-1, 1 << 16, (8, 512), dtype=torch.int32, device=device)
    a_out = torch.empty_like(a_q)
    a_out1 = torch.empty_like(a_q)
    a_ws = torch.empty(ops.sparse_mla_attention_workspace_bytes(8, 32, 4), dtype=torch.uint8, device=device)
    # the V4 insert, the ring-state save and the compress-ratio-1 norm
    v4_kv = torch.empty((16, 64, 584), dtype=torch.uint8, device=device)
    ring_rows = torch.empty((3000, 1024), dtype=torch.float32, device=device)
    ring_slots = torch.randperm(200 * 32, device=device)[:3000].contiguous()
    ring = torch.empty((200, 32, 1024), dtype=torch.float32, device=device)
    n_kv = torch.empty((5000, 512), dtype=torch.float32, device=device)
    n_slots = torch.arange(5000, device=device)
    n_slots[::7] = -1
    n_w = torch.empty(512, dtype=torch.bfloat16, device=device)
    n_out = torch.empty((5000, 512), dtype=torch.bfloat16, device=device)

    def work():
        ops.mxfp4_build_inverse(g_slots, 1, n, inv)
        ops.mxfp4_store_by_slot(g_src, n, inv, g_cache, 1, n, n)
        ops.mxfp4_store(p_src, p_slots, p_cache, 1, 1 << 16, 1 << 16)
        ops.mxfp4_gather_dequant(p_cache, 1, 1 << 16, 1 << 16, 512, p_slots, dq_out)
        ops.mxfp8_rope_store(r_lat, r_pos, r_cs, r_kv, r_slots, rc.compress_ratio)
        ops.nvfp4_rope_store(r1_lat, r1_pos, r_cs, r1_kv, r1_slots, 1)
        ops.sparse_mla_attention(a_q, p_cache, a_idx, 0.04, out=a_out, splits=4, workspace=a_ws)
        ops.sparse_mla_attention(a_q, p_cache, a_idx, 0.04, out=a_out1, splits=1)
        ops.v4_rope_store(r_lat, r_pos, r_cs, v4_kv, r_slots, rc.compress_ratio)
        ops.save_ring_rows(ring_rows, ring_slots, ring)
        ops.fused_save_compress_norm_cr1(n_kv, n_slots, n_w, 1e-6, n_out)

    def reset(seed):
        gen = torch.Generator(device=device)
        gen.manual_seed(seed)
        g_src.uniform_(-4, 4, generator=gen)
        p_src.uniform_(-100, 100, generator=gen)
        g_cache.fill_(0xA5)
        p_cache.fill_(0xA5)
        dq_out.fill_(0)
        r_kv.fill_(0xA5)
        r1_lat.normal_(generator=gen)
        r1_kv.fill_(0xA5)
        a_q.normal_(generator=gen)
        a_out.fill_(0)
        a_out1.fill_(0)
        v4_kv.fill_(0xA5)
        ring_rows.uniform_(-2, 2, generator=gen)
        ring.fill_(1.5)
        n_kv.normal_(generator=gen)
        n_w.uniform_(0.5, 1.5, generator=gen)
        n_out.fill_(0)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        reset(0)
        work()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        work()

    for rep in range(4):
        log(f"graph replay {rep}")
        reset(100 + rep)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = [g_cache.clone(), p_cache.clone(), dq_out.clone(), r_kv.clone(), r1_kv.clone(), a_out.clone(),
               a_out1.clone(), v4_kv.clone(), ring.clone(), n_out.clone()]
        reset(100 + rep)
        work()  # eager
        torch.cuda.synchronize()
        want = [g_cache, p_cache, dq_out, r_kv, r1_kv, a_out, a_out1, v4_kv, ring, n_out]
        names = ("slot-order store", "scatter store", "dequant", "mxfp8 insert", "nvfp4 insert, ratio 1",
                 "attention split", "attention one pass", "v4 insert", "ring save", "cr1 norm")
        for name, a, b in zip(names, got, want):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), (rep, name)
