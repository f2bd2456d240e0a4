"""The binding on empty inputs whose strides carry no layout (tensors made
from empty numpy arrays have zero strides): every entry point accepts them
and writes nothing."""

import numpy as np
import pytest
import torch

import workloads
from mxfp4_paged_cache_store_amd import ops
from tests.gpu_util import log

pytestmark = pytest.mark.gpu


def test_empty_inputs_with_zero_strides(device):
    src = torch.from_numpy(np.zeros((0, 512), dtype=np.int16)).to(device).view(torch.bfloat16)
    slots = torch.from_numpy(np.zeros(0, dtype=np.int64)).to(device)
    log(f"empty bf16 rows: strides {src.stride()}")
    cache = torch.full((64 * 272,), 0xA5, dtype=torch.uint8, device=device)
    ops.mxfp4_store(src, slots, cache, 1, 64, 64)
    inv = ops.mxfp4_inverse_workspace(1, 64, device)
    ops.mxfp4_build_inverse(slots, 1, 64, inv)
    ops.mxfp4_store_by_slot(src, 0, inv, cache, 1, 64, 64)
    ops.mxfp4_store_slot_order_noalloc(src, slots, cache, 1, 64, 64)
    out = torch.from_numpy(np.zeros((0, 512), dtype=np.int16)).to(device).view(torch.bfloat16)
    ops.mxfp4_gather_dequant(cache, 1, 64, 64, 512, slots, out)

    rows = torch.from_numpy(np.zeros((0, 1024), dtype=np.float32)).to(device)
    ring = torch.full((4, 8, 1024), 1.5, dtype=torch.float32, device=device)
    ops.save_ring_rows(rows, slots, ring)

    kv = torch.from_numpy(np.zeros((0, 512), dtype=np.float32)).to(device)
    w = torch.ones(512, dtype=torch.bfloat16, device=device)
    lat = torch.from_numpy(np.zeros((0, 512), dtype=np.int16)).to(device).view(torch.bfloat16)
    ops.fused_save_compress_norm_cr1(kv, slots, w, 1e-6, lat)

    table = torch.from_numpy(workloads.rope_cos_sin_table(rows=64)).to(device)
    pos = torch.from_numpy(np.zeros(0, dtype=np.int64)).to(device)
    rc = torch.full((2, 64, 528), 0xA5, dtype=torch.uint8, device=device)
    ops.mxfp8_rope_store(src, pos, table, rc, slots, 1)

    q = torch.from_numpy(np.zeros((0, 32, 512), dtype=np.int16)).to(device).view(torch.bfloat16)
    idx = torch.from_numpy(np.zeros((0, 64), dtype=np.int32)).to(device)
    a = ops.sparse_mla_attention(q, cache, idx, 0.04, splits=1)
    b = ops.sparse_mla_attention(q, cache, idx, 0.04, splits=4)
    torch.cuda.synchronize()
    assert a.shape == b.shape == (0, 32, 512)
    assert (cache == 0xA5).all() and (ring == 1.5).all() and (rc == 0xA5).all()
