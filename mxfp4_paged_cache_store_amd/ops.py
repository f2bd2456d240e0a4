"""PyTorch-facing binding of libmxstore: tensors in, device pointers out.

Every function here only checks tensor metadata and marshals pointers,
sizes and the current HIP stream into the C ABI (include/mxstore.h); all of
the arithmetic runs in the gfx950 kernels.  PyTorch provides device memory
and streams, nothing else.

Sources:
  [P1] docs page "vllm.v1.attention.ops.mxfp4_mla.store", `store_mxfp4_mla`
  [P2] docs page "vllm.models.deepseek_v41.common.ops.fused_compress_quant_cache",
       `rope_quant_insert`
"""

from __future__ import annotations

import torch

from . import _abi

GROUP_SIZE = 32  # values per E8M0 scale (OCP MX block size)
MXFP8_RECORD_BYTES = 528  # 512 E4M3 values + 16 UE8M0 scales [P2 `rope_quant_insert`]
NVFP4_RECORD_BYTES = 288  # 256 bytes of E2M1 pairs + 32 E4M3 scales [P2 `rope_quant_insert`]
V4_RECORD_BYTES = 584     # 576 value bytes + 8 UE8M0 scales, one of them padding [P2 `rope_quant_insert`]


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream)


def _need_cuda(*tensors: torch.Tensor) -> None:
    for t in tensors:
        if not t.is_cuda:
            raise ValueError("libmxstore works on device tensors only")


def _unit_inner(t: torch.Tensor) -> bool:
    """Unit stride along the last dimension.  An empty tensor's strides say
    nothing about a layout (torch may give it zero strides), so it passes."""
    return t.numel() == 0 or t.stride(-1) == 1


def _strides(t: torch.Tensor) -> tuple:
    """Element strides to hand to the C ABI; an empty tensor goes as dense."""
    if t.numel() == 0:
        out, acc = [], 1
        for n in reversed(t.shape):
            out.append(acc)
            acc *= max(n, 1)
        return tuple(reversed(out))
    return t.stride()


def _extent_bytes(t: torch.Tensor) -> int:
    """Bytes from t's data pointer to the end of its last element (what a
    kernel given only the pointer may touch without leaving the tensor)."""
    if t.numel() == 0:
        return 0
    return (1 + sum((n - 1) * st for n, st in zip(t.shape, t.stride()))) * t.element_size()


def _need_cache_extent(cache: torch.Tensor, num_blocks: int, block_size: int, block_stride_rows: int,
                       latent: int, group: int) -> None:
    """The C ABI receives only the cache pointer: check here that the paged
    geometry stays inside the tensor (other argument errors are the ABI's)."""
    if num_blocks < 1 or block_size < 1 or block_stride_rows < block_size or latent < group \
            or group < 1 or latent % group:
        return
    need = ((num_blocks - 1) * block_stride_rows + block_size) * (latent // 2 + latent // group)
    if _extent_bytes(cache) < need:
        raise ValueError(f"cache holds {_extent_bytes(cache)} bytes from its data pointer; "
                         f"{num_blocks} blocks of {block_size} rows at stride {block_stride_rows} need {need}")


def row_bytes(latent: int, group: int = GROUP_SIZE) -> int:
    """Bytes of one packed MXFP4 row: latent/2 + latent/group."""
    n = int(_abi.lib().mx_row_bytes(latent, group))
    if n < 0:
        raise ValueError(f"latent {latent} is not a positive multiple of group {group}")
    return n


# ------------------------------------------------------------------ C ABI names

def mxfp4_store(src: torch.Tensor, slot_mapping: torch.Tensor, cache: torch.Tensor,
                num_blocks: int, block_size: int, block_stride_rows: int,
                group: int = GROUP_SIZE, stream=None) -> None:
    """``mxfp4_store`` of the C ABI.  ``src``: bf16 [T, latent], unit inner
    stride; ``slot_mapping``: int64 [T] contiguous; ``cache``: uint8 storage
    of the paged view (its data pointer is the cache base)."""
    _need_cuda(src, slot_mapping, cache)
    if src.dtype != torch.bfloat16 or src.dim() != 2 or not _unit_inner(src):
        raise ValueError("src must be a bf16 [tokens, latent] tensor with unit inner stride")
    if slot_mapping.dtype != torch.int64 or not slot_mapping.is_contiguous():
        raise ValueError("slot_mapping must be a contiguous int64 tensor")
    if cache.dtype != torch.uint8:
        raise ValueError(f"the cache is raw bytes (torch.uint8), not {cache.dtype}")
    num_tokens = slot_mapping.numel()
    if num_tokens > src.shape[0]:
        raise ValueError("slot_mapping has more entries than src has rows")
    _need_cache_extent(cache, num_blocks, block_size, block_stride_rows, src.shape[1], group)
    _abi.check(_abi.lib().mxfp4_store(
        src.data_ptr(), num_tokens, src.shape[1], _strides(src)[0], slot_mapping.data_ptr(),
        cache.data_ptr(), num_blocks, block_size, block_stride_rows, group, _stream(stream)))


def mxfp4_inverse_bytes(num_blocks: int, block_size: int) -> int:
    """``mxfp4_inverse_bytes`` of the C ABI: bytes of the inverse map (one
    int32 per slot, padded to 16)."""
    n = int(_abi.lib().mxfp4_inverse_bytes(num_blocks, block_size))
    if n < 0:
        raise ValueError("num_blocks and block_size must be >= 1 with fewer than 2^32 slots")
    return n


def mxfp4_inverse_workspace(num_blocks: int, block_size: int, device="cuda") -> torch.Tensor:
    """A device int32 tensor of ``mxfp4_inverse_bytes`` bytes: the inverse
    map that ``mxfp4_build_inverse`` fills and ``mxfp4_store_by_slot`` reads
    (its first num_blocks * block_size entries)."""
    return torch.empty(mxfp4_inverse_bytes(num_blocks, block_size) // 4, dtype=torch.int32,
                       device=device)


def mxfp4_slot_order_advised(num_tokens: int, latent: int, num_blocks: int, block_size: int) -> bool:
    """``mxfp4_slot_order_advised`` of the C ABI."""
    return bool(_abi.lib().mxfp4_slot_order_advised(num_tokens, latent, num_blocks, block_size))


def mxfp4_build_inverse(slot_mapping: torch.Tensor, num_blocks: int, block_size: int,
                        inverse: torch.Tensor, stream=None) -> torch.Tensor:
    """``mxfp4_build_inverse`` of the C ABI; ``inverse`` is a device int32
    tensor of at least ``mxfp4_inverse_bytes`` bytes (see
    ``mxfp4_inverse_workspace``)."""
    _need_cuda(slot_mapping, inverse)
    if slot_mapping.dtype != torch.int64 or not slot_mapping.is_contiguous():
        raise ValueError("slot_mapping must be a contiguous int64 tensor")
    if inverse.dtype != torch.int32 or not inverse.is_contiguous():
        raise ValueError("inverse must be a contiguous int32 tensor")
    _abi.check(_abi.lib().mxfp4_build_inverse(
        slot_mapping.data_ptr(), slot_mapping.numel(), num_blocks, block_size,
        inverse.data_ptr(), inverse.numel() * 4, _stream(stream)))
    return inverse


def mxfp4_store_by_slot(src: torch.Tensor, num_tokens: int, inverse: torch.Tensor,
                        cache: torch.Tensor, num_blocks: int, block_size: int,
                        block_stride_rows: int, group: int = GROUP_SIZE, stream=None) -> None:
    """``mxfp4_store_by_slot`` of the C ABI: the store in slot order, from the
    inverse map of the batch's slot mapping."""
    _need_cuda(src, inverse, cache)
    if src.dtype != torch.bfloat16 or src.dim() != 2 or not _unit_inner(src):
        raise ValueError("src must be a bf16 [tokens, latent] tensor with unit inner stride")
    if inverse.dtype != torch.int32 or not inverse.is_contiguous():
        raise ValueError("inverse must be a contiguous int32 tensor")
    if cache.dtype != torch.uint8:
        raise ValueError(f"the cache is raw bytes (torch.uint8), not {cache.dtype}")
    if num_tokens > src.shape[0]:
        raise ValueError("num_tokens exceeds the rows of src")
    _need_cache_extent(cache, num_blocks, block_size, block_stride_rows, src.shape[1], group)
    _abi.check(_abi.lib().mxfp4_store_by_slot(
        src.data_ptr(), num_tokens, src.shape[1], _strides(src)[0], inverse.data_ptr(),
        inverse.numel() * 4, cache.data_ptr(), num_blocks, block_size, block_stride_rows, group,
        _stream(stream)))


def mxfp4_store_slot_order_noalloc(src: torch.Tensor, slot_mapping: torch.Tensor,
                                   cache: torch.Tensor, num_blocks: int, block_size: int,
                                   block_stride_rows: int, group: int = GROUP_SIZE,
                                   stream=None) -> None:
    """``mxfp4_store_slot_order_noalloc`` of the C ABI: the slot-order store
    with its inverse map in the library's static per-GPU array (no
    allocation, no workspace; calls that overlap on one GPU race)."""
    _need_cuda(src, slot_mapping, cache)
    if src.dtype != torch.bfloat16 or src.dim() != 2 or not _unit_inner(src):
        raise ValueError("src must be a bf16 [tokens, latent] tensor with unit inner stride")
    if slot_mapping.dtype != torch.int64 or not slot_mapping.is_contiguous():
        raise ValueError("slot_mapping must be a contiguous int64 tensor")
    if cache.dtype != torch.uint8:
        raise ValueError(f"the cache is raw bytes (torch.uint8), not {cache.dtype}")
    num_tokens = slot_mapping.numel()
    if num_tokens > src.shape[0]:
        raise ValueError("slot_mapping has more entries than src has rows")
    _need_cache_extent(cache, num_blocks, block_size, block_stride_rows, src.shape[1], group)
    _abi.check(_abi.lib().mxfp4_store_slot_order_noalloc(
        src.data_ptr(), num_tokens, src.shape[1], _strides(src)[0], slot_mapping.data_ptr(),
        cache.data_ptr(), num_blocks, block_size, block_stride_rows, group, _stream(stream)))


def mxfp4_gather_dequant(cache: torch.Tensor, num_blocks: int, block_size: int,
                         block_stride_rows: int, latent: int, slots: torch.Tensor,
                         out: torch.Tensor, group: int = GROUP_SIZE, stream=None) -> torch.Tensor:
    """``mxfp4_gather_dequant`` of the C ABI; fills bf16 ``out`` [n, latent]."""
    _need_cuda(cache, slots, out)
    if slots.dtype != torch.int64 or not slots.is_contiguous():
        raise ValueError("slots must be a contiguous int64 tensor")
    if out.dtype != torch.bfloat16 or out.dim() != 2 or not _unit_inner(out):
        raise ValueError("out must be a bf16 [n, latent] tensor with unit inner stride")
    if out.shape[0] < slots.numel() or out.shape[1] != latent:
        raise ValueError("out must have at least len(slots) rows of `latent` values")
    _need_cache_extent(cache, num_blocks, block_size, block_stride_rows, latent, group)
    _abi.check(_abi.lib().mxfp4_gather_dequant(
        cache.data_ptr(), num_blocks, block_size, block_stride_rows, latent, group,
        slots.data_ptr(), slots.numel(), out.data_ptr(), _strides(out)[0], _stream(stream)))
    return out


def _rope_args(latent, positions, cos_sin, kv_cache, slot_mapping, width):
    _need_cuda(latent, positions, cos_sin, kv_cache, slot_mapping)
    if latent.dtype != torch.bfloat16 or latent.dim() != 2 or latent.shape[1] != 512 \
            or not latent.is_contiguous():
        raise ValueError("latent must be a contiguous bf16 [tokens, 512] tensor")
    if positions.dtype != torch.int64 or not positions.is_contiguous():
        raise ValueError("positions must be a contiguous int64 tensor")
    if slot_mapping.dtype != torch.int64 or not slot_mapping.is_contiguous():
        raise ValueError("slot_mapping must be a contiguous int64 tensor")
    if cos_sin.dtype != torch.float32 or cos_sin.dim() != 2 or cos_sin.stride(1) != 1:
        raise ValueError("cos_sin must be an fp32 [rows, >=64] table with unit inner stride")
    if kv_cache.dtype != torch.uint8 or kv_cache.dim() != 3 or kv_cache.shape[2] != width \
            or kv_cache.stride(2) != 1 or kv_cache.stride(1) != width:
        raise ValueError(f"kv_cache must be uint8 [blocks, block, {width}] with contiguous pages")
    num_tokens = slot_mapping.numel()
    if num_tokens > min(latent.shape[0], positions.numel()):
        raise ValueError("slot_mapping is longer than latent or positions")
    return (latent.data_ptr(), positions.data_ptr(), cos_sin.data_ptr(), cos_sin.stride(0),
            cos_sin.shape[0], kv_cache.data_ptr(), kv_cache.stride(0), kv_cache.shape[1],
            kv_cache.shape[0], slot_mapping.data_ptr(), num_tokens)


def mxfp8_rope_store(latent, positions, cos_sin, kv_cache, slot_mapping, compress_ratio,
                     sanitize_nans: bool = True, stream=None) -> None:
    """``mxfp8_rope_store`` of the C ABI; ``kv_cache`` is uint8 [blocks, B, 528]."""
    args = _rope_args(latent, positions, cos_sin, kv_cache, slot_mapping, MXFP8_RECORD_BYTES)
    _abi.check(_abi.lib().mxfp8_rope_store(*args, int(compress_ratio), int(bool(sanitize_nans)),
                                           _stream(stream)))


def nvfp4_rope_store(latent, positions, cos_sin, kv_cache, slot_mapping, compress_ratio,
                     sanitize_nans: bool = True, stream=None) -> None:
    """``nvfp4_rope_store`` of the C ABI; ``kv_cache`` is uint8 [blocks, B, 288]."""
    args = _rope_args(latent, positions, cos_sin, kv_cache, slot_mapping, NVFP4_RECORD_BYTES)
    _abi.check(_abi.lib().nvfp4_rope_store(*args, int(compress_ratio), int(bool(sanitize_nans)),
                                           _stream(stream)))


def v4_rope_store(latent, positions, cos_sin, kv_cache, slot_mapping, compress_ratio,
                  sanitize_nans: bool = True, stream=None) -> None:
    """``v4_rope_store`` of the C ABI; ``kv_cache`` is uint8 [blocks, B, 584]."""
    args = _rope_args(latent, positions, cos_sin, kv_cache, slot_mapping, V4_RECORD_BYTES)
    _abi.check(_abi.lib().v4_rope_store(*args, int(compress_ratio), int(bool(sanitize_nans)),
                                        _stream(stream)))


def save_ring_rows(rows: torch.Tensor, slot_mapping: torch.Tensor, state_cache: torch.Tensor,
                   stream=None) -> None:
    """Store fp32 [kv, score] rows to their ring slots, skipping slot -1
    [P2 `save_ring_rows`]: same arguments and checks as the page's wrapper;
    ``state_cache`` is the fp32 ring [blocks, capacity, width]."""
    _need_cuda(rows, slot_mapping, state_cache)
    if rows.dtype != torch.float32 or rows.dim() != 2 or not _unit_inner(rows):
        raise ValueError("rows must be fp32 [n, width] with unit inner stride")
    if state_cache.dtype != torch.float32 or state_cache.dim() != 3 or state_cache.stride(2) != 1 \
            or state_cache.shape[2] != rows.shape[1]:
        raise ValueError("state_cache must be fp32 [blocks, capacity, width] with unit inner stride")
    if slot_mapping.dtype != torch.int64 or not slot_mapping.is_contiguous() \
            or slot_mapping.numel() != rows.shape[0]:
        raise ValueError("slot_mapping must be contiguous int64 with one entry per row")
    _abi.check(_abi.lib().save_ring_rows(
        rows.data_ptr(), rows.shape[0], rows.shape[1], _strides(rows)[0], slot_mapping.data_ptr(),
        state_cache.data_ptr(), state_cache.shape[0], state_cache.shape[1], state_cache.stride(0),
        state_cache.stride(1), _stream(stream)))


def fused_save_compress_norm_cr1(kv_score: torch.Tensor, slot_mapping: torch.Tensor,
                                 rms_norm_weight: torch.Tensor, rms_norm_eps: float,
                                 latent_out: torch.Tensor, stream=None) -> None:
    """Compress ratio 1 of [P2 `fused_save_compress_norm`]: RMSNorm of each
    valid token's fp32 [512] row with the bf16 weight, into bf16
    ``latent_out`` (rows of tokens with slot < 0 are not written)."""
    _need_cuda(kv_score, slot_mapping, rms_norm_weight, latent_out)
    if kv_score.dtype != torch.float32 or kv_score.dim() != 2 or not _unit_inner(kv_score) \
            or kv_score.shape[1] != 512:
        raise ValueError("kv_score must be fp32 [tokens, 512] with unit inner stride")
    if rms_norm_weight.dtype != torch.bfloat16 or rms_norm_weight.numel() != 512 \
            or not rms_norm_weight.is_contiguous():
        raise ValueError("rms_norm_weight must be contiguous bf16 [512]")
    if latent_out.dtype != torch.bfloat16 or latent_out.dim() != 2 or not _unit_inner(latent_out) \
            or latent_out.shape[1] != 512:
        raise ValueError("latent_out must be bf16 [tokens, 512] with unit inner stride")
    n = slot_mapping.numel()
    if slot_mapping.dtype != torch.int64 or not slot_mapping.is_contiguous() \
            or n > kv_score.shape[0] or n > latent_out.shape[0]:
        raise ValueError("slot_mapping must be contiguous int64 with at most one entry per row")
    _abi.check(_abi.lib().fused_save_compress_norm_cr1(
        kv_score.data_ptr(), n, 512, _strides(kv_score)[0], slot_mapping.data_ptr(),
        rms_norm_weight.data_ptr(), float(rms_norm_eps), latent_out.data_ptr(), _strides(latent_out)[0],
        _stream(stream)))


def sparse_mla_attention_splits_advised(num_tokens: int, num_heads: int, topk: int) -> int:
    """Split count the library advises for this shape (1: no split)."""
    return int(_abi.lib().sparse_mla_attention_splits_advised(num_tokens, num_heads, topk))


def sparse_mla_attention_workspace_bytes(num_tokens: int, num_heads: int, splits: int) -> int:
    n = int(_abi.lib().sparse_mla_attention_workspace_bytes(num_tokens, num_heads, splits))
    if n < 0:
        _abi.check(n)
    return n


def sparse_mla_attention(q: torch.Tensor, cache: torch.Tensor, indices: torch.Tensor, scale: float,
                         sink: torch.Tensor | None = None, out: torch.Tensor | None = None,
                         stream=None, splits: int | None = None,
                         workspace: torch.Tensor | None = None) -> torch.Tensor:
    """Sparse MLA attention of bf16 queries [T, H, 512] over the listed slots
    (int32 [T, topk], invalid entries skipped) of a paged MXFP4 cache (the
    view rules of ``store_mxfp4_mla``), keys = values = the dequantized rows;
    optional fp32 per-head sinks [P3 read path].  Returns bf16 [T, H, 512].
    ``splits`` > 1 walks each (token, head block) as that many key ranges
    and merges them (the split form for few tokens); None takes the library's
    advice.  The split form needs a device ``workspace`` (uint8, at least
    ``sparse_mla_attention_workspace_bytes``); one is allocated when None."""
    _need_cuda(q, cache, indices)
    if q.dtype != torch.bfloat16 or q.dim() != 3 or q.shape[2] != 512 or not _unit_inner(q):
        raise ValueError("q must be bf16 [tokens, heads, 512] with unit inner stride")
    if indices.dtype != torch.int32 or indices.dim() != 2 or indices.shape[0] != q.shape[0] \
            or (indices.shape[1] > 1 and not _unit_inner(indices)):
        raise ValueError("indices must be int32 [tokens, topk] with unit inner stride")
    num_blocks, block_size, stride_rows = resolve_paged_view(cache, 512)
    if sink is not None and (sink.dtype != torch.float32 or sink.numel() != q.shape[1]
                             or not sink.is_contiguous()):
        raise ValueError("sink must be contiguous fp32 [heads]")
    if out is None:
        out = torch.empty(q.shape, dtype=torch.bfloat16, device=q.device)
    if out.dtype != torch.bfloat16 or out.shape != q.shape or not _unit_inner(out):
        raise ValueError("out must be bf16 shaped like q with unit inner stride")
    tokens, heads, topk = q.shape[0], q.shape[1], indices.shape[1]
    if splits is None:
        splits = sparse_mla_attention_splits_advised(tokens, heads, topk)
    qs, os_ = _strides(q), _strides(out)
    args = (q.data_ptr(), tokens, heads, 512, qs[0], qs[1], cache.data_ptr(),
            num_blocks, block_size, stride_rows, indices.data_ptr(), topk,
            max(_strides(indices)[0], topk), float(scale), None if sink is None else sink.data_ptr(),
            out.data_ptr(), os_[0], os_[1])
    if splits == 1:
        _abi.check(_abi.lib().sparse_mla_attention(*args, _stream(stream)))
        return out
    need = sparse_mla_attention_workspace_bytes(tokens, heads, splits)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    if workspace.dtype != torch.uint8 or not workspace.is_contiguous() or workspace.device != q.device:
        raise ValueError("workspace must be a contiguous uint8 tensor on the query's device")
    _abi.check(_abi.lib().sparse_mla_attention_split(*args, int(splits), workspace.data_ptr(),
                                                     workspace.numel(), _stream(stream)))
    return out


# ------------------------------------------------------------------ page-level API

def resolve_paged_view(cache: torch.Tensor, latent: int, group: int = GROUP_SIZE):
    """(num_blocks, block_size, block_stride_rows) of a cache tensor [P1
    `store_mxfp4_mla`]: a 3-D paged [blocks, block, row_bytes] view whose block
    stride is a whole number of rows, or any tensor viewable as flat rows."""
    if cache.dtype != torch.uint8:
        raise ValueError(f"the cache is raw bytes (torch.uint8), not {cache.dtype}")
    pitch = row_bytes(latent, group)
    if cache.dim() == 3:
        num_blocks, block_size, width = cache.shape
        if width != pitch or tuple(cache.stride()[1:]) != (pitch, 1) or cache.stride(0) % pitch:
            raise ValueError(
                f"a paged cache is [blocks, block, {pitch}] with {pitch}-byte rows packed "
                f"in each block and blocks a multiple of {pitch} bytes apart; this one has "
                f"shape {tuple(cache.shape)}, strides {cache.stride()}")
        return num_blocks, block_size, cache.stride(0) // pitch
    flat = cache.view(-1)
    if flat.numel() % pitch:
        raise ValueError(f"a flat cache holds whole {pitch}-byte rows; {flat.numel()} bytes do not divide")
    n = flat.numel() // pitch
    return 1, n, n


def store_mxfp4_mla(kv_c_normed: torch.Tensor, slot_mapping: torch.Tensor,
                    cache: torch.Tensor, group: int = GROUP_SIZE, stream=None,
                    inverse: torch.Tensor | None = None) -> None:
    """Quantize the MLA latent to MXFP4 and write it into the paged cache
    [P1 `store_mxfp4_mla`]: same arguments and view resolution as the page's
    wrapper.  The work is one ``mxfp4_store`` launch; when an int32
    ``inverse`` workspace (``mxfp4_inverse_workspace``) is given and the
    library advises the slot-order form for this shape, it is
    ``mxfp4_build_inverse`` + ``mxfp4_store_by_slot`` instead (same bytes)."""
    if kv_c_normed.dim() != 2:
        raise ValueError(f"kv_c_normed is a 2-D [tokens, latent] tensor; this one is {tuple(kv_c_normed.shape)}")
    num_blocks, block_size, stride_rows = resolve_paged_view(cache, kv_c_normed.shape[1], group)
    num_tokens = slot_mapping.numel()
    if num_tokens == 0:
        return
    if inverse is not None and mxfp4_slot_order_advised(num_tokens, kv_c_normed.shape[1],
                                                        num_blocks, block_size):
        mxfp4_build_inverse(slot_mapping, num_blocks, block_size, inverse, stream)
        mxfp4_store_by_slot(kv_c_normed, num_tokens, inverse, cache, num_blocks, block_size,
                            stride_rows, group, stream)
    else:
        mxfp4_store(kv_c_normed, slot_mapping, cache, num_blocks, block_size, stride_rows,
                    group, stream)


def rope_quant_insert(latent, positions, cos_sin_cache, kv_cache, slot_mapping,
                      compress_ratio: int, sanitize_nans: bool = True, stream=None) -> None:
    """GPT-J RoPE + quantized insert into a paged compressed cache whose
    record width selects the format [P2 `rope_quant_insert`]: 528 -> MXFP8,
    288 -> NVFP4, 584 -> V4.  The plain bf16/fp8 rows of the page are not
    provided by this library."""
    width = kv_cache.shape[-1] if kv_cache.dim() == 3 else None
    fns = {MXFP8_RECORD_BYTES: mxfp8_rope_store, NVFP4_RECORD_BYTES: nvfp4_rope_store,
           V4_RECORD_BYTES: v4_rope_store}
    if kv_cache.dtype != torch.uint8 or width not in fns:
        raise ValueError(f"no insert writes {width}-byte records of {kv_cache.dtype} "
                         f"(uint8 records of 528, 288 or 584 bytes are known)")
    fn = fns[width]
    fn(latent, positions, cos_sin_cache, kv_cache, slot_mapping, compress_ratio,
       sanitize_nans, stream)
