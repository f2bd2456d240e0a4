"""MI355X-native MXFP4 paged KV-cache store.

libmxstore.so (hand-written HIP for gfx950, C ABI in include/mxstore.h)
quantizes a bf16 MLA latent to MXFP4 (E2M1 codes + one E8M0 scale per 32
values, 272 bytes per 512-wide token) and scatters it into a paged cache; a
gather-dequant companion unpacks slots back to bf16; two RoPE+quant inserts
write the MXFP8 (528 B), NVFP4 (288 B) and V4 (584 B) compressed-cache records; the
ring-state save and the compress-ratio-1 RMSNorm precede those inserts; a
sparse MLA attention reads the packed cache directly (MFMA).
"""

from .ops import (
    GROUP_SIZE,
    fused_save_compress_norm_cr1,
    MXFP8_RECORD_BYTES,
    NVFP4_RECORD_BYTES,
    V4_RECORD_BYTES,
    mxfp4_gather_dequant,
    mxfp4_store,
    mxfp4_build_inverse,
    mxfp4_inverse_bytes,
    mxfp4_inverse_workspace,
    mxfp4_slot_order_advised,
    mxfp4_store_by_slot,
    mxfp4_store_slot_order_noalloc,
    mxfp8_rope_store,
    nvfp4_rope_store,
    v4_rope_store,
    resolve_paged_view,
    rope_quant_insert,
    row_bytes,
    save_ring_rows,
    sparse_mla_attention,
    sparse_mla_attention_splits_advised,
    sparse_mla_attention_workspace_bytes,
    store_mxfp4_mla,
)
from ._abi import MxError

__all__ = [
    "GROUP_SIZE",
    "MXFP8_RECORD_BYTES",
    "NVFP4_RECORD_BYTES",
    "V4_RECORD_BYTES",
    "MxError",
    "fused_save_compress_norm_cr1",
    "mxfp4_gather_dequant",
    "mxfp4_store",
    "mxfp4_build_inverse",
    "mxfp4_inverse_bytes",
    "mxfp4_inverse_workspace",
    "mxfp4_slot_order_advised",
    "mxfp4_store_by_slot",
    "mxfp4_store_slot_order_noalloc",
    "mxfp8_rope_store",
    "nvfp4_rope_store",
    "v4_rope_store",
    "resolve_paged_view",
    "rope_quant_insert",
    "row_bytes",
    "save_ring_rows",
    "sparse_mla_attention",
    "sparse_mla_attention_splits_advised",
    "sparse_mla_attention_workspace_bytes",
    "store_mxfp4_mla",
]
