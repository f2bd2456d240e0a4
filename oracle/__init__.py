"""CPU oracle for the MXFP4 paged-cache store and its companions.

TEST INFRASTRUCTURE ONLY.  This package is the checker the GPU library is
compared against.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it.  It shares no code with
the HIP library (``mxfp4_paged_cache_store_amd``) and never imports it.

The arithmetic lives in ``mxoracle.c`` (plain scalar C, built with gcc
``-O2 -ffp-contract=off``, no fast-math); this module only builds it and
marshals numpy arrays.  Each C function cites the page section it follows.
``Oracle(path)`` binds one build; the module-level functions use the build of
``mxoracle.c`` itself (the tests also bind deliberately broken builds to show
that the pins catch them).
"""

from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(_HERE, "mxoracle.c")
_BUILD_DIR = os.path.join(_HERE, "_build")
_LIB_PATH = os.path.join(_BUILD_DIR, "libmxoracle.so")

_default = None
_lock = threading.Lock()

_i64 = ctypes.c_int64
_i32 = ctypes.c_int32
_vp = ctypes.c_void_p


def build(src: str = SRC, out: str = _LIB_PATH) -> str:
    """Compile the oracle C source into a shared library (always rebuilds)."""
    os.makedirs(os.path.dirname(out), exist_ok=True)
    tmp = out + ".tmp"
    cmd = [
        "gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math",
        "-fPIC", "-shared", "-Wall", "-Wextra", "-o", tmp, src, "-lm",
    ]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def _bind(lib: ctypes.CDLL) -> ctypes.CDLL:
    lib.orc_row_bytes.restype = _i64
    lib.orc_row_bytes.argtypes = [_i64, _i32]
    lib.orc_ceil_pow2_exponent.restype = ctypes.c_int
    lib.orc_ceil_pow2_exponent.argtypes = [ctypes.c_float]
    lib.orc_e2m1_code.restype = ctypes.c_int
    lib.orc_e2m1_code.argtypes = [ctypes.c_float]
    lib.orc_e4m3_encode.restype = ctypes.c_uint8
    lib.orc_e4m3_encode.argtypes = [ctypes.c_float]
    lib.orc_e4m3_value.restype = ctypes.c_double
    lib.orc_e4m3_value.argtypes = [ctypes.c_uint8]
    lib.orc_e4m3_encode_array.restype = None
    lib.orc_e4m3_encode_array.argtypes = [_vp, _i64, _vp]
    lib.orc_mxfp4_dequant_bf16.restype = ctypes.c_uint16
    lib.orc_mxfp4_dequant_bf16.argtypes = [ctypes.c_int, ctypes.c_int]
    lib.orc_mxfp4_quantize_row.restype = None
    lib.orc_mxfp4_quantize_row.argtypes = [_vp, _i64, _vp]
    lib.orc_mxfp4_store.restype = ctypes.c_int
    lib.orc_mxfp4_store.argtypes = [_vp, _i64, _i64, _i64, _vp, _vp, _i64, _i64, _i64]
    lib.orc_mxfp4_gather_dequant.restype = ctypes.c_int
    lib.orc_mxfp4_gather_dequant.argtypes = [_vp, _i64, _i64, _i64, _i64, _vp, _i64, _vp, _i64]
    for name in ("orc_mxfp8_rope_store", "orc_nvfp4_rope_store", "orc_v4_rope_store"):
        fn = getattr(lib, name)
        fn.restype = ctypes.c_int
        fn.argtypes = [_vp, _vp, _vp, _i64, _i64, _vp, _i64, _i64, _i64, _vp, _i64, _i32, _i32]
    lib.orc_rope_rotate.restype = ctypes.c_int
    lib.orc_rope_rotate.argtypes = [_vp, _vp, _vp, _i64, _i64, _i64, _i32, _i32, _vp, _vp]
    lib.orc_sparse_mla_attention.restype = ctypes.c_int
    lib.orc_sparse_mla_attention.argtypes = [_vp, _i64, _i64, _i64, _vp, _i64, _i64, _i64, _vp, _i64,
                                             ctypes.c_double, _vp, _vp]
    lib.orc_f32_to_bf16.restype = ctypes.c_uint16
    lib.orc_f32_to_bf16.argtypes = [ctypes.c_float]
    lib.orc_rmsnorm_cr1.restype = ctypes.c_int
    lib.orc_rmsnorm_cr1.argtypes = [_vp, _i64, _i64, _i64, _vp, _vp, ctypes.c_float, _vp, _i64]
    lib.orc_save_ring_rows.restype = ctypes.c_int
    lib.orc_save_ring_rows.argtypes = [_vp, _i64, _i64, _i64, _vp, _vp, _i64, _i64, _i64, _i64]
    return lib


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise ValueError(f"oracle {what}: arguments outside the contract (rc={rc})")


def _run_chunks(run, n: int, threads: int) -> None:
    if threads <= 1 or n < 2 * threads:
        run(0, n)
        return
    bounds = [n * i // threads for i in range(threads + 1)]
    workers = [threading.Thread(target=run, args=(bounds[i], bounds[i + 1]))
               for i in range(threads)]
    for w in workers:
        w.start()
    for w in workers:
        w.join()


class Oracle:
    """The oracle's functions over one build of the C source (numpy in/out)."""

    def __init__(self, lib_path: str):
        self.lib = _bind(ctypes.CDLL(lib_path))

    # ------------------------------------------------------------ scalars

    def row_bytes(self, latent: int, group: int = 32) -> int:
        return int(self.lib.orc_row_bytes(latent, group))

    def ceil_pow2_exponent(self, v: float) -> int:
        return int(self.lib.orc_ceil_pow2_exponent(v))

    def e2m1_code(self, q: float) -> int:
        return int(self.lib.orc_e2m1_code(q))

    def e4m3_encode(self, v: float) -> int:
        return int(self.lib.orc_e4m3_encode(v))

    def e4m3_encode_array(self, v: np.ndarray) -> np.ndarray:
        v = np.ascontiguousarray(v, dtype=np.float32)
        out = np.empty(v.shape, dtype=np.uint8)
        self.lib.orc_e4m3_encode_array(_ptr(v), v.size, _ptr(out))
        return out

    def e4m3_value(self, b: int) -> float:
        return float(self.lib.orc_e4m3_value(b))

    def dequant_bf16(self, code: int, scale_byte: int) -> int:
        return int(self.lib.orc_mxfp4_dequant_bf16(code, scale_byte))

    # ------------------------------------------------------------ arrays

    def quantize_row(self, x_bf16_bits: np.ndarray) -> np.ndarray:
        """One latent row (uint16 bf16 bits) -> packed row bytes (uint8)."""
        x = np.ascontiguousarray(x_bf16_bits, dtype=np.uint16)
        out = np.zeros(self.row_bytes(x.size), dtype=np.uint8)
        self.lib.orc_mxfp4_quantize_row(_ptr(x), x.size, _ptr(out))
        return out

    def mxfp4_store(self, src: np.ndarray, slot_mapping: np.ndarray, cache: np.ndarray,
                    num_blocks: int, block_size: int, block_stride_rows: int,
                    threads: int = 1) -> None:
        """Store rows of ``src`` (uint16 [T, latent] bf16 bits) into ``cache``.

        ``src`` may be a row-strided view (unit inner stride).  ``cache`` is
        the flat uint8 buffer holding the paged layer view; it is modified in
        place.  ``threads > 1`` splits the tokens into contiguous ranges run
        concurrently (distinct slots never share bytes).
        """
        assert src.dtype == np.uint16 and src.ndim == 2
        assert slot_mapping.dtype == np.int64 and cache.dtype == np.uint8
        assert cache.flags.c_contiguous and slot_mapping.flags.c_contiguous
        num_tokens = slot_mapping.size
        if num_tokens == 0:  # nothing stored (an empty array's strides mean nothing)
            return
        assert src.strides[1] == 2
        latent = src.shape[1]
        src_row_stride = src.strides[0] // 2
        need = ((num_blocks - 1) * block_stride_rows + block_size) * self.row_bytes(latent)
        assert cache.size >= need, "cache buffer smaller than the paged view"
        assert src.shape[0] >= num_tokens
        lib = self.lib
        base = src.__array_interface__["data"][0]

        def run(lo: int, hi: int) -> None:
            rc = lib.orc_mxfp4_store(
                base + lo * src_row_stride * 2, hi - lo, latent, src_row_stride,
                slot_mapping.ctypes.data + lo * 8, _ptr(cache),
                num_blocks, block_size, block_stride_rows)
            _check(rc, "mxfp4_store")

        _run_chunks(run, num_tokens, threads)

    def mxfp4_gather_dequant(self, cache: np.ndarray, num_blocks: int, block_size: int,
                             block_stride_rows: int, latent: int, slots: np.ndarray,
                             out: np.ndarray | None = None) -> np.ndarray:
        """Dequantize the rows of ``slots`` to bf16 bits, uint16 [n, latent]."""
        assert slots.dtype == np.int64 and slots.flags.c_contiguous
        n = slots.size
        if out is None:
            out = np.zeros((n, latent), dtype=np.uint16)
        assert out.dtype == np.uint16 and out.flags.c_contiguous and out.shape[0] >= n
        rc = self.lib.orc_mxfp4_gather_dequant(
            _ptr(cache), num_blocks, block_size, block_stride_rows, latent,
            _ptr(slots), n, _ptr(out), out.shape[1])
        _check(rc, "mxfp4_gather_dequant")
        return out

    def _rope_store(self, fn_name, width, latent, positions, cos_sin, cache, block, num_blocks,
                    cache_block_stride, slot_mapping, compress_ratio, sanitize, threads) -> None:
        assert latent.dtype == np.uint16 and latent.flags.c_contiguous
        assert latent.shape[1] == 512
        assert positions.dtype == np.int64 and slot_mapping.dtype == np.int64
        assert positions.flags.c_contiguous and slot_mapping.flags.c_contiguous
        assert cos_sin.dtype == np.float32 and cos_sin.strides[1] == 4
        assert cache.dtype == np.uint8 and cache.flags.c_contiguous
        stride = block * width if cache_block_stride is None else cache_block_stride
        assert cache.size >= (num_blocks - 1) * stride + block * width, \
            "cache buffer smaller than the paged view"
        n = slot_mapping.size
        assert n <= min(latent.shape[0], positions.size)
        fn = getattr(self.lib, fn_name)

        def run(lo: int, hi: int) -> None:
            rc = fn(_ptr(latent) + lo * 1024, _ptr(positions) + lo * 8, cos_sin.ctypes.data,
                    cos_sin.strides[0] // 4, cos_sin.shape[0], _ptr(cache), stride, block,
                    num_blocks, _ptr(slot_mapping) + lo * 8, hi - lo, compress_ratio,
                    int(bool(sanitize)))
            _check(rc, fn_name)

        _run_chunks(run, n, threads)

    def rope_rotate(self, latent, positions, cos_sin, compress_ratio, sanitize=True):
        """The inserts' rotated fp32 latent: (float32 [T, 512], bool [T]
        written); rows of tokens the gate rejects are NaN."""
        assert latent.dtype == np.uint16 and latent.flags.c_contiguous
        assert latent.shape[1] == 512
        assert positions.dtype == np.int64 and positions.flags.c_contiguous
        assert cos_sin.dtype == np.float32 and cos_sin.strides[1] == 4
        n = positions.size
        assert latent.shape[0] >= n
        out = np.full((n, 512), np.nan, dtype=np.float32)
        written = np.zeros(n, dtype=np.uint8)
        rc = self.lib.orc_rope_rotate(
            _ptr(latent), _ptr(positions), cos_sin.ctypes.data, cos_sin.strides[0] // 4,
            cos_sin.shape[0], n, compress_ratio, int(bool(sanitize)), _ptr(out), _ptr(written))
        _check(rc, "rope_rotate")
        return out, written.astype(bool)

    def mxfp8_rope_store(self, latent, positions, cos_sin, cache, block, num_blocks,
                         slot_mapping, compress_ratio, sanitize=True,
                         cache_block_stride=None, threads: int = 1) -> None:
        """MXFP8 insert into the flat uint8 ``cache`` (pages ``cache_block_stride``
        bytes apart, default one block of records).  ``threads > 1`` runs
        contiguous token ranges concurrently (distinct slots never share bytes)."""
        self._rope_store("orc_mxfp8_rope_store", 528, latent, positions, cos_sin, cache, block,
                         num_blocks, cache_block_stride, slot_mapping, compress_ratio, sanitize,
                         threads)

    def nvfp4_rope_store(self, latent, positions, cos_sin, cache, block, num_blocks,
                         slot_mapping, compress_ratio, sanitize=True,
                         cache_block_stride=None, threads: int = 1) -> None:
        """NVFP4 insert; arguments as for ``mxfp8_rope_store``."""
        self._rope_store("orc_nvfp4_rope_store", 288, latent, positions, cos_sin, cache, block,
                         num_blocks, cache_block_stride, slot_mapping, compress_ratio, sanitize,
                         threads)

    def v4_rope_store(self, latent, positions, cos_sin, cache, block, num_blocks,
                      slot_mapping, compress_ratio, sanitize=True,
                      cache_block_stride=None, threads: int = 1) -> None:
        """V4 insert; arguments as for ``mxfp8_rope_store``."""
        self._rope_store("orc_v4_rope_store", 584, latent, positions, cos_sin, cache, block,
                         num_blocks, cache_block_stride, slot_mapping, compress_ratio, sanitize,
                         threads)

    def sparse_mla_attention(self, q_bits: np.ndarray, cache: np.ndarray, num_blocks: int,
                             block_size: int, block_stride_rows: int, indices: np.ndarray,
                             scale: float, sink: np.ndarray | None = None) -> np.ndarray:
        """Attention of bf16 queries ``q_bits`` [T, H, latent] (uint16 bit
        patterns) over the listed slots ``indices`` (int32 [T, topk]) of an
        MXFP4 cache; returns float64 [T, H, latent]."""
        q = np.ascontiguousarray(q_bits, dtype=np.uint16)
        assert q.ndim == 3
        idx = np.ascontiguousarray(indices, dtype=np.int32)
        assert idx.ndim == 2 and idx.shape[0] == q.shape[0]
        t, h, latent = q.shape
        out = np.zeros((t, h, latent), dtype=np.float64)
        s = None if sink is None else np.ascontiguousarray(sink, dtype=np.float32)
        assert s is None or s.size == h
        rc = self.lib.orc_sparse_mla_attention(
            _ptr(q), t, h, latent, _ptr(np.ascontiguousarray(cache)), num_blocks, block_size,
            block_stride_rows, _ptr(idx), idx.shape[1], float(scale),
            None if s is None else _ptr(s), _ptr(out))
        _check(rc, "sparse_mla_attention")
        return out

    def f32_to_bf16(self, x: float) -> int:
        return int(self.lib.orc_f32_to_bf16(float(x)))

    def save_ring_rows(self, rows: np.ndarray, slot_mapping: np.ndarray,
                       state: np.ndarray) -> None:
        """Copy fp32 ``rows`` [n, width] (row-strided allowed) into the ring
        ``state`` [blocks, capacity, width] (strided views allowed) in place."""
        assert rows.dtype == np.float32 and rows.ndim == 2
        assert state.dtype == np.float32 and state.ndim == 3 and state.strides[2] == 4
        assert slot_mapping.dtype == np.int64 and slot_mapping.flags.c_contiguous
        assert slot_mapping.size == rows.shape[0] and state.shape[2] == rows.shape[1]
        if rows.shape[0] == 0:  # nothing to copy (an empty array's strides mean nothing)
            return
        assert rows.strides[1] == 4
        rc = self.lib.orc_save_ring_rows(
            rows.ctypes.data, rows.shape[0], rows.shape[1], rows.strides[0] // 4,
            _ptr(slot_mapping), state.ctypes.data, state.shape[0], state.shape[1],
            state.strides[0] // 4, state.strides[1] // 4)
        _check(rc, "save_ring_rows")


    def rmsnorm_cr1(self, kv: np.ndarray, slot_mapping: np.ndarray, weight_bf16: np.ndarray,
                    eps: float, out: np.ndarray | None = None) -> np.ndarray:
        """RMSNorm of the valid fp32 rows of ``kv`` [n, width] (row-strided
        allowed) with a bf16-bits weight, in double; rows of invalid tokens of
        ``out`` (float64 [n, width]) are left as they are (NaN if allocated
        here)."""
        assert kv.dtype == np.float32 and kv.ndim == 2
        assert slot_mapping.dtype == np.int64 and slot_mapping.flags.c_contiguous
        w = np.ascontiguousarray(weight_bf16, dtype=np.uint16)
        n, width = slot_mapping.size, kv.shape[1]
        assert w.size == width and kv.shape[0] >= n
        if out is None:
            out = np.full((n, width), np.nan, dtype=np.float64)
        assert out.dtype == np.float64 and out.flags.c_contiguous
        if n == 0:  # no rows (an empty array's strides mean nothing)
            return out
        assert kv.strides[1] == 4
        rc = self.lib.orc_rmsnorm_cr1(kv.ctypes.data, n, width, kv.strides[0] // 4,
                                      _ptr(slot_mapping), _ptr(w), eps, _ptr(out), out.shape[1])
        _check(rc, "rmsnorm_cr1")
        return out


def default() -> Oracle:
    """The oracle built from oracle/mxoracle.c (built on first use)."""
    global _default
    with _lock:
        if _default is None:
            if not os.path.exists(_LIB_PATH) or (
                os.path.getmtime(_LIB_PATH) < os.path.getmtime(SRC)
            ):
                build()
            _default = Oracle(_LIB_PATH)
        return _default


def _forward(name):
    def fn(*args, **kwargs):
        return getattr(default(), name)(*args, **kwargs)
    fn.__name__ = name
    fn.__doc__ = getattr(Oracle, name).__doc__
    return fn


row_bytes = _forward("row_bytes")
ceil_pow2_exponent = _forward("ceil_pow2_exponent")
e2m1_code = _forward("e2m1_code")
e4m3_encode = _forward("e4m3_encode")
e4m3_encode_array = _forward("e4m3_encode_array")
e4m3_value = _forward("e4m3_value")
dequant_bf16 = _forward("dequant_bf16")
quantize_row = _forward("quantize_row")
mxfp4_store = _forward("mxfp4_store")
mxfp4_gather_dequant = _forward("mxfp4_gather_dequant")
rope_rotate = _forward("rope_rotate")
mxfp8_rope_store = _forward("mxfp8_rope_store")
nvfp4_rope_store = _forward("nvfp4_rope_store")
save_ring_rows = _forward("save_ring_rows")
rmsnorm_cr1 = _forward("rmsnorm_cr1")
v4_rope_store = _forward("v4_rope_store")
f32_to_bf16 = _forward("f32_to_bf16")
sparse_mla_attention = _forward("sparse_mla_attention")
