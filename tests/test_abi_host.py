"""CPU checks of the C ABI: the library loads, exports every symbol that
include/*.h declares, and rejects arguments outside the contract with the
documented status before any device work (these calls never reach HIP)."""

import glob
import os
import re

import pytest

from mxfp4_paged_cache_store_amd import _abi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    names = []
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for m in re.finditer(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?\b([a-z_][a-z0-9_]*)\s*\(", text, re.M):
            names.append(m.group(1))
    return sorted(set(names))


def test_exports_every_declared_symbol(mxlib):
    declared = declared_functions()
    assert set(declared) == set(_abi.EXPORTED), declared
    for name in declared:
        assert hasattr(mxlib, name), name


def test_row_bytes(mxlib):
    assert mxlib.mx_row_bytes(512, 32) == 272
    assert mxlib.mx_row_bytes(128, 32) == 68
    assert mxlib.mx_row_bytes(1024, 32) == 544
    assert mxlib.mx_row_bytes(100, 32) == _abi.MX_E_SHAPE
    assert mxlib.mx_row_bytes(512, 0) == _abi.MX_E_SHAPE


FAKE = 0x10000  # an aligned address that is never dereferenced


def store(mxlib, **kw):
    a = dict(src=FAKE, n=4, latent=512, stride=512, slots=FAKE, cache=FAKE, nb=1, bs=8,
             bsr=8, group=32)
    a.update(kw)
    return mxlib.mxfp4_store(a["src"], a["n"], a["latent"], a["stride"], a["slots"], a["cache"],
                             a["nb"], a["bs"], a["bsr"], a["group"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(group=16), _abi.MX_E_SHAPE),
    (dict(latent=500, stride=512), _abi.MX_E_SHAPE),
    (dict(latent=64, stride=64), _abi.MX_E_SHAPE),
    (dict(latent=4096, stride=4096), _abi.MX_E_SHAPE),
    (dict(bsr=4), _abi.MX_E_STRIDE),
    (dict(stride=256), _abi.MX_E_STRIDE),
    (dict(n=-1), _abi.MX_E_RANGE),
    (dict(nb=0), _abi.MX_E_RANGE),
    (dict(nb=1 << 30, bs=64, bsr=64), _abi.MX_E_RANGE),
    (dict(src=0), _abi.MX_E_NULL),
    (dict(slots=0), _abi.MX_E_NULL),
    (dict(src=FAKE + 8), _abi.MX_E_ALIGN),
    (dict(stride=516), _abi.MX_E_ALIGN),
    (dict(cache=FAKE + 2), _abi.MX_E_ALIGN),
])
def test_store_rejects(mxlib, kw, status):
    assert store(mxlib, **kw) == status
    assert mxlib.mx_last_error().decode()


def test_store_zero_tokens_is_a_noop(mxlib):
    # null pointers are fine when there is nothing to do; nothing is launched
    assert store(mxlib, n=0, src=0, slots=0, cache=0) == _abi.MX_OK
    assert mxlib.mx_last_error().decode() == ""


def dequant(mxlib, **kw):
    a = dict(cache=FAKE, nb=1, bs=8, bsr=8, latent=512, group=32, slots=FAKE, n=3, out=FAKE,
             ostride=512)
    a.update(kw)
    return mxlib.mxfp4_gather_dequant(a["cache"], a["nb"], a["bs"], a["bsr"], a["latent"],
                                      a["group"], a["slots"], a["n"], a["out"], a["ostride"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(group=64), _abi.MX_E_SHAPE),
    (dict(bsr=7), _abi.MX_E_STRIDE),
    (dict(ostride=100), _abi.MX_E_STRIDE),
    (dict(ostride=520 + 4), _abi.MX_E_ALIGN),
    (dict(out=FAKE + 4), _abi.MX_E_ALIGN),
    (dict(n=-2), _abi.MX_E_RANGE),
    (dict(out=0), _abi.MX_E_NULL),
])
def test_dequant_rejects(mxlib, kw, status):
    assert dequant(mxlib, **kw) == status


def test_dequant_empty_list_is_a_noop(mxlib):
    assert dequant(mxlib, n=0, cache=0, slots=0, out=0) == _abi.MX_OK


def rope(mxlib, fn, **kw):
    a = dict(latent=FAKE, pos=FAKE, cs=FAKE, cstride=64, crows=100, cache=FAKE, pstride=64 * 528,
             block=64, nb=4, slots=FAKE, n=5, cr=4, san=1)
    a.update(kw)
    return getattr(mxlib, fn)(a["latent"], a["pos"], a["cs"], a["cstride"], a["crows"], a["cache"],
                              a["pstride"], a["block"], a["nb"], a["slots"], a["n"], a["cr"],
                              a["san"], None)


@pytest.mark.parametrize("fn,width", [("mxfp8_rope_store", 528), ("nvfp4_rope_store", 288),
                                      ("v4_rope_store", 584)])
@pytest.mark.parametrize("kw,status", [
    (dict(cr=0), _abi.MX_E_ARG),
    (dict(pstride=100), _abi.MX_E_STRIDE),
    (dict(cstride=32), _abi.MX_E_STRIDE),
    (dict(block=0), _abi.MX_E_RANGE),
    (dict(n=-1), _abi.MX_E_RANGE),
    (dict(latent=0), _abi.MX_E_NULL),
    (dict(cache=FAKE + 8), _abi.MX_E_ALIGN),
])
def test_rope_rejects(mxlib, fn, width, kw, status):
    if "pstride" not in kw:
        kw = dict(kw, pstride=64 * width)
    assert rope(mxlib, fn, **kw) == status


@pytest.mark.parametrize("fn", ["mxfp8_rope_store", "nvfp4_rope_store", "v4_rope_store"])
def test_rope_empty_is_a_noop(mxlib, fn):
    assert rope(mxlib, fn, n=0, latent=0, pos=0, cs=0, cache=0, slots=0, pstride=64 * 592) == _abi.MX_OK


def test_nvfp4_record_width_checked(mxlib):
    # a 288-byte page stride is too small for the 528-byte record
    assert rope(mxlib, "mxfp8_rope_store", pstride=64 * 288) == _abi.MX_E_STRIDE
    assert rope(mxlib, "v4_rope_store", pstride=64 * 528) == _abi.MX_E_STRIDE


def test_inverse_bytes_and_advice(mxlib):
    assert mxlib.mxfp4_inverse_bytes(1, 4_500_000) == 18_000_000
    assert mxlib.mxfp4_inverse_bytes(1000, 150) == 600_000
    assert mxlib.mxfp4_inverse_bytes(3, 3) == 48           # 36 rounded up to 16
    assert mxlib.mxfp4_inverse_bytes(0, 5) == _abi.MX_E_RANGE
    assert mxlib.mxfp4_inverse_bytes(1 << 30, 64) == _abi.MX_E_RANGE
    adv = mxlib.mxfp4_slot_order_advised
    assert adv(4_500_000, 512, 1, 4_500_000) == 1
    # rows past 256 MiB (986,895 rows of 272 B; 493,447 of 544 B; 246,723 of 1088 B)
    assert adv(986_896, 512, 1, 986_896) == 1 and adv(986_895, 512, 1, 986_895) == 0
    assert adv(493_448, 1024, 1000, 900) == 1 and adv(493_447, 1024, 1000, 900) == 0
    assert adv(246_724, 2048, 1000, 400) == 1 and adv(246_723, 2048, 1000, 400) == 0
    assert adv(1 << 20, 512, 1, 1 << 21) == 1
    assert adv(16_384, 512, 8192, 64) == 0      # sparse prefill: scatter
    assert adv(1 << 17, 512, 1, 1 << 17) == 0   # fits the Infinity Cache: scatter
    assert adv(2_000_000, 256, 1, 2_000_000) == 0   # latent below 512
    assert adv(2_000_000, 512, 1, 4_000_001) == 0   # under half of the slots


def build_inverse(mxlib, **kw):
    a = dict(slots=FAKE, n=10, nb=2, bs=8, inv=FAKE, nbytes=64)
    a.update(kw)
    return mxlib.mxfp4_build_inverse(a["slots"], a["n"], a["nb"], a["bs"], a["inv"], a["nbytes"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(nbytes=60), _abi.MX_E_RANGE),
    (dict(n=-1), _abi.MX_E_RANGE),
    (dict(n=1 << 31), _abi.MX_E_RANGE),
    (dict(nb=0), _abi.MX_E_RANGE),
    (dict(inv=0), _abi.MX_E_NULL),
    (dict(slots=0), _abi.MX_E_NULL),
    (dict(inv=FAKE + 4), _abi.MX_E_ALIGN),
])
def test_build_inverse_rejects(mxlib, kw, status):
    assert build_inverse(mxlib, **kw) == status


def store_by_slot(mxlib, **kw):
    a = dict(src=FAKE, n=4, latent=512, stride=512, inv=FAKE, nbytes=32, cache=FAKE, nb=1, bs=8,
             bsr=8, group=32)
    a.update(kw)
    return mxlib.mxfp4_store_by_slot(a["src"], a["n"], a["latent"], a["stride"], a["inv"], a["nbytes"],
                                     a["cache"], a["nb"], a["bs"], a["bsr"], a["group"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(latent=256, stride=256), _abi.MX_E_SHAPE),
    (dict(group=16), _abi.MX_E_SHAPE),
    (dict(inv=0), _abi.MX_E_NULL),
    (dict(inv=FAKE + 8), _abi.MX_E_ALIGN),
    (dict(bsr=4), _abi.MX_E_STRIDE),
    (dict(n=-3), _abi.MX_E_RANGE),
    (dict(nbytes=16), _abi.MX_E_RANGE),          # 8 slots need 32 bytes of map
    (dict(nb=3, bsr=8, nbytes=64), _abi.MX_E_RANGE),  # 24 slots need 96
])
def test_store_by_slot_rejects(mxlib, kw, status):
    assert store_by_slot(mxlib, **kw) == status


def test_store_by_slot_empty_is_a_noop(mxlib):
    assert store_by_slot(mxlib, n=0, src=0, inv=0, cache=0) == _abi.MX_OK


def ring(mxlib, **kw):
    a = dict(rows=FAKE, n=3, width=1024, rstride=1024, slots=FAKE, state=FAKE, nb=4, cap=8,
             sstride=8 * 1024, srstride=1024)
    a.update(kw)
    return mxlib.save_ring_rows(a["rows"], a["n"], a["width"], a["rstride"], a["slots"], a["state"],
                                a["nb"], a["cap"], a["sstride"], a["srstride"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(width=1022, rstride=1024), _abi.MX_E_SHAPE),
    (dict(width=0), _abi.MX_E_SHAPE),
    (dict(n=-1), _abi.MX_E_RANGE),
    (dict(cap=0), _abi.MX_E_RANGE),
    (dict(rstride=1000), _abi.MX_E_STRIDE),
    (dict(sstride=7 * 1024), _abi.MX_E_STRIDE),
    (dict(rstride=1026), _abi.MX_E_ALIGN),
    (dict(rows=FAKE + 4), _abi.MX_E_ALIGN),
    (dict(state=0), _abi.MX_E_NULL),
])
def test_ring_rows_rejects(mxlib, kw, status):
    assert ring(mxlib, **kw) == status


def test_ring_rows_empty_is_a_noop(mxlib):
    assert ring(mxlib, n=0, rows=0, slots=0, state=0) == _abi.MX_OK


def norm(mxlib, **kw):
    a = dict(kv=FAKE, n=3, width=512, kstride=512, slots=FAKE, w=FAKE, eps=1e-6, out=FAKE,
             ostride=512)
    a.update(kw)
    return mxlib.fused_save_compress_norm_cr1(a["kv"], a["n"], a["width"], a["kstride"], a["slots"],
                                              a["w"], a["eps"], a["out"], a["ostride"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(width=1024, kstride=1024), _abi.MX_E_SHAPE),
    (dict(n=-1), _abi.MX_E_RANGE),
    (dict(eps=-1e-6), _abi.MX_E_ARG),
    (dict(eps=float("nan")), _abi.MX_E_ARG),
    (dict(eps=float("inf")), _abi.MX_E_ARG),
    (dict(kstride=500), _abi.MX_E_STRIDE),
    (dict(ostride=511), _abi.MX_E_STRIDE),
    (dict(kstride=514), _abi.MX_E_ALIGN),
    (dict(kv=FAKE + 8), _abi.MX_E_ALIGN),
    (dict(out=FAKE + 2), _abi.MX_E_ALIGN),
    (dict(w=0), _abi.MX_E_NULL),
])
def test_compress_norm_rejects(mxlib, kw, status):
    assert norm(mxlib, **kw) == status


def test_compress_norm_empty_is_a_noop(mxlib):
    assert norm(mxlib, n=0, kv=0, slots=0, w=0, out=0) == _abi.MX_OK


def attn(mxlib, **kw):
    a = dict(q=FAKE, n=3, h=16, latent=512, qts=16 * 512, qhs=512, cache=FAKE, nb=4, bs=64, bsr=64,
             idx=FAKE, topk=128, istride=128, scale=0.05, sink=None, out=FAKE, ots=16 * 512, ohs=512)
    a.update(kw)
    return mxlib.sparse_mla_attention(a["q"], a["n"], a["h"], a["latent"], a["qts"], a["qhs"], a["cache"],
                                      a["nb"], a["bs"], a["bsr"], a["idx"], a["topk"], a["istride"],
                                      a["scale"], a["sink"], a["out"], a["ots"], a["ohs"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(latent=256, qhs=256, ohs=256), _abi.MX_E_SHAPE),
    (dict(h=24), _abi.MX_E_SHAPE),
    (dict(h=0), _abi.MX_E_SHAPE),
    (dict(n=-1), _abi.MX_E_RANGE),
    (dict(topk=-1), _abi.MX_E_RANGE),
    (dict(nb=1 << 26), _abi.MX_E_RANGE),
    (dict(scale=float("nan")), _abi.MX_E_ARG),
    (dict(scale=float("inf")), _abi.MX_E_ARG),
    (dict(qhs=500), _abi.MX_E_STRIDE),
    (dict(qts=512), _abi.MX_E_STRIDE),
    (dict(istride=100), _abi.MX_E_STRIDE),
    (dict(qhs=516, qts=16 * 516), _abi.MX_E_ALIGN),
    (dict(q=FAKE + 8), _abi.MX_E_ALIGN),
    (dict(cache=FAKE + 4), _abi.MX_E_ALIGN),
    (dict(idx=0), _abi.MX_E_NULL),
    (dict(bsr=32), _abi.MX_E_STRIDE),
])
def test_attention_rejects(mxlib, kw, status):
    assert attn(mxlib, **kw) == status


def test_attention_empty_is_a_noop(mxlib):
    assert attn(mxlib, n=0, q=0, cache=0, idx=0, out=0) == _abi.MX_OK


def attn_split(mxlib, splits, ws, ws_bytes, **kw):
    a = dict(q=FAKE, n=3, h=16, latent=512, qts=16 * 512, qhs=512, cache=FAKE, nb=4, bs=64, bsr=64,
             idx=FAKE, topk=128, istride=128, scale=0.05, sink=None, out=FAKE, ots=16 * 512, ohs=512)
    a.update(kw)
    return mxlib.sparse_mla_attention_split(a["q"], a["n"], a["h"], a["latent"], a["qts"], a["qhs"], a["cache"],
                                            a["nb"], a["bs"], a["bsr"], a["idx"], a["topk"], a["istride"],
                                            a["scale"], a["sink"], a["out"], a["ots"], a["ohs"], splits, ws,
                                            ws_bytes, None)


def test_attention_split_workspace_and_advice(mxlib):
    wsb = mxlib.sparse_mla_attention_workspace_bytes
    assert wsb(3, 16, 1) == 0
    assert wsb(3, 16, 4) == ((3 * 16 * 4 * 514 * 4 + 255) // 256) * 256
    assert wsb(64, 32, 8) == 64 * 32 * 8 * 514 * 4          # already a multiple of 256
    assert wsb(3, 16, 0) == _abi.MX_E_RANGE and wsb(3, 16, 65) == _abi.MX_E_RANGE
    assert wsb(-1, 16, 2) == _abi.MX_E_RANGE and wsb(3, 0, 2) == _abi.MX_E_RANGE
    adv = mxlib.sparse_mla_attention_splits_advised
    assert adv(4096, 32, 2048) == 1          # 4096 workgroups already fill the GPU
    assert adv(64, 32, 2048) == 4            # 64 workgroups -> 256
    assert adv(256, 32, 2048) == 1           # 256 workgroups: one per CU already
    assert adv(128, 32, 2048) == 2
    assert adv(1, 32, 2048) == 16            # capped at two tiles per range (32 tiles)
    assert adv(1, 128, 65536) == 64          # capped at 64 ranges
    assert adv(8, 32, 64) == 1               # one tile: nothing to split
    assert adv(8, 48, 2048) == 11            # 16-head blocks: 8 * 3 workgroups -> 264
    assert adv(0, 32, 2048) == 1 and adv(8, 24, 2048) == 1 and adv(8, 32, 0) == 1


def test_attention_split_rejects(mxlib):
    need = mxlib.sparse_mla_attention_workspace_bytes(3, 16, 4)
    assert attn_split(mxlib, 0, FAKE, need) == _abi.MX_E_RANGE
    assert attn_split(mxlib, 65, FAKE, need) == _abi.MX_E_RANGE
    assert attn_split(mxlib, 4, FAKE, need - 1) == _abi.MX_E_RANGE
    assert attn_split(mxlib, 4, None, need) == _abi.MX_E_NULL
    assert attn_split(mxlib, 4, FAKE + 8, need) == _abi.MX_E_ALIGN
    assert attn_split(mxlib, 4, FAKE, need, h=24) == _abi.MX_E_SHAPE   # the shared checks still apply
    assert attn_split(mxlib, 4, None, 0, n=0, q=0, cache=0, idx=0, out=0) == _abi.MX_OK
