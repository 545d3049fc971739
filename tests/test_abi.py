"""The C-ABI library loads, exports every symbol include/*.h declares, and
rejects bad arguments on the host before touching the device (CPU only: no
call here reaches a kernel launch)."""

from __future__ import annotations

import ctypes
import glob
import os
import re

import pytest

from exact_tiled_attention_fa_amd import _abi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
A16 = 1 << 20  # a 16-byte-aligned dummy address; never dereferenced on these paths


def declared_functions():
    names = []
    for hdr in glob.glob(os.path.join(ROOT, "include", "*.h")):
        src = open(hdr).read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        names += re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*(fa_[a-z0-9_]+)\s*\(",
                            src, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    if not _abi.lib_path().exists():
        pytest.fail(f"{_abi.lib_path()} missing: run `python -c 'import __graft_entry__ as g; g.build()'`")
    return _abi.load()


def test_header_declares_the_abi():
    assert declared_functions() == sorted(
        ["fa_fwd", "fa_fwd_ex", "fa_fwd_fp8", "fa_fwd_fp8_ex", "fa_bwd", "fa_bwd_ex",
         "fa_bwd_workspace_size",
         "fa_decode", "fa_decode_noalloc",
         "fa_decode_paged", "fa_decode_workspace_size", "fa_last_error", "fa_info"])


def test_every_declared_symbol_is_exported(lib):
    raw = ctypes.CDLL(str(_abi.lib_path()))
    for name in declared_functions():
        assert hasattr(raw, name), f"{name} not exported"
        assert name in _abi.SIGNATURES, f"{name} has no binding"


def test_info_names_target(lib):
    info = _abi.fa_info()
    assert "gfx950" in info and "{64,128,256}" in info


def fwd(**kw):
    a = dict(q=A16, k=A16, v=A16, o=A16, lse=A16, B=1, Hq=2, Hkv=1, Lq=8, Lk=8, D=64, scale=0.125,
             causal=0, dtype=_abi.FA_BF16, stream=None)
    a.update(kw)
    return _abi.fa_fwd(*a.values())


@pytest.mark.parametrize("kw,status,text", [
    (dict(q=None), _abi.FA_ERR_INVALID_ARGUMENT, "q is NULL"),
    (dict(lse=None), _abi.FA_ERR_INVALID_ARGUMENT, "lse is NULL"),
    (dict(k=A16 + 2), _abi.FA_ERR_INVALID_ARGUMENT, "not 16-byte aligned"),
    (dict(B=0), _abi.FA_ERR_INVALID_ARGUMENT, "sizes must be >= 1"),
    (dict(Lq=-3), _abi.FA_ERR_INVALID_ARGUMENT, "sizes must be >= 1"),
    (dict(Hq=3, Hkv=2), _abi.FA_ERR_INVALID_ARGUMENT, "not a multiple"),
    (dict(D=96), _abi.FA_ERR_UNSUPPORTED, "head_dim 96"),
    (dict(D=32), _abi.FA_ERR_UNSUPPORTED, "head_dim 32"),
    (dict(dtype=7), _abi.FA_ERR_UNSUPPORTED, "dtype 7"),
    (dict(scale=float("nan")), _abi.FA_ERR_INVALID_ARGUMENT, "not finite"),
    (dict(scale=float("inf")), _abi.FA_ERR_INVALID_ARGUMENT, "not finite"),
    (dict(B=1 << 20, Hq=1 << 10, Hkv=1, Lq=1 << 12), _abi.FA_ERR_INVALID_ARGUMENT, "too large"),
])
def test_fwd_rejects(lib, kw, status, text):
    assert fwd(**kw) == status
    assert text in _abi.fa_last_error()


def dec(**kw):
    a = dict(q=A16, k=A16, v=A16, seqlens=A16, o=A16, lse=A16, B=2, Hq=8, Hkv=2, Lk_max=64,
             D=128, scale=0.1, num_splits=8, workspace=A16, workspace_bytes=1 << 30,
             dtype=_abi.FA_BF16, stream=None)
    a.update(kw)
    return _abi.fa_decode(*a.values())


@pytest.mark.parametrize("kw,status,text", [
    (dict(seqlens=None), _abi.FA_ERR_INVALID_ARGUMENT, "seqlens is NULL"),
    (dict(seqlens=A16 + 2), _abi.FA_ERR_INVALID_ARGUMENT, "4-byte aligned"),
    (dict(workspace=None), _abi.FA_ERR_INVALID_ARGUMENT, "workspace is NULL"),
    (dict(workspace_bytes=100), _abi.FA_ERR_INVALID_ARGUMENT, "needs"),
    (dict(num_splits=0), _abi.FA_ERR_INVALID_ARGUMENT, "num_splits=0"),
    (dict(num_splits=65), _abi.FA_ERR_INVALID_ARGUMENT, "num_splits=65"),
    (dict(Hq=6, Hkv=4), _abi.FA_ERR_INVALID_ARGUMENT, "not a multiple"),
    (dict(D=80), _abi.FA_ERR_UNSUPPORTED, "head_dim 80"),
    (dict(Lk_max=0), _abi.FA_ERR_INVALID_ARGUMENT, "sizes must be >= 1"),
])
def test_decode_rejects(lib, kw, status, text):
    assert dec(**kw) == status
    assert text in _abi.fa_last_error()


def test_workspace_size(lib):
    assert _abi.fa_decode_workspace_size(128, 32, 128, 8) == 128 * 32 * 8 * (128 + 1) * 4
    assert _abi.fa_decode_workspace_size(1, 1, 64, 1) == 65 * 4
    assert _abi.fa_decode_workspace_size(1, 1, 64, 0) == 0
    assert _abi.fa_decode_workspace_size(0, 1, 64, 1) == 0
    assert _abi.fa_decode_workspace_size(1, 1, 64, 65) == 0


def test_binding_refuses_missing_library(monkeypatch, tmp_path):
    monkeypatch.setenv("FA_GFX950_LIB", str(tmp_path / "nope.so"))
    monkeypatch.setattr(_abi, "_lib", None)
    with pytest.raises(RuntimeError, match="no fallback"):
        _abi.load()


def fwd_ex(**kw):
    a = dict(q=A16, k=A16, v=A16, o=A16, lse=A16, cu_q=None, cu_k=None, B=1, Hq=2, Hkv=1, Lq=8,
             Lk=8, total_q=0, total_k=0, D=64, scale=0.125, causal=0, wl=-1, wr=-1,
             dtype=_abi.FA_BF16, stream=None)
    a.update(kw)
    return _abi.fa_fwd_ex(*a.values())


@pytest.mark.parametrize("kw,status,text", [
    (dict(cu_q=A16), _abi.FA_ERR_INVALID_ARGUMENT, "both be set"),
    (dict(cu_k=A16), _abi.FA_ERR_INVALID_ARGUMENT, "both be set"),
    (dict(cu_q=A16 + 2, cu_k=A16, total_q=8, total_k=8), _abi.FA_ERR_INVALID_ARGUMENT,
     "4-byte aligned"),
    (dict(cu_q=A16, cu_k=A16, total_q=0, total_k=8), _abi.FA_ERR_INVALID_ARGUMENT, "total_q=0"),
    (dict(cu_q=A16, cu_k=A16, total_q=8, total_k=0), _abi.FA_ERR_INVALID_ARGUMENT, "total_k=0"),
    (dict(cu_q=A16, cu_k=A16, total_q=1 << 30, total_k=1 << 30, Hq=1, wl=4),
     _abi.FA_ERR_INVALID_ARGUMENT, "2^30"),
    (dict(cu_q=A16, cu_k=A16, total_q=1 << 30, total_k=8, Hq=4, Hkv=1),
     _abi.FA_ERR_INVALID_ARGUMENT, "exceeds 2^31-1"),
    (dict(Hkv=1 << 20, Hq=1 << 20, D=64), _abi.FA_ERR_INVALID_ARGUMENT, "2^25"),
    (dict(o=None), _abi.FA_ERR_INVALID_ARGUMENT, "o is NULL"),
    (dict(D=48), _abi.FA_ERR_UNSUPPORTED, "head_dim 48"),
])
def test_fwd_ex_rejects(lib, kw, status, text):
    assert fwd_ex(**kw) == status
    assert text in _abi.fa_last_error()


def test_fwd_is_fwd_ex_without_masks(lib):
    """fa_fwd validates exactly as fa_fwd_ex with NULL offsets and no window."""
    for kw in (dict(B=0), dict(Hq=3, Hkv=2), dict(D=96), dict(scale=float("nan"))):
        st1 = fwd(**kw)
        e1 = _abi.fa_last_error()
        st2 = fwd_ex(**kw)
        assert (st1, e1) == (st2, _abi.fa_last_error())


def dec_paged(**kw):
    a = dict(q=A16, k=A16, v=A16, ks=None, vs=None, table=A16, seqlens=A16, o=A16, lse=A16, B=2,
             Hq=8, Hkv=2, D=128, num_pages=10, page_size=16, max_pages=4, scale=0.1,
             num_splits=8, kf=_abi.FA_KV_NATIVE, vf=_abi.FA_KV_NATIVE, workspace=A16,
             workspace_bytes=1 << 30, dtype=_abi.FA_BF16, stream=None)
    a.update(kw)
    return _abi.fa_decode_paged(*a.values())


@pytest.mark.parametrize("kw,status,text", [
    (dict(table=None), _abi.FA_ERR_INVALID_ARGUMENT, "block_table is NULL"),
    (dict(seqlens=None), _abi.FA_ERR_INVALID_ARGUMENT, "seqlens is NULL"),
    (dict(table=A16 + 2), _abi.FA_ERR_INVALID_ARGUMENT, "4-byte aligned"),
    (dict(page_size=8), _abi.FA_ERR_INVALID_ARGUMENT, "page_size=8"),
    (dict(page_size=48), _abi.FA_ERR_INVALID_ARGUMENT, "page_size=48"),
    (dict(page_size=1 << 17), _abi.FA_ERR_INVALID_ARGUMENT, "power of two"),
    (dict(kf=_abi.FA_KV_INT8), _abi.FA_ERR_INVALID_ARGUMENT, "k_scales"),
    (dict(kf=_abi.FA_KV_INT8, ks=A16, vf=_abi.FA_KV_INT8), _abi.FA_ERR_INVALID_ARGUMENT,
     "v_scales"),
    (dict(vf=_abi.FA_KV_INT8, vs=A16), _abi.FA_ERR_UNSUPPORTED, "int8 values need int8 keys"),
    (dict(kf=5), _abi.FA_ERR_UNSUPPORTED, "kv formats"),
    (dict(num_pages=0), _abi.FA_ERR_INVALID_ARGUMENT, "sizes must be >= 1"),
    (dict(max_pages=0), _abi.FA_ERR_INVALID_ARGUMENT, "sizes must be >= 1"),
    (dict(max_pages=1 << 20, page_size=1 << 12), _abi.FA_ERR_INVALID_ARGUMENT, "2^31-1"),
    (dict(workspace_bytes=64), _abi.FA_ERR_INVALID_ARGUMENT, "needs"),
    (dict(D=96), _abi.FA_ERR_UNSUPPORTED, "head_dim 96"),
    (dict(num_splits=65), _abi.FA_ERR_INVALID_ARGUMENT, "num_splits=65"),
])
def test_decode_paged_rejects(lib, kw, status, text):
    assert dec_paged(**kw) == status
    assert text in _abi.fa_last_error()


def bwd(**kw):
    a = dict(q=A16, k=A16, v=A16, o=A16, do=A16, lse=A16, dq=A16, dk=A16, dv=A16, B=1, Hq=2, Hkv=1,
             Lq=8, Lk=8, D=64, scale=0.125, causal=1, wl=-1, wr=-1, ws=A16, ws_bytes=1 << 30,
             dtype=_abi.FA_BF16, stream=None)
    a.update(kw)
    return _abi.fa_bwd(*a.values())


@pytest.mark.parametrize("kw,status,text", [
    (dict(do=None), _abi.FA_ERR_INVALID_ARGUMENT, "dout is NULL"),
    (dict(dk=A16 + 8), _abi.FA_ERR_INVALID_ARGUMENT, "dk is not 16-byte aligned"),
    (dict(ws=None), _abi.FA_ERR_INVALID_ARGUMENT, "workspace is NULL"),
    (dict(ws_bytes=16), _abi.FA_ERR_INVALID_ARGUMENT, "needs"),
    (dict(D=96), _abi.FA_ERR_UNSUPPORTED, "head_dim 96"),
    (dict(Hq=3, Hkv=2), _abi.FA_ERR_INVALID_ARGUMENT, "not a multiple"),
    (dict(Lk=0), _abi.FA_ERR_INVALID_ARGUMENT, "sizes must be >= 1"),
    (dict(scale=float("inf")), _abi.FA_ERR_INVALID_ARGUMENT, "not finite"),
    (dict(Hq=1 << 20, Hkv=1 << 20, D=64), _abi.FA_ERR_INVALID_ARGUMENT, "2^25"),
])
def test_bwd_rejects(lib, kw, status, text):
    assert bwd(**kw) == status
    assert text in _abi.fa_last_error()


def bwd_ex(**kw):
    a = dict(q=A16, k=A16, v=A16, o=A16, do=A16, lse=A16, dq=A16, dk=A16, dv=A16, cu_q=None,
             cu_k=None, B=1, Hq=2, Hkv=1, Lq=8, Lk=8, total_q=0, total_k=0, D=64, scale=0.125,
             causal=1, wl=-1, wr=-1, ws=A16, ws_bytes=1 << 30, dtype=_abi.FA_BF16, stream=None)
    a.update(kw)
    return _abi.fa_bwd_ex(*a.values())


@pytest.mark.parametrize("kw,status,text", [
    (dict(cu_q=A16), _abi.FA_ERR_INVALID_ARGUMENT, "both be set"),
    (dict(cu_k=A16), _abi.FA_ERR_INVALID_ARGUMENT, "both be set"),
    (dict(cu_q=A16 + 2, cu_k=A16, total_q=8, total_k=8), _abi.FA_ERR_INVALID_ARGUMENT,
     "4-byte aligned"),
    (dict(cu_q=A16, cu_k=A16, total_q=0, total_k=8), _abi.FA_ERR_INVALID_ARGUMENT, "total_q=0"),
    (dict(cu_q=A16, cu_k=A16, total_q=8, total_k=0), _abi.FA_ERR_INVALID_ARGUMENT, "total_k=0"),
    (dict(cu_q=A16, cu_k=A16, total_q=8, total_k=8, D=32), _abi.FA_ERR_UNSUPPORTED,
     "head_dim 32"),
    (dict(cu_q=A16, cu_k=A16, total_q=1 << 30, total_k=8, Hq=4), _abi.FA_ERR_INVALID_ARGUMENT,
     "exceeds 2^31-1"),
    (dict(cu_q=A16, cu_k=A16, total_q=8, total_k=8, ws_bytes=16), _abi.FA_ERR_INVALID_ARGUMENT,
     "needs"),
])
def test_bwd_ex_rejects(lib, kw, status, text):
    assert bwd_ex(**kw) == status
    assert text in _abi.fa_last_error()


def test_bwd_is_bwd_ex_without_offsets(lib):
    """fa_bwd validates exactly as fa_bwd_ex with NULL offsets."""
    for kw in (dict(B=0), dict(Hq=3, Hkv=2), dict(D=96), dict(scale=float("nan")),
               dict(ws_bytes=16), dict(dk=A16 + 8)):
        st1 = bwd(**kw)
        e1 = _abi.fa_last_error()
        st2 = bwd_ex(**kw)
        assert (st1, e1) == (st2, _abi.fa_last_error())


def test_bwd_workspace_size(lib):
    assert _abi.fa_bwd_workspace_size(2, 3, 33) == 2 * 2 * 3 * 64 * 4
    assert _abi.fa_bwd_workspace_size(1, 1, 32) == 2 * 32 * 4
    assert _abi.fa_bwd_workspace_size(0, 1, 32) == 0


def fp8(**kw):
    a = dict(q=A16, k=A16, vt=A16, o=A16, lse=A16, B=1, Hq=2, Hkv=1, Lq=8, Lk=8, D=128, vts=64,
             scale=0.1, qd=0.0625, kd=0.0625, vd=0.0625, causal=1, wl=-1, wr=-1,
             dtype=_abi.FA_BF16, stream=None)
    a.update(kw)
    return _abi.fa_fwd_fp8(*a.values())


@pytest.mark.parametrize("kw,status,text", [
    (dict(vt=None), _abi.FA_ERR_INVALID_ARGUMENT, "vt8 is NULL"),
    (dict(vts=32), _abi.FA_ERR_INVALID_ARGUMENT, "vt_stride=32"),
    (dict(vts=64, Lk=65), _abi.FA_ERR_INVALID_ARGUMENT, "vt_stride=64"),
    (dict(qd=0.0), _abi.FA_ERR_INVALID_ARGUMENT, "descales"),
    (dict(vd=float("nan")), _abi.FA_ERR_INVALID_ARGUMENT, "descales"),
    (dict(D=96), _abi.FA_ERR_UNSUPPORTED, "fp8 head_dim 96"),
    (dict(dtype=5), _abi.FA_ERR_UNSUPPORTED, "dtype 5"),
    (dict(Hq=3, Hkv=2), _abi.FA_ERR_INVALID_ARGUMENT, "not a multiple"),
])
def test_fp8_rejects(lib, kw, status, text):
    assert fp8(**kw) == status
    assert text in _abi.fa_last_error()


def fp8_ex(**kw):
    a = dict(q=A16, k=A16, vt=A16, o=A16, lse=A16, cu_q=None, cu_k=None, B=1, Hq=2, Hkv=1, Lq=8,
             Lk=8, total_q=0, total_k=0, D=128, vts=64, scale=0.1, qd=0.0625, kd=0.0625,
             vd=0.0625, causal=1, wl=-1, wr=-1, dtype=_abi.FA_BF16, stream=None)
    a.update(kw)
    return _abi.fa_fwd_fp8_ex(*a.values())


PACKED8 = dict(cu_q=A16, cu_k=A16, B=2, Lq=8, Lk=8, total_q=16, total_k=16, vts=128)


@pytest.mark.parametrize("kw,status,text", [
    (dict(cu_q=A16), _abi.FA_ERR_INVALID_ARGUMENT, "both be set"),
    (dict(cu_k=A16), _abi.FA_ERR_INVALID_ARGUMENT, "both be set"),
    (dict(PACKED8, cu_q=A16 + 2), _abi.FA_ERR_INVALID_ARGUMENT, "4-byte aligned"),
    (dict(PACKED8, total_q=0), _abi.FA_ERR_INVALID_ARGUMENT, "total_q=0"),
    (dict(PACKED8, vts=64), _abi.FA_ERR_INVALID_ARGUMENT, "vt_stride=64"),
    (dict(PACKED8, vts=100), _abi.FA_ERR_INVALID_ARGUMENT, "multiple of 64"),
    (dict(PACKED8, D=32), _abi.FA_ERR_UNSUPPORTED, "fp8 head_dim 32"),
    (dict(PACKED8, total_q=1 << 30, Hq=4, Hkv=1), _abi.FA_ERR_INVALID_ARGUMENT, "2^31-1"),
])
def test_fp8_ex_rejects(lib, kw, status, text):
    assert fp8_ex(**kw) == status
    assert text in _abi.fa_last_error()


def test_fp8_is_fp8_ex_without_offsets(lib):
    """fa_fwd_fp8 validates exactly as fa_fwd_fp8_ex with NULL offsets."""
    for kw in (dict(vt=None), dict(vts=32), dict(vts=64, Lk=65), dict(qd=0.0), dict(D=96),
               dict(dtype=5), dict(Hq=3, Hkv=2)):
        st1 = fp8(**kw)
        e1 = _abi.fa_last_error()
        st2 = fp8_ex(**kw)
        assert (st1, e1) == (st2, _abi.fa_last_error())


def test_last_error_is_per_thread(lib):
    """Each host thread sees the text of its own last failing call."""
    import threading

    results = {}
    go = threading.Barrier(2)

    def worker(name, kw, expect):
        go.wait()
        for _ in range(200):
            st = fwd(**kw)
            txt = _abi.fa_last_error()
            if st == _abi.FA_OK or expect not in txt:
                results[name] = txt
                return
        results[name] = "ok"

    a = threading.Thread(target=worker, args=("a", dict(D=96), "head_dim 96"))
    b = threading.Thread(target=worker, args=("b", dict(Hq=3, Hkv=2), "not a multiple"))
    a.start(); b.start(); a.join(); b.join()
    assert results == {"a": "ok", "b": "ok"}, results


def test_probe_library_rejects():
    """The benchmark's MFMA probe lives in its own library (not in libfa's
    ABI) and checks its host arguments before it asks for the device."""
    import ctypes

    from exact_tiled_attention_fa_amd import probe

    if not probe.lib_path().exists():
        pytest.fail(f"{probe.lib_path()} missing: run the build")
    plib = probe.load()
    assert not hasattr(ctypes.CDLL(str(_abi.lib_path())), "fa_probe_mfma_bf16")
    fl = ctypes.c_double(0.0)
    bad = [dict(operands=None), dict(out=None), dict(operand_bytes=0), dict(operand_bytes=24),
           dict(iters=0), dict(iters=(1 << 20) + 1), dict(operands=A16 + 8)]
    for kw in bad:
        a = dict(operands=A16, operand_bytes=1 << 20, out=A16, out_len=1 << 20, iters=4)
        a.update(kw)
        st = plib.fa_probe_mfma_bf16(a["operands"], a["operand_bytes"], a["out"], a["out_len"],
                                     a["iters"], ctypes.byref(fl), None)
        assert st == 1, kw
    assert fl.value == 0.0


def test_decode_noalloc_rejects_before_the_device(lib):
    """fa_decode_noalloc validates like fa_decode and rejects calls whose split
    partials exceed its 32 MiB static array, all before any device call."""
    def call(**kw):
        a = dict(q=A16, k=A16, v=A16, seqlens=A16, o=A16, lse=A16, B=4, Hq=8, Hkv=2, Lk_max=64,
                 D=128, scale=0.1, splits=8, dtype=_abi.FA_BF16)
        a.update(kw)
        return _abi.fa_decode_noalloc(a["q"], a["k"], a["v"], a["seqlens"], a["o"], a["lse"],
                                      a["B"], a["Hq"], a["Hkv"], a["Lk_max"], a["D"], a["scale"],
                                      a["splits"], a["dtype"], None)

    assert call(q=None) == _abi.FA_ERR_INVALID_ARGUMENT
    assert call(splits=0) == _abi.FA_ERR_INVALID_ARGUMENT
    assert call(D=96) == _abi.FA_ERR_UNSUPPORTED
    # 256 sequences x 64 heads x 8 splits x 129 floats = 67.6 MB > 32 MiB
    st = call(B=256, Hq=64, Hkv=8)
    assert st == _abi.FA_ERR_INVALID_ARGUMENT and "static scratch" in _abi.fa_last_error()
