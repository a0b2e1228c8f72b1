"""The C ABI on the host: the library loads, exports what include/gdn.h
declares, and rejects bad calls before touching the GPU (so these run here,
without one; no call below reaches a kernel launch)."""
import ctypes
import os
import re

import pytest

import gated_deltanet_chunked_chunk_amd as gdn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn.h")

OK, INVALID, UNSUPPORTED, MISALIGNED, WORKSPACE = 0, 1, 2, 3, 4
FAKE = 0x10000  # an aligned address that is never dereferenced: every call below fails validation


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    lib = gdn.load()
    names = declared_functions()
    assert "gdn_chunk_fwd" in names and "gdn_chunk_fwd_workspace_size" in names
    for name in names:
        assert hasattr(lib, name), f"libgdn.so does not export {name}"


def test_status_strings_and_version():
    for code, name in gdn.STATUS.items():
        assert gdn.gdn_status_string(code).startswith(name)
    assert "unknown" in gdn.gdn_status_string(99)
    assert gdn.gdn_version() == 100
    assert gdn.gdn_last_hip_error() == 0


def test_workspace_is_zero():
    assert gdn.gdn_chunk_fwd_workspace_size(1, 8, 2048, 16, 16, 128, 128, 8) == 0


def call(dtype=1, B=1, T=64, Hqk=2, Hv=2, dk=128, dv=128, q=FAKE, k=FAKE, v=FAKE, g=FAKE,
         beta=FAKE, h0=None, cu=None, cu_host=None, n_seqs=0, o=FAKE, ht=None, ws=None,
         ws_bytes=0):
    lib = gdn.load()
    host = None
    if cu_host is not None:
        host = ctypes.cast((ctypes.c_int32 * len(cu_host))(*cu_host), ctypes.c_void_p)
    return lib.gdn_chunk_fwd(dtype, B, T, Hqk, Hv, dk, dv, q, k, v, g, beta, 1.0, h0, cu, host,
                             n_seqs, o, ht, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), INVALID), (dict(k=None), INVALID), (dict(v=None), INVALID),
    (dict(g=None), INVALID), (dict(beta=None), INVALID), (dict(o=None), INVALID),
    (dict(B=0), INVALID), (dict(T=0), INVALID), (dict(Hqk=0), INVALID), (dict(dk=0), INVALID),
    (dict(dtype=7), UNSUPPORTED), (dict(Hqk=2, Hv=3), UNSUPPORTED), (dict(dk=64), UNSUPPORTED),
    (dict(dv=96), UNSUPPORTED), (dict(dtype=0, dk=96), UNSUPPORTED),
    (dict(q=FAKE + 8), MISALIGNED), (dict(o=FAKE + 4), MISALIGNED),
    (dict(h0=FAKE + 2), MISALIGNED), (dict(ht=FAKE + 12), MISALIGNED),
    (dict(cu=FAKE, n_seqs=2, B=2), INVALID), (dict(cu=FAKE, n_seqs=0), INVALID),
    # a valid host copy passes its checks; the misaligned g then fails the call
    (dict(cu=FAKE, n_seqs=2, cu_host=[0, 10, 64], g=FAKE + 4), MISALIGNED),
    (dict(cu=FAKE + 4, n_seqs=2, cu_host=[0, 10, 64]), MISALIGNED),
    (dict(cu=FAKE, n_seqs=2, cu_host=[1, 10, 64]), INVALID),
    (dict(cu=FAKE, n_seqs=2, cu_host=[0, 10, 63]), INVALID),
    (dict(cu=FAKE, n_seqs=2, cu_host=[0, 30, 20]), INVALID),
    (dict(cu_host=[0, 64]), INVALID),
    (dict(B=1 << 40, T=1 << 40), INVALID),
])
def test_rejects_before_launch(kw, status):
    assert call(**kw) == status


def test_binding_refuses_to_run_without_library(monkeypatch):
    monkeypatch.setattr(gdn, "_lib", None)
    monkeypatch.setattr(gdn, "_LIB_PATH", os.path.join(ROOT, "no_such_libgdn.so"))
    with pytest.raises(ImportError):
        gdn.load()


def test_binding_checks_tensors_on_host():
    import torch
    x = torch.zeros(1, 4, 1, 128)
    with pytest.raises(gdn.GdnError):
        gdn.gdn_chunk_fwd(x, x, x, torch.zeros(1, 4, 1), torch.zeros(1, 4, 1))  # CPU tensors


def test_bwd_workspace_size():
    ws = gdn.gdn_chunk_bwd_workspace_size
    # 8 rows of 32 chunks, 16 heads: per chunk-head 64*64*4 + 64*64*2 + 64*4 + 2*128*128*2
    per = 64 * 64 * 4 + 64 * 64 * 2 + 64 * 4 + 2 * 128 * 128 * 2
    assert ws(1, 8, 2048, 16, 16, 128, 128, 8) == 8 * 32 * 16 * per
    # one packed row of 5 documents: at most ceil(T / 64) + 5 chunks
    assert ws(1, 1, 2048, 16, 16, 128, 128, 5) == (32 + 5) * 16 * per
    assert ws(0, 8, 2048, 16, 16, 128, 128, 8) == 0   # fp32: no backward kernel
    assert ws(1, 8, 2048, 16, 16, 64, 128, 8) == 0    # dk = 64: none either


def bwd_call(dtype=1, B=1, T=64, Hqk=2, Hv=2, dk=128, dv=128, q=FAKE, k=FAKE, v=FAKE, g=FAKE,
             beta=FAKE, h0=None, cu=None, cu_host=None, n_seqs=0, do=FAKE, dht=None, dq=FAKE,
             dk_=FAKE, dv_=FAKE, dg=FAKE, dbeta=FAKE, dh0=None, ws=FAKE, ws_bytes=1 << 40):
    lib = gdn.load()
    host = None
    if cu_host is not None:
        host = ctypes.cast((ctypes.c_int32 * len(cu_host))(*cu_host), ctypes.c_void_p)
    return lib.gdn_chunk_bwd(dtype, B, T, Hqk, Hv, dk, dv, q, k, v, g, beta, 1.0, h0, cu, host,
                             n_seqs, do, dht, dq, dk_, dv_, dg, dbeta, dh0, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), INVALID), (dict(do=None), INVALID), (dict(dq=None), INVALID),
    (dict(dk_=None), INVALID), (dict(dv_=None), INVALID), (dict(dg=None), INVALID),
    (dict(dbeta=None), INVALID), (dict(T=0), INVALID),
    (dict(dtype=0), UNSUPPORTED), (dict(dk=64), UNSUPPORTED), (dict(dv=96), UNSUPPORTED),
    (dict(Hqk=2, Hv=3), UNSUPPORTED),
    (dict(do=FAKE + 8), MISALIGNED), (dict(dht=FAKE + 4), MISALIGNED),
    (dict(dh0=FAKE + 2), MISALIGNED), (dict(dg=FAKE + 4), MISALIGNED),
    (dict(ws=FAKE + 16), MISALIGNED),
    (dict(ws=None), WORKSPACE), (dict(ws_bytes=1024), WORKSPACE),
    (dict(cu=FAKE, n_seqs=2, B=2), INVALID),
    (dict(cu=FAKE, n_seqs=2, cu_host=[0, 10, 63]), INVALID),
    (dict(cu_host=[0, 64]), INVALID),
])
def test_bwd_rejects_before_launch(kw, status):
    assert bwd_call(**kw) == status
