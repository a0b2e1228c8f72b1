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
    # fp32, short rows, and sizes the forward rejects use no workspace either.
    assert gdn.gdn_chunk_fwd_workspace_size(0, 1, 1 << 20, 1, 1, 128, 128, 1) == 0
    assert gdn.gdn_chunk_fwd_workspace_size(1, 1, 1000, 1, 1, 128, 128, 1) == 0
    assert gdn.gdn_chunk_fwd_workspace_size(1, 1, 1 << 20, 2, 3, 128, 128, 1) == 0


def piece_bytes(B, pieces, Hv, dk, dv):
    per = B * (pieces - 1) * Hv * dk
    return -(-per * (dv + dk) * 4 // 256) * 256 + per * dv * 4


def test_piece_scan_workspace():
    """Rows with few heads are split into pieces (at least 4 chunks each)
    where the planner's cost (workgroup rounds x chunks per piece for both
    passes, plus the scan's serial steps and a fixed launch cost) beats whole
    rows by a twentieth.  The long row (1 x 1,064,960 tokens, 16 heads, two
    64-column tiles) splits into 8 pieces of 2,080 chunks."""
    assert gdn.gdn_chunk_fwd_workspace_size(1, 1, 1_064_960, 16, 16, 128, 128, 1) == \
        piece_bytes(1, 8, 16, 128, 128)
    # 65 chunks, 2 heads: 6 pieces of 11 chunks (the last 10).
    assert gdn.gdn_chunk_fwd_workspace_size(1, 1, 4133, 1, 2, 128, 128, 1) == \
        piece_bytes(1, 6, 2, 128, 128)
    # 94 chunks, two rows, dv = 64: 8 pieces of 12 chunks.
    assert gdn.gdn_chunk_fwd_workspace_size(1, 2, 6000, 1, 1, 128, 64, 2) == \
        piece_bytes(2, 8, 1, 128, 64)
    # 47 chunks, two rows: 6 pieces of 8 chunks.
    assert gdn.gdn_chunk_fwd_workspace_size(1, 2, 3000, 1, 1, 128, 64, 2) == \
        piece_bytes(2, 6, 1, 128, 64)
    # 16 chunks over 64 rows (dk = dv = 64): the scan's steps and the extra
    # launches cost more than they save; whole rows, no workspace.
    assert gdn.gdn_chunk_fwd_workspace_size(1, 8, 1024, 8, 8, 64, 64, 8) == 0
    # 48 chunks at dk = 256 over 2 rows: the scan's steps are dearer there.
    assert gdn.gdn_chunk_fwd_workspace_size(1, 1, 3037, 1, 2, 256, 64, 1) == 0
    # dk = 256 (four transition tiles per piece): 3 pieces of 5,547 chunks;
    # dv = 256 is tiled like any other dv.
    assert gdn.gdn_chunk_fwd_workspace_size(1, 1, 1_064_960, 16, 16, 256, 256, 1) == \
        piece_bytes(1, 3, 16, 256, 256)
    assert gdn.gdn_chunk_fwd_workspace_size(1, 1, 4133, 1, 2, 256, 128, 1) == \
        piece_bytes(1, 4, 2, 256, 128)
    assert gdn.gdn_chunk_fwd_workspace_size(1, 1, 4133, 1, 2, 128, 256, 1) == \
        piece_bytes(1, 6, 2, 128, 256)


def test_piece_scan_workspace_checked_before_launch():
    need = gdn.gdn_chunk_fwd_workspace_size(1, 1, 4133, 1, 2, 128, 128, 1)
    assert call(T=4133, Hqk=1, Hv=2, ws=FAKE, ws_bytes=need - 1) == WORKSPACE
    assert call(T=4133, Hqk=1, Hv=2, ws=FAKE + 16, ws_bytes=need) == MISALIGNED


def call(dtype=1, B=1, T=64, Hqk=2, Hv=2, dk=128, dv=128, q=FAKE, k=FAKE, v=FAKE, g=FAKE,
         beta=FAKE, h0=None, cu=None, cu_host=None, n_seqs=0, o=FAKE, ht=None, ws=None,
         ws_bytes=0, flags=0):
    lib = gdn.load()
    host = None
    if cu_host is not None:
        host = ctypes.cast((ctypes.c_int32 * len(cu_host))(*cu_host), ctypes.c_void_p)
    return lib.gdn_chunk_fwd(dtype, B, T, Hqk, Hv, dk, dv, q, k, v, g, beta, 1.0, flags, h0, cu,
                             host, n_seqs, o, ht, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), INVALID), (dict(k=None), INVALID), (dict(v=None), INVALID),
    (dict(g=None), INVALID), (dict(beta=None), INVALID), (dict(o=None), INVALID),
    (dict(B=0), INVALID), (dict(T=0), INVALID), (dict(Hqk=0), INVALID), (dict(dk=0), INVALID),
    (dict(dtype=7), UNSUPPORTED), (dict(Hqk=2, Hv=3), UNSUPPORTED), (dict(dk=32), UNSUPPORTED),
    (dict(flags=4), INVALID), (dict(flags=0x100), INVALID),
    (dict(dv=96), UNSUPPORTED), (dict(dtype=0, dk=96), UNSUPPORTED),
    (dict(dk=512), UNSUPPORTED), (dict(dv=512), UNSUPPORTED),
    (dict(dk=256, q=FAKE + 8), MISALIGNED), (dict(dtype=0, dk=256, dv=256, o=FAKE + 4), MISALIGNED),
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


def call_noalloc(dtype=1, B=1, T=64, Hqk=2, Hv=2, dk=128, dv=128, q=FAKE, k=FAKE, v=FAKE, g=FAKE,
                 beta=FAKE, h0=None, cu=None, cu_host=None, n_seqs=0, o=FAKE, ht=None, flags=0):
    lib = gdn.load()
    host = None
    if cu_host is not None:
        host = ctypes.cast((ctypes.c_int32 * len(cu_host))(*cu_host), ctypes.c_void_p)
    return lib.gdn_chunk_fwd_noalloc(dtype, B, T, Hqk, Hv, dk, dv, q, k, v, g, beta, 1.0, flags,
                                     h0, cu, host, n_seqs, o, ht, None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), INVALID), (dict(o=None), INVALID), (dict(T=0), INVALID),
    (dict(dtype=7), UNSUPPORTED), (dict(dk=32), UNSUPPORTED), (dict(flags=4), INVALID),
    (dict(q=FAKE + 8), MISALIGNED), (dict(ht=FAKE + 12), MISALIGNED),
    (dict(cu=FAKE, n_seqs=2, cu_host=[0, 30, 20]), INVALID),
    (dict(B=1 << 40, T=1 << 40), INVALID),
])
def test_noalloc_rejects_before_launch(kw, status):
    """The entry point without a workspace validates exactly as
    gdn_chunk_fwd does, before any HIP call."""
    assert call_noalloc(**kw) == status


SCRATCH_LIMIT = 6


def test_noalloc_scratch_limit():
    """A call whose piece plan needs more than the static scratch is refused
    with its own status before anything is enqueued; the planned need is what
    gdn_chunk_fwd_workspace_size reports."""
    limit = gdn.GDN_STATIC_SCRATCH_BYTES
    assert limit == 64 << 20
    # Three rows of 2^22 tokens at 3 heads, dk = dv = 256: many pieces of a
    # large state each (216 MiB).
    need = gdn.gdn_chunk_fwd_workspace_size(1, 3, 1 << 22, 3, 3, 256, 256, 3)
    assert need > limit
    assert call_noalloc(B=3, T=1 << 22, Hqk=3, Hv=3, dk=256, dv=256) == SCRATCH_LIMIT
    # The long rows the library is measured on fit.
    assert 0 < gdn.gdn_chunk_fwd_workspace_size(1, 1, 1_064_960, 16, 16, 128, 128, 1) <= limit
    assert 0 < gdn.gdn_chunk_fwd_workspace_size(1, 1, 65536, 8, 8, 256, 256, 1) <= limit
    assert "GDN_STATIC_SCRATCH_BYTES" in gdn.gdn_status_string(SCRATCH_LIMIT)


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
    # 8 rows of 32 chunks, 16 heads: per chunk-head two bf16 states (dv x 128)
    # and two bf16 row blocks (64 x dv)
    per = 2 * 128 * 128 * 2 + 2 * 64 * 128 * 2
    assert ws(1, 8, 2048, 16, 16, 128, 128, 8) == 8 * 32 * 16 * per
    # one packed row of 5 documents: at most ceil(T / 64) + 5 chunks
    assert ws(1, 1, 2048, 16, 16, 128, 128, 5) == (32 + 5) * 16 * per
    assert ws(0, 8, 2048, 16, 16, 128, 128, 8) == 0   # fp32: no backward kernel
    # dk = 64 keeps the chunk states 128 keys wide (zeros past dk): the same size
    assert ws(1, 8, 2048, 16, 16, 64, 128, 8) == ws(1, 8, 2048, 16, 16, 128, 128, 8)
    # dk = 256: chunks of 32 tokens, 256-key states and 32 Delta and drhs rows
    assert ws(1, 8, 2048, 16, 16, 256, 128, 8) == 8 * 64 * 16 * (2 * 256 * 128 * 2 + 2 * 32 * 128 * 2)
    assert ws(1, 1, 2048, 16, 16, 256, 128, 5) == (64 + 5) * 16 * (2 * 256 * 128 * 2 + 2 * 32 * 128 * 2)
    assert ws(1, 8, 2048, 16, 16, 512, 128, 8) == 0   # no such head dimension
    assert ws(1, 1, 100, 1, 1, 128, 256, 1) > ws(1, 1, 100, 1, 1, 128, 128, 1)
    # the in-op options add the prepared copies: q and k in bf16, g and beta in fp32
    base = ws(1, 8, 2048, 16, 16, 128, 128, 8)
    rows = 8 * 2048 * 16
    assert ws(1, 8, 2048, 16, 16, 128, 128, 8, 1) == base + 2 * rows * 128 * 2
    assert ws(1, 8, 2048, 16, 16, 128, 128, 8, 2) == base + 2 * rows * 4
    assert ws(1, 8, 2048, 16, 16, 128, 128, 8, 3) == base + 2 * rows * 128 * 2 + 2 * rows * 4
    # each region rounded up to 256 bytes: 3 tokens x 1 head x 4 bytes -> 256
    assert ws(1, 1, 3, 1, 1, 128, 128, 1, 2) == ws(1, 1, 3, 1, 1, 128, 128, 1) + 2 * 256
    assert ws(1, 8, 2048, 16, 16, 128, 128, 8, 4) == 0   # unknown option bit


def bwd_call(dtype=1, B=1, T=64, Hqk=2, Hv=2, dk=128, dv=128, q=FAKE, k=FAKE, v=FAKE, g=FAKE,
             beta=FAKE, h0=None, cu=None, cu_host=None, n_seqs=0, do=FAKE, dht=None, dq=FAKE,
             dk_=FAKE, dv_=FAKE, dg=FAKE, dbeta=FAKE, dh0=None, ws=FAKE, ws_bytes=1 << 40,
             flags=0):
    lib = gdn.load()
    host = None
    if cu_host is not None:
        host = ctypes.cast((ctypes.c_int32 * len(cu_host))(*cu_host), ctypes.c_void_p)
    return lib.gdn_chunk_bwd(dtype, B, T, Hqk, Hv, dk, dv, q, k, v, g, beta, 1.0, flags, h0, cu,
                             host,
                             n_seqs, do, dht, dq, dk_, dv_, dg, dbeta, dh0, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), INVALID), (dict(do=None), INVALID), (dict(dq=None), INVALID),
    (dict(dk_=None), INVALID), (dict(dv_=None), INVALID), (dict(dg=None), INVALID),
    (dict(dbeta=None), INVALID), (dict(T=0), INVALID),
    (dict(dtype=0), UNSUPPORTED), (dict(dk=512), UNSUPPORTED), (dict(dv=96), UNSUPPORTED),
    (dict(dk=32), UNSUPPORTED), (dict(dv=512), UNSUPPORTED), (dict(Hqk=2, Hv=3), UNSUPPORTED),
    (dict(dk=64, do=FAKE + 8), MISALIGNED), (dict(dv=256, dht=FAKE + 4), MISALIGNED),
    (dict(do=FAKE + 8), MISALIGNED), (dict(dht=FAKE + 4), MISALIGNED),
    (dict(dh0=FAKE + 2), MISALIGNED), (dict(dg=FAKE + 4), MISALIGNED),
    (dict(ws=FAKE + 16), MISALIGNED),
    (dict(ws=None), WORKSPACE), (dict(ws_bytes=1024), WORKSPACE),
    (dict(cu=FAKE, n_seqs=2, B=2), INVALID),
    (dict(cu=FAKE, n_seqs=2, cu_host=[0, 10, 63]), INVALID),
    (dict(cu_host=[0, 64]), INVALID),
    (dict(flags=4), INVALID), (dict(flags=0x80000002), INVALID),
])
def test_bwd_rejects_before_launch(kw, status):
    assert bwd_call(**kw) == status


def prep_call(dtype=1, rows=4, dk=128, q=FAKE, k=FAKE, qo=FAKE, ko=FAKE, n_gates=4, g=FAKE,
              beta=FAKE, go=FAKE, bo=FAKE, flags=3):
    return gdn.load().gdn_prepare_inputs(dtype, rows, dk, q, k, qo, ko, n_gates, g, beta, go,
                                         bo, flags, None)


@pytest.mark.parametrize("kw,status", [
    (dict(flags=4), INVALID), (dict(flags=0x80000001), INVALID),
    (dict(q=None), INVALID), (dict(ko=None), INVALID), (dict(rows=-1), INVALID),
    (dict(dk=0), INVALID), (dict(dk=257), UNSUPPORTED), (dict(dtype=5), UNSUPPORTED),
    (dict(dk=256, q=FAKE + 4), MISALIGNED),
    (dict(g=None), INVALID), (dict(bo=None), INVALID), (dict(n_gates=-1), INVALID),
    (dict(q=FAKE + 4), MISALIGNED), (dict(go=FAKE + 8), MISALIGNED),
    # Nothing to do (no option, or zero rows and gates) launches nothing.
    (dict(flags=0), OK), (dict(rows=0, n_gates=0), OK),
    # An option not set leaves its pointers unread.
    (dict(flags=1, g=None, beta=None, go=None, bo=None, rows=0), OK),
    (dict(flags=2, q=None, k=None, qo=None, ko=None, n_gates=0), OK),
    (dict(rows=0, n_gates=0, q=None, g=None), OK),
])
def test_prepare_rejects_before_launch(kw, status):
    assert prep_call(**kw) == status


def prep_bwd_call(dtype=1, rows=4, dk=128, q=FAKE, k=FAKE, dq=FAKE, dk_=FAKE, dqo=FAKE,
                  dko=FAKE, n_gates=4, g=FAKE, beta=FAKE, dg=FAKE, db=FAKE, dgo=FAKE, dbo=FAKE,
                  flags=3):
    return gdn.load().gdn_prepare_inputs_bwd(dtype, rows, dk, q, k, dq, dk_, dqo, dko, n_gates,
                                             g, beta, dg, db, dgo, dbo, flags, None)


@pytest.mark.parametrize("kw,status", [
    (dict(flags=4), INVALID), (dict(flags=0x80000001), INVALID),
    (dict(q=None), INVALID), (dict(dk_=None), INVALID), (dict(dko=None), INVALID),
    (dict(rows=-1), INVALID), (dict(dk=0), INVALID), (dict(dk=257), UNSUPPORTED),
    (dict(dtype=5), UNSUPPORTED), (dict(dq=FAKE + 4), MISALIGNED),
    (dict(dko=FAKE + 8), MISALIGNED), (dict(g=None), INVALID), (dict(db=None), INVALID),
    (dict(dgo=None), INVALID), (dict(n_gates=-1), INVALID), (dict(dbo=FAKE + 4), MISALIGNED),
    (dict(flags=0), OK), (dict(rows=0, n_gates=0), OK),
    (dict(flags=1, g=None, beta=None, dg=None, db=None, dgo=None, dbo=None, rows=0), OK),
    (dict(flags=2, q=None, k=None, dq=None, dk_=None, dqo=None, dko=None, n_gates=0), OK),
])
def test_prepare_bwd_rejects_before_launch(kw, status):
    assert prep_bwd_call(**kw) == status


def step_call(dtype=1, N=2, Hqk=2, Hv=2, dk=128, dv=128, q=FAKE, k=FAKE, v=FAKE, g=FAKE,
              beta=FAKE, flags=0, state=FAKE, slots=None, n_slots=2, o=FAKE):
    return gdn.load().gdn_recurrent_step(dtype, N, Hqk, Hv, dk, dv, q, k, v, g, beta, 1.0, flags,
                                         state, slots, n_slots, o, None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), INVALID), (dict(v=None), INVALID), (dict(state=None), INVALID),
    (dict(o=None), INVALID), (dict(N=-1), INVALID), (dict(Hqk=0), INVALID),
    (dict(flags=8), INVALID), (dict(n_slots=1), INVALID), (dict(n_slots=-1), INVALID),
    (dict(dtype=9), UNSUPPORTED), (dict(dk=96), UNSUPPORTED), (dict(dv=512), UNSUPPORTED),
    (dict(dk=32), UNSUPPORTED), (dict(Hqk=2, Hv=3), UNSUPPORTED),
    (dict(state=FAKE + 4), MISALIGNED), (dict(dk=256, dv=256, state=FAKE + 4), MISALIGNED),
    (dict(slots=FAKE + 4, n_slots=1), MISALIGNED), (dict(o=FAKE + 2), MISALIGNED),
    (dict(N=1 << 40, n_slots=1 << 40), INVALID),
    # N = 0 enqueues nothing and reads no pointer.
    (dict(N=0, n_slots=0), OK), (dict(N=0, n_slots=0, q=None, state=None, o=None), OK),
    (dict(N=0, dk=96), UNSUPPORTED),
])
def test_step_rejects_before_launch(kw, status):
    assert step_call(**kw) == status


def test_step_binding_checks_tensors_on_host():
    import torch
    x = torch.zeros(2, 2, 128)
    with pytest.raises(gdn.GdnError):
        gdn.gdn_recurrent_step(x, x, x, torch.zeros(2, 2), torch.zeros(2, 2),
                               torch.zeros(2, 2, 128, 128))
    with pytest.raises(gdn.GdnError):
        gdn.gdn_prepare_inputs(x, x, torch.zeros(2, 2), torch.zeros(2, 2))


def test_piece_plan_properties():
    """Over a grid of shapes: the plan never splits rows once the output pass
    of whole rows already fills every CU (B * H_v * dv / 64 >= 256 workgroups),
    and whatever it picks is a whole number of pieces between 2 and 256."""
    for dk in (64, 128, 256):
        for dv in (64, 128, 256):
            for B, Hv in ((1, 1), (1, 4), (2, 8), (4, 16), (8, 16), (8, 32), (16, 32)):
                for T in (1, 255, 4096, 65536, 1 << 20):
                    need = gdn.gdn_chunk_fwd_workspace_size(1, B, T, 1, Hv, dk, dv, B)
                    if B * Hv * dv // 64 >= 256:
                        assert need == 0, (B, T, Hv, dk, dv)
                    if need == 0:
                        continue
                    found = [p for p in range(2, 257) if piece_bytes(B, p, Hv, dk, dv) == need]
                    assert len(found) == 1, (B, T, Hv, dk, dv, need)
                    assert found[0] <= -(-T // 64), (B, T, Hv, dk, dv)


def test_packed_plan():
    """The plan of packed calls (from the host copy of cu_seqlens): documents
    longest first whenever there is more than one (up to 2,048); long
    documents split only where the cost model gains, within the slots of the
    single-row plan of T tokens (the capacity the size-only query promises);
    short documents never."""
    import gdn_inputs as gi
    plan = gdn.gdn_chunk_fwd_plan
    # One row of 8 heads, ~16 geometric documents of mean 1024: all 256
    # workgroups run at once, so whole documents are best and their order
    # does not matter (no ranking launch).
    cu = [int(x) for x in gi.cu_from_lengths(gi.geometric_lengths(16384, 1024, 1009))]
    assert len(cu) - 1 == 16
    assert plan(1, 1, 16384, 8, 8, 128, 128, cu) == (0, 0, False)
    # One 20,000-token document among seven short ones at 8 heads: split.
    cu = [int(x) for x in gi.cu_from_lengths([20000, 2000, 1500, 3000, 900, 1100, 800, 700])]
    T = cu[-1]
    pl, slots, ordered = plan(1, 1, T, 8, 8, 128, 128, cu)
    _, budget, _ = plan(1, 1, T, 8, 8, 128, 128)
    assert pl > 0 and pl % 64 == 0 and 0 < slots <= budget and not ordered
    assert slots == sum(max(0, -(-(b - a) // pl) - 1) for a, b in zip(cu, cu[1:]))
    # The 32-head packed workload fills the CUs: ordered, not split.
    cu = [int(x) for x in gi.cu_from_lengths(gi.geometric_lengths(16384, 1024, 1002))]
    assert plan(1, 1, 16384, 16, 32, 128, 128, cu) == (0, 0, True)
    # Short documents are never split, whatever the heads.
    cu = list(range(0, 20 * 500 + 1, 20))
    assert plan(1, 1, cu[-1], 1, 1, 128, 128, cu)[:2] == (0, 0)
    # One document: nothing to order; few workgroups: nothing gained by it.
    assert plan(1, 1, 5000, 1, 1, 128, 128, [0, 5000])[2] is False
    assert plan(1, 1, 5000, 1, 1, 128, 128, [0, 1000, 5000])[2] is False
    # fp32: never split, never ordered.
    assert plan(0, 1, 16384, 8, 8, 128, 128, [0, 16000, 16384]) == (0, 0, False)
    # Without the host copy nothing is planned from lengths (batch rows).
    assert plan(1, 2, 2048, 16, 16, 128, 128)[2] is False


def test_packed_workspace_size():
    """A packed call's workspace: the document order (4 bytes per document,
    256-aligned, up to 2,048 documents) plus the single-row piece capacity."""
    base = gdn.gdn_chunk_fwd_workspace_size(1, 1, 16384, 8, 8, 128, 128, 1)
    assert gdn.gdn_chunk_fwd_workspace_size(1, 1, 16384, 8, 8, 128, 128, 16) == base + 256
    assert gdn.gdn_chunk_fwd_workspace_size(1, 1, 16384, 8, 8, 128, 128, 100) == base + 512
    assert gdn.gdn_chunk_fwd_workspace_size(1, 1, 16384, 8, 8, 128, 128, 5000) == base
    assert gdn.gdn_chunk_fwd_workspace_size(0, 1, 16384, 8, 8, 128, 128, 16) == 0


@pytest.mark.parametrize("cu", [[1, 10, 64], [0, 10, 63], [0, 30, 20]])
def test_plan_rejects_bad_host_offsets(cu):
    with pytest.raises(gdn.GdnError):
        gdn.gdn_chunk_fwd_plan(1, 1, 64, 1, 1, 128, 128, cu)
