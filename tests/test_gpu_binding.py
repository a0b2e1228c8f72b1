"""The binding refuses caller-provided buffers that do not match the call
(shape, dtype, device, contiguity) before anything is launched."""
import pytest
import torch

import gated_deltanet_chunked_chunk_amd as gdn

pytestmark = pytest.mark.gpu


def inputs(B=1, T=70, Hqk=1, Hv=2, dk=128, dv=128):
    dev = torch.device("cuda:0")
    q = torch.zeros(B, T, Hqk, dk, dtype=torch.bfloat16, device=dev)
    v = torch.zeros(B, T, Hv, dv, dtype=torch.bfloat16, device=dev)
    g = torch.zeros(B, T, Hv, device=dev)
    return q, q.clone(), v, g, g.clone()


@pytest.mark.parametrize("bad", ["short", "dtype", "strided", "host"])
def test_fwd_rejects_bad_out(bad):
    q, k, v, g, b = inputs()
    out = {"short": torch.empty(1, 69, 2, 128, dtype=torch.bfloat16, device="cuda"),
           "dtype": torch.empty(1, 70, 2, 128, device="cuda"),
           "strided": torch.empty(1, 70, 2, 256, dtype=torch.bfloat16, device="cuda")[..., :128],
           "host": torch.empty(1, 70, 2, 128, dtype=torch.bfloat16)}[bad]
    with pytest.raises(gdn.GdnError):
        gdn.gdn_chunk_fwd(q, k, v, g, b, out=out)


@pytest.mark.parametrize("shape,dtype", [((1, 2, 128, 64), torch.float32),
                                         ((2, 2, 128, 128), torch.float32),
                                         ((1, 2, 128, 128), torch.bfloat16)])
def test_fwd_rejects_bad_final_state(shape, dtype):
    q, k, v, g, b = inputs()
    with pytest.raises(gdn.GdnError):
        gdn.gdn_chunk_fwd(q, k, v, g, b, final_state=torch.empty(shape, dtype=dtype, device="cuda"))


def test_fwd_rejects_small_workspace():
    # One row of 16,384 tokens at 8 heads splits into pieces: its workspace is not empty.
    q, k, v, g, b = inputs(T=16384, Hqk=8, Hv=8)
    need = gdn.gdn_chunk_fwd_workspace_size(1, 1, 16384, 8, 8, 128, 128, 1)
    assert need > 0
    with pytest.raises(gdn.GdnError):
        gdn.gdn_chunk_fwd(q, k, v, g, b, workspace=torch.empty(need - 256, dtype=torch.uint8,
                                                                device="cuda"))
    # A wider element type counts in bytes, not elements.
    ws = torch.empty(-(-need // 4), dtype=torch.float32, device="cuda")
    o, _ = gdn.gdn_chunk_fwd(q, k, v, g, b, workspace=ws)
    torch.cuda.synchronize()
    assert torch.all(o == 0)


def test_bwd_rejects_small_workspace():
    q, k, v, g, b = inputs()
    do = torch.zeros_like(v)
    need = gdn.gdn_chunk_bwd_workspace_size(1, 1, 70, 1, 2, 128, 128, 1)
    with pytest.raises(gdn.GdnError):
        gdn.gdn_chunk_bwd(q, k, v, g, b, do, workspace=torch.empty(need - 1, dtype=torch.uint8,
                                                                     device="cuda"))


def test_step_rejects_bad_out():
    dev = "cuda"
    q = torch.zeros(3, 1, 128, dtype=torch.bfloat16, device=dev)
    v = torch.zeros(3, 2, 128, dtype=torch.bfloat16, device=dev)
    g = torch.zeros(3, 2, device=dev)
    state = torch.zeros(3, 2, 128, 128, device=dev)
    for out in (torch.empty(3, 2, 64, dtype=torch.bfloat16, device=dev),
                torch.empty(3, 2, 128, dtype=torch.float32, device=dev)):
        with pytest.raises(gdn.GdnError):
            gdn.gdn_recurrent_step(q, q, v, g, g, state, out=out)
