"""gdn_chunk_fwd_noalloc, the entry point that allocates nothing, against
gdn_chunk_fwd with a caller workspace: two calls in a row through the C ABI,
the second on a smaller input, both long enough to run the piece scan in the
static scratch (each call must find nothing of the previous one's left there
that it reads), and a sampled head of each against the oracle."""
import numpy as np
import pytest
import torch

import gated_deltanet_chunked_chunk_amd as gdn
import gdn_inputs as gi
import oracle
from gpu_util import TOL, rel_l2, to_device

pytestmark = pytest.mark.gpu


def one_call(B, T, H, seed, h0_std):
    d = gi.make(B, T, H, H, 128, 128, "bf16", seed, h0_std=h0_std)
    need = gdn.gdn_chunk_fwd_workspace_size(1, B, T, H, H, 128, 128, B)
    assert 0 < need <= gdn.GDN_STATIC_SCRATCH_BYTES, need
    print(f"[no-alloc case] B={B} T={T} H={H} seed={seed} piece workspace {need} B", flush=True)
    t = to_device(d)
    o_ref, h_ref = gdn.gdn_chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"],
                                     initial_state=t["h0"], scale=0.5)
    o = torch.empty_like(o_ref)
    ht = torch.empty_like(h_ref)
    gdn.gdn_chunk_fwd_noalloc(t["q"], t["k"], t["v"], t["g"], t["beta"], initial_state=t["h0"],
                              scale=0.5, out=o, final_state=ht)
    torch.cuda.synchronize()
    # The same plan and kernels: bitwise equal.
    assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16))
    assert torch.equal(ht, h_ref)
    # And one sampled (row, head) within the tolerances of the oracle.
    b, j = B - 1, gi.sampled_heads(seed, H, n=1)[0]
    sl = lambda x: gi.widen(x[b:b + 1, :, j:j + 1])
    h0 = None if d["h0"] is None else d["h0"][b:b + 1, j:j + 1].astype(np.float64)
    ro, rh = oracle.gdn_fwd(sl(d["q"]), sl(d["k"]), sl(d["v"]), d["g"][b:b + 1, :, j:j + 1],
                            d["beta"][b:b + 1, :, j:j + 1], scale=0.5, h0=h0)
    eo = rel_l2(o[b:b + 1, :, j:j + 1].float().cpu().numpy(), ro)
    eh = rel_l2(ht[b:b + 1, j:j + 1].cpu().numpy(), rh)
    print(f"  bitwise equal to gdn_chunk_fwd; oracle rel-L2 output {eo:.3e}, state {eh:.3e}",
          flush=True)
    assert eo <= TOL["bf16"][0] and eh <= TOL["bf16"][1]


def test_noalloc_two_calls_second_smaller():
    one_call(1, 16384, 8, 7001, 0.05)
    one_call(1, 8192, 4, 7002, None)
