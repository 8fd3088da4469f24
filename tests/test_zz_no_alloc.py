"""The allocation-free FFN entry point (flag buffer in the library's own device array) against the entry point that
takes a flag workspace, through the C ABI: two calls in a row, the second on a smaller input, each bit for bit the
same as the workspace entry point on the same inputs (the same kernels and item list, so the same arithmetic); also
with the launch landing the token rows itself, whose per-tile flags live in the same array."""
import numpy as np
import pytest
import torch

import moe_inputs as mi
from expert_output_overlap_amd import binding as B
from expert_output_overlap_amd.runtime import MoePath, to_device

pytestmark = pytest.mark.gpu

# 4 k-splits (the flag buffer holds split-K partial sums, 30 MB); then a smaller batch of the same layer
FIRST = mi.Spec("noalloc_splitk", R=4, T_o=600, G=8, E_l=2, k=2, d=256, f=1024, M=32, seed=16)
SECOND = mi.Spec("noalloc_small", R=4, T_o=250, G=8, E_l=2, k=2, d=256, f=1024, M=32, seed=26)


def bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy()


def run_both(s, mode, land=False):
    print("case", s.name, "mode", mode, "land", land, flush=True)
    inp = mi.inputs(s)
    P = MoePath.from_spec(s)
    dev = {k: to_device(v, s.dtype) for k, v in inp.items()}
    P.route(dev["logits"])
    P.layout(dev["x"])
    for r in range(s.R):
        P.recv[r].fill_(float("nan"))
    P.ffn(dev["w_gate_up"], dev["w_down"], mode=mode, consumer_cus=4)
    P.combine()
    torch.cuda.synchronize()
    assert P.status() == B.MOE_OK
    n_r = [int(v) for v in P.scalars()["N_r"]]
    ref = [bits(P.recv[r][: n_r[r]]) for r in range(s.R)]
    ref_out = bits(P.out[: s.T])
    # the allocation-free call on the same buffers, after poisoning the outputs and intermediates
    for r in range(s.R):
        P.recv[r].fill_(float("nan"))
    P.h.fill_(float("nan"))
    P.y_pad.fill_(float("nan"))
    P.out.fill_(float("nan"))
    if land:  # the launch lands the token rows itself: its landing flags must start cleared on every call
        P.x_pad.fill_(float("nan"))
        P.layout(None)
    cfg = B.moe_overlap_cfg(4, mode, 0, 0, 0, None, 0, dev["x"].data_ptr() if land else None)  # epoch ignored
    B.moe_expert_ffn_overlap_noalloc(P.shape, P.L, P.x_pad, dev["w_gate_up"], dev["w_down"], P.h, P.y_pad, P.recv, cfg)
    P.combine()
    torch.cuda.synchronize()
    assert P.status() == B.MOE_OK
    for r in range(s.R):
        np.testing.assert_array_equal(bits(P.recv[r][: n_r[r]]), ref[r], err_msg="owner %d" % r)
    np.testing.assert_array_equal(bits(P.out[: s.T]), ref_out)
    return P


def test_noalloc_matches_workspace_entry_point_twice():
    assert torch.cuda.is_available()
    run_both(FIRST, 0)
    run_both(SECOND, 0)  # the second call, on a smaller input, reuses the array the first one left behind
    run_both(SECOND, 1)  # and sequential mode
    run_both(FIRST, 0, land=True)  # landing the token rows in the launch, twice in a row
    run_both(SECOND, 0, land=True)


def test_noalloc_rejects_what_does_not_fit():
    s = mi.spec("mixtral")  # split-K partial sums for its capacity: 755 MB of flag buffer, over the 64 MiB maximum
    sh = B.moe_shape(s.R, s.T_o, s.G, s.E_l, s.k, 0, s.d, s.f, s.M, s.mgb, B.MOE_BF16)
    assert B.moe_ffn_flags_count(sh) * 4 > 64 << 20
    P = MoePath.from_spec(mi.spec("tiny"))
    dummy = torch.empty(16, dtype=torch.bfloat16, device="cuda")
    cfg = B.moe_overlap_cfg(4, 0, 0, 0, 0, None, 0)
    with pytest.raises(B.MoeError, match="maximum"):
        B.moe_expert_ffn_overlap_noalloc(sh, P.L, dummy, dummy, dummy, dummy, dummy, [dummy] * s.R, cfg)
    cfg2 = B.moe_overlap_cfg(4, 2, 0, 0, 0, None, 0)
    with pytest.raises(B.MoeError, match="mode 2"):
        B.moe_expert_ffn_overlap_noalloc(P.shape, P.L, P.x_pad, dummy, dummy, P.h, P.y_pad, P.recv, cfg2)
