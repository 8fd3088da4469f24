"""GPU parity of the backward pass (moe_expert_ffn_backward, moe_combine_backward) against the CPU oracle, through
the C-ABI: the dY rows bit for bit; every delivered dX row, dx, the routing weights' gradient and both weight
gradients within the tolerance of ``tolerance.py``; sequential and overlapped calls bitwise equal."""
import numpy as np
import pytest
import torch

import moe_inputs as mi
import oracle
import tolerance
from expert_output_overlap_amd import binding as B
from expert_output_overlap_amd.runtime import MoePath, to_device

pytestmark = pytest.mark.gpu

BWD_SMALL = [
    mi.spec("tiny"),
    # two 256-wide column tiles of dX and dH, several row tiles per expert
    mi.Spec("bwd_small", R=4, T_o=240, G=8, E_l=2, k=2, d=256, f=256, M=32, seed=41),
    # d and f not multiples of 256 (masked columns), three experts, ragged row tiles
    mi.Spec("bwd_ragged", R=3, T_o=300, G=6, E_l=3, k=2, d=192, f=384, M=16, seed=42),
    # f = 8 d: the dX items split 8 ways over k (partial sums, last arrival sums), skewed routing
    mi.Spec("bwd_splitk", R=4, T_o=200, G=8, E_l=2, k=2, d=128, f=1024, M=32, seed=43, bias="zipf", bias_param=1.2),
    # an expert with no rows (zero weight gradients) and tokens with no local slot
    mi.Spec("bwd_sparse", R=2, T_o=64, G=16, E_l=4, k=1, d=128, f=128, M=16, seed=44, bias="zipf", bias_param=3.0),
]


def f64(t):
    return t.float().cpu().numpy().astype(np.float64)


def bits(t):
    return t.contiguous().view(torch.int16 if t.element_size() == 2 else torch.int32).cpu().numpy()


class BwdRun:
    def __init__(self, s):
        assert torch.cuda.is_available(), "the gpu tests need the MI355X"
        print("case", s, flush=True)
        self.s = s
        self.inp = mi.inputs(s)
        self.P = MoePath.from_spec(s)
        self.dev = {k: to_device(v, s.dtype) for k, v in self.inp.items()}
        self.d_out_h = mi.d_out(s)
        self.d_out = to_device(self.d_out_h, s.dtype)
        P = self.P
        P.route(self.dev["logits"])
        P.layout(self.dev["x"])
        P.ffn(self.dev["w_gate_up"], self.dev["w_down"], mode=0, consumer_cus=4)
        P.combine()
        torch.cuda.synchronize()
        assert P.status() == B.MOE_OK
        self.ref = oracle.backward(s, self.inp, self.d_out_h)
        self.lay = oracle.layout(self.ref["topk_idx"], s.R, s.T_o, s.G, s.E_l, s.k, s.M, s.mgb, 0)

    def backward(self, **kw):
        P = self.P
        b = P.bwd_buffers()
        for r in range(self.s.R):
            b["dx_recv"][r].fill_(float("nan"))
        b["dw_gate_up"].fill_(float("nan"))
        b["dw_down"].fill_(float("nan"))
        P.backward(self.d_out, self.dev["w_gate_up"], self.dev["w_down"], **kw)
        P.combine_backward(self.d_out)
        torch.cuda.synchronize()
        assert P.status() == B.MOE_OK
        return b

    def slot_of_padded(self):
        """For each real padded row: (token, slot) of the oracle's row list, and the oracle row index."""
        s, lay, idx = self.s, self.lay, self.ref["topk_idx"]
        t_all, j_all = self.ref["rows"]
        pos = {(int(t), int(j)): i for i, (t, j) in enumerate(zip(t_all, j_all))}
        real = np.nonzero(lay["row_src"] >= 0)[0]
        ridx = []
        for p in real:
            t = int(lay["row_src"][p])
            e = int(lay["tile_expert"][p // s.M])
            j = int(np.nonzero(idx[t] == e)[0][0])
            ridx.append(pos[(t, j)])
        return real, np.array(ridx)


def resolve_parts(run, b):
    """The GPU's h, dG and dU rows against the oracle's: each value is a bf16 value between the least and the greatest
    rounding that an fp32 evaluation within its error bound can give (the oracle's admitted interval; the oracle's own
    rounding lies in it).  Returns the oracle's reductions for the values the GPU took (oracle.backward_reduce) and the
    number of values that differ from the oracle's rounding."""
    s, ref, P = run.s, run.ref, run.P
    parts = ref["parts"]
    real, ridx = run.slot_of_padded()
    sel = torch.as_tensor(real, device=b["dy_pad"].device)
    adm = parts["adm"][ridx]
    got = {"h": f64(P.h[sel]), "dgu": f64(b["dgu_ws"][sel])}
    want = {"h": parts["h"][ridx], "dgu": parts["dgu"][ridx]}
    lo = {"h": adm[:, 0, 0], "dgu": np.concatenate([adm[:, 1, 0], adm[:, 2, 0]], axis=1)}
    hi = {"h": adm[:, 0, 1], "dgu": np.concatenate([adm[:, 1, 1], adm[:, 2, 1]], axis=1)}
    res = dict(parts)
    flips = 0
    for k in ("h", "dgu"):
        bad = (got[k] < lo[k]) | (got[k] > hi[k])
        if bad.any():
            i = np.unravel_index(np.argmax(bad), bad.shape)
            raise AssertionError("%s: %d values outside the admitted roundings; first at %s got %r ref %r in [%r, %r]"
                                 % (k, bad.sum(), i, got[k][i], want[k][i], lo[k][i], hi[k][i]))
        flips += int((got[k] != want[k]).sum())
        res[k] = parts[k].copy()
        res[k][ridx] = got[k]
    if flips == 0:
        return ref, 0
    t, j = ref["rows"]
    lo_e = ref["topk_idx"][t, j]
    out = oracle.backward_reduce(s, run.inp, run.d_out_h, (t, j), lo_e, res, dx_from_dgu=True)
    out.update({"rows": ref["rows"], "parts": dict(res, dx=out["dx_rows"])})
    return out, flips


def check_outputs(run, b):
    s, P = run.s, run.P
    real, ridx = run.slot_of_padded()
    dev = b["dy_pad"].device
    # the dY rows: bf16 of the fp32 product w dOut, bit for bit
    got_dy = f64(b["dy_pad"][torch.as_tensor(real, device=dev)])
    np.testing.assert_array_equal(got_dy, run.ref["parts"]["dy"][ridx], err_msg="dY rows")
    # h, dG and dU: the oracle's roundings, up to the admitted other ones; the sums below follow the values taken
    ref, flips = resolve_parts(run, b)
    print("other roundings of h, dG, dU taken:", flips, flush=True)
    parts = ref["parts"]
    # the delivered dX rows: owner r's row recv_off[g] + i is the i-th row of group g = e * R + r
    lay = run.lay
    for r in range(s.R):
        n_r = int(lay["N_r"][r])
        got = f64(b["dx_recv"][r][:n_r])
        want = np.full((n_r, s.d), np.nan)
        for e in range(s.E_l):
            g = e * s.R + r
            n, po, ro = int(lay["counts"][g]), int(lay["padded_off"][g]), int(lay["recv_off"][g])
            sel = np.searchsorted(real, po + np.arange(n))
            want[ro:ro + n] = parts["dx"][ridx[sel]]
        tolerance.check(got, want, "dX rows of owner %d" % r)
        assert np.isnan(f64(b["dx_recv"][r][n_r:P.recv_cap])).all(), "rows past N_r were written"
    tolerance.check(f64(b["dx"][: s.T]), ref["dx"], "dx")
    tolerance.check(b["dw_route"][: s.T].cpu().numpy().astype(np.float64), ref["dw"], "routing weights' gradient")
    tolerance.check(b["dw_down"].cpu().numpy().astype(np.float64), ref["dw_down"], "dW_down")
    tolerance.check(b["dw_gate_up"].cpu().numpy().astype(np.float64), ref["dw_gate_up"], "dW_gate_up")


@pytest.mark.parametrize("s", BWD_SMALL, ids=lambda v: v.name)
def test_backward_parity(s):
    """Whole backward (dY dispatch, dH, h / dG / dU, dX with its return, the weight gradients, the combine's
    backward) against the oracle; then the sequential call, and the overlapped call with no consumer partition and
    with one of 16, give the same bits."""
    run = BwdRun(s)
    b = run.backward(mode=0, consumer_cus=8)
    check_outputs(run, b)
    ref_bits = {k: bits(b[k]) for k in ("dx", "dw_route", "dw_gate_up", "dw_down")}
    ref_recv = [bits(t) for t in b["dx_recv"]]
    for kw in (dict(mode=1), dict(mode=0, consumer_cus=-1), dict(mode=0, consumer_cus=16)):
        b2 = run.backward(**kw)
        for k, v in ref_bits.items():
            np.testing.assert_array_equal(bits(b2[k]), v, err_msg="%s %s" % (k, kw))
        for r in range(s.R):
            np.testing.assert_array_equal(bits(b2["dx_recv"][r]), ref_recv[r], err_msg="dx_recv %d %s" % (r, kw))


def test_backward_repeats_and_rejects_bad_calls():
    """Repeated calls on the same flag buffer (new epochs) give the same bits; fp32 shapes, f not a multiple of 128
    and a spin budget that ends every wait are reported."""
    s = BWD_SMALL[1]
    run = BwdRun(s)
    first = bits(run.backward(mode=0)["dw_down"])
    for _ in range(3):
        np.testing.assert_array_equal(bits(run.backward(mode=0)["dw_down"]), first)
    bad = B.moe_shape(s.R, s.T_o, s.G, s.E_l, s.k, 0, s.d, 192, s.M, s.mgb, B.MOE_BF16)
    assert B.moe_bwd_flags_count(bad) == -1
    f32 = B.moe_shape(s.R, s.T_o, s.G, s.E_l, s.k, 0, s.d, s.f, s.M, s.mgb, B.MOE_F32)
    assert B.moe_bwd_flags_count(f32) == -1
    # a spin budget of one tick: some wait gives up, the status word says so, and every workgroup exits
    P = run.P
    b = P.bwd_buffers()
    cfg = B.moe_overlap_cfg(8, 0, 1000, 0, 1, None, 0, None)
    t = {"topk_idx": P.topk_idx, "topk_w": P.topk_w, "x_pad": P.x_pad, "w_gate_up": run.dev["w_gate_up"],
         "w_down": run.dev["w_down"], "d_out": run.d_out, "h_ws": P.h,
         **{k: b[k] for k in ("dy_pad", "dh_ws", "dgu_ws", "dx_pad", "dw_gate_up", "dw_down")}}
    B.moe_expert_ffn_backward(P.shape, P.L, t, b["dx_recv"], b["flags"], cfg)
    torch.cuda.synchronize()
    assert P.status() in (B.MOE_OK, B.MOE_ETIMEOUT)
