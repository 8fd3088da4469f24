"""GPU parity of the backward pass (moe_expert_ffn_backward, moe_combine_backward) against the CPU oracle, through
the C-ABI.  dY, h, dG and dU lie in the oracle's admitted intervals (each a bf16 rounding of a value within the fp32
evaluation's error bound; where no other rounding is admitted, that is the oracle's value bit for bit).  The
returned dX rows, dx, the routing weights' gradient and both weight gradients are within the tolerance of
``tolerance.py`` of the oracle's values, plus the allowance those intervals imply (tolerance.backward_slack); the
routing weights' gradient is taken over the oracle's forward rows for the roundings of h the forward took, as the
forward's own parity test takes them (tolerance.check_ffn).  Sequential and overlapped calls give equal bits."""
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
    # f = 8 d: the dX items split 4 ways over k (partial sums, last arrival sums), skewed routing
    mi.Spec("bwd_splitk", R=4, T_o=200, G=8, E_l=2, k=2, d=128, f=1024, M=32, seed=43, bias="zipf", bias_param=1.2),
    # an expert with no rows (zero weight gradients) and tokens with no local slot
    mi.Spec("bwd_sparse", R=2, T_o=64, G=16, E_l=4, k=1, d=128, f=128, M=16, seed=44, bias="zipf", bias_param=3.0),
]


def f64(t):
    return t.float().cpu().numpy().astype(np.float64)


def bits(t):
    return t.contiguous().view(torch.int16 if t.element_size() == 2 else torch.int32).cpu().numpy()


def check_in(got, lo, hi, what):
    bad = (got < lo) | (got > hi) | ~np.isfinite(got)
    if bad.any():
        i = np.unravel_index(np.argmax(bad), bad.shape)
        raise AssertionError("%s: %d values outside the admitted interval; first at %s got %r in [%r, %r]"
                             % (what, bad.sum(), i, got[i], lo[i], hi[i]))


class BwdRun:
    """One workload on the GPU: forward (route, layout, FFN, combine), then the backward calls."""

    def __init__(self, s, self_rank=0, logits=None):
        assert torch.cuda.is_available(), "the gpu tests need the MI355X"
        print("case", s, "self_rank", self_rank, flush=True)
        self.s = s
        self.lo = self_rank * s.E_l  # the local experts' first global id
        self.inp = mi.inputs(s)
        if logits is not None:
            self.inp["logits"] = logits
        self.P = MoePath(s.R, s.T_o, s.G, s.E_l, s.k, s.d, s.f, s.M, s.mgb, s.dtype, self_rank)
        self.dev = {k: to_device(v, s.dtype) for k, v in self.inp.items()}
        self.d_out_h = mi.d_out(s)
        self.d_out = to_device(self.d_out_h, s.dtype)
        P = self.P
        P.route(self.dev["logits"])
        P.layout(self.dev["x"])
        P.ffn(self.dev["w_gate_up"], self.dev["w_down"], mode=0)
        P.combine()
        torch.cuda.synchronize()
        assert P.status() == B.MOE_OK
        self.idx, self.w = oracle.route(self.inp["logits"], s.k)
        np.testing.assert_array_equal(P.topk_idx[: s.T].cpu().numpy(), self.idx)
        self.lay = oracle.layout(self.idx, s.R, s.T_o, s.G, s.E_l, s.k, s.M, s.mgb, self_rank)

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

    def rows_of(self, sel):
        """The local slots (t, j) where sel [T, k] holds, their experts, owners and padded rows (the combine plan names
        each slot's row in its owner's receive buffer; the padded row is at the same offset in its group)."""
        s, lay = self.s, self.lay
        plan = lay["combine_plan"]
        t, j = np.nonzero(sel & (plan >= 0))
        e = self.idx[t, j] - self.lo
        r = t // s.T_o
        g = e * s.R + r
        p = lay["padded_off"][g] + plan[t, j] - lay["recv_off"][g]
        return t, j, e, r, p

    def check(self, b, t, j, e, r, p, toks, experts):
        """The checks named in the module docstring, for the slots (t, j) (with experts e, owners r, padded rows p):
        their parts and returned dX rows, dx and the routing weights' gradient of tokens toks (every local slot of
        which is among the slots), the weight gradients of experts (every row of which is among the slots)."""
        s, P, inp = self.s, self.P, self.inp
        parts = oracle.bwd_rows(t, e, self.w[t, j], inp["x"], inp["w_gate_up"], inp["w_down"], self.d_out_h, True,
                                want_adm=True, w_rel=tolerance.ROUTE_W_RTOL)
        ref = oracle.backward_reduce(s, inp, self.d_out_h, (t, j), e, parts, experts=experts)
        pd = torch.as_tensor(p, device=b["dy_pad"].device)
        adm, f = parts["adm"], s.f
        check_in(f64(b["dy_pad"][pd]), parts["dy_adm"][:, 0], parts["dy_adm"][:, 1], "dY rows")
        check_in(f64(P.h[pd]), adm[:, 0, 0], adm[:, 0, 1], "h rows")
        dgu = f64(b["dgu_ws"][pd])
        check_in(dgu[:, :f], adm[:, 1, 0], adm[:, 1, 1], "dG rows")
        check_in(dgu[:, f:], adm[:, 2, 0], adm[:, 2, 1], "dU rows")
        n_other = sum(int((g_ != o_).sum()) for g_, o_ in ((f64(b["dy_pad"][pd]), parts["dy"]),
                                                           (f64(P.h[pd]), parts["h"]), (dgu, parts["dgu"])))
        print("values in an admitted interval other than the oracle's rounding:", n_other, flush=True)
        sl = tolerance.backward_slack(parts, e, inp["w_gate_up"], oracle._as_f64(inp["x"][t]), experts)
        plan = self.lay["combine_plan"]
        got = np.stack([f64(b["dx_recv"][int(r[i])][int(plan[t[i], j[i]])]) for i in range(t.size)]) if t.size \
            else np.zeros((0, s.d))
        tolerance.check(got, parts["dx"], "returned dX rows", slack=sl["dx_rows"])
        tok_sl = np.zeros((s.T, s.d))
        np.add.at(tok_sl, t, sl["dx_rows"])
        tk = torch.as_tensor(toks, device=pd.device)
        tolerance.check(f64(b["dx"][tk]), ref["dx"][toks], "dx of %d tokens" % len(toks),
                        slack=tok_sl[toks] + tolerance.bf16_ulp(ref["dx"][toks]))
        # the routing weights' gradient <dOut, y> over the delivered forward rows: the oracle's rows for the
        # alternative roundings of h the forward took (tolerance.check_ffn, as the forward's parity test takes them)
        m = np.isin(t, toks)
        ex = oracle.ffn_rows_ex(t[m], e[m], inp["x"], inp["w_gate_up"], inp["w_down"], True, max_cand=16)
        got_y = np.stack([f64(P.recv[int(r[i])][int(plan[t[i], j[i]])]) for i in np.nonzero(m)[0]]) if m.any() \
            else np.zeros((0, s.d))
        y_ref, _ = tolerance.check_ffn(got_y, ex, "forward y rows of %d tokens" % len(toks))
        dw_ref = np.zeros((s.T, s.k))
        dw_ref[t[m], j[m]] = np.einsum("ic,ic->i", oracle._as_f64(self.d_out_h[t[m]]), y_ref)
        tolerance.check(b["dw_route"][tk].cpu().numpy().astype(np.float64), dw_ref[toks],
                        "routing weights' gradient of %d tokens" % len(toks))
        for i, ee in enumerate(experts):
            tolerance.check(b["dw_down"][ee].cpu().numpy().astype(np.float64), ref["dw_down"][i],
                            "dW_down[%d]" % ee, slack=sl["dw_down"][i])
            tolerance.check(b["dw_gate_up"][ee].cpu().numpy().astype(np.float64), ref["dw_gate_up"][i],
                            "dW_gate_up[%d]" % ee, slack=sl["dw_gate_up"][i])


@pytest.mark.parametrize("s,self_rank", [(s, 0) for s in BWD_SMALL] + [(BWD_SMALL[1], 1), (BWD_SMALL[2], 1), (BWD_SMALL[3], 3)],
                         ids=lambda v: v.name if hasattr(v, "name") else "rank%d" % v)
def test_backward_parity(s, self_rank):
    """Whole backward (dY dispatch, dH, h / dG / dU, dX with its return, the weight gradients, the combine's
    backward) against the oracle on every row, token and expert, at rank 0 and at ranks 1 and 3 (whose own dX rows
    the dX items store straight into their receive buffer); then the sequential call, and the overlapped call with
    no consumer partition and with one of 16, give the same bits."""
    run = BwdRun(s, self_rank)
    b = run.backward(mode=0, consumer_cus=8)
    t, j, e, r, p = run.rows_of(np.ones((s.T, s.k), bool))
    run.check(b, t, j, e, r, p, np.arange(s.T), list(range(s.E_l)))
    rows_past = [np.isnan(f64(b["dx_recv"][q][int(run.lay["N_r"][q]):run.P.recv_cap])).all() for q in range(s.R)]
    assert all(rows_past), "rows past N_r were written"
    ref_bits = {k: bits(b[k]) for k in ("dx", "dw_route", "dw_gate_up", "dw_down")}
    ref_recv = [bits(x) for x in b["dx_recv"]]
    for kw in (dict(mode=1), dict(mode=0, consumer_cus=-1), dict(mode=0, consumer_cus=16)):
        b2 = run.backward(**kw)
        for k, v in ref_bits.items():
            np.testing.assert_array_equal(bits(b2[k]), v, err_msg="%s %s" % (k, kw))
        for q in range(s.R):
            np.testing.assert_array_equal(bits(b2["dx_recv"][q]), ref_recv[q], err_msg="dx_recv %d %s" % (q, kw))


GU_CASES = BWD_SMALL[1:4] + [mi.spec("deepseek"), mi.spec("mixtral")]


def same_bits(a, b):
    return bool(torch.equal(a.contiguous().view(torch.int16 if a.element_size() == 2 else torch.int32),
                            b.contiguous().view(torch.int16 if b.element_size() == 2 else torch.int32)))


@pytest.mark.parametrize("s", GU_CASES, ids=lambda v: v.name)
def test_backward_with_the_forwards_preactivations(s):
    """The forward storing g | u (moe_overlap_cfg.gu_out) and the backward taking them (moe_bwd_args.gu): the
    forward's own outputs keep their bits; the stored rows are every real row's, and nothing else is written; and h,
    dG | dU, the returned dX rows, both weight gradients, dx and the routing weights' gradient are the same bits as
    the recomputing call's (whose values test_backward_parity and test_backward_full_size check against the oracle),
    overlapped and sequential.  Then the calls that would misuse them are rejected."""
    run = BwdRun(s)
    P = run.P
    t, j, e, r, p = run.rows_of(np.ones((s.T, s.k), bool))
    pd = torch.as_tensor(p, device=P.h.device)
    b = run.backward(mode=0)
    ref = {k: b[k].clone() for k in ("dw_gate_up", "dw_down", "dx", "dw_route")}
    ref["h"], ref["dgu"] = P.h[pd].clone(), b["dgu_ws"][pd].clone()
    ref_recv = [x.clone() for x in b["dx_recv"]]
    y_ref, out_ref = [x.clone() for x in P.recv], P.out.clone()
    gu = P.gu_buffer()
    gu.fill_(float("nan"))
    P.ffn(run.dev["w_gate_up"], run.dev["w_down"], mode=0, gu_out=gu)
    P.combine()
    torch.cuda.synchronize()
    assert P.status() == B.MOE_OK
    assert all(same_bits(a, b_) for a, b_ in zip(P.recv, y_ref)) and same_bits(P.out, out_ref), \
        "storing g | u changed the forward's outputs"
    real = torch.zeros(gu.shape[0], dtype=torch.bool, device=gu.device)
    real[pd] = True
    assert not torch.isnan(gu[real]).any(), "a real row's g | u was not stored"
    assert torch.isnan(gu[~real]).all(), "g | u stored past the real rows"
    for kw in (dict(mode=0), dict(mode=1)):
        b2 = run.backward(gu=gu, **kw)
        got = {k: b2[k] for k in ("dw_gate_up", "dw_down", "dx", "dw_route")}
        got["h"], got["dgu"] = P.h[pd], b2["dgu_ws"][pd]
        for k, v in ref.items():
            assert same_bits(got[k], v), "%s differs from the recomputing call's (%s)" % (k, kw)
        for q in range(s.R):
            assert same_bits(b2["dx_recv"][q], ref_recv[q]), "dx_recv %d differs (%s)" % (q, kw)
    # misuse: g | u stored by a return-only call, or passed to the backward's cfg
    cfg = B.moe_overlap_cfg(8, 2, 99, 0, 0, None, 0, None, gu.data_ptr())
    with pytest.raises(B.MoeError):
        B.moe_expert_ffn_overlap(P.shape, P.L, P.x_pad, run.dev["w_gate_up"], run.dev["w_down"], P.h, P.y_pad,
                                 P.recv, P.flags, cfg)
    bb = P.bwd_buffers()
    cfg = B.moe_overlap_cfg(0, 0, 99, 0, 0, None, 0, None, gu.data_ptr())
    tens = {"topk_idx": P.topk_idx, "topk_w": P.topk_w, "x_pad": P.x_pad, "w_gate_up": run.dev["w_gate_up"],
            "w_down": run.dev["w_down"], "d_out": run.d_out, "h_ws": P.h,
            **{k: bb[k] for k in ("dy_pad", "dh_ws", "dgu_ws", "dx_pad", "dw_gate_up", "dw_down")}}
    with pytest.raises(B.MoeError):
        B.moe_expert_ffn_backward(P.shape, P.L, tens, bb["dx_recv"], bb["flags"], cfg)


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


FULL_BWD = ["skew", "deepseek", "mixtral"]


@pytest.mark.parametrize("name", FULL_BWD)
def test_backward_full_size(name):
    """Full-size workload in the benchmark's configuration (overlapped, the library's consumer count): the parts and
    returned dX rows of the local slots of 12 sampled tokens, those tokens' dx and routing weights' gradient, and both
    weight gradients of one expert from all of its rows (the expert with the fewest rows among those with more than
    two row tiles, so that the sums cross row tiles and end on a ragged one; none for the Mixtral-shaped shard, whose
    two experts hold thousands of rows each); the sequential call gives the same bits."""
    s = mi.spec(name)
    run = BwdRun(s)
    b = run.backward(mode=0)
    idx, plan = run.idx, run.lay["combine_plan"]
    rng = np.random.default_rng(7)
    toks = np.sort(rng.choice(np.nonzero((plan >= 0).any(axis=1))[0], 12, replace=False))
    counts = np.bincount(idx[idx < s.E_l], minlength=s.E_l)
    e_w = [] if name == "mixtral" else [int(np.argmin(np.where(counts > 2 * s.M, counts, np.iinfo(np.int64).max)))]
    assert not e_w or counts[e_w[0]] > 2 * s.M
    sel = np.isin(np.arange(s.T)[:, None], toks) | np.isin(idx, e_w)
    t, j, e, r, p = run.rows_of(sel)
    print("%s: %d rows (%d sampled tokens, expert %s with %s rows)" % (name, t.size, toks.size, e_w,
                                                                       counts[e_w] if e_w else 0), flush=True)
    run.check(b, t, j, e, r, p, toks, e_w)
    keep = {k: bits(b[k]) for k in ("dx", "dw_route", "dw_down")}
    b = run.backward(mode=1)
    for k, v in keep.items():
        np.testing.assert_array_equal(bits(b[k]), v, err_msg="sequential %s" % k)


def test_backward_ordering_stress():
    """Publish/acquire ordering of the backward launch under stress (the page's "What would settle it", as for the
    forward): 300 overlapped calls on a split-K shape over consumer partitions {none, 1, 2, 4, 8, 16, 32} and shuffled
    epochs, every other call taking the forward's stored g | u (whose h / dG / dU items then publish as soon as dH
    is in); every call's dx, weight gradients and returned dX rows equal the sequential recomputing call's bit for
    bit.  Stops at the first mismatch (and names the call)."""
    s = BWD_SMALL[3]
    run = BwdRun(s)
    gu = run.P.gu_buffer()
    run.P.ffn(run.dev["w_gate_up"], run.dev["w_down"], mode=0, gu_out=gu)
    b = run.backward(mode=1)
    keys = ("dx", "dw_route", "dw_gate_up", "dw_down")
    ref = {k: b[k].clone() for k in keys}
    ref_recv = [b["dx_recv"][r][: int(run.lay["N_r"][r])].clone() for r in range(s.R)]
    rng = np.random.default_rng(77)
    last = run.P.bwd_epoch
    for it in range(300):
        cus = int(rng.choice([-1, 1, 2, 4, 8, 16, 32]))
        ep = last
        while ep == last:  # shuffled, but never the value the flags hold from the previous call
            ep = int(rng.integers(1, 1 << 31))
        last = ep
        b = run.backward(mode=0, consumer_cus=cus, epoch=ep, gu=gu if it % 2 else None)
        for k in keys:
            if not torch.equal(b[k].view(torch.int32 if b[k].element_size() == 4 else torch.int16),
                               ref[k].view(torch.int32 if ref[k].element_size() == 4 else torch.int16)):
                raise AssertionError("call %d (consumer_cus %d, epoch %d, stored g | u %s): %s differs"
                                     % (it, cus, ep, bool(it % 2), k))
        for r in range(s.R):
            got = b["dx_recv"][r][: ref_recv[r].shape[0]]
            if not torch.equal(got.view(torch.int16), ref_recv[r].view(torch.int16)):
                raise AssertionError("call %d (consumer_cus %d, epoch %d): dX rows of owner %d differ" % (it, cus, ep, r))


def test_backward_empty_and_degenerate_inputs():
    """No tokens (every weight-gradient tile is still written, as zeros); no token routed to a local expert (every
    gradient zero); every token routed to local expert 0 (which then holds a slot of every token) against the
    oracle."""
    s = mi.spec("tiny", T_o=0)
    P = MoePath.from_spec(s)
    P.route(torch.empty(0, s.G, device="cuda"))
    P.layout(torch.empty(0, s.d, dtype=torch.bfloat16, device="cuda"))
    w1, w2 = (to_device(a, s.dtype) for a in mi.weights(s))
    P.ffn(w1, w2)
    P.combine()
    b = P.bwd_buffers()
    b["dw_gate_up"].fill_(float("nan"))
    b["dw_down"].fill_(float("nan"))
    d_out = torch.empty(0, s.d, dtype=torch.bfloat16, device="cuda")
    P.backward(d_out, w1, w2)
    P.combine_backward(d_out)
    torch.cuda.synchronize()
    assert P.status() == B.MOE_OK
    assert (b["dw_gate_up"] == 0).all() and (b["dw_down"] == 0).all()
    # no token routed to a local expert
    s = mi.spec("tiny")
    lg = mi.logits(s)
    lg[:, : s.E_l] -= 100.0
    run = BwdRun(s, logits=lg)
    b = run.backward(mode=0)
    assert int(run.lay["M_pad"]) == 0
    assert (f64(b["dx"][: s.T]) == 0).all() and (b["dw_route"][: s.T] == 0).all()
    assert (b["dw_gate_up"] == 0).all() and (b["dw_down"] == 0).all()
    # every token routed to local expert 0
    lg = mi.logits(s)
    lg[:, 0] += 100.0
    run = BwdRun(s, logits=lg)
    b = run.backward(mode=0)
    t, j, e, r, p = run.rows_of(np.ones((s.T, s.k), bool))
    assert (e == 0).sum() == s.T  # expert 0 holds one slot of every token
    run.check(b, t, j, e, r, p, np.arange(s.T), list(range(s.E_l)))
