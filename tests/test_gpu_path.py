"""GPU parity of the HIP path against the CPU oracle, through the C-ABI.

Layout arrays and permutations bit for bit; FFN output rows, delivered rows and the combined output within the
tolerance of ``tolerance.py``; delivery bit-equal to the GPU's own y rows; sequential and overlapped runs bitwise
equal.  Small shapes are compared element by element; the full-size workloads compare the complete layout, rows of
every GEMM row tile (every real row of the Mixtral-shaped shard) and tokens, in the launch configuration the
benchmark times.
"""
import dataclasses

import numpy as np
import pytest
import torch

import moe_inputs as mi
import oracle
import schedule_model
import tolerance
from expert_output_overlap_amd import binding as B
from expert_output_overlap_amd.runtime import MoePath, to_device

SELF = 0  # the GPU's own rank among the owners (self_rank) unless a test says otherwise

pytestmark = pytest.mark.gpu

LAYOUT_INT = ["counts", "padded_off", "recv_off"]


def _require_gpu():
    assert torch.cuda.is_available(), "the gpu tests need the MI355X"


def f64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16 if t.element_size() == 2 else torch.int32).cpu().numpy()


class Run:
    """Inputs of one workload on host and device, the GPU path's buffers, and the oracle's routing and layout."""

    def __init__(self, s, logits=None, self_rank=SELF):
        _require_gpu()
        print("case", s, "self_rank", self_rank, flush=True)
        self.s = s
        self.sr = self_rank
        self.inp = mi.inputs(s)
        if logits is not None:
            self.inp["logits"] = logits
        self.P = MoePath(s.R, s.T_o, s.G, s.E_l, s.k, s.d, s.f, s.M, s.mgb, s.dtype, self_rank)
        self.dev = {k: to_device(v, s.dtype) for k, v in self.inp.items()}
        self.P.route(self.dev["logits"])
        self.P.layout(self.dev["x"])
        self.idx, self.w = oracle.route(self.inp["logits"], s.k)
        self.lay = oracle.layout(self.idx, s.R, s.T_o, s.G, s.E_l, s.k, s.M, s.mgb, self_rank)

    def ffn(self, **kw):
        return self.P.ffn(self.dev["w_gate_up"], self.dev["w_down"], **kw)

    def y_at(self, rows) -> torch.Tensor:
        """The GPU's y at padded rows ``rows`` (real rows): from y_pad, except the self-owned groups' rows, which the
        producer stores straight into the self owner's receive buffer."""
        lay, s = self.lay, self.s
        rows = np.asarray(rows, dtype=np.int64)
        g = lay["tile_expert"][rows // s.M] * s.R + lay["tile_owner"][rows // s.M]
        own = lay["tile_owner"][rows // s.M] == self.sr
        dev = self.P.y_pad.device
        out = self.P.y_pad[torch.as_tensor(rows, device=dev)].clone()
        if own.any():
            dst = lay["recv_off"][g[own]] + rows[own] - lay["padded_off"][g[own]]
            out[torch.as_tensor(np.nonzero(own)[0], device=dev)] = self.P.recv[self.sr][torch.as_tensor(dst, device=dev)]
        return out

    def check_rows(self, rows, what="y"):
        """Check the GPU's y at padded rows ``rows`` (real rows) against the oracle, up to the oracle's own
        alternative roundings of h; returns the oracle reference rows that matched."""
        lay, s = self.lay, self.s
        bf = s.dtype == "bf16"
        ex = oracle.ffn_rows_ex(lay["row_src"][rows], lay["tile_expert"][rows // s.M], self.inp["x"],
                                self.inp["w_gate_up"], self.inp["w_down"], bf)
        got = f64(self.y_at(rows))
        ref, flips = tolerance.check_ffn(got, ex, what, bf)
        print("%s: %d rows, %d alternative h roundings taken" % (what, len(rows), flips), flush=True)
        return ref


def out_slack(run, recv_ref):
    """The combined output's allowance for the delivered rows' own admitted roundings (tolerance.combine_slack)."""
    s, lay = run.s, run.lay
    if s.dtype != "bf16":
        return None
    base = np.concatenate([[0], np.cumsum([r.shape[0] for r in recv_ref])])
    y_all = np.concatenate(recv_ref) if len(recv_ref) else np.zeros((0, s.d))
    plan = lay["combine_plan"].reshape(s.T, s.k)
    return tolerance.combine_slack(plan, run.w, y_all, lambda i, j: base[i // s.T_o] + plan[i, j])


def check_route_and_layout(run):
    s, P, lay = run.s, run.P, run.lay
    torch.cuda.synchronize()
    assert P.status() == B.MOE_OK
    np.testing.assert_array_equal(P.topk_idx[: s.T].cpu().numpy(), run.idx)
    np.testing.assert_allclose(P.topk_w[: s.T].cpu().numpy(), run.w, rtol=tolerance.ROUTE_W_RTOL, atol=1e-9)
    for n in LAYOUT_INT:
        np.testing.assert_array_equal(P.array(n).cpu().numpy(), lay[n], err_msg=n)
    sc = P.scalars()
    assert (sc["M_pad"], sc["n_tiles"], sc["n_segs"]) == (lay["M_pad"], lay["n_tiles"], lay["n_segs"])
    assert sc["N_r"] == lay["N_r"].tolist()
    nt, ns = lay["n_tiles"], lay["n_segs"]
    for n in ("tile_owner", "tile_expert", "tile_valid", "tile_order"):
        np.testing.assert_array_equal(P.array(n)[:nt].cpu().numpy(), lay[n], err_msg=n)
    np.testing.assert_array_equal(P.array("seg_desc").view(-1, 8)[:ns].cpu().numpy(), lay["seg_desc"])
    np.testing.assert_array_equal(P.array("row_src")[: lay["M_pad"]].cpu().numpy(), lay["row_src"])
    np.testing.assert_array_equal(P.array("combine_plan").view(-1, s.k).cpu().numpy(), lay["combine_plan"])
    real = np.nonzero(lay["row_src"] >= 0)[0]
    xb = bits(P.x_pad)
    np.testing.assert_array_equal(xb[real], bits(run.dev["x"])[lay["row_src"][real]])
    check_schedule(run)


def check_schedule(run):
    """GEMM row tiles hold every real row exactly once and no padding row, with one expert each; each expert's
    row tiles form one run of consecutive tiles that every tile of it names, all full but the last; every
    segment's row tiles contain all of its rows (host-side property check of the internal schedule)."""
    P, lay, s = run.P, run.lay, run.s
    TR = 256 if s.dtype == "bf16" else 64
    n_mt = P.scalars()["n_mtiles"]
    desc = P.array("mtile_desc").view(-1, B.MT_FIELDS)[:n_mt].cpu().numpy()
    covered = np.zeros(lay["M_pad"], np.int32)
    tile_of_row = np.full(lay["M_pad"], -1)
    runs = {}
    for mt, dsc in enumerate(desc):
        e, nrow, r0, rc = dsc[0], dsc[1], dsc[2], dsc[3]
        gs = e * s.R + run.sr
        assert dsc[4:8].tolist() == [lay["padded_off"][gs], lay["counts"][gs],
                                     lay["recv_off"][gs] - lay["padded_off"][gs], 0]
        H = B.MT_HDR
        dsc = np.concatenate([dsc[:4], dsc[H:]])
        assert 1 <= nrow <= TR and (dsc[4 + nrow:4 + TR] == -1).all()
        assert r0 <= mt < r0 + rc <= n_mt and runs.setdefault(e, (r0, rc)) == (r0, rc)
        assert nrow == TR or mt == r0 + rc - 1
        rows = dsc[4:4 + nrow]
        covered[rows] += 1
        tile_of_row[rows] = mt
        assert (lay["tile_expert"][rows // s.M] == e).all()
    for e, (r0, rc) in runs.items():
        assert (desc[r0:r0 + rc, 0] == e).all()
    real = lay["row_src"] >= 0
    assert (covered[real] == 1).all() and (covered[~real] == 0).all()
    segm = P.array("seg_mtiles").view(-1, 2)[: lay["n_segs"]].cpu().numpy()
    for sd, (m0, mc) in zip(lay["seg_desc"], segm):
        rows = np.arange(sd[4], sd[4] + sd[6])
        assert ((tile_of_row[rows] >= m0) & (tile_of_row[rows] < m0 + mc)).all()
    if s.dtype != "bf16":
        return
    # the row-tile model of the CPU schedule tests is the device's packing, and the device's producer order is its
    # remote-first order; the list the launch runs over these tables passes the CPU checks
    hdr_m, rows_m, pure_m, order_m = schedule_model.packing(lay["counts"], lay["padded_off"], s.R, s.E_l, run.sr, s.M)
    np.testing.assert_array_equal(desc[:, :4], hdr_m)
    for mt in range(n_mt):
        np.testing.assert_array_equal(desc[mt, B.MT_HDR:B.MT_HDR + desc[mt, 1]], rows_m[mt])
    order = P.array("mt_order")[:n_mt].cpu().numpy()
    np.testing.assert_array_equal(order, order_m)
    n_rem = P.scalars()["n_remote_mtiles"]
    assert n_rem == int((~pure_m).sum())
    for mode in (0, 1):
        cfg = B.moe_overlap_cfg(0, mode, 1, 0, 0, None)
        items = B.moe_ffn_schedule(P.shape, torch.cuda.get_device_properties(0).multi_processor_count, cfg,
                                   desc[:, :4], order, n_rem)
        schedule_model.check_list(items, n_mt, s.d, s.f, pure_m)


def check_delivery(run):
    """recv[r] rows of another owner are the GPU's own y rows of group (e, r), bit for bit; the self owner's rows,
    which the producer stores there itself, are all written; rows past N_r untouched (NaN canary)."""
    P, lay, s = run.P, run.lay, run.s
    yb = bits(P.y_pad)
    for r in range(s.R):
        rb = bits(P.recv[r])
        n_r = int(lay["N_r"][r])
        if r == run.sr:
            assert not np.isnan(f64(P.recv[r][:n_r])).any(), "a self-owned row was not written"
        for e in range(s.E_l if r != run.sr else 0):
            g = e * s.R + r
            n, po, ro = lay["counts"][g], lay["padded_off"][g], lay["recv_off"][g]
            np.testing.assert_array_equal(rb[ro:ro + n], yb[po:po + n], err_msg="owner %d expert %d" % (r, e))
        tail = f64(P.recv[r][n_r:P.recv_cap])
        assert np.isnan(tail).all(), "rows past N_r were written"


def check_landing(run, recv_bits, out_bits, **kw):
    """The FFN call landing the token rows itself (layout built without the gather, x_pad poisoned first): the
    rows it lands are x's rows bit for bit, and every delivered row and the combined output are the bits of the call
    that read the gathered x_pad."""
    P, s, lay = run.P, run.s, run.lay
    P.x_pad.fill_(float("nan"))
    P.layout(None)
    run.ffn(x_tokens=run.dev["x"], **kw)
    P.combine()
    torch.cuda.synchronize()
    assert P.status() == B.MOE_OK
    real = np.nonzero(lay["row_src"] >= 0)[0]
    dev = P.x_pad.device
    np.testing.assert_array_equal(bits(P.x_pad[torch.as_tensor(real, device=dev)]),
                                  bits(run.dev["x"][torch.as_tensor(lay["row_src"][real], device=dev)]),
                                  err_msg="landed rows " + str(kw))
    for r in range(s.R):
        np.testing.assert_array_equal(bits(P.recv[r]), recv_bits[r], err_msg="landing " + str(kw))
    np.testing.assert_array_equal(bits(P.out), out_bits, err_msg="landing " + str(kw))


SMALL = [
    mi.spec("tiny"), mi.spec("tiny_f32"), mi.spec("tiny", mgb=2),
    mi.Spec("ragged", R=4, T_o=300, G=16, E_l=4, k=2, d=256, f=512, M=32, seed=11),
    mi.Spec("ragged_skew", R=3, T_o=500, G=12, E_l=4, k=3, d=192, f=320, M=48, seed=12, bias="zipf",
            bias_param=1.2, mgb=2),
    mi.Spec("one_owner", R=1, T_o=200, G=1, E_l=1, k=1, d=128, f=128, M=16, seed=13),
    mi.Spec("k_eq_el", R=2, T_o=70, G=6, E_l=3, k=3, d=128, f=192, M=64, seed=14),
    mi.Spec("f32_ragged", R=3, T_o=90, G=9, E_l=3, k=2, d=128, f=192, M=32, dtype="f32", seed=15),
    # f = 4 d: the second GEMM's output tiles are summed from 4 k-splits (ragged row tiles, two windows)
    mi.Spec("splitk", R=4, T_o=600, G=8, E_l=2, k=2, d=256, f=1024, M=32, seed=16),
    # f = 2 d, 3 d and 6 d: 2, 3 and 6 k-splits (the last summed by the general loop)
    mi.Spec("splitk2", R=4, T_o=300, G=8, E_l=2, k=2, d=256, f=512, M=32, seed=17),
    mi.Spec("splitk3", R=2, T_o=500, G=8, E_l=2, k=2, d=256, f=768, M=64, seed=18),
    mi.Spec("splitk6", R=3, T_o=200, G=6, E_l=2, k=1, d=256, f=1536, M=16, seed=19),
    # 4 k-splits over more than four windows of row tiles: split-major second-GEMM windows (sequential call) and
    # interleaved windows (overlapped call)
    mi.Spec("splitk_windows", R=4, T_o=2400, G=8, E_l=2, k=2, d=256, f=1024, M=32, seed=22),
    # more items than one round of the producers, the last round at most half full (on 256 CUs: 300 items, 48 and
    # 44 in the last round of the overlapped and sequential calls): that round's second-GEMM items run as two
    # half-width items each; with 4 k-splits (halves of splits) and with none (halves counted in by the tile)
    mi.Spec("splitk_halves", R=4, T_o=3150, G=4, E_l=1, k=2, d=256, f=1024, M=32, seed=23),
    mi.Spec("halves", R=4, T_o=12800, G=4, E_l=1, k=2, d=256, f=256, M=32, seed=24),
    # fp32 with more transfer segments than a 128-thread consumer workgroup holds in its window at once
    mi.Spec("f32_many_segs", R=8, T_o=400, G=32, E_l=16, k=2, d=128, f=128, M=16, dtype="f32", seed=20),
]


@pytest.mark.parametrize("s,self_rank", [(s, SELF) for s in SMALL] + [(SMALL[3], 2), (SMALL[4], 1), (SMALL[1], 1)],
                         ids=lambda v: v.name + ("_mgb%d" % v.mgb) if isinstance(v, mi.Spec) else "rank%d" % v)
def test_small_full_parity(s, self_rank):
    """Whole path against the oracle; ranks other than 0 own other experts, and the producer stores their rows."""
    run = Run(s, self_rank=self_rank)
    check_route_and_layout(run)
    P, lay = run.P, run.lay
    for r in range(s.R):
        P.recv[r].fill_(float("nan"))
    run.ffn(mode=0, consumer_cus=4)
    torch.cuda.synchronize()
    assert P.status() == B.MOE_OK
    real = np.nonzero(lay["row_src"] >= 0)[0]
    y_ref = run.check_rows(real)
    check_delivery(run)
    y_pad = np.full((lay["M_pad"], s.d), np.nan)
    y_pad[real] = y_ref
    recv_ref = oracle.deliver(lay, y_pad, s.R, s.E_l)
    for r in range(s.R):
        tolerance.check(f64(P.recv[r][: int(lay["N_r"][r])]), recv_ref[r], "recv[%d]" % r)
    P.combine()
    torch.cuda.synchronize()
    out_ref = oracle.combine(lay, run.w, recv_ref, s.R, s.T_o, s.k, s.dtype == "bf16")
    tolerance.check(f64(P.out[: s.T]), out_ref, "out", slack=out_slack(run, recv_ref))
    # sequential mode, and the producer's other row-tile order, give the same bits
    recv_ovl = [bits(b) for b in P.recv]
    out_ovl = bits(P.out)
    bf = s.dtype == "bf16"
    # bf16 also: the return on the DMA engines, and no consumer partition (the return at the launch's tail)
    for kw in (dict(mode=1), dict(mode=0, tile_order=1)) + ((dict(mode=3), dict(mode=0, consumer_cus=-1)) if bf else ()):
        run.ffn(**{"consumer_cus": 4, **kw})
        P.combine()
        torch.cuda.synchronize()
        assert P.status() == B.MOE_OK
        for r in range(s.R):
            np.testing.assert_array_equal(bits(P.recv[r]), recv_ovl[r], err_msg=str(kw))
        np.testing.assert_array_equal(bits(P.out), out_ovl, err_msg=str(kw))
    if bf:  # the launch landing the token rows itself, overlapped and sequential
        for kw in (dict(mode=0), dict(mode=1), dict(mode=0, tile_order=1), dict(mode=0, consumer_cus=-1)):
            check_landing(run, recv_ovl, out_ovl, **{"consumer_cus": 4, **kw})


FULL = ["mixtral", "skew", "sweep1", "sweep2", "sweep4", "sweep8", "sweep16", "deepseek"]
BENCH_CONSUMER_CUS = 0  # bench.py's default partition, the library's pick for the shape (and its default band window)


@pytest.mark.parametrize("name", FULL)
def test_full_size_parity(name):
    """Full-size workload in the benchmark's launch configuration: the whole layout bit for bit; y on the first, the
    last and four random real rows of every GEMM row tile (every split-K and half-width tile included), on every real
    row for the Mixtral-shaped shard; the combine of every token there, of sampled tokens elsewhere; sequential ==
    overlapped bit for bit, and so is the launch that lands the token rows itself."""
    s = mi.spec(name)
    run = Run(s)
    check_route_and_layout(run)
    P, lay = run.P, run.lay
    for r in range(s.R):
        P.recv[r].fill_(float("nan"))
    run.ffn(mode=0, consumer_cus=BENCH_CONSUMER_CUS)
    P.combine()
    torch.cuda.synchronize()
    assert P.status() == B.MOE_OK
    check_delivery(run)
    rng = np.random.default_rng(0)
    real = np.nonzero(lay["row_src"] >= 0)[0]
    n_mt = P.scalars()["n_mtiles"]
    desc = P.array("mtile_desc").view(-1, B.MT_FIELDS)[:n_mt].cpu().numpy()
    if name == "mixtral":
        rows = real
    else:
        picks = []
        for mt in range(n_mt):
            tr = desc[mt, B.MT_HDR:B.MT_HDR + desc[mt, 1]]
            picks.append(np.concatenate([tr[:1], tr[-1:], rng.choice(tr, min(4, tr.size), replace=False)]))
        rows = np.unique(np.concatenate(picks))
    print("%s: %d of %d real rows over %d row tiles" % (name, rows.size, real.size, n_mt), flush=True)
    y_ref = np.concatenate([run.check_rows(rows[i:i + 96], "y rows") for i in range(0, rows.size, 96)])
    if name == "mixtral":  # every token's combine, from the reference rows of every real row
        y_pad = np.full((lay["M_pad"], s.d), np.nan)
        y_pad[rows] = y_ref
        recv_ref = oracle.deliver(lay, y_pad, s.R, s.E_l)
        out_ref = oracle.combine(lay, run.w, recv_ref, s.R, s.T_o, s.k, True)
        tolerance.check(f64(P.out[: s.T]), out_ref, "out (every token)", slack=out_slack(run, recv_ref))
    else:  # sampled tokens: the oracle's FFN rows of their local slots, the oracle's combine
        toks = rng.choice(s.T, 16, replace=False)
        plan = lay["combine_plan"][toks]
        src_rows = []
        mini_plan = np.full_like(plan, -1)
        for i, t in enumerate(toks):
            r = t // s.T_o
            for j in range(s.k):
                if plan[i, j] >= 0:
                    e = run.idx[t, j]
                    g = e * s.R + r
                    p = lay["padded_off"][g] + plan[i, j] - lay["recv_off"][g]
                    mini_plan[i, j] = len(src_rows)
                    src_rows.append(p)
        y_rows = run.check_rows(np.array(src_rows, dtype=np.int64), "y of sampled tokens") if src_rows else \
            np.zeros((0, s.d))
        mini = {"combine_plan": np.ascontiguousarray(mini_plan, dtype=np.int32)}
        out_ref = oracle.combine(mini, run.w[toks], [y_rows], 1, len(toks), s.k, s.dtype == "bf16")
        slack = tolerance.combine_slack(mini["combine_plan"], run.w[toks], y_rows, lambda i, j: mini_plan[i, j]) \
            if s.dtype == "bf16" else None
        tolerance.check(f64(P.out)[toks], out_ref, "out tokens", slack=slack)
    # sequential == overlapped, bitwise
    recv_ovl = [bits(b) for b in P.recv]
    out_ovl = bits(P.out)
    run.ffn(mode=1, consumer_cus=BENCH_CONSUMER_CUS)
    P.combine()
    torch.cuda.synchronize()
    for r in range(s.R):
        np.testing.assert_array_equal(bits(P.recv[r]), recv_ovl[r])
    np.testing.assert_array_equal(bits(P.out), out_ovl)
    # the launch landing the token rows itself, in the benchmark's configuration
    check_landing(run, recv_ovl, out_ovl, mode=0, consumer_cus=BENCH_CONSUMER_CUS)


STRESS_SHAPES = [
    # 4 k-splits (partial sums handed between workgroups, last-arriver reductions), ragged row tiles
    mi.Spec("stress_splitk", R=4, T_o=600, G=8, E_l=2, k=2, d=256, f=1024, M=32, seed=21),
    # no split, many small segments (16 experts x 4 owners), many flags per segment wait
    mi.Spec("stress_segs", R=4, T_o=512, G=16, E_l=4, k=2, d=512, f=512, M=32, seed=25),
]


@pytest.mark.parametrize("mgb", [1, 2])
@pytest.mark.parametrize("s", STRESS_SHAPES, ids=lambda v: v.name)
def test_overlap_ordering_stress(s, mgb):
    """Publish/acquire ordering under stress (the page's falsifier: "What would settle it"): 500 overlapped calls per
    shape and segment size (2,000 in all) over consumer partitions {1, 2, 4, 8, 16, 32}, band windows {2, 4, 16} and
    shuffled epochs; every call's delivered rows, and the self owner's rows the producer stores, must equal the
    sequential call's bit for bit.  Stops at the first mismatch (and names the call)."""
    s = dataclasses.replace(s, mgb=mgb)
    run = Run(s)
    check_route_and_layout(run)
    P = run.P
    run.ffn(mode=1)
    torch.cuda.synchronize()
    assert P.status() == B.MOE_OK
    ref = [P.recv[r][: int(run.lay["N_r"][r])].clone() for r in range(s.R)]
    rng = np.random.default_rng(1000 + mgb)
    last = P.epoch
    for it in range(500):
        cus = int(rng.choice([1, 2, 4, 8, 16, 32]))
        win = int(rng.choice([2, 4, 16]))
        ep = last
        while ep == last:  # shuffled, but never the value the flags hold from the previous call
            ep = int(rng.integers(1, 1 << 31))
        last = ep
        for r in range(s.R):
            P.recv[r].fill_(float("nan"))
        run.ffn(mode=0, consumer_cus=cus, band_window=win, epoch=ep)
        torch.cuda.synchronize()
        st = P.status()
        assert st == B.MOE_OK, "call %d (consumer_cus %d, band_window %d): status %d" % (it, cus, win, st)
        for r in range(s.R):
            got = P.recv[r][: ref[r].shape[0]]
            if not torch.equal(got.view(torch.int16), ref[r].view(torch.int16)):
                bad = (got.view(torch.int16) != ref[r].view(torch.int16)).any(dim=1).nonzero().flatten()[:8].tolist()
                raise AssertionError("call %d (consumer_cus %d, band_window %d, epoch %d): owner %d rows %s differ"
                                     % (it, cus, win, ep, r, bad))
    check_delivery(run)


@pytest.mark.parametrize("name", ["splitk", "mixtral"])
def test_no_stale_reads_across_calls(name):
    """Results handed between workgroups inside the FFN launch (h tiles, split-K partial sums, y tiles) are read
    only once they are complete and visible: a call on new data after a call on old data, with h and y_pad
    poisoned in between, gives bit for bit what a fresh run on the new data gives."""
    s = [c for c in SMALL if c.name == name][0] if name != "mixtral" else mi.spec("mixtral")
    run = Run(s)
    run.ffn(mode=0)
    torch.cuda.synchronize()
    assert run.P.status() == B.MOE_OK
    neg = -run.dev["x"]  # same routing, different h, partial sums and y everywhere
    run.P.h.fill_(float("nan"))
    run.P.y_pad.fill_(float("nan"))
    run.P.recv[SELF].fill_(float("nan"))
    run.P.layout(neg)
    run.ffn(mode=0)
    fresh = MoePath.from_spec(s)
    fresh.route(run.dev["logits"])
    fresh.layout(neg)
    fresh.ffn(run.dev["w_gate_up"], run.dev["w_down"], mode=1)
    torch.cuda.synchronize()
    assert run.P.status() == B.MOE_OK and fresh.status() == B.MOE_OK
    lay = run.lay
    own = lay["tile_owner"][np.arange(lay["M_pad"]) // s.M] == SELF
    real = np.nonzero((lay["row_src"] >= 0) & ~own)[0]
    np.testing.assert_array_equal(bits(run.P.y_pad)[real], bits(fresh.y_pad)[real])
    # the self owner's rows went straight to its buffer: y_pad keeps the poison there
    mine = np.nonzero((lay["row_src"] >= 0) & own)[0]
    assert np.isnan(f64(run.P.y_pad[torch.as_tensor(mine, device=run.P.y_pad.device)])).all()
    for r in range(s.R):
        n_r = int(run.lay["N_r"][r])
        np.testing.assert_array_equal(bits(run.P.recv[r])[:n_r], bits(fresh.recv[r])[:n_r])


@pytest.mark.parametrize("name", ["tiny", "splitk"])
def test_return_only_repeats(name):
    """The return alone, for flags an overlapped call already published, delivers the same rows again, call after
    call and whatever the partition: every launch hands out its copy units afresh (a new stamp on the counter)."""
    s = [c for c in SMALL if c.name == name][0]
    run = Run(s)
    for r in range(s.R):
        run.P.recv[r].fill_(float("nan"))
    epoch = run.ffn(mode=0, consumer_cus=4)
    torch.cuda.synchronize()
    assert run.P.status() == B.MOE_OK
    check_delivery(run)
    ref = [bits(b) for b in run.P.recv]
    for cus in (3, 16, 1):
        for r in range(s.R):  # the return delivers the other owners' rows (the producer stored the self owner's)
            if r != SELF:
                run.P.recv[r].fill_(float("nan"))
        run.P.ffn(run.dev["w_gate_up"], run.dev["w_down"], mode=2, consumer_cus=cus, epoch=epoch)
        torch.cuda.synchronize()
        assert run.P.status() == B.MOE_OK
        check_delivery(run)
        for a, b in zip(ref, run.P.recv):
            np.testing.assert_array_equal(a, bits(b))


def test_watchdog_ends_a_wait_that_never_ends():
    s = mi.spec("tiny")
    run = Run(s)
    run.ffn(mode=0, consumer_cus=2)
    torch.cuda.synchronize()
    assert run.P.status() == B.MOE_OK
    # return only, for an epoch the producer never published: the consumer must give up, not hang
    run.P.ffn(run.dev["w_gate_up"], run.dev["w_down"], mode=2, consumer_cus=2, watchdog_ticks=100000, epoch=999)
    torch.cuda.synchronize()
    assert run.P.status() == B.MOE_ETIMEOUT
    # later kernels are no-ops until the next layout resets the status
    run.P.out.fill_(7.0)
    run.P.combine()
    torch.cuda.synchronize()
    assert (f64(run.P.out) == 7.0).all()
    run.P.layout(run.dev["x"])
    torch.cuda.synchronize()
    assert run.P.status() == B.MOE_OK


@pytest.mark.parametrize("name", ["splitk", "splitk_windows"])
def test_tiny_spin_budget_ends_every_wait(name):
    """With a one-tick spin budget the producer's waits for h tiles, the consumer's waits and the workgroups that
    join the return give up instead of waiting: the launch ends with MOE_OK (nothing had to wait) or
    MOE_ETIMEOUT, and the next call, on a fresh layout, delivers exactly what a fresh run delivers."""
    s = [c for c in SMALL if c.name == name][0]
    run = Run(s)
    run.ffn(mode=0, consumer_cus=4, watchdog_ticks=1)
    torch.cuda.synchronize()
    assert run.P.status() in (B.MOE_OK, B.MOE_ETIMEOUT)
    run.P.layout(run.dev["x"])
    for r in range(s.R):
        run.P.recv[r].fill_(float("nan"))
    run.ffn(mode=0, consumer_cus=4)
    fresh = MoePath.from_spec(s)
    fresh.route(run.dev["logits"])
    fresh.layout(run.dev["x"])
    fresh.ffn(run.dev["w_gate_up"], run.dev["w_down"], mode=1)
    torch.cuda.synchronize()
    assert run.P.status() == B.MOE_OK and fresh.status() == B.MOE_OK
    check_delivery(run)
    for r in range(s.R):
        n_r = int(run.lay["N_r"][r])
        np.testing.assert_array_equal(bits(run.P.recv[r])[:n_r], bits(fresh.recv[r])[:n_r])


def test_capacity_overflow_reported():
    s = mi.spec("tiny")
    run = Run(s)
    P = run.P
    P.L.cap_rows = s.M
    P.L.cap_tiles = 1
    P.layout(run.dev["x"])
    torch.cuda.synchronize()
    assert P.status() == B.MOE_ECAPACITY
    assert P.scalars()["M_pad"] == 0


def test_empty_and_degenerate_inputs():
    # no tokens
    s = mi.spec("tiny", T_o=0)
    P = MoePath.from_spec(s)
    P.route(torch.empty(0, s.G, device="cuda"))
    P.layout(torch.empty(0, s.d, dtype=torch.bfloat16, device="cuda"))
    w1, w2 = (to_device(a, s.dtype) for a in mi.weights(s))
    P.ffn(w1, w2)
    P.combine()
    torch.cuda.synchronize()
    assert P.status() == B.MOE_OK and P.scalars()["M_pad"] == 0
    # no token routed to a local expert: out is zero
    s = mi.spec("tiny")
    lg = mi.logits(s)
    lg[:, : s.E_l] -= 100.0
    run = Run(s, logits=lg)
    check_route_and_layout(run)
    run.ffn()
    run.P.combine()
    torch.cuda.synchronize()
    assert run.P.scalars()["M_pad"] == 0 and (f64(run.P.out[: s.T]) == 0).all()
    # every token routed to local expert 0
    lg = mi.logits(s)
    lg[:, 0] += 100.0
    run = Run(s, logits=lg)
    check_route_and_layout(run)
    run.ffn()
    torch.cuda.synchronize()
    real = np.nonzero(run.lay["row_src"] >= 0)[0]
    run.check_rows(real)
