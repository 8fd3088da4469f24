"""The FFN launch's work-item list on the CPU (no GPU): the list the library reports (``moe_ffn_schedule``, the
kernel's own code, compiled for the host) over row tiles modelled from the oracle's layout, on every workload, in
overlapped and sequential mode and over band windows and consumer partitions.

Checked: every item exactly once; every wait is on an earlier GEMM1 item; a run of the list with random item times
always finishes (no wait that never ends), also when the half-width items are handed out from a counter instead of
statically; each y tile's arrival target equals the items that arrive; remote-first order of the row tiles.
"""
import ctypes

import numpy as np
import pytest

import moe_inputs as mi
import oracle
import schedule_model as sm
from expert_output_overlap_amd import binding as B

N_CU = 256
SMALL = [
    mi.spec("tiny"),
    mi.Spec("ragged", R=4, T_o=300, G=16, E_l=4, k=2, d=256, f=512, M=32, seed=11),
    mi.Spec("splitk", R=4, T_o=600, G=8, E_l=2, k=2, d=256, f=1024, M=32, seed=16),
    mi.Spec("splitk6", R=3, T_o=200, G=6, E_l=2, k=1, d=256, f=1536, M=16, seed=19),
    mi.Spec("splitk_windows", R=4, T_o=2400, G=8, E_l=2, k=2, d=256, f=1024, M=32, seed=22),
    mi.Spec("splitk_halves", R=4, T_o=3150, G=4, E_l=1, k=2, d=256, f=1024, M=32, seed=23),
    mi.Spec("halves", R=4, T_o=12800, G=4, E_l=1, k=2, d=256, f=256, M=32, seed=24),
    mi.Spec("one_owner", R=1, T_o=200, G=1, E_l=1, k=1, d=128, f=128, M=16, seed=13),
]
FULL = ["mixtral", "skew", "sweep1", "sweep2", "sweep4", "sweep8", "sweep16", "deepseek"]

_cache = {}


def tiles_of(s, self_rank=0):
    key = (s, self_rank)
    if key not in _cache:
        idx, _ = oracle.route(mi.logits(s), s.k)
        lay = oracle.layout(idx, s.R, s.T_o, s.G, s.E_l, s.k, s.M, s.mgb, self_rank)
        _cache[key] = sm.packing(lay["counts"], lay["padded_off"], s.R, s.E_l, self_rank, s.M)
    return _cache[key]


def shape_of(s, self_rank=0):
    return B.moe_shape(s.R, s.T_o, s.G, s.E_l, s.k, self_rank, s.d, s.f, s.M, s.mgb, B.MOE_BF16)


def schedule(s, mode, cus=0, window=0, self_rank=0, tile_order=0):
    hdr, _, pure, order = tiles_of(s, self_rank)
    cfg = B.moe_overlap_cfg(cus, mode, 1, window, 0, None, tile_order)
    items = B.moe_ffn_schedule(shape_of(s, self_rank), N_CU, cfg, hdr, order, int((~pure).sum()))
    # with the row-tile numbering there is no remote-first order to check
    return items, hdr, pure if tile_order == 0 else np.zeros_like(pure)


def consumers_of(s, mode, cus, self_rank=0):
    """The consumer count of the schedule: consumer_cus, or for 0 the launch's rule with default rates on the
    batch (every row of the row tiles holding another owner's row counted as returned), as moe_ffn_schedule takes."""
    if mode != 0 or cus < 0:
        return 0
    if cus > 0:
        return cus
    hdr, _, pure, order = tiles_of(s, self_rank)
    m_real = int(hdr[:, 1].sum())
    m_ret = int(hdr[order[: int((~pure).sum())], 1].sum())
    return B.moe_pick_consumer_cus_observed(shape_of(s, self_rank), N_CU, m_real, m_ret, len(hdr), 0.0, 0.0)


@pytest.mark.parametrize("mode,cus", [(0, 0), (1, 0), (0, 16)])
@pytest.mark.parametrize("name", FULL)
def test_full_workload_lists(name, mode, cus):
    """The bench's launch configuration (the launch's consumer partition, default band window) on every workload,
    and a 16-CU partition; the consumer count the schedule reports for the launch's rule is the rule's."""
    s = mi.spec(name)
    items, hdr, pure = schedule(s, mode, cus)
    waits = sm.check_list(items, len(hdr), s.d, s.f, pure)
    sm.simulate(items, waits, seed=1)
    C = consumers_of(s, mode, cus)
    assert items[:, 0].max() + 1 == N_CU  # every workgroup appears: C consumers first, then the producers
    if mode == 0:  # the consumer workgroups' own share is GEMM1 items only (they wait on nothing)
        cons = items[:, 0] < C
        assert (items[cons, 2] == 1).all()
        if cus == 0 and name in ("deepseek", "mixtral", "skew", "sweep4", "sweep8", "sweep16"):
            assert C == 0  # the return fits in the round-robin's slack
        if cus == 0 and name in ("sweep1", "sweep2"):
            assert C == 8  # full first-GEMM rounds: a partition


@pytest.mark.parametrize("window", [0, 2, 16])
@pytest.mark.parametrize("cus", [1, 8, 32])
@pytest.mark.parametrize("s", SMALL + [mi.spec("mixtral")], ids=lambda v: v.name)
def test_lists_over_partitions_and_windows(s, cus, window):
    for mode in (0, 1):
        for tile_order in (0, 1):
            items, hdr, pure = schedule(s, mode, cus, window, tile_order=tile_order)
            waits = sm.check_list(items, len(hdr), s.d, s.f, pure)
            sm.simulate(items, waits, seed=cus + window)


@pytest.mark.parametrize("s,self_rank", [(SMALL[1], 2), (SMALL[2], 1), (mi.spec("skew"), 3)],
                         ids=lambda v: v.name if isinstance(v, mi.Spec) else "rank%d" % v)
def test_lists_at_other_ranks(s, self_rank):
    items, hdr, pure = schedule(s, 0, self_rank=self_rank)
    sm.check_list(items, len(hdr), s.d, s.f, pure)


@pytest.mark.parametrize("name,mode,cus", [("splitk_halves", 1, 0), ("halves", 1, 0), ("mixtral", 0, 8),
                                           ("mixtral", 1, 0), ("deepseek", 0, 16), ("skew", 1, 0), ("sweep1", 0, 8)])
def test_half_width_items_handed_out_from_a_counter(name, mode, cus):
    """The half-width final round with its halves taken from a counter by whichever workgroup is free first (the
    variant whose GPU test once hung, and was dropped): in any such order every half runs once, its waits (GEMM1
    items) all finish, and the arrival targets, which the list fixes, are those of the static order."""
    s = [c for c in SMALL if c.name == name][0] if name in {c.name for c in SMALL} else mi.spec(name)
    items, hdr, pure = schedule(s, mode, cus)
    assert (items[:, 6] >= 0).any(), "this configuration must halve its last round"
    waits = sm.check_list(items, len(hdr), s.d, s.f, pure)
    for seed in range(3):
        order = sm.simulate(items, waits, claim_halves=True, seed=seed)
        assert sorted(order) == list(range(len(items)))


@pytest.mark.parametrize("name", ["mixtral", "deepseek", "skew"])
def test_remote_first_order_has_self_only_tiles_last(name):
    """Row tiles of self-owned rows only (an expert's self-owned rows, which its run packs last, fill such a tile when
    they reach past the run's last tile boundary) come last in the producer's order, and their second-GEMM items end
    the list in both modes; the other row tiles keep their numbering, expert by expert."""
    s = mi.spec(name)
    _, _, pure, order = tiles_of(s)
    npure = int(pure.sum())
    assert npure >= 1
    assert (order[-npure:] == np.nonzero(pure)[0]).all() and (order[:-npure] == np.nonzero(~pure)[0]).all()
    for mode in (0, 1):
        items, hdr, pure = schedule(s, mode)
        g2 = items[items[:, 2] == 2]
        is_pure = pure[g2[:, 3]]
        # the GEMM2 items of self-owned-only row tiles are exactly the list's last ones
        assert is_pure.sum() > 0 and is_pure[-int(is_pure.sum()):].all()


def test_schedule_rejects_bad_input():
    s = mi.spec("tiny")
    hdr, _, _, order = tiles_of(s)
    cfg = B.moe_overlap_cfg(0, 0, 1, 0, 0, None)
    bad = hdr.copy()
    bad[0, 3] = len(hdr) + 5
    with pytest.raises(B.MoeError):
        B.moe_ffn_schedule(shape_of(s), N_CU, cfg, bad, order, len(hdr))
    f32 = B.moe_shape(s.R, s.T_o, s.G, s.E_l, s.k, 0, s.d, s.f, s.M, s.mgb, B.MOE_F32)
    with pytest.raises(B.MoeError):
        B.moe_ffn_schedule(f32, N_CU, cfg, hdr, order, len(hdr))
    n = ctypes.c_int64(0)
    h = np.ascontiguousarray(hdr, dtype=np.int32)
    o = np.ascontiguousarray(order, dtype=np.int32)
    assert B.lib().moe_ffn_schedule(ctypes.byref(shape_of(s)), N_CU, ctypes.byref(cfg), len(hdr), len(hdr),
                                    h.ctypes.data, o.ctypes.data, None, 0, ctypes.byref(n)) == 0 and n.value > 0
    small = np.zeros((1, 8), np.int32)
    assert B.lib().moe_ffn_schedule(ctypes.byref(shape_of(s)), N_CU, ctypes.byref(cfg), len(hdr), len(hdr),
                                    h.ctypes.data, o.ctypes.data, small.ctypes.data, 1,
                                    ctypes.byref(n)) == B.MOE_EINVAL
