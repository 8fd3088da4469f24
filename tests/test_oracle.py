"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than its own formula: the padding numbers printed on the
review page, invariants that define the layout uniquely, library routines for special cases (softmax, dense
matmul, torch's fp32->bf16 rounding), exact algebraic identities, and hand-worked examples.
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

import moe_inputs as mi
import oracle


# ----------------------------------------------------------------------------------------------------------------
# bf16 rounding

def test_round_bf16_matches_torch_on_fp32_values(orc):
    v = mi.normal_f32(2, 77, (4000,), 0.0, 3.0)
    v = np.concatenate([v, np.array([1e-38, -3e-39, 65504.0, 3.0e38, 1.0 + 2.0 ** -8], np.float32)])
    ref = torch.from_numpy(v).to(torch.bfloat16).double().numpy()
    got = np.array([orc.orc_round_bf16(float(x)) for x in v])
    assert (got == ref).all()


def test_round_bf16_ties_and_direct_rounding(orc):
    assert orc.orc_round_bf16(1.0 + 2.0 ** -8) == 1.0                     # tie, to even
    assert orc.orc_round_bf16(1.0 + 3 * 2.0 ** -8) == 1.0 + 2.0 ** -6     # tie, to even (up)
    # just above a tie: correct rounding goes up; rounding to fp32 first would land on the tie and go down
    assert orc.orc_round_bf16(1.0 + 2.0 ** -8 + 2.0 ** -40) == 1.0 + 2.0 ** -7
    assert orc.orc_round_bf16(-(1.0 + 2.0 ** -8 + 2.0 ** -40)) == -(1.0 + 2.0 ** -7)
    assert orc.orc_round_bf16(0.0) == 0.0


# ----------------------------------------------------------------------------------------------------------------
# routing

def _check_topk_definition(logits, idx):
    """Top-k by logit descending with ties to the lower id, as invariants that fix it uniquely."""
    T, G = logits.shape
    k = idx.shape[1]
    for t in range(T):
        chosen = idx[t]
        assert len(set(chosen.tolist())) == k
        rest = np.setdiff1d(np.arange(G), chosen)
        lc = logits[t, chosen]
        # ordered: descending logit, equal logits by ascending id
        for a in range(k - 1):
            assert lc[a] > lc[a + 1] or (lc[a] == lc[a + 1] and chosen[a] < chosen[a + 1])
        if rest.size:
            worst = lc[-1]
            assert (logits[t, rest] <= worst).all()
            tied = rest[logits[t, rest] == worst]
            assert (tied > chosen[-1]).all()


@pytest.mark.parametrize("G,k", [(8, 2), (64, 6), (4, 4), (256, 8), (1, 1)])
def test_route_topk_invariants_and_softmax(orc, G, k):
    lg = mi.normal_f32(3, 1, (64, G))
    lg[:8] = np.round(lg[:8])  # many exact ties
    idx, w = oracle.route(lg, k, orc)
    _check_topk_definition(lg, idx)
    sm = scipy.special.softmax(lg.astype(np.float64), axis=1)
    ref = np.take_along_axis(sm, idx.astype(np.int64), axis=1)
    np.testing.assert_allclose(w, ref, rtol=1e-6, atol=0)


def test_route_all_equal_logits(orc):
    idx, w = oracle.route(np.zeros((3, 8), np.float32), 3, orc)
    assert (idx == np.array([0, 1, 2])).all()
    assert np.allclose(w, 1.0 / 8.0, rtol=1e-7)


# ----------------------------------------------------------------------------------------------------------------
# padding: the section 4.5 numbers printed by the referee

def test_padding_numbers_from_section_4_5(orc, golden_dir):
    g = json.load(open(os.path.join(golden_dir, "padding_section45.json")))
    E, W, tbM = g["E"], g["W"], g["tbM"]
    worst = np.ones(E * W, np.int32)          # n = 1 (mod tbM) in every group: tbM-1 padding rows each
    assert oracle.padding_rows(worst[:W], 1, W, tbM, 0, False, orc) == g["claimed_bound_rows"]
    assert oracle.padding_rows(worst, E, W, tbM, 0, False, orc) == g["true_bound_rows"]
    bal = np.full(E * W, g["M_rows_per_rank"] // (E * W), np.int32)
    assert bal[0] == g["balanced_rows_per_group"]
    assert oracle.padding_rows(bal[:1], 1, 1, tbM, 1, True, orc) == g["balanced_padding_per_group"]
    assert oracle.padding_rows(bal, E, W, tbM, 0, False, orc) == g["balanced_total_padding_rows"]
    # every group padded (this build pads the self group too): one more group per expert
    assert oracle.padding_rows(bal, E, W, tbM, 0, True, orc) == g["balanced_total_padding_rows"] * W // (W - 1)


def test_layout_balanced_section_4_5_shape(orc, golden_dir):
    """Layout of a balanced routing at the section 4.5 shape: M_pad - M_real is the padding calculator's value."""
    g = json.load(open(os.path.join(golden_dir, "padding_section45.json")))
    E, W, tbM = g["E"], g["W"], g["tbM"]
    T_o = g["M_rows_per_rank"] // W
    # token t of every owner goes to local expert t mod E (k=1, G=E): 64 rows per (expert, owner) group
    idx = np.tile(np.arange(T_o, dtype=np.int32) % E, W).reshape(-1, 1)
    lay = oracle.layout(idx, W, T_o, E, E, 1, tbM, 1, 0, orc)
    assert (lay["counts"] == g["balanced_rows_per_group"]).all()
    assert lay["M_pad"] - g["M_rows_per_rank"] == oracle.padding_rows(lay["counts"], E, W, tbM, 0, True, orc)
    assert lay["M_pad"] == E * W * tbM


# ----------------------------------------------------------------------------------------------------------------
# layout

def check_layout_invariants(lay, idx, R, T_o, E_l, k, M, mgb, self_rank=0):
    """Invariants that define the remote-owner-aligned layout (and so pin it on any input)."""
    T = R * T_o
    lo = self_rank * E_l
    counts, poff, roff = lay["counts"], lay["padded_off"], lay["recv_off"]
    M_pad, n_tiles = lay["M_pad"], lay["n_tiles"]
    local = (idx >= lo) & (idx < lo + E_l)
    assert counts.sum() == local.sum()                               # every local slot has a row
    P = -(-counts // M) * M
    assert M_pad == P.sum() and M_pad % M == 0 and n_tiles == M_pad // M
    order = [(e, r) for e in range(E_l) for r in range(R)]            # expert-major, owner-minor
    run = 0
    for (e, r) in order:
        assert poff[e * R + r] == run and run % M == 0
        run += P[e * R + r]
    for r in range(R):
        assert lay["N_r"][r] == counts[r::R].sum()
        run = 0
        for e in range(E_l):
            assert roff[e * R + r] == run
            run += counts[e * R + r]
    # bands: exactly one owner and expert each, valid rows = real rows inside the band
    row_src = lay["row_src"]
    for b in range(n_tiles):
        rows = row_src[b * M:(b + 1) * M]
        assert lay["tile_valid"][b] == (rows >= 0).sum() >= 1
        assert (rows[: lay["tile_valid"][b]] >= 0).all() and (rows[lay["tile_valid"][b]:] < 0).all()
        e, r = lay["tile_expert"][b], lay["tile_owner"][b]
        assert poff[e * R + r] <= b * M < poff[e * R + r] + P[e * R + r]
        toks = rows[rows >= 0]
        assert (toks // T_o == r).all()                              # rows of one owner only
        assert all(e + lo in idx[t] for t in toks)                   # routed to that expert
    # each local (token, slot) appears exactly once; rows ascend by token inside a group
    plan = lay["combine_plan"]
    seen = np.zeros(M_pad, bool)
    for t in range(T):
        r = t // T_o
        for j in range(k):
            e = idx[t, j] - lo
            if 0 <= e < E_l:
                i = plan[t, j] - roff[e * R + r]
                assert 0 <= i < counts[e * R + r]
                p = poff[e * R + r] + i
                assert row_src[p] == t and not seen[p]
                seen[p] = True
            else:
                assert plan[t, j] == -1
    assert seen.sum() == counts.sum() and ((row_src >= 0) == seen).all()
    for g in range(E_l * R):
        seg = row_src[poff[g]: poff[g] + counts[g]]
        assert (np.diff(seg) > 0).all()
    # remote-first order: a permutation of the bands; groups by (is_self, -P, e, r), bands ascending
    tord = lay["tile_order"]
    assert sorted(tord.tolist()) == list(range(n_tiles))
    keys = [(int(lay["tile_owner"][b] == self_rank), -int(P[lay["tile_expert"][b] * R + lay["tile_owner"][b]]),
             int(lay["tile_expert"][b]), int(lay["tile_owner"][b]), int(b)) for b in tord]
    assert keys == sorted(keys)
    # segments: follow tile_order, at most mgb bands, real rows only, contiguous on both sides
    segs = lay["seg_desc"]
    walked = []
    delivered = 0
    for s in segs:
        r, e, b0, nb, src, dst, rows, g = s.tolist()
        assert 1 <= nb <= mgb and g == e * R + r and src == b0 * M
        walked += list(range(b0, b0 + nb))
        assert dst == roff[g] + (src - poff[g])
        assert 0 < rows <= nb * M and (row_src[src:src + rows] >= 0).all()
        assert rows == nb * M or src + rows == poff[g] + counts[g]
        delivered += rows
    assert walked == tord.tolist() and delivered == counts.sum()


def _tiny_idx(seed, R, T_o, G, k):
    lg = mi.normal_f32(seed, 1, (R * T_o, G))
    return oracle.route(lg, k)[0]


@pytest.mark.parametrize("R,T_o,G,E_l,k,M,mgb", [
    (4, 16, 8, 2, 2, 16, 1), (4, 16, 8, 2, 2, 16, 2), (2, 37, 6, 3, 3, 4, 3), (1, 50, 1, 1, 1, 8, 1),
    (3, 20, 9, 3, 3, 5, 2), (4, 64, 64, 16, 6, 8, 1), (8, 8, 256, 32, 8, 4, 2), (1, 1, 4, 2, 2, 16, 1)])
def test_layout_invariants_random(orc, R, T_o, G, E_l, k, M, mgb):
    idx = _tiny_idx(R * 100 + T_o, R, T_o, G, k)
    lay = oracle.layout(idx, R, T_o, G, E_l, k, M, mgb, 0, orc)
    check_layout_invariants(lay, idx, R, T_o, E_l, k, M, mgb)


def test_layout_nonzero_self_rank(orc):
    R, T_o, G, E_l, k, M = 4, 40, 16, 4, 3, 8
    idx = _tiny_idx(9, R, T_o, G, k)
    lay = oracle.layout(idx, R, T_o, G, E_l, k, M, 2, 2, orc)
    check_layout_invariants(lay, idx, R, T_o, E_l, k, M, 2, self_rank=2)


def test_layout_sorting_formulation(orc):
    """The row permutation equals a stable lexicographic sort of local slots by (expert, owner, token)."""
    R, T_o, G, E_l, k, M = 4, 33, 12, 3, 4, 8
    idx = _tiny_idx(5, R, T_o, G, k)
    lay = oracle.layout(idx, R, T_o, G, E_l, k, M, 1, 0, orc)
    t, j = np.nonzero(idx < E_l)
    e = idx[t, j]
    o = np.lexsort((t, t // T_o, e))
    real_rows = lay["row_src"][lay["row_src"] >= 0]
    assert (real_rows == t[o]).all()


def test_layout_hand_worked_example(orc):
    """R=2 owners x 3 tokens, G=4, E_l=2, k=2, M=2, computed by hand.

    owner 0: t0 -> {0, 2}, t1 -> {1, 0}, t2 -> {3, 2};   owner 1: t3 -> {0, 1}, t4 -> {2, 3}, t5 -> {1, 3}
    groups (e, r): (0,0) = [t0, t1] n=2; (0,1) = [t3] n=1; (1,0) = [t1] n=1; (1,1) = [t3, t5] n=2
    """
    idx = np.array([[0, 2], [1, 0], [3, 2], [0, 1], [2, 3], [1, 3]], np.int32)
    lay = oracle.layout(idx, 2, 3, 4, 2, 2, 2, 1, 0, orc)
    assert lay["counts"].tolist() == [2, 1, 1, 2]
    assert lay["padded_off"].tolist() == [0, 2, 4, 6]
    assert lay["recv_off"].tolist() == [0, 0, 2, 1]
    assert lay["M_pad"] == 8 and lay["n_tiles"] == 4 and lay["N_r"].tolist() == [3, 3]
    assert lay["row_src"].tolist() == [0, 1, 3, -1, 1, -1, 3, 5]
    assert lay["tile_owner"].tolist() == [0, 1, 0, 1] and lay["tile_expert"].tolist() == [0, 0, 1, 1]
    assert lay["tile_valid"].tolist() == [2, 1, 1, 2]
    # remote groups first (owner 1: (0,1) and (1,1), both P=2, by expert), then the self groups
    assert lay["tile_order"].tolist() == [1, 3, 0, 2]
    assert lay["combine_plan"].tolist() == [[0, -1], [2, 1], [-1, -1], [0, 1], [-1, -1], [2, -1]]
    assert lay["seg_desc"][:, :7].tolist() == [[1, 0, 1, 1, 2, 0, 1], [1, 1, 3, 1, 6, 1, 2],
                                               [0, 0, 0, 1, 0, 0, 2], [0, 1, 2, 1, 4, 2, 1]]


def test_layout_edge_cases(orc):
    # empty input
    lay = oracle.layout(np.zeros((0, 2), np.int32), 4, 0, 8, 2, 2, 16, 1, 0, orc)
    assert lay["M_pad"] == 0 and lay["n_tiles"] == 0 and lay["n_segs"] == 0
    # no local expert hit
    idx = np.full((12, 2), 5, np.int32)
    idx[:, 1] = 6
    lay = oracle.layout(idx, 3, 4, 8, 2, 2, 4, 1, 0, orc)
    assert lay["M_pad"] == 0 and (lay["combine_plan"] == -1).all()
    # all tokens to one expert; n a multiple of M (no padding)
    R, T_o, M = 2, 8, 4
    idx = np.zeros((R * T_o, 1), np.int32)
    lay = oracle.layout(idx, R, T_o, 4, 2, 1, M, 2, 0, orc)
    assert lay["counts"].tolist() == [8, 8, 0, 0] and lay["M_pad"] == 16
    check_layout_invariants(lay, idx, R, T_o, 2, 1, M, 2)
    # k = E_l: every token hits every local expert
    idx = np.tile(np.array([1, 0, 2], np.int32), (10, 1))
    lay = oracle.layout(idx, 2, 5, 3, 3, 3, 4, 1, 0, orc)
    assert lay["counts"].tolist() == [5] * 6
    check_layout_invariants(lay, idx, 2, 5, 3, 3, 4, 1)


def test_layout_identity_special_case(orc):
    """R=1, E_l=1, k=1: the layout is the identity permutation followed by padding."""
    T, M = 45, 16
    lay = oracle.layout(np.zeros((T, 1), np.int32), 1, T, 1, 1, 1, M, 1, 0, orc)
    assert lay["M_pad"] == 48
    assert lay["row_src"].tolist() == list(range(T)) + [-1] * 3
    assert lay["combine_plan"][:, 0].tolist() == list(range(T))


@pytest.mark.parametrize("name", ["tiny", "skew", "mixtral", "deepseek", "sweep1", "sweep16"])
def test_layout_invariants_configs(orc, name):
    s = mi.spec(name)
    if name in ("deepseek", "sweep16", "mixtral", "skew"):
        s = mi.spec(name, T_o=256)  # full-size layouts are checked vectorised below; loops here stay quick
    idx, _ = oracle.route(mi.logits(s), s.k, orc)
    lay = oracle.layout(idx, s.R, s.T_o, s.G, s.E_l, s.k, s.M, s.mgb, 0, orc)
    check_layout_invariants(lay, idx, s.R, s.T_o, s.E_l, s.k, s.M, s.mgb)


@pytest.mark.parametrize("name", ["mixtral", "skew", "deepseek", "sweep4"])
def test_layout_full_size_vectorised(orc, name):
    s = mi.spec(name)
    idx, _ = oracle.route(mi.logits(s), s.k, orc)
    lay = oracle.layout(idx, s.R, s.T_o, s.G, s.E_l, s.k, s.M, 2, 0, orc)
    t, j = np.nonzero(idx < s.E_l)
    e = idx[t, j]
    o = np.lexsort((t, t // s.T_o, e))
    assert (lay["row_src"][lay["row_src"] >= 0] == t[o]).all()
    cnt = np.bincount(e * s.R + t // s.T_o, minlength=s.E_l * s.R)
    assert (lay["counts"] == cnt).all()
    assert lay["M_pad"] == (-(-cnt // s.M) * s.M).sum()
    assert (lay["combine_plan"][idx >= s.E_l] == -1).all()
    assert lay["seg_desc"][:, 6].sum() == cnt.sum()


# ----------------------------------------------------------------------------------------------------------------
# FFN

def _silu(v):
    return v / (1.0 + np.exp(-v))


def _rand_expert(seed, E, d, f, dtype):
    gen = mi.normal_bf16 if dtype == "bf16" else mi.normal_f32
    w1 = gen(seed, 100, (E, 2 * f, d), 0.0, 1 / math.sqrt(d))
    w2 = gen(seed, 101, (E, d, f), 0.0, 1 / math.sqrt(d))
    x = gen(seed, 102, (10, d))
    return x, w1, w2


def _to64(a, dtype):
    return mi.bf16_bits_to_f32(a).astype(np.float64) if dtype == "bf16" else a.astype(np.float64)


def test_ffn_dense_mlp_matmul_fp32(orc):
    """In fp32 mode the FFN of each row is the dense SwiGLU MLP: silu(x Wg^T) * (x Wu^T) @ Wd^T."""
    d, f, E = 32, 48, 3
    x, w1, w2 = _rand_expert(1, E, d, f, "f32")
    src = np.arange(10, dtype=np.int32)
    ex = (np.arange(10) % E).astype(np.int32)
    y = oracle.ffn_rows(src, ex, x, w1, w2, False, orc)
    for i in range(10):
        X = x[i:i + 1].astype(np.float64)
        W1, W2 = w1[ex[i]].astype(np.float64), w2[ex[i]].astype(np.float64)
        ref = (_silu(X @ W1[:f].T) * (X @ W1[f:].T)) @ W2.T
        np.testing.assert_allclose(y[i], ref[0], rtol=1e-12, atol=1e-13)


def test_ffn_bf16_close_to_unrounded(orc):
    d, f = 64, 128
    x, w1, w2 = _rand_expert(2, 2, d, f, "bf16")
    src = np.arange(10, dtype=np.int32)
    ex = (np.arange(10) % 2).astype(np.int32)
    yb = oracle.ffn_rows(src, ex, x, w1, w2, True, orc)
    yf = oracle.ffn_rows(src, ex, mi.bf16_bits_to_f32(x), mi.bf16_bits_to_f32(w1), mi.bf16_bits_to_f32(w2), False,
                         orc)
    # outputs are bf16 values
    assert (np.array([orc.orc_round_bf16(v) for v in yb.ravel()]) == yb.ravel()).all()
    assert np.linalg.norm(yb - yf) / np.linalg.norm(yf) < 5e-3


def test_ffn_silu_known_values(orc):
    """One-hot x and identity-like gate weights give g = known values; silu(1), silu(-1), silu(0), silu(20)."""
    d, f = 4, 4
    x = np.eye(d, dtype=np.float32)[:1]                            # x = e_0
    w1 = np.zeros((1, 2 * f, d), np.float32)
    w1[0, :f, 0] = [1.0, -1.0, 0.0, 20.0]                          # g = [1, -1, 0, 20]
    w1[0, f:, 0] = [1.0, 1.0, 1.0, 1.0]                            # u = 1
    w2 = np.eye(d, f, dtype=np.float32)[None]                      # y = h
    y = oracle.ffn_rows(np.zeros(1, np.int32), np.zeros(1, np.int32), x, w1, w2, False, orc)[0]
    expect = [0.7310585786300049, -0.2689414213699951, 0.0, 20.0 / (1.0 + math.exp(-20.0))]
    np.testing.assert_allclose(y, expect, rtol=1e-15, atol=0)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_ffn_scaling_identities(orc, dtype):
    """Doubling Wu or Wd doubles y exactly; doubling Wg does not (it sits inside silu)."""
    d, f = 64, 96
    x, w1, w2 = _rand_expert(4, 1, d, f, dtype)
    src = np.arange(6, dtype=np.int32)
    ex = np.zeros(6, np.int32)
    bf = dtype == "bf16"

    def dbl(a):  # exact doubling of bf16 bits or fp32 values
        return (a + np.uint16(0x80)).astype(np.uint16) if bf else a * np.float32(2)

    y = oracle.ffn_rows(src, ex, x, w1, w2, bf, orc)
    w1u = w1.copy()
    w1u[:, f:] = dbl(w1[:, f:])
    assert (oracle.ffn_rows(src, ex, x, w1u, w2, bf, orc) == 2 * y).all()
    assert (oracle.ffn_rows(src, ex, x, w1, dbl(w2), bf, orc) == 2 * y).all()
    w1g = w1.copy()
    w1g[:, :f] = dbl(w1[:, :f])
    assert not np.allclose(oracle.ffn_rows(src, ex, x, w1g, w2, bf, orc), 2 * y)


def test_ffn_zero_up_gives_zero(orc):
    d, f = 64, 64
    x, w1, w2 = _rand_expert(6, 2, d, f, "f32")
    w1[:, f:] = 0
    y = oracle.ffn_rows(np.arange(4, dtype=np.int32), np.array([0, 1, 0, 1], np.int32), x, w1, w2, False, orc)
    assert (y == 0).all()


# ----------------------------------------------------------------------------------------------------------------
# delivery and combine

def test_delivery_exactly_once_real_rows_only(orc):
    s = mi.spec("tiny", R=3, T_o=21, M=4, mgb=2)
    idx = _tiny_idx(3, s.R, s.T_o, s.G, s.k)
    lay = oracle.layout(idx, s.R, s.T_o, s.G, s.E_l, s.k, s.M, s.mgb, 0, orc)
    tag = np.repeat(np.arange(lay["M_pad"], dtype=np.float64)[:, None], 3, axis=1)   # row p carries p
    recv = oracle.deliver(lay, tag, s.R, s.E_l, orc)
    got = np.concatenate([b[:, 0] for b in recv]).astype(int)
    real = np.nonzero(lay["row_src"] >= 0)[0]
    assert sorted(got.tolist()) == real.tolist()              # each real row once, padding never
    for t in range(s.T):
        for j in range(s.k):
            p = lay["combine_plan"][t, j]
            if p >= 0:
                assert lay["row_src"][int(recv[t // s.T_o][p, 0])] == t


def test_combine_pure_unpermute(orc):
    """k=1 with weight 1 (G=1: softmax of one logit is exactly 1): out is y's row by plan, bit for bit."""
    R, T_o, d = 3, 7, 5
    idx = np.zeros((R * T_o, 1), np.int32)
    w = oracle.route(np.zeros((R * T_o, 1), np.float32), 1, orc)[1]
    assert (w == 1.0).all()
    lay = oracle.layout(idx, R, T_o, 1, 1, 1, 4, 1, 0, orc)
    y = mi.normal_f32(1, 5, (lay["M_pad"], d)).astype(np.float64)
    recv = oracle.deliver(lay, y, R, 1, orc)
    out = oracle.combine(lay, w, recv, R, T_o, 1, False, orc)
    for t in range(R * T_o):
        assert (out[t] == y[lay["padded_off"][t // T_o] + t % T_o]).all()


def test_combine_weighted_sum_and_no_local(orc):
    R, T_o, d, k = 2, 3, 4, 2
    idx = np.array([[0, 1], [1, 5], [4, 5], [1, 0], [0, 7], [6, 1]], np.int32)
    w = np.array([[0.5, 0.25], [0.75, 0.1], [0.3, 0.3], [2.0, -1.0], [1.0, 9.0], [9.0, 0.125]], np.float32)
    lay = oracle.layout(idx, R, T_o, 8, 2, k, 2, 1, 0, orc)
    y = mi.normal_f32(2, 5, (lay["M_pad"], d)).astype(np.float64)
    recv = oracle.deliver(lay, y, R, 2, orc)
    out = oracle.combine(lay, w, recv, R, T_o, k, False, orc)

    def yrow(t, e):  # row of token t for local expert e, found by searching row_src inside the group
        g = e * R + t // T_o
        p0 = lay["padded_off"][g]
        seg = lay["row_src"][p0:p0 + lay["counts"][g]]
        return y[p0 + int(np.nonzero(seg == t)[0][0])]

    np.testing.assert_array_equal(out[2], 0.0)                     # token with no local expert
    np.testing.assert_allclose(out[0], 0.5 * yrow(0, 0) + 0.25 * yrow(0, 1), rtol=1e-15)
    np.testing.assert_allclose(out[1], 0.75 * yrow(1, 1), rtol=1e-15)
    np.testing.assert_allclose(out[3], 2.0 * yrow(3, 1) - 1.0 * yrow(3, 0), rtol=1e-15)
    np.testing.assert_allclose(out[5], 0.125 * yrow(5, 1), rtol=1e-15)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_whole_path_reduces_to_dense_mlp(orc, dtype):
    """R=1, G=E_l=1, k=1: layout, FFN, delivery and combine together are the dense SwiGLU MLP on X."""
    s = mi.spec("tiny", R=1, T_o=37, G=1, E_l=1, k=1, d=64, f=64, M=16, dtype=dtype)
    inp = mi.inputs(s)
    res = oracle.run(s, inp, orc)
    X = _to64(inp["x"], dtype)
    W1, W2 = _to64(inp["w_gate_up"][0], dtype), _to64(inp["w_down"][0], dtype)
    h = _silu(X @ W1[: s.f].T) * (X @ W1[s.f:].T)
    if dtype == "bf16":   # h and y are bf16 activations; torch's fp32->bf16 on fp32-rounded values
        h = torch.from_numpy(h).float().to(torch.bfloat16).double().numpy()
        ref = torch.from_numpy(h @ W2.T).float().to(torch.bfloat16).double().numpy()
        assert np.abs(res["out"] - ref).max() <= 2.0 ** -7 * np.abs(ref).max()
        assert np.mean(res["out"] == ref) > 0.99
    else:
        np.testing.assert_allclose(res["out"], h @ W2.T, rtol=1e-12, atol=1e-12)


# ----------------------------------------------------------------------------------------------------------------
# alternative roundings of h (bf16): what an fp32 evaluation may legitimately round the other way

def _ragged_rows():
    s = mi.Spec("ragged", R=4, T_o=120, G=16, E_l=4, k=2, d=256, f=512, M=32, seed=11)
    inp = mi.inputs(s)
    idx, _ = oracle.route(inp["logits"], s.k)
    lay = oracle.layout(idx, s.R, s.T_o, s.G, s.E_l, s.k, s.M)
    real = np.nonzero(lay["row_src"] >= 0)[0]
    return s, inp, lay["row_src"][real], lay["tile_expert"][real // s.M]


def test_ffn_ex_matches_plain_and_torch_fp64(orc):
    s, inp, src, ex_ = _ragged_rows()
    ex = oracle.ffn_rows_ex(src, ex_, inp["x"], inp["w_gate_up"], inp["w_down"], True, want_h=True, lib=orc)
    assert (ex["y"] == oracle.ffn_rows(src, ex_, inp["x"], inp["w_gate_up"], inp["w_down"], True, orc)).all()
    # h against a float64 torch evaluation of silu(g) * u rounded to bf16 (through fp32: equal except in the
    # rare double-rounding case)
    X = torch.from_numpy(_to64(inp["x"], "bf16")[src])
    W1 = torch.from_numpy(_to64(inp["w_gate_up"], "bf16"))[torch.from_numpy(ex_.astype(np.int64))]
    g = torch.einsum("rc,rnc->rn", X, W1[:, : s.f])
    u = torch.einsum("rc,rnc->rn", X, W1[:, s.f:])
    h_t = (torch.nn.functional.silu(g) * u).float().to(torch.bfloat16).double().numpy()
    assert np.mean(h_t == ex["h"]) > 0.9999
    # y before rounding = h @ Wd^T (float64 library matmul)
    W2 = torch.from_numpy(_to64(inp["w_down"], "bf16"))[torch.from_numpy(ex_.astype(np.int64))]
    y_t = torch.einsum("rn,rmn->rm", torch.from_numpy(ex["h"]), W2).numpy()
    np.testing.assert_allclose(ex["y_unr"], y_t, rtol=1e-12, atol=1e-12)


def test_ffn_ex_candidates_cover_fp32_flips(orc):
    """Every h that an fp32 evaluation (torch, bf16 inputs widened to fp32) rounds differently from the exact
    value is among the oracle's candidates, with the right other value; each candidate vector is exactly the
    change of y when that h takes its other rounding."""
    s, inp, src, ex_ = _ragged_rows()
    ex = oracle.ffn_rows_ex(src, ex_, inp["x"], inp["w_gate_up"], inp["w_down"], True, want_h=True, lib=orc)
    X = torch.from_numpy(mi.bf16_bits_to_f32(inp["x"])[src])
    W1 = torch.from_numpy(mi.bf16_bits_to_f32(inp["w_gate_up"]))[torch.from_numpy(ex_.astype(np.int64))]
    g = torch.einsum("rc,rnc->rn", X, W1[:, : s.f])
    u = torch.einsum("rc,rnc->rn", X, W1[:, s.f:])
    h32 = (torch.nn.functional.silu(g) * u).to(torch.bfloat16).double().numpy()
    rows, cols = np.nonzero(h32 != ex["h"])
    assert rows.size > 0                        # this workload does produce fp32 flips
    W2 = _to64(inp["w_down"], "bf16")
    big = 0
    for r, n in zip(rows, cols):
        if abs(h32[r, n] - ex["h"][r, n]) < 1e-5:
            # near zero the fp32 error spans several bf16 steps; the effect on y is below 1e-5 * |Wd|
            continue
        big += 1
        cand = list(ex["cand_n"][r, : ex["cand_count"][r]])
        assert n in cand, (r, n)
        q = cand.index(n)
        np.testing.assert_allclose(ex["cand_vec"][r, q], (h32[r, n] - ex["h"][r, n]) * W2[ex_[r], :, n], rtol=1e-15)
    assert big > 0
    assert ex["cand_count"].mean() < 64


def test_ffn_ex_flip_resolution_recovers_planted_roundings(orc):
    """A row built from the oracle's y plus some of its own candidates is matched back exactly; a perturbation
    that is not a listed candidate is not absorbed."""
    import tolerance

    s, inp, src, ex_ = _ragged_rows()
    ex = oracle.ffn_rows_ex(src, ex_, inp["x"], inp["w_gate_up"], inp["w_down"], True, lib=orc)
    got = ex["y_unr"].copy()
    planted = 0
    for i in range(got.shape[0]):
        cc = ex["cand_count"][i]
        for q in range(0, cc, 3):
            got[i] += ex["cand_vec"][i, q]
            planted += 1
    got = oracle.round_bf16_array(got, orc)
    ref, flips = tolerance.check_ffn(got, ex)
    assert planted > 0 and flips > 0
    bad = got.copy()
    bad[3, 7] += 0.05
    with pytest.raises(AssertionError):
        tolerance.check_ffn(bad, ex)


# ---- pins of the comparator parts: the bf16 neighbour, the fp32 bound of y, the candidate list at full width ------

def test_bf16_toward_matches_torch_nextafter(orc):
    """orc_bf16_toward_n (the bf16 value next to a bf16 value, toward a target) against torch.nextafter on bfloat16:
    both signs, zero, subnormals, binade edges, and a target equal to the value (itself)."""
    rng = np.random.default_rng(7)
    v = np.concatenate([rng.normal(0, 1, 4000), rng.normal(0, 1e-3, 1000), rng.normal(0, 1e4, 1000),
                        np.ldexp(1.0, np.arange(-130, 20)), -np.ldexp(1.0, np.arange(-130, 20)),
                        [0.0, -0.0, 1e-40, -1e-40, 3.0e38]])
    h = oracle.round_bf16_array(v, orc)
    # targets on both sides of h (the oracle steps toward v; v == h returns h)
    for tgt in (v, h + np.where(h >= 0, 1.0, -1.0) * np.abs(h) * 0.5 + 1e-45, h - np.abs(h) * 0.5 - 1e-45, h):
        got = oracle.bf16_toward(h, tgt, orc)
        th = torch.from_numpy(h).to(torch.bfloat16)
        assert (th.double().numpy() == h).all()  # h is exactly representable
        tt = torch.from_numpy(np.where(tgt > h, np.inf, np.where(tgt < h, -np.inf, h))).to(torch.bfloat16)
        want = torch.nextafter(th, tt).double().numpy()
        want = np.where(tgt == h, h, want)
        np.testing.assert_array_equal(got, want)


def _fp32_seq_matvec(h32: np.ndarray, w32: np.ndarray) -> np.ndarray:
    """y = w h in fp32 with a plain sequential sum over the reduction index (another summation order than torch's)."""
    terms = (w32 * h32[None, :]).astype(np.float32)       # each product rounded to fp32
    return np.add.accumulate(terms, axis=1, dtype=np.float32)[:, -1]


@pytest.mark.parametrize("shape", ["ragged", "wide"])
def test_y_delta_covers_fp32_evaluations(orc, shape):
    """The oracle's y_delta bounds how far an fp32 evaluation of y = h Wd^T can be from the exact value: two independent
    fp32 evaluations (torch's blocked matmul and a sequential fp32 sum) of every element stay within it, and the bound
    is far below half a bf16 step (it lets only near-midpoint roundings go either way)."""
    if shape == "ragged":
        s, inp, src, ex_ = _ragged_rows()
    else:  # full width: d = 4096, f = 14336, a few rows
        s = mi.spec("mixtral")
        inp = mi.inputs(s)
        src, ex_ = np.arange(0, 2048, 512).astype(np.int32), np.array([0, 1, 0, 1], np.int32)
    ex = oracle.ffn_rows_ex(src, ex_, inp["x"], inp["w_gate_up"], inp["w_down"], True, want_h=True, lib=orc)
    W2 = mi.bf16_bits_to_f32(inp["w_down"])
    h32 = ex["h"].astype(np.float32)  # bf16 values, exact in fp32
    for i in range(len(src)):
        w = W2[ex_[i]]
        y_t = (torch.from_numpy(w) @ torch.from_numpy(h32[i])).double().numpy()
        y_s = _fp32_seq_matvec(h32[i], w).astype(np.float64)
        for y32 in (y_t, y_s):
            assert (np.abs(y32 - ex["y_unr"][i]) <= ex["y_delta"][i]).all()
    half_step = np.ldexp(np.abs(ex["y_unr"]), -9)
    # about 1-5% of half a step at these widths; a dropped scale or f in place of sqrt(f) would exceed 10%
    assert np.median(ex["y_delta"] / np.maximum(half_step, 1e-30)) < 0.1


def _silu_coarse(g: np.ndarray, rng) -> np.ndarray:
    """silu(g) in fp32 as coarsely as the kernel may take it: exp as exp2(g * log2 e) (the product rounded to fp32),
    and the reciprocal of 1 + e^-g off by up to one fp32 ulp either way."""
    g = g.astype(np.float32)
    e = np.exp2((-g * np.float32(1.4426950408889634)).astype(np.float32)).astype(np.float32)
    den = (np.float32(1.0) + e).astype(np.float32)
    r = (np.float32(1.0) / den).astype(np.float32)
    nudge = rng.integers(-1, 2, size=r.shape)
    r = np.where(nudge > 0, np.nextafter(r, np.float32(np.inf)), np.where(nudge < 0, np.nextafter(r, np.float32(0)), r))
    return (g * r).astype(np.float32)


@pytest.mark.parametrize("name", ["mixtral", "deepseek"])
def test_ffn_ex_candidates_cover_coarse_fp32_at_full_width(orc, name):
    """At the full widths (d = 4096, f = 14336; d = 7168, f = 2048): every h that an fp32 evaluation with a coarse
    silu (exp2-based exp, reciprocal off by one ulp; the kernel's evaluation is no coarser) rounds to the other bf16
    neighbour is in the oracle's complete list of alternatives; the capped list the comparison uses (64 per row) holds
    the largest steps, so an alternative it leaves out moves h by no more than every one it keeps."""
    s = mi.spec(name)
    inp = mi.inputs(s)
    src = np.arange(0, s.T, s.T // 6).astype(np.int32)[:6]
    ex_ = (np.arange(len(src)) % s.E_l).astype(np.int32)
    full = oracle.ffn_rows_ex(src, ex_, inp["x"], inp["w_gate_up"], inp["w_down"], True, max_cand=s.f, want_h=True,
                              want_vec=False, lib=orc)
    capped = oracle.ffn_rows_ex(src, ex_, inp["x"], inp["w_gate_up"], inp["w_down"], True, want_vec=False, lib=orc)
    X = torch.from_numpy(mi.bf16_bits_to_f32(inp["x"])[src])
    W1 = mi.bf16_bits_to_f32(inp["w_gate_up"])
    rng = np.random.default_rng(3)
    flips = 0
    for i in range(len(src)):
        w = torch.from_numpy(W1[ex_[i]])
        g = (w[: s.f] @ X[i]).numpy()
        u = (w[s.f:] @ X[i]).numpy()
        cand = set(full["cand_n"][i, : full["cand_count"][i]].tolist())
        for trial in range(2):
            h32 = (_silu_coarse(g, rng) * u.astype(np.float32)).astype(np.float32)
            hb = torch.from_numpy(h32).to(torch.bfloat16).double().numpy()
            for n in np.nonzero(hb != full["h"][i])[0]:
                flips += 1
                assert n in cand, (i, n, h32[n], full["h"][i, n])
        # the capped list: the first min(64, count) of the complete one by step size
        step = lambda n: abs(oracle.bf16_toward(full["h"][i, n:n + 1], np.array([np.inf]), orc)[0] - full["h"][i, n])
        kept = capped["cand_n"][i, : capped["cand_count"][i]].tolist()
        assert capped["cand_count"][i] == min(64, full["cand_count"][i]) and set(kept) <= cand
        if full["cand_count"][i] > 64:
            left = cand - set(kept)
            assert max(step(n) for n in left) <= min(step(n) for n in kept)
    assert flips > 0



def test_combine_allowance_admits_one_step_of_each_row_and_no_more(orc):
    """The combined output's allowance (tolerance.combine_slack): an output combined from delivered rows whose elements
    took the other neighbour of their final rounding (one bf16 step; a quarter of them here) passes the check, also
    where the weighted sum cancels to a small value; an output off by three steps of its contributing rows, or by
    2e-3 at a small element, fails."""
    import tolerance

    s, inp, src, ex_ = _ragged_rows()
    idx, w = oracle.route(inp["logits"], s.k)
    lay = oracle.layout(idx, s.R, s.T_o, s.G, s.E_l, s.k, s.M)
    y_pad = oracle.ffn_layout(lay, inp["x"], inp["w_gate_up"], inp["w_down"], True, s.M, orc)
    recv = oracle.deliver(lay, y_pad, s.R, s.E_l, orc)
    out = oracle.combine(lay, w, recv, s.R, s.T_o, s.k, True, orc)
    base = np.concatenate([[0], np.cumsum([r.shape[0] for r in recv])])
    y_all = np.concatenate(recv)
    plan = lay["combine_plan"].reshape(s.T, s.k)
    slack = tolerance.combine_slack(plan, w, y_all, lambda i, j: base[i // s.T_o] + plan[i, j])
    rng = np.random.default_rng(5)
    # a quarter of the delivered elements one bf16 step up or down
    moved = [r + rng.choice([-1.0, 1.0], size=r.shape) * (rng.random(r.shape) < 0.25) * tolerance.bf16_ulp(r)
             for r in recv]
    out_moved = oracle.combine(lay, w, moved, s.R, s.T_o, s.k, True, orc)
    assert np.abs(out_moved - out).max() > 1e-3  # the stated bound alone would not hold everywhere
    tolerance.check(out_moved, out, "one step per row", slack=slack)
    moved3 = [r + 3.0 * tolerance.bf16_ulp(r) for r in recv]
    with pytest.raises(AssertionError):
        tolerance.check(oracle.combine(lay, w, moved3, s.R, s.T_o, s.k, True, orc), out, "three steps", slack=slack)
    small = np.argwhere((np.abs(out) < 0.02) & (slack < 5e-4))
    bad = out.copy()
    bad[tuple(small[0])] += 2e-3
    with pytest.raises(AssertionError):
        tolerance.check(bad, out, "planted", slack=slack)
    # the ulp helper: bf16 spacing at binade edges and below the normal range
    np.testing.assert_array_equal(tolerance.bf16_ulp(np.array([1.0, 1.5, 2.0, -0.75, 0.0, 1e-40])),
                                  [2.0 ** -7, 2.0 ** -7, 2.0 ** -6, 2.0 ** -8, 2.0 ** -133, 2.0 ** -133])


def test_backward_allowance_admits_the_intervals_and_no_more(orc):
    """The backward's allowance (tolerance.backward_slack): sums whose parts took other admitted values (dY, h, dG and
    dU each at the far end of its interval with probability 1/2, the rows' dX recomputed from the moved dG | dU and
    rounded as returned) pass the check, and some fail it without the allowance; an error planted past the stated
    tolerance plus the allowance fails."""
    import tolerance

    s = mi.Spec("bwd_slack", R=2, T_o=160, G=4, E_l=2, k=2, d=256, f=256, M=32, seed=39)
    inp = mi.inputs(s)
    d_out = mi.d_out(s)
    ref = oracle.backward(s, inp, d_out, orc, w_rel=2e-6)
    t, j = ref["rows"]
    p = ref["parts"]
    e = ref["topk_idx"][t, j]
    f = s.f
    rng = np.random.default_rng(9)

    def far(v, lo, hi):
        end = np.where(hi - v >= v - lo, hi, lo)
        return np.where(rng.random(v.shape) < 0.5, end, v)

    adm = p["adm"]
    moved = dict(p)
    moved["dy"] = far(p["dy"], p["dy_adm"][:, 0], p["dy_adm"][:, 1])
    moved["h"] = far(p["h"], adm[:, 0, 0], adm[:, 0, 1])
    moved["dgu"] = np.concatenate([far(p["dgu"][:, :f], adm[:, 1, 0], adm[:, 1, 1]),
                                   far(p["dgu"][:, f:], adm[:, 2, 0], adm[:, 2, 1])], axis=1)
    assert (moved["h"] != p["h"]).sum() > 100 and (moved["dgu"] != p["dgu"]).sum() > 100
    wgu = oracle._as_f64(inp["w_gate_up"])
    moved["dx"] = np.zeros_like(p["dx"])
    for ee in range(s.E_l):
        m = e == ee
        moved["dx"][m] = oracle.round_bf16_array(moved["dgu"][m] @ wgu[ee], orc)
    got = oracle.backward_reduce(s, inp, d_out, (t, j), e, moved, lib=orc)
    sl = tolerance.backward_slack(p, e, inp["w_gate_up"], oracle._as_f64(inp["x"][t]), list(range(s.E_l)))
    failed_without = 0
    for k in ("dx_rows", "dw_down", "dw_gate_up"):
        tolerance.check(got[k], ref[k], k, slack=sl[k])
        try:
            tolerance.check(got[k], ref[k], k)
        except AssertionError:
            failed_without += 1
    assert failed_without > 0
    i = np.unravel_index(np.argmax(sl["dw_down"]), sl["dw_down"].shape)
    bad = got["dw_down"].copy()
    bad[i] = ref["dw_down"][i] + 1.5 * (max(tolerance.RTOL * abs(ref["dw_down"][i]), tolerance.ATOL) + sl["dw_down"][i])
    with pytest.raises(AssertionError):
        tolerance.check(bad, ref["dw_down"], "planted", slack=sl["dw_down"])


# ---- backward of the layer (orc_bwd_rows and oracle.backward) -----------------------------------------------------
BWD_SPEC = mi.Spec("bwd_tiny", R=3, T_o=12, G=6, E_l=2, k=2, d=32, f=48, M=16, dtype="f32", seed=31)


def _forward_loss(orc, s, lay, x, w1, w2, topk_w, d_out, is_bf16=False):
    """L = <dOut, out> through the oracle's own forward (FFN over the layout, delivery, combine) at fixed routing."""
    y_pad = oracle.ffn_layout(lay, x, w1, w2, is_bf16, s.M, orc)
    recv = oracle.deliver(lay, y_pad, s.R, s.E_l, orc)
    out = oracle.combine(lay, topk_w, recv, s.R, s.T_o, s.k, is_bf16, orc)
    return float((d_out.astype(np.float64) * out).sum())


def test_backward_matches_finite_differences_of_the_forward(orc):
    """Each gradient of oracle.backward against central differences of the forward oracle (fp32 mode, no rounding):
    L(theta + v) - L(theta - v) equals <grad, 2 v> up to third-order terms, for random directions v in x, the gate /
    up weights, the down weights and the routing weights.  A dropped term, a wrong sign or a transposed operand in
    any gradient fails this."""
    s = BWD_SPEC
    inp = mi.inputs(s)
    d_out = mi.d_out(s)
    b = oracle.backward(s, inp, d_out, orc)
    idx, w = b["topk_idx"], b["topk_w"]
    lay = oracle.layout(idx, s.R, s.T_o, s.G, s.E_l, s.k, s.M, s.mgb, 0, orc)
    rng = np.random.default_rng(5)
    base = dict(x=inp["x"], w1=inp["w_gate_up"], w2=inp["w_down"], topk_w=w)
    grads = dict(x=b["dx"], w1=b["dw_gate_up"], w2=b["dw_down"], topk_w=b["dw"])
    for name, g in grads.items():
        a = base[name]
        v = rng.standard_normal(a.shape) * 1e-3 * (np.abs(a).mean() + 1e-3)
        if name == "topk_w":
            v *= (idx < s.E_l)  # only slots routed to a local expert enter the local combine
        plus, minus = (a + v).astype(np.float32), (a - v).astype(np.float32)
        args_p, args_m = dict(base), dict(base)
        args_p[name], args_m[name] = plus, minus
        dl = _forward_loss(orc, s, lay, d_out=d_out, **args_p) - _forward_loss(orc, s, lay, d_out=d_out, **args_m)
        pred = float((g * (plus.astype(np.float64) - minus.astype(np.float64))).sum())
        assert abs(dl - pred) <= 1e-6 * abs(pred) + 1e-12, (name, dl, pred)


def test_backward_matches_torch_autograd_fp64(orc):
    """The same gradients from torch autograd over an independent float64 forward of the layer (per token: the sum
    over its local slots of w * FFN_e(x)), fp32 mode."""
    s = BWD_SPEC
    inp = mi.inputs(s)
    d_out = mi.d_out(s)
    b = oracle.backward(s, inp, d_out, orc)
    idx, w = b["topk_idx"], b["topk_w"]
    x = torch.tensor(inp["x"], dtype=torch.float64, requires_grad=True)
    w1 = torch.tensor(inp["w_gate_up"], dtype=torch.float64, requires_grad=True)
    w2 = torch.tensor(inp["w_down"], dtype=torch.float64, requires_grad=True)
    tw = torch.tensor(w, dtype=torch.float64, requires_grad=True)
    out = torch.zeros(s.T, s.d, dtype=torch.float64)
    for t in range(s.T):
        for j in range(s.k):
            e = int(idx[t, j])
            if e >= s.E_l:
                continue
            g = w1[e, : s.f] @ x[t]
            u = w1[e, s.f:] @ x[t]
            out[t] = out[t] + tw[t, j] * (w2[e] @ (torch.nn.functional.silu(g) * u))
    (out * torch.tensor(d_out, dtype=torch.float64)).sum().backward()
    for got, ref in ((b["dx"], x.grad), (b["dw_gate_up"], w1.grad), (b["dw_down"], w2.grad), (b["dw"], tw.grad)):
        np.testing.assert_allclose(got, ref.numpy(), rtol=1e-9, atol=1e-12)


def _bf16(a):
    return torch.tensor(np.asarray(a, dtype=np.float64)).to(torch.float32).to(torch.bfloat16).to(torch.float64).numpy()


def test_backward_bf16_rounding_points(orc):
    """bf16 mode rounds where the GPU rounds, and only there, checked against independent evaluations (numpy products,
    torch's bf16 conversion): dY = bf16 of the fp32 product w * dOut, exactly; h equals the forward oracle's h bit for
    bit; dG, dU and the rows' dX are bf16 roundings of numpy's double evaluation from the rounded operands (one bf16
    step allowed where numpy's summation order lands on the other side of a tie); dx is the rounded sum of the rows."""
    s = mi.spec("tiny")
    inp = mi.inputs(s)
    d_out = mi.d_out(s)
    b = oracle.backward(s, inp, d_out, orc)
    t, j = b["rows"]
    r = b["parts"]
    w, idx = b["topk_w"], b["topk_idx"]
    dout32 = oracle._as_f64(d_out).astype(np.float32)
    np.testing.assert_array_equal(r["dy"], _bf16(w[t, j][:, None].astype(np.float32) * dout32[t]))
    fwd = oracle.ffn_rows_ex(t.astype(np.int32), idx[t, j].astype(np.int32), inp["x"], inp["w_gate_up"],
                             inp["w_down"], True, max_cand=0, want_h=True, want_vec=False, lib=orc)
    np.testing.assert_array_equal(r["h"], fwd["h"])
    np.testing.assert_array_equal(r["y"], fwd["y"])
    x = oracle._as_f64(inp["x"])[t]
    w1 = oracle._as_f64(inp["w_gate_up"])
    w2 = oracle._as_f64(inp["w_down"])
    e = idx[t, j]
    g = np.einsum("ind,id->in", w1[e, : s.f], x)
    u = np.einsum("ind,id->in", w1[e, s.f:], x)
    dh = np.einsum("imn,im->in", w2[e], r["dy"])
    sg = 1.0 / (1.0 + np.exp(-g))
    step = lambda v: np.abs(v) * 2.0 ** -7 + 1e-40
    for got, exact in ((r["dgu"][:, : s.f], dh * u * sg * (1 + g * (1 - sg))), (r["dgu"][:, s.f:], dh * g * sg)):
        assert (np.abs(got - _bf16(exact)) <= step(exact)).all()
        assert (got == _bf16(got)).all()
    dxr = np.einsum("ind,in->id", w1[e], r["dgu"])
    assert (np.abs(r["dx"] - _bf16(dxr)) <= step(dxr)).all() and (r["dx"] == _bf16(r["dx"])).all()
    summed = np.zeros((s.T, s.d))
    np.add.at(summed, t, r["dx"])
    np.testing.assert_array_equal(b["dx"], _bf16(summed))


def test_backward_admitted_roundings_cover_fp32_evaluations(orc):
    """The admitted intervals of dY (routing weights correct to relative w_rel) and of h, dG and dU (the least and
    greatest bf16 values an fp32 evaluation within the error bound can round to) hold: dY = bf16(fp32(w' dOut)) for
    weights w' at both ends of their bound, and the bf16 rounding of fp32 evaluations of h, dG and dU in several
    summation orders (left to right, right to left, numpy's pairwise sum, 16 lanes of 16 terms then a lane sum) from
    dY at the least, the oracle's and the greatest admitted values; the oracle's own roundings lie in them; most values
    admit one rounding only, so the intervals are no blanket allowance."""
    s = mi.Spec("bwd_adm", R=2, T_o=48, G=4, E_l=2, k=2, d=256, f=128, M=16, seed=37)
    inp = mi.inputs(s)
    d_out = mi.d_out(s)
    w_rel = 2e-6
    b = oracle.backward(s, inp, d_out, orc, w_rel=w_rel)
    t, j = b["rows"]
    r = b["parts"]
    e = b["topk_idx"][t, j]
    wt = b["topk_w"][t, j].astype(np.float64)
    dout = oracle._as_f64(d_out)[t]
    for sgn in (-1, 1):
        w_end = (wt * (1 + sgn * w_rel)).astype(np.float32)
        v = _bf16((w_end[:, None] * dout.astype(np.float32)).astype(np.float64))
        assert ((r["dy_adm"][:, 0] <= v) & (v <= r["dy_adm"][:, 1])).all()
    assert ((r["dy_adm"][:, 0] <= r["dy"]) & (r["dy"] <= r["dy_adm"][:, 1])).all()
    assert (r["dy_adm"][:, 0] == r["dy_adm"][:, 1]).mean() > 0.99
    x = oracle._as_f64(inp["x"]).astype(np.float32)[t]
    w1 = oracle._as_f64(inp["w_gate_up"]).astype(np.float32)[e]
    w2 = oracle._as_f64(inp["w_down"]).astype(np.float32)[e]
    tg = w1[:, : s.f] * x[:, None, :]            # [n, f, d], exact in fp32 (bf16 operands)
    tu = w1[:, s.f:] * x[:, None, :]
    ths = [np.swapaxes(w2 * dy.astype(np.float32)[:, :, None], 1, 2)  # [n, f, d]
           for dy in (r["dy_adm"][:, 0], r["dy"], r["dy_adm"][:, 1])]

    def seq(tm, rev=False):
        acc = np.zeros(tm.shape[:2], np.float32)
        for c in (range(tm.shape[2] - 1, -1, -1) if rev else range(tm.shape[2])):
            acc = acc + tm[:, :, c]
        return acc

    def lanes(tm):
        return seq(np.stack([seq(tm[:, :, i::16]) for i in range(16)], axis=2))

    orders = (seq, lambda tm: seq(tm, True), lambda tm: tm.sum(axis=2, dtype=np.float32), lanes)
    lo, hi = r["adm"][:, :, 0], r["adm"][:, :, 1]
    for q, own in enumerate((r["h"], r["dgu"][:, : s.f], r["dgu"][:, s.f:])):
        assert (lo[:, q] <= own).all() and (own <= hi[:, q]).all()
        assert (lo[:, q] == hi[:, q]).mean() > 0.9
    for order, th in [(o, ths[1]) for o in orders] + [(orders[0], ths[0]), (orders[3], ths[2])]:
        g, u, dh = order(tg), order(tu), order(th)
        sg = np.float32(1) / (np.float32(1) + np.exp(-g))
        silu = g * sg
        vals = (silu * u, dh * u * (sg * (np.float32(1) + g * (np.float32(1) - sg))), dh * silu)
        for q, v in enumerate(vals):
            v = _bf16(v.astype(np.float64))
            assert ((lo[:, q] <= v) & (v <= hi[:, q])).all(), q


def test_backward_at_another_rank(orc):
    """Rank 1's gradients (its local experts are the global [E_l, 2 E_l)) of a batch whose routing logits swap global
    experts [0, E_l) and [E_l, 2 E_l) equal rank 0's gradients of the original batch: only the offset of the local
    experts changes."""
    s = BWD_SPEC
    inp = mi.inputs(s)
    d_out = mi.d_out(s)
    sw = dict(inp)
    lg = inp["logits"].copy()
    E = s.E_l
    lg[:, [*range(E, 2 * E), *range(0, E)]] = inp["logits"][:, : 2 * E]
    sw["logits"] = lg
    a = oracle.backward(s, inp, d_out, orc)
    b = oracle.backward(s, sw, d_out, orc, self_rank=1)
    for k in ("dx", "dw", "dw_gate_up", "dw_down"):
        np.testing.assert_array_equal(a[k], b[k], err_msg=k)


def test_backward_no_local_slot_gives_zero(orc):
    """A token none of whose slots is routed to a local expert gets a zero dx row and zero routing gradients; an
    expert with no rows gets zero weight gradients."""
    s = BWD_SPEC
    inp = mi.inputs(s)
    lg = inp["logits"].copy()
    lg[0, :] = -10.0
    lg[0, 2:4] = 10.0  # token 0 to experts 2 and 3, both on another rank
    lg[:, 1] = -50.0   # local expert 1 chosen by nobody
    inp["logits"] = lg
    b = oracle.backward(s, inp, mi.d_out(s), orc)
    assert (b["topk_idx"][0] >= s.E_l).all()
    assert (b["dx"][0] == 0).all() and (b["dw"][0] == 0).all()
    assert (b["topk_idx"] != 1).all()
    assert (b["dw_gate_up"][1] == 0).all() and (b["dw_down"][1] == 0).all()
