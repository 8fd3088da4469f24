"""Floating-point parity bar: per element |got - ref| <= max(2e-2 * |ref|, 1e-3) and, over all compared elements,
||got - ref||_F / ||ref||_F <= 5e-3.  Integer and index results are compared bit for bit elsewhere."""
import numpy as np

RTOL = 2e-2
ATOL = 1e-3
NORM_RTOL = 5e-3
# routing weights: an fp32 softmax's weights against the oracle's, relative (their error bound over the workloads'
# expert counts, well above the few fp32 steps they differ by)
ROUTE_W_RTOL = 2e-6


def check(got, ref, what="", slack=None):
    """Per element |got - ref| <= max(RTOL |ref|, ATOL) (+ slack, an allowance derived from the inputs' own admitted
    roundings; see combine_slack), and the normwise bound."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.isfinite(got).all(), "%s: non-finite values" % what
    err = np.abs(got - ref)
    lim = np.maximum(RTOL * np.abs(ref), ATOL)
    if slack is not None:
        lim = lim + slack
    bad = err > lim
    if bad.any():
        i = np.unravel_index(np.argmax(err - lim), err.shape)
        raise AssertionError("%s: %d of %d elements out of tolerance; worst at %s got %r ref %r"
                             % (what, bad.sum(), bad.size, i, got[i], ref[i]))
    den = np.linalg.norm(ref)
    if den > 0:
        rel = np.linalg.norm(got - ref) / den
        assert rel <= NORM_RTOL, "%s: normwise relative error %.3e" % (what, rel)


def resolve_flips(got, ex, is_bf16=True):
    """Match GPU FFN rows against the oracle's rows, allowing only the oracle's own alternative roundings.

    ``ex`` is ``oracle.ffn_rows_ex`` output.  Where an exact h lies within the kernel's fp32 error bound of a bf16
    rounding midpoint, both roundings are correct results, and the oracle lists the exact change each would make
    to y.  In every row, candidates are taken one at a time while one raises the number of elements whose rounded
    value equals the GPU's bit for bit (a real flip moves the whole row onto the GPU's values; any other candidate
    does not).  Then y's own final rounding may take the other neighbour where the fp32 bound reaches the midpoint.
    Returns (the reference rows as the oracle defines them for the chosen roundings, rounded like the path rounds
    y; number of alternative roundings taken).
    """
    import oracle

    got = np.asarray(got, dtype=np.float64)
    ref = np.array(ex["y_unr"], dtype=np.float64)
    flips = 0
    if is_bf16:
        for i in range(got.shape[0]):
            cc = int(ex["cand_count"][i])
            if cc == 0:
                continue
            V = ex["cand_vec"][i, :cc]
            used = np.zeros(cc, bool)
            match = int((oracle.round_bf16_array(ref[i]) == got[i]).sum())
            while not used.all():
                trial = oracle.round_bf16_array(ref[i][None, :] + V)
                m = (trial == got[i][None, :]).sum(axis=1)
                m[used] = -1
                j = int(np.argmax(m))
                if m[j] <= match:
                    break
                used[j] = True
                ref[i] = ref[i] + V[j]
                match = int(m[j])
                flips += 1
        unr = ref
        ref = oracle.round_bf16_array(unr)
        nb = oracle.bf16_toward(ref, unr)
        alt = (got == nb) & (got != ref) & (np.abs(unr - 0.5 * (ref + nb)) <= ex["y_delta"])
        ref = np.where(alt, nb, ref)
        flips += int(alt.sum())
    return ref, flips


def _row_ok(g, r):
    return bool((np.abs(g - r) <= np.maximum(RTOL * np.abs(r), ATOL)).all())


def check_ffn(got, ex, what="y", is_bf16=True):
    """Tolerance check of FFN rows against the oracle up to the oracle's listed alternative roundings of h.
    Returns the reference rows used (for downstream delivery / combine references) and the flip count."""
    ref, flips = resolve_flips(got, ex, is_bf16)
    check(got, ref, what + " (%d alternative h roundings)" % flips)
    return ref, flips


def bf16_ulp(v):
    """The spacing of bf16 values at |v| (the step of v's binade; 2^-133 below the normal range)."""
    v = np.abs(np.asarray(v, dtype=np.float64))
    e = np.floor(np.log2(np.where(v > 0, v, 1.0)))
    return np.where(v > 0, np.ldexp(1.0, np.maximum(e - 7, -133).astype(int)), np.ldexp(1.0, -133))


def combine_slack(plan, w, y_rows, row_of):
    """The combined output's allowance beyond the stated tolerance: each delivered y element is a correct result up to
    one step of its own final bf16 rounding (near a rounding midpoint either neighbour is, as for h; and the
    alternatives the comparison of y does not list can carry y across such a midpoint), so the weighted sum may differ
    by sum_j |w_j| ulp(y_j).  plan [n, k] (>= 0 for local slots), w [n, k], y_rows [m, d] the reference rows,
    row_of(i, j) the index into y_rows of token i's slot j."""
    n, k = plan.shape
    out = np.zeros((n, y_rows.shape[1]))
    for i in range(n):
        for j in range(k):
            if plan[i, j] >= 0:
                out[i] += abs(float(w[i, j])) * bf16_ulp(y_rows[row_of(i, j)])
    return out


def _f64(a):
    """bf16 bits (uint16) or float32 to float64."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def _width(v, adm_lo, adm_hi):
    """The widest step from v to another admitted value."""
    return np.maximum(adm_hi - v, v - adm_lo)


def backward_slack(parts, e, w_gate_up, x_rows, experts):
    """Allowances of the backward's sums beyond the stated tolerance, from the admitted values of the rows' parts
    (oracle.bwd_rows with want_adm): a part the GPU may take anywhere in its interval moves each sum it feeds by at
    most the interval's width times the other factor's magnitude; the dX rows add one step of their own final bf16
    rounding (either neighbour near a midpoint, as for y).
    parts: for rows with local expert e [n]; w_gate_up [E, 2f, d] (bf16 bits as uint16, or float32; converted one
    expert at a time); x_rows [n, d] (float64); experts: the experts whose weight gradients are checked.  Returns
    {"dx_rows" [n, d], "dw_down" [len, d, f], "dw_gate_up" [len, 2f, d]}."""
    adm, dadm = parts["adm"], parts["dy_adm"]
    f = parts["h"].shape[1]
    wh = _width(parts["h"], adm[:, 0, 0], adm[:, 0, 1])
    wgu = np.concatenate([_width(parts["dgu"][:, :f], adm[:, 1, 0], adm[:, 1, 1]),
                          _width(parts["dgu"][:, f:], adm[:, 2, 0], adm[:, 2, 1])], axis=1)
    wdy = _width(parts["dy"], dadm[:, 0], dadm[:, 1])
    dx = bf16_ulp(parts["dx"])
    for ee in np.unique(e):
        m = e == ee
        dx[m] += wgu[m] @ np.abs(_f64(w_gate_up[ee]))
    dwd = np.stack([np.abs(parts["dy"][e == ee]).T @ wh[e == ee] + wdy[e == ee].T @ (np.abs(parts["h"][e == ee])
                                                                                     + wh[e == ee])
                    for ee in experts]) if len(experts) else np.zeros((0, wdy.shape[1], f))
    dwgu = np.stack([wgu[e == ee].T @ np.abs(x_rows[e == ee]) for ee in experts]) if len(experts) else \
        np.zeros((0, 2 * f, wdy.shape[1]))
    return {"dx_rows": dx, "dw_down": dwd, "dw_gate_up": dwgu}
