"""Floating-point parity bar: per element |got - ref| <= max(2e-2 * |ref|, 1e-3) and, over all compared elements,
||got - ref||_F / ||ref||_F <= 5e-3.  Integer and index results are compared bit for bit elsewhere."""
import numpy as np

RTOL = 2e-2
ATOL = 1e-3
NORM_RTOL = 5e-3


def check(got, ref, what=""):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.isfinite(got).all(), "%s: non-finite values" % what
    err = np.abs(got - ref)
    lim = np.maximum(RTOL * np.abs(ref), ATOL)
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
