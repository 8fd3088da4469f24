"""CPU oracle for the MoE expert-compute-plus-return path (ctypes wrapper over ``oracle.c``).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py``, never by the GPU library or its binding.  It shares no code with the GPU path; only the seeded
input generator (``moe_inputs``) serves both.

The method is the one on the review page of "Fine-grained Computation-Communication Overlap via Tile-level
Signaling and Scheduling for Mixture-of-Experts" (arXiv 2607.19539): routing output, remote-owner-aligned
layout (rows grouped by (expert, owner), padded to the tile height; referee major comment 1 on section 4.5 /
Algorithm 1), the expert SwiGLU FFN, owner delivery of real rows only ("What carries the argument"), and the
top-k weighted combine driven by the precomputed plan (ledger axiom 3, section 3.2.3).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

SEG_FIELDS = 8
SEG_OWNER, SEG_EXPERT, SEG_FIRST_BAND, SEG_NBANDS, SEG_SRC_ROW, SEG_DST_ROW, SEG_ROWS, SEG_GROUP = range(8)


def build(force: bool = True, extra_flags=()) -> str:
    """Compile oracle.c with gcc (-O2, OpenMP, no fast-math)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", *extra_flags, "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


class _LayoutArgs(ctypes.Structure):
    _fields_ = [
        ("topk_idx", ctypes.c_void_p),
        ("R", ctypes.c_int32), ("T_o", ctypes.c_int32), ("G", ctypes.c_int32), ("E_l", ctypes.c_int32),
        ("k", ctypes.c_int32), ("self_rank", ctypes.c_int32), ("M", ctypes.c_int32), ("mgb", ctypes.c_int32),
        ("cap_rows", ctypes.c_int64), ("cap_tiles", ctypes.c_int64),
        ("counts", ctypes.c_void_p), ("padded_off", ctypes.c_void_p), ("recv_off", ctypes.c_void_p),
        ("tile_owner", ctypes.c_void_p), ("tile_expert", ctypes.c_void_p), ("tile_valid", ctypes.c_void_p),
        ("tile_order", ctypes.c_void_p), ("seg_desc", ctypes.c_void_p), ("row_src", ctypes.c_void_p),
        ("combine_plan", ctypes.c_void_p), ("scalars", ctypes.c_void_p),
    ]


_lib = None


def load(path: str | None = None):
    """Load the oracle library (building it first when absent).  ``path`` loads another build of it."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        _lib = _bind(ctypes.CDLL(_LIB))
    return _lib


def _bind(lib):
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
    lib.orc_route.argtypes = [i64, i32, i32, vp, vp, vp]
    lib.orc_route.restype = i32
    lib.orc_layout.argtypes = [ctypes.POINTER(_LayoutArgs)]
    lib.orc_layout.restype = i32
    lib.orc_padding_rows.argtypes = [vp, i32, i32, i32, i32, i32]
    lib.orc_padding_rows.restype = i64
    lib.orc_ffn_rows.argtypes = [i64, vp, vp, i32, i32, i32, vp, vp, vp, vp]
    lib.orc_ffn_rows.restype = i32
    lib.orc_ffn_rows_ex.argtypes = [i64, vp, vp, i32, i32, i32, vp, vp, vp, vp, vp, i32, vp, vp, vp, vp, vp]
    lib.orc_bf16_toward_n.argtypes = [i64, vp, vp, vp]
    lib.orc_bf16_toward_n.restype = None
    lib.orc_ffn_rows_ex.restype = i32
    lib.orc_round_bf16_n.argtypes = [i64, vp, vp]
    lib.orc_round_bf16_n.restype = None
    lib.orc_deliver.argtypes = [i32, i32, i32, vp, vp, vp, vp, vp]
    lib.orc_deliver.restype = i32
    lib.orc_combine.argtypes = [i32, i32, i32, i32, i32, vp, vp, vp, vp]
    lib.orc_combine.restype = i32
    lib.orc_bwd_rows.argtypes = [i64, vp, vp, vp, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                 ctypes.c_double, vp]
    lib.orc_bwd_rows.restype = i32
    lib.orc_round_bf16.argtypes = [ctypes.c_double]
    lib.orc_round_bf16.restype = ctypes.c_double
    lib.orc_bf16_bits.argtypes = [ctypes.c_double]
    lib.orc_bf16_bits.restype = ctypes.c_uint16
    return lib


def _p(a: np.ndarray):
    assert a.flags.c_contiguous
    return a.ctypes.data


def route(logits: np.ndarray, k: int, lib=None):
    """Top-k by logit (ties to the lower id) and softmax weights over all G at those ids."""
    lib = lib or load()
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    T, G = logits.shape
    idx = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float32)
    rc = lib.orc_route(T, G, k, _p(logits), _p(idx), _p(w))
    if rc != 0:
        raise ValueError("orc_route: bad shape")
    return idx, w


def capacity_rows(R, T_o, E_l, k, M) -> int:
    """Upper bound of the padded row count: each token has at most min(k, E_l) local slots and each of
    the E_l*R groups adds at most M-1 padding rows; rounded up to a multiple of M."""
    bound = R * T_o * min(k, E_l) + E_l * R * (M - 1)
    return ((bound + M - 1) // M) * M


def layout(topk_idx: np.ndarray, R: int, T_o: int, G: int, E_l: int, k: int, M: int, mgb: int = 1,
           self_rank: int = 0, lib=None) -> dict:
    """The remote-owner-aligned layout and its metadata; arrays are trimmed to their used sizes."""
    lib = lib or load()
    topk_idx = np.ascontiguousarray(topk_idx, dtype=np.int32).reshape(R * T_o, k)
    cap = capacity_rows(R, T_o, E_l, k, M)
    cap_t = cap // M
    NG = E_l * R
    out = {
        "counts": np.zeros(NG, np.int32), "padded_off": np.zeros(NG, np.int32), "recv_off": np.zeros(NG, np.int32),
        "tile_owner": np.zeros(cap_t, np.int32), "tile_expert": np.zeros(cap_t, np.int32),
        "tile_valid": np.zeros(cap_t, np.int32), "tile_order": np.zeros(cap_t, np.int32),
        "seg_desc": np.zeros((cap_t, SEG_FIELDS), np.int32), "row_src": np.zeros(cap, np.int32),
        "combine_plan": np.zeros((R * T_o, k), np.int32), "scalars": np.zeros(3 + R, np.int32),
    }
    a = _LayoutArgs(topk_idx=_p(topk_idx), R=R, T_o=T_o, G=G, E_l=E_l, k=k, self_rank=self_rank, M=M, mgb=mgb,
                    cap_rows=cap, cap_tiles=cap_t,
                    **{n: _p(out[n]) for n in ("counts", "padded_off", "recv_off", "tile_owner", "tile_expert",
                                               "tile_valid", "tile_order", "seg_desc", "row_src",
                                               "combine_plan", "scalars")})
    rc = lib.orc_layout(ctypes.byref(a))
    if rc != 0:
        raise ValueError("orc_layout failed: %d" % rc)
    M_pad, n_tiles, n_segs = (int(v) for v in out["scalars"][:3])
    for n in ("tile_owner", "tile_expert", "tile_valid", "tile_order"):
        out[n] = out[n][:n_tiles]
    out["seg_desc"] = out["seg_desc"][:n_segs]
    out["row_src"] = out["row_src"][:M_pad]
    out["M_pad"], out["n_tiles"], out["n_segs"] = M_pad, n_tiles, n_segs
    out["N_r"] = out["scalars"][3:].copy()
    return out


def padding_rows(counts: np.ndarray, E: int, R: int, M: int, self_rank: int = 0, count_self: bool = True,
                 lib=None) -> int:
    lib = lib or load()
    counts = np.ascontiguousarray(counts, dtype=np.int32).reshape(E * R)
    return int(lib.orc_padding_rows(_p(counts), E, R, M, self_rank, int(count_self)))


def ffn_rows(src_row, expert, x, w_gate_up, w_down, is_bf16: bool, lib=None) -> np.ndarray:
    """FFN output rows (float64 [n, d]) for token rows ``src_row`` through local experts ``expert``."""
    lib = lib or load()
    src_row = np.ascontiguousarray(src_row, dtype=np.int32)
    expert = np.ascontiguousarray(expert, dtype=np.int32)
    x = np.ascontiguousarray(x)
    w_gate_up = np.ascontiguousarray(w_gate_up)
    w_down = np.ascontiguousarray(w_down)
    d = x.shape[1]
    f = w_down.shape[2]
    assert w_gate_up.shape[1:] == (2 * f, d) and w_down.shape[1:] == (d, f)
    y = np.empty((src_row.size, d), dtype=np.float64)
    rc = lib.orc_ffn_rows(src_row.size, _p(src_row), _p(expert), d, f, int(is_bf16), _p(x), _p(w_gate_up),
                          _p(w_down), _p(y))
    if rc != 0:
        raise ValueError("orc_ffn_rows failed")
    return y


def ffn_rows_ex(src_row, expert, x, w_gate_up, w_down, is_bf16: bool, max_cand: int = 64, want_h: bool = False,
                want_vec: bool = True, lib=None) -> dict:
    """FFN rows plus, in bf16 mode, the roundings of h that an fp32 evaluation does not decide.

    Returns y (float64 [n, d], rounded as the path rounds), y_unr (y before its final rounding), y_delta (bound
    of an fp32 evaluation's error in y_unr), optionally h (the rounded hidden rows [n, f]), and per row
    up to ``max_cand`` alternative roundings, largest step first: cand_count [n], cand_n [n, max_cand] (hidden index),
    cand_vec [n, max_cand, d] (exact change of y_unr when h takes the other bf16 candidate; omitted with
    want_vec=False).
    """
    lib = lib or load()
    src_row = np.ascontiguousarray(src_row, dtype=np.int32)
    expert = np.ascontiguousarray(expert, dtype=np.int32)
    x = np.ascontiguousarray(x)
    w_gate_up = np.ascontiguousarray(w_gate_up)
    w_down = np.ascontiguousarray(w_down)
    d = x.shape[1]
    f = w_down.shape[2]
    n = src_row.size
    out = {"y": np.empty((n, d)), "y_unr": np.empty((n, d)), "cand_count": np.zeros(n, np.int32),
           "cand_n": np.zeros((n, max_cand), np.int32), "y_delta": np.empty((n, d))}
    if want_vec:
        out["cand_vec"] = np.zeros((n, max_cand, d))
    if want_h:
        out["h"] = np.empty((n, f))
    rc = lib.orc_ffn_rows_ex(n, _p(src_row), _p(expert), d, f, int(is_bf16), _p(x), _p(w_gate_up), _p(w_down),
                             _p(out["y"]), _p(out["y_unr"]), max_cand, _p(out["cand_count"]), _p(out["cand_n"]),
                             _p(out["cand_vec"]) if want_vec else None, _p(out["h"]) if want_h else None,
                             _p(out["y_delta"]))
    if rc != 0:
        raise ValueError("orc_ffn_rows_ex failed")
    return out


def round_bf16_array(a: np.ndarray, lib=None) -> np.ndarray:
    lib = lib or load()
    a = np.ascontiguousarray(a, dtype=np.float64)
    out = np.empty_like(a)
    lib.orc_round_bf16_n(a.size, _p(a), _p(out))
    return out


def bf16_toward(h: np.ndarray, v: np.ndarray, lib=None) -> np.ndarray:
    """The bf16 neighbour of each bf16 value h in the direction of v (h where v == h)."""
    lib = lib or load()
    h = np.ascontiguousarray(h, dtype=np.float64)
    v = np.ascontiguousarray(v, dtype=np.float64)
    out = np.empty_like(h)
    lib.orc_bf16_toward_n(h.size, _p(h), _p(v), _p(out))
    return out


def ffn_layout(lay: dict, x, w_gate_up, w_down, is_bf16: bool, M: int, lib=None) -> np.ndarray:
    """FFN over the real rows of the padded layout; padding rows are NaN (they have no defined value)."""
    real = np.nonzero(lay["row_src"] >= 0)[0]
    y_pad = np.full((lay["M_pad"], x.shape[1]), np.nan)
    if real.size:
        y_pad[real] = ffn_rows(lay["row_src"][real], lay["tile_expert"][real // M], x, w_gate_up, w_down, is_bf16,
                               lib)
    return y_pad


def deliver(lay: dict, y_pad: np.ndarray, R: int, E_l: int, lib=None):
    lib = lib or load()
    d = y_pad.shape[1]
    y_pad = np.ascontiguousarray(y_pad, dtype=np.float64)
    recv = [np.full((int(lay["N_r"][r]), d), np.nan) for r in range(R)]
    ptrs = (ctypes.c_void_p * R)(*[_p(b) for b in recv])
    lib.orc_deliver(R, E_l, d, _p(lay["counts"]), _p(lay["padded_off"]), _p(lay["recv_off"]), _p(y_pad), ptrs)
    return recv


def combine(lay: dict, topk_w, recv, R: int, T_o: int, k: int, is_bf16: bool, lib=None) -> np.ndarray:
    lib = lib or load()
    d = recv[0].shape[1] if len(recv) and recv[0].ndim == 2 else 0
    topk_w = np.ascontiguousarray(topk_w, dtype=np.float32)
    recv = [np.ascontiguousarray(b, dtype=np.float64) for b in recv]
    out = np.empty((R * T_o, d), dtype=np.float64)
    ptrs = (ctypes.c_void_p * R)(*[_p(b) for b in recv])
    lib.orc_combine(R, T_o, k, d, int(is_bf16), _p(lay["combine_plan"]), _p(topk_w), ptrs, _p(out))
    return out


def round_bf16(v: float, lib=None) -> float:
    return (lib or load()).orc_round_bf16(float(v))


def bwd_rows(tok, expert, w, x, w_gate_up, w_down, d_out, is_bf16: bool, want_y: bool = True,
             want_parts: bool = True, want_adm: bool = False, w_rel: float = 0.0, lib=None) -> dict:
    """Backward of the expert FFN for rows (token tok[i], local expert expert[i], routing weight w[i]): the row
    gradient dX [n, d], and (want_parts) dY [n, d], h [n, f], dG | dU [n, 2f]; (want_y) the forward output y [n, d];
    (want_adm, bf16) the least and greatest admitted values of h, dG and dU, [n, 3, 2, f], and of dY, [n, 2, d], for
    routing weights correct to relative w_rel (orc_bwd_rows)."""
    lib = lib or load()
    tok = np.ascontiguousarray(tok, dtype=np.int32)
    expert = np.ascontiguousarray(expert, dtype=np.int32)
    w = np.ascontiguousarray(w, dtype=np.float32)
    n = tok.size
    _, d = x.shape
    f = w_down.shape[2]
    out = {"dx": np.empty((n, d))}
    if want_parts:
        out.update(dy=np.empty((n, d)), h=np.empty((n, f)), dgu=np.empty((n, 2 * f)))
    if want_y:
        out["y"] = np.empty((n, d))
    if want_adm:
        out["adm"] = np.zeros((n, 3, 2, f))
        out["dy_adm"] = np.zeros((n, 2, d))
    g = lambda k: _p(out[k]) if k in out else None
    rc = lib.orc_bwd_rows(n, _p(tok), _p(expert), _p(w), d, f, int(is_bf16), _p(np.ascontiguousarray(x)),
                          _p(np.ascontiguousarray(w_gate_up)), _p(np.ascontiguousarray(w_down)),
                          _p(np.ascontiguousarray(d_out)), _p(out["dx"]), g("dy"), g("h"), g("dgu"), g("y"),
                          g("adm"), float(w_rel), g("dy_adm"))
    assert rc == 0
    return out


def backward(s, inputs: dict, d_out: np.ndarray, lib=None, *, w_rel: float = 0.0, self_rank: int = 0) -> dict:
    """Gradients of the MoE layer for the local experts, given dOut = dL/d(combined output) [T, d] (the review page,
    "Where Pith is reading between the lines": MoE training's backward pass): dx [T, d] = sum over the token's
    local slots of the rows' dX (rounded once in bf16 mode, as the combined output is), the routing weights'
    gradient dw [T, k] = <dOut_t, y> (0 for slots routed elsewhere), and the weight gradients
    dw_gate_up [E, 2f, d] = sum over the expert's rows of (dG | dU) x^T and dw_down [E, d, f] = sum of dY h^T
    (numpy matmuls of the rows' parts, in double; backward_reduce).  w_rel: the relative bound to which routing
    weights are taken as correct, for the admitted values of the parts (bwd_rows).  self_rank: the rank whose local
    experts [self_rank E_l, (self_rank + 1) E_l) the gradients are of."""
    lib = lib or load()
    idx, w = route(inputs["logits"], s.k, lib)
    lo = self_rank * s.E_l
    t, j = np.nonzero((idx >= lo) & (idx < lo + s.E_l))
    e = idx[t, j] - lo
    is_bf16 = s.dtype == "bf16"
    r = bwd_rows(t, e, w[t, j], inputs["x"], inputs["w_gate_up"], inputs["w_down"], d_out, is_bf16,
                 want_adm=is_bf16, w_rel=w_rel, lib=lib)
    out = backward_reduce(s, inputs, d_out, (t, j), e, r, lib=lib)
    out.update({"rows": (t, j), "parts": r, "topk_idx": idx, "topk_w": w})
    return out


def backward_reduce(s, inputs: dict, d_out: np.ndarray, rows, e, parts: dict, experts=None, lib=None) -> dict:
    """The sums over rows of the backward: dx, dw, dw_gate_up and dw_down (see backward) from the rows' parts (dy, h,
    dgu, y, dx).  experts: the local experts whose weight gradients are formed (all by default); the weight gradients
    are then indexed like that list."""
    lib = lib or load()
    t, j = rows
    is_bf16 = s.dtype == "bf16"
    dx_rows = parts["dx"]
    dx = np.zeros((s.T, s.d))
    np.add.at(dx, t, dx_rows)
    if is_bf16:
        dx = round_bf16_array(dx, lib)
    dout = _as_f64(d_out)
    dw = np.zeros((s.T, s.k))
    dw[t, j] = np.einsum("ic,ic->i", dout[t], parts["y"])
    experts = list(range(s.E_l)) if experts is None else list(experts)
    xs = _as_f64(inputs["x"][t])
    dwgu = np.zeros((len(experts), 2 * s.f, s.d))
    dwd = np.zeros((len(experts), s.d, s.f))
    for i, ee in enumerate(experts):
        m = e == ee
        dwgu[i] = parts["dgu"][m].T @ xs[m]
        dwd[i] = parts["dy"][m].T @ parts["h"][m]
    return {"dx": dx, "dx_rows": dx_rows, "dw": dw, "dw_gate_up": dwgu, "dw_down": dwd}


def _as_f64(a: np.ndarray) -> np.ndarray:
    """bf16 bits (uint16) or float32 to float64."""
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def run(s, inputs: dict, lib=None) -> dict:
    """The whole path on the CPU for a workload ``s`` (a ``moe_inputs.Spec``) and its generated inputs."""
    lib = lib or load()
    idx, w = route(inputs["logits"], s.k, lib)
    lay = layout(idx, s.R, s.T_o, s.G, s.E_l, s.k, s.M, s.mgb, 0, lib)
    is_bf16 = s.dtype == "bf16"
    y_pad = ffn_layout(lay, inputs["x"], inputs["w_gate_up"], inputs["w_down"], is_bf16, s.M, lib)
    recv = deliver(lay, y_pad, s.R, s.E_l, lib)
    out = combine(lay, w, recv, s.R, s.T_o, s.k, is_bf16, lib)
    return {"topk_idx": idx, "topk_w": w, "layout": lay, "y_pad": y_pad, "recv": recv, "out": out}
