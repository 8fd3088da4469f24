"""Seeded synthetic inputs for the MoE expert-compute-plus-return path.

Shared by the CPU oracle (``oracle/``) and the GPU path; it holds random-number generation and
workload shapes only, none of the method's arithmetic.  Values come from ``gen.c`` (counter-based
splitmix64 streams, Box-Muller normals, fp32 then bf16 round-to-nearest-even).

Workloads (the synthetic stand-ins for the MoE shards the first page measures on; no model weights or
datasets are used): each is R owner ranks x T_o tokens, G global experts of which E_l are local to rank 0,
top-k routing, hidden d, FFN width f, layout tile height M.

Draws: logits ~ N(0, 1) [G per token]; optional per-expert logit bias; X ~ N(0, 1) [T, d];
per local expert, gate and up weights ~ N(0, 1/d) [f, d] each, down weights ~ N(0, 1/d) [d, f].
"""
from __future__ import annotations

import ctypes
import dataclasses
import math
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gen.c")
_LIB = os.path.join(_HERE, "libmoe_inputs.so")

# stream ids of the counter-based generator
STREAM_LOGITS = 1
STREAM_BIAS = 2
STREAM_X = 3
STREAM_DOUT = 4  # the output gradient of the backward pass
STREAM_W0 = 16  # expert e uses 16+3e (gate), 16+3e+1 (up), 16+3e+2 (down)


def build(force: bool = True) -> str:
    """Compile gen.c into libmoe_inputs.so (gcc, OpenMP)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(_LIB)
        u64, i64, dbl, vp = ctypes.c_uint64, ctypes.c_int64, ctypes.c_double, ctypes.c_void_p
        lib.gen_normal_f32.argtypes = [u64, u64, i64, dbl, dbl, vp]
        lib.gen_normal_bf16.argtypes = [u64, u64, i64, dbl, dbl, vp]
        lib.gen_raw_u64.argtypes = [u64, u64, i64, vp]
        lib.gen_splitmix64_seq.argtypes = [u64, i64, vp]
        for fn in (lib.gen_normal_f32, lib.gen_normal_bf16, lib.gen_raw_u64, lib.gen_splitmix64_seq):
            fn.restype = None
        _lib = lib
    return _lib


def normal_f32(seed: int, stream: int, shape, mu: float = 0.0, sigma: float = 1.0) -> np.ndarray:
    out = np.empty(shape, dtype=np.float32)
    _load().gen_normal_f32(seed, stream, out.size, mu, sigma, out.ctypes.data)
    return out


def normal_bf16(seed: int, stream: int, shape, mu: float = 0.0, sigma: float = 1.0) -> np.ndarray:
    """bf16 values as their raw uint16 bit patterns."""
    out = np.empty(shape, dtype=np.uint16)
    _load().gen_normal_bf16(seed, stream, out.size, mu, sigma, out.ctypes.data)
    return out


def raw_u64(seed: int, stream: int, n: int) -> np.ndarray:
    out = np.empty(n, dtype=np.uint64)
    _load().gen_raw_u64(seed, stream, n, out.ctypes.data)
    return out


def splitmix64_seq(state: int, n: int) -> np.ndarray:
    out = np.empty(n, dtype=np.uint64)
    _load().gen_splitmix64_seq(state, n, out.ctypes.data)
    return out


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of raw bf16 bits to fp32 (a bit shift, no rounding)."""
    return (bits.astype(np.uint32) << 16).view(np.float32)


@dataclasses.dataclass(frozen=True)
class Spec:
    name: str
    R: int            # owner ranks
    T_o: int          # tokens per owner
    G: int            # global experts
    E_l: int          # local experts (rank 0 hosts experts [0, E_l))
    k: int            # top-k
    d: int            # hidden
    f: int            # FFN width
    M: int            # layout tile height
    dtype: str = "bf16"   # "bf16" or "f32"
    seed: int = 0
    bias: str = "none"    # "none" | "zipf" | "normal"
    bias_param: float = 0.0
    mgb: int = 1          # row bands per transfer segment

    @property
    def T(self) -> int:
        return self.R * self.T_o


def _preset(name: str) -> Spec:
    if name == "tiny":
        return Spec("tiny", R=4, T_o=16, G=8, E_l=2, k=2, d=64, f=128, M=16, dtype="bf16", seed=1)
    if name == "tiny_f32":
        return Spec("tiny_f32", R=4, T_o=16, G=8, E_l=2, k=2, d=64, f=128, M=16, dtype="f32", seed=1)
    if name == "mixtral":
        return Spec("mixtral", R=4, T_o=1024, G=8, E_l=2, k=2, d=4096, f=14336, M=128, seed=2)
    if name == "skew":
        return Spec("skew", R=4, T_o=2048, G=64, E_l=16, k=6, d=2048, f=1408, M=64, seed=3,
                    bias="zipf", bias_param=1.2)
    if name.startswith("sweep"):
        e = int(name[5:])
        assert e in (1, 2, 4, 8, 16), name
        return Spec(name, R=4, T_o=4096, G=4 * e, E_l=e, k=2, d=4096, f=4096, M=128, seed=40 + e)
    if name == "deepseek":
        return Spec("deepseek", R=8, T_o=2048, G=256, E_l=32, k=8, d=7168, f=2048, M=128, seed=5,
                    bias="normal", bias_param=0.5)
    raise KeyError(name)


CONFIG_NAMES = ["tiny", "tiny_f32", "mixtral", "skew", "sweep1", "sweep2", "sweep4", "sweep8", "sweep16",
                "deepseek"]


def spec(name: str, **overrides) -> Spec:
    s = _preset(name)
    return dataclasses.replace(s, **overrides) if overrides else s


def expert_bias(s: Spec) -> np.ndarray:
    """Per-expert logit bias, float64 [G].

    zipf:   popularity rank q(e) = (e mod E_l) * R + e // E_l spreads popularity round-robin over the
            expert-parallel ranks; bias = -s * ln(q + 1), i.e. softmax mass proportional to (q+1)^-s.
    normal: bias ~ N(0, v) with v = bias_param read as a variance.
    """
    if s.bias == "none":
        return np.zeros(s.G, dtype=np.float64)
    if s.bias == "zipf":
        e = np.arange(s.G)
        q = (e % s.E_l) * s.R + e // s.E_l
        return -s.bias_param * np.log(q.astype(np.float64) + 1.0)
    if s.bias == "normal":
        return normal_f32(s.seed, STREAM_BIAS, (s.G,), 0.0, math.sqrt(s.bias_param)).astype(np.float64)
    raise ValueError(s.bias)


def logits(s: Spec) -> np.ndarray:
    """Router logits fp32 [T, G] = raw N(0,1) + per-expert bias (sum taken in double, rounded once)."""
    raw = normal_f32(s.seed, STREAM_LOGITS, (s.T, s.G)).astype(np.float64)
    return (raw + expert_bias(s)[None, :]).astype(np.float32)


def activations(s: Spec) -> np.ndarray:
    """Token rows X [T, d], owner-major (row r*T_o + t).  uint16 bf16 bits, or float32."""
    if s.dtype == "bf16":
        return normal_bf16(s.seed, STREAM_X, (s.T, s.d))
    return normal_f32(s.seed, STREAM_X, (s.T, s.d))


def weights(s: Spec, experts=None):
    """(w_gate_up [E,2f,d], w_down [E,d,f]) in the (out, in) row-major convention of a linear layer.

    Gate rows are [0, f) of w_gate_up and up rows [f, 2f).  ``experts`` selects local experts (default all).
    """
    experts = list(range(s.E_l)) if experts is None else list(experts)
    sig = 1.0 / math.sqrt(s.d)
    lib = _load()
    fill = lib.gen_normal_bf16 if s.dtype == "bf16" else lib.gen_normal_f32
    dt = np.uint16 if s.dtype == "bf16" else np.float32
    w1 = np.empty((len(experts), 2 * s.f, s.d), dtype=dt)
    w2 = np.empty((len(experts), s.d, s.f), dtype=dt)
    n = s.f * s.d
    for i, e in enumerate(experts):
        base = STREAM_W0 + 3 * e
        fill(s.seed, base + 0, n, 0.0, sig, w1[i, : s.f].ctypes.data)   # gate
        fill(s.seed, base + 1, n, 0.0, sig, w1[i, s.f:].ctypes.data)    # up
        fill(s.seed, base + 2, n, 0.0, sig, w2[i].ctypes.data)          # down
    return w1, w2


def d_out(s: Spec) -> np.ndarray:
    """Gradient of the combined output dOut [T, d] for the backward pass, N(0,1): uint16 bf16 bits, or float32."""
    if s.dtype == "bf16":
        return normal_bf16(s.seed, STREAM_DOUT, (s.T, s.d))
    return normal_f32(s.seed, STREAM_DOUT, (s.T, s.d))


def inputs(s: Spec) -> dict:
    """All host inputs of a workload: logits, x, w_gate_up, w_down."""
    w1, w2 = weights(s)
    return {"logits": logits(s), "x": activations(s), "w_gate_up": w1, "w_down": w2}
