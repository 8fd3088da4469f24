"""ctypes binding of libmoe_overlap.so: the C-ABI entry points under the same names (argument marshalling only).

Tensors are torch tensors on the GPU (device memory); streams are torch streams (their hipStream_t is passed).
Every computation runs in the library's HIP kernels; there is no fallback: if the library is missing this
module raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe_overlap.so")

MOE_OK, MOE_EINVAL, MOE_ECAPACITY, MOE_EHIP, MOE_ETIMEOUT = 0, -1, -2, -3, -4
MOE_BF16, MOE_F32 = 0, 1
MOE_SEG_FIELDS = 8
MOE_OBS_WORDS = 16
MT_HDR = 8
MT_FIELDS = MT_HDR + 256
EXPORTS = ["moe_last_error", "moe_version", "moe_route", "moe_layout_capacity_rows", "moe_layout_workspace_bytes",
           "moe_layout_bind", "moe_layout_build", "moe_read_status", "moe_ffn_flags_count", "moe_pick_consumer_cus",
           "moe_pick_consumer_cus_observed",
           "moe_expert_ffn_overlap", "moe_expert_ffn_overlap_noalloc", "moe_ffn_schedule",
           "moe_combine", "moe_set_kernel_timing", "moe_kernel_times", "moe_bwd_flags_count",
           "moe_expert_ffn_backward", "moe_combine_backward"]


class moe_shape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("R", "tokens_per_owner", "num_global_experts", "num_local_experts",
                                               "top_k", "self_rank", "d", "f", "tile_m", "seg_bands", "dtype")]


LAYOUT_ARRAYS = ["counts", "padded_off", "recv_off", "tile_owner", "tile_expert", "tile_valid", "tile_order",
                 "seg_desc", "row_src", "combine_plan", "scalars", "status", "mtile_desc", "seg_mtiles",
                 "seg_sched", "chunk_counts", "mt_order"]


class moe_layout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in LAYOUT_ARRAYS] + [
        ("cap_rows", ctypes.c_int64), ("cap_tiles", ctypes.c_int64), ("cap_mtiles", ctypes.c_int64)]


class moe_overlap_cfg(ctypes.Structure):
    _fields_ = [("consumer_cus", ctypes.c_int32), ("mode", ctypes.c_int32), ("epoch", ctypes.c_uint32),
                ("band_window", ctypes.c_int32), ("watchdog_ticks", ctypes.c_uint64),
                ("timestamps", ctypes.c_void_p), ("tile_order", ctypes.c_int32), ("x_tokens", ctypes.c_void_p),
                ("gu_out", ctypes.c_void_p)]


BWD_FIELDS = ["topk_idx", "topk_w", "x_pad", "w_gate_up", "w_down", "d_out", "dy_pad", "dh_ws", "h_ws", "dgu_ws",
              "dx_pad", "dx_recv", "dw_gate_up", "dw_down", "gu"]


class moe_bwd_args(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in BWD_FIELDS]


class MoeError(RuntimeError):
    def __init__(self, fn: str, code: int, msg: str):
        super().__init__("%s failed (%d): %s" % (fn, code, msg))
        self.code = code


_lib = None


def lib():
    """The loaded library.  Raises if it has not been built: there is no other implementation to fall to."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libmoe_overlap.so is not built (%s); run __graft_entry__.build()" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
        ps, pl, pc = ctypes.POINTER(moe_shape), ctypes.POINTER(moe_layout), ctypes.POINTER(moe_overlap_cfg)
        sig = {
            "moe_last_error": ([], ctypes.c_char_p), "moe_version": ([], ctypes.c_char_p),
            "moe_route": ([ps, vp, vp, vp, vp], i32),
            "moe_layout_capacity_rows": ([ps], i64), "moe_layout_workspace_bytes": ([ps], i64),
            "moe_layout_bind": ([ps, vp, i64, pl], i32),
            "moe_layout_build": ([ps, vp, vp, pl, vp, vp], i32),
            "moe_read_status": ([pl, vp], i32), "moe_ffn_flags_count": ([ps], i64),
            "moe_pick_consumer_cus": ([ps, i32], i32),
            "moe_pick_consumer_cus_observed": ([ps, i32, i64, i64, i32, ctypes.c_float, ctypes.c_float], i32),
            "moe_expert_ffn_overlap": ([ps, pl, vp, vp, vp, vp, vp, vp, vp, pc, vp], i32),
            "moe_expert_ffn_overlap_noalloc": ([ps, pl, vp, vp, vp, vp, vp, vp, pc, vp], i32),
            "moe_combine": ([ps, pl, vp, vp, vp, vp], i32),
            "moe_ffn_schedule": ([ps, i32, pc, i32, i32, vp, vp, vp, i64, ctypes.POINTER(ctypes.c_int64)], i32),
            "moe_set_kernel_timing": ([i32], i32), "moe_kernel_times": ([ctypes.POINTER(ctypes.c_double)], i32),
            "moe_bwd_flags_count": ([ps], i64),
            "moe_expert_ffn_backward": ([ps, pl, ctypes.POINTER(moe_bwd_args), vp, pc, vp], i32),
            "moe_combine_backward": ([ps, pl, vp, vp, vp, vp, vp, vp], i32),
        }
        for name, (args, res) in sig.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _lib = L
    return _lib


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check(fn: str, rc: int) -> int:
    if rc != MOE_OK:
        raise MoeError(fn, rc, moe_last_error())
    return rc


def _ptr_array(tensors):
    arr = (ctypes.c_void_p * max(1, len(tensors)))()
    for i, t in enumerate(tensors):
        arr[i] = t.data_ptr()
    return arr


# ---- entry points --------------------------------------------------------------------------------------------

def moe_last_error() -> str:
    return lib().moe_last_error().decode()


def moe_version() -> str:
    return lib().moe_version().decode()


def moe_route(shape: moe_shape, logits, topk_idx, topk_w, stream=None) -> int:
    return _check("moe_route", lib().moe_route(ctypes.byref(shape), _ptr(logits), _ptr(topk_idx), _ptr(topk_w),
                                               _stream(stream)))


def moe_layout_capacity_rows(shape: moe_shape) -> int:
    return lib().moe_layout_capacity_rows(ctypes.byref(shape))


def moe_layout_workspace_bytes(shape: moe_shape) -> int:
    return lib().moe_layout_workspace_bytes(ctypes.byref(shape))


def moe_layout_bind(shape: moe_shape, workspace, layout: moe_layout) -> int:
    return _check("moe_layout_bind", lib().moe_layout_bind(ctypes.byref(shape), _ptr(workspace),
                                                           workspace.numel() * workspace.element_size(),
                                                           ctypes.byref(layout)))


def moe_layout_build(shape: moe_shape, topk_idx, x, layout: moe_layout, x_pad, stream=None) -> int:
    return _check("moe_layout_build", lib().moe_layout_build(ctypes.byref(shape), _ptr(topk_idx), _ptr(x),
                                                             ctypes.byref(layout), _ptr(x_pad), _stream(stream)))


def moe_read_status(layout: moe_layout, stream=None) -> int:
    return lib().moe_read_status(ctypes.byref(layout), _stream(stream))


def moe_ffn_flags_count(shape: moe_shape) -> int:
    return lib().moe_ffn_flags_count(ctypes.byref(shape))


def moe_pick_consumer_cus(shape: moe_shape, n_cu: int) -> int:
    return lib().moe_pick_consumer_cus(ctypes.byref(shape), n_cu)


def moe_pick_consumer_cus_observed(shape: moe_shape, n_cu: int, rows_routed: int, rows_returned: int, n_mtiles: int,
                                   ffn_rate: float, copy_rate: float) -> int:
    return lib().moe_pick_consumer_cus_observed(ctypes.byref(shape), n_cu, rows_routed, rows_returned, n_mtiles,
                                                ffn_rate, copy_rate)


def moe_expert_ffn_overlap(shape: moe_shape, layout: moe_layout, x_pad, w_gate_up, w_down, h_ws, y_pad, recv,
                           flags, cfg: moe_overlap_cfg, stream=None) -> int:
    return _check("moe_expert_ffn_overlap", lib().moe_expert_ffn_overlap(
        ctypes.byref(shape), ctypes.byref(layout), _ptr(x_pad), _ptr(w_gate_up), _ptr(w_down), _ptr(h_ws),
        _ptr(y_pad), _ptr_array(recv), _ptr(flags), ctypes.byref(cfg), _stream(stream)))


def moe_expert_ffn_overlap_noalloc(shape: moe_shape, layout: moe_layout, x_pad, w_gate_up, w_down, h_ws, y_pad, recv,
                                   cfg: moe_overlap_cfg, stream=None) -> int:
    return _check("moe_expert_ffn_overlap_noalloc", lib().moe_expert_ffn_overlap_noalloc(
        ctypes.byref(shape), ctypes.byref(layout), _ptr(x_pad), _ptr(w_gate_up), _ptr(w_down), _ptr(h_ws),
        _ptr(y_pad), _ptr_array(recv), ctypes.byref(cfg), _stream(stream)))


def moe_ffn_schedule(shape: moe_shape, n_cu: int, cfg: moe_overlap_cfg, mt_hdr, mt_order, n_remote: int):
    """The bf16 FFN launch's item list (host only): int32 numpy array [n, 8] of {workgroup, sequence, kind, row tile,
    column tile, split, half, target} by list index.  mt_hdr: int32 [n_mtiles, 4]; mt_order: int32 [n_mtiles]."""
    import numpy as np

    mt_hdr = np.ascontiguousarray(mt_hdr, dtype=np.int32).reshape(-1, 4)
    mt_order = np.ascontiguousarray(mt_order, dtype=np.int32).reshape(-1)
    n = ctypes.c_int64(0)
    args = (ctypes.byref(shape), n_cu, ctypes.byref(cfg), mt_hdr.shape[0], n_remote, mt_hdr.ctypes.data,
            mt_order.ctypes.data)
    _check("moe_ffn_schedule", lib().moe_ffn_schedule(*args, None, 0, ctypes.byref(n)))
    out = np.zeros((max(n.value, 1), 8), dtype=np.int32)
    _check("moe_ffn_schedule", lib().moe_ffn_schedule(*args, out.ctypes.data, n.value, ctypes.byref(n)))
    return out[: n.value]


def moe_combine(shape: moe_shape, layout: moe_layout, topk_w, recv, out, stream=None) -> int:
    return _check("moe_combine", lib().moe_combine(ctypes.byref(shape), ctypes.byref(layout), _ptr(topk_w),
                                                   _ptr_array(recv), _ptr(out), _stream(stream)))


def moe_set_kernel_timing(enable: bool) -> int:
    return _check("moe_set_kernel_timing", lib().moe_set_kernel_timing(int(bool(enable))))


def moe_kernel_times():
    """(gemm1 ms, gemm2 ms, consumer ms, calls) summed since the last query."""
    out = (ctypes.c_double * 4)()
    _check("moe_kernel_times", lib().moe_kernel_times(out))
    return out[0], out[1], out[2], int(out[3])


def moe_bwd_flags_count(shape: moe_shape) -> int:
    return lib().moe_bwd_flags_count(ctypes.byref(shape))


def moe_expert_ffn_backward(shape: moe_shape, layout: moe_layout, tensors: dict, dx_recv, flags, cfg: moe_overlap_cfg,
                            stream=None) -> int:
    """tensors: the moe_bwd_args fields other than dx_recv, as device tensors ("gu" optional)."""
    ptrs = _ptr_array(dx_recv)
    a = moe_bwd_args(**{k: (ctypes.cast(ptrs, ctypes.c_void_p) if k == "dx_recv" else
                            _ptr(tensors.get(k) if k == "gu" else tensors[k])) for k in BWD_FIELDS})
    return _check("moe_expert_ffn_backward", lib().moe_expert_ffn_backward(
        ctypes.byref(shape), ctypes.byref(layout), ctypes.byref(a), _ptr(flags), ctypes.byref(cfg), _stream(stream)))


def moe_combine_backward(shape: moe_shape, layout: moe_layout, d_out, y_recv, dx_recv, dx, dw_route, stream=None) -> int:
    return _check("moe_combine_backward", lib().moe_combine_backward(
        ctypes.byref(shape), ctypes.byref(layout), _ptr(d_out), _ptr_array(y_recv), _ptr_array(dx_recv), _ptr(dx),
        _ptr(dw_route), _stream(stream)))
