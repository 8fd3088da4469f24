"""Device buffers and calls of one MoE expert-compute-plus-return problem (torch allocates, the library computes).

``MoePath`` owns every buffer the C-ABI needs for one shape and calls the entry points in order:
route -> layout -> expert FFN with return -> combine.  Nothing here computes anything itself.
"""
from __future__ import annotations

import ctypes

import torch

from . import binding as B

NAME_SIZES = ("counts", "padded_off", "recv_off", "tile_owner", "tile_expert", "tile_valid", "tile_order", "seg_desc",
              "row_src", "combine_plan", "scalars", "status", "mtile_desc", "seg_mtiles")


class MoePath:
    def __init__(self, R, T_o, G, E_l, k, d, f, M, mgb=1, dtype="bf16", self_rank=0, device="cuda"):
        self.R, self.T_o, self.G, self.E_l, self.k, self.d, self.f, self.M = R, T_o, G, E_l, k, d, f, M
        self.T = R * T_o
        self.dtype = dtype
        self.device = torch.device(device)
        self.shape = B.moe_shape(R, T_o, G, E_l, k, self_rank, d, f, M, mgb, B.MOE_BF16 if dtype == "bf16" else B.MOE_F32)
        nbytes = B.moe_layout_workspace_bytes(self.shape)
        if nbytes < 0:
            raise B.MoeError("moe_layout_workspace_bytes", -1, "invalid shape")
        self.ws = torch.empty(nbytes + 256, dtype=torch.uint8, device=self.device)
        base = (self.ws.data_ptr() + 255) // 256 * 256
        self.ws_aligned = self.ws[base - self.ws.data_ptr():]
        self.L = B.moe_layout()
        B.moe_layout_bind(self.shape, self.ws_aligned, self.L)
        cap = self.L.cap_rows
        self.tdtype = torch.bfloat16 if dtype == "bf16" else torch.float32
        z = dict(device=self.device)
        self.x_pad = torch.empty(cap, d, dtype=self.tdtype, **z)
        self.h = torch.empty(cap, f, dtype=self.tdtype, **z)
        self.y_pad = torch.empty(cap, d, dtype=self.tdtype, **z)
        self.recv_cap = T_o * min(k, E_l)
        self.recv = [torch.empty(max(self.recv_cap, 1), d, dtype=self.tdtype, **z) for _ in range(R)]
        self.flags = torch.zeros(B.moe_ffn_flags_count(self.shape), dtype=torch.int32, **z)
        self.topk_idx = torch.empty(max(self.T, 1), k, dtype=torch.int32, **z)
        self.topk_w = torch.empty(max(self.T, 1), k, dtype=torch.float32, **z)
        self.out = torch.empty(max(self.T, 1), d, dtype=self.tdtype, **z)
        self.timestamps = torch.zeros(2 + 2 * self.L.cap_tiles, dtype=torch.int64, **z)
        self.epoch = 0

    @classmethod
    def from_spec(cls, s, device="cuda"):
        return cls(s.R, s.T_o, s.G, s.E_l, s.k, s.d, s.f, s.M, s.mgb, s.dtype, 0, device)

    # ---- views of the layout arrays (int32 tensors in the workspace) ----------------------------------------
    def array(self, name: str) -> torch.Tensor:
        L = self.L
        sizes = {
            "counts": self.E_l * self.R, "padded_off": self.E_l * self.R, "recv_off": self.E_l * self.R,
            "tile_owner": L.cap_tiles, "tile_expert": L.cap_tiles, "tile_valid": L.cap_tiles,
            "tile_order": L.cap_tiles, "seg_desc": L.cap_tiles * B.MOE_SEG_FIELDS, "row_src": L.cap_rows,
            "combine_plan": self.T * self.k, "scalars": 5 + self.R, "status": 1,
            "mtile_desc": L.cap_mtiles * B.MT_FIELDS, "seg_mtiles": L.cap_tiles * 2, "seg_sched": L.cap_tiles,
            "mt_order": L.cap_mtiles,
        }
        off = (getattr(L, name) - self.ws_aligned.data_ptr()) // 4
        return self.ws_aligned.view(torch.int32)[off: off + sizes[name]]

    # ---- calls ---------------------------------------------------------------------------------------------------
    def route(self, logits: torch.Tensor, stream=None):
        B.moe_route(self.shape, logits, self.topk_idx, self.topk_w, stream)

    def layout(self, x: torch.Tensor | None, topk_idx: torch.Tensor | None = None, stream=None):
        """x None: no gather into x_pad (the FFN call lands the rows, ``ffn(x_tokens=...)``)."""
        B.moe_layout_build(self.shape, self.topk_idx if topk_idx is None else topk_idx, x, self.L, self.x_pad, stream)

    def ffn(self, w_gate_up, w_down, mode=0, consumer_cus=0, band_window=0, timestamps=False, watchdog_ticks=0,
            epoch=None, tile_order=0, x_tokens: torch.Tensor | None = None, gu_out: torch.Tensor | None = None,
            stream=None):
        """gu_out: None, or [cap_rows, 2f] fp32 (gu_buffer()) for the first GEMM's pre-activations g | u, which a
        backward call can take instead of recomputing them."""
        if epoch is None:
            self.epoch += 1
            epoch = self.epoch
        cfg = B.moe_overlap_cfg(consumer_cus, mode, epoch, band_window, watchdog_ticks,
                                self.timestamps.data_ptr() if timestamps else None, tile_order,
                                None if x_tokens is None else x_tokens.data_ptr(),
                                None if gu_out is None else gu_out.data_ptr())
        B.moe_expert_ffn_overlap(self.shape, self.L, self.x_pad, w_gate_up, w_down, self.h, self.y_pad, self.recv,
                                 self.flags, cfg, stream)
        return epoch

    # ---- backward ---------------------------------------------------------------------------------------------
    def bwd_buffers(self):
        """The backward call's workspaces and outputs, allocated on first use (bf16 only)."""
        if getattr(self, "_bwd", None) is None:
            cap, d, f, z = self.L.cap_rows, self.d, self.f, dict(device=self.device)
            n = B.moe_bwd_flags_count(self.shape)
            if n < 0:
                raise B.MoeError("moe_bwd_flags_count", -1, "shape has no backward pass")
            self._bwd = {
                "dy_pad": torch.empty(cap, d, dtype=torch.bfloat16, **z),
                "dh_ws": torch.empty(cap, f, dtype=torch.float32, **z),
                "dgu_ws": torch.empty(cap, 2 * f, dtype=torch.bfloat16, **z),
                "dx_pad": torch.empty(cap, d, dtype=torch.bfloat16, **z),
                "dx_recv": [torch.empty(max(self.recv_cap, 1), d, dtype=torch.bfloat16, **z) for _ in range(self.R)],
                "dw_gate_up": torch.empty(self.E_l, 2 * f, d, dtype=torch.float32, **z),
                "dw_down": torch.empty(self.E_l, d, f, dtype=torch.float32, **z),
                "flags": torch.zeros(n, dtype=torch.int32, **z),
                "dx": torch.empty(max(self.T, 1), d, dtype=torch.bfloat16, **z),
                "dw_route": torch.empty(max(self.T, 1), self.k, dtype=torch.float32, **z),
            }
            self.bwd_epoch = 0
        return self._bwd

    def gu_buffer(self):
        """[cap_rows, 2f] fp32 for the forward's g | u (ffn(gu_out=...), backward(gu=...)), allocated on first use."""
        if getattr(self, "_gu", None) is None:
            self._gu = torch.empty(self.L.cap_rows, 2 * self.f, dtype=torch.float32, device=self.device)
        return self._gu

    def backward(self, d_out: torch.Tensor, w_gate_up, w_down, mode=0, consumer_cus=0, watchdog_ticks=0, epoch=None,
                 gu: torch.Tensor | None = None, stream=None):
        """The expert FFN's backward with the dX return (moe_expert_ffn_backward), for the routing, layout and x_pad
        of the last forward; the forward's h workspace receives the recomputed h.  gu: None, or the g | u that forward
        stored (ffn(gu_out=...)), which the h / dG / dU items then read instead of recomputing the first GEMM."""
        b = self.bwd_buffers()
        if epoch is None:
            self.bwd_epoch += 1
            epoch = self.bwd_epoch
        cfg = B.moe_overlap_cfg(consumer_cus, mode, epoch, 0, watchdog_ticks, None, 0, None)
        t = {"topk_idx": self.topk_idx, "topk_w": self.topk_w, "x_pad": self.x_pad, "w_gate_up": w_gate_up,
             "w_down": w_down, "d_out": d_out, "h_ws": self.h, "gu": gu,
             **{k: b[k] for k in ("dy_pad", "dh_ws", "dgu_ws", "dx_pad", "dw_gate_up", "dw_down")}}
        B.moe_expert_ffn_backward(self.shape, self.L, t, b["dx_recv"], b["flags"], cfg, stream)
        return epoch

    def combine_backward(self, d_out: torch.Tensor, stream=None):
        """dx and the routing weights' gradient (moe_combine_backward) from the delivered dX rows and the forward's
        delivered y rows."""
        b = self.bwd_buffers()
        B.moe_combine_backward(self.shape, self.L, d_out, self.recv, b["dx_recv"], b["dx"], b["dw_route"], stream)

    def combine(self, topk_w: torch.Tensor | None = None, stream=None):
        B.moe_combine(self.shape, self.L, self.topk_w if topk_w is None else topk_w, self.recv, self.out, stream)

    def partition_record(self):
        """The launch's consumer-partition record (bf16): (consumer CUs of the last overlapped call, observed producer
        flops per CU-tick, observed consumer bytes per CU-tick, whether both rates hold observations)."""
        import struct

        w = self.flags[-B.MOE_OBS_WORDS:].cpu().numpy().astype("<i4").view("<u4")
        f = lambda v: struct.unpack("<f", struct.pack("<I", int(v)))[0]
        return int(w[12]), f(w[10]), f(w[11]), int(w[13]) == 3

    def status(self, stream=None) -> int:
        return B.moe_read_status(self.L, stream)

    def scalars(self):
        sc = self.array("scalars").cpu().tolist()
        return {"M_pad": sc[0], "n_tiles": sc[1], "n_segs": sc[2], "N_r": sc[3:3 + self.R], "n_mtiles": sc[3 + self.R],
                "n_remote_mtiles": sc[4 + self.R]}


def to_device(a, dtype: str, device="cuda") -> torch.Tensor:
    """Host array from moe_inputs (bf16 bits as uint16, or fp32/int32) to a device tensor of the right type."""
    import numpy as np

    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(a).to(device)
