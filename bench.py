"""Benchmark of the MoE expert-compute-plus-return path on one MI355X.

A step is one pass of the whole path over one batch already resident in HBM: layout build (histogram, scans,
scatter, row gather) -> expert SwiGLU FFN with tile-signalled return of finished row-band segments to the R owner
buffers (producer and consumer overlapped on disjoint CU partitions) -> top-k weighted combine.  Routing is the
path's input and runs once before the timed region.

Prints one JSON line.  ``value`` is useful (algorithmic) TFLOP/s of the whole step, 6 * M_real * d * f flops per
step; the line also carries the FFN-only TFLOP/s and % of the bf16 dense MFMA peak, the return-copy overlap ratio,
the sequential-vs-overlapped comparison, a roofline entry for the dominant kernel and the CPU oracle's rate.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
MFMA_F32_PEAK_TFLOPS = 157.3
HBM_PEAK_GBS = 8000.0
METRIC = "grouped expert-FFN TFLOP/s (% bf16 MFMA peak) + return-copy overlap ratio %"


def workload_name(s) -> str:
    return ("%s: R=%d owners x %d tokens, G=%d experts top-%d, %d local, d=%d, f=%d, tile M=%d, %s, mgb=%d"
            % (s.name, s.R, s.T_o, s.G, s.k, s.E_l, s.d, s.f, s.M, s.dtype, s.mgb))


def overlap_stats(ts: np.ndarray, n_segs: int, tick_ns: float = 10.0) -> dict:
    """Fraction of consumer copy time inside [first producer item start, last flag publish], over the segments the
    consumer copied (the self owner's segments have no copy: the producer stores those rows itself)."""
    p0, p1 = int(ts[0]), int(ts[1])
    s = ts[2:2 + 2 * n_segs:2]
    e = ts[3:3 + 2 * n_segs:2]
    copied = e != 0
    s, e = s[copied].astype(np.int64), e[copied].astype(np.int64)
    n_segs = int(copied.sum())
    dur = np.maximum(e - s, 0)
    inter = np.maximum(np.minimum(e, p1) - np.maximum(s, p0), 0)
    tot = dur.sum()
    return {
        "overlap_ratio": float(inter.sum() / tot) if tot > 0 else None,
        "producer_span_us": (p1 - p0) * tick_ns / 1e3,
        "copy_time_us": float(tot) * tick_ns / 1e3,
        "exposed_tail_us": max(0, int(e.max()) - p1) * tick_ns / 1e3 if n_segs else 0.0,
        "first_copy_after_start_us": (int(s.min()) - p0) * tick_ns / 1e3 if n_segs else None,
        # from the first copy start to the last copy end: the window the overlapped return took
        "copy_window_us": (int(e.max()) - int(s.min())) * tick_ns / 1e3 if n_segs else 0.0,
    }


def hbm_traffic(s, cus: int, band_window: int, land: bool, mode: int):
    """HBM bytes per launch of the FFN kernel from the committed counter summary (FETCH_SIZE and WRITE_SIZE, each
    scaled by the same counter's reading for a plain copy of known size), if one covers this workload and launch
    configuration and the kernel sources are the ones it was taken on; else None."""
    import hashlib

    path = os.path.join(ROOT, "profiles", "k_ffn_bf16_%s_hbm_bytes.json" % s.name)
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    c = rec["configuration"]
    want = {"config": s.name, "mgb": s.mgb, "consumer_cus_option": cus, "band_window": band_window or 4,
            "token_rows_landed_by": "the FFN launch" if land else "the layout's gather kernel", "mode": mode}
    if any(c.get(k) != v for k, v in want.items()):
        return None
    h = hashlib.sha256()
    for p in rec["sources"]:
        h.update(open(os.path.join(ROOT, p), "rb").read())
    return rec["hbm_bytes_per_launch"] if h.hexdigest() == rec["source_sha256"] else None


def _cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _omp_threads(n: int) -> None:
    """Set the OpenMP thread count of this process (the oracle's parallel FFN)."""
    import ctypes

    for name in ("libgomp.so.1", "libgomp.so"):
        try:
            ctypes.CDLL(name).omp_set_num_threads(int(n))
            return
        except OSError:
            continue


def _oracle_ffn_sample(s, inp, lay, target_s: float, seed: int = 1):
    """The oracle's FFN on a random sample of real rows grown until it takes about target_s; (rows, seconds)."""
    import oracle

    real = np.nonzero(lay["row_src"] >= 0)[0]
    rng = np.random.default_rng(seed)
    n = 8
    while True:
        rows = rng.choice(real, min(n, real.size), replace=False)
        t0 = time.perf_counter()
        oracle.ffn_rows(lay["row_src"][rows], lay["tile_expert"][rows // s.M], inp["x"], inp["w_gate_up"],
                        inp["w_down"], s.dtype == "bf16")
        dt = time.perf_counter() - t0
        if dt >= target_s or n >= real.size:
            return rows.size, real.size, dt
        n = min(real.size, int(n * max(2.0, 1.2 * target_s / max(dt, 1e-3))))


def _oracle_bwd_sample(s, inp, lay, idx, w, target_s: float, seed: int = 3):
    """The oracle's backward rows (dY, dH, h, dG, dU, dX; no forward y) on a random sample of local slots grown until
    it takes about target_s; (rows, seconds)."""
    import moe_inputs as mi
    import oracle

    t_all, j_all = np.nonzero(idx < s.E_l)
    d_out = mi.d_out(s)
    rng = np.random.default_rng(seed)
    n = 4
    while True:
        pick = rng.choice(t_all.size, min(n, t_all.size), replace=False)
        t, j = t_all[pick], j_all[pick]
        t0 = time.perf_counter()
        oracle.bwd_rows(t, idx[t, j], w[t, j], inp["x"], inp["w_gate_up"], inp["w_down"], d_out, s.dtype == "bf16",
                        want_y=False)
        dt = time.perf_counter() - t0
        if dt >= target_s or n >= t_all.size:
            return pick.size, dt
        n = min(t_all.size, int(n * max(2.0, 1.2 * target_s / max(dt, 1e-3))))


def cpu_baseline(s, inp, target_s: float):
    """The CPU oracle on the same workload: routing, layout, delivery and combine on the full batch, the FFN on a
    bounded random sample of real rows (useful TFLOP/s), every stage timed, all host threads; plus the whole oracle
    on Tiny and the FFN of Skewed on one thread."""
    import oracle
    import moe_inputs as mi

    oracle.load()
    cores = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    _omp_threads(cores)
    st = {}
    t0 = time.perf_counter()
    idx, w = oracle.route(inp["logits"], s.k)
    st["route_s"] = time.perf_counter() - t0
    t0 = time.perf_counter()
    lay = oracle.layout(idx, s.R, s.T_o, s.G, s.E_l, s.k, s.M, s.mgb, 0)
    st["layout_s"] = time.perf_counter() - t0
    n_rows, n_real, dt = _oracle_ffn_sample(s, inp, lay, target_s)
    st["ffn_sample_s"] = dt
    flops = 6.0 * n_rows * s.d * s.f
    # delivery and combine of the full batch (their cost does not depend on the values)
    y_pad = np.zeros((lay["M_pad"], s.d))
    t0 = time.perf_counter()
    recv = oracle.deliver(lay, y_pad, s.R, s.E_l)
    st["deliver_s"] = time.perf_counter() - t0
    t0 = time.perf_counter()
    oracle.combine(lay, w, recv, s.R, s.T_o, s.k, s.dtype == "bf16")
    st["combine_s"] = time.perf_counter() - t0
    st["ffn_full_batch_s_extrapolated"] = dt * n_real / n_rows
    bwd = None
    if s.dtype == "bf16":  # the backward rows on a sample: 10 d f flops per row (dH 2, g and u 4, dX 4)
        nb, db = _oracle_bwd_sample(s, inp, lay, idx, w, min(5.0, target_s / 2))
        bwd = {"value": 10.0 * nb * s.d * s.f / db / 1e12, "unit": "TFLOP/s",
               "sample": "oracle backward rows (dY, dH, h, dG, dU, dX; fp64) for %d local slots, %.1f s" % (nb, db)}
    # one thread: the whole oracle on Tiny, and the FFN of Skewed on a sample
    _omp_threads(1)
    ts = mi.spec("tiny")
    tin = mi.inputs(ts)
    t0 = time.perf_counter()
    oracle.run(ts, tin)
    one = {"tiny_whole_path_s": time.perf_counter() - t0}
    sk = mi.spec("skew")
    skin = mi.inputs(sk)
    skidx, _ = oracle.route(skin["logits"], sk.k)
    sklay = oracle.layout(skidx, sk.R, sk.T_o, sk.G, sk.E_l, sk.k, sk.M, sk.mgb, 0)
    r1, n1, d1 = _oracle_ffn_sample(sk, skin, sklay, min(3.0, target_s / 3), seed=2)
    one["skew_ffn_tflops"] = 6.0 * r1 * sk.d * sk.f / d1 / 1e12
    one["skew_ffn_sample"] = "%d of %d real rows, %.1f s" % (r1, n1, d1)
    _omp_threads(cores)
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": "oracle FFN (fp64, h and y rounded to bf16) on %d of %d real rows, %.1f s; routing, layout, "
                      "delivery and combine of the full batch" % (n_rows, n_real, dt),
            "cpu_model": _cpu_model(), "stages_s": {k: round(v, 4) for k, v in st.items()},
            "one_thread": one, "backward_rows": bwd}


def bench_backward(P, s, w1, w2, reps: int, M_real: int, ffn_call) -> dict:
    """The backward pass for the last forward's routing and layout: dY dispatch, the persistent launch (dH, h / dG /
    dU, dX with its return to the owners, the weight gradients) and the combine's backward, as one call; overlapped
    (consumer workgroups return dX rows while the weight gradients run) and sequential (the return after the launch).
    Flops: 12 M d f for the gradients (dH 2, dX 4, dW_down 2, dW_gate_up 4), 16 M d f with the launch's recompute of
    the gate and up projections.  Then the same with the gate and up pre-activations stored by the forward
    (ffn_call(gu_out), the step's FFN call) instead of recomputed: that forward call's time with and without storing
    them, the backward taking them, and the two forward + backward sums."""
    import torch

    import moe_inputs as mi
    from expert_output_overlap_amd import binding as B
    from expert_output_overlap_amd.runtime import to_device

    d_out = to_device(mi.d_out(s), s.dtype)
    P.bwd_buffers()

    gu = None

    def call(mode):
        P.backward(d_out, w1, w2, mode=mode, gu=gu)
        P.combine_backward(d_out)

    for _ in range(3):
        call(0)
    torch.cuda.synchronize()
    assert P.status() == B.MOE_OK

    def timed(mode):
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        B.moe_set_kernel_timing(True)
        B.moe_kernel_times()
        ts = []
        for _ in range(reps):
            ev0.record()
            call(mode)
            ev1.record()
            ev1.synchronize()
            ts.append(ev0.elapsed_time(ev1))
        k_ms, _, c_ms, n = B.moe_kernel_times()
        B.moe_set_kernel_timing(False)
        assert P.status() == B.MOE_OK
        return float(np.median(ts)), k_ms / n, c_ms / n

    t_ovl, k_ovl, _ = timed(0)
    t_seq, k_seq, c_seq = timed(1)
    grads = 12.0 * M_real * s.d * s.f
    executed = 16.0 * M_real * s.d * s.f
    ret_bytes = 2.0 * (M_real - int(P.scalars()["N_r"][P.shape.self_rank])) * s.d * 2

    def time_fwd(g):
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ffn_call(g)
        ts = []
        for _ in range(reps):
            ev0.record()
            ffn_call(g)
            ev1.record()
            ev1.synchronize()
            ts.append(ev0.elapsed_time(ev1))
        assert P.status() == B.MOE_OK
        return float(np.median(ts))

    f_plain = time_fwd(None)
    gu = P.gu_buffer()
    f_gu = time_fwd(gu)  # leaves this routing's g | u in gu for the calls below
    t_gu, k_gu, _ = timed(0)
    saved = {
        "ms": round(t_gu, 4), "launch_ms": round(k_gu, 4),
        "tflops_gradients": round(grads / (t_gu * 1e-3) / 1e12, 2),
        "launch_tflops_executed": round(grads / (k_gu * 1e-3) / 1e12, 2),
        "forward_ffn_ms": round(f_plain, 4), "forward_ffn_ms_storing": round(f_gu, 4),
        "forward_plus_backward_ms_recompute": round(f_plain + t_ovl, 4),
        "forward_plus_backward_ms_stored": round(f_gu + t_gu, 4),
    }
    return {
        "ms": round(t_ovl, 4), "ms_sequential": round(t_seq, 4),
        "saved_vs_sequential_us": round(1e3 * (t_seq - t_ovl), 1),
        "tflops_gradients": round(grads / (t_ovl * 1e-3) / 1e12, 2),
        "pct_bf16_peak_gradients": round(100 * grads / (t_ovl * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 2),
        "launch_ms": {"overlapped": round(k_ovl, 4), "sequential_producer": round(k_seq, 4),
                      "sequential_return": round(c_seq, 4)},
        "launch_tflops_executed": round(executed / (k_ovl * 1e-3) / 1e12, 2),
        "launch_pct_bf16_peak_executed": round(100 * executed / (k_ovl * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 2),
        "return_gbs_sequential": round(ret_bytes / (c_seq * 1e-3) / 1e9, 1),
        "with_stored_preactivations": saved,
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="deepseek")
    ap.add_argument("--consumer-cus", type=int, default=0,
                    help="consumer CUs of the overlapped launch (0 = the launch picks them from the batch's routing "
                         "and the rates it observed, 0 included; -1 = none: the return at the launch's tail)")
    ap.add_argument("--mgb", type=int, default=1)
    ap.add_argument("--band-window", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--kernels-only", action="store_true", help="timed loop only (for profiler runs)")
    ap.add_argument("--mode", type=int, default=0, choices=(0, 1, 3),
                    help="FFN mode of the timed steps: 0 overlapped, 1 sequential (the consumer alone after the "
                         "producer, for profiling the copy), 3 the return on the DMA engines")
    ap.add_argument("--backward", type=int, default=1, choices=(0, 1, 2),
                    help="1 (default, bf16): also time the layer's backward pass after the forward steps; 2: with "
                         "--kernels-only, the backward calls take the forward's stored pre-activations")
    ap.add_argument("--land", type=int, default=1, choices=(0, 1),
                    help="where x_pad's token rows come from: 1 (default) the FFN launch lands them itself, row tile "
                         "by row tile, while its first GEMM starts; 0 the layout's gather kernel")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: this path runs on a single MI355X (the owner ranks are receive buffers in "
              "its HBM); --gpus %d is not supported" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch

    import moe_inputs as mi
    from expert_output_overlap_amd import binding as B
    from expert_output_overlap_amd.runtime import MoePath, to_device

    assert torch.cuda.is_available(), "bench.py needs the GPU"
    s = mi.spec(args.config, mgb=args.mgb)
    t0 = time.perf_counter()
    inp = mi.inputs(s)
    t_gen = time.perf_counter() - t0
    print("inputs generated in %.1f s" % t_gen, file=sys.stderr, flush=True)
    P = MoePath.from_spec(s)
    dev = {k: to_device(v, s.dtype) for k, v in inp.items()}
    P.route(dev["logits"])
    torch.cuda.synchronize()
    w1, w2 = dev["w_gate_up"], dev["w_down"]
    # consumer_cus = 0: every overlapped launch picks its partition from the batch's routing and observed rates
    cus = args.consumer_cus

    land = args.land == 1 and s.dtype == "bf16" and args.mode in (0, 1)

    def step(mode=0, timestamps=False):
        P.layout(None if land else dev["x"])
        P.ffn(w1, w2, mode=mode, consumer_cus=cus, band_window=args.band_window, timestamps=timestamps,
              x_tokens=dev["x"] if land else None)
        P.combine()

    for _ in range(args.warmup):
        step(mode=args.mode)
    torch.cuda.synchronize()
    assert P.status() == B.MOE_OK, "device status %d" % P.status()
    sc = P.scalars()
    M_real = int(sum(sc["N_r"]))
    M_pad = sc["M_pad"]
    useful = 6.0 * M_real * s.d * s.f
    # executed MFMA work: the GEMMs skip the 32-row MFMA blocks of a row tile that hold no real row
    n_mt = sc["n_mtiles"]
    mt_rows = P.array("mtile_desc").view(-1, B.MT_FIELDS)[:n_mt, 1].cpu().numpy().astype(np.int64)
    executed = 6.0 * float(((mt_rows + 31) // 32 * 32).sum()) * s.d * s.f if s.dtype == "bf16" else useful

    # timed region: K whole steps, kernel events recorded on the streams the kernels run on
    B.moe_set_kernel_timing(True)
    B.moe_kernel_times()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(mode=args.mode)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    g1_ms, g2_ms, cons_ms, ncalls = B.moe_kernel_times()
    B.moe_set_kernel_timing(False)
    assert P.status() == B.MOE_OK
    ms_step = wall * 1e3 / args.steps
    print("timed %d steps: %.3f ms/step" % (args.steps, ms_step), file=sys.stderr, flush=True)
    if args.kernels_only:
        line = {"ms_per_step": ms_step}
        if args.backward and s.dtype == "bf16":  # the backward calls too, for profiles of their kernels
            d_out = to_device(mi.d_out(s), s.dtype)
            P.bwd_buffers()
            gu = None
            if args.backward == 2:  # one forward call that stores g | u, which every backward call then reads
                gu = P.gu_buffer()
                P.ffn(w1, w2, mode=0, consumer_cus=cus, band_window=args.band_window,
                      x_tokens=dev["x"] if land else None, gu_out=gu)
            for i in range(args.warmup + args.steps):
                if i == args.warmup:
                    torch.cuda.synchronize()
                    t0 = time.perf_counter()
                P.backward(d_out, w1, w2, mode=0, gu=gu)
                P.combine_backward(d_out)
            torch.cuda.synchronize()
            assert P.status() == B.MOE_OK
            line["backward_ms"] = (time.perf_counter() - t0) * 1e3 / max(args.steps, 1)
        print(json.dumps(line))
        return

    # FFN call alone, overlapped and sequential (events on the caller stream around the call)
    def time_ffn(mode, reps, xt=None):
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        c = cus if mode != 3 else max(cus, 0)  # the DMA return has no consumer workgroups to leave out
        P.ffn(w1, w2, mode=mode, consumer_cus=c, band_window=args.band_window, x_tokens=xt)
        ts = []
        for _ in range(reps):
            ev0.record()
            P.ffn(w1, w2, mode=mode, consumer_cus=c, band_window=args.band_window, x_tokens=xt)
            ev1.record()
            ev1.synchronize()
            ts.append(ev0.elapsed_time(ev1))
        return float(np.median(ts)), float(np.min(ts)), float(np.max(ts))

    reps = max(5, args.steps)
    t_ovl = time_ffn(0, reps)
    t_land = time_ffn(0, reps, dev["x"]) if land else None
    part = P.partition_record() if s.dtype == "bf16" else (cus, 0.0, 0.0, False)
    t_seq = time_ffn(1, reps)
    t_dma = time_ffn(3, max(3, reps // 4)) if s.dtype == "bf16" else None
    B.moe_set_kernel_timing(True)
    B.moe_kernel_times()
    for _ in range(reps):
        P.ffn(w1, w2, mode=1, consumer_cus=cus, band_window=args.band_window)
    torch.cuda.synchronize()
    s1, s2, sc_ms, sn = B.moe_kernel_times()
    B.moe_set_kernel_timing(False)
    copy_seq_ms = sc_ms / sn
    # overlap ratio from device timestamps (100 MHz clock), median over reps
    ovl = []
    for _ in range(reps):
        P.ffn(w1, w2, mode=0, consumer_cus=cus, band_window=args.band_window, timestamps=True)
        torch.cuda.synchronize()
        ovl.append(overlap_stats(P.timestamps.cpu().numpy().view(np.uint64), sc["n_segs"]))
    ratio = float(np.median([o["overlap_ratio"] for o in ovl if o["overlap_ratio"] is not None]))
    o_med = {k: float(np.median([o[k] for o in ovl])) for k in ("producer_span_us", "copy_time_us",
                                                                   "exposed_tail_us", "copy_window_us")}
    torch.cuda.synchronize()
    assert P.status() == B.MOE_OK

    g1_avg, g2_avg = g1_ms / ncalls, g2_ms / ncalls
    ffn_tflops = useful / (t_ovl[0] * 1e-3) / 1e12
    # the dominant launch: for bf16 the whole FFN (6 M_real d f flops), for fp32 the first GEMM (4 M_real d f)
    roof_flops = useful if s.dtype == "bf16" else 4.0 * M_real * s.d * s.f
    # the return moves the other owners' rows (the producer stores the self owner's rows into its buffer itself)
    M_ret = M_real - int(sc["N_r"][P.shape.self_rank])
    copy_bytes = 2.0 * M_ret * s.d * (2 if s.dtype == "bf16" else 4)
    peak = MFMA_BF16_PEAK_TFLOPS if s.dtype == "bf16" else MFMA_F32_PEAK_TFLOPS
    value = useful / (ms_step * 1e-3) / 1e12
    res = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": s.dtype, "data": "synthetic",
        "config": {"workload": workload_name(s), "M_real": M_real, "M_returned": M_ret, "M_pad": M_pad,
                   "gemm_row_tiles": sc["n_mtiles"],
                   # 0: no consumer partition (every workgroup takes copy units once its items are done)
                   "consumer_cus": max(args.consumer_cus, 0) if args.consumer_cus else part[0],
                   "consumer_cus_chosen_by": "option" if args.consumer_cus else "the launch (routing + observed rates)",
                   "band_window": args.band_window or 4, "producer_order": "remote first",
                   "token_rows_landed_by": "the FFN launch" if land else "the layout's gather kernel",
                   "mode": {0: "overlapped", 1: "sequential", 3: "DMA return"}[args.mode]},
        "pct_bf16_peak_step": round(100 * value / peak, 2),
        "ffn_tflops_overlapped": round(ffn_tflops, 2),
        "pct_bf16_peak_ffn": round(100 * ffn_tflops / peak, 2),
        "overlap_ratio_pct": round(100 * ratio, 2),
        "ffn_ms_overlapped": [round(v, 4) for v in t_ovl],
        # the FFN call that also lands the token rows (the timed steps' form when the launch lands them)
        "ffn_ms_overlapped_landing": [round(v, 4) for v in t_land] if t_land else None,
        "ffn_ms_sequential": [round(v, 4) for v in t_seq],
        "speedup_seq_over_ovl": round(t_seq[0] / t_ovl[0], 4),
        "copy_ms_sequential": round(copy_seq_ms, 4),
        "copy_gbs_sequential": round(copy_bytes / (copy_seq_ms * 1e-3) / 1e9, 1),
        "copy_pct_hbm_peak_sequential": round(100 * copy_bytes / (copy_seq_ms * 1e-3) / 8e12, 2),
        # the overlapped return over the window it took (first copy start to last copy end), and what share of the
        # sequential return's time the overlapped call saved
        "copy_gbs_overlapped_window": round(copy_bytes / (o_med["copy_window_us"] * 1e-6) / 1e9, 1)
        if o_med["copy_window_us"] > 0 else None,
        "hidden_fraction_of_sequential_copy": round((t_seq[0] - t_ovl[0]) / copy_seq_ms, 3) if copy_seq_ms > 0 else None,
        # sequential = the FFN launch on every CU, then the return alone on every CU: its two parts, and what the
        # overlapped launch saves against their sum (medians)
        "sequential_parts_ms": {"ffn": round(s1 / sn, 4), "return": round(copy_seq_ms, 4)},
        "saved_vs_sequential_us": round(1e3 * (t_seq[0] - t_ovl[0]), 1),
        "timestamps_us": {k: round(v, 2) for k, v in o_med.items()},
        "kernel_ms_avg": {"ffn_producer_launch": round(g1_avg, 4), "second_launch": round(g2_avg, 4),
                          "consumer_alone_seq": round(s1 and sc_ms / sn, 4)},
        "executed_mfma_tflop": round(executed / 1e12, 4),
        "executed_over_useful_pct": round(100.0 * (executed - useful) / useful, 2),
        "layout_padding_pct": round(100.0 * (M_pad - M_real) / max(M_real, 1), 2),
        "observed_rates": {"producer_tflops_per_cu": round(part[1] * 1e8 / 1e12, 4),
                           "consumer_copy_gbs_per_cu": round(part[2] * 1e8 / 1e9, 2), "valid": part[3]},
        "ffn_ms_dma_return": [round(v, 4) for v in t_dma] if t_dma else None,
        "roofline": {"bound": "mfma",
                     "kernel": ("k_ffn_bf16: whole expert FFN in one persistent launch (gate/up + SwiGLU, "
                                "down projection with split-K, flag publish; the return inside)"
                                if s.dtype == "bf16" else "k_gemm<float> first GEMM"),
                     "achieved": round(roof_flops / (g1_avg * 1e-3) / 1e12, 2), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(roof_flops / (g1_avg * 1e-3) / 1e12 / peak, 4),
                     "traffic": hbm_traffic(s, cus, args.band_window, land, args.mode),
                     "traffic_unit": "HBM bytes per launch"},
    }
    if args.backward and s.dtype == "bf16":
        res["backward"] = bench_backward(
            P, s, w1, w2, reps, M_real,
            lambda g: P.ffn(w1, w2, mode=0, consumer_cus=cus, band_window=args.band_window,
                            x_tokens=dev["x"] if land else None, gu_out=g))
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(s, inp, args.cpu_seconds)
    print(json.dumps(res))


if __name__ == "__main__":
    main()
