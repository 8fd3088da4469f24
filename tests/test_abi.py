"""The C-ABI library loads and exports every entry point its header declares; host-only helpers (sizes,
workspace carving, argument checks) behave as documented.  No kernel is launched here."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
from expert_output_overlap_amd import binding as B

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "moe_overlap.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(moe_[a-z_0-9]+)\s*\(", src, flags=re.M)))


def test_library_exports_every_declared_symbol():
    lib = B.lib()
    names = declared_functions()
    assert len(names) >= 11
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(B.EXPORTS) == names


def test_version():
    assert "gfx950" in B.moe_version()


def shape(**kw):
    base = dict(R=4, tokens_per_owner=1024, num_global_experts=8, num_local_experts=2, top_k=2, self_rank=0, d=4096,
                f=14336, tile_m=128, seg_bands=1, dtype=B.MOE_BF16)
    base.update(kw)
    return B.moe_shape(**base)


@pytest.mark.parametrize("kw", [dict(), dict(R=8, tokens_per_owner=2048, num_global_experts=256, num_local_experts=32,
                                            top_k=8, d=7168, f=2048), dict(tile_m=64, top_k=6, num_local_experts=16,
                                                                           num_global_experts=64)])
def test_capacity_matches_bound(kw):
    s = shape(**kw)
    cap = B.moe_layout_capacity_rows(s)
    assert cap == oracle.capacity_rows(s.R, s.tokens_per_owner, s.num_local_experts, s.top_k, s.tile_m)


def _tail_fits(n_cu, m_ret, d, n_g1, ffn_rate=31250.0, copy_rate=450.0):
    """The rule's no-partition test, restated: the workgroups without a first-GEMM item in the last, partly filled,
    round copy the returned rows (4 d bytes each, at 50000 bytes per tick or their own rate if lower) within one
    first-GEMM item's time (2 x 256 x 256 x d flops at the producers' rate)."""
    q1 = n_g1 % n_cu
    if q1 == 0 or m_ret == 0:
        return m_ret == 0
    return 4.0 * m_ret * d / min(50000.0, (n_cu - q1) * copy_rate) <= 2.0 * 256 * 256 * d / ffn_rate


@pytest.mark.parametrize("kw,want", [
    (dict(), 8),                                                       # f = 14336
    (dict(tokens_per_owner=4096, num_global_experts=8, num_local_experts=2, f=4096), 8),
    (dict(R=8, tokens_per_owner=2048, num_global_experts=256, num_local_experts=32, top_k=8, d=7168, f=2048), 16),
    (dict(tokens_per_owner=2048, num_global_experts=64, num_local_experts=16, top_k=6, d=2048, f=1408,
          tile_m=64), 16),
    (dict(d=64, f=128, tile_m=16), 32),                                # capped at 32
    (dict(d=64, f=128, tile_m=16, dtype=B.MOE_F32), 8),
])
def test_consumer_partition_pick(kw, want):
    """The shape-only partition estimate: the launch's rule with default rates, R - 1 of every R of a nominal 10^6
    rows returned, in full row tiles.  So many returned rows never fit in the round-robin's slack, so the pick is the
    partition: the smallest multiple of 8 at which the consumers alone return the rows in half the FFN's time, within
    [8, min(32, CUs/4)]; a device with under 32 CUs takes a quarter of them."""
    s = shape(**kw)
    c = B.moe_pick_consumer_cus(s, 256)
    assert c == want
    if s.dtype == B.MOE_BF16:
        ratio = lambda c: 4.0 * (s.R - 1) / s.R * 31250.0 * (256 - c) / (6.0 * 450.0 * c * s.f)
        assert ratio(c) <= 0.5 or c == 32
        assert c == 8 or ratio(c - 8) > 0.5
        m = 10 ** 6
        n1 = s.f // (128 if s.f % 128 == 0 else 64)
        assert not _tail_fits(256, m * (s.R - 1) // s.R, s.d, (m + 255) // 256 * n1)
    assert B.moe_pick_consumer_cus(s, 16) == 4   # a quarter of a small device's CUs
    assert B.moe_pick_consumer_cus(s, 4) == 1
    assert B.moe_pick_consumer_cus(s, 1) == -1
    assert B.moe_pick_consumer_cus(shape(f=0), 256) == -1


@pytest.mark.parametrize("bad", [dict(R=0), dict(R=17), dict(d=96), dict(f=0), dict(tile_m=24), dict(tile_m=272),
                                 dict(top_k=0), dict(top_k=9), dict(num_local_experts=3), dict(self_rank=4),
                                 dict(dtype=7), dict(seg_bands=0), dict(tokens_per_owner=-1),
                                 dict(num_local_experts=65, num_global_experts=130)])
def test_invalid_shapes_rejected(bad):
    s = shape(**bad)
    assert B.moe_layout_capacity_rows(s) == -1
    assert B.moe_layout_workspace_bytes(s) == -1
    assert B.moe_ffn_flags_count(s) == -1
    L = B.moe_layout()
    buf = np.zeros(1 << 16, np.uint8)
    assert B.lib().moe_layout_bind(ctypes.byref(s), ctypes.c_void_p(buf.ctypes.data), buf.size,
                                   ctypes.byref(L)) == B.MOE_EINVAL
    assert B.moe_last_error() != ""


def test_bind_carves_disjoint_aligned_arrays():
    s = shape(R=3, tokens_per_owner=300, num_global_experts=12, num_local_experts=4, d=256, f=512, tile_m=32)
    nbytes = B.moe_layout_workspace_bytes(s)
    buf = np.zeros(nbytes + 512, np.uint8)
    base = (buf.ctypes.data + 255) // 256 * 256
    L = B.moe_layout()
    lib = B.lib()
    assert lib.moe_layout_bind(ctypes.byref(s), ctypes.c_void_p(base), nbytes - 1, ctypes.byref(L)) == B.MOE_EINVAL
    assert lib.moe_layout_bind(ctypes.byref(s), ctypes.c_void_p(base + 4), nbytes, ctypes.byref(L)) == B.MOE_EINVAL
    assert lib.moe_layout_bind(ctypes.byref(s), ctypes.c_void_p(base), nbytes, ctypes.byref(L)) == B.MOE_OK
    NG = s.num_local_experts * s.R
    T = s.R * s.tokens_per_owner
    sizes = {"counts": NG, "padded_off": NG, "recv_off": NG, "tile_owner": L.cap_tiles, "tile_expert": L.cap_tiles,
             "tile_valid": L.cap_tiles, "tile_order": L.cap_tiles, "seg_desc": 8 * L.cap_tiles,
             "row_src": L.cap_rows, "combine_plan": T * s.top_k, "scalars": 4 + s.R, "status": 1,
             "mtile_desc": 264 * L.cap_mtiles, "seg_mtiles": 2 * L.cap_tiles, "seg_sched": L.cap_tiles,
             "chunk_counts": s.R * ((s.tokens_per_owner + 63) // 64) * s.num_local_experts}
    spans = sorted((getattr(L, n) - base, getattr(L, n) - base + 4 * sizes[n], n) for n in sizes)
    for (a0, a1, n), (b0, b1, m) in zip(spans, spans[1:]):
        assert a1 <= b0, (n, m)
    assert spans[0][0] >= 0 and spans[-1][1] <= nbytes
    assert all(a % 256 == 0 for a, _, _ in spans)
    assert L.cap_tiles * s.tile_m == L.cap_rows


def test_flag_count_covers_row_tiles():
    s = shape()
    L = B.moe_layout()
    nbytes = B.moe_layout_workspace_bytes(s)
    buf = np.zeros(nbytes + 256, np.uint8)
    base = (buf.ctypes.data + 255) // 256 * 256
    assert B.lib().moe_layout_bind(ctypes.byref(s), ctypes.c_void_p(base), nbytes, ctypes.byref(L)) == 0
    nflags = B.moe_ffn_flags_count(s)
    n_nt2 = s.d // 256  # 256-wide output tiles of the second GEMM
    assert nflags >= L.cap_mtiles * n_nt2
    # f = 3.5 d: the second GEMM's tiles are split 4 ways over k, and the four splits' fp32 partial 256 x 256
    # tiles per output tile live in the same buffer
    assert nflags >= L.cap_mtiles * n_nt2 * (1 + 4 * 256 * 256)
    # an fp32 shape has one flag per output tile of the second GEMM (64 wide), then (64-word aligned) the
    # return's 64-bit copy-unit counter
    sf = shape(dtype=B.MOE_F32, d=256, f=512)
    Lf = B.moe_layout()
    nb = B.moe_layout_workspace_bytes(sf)
    buf2 = np.zeros(nb + 256, np.uint8)
    base2 = (buf2.ctypes.data + 255) // 256 * 256
    assert B.lib().moe_layout_bind(ctypes.byref(sf), ctypes.c_void_p(base2), nb, ctypes.byref(Lf)) == 0
    assert B.moe_ffn_flags_count(sf) == (Lf.cap_mtiles * (256 // 64) + 63) // 64 * 64 + 2


def _cap_mtiles(s):
    L = B.moe_layout()
    nbytes = B.moe_layout_workspace_bytes(s)
    buf = np.zeros(nbytes + 256, np.uint8)
    base = (buf.ctypes.data + 255) // 256 * 256
    assert B.lib().moe_layout_bind(ctypes.byref(s), ctypes.c_void_p(base), nbytes, ctypes.byref(L)) == 0
    return L.cap_mtiles


def test_backward_flag_count():
    """The backward's flag buffer holds a flag per dX, dH and h / dG / dU tile, the k-split arrival counters, the
    split-K partial sums (4 splits where f = 3.5 d, none where f < d), the copy-unit and weight-gradient counters;
    fp32 shapes and f not a multiple of 128 have no backward."""
    s = shape(d=4096, f=14336)
    cap = _cap_mtiles(s)
    n = B.moe_bwd_flags_count(s)
    n_x, n_h, n_g = 4096 // 256, 14336 // 256, 14336 // 128
    assert n >= cap * (n_x + n_h + n_g + 2 * n_x) + cap * n_x * 4 * 256 * 256 + 4
    assert n < cap * (n_x + n_h + n_g + 2 * n_x) + cap * n_x * 5 * 256 * 256  # 4 splits, not more
    s1 = shape(d=7168, f=2048)
    cap1 = _cap_mtiles(s1)
    n1 = B.moe_bwd_flags_count(s1)
    assert cap1 * (7168 // 256 + 2048 // 256 + 2048 // 128) <= n1 < cap1 * 256 * 256  # no partial sums
    assert B.moe_bwd_flags_count(shape(d=256, f=192)) == -1
    assert B.moe_bwd_flags_count(shape(dtype=B.MOE_F32, d=256, f=512)) == -1


CSRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "expert_output_overlap_amd", "csrc")


def test_inline_asm_carries_its_wait_states():
    """The compiler inserts hazard wait states only around instructions it emits itself, so every inline-assembly
    statement that needs them carries its own: a store wider than 8 bytes is followed by two wait states before
    its data registers may be rewritten (s_nop 1), and every SALU write of M0 by one (s_nop), which the LDS-DMA
    load that reads M0 needs.  M0 is a reserved register that a clobber list may not name, so a statement that
    writes M0 first saves it in an output register and writes the saved value back as its last M0 write."""
    found = {"store": 0, "m0": 0}
    for fn in sorted(os.listdir(CSRC)):
        if not fn.endswith((".hip", ".h", ".cpp")):
            continue
        src = open(os.path.join(CSRC, fn)).read()
        for stmt in re.findall(r'asm\s+volatile\s*\(\s*((?:"[^"]*"\s*)+)', src):
            text = "".join(re.findall(r'"([^"]*)"', stmt)).replace("\\n", "\n").replace("\\t", " ")
            ins = [l.strip() for l in text.split("\n") if l.strip()]
            assert not re.search(r'"m0"', src[src.index(stmt):src.index(stmt) + len(stmt) + 400].split(";")[0]), \
                (fn, "M0 named in a clobber list")
            m0_writes = [i for i, op in enumerate(ins) if re.match(r"s_mov_b32\s+m0\s*,", op)]
            for i, op in enumerate(ins):
                if re.match(r"(global|buffer|flat)_store_dwordx(3|4)\b", op):
                    found["store"] += 1
                    assert i + 1 < len(ins) and re.match(r"s_nop\s+[1-9]", ins[i + 1]), (fn, text)
                if "_lds_" in op or op.endswith(" lds"):
                    # the LDS-DMA load reads the M0 set before it, one wait state after that write
                    assert any(w + 1 < i and ins[w + 1].startswith("s_nop") for w in m0_writes), (fn, text)
            if m0_writes:
                found["m0"] += 1
                save = re.match(r"s_mov_b32\s+(%\d+)\s*,\s*m0$", ins[0])
                assert save, (fn, "M0 not saved first", text)
                last = ins[m0_writes[-1]]
                assert re.match(r"s_mov_b32\s+m0\s*,\s*" + re.escape(save.group(1)) + r"$", last), (fn, text)
                for w in m0_writes:
                    assert w + 1 < len(ins) and ins[w + 1].startswith("s_nop"), (fn, text)
    assert found["store"] >= 1 and found["m0"] >= 1, found


def test_full_size_parity_runs_in_the_bench_configuration():
    """The full-size GPU parity tests use the consumer partition that bench.py times by default."""
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    bench = open(os.path.join(root, "bench.py")).read()
    m = re.search(r'"--consumer-cus", type=int, default=(\d+)', bench)
    tests = open(os.path.join(root, "tests", "test_gpu_path.py")).read()
    t = re.search(r"^BENCH_CONSUMER_CUS = (\d+)", tests, re.M)
    assert m and t and int(m.group(1)) == int(t.group(1))


def test_partition_rule():
    """The consumer-partition rule (the launch's own code, compiled for the host).  No partition (0) when nothing is
    returned, or when the first-GEMM items fill their last round over the CUs only in part and the workgroups left
    without one copy the returned rows within one first-GEMM item's time; else the partition: more returned rows or a
    faster FFN take more consumer CUs, multiples of 8 within [8, min(32, CUs / 4)]; defaults for rates <= 0."""
    s = shape(d=2048, f=1408, R=4)
    n1 = 1408 // 128
    pick = lambda routed, ret, n_mt, fr=0.0, cr=0.0, n=256: B.moe_pick_consumer_cus_observed(s, n, routed, ret, n_mt,
                                                                                              fr, cr)
    assert pick(15000, 0, 60) == 0
    # 60 row tiles x 11 = 660 first-GEMM items: 148 in the last round over 256 CUs, 108 workgroups free
    assert 660 % 256 == 148 and _tail_fits(256, 3000, 2048, 660) and pick(15000, 3000, 60) == 0
    assert not _tail_fits(256, 60000, 2048, 660) and pick(65536, 60000, 60) in (8, 16, 24, 32)
    # full rounds (256 row tiles x 11 = 2816 = 11 x 256): no slack, a partition whatever is returned
    assert pick(65536, 100, 256) == 8 and not _tail_fits(256, 100, 2048, 2816)
    vals = [pick(15000, r, 256) for r in (3000, 6000, 9000, 12000, 15000)]
    assert vals == sorted(vals) and vals[-1] > vals[0] and all(v % 8 == 0 and 8 <= v <= 32 for v in vals)
    assert pick(15000, 15000, 256, cr=100.0) > pick(15000, 15000, 256, cr=450.0) > pick(15000, 15000, 256, cr=2000.0)
    assert pick(15000, 12000, 256, fr=60000.0) >= pick(15000, 12000, 256, fr=31250.0)
    assert pick(15000, 12000, 60, 0.0, 0.0) == pick(15000, 12000, 60, 31250.0, 450.0)
    assert pick(15000, 15000, 256, cr=1.0, n=64) == 16  # capped at a quarter of the CUs
    # the workloads as routed: the Mixtral-like and DeepSeek-V3-like shards return within the slack; d = f = 4096
    # with one expert fills its first-GEMM rounds
    mix = shape()
    assert B.moe_pick_consumer_cus_observed(mix, 256, 2043, 1510, 9, 0.0, 0.0) == 0
    ds = shape(R=8, tokens_per_owner=2048, num_global_experts=256, num_local_experts=32, top_k=8, d=7168, f=2048)
    assert B.moe_pick_consumer_cus_observed(ds, 256, 24232, 21203, 114, 0.0, 0.0) == 0
    sw1 = shape(tokens_per_owner=4096, num_global_experts=4, num_local_experts=1, d=4096, f=4096)
    assert B.moe_pick_consumer_cus_observed(sw1, 256, 8181, 6076, 32, 0.0, 0.0) == 8
    assert pick(100, 200, 1) == -1 and pick(100, 50, -1) == -1


def test_landing_rejected_where_it_does_not_apply():
    """The launch lands token rows (cfg.x_tokens) for bf16 in modes 0 and 1 only; the call rejects the rest before
    any device work."""
    for dtype, mode in ((B.MOE_F32, 0), (B.MOE_BF16, 2), (B.MOE_BF16, 3)):
        s = shape(dtype=dtype, d=256, f=512)
        nbytes = B.moe_layout_workspace_bytes(s)
        buf = np.zeros(nbytes + 256, np.uint8)
        base = (buf.ctypes.data + 255) // 256 * 256
        L = B.moe_layout()
        assert B.lib().moe_layout_bind(ctypes.byref(s), ctypes.c_void_p(base), nbytes, ctypes.byref(L)) == 0
        fake = np.zeros(64, np.uint64)  # never dereferenced: the call fails its checks first
        p = ctypes.c_void_p(fake.ctypes.data)
        recv = (ctypes.c_void_p * s.R)(*([fake.ctypes.data] * s.R))
        cfg = B.moe_overlap_cfg(4, mode, 1, 0, 0, None, 0, fake.ctypes.data)
        rc = B.lib().moe_expert_ffn_overlap(ctypes.byref(s), ctypes.byref(L), p, p, p, p, p, recv, p,
                                            ctypes.byref(cfg), None)
        assert rc == B.MOE_EINVAL and "x_tokens" in B.moe_last_error(), (dtype, mode, B.moe_last_error())


def test_preactivation_store_rejected_where_the_backward_cannot_take_it():
    """The forward stores g | u (cfg.gu_out) for bf16 shapes with f a multiple of 128 in modes 0, 1 and 3 only, and
    the backward takes them through its argument struct, not its cfg; both calls reject the rest before any device
    work."""
    fake = np.zeros(64, np.uint64)  # never dereferenced: the calls fail their checks first
    p = ctypes.c_void_p(fake.ctypes.data)
    for dtype, f, mode in ((B.MOE_F32, 512, 0), (B.MOE_BF16, 192, 0), (B.MOE_BF16, 512, 2)):
        s = shape(dtype=dtype, d=256, f=f)
        nbytes = B.moe_layout_workspace_bytes(s)
        buf = np.zeros(nbytes + 256, np.uint8)
        base = (buf.ctypes.data + 255) // 256 * 256
        L = B.moe_layout()
        assert B.lib().moe_layout_bind(ctypes.byref(s), ctypes.c_void_p(base), nbytes, ctypes.byref(L)) == 0
        recv = (ctypes.c_void_p * s.R)(*([fake.ctypes.data] * s.R))
        cfg = B.moe_overlap_cfg(4, mode, 1, 0, 0, None, 0, None, fake.ctypes.data)
        rc = B.lib().moe_expert_ffn_overlap(ctypes.byref(s), ctypes.byref(L), p, p, p, p, p, recv, p,
                                            ctypes.byref(cfg), None)
        assert rc == B.MOE_EINVAL and "gu_out" in B.moe_last_error(), (dtype, f, mode, B.moe_last_error())
    s = shape(d=256, f=512)
    nbytes = B.moe_layout_workspace_bytes(s)
    buf = np.zeros(nbytes + 256, np.uint8)
    base = (buf.ctypes.data + 255) // 256 * 256
    L = B.moe_layout()
    assert B.lib().moe_layout_bind(ctypes.byref(s), ctypes.c_void_p(base), nbytes, ctypes.byref(L)) == 0
    recv = (ctypes.c_void_p * s.R)(*([fake.ctypes.data] * s.R))
    args = B.moe_bwd_args(**{k: (ctypes.cast(recv, ctypes.c_void_p) if k == "dx_recv" else p) for k in B.BWD_FIELDS})
    cfg = B.moe_overlap_cfg(0, 0, 1, 0, 0, None, 0, None, fake.ctypes.data)
    rc = B.lib().moe_expert_ffn_backward(ctypes.byref(s), ctypes.byref(L), ctypes.byref(args), p, ctypes.byref(cfg),
                                         None)
    assert rc == B.MOE_EINVAL and "gu_out" in B.moe_last_error(), B.moe_last_error()
