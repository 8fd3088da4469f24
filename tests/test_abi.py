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


@pytest.mark.parametrize("kw,c_copy,want", [
    # (kw, the partition the consumers' copy rate asks for, the pick)
    (dict(), 8, 0),                                                    # f = 14336
    (dict(tokens_per_owner=4096, num_global_experts=8, num_local_experts=2, f=4096), 8, 0),
    (dict(R=8, tokens_per_owner=2048, num_global_experts=256, num_local_experts=32, top_k=8, d=7168, f=2048), 16, 0),
    (dict(tokens_per_owner=2048, num_global_experts=64, num_local_experts=16, top_k=6, d=2048, f=1408,
          tile_m=64), 16, 0),
    (dict(d=64, f=128, tile_m=16), 32, 32),                            # capped at 32; the tail return costs more
    (dict(d=64, f=128, tile_m=16, dtype=B.MOE_F32), 8, 8),
])
def test_consumer_partition_pick(kw, c_copy, want):
    """The shape-only partition estimate: the launch's rule with default rates and R - 1 of every R rows returned.
    The partition size is the smallest multiple of 8 at which the consumers alone return the rows in half the FFN's
    time, within [8, min(32, CUs/4)]; the pick is 0 (no partition, the return at the launch's tail) when the chip
    copies the rows in less time than those CUs add to the FFN; a device with under 32 CUs takes a quarter of them."""
    s = shape(**kw)
    c = B.moe_pick_consumer_cus(s, 256)
    assert c == want
    if s.dtype == B.MOE_BF16:
        ratio = lambda c: 4.0 * (s.R - 1) / s.R * 31250.0 * (256 - c) / (6.0 * 450.0 * c * s.f)
        assert ratio(c_copy) <= 0.5 or c_copy == 32
        assert c_copy == 8 or ratio(c_copy - 8) > 0.5
        m = 1e6  # the rule's nominal rows
        tail = 4.0 * m * (s.R - 1) / s.R * s.d / 50000.0
        ffn0 = 6.0 * m * s.d * s.f / (256 * 31250.0)
        assert (tail <= ffn0 * c_copy / (256 - c_copy)) == (want == 0)
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
    """The consumer-partition rule (the launch's own code, compiled for the host): more returned rows take more
    consumer CUs, a faster FFN too; nothing to return, or a return cheaper at the launch's tail than the CUs
    a partition takes, takes none (0); otherwise multiples of 8 within [8, min(32, CUs / 4)]; defaults for rates <= 0."""
    s = shape(d=2048, f=1408, R=4)
    pick = lambda routed, ret, fr=0.0, cr=0.0, n=256: B.moe_pick_consumer_cus_observed(s, n, routed, ret, fr, cr)
    assert pick(15000, 0) == 0
    vals = [pick(15000, r) for r in (0, 3000, 6000, 9000, 12000, 15000)]
    assert vals == sorted(vals) and vals[0] == 0 and vals[-1] >= 16
    assert all(v == 0 or (v % 8 == 0 and 8 <= v <= 32) for v in vals)
    # the tail return against the partition, by the rule's own terms: 4 d bytes per returned row over the chip at
    # 50000 bytes per tick, against the c CUs' share of 6 d f flops per routed row at the default rate
    tail = lambda ret: 4.0 * ret * 2048 / 50000.0
    ffn0 = 6.0 * 15000 * 2048 * 1408 / (256 * 31250.0)
    assert pick(15000, 15000) == 16 and tail(15000) > ffn0 * 16 / 240
    assert pick(15000, 3000) == 0 and tail(3000) <= ffn0 * 8 / 248
    # the Mixtral-like and DeepSeek-V3-like shards return less than that costs: no partition
    mix = shape()
    assert B.moe_pick_consumer_cus_observed(mix, 256, 2048, 1536, 0.0, 0.0) == 0
    ds = shape(R=8, tokens_per_owner=2048, num_global_experts=256, num_local_experts=32, top_k=8, d=7168, f=2048)
    assert B.moe_pick_consumer_cus_observed(ds, 256, 24232, 21203, 0.0, 0.0) == 0
    # slower copies take more consumers (where the return stays with a partition: faster copies also make a small
    # partition cheaper than the tail return, so they can turn a pick of 0 into 8)
    assert pick(15000, 15000, cr=100.0) > pick(15000, 15000, cr=450.0) > pick(15000, 15000, cr=2000.0) == 8
    assert pick(15000, 12000, cr=450.0) == 0 and pick(15000, 12000, cr=2000.0) == 8
    assert pick(15000, 12000, fr=60000.0) >= pick(15000, 12000, fr=31250.0)
    assert pick(15000, 12000, 0.0, 0.0) == pick(15000, 12000, 31250.0, 450.0)
    assert pick(15000, 15000, cr=1.0, n=64) == 16  # capped at a quarter of the CUs
    # the shape-only estimate is the rule with 3 of 4 owners' rows returned and default rates
    assert B.moe_pick_consumer_cus(s, 256) == pick(4000, 3000)
    assert pick(100, 200) == -1


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
