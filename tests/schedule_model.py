"""The FFN launch's work-item list, checked on the CPU.

``packing`` models how the layout cuts real rows into GEMM row tiles (each expert's groups together, the other
owners' groups by decreasing padded size then owner, the self-owned group last; tiles of 256 rows), and the
producer's row-tile order (every tile holding another owner's row by number, then the self-owned-only tiles).  The
GPU tests pin this model to the tables the device builds.  ``check_list`` takes the list the library reports
(``moe_ffn_schedule``, the kernel's own code) and checks what the launch relies on.
"""
import numpy as np

TILE_ROWS = 256


def packing(counts: np.ndarray, padded_off: np.ndarray, R: int, E: int, self_rank: int, M: int):
    """Row tiles of the layout: (headers [n, 4] = expert, rows, run_first, run_count; rows per tile (padded
    positions); pure-self flag per tile; the producer's order [n])."""
    hdr, tile_rows, pure = [], [], []
    for e in range(E):
        groups = [e * R + r for r in range(R) if counts[e * R + r] > 0]
        P = {g: -(-counts[g] // M) * M for g in groups}
        remote = sorted([g for g in groups if g % R != self_rank], key=lambda g: (-P[g], g % R))
        selfg = [g for g in groups if g % R == self_rank]
        rows = np.concatenate([padded_off[g] + np.arange(counts[g]) for g in remote + selfg]) if groups else []
        nself = sum(counts[g] for g in selfg)
        if len(rows) == 0:
            continue
        first, cnt = len(hdr), -(-len(rows) // TILE_ROWS)
        for t in range(cnt):
            rr = rows[t * TILE_ROWS:(t + 1) * TILE_ROWS]
            hdr.append((e, len(rr), first, cnt))
            tile_rows.append(np.asarray(rr))
            pure.append(t * TILE_ROWS >= len(rows) - nself)
    pure = np.array(pure, dtype=bool)
    order = np.concatenate([np.nonzero(~pure)[0], np.nonzero(pure)[0]]).astype(np.int32)
    return np.array(hdr, dtype=np.int32).reshape(-1, 4), tile_rows, pure, order


def list_params(d: int, f: int):
    bn1 = 256 if f % 128 == 0 else 128
    bn2 = 256 if d % 256 == 0 else (128 if d % 128 == 0 else 64)
    n1, n2 = f // (bn1 // 2), d // bn2
    want = min(8, max(1, (2 * f + d) // (2 * d)))
    S = 1
    for c in range(want, 1, -1):
        if n1 % c == 0 and (f // 64) % c == 0:
            S = c
            break
    return n1, n2, S


def check_list(items: np.ndarray, n_mt: int, d: int, f: int, pure: np.ndarray):
    """Properties of the launch's item list ``items`` [n, 8] = {workgroup, seq, kind, mt, nt, s, half, target}."""
    n1, n2, S = list_params(d, f)
    per = n1 // S
    idx_of = {}
    for i, (wg, seq, kind, mt, nt, s, half, target) in enumerate(items):
        key = (int(kind), int(mt), int(nt), int(s), int(half))
        assert key not in idx_of, ("item listed twice", key)
        idx_of[key] = i
    # every item exactly once: every h tile, and every split of every y tile (whole, or both of its halves)
    for mt in range(n_mt):
        for nt in range(n1):
            assert (1, mt, nt, 0, -1) in idx_of, ("missing GEMM1 item", mt, nt)
        for nt in range(n2):
            for s in range(S):
                whole = (2, mt, nt, s, -1) in idx_of
                halves = (2, mt, nt, s, 0) in idx_of and (2, mt, nt, s, 1) in idx_of
                assert whole != halves, ("split listed neither whole nor as two halves", mt, nt, s)
    assert len(idx_of) == len(items)
    kind, mt, nt, s, half, target = (items[:, j] for j in range(2, 8))
    # each workgroup runs its items in increasing list order
    for wg in np.unique(items[:, 0]):
        m = np.nonzero(items[:, 0] == wg)[0]
        assert (np.diff(m) > 0).all() and (items[m, 1] == np.arange(m.size)).all()
    # every GEMM2 item waits only on GEMM1 items earlier in the list (its split's h column tiles)
    waits = {}
    for i in np.nonzero(kind == 2)[0]:
        w = [idx_of[(1, int(mt[i]), c, 0, -1)] for c in range(int(s[i]) * per, (int(s[i]) + 1) * per)]
        assert max(w) < i, ("wait on a later item", i)
        waits[i] = w
    # the number of items that count themselves in at a y tile equals the target each of them carries
    tiles = {}
    for i in np.nonzero(kind == 2)[0]:
        tiles.setdefault((int(mt[i]), int(nt[i])), []).append(i)
    for key, its in tiles.items():
        tg = set(int(target[i]) for i in its)
        assert tg == {len(its)}, ("arrival target", key, tg, len(its))
    # remote first: every GEMM2 item of a self-owned-only row tile after every GEMM2 item of the other row tiles
    g2 = kind == 2
    if pure.any() and (~pure).any():
        last_remote = np.nonzero(g2 & ~pure[mt])[0].max()
        first_self = np.nonzero(g2 & pure[mt])[0].min()
        assert last_remote < first_self, ("remote-first order", last_remote, first_self)
    return waits


def simulate(items: np.ndarray, waits: dict, claim_halves: bool = False, seed: int = 0):
    """Runs the list as the launch does: each workgroup takes its items in order, an item runs once the items it waits
    on have finished, and items take random positive times.  With claim_halves, the half-width items are not
    assigned statically but taken from a counter, in list order, by whichever workgroup is free first.  Returns the
    finish order; fails if the run stops with items left (a wait that never ends)."""
    rng = np.random.default_rng(seed)
    n = len(items)
    halves = np.nonzero(items[:, 6] >= 0)[0] if claim_halves else np.zeros(0, int)
    is_half = np.zeros(n, bool)
    is_half[halves] = True
    queues = {}
    for i in range(n):
        if not is_half[i]:
            queues.setdefault(int(items[i, 0]), []).append(i)
    wgs = sorted(set(int(w) for w in items[:, 0]))
    for w in wgs:
        queues.setdefault(w, [])
    done = np.zeros(n, bool)
    busy_until = {w: 0.0 for w in wgs}
    running = {}
    claim = 0
    t = 0.0
    order = []
    while not done.all():
        progressed = False
        for w in wgs:
            if w in running:
                continue
            q = queues[w]
            if not q and claim < len(halves):  # a free workgroup takes the next half from the counter
                q.append(int(halves[claim]))
                claim += 1
            if q and all(done[j] for j in waits.get(q[0], [])):
                i = q.pop(0)
                running[w] = i
                busy_until[w] = t + rng.uniform(0.5, 1.5)
                progressed = True
        if not running:
            assert progressed, "no workgroup can run: %d items left" % int((~done).sum())
            continue
        w = min(running, key=lambda k: busy_until[k])
        t = busy_until[w]
        i = running.pop(w)
        done[i] = True
        order.append(i)
    return order
