// The work-item list of the fused bf16 FFN launch (review page: "Core claim" and "What carries the argument": one
// rank-wide persistent GEMM whose tiles are scheduled remote-bound first).  Shared, as __host__ __device__ code, by
// the kernel (ffn.hip) and the host-side schedule entry point (moe_ffn_schedule), so that the list the tests check
// on the CPU is the one the GPU runs.
//
// Items: a GEMM1 item is (row tile mt, h column tile nt); a GEMM2 item is (row tile mt, y column tile nt, k-split
// s).  Row tiles are visited through positions: position p is row tile mt_order[p], every row tile that holds a
// row bound for another owner before every row tile that holds only self-owned rows (the layout builds the order).
// The list, by list index:
//  - GEMM1 first (interleave = 0): every GEMM1 item, expert by expert by row-tile number (each expert's row tiles are
//    one run; the descriptor gives its first tile and count), column-tile major inside an expert; then the GEMM2
//    items window by window over positions (windows of W positions).  With at most four windows, every window but
//    the first goes row tile by row tile (split-major inside a row tile); the others, and the first, split-major
//    then column-tile major over the window, so consecutive items share a down-projection weight tile.  The last
//    window, and every window from the one holding the first self-owned-only row tile on, go row tile by row tile.
//  - interleaved (interleave = 1): G1(0), G1(1), G2(0), G1(2), G2(1), ..., G1(nw-1), G2(nw-2), G2(nw-1), windows
//    over positions; the last two GEMM2 windows, and those from the first self-owned-only row tile on, row tile by
//    row tile.
// In both, every GEMM2 item follows the GEMM1 items it reads, and the last split of a y tile follows its others.
// Workgroups: the first C run the consumer role and first take kc GEMM1 items each from the head of the list; the
// G producer workgroups take the rest round-robin, producer b taking items C kc + b', C kc + b' + G, ... with b'
// remapped so that a run of consecutive items goes to one XCD (workgroup b sits on XCD b % 8).  When the producers'
// last round is at most half full and holds only GEMM2 items, each of its items becomes two half-width items
// (list indices >= i_tail, two per item).
#pragma once

#include <stdint.h>

#define MOE_HD __host__ __device__ inline

MOE_HD int li_min(int a, int b) { return a < b ? a : b; }

struct FfnList {
  int n_mt, n_nt1, n_nt2, S, W, interleave;  // row tiles, column tiles of GEMM1 / GEMM2, k-splits, window, order
  int n_rem;                                 // positions [0, n_rem) hold the row tiles with another owner's rows
  int C, G;                                  // consumer and producer workgroups
  int n_items, kc, i_tail, n_list;           // items, consumers' GEMM1 share, first half item, list length
};

// Interleave when the return is large next to the FFN and re-streaming weights is cheap.  At about 45 GB/s of copy
// per consumer CU and 0.8 PFLOP/s of FFN, copy time / FFN time = 4 M d / (45e9 C) / (6 M d f / 0.8e15)
// ~= 11850 / (C f), whatever M and d are; GEMM1 first leaves the last part of the launch for the copies, and the
// workgroups that finish early help with what is left, so it is used while that ratio stays under about 1/4.
// Interleaved windows stream an expert's weight tiles once per window holding its rows, and consecutive items share
// fewer of them, which pays only while the local experts' weights (3 d f per expert) take at most half of the
// 256 MB last-level cache; measured with d = f = 4096: one expert (100 MB) gains 4%, two (201 MB) lose 3%.
MOE_HD int ffn_interleave(int n_cons, int d, int f, int E) {
  const double w_bytes = 3.0 * d * (double)f * 2.0 * E;
  return n_cons > 0 && (int64_t)n_cons * f < 48000 && w_bytes <= 128.0 * 1024 * 1024;
}

MOE_HD FfnList ffn_list_make(int n_mt, int n_rem, int n_nt1, int n_nt2, int S, int W, int interleave, int C, int G,
                             bool halves) {
  FfnList L;
  L.n_mt = n_mt;
  L.n_rem = n_rem;
  L.n_nt1 = n_nt1;
  L.n_nt2 = n_nt2;
  L.S = S;
  L.W = W;
  L.interleave = interleave;
  L.C = C;
  L.G = G;
  L.n_items = n_mt * (n_nt1 + n_nt2 * S);
  // With every GEMM1 item first, no row tile is returned before the GEMM1 part of the list is done, so the
  // consumer workgroups first take kc GEMM1 items each from the head of the list: just enough that the producers'
  // share fits in as few rounds as the whole list would on all workgroups, and no more than the consumers finish
  // before the GEMM1 part ends.  GEMM1 items wait on nothing, so the consumers' later waits still end.
  L.kc = 0;
  if (C > 0 && interleave == 0) {
    const int rounds = (L.n_items + G + C - 1) / (G + C), over = L.n_items - rounds * G;
    L.kc = over > 0 ? (over + C - 1) / C : 0;
    L.kc = li_min(L.kc, n_mt * n_nt1 / (G + C));
  }
  // The producers' last round holds q items.  When they are GEMM2 items and at most half a round, each becomes two
  // items of half the tile width, so that the round keeps twice as many CUs busy (a half-width tile takes ~0.7 of
  // a full one's time).  Every output element is accumulated as before, so results do not change.
  L.i_tail = L.n_items;
  L.n_list = L.n_items;
  if (halves && L.n_items > C * L.kc) {
    const int np = L.n_items - C * L.kc, q = np - (np - 1) / G * G;
    const int nw = (n_mt + W - 1) / W, Wl = n_mt - (nw - 1) * W;
    const int g2_tail = interleave == 0 ? n_mt * n_nt2 * S : (Wl + (nw > 1 ? W : 0)) * n_nt2 * S;
    if (2 * q <= G && q <= g2_tail) {
      L.i_tail = L.n_items - q;
      L.n_list = L.n_items + q;
    }
  }
  return L;
}

// The list indices workgroup `block` runs: i0, i0 + step, ... while < i1.
MOE_HD void ffn_list_range(const FfnList& L, int block, int* i0, int* i1, int* step) {
  if (block < L.C) {
    *i0 = block * L.kc;
    *i1 = *i0 + L.kc;
    *step = 1;
    return;
  }
  int bid = block - L.C;
  if ((L.G & 7) == 0 && (L.C & 7) == 0) bid = (bid & 7) * (L.G >> 3) + (bid >> 3);
  *i0 = L.C * L.kc + bid;
  *i1 = L.n_list;
  *step = L.G;
}

struct FfnItem {
  int kind;    // 1: GEMM1 tile, 2: GEMM2 split
  int mt;      // row tile (its number, not its position)
  int nt, s;   // column tile; k-split (GEMM2)
  int half;    // -1, or which half-width half (GEMM2)
  int target;  // GEMM2: items that complete the y tile (its S splits and one more per halved split)
};

// Position part of the list (GEMM2 items, and GEMM1 items when interleaved): item i -> kind, position, nt, s, and
// the list distance between consecutive splits of the item's y tile.
struct FfnSlot {
  int kind, pos, nt, s, stride;
};

MOE_HD FfnSlot ffn_slot(int i, const FfnList& L) {
  const int n_mt = L.n_mt, W = L.W, n1 = L.n_nt1, n2 = L.n_nt2, S = L.S;
  const bool interleave = L.interleave != 0;
  const int n2S = n2 * S;
  const int nw = (n_mt + W - 1) / W;
  const bool by_tile = !interleave && nw <= 4;
  // the window holding the first self-owned-only row tile, and every later one, go row tile by row tile, so that
  // every item of a row tile with another owner's rows precedes every item of a self-owned-only one
  const int wb = L.n_rem < n_mt ? L.n_rem / W : nw;
  auto g1 = [&](int w, int j, int Wc) {  // GEMM1 item j of a window of Wc positions starting at w*W
    FfnSlot it;
    it.kind = 1;
    it.nt = j / Wc;
    it.pos = w * W + (j - it.nt * Wc);
    it.s = 0;
    it.stride = 0;
    return it;
  };
  auto g2 = [&](int w, int j, int Wc) {
    FfnSlot it;
    it.kind = 2;
    if ((by_tile && w >= 1) || w >= nw - (interleave ? 2 : 1) || w >= wb) {  // row tile by row tile
      const int ml = j / n2S, r = j - ml * n2S;
      it.s = r / n2;
      it.nt = r - it.s * n2;
      it.pos = w * W + ml;
      it.stride = n2;
      return it;
    }
    const int per = Wc * n2;  // split-major, then column-tile major
    it.s = j / per;
    const int r = j - it.s * per;
    it.nt = r / Wc;
    it.pos = w * W + (r - it.nt * Wc);
    it.stride = per;
    return it;
  };
  const int Wl = n_mt - (nw - 1) * W;
  if (!interleave) {  // i >= n_mt * n1
    const int j = i - n_mt * n1, w = j / (W * n2S);
    return w < nw - 1 ? g2(w, j - w * W * n2S, W) : g2(nw - 1, j - (nw - 1) * W * n2S, Wl);
  }
  const int W0 = nw == 1 ? Wl : W;
  if (i < W0 * n1) return g1(0, i, W0);
  i -= W0 * n1;
  if (nw == 1) return g2(0, i, Wl);
  const int pz = W * (n1 + n2S);  // a pair (G1(p), G2(p-1)) of two full windows, p = 1 .. nw-2
  if (i < (nw - 2) * pz) {
    const int p = 1 + i / pz, j = i - (p - 1) * pz;
    return j < W * n1 ? g1(p, j, W) : g2(p - 1, j - W * n1, W);
  }
  i -= (nw - 2) * pz;
  if (i < Wl * n1) return g1(nw - 1, i, Wl);
  i -= Wl * n1;
  if (i < W * n2S) return g2(nw - 2, i, W);
  return g2(nw - 1, i - W * n2S, Wl);
}

// List index `idx` (< n_list).  run_of(mt, &first, &count) gives the run of consecutive row tiles of mt's expert;
// order[p] the row tile at position p.
template <typename RunOf, typename OrderOf>
MOE_HD FfnItem ffn_list_item(const FfnList& L, int idx, RunOf run_of, OrderOf order) {
  FfnItem it;
  it.half = -1;
  int item = idx;
  if (item >= L.i_tail) {
    it.half = (item - L.i_tail) & 1;
    item = L.i_tail + ((item - L.i_tail) >> 1);
  }
  it.target = 1;
  if (L.interleave == 0 && item < L.n_mt * L.n_nt1) {
    // GEMM1 part with every GEMM1 item first: item i lies in the run of row tile i / n_nt1, since a run of c tiles
    // holds c * n_nt1 items
    int r0 = 0, rc = 1;
    run_of(item / L.n_nt1, &r0, &rc);
    const int j = item - r0 * L.n_nt1;
    it.kind = 1;
    it.nt = j / rc;
    it.mt = r0 + (j - it.nt * rc);
    it.s = 0;
    return it;
  }
  const FfnSlot sl = ffn_slot(item, L);
  it.kind = sl.kind;
  it.mt = order(sl.pos);
  it.nt = sl.nt;
  it.s = sl.s;
  if (sl.kind == 2) {
    // items that complete the y tile: its S splits, one more for each split that is halved
    const int last = item + (L.S - 1 - sl.s) * sl.stride;
    it.target = L.S;
    for (int sp = 0; sp < L.S; ++sp) it.target += last - (L.S - 1 - sp) * sl.stride >= L.i_tail;
  }
  return it;
}

// ---- the consumer partition, picked at run time -------------------------------------------------------------
// The review page ("If this is right": the overlap collapses with too few consumer SMs; "Where Pith is reading between
// the lines": size the partition at run time) leaves the size open.  The launch picks it itself, every workgroup
// identically, from this batch's routing (rows routed to the local experts and rows to return to other owners, from
// the layout) and from rates observed in earlier calls: the producers' flops per CU-tick and the consumers' copied
// bytes per CU-tick (100 MHz ticks).  The consumers have to return 4 d bytes per returned row (read and write, bf16)
// while the producers run 6 d f flops per routed row; copies can start only once row tiles complete, in about the
// second half of the launch, so the pick is the smallest multiple of 8 (the same count on each XCD) in [8, cmax] at
// which the consumers alone would finish the return in half the FFN's time; cmax = min(32, n_cu / 4) (a device with
// under 32 CUs: a quarter of them).  The pick is 0, no partition, when the return fits in the slack the producers'
// round-robin leaves anyway: when the first-GEMM items (n_g1, each 2 x 256 x 256 x d flops) fill their last round only
// in part, the workgroups without one run a whole first-GEMM item ahead of the others, and each takes copy units once
// its own items are done, so a return that those workgroups finish within one first-GEMM item's time runs behind the
// others' GEMM at no cost, and every CU produces.  On one device the return is a copy in HBM, at up to
// MOE_TAIL_COPY_RATE over the chip or the free CUs' copy rate if lower.  Measured: the DeepSeek-V3-like and
// Mixtral-like shards run 1-4% faster with the return hidden this way than with the best partition (100% of the copy
// inside the producers' span); with d = f = 4096 and one or two experts the first-GEMM rounds are full, the copy
// would run after the GEMM (8-24% hidden), and a partition keeps it hidden.
#ifndef MOE_OBS_WORDS
#define MOE_OBS_WORDS 16  // words of the partition record (also in moe_overlap.h)
#endif
// defaults before any observation: ~45 GB/s of copy per CU, ~0.8 PFLOP/s of FFN over 256 CUs
#define MOE_COPY_RATE0 450.0f    // bytes per tick per consumer CU
#define MOE_FFN_RATE0 31250.0f   // flops per tick per producer CU
#define MOE_TAIL_COPY_RATE 50000.0f  // bytes per tick over the whole chip (5 TB/s: an HBM copy, read and write)

MOE_HD int ffn_adaptive_consumers(int n_cu, int64_t m_real, int64_t m_ret, int d, int f, int64_t n_g1, float ffn_rate,
                                  float copy_rate) {
  const int cmax = li_min(32, n_cu / 4) / 8 * 8;
  if (cmax < 8) return n_cu / 4 > 1 ? n_cu / 4 : 1;  // a small device: a quarter of its CUs
  if (!(ffn_rate > 0.f)) ffn_rate = MOE_FFN_RATE0;
  if (!(copy_rate > 0.f)) copy_rate = MOE_COPY_RATE0;
  const int q1 = (int)(n_g1 % n_cu);  // workgroups with one first-GEMM item more than the others, with no partition
  if (q1 > 0 && m_ret > 0) {
    const double free_rate = (double)(n_cu - q1) * copy_rate;
    const double rate = free_rate < MOE_TAIL_COPY_RATE ? free_rate : MOE_TAIL_COPY_RATE;
    if (4.0 * (double)m_ret * d / rate <= 2.0 * 256 * 256 * (double)d / ffn_rate) return 0;
  }
  if (m_ret == 0) return 0;  // nothing to return
  int c = 8;
  for (; c < cmax; c += 8) {
    const double copy_t = 4.0 * (double)m_ret * d / ((double)c * copy_rate);
    const double ffn_t = 6.0 * (double)m_real * d * (double)f / ((double)(n_cu - c) * ffn_rate);
    if (copy_t <= 0.5 * ffn_t) break;
  }
  return c;
}
