// Remote-owner-aligned layout on the GPU (review page: "What carries the argument"; referee major
// comment 1, section 4.5 / Algorithm 1): rows of each local expert grouped by owner rank, each
// (expert, owner) group padded to a multiple of the tile height M, remote groups scheduled first.
//
//   k_layout_count   per 64-token chunk of one owner: histogram of local experts (wave ballots); row_src to -1
//   k_layout_scan    one workgroup: chunk prefixes, group sizes, wavefront prefix scans of padded sizes,
//                    band tables, remote-first order, transfer segments, GEMM row tiles
//   k_layout_scatter per chunk: stable rank of each (token, slot) in its group -> row_src, combine plan
//   k_gather_rows    x_pad[p] = x[row_src[p]] for real rows, 16-byte lanes
#include "common.h"
#include "launch.h"

#define SCAN_THREADS 1024
#define MAX_GROUPS (MOE_MAX_OWNERS * MOE_MAX_LOCAL_EXPERTS)
#define SCAN_KEYS 4096  // segments whose consumer-order keys are staged in LDS

__device__ __forceinline__ uint64_t lanemask_lt() {
  const int l = lane_id();
  return l == 0 ? 0ull : (~0ull >> (64 - l));
}

__global__ __launch_bounds__(256) void k_layout_count(const int32_t* __restrict__ topk_idx, int T_o, int G, int k,
                                                      int lo, int E, int n_chunks, int32_t* __restrict__ chunk_counts,
                                                      int32_t* __restrict__ row_src, int64_t cap_rows) {
  // every padded row starts as padding (-1); the scatter writes the real rows after the scan
  const int64_t nthr = (int64_t)gridDim.x * gridDim.y * blockDim.x;
  for (int64_t p = ((int64_t)blockIdx.y * gridDim.x + blockIdx.x) * blockDim.x + threadIdx.x; p < cap_rows; p += nthr)
    row_src[p] = -1;
  const int wave = threadIdx.x / MOE_WAVE, lane = lane_id();
  const int r = blockIdx.y;
  const int c = blockIdx.x * 4 + wave;
  if (c >= n_chunks) return;
  const int t = c * 64 + lane;
  uint64_t mask = 0;
  bool bad = false;
  if (t < T_o) {
    const int32_t* ids = topk_idx + ((int64_t)r * T_o + t) * k;
    for (int j = 0; j < k; ++j) {
      const int g = ids[j];
      bad |= (g < 0 || g >= G);
      const int e = g - lo;
      if (e >= 0 && e < E) {
        bad |= ((mask >> e) & 1ull) != 0;  // the same local expert twice in one token
        mask |= 1ull << e;
      }
    }
  }
  // a chunk with an invalid token records -1 counts; the scan turns that into MOE_EINVAL
  const bool chunk_bad = __ballot(bad) != 0ull;
  int mine = 0;
  for (int e = 0; e < E; ++e) {
    const int cnt = __popcll(__ballot((mask >> e) & 1ull));
    if (lane == e) mine = cnt;
  }
  if (lane < E) chunk_counts[((int64_t)r * n_chunks + c) * E + lane] = chunk_bad ? -1 : mine;
}

// Exclusive scans of N values per thread over the 1024-thread block, with two barriers: the waves' sums go to LDS,
// then every wave scans the 16 sums itself.  out[i] gets the thread's exclusive prefix, total[i] the block's sum.
// s_wsum holds N * 16 ints; every thread of the block calls this.
template <int N>
__device__ void block_excl_scan_n(const int (&v)[N], int (&out)[N], int (&total)[N], int* s_wsum) {
  constexpr int W = SCAN_THREADS / MOE_WAVE;
  const int wave = threadIdx.x / MOE_WAVE, lane = lane_id();
  int incl[N];
#pragma unroll
  for (int i = 0; i < N; ++i) {
    incl[i] = wave_incl_scan(v[i]);
    if (lane == MOE_WAVE - 1) s_wsum[i * W + wave] = incl[i];
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const int w = lane < W ? s_wsum[i * W + lane] : 0;
    const int wi = wave_incl_scan(w);
    out[i] = __builtin_amdgcn_readlane(wi - w, wave) + incl[i] - v[i];
    total[i] = __builtin_amdgcn_readlane(wi, W - 1);
  }
  __syncthreads();  // the sums are read before the next call writes them
}

__device__ __forceinline__ int block_excl_scan(int v, int* s_wsum, int* total) {
  const int in[1] = {v};
  int out[1], tot[1];
  block_excl_scan_n<1>(in, out, tot, s_wsum);
  *total = tot[0];
  return out[0];
}

struct ScanArgs {
  int R, T_o, E, M, mgb, self_rank, n_chunks, mt_rows;
  int64_t cap_rows, cap_tiles, cap_mtiles;
  int32_t *chunk_counts, *counts, *padded_off, *recv_off, *tile_owner, *tile_expert, *tile_valid, *tile_order,
      *seg_desc, *row_src, *scalars, *status, *mtile_desc, *seg_mtiles, *seg_sched, *mt_order;
};

__global__ __launch_bounds__(SCAN_THREADS) void k_layout_scan(ScanArgs a) {
  __shared__ int s_n[MAX_GROUPS];      // n_g
  __shared__ int s_poff[MAX_GROUPS];   // padded offset of g
  __shared__ int s_order[MAX_GROUPS];  // q -> g (non-empty groups, remote-first)
  __shared__ int s_q2[MAX_GROUPS];     // g -> position in the row-tile packing order
  __shared__ int s_band_pos[MAX_GROUPS], s_seg_pos[MAX_GROUPS], s_row_pos[MAX_GROUPS];
  __shared__ int s_order2[MAX_GROUPS];  // q2 -> g, row-tile packing order
  __shared__ int s_tile_base[MAX_GROUPS], s_run_off[MAX_GROUPS], s_run_rows[MAX_GROUPS];  // by q2
  __shared__ int s_roff[MAX_GROUPS];    // receive offset of g
  __shared__ int s_wsum[3 * SCAN_THREADS / MOE_WAVE];
  __shared__ int s_misc[4];
  // scratch reused by steps that never overlap: 64-bit sort keys of the groups (e), run tables (g), segment
  // keys (i)
  __shared__ uint64_t s_scratch[SCAN_KEYS / 2];

  const int tid = threadIdx.x;
  const int R = a.R, E = a.E, M = a.M, NG = E * R;

  // (a) group sizes; per-(owner, expert) chunk counts become exclusive prefixes in place.  A group's chunks are
  // cut into P parts of at most 8 consecutive chunks (P <= 1024 / groups), one thread per (group, part): it loads
  // its part's counts at once, the part sums meet in LDS, then it writes its part's prefixes.  A chunk that saw
  // an invalid token holds -1 counts.
  int bad = 0;
  {
    int* s_part = (int*)s_scratch;  // [P][NG] part sums
    int P = SCAN_THREADS / NG;
    if (P > (a.n_chunks + 7) / 8) P = (a.n_chunks + 7) / 8;
    if (P < 1) P = 1;
    const int L = (a.n_chunks + P - 1) / P;  // chunks per part
    // consecutive threads take consecutive experts of one owner, whose counts are adjacent in memory
    const int gi = tid % NG, p = tid / NG;
    const bool act = p < P;
    const int r = gi / E, e = gi - r * E, g = e * R + r;
    int32_t* base = a.chunk_counts + (int64_t)r * a.n_chunks * E + e;
    const int c0 = p * L, c1 = min(c0 + L, a.n_chunks);
    int v[8];
    int sum = 0;
    if (act) {
      if (L <= 8) {
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = c0 + u < c1 ? base[(int64_t)(c0 + u) * E] : 0;
#pragma unroll
        for (int u = 0; u < 8; ++u) sum += v[u];
      } else {
        for (int c = c0; c < c1; ++c) sum += base[(int64_t)c * E];
      }
      s_part[p * NG + gi] = sum;
    }
    __syncthreads();
    if (act) {
      int run = 0;
      for (int q = 0; q < p; ++q) run += s_part[q * NG + gi];
      if (L <= 8) {
#pragma unroll
        for (int u = 0; u < 8; ++u)
          if (c0 + u < c1) {
            base[(int64_t)(c0 + u) * E] = run;
            bad |= v[u] < 0;
            run += v[u];
          }
      } else {
        for (int c = c0; c < c1; ++c) {
          const int x = base[(int64_t)c * E];
          base[(int64_t)c * E] = run;
          bad |= x < 0;
          run += x;
        }
      }
      if (p == P - 1) {
        s_n[g] = run;
        a.counts[g] = run;
      }
    }
  }
  // the layout build sets the status word: MOE_EINVAL for an invalid token, then MOE_ECAPACITY, else MOE_OK
  const int any_bad = __syncthreads_or(bad);
  const int32_t status0 = any_bad ? MOE_EINVAL : MOE_OK;
  if (tid == 0) *a.status = status0;

  // (b) padded offsets: exclusive scan of P = ceil(n/M)*M in (e, r) order
  int total = 0;
  {
    const int n = tid < NG ? s_n[tid] : 0;
    const int P = ((n + M - 1) / M) * M;
    const int off = block_excl_scan(P, s_wsum, &total);
    if (tid < NG) {
      s_poff[tid] = off;
      a.padded_off[tid] = off;
    }
  }
  const int M_pad = total;
  const int n_tiles = M_pad / M;
  // (c) receive offsets per owner: sum over e' < e of n_{e', r}
  if (tid < R) {
    int run = 0;
    for (int e = 0; e < E; ++e) {
      a.recv_off[e * R + tid] = run;
      s_roff[e * R + tid] = run;
      run += s_n[e * R + tid];
    }
    a.scalars[SC_NR + tid] = run;
  }
  if ((int64_t)M_pad > a.cap_rows || status0 != 0) {
    if (tid == 0) {
      if (status0 == 0) set_status(a.status, MOE_ECAPACITY);
      a.scalars[SC_MPAD] = 0;
      a.scalars[SC_NTILES] = 0;
      a.scalars[SC_NSEGS] = 0;
      a.scalars[SC_NR + R] = 0;
      a.scalars[SC_NR + R + 1] = 0;
    }
    return;
  }
  __syncthreads();

  // (d) band tables (row_src holds -1 everywhere from the count kernel; the scatter writes the real rows)
  for (int g = tid; g < NG; g += SCAN_THREADS) {
    const int n = s_n[g], off = s_poff[g], e = g / R, r = g - e * R;
    for (int row = 0, b = off / M; row < n; row += M, ++b) {
      a.tile_owner[b] = r;
      a.tile_expert[b] = e;
      a.tile_valid[b] = (n - row) < M ? (n - row) : M;
    }
  }

  // (e) remote-first order of non-empty groups: key (owner == self, -P, e, r) ascending (bands, segments);
  // row-tile packing order: key (e, owner == self, -P, r): each expert's groups together, so that a GEMM row tile
  // (one expert) is as full as possible, and inside an expert the self-owned group last.  (Keeping
  // every self-owned group behind all remote ones instead gives each expert a second, mostly empty tile when R is
  // large: 142 row tiles instead of about 100 for 32 experts and 8 owners.)  Both keys are packed into one
  // unsigned 64-bit value per group (unique, since (e, r) is), so a group's rank is the count of smaller keys.
  {
    uint64_t* key1 = s_scratch;
    uint64_t* key2 = s_scratch + MAX_GROUPS;
    const bool mine = tid < NG && s_n[tid] > 0;
    const uint64_t none = ~0ull;
    uint64_t k1 = none, k2 = none;
    if (mine) {
      const int g = tid, e = g / R, r = g - e * R;
      const uint64_t self = r == a.self_rank, nP = (uint64_t)((1 << 30) - ((s_n[g] + M - 1) / M) * M);
      k1 = (self << 63) | (nP << 32) | ((uint64_t)e << 16) | (uint64_t)r;
      k2 = ((uint64_t)e << 50) | (self << 49) | (nP << 16) | (uint64_t)r;
    }
    if (tid < NG) {
      key1[tid] = k1;
      key2[tid] = k2;
    }
    int* s_rank = s_order;  // [NG] ranks by key1, then [NG] by key2 (s_order2), before either order is written
    if (tid < NG) {
      s_rank[tid] = 0;
      s_order2[tid] = 0;
    }
    __syncthreads();
    // the ranks of a group's keys are counted by NP threads, each over a slice of the groups
    {
      const int NP = SCAN_THREADS / NG >= 4 ? 4 : SCAN_THREADS / NG;
      const int gi = tid % NG, part = tid / NG;
      if (part < NP && gi < NG && s_n[gi] > 0) {
        const uint64_t c1 = key1[gi], c2 = key2[gi];
        const int h0 = part * NG / NP, h1 = (part + 1) * NG / NP;
        int r1 = 0, r2 = 0;
#pragma unroll 8
        for (int h = h0; h < h1; ++h) {
          r1 += key1[h] < c1;
          r2 += key2[h] < c2;
        }
        atomicAdd(&s_rank[gi], r1);
        atomicAdd(&s_order2[gi], r2);
      }
    }
    __syncthreads();
    int rank = 0, rank2 = 0;
    if (mine) {
      rank = s_rank[tid];
      rank2 = s_order2[tid];
    }
    __syncthreads();  // the ranks are read before the orders are written over them
    int n_ne = 0;
    block_excl_scan(mine ? 1 : 0, s_wsum, &n_ne);
    if (mine) {
      s_order[rank] = tid;
      s_order2[rank2] = tid;
      s_q2[tid] = rank2;
    }
    if (tid == 0) s_misc[0] = n_ne;
    __syncthreads();
  }
  const int n_ne = s_misc[0];

  // (f) band and segment positions in remote-first order, real-row positions in packing order
  {
    const int q = tid;
    int nb = 0, ns = 0, nrow = 0;
    if (q < n_ne) {
      const int n = s_n[s_order[q]];
      nb = (n + M - 1) / M;
      ns = (nb + a.mgb - 1) / a.mgb;
      nrow = s_n[s_order2[q]];
    }
    const int in3[3] = {nb, ns, nrow};
    int pre3[3], tot3[3];
    block_excl_scan_n<3>(in3, pre3, tot3, s_wsum);
    const int pb = pre3[0], ps = pre3[1], prow = pre3[2], ts = tot3[1], trow = tot3[2];
    if (q < n_ne) {
      s_band_pos[q] = pb;
      s_seg_pos[q] = ps;
      s_row_pos[q] = prow;  // indexed by q2
    }
    if (tid == 0) {
      s_misc[1] = ts;
      s_misc[2] = trow;
    }
    __syncthreads();
  }
  const int n_segs = s_misc[1];

  // (g) GEMM row tiles: runs of consecutive same-expert groups in packing order (one per expert), each run's real
  // rows cut into tiles of mt_rows rows (run starts, then two block scans: runs' tile counts, positions inside a
  // run)
  {
    int* s_e2 = (int*)s_scratch;               // expert of packing position q
    int* s_first = s_e2 + MAX_GROUPS;          // first packing position of run j
    int* s_tbase = s_first + MAX_GROUPS;       // first row tile of run j
    int* s_rrows = s_tbase + MAX_GROUPS;       // real rows of run j
    const int q = tid;
    const bool in = q < n_ne;
    if (in) s_e2[q] = s_order2[q] / R;
    __syncthreads();
    const int start = in && (q == 0 || s_e2[q - 1] != s_e2[q]);
    int n_runs = 0;
    const int run = block_excl_scan(start, s_wsum, &n_runs) + start - 1;  // run of q
    if (start) s_first[run] = q;
    __syncthreads();
    int tiles = 0, rrows = 0, fp = 0;
    if (tid < n_runs) {
      const int q0 = s_first[tid], q1 = tid + 1 < n_runs ? s_first[tid + 1] : n_ne;
      rrows = (q1 < n_ne ? s_row_pos[q1] : s_misc[2]) - s_row_pos[q0];
      tiles = (rrows + a.mt_rows - 1) / a.mt_rows;
      // the run's self-owned rows come last: its tiles from fp on hold self-owned rows only
      const int nself = s_n[s_e2[q0] * R + a.self_rank];
      fp = (rrows - nself + a.mt_rows - 1) / a.mt_rows;
    }
    int n_mt = 0, n_pure = 0;
    const int tb = block_excl_scan(tiles, s_wsum, &n_mt);
    const int pre = block_excl_scan(tiles - fp, s_wsum, &n_pure);
    if (tid < n_runs) {
      s_tbase[tid] = tb;
      s_rrows[tid] = rrows;
      // the producer's order: tiles holding another owner's rows by number, then the self-owned-only tiles
      for (int t = 0; t < tiles; ++t)
        a.mt_order[t < fp ? tb - pre + t : n_mt - n_pure + pre + (t - fp)] = tb + t;
    }
    __syncthreads();
    if (in) {
      s_tile_base[q] = s_tbase[run];
      s_run_off[q] = s_row_pos[q] - s_row_pos[s_first[run]];
      s_run_rows[q] = s_rrows[run];
    }
    if (tid == 0) {
      s_misc[3] = n_mt;
      a.scalars[SC_NR + R + 1] = n_mt - n_pure;
    }
    __syncthreads();
  }
  const int n_mtiles = s_misc[3];
  if ((int64_t)n_mtiles > a.cap_mtiles) {  // cannot happen within the capacity bound; guard anyway
    if (tid == 0) {
      set_status(a.status, MOE_ECAPACITY);
      a.scalars[SC_MPAD] = 0;
      a.scalars[SC_NTILES] = 0;
      a.scalars[SC_NSEGS] = 0;
      a.scalars[SC_NR + R] = 0;
    }
    return;
  }

  // (h) tile_order, row-tile entries and segments, one thread per band and segment; the group of an
  // entry is the last one whose first position (prefix over non-empty groups) is not after it
  auto find = [&](const int* first, int pos) {
    int lo = 0, hi = n_ne - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (first[mid] <= pos) lo = mid;
      else hi = mid - 1;
    }
    return lo;
  };
  for (int pos = tid; pos < n_tiles; pos += SCAN_THREADS) {
    const int q = find(s_band_pos, pos);
    a.tile_order[pos] = s_poff[s_order[q]] / M + (pos - s_band_pos[q]);
  }
  const int mt_mask = a.mt_rows - 1, mt_shift = __builtin_ctz(a.mt_rows);  // mt_rows is a power of two
  // row-tile entries: one wave per group of the packing order, 64 of its rows at a time; row j of group g is
  // row u = run offset + j of its expert's run, slot u % mt_rows of tile (run base + u / mt_rows).  The group that
  // ends a run marks the slots of its last tile past the run's rows with -1.  Lane l of wave w first loads the
  // tables of packing position w + 16 l, and the wave takes them from there one group at a time.
  {
    constexpr int W = SCAN_THREADS / MOE_WAVE;
    const int wave = tid / MOE_WAVE, lane = tid % MOE_WAVE;
    const int ql = wave + W * lane;  // < 64 W = MAX_GROUPS
    int g_l = 0, n_l = 0, base_l = 0, roff_l = 0, rrows_l = 0, poff_l = 0;
    if (ql < n_ne) {
      g_l = s_order2[ql];
      n_l = s_n[g_l];
      base_l = s_tile_base[ql];
      roff_l = s_run_off[ql];
      rrows_l = s_run_rows[ql];
      poff_l = s_poff[g_l];
    }
    for (int i = 0; wave + W * i < n_ne; ++i) {
      const int g = __builtin_amdgcn_readlane(g_l, i), n = __builtin_amdgcn_readlane(n_l, i);
      const int base = __builtin_amdgcn_readlane(base_l, i), roff = __builtin_amdgcn_readlane(roff_l, i);
      const int rrows = __builtin_amdgcn_readlane(rrows_l, i), poff = __builtin_amdgcn_readlane(poff_l, i);
      for (int j = lane; j < n; j += MOE_WAVE) {
        const int u = roff + j, slot = u & mt_mask;
        int32_t* d = a.mtile_desc + (int64_t)(base + (u >> mt_shift)) * MOE_MT_FIELDS;
        d[MOE_MT_HDR + slot] = poff + j;
        if (slot == 0) {
          const int left = rrows - u;
          d[0] = g / R;
          d[1] = left < a.mt_rows ? left : a.mt_rows;
          d[2] = base;
          d[3] = (rrows + a.mt_rows - 1) >> mt_shift;
          const int gs = (g / R) * R + a.self_rank;
          d[MT_SELF_LO] = s_poff[gs];
          d[MT_SELF_N] = s_n[gs];
          d[MT_SELF_DELTA] = s_roff[gs] - s_poff[gs];
          d[7] = 0;
        }
      }
      const int used = rrows & mt_mask;
      if (roff + n == rrows && used != 0) {
        int32_t* d = a.mtile_desc + (int64_t)(base + (rrows >> mt_shift)) * MOE_MT_FIELDS;
        for (int sl = used + lane; sl < a.mt_rows; sl += MOE_WAVE) d[MOE_MT_HDR + sl] = -1;
      }
    }
  }
  for (int sp = tid; sp < n_segs; sp += SCAN_THREADS) {
    const int q = find(s_seg_pos, sp);
    const int g = s_order[q], e = g / R, r = g - e * R, n = s_n[g], off = s_poff[g];
    const int nb = (n + M - 1) / M, b = (sp - s_seg_pos[q]) * a.mgb;
    const int cnt = (nb - b) < a.mgb ? (nb - b) : a.mgb;
    int rows = n - b * M;
    if (rows > cnt * M) rows = cnt * M;
    int32_t* sd = a.seg_desc + (int64_t)sp * MOE_SEG_FIELDS;
    sd[SEG_OWNER] = r;
    sd[SEG_EXPERT] = e;
    sd[SEG_FIRST_BAND] = off / M + b;
    sd[SEG_NBANDS] = cnt;
    sd[SEG_SRC_ROW] = off + b * M;
    sd[SEG_DST_ROW] = s_roff[g] + b * M;
    sd[SEG_ROWS] = rows;
    sd[SEG_GROUP] = g;
    const int q2 = s_q2[g], base = s_tile_base[q2], roff = s_run_off[q2];
    const int mt0 = base + ((roff + b * M) >> mt_shift), mt1 = base + ((roff + b * M + rows - 1) >> mt_shift);
    a.seg_mtiles[2 * sp] = mt0;
    a.seg_mtiles[2 * sp + 1] = mt1 - mt0 + 1;
  }
  __syncthreads();
  // (i) consumer order: segments by the last GEMM row tile they wait for, ties by segment index (stable).  In LDS a
  // counting sort over the row tiles: per-tile counts (LDS atomics), their exclusive scan, each segment dropped
  // into its tile's bucket, then placed inside the bucket by the segments of the bucket with a smaller index (at
  // most mt_rows segments end in one row tile, since each has a row in it).  Larger layouts rank every segment
  // against all others in global memory.
  if (n_mtiles + 1 + n_segs <= SCAN_KEYS) {
    int* s_start = (int*)s_scratch;          // [n_mtiles + 1]: counts per last tile, then bucket starts
    int* s_list = s_start + n_mtiles + 1;    // [n_segs]: bucket members
    constexpr int PER = SCAN_KEYS / SCAN_THREADS;
    for (int t = tid; t <= n_mtiles; t += SCAN_THREADS) s_start[t] = 0;
    __syncthreads();
    int key[PER], slot[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int sg = tid + j * SCAN_THREADS;
      key[j] = 0;
      slot[j] = 0;
      if (sg < n_segs) {
        key[j] = a.seg_mtiles[2 * sg] + a.seg_mtiles[2 * sg + 1] - 1;
        slot[j] = atomicAdd(&s_start[key[j]], 1);
      }
    }
    __syncthreads();
    {  // buckets [PER tid, PER tid + PER) of this thread; bucket n_mtiles (empty) gets start n_segs
      int c[PER], sum = 0;
#pragma unroll
      for (int j = 0; j < PER; ++j) {
        const int t = PER * tid + j;
        c[j] = t <= n_mtiles ? s_start[t] : 0;
        sum += c[j];
      }
      int tot = 0;
      int run = block_excl_scan(sum, s_wsum, &tot);
#pragma unroll
      for (int j = 0; j < PER; ++j) {
        const int t = PER * tid + j;
        if (t <= n_mtiles) s_start[t] = run;
        run += c[j];
      }
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int sg = tid + j * SCAN_THREADS;
      if (sg < n_segs) s_list[s_start[key[j]] + slot[j]] = sg;
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int sg = tid + j * SCAN_THREADS;
      if (sg < n_segs) {
        const int b0 = s_start[key[j]], b1 = s_start[key[j] + 1];
        int rank = b0;
        for (int o = b0; o < b1; ++o) rank += s_list[o] < sg;
        a.seg_sched[rank] = sg;
      }
    }
  } else {
    for (int sg = tid; sg < n_segs; sg += SCAN_THREADS) {
      const int last = a.seg_mtiles[2 * sg] + a.seg_mtiles[2 * sg + 1];
      int rank = 0;
      for (int o = 0; o < n_segs; ++o) {
        const int lo2 = a.seg_mtiles[2 * o] + a.seg_mtiles[2 * o + 1];
        rank += (lo2 < last) || (lo2 == last && o < sg);
      }
      a.seg_sched[rank] = sg;
    }
  }
  if (tid == 0) {
    a.scalars[SC_MPAD] = M_pad;
    a.scalars[SC_NTILES] = n_tiles;
    a.scalars[SC_NSEGS] = n_segs;
    a.scalars[SC_NR + R] = n_mtiles;
  }
}

__global__ __launch_bounds__(256) void k_layout_scatter(const int32_t* __restrict__ topk_idx, int R, int T_o, int k,
                                                        int lo, int E, int n_chunks,
                                                        const int32_t* __restrict__ chunk_prefix,
                                                        const int32_t* __restrict__ padded_off,
                                                        const int32_t* __restrict__ recv_off,
                                                        int32_t* __restrict__ row_src, int32_t* __restrict__ plan,
                                                        const int32_t* __restrict__ status) {
  if (load_status(status) != 0) return;
  const int wave = threadIdx.x / MOE_WAVE, lane = lane_id();
  const int r = blockIdx.y;
  const int c = blockIdx.x * 4 + wave;
  if (c >= n_chunks) return;
  const int t = c * 64 + lane;
  const bool valid = t < T_o;
  const int64_t tok = (int64_t)r * T_o + t;
  constexpr int KMAX = 16;  // top-k <= 16
  uint64_t mask = 0;
  int e_of[KMAX];  // slot j -> local expert or -1 (compile-time indices: registers)
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    int e = -1;
    if (j < k && valid) {
      e = topk_idx[tok * k + j] - lo;
      if (e < 0 || e >= E) e = -1;
      if (e < 0) plan[tok * k + j] = -1;
    }
    e_of[j] = e;
    if (e >= 0) mask |= 1ull << e;
  }
  // lane e holds local expert e's chunk prefix and group offsets (E <= 64), read below with readlane
  const int32_t* pre = chunk_prefix + ((int64_t)r * n_chunks + c) * E;
  int pre_l = 0, poff_l = 0, roff_l = 0;
  if (lane < E) {
    pre_l = pre[lane];
    poff_l = padded_off[lane * R + r];
    roff_l = recv_off[lane * R + r];
  }
  const uint64_t lt = lanemask_lt();
  for (int e = 0; e < E; ++e) {
    const uint64_t b = __ballot((mask >> e) & 1ull);
    if (b == 0) continue;
    const int pe = __builtin_amdgcn_readlane(pre_l, e), po = __builtin_amdgcn_readlane(poff_l, e);
    const int ro = __builtin_amdgcn_readlane(roff_l, e);
    if ((mask >> e) & 1ull) {
      const int rank = pe + __popcll(b & lt);
      row_src[(int64_t)po + rank] = (int32_t)tok;
#pragma unroll
      for (int j = 0; j < KMAX; ++j)
        if (e_of[j] == e) plan[tok * k + j] = ro + rank;
    }
  }
}

// x_pad[p] = x[row_src[p]] for the real rows; one wavefront per row, 16-byte lanes.
__global__ __launch_bounds__(256) void k_gather_rows(const uint4* __restrict__ x, uint4* __restrict__ x_pad,
                                                     const int32_t* __restrict__ row_src,
                                                     const int32_t* __restrict__ scalars, int row_vec,
                                                     const int32_t* __restrict__ status) {
  if (load_status(status) != 0) return;
  const int M_pad = scalars[SC_MPAD];
  const int wave = threadIdx.x / MOE_WAVE, lane = lane_id();
  for (int p = blockIdx.x * 4 + wave; p < M_pad; p += gridDim.x * 4) {
    const int src = row_src[p];
    if (src < 0) continue;
    const uint4* s = x + (int64_t)src * row_vec;
    uint4* d = x_pad + (int64_t)p * row_vec;
    int i = lane;
    for (; i + 192 < row_vec; i += 256) {
      const uint4 v0 = s[i], v1 = s[i + 64], v2 = s[i + 128], v3 = s[i + 192];
      d[i] = v0;
      d[i + 64] = v1;
      d[i + 128] = v2;
      d[i + 192] = v3;
    }
    for (; i < row_vec; i += 64) d[i] = s[i];
  }
}

int launch_layout(const LayoutLaunch& p, hipStream_t st) {
  const int n_chunks = (p.T_o + 63) / 64;
  if (n_chunks > 0)
    hipLaunchKernelGGL(k_layout_count, dim3((n_chunks + 3) / 4, p.R), dim3(256), 0, st, p.topk_idx, p.T_o, p.G, p.k,
                       p.lo, p.E, n_chunks, p.L->chunk_counts, p.L->row_src, p.L->cap_rows);
  ScanArgs a;
  a.R = p.R;
  a.T_o = p.T_o;
  a.E = p.E;
  a.M = p.M;
  a.mgb = p.mgb;
  a.self_rank = p.self_rank;
  a.n_chunks = n_chunks;
  a.mt_rows = p.mt_rows;
  a.cap_rows = p.L->cap_rows;
  a.cap_tiles = p.L->cap_tiles;
  a.cap_mtiles = p.L->cap_mtiles;
  a.chunk_counts = p.L->chunk_counts;
  a.counts = p.L->counts;
  a.padded_off = p.L->padded_off;
  a.recv_off = p.L->recv_off;
  a.tile_owner = p.L->tile_owner;
  a.tile_expert = p.L->tile_expert;
  a.tile_valid = p.L->tile_valid;
  a.tile_order = p.L->tile_order;
  a.seg_desc = p.L->seg_desc;
  a.row_src = p.L->row_src;
  a.scalars = p.L->scalars;
  a.status = p.L->status;
  a.mtile_desc = p.L->mtile_desc;
  a.seg_mtiles = p.L->seg_mtiles;
  a.seg_sched = p.L->seg_sched;
  a.mt_order = p.L->mt_order;
  hipLaunchKernelGGL(k_layout_scan, dim3(1), dim3(SCAN_THREADS), 0, st, a);
  if (n_chunks > 0)
    hipLaunchKernelGGL(k_layout_scatter, dim3((n_chunks + 3) / 4, p.R), dim3(256), 0, st, p.topk_idx, p.R, p.T_o,
                       p.k, p.lo, p.E, n_chunks, p.L->chunk_counts, p.L->padded_off, p.L->recv_off, p.L->row_src,
                       p.L->combine_plan, p.L->status);
  const int row_vec = (int)(p.row_bytes / 16);
  int64_t blocks = (p.L->cap_rows + 3) / 4;
  if (blocks > 4096) blocks = 4096;
  if (blocks > 0 && p.x != nullptr)  // no x: the FFN launch lands the rows itself
    hipLaunchKernelGGL(k_gather_rows, dim3((unsigned)blocks), dim3(256), 0, st, (const uint4*)p.x, (uint4*)p.x_pad,
                       p.L->row_src, p.L->scalars, row_vec, p.L->status);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}
