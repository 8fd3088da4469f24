// The backward pass of the expert FFN (review page, "Where Pith is reading between the lines": the producer-consumer
// signalling applied to MoE training's backward pass, which has the same GEMM-then-transfer structure).  Given the
// gradient of the combined output, per routed row p of token t, slot weight w and local expert e:
//   dY = bf16(w dOut[t])                                   (k_bwd_dy: the gradient's dispatch into the padded layout)
//   dH = dY Wd,  g = x Wg^T,  u = x Wu^T                   (recomputed as the forward computes them, or read from
//                                                           the forward's stored copy: the same bits)
//   h = bf16(silu(g) u),  dU = bf16(dH silu(g)),  dG = bf16(dH u silu'(g))
//   dX = (dG | dU) (Wg | Wu)                                (rows returned to their owners: the overlapped transfer)
//   dWd[e] = sum_p dY^T h,  dWgu[e] = sum_p (dG | dU)^T x   (fp32, over the expert's rows)
// and the combine's backward (k_bwd_combine): dx[t] = sum of the token's delivered dX rows, and the routing weight's
// gradient <dOut[t], y> from the forward's delivered rows.
//
// One persistent launch runs four kinds of items, each a 256 x 256 output tile of bf16 MFMAs (32x32x16) over
// k-tiles of 64, in list order: H (row tile, 256 columns of f) -> dH, fp32, flag fh; G (row tile, 128 columns of f)
// -> h, dG, dU after its dH tile's flag, flag fg; X (row tile, 256 columns of d, k-split) -> dX rows after the fg
// flags of its split, split-K partial sums summed in split order by the last to arrive, flag fx, which the
// consumer role waits on to copy the other owners' rows (the self owner's rows are stored straight into its buffer,
// as in the forward); W (expert, 256 x 256 tile of dWd or dWgu, k over the expert's rows) after the fg flags of the
// expert's row tiles.  H, G and X go round-robin over the workgroups, each in list order, and every wait of one is
// on an earlier item, so the earliest unfinished item can always run; W tiles, which nobody waits on, are handed out
// at run time once a workgroup's H, G and X items are done.
//
// Operands whose k runs along rows of memory (x, dY, (dG | dU) as the rows of a row tile; Wgu rows for g and u) are
// staged as in the forward.  Operands whose k runs down columns (Wd and Wgu as the second operand of dH and dX; all
// four operands of the weight gradients, whose k is the expert's rows) are staged as 64 rows x 256 columns, and
// their MFMA fragments are read with the LDS transpose read (ds_read_b64_tr_b16): in a group of 16 lanes, lane j
// gives the address of row r0 + j / 4, columns c0 + 4 (j % 4) .. + 3, and lane l receives column c0 + l of rows
// r0 .. r0 + 3, so two reads give a lane the 8 consecutive k of its column that the MFMA takes.  Such a tile keeps
// 32-byte column granule g of row r at granule col_swz(g, r), so that each half-wave of a read hits 64 distinct
// banks.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <algorithm>

#include "common.h"
#include "consumer.h"
#include "launch.h"
#include "tile_util.h"

#define BWD_THREADS 512  // 8 waves: 2 (rows) x 4 (columns) of 128 x 64 wave tiles
#define BWD_BM 256
#define BWD_BK 64
#define BWD_STAGE (2 * BWD_BM * BWD_BK * 2)  // A and B tiles of one k-tile, 64 KB

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

struct BwdArgs {
  const unsigned char* x;    // x_pad [cap_rows, d] bf16
  const unsigned char* w1;   // w_gate_up [E, 2f, d]
  const unsigned char* w2;   // w_down [E, d, f]
  const unsigned char* dy;   // dY rows [cap_rows, d]
  float* dh;                 // [cap_rows, f]
  unsigned char* h;          // [cap_rows, f] bf16
  unsigned char* dgu;        // [cap_rows, 2f] bf16: dG | dU
  const float* gu;           // null, or [cap_rows, 2f] fp32: g | u as the forward stored them (G items skip the GEMM)
  unsigned char* dxp;        // dX rows of the other owners [cap_rows, d]
  unsigned char* self_recv;  // the self owner's dX buffer
  float* dw1;                // [E, 2f, d]
  float* dw2;                // [E, d, f]
  int d, f, E, S;            // S: k-splits of the dX items
  int n_h, n_g, n_x;         // column tiles of H (256 of f), G (128 of f), X (256 of d) items
  const int32_t* mtile_desc;
  const int32_t* mt_order;
  const int32_t* scalars;
  int sc_nmt;
  int32_t* status;
  uint32_t* fh;
  uint32_t* fg;
  uint32_t* fx;
  uint64_t* scount;  // [cap_mtiles][n_x] arrivals of the dX k-splits
  float* partial;    // [cap_mtiles][n_x][S][256 x 256] fp32 partial sums
  uint64_t* wclaim;  // weight-gradient tiles handed out: this launch's stamp << 32 | count
  uint32_t wstamp;
  uint32_t epoch;
  uint64_t budget;
  int n_cons;  // consumer workgroups (the first n_cons of the grid)
  int join;    // producers take copy units once their items are done
  ConsumerArgs cons;
};

// Column-staged tiles (64 k-rows x 256 columns, 512 bytes per row): the 32-byte granule g (16 columns) of k-row r
// sits at granule col_swz(g, r) of the row.  A transposed fragment read has lanes 0-15 and 16-31 on columns 16
// apart (granules g and g + 1, g even) of the same four k-rows; col_swz puts g and g + 1 in opposite halves of the
// 64 banks (bit 2 of the granule, from bit 0 of g) and the four rows of each in distinct granules of that half
// (XOR with r & 3), so each half-wave reads 64 distinct banks.  (Granule g ^ (r & 3) kept g and g + 1 in one half:
// 31% of the launch's LDS cycles were bank conflicts.)
__device__ __forceinline__ int col_swz(int g, int r) {
  const int x = g & 7;
  return (g & 8) | ((((x & 1) << 2) | (x >> 1)) ^ (r & 3));
}
__device__ __forceinline__ int col_unswz(int p, int r) {  // the logical granule at granule p of k-row r
  const int y = (p & 7) ^ (r & 3);
  return (p & 8) | (((y & 3) << 1) | (y >> 2));
}

// Fragment of a column-staged tile at column cb (a multiple of 32), k-step ks: the 8 consecutive k of column
// cb + lane % 32 starting at 16 ks + 8 (lane / 32), as the MFMA takes them.
__device__ __forceinline__ bf16x8_t frag_tr(const unsigned char* st, int cb, int ks, int lane) {
  const int gi = lane >> 4, j = lane & 15;
  const int n = cb + 16 * (gi & 1) + 4 * (j & 3);
  s16x4_t v[2];
#pragma unroll
  for (int hk = 0; hk < 2; ++hk) {
    const int k = 16 * ks + 8 * (gi >> 1) + 4 * hk + (j >> 2);
    const unsigned char* p = st + k * 512 + ((col_swz(n >> 4, k) << 5) | ((n & 15) << 1));
    v[hk] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)p);
  }
  return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(v[0], v[1], 0, 1, 2, 3, 4, 5, 6, 7));
}

// Fragment of a row-staged tile (256 rows x 64 k, 16-byte k-chunk c of row r at slot c ^ (r & 7) ^ ((r >> 3) & 1)):
// row rb + lane % 32, k 16 ks + 8 (lane / 32) ..
__device__ __forceinline__ bf16x8_t frag_row(const unsigned char* st, int rb, int ks, int lane) {
  const int swz = (lane & 7) ^ ((lane >> 3) & 1);
  return __builtin_bit_cast(bf16x8_t,
                            *(const u32x4_t*)(st + (rb + (lane & 31)) * 128 + (((2 * ks + (lane >> 5)) ^ swz) << 4)));
}

// Item kinds
enum { BK_H = 1, BK_G = 2, BK_X = 3, BK_WD = 4, BK_WGU = 5 };

struct BwdItem {
  int kind, mt, nt, s;  // H/G/X: row tile, column tile, split
  int e, it, jt;        // W: expert, output row tile, output column tile
};

// Items H, G and X, in list order (assigned round-robin before the run starts): i < bwd_n_static
__device__ __forceinline__ BwdItem bwd_item(const BwdArgs& a, int n_mt, int i) {
  BwdItem it{};
  const int NH = n_mt * a.n_h, NG = n_mt * a.n_g;
  if (i < NH) {
    it.kind = BK_H;
    it.mt = i / a.n_h;
    it.nt = i - it.mt * a.n_h;
  } else if ((i -= NH) < NG) {
    it.kind = BK_G;
    it.mt = i / a.n_g;
    it.nt = i - it.mt * a.n_g;
  } else {
    i -= NG;
    it.kind = BK_X;
    const int per = a.n_x * a.S, p = i / per, r = i - p * per;
    it.mt = a.mt_order[p];  // remote first: the row tiles holding another owner's rows come first
    it.s = r / a.n_x;
    it.nt = r - it.s * a.n_x;
  }
  return it;
}

__device__ __forceinline__ int bwd_n_static(const BwdArgs& a, int n_mt) { return n_mt * (a.n_h + a.n_g + a.n_x * a.S); }

// Weight-gradient tiles per expert: every dW_down and every dW_gate_up tile
__device__ __forceinline__ int bwd_w_per_expert(const BwdArgs& a) {
  const int nd = (a.d + 255) / 256, nf = (a.f + 255) / 256, n2 = 2 * a.f / 256;
  return nd * nf + n2 * nd;
}

// Shared state of an item (in LDS)
struct BwdShared {
  int rows[BWD_BM];  // padded rows of the row tile
  int hdr[MOE_MT_HDR];
  int run_first, run_count, k_rows;  // W items: the expert's run of row tiles and its row count
  int stop;
  int next;  // W items: the tile the workgroup claimed during its current one
  // per local expert, built once by a workgroup before its first W item: rows, first row tile and tile count of its
  // run, and the experts by decreasing rows (the order W tiles are handed out in)
  int e_rows[MOE_MAX_LOCAL_EXPERTS], e_first[MOE_MAX_LOCAL_EXPERTS], e_count[MOE_MAX_LOCAL_EXPERTS];
  int e_order[MOE_MAX_LOCAL_EXPERTS];
};

// W tile number w (0 .. E x per): expert e_order[w / per], then its dW_down tiles, then its dW_gate_up tiles
__device__ __forceinline__ BwdItem bwd_w_item(const BwdArgs& a, const BwdShared& sh, int w) {
  BwdItem it{};
  const int nd = (a.d + 255) / 256, nf = (a.f + 255) / 256, per = bwd_w_per_expert(a);
  const int k = w / per, r = w - k * per;
  it.e = sh.e_order[k];
  if (r < nd * nf) {
    it.kind = BK_WD;
    it.it = r / nf;
    it.jt = r - it.it * nf;
  } else {
    it.kind = BK_WGU;
    it.it = (r - nd * nf) / nd;
    it.jt = (r - nd * nf) - it.it * nd;
  }
  return it;
}


template <int KIND>
__device__ __forceinline__ bool bwd_tile(const BwdArgs& a, unsigned char* smem, BwdShared& sh, const BwdItem& it) {
  constexpr bool A_TR = KIND == BK_WD || KIND == BK_WGU;        // A staged by columns (k along rows of memory)
  constexpr bool B_TR = KIND != BK_G;                            // B staged by columns
  constexpr int MI = 4, NI = 2, A_BYTES = BWD_BM * BWD_BK * 2;
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 2, wn = wave & 3;
  const int d = a.d, f = a.f;
  const int e = (KIND == BK_WD || KIND == BK_WGU) ? it.e : sh.hdr[0];
  const int n_rows = (KIND == BK_WD || KIND == BK_WGU) ? 0 : sh.hdr[1];

  // ---- operand geometry ------------------------------------------------------------------------------------
  // A: H dY rows (K = d); G x rows (K = d); X (dG | dU) rows (K = 2f, split s); WD dY by columns, WGU (dG | dU) by
  // columns (K = the expert's rows).  B: H Wd by columns (k = d index, columns of f); G Wgu rows (gate | up);
  // X Wgu by columns (k = 2f index, columns of d); WD h by columns; WGU x by columns.
  int K, k0 = 0;
  if (KIND == BK_H) K = d;
  else if (KIND == BK_G) K = a.gu != nullptr ? 0 : d;  // with g | u from the forward, no GEMM
  else if (KIND == BK_X) {
    K = 2 * f / a.S;
    k0 = it.s * K;
  } else K = sh.k_rows;
  const int nk = (K + BWD_BK - 1) / BWD_BK;
  const unsigned char* Abase;
  uint32_t a_stride;  // bytes per row of A's memory
  if (KIND == BK_H) { Abase = a.dy; a_stride = d * 2; }
  else if (KIND == BK_G) { Abase = a.x; a_stride = d * 2; }
  else if (KIND == BK_X) { Abase = a.dgu; a_stride = 4 * f; }
  else if (KIND == BK_WD) { Abase = a.dy; a_stride = d * 2; }
  else { Abase = a.dgu; a_stride = 4 * f; }
  const unsigned char* Bbase;
  uint32_t b_stride;
  int b_cols = 0, b_col0 = 0;  // transposed B: columns of its memory, and this tile's first column
  if (KIND == BK_H) { Bbase = a.w2 + (int64_t)e * d * f * 2; b_stride = f * 2; b_cols = f; b_col0 = it.nt * 256; }
  else if (KIND == BK_G) { Bbase = a.w1 + (int64_t)e * 2 * f * d * 2; b_stride = d * 2; }
  else if (KIND == BK_X) { Bbase = a.w1 + (int64_t)e * 2 * f * d * 2; b_stride = d * 2; b_cols = d; b_col0 = it.nt * 256; }
  else if (KIND == BK_WD) { Bbase = a.h; b_stride = f * 2; b_cols = f; b_col0 = it.jt * 256; }
  else { Bbase = a.x; b_stride = d * 2; b_cols = d; b_col0 = it.jt * 256; }
  const int a_cols = KIND == BK_WD ? d : 2 * f, a_col0 = it.it * 256;  // transposed A

  // the memory row of k index kk (0 .. nk*64) of a transposed operand whose k runs over memory rows: weights (H, X)
  // by k directly; W items through the expert's row list (absent rows read the expert's first row; zeroed below)
  auto krow = [&](int kk) -> int64_t {
    if (KIND == BK_H || KIND == BK_X) return (int64_t)(k0 + kk);
    const int r = kk < sh.k_rows ? kk : 0, t = sh.run_first + (r >> 8);
    return a.mtile_desc[(int64_t)t * MOE_MT_FIELDS + MOE_MT_HDR + (r & 255)];
  };

  const uint32_t lds0 = (uint32_t)(uintptr_t)smem;
  // ---- loads: per k-tile each wave issues 4 A and 4 B 16-byte LDS-DMA loads (load u < 4: A instruction
  // q = 4 wave + u, else B instruction q = 4 wave + u - 4; one instruction fills 1 KB of the stage).
  // Row-staged tiles (256 rows x 64 k): lane -> row 8q + lane/8, slot lane & 7 holding k-chunk
  // (lane & 7) ^ (lane >> 3) ^ (q & 1).  Column-staged tiles (64 k x 256 columns): lanes 0-31 k-row 2q, 32-63 k-row
  // 2q + 1, slot lane & 31 of the row holding 16-byte column chunk c of granule c / 2 = col_unswz(slot / 2, k);
  // columns past the matrix read column 0.  A lane's offsets are fixed but for the k-tile: + kt * step, or, for the W
  // items (k over the expert's rows), + the memory row of each of its four k-rows times the stride, read from the
  // row-tile descriptors in global memory three k-tiles ahead (a read just before each load put a global-memory
  // latency in front of every k-tile's loads).
  const uint32_t chunk0 = (uint32_t)(((lane & 7) ^ (lane >> 3)) << 4);
  uint32_t aoff[4], boff[4];
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) {
    const int q = wave * 4 + jj;
    const int r = 8 * q + (lane >> 3);                                // row-staged row
    const int kq = 2 * q + (lane >> 5), cs = lane & 31;               // column-staged k-row and slot
    const int c = (col_unswz(cs >> 1, kq) << 1) | (cs & 1);           // the 16-byte column chunk it holds
    const uint32_t rchunk = (uint32_t)k0 * 2u + (chunk0 ^ ((uint32_t)(q & 1) << 4));
    if (A_TR) {
      aoff[jj] = (uint32_t)(a_col0 + 8 * c < a_cols ? a_col0 + 8 * c : 0) * 2u;
    } else {
      aoff[jj] = (uint32_t)sh.rows[r < n_rows ? r : 0] * a_stride + rchunk;  // absent rows read a real row
    }
    if (B_TR) {
      const uint32_t cpart = (uint32_t)(b_col0 + 8 * c < b_cols ? b_col0 + 8 * c : 0) * 2u;
      boff[jj] = A_TR ? cpart : (uint32_t)(k0 + kq) * b_stride + cpart;  // weights: k runs over their rows
    } else {  // G: gate rows, then up rows of the column tile
      const int wr = r < 128 ? it.nt * 128 + r : f + it.nt * 128 + (r - 128);
      boff[jj] = (uint32_t)wr * b_stride + rchunk;
    }
  }
  const uint32_t a_step = A_TR ? 0u : (uint32_t)BWD_BK * 2u;
  const uint32_t b_step = A_TR ? 0u : B_TR ? (uint32_t)BWD_BK * b_stride : (uint32_t)BWD_BK * 2u;
  // W: memory rows of this lane's k-rows: ids1 of the k-tile whose loads go out next, ids2 and ids3 of the next two
  int ids1[4] = {0, 0, 0, 0}, ids2[4] = {0, 0, 0, 0}, ids3[4] = {0, 0, 0, 0};
  auto fetch_ids = [&](int kt, int (&ids)[4]) {
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) ids[jj] = (int)krow(kt * BWD_BK + 2 * (wave * 4 + jj) + (lane >> 5));
  };
  // load u of k-tile kt into the stage at LDS address st (ids: the W item's rows of k-tile kt)
  auto dma1 = [&](int kt, uint32_t st, int u, const int (&ids)[4]) {
    if (u < 4) {
      const uint32_t off = aoff[u] + (A_TR ? (uint32_t)ids[u] * a_stride : (uint32_t)kt * a_step);
      dma16(Abase, off, st + (wave * 4 + u) * 1024);
    } else {
      const int jj = u - 4;
      const uint32_t off = boff[jj] + (A_TR ? (uint32_t)ids[jj] * b_stride : (uint32_t)kt * b_step);
      dma16(Bbase, off, st + A_BYTES + (wave * 4 + jj) * 1024);
    }
  };
  // W items: the k-rows of the last k-tile past the expert's rows hold real rows' values; zero them in both tiles
  auto zero_tail = [&](int stage) {
    const int cnt = sh.k_rows - (nk - 1) * BWD_BK;
    if (!A_TR || cnt >= BWD_BK) return;
    unsigned char* st = smem + stage * BWD_STAGE;
    for (int i = tid; i < (BWD_BK - cnt) * 2 * 32; i += BWD_THREADS) {  // 16-byte chunks of the rows, A then B
      const int t = i / ((BWD_BK - cnt) * 32), r = cnt + (i / 32) % (BWD_BK - cnt), c = i & 31;
      *(u32x4_t*)(st + t * A_BYTES + r * 512 + c * 16) = u32x4_t{0u, 0u, 0u, 0u};
    }
    __syncthreads();
  };

  f32x16_t acc[MI][NI];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int ni = 0; ni < NI; ++ni)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[mi][ni][q] = 0.f;

  // ---- the k-loop (the forward's pipeline): a k-tile is four k-steps of MI x NI MFMAs per wave; the fragments of
  // k-step s+1 are read in the first two MFMA slots of k-step s (two register sets); one barrier per k-tile, between
  // k-steps 2 and 3, after which k-tile kt+1 is in LDS and the stage of kt is free: the A loads of k-tile kt+2 go
  // into it during k-step 3 and the B loads of kt+1 went out during k-step 0, so every load has about three k-steps
  // to land.  Each slot's work is pinned with sched_barrier.
  constexpr int NSLOT = MI * NI, RS = 2, RPS = (MI + NI + RS - 1) / RS, FIRST = RS, HALF = 4;
  constexpr int DPS = (HALF + (NSLOT - FIRST) - 1) / (NSLOT - FIRST);
  bf16x8_t fa[2][MI], fb[2][NI];
  // 32-row MFMA blocks of this wave that hold real rows of the row tile (all MI for W items and full tiles): the
  // others' MFMAs and A fragment reads are skipped (an expert's last row tile is partly empty)
  const int mact = A_TR ? MI : min(MI, max(0, (n_rows - wm * 128 + 31) / 32));
  auto frag1 = [&](const unsigned char* sa, int ks, int i, bf16x8_t* A_, bf16x8_t* B_, bool full) {
    const unsigned char* sb = sa + A_BYTES;
    if (i < MI) {
      if (!full && i >= mact) return;
      A_[i] = A_TR ? frag_tr(sa, wm * 128 + i * 32, ks, lane) : frag_row(sa, wm * 128 + i * 32, ks, lane);
    } else {
      const int ni = i - MI;
      if (B_TR) B_[ni] = frag_tr(sb, wn * 64 + ni * 32, ks, lane);
      else B_[ni] = frag_row(sb, ni == 0 ? wn * 32 : 128 + wn * 32, ks, lane);  // gate block, up block
    }
  };
  auto step = [&](auto ks_tag, auto m1_tag, auto m2_tag, auto full_tag, int kt) {
    constexpr int ks = decltype(ks_tag)::value;
    constexpr bool M1 = decltype(m1_tag)::value, M2 = decltype(m2_tag)::value;
    constexpr bool FULL = decltype(full_tag)::value;
    constexpr int c = ks & 1;
    const unsigned char* sa = smem + (kt & 1) * BWD_STAGE;
    const unsigned char* nsa = smem + ((kt + 1) & 1) * BWD_STAGE;
#pragma unroll
    for (int i = 0; i < NSLOT; ++i) {
      const int mi = i / NI, ni = i % NI;
      if (FULL || mi < mact)
        acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[c][mi], fb[c][ni], acc[mi][ni], 0, 0, 0);
      if (i < RS) {
#pragma unroll
        for (int r = i * RPS; r < (i + 1) * RPS && r < MI + NI; ++r) {
          if (ks < 3) frag1(sa, ks + 1, r, fa[c ^ 1], fb[c ^ 1], FULL);
          else if (M1) frag1(nsa, 0, r, fa[c ^ 1], fb[c ^ 1], FULL);
        }
      }
      if (i >= FIRST && ((ks == 3 && M2) || (ks == 0 && M1))) {
#pragma unroll
        for (int t = 0; t < DPS; ++t) {
          const int v = (i - FIRST) * DPS + t;
          if (v < HALF) {
            if (ks == 3) dma1(kt + 2, lds0 + (kt & 1) * BWD_STAGE, v, ids1);             // A of kt+2
            else dma1(kt + 1, lds0 + ((kt + 1) & 1) * BWD_STAGE, HALF + v, ids1);        // B of kt+1
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if (ks == 1 && A_TR) fetch_ids(kt + 3, ids3);  // lands under k-step 2, before the barrier's vmcnt(0)
    if (ks == 2) {
      // this wave's fragment reads of k-tile kt and loads of k-tile kt+1 are done; then everyone's are
      asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
      if (M1 && !M2) zero_tail((kt + 1) & 1);  // k-tile kt+1 is the last
      if (A_TR) {
        // W rows: kt+2's for the A loads of k-step 3 and the B loads of the next k-step 0, and kt+3's; moved here,
        // where nothing is in flight, so that waiting for the row reads stalls no load
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          ids1[jj] = ids2[jj];
          ids2[jj] = ids3[jj];
        }
      }
    }
  };
  auto tile = [&](auto m1, auto m2, auto full, int kt) {
    step(std::integral_constant<int, 0>{}, m1, m2, full, kt);
    step(std::integral_constant<int, 1>{}, m1, m2, full, kt);
    step(std::integral_constant<int, 2>{}, m1, m2, full, kt);
    step(std::integral_constant<int, 3>{}, m1, m2, full, kt);
  };
  auto kloop = [&](auto full) {
    // prologue: k-tile 0 whole, the A loads of k-tile 1 (its B loads go out in k-step 0 of k-tile 0)
    int ids0[4] = {0, 0, 0, 0};
    if (A_TR) {
      fetch_ids(0, ids0);
      fetch_ids(1, ids1);
      fetch_ids(2, ids2);
    }
#pragma unroll
    for (int u = 0; u < 2 * HALF; ++u) dma1(0, lds0, u, ids0);
    wait_loads_barrier();
    if (nk == 1) zero_tail(0);
#pragma unroll
    for (int i = 0; i < MI + NI; ++i) frag1(smem, 0, i, fa[0], fb[0], decltype(full)::value);
    if (nk > 1) {
#pragma unroll
      for (int u = 0; u < HALF; ++u) dma1(1, lds0 + BWD_STAGE, u, ids1);
    }
    int kt = 0;
    for (; kt + 2 < nk; ++kt) tile(std::true_type{}, std::true_type{}, full, kt);
    if (kt + 1 < nk) {
      tile(std::true_type{}, std::false_type{}, full, kt);
      ++kt;
    }
    tile(std::false_type{}, std::false_type{}, full, kt);
  };
  if (nk > 0) {
    if (mact == MI) kloop(std::true_type{});
    else kloop(std::false_type{});
  }

  // ---- epilogues ---------------------------------------------------------------------------------------------
  // accumulator (mi, ni), element q: row wm*128 + mi*32 + 8 (q / 4) + 4 (lane / 32) + q % 4, column
  // wn*64 + ni*32 + lane % 32 (G: ni = 0 the gate block, 1 the up block of columns wn*32 + lane % 32).  Each group
  // of four q (q4 = q / 4) is transposed inside its quad of lanes (quad_transpose), after which lane l holds row
  // wm*128 + mi*32 + 8 q4 + 4 (l / 32) + l % 4 at the four consecutive columns from wn*64 + ni*32 + 4 ((l % 32) / 4):
  // one wave store then writes eight rows of 32 consecutive columns (16 bytes per lane for fp32, 8 for bf16)
  auto row_t = [&](int mi, int q4) { return wm * 128 + mi * 32 + 8 * q4 + 4 * (lane >> 5) + (lane & 3); };
  const int col_t = 4 * ((lane & 31) >> 2);  // + wn*64 + ni*32 (G: + wn*32)
  auto quad = [&](const f32x16_t& v, int q4) {
    return quad_transpose(f32x4_t{v[4 * q4], v[4 * q4 + 1], v[4 * q4 + 2], v[4 * q4 + 3]}, lane);
  };
  auto bf16x4 = [&](float v0, float v1, float v2, float v3) {
    return u32x2_t{bf16_bits(v0) | (bf16_bits(v1) << 16), bf16_bits(v2) | (bf16_bits(v3) << 16)};
  };
  if (KIND == BK_H) {
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int r = row_t(mi, q4);
        const int64_t p = sh.rows[r < n_rows ? r : 0];
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) {
          const f32x4_t v = quad(acc[mi][ni], q4);
          const int col = it.nt * 256 + wn * 64 + ni * 32 + col_t;
          if (r < n_rows && col < f) store16_coherent(a.dh + p * f + col, __builtin_bit_cast(u32x4_t, v));
        }
      }
    publish(&a.fh[(int64_t)it.mt * a.n_h + it.nt], a.epoch);
    return true;
  }
  if (KIND == BK_G) {
    // dH of these columns comes from the H item of the 256 columns that hold them
    if (tid == 0) sh.stop = poll_flags(&a.fh[(int64_t)it.mt * a.n_h + (it.nt * 128) / 256], 1, a.epoch, a.budget,
                                       a.status, 1);
    __syncthreads();
    if (sh.stop) {
      if (sh.stop == 1 && tid == 0) set_status(a.status, MOE_ETIMEOUT);
      return false;
    }
    flag_acquire();
    const int col = it.nt * 128 + wn * 32 + col_t;
    const bool saved = a.gu != nullptr;
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        // g and u of row r at columns col ..: the accumulators, transposed, or the forward's stored values (the
        // same bits: the same k-tiles in the same order)
        f32x4_t g4, u4;
        if (!saved) {
          g4 = quad(acc[mi][0], q4);
          u4 = quad(acc[mi][1], q4);
        }
        const int r = row_t(mi, q4);
        if (r >= n_rows) continue;
        const int64_t p = sh.rows[r];
        if (saved) {
          g4 = *(const f32x4_t*)(a.gu + p * 2 * f + col);
          u4 = *(const f32x4_t*)(a.gu + p * 2 * f + f + col);
        }
        const f32x4_t dh = *(const f32x4_t*)(a.dh + p * f + col);
        float hv[4], dg[4], du[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const float g = g4[c], u = u4[c];
          const float sg = __builtin_amdgcn_rcpf(1.0f + __expf(-g));
          const float silu = silu_fast(g);  // the forward's h, bit for bit
          const float dsilu = sg * (1.0f + g * (1.0f - sg));
          hv[c] = silu * u;
          dg[c] = dh[c] * u * dsilu;
          du[c] = dh[c] * silu;
        }
        store8_coherent(a.h + (p * f + col) * 2, bf16x4(hv[0], hv[1], hv[2], hv[3]));
        store8_coherent(a.dgu + (p * 2 * f + col) * 2, bf16x4(dg[0], dg[1], dg[2], dg[3]));
        store8_coherent(a.dgu + (p * 2 * f + f + col) * 2, bf16x4(du[0], du[1], du[2], du[3]));
      }
    publish(&a.fg[(int64_t)it.mt * a.n_g + it.nt], a.epoch);
    return true;
  }
  if (KIND == BK_X) {
    const int64_t tile = (int64_t)it.mt * a.n_x + it.nt;
    if (a.S > 1) {
      // every split stores its fp32 partial sums (thread t keeps its accumulators at float4 chunk
      // ((mi * 2 + ni) * 4 + q4) * 512 + t of its slot) and counts itself in; the last to arrive sums the slots in
      // split order, the same association whichever split completes the tile
      f32x4_t* slot = (f32x4_t*)(a.partial + tile * a.S * (256 * 256)) + (int64_t)it.s * (256 * 256 / 4);
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int ni = 0; ni < NI; ++ni)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            const f32x16_t v = acc[mi][ni];
            const f32x4_t w4 = {v[4 * q4], v[4 * q4 + 1], v[4 * q4 + 2], v[4 * q4 + 3]};
            store16_coherent(slot + ((mi * NI + ni) * 4 + q4) * BWD_THREADS + tid, __builtin_bit_cast(u32x4_t, w4));
          }
      wait_stores();
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
      __syncthreads();
      if (tid == 0) sh.stop = (int)arrive(&a.scount[tile], a.epoch);
      __syncthreads();
      if (sh.stop != a.S - 1) return true;  // not the last split
      flag_acquire();
      const f32x4_t* slots = (const f32x4_t*)(a.partial + tile * a.S * (256 * 256));
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int ni = 0; ni < NI; ++ni)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            const int o = ((mi * NI + ni) * 4 + q4) * BWD_THREADS + tid;
            f32x4_t t = __builtin_nontemporal_load(slots + o);
            for (int sp = 1; sp < a.S; ++sp) t += __builtin_nontemporal_load(slots + (int64_t)sp * (256 * 256 / 4) + o);
            acc[mi][ni][4 * q4] = t[0];
            acc[mi][ni][4 * q4 + 1] = t[1];
            acc[mi][ni][4 * q4 + 2] = t[2];
            acc[mi][ni][4 * q4 + 3] = t[3];
          }
    }
    // bf16 rows: the self owner's rows straight into its buffer, the other owners' into the padded layout
    const int lo = sh.hdr[MT_SELF_LO], ns = sh.hdr[MT_SELF_N], delta = sh.hdr[MT_SELF_DELTA];
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int r = row_t(mi, q4);
        const int p = sh.rows[r < n_rows ? r : 0];
        const bool self = (unsigned)(p - lo) < (unsigned)ns;
        unsigned char* rowp = self ? a.self_recv + (int64_t)(p + delta) * d * 2 : a.dxp + (int64_t)p * d * 2;
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) {
          const f32x4_t v = quad(acc[mi][ni], q4);
          const int col = it.nt * 256 + wn * 64 + ni * 32 + col_t;
          if (r < n_rows && col < d) store8_coherent(rowp + col * 2, bf16x4(v[0], v[1], v[2], v[3]));
        }
      }
    publish(&a.fx[tile], a.epoch);
    return true;
  }
  // W items: the fp32 tile into the weight gradient (read by nobody inside the launch).  Thread 0 claims the
  // workgroup's next tile first, so that the atomic's round trip overlaps these stores
  int nxt = 0;
  if (tid == 0) nxt = (int)(uint32_t)__hip_atomic_fetch_add(a.wclaim, (uint64_t)1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  float* out = KIND == BK_WD ? a.dw2 + (int64_t)e * d * f : a.dw1 + (int64_t)e * 2 * f * d;
  const int out_rows = KIND == BK_WD ? d : 2 * f, out_cols = KIND == BK_WD ? f : d;
  // straight from the accumulators: for each element q, the 4-byte stores of lanes 0-31 and of lanes 32-63 each
  // write 128 consecutive bytes of one row (the quad transpose and 16-byte stores took the DeepSeek-V3-shaped
  // backward 3.6% longer; streaming these stores past the caches made no difference on six workloads)
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int r = it.it * 256 + wm * 128 + mi * 32 + 8 * (q >> 2) + 4 * (lane >> 5) + (q & 3);
#pragma unroll
      for (int ni = 0; ni < NI; ++ni) {
        const int col = it.jt * 256 + wn * 64 + ni * 32 + (lane & 31);
        if (r < out_rows && col < out_cols) out[(int64_t)r * out_cols + col] = acc[mi][ni][q];
      }
    }
  if (tid == 0) sh.next = nxt;
  return true;
}

__global__ __launch_bounds__(BWD_THREADS, 1) void k_bwd_ffn(BwdArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ BwdShared sh;
  launch_acquire();  // drop cache lines older than this launch (the publish protocol in common.h)
  const int C = a.n_cons, tid = threadIdx.x;
  if (blockIdx.x == 0 && tid == 0)  // the W-tile counter starts at zero for this launch
    __hip_atomic_store(a.wclaim, (uint64_t)a.wstamp << 32, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (load_status(a.status) != 0) return;
  if ((a.join || C > 0) && blockIdx.x == 0) consumer_stamp(a.cons);
  const int n_mt = a.scalars[a.sc_nmt];
  // H, G and X items: round-robin over every workgroup, consecutive items on the workgroups of one XCD
  const int n_static = bwd_n_static(a, n_mt);
  const int G = gridDim.x;
  int bid = blockIdx.x;
  if ((G & 7) == 0) bid = (bid & 7) * (G >> 3) + (bid >> 3);
  auto stop_on = [&](int st) {  // after a wait: true when the workgroup must end (status set)
    if (st == 1 && tid == 0) set_status(a.status, MOE_ETIMEOUT);
    return st != 0;
  };
  for (int i = bid; i < n_static; i += G) {
    const BwdItem it = bwd_item(a, n_mt, i);
    __syncthreads();  // the previous item is done with sh
    const int32_t* dsc = a.mtile_desc + (int64_t)it.mt * MOE_MT_FIELDS;
    if (tid < MOE_MT_HDR) sh.hdr[tid] = dsc[tid];
    if (tid < BWD_BM) sh.rows[tid] = dsc[MOE_MT_HDR + tid];
    bool ok = true;
    if (it.kind == BK_X) {  // the (dG | dU) columns of this split: the G items of their 128-column blocks
      if (tid < 64) {
        const int kk = 2 * a.f / a.S, c0 = it.s * kk;
        const uint32_t* fg = a.fg + (int64_t)it.mt * a.n_g;
        const int st = poll_flags_wave([&](int j) { return &fg[((c0 + 128 * j) % a.f) / 128]; }, kk / 128, a.epoch,
                                       a.budget, a.status, 1);
        if (tid == 0) sh.stop = st;
      }
      __syncthreads();
      if (stop_on(sh.stop)) return;
      flag_acquire();
      ok = bwd_tile<BK_X>(a, smem, sh, it);
    } else {
      __syncthreads();
      ok = it.kind == BK_H ? bwd_tile<BK_H>(a, smem, sh, it) : bwd_tile<BK_G>(a, smem, sh, it);
    }
    if (!ok) return;
  }
  // The first C workgroups return dX rows now, while the others start on the weight-gradient tiles (the dX tiles
  // complete with the static items), and take W tiles too once every copy unit is handed out.  (C workgroups
  // returning from the start and running no static items cost the launch more than the return takes on the
  // whole chip after it.)
  if ((int)blockIdx.x < C) consumer_role(a.cons);
  // W tiles: nobody waits on them, and their lengths follow the experts' row counts, so they are handed out at run
  // time from the launch's counter, longest experts first (a static share left some workgroups 20-25% more work
  // than others)
  {
    __syncthreads();
    if (tid < a.E) {
      sh.e_rows[tid] = 0;
      sh.e_first[tid] = 0;
      sh.e_count[tid] = 0;
    }
    __syncthreads();
    for (int t = tid; t < n_mt; t += BWD_THREADS) {
      const int32_t* dsc = a.mtile_desc + (int64_t)t * MOE_MT_FIELDS;
      atomicAdd(&sh.e_rows[dsc[0]], dsc[1]);
      if (dsc[2] == t) {  // the first tile of the expert's run
        sh.e_first[dsc[0]] = t;
        sh.e_count[dsc[0]] = dsc[3];
      }
    }
    __syncthreads();
    if (tid < a.E) {
      int rank = 0;
      for (int e = 0; e < a.E; ++e)
        rank += sh.e_rows[e] > sh.e_rows[tid] || (sh.e_rows[e] == sh.e_rows[tid] && e < tid);
      sh.e_order[rank] = tid;
    }
    const int n_w = a.E * bwd_w_per_expert(a);
    // Each tile's thread 0 claims the workgroup's next tile before its epilogue's stores (bwd_tile), so the
    // atomic's round trip overlaps them; the counter's stamp is looked at only before the first claim (DeepSeek-V3-
    // and Mixtral-shaped and skewed backward 0.7-4% shorter).  Claiming a whole tile ahead held long tiles back
    // from idle workgroups at the end (skewed 8-10% slower); one wait per expert for all of its G flags instead of
    // one per tile for the columns it reads gained nothing.
    if (tid == 0) {
      const uint64_t t0 = moe_clock();
      bool stamped;
      while (!(stamped = (uint32_t)(__hip_atomic_load(a.wclaim, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >> 32) ==
                         a.wstamp) &&
             moe_clock() - t0 <= a.budget)
        __builtin_amdgcn_s_sleep(1);
      if (stamped)
        sh.next = (int)(uint32_t)__hip_atomic_fetch_add(a.wclaim, (uint64_t)1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      else {
        sh.next = -1;
        set_status(a.status, MOE_ETIMEOUT);
      }
    }
    for (;;) {
      __syncthreads();  // the previous item is done with sh (and the table and the claim are complete)
      const int w = sh.next;
      if (w < 0 || w >= n_w) break;
      const BwdItem it = bwd_w_item(a, sh, w);
      // the expert's run of row tiles (none: no rows, a zero tile); WD reads h columns jt*256 .., WGU (dG | dU)
      // columns it*256 ..: their G items in every row tile of the run
      if (tid == 0) {
        sh.run_first = sh.e_first[it.e];
        sh.run_count = sh.e_count[it.e];
        sh.k_rows = sh.e_rows[it.e];
      }
      if (tid < 64) {
        const int c0 = it.kind == BK_WD ? it.jt * 256 : it.it * 256;
        const int nc = (min(c0 + 256, it.kind == BK_WD ? a.f : 2 * a.f) - c0 + 127) / 128;
        const int first = sh.e_first[it.e];
        const int st = poll_flags_wave(
            [&](int j) { return &a.fg[(int64_t)(first + j / nc) * a.n_g + ((c0 + 128 * (j % nc)) % a.f) / 128]; },
            sh.e_count[it.e] * nc, a.epoch, a.budget, a.status, 1);
        if (tid == 0) sh.stop = st;
      }
      __syncthreads();
      if (stop_on(sh.stop)) return;
      flag_acquire();
      const bool ok = it.kind == BK_WD ? bwd_tile<BK_WD>(a, smem, sh, it) : bwd_tile<BK_WGU>(a, smem, sh, it);
      if (!ok) return;
    }
  }
  // with join, every workgroup takes the copy units left once the W tiles are handed out
  if (a.join) consumer_role(a.cons);
}

// dY rows of the padded layout: row p (token t, local expert e of its band) = bf16(w dOut[t]) with w the weight of
// t's slot routed to e (an fp32 product, then bf16).  One wavefront per row, 16-byte lanes.
__global__ __launch_bounds__(256) void k_bwd_dy(const uint16_t* __restrict__ d_out, const int32_t* __restrict__ topk_idx,
                                                const float* __restrict__ topk_w, const int32_t* __restrict__ row_src,
                                                const int32_t* __restrict__ tile_expert, const int32_t* scalars, int M,
                                                int k, int lo, int d, uint16_t* __restrict__ dy) {
  const int64_t n_pad = scalars[SC_MPAD];
  const int lane = threadIdx.x & 63;
  for (int64_t p = blockIdx.x * 4 + (threadIdx.x >> 6); p < n_pad; p += (int64_t)gridDim.x * 4) {
    const int t = row_src[p];
    if (t < 0) continue;  // padding
    const int eg = lo + tile_expert[p / M];
    float w = 0.f;
    for (int j = 0; j < k; ++j)
      if (topk_idx[(int64_t)t * k + j] == eg) w = topk_w[(int64_t)t * k + j];
    const uint4* src = (const uint4*)(d_out + (int64_t)t * d);
    uint4* dst = (uint4*)(dy + p * d);
    constexpr int U = 4;  // chunks per lane whose loads all go out before any is used
    const int rv = d / 8;
    for (int c0 = lane; c0 < rv; c0 += U * 64) {
      uint4 v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) v[u] = c0 + u * 64 < rv ? src[c0 + u * 64] : make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (c0 + u * 64 >= rv) break;
        const uint32_t in[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
        uint32_t o[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float lo16 = __uint_as_float(in[q] << 16) * w, hi16 = __uint_as_float(in[q] & 0xffff0000u) * w;
          o[q] = bf16_bits(lo16) | (bf16_bits(hi16) << 16);
        }
        dst[c0 + u * 64] = make_uint4(o[0], o[1], o[2], o[3]);
      }
    }
  }
}

// The combine's backward, one wave per token (out = sum_j w_j y_j over the token's local slots): dx = bf16 of the sum
// of the slots' returned dX rows in ascending slot order, and the routing weights' gradient dw[t][j] = <dOut_t, y_j>
// over the delivered forward row (0 for slots routed elsewhere).  16-byte loads, two chunks per lane at a time; the
// dOut chunk is loaded once for all the token's slots, and each slot's dot product stays in a register until one
// wave sum at the end.  (A workgroup per token with 2-byte loads and a barrier per slot ran at 1.9 TB/s.)  NT: every
// row read streams past the caches (nontemporal), for row sets larger than the last-level cache.
#define BWD_MAX_K 16
__device__ __forceinline__ uint4 load16(const uint4* p, bool nt) {
  if (!nt) return *p;
  const u32x4_t v = __builtin_nontemporal_load((const u32x4_t*)p);
  return make_uint4(v[0], v[1], v[2], v[3]);
}
template <bool NT>
__global__ __launch_bounds__(256) void k_bwd_combine(const uint16_t* __restrict__ d_out, const int32_t* __restrict__ plan,
                                                     RecvPtrs y_recv, RecvPtrs dx_recv, int T, int T_o, int k, int d,
                                                     uint16_t* __restrict__ dx, float* __restrict__ dw) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const int r = (int)(t / T_o), rv = d / 8;  // 16-byte chunks per row
  int pj[BWD_MAX_K];
#pragma unroll
  for (int j = 0; j < BWD_MAX_K; ++j) pj[j] = j < k ? plan[t * k + j] : -1;
  const uint4* o = (const uint4*)(d_out + t * d);
  const uint4* yb = (const uint4*)y_recv.p[r];
  const uint4* xb = (const uint4*)dx_recv.p[r];
  uint4* dst = (uint4*)(dx + t * d);
  auto lo = [](uint32_t v) { return __uint_as_float(v << 16); };
  auto hi = [](uint32_t v) { return __uint_as_float(v & 0xffff0000u); };
  float dot[BWD_MAX_K];
#pragma unroll
  for (int j = 0; j < BWD_MAX_K; ++j) dot[j] = 0.f;
  constexpr int U = 2;
  for (int c0 = lane; c0 < rv; c0 += U * 64) {
    uint4 ov[U];
    float acc[U][8];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = c0 + u * 64;
      ov[u] = c < rv ? load16(&o[c], NT) : make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[u][i] = 0.f;
    }
#pragma unroll
    for (int j = 0; j < BWD_MAX_K; ++j) {
      if (pj[j] < 0) continue;  // the same for the whole wave
      uint4 yv[U], xv[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = c0 + u * 64;
        yv[u] = c < rv ? load16(&yb[(int64_t)pj[j] * rv + c], NT) : make_uint4(0, 0, 0, 0);
        xv[u] = c < rv ? load16(&xb[(int64_t)pj[j] * rv + c], NT) : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const uint32_t oq[4] = {ov[u].x, ov[u].y, ov[u].z, ov[u].w}, yq[4] = {yv[u].x, yv[u].y, yv[u].z, yv[u].w};
        const uint32_t xq[4] = {xv[u].x, xv[u].y, xv[u].z, xv[u].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          dot[j] += lo(oq[i]) * lo(yq[i]) + hi(oq[i]) * hi(yq[i]);
          acc[u][2 * i] += lo(xq[i]);
          acc[u][2 * i + 1] += hi(xq[i]);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = c0 + u * 64;
      if (c < rv)
        dst[c] = make_uint4(bf16_bits(acc[u][0]) | (bf16_bits(acc[u][1]) << 16),
                            bf16_bits(acc[u][2]) | (bf16_bits(acc[u][3]) << 16),
                            bf16_bits(acc[u][4]) | (bf16_bits(acc[u][5]) << 16),
                            bf16_bits(acc[u][6]) | (bf16_bits(acc[u][7]) << 16));
    }
  }
#pragma unroll
  for (int j = 0; j < BWD_MAX_K; ++j) {
    if (j >= k) break;
    const float sj = pj[j] >= 0 ? wave_sum_f(dot[j]) : 0.f;
    if (lane == 0) dw[t * k + j] = sj;
  }
}

// ---- host side -------------------------------------------------------------------------------------------------

namespace {
void bwd_fill_consumer(ConsumerArgs& c, const BwdLaunch& p, const uint32_t* flags, uint64_t* claim, int n_x) {
  c.y = (const uint4*)p.dx_pad;
  for (int r = 0; r < MOE_MAX_OWNERS; ++r) c.recv.p[r] = r < p.R ? p.dx_recv[r] : nullptr;
  c.seg_desc = p.L->seg_desc;
  c.seg_mtiles = p.L->seg_mtiles;
  c.seg_sched = p.L->seg_sched;
  c.scalars = p.L->scalars;
  c.status = p.L->status;
  c.flags = flags;
  c.claim = claim;
  c.stamp = next_stamp();
  c.epoch = p.epoch;
  c.n_nt = n_x;
  c.row_vec = p.d * 2 / 16;
  c.budget = p.watchdog_ticks;
  c.ts = nullptr;
  c.self_rank = p.self_rank;
  c.obs = nullptr;
}

// the dX items' k-splits: an item's k about d (2f / S ~ d, as long as the H and G items'), each split a multiple of
// 128 columns of (dG | dU) (the G items' width), at most 4: the last split to arrive reads every slot alone, and
// 7 splits on the Mixtral-like shard (2 MB of partial sums per tile) cost the dX items 17% more CU time than 4
int bwd_splits(int d, int f) {
  const int want = std::min(4, std::max(1, (4 * f + d) / (2 * d)));
  for (int c = want; c > 1; --c)
    if ((2 * f / 128) % c == 0) return c;
  return 1;
}

struct BwdCarve {
  int64_t fh, fg, fx, scount, partial, claim, wclaim, total;  // 4-byte words
};
BwdCarve bwd_carve(int d, int f, int64_t cap_mtiles) {
  auto up = [](int64_t v) { return (v + 63) / 64 * 64; };
  const int64_t n_h = (f + 255) / 256, n_g = f / 128, n_x = (d + 255) / 256, S = bwd_splits(d, f);
  BwdCarve c;
  c.fx = 0;  // the consumer's flags first (consumer_role indexes them from its flag pointer)
  c.fh = up(cap_mtiles * n_x);
  c.fg = c.fh + up(cap_mtiles * n_h);
  c.scount = c.fg + up(cap_mtiles * n_g);
  c.partial = c.scount + up(2 * cap_mtiles * n_x);
  c.claim = c.partial + (S > 1 ? cap_mtiles * n_x * S * 256 * 256 : 0);
  c.wclaim = c.claim + 2;
  c.total = c.wclaim + 2;
  return c;
}
}  // namespace

int64_t bwd_flag_words(int d, int f, int64_t cap_mtiles) { return bwd_carve(d, f, cap_mtiles).total; }

int launch_bwd_dy(const BwdLaunch& p, hipStream_t st) {
  int64_t blocks = (p.L->cap_rows + 3) / 4;
  if (blocks > 4096) blocks = 4096;
  if (blocks > 0)
    hipLaunchKernelGGL(k_bwd_dy, dim3((unsigned)blocks), dim3(256), 0, st, (const uint16_t*)p.d_out, p.topk_idx,
                       p.topk_w, p.L->row_src, p.L->tile_expert, p.L->scalars, p.M, p.k, p.lo, p.d,
                       (uint16_t*)p.dy_pad);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_bwd_ffn(const BwdLaunch& p, int grid, int n_cons, int join, hipStream_t st, hipEvent_t ev0, hipEvent_t ev1) {
  const BwdCarve c = bwd_carve(p.d, p.f, p.cap_mtiles);
  BwdArgs a;
  a.x = (const unsigned char*)p.x_pad;
  a.w1 = (const unsigned char*)p.w_gate_up;
  a.w2 = (const unsigned char*)p.w_down;
  a.dy = (const unsigned char*)p.dy_pad;
  a.dh = p.dh_ws;
  a.h = (unsigned char*)p.h_ws;
  a.dgu = (unsigned char*)p.dgu_ws;
  a.gu = p.gu;
  a.dxp = (unsigned char*)p.dx_pad;
  a.self_recv = (unsigned char*)p.dx_recv[p.self_rank];
  a.dw1 = p.dw_gate_up;
  a.dw2 = p.dw_down;
  a.d = p.d;
  a.f = p.f;
  a.E = p.E;
  a.S = bwd_splits(p.d, p.f);
  a.n_h = (p.f + 255) / 256;
  a.n_g = p.f / 128;
  a.n_x = (p.d + 255) / 256;
  a.mtile_desc = p.L->mtile_desc;
  a.mt_order = p.L->mt_order;
  a.scalars = p.L->scalars;
  a.sc_nmt = SC_NR + p.R;
  a.status = p.L->status;
  a.fh = p.flags + c.fh;
  a.fg = p.flags + c.fg;
  a.fx = p.flags + c.fx;
  a.scount = (uint64_t*)(p.flags + c.scount);
  a.partial = (float*)(p.flags + c.partial);
  a.wclaim = (uint64_t*)(p.flags + c.wclaim);
  a.wstamp = next_stamp();
  a.epoch = p.epoch;
  a.budget = p.watchdog_ticks;
  a.n_cons = n_cons;
  a.join = join;
  bwd_fill_consumer(a.cons, p, p.flags + c.fx, (uint64_t*)(p.flags + c.claim), a.n_x);
  hipExtLaunchKernelGGL(k_bwd_ffn, dim3(grid), dim3(BWD_THREADS), 2 * BWD_STAGE, st, ev0, ev1, 0, a);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

__global__ __launch_bounds__(256) void k_bwd_consumer(ConsumerArgs c) {
  launch_acquire();
  if (blockIdx.x == 0) consumer_stamp(c);
  consumer_role(c);
}

int launch_bwd_consumer(const BwdLaunch& p, int n_cons, hipStream_t st, hipEvent_t ev0, hipEvent_t ev1) {
  const BwdCarve c = bwd_carve(p.d, p.f, p.cap_mtiles);
  ConsumerArgs cons;
  bwd_fill_consumer(cons, p, p.flags + c.fx, (uint64_t*)(p.flags + c.claim), (p.d + 255) / 256);
  hipExtLaunchKernelGGL(k_bwd_consumer, dim3(n_cons), dim3(256), 0, st, ev0, ev1, 0, cons);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_bwd_combine(const BwdLaunch& p, int T_o, int G, const int32_t* plan, void* const* y_recv, void* dx,
                       float* dw, hipStream_t st) {
  RecvPtrs yr, xr;
  for (int r = 0; r < MOE_MAX_OWNERS; ++r) {
    yr.p[r] = r < p.R ? y_recv[r] : nullptr;
    xr.p[r] = r < p.R ? p.dx_recv[r] : nullptr;
  }
  const int64_t T = (int64_t)p.R * T_o;
  // rows read and written at the routing's expected share of local slots (T k E_l / G): dOut, y and dX rows, dx.
  // Past the 256 MB last-level cache the reads stream (DeepSeek-V3-like shard, ~0.9 GB: 253 -> 215 us)
  const bool nt = (2.0 * T * p.k * p.E / G + 2.0 * T) * p.d * 2.0 > 256.0 * 1024 * 1024;
  if (T > 0) {
    const dim3 grid((unsigned)((T + 3) / 4));
    if (nt)
      hipLaunchKernelGGL(k_bwd_combine<true>, grid, dim3(256), 0, st, (const uint16_t*)p.d_out, plan, yr, xr, (int)T,
                         T_o, p.k, p.d, (uint16_t*)dx, dw);
    else
      hipLaunchKernelGGL(k_bwd_combine<false>, grid, dim3(256), 0, st, (const uint16_t*)p.d_out, plan, yr, xr, (int)T,
                         T_o, p.k, p.d, (uint16_t*)dx, dw);
  }
  return hipGetLastError() == hipSuccess ? 0 : -1;
}
