// Producer: persistent grouped SwiGLU expert FFN on CDNA4 MFMA (review page: "The pith" and "Core claim":
// one rank-wide persistent GEMM over all local experts that publishes a readiness flag per output tile;
// "What carries the argument": remote-bound tiles first).
//
//   GEMM1 (GLU):  h[rows, f] = bf16(silu(x Wg^T) * (x Wu^T)),  one tile = BN/2 gate + BN/2 up columns
//   GEMM2:        y[rows, d] = h Wd^T, then the y tile's flag = epoch once its stores are visible device-wide
// bf16: both GEMMs are one persistent launch (k_ffn_bf16) over a list of GEMM1 tiles and GEMM2 k-splits, each
// GEMM2 item waiting for the flags of the h tiles it reads; fp32: two launches (k_gemm), the second publishing.
// The first C workgroups of the publishing launch are the consumer partition (consumer.h): round-robin dispatch
// puts workgroup b on XCD b % 8, so C consumers spread over the XCDs, one per CU, co-resident with the producers
// by construction; every producer workgroup joins the return once its own items are done.
// Row tiles are the layout's GEMM row tiles: up to BM real rows of one expert, each expert's rows packed into
// consecutive tiles, so padding rows cost nothing.  Items (row tile, column tile) are visited window by window
// (band_window row tiles) for weight reuse, and consecutive items go to workgroups on the same XCD.  When the
// producers' last round is at most half full, its GEMM2 items run as two half-width items each.  A tile that one
// item completes is published at the start of the workgroup's next item (before any of its waits), so that the
// stores drain under that item's first loads.
#include <hip/hip_ext.h>

#include <algorithm>
#include <atomic>
#include <mutex>
#include <type_traits>
#include <vector>

#include "common.h"
#include "consumer.h"
#include "item_list.h"
#include "launch.h"
#include "tile_util.h"


template <typename T>
struct Mfma;

// v_mfma_f32_32x32x16_bf16: lane l holds row (l % 32) of A and column (l % 32) of B, 8 consecutive k at
// 8 * (l / 32); D[i][j] with j = l % 32 and i = 8 * (reg / 4) + 4 * (l / 32) + reg % 4.
template <>
struct Mfma<bf16_t> {
  static constexpr int KM = 16, EPL = 8, BK = 64;
  typedef bf16x8_t frag;
  static __device__ __forceinline__ frag load(const bf16_t* p) {
    return __builtin_bit_cast(frag, *(const u32x4_t*)p);
  }
  static __device__ __forceinline__ f32x16_t mma(frag a, frag b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ bf16_t out(float v) { return f32_to_bf16(v); }
};

// v_mfma_f32_32x32x2_f32: one k per lane at (l / 32); same D layout.
template <>
struct Mfma<float> {
  static constexpr int KM = 2, EPL = 1, BK = 32;
  typedef float frag;
  static __device__ __forceinline__ frag load(const float* p) { return *p; }
  static __device__ __forceinline__ f32x16_t mma(frag a, frag b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ float out(float v) { return v; }
};

struct GemmArgs {
  const void* A;  // [rows, K]: x_pad (GEMM1) or h (GEMM2)
  const void* W;  // [E, w_rows, K]
  void* C;        // [rows, ldc]
  int K, w_rows, ldc, f;
  int n_nt;  // column tiles
  const int32_t* mtile_desc;
  const int32_t* scalars;
  int sc_nmt;
  const int32_t* status;
  uint32_t* flags;
  uint32_t epoch;
  int window;
  uint64_t* ts;
  int n_cons;  // GEMM2 only: workgroups [0, n_cons) run the consumer role
  ConsumerArgs cons;
  void* self_recv;  // GEMM2 only: its rows of the self-owned groups go straight to the self owner's buffer
};

__device__ __forceinline__ float silu_f32(float g) { return g / (1.0f + __expf(-g)); }

template <typename T, int BM, int BN, int WGM, int WGN, bool GLU, bool PUBLISH>
__global__ __launch_bounds__(WGM* WGN * 64) void k_gemm(GemmArgs a) {
  using Tr = Mfma<T>;
  constexpr int BK = Tr::BK, NTHR = WGM * WGN * 64;
  constexpr int VEC = 16 / sizeof(T);  // elements per 16-byte chunk
  constexpr int LDK = BK + VEC;        // padded LDS row stride (elements)
  constexpr int WM = BM / WGM, WN = BN / WGN, MI = WM / 32, NI = WN / 32;
  constexpr int CPR = BK / VEC;     // chunks per tile row
  constexpr int RPP = NTHR / CPR;   // tile rows per load pass
  constexpr int PA = BM / RPP, PB = BN / RPP;
  constexpr int OUT_BN = GLU ? BN / 2 : BN;  // output columns per tile
  static_assert(!GLU || NI % 2 == 0, "GLU pairs gate and up blocks");
  static_assert(BM % RPP == 0 && BN % RPP == 0 && BM <= MOE_MT_ROWS, "tile shape");

  __shared__ __align__(16) T sA[2][BM * LDK];
  __shared__ __align__(16) T sB[2][BN * LDK];
  __shared__ int s_rows[BM];
  __shared__ int s_hdr[MOE_MT_HDR];

  if (PUBLISH) launch_acquire();
  if (PUBLISH && a.n_cons > 0 && blockIdx.x == 0) consumer_stamp(a.cons);
  if (PUBLISH && (int)blockIdx.x < a.n_cons) {
    consumer_role(a.cons);
    return;
  }
  if (load_status(a.status) != 0) return;
  const int n_mt = a.scalars[a.sc_nmt];
  const int n_items = n_mt * a.n_nt;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WGN, wn = wave % WGN;
  const int n_cons = PUBLISH ? a.n_cons : 0;
  const int G = gridDim.x - n_cons;  // producer workgroups
  int bid = blockIdx.x - n_cons;
  // producers of one XCD (workgroup index mod 8) take consecutive items, which share a weight tile
  if ((G & 7) == 0 && (n_cons & 7) == 0) bid = (bid & 7) * (G >> 3) + (bid >> 3);
  const T* __restrict__ A = (const T*)a.A;
  const T* __restrict__ Wt = (const T*)a.W;
  T* __restrict__ C = (T*)a.C;
  const int K = a.K;
  const int nk = K / BK;
  const int cr = tid / CPR, cc = (tid % CPR) * VEC;
  bool first = true;

  for (int item = bid; item < n_items; item += G) {
    const int per_win = a.window * a.n_nt;
    const int w = item / per_win, j = item - w * per_win;
    const int mt0 = w * a.window;
    const int Wc = min(a.window, n_mt - mt0);
    const int nt = j / Wc, mt = mt0 + (j - nt * Wc);

    __syncthreads();  // previous item finished with LDS and the header
    {
      const int32_t* dsc = a.mtile_desc + (int64_t)mt * MOE_MT_FIELDS;
      if (tid < MOE_MT_HDR) s_hdr[tid] = dsc[tid];
      for (int i = tid; i < BM; i += NTHR) s_rows[i] = dsc[MOE_MT_HDR + i];
    }
    if (PUBLISH && a.ts != nullptr && first && tid == 0)
      atomicMin((unsigned long long*)&a.ts[0], (unsigned long long)moe_clock());
    first = false;
    __syncthreads();
    const int e = s_hdr[0], n_rows = s_hdr[1];

    const T* pa[PA];
#pragma unroll
    for (int p = 0; p < PA; ++p) {
      const int r = p * RPP + cr;
      pa[p] = A + (int64_t)(r < n_rows ? s_rows[r] : s_rows[0]) * K + cc;  // absent rows read a real row
    }
    const T* pb[PB];
    const T* wbase = Wt + (int64_t)e * a.w_rows * K;
#pragma unroll
    for (int p = 0; p < PB; ++p) {
      const int i = p * RPP + cr;
      int wrow;
      if (GLU) wrow = i < BN / 2 ? nt * (BN / 2) + i : a.f + nt * (BN / 2) + (i - BN / 2);
      else wrow = nt * BN + i;
      pb[p] = wbase + (int64_t)wrow * K + cc;
    }
    bool mvalid[MI];
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) mvalid[mi] = wm * WM + mi * 32 < n_rows;

    f32x16_t acc[MI][NI];
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int ni = 0; ni < NI; ++ni)
#pragma unroll
        for (int q = 0; q < 16; ++q) acc[mi][ni][q] = 0.f;

    // Absent rows (past the tile's row count) read the tile's first row instead; their outputs are never
    // stored, and rows are independent in both GEMMs.
    {
      u32x4_t ra[PA], rb[PB];
#pragma unroll
      for (int p = 0; p < PA; ++p) ra[p] = *(const u32x4_t*)(pa[p]);
#pragma unroll
      for (int p = 0; p < PB; ++p) rb[p] = *(const u32x4_t*)(pb[p]);
#pragma unroll
      for (int p = 0; p < PA; ++p) *(u32x4_t*)&sA[0][(p * RPP + cr) * LDK + cc] = ra[p];
#pragma unroll
      for (int p = 0; p < PB; ++p) *(u32x4_t*)&sB[0][(p * RPP + cr) * LDK + cc] = rb[p];
    }
    __syncthreads();

    for (int kt = 0; kt < nk; ++kt) {
      const int cur = kt & 1;
      const bool more = kt + 1 < nk;
      u32x4_t ra[PA], rb[PB];
      if (more) {
        const int k0 = (kt + 1) * BK;
#pragma unroll
        for (int p = 0; p < PA; ++p) ra[p] = *(const u32x4_t*)(pa[p] + k0);
#pragma unroll
        for (int p = 0; p < PB; ++p) rb[p] = *(const u32x4_t*)(pb[p] + k0);
      }
      const T* cA = sA[cur];
      const T* cB = sB[cur];
#pragma unroll
      for (int s = 0; s < BK / Tr::KM; ++s) {
        const int kk = s * Tr::KM + (lane >> 5) * Tr::EPL;
        typename Tr::frag fa[MI], fb[NI];
#pragma unroll
        for (int mi = 0; mi < MI; ++mi) fa[mi] = Tr::load(&cA[(wm * WM + mi * 32 + (lane & 31)) * LDK + kk]);
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) {
          int row;
          if (GLU) row = ni < NI / 2 ? wn * (WN / 2) + ni * 32 : BN / 2 + wn * (WN / 2) + (ni - NI / 2) * 32;
          else row = wn * WN + ni * 32;
          fb[ni] = Tr::load(&cB[(row + (lane & 31)) * LDK + kk]);
        }
#pragma unroll
        for (int mi = 0; mi < MI; ++mi) {
          if (!mvalid[mi]) continue;
#pragma unroll
          for (int ni = 0; ni < NI; ++ni) acc[mi][ni] = Tr::mma(fa[mi], fb[ni], acc[mi][ni]);
        }
      }
      if (more) {
        const int nxt = cur ^ 1;
#pragma unroll
        for (int p = 0; p < PA; ++p) *(u32x4_t*)&sA[nxt][(p * RPP + cr) * LDK + cc] = ra[p];
#pragma unroll
        for (int p = 0; p < PB; ++p) *(u32x4_t*)&sB[nxt][(p * RPP + cr) * LDK + cc] = rb[p];
      }
      __syncthreads();
    }

    // epilogue: store the tile's real rows (the second GEMM's self-owned rows into the self owner's buffer)
    constexpr int NO = GLU ? NI / 2 : NI;
    const int self_lo = s_hdr[MT_SELF_LO], self_n = PUBLISH ? s_hdr[MT_SELF_N] : 0, self_delta = s_hdr[MT_SELF_DELTA];
    T* __restrict__ Cs = (T*)a.self_recv;
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
      if (!mvalid[mi]) continue;
#pragma unroll
      for (int ni = 0; ni < NO; ++ni) {
        const int col = nt * OUT_BN + (GLU ? wn * (WN / 2) : wn * WN) + ni * 32 + (lane & 31);
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const int row = wm * WM + mi * 32 + (q >> 2) * 8 + (lane >> 5) * 4 + (q & 3);
          if (row < n_rows) {
            const int64_t grow = s_rows[row];
            float v = acc[mi][ni][q];
            if (GLU) v = silu_f32(v) * acc[mi][ni + NI / 2][q];
            if (PUBLISH && (uint32_t)(grow - self_lo) < (uint32_t)self_n) Cs[(grow + self_delta) * a.ldc + col] = Tr::out(v);
            else C[grow * a.ldc + col] = Tr::out(v);
          }
        }
      }
    }
    if (PUBLISH) {
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");  // this thread's tile stores, agent-visible
      __syncthreads();
      if (tid == 0) {
        __hip_atomic_store(&a.flags[(int64_t)mt * a.n_nt + nt], a.epoch, __ATOMIC_RELEASE,
                           __HIP_MEMORY_SCOPE_AGENT);
        if (a.ts != nullptr) atomicMax((unsigned long long*)&a.ts[1], (unsigned long long)moe_clock());
      }
    }
  }
  // then every producer returns segments until no copy unit is left
  if (PUBLISH && n_cons > 0) consumer_role(a.cons);
}

// ---- bf16 GEMM: 256-row tiles, direct global->LDS loads ------------------------------------------------
//
// Workgroup tile 256 x BN x 64 (k), 8 waves (two per SIMD) in (8 / (BN / 64)) x (BN / 64), wave tile
// (64 * BN / 256 ... 128) x 64: MI x 2 MFMA blocks of 32 x 32, accumulators in AGPRs.  Two waves per SIMD, not
// one: a wave's global->LDS loads go out at a bounded rate (about 30 GB/s per CU from four waves whatever the
// number in flight, 75 GB/s from eight, measured from L2-resident data), and a 256 x 256 tile at the MFMA rate
// needs about 45 GB/s per CU at the clock this chip holds under a dense bf16 load.  Operand tiles are staged in
// LDS without padding, 128 bytes per row; a 16-byte k-chunk c of row r sits at slot c ^ swz(r),
// swz(r) = (r & 7) ^ ((r >> 3) & 1), so the 16-byte fragment reads of 16 consecutive rows hit distinct banks.
// global_load_lds_dwordx4 moves each 16-byte chunk straight from global memory into its swizzled LDS slot (one
// wave instruction fills 8 rows, 1 KB).
//
// Pipeline, two LDS stages, one barrier per k-tile.  A k-tile is four k-steps of MI x 2 MFMAs per wave; the
// fragments of k-step s+1 are read while the MFMAs of k-step s run.  The barrier sits between k-steps 2 and
// 3 of k-tile kt: past it, k-tile kt+1 is in LDS for every wave (its first fragments are read during
// k-step 3) and no wave reads the stage of kt any more, so the loads of k-tile kt+2 go into that stage, half
// in k-step 3 of kt and half in k-step 0 of kt+1.  Every load thus has about three k-steps to land, and the
// address unit sees an even trickle of 1 KB requests rather than one burst.  MFMAs, LDS reads and loads are
// placed one group at a time (sched_barrier between groups), so the schedule is the one written here.
//
// The loads are issued from inline assembly and the per-k-tile wait is an explicit "vmcnt(0); s_barrier":
// the compiler's own waitcnt insertion cannot tell an LDS-DMA store from the fragment reads of the other stage
// and would drain every load in flight before each LDS read, serialising loads and MFMAs.  The stage
// discipline makes that unnecessary: a stage is written only after the barrier that ends every read of it.

#define FFN_THREADS 512  // 8 waves, two per SIMD
#define FFN_WAVES (FFN_THREADS / 64)



// The expert FFN as one persistent launch.  Work items:
//   GEMM1 item (row tile mt, column tile nt): h[rows, nt*BN1/2 ...] = bf16(silu(x Wg^T) * (x Wu^T)), then
//     flags1[mt][nt] = epoch;
//   GEMM2 item (mt, nt, split s): the k-tiles of split s of y[rows, nt*BN2 ...] = h Wd^T, after acquiring the
//     flags1 of the h columns that split reads.  With S > 1 splits, each split stores fp32 partial sums and
//     counts itself in; the last to arrive adds the partial sums in split order, stores the bf16 y tile and
//     publishes flags2[mt][nt], which the consumer waits on.
// The list and who runs which item are in item_list.h: GEMM2 items go window by window over the row tiles in
// remote-first order (every row tile holding a row bound for another owner before every row tile of self-owned
// rows only), so row tiles complete (and are returned) one window after another during the second part of the
// launch.  Every wait is on an item earlier in the list, so the lowest unfinished item can always run: the waits
// end while every workgroup is resident, and a spin budget bounds them otherwise.

struct FusedArgs {
  const unsigned char* x;   // x_pad [cap_rows, d]
  const unsigned char* w1;  // [E_l, 2f, d]
  const unsigned char* w2;  // [E_l, d, f]
  unsigned char* h;         // [cap_rows, f]
  unsigned char* y;         // y_pad [cap_rows, d]
  int d, f;
  int n_nt1, n_nt2, S, window;
  int interleave;  // item order: 0 = GEMM1 first, 1 = interleaved windows
  int halves;      // the half-width final round is allowed
  int item_begin, item_end;  // this launch runs the list indices in [item_begin, item_end) (one chunk of the list)
  const int32_t* mtile_desc;
  const int32_t* mt_order;  // [n_mt] row tile at each position of the list (remote-bound row tiles first), or
                            // null: row-tile numbering
  const int32_t* scalars;
  int sc_nmt;
  int32_t* status;
  uint32_t* flags2;  // [cap_mtiles][n_nt2]: y tile published (the consumer's flags)
  uint32_t* flags1;  // [cap_mtiles][n_nt1]: h tile finished
  uint64_t* scount;  // [cap_mtiles][n_nt2]: splits of a y tile that have stored their partial sums
  float* partial;    // [cap_mtiles][n_nt2][S][256 * BN2]
  uint32_t epoch;
  uint64_t budget;
  uint64_t* ts;
  int n_cons;      // consumer workgroups; -1: picked by the launch (ffn_adaptive_consumers)
  int join;        // the launch runs the return: every workgroup takes copy units once its own items are done
  int E;           // local experts (the interleave rule, when the launch picks the partition)
  uint32_t* obs;   // the partition record (MOE_OBS_WORDS words, see obs_*), or null
  // dispatch landing inside the launch (xtok non-null): the token rows of x_pad are copied here, row tile by row tile
  const unsigned char* xtok;  // token rows X [T, d]
  float* gu;                  // null, or [cap_rows, 2f] fp32: the first GEMM's items store g | u of their rows here
  const int32_t* row_src;     // padded row -> token row
  uint32_t* flags0;           // [cap_mtiles]: the row tile's input rows have landed
  uint64_t* gcount;           // [cap_mtiles]: landed units of the row tile (epoch << 32 | count)
  uint64_t* gclaim;           // landing units handed out: stamp << 32 | count
  uint32_t gstamp;
  ConsumerArgs cons;
  unsigned char* self_recv;  // the self owner's buffer: y rows of the self-owned groups go straight there
};

// The partition record in the flag buffer (64-bit fields at even words): [0] arrival counter of this call's
// workgroups (the last one resets it; a call that fails leaves a count the next calls absorb), [2] ~(first producer item start), [4] last producer item end, [6] bytes the
// consumer role copied, [8] its copy ticks summed over workgroups; [10] producers' flops per CU-tick and [11]
// consumers' bytes per CU-tick (fp32, running estimates from earlier calls), [12] the partition of the last call,
// [13] bit 0 / bit 1 set once [10] / [11] hold observations.
__device__ __forceinline__ unsigned long long* obs64(uint32_t* obs, int w) { return (unsigned long long*)(obs + w); }

// All threads of the workgroup: wait until the n flags equal epoch, then acquire (compiler ordering; see the
// publish protocol in common.h).  False if the spin budget ran
// out (status set to MOE_ETIMEOUT) or another workgroup reported an error.
__device__ bool wait_flags(const uint32_t* fl, int n, uint32_t epoch, uint64_t budget, int32_t* status, int* s_stop) {
  __syncthreads();  // every thread has read *s_stop of the previous wait
  if (threadIdx.x < 64) {  // a producer waits briefly
    const int st = poll_flags_wave([&](int j) { return &fl[j]; }, n, epoch, budget, status, 1);
    if (threadIdx.x == 0) *s_stop = st;
  }
  __syncthreads();
  if (*s_stop) {
    if (*s_stop == 1 && threadIdx.x == 0) set_status(status, MOE_ETIMEOUT);
    return false;
  }
  flag_acquire();  // no stale copies to drop: the publish protocol in common.h
  return true;
}

// Results that other workgroups read inside this launch (h tiles, split partial sums, y tiles) are written with
// agent-scope atomic stores: on this chip those are coherent across the XCDs' separate L2 caches (they carry the
// device-scope cache policy), and a store's completion, which s_waitcnt vmcnt waits for, means it is visible
// device-wide.  Publishing is then: every thread's stores completed (a release fence at workgroup scope, which is
// that vmcnt(0), and the barrier), then the flag, an agent-scope atomic store.  An agent-scope release fence would
// write back the whole L2 of the XCD instead, once per published tile, which stalls every workgroup on that XCD
// (nothing the tile needs is dirty in L2: its data went out with device-scope stores).  The reader's side is in
// common.h.
typedef float f32x8_t __attribute__((ext_vector_type(8)));

// 16 fp32 partial sums of one thread in one 32 x 32 accumulator block (the layout the splits store them in:
// float4 chunk q4 of block b of thread t at (b * 4 + q4) * FFN_THREADS + t)
__device__ __forceinline__ f32x16_t load_block16(const f32x4_t* src) {
  constexpr int T = FFN_THREADS;
  const f32x4_t q0 = __builtin_nontemporal_load(src), q1 = __builtin_nontemporal_load(src + T);
  const f32x4_t q2 = __builtin_nontemporal_load(src + 2 * T), q3 = __builtin_nontemporal_load(src + 3 * T);
  const f32x8_t h0 = __builtin_shufflevector(q0, q1, 0, 1, 2, 3, 4, 5, 6, 7);
  const f32x8_t h1 = __builtin_shufflevector(q2, q3, 0, 1, 2, 3, 4, 5, 6, 7);
  return (f32x16_t)__builtin_shufflevector(h0, h1, 0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15);
}

// Stores the real rows of a 256 x OUT_BN bf16 tile staged in LDS (16-byte chunk ch of row r at chunk ch ^ (r & 7)):
// row r, at padded row p = s_rows[r], goes to base + p * ldc elements, or to dst.alt + (p + dst.delta) * ldc if p
// is in the self-owned range of dst; 4 chunks per thread at a time (their LDS reads first, then their stores, so
// neither latency is paid per chunk; 8 at a time held more registers and ran 1-2% slower).
template <int OUT_BN>
__device__ __forceinline__ void store_rows(const unsigned char* smem, unsigned char* base, int64_t ldc,
                                           const int* s_rows, int n_rows, int tid, const RowDst& dst) {
  constexpr int BM = 256, OUT_ROW = OUT_BN * 2, CPR = OUT_ROW / 16, NT = FFN_THREADS;
  constexpr int ITER = BM * CPR / NT, UN = ITER < 4 ? ITER : 4;
  static_assert(ITER >= 1 && ITER % UN == 0, "store loop unroll");
#pragma unroll 1
  for (int i0 = 0; i0 < ITER; i0 += UN) {
    u32x4_t v[UN];
#pragma unroll
    for (int u = 0; u < UN; ++u) {
      const int idx = tid + (i0 + u) * NT, row = idx / CPR, ch = idx - row * CPR;
      v[u] = *(const u32x4_t*)(smem + row * OUT_ROW + ((ch ^ (row & 7)) << 4));
    }
#pragma unroll
    for (int u = 0; u < UN; ++u) {
      const int idx = tid + (i0 + u) * NT, row = idx / CPR, ch = idx - row * CPR;
      if (row < n_rows) {
        const int p = s_rows[row];
        const bool self = (unsigned)(p - dst.lo) < (unsigned)dst.n;
        unsigned char* b = self ? dst.alt : base;
        store16_coherent(b + (int64_t)(self ? p + dst.delta : p) * ldc * 2 + ch * 16, v[u]);
      }
    }
  }
}

// The sum of split-K y tile (mt, nt), BN columns wide, by the item that completed it: the splits' fp32 partial
// sums added in split order, y = ((p_0 + p_1) + ...) + p_{S-1} (the same association whichever item completes the
// tile, so the result is the same on every call and in every mode), rounded to bf16 into LDS, then the tile's real
// rows stored and its flag published.  Every thread's own partial sums were stored like the others', so all slots
// are read back.  With the split count fixed at compile time, every slot of a 32 x 32 block is loaded in one go, D
// blocks ahead of the one being summed, so about D round trips of the reads are in flight instead of one; other
// split counts sum one block and split at a time.
template <int BN>
__device__ __forceinline__ void reduce_tile(const FusedArgs& a, unsigned char* smem, const int* s_rows,
                                            const int* s_hdr, int n_rows, int mt, int nt) {
  constexpr int BM = 256, WGN = BN / 64, WGM = FFN_WAVES / WGN, WM = BM / WGM, MI = WM / 32, NI = 2, NB = MI * NI;
  constexpr int OUT_ROW = BN * 2, SLOT4 = BM * BN / 4;
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int lane = tid & 63, wave = tid >> 6, wm = wave / WGN, wn = wave % WGN;
  const int64_t tile = (int64_t)mt * a.n_nt2 + nt;
  const f32x4_t* slots = (const f32x4_t*)(a.partial + tile * a.S * (BM * BN));
  auto stage = [&](int b, const f32x16_t& v) {  // block b of this thread's accumulators, as bf16, into LDS
    const int mi = b / NI, ni = b - mi * NI, col = wn * 64 + ni * 32 + (lane & 31);
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int row = wm * WM + mi * 32 + (q >> 2) * 8 + (lane >> 5) * 4 + (q & 3);
      const int chunk = (col >> 3) ^ (row & 7);
      *(__bf16*)(smem + row * OUT_ROW + chunk * 16 + (col & 7) * 2) = (__bf16)v[q];  // round to nearest even
    }
  };
  auto ring_sum = [&](auto S_) {
    constexpr int SC = decltype(S_)::value, D = SC <= 2 ? 2 : 1;
    f32x16_t ring[D + 1][SC];
    auto load = [&](int b) {
#pragma unroll
      for (int sp = 0; sp < SC; ++sp)
        ring[b % (D + 1)][sp] = load_block16(slots + (int64_t)sp * SLOT4 + b * 4 * FFN_THREADS + tid);
    };
#pragma unroll
    for (int b = 0; b < D; ++b) load(b);
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      if (b + D < NB) load(b + D);
      __builtin_amdgcn_sched_barrier(0);
      f32x16_t t = ring[b % (D + 1)][0];
#pragma unroll
      for (int sp = 1; sp < SC; ++sp) t += ring[b % (D + 1)][sp];
      stage(b, t);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  if (a.S == 2) ring_sum(std::integral_constant<int, 2>{});
  else if (a.S == 3) ring_sum(std::integral_constant<int, 3>{});
  else if (a.S == 4) ring_sum(std::integral_constant<int, 4>{});
  else {
#pragma unroll 1
    for (int b = 0; b < NB; ++b) {
      const f32x4_t* src = slots + b * 4 * FFN_THREADS + tid;
      f32x16_t t = load_block16(src);
      for (int sp = 1; sp < a.S; ++sp) t += load_block16(src + (int64_t)sp * SLOT4);
      stage(b, t);
    }
  }
  __syncthreads();
  store_rows<BN>(smem, a.y + (int64_t)nt * BN * 2, a.d, s_rows, n_rows, tid, self_dst(a.self_recv, s_hdr, (int64_t)nt * BN * 2));
  publish(&a.flags2[tile], a.epoch);
  if (a.ts != nullptr && tid == 0) atomicMax((unsigned long long*)&a.ts[1], (unsigned long long)moe_clock());
}

// One item: output tile (row tile with rows s_rows[0, n_rows) of expert e, column tile nt), k-tiles of
// split s.  GLU: the first GEMM (A = x_pad rows, B = gate rows nt*BN/2.. and up rows f + nt*BN/2..); else the
// second (A = h rows, B = down-projection rows col0.., output columns col0..), whose y tile (mt, nt) is complete
// after `target` items have counted themselves in (1: this item alone).  HALF_TILE: this item computes half (`half`,
// 0 or 1) of a y tile twice as wide; its partial sums go to their places in that tile's layout.  A tile that this
// item completes alone (an h tile, an unsplit y tile) is not published here: its flag goes to *s_pend (*s_pend_y:
// a y tile), and the workgroup publishes it once the stores have completed, at the start of its next item or after
// its last, so that the stores drain while the next item's row list loads.  False if a wait gave up (the
// workgroup must exit).
template <int BN, bool GLU, bool HALF_TILE = false>
__device__ __forceinline__ bool ffn_tile(const FusedArgs& a, unsigned char* smem, const int* s_rows, const int* s_hdr,
                                         int e, int n_rows,
                                         int mt, int nt, int s, int col0, int target, int half, int* s_stop,
                                         uint32_t** s_pend, int* s_pend_y) {
  // waves: WGM x WGN, each a WM x 64 wave tile of MI x 2 MFMA blocks (GLU: one block of gate columns and the
  // block of up columns that pairs with it)
  constexpr int BM = 256, BK = 64;
  constexpr int WGN = BN / 64, WGM = FFN_WAVES / WGN, WM = BM / WGM, MI = WM / 32, NI = 2;
  constexpr int OUT_BN = GLU ? BN / 2 : BN;
  constexpr int A_BYTES = BM * BK * 2, B_BYTES = BN * BK * 2, STAGE = A_BYTES + B_BYTES;
  constexpr int A_LOADS = BM / 8 / FFN_WAVES, B_LOADS = BN / 8 / FFN_WAVES;  // 1 KB wave loads (8 rows) per k-tile
  constexpr int N_LOADS = A_LOADS + B_LOADS;
  static_assert(WGN >= 1 && WGM * WGN == FFN_WAVES && MI >= 1, "wave grid");
  static_assert(B_LOADS >= 1, "tile width");

  // the thread index, made opaque per item, so that lane-derived addresses are computed here instead of being
  // hoisted out of the item loop for both GEMMs at once (that would hold, and spill, their registers throughout)
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WGN, wn = wave % WGN;
  const int K = GLU ? a.d : a.f;
  const int nk = GLU ? K / BK : K / BK / a.S;
  const int kt0 = GLU ? 0 : s * nk;
  const uint32_t row_bytes = (uint32_t)K * 2u;
  const unsigned char* __restrict__ Ab = (GLU ? a.x : a.h) + (uint32_t)kt0 * (BK * 2);
  const unsigned char* __restrict__ Wb = GLU ? a.w1 : a.w2;
  const int w_rows = GLU ? 2 * a.f : a.d;
  unsigned char* __restrict__ Cb = GLU ? a.h : a.y;
  const int64_t ldc = GLU ? a.f : a.d;
  const uint32_t lds0 = (uint32_t)(uintptr_t)smem;  // LDS byte address of the stages
  // load mapping: wave instruction q fills tile rows [8q, 8q+8); lane -> row 8q + lane/8, LDS slot lane & 7,
  // which holds k-chunk (lane & 7) ^ swz(row) = (lane & 7) ^ (lane >> 3) ^ (q & 1)
  const uint32_t chunk0 = (uint32_t)(((lane & 7) ^ (lane >> 3)) << 4);
  // fragment mapping: row = base + (lane & 31), k-chunk c = 2 * kstep + (lane >> 5)
  const int swz = (lane & 7) ^ ((lane >> 3) & 1);

  uint32_t aoff[A_LOADS], boff[B_LOADS];
#pragma unroll
  for (int jj = 0; jj < A_LOADS; ++jj) {
    const int q = wave * A_LOADS + jj;
    const int r = 8 * q + (lane >> 3);
    const int row = r < n_rows ? s_rows[r] : s_rows[0];  // absent rows read a real row
    aoff[jj] = (uint32_t)row * row_bytes + (chunk0 ^ ((uint32_t)(q & 1) << 4));
  }
  const unsigned char* wbase = Wb + (int64_t)e * w_rows * row_bytes + (uint32_t)kt0 * (BK * 2);
#pragma unroll
  for (int jj = 0; jj < B_LOADS; ++jj) {
    const int q = wave * B_LOADS + jj;
    const int i = 8 * q + (lane >> 3);
    int wrow;
    if (GLU) wrow = i < BN / 2 ? nt * (BN / 2) + i : a.f + nt * (BN / 2) + (i - BN / 2);
    else wrow = col0 + i;
    boff[jj] = (uint32_t)wrow * row_bytes + (chunk0 ^ ((uint32_t)(q & 1) << 4));
  }
  f32x16_t acc[MI][NI];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int ni = 0; ni < NI; ++ni)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[mi][ni][q] = 0.f;

  // 32-row MFMA blocks of this wave that hold real rows: all MI except in the last tile of an expert's run
  const int mact = min(MI, max(0, (n_rows - wm * WM + 31) / 32));
  auto kloop = [&](auto full_tag) {
    constexpr bool FULL = decltype(full_tag)::value;
    // slots of a k-step: MFMA i (if i < MI*NI); the next k-step's fragment reads all go out in the first RS
    // slots, so that each has most of the k-step's MFMAs to land in (spread one per slot, the last ones arrived
    // two MFMAs before they were needed: ~8% slower first-GEMM k-loops); the loads go in the slots after those
    constexpr int NSLOT = MI * NI > MI + NI ? MI * NI : MI + NI;
    constexpr int RS = NSLOT >= 4 ? 2 : 1, RPS = (MI + NI + RS - 1) / RS;  // read slots, reads per slot
    constexpr int FIRST = NSLOT > RS ? RS : 0;
    constexpr int HALF = (N_LOADS + 1) / 2;  // loads per half k-tile
    constexpr int DPS = (HALF + (NSLOT - FIRST) - 1) / (NSLOT - FIRST);
    // fragment i of k-step ks (i < MI: A block i, else B block i - MI) from the stage at sa
    auto frag1 = [&](const unsigned char* sa, int ks, int i, bf16x8_t* A_, bf16x8_t* B_) {
      const int sl = (((2 * ks + (lane >> 5)) ^ swz) << 4);
      if (i < MI) {
        A_[i] = __builtin_bit_cast(bf16x8_t, *(const u32x4_t*)(sa + (wm * WM + i * 32 + (lane & 31)) * 128 + sl));
      } else {
        const int ni = i - MI;
        int row;
        if (GLU) row = ni == 0 ? wn * 32 : BN / 2 + wn * 32;
        else row = wn * 64 + ni * 32;
        B_[ni] = __builtin_bit_cast(bf16x8_t, *(const u32x4_t*)(sa + A_BYTES + (row + (lane & 31)) * 128 + sl));
      }
    };
    // this wave's load u of k-tile kt into the stage at LDS address sb
    auto dma1 = [&](int kt, uint32_t sb, int u) {
      const unsigned char* ak = Ab + (uint32_t)kt * (BK * 2);
      const unsigned char* bk = wbase + (uint32_t)kt * (BK * 2);
      if (u < A_LOADS) dma16(ak, aoff[u], sb + (wave * A_LOADS + u) * 1024);
      else dma16(bk, boff[u - A_LOADS], sb + A_BYTES + (wave * B_LOADS + u - A_LOADS) * 1024);
    };
    bf16x8_t fa[2][MI], fb[2][NI];
    // one k-step of k-tile kt; M1: k-tile kt+1 exists, M2: k-tile kt+2 exists
    auto step = [&](auto ks_tag, auto m1_tag, auto m2_tag, int kt) {
      constexpr int ks = decltype(ks_tag)::value;
      constexpr bool M1 = decltype(m1_tag)::value, M2 = decltype(m2_tag)::value;
      constexpr int c = ks & 1;
      const unsigned char* sa = smem + (kt & 1) * STAGE;
      const unsigned char* nsa = smem + ((kt + 1) & 1) * STAGE;
#pragma unroll
      for (int i = 0; i < NSLOT; ++i) {
        const int mi = i / NI, ni = i % NI;
        if (i < MI * NI && (FULL || mi < mact))
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[c][mi], fb[c][ni], acc[mi][ni], 0, 0, 0);
        if (i < RS) {
#pragma unroll
          for (int r = i * RPS; r < (i + 1) * RPS && r < MI + NI; ++r) {
            if (ks < 3) frag1(sa, ks + 1, r, fa[c ^ 1], fb[c ^ 1]);
            else if (M1) frag1(nsa, 0, r, fa[c ^ 1], fb[c ^ 1]);
          }
        }
        if (i >= FIRST && ((ks == 3 && M2) || (ks == 0 && M1))) {
          // first half of k-tile kt+2 after this tile's barrier; second half of k-tile kt+1 in k-step 0
#pragma unroll
          for (int t = 0; t < DPS; ++t) {
            const int v = (i - FIRST) * DPS + t;
            if (v < HALF) {
              if (ks == 3) dma1(kt + 2, lds0 + (kt & 1) * STAGE, v);
              else if (HALF + v < N_LOADS) dma1(kt + 1, lds0 + ((kt + 1) & 1) * STAGE, HALF + v);
            }
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      if (ks == 2) {
        // this wave's fragment reads of k-tile kt and loads of k-tile kt+1 are done; then everyone's are
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    auto tile = [&](auto m1, auto m2, int kt) {
      step(std::integral_constant<int, 0>{}, m1, m2, kt);
      step(std::integral_constant<int, 1>{}, m1, m2, kt);
      step(std::integral_constant<int, 2>{}, m1, m2, kt);
      step(std::integral_constant<int, 3>{}, m1, m2, kt);
    };
    // prologue: k-tile 0 whole, first half of k-tile 1 (its second half goes out in k-step 0 of k-tile 0)
#pragma unroll
    for (int u = 0; u < N_LOADS; ++u) dma1(0, lds0, u);
    wait_loads_barrier();
#pragma unroll
    for (int i = 0; i < MI + NI; ++i) frag1(smem, 0, i, fa[0], fb[0]);
    if (nk > 1) {
#pragma unroll
      for (int u = 0; u < HALF; ++u) dma1(1, lds0 + STAGE, u);
    }
    int kt = 0;
    for (; kt + 2 < nk; ++kt) tile(std::true_type{}, std::true_type{}, kt);
    if (kt + 1 < nk) {
      tile(std::true_type{}, std::false_type{}, kt);
      ++kt;
    }
    tile(std::false_type{}, std::false_type{}, kt);
  };
  if (mact == MI) kloop(std::true_type{});
  else kloop(std::false_type{});
  // epilogue: every wave writes its bf16 outputs into LDS as a 256 x OUT_BN tile (16-byte chunk ch of row r at
  // chunk ch ^ (r & 7), so neither the column writes nor the row reads collide), then 16-byte stores of the
  // tile's real rows
  constexpr int NO = GLU ? 1 : NI;
  constexpr int OUT_ROW = OUT_BN * 2;
  // the thread index, made opaque here, so that the many epilogue addresses are computed per item instead of
  // being hoisted out of the item loop, where they would hold (and spill) registers through the k-loop
  int tid_e = tid;
  asm volatile("" : "+v"(tid_e));
  const int lane_e = tid_e & 63;
  if constexpr (GLU) {
    if (a.gu != nullptr) {
      // the pre-activations g | u of the real rows, fp32, for a backward call that takes them instead of
      // recomputing this GEMM.  Accumulator element q of a lane is row 8 (q / 4) + 4 (lane / 32) + q % 4 of the
      // block at column lane % 32, so for each q the 4-byte stores of lanes 0-31 and of lanes 32-63 each write 128
      // consecutive bytes of one row: no transpose needed (a DPP quad transpose and 16-byte stores made this part
      // of the epilogue ~25% longer).  The stores stream past the caches (nontemporal): nothing reads them in this
      // launch, and cached they would push the GEMMs' operand tiles out of L2.
      const int64_t ld = 2 * (int64_t)a.f;
      const int col = nt * (BN / 2) + wn * 32 + (lane_e & 31);
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const int r = wm * WM + mi * 32 + 8 * (q >> 2) + 4 * (lane_e >> 5) + (q & 3);
          if (r < n_rows) {
            float* row = a.gu + (int64_t)s_rows[r] * ld;
            __builtin_nontemporal_store(acc[mi][0][q], &row[col]);
            __builtin_nontemporal_store(acc[mi][1][q], &row[a.f + col]);
          }
          __builtin_amdgcn_sched_barrier(0);  // one row group at a time
        }
    }
  }
  auto stage = [&](int mi, int ni, const f32x16_t& v, const f32x16_t& up) {  // one 32 x 32 block into LDS
    const int col = (GLU ? wn * 32 : wn * 64 + ni * 32) + (lane_e & 31);
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int row = wm * WM + mi * 32 + (q >> 2) * 8 + (lane_e >> 5) * 4 + (q & 3);
      const float o = GLU ? silu_fast(v[q]) * up[q] : v[q];
      const int chunk = (col >> 3) ^ (row & 7);
      *(__bf16*)(smem + row * OUT_ROW + chunk * 16 + (col & 7) * 2) = (__bf16)o;  // round to nearest even
    }
  };
  if (!GLU && a.S > 1) {
    // split-K: every split stores its fp32 partial sums (thread tid keeps its accumulators at float4 chunk
    // ((mi * NI + ni) * 4 + q4) * 256 + tid of its slot; a half item writes the chunks that the full tile's
    // threads of its columns would), waits for the stores to complete, and counts itself in; the item that
    // completes the tile sums it (reduce_tile)
    // the full tile's wave grid (a half item's blocks go where the full tile's thread for those rows and columns
    // keeps them)
    constexpr int BNF = HALF_TILE ? 2 * BN : BN, SLOT4 = BM * BNF / 4, NT = FFN_THREADS;
    constexpr int WGN_F = BNF / 64, WM_F = BM / (FFN_WAVES / WGN_F);
    const int64_t tile = (int64_t)mt * a.n_nt2 + nt;
    f32x4_t* slot = (f32x4_t*)(a.partial + tile * a.S * (BM * BNF)) + (int64_t)s * SLOT4;
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int ni = 0; ni < NI; ++ni) {
        const int row0 = wm * WM + mi * 32, col0 = (HALF_TILE ? half * BN : 0) + wn * 64 + ni * 32;
        const int tid_f = ((row0 / WM_F) * WGN_F + col0 / 64) * 64 + lane;
        const int b = ((row0 % WM_F) / 32) * NI + ni;
        f32x4_t* dst = slot + b * 4 * NT + tid_f;
        const f32x16_t v = acc[mi][ni];
        store16_coherent(dst, __builtin_bit_cast(u32x4_t, __builtin_shufflevector(v, v, 0, 1, 2, 3)));
        store16_coherent(dst + NT, __builtin_bit_cast(u32x4_t, __builtin_shufflevector(v, v, 4, 5, 6, 7)));
        store16_coherent(dst + 2 * NT, __builtin_bit_cast(u32x4_t, __builtin_shufflevector(v, v, 8, 9, 10, 11)));
        store16_coherent(dst + 3 * NT, __builtin_bit_cast(u32x4_t, __builtin_shufflevector(v, v, 12, 13, 14, 15)));
      }
    wait_stores();
    __syncthreads();  // every thread's partial stores completed; every wave is done with the operand stages
    if (tid == 0) *s_stop = (int)arrive(&a.scount[tile], a.epoch);
    __syncthreads();
    if (*s_stop != target - 1) return true;  // the tile is not complete yet
    flag_acquire();  // the other splits' partial sums completed before they counted themselves in
    reduce_tile<BNF>(a, smem, s_rows, s_hdr, n_rows, mt, nt);
    return true;
  }
  __syncthreads();  // every wave is done with the operand stages
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int ni = 0; ni < NO; ++ni) stage(mi, ni, acc[mi][ni], acc[mi][GLU ? 1 : ni]);
  __syncthreads();
  const RowDst dst = GLU ? RowDst{nullptr, 0, 0, 0} : self_dst(a.self_recv, s_hdr, (int64_t)col0 * 2);
  store_rows<OUT_BN>(smem, Cb + (GLU ? (int64_t)nt * OUT_BN : (int64_t)col0) * 2, ldc, s_rows, n_rows, tid_e, dst);
  if (GLU || target == 1) {
    if (tid == 0) {
      *s_pend = GLU ? &a.flags1[(int64_t)mt * a.n_nt1 + nt] : &a.flags2[(int64_t)mt * a.n_nt2 + nt];
      *s_pend_y = GLU ? 0 : 1;
    }
  } else {  // a half of an unsplit tile: the second half to finish publishes
    wait_stores();
    __syncthreads();
    const int64_t tile = (int64_t)mt * a.n_nt2 + nt;
    if (tid == 0 && (int)arrive(&a.scount[tile], a.epoch) == target - 1) {
      __hip_atomic_store(&a.flags2[tile], a.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (a.ts != nullptr) atomicMax((unsigned long long*)&a.ts[1], (unsigned long long)moe_clock());
    }
  }
  return true;
}

// ---- dispatch landing inside the launch ---------------------------------------------------------------------
// The first all-to-all lands token rows in x_pad (review page, "Where Pith is reading between the lines": the same
// tile signalling applied to the dispatch).  With x_tokens given, the launch copies them itself: units of LAND_ROWS
// rows of one row tile, numbered in the order the first GEMM needs its row tiles, handed out from a stamped counter
// like the return's copy units.  A unit's rows go out with device-coherent stores; once they have completed the
// unit counts itself in at its row tile, and the unit that completes the tile publishes the tile's input flag.  A
// first-GEMM item waits for its row tile's flag and takes landing units itself while it waits; the consumer
// workgroups, once done with their own first-GEMM items, land what is left, so the copy runs ahead of the producers
// while the consumers would otherwise wait for the first finished segment.  (The consumers landing everything before
// their own first-GEMM items held up the second GEMM of the first row tiles: 0.4 ms more on a 2.3 ms launch.)
#define LAND_ROWS 32
#define LAND_DEPTH 8  // 16-byte loads in flight per thread
#define LAND_UNITS_PER_TILE (MOE_MT_ROWS / LAND_ROWS)

// One landing unit u (row tile mt_of(u / LAND_UNITS_PER_TILE), its rows [sub * LAND_ROWS, ...)).  All threads.
__device__ void land_unit(const FusedArgs& a, int mt, int sub, int* s_p, int* s_t) {
  const int tid = threadIdx.x;
  const int32_t* dsc = a.mtile_desc + (int64_t)mt * MOE_MT_FIELDS;
  const int n_rows = dsc[1], r0 = sub * LAND_ROWS, nr = min(LAND_ROWS, n_rows - r0);
  __syncthreads();  // s_p / s_t of the previous unit are no longer read
  if (tid < nr) {
    const int p = dsc[MOE_MT_HDR + r0 + tid];
    s_p[tid] = p;
    s_t[tid] = a.row_src[p];
  }
  __syncthreads();
  const int row_vec = a.d * 2 / 16;
  const int64_t row_bytes = (int64_t)a.d * 2;
  unsigned char* xp = (unsigned char*)a.x;
  const int n = nr > 0 ? nr * row_vec : 0;
  int i = tid;
  for (; i + (LAND_DEPTH - 1) * FFN_THREADS < n; i += LAND_DEPTH * FFN_THREADS) {  // LAND_DEPTH loads in flight
    u32x4_t v[LAND_DEPTH];
#pragma unroll
    for (int k = 0; k < LAND_DEPTH; ++k) {
      const int j = i + k * FFN_THREADS, r = j / row_vec, c = j - r * row_vec;
      v[k] = *(const u32x4_t*)(a.xtok + (int64_t)s_t[r] * row_bytes + c * 16);
    }
#pragma unroll
    for (int k = 0; k < LAND_DEPTH; ++k) {
      const int j = i + k * FFN_THREADS, r = j / row_vec, c = j - r * row_vec;
      store16_coherent(xp + (int64_t)s_p[r] * row_bytes + c * 16, v[k]);
    }
  }
  for (; i < n; i += FFN_THREADS) {
    const int r = i / row_vec, c = i - r * row_vec;
    store16_coherent(xp + (int64_t)s_p[r] * row_bytes + c * 16,
                     *(const u32x4_t*)(a.xtok + (int64_t)s_t[r] * row_bytes + c * 16));
  }
  wait_stores();
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __syncthreads();  // every thread's stores of the unit have completed
  if (tid == 0 && (int)arrive(&a.gcount[mt], a.epoch) == LAND_UNITS_PER_TILE - 1)
    __hip_atomic_store(&a.flags0[mt], a.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The next number from a counter that holds stamp << 32 | count, once the launch's stamp is there (workgroup 0
// stores it at the start); -1 if the stamp does not come within the spin budget.  One thread.
__device__ int claim_stamped(uint64_t* ctr, uint32_t stamp, uint64_t budget) {
  const uint64_t t0 = moe_clock();
  while ((uint32_t)(__hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >> 32) != stamp) {
    if (moe_clock() - t0 > budget) return -1;
    __builtin_amdgcn_s_sleep(1);
  }
  return (int)(uint32_t)__hip_atomic_fetch_add(ctr, (uint64_t)1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Takes the next landing unit and lands it; false once every unit has been handed out (or the stamp never came).
// All threads; s_u is workgroup-shared.
template <typename OrderOf>
__device__ bool land_next(const FusedArgs& a, int n_mt, OrderOf mt_of, int* s_u, int* s_p, int* s_t) {
  __syncthreads();  // s_u of the previous call has been read
  if (threadIdx.x == 0) *s_u = claim_stamped(a.gclaim, a.gstamp, a.budget);
  __syncthreads();
  const int u = *s_u;
  if (u < 0 || u >= n_mt * LAND_UNITS_PER_TILE) return false;
  land_unit(a, mt_of(u / LAND_UNITS_PER_TILE), u % LAND_UNITS_PER_TILE, s_p, s_t);
  return true;
}

// A first-GEMM item's wait for its row tile's input rows: lands units while they last, else spins (spin budget).
template <typename OrderOf>
__device__ bool wait_landed(const FusedArgs& a, int mt, int n_mt, OrderOf mt_of, int* s_u, int* s_p, int* s_t,
                            int* s_stop) {
  const uint64_t t0 = moe_clock();
  bool more = true;
  for (;;) {
    __syncthreads();
    if (threadIdx.x == 0) {
      const bool ok = __hip_atomic_load(&a.flags0[mt], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == a.epoch;
      *s_stop = ok ? 3 : ((moe_clock() - t0 > a.budget) ? 1 : (load_status(a.status) != 0 ? 2 : 0));
    }
    __syncthreads();
    const int st = *s_stop;
    if (st == 3) break;
    if (st != 0) {
      if (st == 1 && threadIdx.x == 0) set_status(a.status, MOE_ETIMEOUT);
      return false;
    }
    if (more) more = land_next(a, n_mt, mt_of, s_u, s_p, s_t);
    else __builtin_amdgcn_s_sleep(2);
  }
  flag_acquire();  // the rows were written by this launch (the publish protocol in common.h)
  __syncthreads();  // every thread has read s_stop before the item's own waits write it
  return true;
}

template <int BN1, int BN2>
__global__ __launch_bounds__(FFN_THREADS, 1) void k_ffn_bf16(FusedArgs a) {
  constexpr int BM = 256, BK = 64, BNX = BN1 > BN2 ? BN1 : BN2;
  constexpr int STAGE = (BM + BNX) * BK * 2;
  static_assert(BM * BN2 * 2 <= 2 * STAGE && BM * BN1 <= 2 * STAGE, "output staging fits the operand stages");
  __shared__ __align__(1024) unsigned char smem[2 * STAGE];
  __shared__ int s_rows[MOE_MT_ROWS];
  __shared__ int s_hdr[MOE_MT_HDR];
  __shared__ int s_stop;
  __shared__ uint32_t* s_pend;  // flag of the previous item, published once its stores have completed
  __shared__ int s_pend_y;
  __shared__ int s_land_u, s_land_p[LAND_ROWS], s_land_t[LAND_ROWS];

  launch_acquire();  // drop cache lines older than this launch (the publish protocol in common.h)
  if (load_status(a.status) != 0) return;
  const int n_mt = a.scalars[a.sc_nmt];
  // this batch's routed and returned rows (the layout's per-owner counts)
  int64_t m_real = 0, m_self = 0;
  for (int r = 0; r < a.sc_nmt - SC_NR; ++r) {
    const int n = a.scalars[SC_NR + r];
    m_real += n;
    if (r == a.cons.self_rank) m_self = n;
  }
  int C = a.n_cons, interleave = a.interleave;
  if (C < 0) {  // the launch picks its consumer partition: every workgroup computes the same value
    // a rate never observed reads 0 (the buffer starts zeroed) and the rule takes its default
    const float fr = (a.obs[13] & 1) ? __uint_as_float(a.obs[10]) : 0.f, cr = (a.obs[13] & 2) ? __uint_as_float(a.obs[11]) : 0.f;
    C = ffn_adaptive_consumers(gridDim.x, m_real, m_real - m_self, a.d, a.f, (int64_t)n_mt * a.n_nt1, fr, cr);
    interleave = ffn_interleave(C, a.d, a.f, a.E);
    if (blockIdx.x == 0 && threadIdx.x == 0) a.obs[12] = (uint32_t)C;
  }
  if (a.join && blockIdx.x == 0) consumer_stamp(a.cons);
  if (a.xtok != nullptr && blockIdx.x == 0 && threadIdx.x == 0)  // open the landing counter for this launch
    __hip_atomic_store(a.gclaim, (uint64_t)a.gstamp << 32, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const int tid = threadIdx.x;
  if (tid == 0) s_pend = nullptr;
  // every wave's stores of the previous item have completed, then its flag (a wait on it may come next)
  auto flush = [&]() {
    uint32_t* f = s_pend;
    if (f == nullptr) return;
    const int y = s_pend_y;
    wait_stores();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __syncthreads();
    if (tid == 0) {
      __hip_atomic_store(f, a.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (y && a.ts != nullptr) atomicMax((unsigned long long*)&a.ts[1], (unsigned long long)moe_clock());
      s_pend = nullptr;
    }
  };
  const int G = gridDim.x - C;
  // the item list (item_list.h): the consumers' share of GEMM1 items, the producers' round-robin share, and the
  // half-width items of a last round at most half full
  const FfnList L = ffn_list_make(n_mt, a.mt_order ? a.scalars[a.sc_nmt + 1] : n_mt, a.n_nt1, a.n_nt2, a.S, a.window,
                                  interleave, C, G, BN2 >= 128 && a.halves);
  auto run_of = [&](int mt, int* r0, int* rc) {
    const int32_t* d = a.mtile_desc + (int64_t)mt * MOE_MT_FIELDS;
    *r0 = d[2];
    *rc = d[3];
  };
  auto order = [&](int p) { return a.mt_order ? (int)a.mt_order[p] : p; };
  // the order in which the first GEMM needs its row tiles: by number (GEMM1 first), by position (interleaved)
  auto land_of = [&](int k) { return interleave ? order(k) : k; };
  bool first = true;
  auto run = [&](int idx) {  // one item of the list; false once the launch has failed
    __syncthreads();  // previous item done with LDS and the header
    const FfnItem it = ffn_list_item(L, idx, run_of, order);
    {
      const int32_t* dsc = a.mtile_desc + (int64_t)it.mt * MOE_MT_FIELDS;
      if (tid < MOE_MT_HDR) s_hdr[tid] = dsc[tid];
      if (tid < MOE_MT_ROWS) s_rows[tid] = dsc[MOE_MT_HDR + tid];
    }
    if (first && tid == 0) {
      const unsigned long long t = moe_clock();
      if (a.ts != nullptr) atomicMin((unsigned long long*)&a.ts[0], t);
      if (a.obs != nullptr) atomicMax(obs64(a.obs, 2), ~t);
    }
    first = false;
    __syncthreads();
    flush();
    const int e = __builtin_amdgcn_readfirstlane(s_hdr[0]), n_rows = __builtin_amdgcn_readfirstlane(s_hdr[1]);
    if (it.kind == 1) {
      if (a.xtok != nullptr && !wait_landed(a, it.mt, n_mt, land_of, &s_land_u, s_land_p, s_land_t, &s_stop))
        return false;
      return ffn_tile<BN1, true>(a, smem, s_rows, s_hdr, e, n_rows, it.mt, it.nt, 0, 0, 1, -1, &s_stop, &s_pend, &s_pend_y);
    }
    // the h columns this split reads: column tiles [s, s+1) * n_nt1 / S of the first GEMM
    const int per = a.n_nt1 / a.S;
    if (!wait_flags(a.flags1 + (int64_t)it.mt * a.n_nt1 + it.s * per, per, a.epoch, a.budget, a.status, &s_stop))
      return false;
    if (it.half < 0)
      return ffn_tile<BN2, false>(a, smem, s_rows, s_hdr, e, n_rows, it.mt, it.nt, it.s, it.nt * BN2, it.target, -1,
                                  &s_stop, &s_pend, &s_pend_y);
    if constexpr (BN2 >= 128)
      return ffn_tile<BN2 / 2, false, true>(a, smem, s_rows, s_hdr, e, n_rows, it.mt, it.nt, it.s,
                                            it.nt * BN2 + it.half * (BN2 / 2), it.target, it.half, &s_stop, &s_pend,
                                            &s_pend_y);
    return false;
  };
  // Producer workgroups move through the list in step, a run of consecutive items on one XCD, whose workgroups share
  // operand tiles in its L2.  Two ways of balancing the end were measured and dropped: taking items (or XCD-sized
  // runs of them) from counters at run time costs 4-16% in claim latency and lost L2 sharing; handing runs to the
  // XCDs by a cost model shortens the producers' span (the round-robin leaves the workgroups that take one more
  // first-GEMM item, each ~d / (f / S) second-GEMM items long, behind at the end) by 6% on the DeepSeek-V3-like
  // shard, but the workgroups that finish early under the round-robin are the ones that run the return while the
  // others finish, and with the producers balanced that return is exposed: no faster overall.
  int i0, i1, step;
  ffn_list_range(L, (int)blockIdx.x, &i0, &i1, &step);
  if (a.item_begin > i0) i0 += (a.item_begin - i0 + step - 1) / step * step;  // this launch's chunk of the list
  i1 = min(i1, a.item_end);
  for (int item = i0; item < i1; item += step)
    if (!run(item)) return;
  __syncthreads();
  flush();
  // the consumer workgroups, done with their share of first-GEMM items (none when interleaved), land the token
  // rows that are left, ahead of the producers, until every unit is handed out; then they return segments
  if (a.xtok != nullptr && (int)blockIdx.x < C)
    while (land_next(a, n_mt, land_of, &s_land_u, s_land_p, s_land_t)) {
    }
  if (a.obs != nullptr && tid == 0 && !first) atomicMax(obs64(a.obs, 4), (unsigned long long)moe_clock());
  // then every workgroup returns segments until no copy unit is left (with no consumer partition, the return is
  // the tail of the launch: workgroups take copy units as they run out of items)
  if (a.join) consumer_role(a.cons);
  // the last workgroup to finish folds this call's rates into the record (an error on the way leaves it as it was)
  if (a.obs != nullptr) {
    __syncthreads();
    // a plain counter (fetch-and-add, reset by the last arrival): 256 compare-and-swap loops on one word at the
    // end of the launch serialised for ~0.2 ms
    if (tid == 0 && atomicAdd(obs64(a.obs, 0), 1ull) == (unsigned long long)gridDim.x - 1) {
      auto ld = [&](int w) { return __hip_atomic_load(obs64(a.obs, w), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); };
      const unsigned long long s_inv = ld(2), e = ld(4), bytes = ld(6), ticks = ld(8);
      float fr = (a.obs[13] & 1) ? __uint_as_float(a.obs[10]) : 0.f, cr = (a.obs[13] & 2) ? __uint_as_float(a.obs[11]) : 0.f;
      if (s_inv != 0 && e > ~s_inv && G > 0) {
        const float nf = (float)(6.0 * (double)m_real * a.d * (double)a.f / ((double)(e - ~s_inv) * G));
        fr = fr > 0.f ? 0.5f * (fr + nf) : nf;
      }
      if (ticks > 0 && bytes > 0 && C > 0) {  // a consumer CU's rate (a tail return shares the chip's bandwidth)
        const float nc = (float)((double)bytes / (double)ticks);
        cr = cr > 0.f ? 0.5f * (cr + nc) : nc;
      }
      a.obs[10] = __float_as_uint(fr);
      a.obs[11] = __float_as_uint(cr);
      a.obs[13] = (fr > 0.f ? 1u : 0u) | (cr > 0.f ? 2u : 0u);  // which rates hold observations
      for (int w = 0; w < 10; w += 2) __hip_atomic_store(obs64(a.obs, w), 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

__global__ __launch_bounds__(256) void k_consumer(ConsumerArgs c) {
  launch_acquire();
  if (blockIdx.x == 0) consumer_stamp(c);
  consumer_role(c);
}

// ---- tile configurations --------------------------------------------------------------------------------
#define BF_BM 256
#define F32_BM 64
#define F32_BN 64

int ffn_gemm_bm(int dtype) { return dtype == MOE_BF16 ? BF_BM : F32_BM; }

static int gemm1_bn(int dtype, int f) {
  if (dtype == MOE_BF16) return f % 128 == 0 ? 256 : 128;
  return F32_BN;
}

int ffn_gemm2_bn(int dtype, int d) {
  if (dtype == MOE_BF16) return d % 256 == 0 ? 256 : (d % 128 == 0 ? 128 : 64);
  return F32_BN;
}

// k-splits of a second-GEMM tile: about as many as make its k-loop as long as a first-GEMM tile's
// (f / d rounded, at most 8), restricted so that each split reads whole first-GEMM column tiles of h
int ffn_splits(int dtype, int d, int f) {
  if (dtype != MOE_BF16) return 1;
  const int n_nt1 = f / (gemm1_bn(dtype, f) / 2), nk2 = f / 64;
  int want = (2 * f + d) / (2 * d);
  want = want < 1 ? 1 : (want > 8 ? 8 : want);
  for (int S = want; S > 1; --S)
    if (n_nt1 % S == 0 && nk2 % S == 0) return S;
  return 1;
}

// A nonzero value distinct for every launch that runs the consumer role (the unit counter's stamp).
uint32_t next_stamp() {
  static std::atomic<uint32_t> seq{0};
  uint32_t v;
  do v = ++seq;
  while (v == 0);
  return v;
}

namespace {
struct FlagCarve {
  int64_t flags2, flags1, scount, partial, claim, flags0, gcount, gclaim, obs, total;  // offsets and size in words
};
FlagCarve flag_carve(int dtype, int d, int f, int64_t cap_mtiles) {
  FlagCarve c;
  const int64_t n2 = d / ffn_gemm2_bn(dtype, d);
  auto up = [](int64_t v) { return (v + 63) / 64 * 64; };
  c.flags2 = 0;
  if (dtype != MOE_BF16) {
    c.flags1 = c.scount = c.partial = cap_mtiles * n2;
    c.claim = up(c.partial);
  } else {
    const int64_t n1 = f / (gemm1_bn(dtype, f) / 2), S = ffn_splits(dtype, d, f);
    c.flags1 = up(cap_mtiles * n2);
    c.scount = c.flags1 + up(cap_mtiles * n1);
    c.partial = c.scount + up(2 * cap_mtiles * n2);  // split counts; also the halves of unsplit tiles
    c.claim = c.partial + (S > 1 ? cap_mtiles * n2 * S * (int64_t)BF_BM * ffn_gemm2_bn(dtype, d) : 0);
  }
  if (dtype == MOE_BF16) {  // the dispatch landing: tile flags, per-tile unit counts, the unit counter
    c.flags0 = c.claim + 2;
    c.gcount = c.flags0 + up(cap_mtiles);
    c.gclaim = c.gcount + up(2 * cap_mtiles);
    c.obs = c.gclaim + 2;  // the partition record, last
  } else {
    c.flags0 = c.gcount = c.gclaim = c.obs = c.claim + 2;
  }
  c.total = c.obs + (dtype == MOE_BF16 ? MOE_OBS_WORDS : 0);
  return c;
}


void fill_consumer(ConsumerArgs& c, const FfnLaunch& p, int n_nt2) {
  c.y = (const uint4*)p.y_pad;
  for (int r = 0; r < MOE_MAX_OWNERS; ++r) c.recv.p[r] = r < p.R ? p.recv[r] : nullptr;
  c.seg_desc = p.L->seg_desc;
  c.seg_mtiles = p.L->seg_mtiles;
  c.seg_sched = p.L->seg_sched;
  c.scalars = p.L->scalars;
  c.status = p.L->status;
  c.flags = p.flags;
  c.claim = (uint64_t*)(p.flags + flag_carve(p.dtype, p.d, p.f, p.cap_mtiles).claim);
  c.stamp = next_stamp();
  c.epoch = p.epoch;
  c.n_nt = n_nt2;
  c.row_vec = p.d * (p.dtype == MOE_BF16 ? 2 : 4) / 16;
  c.budget = p.watchdog_ticks;
  c.ts = p.timestamps;
  c.self_rank = p.self_rank;
  c.obs = nullptr;
}


GemmArgs base_args(const FfnLaunch& p) {
  GemmArgs a;
  a.mtile_desc = p.L->mtile_desc;
  a.scalars = p.L->scalars;
  a.sc_nmt = SC_NR + p.R;
  a.status = p.L->status;
  a.window = p.band_window > 0 ? p.band_window : 4;
  a.ts = p.timestamps;
  a.epoch = p.epoch;
  a.flags = nullptr;
  a.n_cons = 0;
  a.self_recv = p.recv[p.self_rank];
  return a;
}

int launch_bf16(const FfnLaunch& p, int grid, int n_cons, hipStream_t st, hipEvent_t ev0, hipEvent_t ev1) {
  FusedArgs a;
  const FlagCarve fc = flag_carve(p.dtype, p.d, p.f, p.cap_mtiles);
  a.x = (const unsigned char*)p.x_pad;
  a.w1 = (const unsigned char*)p.w_gate_up;
  a.w2 = (const unsigned char*)p.w_down;
  a.h = (unsigned char*)p.h;
  a.y = (unsigned char*)p.y_pad;
  a.d = p.d;
  a.f = p.f;
  const int bn1 = gemm1_bn(p.dtype, p.f), bn2 = ffn_gemm2_bn(p.dtype, p.d);
  a.n_nt1 = p.f / (bn1 / 2);
  a.n_nt2 = p.d / bn2;
  a.S = ffn_splits(p.dtype, p.d, p.f);
  a.window = p.band_window > 0 ? p.band_window : 4;
  // item order: GEMM1 first or interleaved windows (the rule is in item_list.h)
  // chunks: GEMM1 first; a launch that picks its partition decides the order itself
  a.interleave = p.item_end >= 0 ? 0 : (n_cons < 0 ? -1 : ffn_interleave(n_cons, p.d, p.f, p.E));
  a.halves = p.item_end >= 0 ? 0 : 1;  // a chunked list has no single last round
  a.item_begin = p.item_end >= 0 ? p.item_begin : 0;
  a.item_end = p.item_end >= 0 ? p.item_end : INT32_MAX;
  a.mtile_desc = p.L->mtile_desc;
  a.mt_order = p.tile_order == 0 ? p.L->mt_order : nullptr;
  a.scalars = p.L->scalars;
  a.sc_nmt = SC_NR + p.R;
  a.status = p.L->status;
  a.flags2 = p.flags + fc.flags2;
  a.flags1 = p.flags + fc.flags1;
  a.scount = (uint64_t*)(p.flags + fc.scount);
  a.partial = (float*)(p.flags + fc.partial);
  a.epoch = p.epoch;
  a.budget = p.watchdog_ticks;
  a.ts = p.timestamps;
  a.n_cons = n_cons;
  a.join = p.join;
  a.E = p.E;
  a.obs = p.item_end >= 0 ? nullptr : p.flags + fc.obs;  // a chunk of the list observes no whole-call rate
  a.xtok = (const unsigned char*)p.x_tokens;
  a.gu = p.gu_out;
  a.row_src = p.L->row_src;
  a.flags0 = p.flags + fc.flags0;
  a.gcount = (uint64_t*)(p.flags + fc.gcount);
  a.gclaim = (uint64_t*)(p.flags + fc.gclaim);
  a.gstamp = next_stamp();
  fill_consumer(a.cons, p, a.n_nt2);
  a.cons.obs = a.obs;
  a.self_recv = (unsigned char*)p.recv[p.self_rank];
  const dim3 g(grid), b(FFN_THREADS);
  if (bn1 == 256 && bn2 == 256) hipExtLaunchKernelGGL((k_ffn_bf16<256, 256>), g, b, 0, st, ev0, ev1, 0, a);
  else if (bn1 == 256 && bn2 == 128) hipExtLaunchKernelGGL((k_ffn_bf16<256, 128>), g, b, 0, st, ev0, ev1, 0, a);
  else if (bn1 == 256) hipExtLaunchKernelGGL((k_ffn_bf16<256, 64>), g, b, 0, st, ev0, ev1, 0, a);
  else if (bn2 == 256) hipExtLaunchKernelGGL((k_ffn_bf16<128, 256>), g, b, 0, st, ev0, ev1, 0, a);
  // narrower tiles hold under 80 KB of LDS; pad them so that one workgroup still fills a CU
  else if (bn2 == 128) hipExtLaunchKernelGGL((k_ffn_bf16<128, 128>), g, b, 16384, st, ev0, ev1, 0, a);
  else hipExtLaunchKernelGGL((k_ffn_bf16<128, 64>), g, b, 16384, st, ev0, ev1, 0, a);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}
}  // namespace

int64_t ffn_flag_words(int dtype, int d, int f, int64_t cap_mtiles) { return flag_carve(dtype, d, f, cap_mtiles).total; }

void ffn_list_dims(int d, int f, int* n_nt1, int* n_nt2, int* S) {
  *n_nt1 = f / (gemm1_bn(MOE_BF16, f) / 2);
  *n_nt2 = d / ffn_gemm2_bn(MOE_BF16, d);
  *S = ffn_splits(MOE_BF16, d, f);
}

int ffn_schedule_host(int d, int f, int E, int n_cons, int n_producers, int band_window, int n_mt, int n_rem,
                      const int32_t* mt_hdr, const int32_t* mt_order, int32_t* items, int64_t cap, int64_t* n_out) {
  const int bn1 = gemm1_bn(MOE_BF16, f), bn2 = ffn_gemm2_bn(MOE_BF16, d);
  const int n_nt1 = f / (bn1 / 2), n_nt2 = d / bn2, S = ffn_splits(MOE_BF16, d, f);
  const int W = band_window > 0 ? band_window : 4;
  const FfnList L = ffn_list_make(n_mt, n_rem, n_nt1, n_nt2, S, W, ffn_interleave(n_cons, d, f, E), n_cons,
                                  n_producers, bn2 >= 128);
  *n_out = L.n_list;
  if (cap < L.n_list) return -1;
  auto run_of = [&](int mt, int* r0, int* rc) {
    *r0 = mt_hdr[4 * mt + 2];
    *rc = mt_hdr[4 * mt + 3];
  };
  auto order = [&](int p) { return (int)mt_order[p]; };
  auto put = [&](int idx, int b, int seq) {
    const FfnItem it = ffn_list_item(L, idx, run_of, order);
    int32_t* o = items + 8 * (int64_t)idx;
    o[0] = b;
    o[1] = seq;
    o[2] = it.kind;
    o[3] = it.mt;
    o[4] = it.nt;
    o[5] = it.s;
    o[6] = it.half;
    o[7] = it.target;
  };
  for (int b = 0; b < n_cons + n_producers; ++b) {
    int i0, i1, step;
    ffn_list_range(L, b, &i0, &i1, &step);
    int seq = 0;
    for (int idx = i0; idx < i1; idx += step, ++seq) put(idx, b, seq);
  }
  return 0;
}

int launch_ffn_producer(const FfnLaunch& p, int grid, int n_cons, hipStream_t st, hipEvent_t ev0, hipEvent_t ev1) {
  if (p.dtype == MOE_BF16) return launch_bf16(p, grid, n_cons, st, ev0, ev1);
  GemmArgs a = base_args(p);
  a.A = p.x_pad;
  a.W = p.w_gate_up;
  a.C = p.h;
  a.K = p.d;
  a.w_rows = 2 * p.f;
  a.ldc = p.f;
  a.f = p.f;
  a.n_nt = p.f / (F32_BN / 2);
  hipExtLaunchKernelGGL((k_gemm<float, F32_BM, F32_BN, 2, 1, true, false>), dim3(grid), dim3(128), 0, st, ev0, ev1, 0,
                        a);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_ffn_producer2(const FfnLaunch& p, int grid, int n_cons, hipStream_t st, hipEvent_t ev0, hipEvent_t ev1) {
  if (p.dtype == MOE_BF16) return 0;  // one launch does both GEMMs
  GemmArgs a = base_args(p);
  a.A = p.h;
  a.W = p.w_down;
  a.C = p.y_pad;
  a.K = p.f;
  a.w_rows = p.d;
  a.ldc = p.d;
  a.f = p.f;
  a.flags = p.flags;
  a.n_nt = p.d / F32_BN;
  a.n_cons = n_cons;
  fill_consumer(a.cons, p, a.n_nt);
  hipExtLaunchKernelGGL((k_gemm<float, F32_BM, F32_BN, 2, 1, false, true>), dim3(grid), dim3(128), 0, st, ev0, ev1, 0,
                        a);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_ffn_consumer(const FfnLaunch& p, int n_cons, hipStream_t st, hipEvent_t ev0, hipEvent_t ev1) {
  ConsumerArgs c;
  fill_consumer(c, p, p.d / ffn_gemm2_bn(p.dtype, p.d));
  hipExtLaunchKernelGGL(k_consumer, dim3(n_cons), dim3(256), 0, st, ev0, ev1, 0, c);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// ---- the allocation-free variant's flag buffer --------------------------------------------------------------
// moe_expert_ffn_overlap_noalloc keeps the FFN launch's flag buffer (tile flags, split arrival counters, split-K
// partial sums, the copy-unit counter) in this file-scope array instead of a caller's workspace.  Every device the
// library runs on holds its own copy until the process ends.  In host code `scratch` names a host-side stand-in,
// not device memory: only the address hipGetSymbolAddress returns, taken once per device with that device current,
// is ever passed to a kernel or a copy.
#define MOE_NOALLOC_SCRATCH_BYTES (64ll << 20)
static __device__ __align__(256) uint32_t scratch[MOE_NOALLOC_SCRATCH_BYTES / 4];

namespace {
std::mutex g_scratch_mu;
std::vector<uint32_t*> g_scratch_ptr;  // per device: the device address of `scratch`, null until looked up
}  // namespace

int64_t ffn_noalloc_scratch_words() { return MOE_NOALLOC_SCRATCH_BYTES / 4; }

uint32_t* ffn_noalloc_scratch(int dev) {
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (dev < 0) return nullptr;
  if ((int)g_scratch_ptr.size() <= dev) g_scratch_ptr.resize(dev + 1, nullptr);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return nullptr;
    g_scratch_ptr[dev] = (uint32_t*)p;
  }
  return g_scratch_ptr[dev];
}

__global__ void k_fill_u32(uint32_t* __restrict__ p, int64_t n) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) p[i] = 0u;
}

int launch_flags_clear(int dtype, int d, int f, int64_t cap_mtiles, uint32_t* flags, hipStream_t st) {
  // everything that is read before this call writes it: tile flags, arrival counters, the copy-unit counter (the
  // split-K partial sums are always written before they are read)
  const FlagCarve c = flag_carve(dtype, d, f, cap_mtiles);
  const int64_t blocks = std::min<int64_t>((c.partial + 255) / 256, 1024);
  if (c.partial > 0) hipLaunchKernelGGL(k_fill_u32, dim3((unsigned)blocks), dim3(256), 0, st, flags, c.partial);
  // the copy-unit counter, the dispatch landing's flags and counters, and the partition record's arrival counter
  // and per-call sums (its running rate estimates stay)
  const int64_t tail = (dtype == MOE_BF16 ? c.obs + 10 : c.claim + 2) - c.claim;  // up to the record's estimates
  hipLaunchKernelGGL(k_fill_u32, dim3((unsigned)std::min<int64_t>((tail + 255) / 256, 1024)), dim3(256), 0, st,
                     flags + c.claim, tail);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// even entries (starts, taken with atomicMin) to the largest value, odd ones (ends, atomicMax) to zero
__global__ void k_ts_init(uint64_t* ts, int64_t n) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    ts[i] = (i & 1) ? 0ull : ~0ull;
}

int launch_ts_init(uint64_t* timestamps, int64_t n, hipStream_t st) {
  hipLaunchKernelGGL(k_ts_init, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, timestamps, n);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}
