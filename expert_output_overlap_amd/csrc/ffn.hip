// Producer: persistent grouped SwiGLU expert FFN on CDNA4 MFMA (review page: "The pith" and "Core claim":
// one rank-wide persistent GEMM over all local experts that publishes a readiness flag per output tile;
// "What carries the argument": remote-bound tiles first).
//
// Two persistent launches, one workgroup per CU:
//   GEMM1 (GLU):  h[rows, f] = bf16(silu(x Wg^T) * (x Wu^T)),  one tile = BN/2 gate + BN/2 up columns
//   GEMM2:        y[rows, d] = h Wd^T, then flags[tile] = epoch with an agent-scope release.  The first C
//                 workgroups of this launch are the consumer partition instead (consumer.h): round-robin
//                 dispatch puts workgroup b on XCD b % 8, so C consumers spread over the XCDs, one per CU,
//                 and the producer and consumer are co-resident by construction.
// Row tiles are the layout's GEMM row tiles: up to BM/16 sub-blocks of 16 rows of one expert, walked in
// the remote-first group order, so all-padding sub-blocks cost nothing.  Items (row tile, column tile)
// are visited window by window (band_window row tiles, column-tile-major inside a window) for weight
// reuse, and consecutive items go to workgroups on the same XCD.
#include <type_traits>

#include "common.h"
#include "consumer.h"
#include "launch.h"

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));  // 16-byte chunk (native vector: stays in VGPRs)

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
  static_assert(BM % RPP == 0 && BN % RPP == 0 && BM / 16 <= MOE_MT_SUB, "tile shape");

  __shared__ __align__(16) T sA[2][BM * LDK];
  __shared__ __align__(16) T sB[2][BN * LDK];
  __shared__ int s_sub[MOE_MT_SUB];
  __shared__ int s_hdr[2];

  if (PUBLISH && (int)blockIdx.x < a.n_cons) {
    consumer_role(a.cons, blockIdx.x, a.n_cons);
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
    if (tid < MOE_MT_FIELDS) {
      const int v = a.mtile_desc[(int64_t)mt * MOE_MT_FIELDS + tid];
      if (tid < 2) s_hdr[tid] = v;
      else s_sub[tid - 2] = v;
    }
    if (PUBLISH && a.ts != nullptr && first && tid == 0)
      atomicMin((unsigned long long*)&a.ts[0], (unsigned long long)moe_clock());
    first = false;
    __syncthreads();
    const int e = s_hdr[0], n_sub = s_hdr[1];

    const T* pa[PA];
#pragma unroll
    for (int p = 0; p < PA; ++p) {
      const int r = p * RPP + cr;
      const int sub = r >> 4;
      pa[p] = A + (int64_t)(sub < n_sub ? s_sub[sub] + (r & 15) : 0) * K + cc;
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
    for (int mi = 0; mi < MI; ++mi) mvalid[mi] = ((wm * WM + mi * 32) >> 4) < n_sub;

    f32x16_t acc[MI][NI];
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int ni = 0; ni < NI; ++ni)
#pragma unroll
        for (int q = 0; q < 16; ++q) acc[mi][ni][q] = 0.f;

    // Rows of absent sub-blocks read row 0 of the tile's source instead (always allocated); their outputs are
    // never stored, and rows are independent in both GEMMs.
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

    // epilogue: store the tile's real sub-blocks (padding rows inside a present sub-block included)
    constexpr int NO = GLU ? NI / 2 : NI;
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
      if (!mvalid[mi]) continue;
#pragma unroll
      for (int ni = 0; ni < NO; ++ni) {
        const int col = nt * OUT_BN + (GLU ? wn * (WN / 2) : wn * WN) + ni * 32 + (lane & 31);
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const int row = wm * WM + mi * 32 + (q >> 2) * 8 + (lane >> 5) * 4 + (q & 3);
          const int sub = row >> 4;
          if (sub < n_sub) {
            const int64_t grow = s_sub[sub] + (row & 15);
            float v = acc[mi][ni][q];
            if (GLU) v = silu_f32(v) * acc[mi][ni + NI / 2][q];
            C[grow * a.ldc + col] = Tr::out(v);
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
}

// ---- bf16 GEMM: 256-row tiles, direct global->LDS loads ------------------------------------------------
//
// Workgroup tile 256 x BN x 64 (k), 4 waves in 2 x 2, wave tile 128 x BN/2 (4 x BN/64 MFMA blocks of 32 x 32,
// accumulators in AGPRs).  Operand tiles are staged in LDS without padding, 128 bytes per row; a 16-byte
// k-chunk c of row r sits at slot c ^ swz(r), swz(r) = (r & 7) ^ ((r >> 3) & 1), so the 16-byte fragment
// reads of 16 consecutive rows hit distinct banks.  global_load_lds_dwordx4 moves each 16-byte chunk straight
// from global memory into its swizzled LDS slot (one wave instruction fills 8 rows, 1 KB).
//
// Pipeline, two LDS stages, one barrier per k-tile.  A k-tile is four k-steps of 16 MFMAs per wave; the
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

// global_load_lds_dwordx4 in its scalar-base form: lane i moves 16 bytes from base + off into LDS at
// m0 + 16 * i (m0 is set in the same statement, so no other code depends on it)
__device__ __forceinline__ void dma16(const void* base, uint32_t off, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(__builtin_amdgcn_readfirstlane(lds_addr)),
               "v"(off), "s"(base) : "memory");
}

// this wave's loads have landed in LDS, then the workgroup barrier: after it every wave's have
__device__ __forceinline__ void wait_loads_barrier() { asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory"); }

// SiLU with the hardware reciprocal (about 1 ulp), rounded to bf16 right after
__device__ __forceinline__ float silu_fast(float g) { return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)); }

template <int BN, bool GLU, bool PUBLISH>
__global__ __launch_bounds__(256, 1) void k_gemm_bf16(GemmArgs a) {
  constexpr int BM = 256, BK = 64;
  constexpr int WM = 128, WN = BN / 2, MI = WM / 32, NI = WN / 32;
  constexpr int OUT_BN = GLU ? BN / 2 : BN;
  constexpr int A_BYTES = BM * BK * 2, B_BYTES = BN * BK * 2, STAGE = A_BYTES + B_BYTES;
  constexpr int A_LOADS = BM / 8 / 4, B_LOADS = BN / 8 / 4;  // 1 KB wave loads (8 rows) per wave per k-tile
  constexpr int N_LOADS = A_LOADS + B_LOADS;
  static_assert(!GLU || NI % 2 == 0, "GLU pairs gate and up blocks");
  static_assert(B_LOADS >= 1, "tile width");
  static_assert(BM * OUT_BN * 2 <= 2 * STAGE, "output staging fits the operand stages");

  __shared__ __align__(1024) unsigned char smem[2 * STAGE];
  __shared__ int s_sub[MOE_MT_SUB];
  __shared__ int s_hdr[2];

  if (PUBLISH && (int)blockIdx.x < a.n_cons) {
    consumer_role(a.cons, blockIdx.x, a.n_cons);
    return;
  }
  if (load_status(a.status) != 0) return;
  const int n_mt = a.scalars[a.sc_nmt];
  const int n_items = n_mt * a.n_nt;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int n_cons = PUBLISH ? a.n_cons : 0;
  const int G = gridDim.x - n_cons;
  int bid = blockIdx.x - n_cons;
  if ((G & 7) == 0 && (n_cons & 7) == 0) bid = (bid & 7) * (G >> 3) + (bid >> 3);
  const unsigned char* __restrict__ Ab = (const unsigned char*)a.A;
  const unsigned char* __restrict__ Wb = (const unsigned char*)a.W;
  unsigned char* __restrict__ Cb = (unsigned char*)a.C;
  const int K = a.K;
  const uint32_t row_bytes = (uint32_t)K * 2u;
  const int nk = K / BK;
  const uint32_t lds0 = (uint32_t)(uintptr_t)smem;  // LDS byte address of the stages
  // load mapping: wave instruction q fills tile rows [8q, 8q+8); lane -> row 8q + lane/8, LDS slot lane & 7,
  // which holds k-chunk (lane & 7) ^ swz(row) = (lane & 7) ^ (lane >> 3) ^ (q & 1)
  const uint32_t chunk0 = (uint32_t)(((lane & 7) ^ (lane >> 3)) << 4);
  // fragment mapping: row = base + (lane & 31), k-chunk c = 2 * kstep + (lane >> 5)
  const int swz = (lane & 7) ^ ((lane >> 3) & 1);
  bool first = true;

  for (int item = bid; item < n_items; item += G) {
    const int per_win = a.window * a.n_nt;
    const int w = item / per_win, j = item - w * per_win;
    const int mt0 = w * a.window;
    const int Wc = min(a.window, n_mt - mt0);
    const int nt = j / Wc, mt = mt0 + (j - nt * Wc);

    __syncthreads();  // previous item done with LDS and the header
    if (tid < MOE_MT_FIELDS) {
      const int v = a.mtile_desc[(int64_t)mt * MOE_MT_FIELDS + tid];
      if (tid < 2) s_hdr[tid] = v;
      else s_sub[tid - 2] = v;
    }
    if (PUBLISH && a.ts != nullptr && first && tid == 0)
      atomicMin((unsigned long long*)&a.ts[0], (unsigned long long)moe_clock());
    first = false;
    __syncthreads();
    const int e = s_hdr[0], n_sub = s_hdr[1];

    uint32_t aoff[A_LOADS], boff[B_LOADS];
#pragma unroll
    for (int jj = 0; jj < A_LOADS; ++jj) {
      const int q = wave * A_LOADS + jj;
      const int r = 8 * q + (lane >> 3);
      const int sub = r >> 4;
      const int row = sub < n_sub ? s_sub[sub] + (r & 15) : s_sub[0];  // absent sub-blocks read a real row
      aoff[jj] = (uint32_t)row * row_bytes + (chunk0 ^ ((uint32_t)(q & 1) << 4));
    }
    const unsigned char* wbase = Wb + (int64_t)e * a.w_rows * row_bytes;
#pragma unroll
    for (int jj = 0; jj < B_LOADS; ++jj) {
      const int q = wave * B_LOADS + jj;
      const int i = 8 * q + (lane >> 3);
      int wrow;
      if (GLU) wrow = i < BN / 2 ? nt * (BN / 2) + i : a.f + nt * (BN / 2) + (i - BN / 2);
      else wrow = nt * BN + i;
      boff[jj] = (uint32_t)wrow * row_bytes + (chunk0 ^ ((uint32_t)(q & 1) << 4));
    }
    f32x16_t acc[MI][NI];
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int ni = 0; ni < NI; ++ni)
#pragma unroll
        for (int q = 0; q < 16; ++q) acc[mi][ni][q] = 0.f;

    // 32-row MFMA blocks of this wave that hold present sub-blocks: all MI except in a tile's ragged tail
    const int mact = min(MI, max(0, (n_sub * 16 - wm * WM + 31) / 32));
    auto kloop = [&](auto full_tag) {
      constexpr bool FULL = decltype(full_tag)::value;
      // slots of a k-step: MFMA i (if i < MI*NI), then fragment read i (if i < MI+NI), then loads; the loads go
      // after the slots with a read where there are such slots, else spread over all of them
      constexpr int NSLOT = MI * NI > MI + NI ? MI * NI : MI + NI;
      constexpr int FIRST = MI * NI > MI + NI ? MI + NI : 0;
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
          if (GLU) row = ni < NI / 2 ? wn * (WN / 2) + ni * 32 : BN / 2 + wn * (WN / 2) + (ni - NI / 2) * 32;
          else row = wn * WN + ni * 32;
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
          if (i < MI + NI) {
            if (ks < 3) frag1(sa, ks + 1, i, fa[c ^ 1], fb[c ^ 1]);
            else if (M1) frag1(nsa, 0, i, fa[c ^ 1], fb[c ^ 1]);
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
    // chunk ch ^ (r & 7), so neither the column writes nor the row reads collide), then 16-byte stores of the rows
    // of present sub-blocks (padding rows inside them included, never read for a result)
    constexpr int NO = GLU ? NI / 2 : NI;
    constexpr int OUT_ROW = OUT_BN * 2, CPR = OUT_ROW / 16;
    // the thread index, made opaque here, so that the many epilogue addresses are computed per item instead of
    // being hoisted out of the item loop, where they would hold (and spill) registers through the k-loop
    int tid_e = tid;
    asm volatile("" : "+v"(tid_e));
    const int lane_e = tid_e & 63;
    __syncthreads();  // every wave is done with the operand stages
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
#pragma unroll
      for (int ni = 0; ni < NO; ++ni) {
        const int col = (GLU ? wn * (WN / 2) : wn * WN) + ni * 32 + (lane_e & 31);
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const int row = wm * WM + mi * 32 + (q >> 2) * 8 + (lane_e >> 5) * 4 + (q & 3);
          float v = acc[mi][ni][q];
          if (GLU) v = silu_fast(v) * acc[mi][ni + NI / 2][q];
          const int chunk = (col >> 3) ^ (row & 7);
          *(__bf16*)(smem + row * OUT_ROW + chunk * 16 + (col & 7) * 2) = (__bf16)v;  // round to nearest even
        }
      }
    }
    __syncthreads();
    for (int idx = tid_e; idx < BM * CPR; idx += 256) {
      const int row = idx / CPR, ch = idx - row * CPR;
      const int sub = row >> 4;
      if (sub >= n_sub) continue;
      const u32x4_t v = *(const u32x4_t*)(smem + row * OUT_ROW + ((ch ^ (row & 7)) << 4));
      const int64_t grow = s_sub[sub] + (row & 15);
      *(u32x4_t*)(Cb + (grow * a.ldc + (int64_t)nt * OUT_BN) * 2 + ch * 16) = v;
    }
    if (PUBLISH) {
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");  // this thread's tile stores, agent-visible
      __syncthreads();
      if (tid == 0) {
        __hip_atomic_store(&a.flags[(int64_t)mt * a.n_nt + nt], a.epoch, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
        if (a.ts != nullptr) atomicMax((unsigned long long*)&a.ts[1], (unsigned long long)moe_clock());
      }
    }
  }
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

static GemmArgs base_args(const FfnLaunch& p) {
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
  return a;
}

int launch_ffn_gemm1(const FfnLaunch& p, int grid, hipStream_t st) {
  GemmArgs a = base_args(p);
  a.A = p.x_pad;
  a.W = p.w_gate_up;
  a.C = p.h;
  a.K = p.d;
  a.w_rows = 2 * p.f;
  a.ldc = p.f;
  a.f = p.f;
  const int bn = gemm1_bn(p.dtype, p.f);
  a.n_nt = p.f / (bn / 2);
  if (p.dtype == MOE_BF16) {
    if (bn == 256) hipLaunchKernelGGL((k_gemm_bf16<256, true, false>), dim3(grid), dim3(256), 0, st, a);
    else hipLaunchKernelGGL((k_gemm_bf16<128, true, false>), dim3(grid), dim3(256), 0, st, a);
  } else {
    hipLaunchKernelGGL((k_gemm<float, F32_BM, F32_BN, 2, 1, true, false>), dim3(grid), dim3(128), 0, st, a);
  }
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_ffn_gemm2(const FfnLaunch& p, int grid, int n_cons, hipStream_t st) {
  GemmArgs a = base_args(p);
  a.A = p.h;
  a.W = p.w_down;
  a.C = p.y_pad;
  a.K = p.f;
  a.w_rows = p.d;
  a.ldc = p.d;
  a.f = p.f;
  a.flags = p.flags;
  const int bn = ffn_gemm2_bn(p.dtype, p.d);
  a.n_nt = p.d / bn;
  a.n_cons = n_cons;
  ConsumerArgs& c = a.cons;
  c.y = (const uint4*)p.y_pad;
  for (int r = 0; r < MOE_MAX_OWNERS; ++r) c.recv.p[r] = r < p.R ? p.recv[r] : nullptr;
  c.seg_desc = p.L->seg_desc;
  c.seg_mtiles = p.L->seg_mtiles;
  c.seg_sched = p.L->seg_sched;
  c.scalars = p.L->scalars;
  c.status = p.L->status;
  c.flags = p.flags;
  c.epoch = p.epoch;
  c.n_nt = a.n_nt;
  c.row_vec = p.d * (p.dtype == MOE_BF16 ? 2 : 4) / 16;
  c.budget = p.watchdog_ticks;
  c.ts = p.timestamps;
  // the bf16 workgroups hold over 80 KB of LDS (one per CU); pad the narrow variants to keep that true
  if (p.dtype == MOE_BF16) {
    if (bn == 256) hipLaunchKernelGGL((k_gemm_bf16<256, false, true>), dim3(grid), dim3(256), 0, st, a);
    else if (bn == 128) hipLaunchKernelGGL((k_gemm_bf16<128, false, true>), dim3(grid), dim3(256), 0, st, a);
    else hipLaunchKernelGGL((k_gemm_bf16<64, false, true>), dim3(grid), dim3(256), 16384, st, a);
  } else {
    hipLaunchKernelGGL((k_gemm<float, F32_BM, F32_BN, 2, 1, false, true>), dim3(grid), dim3(128), 0, st, a);
  }
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

__global__ void k_ts_init(uint64_t* ts) {
  ts[0] = ~0ull;
  ts[1] = 0ull;
}

int launch_ts_init(uint64_t* timestamps, hipStream_t st) {
  hipLaunchKernelGGL(k_ts_init, dim3(1), dim3(1), 0, st, timestamps);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}
