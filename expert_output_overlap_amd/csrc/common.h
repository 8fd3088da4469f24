// Device-side helpers shared by the gfx950 kernels of this library (never by the CPU oracle).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe_overlap.h"

#define MOE_WAVE 64

// GEMM row tile: up to MOE_MT_ROWS real rows of one expert (the kernel's tile height: 256 bf16, 64 fp32).
// Descriptor: MOE_MT_HDR header fields (expert, row count, first row tile and row-tile count of the expert's run,
// whose row tiles are consecutive, and the expert's self-owned group), then the rows' positions in the padded
// layout (-1 past the row count).
#define MOE_MT_ROWS 256
#define MOE_MT_HDR 8
// header fields of a row tile: expert, real rows, first row tile and row-tile count of the expert's run, then the
// self-owned group of the expert: first padded row, rows, and receive row minus padded row
#define MT_SELF_LO 4
#define MT_SELF_N 5
#define MT_SELF_DELTA 6
#define MOE_MT_FIELDS (MOE_MT_HDR + MOE_MT_ROWS)

// scalars[] indices
#define SC_MPAD 0
#define SC_NTILES 1
#define SC_NSEGS 2
#define SC_NR 3
// n_mtiles sits at 3 + R

// segment descriptor fields
#define SEG_OWNER 0
#define SEG_EXPERT 1
#define SEG_FIRST_BAND 2
#define SEG_NBANDS 3
#define SEG_SRC_ROW 4
#define SEG_DST_ROW 5
#define SEG_ROWS 6
#define SEG_GROUP 7

typedef uint16_t bf16_t;  // raw bf16 storage

__device__ __forceinline__ float bf16_to_f32(bf16_t v) { return __uint_as_float(((uint32_t)v) << 16); }

// fp32 -> bf16, round to nearest even (inputs here are finite; NaN kept quiet)
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (bf16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (bf16_t)(u >> 16);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return (uint32_t)f32_to_bf16(a) | ((uint32_t)f32_to_bf16(b) << 16);
}

// 100 MHz constant-rate device clock, comparable across CUs
__device__ __forceinline__ uint64_t moe_clock() { return wall_clock64(); }

// Status word helpers: first error wins.
__device__ __forceinline__ void set_status(int32_t* status, int32_t code) { atomicCAS(status, 0, code); }

__device__ __forceinline__ int32_t load_status(const int32_t* status) {
  return __hip_atomic_load(status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// One thread: waits until the n flags fl[0 .. n) all equal epoch, taking them one at a time and sleeping longer while
// one stays unset (up to max_nap + 1 sleeps of ~512 clocks between loads), so that a long wait sends few loads to the flags' lines (every
// workgroup of a launch polls a handful of lines: polling every flag of a segment from every thread each ~0.1 us
// slowed the producers' own loads).  The status word is looked at every 16 loads.  0: all set; 1: the spin budget
// ran out; 2: another workgroup reported an error.
__device__ inline int poll_flags(const uint32_t* fl, int n, uint32_t epoch, uint64_t budget, const int32_t* status,
                                  int max_nap) {
  const uint64_t t0 = moe_clock();
  int polls = 0;
  for (int i = 0; i < n; ++i) {
    int nap = 0;
    while (__hip_atomic_load(&fl[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != epoch) {
      if (moe_clock() - t0 > budget) return 1;
      if ((++polls & 15) == 0 && load_status(status) != 0) return 2;
      for (int k = 0; k <= nap; ++k) __builtin_amdgcn_s_sleep(8);  // ~512 clocks each
      nap = nap < max_nap ? nap + 1 : max_nap;
    }
  }
  return 0;
}

// The first wave of a workgroup: waits until *flag_at(j) == epoch for every j < n, with one load per lane in flight
// (64 at a time; flags that sit side by side share a cache line, so one wave load reads them all) and a sleep
// between rounds while one stays unset (up to max_nap + 1 sleeps of ~512 clocks).  The status word is looked at
// every 16 rounds.  0: all set; 1: the spin budget ran out; 2: another workgroup reported an error.  (One thread
// taking the flags one at a time put a memory round trip per flag in front of items that wait on dozens of them.)
template <typename FlagAt>
__device__ __forceinline__ int poll_flags_wave(FlagAt flag_at, int n, uint32_t epoch, uint64_t budget,
                                               const int32_t* status, int max_nap) {
  const int lane = threadIdx.x & 63;
  const uint64_t t0 = moe_clock();
  int polls = 0;
  for (int base = 0; base < n; base += 64) {
    bool done = base + lane >= n;
    int nap = 0;
    for (;;) {
      if (!done) done = __hip_atomic_load(flag_at(base + lane), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == epoch;
      if (__ballot(!done) == 0) break;
      if (moe_clock() - t0 > budget) return 1;
      if ((++polls & 15) == 0 && load_status(status) != 0) return 2;
      for (int k = 0; k <= nap; ++k) __builtin_amdgcn_s_sleep(8);  // ~512 clocks each
      nap = nap < max_nap ? nap + 1 : max_nap;
    }
  }
  return 0;
}

// ---- the in-launch publish protocol ----------------------------------------------------------------------
// Results one workgroup hands to another inside a launch (h tiles, split-K partial sums, y tiles) go out with
// device-scope stores, which write through to the level shared by the XCDs; the producer waits for their
// completion (s_waitcnt vmcnt(0), ordered by a release fence at workgroup scope) and then stores the flag with an
// agent-scope atomic.  A reader polls the flag with agent-scope atomic loads.  What it reads next cannot be stale in
// its own caches: every line that is read after a flag wait is read only after this launch wrote it (each such
// result is read only once its flag is set, and no two results share a cache line), so the only stale copies a
// CU's L1 or an XCD's L2 can hold are from before the launch, and every workgroup drops those with one
// agent-scope acquire when it starts (launch_acquire).  After a flag wait the reader then needs only compiler
// ordering (flag_acquire), not the agent-scope acquire that invalidates the XCD's whole L2 on every wait, which
// made every second-GEMM k-loop on the XCD refetch its operands (measured ~3200 against ~2450 shader cycles per
// 256 x 256 x 64 k-tile).
__device__ __forceinline__ void launch_acquire() { __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent"); }
__device__ __forceinline__ void flag_acquire() { __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup"); }

// wave-level helpers
__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Inclusive prefix sum over the 64 lanes of a wave with DPP moves: shifts by 1, 2, 4 and 8 lanes inside each
// 16-lane row (lanes with no source add the zero `old`), then lane 15 into row 1 and lane 47 into row 3
// (row_bcast:15), then lane 31 into rows 2 and 3 (row_bcast:31).  Every lane of the wave must be active.
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15, rows 1 and 3
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31, rows 2 and 3
  return v;
}

__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ float wave_sum_f(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Owner receive-buffer table passed by value in the kernel arguments.
struct RecvPtrs {
  void* p[MOE_MAX_OWNERS];
};

// Store destinations of an output tile whose first column is col_bytes into the row: padded rows [lo, lo + n) (the
// self-owned group of the tile's expert) go to alt + (p + delta) rows, every other row p to the padded layout.  The
// self owner's rows need no transfer, so the producer stores them straight into the self owner's receive buffer
// and the consumer returns only the other owners' groups.
struct RowDst {
  unsigned char* alt;
  int lo, n, delta;
};

// from the row-tile header (in LDS)
__device__ __forceinline__ RowDst self_dst(unsigned char* self_recv, const int* s_hdr, int64_t col_bytes) {
  RowDst d;
  d.lo = s_hdr[MT_SELF_LO];
  d.n = s_hdr[MT_SELF_N];
  d.delta = s_hdr[MT_SELF_DELTA];
  d.alt = self_recv + col_bytes;
  return d;
}
