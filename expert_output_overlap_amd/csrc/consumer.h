// Consumer role: persistent return of finished row-band segments to their owners (review page: "The pith" and
// "What carries the argument": a persistent communication kernel on a small partition polls the per-tile
// readiness flags and moves each ready segment -- a contiguous strip of output rows spanning the full
// width -- to its owner as one contiguous write).  On one GPU the owner ranks are receive buffers in HBM,
// so a transfer is a device-memory copy by the consumer's CUs.
//
// The copy work is cut into units of at most CONSUMER_UNIT bytes: a segment of n bytes is ceil(n / unit) units
// of whole 16-byte chunks.  Segments of the self owner have none: their rows need no transfer, and the producer
// stores them into the self owner's buffer itself.  Units are numbered in the order in which their segments' GEMM row tiles complete,
// and every workgroup in the role takes the next unit from a counter, one at a time: the consumer partition
// during the FFN, and every producer workgroup as soon as its own items are done, so the copies still pending
// when the last tile is published are spread over the whole chip.  For a unit whose segment it has not seen
// complete yet, a workgroup polls the flags of the segment's GEMM row tiles with relaxed agent-scope loads, then
// reads the rows (the publish protocol in common.h: every workgroup of the launch dropped stale cache lines at its
// start, and rows are read only after this launch wrote them); a spin budget on the 100 MHz clock bounds every
// wait.
//
// The counter is one 64-bit word: the launch's stamp (nonzero, distinct for every launch) in the high half and
// the units handed out in the low half.  One workgroup writes the stamp with a zero count at the start of the
// launch; a workgroup takes its first unit only once it sees the stamp, so no count of an earlier launch is
// ever used.
#pragma once
#include "common.h"

#define CONSUMER_UNIT_CHUNKS 8192  // 16-byte chunks per copy unit (128 KB)

typedef uint32_t v4u32 __attribute__((ext_vector_type(4)));

struct ConsumerArgs {
  const uint4* y;  // y_pad rows, row_vec 16-byte chunks per row
  RecvPtrs recv;
  const int32_t* seg_desc;
  const int32_t* seg_mtiles;
  const int32_t* seg_sched;
  const int32_t* scalars;
  int32_t* status;
  const uint32_t* flags;
  uint64_t* claim;  // unit counter: stamp << 32 | units handed out
  uint32_t epoch;
  uint32_t stamp;
  int self_rank;  // segments of this owner are stored by the producer itself: no copy units
  int n_nt;
  int row_vec;
  uint64_t budget;
  uint64_t* ts;
  uint32_t* obs;  // the launch's partition record: copied bytes (64-bit word 6) and copy ticks (word 8), or null
};

// Opens the counter for this launch; called by one workgroup at its start, before it claims.
__device__ __forceinline__ void consumer_stamp(const ConsumerArgs& a) {
  if (threadIdx.x == 0)
    __hip_atomic_store(a.claim, (uint64_t)a.stamp << 32, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

#define CONSUMER_MAX_THREADS 512

// Runs in a workgroup of up to CONSUMER_MAX_THREADS threads (whole waves) until every unit has been handed out.
__device__ __forceinline__ void consumer_role(const ConsumerArgs& a) {
  // a window of up to blockDim.x scheduled segments: their ids and, relative to the window, the units before them
  __shared__ int s_seg[CONSUMER_MAX_THREADS];
  __shared__ uint32_t s_pre[CONSUMER_MAX_THREADS + 1];
  __shared__ int s_wsum[CONSUMER_MAX_THREADS / 64];
  __shared__ uint32_t s_cur;
  __shared__ int s_hit, s_stop;
  const int tid = threadIdx.x, nthr = blockDim.x;
  if (load_status(a.status) != 0) return;
  const int n_segs = a.scalars[SC_NSEGS];
  const uint64_t t0 = moe_clock();
  uint32_t next = 0;  // thread 0: the unit claimed for the next round
  if (tid == 0) {
    int stop = 0;
    while ((uint32_t)(__hip_atomic_load(a.claim, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >> 32) != a.stamp) {
      if (moe_clock() - t0 > a.budget) {
        stop = 1;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    if (stop) set_status(a.status, MOE_ETIMEOUT);
    else next = (uint32_t)__hip_atomic_fetch_add(a.claim, (uint64_t)1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_stop = stop;
  }
  __syncthreads();
  if (s_stop) return;
  int base = 0, span = 0;  // scheduled segments [base, base + span) are in the window
  uint32_t ubase = 0;      // units before segment base
  int seen = -1;           // the last segment whose flags this workgroup found complete
  for (;;) {
    __syncthreads();  // the previous unit's s_cur and s_hit have been read
    if (tid == 0) s_cur = next;
    __syncthreads();
    const uint32_t cur = s_cur;
    // move the window forward to the one holding unit cur (claims only grow)
    while (span == 0 || cur - ubase >= s_pre[span]) {
      if (span > 0) {
        ubase += s_pre[span];
        base += span;
      }
      if (base >= n_segs) return;  // every unit has been handed out
      span = min(nthr, n_segs - base);
      __syncthreads();  // the old window is no longer read
      uint32_t u = 0;
      if (tid < span) {
        const int s = a.seg_sched[base + tid];
        s_seg[tid] = s;
        const int32_t* sd = a.seg_desc + (int64_t)s * MOE_SEG_FIELDS;
        const int64_t n = sd[SEG_OWNER] == a.self_rank ? 0 : (int64_t)sd[SEG_ROWS] * a.row_vec;
        u = (uint32_t)((n + CONSUMER_UNIT_CHUNKS - 1) / CONSUMER_UNIT_CHUNKS);
      }
      int v = wave_incl_scan((int)u);
      if ((tid & 63) == 63) s_wsum[tid >> 6] = v;
      __syncthreads();
      for (int w = 0; w < (tid >> 6); ++w) v += s_wsum[w];
      if (tid < span) s_pre[tid + 1] = (uint32_t)v;
      if (tid == 0) s_pre[0] = 0;
      __syncthreads();
    }
    const uint32_t r = cur - ubase;
    if (tid < span && s_pre[tid] <= r && r < s_pre[tid + 1]) s_hit = tid;
    __syncthreads();
    const int t = s_hit;
    const int s = s_seg[t];
    const int64_t c0 = (int64_t)(r - s_pre[t]) * CONSUMER_UNIT_CHUNKS;
    // the next claim goes out now; its reply is needed only at the top of the next round
    if (tid == 0) next = (uint32_t)__hip_atomic_fetch_add(a.claim, (uint64_t)1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int32_t* sd = a.seg_desc + (int64_t)s * MOE_SEG_FIELDS;
    if (s != seen) {
      const int mt0 = a.seg_mtiles[2 * s], mcnt = a.seg_mtiles[2 * s + 1];
      const int nflags = mcnt * a.n_nt;
      const uint32_t* fl = a.flags + (int64_t)mt0 * a.n_nt;
      if (tid < 64) {
        const int st = poll_flags_wave([&](int j) { return &fl[j]; }, nflags, a.epoch, a.budget, a.status, 3);
        if (tid == 0) s_stop = st;
      }
      __syncthreads();
      if (s_stop) {
        if (s_stop == 1 && tid == 0) set_status(a.status, MOE_ETIMEOUT);
        return;
      }
      flag_acquire();  // the launch_acquire of this launch left no stale copy of these rows (common.h)
      seen = s;
    }
    const int64_t n = (int64_t)sd[SEG_ROWS] * a.row_vec;
    const int64_t c1 = c0 + CONSUMER_UNIT_CHUNKS < n ? c0 + CONSUMER_UNIT_CHUNKS : n;
    const int owner = sd[SEG_OWNER], src = sd[SEG_SRC_ROW], dst = sd[SEG_DST_ROW];
    const uint64_t tc0 = moe_clock();
    if (a.ts != nullptr && tid == 0) atomicMin((unsigned long long*)&a.ts[2 + 2 * s], (unsigned long long)tc0);
    const v4u32* __restrict__ f4 = (const v4u32*)(a.y + (int64_t)src * a.row_vec);
    v4u32* __restrict__ t4 = (v4u32*)((uint4*)a.recv.p[owner] + (int64_t)dst * a.row_vec);
    const int64_t B = nthr;
    int64_t i = c0 + tid;
    for (; i + 7 * B < c1; i += 8 * B) {  // 8 loads in flight per thread (128 B per thread)
      v4u32 v[8];  // a native vector type: an array of it stays in registers
#pragma unroll
      for (int k = 0; k < 8; ++k) v[k] = f4[i + k * B];
#pragma unroll
      for (int k = 0; k < 8; ++k) t4[i + k * B] = v[k];
    }
    for (; i < c1; i += B) t4[i] = f4[i];
    if (a.ts != nullptr) {
      __syncthreads();  // the unit is copied (loads returned; the stores need not have landed)
      if (tid == 0) atomicMax((unsigned long long*)&a.ts[3 + 2 * s], (unsigned long long)moe_clock());
    }
    if (a.obs != nullptr && tid == 0) {  // thread 0's share of the unit stands for the workgroup's (no barrier)
      atomicAdd((unsigned long long*)(a.obs + 6), (unsigned long long)((c1 - c0) * 16));
      atomicAdd((unsigned long long*)(a.obs + 8), (unsigned long long)(moe_clock() - tc0));
    }
  }
}
