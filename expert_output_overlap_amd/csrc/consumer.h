// Consumer role: persistent return of finished row-band segments to their owners (review page: "The pith" and
// "What carries the argument": a persistent communication kernel on a small partition polls the per-tile
// readiness flags and moves each ready segment -- a contiguous strip of output rows spanning the full
// width -- to its owner as one contiguous write).  On one GPU the owner ranks are receive buffers in HBM,
// so a transfer is a device-memory copy by the consumer's CUs.
//
// Every consumer workgroup walks all segments in the order in which their GEMM row tiles complete and copies
// its 1/C share of each (16-byte chunks w*B + t, then every C*B chunks for B threads): all C CUs work on the
// segment that became ready last, so the copy that remains after the producer's final tile is short.  For a
// segment it polls the flags of the GEMM row tiles the segment depends on with relaxed agent-scope loads,
// then issues one agent-scope acquire fence (pairing with the producer's publish) before reading the rows;
// a spin budget on the 100 MHz clock bounds every wait.
#pragma once
#include "common.h"

struct ConsumerArgs {
  const uint4* y;  // y_pad rows, row_vec 16-byte chunks per row
  RecvPtrs recv;
  const int32_t* seg_desc;
  const int32_t* seg_mtiles;
  const int32_t* seg_sched;
  const int32_t* scalars;
  int32_t* status;
  const uint32_t* flags;
  uint32_t epoch;
  int n_nt;
  int row_vec;
  uint64_t budget;
  uint64_t* ts;
};

// Runs in consumer workgroup `cid` of `n_cons`, blockDim.x threads.
__device__ void consumer_role(const ConsumerArgs& a, int cid, int n_cons) {
  __shared__ int s_stop;
  const int tid = threadIdx.x;
  if (load_status(a.status) != 0) return;
  const int n_segs = a.scalars[SC_NSEGS];
  const uint64_t t0 = moe_clock();
  for (int si = 0; si < n_segs; ++si) {
    const int s = a.seg_sched[si];
    const int mt0 = a.seg_mtiles[2 * s], mcnt = a.seg_mtiles[2 * s + 1];
    const int nflags = mcnt * a.n_nt;
    const uint32_t* fl = a.flags + (int64_t)mt0 * a.n_nt;
    // wait for every tile of the segment
    for (;;) {
      int ok = 1;
      for (int i = tid; i < nflags; i += blockDim.x)
        ok &= __hip_atomic_load(&fl[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == a.epoch;
      if (__syncthreads_and(ok)) break;
      if (tid == 0) s_stop = (moe_clock() - t0 > a.budget) ? 1 : (load_status(a.status) != 0 ? 2 : 0);
      __syncthreads();
      if (s_stop) {
        if (s_stop == 1 && tid == 0) set_status(a.status, MOE_ETIMEOUT);
        return;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    const int32_t* sd = a.seg_desc + (int64_t)s * MOE_SEG_FIELDS;
    const int owner = sd[SEG_OWNER], src = sd[SEG_SRC_ROW], dst = sd[SEG_DST_ROW], rows = sd[SEG_ROWS];
    if (a.ts != nullptr && tid == 0) atomicMin((unsigned long long*)&a.ts[2 + 2 * s], (unsigned long long)moe_clock());
    const uint4* __restrict__ from = a.y + (int64_t)src * a.row_vec;
    uint4* __restrict__ to = (uint4*)a.recv.p[owner] + (int64_t)dst * a.row_vec;
    const int64_t n = (int64_t)rows * a.row_vec;
    const int64_t stride = (int64_t)n_cons * blockDim.x;
    int64_t i = (int64_t)cid * blockDim.x + tid;
    for (; i + 3 * stride < n; i += 4 * stride) {
      const uint4 v0 = from[i], v1 = from[i + stride], v2 = from[i + 2 * stride], v3 = from[i + 3 * stride];
      to[i] = v0;
      to[i + stride] = v1;
      to[i + 2 * stride] = v2;
      to[i + 3 * stride] = v3;
    }
    for (; i < n; i += stride) to[i] = from[i];
    if (a.ts != nullptr) {
      __syncthreads();
      if (tid == 0) atomicMax((unsigned long long*)&a.ts[3 + 2 * s], (unsigned long long)moe_clock());
    }
  }
}
