// Consumer role: persistent return of finished row-band segments to their owners (review page: "The pith" and
// "What carries the argument": a persistent communication kernel on a small partition polls the per-tile
// readiness flags and moves each ready segment -- a contiguous strip of output rows spanning the full
// width -- to its owner as one contiguous write).  On one GPU the owner ranks are receive buffers in HBM,
// so a transfer is a device-memory copy by the consumer's CUs.
//
// The copy work is cut into units of at most CONSUMER_UNIT bytes: a segment of n bytes is ceil(n / unit) units
// of whole 16-byte chunks.  Units are numbered in the order in which their segments' GEMM row tiles complete,
// and consumer workgroup w of C takes units w, w + C, ...: a small segment goes to one workgroup whole, a large
// one is spread over several, so the copy that remains after the producer's final tile is short and no
// workgroup pays a wait per segment for segments it has no part of.  For a unit it polls the flags of the GEMM
// row tiles its segment depends on with relaxed agent-scope loads, then issues one agent-scope acquire fence
// (pairing with the producer's publish) before reading the rows; a spin budget on the 100 MHz clock bounds
// every wait.
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
  int64_t u0 = 0;  // first unit of the current segment
  for (int si = 0; si < n_segs; ++si) {
    const int s = a.seg_sched[si];
    const int32_t* sd = a.seg_desc + (int64_t)s * MOE_SEG_FIELDS;
    const int64_t n = (int64_t)sd[SEG_ROWS] * a.row_vec;  // 16-byte chunks of the segment
    const int64_t units = (n + CONSUMER_UNIT_CHUNKS - 1) / CONSUMER_UNIT_CHUNKS;
    // this workgroup's first unit of the segment: the smallest u >= u0 with u % n_cons == cid
    int64_t u = u0 + ((cid - u0 % n_cons) % n_cons + n_cons) % n_cons;
    u0 += units;
    if (u >= u0) continue;  // no part of this segment
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
    const int owner = sd[SEG_OWNER], src = sd[SEG_SRC_ROW], dst = sd[SEG_DST_ROW];
    if (a.ts != nullptr && tid == 0) atomicMin((unsigned long long*)&a.ts[2 + 2 * s], (unsigned long long)moe_clock());
    const uint4* __restrict__ from = a.y + (int64_t)src * a.row_vec;
    uint4* __restrict__ to = (uint4*)a.recv.p[owner] + (int64_t)dst * a.row_vec;
    const int64_t B = blockDim.x;
    for (; u < u0; u += n_cons) {
      const int64_t c0 = (u - (u0 - units)) * CONSUMER_UNIT_CHUNKS;
      const int64_t c1 = c0 + CONSUMER_UNIT_CHUNKS < n ? c0 + CONSUMER_UNIT_CHUNKS : n;
      int64_t i = c0 + tid;
      const v4u32* __restrict__ f4 = (const v4u32*)from;
      v4u32* __restrict__ t4 = (v4u32*)to;
      for (; i + 7 * B < c1; i += 8 * B) {  // 8 loads in flight per thread (32 KB per workgroup)
        v4u32 v[8];  // a native vector type: an array of it stays in registers
#pragma unroll
        for (int k = 0; k < 8; ++k) v[k] = f4[i + k * B];
#pragma unroll
        for (int k = 0; k < 8; ++k) t4[i + k * B] = v[k];
      }
      for (; i < c1; i += B) t4[i] = f4[i];
    }
    if (a.ts != nullptr) {
      __syncthreads();
      if (tid == 0) atomicMax((unsigned long long*)&a.ts[3 + 2 * s], (unsigned long long)moe_clock());
    }
  }
}
