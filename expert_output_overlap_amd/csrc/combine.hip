// Top-k weighted combine at the owners (review page ledger, axiom 3: the router output, hence the combine
// plan, is known before the return): out[r*T_o+t] = sum_j w[t,j] * recv[r][plan[t,j]] over the slots with a
// local expert, fp32 accumulation in ascending j, rounded once to the element type.
// One wavefront per token, 16-byte lanes along the hidden dimension, four 16-byte chunks of two slots per lane
// in flight.  The token index is wave-uniform, so its plan and weights come through scalar loads.  Every row is
// read once and every output row written once: the launch streams one side past the caches (nontemporal), the
// reads when the rows moved exceed the last-level cache, the stores otherwise (see launch_combine).
#include "common.h"
#include "launch.h"

#define COMBINE_MAX_K 16

typedef uint32_t cmb_u32x4 __attribute__((ext_vector_type(4)));

struct CombineArgs {
  const float* w;
  const int32_t* plan;
  RecvPtrs recv;
  void* out;
  const int32_t* status;
  int T, T_o, k, row_vec;
};

template <typename T, bool NT_LOAD, bool NT_STORE>
__global__ __launch_bounds__(256) void k_combine(CombineArgs a) {
  constexpr int VEC = 16 / sizeof(T);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / MOE_WAVE), lane = lane_id();
  const int tok = blockIdx.x * 4 + wave;
  // the status word and the token's plan and weights are independent loads: one round trip for all
  const int32_t st = load_status(a.status);
  if (tok >= a.T) return;
  const int r = tok / a.T_o;
  int p[COMBINE_MAX_K];
  float w[COMBINE_MAX_K];
  int nloc = 0;
  for (int j = 0; j < a.k; ++j) {
    const int pj = a.plan[(int64_t)tok * a.k + j];
    const float wj = a.w[(int64_t)tok * a.k + j];
    if (pj >= 0) {
      p[nloc] = pj;
      w[nloc] = wj;
      ++nloc;
    }
  }
  if (st != 0) return;
  const cmb_u32x4* src = (const cmb_u32x4*)a.recv.p[r];
  cmb_u32x4* dst = (cmb_u32x4*)a.out + (int64_t)tok * a.row_vec;
  auto ld = [&](int slot, int c) -> cmb_u32x4 {
    if (c >= a.row_vec) return cmb_u32x4{0u, 0u, 0u, 0u};
    const cmb_u32x4* q = src + (int64_t)p[slot] * a.row_vec + c;
    return NT_LOAD ? __builtin_nontemporal_load(q) : *q;
  };
  auto add = [&](float (&acc)[VEC], const cmb_u32x4& v, float wj) {
    if (sizeof(T) == 2) {
      const uint32_t q[4] = {v[0], v[1], v[2], v[3]};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[2 * i] += wj * bf16_to_f32((bf16_t)(q[i] & 0xffffu));
        acc[2 * i + 1] += wj * bf16_to_f32((bf16_t)(q[i] >> 16));
      }
    } else {
      acc[0] += wj * __uint_as_float(v[0]);
      acc[1] += wj * __uint_as_float(v[1]);
      acc[2] += wj * __uint_as_float(v[2]);
      acc[3] += wj * __uint_as_float(v[3]);
    }
  };
  // U chunks of the row per lane, for two slots at a time: all their loads go out before any is used; the
  // sums still run in ascending slot order
  constexpr int U = 4;
  for (int c0 = lane; c0 < a.row_vec; c0 += U * MOE_WAVE) {
    float acc[U][VEC];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int i = 0; i < VEC; ++i) acc[u][i] = 0.f;
    int j = 0;
    for (; j + 1 < nloc; j += 2) {
      cmb_u32x4 v0[U], v1[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        v0[u] = ld(j, c0 + u * MOE_WAVE);
        v1[u] = ld(j + 1, c0 + u * MOE_WAVE);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) add(acc[u], v0[u], w[j]);
#pragma unroll
      for (int u = 0; u < U; ++u) add(acc[u], v1[u], w[j + 1]);
    }
    if (j < nloc) {
      cmb_u32x4 v0[U];
#pragma unroll
      for (int u = 0; u < U; ++u) v0[u] = ld(j, c0 + u * MOE_WAVE);
#pragma unroll
      for (int u = 0; u < U; ++u) add(acc[u], v0[u], w[j]);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = c0 + u * MOE_WAVE;
      if (c >= a.row_vec) break;
      cmb_u32x4 o;
      if (sizeof(T) == 2) {
        o = cmb_u32x4{pack_bf16x2(acc[u][0], acc[u][1]), pack_bf16x2(acc[u][2], acc[u][3]),
                      pack_bf16x2(acc[u][4], acc[u][5]), pack_bf16x2(acc[u][6], acc[u][7])};
      } else {
        o = cmb_u32x4{__float_as_uint(acc[u][0]), __float_as_uint(acc[u][1]), __float_as_uint(acc[u][2]),
                      __float_as_uint(acc[u][3])};
      }
      if (NT_STORE) __builtin_nontemporal_store(o, &dst[c]);
      else dst[c] = o;
    }
  }
}

int launch_combine(const CombineLaunch& p, hipStream_t st) {
  const int T = p.R * p.T_o;
  if (T == 0) return 0;
  CombineArgs a;
  a.w = p.topk_w;
  a.plan = p.L->combine_plan;
  for (int r = 0; r < MOE_MAX_OWNERS; ++r) a.recv.p[r] = r < p.R ? p.recv[r] : nullptr;
  a.out = p.out;
  a.status = p.L->status;
  a.T = T;
  a.T_o = p.T_o;
  a.k = p.k;
  a.row_vec = p.d * (p.dtype == MOE_BF16 ? 2 : 4) / 16;
  const dim3 grid((T + 3) / 4);
  // The rows this combine moves, at the routing's expected share of local slots (T k E_l / G rows read, T
  // written): past the 256 MB last-level cache, the row reads stream (DeepSeek-V3-like shard, ~470 MB: 123 -> 97
  // us; streaming the stores as well, 111 us); below it the rows read are still in the cache that the return just
  // wrote them through, and the stores stream instead (Mixtral-like, ~50 MB: 11 -> 8.7 us; skewed 19 -> 17 us;
  // streaming the reads there cost 10-15%).
  const double elem = p.dtype == MOE_BF16 ? 2.0 : 4.0;
  const bool big = ((double)T * p.k * p.E / p.G + (double)T) * p.d * elem > 256.0 * 1024 * 1024;
  if (p.dtype == MOE_BF16) {
    if (big) hipLaunchKernelGGL((k_combine<bf16_t, true, false>), grid, dim3(256), 0, st, a);
    else hipLaunchKernelGGL((k_combine<bf16_t, false, true>), grid, dim3(256), 0, st, a);
  } else {
    if (big) hipLaunchKernelGGL((k_combine<float, true, false>), grid, dim3(256), 0, st, a);
    else hipLaunchKernelGGL((k_combine<float, false, true>), grid, dim3(256), 0, st, a);
  }
  return hipGetLastError() == hipSuccess ? 0 : -1;
}
