// Top-k weighted combine at the owners (review page ledger, axiom 3: the router output, hence the combine
// plan, is known before the return): out[r*T_o+t] = sum_j w[t,j] * recv[r][plan[t,j]] over the slots with a
// local expert, fp32 accumulation in ascending j, rounded once to the element type.
// One wavefront per token, 16-byte lanes along the hidden dimension, four 16-byte chunks of two slots per lane
// in flight.
#include "common.h"
#include "launch.h"

#define COMBINE_MAX_K 16

struct CombineArgs {
  const float* w;
  const int32_t* plan;
  RecvPtrs recv;
  void* out;
  const int32_t* status;
  int T, T_o, k, row_vec;
};

template <typename T>
__global__ __launch_bounds__(256) void k_combine(CombineArgs a) {
  constexpr int VEC = 16 / sizeof(T);
  const int wave = threadIdx.x / MOE_WAVE, lane = lane_id();
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
  const uint4* src = (const uint4*)a.recv.p[r];
  uint4* dst = (uint4*)a.out + (int64_t)tok * a.row_vec;
  auto add = [&](float (&acc)[VEC], const uint4& v, float wj) {
    if (sizeof(T) == 2) {
      const uint32_t q[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[2 * i] += wj * bf16_to_f32((bf16_t)(q[i] & 0xffffu));
        acc[2 * i + 1] += wj * bf16_to_f32((bf16_t)(q[i] >> 16));
      }
    } else {
      acc[0] += wj * __uint_as_float(v.x);
      acc[1] += wj * __uint_as_float(v.y);
      acc[2] += wj * __uint_as_float(v.z);
      acc[3] += wj * __uint_as_float(v.w);
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
      uint4 v0[U], v1[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = c0 + u * MOE_WAVE;
        v0[u] = c < a.row_vec ? src[(int64_t)p[j] * a.row_vec + c] : make_uint4(0, 0, 0, 0);
        v1[u] = c < a.row_vec ? src[(int64_t)p[j + 1] * a.row_vec + c] : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) add(acc[u], v0[u], w[j]);
#pragma unroll
      for (int u = 0; u < U; ++u) add(acc[u], v1[u], w[j + 1]);
    }
    if (j < nloc) {
      uint4 v0[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = c0 + u * MOE_WAVE;
        v0[u] = c < a.row_vec ? src[(int64_t)p[j] * a.row_vec + c] : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) add(acc[u], v0[u], w[j]);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = c0 + u * MOE_WAVE;
      if (c >= a.row_vec) break;
      uint4 o;
      if (sizeof(T) == 2) {
        o.x = pack_bf16x2(acc[u][0], acc[u][1]);
        o.y = pack_bf16x2(acc[u][2], acc[u][3]);
        o.z = pack_bf16x2(acc[u][4], acc[u][5]);
        o.w = pack_bf16x2(acc[u][6], acc[u][7]);
      } else {
        o.x = __float_as_uint(acc[u][0]);
        o.y = __float_as_uint(acc[u][1]);
        o.z = __float_as_uint(acc[u][2]);
        o.w = __float_as_uint(acc[u][3]);
      }
      dst[c] = o;
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
  if (p.dtype == MOE_BF16) hipLaunchKernelGGL(k_combine<bf16_t>, grid, dim3(256), 0, st, a);
  else hipLaunchKernelGGL(k_combine<float>, grid, dim3(256), 0, st, a);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}
