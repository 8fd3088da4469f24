// Router output for the path: per token, top-k of G logits (descending, equal logits to the lower id)
// and the softmax weight over all G logits at each chosen id (no renormalisation over the k).
// One wavefront per token; lane l holds logits l, l+64, l+128, ...
#include "common.h"
#include "launch.h"

#define ROUTE_MAX_PER_LANE 16  // G <= 1024

__device__ __forceinline__ bool better(float va, int ia, float vb, int ib) {
  return va > vb || (va == vb && ia < ib);
}

__global__ __launch_bounds__(256) void k_route(const float* __restrict__ logits, int T, int G, int k,
                                               int32_t* __restrict__ topk_idx, float* __restrict__ topk_w) {
  const int wave = threadIdx.x / MOE_WAVE, lane = lane_id();
  const int t = blockIdx.x * (blockDim.x / MOE_WAVE) + wave;
  if (t >= T) return;
  const float* l = logits + (int64_t)t * G;
  float v[ROUTE_MAX_PER_LANE];
  uint32_t taken = 0;  // bit i: logit lane + 64 i already chosen
  float mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < ROUTE_MAX_PER_LANE; ++i) {
    const int g = lane + 64 * i;
    v[i] = g < G ? l[g] : -INFINITY;
    mx = fmaxf(mx, v[i]);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
  float den = 0.f;
#pragma unroll
  for (int i = 0; i < ROUTE_MAX_PER_LANE; ++i)
    if (lane + 64 * i < G) den += expf(v[i] - mx);
  den = wave_sum_f(den);

  for (int j = 0; j < k; ++j) {
    float bv = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < ROUTE_MAX_PER_LANE; ++i) {
      const int g = lane + 64 * i;
      if (g < G && !((taken >> i) & 1u) && better(v[i], g, bv, bi)) {
        bv = v[i];
        bi = g;
      }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float ov = __shfl_xor(bv, o, 64);
      const int oi = __shfl_xor(bi, o, 64);
      if (better(ov, oi, bv, bi)) {
        bv = ov;
        bi = oi;
      }
    }
    if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
    if (lane == 0) {
      topk_idx[(int64_t)t * k + j] = bi;
      topk_w[(int64_t)t * k + j] = expf(bv - mx) / den;
    }
  }
}

int launch_route(int T, int G, int k, const float* logits, int32_t* topk_idx, float* topk_w, hipStream_t st) {
  if (T == 0) return 0;
  const int per_block = 4;
  hipLaunchKernelGGL(k_route, dim3((T + per_block - 1) / per_block), dim3(64 * per_block), 0, st, logits, T, G,
                     k, topk_idx, topk_w);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}
