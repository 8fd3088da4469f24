// Device helpers shared by the forward and backward FFN launches: operand vector types, the LDS DMA load, stores
// with the device-scope cache policy, the quad transpose of MFMA accumulators, the tile publish and arrival
// counters, SiLU.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));  // 16-byte chunk (native vector: stays in VGPRs)
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// global_load_lds_dwordx4 in its scalar-base form: lane i moves 16 bytes from base + off into LDS at
// m0 + 16 * i.  The statement leaves M0 as it found it: it saves M0 in a scratch SGPR, sets it, issues the load
// (which reads M0 when it issues) and restores it, so no code outside depends on the compiler honouring an M0
// clobber (M0 is a reserved register, which an inline-asm clobber list may not name).
__device__ __forceinline__ void dma16(const void* base, uint32_t off, uint32_t lds_addr) {
  // base and lds_addr are the same in every lane; readfirstlane puts them in scalar registers.  The load takes its
  // LDS address from M0, which needs one wait state after an SALU write (the first s_nop); the second covers a
  // read of M0 right after the statement (the compiler inserts such wait states only around its own M0 writes)
  const uint64_t b = (uint64_t)base;
  const uint64_t sb = ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32)) << 32) |
                      (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %2, %3\n\ts_mov_b32 m0, %0\n\ts_nop 0"
      : "=&s"(saved)
      : "s"(__builtin_amdgcn_readfirstlane(lds_addr)), "v"(off), "s"((const void*)sb)
      : "memory");
}

// this wave's loads have landed in LDS, then the workgroup barrier: after it every wave's have
__device__ __forceinline__ void wait_loads_barrier() { asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory"); }

// 8-byte stores with the device-scope cache policy (data other workgroups read inside the launch; the s_nop as in
// store16_coherent below)
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void store8_coherent(void* p, u32x2_t v) {
  asm volatile("global_store_dwordx2 %0, %1, off sc1\n\ts_nop 1" ::"v"(p), "v"(v) : "memory");
}

// 4 x 4 transpose inside each quad of lanes (DPP quad permutations; every lane of the quad takes part): lane p's
// v[r] becomes lane r's v[p].  Two exchange steps, with lane p ^ 1 for the registers whose bit 0 differs from p's,
// then with lane p ^ 2 for bit 1.  In an MFMA 32 x 32 accumulator a lane holds four consecutive rows of one column
// in each group of four registers; after the transpose it holds one row at four consecutive columns.
template <int CTRL>
__device__ __forceinline__ float quad_perm(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ f32x4_t quad_transpose(f32x4_t v, int lane) {
  constexpr int X1 = 0xB1, X2 = 0x4E;  // quad_perm [1,0,3,2] and [2,3,0,1]
  const bool o1 = lane & 1, o2 = lane & 2;
  float t0 = quad_perm<X1>(v[1]), t1 = quad_perm<X1>(v[0]), t2 = quad_perm<X1>(v[3]), t3 = quad_perm<X1>(v[2]);
  v = f32x4_t{o1 ? t0 : v[0], o1 ? v[1] : t1, o1 ? t2 : v[2], o1 ? v[3] : t3};
  t0 = quad_perm<X2>(v[2]);
  t1 = quad_perm<X2>(v[3]);
  t2 = quad_perm<X2>(v[0]);
  t3 = quad_perm<X2>(v[1]);
  return f32x4_t{o2 ? t0 : v[0], o2 ? t1 : v[1], o2 ? v[2] : t2, o2 ? v[3] : t3};
}

__device__ __forceinline__ uint32_t bf16_bits(float v) {  // round to nearest even
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)v);
}

// SiLU with the hardware reciprocal (about 1 ulp), rounded to bf16 right after
__device__ __forceinline__ float silu_fast(float g) { return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)); }

// 16 bytes with the device-scope cache policy (the one agent-scope atomic stores use), as one dwordx4 store:
// two 8-byte atomic stores per 16 bytes measured 2-3 times slower.  The compiler does not count this store, so
// whoever needs it complete waits with an explicit vmcnt(0) (wait_stores).  Nor does it see that the registers of
// v are store data: on this chip a VALU write to the data registers of a store wider than 8 bytes needs two wait
// states after the store (else the store can send the new value), which the compiler inserts only for stores it
// recognises, so the s_nop is part of the statement.
__device__ __forceinline__ void store16_coherent(void* p, u32x4_t v) {
  asm volatile("global_store_dwordx4 %0, %1, off sc1\n\ts_nop 1" ::"v"(p), "v"(v) : "memory");
}

__device__ __forceinline__ void wait_stores() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

__device__ __forceinline__ void publish(uint32_t* flag, uint32_t epoch) {
  wait_stores();  // this wave's stores are complete
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __syncthreads();  // and every wave's
  if (threadIdx.x == 0) __hip_atomic_store(flag, epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Arrival count of this call at a counter that holds (epoch << 32) | count: returns how many arrived before.  A
// counter that still carries another call's epoch counts from zero, so no reset between calls is needed.
__device__ __forceinline__ uint32_t arrive(uint64_t* ctr, uint32_t epoch) {
  uint64_t old = __hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  for (;;) {
    const bool cur = (uint32_t)(old >> 32) == epoch;
    const uint64_t nw = cur ? old + 1 : (((uint64_t)epoch << 32) | 1u);
    if (__hip_atomic_compare_exchange_strong(ctr, &old, nw, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT))
      return cur ? (uint32_t)old : 0u;
  }
}

