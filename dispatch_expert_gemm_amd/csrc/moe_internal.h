// Internal helpers shared by the libmoe HIP sources (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace moe {

constexpr int kWave = 64;  // CDNA wavefront width

typedef uint16_t bf16_t;  // bfloat16 storage word

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_to_f32(bf16_t v) {
  return __uint_as_float(static_cast<uint32_t>(v) << 16);
}

// fp32 -> bf16, round to nearest even (NaN kept quiet).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<bf16_t>((u >> 16) | 0x40);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<bf16_t>(u >> 16);
}

template <typename T>
__device__ __forceinline__ float load_f32(const T* p);
template <>
__device__ __forceinline__ float load_f32<float>(const float* p) { return *p; }
template <>
__device__ __forceinline__ float load_f32<bf16_t>(const bf16_t* p) { return bf16_to_f32(*p); }

template <typename T>
__device__ __forceinline__ void store_f32(T* p, float v);
template <>
__device__ __forceinline__ void store_f32<float>(float* p, float v) { *p = v; }
template <>
__device__ __forceinline__ void store_f32<bf16_t>(bf16_t* p, float v) { *p = f32_to_bf16(v); }

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

// HBM -> LDS copy of 16 bytes per lane from base + off (base wave-uniform, off per lane): lane l
// of the wave writes LDS bytes lds + 16 l .. +15. Issued from inline asm so the compiler does not
// track it as an LDS write (it would otherwise drain every in-flight copy before unrelated LDS
// reads); completion is waited for explicitly with wait_vmcnt and published to the other waves
// with raw_barrier. M0 is restored.
__device__ __forceinline__ uint32_t lds_addr(const char* lds) {
  return __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const char*)(lds))));
}
__device__ __forceinline__ const char* uniform_ptr(const char* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
  return reinterpret_cast<const char*>((static_cast<uint64_t>(hi) << 32) | lo);
}
// lds: wave-uniform LDS byte address
__device__ __forceinline__ void dma16(const char* base, uint32_t off, uint32_t lds) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "global_load_lds_dwordx4 %2, %3\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds), "v"(off), "s"(base)
      : "memory");
}
// s_waitcnt vmcnt(VM) (gfx9 encoding: vmcnt bits [3:0] and [15:14]; expcnt, lgkmcnt not waited)
template <int VM>
__device__ __forceinline__ void wait_vmcnt() {
  __builtin_amdgcn_s_waitcnt((VM & 0xF) | ((VM >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}
// s_waitcnt vmcnt(VM) lgkmcnt(0)
template <int VM>
__device__ __forceinline__ void wait_vm_lgkm() {
  __builtin_amdgcn_s_waitcnt((VM & 0xF) | ((VM >> 4) << 14) | (0x7 << 4));
}
// s_waitcnt lgkmcnt(0) (vmcnt 63 and expcnt 7: not waited)
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }
// Workgroup barrier without a memory fence (the fence would drain the in-flight LDS loads);
// the memory clobber keeps the compiler from moving LDS accesses across it.
__device__ __forceinline__ void raw_barrier() { asm volatile("s_barrier" ::: "memory"); }


// Rank of expert e under `placement` (NULL = contiguous, E_loc experts per rank).
__device__ __forceinline__ int rank_of(const int32_t* placement, int e, int e_loc) {
  return placement ? placement[e] : e / e_loc;
}

}  // namespace moe

// Host-side helpers (defined in api.cpp).
namespace moe_host {
moe_status launch_status();                // checks hipGetLastError after launches
void set_error(const char* msg);           // records a message for moe_last_error
inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }
inline int min_i(int a, int b) { return a < b ? a : b; }
// The count outputs of moe_route / moe_gate_route: absent, or W in 1..MOE_MAX_RANKS dividing E
// and N (defined in route.hip).
bool route_counts_ok(int N, int E, int W, const void* layout_ws);
inline bool shape_ok(const moe_shape* s) {
  return s && s->N >= 0 && s->E >= 1 && s->E <= MOE_MAX_EXPERTS && s->W >= 1 &&
         s->W <= MOE_MAX_RANKS && s->E % s->W == 0 && s->N % s->W == 0 && s->k >= 1 &&
         s->k <= s->E && s->k <= MOE_MAX_TOPK && s->H >= 0;
}
}  // namespace moe_host
