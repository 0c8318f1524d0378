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
inline bool shape_ok(const moe_shape* s) {
  return s && s->N >= 0 && s->E >= 1 && s->E <= MOE_MAX_EXPERTS && s->W >= 1 &&
         s->W <= MOE_MAX_RANKS && s->E % s->W == 0 && s->N % s->W == 0 && s->k >= 1 &&
         s->k <= s->E && s->k <= MOE_MAX_TOPK && s->H >= 0;
}
}  // namespace moe_host
