// Device-side helpers shared by the ACache HIP kernels (gfx950).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/acache.h"

namespace acache {

typedef uint16_t bf16_t;  // storage type of a bfloat16 element

// bf16 -> fp32 is exact: a bf16 number is the high half of an fp32.
__device__ __forceinline__ float bf16_to_f32(bf16_t x) {
  return __uint_as_float(((uint32_t)x) << 16);
}

// fp32 -> bf16, round to nearest even (IEEE conversion; quiet NaN preserved).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (bf16_t)((u >> 16) | 0x0040u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (bf16_t)(u >> 16);
}

template <typename T> struct Elem;
template <> struct Elem<float> {
  static __device__ __forceinline__ float load(const float* p) { return *p; }
  static __device__ __forceinline__ void store(float* p, float x) { *p = x; }
};
template <> struct Elem<bf16_t> {
  static __device__ __forceinline__ float load(const bf16_t* p) { return bf16_to_f32(*p); }
  static __device__ __forceinline__ void store(bf16_t* p, float x) { *p = f32_to_bf16(x); }
};

// Paged pool geometry: [n_layers][n_pages][n_kv_heads][page_size][head_dim].
struct PoolGeom {
  int32_t n_pages, page_size, page_shift, n_kv_heads, head_dim;
  // element offset of (layer, slot, kv head) row start
  __device__ __forceinline__ size_t row(int layer, int32_t slot, int g) const {
    size_t page = (uint32_t)slot >> page_shift;
    size_t off = (uint32_t)slot & (page_size - 1);
    return ((((size_t)layer * n_pages + page) * n_kv_heads + g) * page_size + off) * head_dim;
  }
};

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

}  // namespace acache
