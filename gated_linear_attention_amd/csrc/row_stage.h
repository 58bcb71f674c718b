// Staging of token-major rows into LDS as fp32 for the fp32 matrix-core
// kernels: a register load, then an LDS store, so that every load of a stage
// is in flight before the first store (the stores go through a generic
// pointer the compiler cannot separate from the loads) and a stage can be
// loaded one step ahead of its use.  bf16 rows stay packed in registers
// until they are widened on the way into LDS.
#pragma once

#include <hip/hip_runtime.h>

#include "sgla_internal.h"

namespace sgla {
namespace stage {

typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 load4(const float* p) { return *reinterpret_cast<const f32x4*>(p); }

// Four consecutive input elements as loaded (bf16 kept packed until they are
// widened on their way into LDS, which halves the registers a prefetch holds).
template <typename T> struct Raw4;
template <> struct Raw4<float> { typedef f32x4 type; };
template <> struct Raw4<__bf16> { typedef uint2 type; };
__device__ __forceinline__ f32x4 raw_load(const float* p) { return load4(p); }
__device__ __forceinline__ uint2 raw_load(const __bf16* p) { return *reinterpret_cast<const uint2*>(p); }
__device__ __forceinline__ void raw_zero(f32x4& x) { x = f32x4{0.f, 0.f, 0.f, 0.f}; }
__device__ __forceinline__ void raw_zero(uint2& x) { x = make_uint2(0u, 0u); }
__device__ __forceinline__ f32x4 widen(f32x4 x) { return x; }
__device__ __forceinline__ f32x4 widen(uint2 u) {
  return f32x4{__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
               __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u)};
}

// Rows [0, 64) x columns [0, W) of a token-major input (row stride RS
// elements) staged by NTH threads into LDS as fp32 (row stride LD floats);
// rows at or past `rows` read as zero.
template <int W, int NTH, typename T>
struct RowTile {
  static constexpr int P = kChunk * (W / 4);      // 4-element pieces
  static constexpr int N = (P + NTH - 1) / NTH;   // per thread
  typename Raw4<T>::type x[N];
  __device__ __forceinline__ void load(const T* src, int64_t RS, int rows) {
#pragma unroll
    for (int u = 0; u < N; ++u) {
      const int i = threadIdx.x + u * NTH;
      const int c = i / (W / 4), c4 = i % (W / 4);
      raw_zero(x[u]);
      if ((P % NTH == 0 || i < P) && c < rows) x[u] = raw_load(src + c * RS + 4 * c4);
    }
  }
  __device__ __forceinline__ void store(float* dst, int LD) const {
#pragma unroll
    for (int u = 0; u < N; ++u) {
      const int i = threadIdx.x + u * NTH;
      if (P % NTH == 0 || i < P)
        *reinterpret_cast<f32x4*>(dst + (i / (W / 4)) * LD + 4 * (i % (W / 4))) = widen(x[u]);
    }
  }
};

}  // namespace stage
}  // namespace sgla
