// Device helpers shared by the bf16 chunk kernels (gfx950, wave64,
// v_mfma_f32_16x16x32_bf16).  Operand layouts of the 16x16x32 MFMA, per lane
// l with group g = l / 16 and r = l % 16:
//   A operand: A[m = r][k = 8g + 0..7]      B operand: B[k = 8g + 0..7][n = r]
//   result   : D[m = 4g + i][n = r], i = 0..3
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace sgla {
namespace mf {

constexpr float kRcpLn2f = 1.44269504088896341f;

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));


__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// v_mfma_f32_32x32x16_bf16, per lane l with h = l / 32 and n = l % 32:
//   A operand: A[m = n][k = 8h + 0..7]     B operand: B[k = 8h + 0..7][n]
//   result   : acc[4j + i] = D[m = 8j + 4h + i][n], j, i = 0..3
typedef float f32x16 __attribute__((ext_vector_type(16)));
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// 2^x with the hardware v_exp_f32 (results below 2^-126 may flush to zero,
// far below any contribution that matters at fp32 accumulation).
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ bf16x8 cat(bf16x4 a, bf16x4 b) {
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Transposed fragment read: lane r of each 16-lane group receives
// base[(row0 + e) * ld + col0 + r] for e = 0..3.  row0 and col0 must be the
// same for the 16 lanes of a group; addresses must be 8-byte aligned.
__device__ __forceinline__ bf16x4 tr_read(const bf16* base, int ld, int row0, int col0) {
  const int lane = threadIdx.x & 15;
  const bf16* p = base + (row0 + (lane >> 2)) * ld + col0 + 4 * (lane & 3);
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p));
}

// Transposed LDS read with the key order used by the wide-key state layout:
// lane r of each 16-lane group receives base[(row0 + e) * ld + col0 + perm(r)]
// for e = 0..3, where perm swaps the middle two 4-key blocks of the 16
// (0-3, 8-11, 4-7, 12-15).
__device__ __forceinline__ bf16x4 tr_read_perm(const bf16* base, int ld, int row0, int col0) {
  const int lane = threadIdx.x & 15;
  const int blk = ((lane & 1) << 3) | ((lane & 2) << 1);
  const bf16* p = base + (row0 + (lane >> 2)) * ld + col0 + blk;
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p));
}

// Raw buffer descriptor over [base, base + bytes).  Loads past the end return
// zeros and stores past the end are dropped, which is how a chunk's tail rows
// (and a chunk past the sequence's end, with bytes = 0) are handled without
// branches: every wave issues the same memory instructions on every chunk.
// Callers pass workgroup-uniform values; they are moved to scalar registers
// explicitly so the descriptor never has to be rebuilt per lane.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  void* p = reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(p, 0, (int)__builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// bf16 pair <-> two floats (element 0 is the low half of the 32-bit word)
__device__ __forceinline__ float bf_lo(uint32_t u) { return __builtin_bit_cast(float, u << 16); }
__device__ __forceinline__ float bf_hi(uint32_t u) { return __builtin_bit_cast(float, u & 0xffff0000u); }

// (a, b) = hi + lo with hi = bf16(x) and lo = bf16(x - hi), both rounded to
// nearest even; 6 VALU per pair (one paired convert for each half).
__device__ __forceinline__ void split2(float a, float b, uint32_t& hi, uint32_t& lo) {
  const f32x2 v = {a, b};
  hi = __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
  const f32x2 hf = {bf_lo(hi), bf_hi(hi)};
  lo = __builtin_bit_cast(uint32_t, __builtin_convertvector(v - hf, bf16x2));
}

__device__ __forceinline__ void split8(const float (&x)[8], bf16x8& hi, bf16x8& lo) {
  u32x4 h, l;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t a, b;
    split2(x[2 * i], x[2 * i + 1], a, b);
    h[i] = a;
    l[i] = b;
  }
  hi = __builtin_bit_cast(bf16x8, h);
  lo = __builtin_bit_cast(bf16x8, l);
}

// Causal 16x16 tiles (c tile, j tile) of the 64 x 64 A matrix, packed 4 bits
// per tile (c | j << 2) so a wave picks its tiles with scalar shifts instead
// of a memory load: (0,0) (1,0) (1,1) (2,0) (2,1) (2,2) (3,0) (3,1) (3,2) (3,3).
constexpr uint64_t kCausalTiles = 0xFB73A62510ull;
__device__ __forceinline__ int tile_c(int ti) { return (int)(kCausalTiles >> (4 * ti)) & 3; }
__device__ __forceinline__ int tile_j(int ti) { return (int)(kCausalTiles >> (4 * ti + 2)) & 3; }

template <typename TOut>
__device__ __forceinline__ void store4(__amdgpu_buffer_rsrc_t rs, uint32_t off, f32x4 x);
template <>
__device__ __forceinline__ void store4<float>(__amdgpu_buffer_rsrc_t rs, uint32_t off, f32x4 x) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, x), rs, off, 0, 0);
}
template <>
__device__ __forceinline__ void store4<bf16>(__amdgpu_buffer_rsrc_t rs, uint32_t off, f32x4 x) {
  bf16x4 y;
#pragma unroll
  for (int i = 0; i < 4; ++i) y[i] = (bf16)x[i];
  __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, y), rs, off, 0, 0);
}


}  // namespace mf
}  // namespace sgla
