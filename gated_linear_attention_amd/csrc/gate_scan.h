// Chunk-local cumulative log gate, pre-scaled by 1/ln 2 (page "flash-linear-
// attention 中的 Simple GLA", section 三: chunk_local_cumsum with the RCP_LN2
// scale, so that decays downstream are hardware exp2).  Shared by the
// standalone gate kernel and the prologue of the chunk kernels.
#pragma once

#include <hip/hip_runtime.h>

namespace sgla {

constexpr double kRcpLn2d = 1.4426950408889634074;  // 1 / ln 2

// Cross-lane moves of a float64 through the gfx9 data-parallel (DPP) lane
// swizzles, applied to both 32-bit halves; lanes that receive nothing get 0.
// They run in the vector ALU, so a wave scan built from them has no LDS
// round trips (a __shfl_up of a double is two ds_bpermute per step).
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ double dpp_f64(double x) {
  const long long b = __builtin_bit_cast(long long, x);
  const int lo = __builtin_amdgcn_update_dpp(0, (int)b, CTRL, ROW_MASK, 0xf, true);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(b >> 32), CTRL, ROW_MASK, 0xf, true);
  return __builtin_bit_cast(double, ((long long)hi << 32) | (unsigned int)lo);
}
constexpr int kDppRowShr = 0x110;     // + n: lane i of a 16-lane row reads lane i - n of the row
constexpr int kDppRowBcast15 = 0x142; // rows 1, 2, 3 read lane 15, 31, 47 (the previous row's last)
constexpr int kDppRowBcast31 = 0x143; // rows 2, 3 read lane 31

// Inclusive prefix sum over the lanes of each `seg`-lane segment of a wave
// (seg a power of two <= 64): row-local steps of 1, 2, 4 and 8 lanes, then
// the row totals carried across rows (16 -> 32 -> 64 lanes).
__device__ __forceinline__ double wave_scan_f64(double s, int seg) {
  const int pos = (threadIdx.x & 63) & (seg - 1);
  double t;
  t = dpp_f64<kDppRowShr + 1, 0xf>(s);
  if (pos >= 1) s += t;
  t = dpp_f64<kDppRowShr + 2, 0xf>(s);
  if (pos >= 2) s += t;
  t = dpp_f64<kDppRowShr + 4, 0xf>(s);
  if (pos >= 4) s += t;
  t = dpp_f64<kDppRowShr + 8, 0xf>(s);
  if (pos >= 8) s += t;
  if (seg > 16) {
    t = dpp_f64<kDppRowBcast15, 0xa>(s);   // rows 1 and 3 add the previous row's total
    s += t;
  }
  if (seg > 32) {
    t = dpp_f64<kDppRowBcast31, 0xc>(s);   // rows 2 and 3 add the first half's total
    s += t;
  }
  return s;
}

// Inclusive prefix sum over the 64 lanes of a wavefront (lane i receives
// x_0 + ... + x_i), accumulated in float64, times 1/ln 2, rounded once to
// float32.  Must be called by all 64 lanes of the wave.
__device__ __forceinline__ float wave_cumsum_log2(float x) {
  return (float)(wave_scan_f64((double)x, 64) * kRcpLn2d);
}

// wave_cumsum_log2 with the rounding remainder: returns hi = float(s / ln 2)
// and sets lo = float(s / ln 2 - hi), so hi + lo carries the running gate to
// ~2^-48 relative.  Differences of two such running gates of similar size
// (hi_c - hi_j is then exact) stay accurate even after a very negative gate
// has pushed both far from zero.  Must be called by all 64 lanes of the wave.
__device__ __forceinline__ float wave_cumsum_log2_split(float x, float& lo) {
  const double t = wave_scan_f64((double)x, 64) * kRcpLn2d;
  const float hi = (float)t;
  lo = (float)(t - (double)hi);
  return hi;
}

// The same scan restarting every `seg` lanes (seg a power of two <= 64): lane
// i receives the sum over lanes [i - i % seg, i], times 1/ln 2.  Must be
// called by all 64 lanes of the wave.
__device__ __forceinline__ float wave_segmented_cumsum_log2(float x, int seg) {
  return (float)(wave_scan_f64((double)x, seg) * kRcpLn2d);
}

}  // namespace sgla
