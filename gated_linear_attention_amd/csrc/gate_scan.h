// Chunk-local cumulative log gate, pre-scaled by 1/ln 2 (page "flash-linear-
// attention 中的 Simple GLA", section 三: chunk_local_cumsum with the RCP_LN2
// scale, so that decays downstream are hardware exp2).  Shared by the
// standalone gate kernel and the prologue of the chunk kernels.
#pragma once

#include <hip/hip_runtime.h>

namespace sgla {

constexpr double kRcpLn2d = 1.4426950408889634074;  // 1 / ln 2

// Inclusive prefix sum over the 64 lanes of a wavefront (lane i receives
// x_0 + ... + x_i), accumulated in float64, times 1/ln 2, rounded once to
// float32.  Must be called by all 64 lanes of the wave.
__device__ __forceinline__ float wave_cumsum_log2(float x) {
  const int lane = threadIdx.x & 63;
  double s = (double)x;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const double y = __shfl_up(s, d, 64);
    if (lane >= d) s += y;
  }
  return (float)(s * kRcpLn2d);
}

// wave_cumsum_log2 with the rounding remainder: returns hi = float(s / ln 2)
// and sets lo = float(s / ln 2 - hi), so hi + lo carries the running gate to
// ~2^-48 relative.  Differences of two such running gates of similar size
// (hi_c - hi_j is then exact) stay accurate even after a very negative gate
// has pushed both far from zero.  Must be called by all 64 lanes of the wave.
__device__ __forceinline__ float wave_cumsum_log2_split(float x, float& lo) {
  const int lane = threadIdx.x & 63;
  double s = (double)x;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const double y = __shfl_up(s, d, 64);
    if (lane >= d) s += y;
  }
  const double t = s * kRcpLn2d;
  const float hi = (float)t;
  lo = (float)(t - (double)hi);
  return hi;
}

// The same scan restarting every `seg` lanes (seg a power of two <= 64): lane
// i receives the sum over lanes [i - i % seg, i], times 1/ln 2.  Must be
// called by all 64 lanes of the wave.
__device__ __forceinline__ float wave_segmented_cumsum_log2(float x, int seg) {
  const int lane = threadIdx.x & 63;
  const int pos = lane & (seg - 1);
  double s = (double)x;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const double y = __shfl_up(s, d, 64);
    if (d < seg && pos >= d) s += y;
  }
  return (float)(s * kRcpLn2d);
}

}  // namespace sgla
