// Per-chunk preparation for the wide-key bf16 forward (K = 256 or 512):
// everything about a 64-token chunk that does not depend on the state, done
// once per (chunk, head) instead of once per V tile (page "flash-linear-
// attention 中的 Simple GLA", section 三: the chunk-local cumulative gate and
// the decay-masked intra-chunk q k^T of the output pass; section 一 for the
// chunk algebra).
//
// For chunk n of a head, with b the chunk-local cumulative log2 gate (b_c =
// (1/ln 2) * sum of g over the chunk's tokens 0..c) and L the chunk length:
//   gates: sc[c]  = scale * 2^b_c           (weight of q_c . h_n)
//          dv[j]  = 2^(b_last - b_j)        (decay of k_j v_j^T to the chunk end)
//          dall   = 2^b_last                (decay of h_n across the chunk)
//   A[c][j] = scale * (q_c . k_j) * 2^(b_c - b_j) for j <= c, 0 otherwise,
//             stored as bf16 hi + lo planes (A = hi + lo to ~2^-16 relative).
// Tokens at or past L read as zeros (q, k, g), so their A rows and columns are
// zero and b stays at b_last; the consumer never stores their outputs.
//
// One workgroup of two waves per (chunk, head).  Q K^T runs on
// v_mfma_f32_16x16x32_bf16 with operands loaded straight from HBM in MFMA
// layout (16 contiguous bytes per lane): wave 0 computes the causal 16 x 16
// tiles of c-tiles 0 and 3, wave 1 those of c-tiles 1 and 2 (five each).
#include <hip/hip_runtime.h>

#include "gate_scan.h"
#include "mfma_common.h"
#include "sgla_internal.h"

namespace sgla {
namespace {

using namespace mf;

constexpr int C = kChunk;
constexpr int LDA = C + 8;   // LDS row stride of the A staging planes (elements)

template <int K>
__global__ void __launch_bounds__(128)
chunk_prep_bf16_kernel(const bf16* __restrict__ q, const bf16* __restrict__ k,
                       const float* __restrict__ g, const float* __restrict__ g_gamma, float scale,
                       int32_t H, SeqLayout seqs, int32_t chunks_per_row, float* __restrict__ gates,
                       bf16* __restrict__ amat) {
  __shared__ __attribute__((aligned(16))) bf16 sA[2][C * LDA];
  __shared__ float sb[2][C];

  const int gc = blockIdx.x;      // global chunk index
  const int hd = blockIdx.y;
  int64_t t0;
  int cl;
  if (seqs.chunk_table != nullptr) {
    const ChunkEntry e = seqs.chunk_table[gc];
    t0 = __builtin_amdgcn_readfirstlane(e.t0);
    cl = __builtin_amdgcn_readfirstlane(e.len);
  } else {
    const int row = gc / chunks_per_row;
    const int m = gc - row * chunks_per_row;
    t0 = (int64_t)row * seqs.T + (int64_t)m * C;
    cl = min(C, seqs.T - m * C);
  }
  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int lane = tid & 63;
  const int g4 = lane >> 4;
  const int r = lane & 15;
  const int64_t task = (int64_t)gc * H + hd;

  // ---- gates (each wave scans for itself) ----------------------------------
  float b;
  if (g != nullptr) {
    const auto rg = make_rsrc(g + t0 * H + hd, (uint32_t)cl * H * 4);
    b = wave_cumsum_log2(__builtin_bit_cast(
        float, __builtin_amdgcn_raw_buffer_load_b32(rg, (uint32_t)(lane * H * 4), 0, 0)));
  } else if (g_gamma != nullptr) {
    b = (float)min(lane + 1, cl) * (g_gamma[hd] * kRcpLn2f);
  } else {
    b = 0.f;
  }
  const float blast = __shfl(b, C - 1, 64);
  sb[w][lane] = b;
  if (w == 0) {
    float* gt = gates + task * kGateStride;
    gt[lane] = exp2_hw(b) * scale;
    gt[C + lane] = exp2_hw(blast - b);
    if (lane == 0) gt[2 * C] = exp2_hw(blast);
  }

  // ---- zero the staging planes (upper-triangle tiles stay zero) -----------
  for (int i = tid; i < 2 * C * LDA / 8; i += 128)
    reinterpret_cast<u32x4*>(&sA[0][0])[i] = u32x4{0u, 0u, 0u, 0u};

  // ---- Q K^T over the key dimension ----------------------------------------
  // wave 0: c tiles 0, 3; wave 1: c tiles 1, 2.  Tile (ct, jt) for jt <= ct.
  const int cA = w == 0 ? 0 : 1;
  const int cB = w == 0 ? 3 : 2;
  const int RS = H * K;             // elements between consecutive tokens
  const auto rq = make_rsrc(q + (t0 * H + hd) * (int64_t)K, (uint32_t)cl * RS * 2);
  const auto rk = make_rsrc(k + (t0 * H + hd) * (int64_t)K, (uint32_t)cl * RS * 2);
  f32x4 acc[5];
#pragma unroll
  for (int i = 0; i < 5; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
  for (int u = 0; u < K / 32; ++u) {
    const uint32_t col = (uint32_t)(32 * u + 8 * g4) * 2;
    const bf16x8 qa = __builtin_bit_cast(
        bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rq, (uint32_t)(16 * cA + r) * RS * 2 + col, 0, 0));
    const bf16x8 qb = __builtin_bit_cast(
        bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rq, (uint32_t)(16 * cB + r) * RS * 2 + col, 0, 0));
    bf16x8 kf[4];
#pragma unroll
    for (int jt = 0; jt < 4; ++jt)
      kf[jt] = __builtin_bit_cast(
          bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rk, (uint32_t)(16 * jt + r) * RS * 2 + col, 0, 0));
    if (w == 0) {
      acc[0] = mfma(qa, kf[0], acc[0]);   // (0, 0)
#pragma unroll
      for (int jt = 0; jt < 4; ++jt) acc[1 + jt] = mfma(qb, kf[jt], acc[1 + jt]);   // (3, jt)
    } else {
      acc[0] = mfma(qa, kf[0], acc[0]);   // (1, 0)
      acc[1] = mfma(qa, kf[1], acc[1]);   // (1, 1)
#pragma unroll
      for (int jt = 0; jt < 3; ++jt) acc[2 + jt] = mfma(qb, kf[jt], acc[2 + jt]);   // (2, jt)
    }
  }
  __syncthreads();   // zero fill done before tiles land

  // ---- mask, decay, scale, split; stage in LDS ------------------------------
  // acc element i of tile (ct, jt): A[16 ct + 4 g + i][16 jt + r]
  auto emit = [&](int ct, int jt, f32x4 a) {
    const int j = 16 * jt + r;
    const float bj = sb[w][j];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = 16 * ct + 4 * g4 + i;
      const float x = j <= c ? a[i] * exp2_hw(sb[w][c] - bj) * scale : 0.f;
      const bf16 hi = (bf16)x;
      const bf16 lo = (bf16)(x - (float)hi);
      sA[0][c * LDA + j] = hi;
      sA[1][c * LDA + j] = lo;
    }
  };
  if (w == 0) {
    emit(0, 0, acc[0]);
#pragma unroll
    for (int jt = 0; jt < 4; ++jt) emit(3, jt, acc[1 + jt]);
  } else {
    emit(1, 0, acc[0]);
    emit(1, 1, acc[1]);
#pragma unroll
    for (int jt = 0; jt < 3; ++jt) emit(2, jt, acc[2 + jt]);
  }
  __syncthreads();

  // ---- store both planes row-major [2][64][64] ------------------------------
  bf16* at = amat + task * (2 * C * C);
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int p = tid + 128 * u;          // 1024 pieces of 8 elements
    const int plane = p >> 9;
    const int row = (p >> 3) & 63;
    const int c8 = p & 7;
    *reinterpret_cast<u32x4*>(at + plane * C * C + row * C + 8 * c8) =
        *reinterpret_cast<const u32x4*>(&sA[plane][row * LDA + 8 * c8]);
  }
}

template <int K>
hipError_t launch_k(const ChunkPrepParams& p, hipStream_t stream) {
  const dim3 grid((unsigned)p.seqs.num_chunks, (unsigned)p.H);
  const int per_row = p.seqs.T > 0 ? (p.seqs.T + C - 1) / C : 1;
  hipLaunchKernelGGL((chunk_prep_bf16_kernel<K>), grid, dim3(128), 0, stream,
                     static_cast<const bf16*>(p.q), static_cast<const bf16*>(p.k), p.g, p.g_gamma,
                     p.scale, p.H, p.seqs, per_row, p.gates, static_cast<bf16*>(p.amat));
  return hipGetLastError();
}

}  // namespace

hipError_t launch_chunk_prep_bf16(const ChunkPrepParams& p, hipStream_t stream) {
  if (p.seqs.num_chunks == 0) return hipSuccess;
  switch (p.K) {
    case 256: return launch_k<256>(p, stream);
    case 512: return launch_k<512>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace sgla
