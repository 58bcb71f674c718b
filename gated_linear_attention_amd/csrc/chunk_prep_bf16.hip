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
//   K^T     : the chunk's keys transposed into the operand order of the state
//             update of chunk_fwd_bf16_wide.hip (layout at the K^T step below), so
//             that kernel loads them with one contiguous 1 KB read per MFMA
//             operand instead of transposing through LDS in every V tile.
// Tokens at or past L read as zeros (q, k, g), so their A rows and columns
// and K^T entries are zero and b stays at b_last.
//
// One workgroup of four waves per (chunk, head).  The K chunk is staged in
// LDS once; Q K^T runs on v_mfma_f32_16x16x32_bf16 with the Q operand loaded
// from HBM in MFMA layout and the K operand read from LDS.
#include <hip/hip_runtime.h>

#include "gate_scan.h"
#include "mfma_common.h"
#include "sgla_internal.h"

namespace sgla {
namespace {

using namespace mf;

constexpr int C = kChunk;
constexpr int NTP = 256;          // threads
constexpr int LDA = C + 8;        // A staging row stride (elements)

// Causal 16 x 16 tiles (c tile, j tile) of each wave, packed 4 bits per tile
// (c | j << 2), up to three per wave:
//   wave 0: (3,0) (3,1) (3,2)   wave 1: (3,3) (0,0)
//   wave 2: (2,0) (2,1) (2,2)   wave 3: (1,0) (1,1)
constexpr uint32_t kPrepTiles[4] = {0xB73u, 0x0Fu, 0xA62u, 0x51u};
constexpr int kPrepCount[4] = {3, 2, 3, 2};

template <int K>
__global__ void __launch_bounds__(NTP)
chunk_prep_bf16_kernel(const bf16* __restrict__ q, const bf16* __restrict__ k,
                       const float* __restrict__ g, const float* __restrict__ g_gamma, float scale,
                       int32_t H, SeqLayout seqs, int32_t chunks_per_row, float* __restrict__ gates,
                       bf16* __restrict__ amat, bf16* __restrict__ ktf) {
  constexpr int LDK = K + 8;      // row stride: conflict-free 16-byte row reads
  constexpr int KP = K / 8;       // 16-byte pieces per key row
  constexpr int NKS = C * KP / NTP;
  __shared__ __attribute__((aligned(16))) bf16 sK[C * LDK];   // later: A staging
  __shared__ float sb[C];

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
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int g4 = lane >> 4;
  const int r = lane & 15;
  const int64_t task = (int64_t)gc * H + hd;
  const int RS = H * K;             // elements between consecutive tokens

  // ---- stage the K chunk (rows past L read as zeros) -----------------------
  {
    const auto rk = make_rsrc(k + (t0 * H + hd) * (int64_t)K, (uint32_t)cl * RS * 2);
    u32x4 x[NKS];
#pragma unroll
    for (int u = 0; u < NKS; ++u) {
      const int p = tid + NTP * u;
      x[u] = __builtin_amdgcn_raw_buffer_load_b128(rk, (uint32_t)((p / KP) * RS + (p % KP) * 8) * 2, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < NKS; ++u) {
      const int p = tid + NTP * u;
      *reinterpret_cast<u32x4*>(sK + (p / KP) * LDK + (p % KP) * 8) = x[u];
    }
  }

  // ---- gates ----------------------------------------------------------------
  if (w == 0) {
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
    sb[lane] = b;
    float* gt = gates + task * kGateStride;
    gt[lane] = exp2_hw(b) * scale;
    gt[C + lane] = exp2_hw(blast - b);
    if (lane == 0) gt[2 * C] = exp2_hw(blast);
  }
  __syncthreads();

  // ---- K^T fragments ----------------------------------------------------------
  // Fragment (kb, ts), kb = 32-key block, ts = 16-token step: lane l holds
  // K[t = 16 ts + 8 (l / 32) + e][key = 32 kb + perm(l % 32)], e = 0..7, with
  // perm swapping the middle two 4-key blocks of each 16.  1 KB per fragment,
  // lane-major, fragments ordered (kb, ts).
  {
    bf16* kt = ktf + task * (int64_t)K * C;
    const int grp = lane >> 4;
#pragma unroll
    for (int f = w; f < (K / 32) * 4; f += 4) {
      const int kb = f >> 2, ts = f & 3;
      const int row0 = 16 * ts + 8 * (grp >> 1);
      const int col0 = 32 * kb + 16 * (grp & 1);
      const bf16x8 x = cat(tr_read_perm(sK, LDK, row0, col0), tr_read_perm(sK, LDK, row0 + 4, col0));
      *reinterpret_cast<bf16x8*>(kt + (f * 64 + lane) * 8) = x;
    }
  }

  // ---- Q K^T: Q operand from HBM, K operand from LDS --------------------------
  const uint32_t tiles = kPrepTiles[w];
  const int ntile = kPrepCount[w];
  const auto rq = make_rsrc(q + (t0 * H + hd) * (int64_t)K, (uint32_t)cl * RS * 2);
  f32x4 acc[3];
#pragma unroll
  for (int i = 0; i < 3; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
  for (int u = 0; u < K / 32; ++u) {
#pragma unroll
    for (int t = 0; t < 3; ++t) {
      if (t >= ntile) continue;
      const int ct = (tiles >> (4 * t)) & 3, jt = (tiles >> (4 * t + 2)) & 3;
      const bf16x8 qa = __builtin_bit_cast(
          bf16x8, __builtin_amdgcn_raw_buffer_load_b128(
                      rq, (uint32_t)((16 * ct + r) * RS + 32 * u + 8 * g4) * 2, 0, 0));
      const bf16x8 kf = *reinterpret_cast<const bf16x8*>(sK + (16 * jt + r) * LDK + 32 * u + 8 * g4);
      acc[t] = mfma(qa, kf, acc[t]);
    }
  }
  __syncthreads();   // every read of the K chunk is done: reuse it for A

  // ---- mask, decay, scale, split; stage both planes in LDS -----------------
  bf16* sA = sK;     // [2][C][LDA]
  for (int i = tid; i < 2 * C * LDA / 8; i += NTP)
    reinterpret_cast<u32x4*>(sA)[i] = u32x4{0u, 0u, 0u, 0u};
  __syncthreads();
#pragma unroll
  for (int t = 0; t < 3; ++t) {
    if (t >= ntile) continue;
    const int ct = (tiles >> (4 * t)) & 3, jt = (tiles >> (4 * t + 2)) & 3;
    // acc element i: A[16 ct + 4 g + i][16 jt + r]
    const int j = 16 * jt + r;
    const float bj = sb[j];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = 16 * ct + 4 * g4 + i;
      const float x = j <= c ? acc[t][i] * exp2_hw(sb[c] - bj) * scale : 0.f;
      const bf16 hi = (bf16)x;
      const bf16 lo = (bf16)(x - (float)hi);
      sA[c * LDA + j] = hi;
      sA[C * LDA + c * LDA + j] = lo;
    }
  }
  __syncthreads();

  // ---- store both planes row-major [2][64][64] ------------------------------
  bf16* at = amat + task * (2 * C * C);
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int p = tid + NTP * u;          // 1024 pieces of 8 elements
    const int plane = p >> 9;
    const int row = (p >> 3) & 63;
    const int c8 = p & 7;
    *reinterpret_cast<u32x4*>(at + plane * C * C + row * C + 8 * c8) =
        *reinterpret_cast<const u32x4*>(sA + plane * C * LDA + row * LDA + 8 * c8);
  }
}

template <int K>
hipError_t launch_k(const ChunkPrepParams& p, hipStream_t stream) {
  const dim3 grid((unsigned)p.seqs.num_chunks, (unsigned)p.H);
  const int per_row = p.seqs.T > 0 ? (p.seqs.T + C - 1) / C : 1;
  hipLaunchKernelGGL((chunk_prep_bf16_kernel<K>), grid, dim3(NTP), 0, stream,
                     static_cast<const bf16*>(p.q), static_cast<const bf16*>(p.k), p.g, p.g_gamma,
                     p.scale, p.H, p.seqs, per_row, p.gates, static_cast<bf16*>(p.amat),
                     static_cast<bf16*>(p.ktf));
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
