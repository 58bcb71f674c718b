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
//             as bf16 hi + lo (A = hi + lo to ~2^-16 relative).
// Besides the gates, three operand streams of chunk_fwd_bf16_wide.hip are
// written in that kernel's MFMA operand order, one 1 KB block (64 lanes x
// 16 bytes, lane-major) per operand, so every load there is one contiguous
// kilobyte:
//   Q   blocks (kb, c2, s): lane (n = l % 32, h = l / 32) holds
//       Q[32 c2 + n][32 kb + 16 s + 8 h + e], e = 0..7       (q.h A operand)
//   K^T blocks (kb, ts):    lane (n, h) holds
//       K[16 ts + 8 h + e][32 kb + perm(n)]                  (update A operand)
//       with perm swapping the middle two 4-key blocks of each 16, the state
//       row order of that kernel
//   A   blocks (ct, u, plane): lane (r = l % 16, g = l / 16) holds
//       A[16 ct + r][32 u + 8 g + e]                         (intra A operand)
// Tokens at or past L read as zeros (q, k, g), so their A rows and columns,
// Q rows and K^T entries are zero and b stays at b_last.
//
// With grouped kv heads the K^T blocks depend on the kv head alone: they are
// stored once per (chunk, kv head), by the group's first query head.
//
// One workgroup of four waves per (chunk, query head), walking the keys in
// slices of 128.  Every slice's K rows and Q blocks are loaded into registers
// up front (a slice staged while only the next one was loading waited a full
// memory latency per slice: -4 % on the K = 512 call), then each slice's K
// rows go to LDS and its Q and K^T blocks are written out.  Q K^T runs on
// v_mfma_f32_32x32x16_bf16: wave w covers query rows [32 (w / 2), +32) over
// half of every slice's keys (blocks 4 sl + 2 (w % 2) + {0, 1}); the two halves
// are added in LDS.
#include <hip/hip_runtime.h>

#include "gate_scan.h"
#include "mfma_common.h"
#include "sgla_internal.h"

namespace sgla {
namespace {

using namespace mf;

constexpr int C = kChunk;
constexpr int NTP = 256;          // threads
constexpr int LDS_ACC = C + 4;    // row stride of the fp32 A accumulator (floats)

template <int K>
__global__ void __launch_bounds__(NTP)
chunk_prep_bf16_kernel(const bf16* __restrict__ q, const bf16* __restrict__ k,
                       const float* __restrict__ g, const float* __restrict__ g_gamma, float scale,
                       int32_t H, int32_t Hkv, SeqLayout seqs, int32_t chunks_per_row,
                       float* __restrict__ gates,
                       bf16* __restrict__ amat, bf16* __restrict__ ktf, bf16* __restrict__ qfr) {
  constexpr int KSL = 128;              // keys per slice
  constexpr int NS = K / KSL;           // slices
  constexpr int LDK = KSL + 8;          // slice row stride: conflict-free 16-byte row reads
  constexpr int KP = KSL / 8;           // 16-byte pieces per slice row
  constexpr int NKS = C * KP / NTP;     // K pieces per thread and slice
  static_assert(NKS * NTP == C * KP, "slice split");
  static_assert(C * LDS_ACC * 4 <= C * LDK * 2, "A accumulator aliases the K slice");
  __shared__ __attribute__((aligned(16))) bf16 sK[C * LDK];
  __shared__ float sb[C];

  // ---- which (chunk, query head) this workgroup prepares ------------------
  // Work units wu = hk * num_chunks + chunk (chunk fastest) are dealt to the
  // XCDs round-robin; the n_rep query heads of a unit follow each other on its
  // XCD, so the K chunk they share is re-read from that XCD's L2.
  const int n_rep = H / Hkv;
  const int xcd = blockIdx.x % kXcds;
  const int slot = blockIdx.x / kXcds;
  const int gs = slot / n_rep;
  const int wu = gs * kXcds + xcd;
  if (wu >= seqs.num_chunks * Hkv) return;
  const int hk = wu / seqs.num_chunks;
  const int gc = wu - hk * seqs.num_chunks;   // global chunk index
  const int hd = hk * n_rep + (slot - gs * n_rep);
  const bool write_kt = hd == hk * n_rep;
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
  const int l32 = lane & 31;
  const int hf = lane >> 5;
  const int grp = lane >> 4;
  const int g4 = lane >> 4;
  const int r = lane & 15;
  const int c2 = w >> 1;           // query rows [32 c2, +32)
  const int kh2 = w & 1;           // key half of every slice: blocks 4 sl + 2 kh2 + {0, 1}
  const int64_t task = (int64_t)gc * H + hd;
  const int RS = H * K;            // elements between consecutive tokens of q
  const int RSK = Hkv * K;         //                                     of k

  // ---- slice loads: the K slice (all rows) and this wave's Q blocks ---------
  const auto rk = make_rsrc(k + (t0 * Hkv + hk) * (int64_t)K, (uint32_t)cl * RSK * 2);
  const auto rq = make_rsrc(q + (t0 * H + hd) * (int64_t)K, (uint32_t)cl * RS * 2);
  // the gate word first: the gate scan waits for it alone, not for the rows
  float gx = 0.f;
  if (w == 0 && g != nullptr) {
    const auto rg = make_rsrc(g + t0 * H + hd, (uint32_t)cl * H * 4);
    gx = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rg, (uint32_t)(lane * H * 4), 0, 0));
  }
  // every slice's K rows and Q blocks, loaded up front
  u32x4 kx[NS][NKS];
  bf16x8 qx[NS][2][2];
#pragma unroll
  for (int sl = 0; sl < NS; ++sl) {
#pragma unroll
    for (int i = 0; i < NKS; ++i) {
      const int p = tid + NTP * i;
      kx[sl][i] = __builtin_amdgcn_raw_buffer_load_b128(
          rk, (uint32_t)((p / KP) * RSK + KSL * sl + (p % KP) * 8) * 2, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int s = 0; s < 2; ++s)
        qx[sl][i][s] = __builtin_bit_cast(
            bf16x8, __builtin_amdgcn_raw_buffer_load_b128(
                        rq, (uint32_t)((32 * c2 + l32) * RS + 32 * (4 * sl + 2 * kh2 + i) + 16 * s + 8 * hf) * 2,
                        0, 0));
  }

  // ---- gates ----------------------------------------------------------------
  if (w == 0) {
    float b;
    if (g != nullptr) {
      b = wave_cumsum_log2(gx);
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

  // ---- per slice: K slice to LDS, Q and K^T blocks out, partial Q K^T ------
  f32x16 acc[2];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int a = 0; a < 16; ++a) acc[t][a] = 0.f;
  bf16* qo = qfr + task * (int64_t)K * C;
  bf16* kt = ktf + ((int64_t)gc * Hkv + hk) * K * C;
  auto slice = [&](const int sl) {
#pragma unroll
    for (int i = 0; i < NKS; ++i) {
      const int p = tid + NTP * i;
      *reinterpret_cast<u32x4*>(sK + (p / KP) * LDK + (p % KP) * 8) = kx[sl][i];
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int s = 0; s < 2; ++s)
        *reinterpret_cast<bf16x8*>(qo + ((((4 * sl + 2 * kh2 + i) * 2 + c2) * 2 + s) * 64 + lane) * 8) = qx[sl][i][s];
    __syncthreads();   // slice sl staged
    // K^T blocks (kb, ts) of this slice's four key blocks, once per kv head
    if (write_kt) {
#pragma unroll
      for (int f = w; f < 16; f += 4) {
        const int kbl = f >> 2, ts = f & 3;
        const int row0 = 16 * ts + 8 * (grp >> 1);
        const int col0 = 32 * kbl + 16 * (grp & 1);
        const bf16x8 x = cat(tr_read_perm(sK, LDK, row0, col0), tr_read_perm(sK, LDK, row0 + 4, col0));
        *reinterpret_cast<bf16x8*>(kt + (((4 * sl + kbl) * 4 + ts) * 64 + lane) * 8) = x;
      }
    }
    // partial Q K^T over this wave's two key blocks: tiles (c2, j2), j2 <= c2
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const int col = 32 * (2 * kh2 + i) + 16 * s + 8 * hf;
        const bf16x8 k0f = *reinterpret_cast<const bf16x8*>(sK + l32 * LDK + col);
        acc[0] = mfma32(qx[sl][i][s], k0f, acc[0]);
        if (c2 == 1) {
          const bf16x8 k1f = *reinterpret_cast<const bf16x8*>(sK + (32 + l32) * LDK + col);
          acc[1] = mfma32(qx[sl][i][s], k1f, acc[1]);
        }
      }
    __syncthreads();   // every read of the slice is done
  };
#pragma unroll
  for (int sl = 0; sl < NS; ++sl) slice(sl);

  // ---- add the two key halves in LDS (fixed order: deterministic) ---------
  // acc[t][4 jj + i] = D[c = 32 c2 + 8 jj + 4 hf + i][j = 32 t + l32]
  float* sacc = reinterpret_cast<float*>(sK);
  auto tile_io = [&](bool add) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      if (t > c2) continue;
#pragma unroll
      for (int a = 0; a < 16; ++a) {
        float* p = sacc + (32 * c2 + 8 * (a >> 2) + 4 * hf + (a & 3)) * LDS_ACC + 32 * t + l32;
        *p = add ? *p + acc[t][a] : acc[t][a];
      }
    }
  };
  if ((w & 1) == 0) tile_io(false);
  __syncthreads();
  if ((w & 1) == 1) tile_io(true);
  __syncthreads();

  // ---- mask, decay, scale, split; A blocks out ------------------------------
  // wave w: c tile ct = w, u = 0 and (ct >= 2) u = 1
  {
    const int ct = w;
    const int c = 16 * ct + r;
    const float bc = sb[c];
    bf16* ao = amat + task * (2 * C * C);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      if (u == 1 && ct < 2) continue;
      const int j0 = 32 * u + 8 * g4;
      const f32x4 a0 = *reinterpret_cast<const f32x4*>(sacc + c * LDS_ACC + j0);
      const f32x4 a1 = *reinterpret_cast<const f32x4*>(sacc + c * LDS_ACC + j0 + 4);
      const f32x4 b0 = *reinterpret_cast<const f32x4*>(sb + j0);
      const f32x4 b1 = *reinterpret_cast<const f32x4*>(sb + j0 + 4);
      float x[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[e] = j0 + e <= c ? a0[e] * exp2_hw(bc - b0[e]) * scale : 0.f;
        x[4 + e] = j0 + 4 + e <= c ? a1[e] * exp2_hw(bc - b1[e]) * scale : 0.f;
      }
      bf16x8 hi, lo;
      split8(x, hi, lo);
      *reinterpret_cast<bf16x8*>(ao + (((ct * 2 + u) * 2 + 0) * 64 + lane) * 8) = hi;
      *reinterpret_cast<bf16x8*>(ao + (((ct * 2 + u) * 2 + 1) * 64 + lane) * 8) = lo;
    }
  }
}

template <int K>
hipError_t launch_k(const ChunkPrepParams& p, hipStream_t stream) {
  const int64_t units = (int64_t)p.seqs.num_chunks * p.Hkv;
  const dim3 grid((unsigned)((units + kXcds - 1) / kXcds * kXcds * (p.H / p.Hkv)));
  const int per_row = p.seqs.T > 0 ? (p.seqs.T + C - 1) / C : 1;
  hipLaunchKernelGGL((chunk_prep_bf16_kernel<K>), grid, dim3(NTP), 0, stream,
                     static_cast<const bf16*>(p.q), static_cast<const bf16*>(p.k), p.g, p.g_gamma,
                     p.scale, p.H, p.Hkv, p.seqs, per_row, p.gates, static_cast<bf16*>(p.amat),
                     static_cast<bf16*>(p.ktf), static_cast<bf16*>(p.qfr));
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
