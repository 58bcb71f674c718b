// Chunked forward of elementwise-gate GLA: the general form that page
// "flash-linear-attention 中的 Simple GLA" contrasts Simple GLA with (section
// 一: the elementwise gate decays every state element on its own; section 三:
// its chunk-local cumulative gate is a [B, T, H, K] cumsum instead of a
// scalar one), with the gate a vector over the key dimension as the relinear
// pages pass it to fla's chunk_gla:
//
//     S_t = diag(exp(gk_t)) S_{t-1} + k_t v_t^T ,   o_t = scale * S_t^T q_t .
//
// Per chunk, with B[c][a] the chunk-local cumulative log2 gate of key a:
//   O = scale * ( (Q (.) 2^B) h_n + A V ),
//   A[c][j] = sum_a q_c[a] k_j[a] 2^(B[c][a] - B[j][a])  for j <= c, else 0
//   h_n+1 = diag(2^B_last) h_n + (K (.) 2^(B_last - B))^T V
// Unlike the head-wise gate, the decay between two tokens differs per key, so
// A is no plain product of Q and K^T.  It is formed by 16 x 16 blocks on the
// matrix cores, each with both operands rescaled against a reference token r
// of the block: (q_c 2^(B_c - B_r)) . (k_j 2^(B_r - B_j)) = q_c k_j 2^(B_c -
// B_j) per key.
//   * Below the diagonal (c-block I > j-block J) r is the first token of
//     block I, so both factors are <= 1 for non-positive gates: nothing can
//     overflow whatever the gates.
//   * On the diagonal r is the block's middle token; the factors are then
//     bounded by the decay over half a block, which is checked per block
//     (every key's exponent span within 2^+-100); a block whose gates are
//     stronger than that is formed elementwise, 2^(B_c - B_j) per term.
// Everything runs in fp32 (the state, the accumulation, the fp32 matrix
// cores v_mfma_f32_16x16x4_f32), so the only rounding is fp32's.
//
// Two launches.  The preparation kernel, one 8-wave workgroup per (chunk,
// head) and so parallel over every chunk, forms B and the 64 x 64 A of its
// chunk (scale folded in, zeros above the diagonal) into the workspace.  The
// chunk kernel then walks each sequence: one workgroup of 4 waves per
// (sequence, head, 32-wide V tile), the K x 32 state in MFMA accumulators with
// an LDS copy read as the q.h operand; it forms B again (a cheap per-key scan,
// needed for the q and k scaling) and reads A with the chunk's rows, the next
// chunk's rows and A being loaded into registers while the current chunk
// computes.
// v_mfma_f32_16x16x4_f32 operands, per lane l with g = l / 16, r = l % 16:
//   A operand A[m = r][k = g], B operand B[k = g][n = r],
//   result acc[i] = D[m = 4 g + i][n = r].
#include <hip/hip_runtime.h>

#include "row_stage.h"
#include "sgla_internal.h"
#include "unit_map.h"

namespace sgla {
namespace {

using stage::f32x4;
using stage::RowTile;

constexpr int C = kChunk;
constexpr int VT = 32;
constexpr int NT = 256;
constexpr int LDV = VT + 4;
constexpr int LDA = C + 4;
constexpr int LDH = VT + 4;
constexpr double kRcpLn2d = 1.4426950408889634074;
constexpr float kMaxSpan = 100.f;   // |log2 factor| allowed for a diagonal block's operands

__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ f32x4 mfma4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

template <typename TOut>
__device__ __forceinline__ TOut out_cast(float x) { return (TOut)x; }

// Chunk-local cumulative log2 gate of every key, in place over the log gates
// staged in sB (row stride LD; padding rows hold 0, so they add nothing).
// Thread (key a, part p) of NTH sums tokens [p TL, +TL) in double; the
// parts' totals are exchanged through sTot (NTH doubles), then each part
// writes its running sums with the earlier parts' total added.  With LO the
// rounding remainder of each running sum goes to sBl (hi + lo carries the
// running gate to ~2^-48 relative, so the difference of two running gates
// stays exact to float32 after a very negative gate has pushed both far from
// zero).  Ends with the workgroup's barrier.
template <int K, int NTH, int LD, bool LO>
__device__ __forceinline__ void key_cumsum_log2(float* sB, float* sBl, double* sTot) {
  constexpr int NPART = NTH / K;      // token parts of the per-key scan
  constexpr int TL = C / NPART;       // tokens per part
  static_assert(NPART * K == NTH && TL * NPART == C, "scan split");
  const int tid = threadIdx.x;
  const int a = tid % K, p = tid / K;
  float gv[TL];
  double tot = 0.0;
#pragma unroll
  for (int u = 0; u < TL; ++u) {
    gv[u] = sB[(p * TL + u) * LD + a];
    tot += (double)gv[u];
  }
  sTot[p * K + a] = tot;
  __syncthreads();
  double b = 0.0;
  for (int pp = 0; pp < p; ++pp) b += sTot[pp * K + a];
#pragma unroll
  for (int u = 0; u < TL; ++u) {
    b += (double)gv[u];
    const double t = b * kRcpLn2d;
    const float hi = (float)t;
    sB[(p * TL + u) * LD + a] = hi;
    if constexpr (LO) sBl[(p * TL + u) * LD + a] = (float)(t - (double)hi);
  }
  __syncthreads();
}

// The chunk chain's per-key scan fused with its operand scaling, over the
// log gates staged in sG: q_c (.) 2^B_c and k_c (.) 2^(B_last - B_c) in place
// in sQ and sK, and 2^B_last per key into sDl.  The suffix B_last - B_c is
// formed in double before its one rounding, so the decay of k stays exact to
// float32 whatever the gates.  Thread (key a, part p) as in key_cumsum_log2.
// Ends with the workgroup's barrier.
template <int K, int NTH, int LD>
__device__ __forceinline__ void key_scan_scale(const float* sG, float* sQ, float* sK, float* sDl,
                                               double* sTot) {
  constexpr int NPART = NTH / K;
  constexpr int TL = C / NPART;
  static_assert(NPART * K == NTH && TL * NPART == C, "scan split");
  const int tid = threadIdx.x;
  const int a = tid % K, p = tid / K;
  float gv[TL];
  double part = 0.0;
#pragma unroll
  for (int u = 0; u < TL; ++u) {
    gv[u] = sG[(p * TL + u) * LD + a];
    part += (double)gv[u];
  }
  sTot[p * K + a] = part;
  __syncthreads();
  double b = 0.0, total = 0.0;
#pragma unroll
  for (int pp = 0; pp < NPART; ++pp) {
    const double x = sTot[pp * K + a];
    if (pp < p) b += x;
    total += x;
  }
#pragma unroll
  for (int u = 0; u < TL; ++u) {
    b += (double)gv[u];
    const int c = p * TL + u;
    sQ[c * LD + a] *= exp2_hw((float)(b * kRcpLn2d));
    sK[c * LD + a] *= exp2_hw((float)((total - b) * kRcpLn2d));
  }
  if (p == NPART - 1) sDl[a] = exp2_hw((float)(total * kRcpLn2d));
  __syncthreads();
}

constexpr int NTP = 512;   // preparation threads (8 waves)

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// bf16 pair of x: hi = bf16(x), lo = bf16(x - hi), both rounded to nearest
// even.
__device__ __forceinline__ void split1(float x, __bf16& hi, __bf16& lo) {
  hi = (__bf16)x;
  lo = (__bf16)(x - (float)hi);
}

// split1 of a and b, packed two to a word (a in the low half)
__device__ __forceinline__ void split2(float a, float b, uint32_t& hi, uint32_t& lo) {
  __bf16 ha, la, hb, lb;
  split1(a, ha, la);
  split1(b, hb, lb);
  hi = (uint32_t)__builtin_bit_cast(unsigned short, ha) | ((uint32_t)__builtin_bit_cast(unsigned short, hb) << 16);
  lo = (uint32_t)__builtin_bit_cast(unsigned short, la) | ((uint32_t)__builtin_bit_cast(unsigned short, lb) << 16);
}

// Preparation of one (chunk, query head): A, 64 x 64 row-major, scale folded
// in, zeros above the diagonal -- as float32 into amat (HL = false, for the
// fp32 chain), or (HL = true, for the bf16 chain) as bf16 hi/lo planes into
// a_hl together with q~ = scale q (.) 2^B and k~ = k (.) 2^(B_last - B) as
// hi/lo planes into qk_hl and the per-key chunk decay 2^B_last into dl.
template <int K, typename TIn, bool HL>
__global__ void __launch_bounds__(NTP)
gla_prep_kernel(const TIn* __restrict__ q, const TIn* __restrict__ k, const float* __restrict__ gk,
                float* __restrict__ amat, __bf16* __restrict__ qk_hl, __bf16* __restrict__ a_hl,
                float* __restrict__ dl, float scale, int32_t H, int32_t Hkv, SeqLayout seqs) {
  constexpr int LDQ = K + 4;                    // sB row stride (floats)
  constexpr int EPL = 16 / (int)sizeof(TIn);    // elements per 16-byte piece
  constexpr int LDX = K + EPL;                  // q / k row stride (elements; 16-byte rows)
  constexpr int PR = K / EPL;                   // pieces per row
  constexpr int NPC = (C * PR + NTP - 1) / NTP; // pieces per thread
  // q and k stay in their input type in LDS (bf16: half the space, so two
  // workgroups fit a CU); the gates are float
  __shared__ __attribute__((aligned(16))) TIn sQ[C * LDX];
  __shared__ __attribute__((aligned(16))) TIn sK[C * LDX];
  // float32 inputs carry B as hi + lo (sB + sBl) so decays stay float32-exact
  // after a very negative gate; bf16 inputs keep one float (their error bar
  // is met with it, and the smaller footprint keeps two workgroups per CU)
  constexpr bool LO = sizeof(TIn) == 4;
  __shared__ __attribute__((aligned(16))) float sB[C * LDQ];   // gates, then B
  __shared__ __attribute__((aligned(16))) float sBl[LO ? C * LDQ : 1];
  __shared__ double sTot[NTP];

  const UnitMap um = map_unit(blockIdx.x, 1, Hkv, H / Hkv, seqs.num_chunks);
  if (!um.valid) return;
  const int32_t chunk = um.rank;
  const int hd = um.hd, hk = um.hk;
  int64_t t0;
  int cl;
  if (seqs.chunk_table != nullptr) {
    const ChunkEntry e = seqs.chunk_table[chunk];
    t0 = e.t0;
    cl = e.len;
  } else {
    const int32_t ncs = (seqs.T + seqs.chunk - 1) / seqs.chunk;
    const int32_t row = chunk / ncs, m = chunk - row * ncs;
    t0 = (int64_t)row * seqs.T + (int64_t)m * seqs.chunk;
    cl = min(seqs.chunk, seqs.T - m * seqs.chunk);
  }
  const int tid = threadIdx.x;
  const int lane = tid & 63, g4 = lane >> 4, r = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index, uniform
  {
    // rows past the chunk's end are zero
    uint4 qx[NPC], kx[NPC];
    const TIn* qb = q + (t0 * H + hd) * K;
    const TIn* kb = k + (t0 * Hkv + hk) * K;
#pragma unroll
    for (int u = 0; u < NPC; ++u) {
      const int p = tid + NTP * u;
      const int c = p / PR, e = (p % PR) * EPL;
      qx[u] = make_uint4(0u, 0u, 0u, 0u);
      kx[u] = make_uint4(0u, 0u, 0u, 0u);
      if ((C * PR % NTP == 0 || p < C * PR) && c < cl) {
        qx[u] = *reinterpret_cast<const uint4*>(qb + c * (int64_t)H * K + e);
        kx[u] = *reinterpret_cast<const uint4*>(kb + c * (int64_t)Hkv * K + e);
      }
    }
    RowTile<K, NTP, float> gt;
    gt.load(gk + (t0 * H + hd) * K, (int64_t)H * K, cl);
#pragma unroll
    for (int u = 0; u < NPC; ++u) {
      const int p = tid + NTP * u;
      if (C * PR % NTP == 0 || p < C * PR) {
        *reinterpret_cast<uint4*>(sQ + (p / PR) * LDX + (p % PR) * EPL) = qx[u];
        *reinterpret_cast<uint4*>(sK + (p / PR) * LDX + (p % PR) * EPL) = kx[u];
      }
    }
    gt.store(sB, LDQ);
  }
  __syncthreads();
  key_cumsum_log2<K, NTP, LDQ, LO>(sB, sBl, sTot);
  auto fq = [&](int c, int a) { return (float)sQ[c * LDX + a]; };
  auto fk = [&](int c, int a) { return (float)sK[c * LDX + a]; };
  // log2 decay B[c][a] - B[j][a] (hi + lo when carried)
  auto dB = [&](int c, int j, int a) {
    const float d = sB[c * LDQ + a] - sB[j * LDQ + a];
    if constexpr (LO) return d + (sBl[c * LDQ + a] - sBl[j * LDQ + a]);
    return d;
  };

  const int64_t rec = (int64_t)chunk * H + hd;
  float* ab = HL ? nullptr : amat + rec * (C * C);
  __bf16* ahl = HL ? a_hl + rec * (2 * C * C) : nullptr;
  auto put_a = [&](int c, int j, float x) {
    if constexpr (HL) {
      __bf16 hi, lo;
      split1(x, hi, lo);
      ahl[c * C + j] = hi;
      ahl[C * C + c * C + j] = lo;
    } else {
      ab[c * C + j] = x;
    }
  };
  if constexpr (HL) {
    // q~ and k~, eight keys of one row per thread and step, as 16-byte stores
    // of each plane (rows past the chunk's end are zero in sQ and sK); the
    // chunk's decay per key
    __bf16* qo = qk_hl + rec * (4 * C * K);
    __bf16* ko = qo + 2 * C * K;
    for (int i = tid; i < C * K / 8; i += NTP) {
      const int c = i / (K / 8), a0 = (i % (K / 8)) * 8;
      u32x4 qh, ql, kh, kl;
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        float xq[2], xk[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int a = a0 + e + u;
          const float b = sB[c * LDQ + a];
          xq[u] = scale * fq(c, a) * exp2_hw(b);
          xk[u] = fk(c, a) * exp2_hw(sB[(C - 1) * LDQ + a] - b);
        }
        uint32_t h2, l2;
        split2(xq[0], xq[1], h2, l2);
        qh[e / 2] = h2;
        ql[e / 2] = l2;
        split2(xk[0], xk[1], h2, l2);
        kh[e / 2] = h2;
        kl[e / 2] = l2;
      }
      *reinterpret_cast<u32x4*>(qo + 8 * i) = qh;
      *reinterpret_cast<u32x4*>(qo + C * K + 8 * i) = ql;
      *reinterpret_cast<u32x4*>(ko + 8 * i) = kh;
      *reinterpret_cast<u32x4*>(ko + C * K + 8 * i) = kl;
    }
    for (int a = tid; a < K; a += NTP) dl[rec * K + a] = exp2_hw(sB[(C - 1) * LDQ + a]);
  }
  if (w < 3) {
    // ---- below the diagonal: blocks (I, J) in the order (1,0) (2,0) (2,1)
    //      (3,0) (3,1) (3,2), two per wave as interleaved chains; the
    //      reference token is the first of block I, so both factors are <= 1
    auto block_ij = [](int bi, int& I, int& J) {
      I = bi == 0 ? 1 : (bi < 3 ? 2 : 3);
      J = bi == 0 ? 0 : (bi < 3 ? bi - 1 : bi - 3);
    };
    int I0, J0, I1, J1;
    block_ij(2 * w, I0, J0);
    block_ij(2 * w + 1, I1, J1);
    f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = acc0;
#pragma unroll 4
    for (int ks = 0; ks < K / 4; ++ks) {
      const int a = 4 * ks + g4;
      const int r0 = 16 * I0, r1 = 16 * I1;
      const int c0 = 16 * I0 + r, j0 = 16 * J0 + r, c1 = 16 * I1 + r, j1 = 16 * J1 + r;
      acc0 = mfma4(fq(c0, a) * exp2_hw(dB(c0, r0, a)), fk(j0, a) * exp2_hw(dB(r0, j0, a)), acc0);
      acc1 = mfma4(fq(c1, a) * exp2_hw(dB(c1, r1, a)), fk(j1, a) * exp2_hw(dB(r1, j1, a)), acc1);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      put_a(16 * I0 + 4 * g4 + i, 16 * J0 + r, acc0[i] * scale);
      put_a(16 * I1 + 4 * g4 + i, 16 * J1 + r, acc1[i] * scale);
    }
  } else if (w < 7) {
    // ---- on the diagonal: block I = w - 3, reference its middle token; a
    //      block whose exponent span is too wide is formed elementwise -------
    const int I = w - 3, rr = 16 * I + 8;
    float span = 0.f;
    for (int a = lane; a < K; a += 64) {
      const float br = sB[rr * LDQ + a];
      span = fmaxf(span, fmaxf(sB[(16 * I) * LDQ + a] - br, br - sB[(16 * I + 15) * LDQ + a]));
    }
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) span = fmaxf(span, __shfl_xor(span, d, 64));
    if (span <= kMaxSpan) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
      for (int ks = 0; ks < K / 4; ++ks) {
        const int a = 4 * ks + g4;
        const int ci = 16 * I + r;
        acc = mfma4(fq(ci, a) * exp2_hw(dB(ci, rr, a)), fk(ci, a) * exp2_hw(dB(rr, ci, a)), acc);
      }
      const int j = 16 * I + r;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int c = 16 * I + 4 * g4 + i;
        put_a(c, j, j <= c ? acc[i] * scale : 0.f);   // a select: an overflowed upper entry is dropped
      }
    } else {
      // elementwise: one (c, j) entry of the block per lane and pass
      for (int pp = 0; pp < 4; ++pp) {
        const int e = lane + 64 * pp;
        const int c = 16 * I + (e >> 4), j = 16 * I + (e & 15);
        float x = 0.f;
        if (j <= c) {
          for (int a = 0; a < K; ++a) x = fmaf(fq(c, a) * fk(j, a), exp2_hw(dB(c, j, a)), x);
        }
        put_a(c, j, x * scale);
      }
    }
  } else {
    // ---- the six blocks above the diagonal are zero ----------------------
    for (int i = lane; i < 6 * 256; i += 64) {
      const int tt = i >> 8, e = i & 255;
      const int ctile = tt < 3 ? 0 : (tt < 5 ? 1 : 2);
      const int jtile = tt < 3 ? tt + 1 : (tt < 5 ? tt - 1 : 3);
      put_a(16 * ctile + (e >> 4), 16 * jtile + (e & 15), 0.f);
    }
  }
}

template <int K, typename TIn, typename TOut>
__global__ void __launch_bounds__(NT)
gla_chunk_fwd_kernel(const TIn* __restrict__ q, const TIn* __restrict__ k,
                     const TIn* __restrict__ v, const float* __restrict__ gk,
                     const float* __restrict__ h0, const float* __restrict__ amat, TOut* __restrict__ o,
                     float* __restrict__ ht, float scale, int32_t H, int32_t Hkv, int32_t V, StateLayout sl,
                     SeqLayout seqs) {
  constexpr int LDQ = K + 4;          // row stride of Q, K, B (floats; 16-byte rows)
  constexpr int NKT = K / 16;
  constexpr int NST = NKT * 2;        // 16 x 16 state tiles (x 2 column tiles)
  constexpr int SPW = (NST + 3) / 4;  // per wave
  __shared__ __attribute__((aligned(16))) float sQ[C * LDQ];
  __shared__ __attribute__((aligned(16))) float sK[C * LDQ];
  __shared__ __attribute__((aligned(16))) float sB[C * LDQ];   // log gates
  __shared__ __attribute__((aligned(16))) float sV[C * LDV];
  __shared__ __attribute__((aligned(16))) float sA[C * LDA];
  __shared__ float sH[K * LDH];
  __shared__ float sDl[K];                                      // 2^B_last per key
  __shared__ double sTot[NT];

  const UnitMap um = map_unit(blockIdx.x, V / VT, Hkv, H / Hkv, seqs.num_seqs);
  if (!um.valid) return;
  const int hd = um.hd, hk = um.hk, vt = um.vt;
  int64_t bos;
  int32_t len, seq, chunk0;
  if (seqs.seq_table != nullptr) {
    const SeqEntry e = seqs.seq_table[um.rank];
    bos = e.bos;
    len = e.len;
    seq = e.seq;
    chunk0 = e.chunk0;
  } else {
    bos = (int64_t)um.rank * seqs.T;
    len = seqs.T;
    seq = um.rank;
    chunk0 = um.rank * ((seqs.T + seqs.chunk - 1) / seqs.chunk);
  }
  const int tid = threadIdx.x;
  const int lane = tid & 63, g4 = lane >> 4, r = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index, uniform
  const int64_t su = ((int64_t)seq * H + hd) * K * V;
  auto sidx = [&](int row, int c) { return su + (int64_t)row * sl.rs + (int64_t)(vt * VT + c) * sl.cs; };

  f32x4 hs[SPW];
#pragma unroll
  for (int s = 0; s < SPW; ++s) {
    const int st = w + 4 * s;
    hs[s] = f32x4{0.f, 0.f, 0.f, 0.f};
    if ((NST % 4 == 0 || st < NST) && h0 != nullptr) {
      const int kt = st >> 1, ctl = st & 1;
#pragma unroll
      for (int i = 0; i < 4; ++i) hs[s][i] = h0[sidx(16 * kt + 4 * g4 + i, 16 * ctl + r)];
    }
  }
  auto publish_state = [&]() {
#pragma unroll
    for (int s = 0; s < SPW; ++s) {
      const int st = w + 4 * s;
      if (NST % 4 == 0 || st < NST) {
        const int kt = st >> 1, ctl = st & 1;
#pragma unroll
        for (int i = 0; i < 4; ++i) sH[(16 * kt + 4 * g4 + i) * LDH + 16 * ctl + r] = hs[s][i];
      }
    }
  };
  publish_state();

  // next chunk's rows and A, loaded one chunk ahead
  RowTile<K, NT, TIn> qt, kt;
  RowTile<K, NT, float> gt;
  RowTile<VT, NT, TIn> vtl;
  RowTile<C, NT, float> at;
  const int nchunks = (len + seqs.chunk - 1) / seqs.chunk;
  auto load_chunk = [&](int m) {
    const int64_t t0 = bos + (int64_t)m * seqs.chunk;
    const int cl = min(seqs.chunk, len - m * seqs.chunk);
    qt.load(q + (t0 * H + hd) * K, (int64_t)H * K, cl);
    kt.load(k + (t0 * Hkv + hk) * K, (int64_t)Hkv * K, cl);
    gt.load(gk + (t0 * H + hd) * K, (int64_t)H * K, cl);
    vtl.load(v + (t0 * Hkv + hk) * V + vt * VT, (int64_t)Hkv * V, cl);
    at.load(amat + ((int64_t)(chunk0 + m) * H + hd) * (C * C), C, C);
  };
  if (nchunks > 0) load_chunk(0);

  // A chunk's outputs are stored at the start of the next iteration (or after
  // the loop): the wait for the prefetched rows at the top of an iteration
  // covers every memory operation issued before it, stores included, so
  // stores issued right after that wait have a whole iteration to complete.
  const int ct0 = w >> 1, ct1 = ct0 + 2, cv = w & 1;
  float pend[8];
  int64_t pend_t0 = 0;
  int pend_cl = 0;
  auto flush_out = [&]() {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c0 = 16 * ct0 + 4 * g4 + i, c1 = 16 * ct1 + 4 * g4 + i;
      if (c0 < pend_cl)
        o[((pend_t0 + c0) * H + hd) * (int64_t)V + vt * VT + 16 * cv + r] = out_cast<TOut>(pend[i]);
      if (c1 < pend_cl)
        o[((pend_t0 + c1) * H + hd) * (int64_t)V + vt * VT + 16 * cv + r] = out_cast<TOut>(pend[4 + i]);
    }
  };

  for (int m = 0; m < nchunks; ++m) {
    const int64_t t0 = bos + (int64_t)m * seqs.chunk;
    const int cl = min(seqs.chunk, len - m * seqs.chunk);
    qt.store(sQ, LDQ);
    kt.store(sK, LDQ);
    gt.store(sB, LDQ);
    vtl.store(sV, LDV);
    at.store(sA, LDA);
    if (m > 0) flush_out();
    __syncthreads();

    // ---- B, the chunk-local cumulative log2 gate of every key, applied in
    //      place: Q (.) 2^B and K (.) 2^(B_last - B) ------------------------
    key_scan_scale<K, NT, LDQ>(sB, sQ, sK, sDl, sTot);
    // the next chunk's rows go into registers now: they are held through the
    // rest of this chunk
    if (m + 1 < nchunks) load_chunk(m + 1);

    // ---- output tiles (ct, cv) and (ct + 2, cv), ct = w / 2, cv = w % 2: the
    //      two tiles share their B operands and run as interleaved chains ------
    {
      f32x4 in0 = {0.f, 0.f, 0.f, 0.f}, in1 = in0, ia0 = in0, ia1 = in0;
#pragma unroll 8
      for (int ks = 0; ks < K / 4; ++ks) {
        const float b = sH[(4 * ks + g4) * LDH + 16 * cv + r];
        in0 = mfma4(sQ[(16 * ct0 + r) * LDQ + 4 * ks + g4], b, in0);
        in1 = mfma4(sQ[(16 * ct1 + r) * LDQ + 4 * ks + g4], b, in1);
      }
      for (int js = 0; js < 4 * (ct0 + 1); ++js) {
        const float b = sV[(4 * js + g4) * LDV + 16 * cv + r];
        ia0 = mfma4(sA[(16 * ct0 + r) * LDA + 4 * js + g4], b, ia0);
        ia1 = mfma4(sA[(16 * ct1 + r) * LDA + 4 * js + g4], b, ia1);
      }
      for (int js = 4 * (ct0 + 1); js < 4 * (ct1 + 1); ++js)
        ia1 = mfma4(sA[(16 * ct1 + r) * LDA + 4 * js + g4], sV[(4 * js + g4) * LDV + 16 * cv + r], ia1);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pend[i] = ia0[i] + scale * in0[i];
        pend[4 + i] = ia1[i] + scale * in1[i];
      }
      pend_t0 = t0;
      pend_cl = cl;
    }

    // ---- state: h <- diag(2^B_last) h + (K (.) 2^(B_last - B))^T V ---------------
    //      (the wave's tiles share the column tile ctl = w % 2, so they share
    //      the V operand and run as interleaved chains)
    {
      const int ctl = w & 1;
#pragma unroll
      for (int s = 0; s < SPW; ++s) {
        const int st = w + 4 * s;
        if (NST % 4 != 0 && st >= NST) continue;
        const int kt = st >> 1;
#pragma unroll
        for (int i = 0; i < 4; ++i) hs[s][i] *= sDl[16 * kt + 4 * g4 + i];
      }
#pragma unroll 4
      for (int cs = 0; cs < C / 4; ++cs) {
        const int c = 4 * cs + g4;
        const float b = sV[c * LDV + 16 * ctl + r];
#pragma unroll
        for (int s = 0; s < SPW; ++s) {
          const int st = w + 4 * s;
          if (NST % 4 != 0 && st >= NST) continue;
          hs[s] = mfma4(sK[c * LDQ + 16 * (st >> 1) + r], b, hs[s]);
        }
      }
    }
    __syncthreads();   // every read of sQ, sK, sV, sA, sDl and the old sH is done
    publish_state();
  }
  if (nchunks > 0) flush_out();
  if (ht != nullptr) {
#pragma unroll
    for (int s = 0; s < SPW; ++s) {
      const int st = w + 4 * s;
      if (NST % 4 == 0 || st < NST) {
        const int kt = st >> 1, ctl = st & 1;
#pragma unroll
        for (int i = 0; i < 4; ++i) ht[sidx(16 * kt + 4 * g4 + i, 16 * ctl + r)] = hs[s][i];
      }
    }
  }
}

template <int K, typename TIn, typename TOut>
hipError_t launch_k(const GlaFwdParams& p, hipStream_t stream) {
  if (p.seqs.num_seqs == 0) return hipSuccess;
  const bool hl = gla_bf16_chain(sizeof(TIn) == 2, K, p.V);
  if (p.seqs.num_chunks > 0) {
    const dim3 pgrid((unsigned)unit_grid(p.seqs.num_chunks, p.Hkv, p.H / p.Hkv, 1));
    if (hl) {
      hipLaunchKernelGGL((gla_prep_kernel<K, TIn, true>), pgrid, dim3(NTP), 0, stream,
                         static_cast<const TIn*>(p.q), static_cast<const TIn*>(p.k), p.gk, nullptr,
                         static_cast<__bf16*>(p.qk_hl), static_cast<__bf16*>(p.a_hl), p.dl, p.scale, p.H,
                         p.Hkv, p.seqs);
    } else {
      hipLaunchKernelGGL((gla_prep_kernel<K, TIn, false>), pgrid, dim3(NTP), 0, stream,
                         static_cast<const TIn*>(p.q), static_cast<const TIn*>(p.k), p.gk, p.amat, nullptr,
                         nullptr, nullptr, p.scale, p.H, p.Hkv, p.seqs);
    }
  }
  if (hl) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_gla_chain_bf16(p, stream);
  }
  const dim3 grid((unsigned)unit_grid(p.seqs.num_seqs, p.Hkv, p.H / p.Hkv, p.V / VT));
  hipLaunchKernelGGL((gla_chunk_fwd_kernel<K, TIn, TOut>), grid, dim3(NT), 0, stream,
                     static_cast<const TIn*>(p.q), static_cast<const TIn*>(p.k),
                     static_cast<const TIn*>(p.v), p.gk, p.h0, p.amat, static_cast<TOut*>(p.o), p.ht,
                     p.scale, p.H, p.Hkv, p.V, p.sl, p.seqs);
  return hipGetLastError();
}

template <typename TIn, typename TOut>
hipError_t launch_io(const GlaFwdParams& p, hipStream_t stream) {
  switch (p.K) {
    case 16: return launch_k<16, TIn, TOut>(p, stream);
    case 32: return launch_k<32, TIn, TOut>(p, stream);
    case 64: return launch_k<64, TIn, TOut>(p, stream);
    case 128: return launch_k<128, TIn, TOut>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_gla_chunk_fwd(const GlaFwdParams& p, hipStream_t stream) {
  if (p.qkv_bf16) return p.o_bf16 ? launch_io<__bf16, __bf16>(p, stream) : launch_io<__bf16, float>(p, stream);
  return p.o_bf16 ? launch_io<float, __bf16>(p, stream) : launch_io<float, float>(p, stream);
}

}  // namespace sgla
