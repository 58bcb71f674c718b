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
// A is no plain product of Q and K^T.  It is formed by 16 x 16 blocks:
//   * blocks below the diagonal (c-block I > j-block J) on the matrix cores,
//     both operands rescaled against the first token r of block I:
//     (q_c 2^(B_c - B_r)) . (k_j 2^(B_r - B_j)), each factor <= 1 for
//     non-positive gates, so nothing can overflow whatever the gates;
//   * the four diagonal blocks elementwise, 2^(B_c - B_j) per key.
// Everything runs in fp32 (the state, the accumulation, the fp32 matrix
// cores v_mfma_f32_16x16x4_f32), so the only rounding is fp32's.
//
// Work layout as the fp32 head-wise kernel: one workgroup of 4 waves per
// (sequence, head, 32-wide V tile), the K x 32 state in MFMA accumulators
// with an LDS copy read as the q.h operand; the next chunk's rows are loaded
// into registers while the current chunk computes.
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
constexpr double kRcpLn2 = 1.4426950408889634074;

__device__ __forceinline__ f32x4 mfma4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

template <typename TOut>
__device__ __forceinline__ TOut out_cast(float x) { return (TOut)x; }

template <int K, typename TIn, typename TOut>
__global__ void __launch_bounds__(NT)
gla_chunk_fwd_kernel(const TIn* __restrict__ q, const TIn* __restrict__ k,
                     const TIn* __restrict__ v, const float* __restrict__ gk,
                     const float* __restrict__ h0, TOut* __restrict__ o, float* __restrict__ ht,
                     float scale, int32_t H, int32_t Hkv, int32_t V, StateLayout sl, SeqLayout seqs) {
  constexpr int LDQ = K + 4;          // row stride of Q, K, B (floats; 16-byte rows)
  constexpr int NKT = K / 16;
  constexpr int NST = NKT * 2;        // 16 x 16 state tiles (x 2 column tiles)
  constexpr int SPW = (NST + 3) / 4;  // per wave
  __shared__ __attribute__((aligned(16))) float sQ[C * LDQ];
  __shared__ __attribute__((aligned(16))) float sK[C * LDQ];
  __shared__ __attribute__((aligned(16))) float sB[C * LDQ];   // gates, then B
  __shared__ float sV[C * LDV];
  __shared__ float sA[C * LDA];
  __shared__ float sH[K * LDH];

  const UnitMap um = map_unit(blockIdx.x, V / VT, Hkv, H / Hkv, seqs.num_seqs);
  if (!um.valid) return;
  const int hd = um.hd, hk = um.hk, vt = um.vt;
  int64_t bos;
  int32_t len, seq;
  if (seqs.seq_table != nullptr) {
    const SeqEntry e = seqs.seq_table[um.rank];
    bos = e.bos;
    len = e.len;
    seq = e.seq;
  } else {
    bos = (int64_t)um.rank * seqs.T;
    len = seqs.T;
    seq = um.rank;
  }
  const int tid = threadIdx.x;
  const int lane = tid & 63, g4 = lane >> 4, r = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index, uniform
  const int64_t su = ((int64_t)seq * H + hd) * K * V;
  auto sidx = [&](int row, int c) { return su + (int64_t)row * sl.rs + (int64_t)(vt * VT + c) * sl.cs; };

  // blocks above the diagonal of A are never written: zero them once
  for (int i = tid; i < 6 * 256; i += NT) {
    const int tt = i >> 8, e = i & 255;
    const int ctile = tt < 3 ? 0 : (tt < 5 ? 1 : 2);
    const int jtile = tt < 3 ? tt + 1 : (tt < 5 ? tt - 1 : 3);
    sA[(16 * ctile + (e >> 4)) * LDA + 16 * jtile + (e & 15)] = 0.f;
  }

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

  // next chunk's rows, loaded one chunk ahead
  RowTile<K, NT, TIn> qt, kt;
  RowTile<K, NT, float> gt;
  RowTile<VT, NT, TIn> vtl;
  const int nchunks = (len + C - 1) / C;
  auto load_chunk = [&](int m) {
    const int64_t t0 = bos + (int64_t)m * C;
    const int cl = min(C, len - m * C);
    qt.load(q + (t0 * H + hd) * K, (int64_t)H * K, cl);
    kt.load(k + (t0 * Hkv + hk) * K, (int64_t)Hkv * K, cl);
    gt.load(gk + (t0 * H + hd) * K, (int64_t)H * K, cl);
    vtl.load(v + (t0 * Hkv + hk) * V + vt * VT, (int64_t)Hkv * V, cl);
  };
  if (nchunks > 0) load_chunk(0);

  for (int m = 0; m < nchunks; ++m) {
    const int64_t t0 = bos + (int64_t)m * C;
    const int cl = min(C, len - m * C);
    qt.store(sQ, LDQ);
    kt.store(sK, LDQ);
    gt.store(sB, LDQ);
    vtl.store(sV, LDV);
    __syncthreads();
    if (m + 1 < nchunks) load_chunk(m + 1);

    // ---- B: chunk-local cumulative log2 gate of every key (padding adds 0) --
    for (int a = tid; a < K; a += NT) {
      double b = 0.0;
      for (int c = 0; c < C; ++c) {
        b += (double)sB[c * LDQ + a];
        sB[c * LDQ + a] = (float)(b * kRcpLn2);
      }
    }
    __syncthreads();

    // ---- A, blocks below the diagonal: wave w takes blocks w and w + 4 ------
    //      (I, J) in order (1,0) (2,0) (2,1) (3,0) (3,1) (3,2)
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int bi = w + 4 * t;
      if (bi >= 6) continue;
      const int I = bi == 0 ? 1 : (bi < 3 ? 2 : 3);
      const int J = bi == 0 ? 0 : (bi < 3 ? bi - 1 : bi - 3);
      const int rr = 16 * I;           // reference token: first of block I
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
      for (int ks = 0; ks < K / 4; ++ks) {
        const int a = 4 * ks + g4;
        const float br = sB[rr * LDQ + a];
        const int ci = (16 * I + r) * LDQ + a, ji = (16 * J + r) * LDQ + a;
        acc = mfma4(sQ[ci] * exp2f(sB[ci] - br), sK[ji] * exp2f(br - sB[ji]), acc);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) sA[(16 * I + 4 * g4 + i) * LDA + 16 * J + r] = acc[i] * scale;
    }
    // ---- A, diagonal blocks: wave w takes block w, one (c, j) pair per lane
    //      and pass over the block's 256 entries (the upper ones are zero) ----
#pragma unroll
    for (int pp = 0; pp < 4; ++pp) {
      const int e = lane + 64 * pp;
      const int cl16 = e >> 4, jl16 = e & 15;
      const int c = 16 * w + cl16, j = 16 * w + jl16;
      float x = 0.f;
      if (jl16 <= cl16) {
        const f32x4* qc = reinterpret_cast<const f32x4*>(sQ + c * LDQ);
        const f32x4* bc = reinterpret_cast<const f32x4*>(sB + c * LDQ);
        const f32x4* kj = reinterpret_cast<const f32x4*>(sK + j * LDQ);
        const f32x4* bj = reinterpret_cast<const f32x4*>(sB + j * LDQ);
#pragma unroll 4
        for (int a4 = 0; a4 < K / 4; ++a4) {
          const f32x4 qv = qc[a4], bcv = bc[a4], kv = kj[a4], bjv = bj[a4];
#pragma unroll
          for (int u = 0; u < 4; ++u) x = fmaf(qv[u] * kv[u], exp2f(bcv[u] - bjv[u]), x);
        }
      }
      sA[c * LDA + j] = x * scale;
    }
    __syncthreads();

    // ---- Q (.) 2^B and K (.) 2^(B_last - B), in place ------------------------
    for (int i = tid; i < C * K; i += NT) {
      const int c = i / K, a = i % K;
      const float b = sB[c * LDQ + a];
      sQ[c * LDQ + a] *= exp2f(b);
      sK[c * LDQ + a] *= exp2f(sB[(C - 1) * LDQ + a] - b);
    }
    __syncthreads();

    // ---- output tiles (ct, cv), two per wave ---------------------------------
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int ot = w + 4 * t;
      const int ctile = ot >> 1, cv = ot & 1;
      f32x4 inter = {0.f, 0.f, 0.f, 0.f}, intra = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
      for (int ks = 0; ks < K / 4; ++ks)
        inter = mfma4(sQ[(16 * ctile + r) * LDQ + 4 * ks + g4], sH[(4 * ks + g4) * LDH + 16 * cv + r], inter);
      for (int js = 0; js < 4 * (ctile + 1); ++js)
        intra = mfma4(sA[(16 * ctile + r) * LDA + 4 * js + g4], sV[(4 * js + g4) * LDV + 16 * cv + r], intra);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int c = 16 * ctile + 4 * g4 + i;
        if (c < cl)
          o[((t0 + c) * H + hd) * (int64_t)V + vt * VT + 16 * cv + r] = out_cast<TOut>(intra[i] + scale * inter[i]);
      }
    }

    // ---- state: h <- diag(2^B_last) h + (K (.) 2^(B_last - B))^T V ---------------
#pragma unroll
    for (int s = 0; s < SPW; ++s) {
      const int st = w + 4 * s;
      if (NST % 4 != 0 && st >= NST) continue;
      const int kt = st >> 1, ctl = st & 1;
      f32x4 acc = hs[s];
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] *= exp2f(sB[(C - 1) * LDQ + 16 * kt + 4 * g4 + i]);
#pragma unroll 8
      for (int cs = 0; cs < C / 4; ++cs) {
        const int c = 4 * cs + g4;
        acc = mfma4(sK[c * LDQ + 16 * kt + r], sV[c * LDV + 16 * ctl + r], acc);
      }
      hs[s] = acc;
    }
    __syncthreads();   // every read of sQ, sK, sB, sV, sA and the old sH is done
    publish_state();
  }
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
  const dim3 grid((unsigned)unit_grid(p.seqs.num_seqs, p.Hkv, p.H / p.Hkv, p.V / VT));
  hipLaunchKernelGGL((gla_chunk_fwd_kernel<K, TIn, TOut>), grid, dim3(NT), 0, stream,
                     static_cast<const TIn*>(p.q), static_cast<const TIn*>(p.k),
                     static_cast<const TIn*>(p.v), p.gk, p.h0, static_cast<TOut*>(p.o), p.ht, p.scale,
                     p.H, p.Hkv, p.V, p.sl, p.seqs);
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
