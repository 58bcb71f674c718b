// Steps (1)-(3) of the chunked Simple GLA forward for float32 q/k/v (page
// "flash-linear-attention 中的 Simple GLA", section 一 chunk view and section
// 三 state/output passes), in fp32 end to end: every product runs on the fp32
// matrix cores (v_mfma_f32_16x16x4_f32: fp32 operands, fp32 accumulation), so
// float32 inputs keep float32 accuracy (no bf16 rounding anywhere on this
// path).
//
// Same per-chunk algebra as the bf16 kernels, with b the chunk-local
// cumulative log2 gate (formed in the chunk prologue by a wave scan):
//   A = (Q K^T) (.) M,   M[c][j] = 2^(b_c - b_j) (j <= c), 0 otherwise
//   O = scale * (A V + diag(2^b) Q h)
//   h <- 2^b_last h + K^T (diag(2^(b_last - b)) V)
// One 256-thread workgroup (4 waves) per (sequence, head, 32-wide V tile).
// The K x 32 state lives in MFMA accumulators of the wave that owns its
// 16 x 16 tiles, with a copy in LDS that all waves read as the q.h operand.
// Per chunk: stage Q, K, V and the gates in LDS (from registers the previous
// chunk loaded them into); the waves split the ten causal 16 x 16 tiles of A,
// then the eight 16 x 16 output tiles and the state tiles.
//
// v_mfma_f32_16x16x4_f32 operands, per lane l with g = l / 16, r = l % 16:
//   A operand A[m = r][k = g], B operand B[k = g][n = r],
//   result acc[i] = D[m = 4 g + i][n = r].
#include <hip/hip_runtime.h>

#include "gate_scan.h"
#include "sgla_internal.h"
#include "unit_map.h"

namespace sgla {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int C = kChunk;
constexpr int VT = 32;
constexpr int NTHREADS = 256;
constexpr float kRcpLn2f = 1.44269504088896341f;
constexpr int LDV = VT + 4;       // V tile row stride (floats)
constexpr int LDA = C + 4;        // A row stride
constexpr int LDH = VT + 4;       // state row stride

__device__ __forceinline__ f32x4 mfma4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Causal 16 x 16 tiles of A, packed 4 bits per tile (c | j << 2), listed so
// that wave w takes tiles w, w + 4, w + 8 (at most three).
constexpr uint64_t kTiles = 0xFB73A62510ull;   // (0,0) (1,0) (1,1) (2,0) (2,1) (2,2) (3,0) (3,1) (3,2) (3,3)

template <int K, typename TOut>
__global__ void __launch_bounds__(NTHREADS)
chunk_fwd_f32_kernel(const float* __restrict__ q, const float* __restrict__ k,
                     const float* __restrict__ v, const float* __restrict__ g,
                     const float* __restrict__ g_gamma, const float* __restrict__ h0,
                     TOut* __restrict__ o, float* __restrict__ ht, float scale, int32_t H,
                     int32_t Hkv, int32_t V, StateLayout sl, SeqLayout seqs) {
  constexpr int LDQ = K + 4;          // Q / K row stride (floats)
  constexpr int NKT = K / 16;         // 16-row state tiles
  constexpr int NST = NKT * 2;        // state tiles (x 2 column tiles)
  constexpr int SPW = (NST + 3) / 4;  // state tiles per wave
  __shared__ float sQ[C * LDQ];
  __shared__ float sK[C * LDQ];
  __shared__ float sV[C * LDV];
  __shared__ float sA[C * LDA];
  __shared__ float sH[K * LDH];
  __shared__ float sG[C], sGl[C], sEb[C], sDk[C];   // sG + sGl: the running log2 gate

  const UnitMap um = map_unit(blockIdx.x, V / VT, Hkv, H / Hkv, seqs.num_seqs);
  if (!um.valid) return;
  const int rank = um.rank, hd = um.hd, hk = um.hk, vt = um.vt;
  int64_t bos;
  int32_t len, seq;
  if (seqs.seq_table != nullptr) {
    const SeqEntry e = seqs.seq_table[rank];
    bos = e.bos;
    len = e.len;
    seq = e.seq;
  } else {
    bos = (int64_t)rank * seqs.T;
    len = seqs.T;
    seq = rank;
  }
  const int tid = threadIdx.x;
  // wave index as a scalar, so per-wave tile choices are scalar branches
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int g4 = lane >> 4;
  const int r = lane & 15;
  const float gam2 = g_gamma != nullptr ? g_gamma[hd] * kRcpLn2f : 0.f;
  const int64_t su = ((int64_t)seq * H + hd) * K * V;
  // state element (row, column c of this tile)
  auto sidx = [&](int row, int c) { return su + (int64_t)row * sl.rs + (int64_t)(vt * VT + c) * sl.cs; };

  // state tiles of this wave: st = w + 4 s, rows [16 (st >> 1), +16),
  // columns [16 (st & 1), +16); acc element i = h[16 kt + 4 g + i][16 ct + r]
  f32x4 hs[SPW];
#pragma unroll
  for (int s = 0; s < SPW; ++s) {
    const int st = w + 4 * s;
    hs[s] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (st < NST && h0 != nullptr) {
      const int kt = st >> 1, ctl = st & 1;
#pragma unroll
      for (int i = 0; i < 4; ++i) hs[s][i] = h0[sidx(16 * kt + 4 * g4 + i, 16 * ctl + r)];
    }
  }
  auto publish_state = [&]() {
#pragma unroll
    for (int s = 0; s < SPW; ++s) {
      const int st = w + 4 * s;
      if (st < NST) {
        const int kt = st >> 1, ctl = st & 1;
#pragma unroll
        for (int i = 0; i < 4; ++i) sH[(16 * kt + 4 * g4 + i) * LDH + 16 * ctl + r] = hs[s][i];
      }
    }
  };
  publish_state();

  const int nchunks = (len + C - 1) / C;
  // ---- chunk staging registers: every thread's share of the Q, K and V
  //      rows and (first wave) its token's log gate; rows past the chunk's
  //      end read as zeros
  constexpr int NQ4 = C * (K / 4) / NTHREADS;   // float4 pieces of Q (and K) per thread
  constexpr int NV4 = C * (VT / 4) / NTHREADS;  // float4 pieces of the V tile per thread
  static_assert(NQ4 * NTHREADS == C * (K / 4) && NV4 * NTHREADS == C * (VT / 4), "staging split");
  f32x4 pq[NQ4], pk[NQ4], pv[NV4];
  float pg = 0.f;
  auto load_chunk = [&](int m) {
    const int64_t t0 = bos + (int64_t)m * C;
    const int cl = m < nchunks ? min(C, len - m * C) : 0;
#pragma unroll
    for (int u = 0; u < NQ4; ++u) {
      const int i = tid + NTHREADS * u;
      const int c = i / (K / 4), k4 = i % (K / 4);
      pq[u] = f32x4{0.f, 0.f, 0.f, 0.f};
      pk[u] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (c < cl) {
        pq[u] = *reinterpret_cast<const f32x4*>(q + ((t0 + c) * H + hd) * (int64_t)K + 4 * k4);
        pk[u] = *reinterpret_cast<const f32x4*>(k + ((t0 + c) * Hkv + hk) * (int64_t)K + 4 * k4);
      }
    }
#pragma unroll
    for (int u = 0; u < NV4; ++u) {
      const int i = tid + NTHREADS * u;
      const int c = i / (VT / 4), v4 = i % (VT / 4);
      pv[u] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (c < cl) pv[u] = *reinterpret_cast<const f32x4*>(v + ((t0 + c) * Hkv + hk) * (int64_t)V + vt * VT + 4 * v4);
    }
    pg = (g != nullptr && tid < cl) ? g[(t0 + tid) * H + hd] : 0.f;
  };
  load_chunk(0);
  for (int m = 0; m < nchunks; ++m) {
    const int64_t t0 = bos + (int64_t)m * C;
    const int cl = min(C, len - m * C);
    // ---- stage the chunk -------------------------------------------------
#pragma unroll
    for (int u = 0; u < NQ4; ++u) {
      const int i = tid + NTHREADS * u;
      const int c = i / (K / 4), k4 = i % (K / 4);
      *reinterpret_cast<f32x4*>(sQ + c * LDQ + 4 * k4) = pq[u];
      *reinterpret_cast<f32x4*>(sK + c * LDQ + 4 * k4) = pk[u];
    }
#pragma unroll
    for (int u = 0; u < NV4; ++u) {
      const int i = tid + NTHREADS * u;
      const int c = i / (VT / 4), v4 = i % (VT / 4);
      *reinterpret_cast<f32x4*>(sV + c * LDV + 4 * v4) = pv[u];
    }
    if (w == 0) {
      // step (1): chunk-local cumulative log2 gate (padding rows add 0)
      float b, bl = 0.f;
      if (g != nullptr) b = wave_cumsum_log2_split(pg, bl);
      else b = (float)min(tid + 1, cl) * gam2;
      const float blast = __shfl(b, C - 1, 64), bllast = __shfl(bl, C - 1, 64);
      sG[tid] = b;
      sGl[tid] = bl;
      sEb[tid] = exp2f(b) * scale;
      sDk[tid] = exp2f((blast - b) + (bllast - bl));
    }
    __syncthreads();
    load_chunk(m + 1);   // in flight while this chunk computes
    __syncthreads();

    // ---- A tiles: (Q K^T) (.) M, scale folded in --------------------------
#pragma unroll
    for (int t = 0; t < 3; ++t) {
      const int ti = w + 4 * t;
      if (ti >= 10) continue;
      const int ctile = (int)(kTiles >> (4 * ti)) & 3, jtile = (int)(kTiles >> (4 * ti + 2)) & 3;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
      for (int ks = 0; ks < K / 4; ++ks)
        acc = mfma4(sQ[(16 * ctile + r) * LDQ + 4 * ks + g4], sK[(16 * jtile + r) * LDQ + 4 * ks + g4], acc);
      const int j = 16 * jtile + r;
      const float bj = sG[j], blj = sGl[j];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int c = 16 * ctile + 4 * g4 + i;
        sA[c * LDA + j] = j <= c ? acc[i] * exp2f((sG[c] - bj) + (sGl[c] - blj)) * scale : 0.f;
      }
    }
    // zero the upper-triangle tiles (0,1) (0,2) (0,3) (1,2) (1,3) (2,3)
    for (int i = tid; i < 6 * 256; i += NTHREADS) {
      const int tt = i >> 8, e = i & 255;
      const int ctile = tt < 3 ? 0 : (tt < 5 ? 1 : 2);
      const int jtile = tt < 3 ? tt + 1 : (tt < 5 ? tt - 1 : 3);
      sA[(16 * ctile + (e >> 4)) * LDA + 16 * jtile + (e & 15)] = 0.f;
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
          o[((t0 + c) * H + hd) * (int64_t)V + vt * VT + 16 * cv + r] = (TOut)(intra[i] + sEb[c] * inter[i]);
      }
    }

    // ---- state tiles: h <- 2^b_last h + K^T diag(2^(b_last - b)) V ------------
    const float dall = exp2f(sG[C - 1]);
#pragma unroll
    for (int s = 0; s < SPW; ++s) {
      const int st = w + 4 * s;
      if (st >= NST) continue;
      const int kt = st >> 1, ctl = st & 1;
      f32x4 acc = hs[s] * dall;
#pragma unroll 8
      for (int cs = 0; cs < C / 4; ++cs) {
        const int c = 4 * cs + g4;
        acc = mfma4(sK[c * LDQ + 16 * kt + r] * sDk[c], sV[c * LDV + 16 * ctl + r], acc);
      }
      hs[s] = acc;
    }
    __syncthreads();   // every read of sQ, sK, sV, sA and the old sH is done
    publish_state();
    // (the next chunk's staging barrier also orders these writes)
  }
  if (ht != nullptr) {
#pragma unroll
    for (int s = 0; s < SPW; ++s) {
      const int st = w + 4 * s;
      if (st < NST) {
        const int kt = st >> 1, ctl = st & 1;
#pragma unroll
        for (int i = 0; i < 4; ++i) ht[sidx(16 * kt + 4 * g4 + i, 16 * ctl + r)] = hs[s][i];
      }
    }
  }
}

template <int K, typename TOut>
hipError_t launch_k(const ChunkFwdParams& p, hipStream_t stream) {
  if (p.seqs.num_seqs == 0) return hipSuccess;
  const dim3 grid((unsigned)unit_grid(p.seqs.num_seqs, p.Hkv, p.H / p.Hkv, p.V / VT));
  hipLaunchKernelGGL((chunk_fwd_f32_kernel<K, TOut>), grid, dim3(NTHREADS), 0, stream,
                     static_cast<const float*>(p.q), static_cast<const float*>(p.k),
                     static_cast<const float*>(p.v), p.g, p.g_gamma, p.h0,
                     static_cast<TOut*>(p.o), p.ht, p.scale, p.H, p.Hkv, p.V, p.sl, p.seqs);
  return hipGetLastError();
}

template <typename TOut>
hipError_t launch_out(const ChunkFwdParams& p, hipStream_t stream) {
  switch (p.K) {
    case 16: return launch_k<16, TOut>(p, stream);
    case 32: return launch_k<32, TOut>(p, stream);
    case 64: return launch_k<64, TOut>(p, stream);
    case 128: return launch_k<128, TOut>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_chunk_fwd_f32(const ChunkFwdParams& p, hipStream_t stream) {
  return p.o_bf16 ? launch_out<__bf16>(p, stream) : launch_out<float>(p, stream);
}

}  // namespace sgla
