// Chunked Simple GLA forward at chunk sizes 16 and 32 (page "flash-linear-
// attention 中的 Simple GLA", section 二: chunk_size is any power of two;
// section 五 runs the chunk kernels at 16, 32 and 64).  The chunk size is a
// tiling choice of the chunk form -- the result equals the recurrence's at
// any size, only the rounding differs -- so this kernel serves the sizes
// below 64 for every supported dtype and key width with one generic design;
// the tuned kernels keep 64.
//
// Per chunk of C tokens of one (sequence, head), with b the chunk-local
// cumulative log2 gate restarting at the chunk (step 1, a wave scan in the
// chunk prologue, kept as hi + lo so decay exponents stay exact after a very
// negative gate), b_last its value at the chunk's last token and h the K x V
// state entering the chunk (section 一 and 三):
//   A      = (Q K^T) (.) M,  M[c][j] = 2^(b_c - b_j) for j <= c, else 0
//   O      = scale * ( A V + diag(2^b) Q h )
//   h_next = 2^b_last h + K^T diag(2^(b_last - b)) V
//
// Everything runs on the fp32 matrix cores (v_mfma_f32_16x16x4_f32): bf16
// inputs are exact in fp32, so no operand is rounded and the result has
// float32 accuracy for either input dtype.  One 256-thread workgroup (4
// waves) per (sequence, head, 16-wide V tile); the K x 16 state sits in MFMA
// accumulators of the waves that own its 16 x 16 tiles, with a copy in LDS
// that the output tiles read as the q.h operand.  Q and K are staged in LDS
// in the input dtype (bf16 staging halves the footprint for K up to 512),
// V, A and the state copy in fp32; the next chunk's rows load into
// registers while the current chunk computes.
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
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int VT = 16;            // state / output columns per workgroup
constexpr int NTHREADS = 256;
constexpr float kRcpLn2f = 1.44269504088896341f;
constexpr int LDV = VT + 4;       // V tile row stride (floats)
constexpr int LDH = VT + 4;       // state copy row stride (floats)

__device__ __forceinline__ f32x4 mfma4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(__bf16 x) { return (float)x; }

// One 16-byte piece of a row: 8 bf16 or 4 float32 elements.
template <typename Tin> struct Piece { static constexpr int N = 16 / (int)sizeof(Tin); };

template <typename Tin, int C, int K, typename TOut>
__global__ void __launch_bounds__(NTHREADS)
chunk_fwd_small_kernel(const Tin* __restrict__ q, const Tin* __restrict__ k, const Tin* __restrict__ v,
                       const float* __restrict__ g, const float* __restrict__ g_gamma,
                       const float* __restrict__ h0, TOut* __restrict__ o, float* __restrict__ ht,
                       float scale, int32_t H, int32_t Hkv, int32_t V, StateLayout sl, SeqLayout seqs) {
  static_assert(C == 16 || C == 32, "chunk sizes below 64");
  constexpr int EP = Piece<Tin>::N;       // elements per 16-byte piece
  constexpr int LDQ = K + EP;             // Q / K row stride (elements)
  constexpr int LDA = C + 4;              // A row stride (floats)
  constexpr int CT = C / 16;              // 16-row token tiles
  constexpr int NAT = CT * (CT + 1) / 2;  // causal A tiles
  constexpr int NST = K / 16;             // 16-row state tiles
  constexpr int SPW = (NST + 3) / 4;      // state tiles per wave
  constexpr int QP = C * K / EP;          // 16-byte pieces of Q (and of K) per chunk
  constexpr int NQP = (QP + NTHREADS - 1) / NTHREADS;
  constexpr int VP = C * VT / EP;         // pieces of the V tile
  static_assert(VP <= NTHREADS, "one V piece per thread at most");
  __shared__ __attribute__((aligned(16))) Tin sQ[C * LDQ];
  __shared__ __attribute__((aligned(16))) Tin sK[C * LDQ];
  __shared__ float sV[C * LDV];
  __shared__ float sA[C * LDA];
  __shared__ float sH[K * LDH];
  __shared__ float sG[64], sGl[64], sEb[64], sDk[64];   // sG + sGl: the running log2 gate

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
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int g4 = lane >> 4;
  const int r = lane & 15;
  const float gam2 = g_gamma != nullptr ? g_gamma[hd] * kRcpLn2f : 0.f;
  const int64_t su = ((int64_t)seq * H + hd) * K * V;
  auto sidx = [&](int row, int c) { return su + (int64_t)row * sl.rs + (int64_t)(vt * VT + c) * sl.cs; };

  // state tiles of this wave: st = w + 4 s covers rows [16 st, 16 st + 16);
  // acc element i = h[16 st + 4 g + i][r]
  f32x4 hs[SPW];
#pragma unroll
  for (int s = 0; s < SPW; ++s) {
    const int st = w + 4 * s;
    hs[s] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (st < NST && h0 != nullptr) {
#pragma unroll
      for (int i = 0; i < 4; ++i) hs[s][i] = h0[sidx(16 * st + 4 * g4 + i, r)];
    }
  }
  auto publish_state = [&]() {
#pragma unroll
    for (int s = 0; s < SPW; ++s) {
      const int st = w + 4 * s;
      if (st < NST) {
#pragma unroll
        for (int i = 0; i < 4; ++i) sH[(16 * st + 4 * g4 + i) * LDH + r] = hs[s][i];
      }
    }
  };
  publish_state();

  const int nchunks = (len + C - 1) / C;
  // ---- chunk staging registers (rows past the chunk's end read as zeros)
  u32x4 pq[NQP], pk[NQP], pv;
  float pg = 0.f;
  auto load_chunk = [&](int m) {
    const int64_t t0 = bos + (int64_t)m * C;
    const int cl = m < nchunks ? min(C, len - m * C) : 0;
#pragma unroll
    for (int u = 0; u < NQP; ++u) {
      const int i = tid + NTHREADS * u;
      const int c = i / (K / EP), e = i % (K / EP);
      pq[u] = u32x4{0u, 0u, 0u, 0u};
      pk[u] = u32x4{0u, 0u, 0u, 0u};
      if (i < QP && c < cl) {
        pq[u] = *reinterpret_cast<const u32x4*>(q + ((t0 + c) * H + hd) * (int64_t)K + EP * e);
        pk[u] = *reinterpret_cast<const u32x4*>(k + ((t0 + c) * Hkv + hk) * (int64_t)K + EP * e);
      }
    }
    {
      const int c = tid / (VT / EP), e = tid % (VT / EP);
      pv = u32x4{0u, 0u, 0u, 0u};
      if (tid < VP && c < cl)
        pv = *reinterpret_cast<const u32x4*>(v + ((t0 + c) * Hkv + hk) * (int64_t)V + vt * VT + EP * e);
    }
    pg = (g != nullptr && tid < cl) ? g[(t0 + tid) * H + hd] : 0.f;
  };
  load_chunk(0);
  for (int m = 0; m < nchunks; ++m) {
    const int64_t t0 = bos + (int64_t)m * C;
    const int cl = min(C, len - m * C);
    // ---- stage the chunk -------------------------------------------------
#pragma unroll
    for (int u = 0; u < NQP; ++u) {
      const int i = tid + NTHREADS * u;
      const int c = i / (K / EP), e = i % (K / EP);
      if (i < QP) {
        *reinterpret_cast<u32x4*>(sQ + c * LDQ + EP * e) = pq[u];
        *reinterpret_cast<u32x4*>(sK + c * LDQ + EP * e) = pk[u];
      }
    }
    if (tid < VP) {
      const int c = tid / (VT / EP), e = tid % (VT / EP);
      const Tin* x = reinterpret_cast<const Tin*>(&pv);
#pragma unroll
      for (int j = 0; j < EP; ++j) sV[c * LDV + EP * e + j] = to_f32(x[j]);
    }
    if (w == 0) {
      // step (1): cumulative log2 gate over the chunk's tokens (lanes past
      // the chunk's end add 0, so they carry the last token's value)
      float b, bl = 0.f;
      if (g != nullptr) b = wave_cumsum_log2_split(pg, bl);
      else b = (float)min(lane + 1, cl) * gam2;
      const float blast = __shfl(b, C - 1, 64), bllast = __shfl(bl, C - 1, 64);
      sG[lane] = b;
      sGl[lane] = bl;
      sEb[lane] = exp2f(b) * scale;
      sDk[lane] = exp2f((blast - b) + (bllast - bl));
    }
    __syncthreads();
    load_chunk(m + 1);   // in flight while this chunk computes

    // ---- A tiles: (Q K^T) (.) M, scale folded in --------------------------
    if (w < NAT) {
      // causal tile w: (ct, jt) = (0,0) | (1,0) (1,1)
      const int ct = w == 0 ? 0 : 1, jt = w == 2 ? 1 : 0;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
      for (int ks = 0; ks < K / 4; ++ks)
        acc = mfma4(to_f32(sQ[(16 * ct + r) * LDQ + 4 * ks + g4]), to_f32(sK[(16 * jt + r) * LDQ + 4 * ks + g4]),
                    acc);
      const int j = 16 * jt + r;
      const float bj = sG[j], blj = sGl[j];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int c = 16 * ct + 4 * g4 + i;
        sA[c * LDA + j] = j <= c ? acc[i] * exp2f((sG[c] - bj) + (sGl[c] - blj)) * scale : 0.f;
      }
    } else if (CT == 2 && w == 3) {
      // the tile above the diagonal (rows 0-15, columns 16-31) is zero
      for (int e = lane; e < 256; e += 64) sA[(e >> 4) * LDA + 16 + (e & 15)] = 0.f;
    }
    __syncthreads();

    // ---- output tiles: 16 token rows each ----------------------------------
    if (w < CT) {
      const int ct = w;
      f32x4 inter = {0.f, 0.f, 0.f, 0.f}, intra = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
      for (int ks = 0; ks < K / 4; ++ks)
        inter = mfma4(to_f32(sQ[(16 * ct + r) * LDQ + 4 * ks + g4]), sH[(4 * ks + g4) * LDH + r], inter);
#pragma unroll
      for (int js = 0; js < 4 * (ct + 1); ++js)
        intra = mfma4(sA[(16 * ct + r) * LDA + 4 * js + g4], sV[(4 * js + g4) * LDV + r], intra);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int c = 16 * ct + 4 * g4 + i;
        if (c < cl) o[((t0 + c) * H + hd) * (int64_t)V + vt * VT + r] = (TOut)(intra[i] + sEb[c] * inter[i]);
      }
    }

    // ---- state tiles: h <- 2^b_last h + K^T diag(2^(b_last - b)) V ------------
    const float dall = exp2f(sG[C - 1] + sGl[C - 1]);
#pragma unroll
    for (int s = 0; s < SPW; ++s) {
      const int st = w + 4 * s;
      if (st >= NST) continue;
      f32x4 acc = hs[s] * dall;
#pragma unroll
      for (int cs = 0; cs < C / 4; ++cs) {
        const int c = 4 * cs + g4;
        acc = mfma4(to_f32(sK[c * LDQ + 16 * st + r]) * sDk[c], sV[c * LDV + r], acc);
      }
      hs[s] = acc;
    }
    __syncthreads();   // every read of sQ, sK, sV, sA and the old state copy is done
    publish_state();   // ordered before the next reads by the next staging barrier
  }
  if (ht != nullptr) {
#pragma unroll
    for (int s = 0; s < SPW; ++s) {
      const int st = w + 4 * s;
      if (st < NST) {
#pragma unroll
        for (int i = 0; i < 4; ++i) ht[sidx(16 * st + 4 * g4 + i, r)] = hs[s][i];
      }
    }
  }
}

template <typename Tin, int C, int K, typename TOut>
hipError_t launch_ck(const ChunkFwdParams& p, hipStream_t stream) {
  const dim3 grid((unsigned)unit_grid(p.seqs.num_seqs, p.Hkv, p.H / p.Hkv, p.V / VT));
  hipLaunchKernelGGL((chunk_fwd_small_kernel<Tin, C, K, TOut>), grid, dim3(NTHREADS), 0, stream,
                     static_cast<const Tin*>(p.q), static_cast<const Tin*>(p.k), static_cast<const Tin*>(p.v),
                     p.g, p.g_gamma, p.h0, static_cast<TOut*>(p.o), p.ht, p.scale, p.H, p.Hkv, p.V, p.sl,
                     p.seqs);
  return hipGetLastError();
}

// Key widths: 16-128 for float32 inputs, 64-512 for bf16 inputs (the sets
// the tuned 64-token kernels support).
template <typename Tin, int C, typename TOut>
hipError_t launch_c(const ChunkFwdParams& p, hipStream_t stream) {
  if constexpr (sizeof(Tin) == 4) {
    switch (p.K) {
      case 16: return launch_ck<Tin, C, 16, TOut>(p, stream);
      case 32: return launch_ck<Tin, C, 32, TOut>(p, stream);
      case 64: return launch_ck<Tin, C, 64, TOut>(p, stream);
      case 128: return launch_ck<Tin, C, 128, TOut>(p, stream);
      default: return hipErrorInvalidValue;
    }
  } else {
    switch (p.K) {
      case 64: return launch_ck<Tin, C, 64, TOut>(p, stream);
      case 128: return launch_ck<Tin, C, 128, TOut>(p, stream);
      case 256: return launch_ck<Tin, C, 256, TOut>(p, stream);
      case 512: return launch_ck<Tin, C, 512, TOut>(p, stream);
      default: return hipErrorInvalidValue;
    }
  }
}

template <typename Tin, typename TOut>
hipError_t launch_t(const ChunkFwdParams& p, int chunk, hipStream_t stream) {
  return chunk == 16 ? launch_c<Tin, 16, TOut>(p, stream) : launch_c<Tin, 32, TOut>(p, stream);
}

}  // namespace

hipError_t launch_chunk_fwd_small(const ChunkFwdParams& p, int chunk, bool qkv_bf16, hipStream_t stream) {
  if (p.seqs.num_seqs == 0) return hipSuccess;
  if (chunk != 16 && chunk != 32) return hipErrorInvalidValue;
  if (qkv_bf16)
    return p.o_bf16 ? launch_t<__bf16, __bf16>(p, chunk, stream) : launch_t<__bf16, float>(p, chunk, stream);
  return p.o_bf16 ? launch_t<float, __bf16>(p, chunk, stream) : launch_t<float, float>(p, chunk, stream);
}

}  // namespace sgla
