// Steps (2) and (3) of the chunked Simple GLA forward for float32 q/k/v
// (page "flash-linear-attention 中的 Simple GLA", section 一 chunk view and
// section 三 state/output passes), evaluated entirely in fp32 on the vector
// ALUs so that float32 inputs keep float32 accuracy end to end (no bf16
// rounding anywhere on this path).  On MI355X the fp32 vector and fp32 matrix
// peaks are the same, so MFMA would not buy throughput here.
//
// Same per-chunk algebra as the bf16 kernel, with b the chunk-local
// cumulative log2 gate (formed in the chunk prologue by a wave scan):
//   A = (Q K^T) (.) M,   M[c][j] = 2^(b_c - b_j) (j <= c), 0 otherwise
//   O = scale * (A V + diag(2^b) Q h)
//   h <- 2^b_last h + K^T (diag(2^(b_last - b)) V)
// One 256-thread workgroup per (sequence, head, 32-wide V tile); the state
// tile lives in LDS for the whole sequence.
#include <hip/hip_runtime.h>

#include "gate_scan.h"
#include "sgla_internal.h"

namespace sgla {
namespace {

constexpr int C = kChunk;
constexpr int VT = 32;
constexpr int NTHREADS = 256;
constexpr float kRcpLn2f = 1.44269504088896341f;

template <int K, typename TOut>
__global__ void __launch_bounds__(NTHREADS)
chunk_fwd_f32_kernel(const float* __restrict__ q, const float* __restrict__ k,
                     const float* __restrict__ v, const float* __restrict__ g,
                     const float* __restrict__ g_gamma, const float* __restrict__ h0,
                     TOut* __restrict__ o, float* __restrict__ ht, float scale, int32_t H,
                     int32_t V, SeqLayout seqs) {
  constexpr int LDQ = K + 1;
  __shared__ float sQ[C][LDQ];
  __shared__ float sK[C][LDQ];
  __shared__ float sV[C][VT + 1];
  __shared__ float sA[C][C + 1];
  __shared__ float sH[K][VT + 1];
  __shared__ float sG[C], sEb[C], sDk[C];

  const int nvt = V / VT;
  const int num_units = seqs.num_seqs * H;
  const int xcd = blockIdx.x % kXcds;
  const int slot = blockIdx.x / kXcds;
  const int unit = (slot / nvt) * kXcds + xcd;
  const int vt = slot % nvt;
  if (unit >= num_units) return;
  const int rank = unit / H;
  const int hd = unit - rank * H;
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
  const float gam2 = g_gamma != nullptr ? g_gamma[hd] * kRcpLn2f : 0.f;
  const int64_t su = ((int64_t)seq * H + hd) * K * V;

  for (int i = tid; i < K * VT; i += NTHREADS) {
    const int kk = i / VT, vv = i % VT;
    sH[kk][vv] = h0 != nullptr ? h0[su + (int64_t)kk * V + vt * VT + vv] : 0.f;
  }

  const int nchunks = (len + C - 1) / C;
  for (int m = 0; m < nchunks; ++m) {
    const int64_t t0 = bos + (int64_t)m * C;
    const int cl = min(C, len - m * C);
    for (int i = tid; i < C * K; i += NTHREADS) {
      const int c = i / K, kk = i % K;
      const bool ok = c < cl;
      const int64_t off = ((t0 + c) * H + hd) * (int64_t)K + kk;
      sQ[c][kk] = ok ? q[off] : 0.f;
      sK[c][kk] = ok ? k[off] : 0.f;
    }
    for (int i = tid; i < C * VT; i += NTHREADS) {
      const int c = i / VT, vv = i % VT;
      sV[c][vv] = c < cl ? v[((t0 + c) * H + hd) * (int64_t)V + vt * VT + vv] : 0.f;
    }
    if (tid < C) {
      // step (1): chunk-local cumulative log2 gate (padding rows add 0)
      if (g != nullptr) sG[tid] = wave_cumsum_log2(tid < cl ? g[(t0 + tid) * H + hd] : 0.f);
      else sG[tid] = (float)min(tid + 1, cl) * gam2;
    }
    __syncthreads();
    const float blast = sG[C - 1];
    if (tid < C) {
      sEb[tid] = exp2f(sG[tid]);
      sDk[tid] = exp2f(blast - sG[tid]);
    }
    // A[c][j], j interleaved over the 4 threads of a row
    {
      const int c = tid >> 2;
      for (int j = tid & 3; j < C; j += 4) {
        float a = 0.f;
        if (j <= c) {
          float dot = 0.f;
          for (int kk = 0; kk < K; ++kk) dot = fmaf(sQ[c][kk], sK[j][kk], dot);
          a = dot * exp2f(sG[c] - sG[j]);
        }
        sA[c][j] = a;
      }
    }
    __syncthreads();
    // O[c][v]
    {
      const int c = tid >> 2;
      for (int vv = tid & 3; vv < VT; vv += 4) {
        float inter = 0.f;
        for (int kk = 0; kk < K; ++kk) inter = fmaf(sQ[c][kk], sH[kk][vv], inter);
        float intra = 0.f;
        for (int j = 0; j <= c; ++j) intra = fmaf(sA[c][j], sV[j][vv], intra);
        if (c < cl)
          o[((t0 + c) * H + hd) * (int64_t)V + vt * VT + vv] =
              (TOut)(scale * (intra + sEb[c] * inter));
      }
    }
    __syncthreads();
    // h[k][v] <- 2^b_last h + sum_c K[c][k] 2^(b_last - b_c) V[c][v]
    {
      const float dall = exp2f(blast);
      const int vv = tid & 31;
      for (int kk = tid >> 5; kk < K; kk += NTHREADS / 32) {
        float acc = 0.f;
        for (int c = 0; c < C; ++c) acc = fmaf(sK[c][kk] * sDk[c], sV[c][vv], acc);
        sH[kk][vv] = fmaf(dall, sH[kk][vv], acc);
      }
    }
    __syncthreads();
  }
  if (ht != nullptr) {
    __syncthreads();
    for (int i = tid; i < K * VT; i += NTHREADS) {
      const int kk = i / VT, vv = i % VT;
      ht[su + (int64_t)kk * V + vt * VT + vv] = sH[kk][vv];
    }
  }
}

template <int K, typename TOut>
hipError_t launch_k(const ChunkFwdParams& p, hipStream_t stream) {
  const int num_units = p.seqs.num_seqs * p.H;
  if (num_units == 0) return hipSuccess;
  const int nvt = p.V / VT;
  const int groups = (num_units + kXcds - 1) / kXcds;
  const dim3 grid((unsigned)(groups * kXcds * nvt));
  hipLaunchKernelGGL((chunk_fwd_f32_kernel<K, TOut>), grid, dim3(NTHREADS), 0, stream,
                     static_cast<const float*>(p.q), static_cast<const float*>(p.k),
                     static_cast<const float*>(p.v), p.g, p.g_gamma, p.h0,
                     static_cast<TOut*>(p.o), p.ht, p.scale, p.H, p.V, p.seqs);
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
