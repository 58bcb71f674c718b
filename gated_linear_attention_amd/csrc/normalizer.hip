// The running normalizer of normalized linear attention (page "relinear": it
// divides by q . z, recovered in one call by appending a column of ones to v
// -- the "augmented value" -- whose state column is z and whose output is the
// normalizer):
//
//     z_t = exp(g_t) z_{t-1} + k_t          (K-vector per sequence and head)
//     den_t = scale * q_t . z_t
//
// computed here without widening V: the ones column on its own.  It is a
// stream over q and k with a K-float state, so it is bound by how fast q and
// k arrive, not by arithmetic.
//
// Chunked form, parallel over chunks (three launches, every one of them
// spread over all (chunk, head) or (sequence, head) units):
//   1. per (chunk, head): the chunk's own contribution to z at its last
//      token, u = sum_j 2^(b_last - b_j) k_j (b the chunk-local cumulative
//      log2 gate), and its total log2 decay b_last;
//   2. per (sequence, head): z entering each chunk, z_(n+1) = 2^(b_last,n) z_n
//      + u_n from z_0 = initial z, written over u_n; the last one is final z;
//   3. per (chunk, head): starting from the chunk's entering z, key i runs
//      its recurrence over the chunk's tokens (one thread per key, rows
//      staged in LDS as float32), leaving q_t[i] z_t[i] in LDS, and every
//      token's products are summed over the keys.
// Passes 1 and 3 read k, pass 3 reads q; the per-chunk z records (K floats
// per chunk and head) are the only extra traffic.
//
// Decode: one wave per (sequence, head); lanes own keys.
#include <hip/hip_runtime.h>

#include "gate_scan.h"
#include "sgla_internal.h"
#include "unit_map.h"

namespace sgla {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int C = kChunk;
constexpr int NT = 256;

template <typename T>
__device__ __forceinline__ float to_f32(T x);
template <>
__device__ __forceinline__ float to_f32<float>(float x) { return x; }
template <>
__device__ __forceinline__ float to_f32<__bf16>(__bf16 x) { return (float)x; }

// Token range of chunk `chunk` (dense: chunks of every row in order).
struct ChunkRange {
  int64_t t0;   // first token (packed index)
  int32_t len;  // 1..C
};

__device__ __forceinline__ ChunkRange chunk_range(const SeqLayout& seqs, int32_t chunk) {
  ChunkRange r;
  if (seqs.chunk_table != nullptr) {
    const ChunkEntry e = seqs.chunk_table[chunk];
    r.t0 = e.t0;
    r.len = e.len;
  } else {
    const int32_t ncs = (seqs.T + seqs.chunk - 1) / seqs.chunk;
    const int32_t row = chunk / ncs, m = chunk - row * ncs;
    r.t0 = (int64_t)row * seqs.T + (int64_t)m * seqs.chunk;
    r.len = min(seqs.chunk, seqs.T - m * seqs.chunk);
  }
  return r;
}

// Per-token log gate of chunk token `c` (0 past the chunk's end, so the
// cumulative gate there equals the last real token's).
__device__ __forceinline__ float token_gate(const float* g, const float* g_gamma, int64_t t0, int c,
                                            int len, int32_t H, int hd) {
  if (c >= len) return 0.f;
  if (g != nullptr) return g[(t0 + c) * H + hd];
  return g_gamma != nullptr ? g_gamma[hd] : 0.f;
}

template <typename TIn>
struct Pieces {
  static constexpr int EPL = 16 / sizeof(TIn);   // elements per 16-byte load
};

// Widens one 16-byte piece to float32.
template <typename TIn>
__device__ __forceinline__ void widen(const uint4& x, float (&f)[Pieces<TIn>::EPL]) {
  const uint32_t w[4] = {x.x, x.y, x.z, x.w};
  if constexpr (sizeof(TIn) == 2) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(w[i] << 16);
      f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(w[i]);
  }
}

// Pass 1: u[chunk, hd, :] = sum_j 2^(b_last - b_j) k_j, dlog[chunk, hd] = b_last.
template <int K, typename TIn>
__global__ void __launch_bounds__(NT)
norm_chunk_sum_kernel(const TIn* __restrict__ k, const float* __restrict__ g,
                      const float* __restrict__ g_gamma, float* __restrict__ u,
                      float* __restrict__ dlog, int32_t H, int32_t Hkv, SeqLayout seqs) {
  constexpr int EPL = Pieces<TIn>::EPL;
  constexpr int PR = K / EPL;                    // pieces per row
  constexpr int NP = (C * PR + NT - 1) / NT;     // pieces per thread
  constexpr int RG = NT / PR;                    // row groups (threads sharing a piece column)
  static_assert(K % EPL == 0 && NT % PR == 0, "K");
  __shared__ float sW[C];
  __shared__ float sPart[RG * K];

  const UnitMap um = map_unit(blockIdx.x, 1, Hkv, H / Hkv, seqs.num_chunks);
  if (!um.valid) return;
  const int32_t chunk = um.rank;
  const int hd = um.hd, hk = um.hk;
  const ChunkRange cr = chunk_range(seqs, chunk);
  const int tid = threadIdx.x;
  const TIn* kb = k + (cr.t0 * Hkv + hk) * K;
  const int64_t RSK = (int64_t)Hkv * K;

  uint4 kx[NP];
#pragma unroll
  for (int v = 0; v < NP; ++v) {
    const int p = tid + NT * v;
    const int c = p / PR;
    kx[v] = make_uint4(0u, 0u, 0u, 0u);
    if ((C * PR % NT == 0 || p < C * PR) && c < cr.len)
      kx[v] = *reinterpret_cast<const uint4*>(kb + c * RSK + (p % PR) * EPL);
  }
  if (tid < C) {
    const float lg = token_gate(g, g_gamma, cr.t0, tid, cr.len, H, hd);
    // chunk-local cumulative log2 gate (closed form for a per-head decay)
    // (per-token gates: carried as hi + lo, so 2^(b_last - b) stays exact to
    // fp32 after a very negative gate inside the chunk)
    float bl = 0.f;
    const float b = g != nullptr         ? wave_cumsum_log2_split(lg, bl)
                    : g_gamma != nullptr ? (float)min(tid + 1, cr.len) * (g_gamma[hd] * (float)kRcpLn2d)
                                         : 0.f;
    const float blast = __shfl(b, C - 1, 64), bllast = __shfl(bl, C - 1, 64);
    sW[tid] = exp2f((blast - b) + (bllast - bl));
    if (tid == C - 1) dlog[(int64_t)chunk * H + hd] = blast;
  }
  __syncthreads();
  float acc[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = 0.f;
#pragma unroll
  for (int v = 0; v < NP; ++v) {
    const int p = tid + NT * v;
    if (C * PR % NT == 0 || p < C * PR) {
      float f[EPL];
      widen<TIn>(kx[v], f);
      const float w = sW[p / PR];
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[e] = fmaf(w, f[e], acc[e]);
    }
  }
  // thread tid holds keys (tid % PR) * EPL + e of row group tid / PR
#pragma unroll
  for (int e = 0; e < EPL; ++e) sPart[(tid / PR) * K + (tid % PR) * EPL + e] = acc[e];
  __syncthreads();
  for (int key = tid; key < K; key += NT) {
    float s = 0.f;
#pragma unroll 8
    for (int rg = 0; rg < RG; ++rg) s += sPart[rg * K + key];
    u[((int64_t)chunk * H + hd) * K + key] = s;
  }
}

// Pass 2: per (sequence, head), z entering each chunk over u; final z.
// Thread `key` runs key's chain.
template <int K>
__global__ void __launch_bounds__(NT)
norm_scan_kernel(float* __restrict__ zrec, const float* __restrict__ dlog,
                 const float* __restrict__ z0, float* __restrict__ zt, int32_t H, SeqLayout seqs) {
  static_assert(K <= NT, "one key per thread");
  const int32_t unit = blockIdx.x;
  const int32_t rank = unit / H, hd = unit - rank * H;
  int32_t len, seq, cbase;
  if (seqs.seq_table != nullptr) {
    const SeqEntry e = seqs.seq_table[rank];
    len = e.len;
    seq = e.seq;
    cbase = e.chunk0;
  } else {
    len = seqs.T;
    seq = rank;
    cbase = rank * ((seqs.T + seqs.chunk - 1) / seqs.chunk);
  }
  const int nch = (len + seqs.chunk - 1) / seqs.chunk;
  const int key = threadIdx.x;
  const int lane = key & 63;
  const bool mine = key < K;
  float z = mine && z0 != nullptr ? z0[((int64_t)seq * H + hd) * K + key] : 0.f;
  // BATCH chunks per step: their records and decays are loaded together
  // (indices clamped to the last chunk, so every load is in range), then the
  // chain runs through them.  Every lane loads chunk m0 + lane's decay, so
  // lane j of each wave holds the factor of chunk m0 + j.
  constexpr int BATCH = 32;
  for (int m0 = 0; m0 < nch; m0 += BATCH) {
    const float dv = exp2f(dlog[(int64_t)(cbase + min(m0 + lane, nch - 1)) * H + hd]);
    if (mine) {
      float uu[BATCH];
#pragma unroll
      for (int j = 0; j < BATCH; ++j)
        uu[j] = zrec[((int64_t)(cbase + min(m0 + j, nch - 1)) * H + hd) * K + key];
#pragma unroll
      for (int j = 0; j < BATCH; ++j) {
        if (m0 + j < nch) {
          zrec[((int64_t)(cbase + m0 + j) * H + hd) * K + key] = z;
          z = fmaf(__builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, dv), j)), z, uu[j]);
        }
      }
    }
  }
  if (mine && zt != nullptr) zt[((int64_t)seq * H + hd) * K + key] = z;
}

// Pass 3: den over one chunk from the z entering it.  q stays in the
// registers it was loaded into; only k (then z) goes through LDS.
template <int K, typename TIn>
__global__ void __launch_bounds__(NT)
norm_chunk_out_kernel(const TIn* __restrict__ q, const TIn* __restrict__ k,
                      const float* __restrict__ g, const float* __restrict__ g_gamma,
                      const float* __restrict__ zrec, float* __restrict__ den, float scale,
                      int32_t H, int32_t Hkv, SeqLayout seqs) {
  constexpr int EPL = Pieces<TIn>::EPL;
  constexpr int PR = K / EPL;                    // 16-byte pieces per row (divides 64)
  constexpr int NP = (C * PR + NT - 1) / NT;     // pieces per thread per matrix
  constexpr int RG = NT / PR;                    // rows covered by one sweep of the threads
  constexpr int KPT = (K + NT - 1) / NT;         // keys per thread
  constexpr int LDK = K + 4;                     // LDS row stride (floats), 16-byte aligned rows
  static_assert(K % EPL == 0 && 64 % PR == 0, "K");
  __shared__ __attribute__((aligned(16))) float sZ[C * LDK];   // k rows, then z rows
  __shared__ float sGam[C];

  const UnitMap um = map_unit(blockIdx.x, 1, Hkv, H / Hkv, seqs.num_chunks);
  if (!um.valid) return;
  const int32_t chunk = um.rank;
  const int hd = um.hd, hk = um.hk;
  const ChunkRange cr = chunk_range(seqs, chunk);
  const int cl = cr.len;
  const int tid = threadIdx.x;
  const int64_t RSQ = (int64_t)H * K, RSK = (int64_t)Hkv * K;
  const TIn* qb = q + (cr.t0 * H + hd) * K;
  const TIn* kb = k + (cr.t0 * Hkv + hk) * K;
  const int e0 = (tid % PR) * EPL;               // this thread's keys [e0, e0 + EPL) of each of its rows

  uint4 qx[NP], kx[NP];
#pragma unroll
  for (int v = 0; v < NP; ++v) {
    const int c = tid / PR + RG * v;
    qx[v] = make_uint4(0u, 0u, 0u, 0u);
    kx[v] = make_uint4(0u, 0u, 0u, 0u);
    if (c < cl) {
      qx[v] = *reinterpret_cast<const uint4*>(qb + c * RSQ + e0);
      kx[v] = *reinterpret_cast<const uint4*>(kb + c * RSK + e0);
    }
  }
  float z[KPT];
#pragma unroll
  for (int kk = 0; kk < KPT; ++kk) {
    const int key = tid + NT * kk;
    z[kk] = key < K ? zrec[((int64_t)chunk * H + hd) * K + key] : 0.f;
  }
  if (tid < C) sGam[tid] = expf(token_gate(g, g_gamma, cr.t0, tid, cl, H, hd));
#pragma unroll
  for (int v = 0; v < NP; ++v) {
    const int c = tid / PR + RG * v;
    if (c < C) {
      float f[EPL];
      widen<TIn>(kx[v], f);
#pragma unroll
      for (int i = 0; i < EPL; i += 4)
        *reinterpret_cast<f32x4*>(sZ + c * LDK + e0 + i) = f32x4{f[i], f[i + 1], f[i + 2], f[i + 3]};
    }
  }
  __syncthreads();
  // recurrence of each key over the chunk; z_t replaces k_t (padding rows
  // add 0 with decay 1)
#pragma unroll
  for (int kk = 0; kk < KPT; ++kk) {
    const int key = tid + NT * kk;
    if (key < K) {
      float zz = z[kk];
#pragma unroll 8
      for (int c = 0; c < C; ++c) {
        zz = fmaf(sGam[c], zz, sZ[c * LDK + key]);
        sZ[c * LDK + key] = zz;
      }
    }
  }
  __syncthreads();
  // den_c = scale * q_c . z_c: each thread its EPL keys of its rows, then
  // a sum over the PR lanes holding the rest of the row
#pragma unroll
  for (int v = 0; v < NP; ++v) {
    const int c = tid / PR + RG * v;
    float s = 0.f;
    if (c < C) {
      float f[EPL];
      widen<TIn>(qx[v], f);
#pragma unroll
      for (int i = 0; i < EPL; i += 4) {
        const f32x4 zz = *reinterpret_cast<const f32x4*>(sZ + c * LDK + e0 + i);
        s = fmaf(f[i], zz[0], s);
        s = fmaf(f[i + 1], zz[1], s);
        s = fmaf(f[i + 2], zz[2], s);
        s = fmaf(f[i + 3], zz[3], s);
      }
    }
#pragma unroll
    for (int d = PR / 2; d >= 1; d >>= 1) s += __shfl_xor(s, d, 64);
    if (tid % PR == 0 && c < cl) den[(cr.t0 + c) * H + hd] = s * scale;
  }
}

// Decode: 4 (sequence, head) units per workgroup, one wave each, z in place.
template <typename TIn>
__global__ void __launch_bounds__(NT)
step_normalizer_kernel(const TIn* __restrict__ q, const TIn* __restrict__ k,
                       const float* __restrict__ g, const float* __restrict__ g_gamma,
                       float* __restrict__ z, float* __restrict__ den, float scale, int32_t units,
                       int32_t H, int32_t Hkv, int32_t K) {
  const int lane = threadIdx.x & 63;
  const int64_t unit = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (unit >= units) return;
  const int64_t n = unit / H;
  const int h = (int)(unit - n * H);
  const int64_t ukv = n * Hkv + h / (H / Hkv);
  const float gamma = expf(g != nullptr ? g[unit] : (g_gamma != nullptr ? g_gamma[h] : 0.f));
  float s = 0.f;
  for (int key = lane; key < K; key += 64) {
    const float zz = fmaf(gamma, z[unit * K + key], to_f32(k[ukv * K + key]));
    z[unit * K + key] = zz;
    s = fmaf(to_f32(q[unit * K + key]), zz, s);
  }
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) s += __shfl_xor(s, d, 64);
  if (lane == 0) den[unit] = s * scale;
}

template <int K, typename TIn>
hipError_t launch_k(const NormalizerParams& p, hipStream_t stream) {
  const int32_t n_rep = p.H / p.Hkv;
  if (p.seqs.num_chunks > 0) {
    const dim3 grid((unsigned)unit_grid(p.seqs.num_chunks, p.Hkv, n_rep, 1));
    hipLaunchKernelGGL((norm_chunk_sum_kernel<K, TIn>), grid, dim3(NT), 0, stream,
                       static_cast<const TIn*>(p.k), p.g, p.g_gamma, p.zrec, p.dlog, p.H, p.Hkv, p.seqs);
  }
  if (p.seqs.num_seqs > 0) {
    const dim3 grid((unsigned)((int64_t)p.seqs.num_seqs * p.H));
    hipLaunchKernelGGL((norm_scan_kernel<K>), grid, dim3(NT), 0, stream, p.zrec, p.dlog, p.z0, p.zt, p.H,
                       p.seqs);
  }
  if (p.seqs.num_chunks > 0) {
    const dim3 grid((unsigned)unit_grid(p.seqs.num_chunks, p.Hkv, n_rep, 1));
    hipLaunchKernelGGL((norm_chunk_out_kernel<K, TIn>), grid, dim3(NT), 0, stream,
                       static_cast<const TIn*>(p.q), static_cast<const TIn*>(p.k), p.g, p.g_gamma, p.zrec,
                       p.den, p.scale, p.H, p.Hkv, p.seqs);
  }
  return hipGetLastError();
}

template <typename TIn>
hipError_t launch_in(const NormalizerParams& p, hipStream_t stream) {
  switch (p.K) {
    case 16: return launch_k<16, TIn>(p, stream);
    case 32: return launch_k<32, TIn>(p, stream);
    case 64: return launch_k<64, TIn>(p, stream);
    case 128: return launch_k<128, TIn>(p, stream);
    case 256: return launch_k<256, TIn>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_chunk_normalizer(const NormalizerParams& p, hipStream_t stream) {
  return p.qkv_bf16 ? launch_in<__bf16>(p, stream) : launch_in<float>(p, stream);
}

hipError_t launch_step_normalizer(const StepNormalizerParams& p, hipStream_t stream) {
  const int64_t units = (int64_t)p.N * p.H;
  if (units == 0) return hipSuccess;
  const dim3 grid((unsigned)((units + 3) / 4));
  if (p.qkv_bf16) {
    hipLaunchKernelGGL(step_normalizer_kernel<__bf16>, grid, dim3(NT), 0, stream,
                       static_cast<const __bf16*>(p.q), static_cast<const __bf16*>(p.k), p.g, p.g_gamma,
                       p.z, p.den, p.scale, (int32_t)units, p.H, p.Hkv, p.K);
  } else {
    hipLaunchKernelGGL(step_normalizer_kernel<float>, grid, dim3(NT), 0, stream,
                       static_cast<const float*>(p.q), static_cast<const float*>(p.k), p.g, p.g_gamma,
                       p.z, p.den, p.scale, (int32_t)units, p.H, p.Hkv, p.K);
  }
  return hipGetLastError();
}

}  // namespace sgla
