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
// Chunked form: one workgroup per (sequence, head), chunks of 64 tokens in
// order.  The next chunk's q and k rows are loaded into registers (16-byte
// loads) while the current chunk is processed: rows to LDS, then thread i
// runs the recurrence of key i over the chunk's 64 tokens (z carried across
// chunks in a register) and leaves q_t[i] z_t[i] in LDS, and finally every
// token's products are summed over the keys.
//
// Decode: one wave per (sequence, head); lanes own keys.
#include <hip/hip_runtime.h>

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

template <int K, typename TIn>
__global__ void __launch_bounds__(NT)
chunk_normalizer_kernel(const TIn* __restrict__ q, const TIn* __restrict__ k,
                        const float* __restrict__ g, const float* __restrict__ g_gamma,
                        const float* __restrict__ z0, float* __restrict__ den, float* __restrict__ zt,
                        float scale, int32_t H, int32_t Hkv, SeqLayout seqs) {
  constexpr int EPL = 16 / sizeof(TIn);          // elements per 16-byte load
  constexpr int PR = K / EPL;                    // 16-byte pieces per row
  constexpr int NP = (C * PR + NT - 1) / NT;     // pieces per thread per matrix
  constexpr int KPT = (K + NT - 1) / NT;         // keys per thread
  constexpr int LDK = K + 1;                     // LDS row stride (floats)
  constexpr int RPT = NT / C;                    // reducer threads per token
  static_assert(K % EPL == 0, "K");
  __shared__ float sQ[C * LDK];
  __shared__ float sK[C * LDK];                  // k rows, then q_t[i] z_t[i]
  __shared__ float sGam[C];

  const UnitMap um = map_unit(blockIdx.x, 1, Hkv, H / Hkv, seqs.num_seqs);
  if (!um.valid) return;
  const int hd = um.hd, hk = um.hk;
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
  const int nchunks = (len + C - 1) / C;
  const int64_t RSQ = (int64_t)H * K, RSK = (int64_t)Hkv * K;
  const TIn* qb = q + (bos * H + hd) * K;
  const TIn* kb = k + (bos * Hkv + hk) * K;

  float z[KPT];
#pragma unroll
  for (int u = 0; u < KPT; ++u) {
    const int key = tid + NT * u;
    z[u] = (key < K && z0 != nullptr) ? z0[((int64_t)seq * H + hd) * K + key] : 0.f;
  }

  uint4 qx[NP], kx[NP];
  float gx = 0.f;
  auto load_chunk = [&](int m) {
    const int cl = min(C, len - m * C);
#pragma unroll
    for (int u = 0; u < NP; ++u) {
      const int p = tid + NT * u;
      const int c = p / PR, e = (p % PR) * EPL;
      qx[u] = make_uint4(0u, 0u, 0u, 0u);
      kx[u] = make_uint4(0u, 0u, 0u, 0u);
      if ((C * PR % NT == 0 || p < C * PR) && c < cl) {
        qx[u] = *reinterpret_cast<const uint4*>(qb + ((int64_t)m * C + c) * RSQ + e);
        kx[u] = *reinterpret_cast<const uint4*>(kb + ((int64_t)m * C + c) * RSK + e);
      }
    }
    if (tid < C) {
      const float lg = g != nullptr ? (tid < cl ? g[(bos + (int64_t)m * C + tid) * H + hd] : 0.f)
                                    : (g_gamma != nullptr ? g_gamma[hd] : 0.f);
      gx = tid < cl ? lg : 0.f;
    }
  };
  auto widen_store = [&](float* dst, const uint4& x, int c, int e) {
    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
    if constexpr (sizeof(TIn) == 2) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        dst[c * LDK + e + 2 * i] = __uint_as_float(w[i] << 16);
        dst[c * LDK + e + 2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) dst[c * LDK + e + i] = __uint_as_float(w[i]);
    }
  };

  if (nchunks > 0) load_chunk(0);
  for (int m = 0; m < nchunks; ++m) {
    const int cl = min(C, len - m * C);
#pragma unroll
    for (int u = 0; u < NP; ++u) {
      const int p = tid + NT * u;
      if (C * PR % NT == 0 || p < C * PR) {
        widen_store(sQ, qx[u], p / PR, (p % PR) * EPL);
        widen_store(sK, kx[u], p / PR, (p % PR) * EPL);
      }
    }
    if (tid < C) sGam[tid] = expf(gx);
    __syncthreads();
    if (m + 1 < nchunks) load_chunk(m + 1);
    // recurrence of each key over the chunk; products replace the k rows
#pragma unroll
    for (int u = 0; u < KPT; ++u) {
      const int key = tid + NT * u;
      if (key < K) {
        float zz = z[u];
        for (int c = 0; c < C; ++c) {
          zz = fmaf(sGam[c], zz, sK[c * LDK + key]);
          sK[c * LDK + key] = sQ[c * LDK + key] * zz;
        }
        z[u] = zz;   // padding tokens add 0 with decay 1: z is the state after the last real token
      }
    }
    __syncthreads();
    // den_c = scale * sum over keys, RPT threads per token
    {
      const int c = tid / RPT, part = tid % RPT;
      float s = 0.f;
      for (int i = part; i < K; i += RPT) s += sK[c * LDK + i];
#pragma unroll
      for (int d = RPT / 2; d >= 1; d >>= 1) s += __shfl_xor(s, d, 64);
      if (part == 0 && c < cl) den[(bos + (int64_t)m * C + c) * H + hd] = s * scale;
    }
    __syncthreads();
  }
  if (zt != nullptr) {
#pragma unroll
    for (int u = 0; u < KPT; ++u) {
      const int key = tid + NT * u;
      if (key < K) zt[((int64_t)seq * H + hd) * K + key] = z[u];
    }
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
  if (p.seqs.num_seqs == 0) return hipSuccess;
  const dim3 grid((unsigned)unit_grid(p.seqs.num_seqs, p.Hkv, p.H / p.Hkv, 1));
  hipLaunchKernelGGL((chunk_normalizer_kernel<K, TIn>), grid, dim3(NT), 0, stream,
                     static_cast<const TIn*>(p.q), static_cast<const TIn*>(p.k), p.g, p.g_gamma,
                     p.z0, p.den, p.zt, p.scale, p.H, p.Hkv, p.seqs);
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
