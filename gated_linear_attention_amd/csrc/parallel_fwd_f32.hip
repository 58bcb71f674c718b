// Parallel form of Simple GLA for float32 q, k and v: the decayed attention
// matrix written out and o = A v (page "flash-linear-attention 中的 Simple
// GLA", section 二: the parallel entry builds A explicitly; section 五: its
// test checks A, with float32 inputs among the cases).  Per batch row and
// query head, with G_t = g_0 + ... + g_t the running log gate:
//
//     A[i][j] = scale * (q_i . k_j) * exp(G_i - G_j)   for j <= i, else 0
//     o_i     = sum_j A[i][j] v_j
//
// No operand is rounded below float32.  One workgroup (4 waves, 16 query
// rows each) owns 64 query rows of one (batch row, query head) and walks the
// 64-key tiles from the one holding its diagonal back to the first:
//   S^T = K_j Q_i^T      on the fp64 matrix cores (v_mfma_f64_16x16x4_f64:
//                        the float32 inputs' products are exact in float64
//                        and so is nearly all of their sum), queries in
//                        registers, the key tile from LDS; A = scale S decay
//                        is formed in float64 and rounded once.  A is mostly
//                        zeros and decayed entries, so its RMS is a few
//                        hundredths of its largest entries: a float32 dot
//                        product's ~10 ulp on those entries would already
//                        exceed 1e-4 of the RMS;
//   O^T += V_j^T A^T     on the fp32 matrix cores (v_mfma_f32_16x16x4_f32);
//                        the lane's A values are already the B operand of
//                        this product (the key order of the k-steps follows
//                        the result layout of S^T, which puts four
//                        consecutive keys of one query row in each lane: one
//                        16-byte store of A), so A never leaves registers.
// The decay exponent is formed in float64 before its one rounding to float32:
// the query's running gate inside the query tile, plus the gate totals of the
// key tiles walked so far, minus the key's running gate inside its tile.  A
// reset gate (-1e4) therefore never leaves an exponent as the difference of
// two large float32 sums.
//
// Key dimensions and value widths are padded with zeros to the template
// width (64, 128 or 256); A rows past T are dropped by the store descriptor's
// bound and columns past T by the key-tile test, as in the bf16 kernel.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "gate_scan.h"
#include "mfma_common.h"
#include "sgla_internal.h"
#include "unit_map.h"

namespace sgla {
namespace {

using namespace mf;

constexpr int C = 64;     // query rows per workgroup, keys per key tile
constexpr int NTH = 256;  // 4 waves

// v_mfma_f32_16x16x4_f32, per lane l with g = l / 16, r = l % 16:
//   A operand: A[m = r][k = g]   B operand: B[k = g][n = r]   result D[m = 4g + i][n = r]
__device__ __forceinline__ f32x4 mfma4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// v_mfma_f64_16x16x4_f64: the same operand layout, float64 values, but the
// result rows interleaved: result D[m = g + 4i][n = r] (measured)
typedef double f64x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ f64x4 mfma4d(double a, double b, f64x4 c) {
  return __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ double gate_at(const ParallelParams& p, int b, int h, int t) {
  if (t >= p.T) return 0.0;
  if (p.g != nullptr) return (double)p.g[((int64_t)b * p.T + t) * p.H + h];
  return p.g_gamma != nullptr ? (double)p.g_gamma[h] : 0.0;
}

template <int KM, int VM, typename TOut>
__global__ __launch_bounds__(NTH) void parallel_fwd_f32_kernel(ParallelParams p) {
  constexpr int LDK = KM + 4;   // row pitch of the key tile (floats)
  constexpr int LDV = VM + 4;   // row pitch of the value tile
  constexpr int NKB = KM / 16;  // 16-wide blocks of the key dimension
  constexpr int NVT = VM / 16;  // 16-wide blocks of the value dimension
  constexpr int KF4 = KM / 4;   // float4 pieces of one key row
  constexpr int VF4 = VM / 4;
  __shared__ __attribute__((aligned(16))) float sK[C * LDK];
  __shared__ __attribute__((aligned(16))) float sV[C * LDV];
  __shared__ __attribute__((aligned(16))) double sL[C];  // key gates inside the tile, inclusive, log2 units
  __shared__ double sTot;                                // the tile's gate total, natural log

  const int T = p.T, H = p.H, Hkv = p.Hkv, K = p.K, V = p.V;
  const int nT = (T + C - 1) / C;
  const UnitMap u = map_unit((int32_t)blockIdx.x, nT, Hkv, H / Hkv, p.B);
  if (!u.valid) return;
  const int iq = nT - 1 - u.vt;  // longest walks first
  const int b = u.rank, h = u.hd, hk = u.hk;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g4 = lane >> 4, r = lane & 15;
  const int i0 = iq * C;
  const int qrow = 16 * w + r;   // this lane's query row inside the tile
  const int qi = i0 + qrow;
  const int nkb = K / 16, nvt = V / 16;   // blocks past these are zero padding

  // qf[m][e] = q[qi][16 m + 4 g4 + e]: the B operand of S^T for k-step (m, e)
  const float* qg = static_cast<const float*>(p.q);
  f32x4 qf[NKB];
#pragma unroll
  for (int m = 0; m < NKB; ++m) {
    qf[m] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (qi < T && m < nkb) qf[m] = *reinterpret_cast<const f32x4*>(qg + (((int64_t)b * T + qi) * H + h) * K + 16 * m + 4 * g4);
  }
  // running gate of the query rows from the tile start, inclusive (log2, float64)
  const double Rall = wave_scan_f64(gate_at(p, b, h, i0 + lane), 64) * kRcpLn2d;
  const double Rq = __shfl(Rall, qrow, 64);

  const float* kg = static_cast<const float*>(p.k);
  const float* vg = static_cast<const float*>(p.v);
  const float scale = p.scale;

  // A rows of this workgroup through one descriptor (rows past T dropped by
  // its bound, every store when no A is wanted: bound 0).  16-byte stores need
  // 16-byte aligned rows (T % 4 == 0); otherwise every tile stores elements.
  const int tlim = (T & 3) == 0 ? T : 0;
  const int rows = min(C, T - i0);
  const __amdgpu_buffer_rsrc_t ra =
      make_rsrc(p.attn != nullptr ? p.attn + (((int64_t)b * H + h) * T + i0) * (int64_t)T : nullptr,
                p.attn != nullptr ? (uint32_t)rows * (uint32_t)T * 4u : 0u);
  const uint32_t arow = (uint32_t)qrow * (uint32_t)T * 4u;

  f32x4 O[NVT];
#pragma unroll
  for (int vt = 0; vt < NVT; ++vt) O[vt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Key and value tiles (zeros past T, past K and past V).  Where the
  // registers allow (K + V <= 256 after padding), the next tile is loaded
  // into registers while the current one computes; otherwise each tile is
  // loaded when it is staged.
  constexpr bool PREF = KM + VM <= 256;
  constexpr int NKL = KF4 * C / NTH, NVL = VF4 * C / NTH;
  f32x4 kr[NKL], vr[NVL];
  double gr = 0.0;
  auto load_tile = [&](int jt) {
    const int j0 = jt * C;
#pragma unroll
    for (int n = 0; n < NKL; ++n) {
      const int f = tid + NTH * n, row = f / KF4, c4 = f % KF4;
      kr[n] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (j0 + row < T && 4 * c4 < K)
        kr[n] = *reinterpret_cast<const f32x4*>(kg + (((int64_t)b * T + j0 + row) * Hkv + hk) * K + 4 * c4);
    }
#pragma unroll
    for (int n = 0; n < NVL; ++n) {
      const int f = tid + NTH * n, row = f / VF4, c4 = f % VF4;
      vr[n] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (j0 + row < T && 4 * c4 < V)
        vr[n] = *reinterpret_cast<const f32x4*>(vg + (((int64_t)b * T + j0 + row) * Hkv + hk) * V + 4 * c4);
    }
    if (w == 0) gr = gate_at(p, b, h, j0 + lane);
  };
  auto stage_tile = [&]() {
#pragma unroll
    for (int n = 0; n < NKL; ++n) {
      const int f = tid + NTH * n;
      *reinterpret_cast<f32x4*>(sK + (f / KF4) * LDK + 4 * (f % KF4)) = kr[n];
    }
#pragma unroll
    for (int n = 0; n < NVL; ++n) {
      const int f = tid + NTH * n;
      *reinterpret_cast<f32x4*>(sV + (f / VF4) * LDV + 4 * (f % VF4)) = vr[n];
    }
    if (w == 0) {
      const double s = wave_scan_f64(gr, 64);
      sL[lane] = s * kRcpLn2d;
      if (lane == 63) sTot = s;
    }
  };

  double D = 0.0;  // gate sum from the key tile's start to the query tile's start (natural log)
  if (PREF) load_tile(iq);
#pragma nounroll
  for (int jt = iq; jt >= 0; --jt) {
    const int j0 = jt * C;
    __syncthreads();  // the previous tile's LDS reads are done
    if (!PREF) load_tile(jt);
    stage_tile();
    __syncthreads();
    if (PREF && jt > 0) load_tile(jt - 1);   // in flight while this tile computes
    if (jt < iq) D += sTot;
    const double base = Rq + D * kRcpLn2d;  // exponent of A = base - sL[key] (log2)

    // S^T = K_j Q_i^T: sd[kb][e] = k_j . q_i for key j = j0 + 16 kb + 4 g4 + e.
    // Product row m holds key 4 (m % 4) + m / 4 of the 16-key block, so that
    // the interleaved result rows g4 + 4 e are the keys 4 g4 + e.
    const int krow = 4 * (r & 3) + (r >> 2);
    f64x4 sd[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) sd[kb] = f64x4{0.0, 0.0, 0.0, 0.0};
    // (padding columns of q and of the key tile are zeros: every product is
    // issued, a runtime bound here would make the compiler copy accumulators)
#pragma unroll
    for (int m = 0; m < NKB; ++m) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const f32x4 ka = *reinterpret_cast<const f32x4*>(sK + (16 * kb + krow) * LDK + 16 * m + 4 * g4);
#pragma unroll
        for (int e = 0; e < 4; ++e) sd[kb] = mfma4d((double)ka[e], (double)qf[m][e], sd[kb]);
      }
    }
    // decay, scale and (in the diagonal tile) the causal mask; A rounded once
    f32x4 s[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int jj = 16 * kb + 4 * g4 + e;
        const float dec = exp2_hw((float)(base - sL[jj]));
        const float x = (float)(sd[kb][e] * (double)scale * (double)dec);
        s[kb][e] = (jt == iq && jj > qrow) ? 0.f : x;
      }
    }
    if (j0 + C <= tlim) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, s[kb]), ra,
                                               arow + (uint32_t)(j0 + 16 * kb + 4 * g4) * 4u, 0, 0);
    } else {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int j = j0 + 16 * kb + 4 * g4 + e;
          const float x = s[kb][e];
          if (j < T)
            __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, x), ra, arow + (uint32_t)j * 4u, 0, 0);
        }
    }
    // O^T += V^T A^T: k-step (kb, e) takes keys 16 kb + 4 g' + e (g' = 0..3),
    // whose A values this lane holds as s[kb][e]
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float* vrow = sV + (16 * kb + 4 * g4 + e) * LDV + r;
#pragma unroll
        for (int vt = 0; vt < NVT; ++vt) O[vt] = mfma4(vrow[16 * vt], s[kb][e], O[vt]);   // zeros past V
      }
  }

  // o: the lane holds o[qi][16 vt + 4 g4 + i]
  if (qi < T) {
    TOut* orow = static_cast<TOut*>(p.o) + (((int64_t)b * T + qi) * H + h) * V;
#pragma unroll
    for (int vt = 0; vt < NVT; ++vt) {
      if (vt < nvt) {
        if constexpr (sizeof(TOut) == 4) {
          *reinterpret_cast<f32x4*>(orow + 16 * vt + 4 * g4) = O[vt];
        } else {
          bf16x4 y;
#pragma unroll
          for (int e = 0; e < 4; ++e) y[e] = (bf16)O[vt][e];
          *reinterpret_cast<bf16x4*>(orow + 16 * vt + 4 * g4) = y;
        }
      }
    }
  }

  // zeros right of the diagonal tile, one row of the wave at a time
  {
    const int cz = p.attn != nullptr ? min(T, i0 + C) : T;
    const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};
    for (int rr = 16 * w; rr < 16 * w + 16 && rr < rows && cz < T; ++rr) {
      const uint32_t ro = (uint32_t)rr * (uint32_t)T * 4u;
      if (tlim != 0) {
        for (int c = cz + 4 * lane; c < T; c += 256)
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, z4), ra, ro + (uint32_t)c * 4u, 0, 0);
      } else {
        for (int c = cz + lane; c < T; c += 64)
          __builtin_amdgcn_raw_buffer_store_b32(0u, ra, ro + (uint32_t)c * 4u, 0, 0);
      }
    }
  }
}

template <int KM, int VM>
hipError_t launch_kv(const ParallelParams& p, hipStream_t stream) {
  const dim3 grid((uint32_t)unit_grid(p.B, p.Hkv, p.H / p.Hkv, (p.T + C - 1) / C));
  if (p.o_f32)
    hipLaunchKernelGGL((parallel_fwd_f32_kernel<KM, VM, float>), grid, dim3(NTH), 0, stream, p);
  else
    hipLaunchKernelGGL((parallel_fwd_f32_kernel<KM, VM, bf16>), grid, dim3(NTH), 0, stream, p);
  return hipGetLastError();
}

template <int KM>
hipError_t launch_k(const ParallelParams& p, hipStream_t stream) {
  if (p.V <= 64) return launch_kv<KM, 64>(p, stream);
  return p.V <= 128 ? launch_kv<KM, 128>(p, stream) : launch_kv<KM, 256>(p, stream);
}

}  // namespace

hipError_t launch_parallel_fwd_f32(const ParallelParams& p, hipStream_t stream) {
  if (p.B == 0 || p.T == 0) return hipSuccess;
  if (!parallel_f32_supported(p.K, p.V) || p.Hkv <= 0 || p.H % p.Hkv != 0) return hipErrorInvalidValue;
  if (p.K <= 64) return launch_k<64>(p, stream);
  return p.K <= 128 ? launch_k<128>(p, stream) : launch_k<256>(p, stream);
}

}  // namespace sgla
