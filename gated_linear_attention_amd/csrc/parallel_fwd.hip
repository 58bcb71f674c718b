// Parallel form of Simple GLA: the decayed attention matrix written out
// (page "flash-linear-attention 中的 Simple GLA", section 二: the parallel
// entry builds the matrix A explicitly; section 五: its test checks A).
// Per batch row and query head, with b the running log2 gate (b_t = (g_0 +
// ... + g_t) / ln 2):
//
//     A[i][j] = scale * (q_i . k_j) * 2^(b_i - b_j)   for j <= i, else 0
//     o_i     = sum_j A[i][j] v_j
//
// One workgroup owns 64 query rows of one (batch row, query head) and walks
// the key tiles from its diagonal tile back to the first one.  Every tile is
// a dense contraction on the bf16 matrix cores: S^T = K_j Q_i^T with the
// queries held in registers, then O^T += V_j^T A^T with A split into bf16
// hi + lo halves (A itself is an fp32 product with a decay, not a bf16
// value).  The exponent never needs the absolute running gate: it is the
// query's gate inside its tile, minus the key's gate inside its tile, plus the
// sum of the whole-tile gates in between, accumulated as the walk moves left,
// so far-apart tokens do not cancel two large running sums.
//
// Written A is T x T float32 per head, written once and never read again:
// the kernel is bound by those stores, and every workgroup writes the same 64
// full rows (computed tiles on and left of the diagonal, zeros right of it),
// so the work per workgroup is even whatever its position.
#include <hip/hip_runtime.h>

#include "gate_scan.h"
#include "mfma_common.h"
#include "sgla_internal.h"
#include "unit_map.h"

namespace sgla {
namespace {

using namespace mf;

constexpr int C = 64;     // query rows per workgroup, keys per key tile
constexpr int NTH = 256;  // 4 waves, 16 query rows each

__device__ __forceinline__ float log_gate(const ParallelParams& p, int b, int h, int t) {
  if (t >= p.T) return 0.f;
  if (p.g != nullptr) return p.g[((int64_t)b * p.T + t) * p.H + h];
  return p.g_gamma != nullptr ? p.g_gamma[h] : 0.f;
}

template <int K, int VMAX, typename TOut>
__global__ __launch_bounds__(NTH) void parallel_fwd_kernel(ParallelParams p) {
  constexpr int LDK = K + 8;     // row pitch of the key tile (bf16), padded against bank conflicts
  constexpr int LDV = VMAX + 8;  // row pitch of the value tile
  constexpr int NKP = K / 32;    // 16-byte pieces of the key tile per thread
  constexpr int NVP = VMAX / 32; // 16-byte pieces of the value tile per thread
  constexpr int NVT = VMAX / 16; // 16-column value blocks (those past V are zeros)
  __shared__ __attribute__((aligned(16))) bf16 sK[C * LDK];
  __shared__ __attribute__((aligned(16))) bf16 sV[C * LDV];
  __shared__ __attribute__((aligned(16))) float sL[C];   // key gates inside the tile (log2)

  const int T = p.T, H = p.H, Hkv = p.Hkv, V = p.V;
  const int nT = (T + C - 1) / C;
  const UnitMap u = map_unit((int32_t)blockIdx.x, nT, Hkv, H / Hkv, p.B);
  if (!u.valid) return;
  const int it = nT - 1 - u.vt;  // longest row tiles first
  const int b = u.rank, h = u.hd, hk = u.hk;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g4 = lane >> 4, r = lane & 15;
  const int i0 = it * C;
  const int qi = i0 + 16 * w + r;  // query row this lane accumulates
  const int nvt = V / 16;

  const bf16* qg = static_cast<const bf16*>(p.q);

  // queries of this lane's row, as the B operand of S^T = K Q^T
  bf16x8 qf[NKP];
#pragma unroll
  for (int kk = 0; kk < NKP; ++kk) {
    u32x4 x = {0u, 0u, 0u, 0u};
    if (qi < T) x = *reinterpret_cast<const u32x4*>(qg + (((int64_t)b * T + qi) * H + h) * K + 32 * kk + 8 * g4);
    qf[kk] = __builtin_bit_cast(bf16x8, x);
  }
  // running log2 gate of the query rows inside their tile
  const float Lrow = wave_cumsum_log2(log_gate(p, b, h, i0 + lane));
  const float Lq = __shfl(Lrow, 16 * w + r, 64);

  // Key and value tiles come through buffer descriptors that start at the
  // tile: rows past T read as zeros, and so do the value columns past V (their
  // lanes get an offset beyond any bound), so the LDS tiles are always whole.
  const bf16* kbase = static_cast<const bf16*>(p.k) + (int64_t)b * T * Hkv * K;
  const bf16* vbase = static_cast<const bf16*>(p.v) + (int64_t)b * T * Hkv * V;
  constexpr int KRS = NTH / (K / 8);     // key rows per pass of the workgroup
  constexpr int VRS = NTH / (VMAX / 8);  // value rows per pass
  const uint32_t kof = (uint32_t)(((tid / (K / 8)) * Hkv + hk) * K + 8 * (tid % (K / 8))) * 2u;
  const uint32_t kstep = (uint32_t)KRS * Hkv * K * 2u;
  const int kls = (tid / (K / 8)) * LDK + 8 * (tid % (K / 8));
  const bool vok = 8 * (tid % (VMAX / 8)) < V;
  const uint32_t vof = (uint32_t)(((tid / (VMAX / 8)) * Hkv + hk) * V + 8 * (tid % (VMAX / 8))) * 2u;
  const uint32_t vstep = (uint32_t)VRS * Hkv * V * 2u;
  const int vls = (tid / (VMAX / 8)) * LDV + 8 * (tid % (VMAX / 8));

  u32x4 kr[NKP], vr[NVP];
  float gr = 0.f;
  auto load = [&](int jt) {
    const int j0 = jt * C;
    const __amdgpu_buffer_rsrc_t rk =
        make_rsrc(kbase + (int64_t)j0 * Hkv * K, (uint32_t)(T - j0) * Hkv * K * 2u);
    const __amdgpu_buffer_rsrc_t rv =
        make_rsrc(vbase + (int64_t)j0 * Hkv * V, (uint32_t)(T - j0) * Hkv * V * 2u);
#pragma unroll
    for (int m = 0; m < NKP; ++m) kr[m] = __builtin_amdgcn_raw_buffer_load_b128(rk, kof + m * kstep, 0, 0);
#pragma unroll
    for (int m = 0; m < NVP; ++m)
      vr[m] = __builtin_amdgcn_raw_buffer_load_b128(rv, vok ? vof + m * vstep : 0xfffffff0u, 0, 0);
    if (w == 0) gr = log_gate(p, b, h, j0 + lane);
  };
  auto stage = [&]() {
#pragma unroll
    for (int m = 0; m < NKP; ++m) *reinterpret_cast<u32x4*>(sK + kls + m * KRS * LDK) = kr[m];
#pragma unroll
    for (int m = 0; m < NVP; ++m) *reinterpret_cast<u32x4*>(sV + vls + m * VRS * LDV) = vr[m];
    if (w == 0) sL[lane] = wave_cumsum_log2(gr);
  };

  // The 64 A rows of this workgroup through one descriptor: rows past T are
  // dropped by its bound (and every store when no A is wanted: bound 0);
  // columns past T are kept out by the key-tile test.  16-byte stores need
  // rows 16-byte aligned (T % 4 == 0); otherwise every tile takes the
  // element-wise stores (tlim = 0).
  const int tlim = (T & 3) == 0 ? T : 0;
  const int rows = min(C, T - i0);
  const __amdgpu_buffer_rsrc_t ra =
      make_rsrc(p.attn + (((int64_t)b * H + h) * T + i0) * (int64_t)T,
                p.attn != nullptr ? (uint32_t)rows * (uint32_t)T * 4u : 0u);
  const uint32_t arow = (uint32_t)(16 * w + r) * (uint32_t)T * 4u;  // this lane's row in the descriptor

  f32x4 O[NVT];
#pragma unroll
  for (int vt = 0; vt < NVT; ++vt) O[vt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float D = 0.f;  // log2 decay over the whole key tiles between this key tile and the query tile

  load(it);
#pragma nounroll
  for (int jt = it; jt >= 0; --jt) {
    __syncthreads();  // the previous tile's LDS reads are done
    stage();
    __syncthreads();
    if (jt > 0) load(jt - 1);
    const int j0 = jt * C;
    if (jt < it) D += sL[C - 1];

    f32x4 s[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      s[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < NKP; ++kk) {
        const bf16x8 ka = *reinterpret_cast<const bf16x8*>(sK + (16 * kb + r) * LDK + 32 * kk + 8 * g4);
        s[kb] = mfma(ka, qf[kk], s[kb]);
      }
    }
    // s[kb][e] = (k_j . q_i) for key j = j0 + 16 kb + 4 g4 + e and query qi
    const float base = Lq + D;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const f32x4 Lk = *reinterpret_cast<const f32x4*>(sL + 16 * kb + 4 * g4);
#pragma unroll
      for (int e = 0; e < 4; ++e) s[kb][e] = p.scale * s[kb][e] * exp2_hw(base - Lk[e]);
    }
    // causal mask: inside the diagonal tile keys past the lane's query row are
    // dropped; further left every key is kept
    const int lim = jt == it ? 16 * w + r - 4 * g4 : C;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (16 * kb + e > lim) s[kb][e] = 0.f;
    {
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
            const float x = s[kb][e];  // element copied out first: a bit_cast of a vector element
                                       // subscript would reinterpret the vector's first element
            if (j < T)
              __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, x), ra,
                                                    arow + (uint32_t)j * 4u, 0, 0);
          }
      }
    }
    // O^T += V^T A^T: the lane's A values for keys 32 hf + {4 g4 .. 4 g4 + 3,
    // 16 + 4 g4 .. 16 + 4 g4 + 3} are the B operand in that key order, and the
    // two transposed reads of V take the same keys.
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const float x[8] = {s[2 * hf][0], s[2 * hf][1], s[2 * hf][2], s[2 * hf][3],
                          s[2 * hf + 1][0], s[2 * hf + 1][1], s[2 * hf + 1][2], s[2 * hf + 1][3]};
      bf16x8 ah, al;
      split8(x, ah, al);
#pragma unroll
      for (int vt = 0; vt < NVT; ++vt) {  // value columns past V are zeros in the tile
        const bf16x8 vt8 = cat(tr_read(sV, LDV, 32 * hf + 4 * g4, 16 * vt),
                               tr_read(sV, LDV, 32 * hf + 16 + 4 * g4, 16 * vt));
        O[vt] = mfma(vt8, ah, O[vt]);
        O[vt] = mfma(vt8, al, O[vt]);
      }
    }
  }

  // o: lane holds o[qi][16 vt + 4 g4 + e]
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

  // zeros right of the diagonal tile, one row per wave at a time
  {
    const int cz = p.attn != nullptr ? min(T, i0 + C) : T;
    const bool vec = tlim != 0;
    const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};
    for (int rr = w; rr < rows && cz < T; rr += 4) {
      const uint32_t ro = (uint32_t)rr * (uint32_t)T * 4u;
      if (vec) {
        for (int c = cz + 4 * lane; c < T; c += 256)
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, z4), ra, ro + (uint32_t)c * 4u, 0, 0);
      } else {
        for (int c = cz + lane; c < T; c += 64)
          __builtin_amdgcn_raw_buffer_store_b32(0u, ra, ro + (uint32_t)c * 4u, 0, 0);
      }
    }
  }
}

template <int K, int VMAX>
hipError_t launch_kv(const ParallelParams& p, dim3 grid, hipStream_t stream) {
  if (p.o_f32)
    hipLaunchKernelGGL((parallel_fwd_kernel<K, VMAX, float>), grid, dim3(NTH), 0, stream, p);
  else
    hipLaunchKernelGGL((parallel_fwd_kernel<K, VMAX, bf16>), grid, dim3(NTH), 0, stream, p);
  return hipGetLastError();
}

template <int K>
hipError_t launch_k(const ParallelParams& p, dim3 grid, hipStream_t stream) {
  if (p.V <= 64) return launch_kv<K, 64>(p, grid, stream);
  return p.V <= 128 ? launch_kv<K, 128>(p, grid, stream) : launch_kv<K, 256>(p, grid, stream);
}

}  // namespace

hipError_t launch_parallel_fwd(const ParallelParams& p, hipStream_t stream) {
  if (p.B == 0 || p.T == 0) return hipSuccess;
  if (!parallel_supported(p.K, p.V) || p.Hkv <= 0 || p.H % p.Hkv != 0) return hipErrorInvalidValue;
  const int32_t nT = (p.T + C - 1) / C;
  const dim3 grid((uint32_t)unit_grid(p.B, p.Hkv, p.H / p.Hkv, nT));
  switch (p.K) {
    case 64: return launch_k<64>(p, grid, stream);
    case 128: return launch_k<128>(p, grid, stream);
    default: return launch_k<256>(p, grid, stream);
  }
}

}  // namespace sgla
