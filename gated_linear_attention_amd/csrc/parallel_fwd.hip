// Parallel form of Simple GLA: the decayed attention matrix written out
// (page "flash-linear-attention 中的 Simple GLA", section 二: the parallel
// entry builds the matrix A explicitly; section 五: its test checks A).
// Per batch row and query head, with b the running log2 gate (b_t = (g_0 +
// ... + g_t) / ln 2):
//
//     A[i][j] = scale * (q_i . k_j) * 2^(b_i - b_j)   for j <= i, else 0
//     o_i     = sum_j A[i][j] v_j
//
// One workgroup owns 128 query rows (64 when K or V is 256) of one (batch
// row, query head) and walks the 64-key tiles from the tiles that hold its
// diagonal back to the first one.  Every tile is a dense contraction on the
// bf16 matrix cores: S^T = K_j Q_i^T with the queries held in registers, then
// O^T += V_j^T A^T with A split into bf16 hi + lo halves (A itself is an fp32
// product with a decay, not a bf16 value).  The exponent never needs the
// absolute running gate: it is the query's gate inside its query tile, minus
// the key's gate inside its key tile, plus the sum of the whole-tile gates in
// between, accumulated in float64 as the walk moves left, so far-apart tokens
// do not cancel two large running sums.
//
// Written A is T x T float32 per head, written once and never read again:
// the kernel is bound by those stores.  Every workgroup writes the same
// number of full rows (computed tiles on and left of the diagonal, zeros
// right of it), so the store work per workgroup is even whatever its
// position; the 256-byte row segments of the computed tiles are what keeps
// it below a plain fill's write rate.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "gate_scan.h"
#include "mfma_common.h"
#include "sgla_internal.h"
#include "unit_map.h"

namespace sgla {
namespace {

using namespace mf;

constexpr int C = 64;     // keys per key tile
constexpr int NTH = 256;  // 4 waves

// 16-row query blocks per wave: 2 (128 query rows per workgroup) where the
// registers allow, so every key and value fragment read from LDS feeds two
// products; 1 (64 rows) for the widest heads.
template <int K, int VMAX>
constexpr int row_blocks() { return (K <= 128 && VMAX <= 128) ? 2 : 1; }

__device__ __forceinline__ float log_gate(const ParallelParams& p, int b, int h, int t) {
  if (t >= p.T) return 0.f;
  if (p.g != nullptr) return p.g[((int64_t)b * p.T + t) * p.H + h];
  return p.g_gamma != nullptr ? p.g_gamma[h] : 0.f;
}

// Inclusive scan of one 64-token gate tile over the wave (lane i: the sum of
// tokens 0..i times 1/ln 2, rounded to float32), and the tile's total in
// float64 natural-log units (every lane).
__device__ __forceinline__ float tile_scan(float x, double& total) {
  const int lane = threadIdx.x & 63;
  double s = (double)x;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const double y = __shfl_up(s, d, 64);
    if (lane >= d) s += y;
  }
  total = __shfl(s, 63, 64);
  return (float)(s * kRcpLn2d);
}

template <int K, int VMAX, typename TOut>
__global__ __launch_bounds__(NTH, (K == 256 && VMAX == 256) ? 1 : 2) void parallel_fwd_kernel(ParallelParams p) {
  constexpr int QB = row_blocks<K, VMAX>();
  constexpr int QR = 64 * QB;    // query rows per workgroup
  constexpr int WR = 16 * QB;    // query rows per wave
  constexpr int LDK = K + 8;     // row pitch of the key tile (bf16), padded against bank conflicts
  constexpr int LDV = VMAX + 8;  // row pitch of the value tile
  constexpr int NKP = K / 32;    // 16-byte pieces of the key tile per thread
  constexpr int NVP = VMAX / 32; // 16-byte pieces of the value tile per thread
  constexpr int NVT = VMAX / 16; // 16-column value blocks (those past V are zeros)
  __shared__ __attribute__((aligned(16))) bf16 sK[C * LDK];
  __shared__ __attribute__((aligned(16))) bf16 sV[C * LDV];
  __shared__ __attribute__((aligned(16))) float sL[C];   // key gates inside the tile (log2)
  __shared__ double sTot;                                 // the tile's gate total (natural log)

  const int T = p.T, H = p.H, Hkv = p.Hkv, V = p.V;
  const int nT = (T + C - 1) / C;
  const int nQ = (T + QR - 1) / QR;
  const UnitMap u = map_unit((int32_t)blockIdx.x, nQ, Hkv, H / Hkv, p.B);
  if (!u.valid) return;
  const int iq = nQ - 1 - u.vt;  // longest query tiles first
  const int b = u.rank, h = u.hd, hk = u.hk;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g4 = lane >> 4, r = lane & 15;
  const int i0 = iq * QR;
  const int wr0 = WR * w;        // first row of this wave inside the query tile
  const int nvt = V / 16;

  // queries of this lane's rows (i0 + wr0 + 16 qb + r), the B operand of S^T = K Q^T
  const bf16* qg = static_cast<const bf16*>(p.q);
  // scale enters as log2|scale| in the exponent and its sign on q (a bf16
  // sign flip is exact)
  const float lscale = log2f(fabsf(p.scale));
  const uint32_t qsign = p.scale < 0.f ? 0x80008000u : 0u;
  bf16x8 qf[QB][NKP];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int qi = i0 + wr0 + 16 * qb + r;
#pragma unroll
    for (int kk = 0; kk < NKP; ++kk) {
      u32x4 x = {0u, 0u, 0u, 0u};
      if (qi < T) x = *reinterpret_cast<const u32x4*>(qg + (((int64_t)b * T + qi) * H + h) * K + 32 * kk + 8 * g4);
      qf[qb][kk] = __builtin_bit_cast(bf16x8, x ^ qsign);
    }
  }
  // running log2 gate R of the query rows from the start of their 64-row
  // half of the query tile (one scan per half, each from zero, so a very
  // negative gate in the first half does not leave the second half's R as a
  // small difference of two large floats)
  float Rh[QB];
#pragma unroll
  for (int hh = 0; hh < QB; ++hh) Rh[hh] = wave_cumsum_log2(log_gate(p, b, h, i0 + 64 * hh + lane));
  const float R63 = QB == 2 ? __shfl(Rh[0], 63, 64) : 0.f;   // the first half's total
  const bool upper = QB == 2 && wr0 >= 64;   // this wave's rows are in the second half
  float Lq[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) Lq[qb] = __shfl(Rh[upper ? 1 : 0], (wr0 + 16 * qb + r) & 63, 64);

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

  // The A rows of this workgroup through one descriptor: rows past T are
  // dropped by its bound (and every store when no A is wanted: bound 0);
  // columns past T are kept out by the key-tile test.  16-byte stores need
  // rows 16-byte aligned (T % 4 == 0); otherwise every tile takes the
  // element-wise stores (tlim = 0).
  const int tlim = (T & 3) == 0 ? T : 0;
  const int rows = min(QR, T - i0);
  const __amdgpu_buffer_rsrc_t ra =
      make_rsrc(p.attn != nullptr ? p.attn + (((int64_t)b * H + h) * T + i0) * (int64_t)T : nullptr,
                p.attn != nullptr ? (uint32_t)rows * (uint32_t)T * 4u : 0u);

  f32x4 O[QB][NVT];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int vt = 0; vt < NVT; ++vt) O[qb][vt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // The exponent of A[i][j] is R_i + D - L_j (log2 units): L_j the key's
  // running gate inside its tile and D the gate sum from the key tile's start
  // to the start of the row's half of the query tile.  Key tiles are walked
  // from the query tile leftwards, so D grows by each tile's total
  // (accumulated in float64); workgroups of one head start at different key
  // tiles, which spreads their A stores over the memory channels.
  const int jd = QB * iq;                      // first key tile inside the query tile
  const int jlast = min(jd + QB - 1, nT - 1);  // last key tile any row of the tile reaches
  double Dacc = 0.0;   // gate total of the key tiles walked so far before the query tile
  double Tjd = 0.0;    // gate total of key tile jd (the query tile's first half)
  double Tnext = 0.0;  // gate total and running gates of the next key tile to stage (wave 0)
  float Lnext = 0.f;

  // One key tile: S^T on the matrix cores, the decay and (in the tiles that
  // hold a diagonal) the causal mask, the A stores, then O^T += V^T A^T.
  auto tile = [&](int jt, auto masked) {
    const int j0 = jt * C;
    if (jt < jd) Dacc += sTot;
    if (jt == jd) Tjd = sTot;
    float D;
    if (!upper) D = jt > jd ? -R63 : (float)(Dacc * kRcpLn2d);   // tile jd + 1 is masked for these rows
    else D = jt > jd ? 0.f : (float)((Dacc + Tjd) * kRcpLn2d);
    f32x4 s[QB][4];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) s[qb][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int kk = 0; kk < NKP; ++kk) {
        const bf16x8 ka = *reinterpret_cast<const bf16x8*>(sK + (16 * kb + r) * LDK + 32 * kk + 8 * g4);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) s[qb][kb] = mfma(ka, qf[qb][kk], s[qb][kb]);
      }
    // s[qb][kb][e] = (k_j . q_i) for key j = j0 + 16 kb + 4 g4 + e and
    // query i = i0 + wr0 + 16 qb + r (q already carries the sign of scale)
    f32x4 Lk[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) Lk[kb] = *reinterpret_cast<const f32x4*>(sL + 16 * kb + 4 * g4);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float base = Lq[qb] + D + lscale;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int e = 0; e < 4; ++e) s[qb][kb][e] = s[qb][kb][e] * exp2_hw(base - Lk[kb][e]);
      if constexpr (decltype(masked)::value) {
        // keys past the lane's query row are dropped (a wave whose rows all
        // precede the tile computes it fully masked)
        const int off = i0 + wr0 + 16 * qb - j0;
        const int lim = off < C - 1 ? off + r - 4 * g4 : C;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (16 * kb + e > lim) s[qb][kb][e] = 0.f;
      }
      const uint32_t arow = (uint32_t)(wr0 + 16 * qb + r) * (uint32_t)T * 4u;
      if (j0 + C <= tlim) {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, s[qb][kb]), ra,
                                                 arow + (uint32_t)(j0 + 16 * kb + 4 * g4) * 4u, 0, 0);
      } else {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int j = j0 + 16 * kb + 4 * g4 + e;
            const float x = s[qb][kb][e];  // element copied out first: a bit_cast of a vector
                                           // element subscript reinterprets the first element
            if (j < T)
              __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, x), ra,
                                                    arow + (uint32_t)j * 4u, 0, 0);
          }
      }
    }
    // O^T += V^T A^T: the lane's A values for keys 32 hf + {4 g4 .. 4 g4 + 3,
    // 16 + 4 g4 .. 16 + 4 g4 + 3} are the B operand in that key order, and
    // the two transposed reads of V take the same keys.
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      bf16x8 ah[QB], al[QB];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const float x[8] = {s[qb][2 * hf][0], s[qb][2 * hf][1], s[qb][2 * hf][2], s[qb][2 * hf][3],
                            s[qb][2 * hf + 1][0], s[qb][2 * hf + 1][1], s[qb][2 * hf + 1][2],
                            s[qb][2 * hf + 1][3]};
        split8(x, ah[qb], al[qb]);
      }
#pragma unroll
      for (int vt = 0; vt < NVT; ++vt) {  // value columns past V are zeros in the tile
        const bf16x8 vt8 = cat(tr_read(sV, LDV, 32 * hf + 4 * g4, 16 * vt),
                               tr_read(sV, LDV, 32 * hf + 16 + 4 * g4, 16 * vt));
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          O[qb][vt] = mfma(vt8, ah[qb], O[qb][vt]);
          O[qb][vt] = mfma(vt8, al[qb], O[qb][vt]);
        }
      }
    }
  };
  // Stage key tile jt (loaded into registers one step earlier) and prefetch
  // the next one.
  auto next = [&](int jt) {
    __syncthreads();  // the previous tile's LDS reads are done
#pragma unroll
    for (int m = 0; m < NKP; ++m) *reinterpret_cast<u32x4*>(sK + kls + m * KRS * LDK) = kr[m];
#pragma unroll
    for (int m = 0; m < NVP; ++m) *reinterpret_cast<u32x4*>(sV + vls + m * VRS * LDV) = vr[m];
    if (w == 0) {
      sL[lane] = Lnext;
      if (lane == 0) sTot = Tnext;
    }
    __syncthreads();
    if (jt > 0) load(jt - 1);
  };
  auto after = [&](int jt) {
    if (w == 0 && jt > 0) Lnext = tile_scan(gr, Tnext);  // gates of the tile loaded above
  };

  load(jlast);
  Lnext = w == 0 ? tile_scan(gr, Tnext) : 0.f;
#pragma nounroll
  for (int jt = jlast; jt >= jd; --jt) {  // key tiles inside the query tile: causal mask
    next(jt);
    tile(jt, std::true_type{});
    after(jt);
  }
#pragma nounroll
  for (int jt = jd - 1; jt >= 0; --jt) {  // key tiles wholly before it
    next(jt);
    tile(jt, std::false_type{});
    after(jt);
  }

  // o: lane holds o[i][16 vt + 4 g4 + e] for its rows i
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int qi = i0 + wr0 + 16 * qb + r;
    if (qi < T) {
      TOut* orow = static_cast<TOut*>(p.o) + (((int64_t)b * T + qi) * H + h) * V;
#pragma unroll
      for (int vt = 0; vt < NVT; ++vt) {
        if (vt < nvt) {
          if constexpr (sizeof(TOut) == 4) {
            *reinterpret_cast<f32x4*>(orow + 16 * vt + 4 * g4) = O[qb][vt];
          } else {
            bf16x4 y;
#pragma unroll
            for (int e = 0; e < 4; ++e) y[e] = (bf16)O[qb][vt][e];
            *reinterpret_cast<bf16x4*>(orow + 16 * vt + 4 * g4) = y;
          }
        }
      }
    }
  }

  // zeros right of the tile that holds this wave's diagonal, one row at a time
  {
    const int cz = p.attn != nullptr ? min(T, ((i0 + wr0) / C + 1) * C) : T;
    const bool vec = tlim != 0;
    const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};
    for (int rr = wr0; rr < wr0 + WR && rr < rows && cz < T; ++rr) {
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
hipError_t launch_kv(const ParallelParams& p, hipStream_t stream) {
  constexpr int QR = 64 * row_blocks<K, VMAX>();
  const dim3 grid((uint32_t)unit_grid(p.B, p.Hkv, p.H / p.Hkv, (p.T + QR - 1) / QR));
  if (p.o_f32)
    hipLaunchKernelGGL((parallel_fwd_kernel<K, VMAX, float>), grid, dim3(NTH), 0, stream, p);
  else
    hipLaunchKernelGGL((parallel_fwd_kernel<K, VMAX, bf16>), grid, dim3(NTH), 0, stream, p);
  return hipGetLastError();
}

template <int K>
hipError_t launch_k(const ParallelParams& p, hipStream_t stream) {
  if (p.V <= 64) return launch_kv<K, 64>(p, stream);
  return p.V <= 128 ? launch_kv<K, 128>(p, stream) : launch_kv<K, 256>(p, stream);
}

}  // namespace

hipError_t launch_parallel_fwd(const ParallelParams& p, hipStream_t stream) {
  if (p.B == 0 || p.T == 0) return hipSuccess;
  if (!parallel_supported(p.K, p.V) || p.Hkv <= 0 || p.H % p.Hkv != 0) return hipErrorInvalidValue;
  switch (p.K) {
    case 64: return launch_k<64>(p, stream);
    case 128: return launch_k<128>(p, stream);
    default: return launch_k<256>(p, stream);
  }
}

}  // namespace sgla
