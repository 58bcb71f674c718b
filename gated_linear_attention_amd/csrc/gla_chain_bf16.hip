// Chunk chain of elementwise-gate GLA on the bf16 matrix cores (page
// "flash-linear-attention 中的 Simple GLA", section 一: the elementwise gate
// decays every state element on its own; section 三: the state pass and the
// output pass), for bf16 inputs with K in {64, 128}.  It reads the records
// the preparation kernel (gla_chunk_fwd.hip) wrote for every (chunk, query
// head), with B the chunk-local cumulative log2 gate of each key:
//   q~ = scale q (.) 2^B,   k~ = k (.) 2^(B_last - B)     bf16 hi + lo planes
//   A  = the decay-masked, scaled intra-chunk matrix      bf16 hi + lo planes
//   d  = 2^B_last per key                                  float32
// and per chunk, with h the K x V state entering it (fp32):
//   O      = q~ h + A V
//   h_n+1  = diag(d) h + k~^T V
// Every factor 2^(...) is <= 1 for non-positive gates.
//
// Work layout as the head-wise bf16 kernel for K <= 128: one workgroup of 8
// waves (two per SIMD) per (sequence, head, 64-wide V tile); wave w owns
// state columns [16 (w % 4), +16) of the tile and state rows [(w / 4) K/2,
// +K/2) as 16 x 16 MFMA accumulators (v_mfma_f32_16x16x32_bf16) for the
// whole sequence.  Each wave forms q~ h over its K/2 rows for all 64 tokens;
// the two halves meet through LDS, each wave finishing two of the four
// 16-token output tiles (with A V added).  One chunk's records are staged in
// LDS, the next chunk's are loaded into registers while this one computes.
//
// Precision: q~ h is issued as hi.hi + lo.hi + hi.lo (q~ and h both split,
// the lo.lo term, 2^-16 of the product, dropped); A V and k~^T V as hi + lo
// against the exact bf16 V.  State, accumulation and output are fp32.
#include <hip/hip_runtime.h>

#include "mfma_common.h"
#include "sgla_internal.h"
#include "unit_map.h"

namespace sgla {
namespace {

using namespace mf;

constexpr int C = kChunk;
constexpr int VT = 64;          // state / output columns per workgroup
constexpr int NW = 8;           // waves
constexpr int NT = 64 * NW;     // threads
constexpr int LDV = VT + 16;    // V tile row stride (elements)
constexpr int LDA = C + 8;      // A row stride (elements)

template <int K>
struct ChainLayout {
  static constexpr int LDQ = K + 8;            // q~ row stride (elements)
  static constexpr int LDK = K + 16;           // k~ row stride (elements)
  static constexpr int OFF_Q = 0;              // q~ hi plane, then lo plane
  static constexpr int SZ_Q = 2 * C * LDQ * 2;
  static constexpr int OFF_K = OFF_Q + SZ_Q;   // k~ hi, lo
  static constexpr int SZ_K = 2 * C * LDK * 2;
  static constexpr int OFF_A = OFF_K + SZ_K;   // A hi, lo
  static constexpr int SZ_A = 2 * C * LDA * 2;
  static constexpr int OFF_V = OFF_A + SZ_A;   // V tile
  static constexpr int SZ_V = C * LDV * 2;
  static constexpr int OFF_D = OFF_V + SZ_V;   // per-key decay d
  static constexpr int SZ_D = K * 4;
  static constexpr int OFF_X = OFF_D + SZ_D;   // q~ h partials exchanged between row halves
  static constexpr int SZ_X = NW * 2 * 64 * 16;
  static constexpr int BYTES = OFF_X + SZ_X;
  static_assert(BYTES <= 160 * 1024, "LDS budget");
  static_assert(OFF_K % 16 == 0 && OFF_A % 16 == 0 && OFF_V % 16 == 0 && OFF_D % 16 == 0 &&
                    OFF_X % 16 == 0,
                "16-byte aligned areas");
};

template <int K, typename TOut>
__global__ void __launch_bounds__(NT)
gla_chain_bf16_kernel(const bf16* __restrict__ v, const bf16* __restrict__ qk_hl,
                      const bf16* __restrict__ a_hl, const float* __restrict__ dl,
                      const float* __restrict__ h0, TOut* __restrict__ o, float* __restrict__ ht,
                      int32_t H, int32_t Hkv, int32_t V, StateLayout sl, SeqLayout seqs) {
  using L = ChainLayout<K>;
  constexpr int KH = K / 2;              // state rows per wave
  constexpr int KT = KH / 16;            // 16-row state tiles per wave
  constexpr int KS = KH / 32;            // 32-deep steps over a wave's rows
  constexpr int SEGQ = K / 8;            // 16-byte pieces per q~ / k~ row
  constexpr int PQ = 2 * C * SEGQ;       // pieces of q~ (both planes); k~ alike
  constexpr int NQ = PQ / NT;
  constexpr int PA = 2 * C * (C / 8);    // pieces of A (both planes)
  constexpr int NA = PA / NT;
  constexpr int PV = C * (VT / 8);       // pieces of the V tile
  constexpr int NV = PV / NT;
  static_assert(NQ * NT == PQ && NA * NT == PA && NV * NT == PV, "staging split");
  static_assert(KS >= 1 && K / 4 <= NT, "K");
  __shared__ __attribute__((aligned(16))) char smem[L::BYTES];
  bf16* const sQ = reinterpret_cast<bf16*>(smem + L::OFF_Q);
  bf16* const sK = reinterpret_cast<bf16*>(smem + L::OFF_K);
  bf16* const sA = reinterpret_cast<bf16*>(smem + L::OFF_A);
  bf16* const sV = reinterpret_cast<bf16*>(smem + L::OFF_V);
  float* const sD = reinterpret_cast<float*>(smem + L::OFF_D);
  f32x4* const sX = reinterpret_cast<f32x4*>(smem + L::OFF_X);

  // ---- which (sequence, head, V tile) this workgroup owns ----------------
  const UnitMap um = map_unit(blockIdx.x, V / VT, Hkv, H / Hkv, seqs.num_seqs);
  if (!um.valid) return;
  const int hd = um.hd, hk = um.hk, vt = um.vt;
  int64_t bos;
  int32_t len, seq, chunk0;
  if (seqs.seq_table != nullptr) {
    const SeqEntry e = seqs.seq_table[um.rank];
    bos = __builtin_amdgcn_readfirstlane(e.bos);
    len = __builtin_amdgcn_readfirstlane(e.len);
    seq = __builtin_amdgcn_readfirstlane(e.seq);
    chunk0 = __builtin_amdgcn_readfirstlane(e.chunk0);
  } else {
    bos = (int64_t)um.rank * seqs.T;
    len = seqs.T;
    seq = um.rank;
    chunk0 = um.rank * ((seqs.T + seqs.chunk - 1) / seqs.chunk);
  }
  const int nchunks = (len + seqs.chunk - 1) / seqs.chunk;

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int g4 = lane >> 4;
  const int r = lane & 15;
  const int kh = w >> 2;                    // state row half
  const int vc = w & 3;                     // 16-column group
  const int krow0 = kh * KH;
  const int vcol = vt * VT + 16 * vc + r;   // this lane's state column
  const int own0 = kh == 0 ? 0 : 1;         // output tiles this wave finishes
  const int own1 = kh == 0 ? 3 : 2;
  // output tiles in q~ h order: this wave's two, then its partner's (w ^ 4)
  const int ctile[4] = {own0, own1, kh == 0 ? 1 : 0, kh == 0 ? 2 : 3};
  const int64_t RSV = (int64_t)Hkv * V;     // token stride of v
  const int RSO = H * V;                    // token stride of o
  const bf16* vb = v + (bos * Hkv + hk) * (int64_t)V + vt * VT;
  TOut* ob = o + (bos * H + hd) * (int64_t)V + vt * VT;
  const uint32_t ocol = (16 * vc + 4 * g4) * (uint32_t)sizeof(TOut);

  // ---- state: h[kt][i] = S[krow0 + 16 kt + 4 g + i][vcol] ------------------
  f32x4 h[KT];
  {
    const float* h0u = h0 != nullptr ? h0 + ((int64_t)seq * H + hd) * K * V : nullptr;
#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        h[kt][i] = h0u != nullptr
                       ? h0u[(int64_t)(krow0 + 16 * kt + 4 * g4 + i) * sl.rs + (int64_t)vcol * sl.cs]
                       : 0.f;
  }

  // ---- chunk records: registers, then LDS ---------------------------------
  struct Stage {
    u32x4 q[NQ], k[NQ], a[NA], v[NV], d;
  };
  const u32x4 zero4 = {0u, 0u, 0u, 0u};
  auto load_chunk = [&](int m, Stage& st) {
    const int64_t rec = (int64_t)(chunk0 + m) * H + hd;
    const bf16* qrec = qk_hl + rec * (4 * C * K);
    const bf16* krec = qrec + 2 * C * K;
    const bf16* arec = a_hl + rec * (2 * C * C);
#pragma unroll
    for (int u = 0; u < NQ; ++u) {
      const int p = tid + NT * u;
      st.q[u] = *reinterpret_cast<const u32x4*>(qrec + 8 * p);
      st.k[u] = *reinterpret_cast<const u32x4*>(krec + 8 * p);
    }
#pragma unroll
    for (int u = 0; u < NA; ++u) st.a[u] = *reinterpret_cast<const u32x4*>(arec + 8 * (tid + NT * u));
    const int cl = min(seqs.chunk, len - m * seqs.chunk);
#pragma unroll
    for (int u = 0; u < NV; ++u) {
      const int p = tid + NT * u;
      const int row = p / (VT / 8), seg = p % (VT / 8);
      st.v[u] = row < cl ? *reinterpret_cast<const u32x4*>(vb + ((int64_t)m * seqs.chunk + row) * RSV + 8 * seg) : zero4;
    }
    st.d = tid < K / 4 ? *reinterpret_cast<const u32x4*>(dl + rec * K + 4 * tid) : zero4;
  };
  auto store_chunk = [&](const Stage& st) {
#pragma unroll
    for (int u = 0; u < NQ; ++u) {
      const int p = tid + NT * u;
      const int plane = p / (C * SEGQ), rem = p % (C * SEGQ);
      const int row = rem / SEGQ, seg = rem % SEGQ;
      *reinterpret_cast<u32x4*>(sQ + (plane * C + row) * L::LDQ + 8 * seg) = st.q[u];
      *reinterpret_cast<u32x4*>(sK + (plane * C + row) * L::LDK + 8 * seg) = st.k[u];
    }
#pragma unroll
    for (int u = 0; u < NA; ++u) {
      const int p = tid + NT * u;
      const int plane = p / (C * C / 8), rem = p % (C * C / 8);
      *reinterpret_cast<u32x4*>(sA + (plane * C + rem / 8) * LDA + 8 * (rem % 8)) = st.a[u];
    }
#pragma unroll
    for (int u = 0; u < NV; ++u) {
      const int p = tid + NT * u;
      *reinterpret_cast<u32x4*>(sV + (p / (VT / 8)) * LDV + 8 * (p % (VT / 8))) = st.v[u];
    }
    if (tid < K / 4) *reinterpret_cast<u32x4*>(sD + 4 * tid) = st.d;
  };

  Stage st;
  if (nchunks > 0) load_chunk(0, st);
  for (int m = 0; m < nchunks; ++m) {
    const int cl = min(seqs.chunk, len - m * seqs.chunk);
    store_chunk(st);
    __syncthreads();   // chunk m staged; the previous chunk's exchange tiles read
    if (m + 1 < nchunks) load_chunk(m + 1, st);

    // ---- q~ h over this wave's K/2 state rows, the four output tiles -------
    f32x4 oacc[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) oacc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      // A operand from the state: rows krow0 + 32 s + 4 g + {0..3} and
      // krow0 + 32 s + 16 + 4 g + {0..3}; q~ is read in the same key order
      float x[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[i] = h[2 * s][i];
        x[4 + i] = h[2 * s + 1][i];
      }
      bf16x8 hh, hl;
      split8(x, hh, hl);
      bf16x8 bh[4], bl[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const bf16* qrow = sQ + (16 * ctile[t] + r) * L::LDQ + krow0 + 32 * s + 4 * g4;
        bh[t] = cat(*reinterpret_cast<const bf16x4*>(qrow), *reinterpret_cast<const bf16x4*>(qrow + 16));
        bl[t] = cat(*reinterpret_cast<const bf16x4*>(qrow + C * L::LDQ),
                    *reinterpret_cast<const bf16x4*>(qrow + C * L::LDQ + 16));
      }
#pragma unroll
      for (int t = 0; t < 4; ++t) oacc[t] = mfma(hh, bh[t], oacc[t]);
#pragma unroll
      for (int t = 0; t < 4; ++t) oacc[t] = mfma(hl, bh[t], oacc[t]);
#pragma unroll
      for (int t = 0; t < 4; ++t) oacc[t] = mfma(hh, bl[t], oacc[t]);
    }
    // the partner's two tiles go through LDS
    sX[(w * 2 + 0) * 64 + lane] = oacc[2];
    sX[(w * 2 + 1) * 64 + lane] = oacc[3];

    // ---- V fragments vf[s][e] = V[32 s + 8 g + e][16 vc + r] ---------------
    bf16x8 vf[2];
#pragma unroll
    for (int s = 0; s < 2; ++s)
      vf[s] = cat(tr_read(sV, LDV, 32 * s + 8 * g4, 16 * vc), tr_read(sV, LDV, 32 * s + 8 * g4 + 4, 16 * vc));

    // ---- A V for this wave's own tiles: own0 needs tokens j < 32, own1 all --
    f32x4 mine0 = oacc[0], mine1 = oacc[1];
    {
      const bf16* ah0 = sA + (16 * own0 + r) * LDA + 8 * g4;
      const bf16* ah1 = sA + (16 * own1 + r) * LDA + 8 * g4;
      const bf16x8 p0h = *reinterpret_cast<const bf16x8*>(ah0);
      const bf16x8 p0l = *reinterpret_cast<const bf16x8*>(ah0 + C * LDA);
      const bf16x8 p1h = *reinterpret_cast<const bf16x8*>(ah1);
      const bf16x8 p1l = *reinterpret_cast<const bf16x8*>(ah1 + C * LDA);
      const bf16x8 p2h = *reinterpret_cast<const bf16x8*>(ah1 + 32);
      const bf16x8 p2l = *reinterpret_cast<const bf16x8*>(ah1 + 32 + C * LDA);
      mine0 = mfma(vf[0], p0h, mine0);
      mine1 = mfma(vf[0], p1h, mine1);
      mine0 = mfma(vf[0], p0l, mine0);
      mine1 = mfma(vf[0], p1l, mine1);
      mine1 = mfma(vf[1], p2h, mine1);
      mine1 = mfma(vf[1], p2l, mine1);
    }

    // ---- h <- diag(d) h + k~^T V for this wave's rows ----------------------
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) h[kt] *= *reinterpret_cast<const f32x4*>(sD + krow0 + 16 * kt + 4 * g4);
    constexpr int KG = KT < 4 ? KT : 4;   // state tiles per MFMA group
#pragma unroll
    for (int s = 0; s < 2; ++s) {
#pragma unroll
      for (int k0 = 0; k0 < KT; k0 += KG) {
        // A operands: k~^T[krow0 + 16 kt + r][32 s + 8 g + e], hi and lo planes
        bf16x8 ah[KG], al[KG];
#pragma unroll
        for (int u = 0; u < KG; ++u) {
          const int col = krow0 + 16 * (k0 + u);
          ah[u] = cat(tr_read(sK, L::LDK, 32 * s + 8 * g4, col), tr_read(sK, L::LDK, 32 * s + 8 * g4 + 4, col));
          al[u] = cat(tr_read(sK + C * L::LDK, L::LDK, 32 * s + 8 * g4, col),
                      tr_read(sK + C * L::LDK, L::LDK, 32 * s + 8 * g4 + 4, col));
        }
#pragma unroll
        for (int u = 0; u < KG; ++u) h[k0 + u] = mfma(ah[u], vf[s], h[k0 + u]);
#pragma unroll
        for (int u = 0; u < KG; ++u) h[k0 + u] = mfma(al[u], vf[s], h[k0 + u]);
      }
    }
    __syncthreads();   // exchange tiles visible; every read of this chunk's stage done

    // ---- own tiles + partner's partial, stored (rows past the chunk's end
    //      fall outside the descriptor and are dropped) ---------------------
    {
      const f32x4 x0 = sX[((w ^ 4) * 2 + 0) * 64 + lane];
      const f32x4 x1 = sX[((w ^ 4) * 2 + 1) * 64 + lane];
      const auto ro = make_rsrc(ob + (int64_t)m * seqs.chunk * RSO, (uint32_t)cl * RSO * (uint32_t)sizeof(TOut));
      const uint32_t c0 = 16 * own0 + r, c1 = 16 * own1 + r;
      store4<TOut>(ro, c0 * RSO * (uint32_t)sizeof(TOut) + ocol, mine0 + x0);
      store4<TOut>(ro, c1 * RSO * (uint32_t)sizeof(TOut) + ocol, mine1 + x1);
    }
  }

  if (ht != nullptr) {
    float* htu = ht + ((int64_t)seq * H + hd) * K * V;
#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        htu[(int64_t)(krow0 + 16 * kt + 4 * g4 + i) * sl.rs + (int64_t)vcol * sl.cs] = h[kt][i];
  }
}

template <int K, typename TOut>
hipError_t launch_k(const GlaFwdParams& p, hipStream_t stream) {
  if (p.seqs.num_seqs == 0) return hipSuccess;
  const dim3 grid((unsigned)unit_grid(p.seqs.num_seqs, p.Hkv, p.H / p.Hkv, p.V / VT));
  hipLaunchKernelGGL((gla_chain_bf16_kernel<K, TOut>), grid, dim3(NT), 0, stream,
                     static_cast<const bf16*>(p.v), static_cast<const bf16*>(p.qk_hl),
                     static_cast<const bf16*>(p.a_hl), p.dl, p.h0, static_cast<TOut*>(p.o), p.ht, p.H,
                     p.Hkv, p.V, p.sl, p.seqs);
  return hipGetLastError();
}

template <typename TOut>
hipError_t launch_out(const GlaFwdParams& p, hipStream_t stream) {
  switch (p.K) {
    case 64: return launch_k<64, TOut>(p, stream);
    case 128: return launch_k<128, TOut>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_gla_chain_bf16(const GlaFwdParams& p, hipStream_t stream) {
  if (!gla_bf16_chain(p.qkv_bf16 != 0, p.K, p.V)) return hipErrorInvalidValue;
  return p.o_bf16 ? launch_out<__bf16>(p, stream) : launch_out<float>(p, stream);
}

}  // namespace sgla
