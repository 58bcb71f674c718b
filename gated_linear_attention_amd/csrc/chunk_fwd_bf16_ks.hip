// Steps (2) and (3) of the chunked Simple GLA forward for bf16 q/k/v with a
// large key dimension (K = 256 or 512), fused in one kernel (page
// "flash-linear-attention 中的 Simple GLA", section 一: chunk view with the
// decay-masked q k^T inside a chunk and the scalar-decayed state between
// chunks; section 三: the inter-chunk state pass and the output pass).
//
// Same per-chunk algebra as the K <= 128 kernel (b = chunk-local cumulative
// log2 gate, h_n the K x V state entering chunk n):
//   A      = (Q K^T) (.) M,  M[c][j] = 2^(b_c - b_j) for j <= c, else 0
//   O      = scale * ( A V + diag(2^b) Q h_n )
//   h_n+1  = 2^b_last h_n + K^T (diag(2^(b_last - b)) V)
// All three products are sums over the key dimension split into 128-wide
// slices, so each chunk is processed as K/128 slice steps:
//   step (n, s): stage Q[:, slice s] and K[:, slice s] (64 x 128 each) in LDS;
//                accumulate Q K^T over the slice into the A tiles;
//                accumulate the q.h contribution of the slice's state rows;
//                update those state rows with the slice's K^T.
// A slice's state rows are touched only in its own step, so the q.h term of
// every row still sees h_n.  A V and the output store of chunk n run in the
// first step of chunk n+1.  Staging is double buffered by step, loads run two
// steps ahead, and there is one barrier per step.
//
// Work split (8 waves, two per SIMD; workgroup = (sequence, head, 32-wide V
// tile), so a 512-wide V gives 16 workgroups per (sequence, head)): wave
// w = 2 kr + vc owns state columns [16 vc, +16) of the tile and, in every
// slice, the 32 state rows [32 kr, +32).  Its q.h partials for the four
// 16-token c tiles are summed with those of the three waves sharing its
// columns through LDS; wave (kr, vc) owns output c tile kr.
//
// Precision: fp32 state, accumulation and output; the decay-masked A, the
// state h in q.h and the decayed V in the update are split into bf16 hi + lo
// and each product is issued twice, as in the K <= 128 kernel.
#include <hip/hip_runtime.h>

#include "gate_scan.h"
#include "mfma_common.h"
#include "sgla_internal.h"

namespace sgla {
namespace {

using namespace mf;

constexpr int C = kChunk;        // tokens per chunk
constexpr int VT = 32;           // state / output columns per workgroup
constexpr int KSL = 128;         // key slice per step
constexpr int NW = 8;            // waves
constexpr int NT = 64 * NW;      // threads
constexpr int LDQ = KSL + 8;     // LDS row strides (elements)
constexpr int LDK = KSL + 16;
constexpr int LDV = VT + 16;
constexpr int LDA = C + 8;

struct KsLayout {
  static constexpr int SZ_Q = C * LDQ * 2;
  static constexpr int SZ_K = C * LDK * 2;
  static constexpr int SZ_STEP = SZ_Q + SZ_K;          // one slice of Q and K
  static constexpr int OFF_V = 2 * SZ_STEP;
  static constexpr int SZ_V = C * LDV * 2;
  static constexpr int OFF_G = OFF_V + SZ_V;           // two chunk-parity copies
  static constexpr int SZ_G = 3 * C * 4;               // b, scale 2^b, 2^(b_last - b)
  static constexpr int OFF_A = OFF_G + 2 * SZ_G;
  static constexpr int SZ_A = 2 * C * LDA * 2;         // hi and lo
  static constexpr int OFF_X = OFF_A + SZ_A;
  static constexpr int SZ_X = NW * 3 * 64 * 16;        // three 16x16 fp32 tiles per wave
  static constexpr int BYTES = OFF_X + SZ_X;
  static_assert(BYTES <= 160 * 1024, "LDS budget");
};

template <int K, typename TOut>
__global__ void __launch_bounds__(NT)
chunk_fwd_bf16_ks_kernel(const bf16* __restrict__ q, const bf16* __restrict__ k,
                         const bf16* __restrict__ v, const float* __restrict__ g,
                         const float* __restrict__ g_gamma, const float* __restrict__ h0,
                         TOut* __restrict__ o, float* __restrict__ ht, float scale, int32_t H,
                         int32_t V, SeqLayout seqs) {
  using L = KsLayout;
  constexpr int NSL = K / KSL;        // slice steps per chunk
  static_assert(NSL >= 2, "single-buffered A, V and exchange areas need two steps per chunk");
  __shared__ __attribute__((aligned(16))) char smem[L::BYTES];

  // ---- which (sequence, head, V tile) this workgroup owns ----------------
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
    bos = __builtin_amdgcn_readfirstlane(e.bos);
    len = __builtin_amdgcn_readfirstlane(e.len);
    seq = __builtin_amdgcn_readfirstlane(e.seq);
  } else {
    bos = (int64_t)rank * seqs.T;
    len = seqs.T;
    seq = rank;
  }
  const int nchunks = (len + C - 1) / C;
  const int nsteps = nchunks * NSL;

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int g4 = lane >> 4;
  const int r = lane & 15;
  const int vc = w & 1;           // 16-column group
  const int kr = w >> 1;          // 32-row group within every slice = owned c tile
  const int vcol = vt * VT + 16 * vc + r;
  const int RSK = H * K;
  const int RSV = H * V;
  const bf16* qb = q + (bos * H + hd) * (int64_t)K;
  const bf16* kb = k + (bos * H + hd) * (int64_t)K;
  const bf16* vb = v + (bos * H + hd) * (int64_t)V + vt * VT;
  const float* gb = g != nullptr ? g + bos * H + hd : nullptr;
  TOut* ob = o + (bos * H + hd) * (int64_t)V + vt * VT;
  const uint32_t ocol = (16 * vc + 4 * g4) * (uint32_t)sizeof(TOut);
  const float gam2 = g_gamma != nullptr
                         ? __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(
                                                         __builtin_bit_cast(int, g_gamma[hd]))) * kRcpLn2f
                         : 0.f;

  auto sQ = [&](int p) { return reinterpret_cast<bf16*>(smem + p * L::SZ_STEP); };
  auto sK = [&](int p) { return reinterpret_cast<bf16*>(smem + p * L::SZ_STEP + L::SZ_Q); };
  bf16* sV = reinterpret_cast<bf16*>(smem + L::OFF_V);
  auto sG = [&](int p) { return reinterpret_cast<float*>(smem + L::OFF_G + p * L::SZ_G); };
  bf16* sAh = reinterpret_cast<bf16*>(smem + L::OFF_A);
  bf16* sAl = sAh + C * LDA;
  f32x4* sX = reinterpret_cast<f32x4*>(smem + L::OFF_X);

  // Upper-triangle A tiles are never written: zero the A area once.
  for (int i = tid; i < L::SZ_A / 16; i += NT) reinterpret_cast<uint4*>(sAh)[i] = make_uint4(0, 0, 0, 0);

  // ---- state: h[s][kt][i] = S[128 s + 32 kr + 16 kt + 4 g + i][vcol] -------
  f32x4 h[NSL][2];
  {
    const float* h0u = h0 != nullptr ? h0 + ((int64_t)seq * H + hd) * K * V : nullptr;
#pragma unroll
    for (int s = 0; s < NSL; ++s)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          h[s][kt][i] = h0u != nullptr
                            ? h0u[(int64_t)(KSL * s + 32 * kr + 16 * kt + 4 * g4 + i) * V + vcol]
                            : 0.f;
  }

  // ---- step staging registers ---------------------------------------------
  // step i covers chunk i / NSL, key slice i % NSL; V and g come with slice 0
  struct Stage {
    u32x4 q[2], k[2], v;
    float g;
    int len;   // tokens in the chunk
  };
  auto load_step = [&](int i, Stage& st) {
    const int m = i / NSL;
    const int s = i - m * NSL;
    const int cl = max(0, min(C, len - m * C));
    st.len = cl;
    const int64_t tok = (int64_t)m * C;
    const auto rq = make_rsrc(qb + tok * RSK + s * KSL, (uint32_t)cl * RSK * 2);
    const auto rk = make_rsrc(kb + tok * RSK + s * KSL, (uint32_t)cl * RSK * 2);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int seg = tid + u * NT;                        // 16 segments per 128-wide row
      const uint32_t off = ((seg >> 4) * RSK + (seg & 15) * 8) * 2;
      st.q[u] = __builtin_amdgcn_raw_buffer_load_b128(rq, off, 0, 0);
      st.k[u] = __builtin_amdgcn_raw_buffer_load_b128(rk, off, 0, 0);
    }
    // V tile rows: 4 segments per 32-wide row, threads 0..255 (others read
    // past the descriptor and get zeros without touching memory)
    const auto rv = make_rsrc(vb + tok * RSV, s == 0 ? (uint32_t)cl * RSV * 2 : 0u);
    const uint32_t voff = tid < 256 ? ((tid >> 2) * RSV + (tid & 3) * 8) * 2 : 0xFFFFFFF0u;
    st.v = __builtin_amdgcn_raw_buffer_load_b128(rv, voff, 0, 0);
    st.g = 0.f;
    if (gb != nullptr) {
      const auto rg = make_rsrc(gb + tok * H, s == 0 ? (uint32_t)cl * H * 4 : 0u);
      st.g = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rg, (uint32_t)(lane * H * 4), 0, 0));
    }
  };
  auto store_step = [&](int p, int gp, int s, const Stage& st) {
    bf16* q_s = sQ(p);
    bf16* k_s = sK(p);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int seg = tid + u * NT;
      *reinterpret_cast<u32x4*>(q_s + (seg >> 4) * LDQ + (seg & 15) * 8) = st.q[u];
      *reinterpret_cast<u32x4*>(k_s + (seg >> 4) * LDK + (seg & 15) * 8) = st.k[u];
    }
    if (s == 0) {
      if (tid < 256) *reinterpret_cast<u32x4*>(sV + (tid >> 2) * LDV + (tid & 3) * 8) = st.v;
      if (w == NW - 1) {
        // step (1): chunk-local cumulative log2 gate b, plus scale * 2^b and
        // 2^(b_last - b)
        float* g_s = sG(gp);
        const float b = gb != nullptr ? wave_cumsum_log2(st.g) : (float)min(lane + 1, st.len) * gam2;
        const float blast = __shfl(b, C - 1, 64);
        g_s[lane] = b;
        g_s[C + lane] = exp2_hw(b) * scale;
        g_s[2 * C + lane] = exp2_hw(blast - b);
      }
    }
  };

  // ---- per-chunk registers --------------------------------------------------
  f32x4 sacc[2];                 // A tiles w and w + 8 (accumulated over slices)
  f32x4 oacc[4];                 // q.h partial, c tiles 0..3
  bf16x8 vf[2], vth[2], vtl[2];  // V and decayed V (hi, lo) fragments of the chunk
  bf16x8 vf_prev[2] = {};
  f32x4 mine = {0.f, 0.f, 0.f, 0.f};
  int prev_m = 0, prev_cl = 0;
  float dall = 1.f;
  const int ti1 = w + 8;         // second A tile (waves 0 and 1 only)

  // A V for the previous chunk's own c tile, then combine with the three
  // partners' q.h partials and store (cl = 0 stores nothing)
  auto finish_prev = [&]() {
    const bf16* arow = sAh + (16 * kr + r) * LDA + 8 * g4;
    {
      const bf16x8 ph = *reinterpret_cast<const bf16x8*>(arow);
      const bf16x8 pl = *reinterpret_cast<const bf16x8*>(arow + C * LDA);
      mine = mfma(vf_prev[0], ph, mine);
      mine = mfma(vf_prev[0], pl, mine);
    }
    if (kr >= 2) {   // c tiles 2 and 3 also see tokens 32..63
      const bf16x8 ph = *reinterpret_cast<const bf16x8*>(arow + 32);
      const bf16x8 pl = *reinterpret_cast<const bf16x8*>(arow + 32 + C * LDA);
      mine = mfma(vf_prev[1], ph, mine);
      mine = mfma(vf_prev[1], pl, mine);
    }
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      const int kp = j < kr ? j : j + 1;                 // partner row group
      const int slot_in_p = kr < kp ? kr : kr - 1;       // its slot for my tile
      mine += sX[((2 * kp + vc) * 3 + slot_in_p) * 64 + lane];
    }
    const auto ro = make_rsrc(ob + (int64_t)prev_m * C * RSV, (uint32_t)prev_cl * RSV * sizeof(TOut));
    store4<TOut>(ro, (uint32_t)(16 * kr + r) * RSV * (uint32_t)sizeof(TOut) + ocol, mine);
  };

  Stage st0, st1;
  load_step(0, st0);
  load_step(1, st1);

  auto step = [&](const int i, const int p, Stage& st) {
    const int m = i / NSL;
    const int s = i - m * NSL;
    const int cl = __builtin_amdgcn_readfirstlane(st.len);
    const int gp = m & 1;
    store_step(p, gp, s, st);
    __syncthreads();   // step i staged
    const float* g_s = sG(gp);
    if (s == 0) {
      finish_prev();
      // this chunk's V fragments vf[t][e] = V[32t + 8g + e][16vc + r] and
      // the decayed V = diag(2^(b_last - b)) V split into hi + lo
#pragma unroll
      for (int t = 0; t < 2; ++t)
        vf[t] = cat(tr_read(sV, LDV, 32 * t + 8 * g4, 16 * vc), tr_read(sV, LDV, 32 * t + 8 * g4 + 4, 16 * vc));
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const f32x4 d0 = *reinterpret_cast<const f32x4*>(g_s + 2 * C + 32 * t + 8 * g4);
        const f32x4 d1 = *reinterpret_cast<const f32x4*>(g_s + 2 * C + 32 * t + 8 * g4 + 4);
        const u32x4 raw = __builtin_bit_cast(u32x4, vf[t]);
        float x[8];
        x[0] = bf_lo(raw[0]) * d0[0];
        x[1] = bf_hi(raw[0]) * d0[1];
        x[2] = bf_lo(raw[1]) * d0[2];
        x[3] = bf_hi(raw[1]) * d0[3];
        x[4] = bf_lo(raw[2]) * d1[0];
        x[5] = bf_hi(raw[2]) * d1[1];
        x[6] = bf_lo(raw[3]) * d1[2];
        x[7] = bf_hi(raw[3]) * d1[3];
        split8(x, vth[t], vtl[t]);
      }
      dall = exp2_hw(g_s[C - 1]);
#pragma unroll
      for (int t = 0; t < 2; ++t) sacc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int t = 0; t < 4; ++t) oacc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    load_step(i + 2, st);
    const bf16* q_s = sQ(p);
    const bf16* k_s = sK(p);

    // ---- A tiles: accumulate this slice of Q K^T -------------------------
    {
      const int ct = tile_c(w), jt = tile_j(w);
#pragma unroll
      for (int u = 0; u < KSL / 32; ++u) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(k_s + (16 * jt + r) * LDK + 32 * u + 8 * g4);
        const bf16x8 b = *reinterpret_cast<const bf16x8*>(q_s + (16 * ct + r) * LDQ + 32 * u + 8 * g4);
        sacc[0] = mfma(a, b, sacc[0]);
      }
    }
    if (ti1 < 10) {
      const int ct = tile_c(ti1), jt = tile_j(ti1);
#pragma unroll
      for (int u = 0; u < KSL / 32; ++u) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(k_s + (16 * jt + r) * LDK + 32 * u + 8 * g4);
        const bf16x8 b = *reinterpret_cast<const bf16x8*>(q_s + (16 * ct + r) * LDQ + 32 * u + 8 * g4);
        sacc[1] = mfma(a, b, sacc[1]);
      }
    }

    // ---- q.h over this slice's 32 own state rows (before their update) ---
    // registers are indexed by compile-time slice numbers only
#pragma unroll
    for (int ss = 0; ss < NSL; ++ss) {
      if (ss != s) continue;
      float x[8];
#pragma unroll
      for (int i2 = 0; i2 < 4; ++i2) {
        x[i2] = h[ss][0][i2];
        x[4 + i2] = h[ss][1][i2];
      }
      bf16x8 hh, hl;
      split8(x, hh, hl);
      bf16x8 b[4];
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        const bf16* qrow = q_s + (16 * ct + r) * LDQ + 32 * kr + 4 * g4;
        b[ct] = cat(*reinterpret_cast<const bf16x4*>(qrow), *reinterpret_cast<const bf16x4*>(qrow + 16));
      }
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) oacc[ct] = mfma(hh, b[ct], oacc[ct]);
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) oacc[ct] = mfma(hl, b[ct], oacc[ct]);

      // ---- state rows of this slice: h <- 2^b_last h + K^T Vdecayed -------
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) h[ss][kt] *= dall;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        bf16x8 a[2];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
          a[kt] = cat(tr_read(k_s, LDK, 32 * t + 8 * g4, 32 * kr + 16 * kt),
                      tr_read(k_s, LDK, 32 * t + 8 * g4 + 4, 32 * kr + 16 * kt));
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) h[ss][kt] = mfma(a[kt], vth[t], h[ss][kt]);
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) h[ss][kt] = mfma(a[kt], vtl[t], h[ss][kt]);
      }
    }

    if (s == NSL - 1) {
      // ---- end of chunk m: A tiles to LDS, q.h partials to the partners ---
      auto emit_A = [&](int ti, f32x4 acc) {
        const int ct = tile_c(ti), jt = tile_j(ti);
        const int c = 16 * ct + r;
        const float bc = g_s[c];
        const f32x4 bj = *reinterpret_cast<const f32x4*>(g_s + 16 * jt + 4 * g4);
        float x[4];
#pragma unroll
        for (int i2 = 0; i2 < 4; ++i2) {
          const int j = 16 * jt + 4 * g4 + i2;
          x[i2] = (j <= c) ? acc[i2] * exp2_hw(bc - bj[i2]) * scale : 0.f;
        }
        uint32_t h0w, l0w, h1w, l1w;
        split2(x[0], x[1], h0w, l0w);
        split2(x[2], x[3], h1w, l1w);
        *reinterpret_cast<u32x2*>(sAh + c * LDA + 16 * jt + 4 * g4) = u32x2{h0w, h1w};
        *reinterpret_cast<u32x2*>(sAl + c * LDA + 16 * jt + 4 * g4) = u32x2{l0w, l1w};
      };
      emit_A(w, sacc[0]);
      if (ti1 < 10) emit_A(ti1, sacc[1]);
      // scale * diag(2^b) on the q.h partials (O^T column c = 16 ct + r)
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) oacc[ct] *= g_s[C + 16 * ct + r];
#pragma unroll
      for (int j = 0; j < 3; ++j) {
        const int ct = j < kr ? j : j + 1;
        f32x4 val = oacc[0];
        val = ct == 1 ? oacc[1] : val;
        val = ct == 2 ? oacc[2] : val;
        val = ct == 3 ? oacc[3] : val;
        sX[(w * 3 + j) * 64 + lane] = val;
      }
      f32x4 own = oacc[0];
      own = kr == 1 ? oacc[1] : own;
      own = kr == 2 ? oacc[2] : own;
      own = kr == 3 ? oacc[3] : own;
      mine = own;
      vf_prev[0] = vf[0];
      vf_prev[1] = vf[1];
      prev_m = m;
      prev_cl = cl;
    }
  };

  int i = 0;
  for (; i + 1 < nsteps; i += 2) {
    step(i, 0, st0);
    step(i + 1, 1, st1);
  }
  if (i < nsteps) step(i, 0, st0);
  __syncthreads();
  if (nchunks > 0) finish_prev();

  if (ht != nullptr) {
    float* htu = ht + ((int64_t)seq * H + hd) * K * V;
#pragma unroll
    for (int s = 0; s < NSL; ++s)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i2 = 0; i2 < 4; ++i2)
          htu[(int64_t)(KSL * s + 32 * kr + 16 * kt + 4 * g4 + i2) * V + vcol] = h[s][kt][i2];
  }
}

template <int K, typename TOut>
hipError_t launch_k(const ChunkFwdParams& p, hipStream_t stream) {
  const int num_units = p.seqs.num_seqs * p.H;
  if (num_units == 0) return hipSuccess;
  const int nvt = p.V / VT;
  const int groups = (num_units + kXcds - 1) / kXcds;
  const dim3 grid((unsigned)(groups * kXcds * nvt));
  hipLaunchKernelGGL((chunk_fwd_bf16_ks_kernel<K, TOut>), grid, dim3(NT), 0, stream,
                     static_cast<const bf16*>(p.q), static_cast<const bf16*>(p.k),
                     static_cast<const bf16*>(p.v), p.g, p.g_gamma, p.h0, static_cast<TOut*>(p.o),
                     p.ht, p.scale, p.H, p.V, p.seqs);
  return hipGetLastError();
}

template <typename TOut>
hipError_t launch_out(const ChunkFwdParams& p, hipStream_t stream) {
  switch (p.K) {
    case 256: return launch_k<256, TOut>(p, stream);
    case 512: return launch_k<512, TOut>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_chunk_fwd_bf16_ks(const ChunkFwdParams& p, hipStream_t stream) {
  return p.o_bf16 ? launch_out<__bf16>(p, stream) : launch_out<float>(p, stream);
}

}  // namespace sgla
