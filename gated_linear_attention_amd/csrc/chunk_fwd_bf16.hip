// Steps (2) and (3) of the chunked Simple GLA forward for bf16 q/k/v, fused in
// one kernel (page "flash-linear-attention 中的 Simple GLA", section 一: the
// chunk view with a decay-masked q k^T inside a chunk and a scalar-decayed
// state between chunks; section 三: the inter-chunk state pass and the output
// pass, which with a head-wise gate are plain matrix products).
//
// For chunk n of one (sequence, head), with b the chunk-local cumulative log2
// gate of step (1) -- formed in each chunk's prologue by a wave scan, so the
// whole forward is a single launch -- b_last = b at the chunk's last token, and h_n the K x V
// state entering the chunk:
//
//   A      = (Q K^T) (.) M,  M[c][j] = 2^(b_c - b_j) for j <= c, else 0
//   O      = scale * ( A V + diag(2^b) Q h_n )
//   h_n+1  = 2^b_last h_n + K^T (diag(2^(b_last - b)) V)
//
// The mask is applied to the exponent before exp2, so no factor ever exceeds
// 1 for non-positive gates (the reason the page gives for the head-wise gate
// being numerically stable).
//
// Layout of the work (gfx950, wave64, v_mfma_f32_16x16x32_bf16):
//   * one workgroup of 8 waves per (unit, head, 64-wide V tile), where a unit
//     is a whole sequence or, for segmented chains, a bin of sequence pieces
//     processed one after another (each piece from its own entering state:
//     the sequence's initial state or the record the segment state pass
//     wrote); the workgroups of one (unit, kv head) share an XCD so repeated
//     reads of its q, k and v rows (other V tiles, other query heads of a kv
//     group) are served by that XCD's L2;
//   * the state lives in MFMA accumulator registers (fp32), split over the
//     waves as described at Layout below, carried across chunks without ever
//     leaving the chip -- only the final state is written;
//   * each chunk's Q, K (64 x K) and V tile (64 x 64) are staged in LDS
//     row-major; the operands that need the token index contiguous per lane
//     (K^T and V as MFMA operands reduced over tokens) are fetched with the
//     gfx950 transposing LDS read ds_read_b64_tr_b16;
//   * staging is double-buffered in LDS with one barrier per chunk, the rows
//     of chunk m + 1 loading into registers while chunk m computes;
//   * the phases of a chunk step are independent of one another: the two
//     waves that share a SIMD (kh = 0 and kh = 1) take them in different
//     orders (A first or last), so that one of them forms A while the other
//     runs its q.h and state-update products, and every wave issues other
//     products before it waits for a product's result (the step is a latency
//     chain; where a wave stalls decides its length).
//
// Precision: the state, the accumulation and the output are fp32.  The three
// MFMA operands that are not exact bf16 inputs -- the decay-masked A, the
// state h used in Q h, and the decayed V used in the state update -- are split
// as x = hi + lo with hi = bf16(x), lo = bf16(x - hi), and each product is
// issued twice (hi and lo), keeping ~16 significant bits for those operands.
#include <hip/hip_runtime.h>

#include "gate_scan.h"
#include "mfma_common.h"
#include "sgla_internal.h"
#include "unit_map.h"

namespace sgla {
namespace {

constexpr int C = kChunk;  // 64 tokens per chunk
constexpr int VT = 64;     // state / output columns per workgroup
constexpr int LDV = VT + 16;  // V tile row stride (elements)
constexpr int LDA = C + 8;    // A tile row stride (elements)
constexpr float kRcpLn2f = mf::kRcpLn2f;
using namespace mf;

// Work split inside a workgroup (8 waves, two per SIMD): wave w owns state
// columns [16*(w%4), +16) of the workgroup's V tile and state rows
// [kh*K/2, +K/2) with kh = w/4.  Each wave forms the q.h contribution of its
// own K/2 rows for all 64 tokens; the two halves are summed through LDS.  The
// output rows are split between the two waves of a column group (c tiles
// {0,3} for kh = 0, {1,2} for kh = 1, which also balances the causal A V work).
template <int K>
struct Layout {
  static constexpr int NW = 8;
  static constexpr int NT = 64 * NW;
  static constexpr int KH = K / 2;            // state rows per wave
  static constexpr int KT = KH / 16;          // 16-row state tiles per wave
  static constexpr int KS = KH / 32;          // 32-deep steps over a wave's rows
  static constexpr int KSF = K / 32;          // 32-deep steps over all K
  static constexpr int NBUF = 2;              // double-buffered chunk staging
  static constexpr int LDQ = K + 8;           // row strides in elements; padding
  static constexpr int LDK = K + 16;          // keeps the 16-byte and transposing
  static constexpr int SZ_Q = C * LDQ * 2;    // reads free of bank conflicts
  static constexpr int SZ_K = C * LDK * 2;
  static constexpr int SZ_V = C * LDV * 2;
  static constexpr int SZ_G = 3 * C * 4;      // b, 2^b, 2^(b_last - b)
  static constexpr int SZ_A = 2 * C * LDA * 2;   // hi and lo
  static constexpr int SZ_STAGE = SZ_Q + SZ_K + SZ_V + SZ_G + SZ_A;
  static constexpr int SZ_X = NW * 2 * 64 * 16;  // two 16x16 fp32 tiles per wave
  static constexpr int OFF_X = NBUF * SZ_STAGE;   // one exchange area per chunk parity
  static constexpr int BYTES = NBUF * SZ_STAGE + 2 * SZ_X;
  static_assert(BYTES <= 160 * 1024, "LDS budget");
};

template <int K, typename TOut>
__global__ void __launch_bounds__(Layout<K>::NT)
chunk_fwd_bf16_kernel(const bf16* __restrict__ q, const bf16* __restrict__ k,
                      const bf16* __restrict__ v, const float* __restrict__ g,
                      const float* __restrict__ g_gamma, const float* __restrict__ h0,
                      TOut* __restrict__ o, float* __restrict__ ht, float scale, int32_t H,
                      int32_t Hkv, int32_t V, StateLayout sl, SeqLayout seqs,
                      const SegEntry* __restrict__ segs, const BinEntry* __restrict__ bins, int32_t num_bins,
                      const float* __restrict__ sin) {
  using L = Layout<K>;
  constexpr int NT = L::NT;
  constexpr int SEG = K / 8;                 // 16-byte segments per q/k row
  constexpr int NQ = C * SEG / NT;           // q (and k) segments per thread
  constexpr int NV = C * (VT / 8) / NT;      // v segments per thread
  static_assert(NQ * NT == C * SEG && NV * NT == C * (VT / 8), "load split");

  __shared__ __attribute__((aligned(16))) char smem[L::BYTES];

  // ---- which (sequence or bin of segments, head, V tile) this workgroup owns
  const UnitMap um = map_unit(blockIdx.x, V / VT, Hkv, H / Hkv, segs != nullptr ? num_bins : seqs.num_seqs);
  if (!um.valid) return;
  const int rank = um.rank, hd = um.hd, hk = um.hk, vt = um.vt;


  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int g4 = lane >> 4;   // 16-lane group 0..3
  const int r = lane & 15;
  const int kh = w >> 2;      // state row half
  const int vc = w & 3;       // 16-column group
  const int krow0 = kh * L::KH;
  const int vcol = vt * VT + 16 * vc + r;   // this lane's state column
  const int own0 = kh == 0 ? 0 : 1;         // output c tiles owned by this wave
  const int own1 = kh == 0 ? 3 : 2;
  // c tiles in q.h order: this wave's two, then its partner's (w ^ 4) two
  const int ctile[4] = {own0, own1, kh == 0 ? 1 : 0, kh == 0 ? 2 : 3};
  const int RSQ = H * K;                    // token stride of q (elements)
  const int RSK = Hkv * K;                  // token stride of k
  const int RSV = Hkv * V;                  // token stride of v
  const int RSO = H * V;                    // token stride of o
  const uint32_t ocol = (16 * vc + 4 * g4) * (uint32_t)sizeof(TOut);   // lane's 4 columns
  const float gam2 = g_gamma != nullptr
                         ? __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(
                                                         __builtin_bit_cast(int, g_gamma[hd]))) * kRcpLn2f
                         : 0.f;

  auto sQ = [&](int p) { return reinterpret_cast<bf16*>(smem + p * L::SZ_STAGE); };
  auto sK = [&](int p) { return reinterpret_cast<bf16*>(smem + p * L::SZ_STAGE + L::SZ_Q); };
  auto sV = [&](int p) {
    return reinterpret_cast<bf16*>(smem + p * L::SZ_STAGE + L::SZ_Q + L::SZ_K);
  };
  auto sG = [&](int p) {
    return reinterpret_cast<float*>(smem + p * L::SZ_STAGE + L::SZ_Q + L::SZ_K + L::SZ_V);
  };
  auto sA = [&](int p) {
    return reinterpret_cast<bf16*>(smem + p * L::SZ_STAGE + L::SZ_Q + L::SZ_K + L::SZ_V + L::SZ_G);
  };
  auto sX = [&](int p) { return reinterpret_cast<f32x4*>(smem + L::OFF_X + p * L::SZ_X); };

  // Upper-triangle A tiles are never written: zero the A buffers once.
  for (int p = 0; p < L::NBUF; ++p)
    for (int i = tid; i < L::SZ_A / 16; i += NT)
      reinterpret_cast<uint4*>(sA(p))[i] = make_uint4(0, 0, 0, 0);

  // One unit (a sequence, or each segment of this workgroup's bin in turn).
  // A unit's first barrier orders every LDS access of the previous unit
  // before its own writes of the A and exchange buffers.
  int32_t seg0 = 0, nunits = 1;
  if (segs != nullptr) {
    const BinEntry be = bins[rank];
    seg0 = __builtin_amdgcn_readfirstlane(be.first);
    nunits = __builtin_amdgcn_readfirstlane(be.count);
  }
  for (int32_t u = 0; u < nunits; ++u) {
    int64_t bos;
    int32_t len, seq;
    int32_t init = -1;      // segment entering-state record (-1: the sequence's initial state)
    bool last = true;       // writes the final state
    // workgroup-uniform: kept in scalar registers so buffer descriptors built
    // from them stay scalar
    if (segs != nullptr) {
      const SegEntry e = segs[seg0 + u];
      bos = __builtin_amdgcn_readfirstlane(e.bos);
      len = __builtin_amdgcn_readfirstlane(e.len);
      seq = __builtin_amdgcn_readfirstlane(e.seq);
      init = __builtin_amdgcn_readfirstlane(e.init);
      last = __builtin_amdgcn_readfirstlane(e.last) != 0;
    } else if (seqs.seq_table != nullptr) {
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
    const bf16* qb = q + (bos * H + hd) * (int64_t)K;
    const bf16* kb = k + (bos * Hkv + hk) * (int64_t)K;
    const bf16* vb = v + (bos * Hkv + hk) * (int64_t)V + vt * VT;
    const float* gb = g != nullptr ? g + bos * H + hd : nullptr;
    TOut* ob = o + (bos * H + hd) * (int64_t)V + vt * VT;     // workgroup-uniform base

    // ---- state in registers: h[kt][i] = S[krow0 + 16kt + 4g + i][vcol] ------
    f32x4 h[L::KT];
    {
      // a later segment starts from its entering-state record ([K][V] rows);
      // the first from the sequence's initial state (layout sl) or zeros
      const float* h0u = init >= 0 ? sin + ((int64_t)init * H + hd) * K * V
                                   : (h0 != nullptr ? h0 + ((int64_t)seq * H + hd) * K * V : nullptr);
      const int64_t rs = init >= 0 ? V : sl.rs, cs = init >= 0 ? 1 : sl.cs;
#pragma unroll
      for (int kt = 0; kt < L::KT; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          h[kt][i] = h0u != nullptr ? h0u[(int64_t)(krow0 + 16 * kt + 4 * g4 + i) * rs + (int64_t)vcol * cs] : 0.f;
    }

    // ---- chunk staging registers -------------------------------------------
    struct Stage {
      u32x4 q[NQ], k[NQ], v[NV];
      float g;
      int len;
    };
    // Loads chunk m (zeros past the sequence's end) into st; every thread issues
    // the same instructions whatever m is.
    auto load_chunk = [&](int m, Stage& st) {
      const int cl = max(0, min(C, len - m * C));
      st.len = cl;
      const int64_t tok = (int64_t)m * C;
      const auto rq = make_rsrc(qb + tok * RSQ, (uint32_t)cl * RSQ * 2);
      const auto rk = make_rsrc(kb + tok * RSK, (uint32_t)cl * RSK * 2);
      const auto rv = make_rsrc(vb + tok * RSV, (uint32_t)cl * RSV * 2);
#pragma unroll
      for (int i = 0; i < NQ; ++i) {
        const int s = tid + i * NT;
        st.q[i] = __builtin_amdgcn_raw_buffer_load_b128(rq, ((s / SEG) * RSQ + (s % SEG) * 8) * 2, 0, 0);
        st.k[i] = __builtin_amdgcn_raw_buffer_load_b128(rk, ((s / SEG) * RSK + (s % SEG) * 8) * 2, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        const int s = tid + i * NT;
        const uint32_t off = ((s / (VT / 8)) * RSV + (s % (VT / 8)) * 8) * 2;
        st.v[i] = __builtin_amdgcn_raw_buffer_load_b128(rv, off, 0, 0);
      }
      // per-token log gate; rows past the chunk's end read 0, so their
      // cumulative value equals the last real token's (a finite decay for their
      // zero k and v rows)
      // issued whether or not there is a per-token gate (an empty descriptor
      // reads zeros), so every chunk's loads are the same count of memory
      // instructions and waiting for them never waits for a later store
      const auto rg = make_rsrc(gb != nullptr ? (const void*)(gb + tok * H) : (const void*)qb,
                                gb != nullptr ? (uint32_t)cl * H * 4 : 0u);
      st.g = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rg, (uint32_t)(lane * H * 4), 0, 0));
    };
    auto store_chunk = [&](int p, const Stage& st) {
      bf16* q_s = sQ(p);
      bf16* k_s = sK(p);
      bf16* v_s = sV(p);
#pragma unroll
      for (int i = 0; i < NQ; ++i) {
        const int s = tid + i * NT;
        *reinterpret_cast<u32x4*>(q_s + (s / SEG) * L::LDQ + (s % SEG) * 8) = st.q[i];
        *reinterpret_cast<u32x4*>(k_s + (s / SEG) * L::LDK + (s % SEG) * 8) = st.k[i];
      }
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        const int s = tid + i * NT;
        *reinterpret_cast<u32x4*>(v_s + (s / (VT / 8)) * LDV + (s % (VT / 8)) * 8) = st.v[i];
      }
      // Every wave takes delivery of the gate word here, although only the last
      // wave uses it: a load whose register is still pending when the register
      // is reused makes the compiler wait on the vector-memory counter there,
      // and that counter retires loads and stores in issue order -- at the
      // next chunk's start that wait would include this chunk's output stores.
      asm volatile("" ::"v"(st.g));
      if (w == 3) {
        // step (1) on wave 3: it owns one A tile (waves 0 and 1 own two) and
        // forms it first, so it reaches the barrier early; chunk-local
        // cumulative log2 gate b, plus the per-token factors scale * 2^b
        // (inter-chunk term) and 2^(b_last - b) (state update)
        float* g_s = sG(p);
        const float b = gb != nullptr ? wave_cumsum_log2(st.g)
                                      : (float)min(lane + 1, st.len) * gam2;
        const float blast = __shfl(b, C - 1, 64);
        g_s[lane] = b;
        g_s[C + lane] = exp2_hw(b) * scale;
        g_s[2 * C + lane] = exp2_hw(blast - b);
      }
    };

    // ---- per-chunk phases ----------------------------------------------------
    // A = (Q K^T) (.) M, split into bf16 hi + lo, into sA(p), for this wave's
    // tiles (w, and w + 8 on waves 0 and 1).  The products and the epilogue
    // that needs their results are separate calls so that other products can
    // be issued between them; nmax bounds the tile count where the caller
    // knows it, so unused accumulators take no registers.
    auto phase_A_mma = [&](int p, f32x4 (&acc)[2][2], const int nmax) {
      const bf16* q_s = sQ(p);
      const bf16* k_s = sK(p);
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int ti = w + L::NW * u;
        if (u < nmax && ti < 10) {
          const int ct = tile_c(ti), jt = tile_j(ti);
          // every operand read first (one wait instead of one per step), then
          // two independent accumulation chains
          bf16x8 a[L::KSF], b[L::KSF];
#pragma unroll
          for (int s = 0; s < L::KSF; ++s) {
            a[s] = *reinterpret_cast<const bf16x8*>(k_s + (16 * jt + r) * L::LDK + 32 * s + 8 * g4);
            b[s] = *reinterpret_cast<const bf16x8*>(q_s + (16 * ct + r) * L::LDQ + 32 * s + 8 * g4);
          }
          acc[u][0] = f32x4{0.f, 0.f, 0.f, 0.f};
          acc[u][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s = 0; s < L::KSF; ++s) acc[u][s & 1] = mfma(a[s], b[s], acc[u][s & 1]);
        }
      }
    };
    auto phase_A_epi = [&](int p, const f32x4 (&accs)[2][2], const int nmax) {
      const float* g_s = sG(p);
      bf16* a_hi = sA(p);
      bf16* a_lo = a_hi + C * LDA;
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int ti = w + L::NW * u;
        if (u < nmax && ti < 10) {
          const int ct = tile_c(ti), jt = tile_j(ti);
          const f32x4 acc = accs[u][0] + accs[u][1];   // acc[i] = q_c . k_j, c = 16ct + r, j = 16jt + 4g + i
          const int c = 16 * ct + r;
          const float bc = g_s[c];
          const f32x4 bj = *reinterpret_cast<const f32x4*>(g_s + 16 * jt + 4 * g4);
          float x[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int j = 16 * jt + 4 * g4 + i;
            x[i] = (j <= c) ? acc[i] * exp2_hw(bc - bj[i]) * scale : 0.f;
          }
          uint32_t h0, l0, h1, l1;
          split2(x[0], x[1], h0, l0);
          split2(x[2], x[3], h1, l1);
          const u32x2 hi = {h0, h1}, lo = {l0, l1};
          *reinterpret_cast<u32x2*>(a_hi + c * LDA + 16 * jt + 4 * g4) = hi;
          *reinterpret_cast<u32x2*>(a_lo + c * LDA + 16 * jt + 4 * g4) = lo;
        }
      }
    };
    // O^T partial = scale diag(2^b) (h^T Q^T) over this wave's K/2 state rows,
    // for c tiles in the order (own0, own1, partner's two)
    auto phase_inter = [&](int p, f32x4 (&oacc)[4]) {
      const bf16* q_s = sQ(p);
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) oacc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < L::KS; ++s) {
        // A operand from the state: rows krow0 + 32s + 4g + {0..3} and
        // krow0 + 32s + 16 + 4g + {0..3}; q is read with the same k order
        float x[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          x[i] = h[2 * s][i];
          x[4 + i] = h[2 * s + 1][i];
        }
        bf16x8 hh, hl;
        split8(x, hh, hl);
        bf16x8 b[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const bf16* qrow = q_s + (16 * ctile[t] + r) * L::LDQ + krow0 + 32 * s + 4 * g4;
          b[t] = cat(*reinterpret_cast<const bf16x4*>(qrow), *reinterpret_cast<const bf16x4*>(qrow + 16));
        }
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) oacc[ct] = mfma(hh, b[ct], oacc[ct]);
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) oacc[ct] = mfma(hl, b[ct], oacc[ct]);
      }
    };
    // scale * diag(2^b): O^T column c = 16 ctile + r (a separate call, so
    // that the wait for the q.h products falls after the update is issued)
    auto inter_scale = [&](int p, f32x4 (&oacc)[4]) {
      // the four factors from one base (immediate offsets, one wait); ctile
      // is {0, 3, 1, 2} for kh = 0 and {1, 2, 0, 3} for kh = 1
      const float* gs = sG(p) + C + r;
      const float s0 = gs[0], s1 = gs[16], s2 = gs[32], s3 = gs[48];
      oacc[0] *= kh == 0 ? s0 : s1;
      oacc[1] *= kh == 0 ? s3 : s2;
      oacc[2] *= kh == 0 ? s1 : s0;
      oacc[3] *= kh == 0 ? s2 : s3;
    };
    // V fragments vf[s][e] = V[32s + 8g + e][16vc + r]
    auto load_vf = [&](int p, bf16x8 (&vf)[2]) {
      const bf16* v_s = sV(p);
#pragma unroll
      for (int s = 0; s < 2; ++s)
        vf[s] = cat(tr_read(v_s, LDV, 32 * s + 8 * g4, 16 * vc),
                    tr_read(v_s, LDV, 32 * s + 8 * g4 + 4, 16 * vc));
    };
    // h <- 2^b_last h + K^T (diag(2^(b_last - b)) V) for this wave's rows
    auto phase_update = [&](int p, const bf16x8 (&vf)[2]) {
      const bf16* k_s = sK(p);
      const float* g_s = sG(p);
      const float dall = exp2_hw(g_s[C - 1]);   // 2^b_last
#pragma unroll
      for (int kt = 0; kt < L::KT; ++kt) h[kt] *= dall;
      bf16x8 vth[2], vtl[2];
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const f32x4 d0 = *reinterpret_cast<const f32x4*>(g_s + 2 * C + 32 * s + 8 * g4);
        const f32x4 d1 = *reinterpret_cast<const f32x4*>(g_s + 2 * C + 32 * s + 8 * g4 + 4);
        const u32x4 raw = __builtin_bit_cast(u32x4, vf[s]);
        float x[8];
        x[0] = bf_lo(raw[0]) * d0[0];
        x[1] = bf_hi(raw[0]) * d0[1];
        x[2] = bf_lo(raw[1]) * d0[2];
        x[3] = bf_hi(raw[1]) * d0[3];
        x[4] = bf_lo(raw[2]) * d1[0];
        x[5] = bf_hi(raw[2]) * d1[1];
        x[6] = bf_lo(raw[3]) * d1[2];
        x[7] = bf_hi(raw[3]) * d1[3];
        split8(x, vth[s], vtl[s]);
      }
      constexpr int KG = L::KT < 4 ? L::KT : 4;   // state tiles per MFMA group
#pragma unroll
      for (int s = 0; s < 2; ++s) {
#pragma unroll
        for (int k0 = 0; k0 < L::KT; k0 += KG) {
          // A operands: K^T[krow0 + 16kt + r][32s + 8g + e]
          bf16x8 a[KG];
#pragma unroll
          for (int u = 0; u < KG; ++u)
            a[u] = cat(tr_read(k_s, L::LDK, 32 * s + 8 * g4, krow0 + 16 * (k0 + u)),
                       tr_read(k_s, L::LDK, 32 * s + 8 * g4 + 4, krow0 + 16 * (k0 + u)));
#pragma unroll
          for (int u = 0; u < KG; ++u) h[k0 + u] = mfma(a[u], vth[s], h[k0 + u]);
#pragma unroll
          for (int u = 0; u < KG; ++u) h[k0 + u] = mfma(a[u], vtl[s], h[k0 + u]);
        }
      }
    };
    // own c tiles: kh = 0 -> c tiles 0 (j < 32) and 3 (j < 64);
    //              kh = 1 -> c tiles 1 (j < 32) and 2 (j < 64)
    // O^T (own tiles) += V^T A^T with A from sA(p)
    auto phase_intra = [&](int p, const bf16x8 (&vf)[2], f32x4& mine0, f32x4& mine1) {
      const bf16* ah0 = sA(p) + (16 * own0 + r) * LDA + 8 * g4;
      const bf16* ah1 = sA(p) + (16 * own1 + r) * LDA + 8 * g4;
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
    };
    // the partner's two c tiles of this wave's q.h partial go through LDS
    auto exchange_write = [&](int px, const f32x4 (&oacc)[4]) {
      f32x4* x = sX(px);
      x[(w * 2 + 0) * 64 + lane] = oacc[2];
      x[(w * 2 + 1) * 64 + lane] = oacc[3];
    };
    // the partner's two tiles of this wave's own output rows
    auto exchange_read = [&](int px, f32x4& x0, f32x4& x1) {
      const f32x4* x = sX(px);
      x0 = x[((w ^ 4) * 2 + 0) * 64 + lane];
      x1 = x[((w ^ 4) * 2 + 1) * 64 + lane];
    };
    // own tiles + partner's partial (x0, x1), stored (rows past the chunk's end
    // fall outside the descriptor and are dropped; cl = 0 stores nothing)
    auto finalize = [&](int m, int cl, f32x4 mine0, f32x4 mine1, const f32x4& x0, const f32x4& x1) {
      const auto ro = make_rsrc(ob + (int64_t)m * C * RSO, (uint32_t)cl * RSO * sizeof(TOut));
      const uint32_t c0 = 16 * own0 + r, c1 = 16 * own1 + r;
      store4<TOut>(ro, c0 * RSO * (uint32_t)sizeof(TOut) + ocol, mine0 + x0);
      store4<TOut>(ro, c1 * RSO * (uint32_t)sizeof(TOut) + ocol, mine1 + x1);
    };

    // Pipelined, one barrier per chunk, loads running one chunk ahead.
    // Iteration m stages chunk m, forms chunk m-1's A V (from buffers of
    // parity p^1 and registers carried over), chunk m's A, q.h partials and
    // state update, and then stores chunk m-1's output.
    Stage st;
    load_chunk(0, st);
    bf16x8 vf_prev[2] = {};
    f32x4 mine0 = {0.f, 0.f, 0.f, 0.f}, mine1 = {0.f, 0.f, 0.f, 0.f};
    int prev_m = 0, prev_cl = 0;   // prev_cl = 0: nothing to store yet
    auto step = [&](const int m, const int p) {
      const int cl = st.len;
      store_chunk(p, st);
      __syncthreads();   // chunk m staged; chunk m-1's A and exchange tiles visible
      // Every wait for a product's result is placed after other products
      // have been issued (measured on the long and packed workloads; each
      // earlier placement cost 1-10 % of the step):
      //  - A on the first wave of each SIMD: products, then q.h, then the
      //    epilogue; on the second wave A comes last, after the exchange;
      //  - chunk m-1's A V after q.h, the q.h scaling after the update;
      //  - chunk m-1's output stores last, the partner's exchange tiles
      //    for them read before the update.
      // The loads of chunk m + 1 go out after the first wave's A products
      // (before them they held up the step's first products: 4-6 % of the
      // step) and before chunk m - 1's output stores, so waiting for them
      // never waits for the stores.
      f32x4 accA[2][2];
      if (kh == 0) phase_A_mma(p, accA, 2);
      load_chunk(m + 1, st);
      f32x4 oacc[4];
      phase_inter(p, oacc);
      if (kh == 0) phase_A_epi(p, accA, 2);
      phase_intra(p ^ 1, vf_prev, mine0, mine1);
      load_vf(p, vf_prev);
      f32x4 x0, x1;
      exchange_read(p ^ 1, x0, x1);
      phase_update(p, vf_prev);
      inter_scale(p, oacc);
      finalize(prev_m, prev_cl, mine0, mine1, x0, x1);
      exchange_write(p, oacc);
      if (kh != 0) {
        phase_A_mma(p, accA, 1);
        phase_A_epi(p, accA, 1);
      }
      mine0 = oacc[0];
      mine1 = oacc[1];
      prev_m = m;
      prev_cl = cl;
    };
    int m = 0;
    for (; m + 1 < nchunks; m += 2) {
      step(m, 0);
      step(m + 1, 1);
    }
    if (m < nchunks) step(m, 0);
    __syncthreads();
    const int pl = (nchunks - 1) & 1;
    phase_intra(pl, vf_prev, mine0, mine1);
    {
      f32x4 x0, x1;
      exchange_read(pl, x0, x1);
      finalize(prev_m, prev_cl, mine0, mine1, x0, x1);
    }

    if (ht != nullptr && last) {
      float* htu = ht + ((int64_t)seq * H + hd) * K * V;
#pragma unroll
      for (int kt = 0; kt < L::KT; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          htu[(int64_t)(krow0 + 16 * kt + 4 * g4 + i) * sl.rs + (int64_t)vcol * sl.cs] = h[kt][i];
    }
  }  // unit
}

template <int K, typename TOut>
hipError_t launch_k(const ChunkFwdParams& p, hipStream_t stream) {
  const int32_t units = p.segs != nullptr ? p.num_bins : p.seqs.num_seqs;
  if (units == 0) return hipSuccess;
  const dim3 grid((unsigned)unit_grid(units, p.Hkv, p.H / p.Hkv, p.V / VT));
  hipLaunchKernelGGL((chunk_fwd_bf16_kernel<K, TOut>), grid, dim3(Layout<K>::NT), 0, stream,
                     static_cast<const bf16*>(p.q), static_cast<const bf16*>(p.k),
                     static_cast<const bf16*>(p.v), p.g, p.g_gamma, p.h0,
                     static_cast<TOut*>(p.o), p.ht, p.scale, p.H, p.Hkv, p.V, p.sl, p.seqs, p.segs,
                     p.bins, p.num_bins, p.sin);
  return hipGetLastError();
}

template <typename TOut>
hipError_t launch_out(const ChunkFwdParams& p, hipStream_t stream) {
  switch (p.K) {
    case 64: return launch_k<64, TOut>(p, stream);
    case 128: return launch_k<128, TOut>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

int chunk_fwd_bf16_vtile(int32_t) { return VT; }

hipError_t launch_chunk_fwd_bf16(const ChunkFwdParams& p, hipStream_t stream) {
  return p.o_bf16 ? launch_out<__bf16>(p, stream) : launch_out<float>(p, stream);
}

}  // namespace sgla
