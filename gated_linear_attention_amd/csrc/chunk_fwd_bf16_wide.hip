// Inter-chunk state pass and output pass of the chunked Simple GLA forward for
// bf16 q/k/v with a wide key dimension (K = 256 or 512), fused in one kernel
// (page "flash-linear-attention 中的 Simple GLA", section 一: chunk view with a
// scalar-decayed state between chunks; section 三: the state pass and the
// output pass).  The per-chunk gates and the decay-masked A = scale (Q K^T (.)
// M) come from the preparation kernel (chunk_prep_bf16.hip).
//
// For chunk n with state h_n (K x V, fp32):
//   O_n     = diag(sc) Q_n h_n + A_n V_n,        sc = scale 2^b
//   h_n+1   = dall h_n + K_n^T diag(dv) V_n,     dv = 2^(b_last - b), dall = 2^b_last
//
// Workgroup = (sequence, head, 32-wide V tile), 8 waves (two per SIMD).  Wave
// w owns the K/8 state rows [K/8 w, +K/8) of the tile's 32 columns, as 32 x 32
// fp32 MFMA accumulators (v_mfma_f32_32x32x16_bf16) that stay in registers
// for the whole sequence.  Per chunk each wave
//   1. multiplies its rows of Q (loaded from HBM straight into MFMA operand
//      layout) with its state rows: a 64 x 32 partial of Q h_n;
//   2. updates its state rows with K^T (transposed LDS reads of the staged K
//      chunk) times the decayed V (hi + lo);
//   3. writes its partial to LDS; after a barrier, wave (ct, vh) sums the
//      eight partials of output tile rows [16 ct, +16) x columns [16 vh, +16),
//      scales them by sc, adds the intra-chunk A V (16x16x32 MFMAs, A read
//      from the preparation output) and stores the tile.
// The next chunk's K, V and gates are loaded into registers one chunk ahead
// and written to LDS after the barrier; Q and A fragments are loaded one
// chunk ahead straight into the registers that use them.
//
// State row order: accumulator element a of lane (n = l % 32, h = l / 32) in
// row tile rt holds S[K/8 w + 32 rt + 16 (a / 8) + 8 h + a % 8][column n], so
// the eight state values a lane feeds to one q.h MFMA are eight consecutive
// keys and the matching Q operand is one 16-byte load.  The update's K^T
// operand reads keys in the same order (a 4-key block permutation inside each
// transposed LDS read).
//
// Precision: fp32 state, accumulation and output; h in q.h and the decayed V
// in the update are split into bf16 hi + lo and issued as two MFMAs each
// (A arrives already split).
#include <hip/hip_runtime.h>

#include "mfma_common.h"
#include "sgla_internal.h"

namespace sgla {
namespace {

using namespace mf;

constexpr int C = kChunk;
constexpr int VT = 32;           // state / output columns per workgroup
constexpr int NW = 8;            // waves
constexpr int NT = 64 * NW;      // threads
constexpr int LDV = VT + 16;     // V tile row stride (elements)
constexpr int LDP = C + 4;       // partial row stride (floats)

template <int K>
struct WideLayout {
  static constexpr int LDK = K + 32;                 // K chunk row stride (elements)
  static constexpr int SZ_K = C * LDK * 2;
  static constexpr int OFF_P = SZ_K;
  static constexpr int SZ_P = NW * VT * LDP * 4;     // per-wave partials [w][v][c]
  static constexpr int OFF_V = OFF_P + SZ_P;
  static constexpr int SZ_V = C * LDV * 2;           // per buffer (two)
  static constexpr int OFF_G = OFF_V + 2 * SZ_V;
  static constexpr int SZ_G = kGateStride * 4;       // per buffer (two)
  static constexpr int BYTES = OFF_G + 2 * SZ_G;
  static_assert(BYTES <= 160 * 1024, "LDS budget");
};

// Transposed LDS read with the key order of the state rows: lane r of each
// 16-lane group receives base[(row0 + e) * ld + col0 + perm(r)] for e = 0..3,
// where perm swaps the middle two 4-key blocks of the 16 (0-3, 8-11, 4-7,
// 12-15).
__device__ __forceinline__ bf16x4 tr_read_perm(const bf16* base, int ld, int row0, int col0) {
  const int lane = threadIdx.x & 15;
  const int blk = ((lane & 1) << 3) | ((lane & 2) << 1);
  const bf16* p = base + (row0 + (lane >> 2)) * ld + col0 + blk;
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p));
}

template <typename TOut>
__device__ __forceinline__ void store1(__amdgpu_buffer_rsrc_t rs, uint32_t off, float x);
template <>
__device__ __forceinline__ void store1<float>(__amdgpu_buffer_rsrc_t rs, uint32_t off, float x) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, x), rs, off, 0, 0);
}
template <>
__device__ __forceinline__ void store1<bf16>(__amdgpu_buffer_rsrc_t rs, uint32_t off, float x) {
  __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, (bf16)x), rs, off, 0, 0);
}

template <int K, typename TOut>
__global__ void __launch_bounds__(NT)
chunk_fwd_bf16_wide_kernel(const bf16* __restrict__ q, const bf16* __restrict__ k,
                           const bf16* __restrict__ v, const float* __restrict__ h0,
                           TOut* __restrict__ o, float* __restrict__ ht, int32_t H, int32_t V,
                           SeqLayout seqs, int32_t chunks_per_row, const float* __restrict__ gates,
                           const bf16* __restrict__ amat) {
  using L = WideLayout<K>;
  constexpr int LDK = L::LDK;
  constexpr int RW = K / NW;           // state rows per wave
  constexpr int NRT = RW / 32;         // 32-row accumulator tiles per wave
  constexpr int KP = K / 8;            // 16-byte pieces per K row
  constexpr int NKS = C * KP / NT;     // K staging pieces per thread
  static_assert(NRT >= 1 && NKS >= 1, "K too small for this kernel");
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
  int32_t len, seq, chunk0;
  if (seqs.seq_table != nullptr) {
    const SeqEntry e = seqs.seq_table[rank];
    bos = __builtin_amdgcn_readfirstlane(e.bos);
    len = __builtin_amdgcn_readfirstlane(e.len);
    seq = __builtin_amdgcn_readfirstlane(e.seq);
    chunk0 = __builtin_amdgcn_readfirstlane(e.chunk0);
  } else {
    bos = (int64_t)rank * seqs.T;
    len = seqs.T;
    seq = rank;
    chunk0 = rank * chunks_per_row;
  }
  const int nchunks = (len + C - 1) / C;

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l32 = lane & 31;       // 32x32 layouts: column / row index
  const int hf = lane >> 5;        //                 key half
  const int grp = lane >> 4;       // 16-lane group
  const int r = lane & 15;         // 16x16 layouts
  const int g4 = lane >> 4;
  const int k0w = RW * w;
  const int ct = w >> 1;           // output tile of this wave: rows [16 ct, +16)
  const int vh = w & 1;            //                           columns [16 vh, +16)
  const int RSK = H * K;
  const int RSV = H * V;
  const bf16* qb = q + (bos * H + hd) * (int64_t)K;
  const bf16* kb = k + (bos * H + hd) * (int64_t)K;
  const bf16* vb = v + (bos * H + hd) * (int64_t)V + vt * VT;
  TOut* ob = o + (bos * H + hd) * (int64_t)V + vt * VT;
  const int64_t gstep = (int64_t)H * kGateStride;          // gate records between chunks
  const int64_t astep = (int64_t)H * 2 * C * C;             // A records between chunks
  const float* gbase = gates + ((int64_t)chunk0 * H + hd) * kGateStride;
  const bf16* abase = amat + ((int64_t)chunk0 * H + hd) * 2 * C * C;

  bf16* sK = reinterpret_cast<bf16*>(smem);
  float* sP = reinterpret_cast<float*>(smem + L::OFF_P);
  auto sV = [&](int p) { return reinterpret_cast<bf16*>(smem + L::OFF_V + p * L::SZ_V); };
  auto sG = [&](int p) { return reinterpret_cast<float*>(smem + L::OFF_G + p * L::SZ_G); };

  // ---- state ---------------------------------------------------------------
  f32x16 h[NRT];
  {
    const float* h0u = h0 != nullptr ? h0 + ((int64_t)seq * H + hd) * K * V : nullptr;
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
      for (int a = 0; a < 16; ++a) {
        const int key = k0w + 32 * rt + 16 * (a >> 3) + 8 * hf + (a & 7);
        h[rt][a] = h0u != nullptr ? h0u[(int64_t)key * V + vt * VT + l32] : 0.f;
      }
  }

  // ---- staging: K chunk, V tile and gates of one chunk, in registers ------
  struct Stage {
    u32x4 kk[NKS];
    u32x4 vg;    // waves 0-3: a V piece; waves 4-7: a gate piece
  };
  auto load_stage = [&](int m, Stage& st) {
    const int cl = max(0, min(C, len - m * C));
    const int64_t tok = (int64_t)m * C;
    const auto rk = make_rsrc(kb + tok * RSK, (uint32_t)cl * RSK * 2);
#pragma unroll
    for (int u = 0; u < NKS; ++u) {
      const int p = tid + NT * u;
      st.kk[u] = __builtin_amdgcn_raw_buffer_load_b128(rk, (uint32_t)((p / KP) * RSK + (p % KP) * 8) * 2, 0, 0);
    }
    if (w < 4) {
      const auto rv = make_rsrc(vb + tok * RSV, (uint32_t)cl * RSV * 2);
      st.vg = __builtin_amdgcn_raw_buffer_load_b128(rv, (uint32_t)((tid >> 2) * RSV + (tid & 3) * 8) * 2, 0, 0);
    } else {
      const auto rg = make_rsrc(gbase + m * gstep, m < nchunks ? (uint32_t)kGateStride * 4 : 0u);
      st.vg = __builtin_amdgcn_raw_buffer_load_b128(rg, (uint32_t)(tid - 256) * 16, 0, 0);
    }
  };
  auto store_stage = [&](const Stage& st, int p) {
#pragma unroll
    for (int u = 0; u < NKS; ++u) {
      const int pc = tid + NT * u;
      *reinterpret_cast<u32x4*>(sK + (pc / KP) * LDK + (pc % KP) * 8) = st.kk[u];
    }
    if (w < 4) {
      *reinterpret_cast<u32x4*>(sV(p) + (tid >> 2) * LDV + (tid & 3) * 8) = st.vg;
    } else if (tid - 256 < kGateStride / 4) {
      *reinterpret_cast<u32x4*>(sG(p) + (tid - 256) * 4) = st.vg;
    }
  };

  // ---- Q operand of q.h: rows 32 c2 + l32, keys k0w + 32 rt + 16 s + 8 hf ---
  bf16x8 qf[2][NRT][2];
  auto load_q = [&](int m) {
    const int cl = max(0, min(C, len - m * C));
    const auto rq = make_rsrc(qb + (int64_t)m * C * RSK, (uint32_t)cl * RSK * 2);
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
        for (int s = 0; s < 2; ++s)
          qf[c2][rt][s] = __builtin_bit_cast(
              bf16x8, __builtin_amdgcn_raw_buffer_load_b128(
                          rq, (uint32_t)((32 * c2 + l32) * RSK + k0w + 32 * rt + 16 * s + 8 * hf) * 2, 0, 0));
  };

  // ---- A operand of the intra product: rows 16 ct + r, tokens 32 u + 8 g4 --
  bf16x8 af[2][2];   // [u][hi, lo]
  auto load_a = [&](int m) {
    const uint32_t bytes = m < nchunks ? (uint32_t)(2 * C * C * 2) : 0u;
    const auto ra0 = make_rsrc(abase + m * astep, bytes);
    const auto ra1 = make_rsrc(abase + m * astep, ct >= 2 ? bytes : 0u);   // tokens 32..63
#pragma unroll
    for (int pl = 0; pl < 2; ++pl) {
      const uint32_t off = (uint32_t)(pl * C * C + (16 * ct + r) * C + 8 * g4) * 2;
      af[0][pl] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(ra0, off, 0, 0));
      af[1][pl] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(ra1, off + 64, 0, 0));
    }
  };

  Stage st;
  load_stage(0, st);
  store_stage(st, 0);
  load_stage(1, st);
  load_q(0);
  load_a(0);
  __syncthreads();

  for (int m = 0; m < nchunks; ++m) {
    const int p = m & 1;
    const float* sg = sG(p);
    const bf16* sv = sV(p);
    const int cl = min(C, len - m * C);

    // ---- 1. partial q.h over this wave's state rows ----------------------
    f32x16 pacc[2];
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
      for (int a = 0; a < 16; ++a) pacc[c2][a] = 0.f;
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = h[rt][8 * s + e];
        bf16x8 hh, hl;
        split8(x, hh, hl);
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2) {
          pacc[c2] = mfma32(qf[c2][rt][s], hh, pacc[c2]);
          pacc[c2] = mfma32(qf[c2][rt][s], hl, pacc[c2]);
        }
      }
    load_q(m + 1);

    // ---- 2. state update: h <- dall h + K^T diag(dv) V -------------------
    const float dall = sg[2 * C];
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) h[rt] *= dall;
#pragma unroll
    for (int ts = 0; ts < 4; ++ts) {
      const int row0 = 16 * ts + 8 * (grp >> 1);
      const bf16x8 vraw = cat(tr_read(sv, LDV, row0, 16 * (grp & 1)), tr_read(sv, LDV, row0 + 4, 16 * (grp & 1)));
      const f32x4 d0 = *reinterpret_cast<const f32x4*>(sg + C + 16 * ts + 8 * hf);
      const f32x4 d1 = *reinterpret_cast<const f32x4*>(sg + C + 16 * ts + 8 * hf + 4);
      const u32x4 raw = __builtin_bit_cast(u32x4, vraw);
      float x[8];
      x[0] = bf_lo(raw[0]) * d0[0];
      x[1] = bf_hi(raw[0]) * d0[1];
      x[2] = bf_lo(raw[1]) * d0[2];
      x[3] = bf_hi(raw[1]) * d0[3];
      x[4] = bf_lo(raw[2]) * d1[0];
      x[5] = bf_hi(raw[2]) * d1[1];
      x[6] = bf_lo(raw[3]) * d1[2];
      x[7] = bf_hi(raw[3]) * d1[3];
      bf16x8 vth, vtl;
      split8(x, vth, vtl);
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt) {
        const int kc = k0w + 32 * rt + 16 * (grp & 1);
        const bf16x8 kf = cat(tr_read_perm(sK, LDK, row0, kc), tr_read_perm(sK, LDK, row0 + 4, kc));
        h[rt] = mfma32(kf, vth, h[rt]);
        h[rt] = mfma32(kf, vtl, h[rt]);
      }
    }

    // ---- 3. partials to LDS: pacc[c2][4 j + i] = P[32 c2 + 8 j + 4 hf + i][l32]
    {
      float* pw = sP + (w * VT + l32) * LDP + 4 * hf;
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          *reinterpret_cast<f32x4*>(pw + 32 * c2 + 8 * j) =
              f32x4{pacc[c2][4 * j], pacc[c2][4 * j + 1], pacc[c2][4 * j + 2], pacc[c2][4 * j + 3]};
    }
    __syncthreads();

    // ---- 4. output tile (ct, vh): rows 16 ct + 4 g4 + i, column 16 vh + r --
    {
      f32x4 acc = *reinterpret_cast<const f32x4*>(sP + (16 * vh + r) * LDP + 16 * ct + 4 * g4);
#pragma unroll
      for (int w2 = 1; w2 < NW; ++w2)
        acc += *reinterpret_cast<const f32x4*>(sP + (w2 * VT + 16 * vh + r) * LDP + 16 * ct + 4 * g4);
      acc *= *reinterpret_cast<const f32x4*>(sg + 16 * ct + 4 * g4);
      {
        const bf16x8 vf = cat(tr_read(sv, LDV, 8 * g4, 16 * vh), tr_read(sv, LDV, 8 * g4 + 4, 16 * vh));
        acc = mfma(af[0][0], vf, acc);
        acc = mfma(af[0][1], vf, acc);
      }
      if (ct >= 2) {
        const bf16x8 vf = cat(tr_read(sv, LDV, 32 + 8 * g4, 16 * vh), tr_read(sv, LDV, 36 + 8 * g4, 16 * vh));
        acc = mfma(af[1][0], vf, acc);
        acc = mfma(af[1][1], vf, acc);
      }
      const auto ro = make_rsrc(ob + (int64_t)m * C * RSV, (uint32_t)cl * RSV * (uint32_t)sizeof(TOut));
#pragma unroll
      for (int i = 0; i < 4; ++i)
        store1<TOut>(ro, (uint32_t)((16 * ct + 4 * g4 + i) * RSV + 16 * vh + r) * (uint32_t)sizeof(TOut), acc[i]);
    }
    load_a(m + 1);

    // ---- 5. next chunk's K, V and gates into LDS; prefetch the one after --
    store_stage(st, p ^ 1);
    load_stage(m + 2, st);
    __syncthreads();
  }

  if (ht != nullptr) {
    float* htu = ht + ((int64_t)seq * H + hd) * K * V;
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
      for (int a = 0; a < 16; ++a) {
        const int key = k0w + 32 * rt + 16 * (a >> 3) + 8 * hf + (a & 7);
        htu[(int64_t)key * V + vt * VT + l32] = h[rt][a];
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
  const int per_row = p.seqs.T > 0 ? (p.seqs.T + C - 1) / C : 0;
  hipLaunchKernelGGL((chunk_fwd_bf16_wide_kernel<K, TOut>), grid, dim3(NT), 0, stream,
                     static_cast<const bf16*>(p.q), static_cast<const bf16*>(p.k),
                     static_cast<const bf16*>(p.v), p.h0, static_cast<TOut*>(p.o), p.ht, p.H, p.V,
                     p.seqs, per_row, p.gates, static_cast<const bf16*>(p.amat));
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

hipError_t launch_chunk_fwd_bf16_wide(const ChunkFwdParams& p, hipStream_t stream) {
  return p.o_bf16 ? launch_out<__bf16>(p, stream) : launch_out<float>(p, stream);
}

}  // namespace sgla
