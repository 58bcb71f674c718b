// Inter-chunk state pass and output pass of the chunked Simple GLA forward for
// bf16 q/k/v with a wide key dimension (K = 256 or 512), fused in one kernel
// (page "flash-linear-attention 中的 Simple GLA", section 一: chunk view with a
// scalar-decayed state between chunks; section 三: the state pass and the
// output pass).  The per-chunk gates, the decay-masked A = scale (Q K^T (.) M)
// and the Q, K^T and A operands in MFMA operand order come from the
// preparation kernel (chunk_prep_bf16.hip), so every operand load here is one
// contiguous 1 KB block.
//
// For chunk n with state h_n (K x V, fp32):
//   O_n     = diag(sc) Q_n h_n + A_n V_n,        sc = scale 2^b
//   h_n+1   = dall h_n + K_n^T diag(dv) V_n,     dv = 2^(b_last - b), dall = 2^b_last
//
// Workgroup = (sequence, head, 32-wide V tile), 8 waves (two per SIMD).  Wave
// w owns the K/8 state rows [K/8 w, +K/8) of the tile's 32 columns, as 32 x 32
// fp32 MFMA accumulators (v_mfma_f32_32x32x16_bf16) that stay in registers
// for the whole sequence.  Per chunk each wave
//   1. multiplies the chunk's Q, restricted to its keys, with its state rows:
//      a 64 x 32 partial of Q h_n;
//   2. updates its state rows with K^T times the decayed V (hi + lo), read
//      from LDS where the eight waves computed it together (each wave an
//      eighth of the tile) during the previous chunk;
//   3. after a barrier, writes its partial to LDS and stages the V tile and
//      gates two chunks ahead; a second barrier closes the chunk.  In the next
//      chunk, once its q.h products are issued, wave (ct, vh) sums the eight
//      partials of output rows [16 ct, +16) x columns [16 vh, +16), scales
//      them by sc, adds the intra-chunk A V (16x16x32 MFMAs, A from the
//      preparation output) and stores the tile after that chunk's update is
//      issued -- so the output's LDS round trips and product latency overlap
//      matrix work instead of sitting between barriers (-6 %).  The next
//      decayed V tile is formed at the top of the chunk.
// Q and K^T fragments are loaded one chunk ahead, A fragments one output
// tile ahead, into the registers that use them.
//
// State row order: accumulator element a of lane (n = l % 32, h = l / 32) in
// row tile rt holds S[K/8 w + 32 rt + 16 (a / 8) + 8 h + a % 8][column n], so
// the eight state values a lane feeds to one q.h MFMA are eight consecutive
// keys and the matching Q operand is one 16-byte load.  The K^T operand of the
// update uses the same key order (the preparation kernel writes it so).
//
// Precision: fp32 state, accumulation and output; h in q.h and the decayed V
// in the update are split into bf16 hi + lo and issued as two MFMAs each
// (A arrives already split).
#include <hip/hip_runtime.h>

#include "mfma_common.h"
#include "sgla_internal.h"
#include "unit_map.h"

namespace sgla {
namespace {

using namespace mf;

constexpr int C = kChunk;
constexpr int VT = 32;           // state / output columns per workgroup
constexpr int NW = 8;            // waves
constexpr int NT = 64 * NW;      // threads
constexpr int LDV = VT + 8;      // V tile row stride (elements)
constexpr int LDP = C + 4;       // partial row stride (floats)

struct WideLayout {
  static constexpr int SZ_P = NW * VT * LDP * 4;     // per-wave partials [w][v][c]
  static constexpr int OFF_V = SZ_P;
  static constexpr int SZ_V = C * LDV * 2;           // V tile, three buffers
  static constexpr int OFF_G = OFF_V + 3 * SZ_V;
  static constexpr int SZ_G = kGateStride * 4;       // gates, three buffers
  static constexpr int OFF_T = OFF_G + 3 * SZ_G;
  static constexpr int SZ_T = 2 * C * LDV * 2;       // decayed V hi + lo, two buffers
  static constexpr int BYTES = OFF_T + 2 * SZ_T;
  static_assert(BYTES <= 160 * 1024, "LDS budget");
};

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
chunk_fwd_bf16_wide_kernel(const bf16* __restrict__ qfr, const bf16* __restrict__ v,
                           const float* __restrict__ h0, TOut* __restrict__ o,
                           float* __restrict__ ht, int32_t H, int32_t Hkv, int32_t V, StateLayout sl,
                           SeqLayout seqs,
                           int32_t chunks_per_row, const float* __restrict__ gates,
                           const bf16* __restrict__ amat, const bf16* __restrict__ ktf) {
  using L = WideLayout;
  constexpr int RW = K / NW;           // state rows per wave
  constexpr int NRT = RW / 32;         // 32-row accumulator tiles per wave
  static_assert(NRT >= 1, "K too small for this kernel");
  __shared__ __attribute__((aligned(16))) char smem[L::BYTES];

  // ---- which (sequence, head, V tile) this workgroup owns ----------------
  const UnitMap um = map_unit(blockIdx.x, V / VT, Hkv, H / Hkv, seqs.num_seqs);
  if (!um.valid) return;
  const int rank = um.rank, hd = um.hd, hk = um.hk, vt = um.vt;
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
  const int RSV = Hkv * V;                                 // token stride of v
  const int RSO = H * V;                                   // token stride of o
  const bf16* vb = v + (bos * Hkv + hk) * (int64_t)V + vt * VT;
  TOut* ob = o + (bos * H + hd) * (int64_t)V + vt * VT;
  const int64_t task0 = (int64_t)chunk0 * H + hd;          // preparation record of chunk 0
  const float* gbase = gates + task0 * kGateStride;
  const bf16* abase = amat + task0 * (2 * C * C);
  const bf16* qbase = qfr + task0 * (int64_t)K * C;
  const bf16* ktbase = ktf + ((int64_t)chunk0 * Hkv + hk) * K * C;   // K^T is per kv head
  const int64_t gstep = (int64_t)H * kGateStride;          // record strides between chunks
  const int64_t astep = (int64_t)H * 2 * C * C;
  const int64_t qstep = (int64_t)H * K * C;
  const int64_t kstep = (int64_t)Hkv * K * C;

  float* sPb = reinterpret_cast<float*>(smem);
  auto sV = [&](int p) { return reinterpret_cast<bf16*>(smem + L::OFF_V + p * L::SZ_V); };
  auto sG = [&](int p) { return reinterpret_cast<float*>(smem + L::OFF_G + p * L::SZ_G); };
  auto sT = [&](int p) { return reinterpret_cast<bf16*>(smem + L::OFF_T + p * L::SZ_T); };

  // ---- state ---------------------------------------------------------------
  f32x16 h[NRT];
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
    for (int a = 0; a < 16; ++a) h[rt][a] = 0.f;
  if (h0 != nullptr) {
    const float* h0u = h0 + ((int64_t)seq * H + hd) * K * V + (int64_t)(vt * VT + l32) * sl.cs;
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
      for (int a = 0; a < 16; ++a)
        h[rt][a] = h0u[(int64_t)(k0w + 32 * rt + 16 * (a >> 3) + 8 * hf + (a & 7)) * sl.rs];
  }

  // ---- V tile and gates of one chunk: waves 0-3 load a V piece each, waves
  //      4-7 a piece of the gate record --------------------------------------
  auto load_vg = [&](int m) -> u32x4 {
    const int cl = max(0, min(C, len - m * C));
    if (w < 4) {
      const auto rv = make_rsrc(vb + (int64_t)m * C * RSV, (uint32_t)cl * RSV * 2);
      return __builtin_amdgcn_raw_buffer_load_b128(rv, (uint32_t)((tid >> 2) * RSV + (tid & 3) * 8) * 2, 0, 0);
    }
    const auto rg = make_rsrc(gbase + m * gstep, m < nchunks ? (uint32_t)kGateStride * 4 : 0u);
    return __builtin_amdgcn_raw_buffer_load_b128(rg, (uint32_t)(tid - 256) * 16, 0, 0);
  };
  auto store_vg = [&](u32x4 x, int p) {
    if (w < 4) {
      *reinterpret_cast<u32x4*>(sV(p) + (tid >> 2) * LDV + (tid & 3) * 8) = x;
    } else if (tid - 256 < kGateStride / 4) {
      *reinterpret_cast<u32x4*>(sG(p) + (tid - 256) * 4) = x;
    }
  };

  // ---- Q operand of q.h: blocks (key block, c2, s) -------------------------
  bf16x8 qf[2][NRT][2];
  auto load_q = [&](int m) {
    const auto rq = make_rsrc(qbase + m * qstep, m < nchunks ? (uint32_t)K * C * 2 : 0u);
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
        for (int s = 0; s < 2; ++s)
          qf[c2][rt][s] = __builtin_bit_cast(
              bf16x8, __builtin_amdgcn_raw_buffer_load_b128(
                          rq, (uint32_t)(((((k0w >> 5) + rt) * 2 + c2) * 2 + s) * 64 + lane) * 16, 0, 0));
  };

  // ---- K^T operand of the update: fragments (key block, token step) --------
  bf16x8 kt[4][NRT];
  auto load_kt = [&](int m) {
    const auto rk = make_rsrc(ktbase + m * kstep, m < nchunks ? (uint32_t)K * C * 2 : 0u);
#pragma unroll
    for (int ts = 0; ts < 4; ++ts)
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt)
        kt[ts][rt] = __builtin_bit_cast(
            bf16x8, __builtin_amdgcn_raw_buffer_load_b128(
                        rk, (uint32_t)((((k0w >> 5) + rt) * 4 + ts) * 64 + lane) * 16, 0, 0));
  };

  // ---- A operand of the intra product: blocks (ct, u, plane) --------------
  bf16x8 af[2][2];   // [u][hi, lo]
  auto load_a = [&](int m) {
    const uint32_t bytes = m < nchunks ? (uint32_t)(2 * C * C * 2) : 0u;
    const auto ra0 = make_rsrc(abase + m * astep, bytes);
    const auto ra1 = make_rsrc(abase + m * astep, ct >= 2 ? bytes : 0u);   // tokens 32..63
#pragma unroll
    for (int pl = 0; pl < 2; ++pl) {
      af[0][pl] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(
                                                 ra0, (uint32_t)((((ct * 2 + 0) * 2 + pl) * 64 + lane) * 16), 0, 0));
      af[1][pl] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(
                                                 ra1, (uint32_t)((((ct * 2 + 1) * 2 + pl) * 64 + lane) * 16), 0, 0));
    }
  };

  // ---- output tile (ct, vh) of chunk m: rows 16 ct + 4 g4 + i, column
  //      16 vh + r ---------------------------------------------------------------
  auto finish = [&](int m) -> f32x4 {
    const float* sg = sG(m % 3);
    const bf16* sv = sV(m % 3);
    f32x4 acc = *reinterpret_cast<const f32x4*>(sPb + (16 * vh + r) * LDP + 16 * ct + 4 * g4);
#pragma unroll
    for (int w2 = 1; w2 < NW; ++w2)
      acc += *reinterpret_cast<const f32x4*>(sPb + (w2 * VT + 16 * vh + r) * LDP + 16 * ct + 4 * g4);
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
    return acc;
  };
  // stored after the update products of the chunk that forms the tile are
  // issued, so the wait for this tile's A V products does not hold the wave
  auto store_out = [&](int m, const f32x4& acc) {
    const int cl = min(C, len - m * C);
    const auto ro = make_rsrc(ob + (int64_t)m * C * RSO, (uint32_t)cl * RSO * (uint32_t)sizeof(TOut));
#pragma unroll
    for (int i = 0; i < 4; ++i)
      store1<TOut>(ro, (uint32_t)((16 * ct + 4 * g4 + i) * RSO + 16 * vh + r) * (uint32_t)sizeof(TOut), acc[i]);
  };

  // ---- decayed V of chunk m, hi + lo: wave w computes tokens [8 w, +8) ------
  auto decay_v = [&](int m) {
    const bf16* sv = sV(m % 3);
    const float* sg = sG(m % 3);
    bf16* st = sT(m & 1);
    const int row = 8 * w + (lane >> 3);
    const int col = 4 * (lane & 7);
    const u32x2 raw = *reinterpret_cast<const u32x2*>(sv + row * LDV + col);
    const float d = sg[C + row];
    float x[4] = {bf_lo(raw[0]) * d, bf_hi(raw[0]) * d, bf_lo(raw[1]) * d, bf_hi(raw[1]) * d};
    uint32_t h0w, l0w, h1w, l1w;
    split2(x[0], x[1], h0w, l0w);
    split2(x[2], x[3], h1w, l1w);
    *reinterpret_cast<u32x2*>(st + row * LDV + col) = u32x2{h0w, h1w};
    *reinterpret_cast<u32x2*>(st + C * LDV + row * LDV + col) = u32x2{l0w, l1w};
  };

  store_vg(load_vg(0), 0);
  store_vg(load_vg(1), 1);
  u32x4 vg = load_vg(2);
  load_q(0);
  load_kt(0);
  __syncthreads();
  decay_v(0);
  __syncthreads();

  f32x4 oprev = {0.f, 0.f, 0.f, 0.f};
  for (int m = 0; m < nchunks; ++m) {
    const float* sg = sG(m % 3);
    const bf16* stv = sT(m & 1);
    // the next chunk's decayed V (its V and gates were staged two chunks
    // ahead; its buffer was last read before the previous chunk's barriers):
    // formed here, its LDS round trip overlaps the q.h products instead of
    // sitting between the two barriers (-2.5 %)
    if (m + 1 < nchunks) decay_v(m + 1);

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
    // chunk m-1's output tile while the q.h products run: its partials, V
    // tile and gates were published by the previous chunk's last barrier
    if (m > 0) oprev = finish(m - 1);
    load_a(m);

    // ---- 2. state update: h <- dall h + K^T (decayed V hi + lo) ------------
    const float dall = sg[2 * C];
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) h[rt] *= dall;
#pragma unroll
    for (int ts = 0; ts < 4; ++ts) {
      const int row0 = 16 * ts + 8 * (grp >> 1);
      const int col0 = 16 * (grp & 1);
      const bf16x8 vth = cat(tr_read(stv, LDV, row0, col0), tr_read(stv, LDV, row0 + 4, col0));
      const bf16x8 vtl = cat(tr_read(stv + C * LDV, LDV, row0, col0), tr_read(stv + C * LDV, LDV, row0 + 4, col0));
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt) {
        h[rt] = mfma32(kt[ts][rt], vth, h[rt]);
        h[rt] = mfma32(kt[ts][rt], vtl, h[rt]);
      }
    }
    if (m > 0) store_out(m - 1, oprev);
    load_kt(m + 1);
    __syncthreads();   // every read of chunk m-1's partials, V tile and gates done

    // ---- 3. partials to LDS: pacc[c2][4 j + i] = P[32 c2 + 8 j + 4 hf + i][l32]
    {
      float* pw = sPb + (w * VT + l32) * LDP + 4 * hf;
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          *reinterpret_cast<f32x4*>(pw + 32 * c2 + 8 * j) =
              f32x4{pacc[c2][4 * j], pacc[c2][4 * j + 1], pacc[c2][4 * j + 2], pacc[c2][4 * j + 3]};
    }
    // ---- 4. V tile and gates two chunks ahead (into chunk m-1's buffers) ----
    store_vg(vg, (m + 2) % 3);
    vg = load_vg(m + 3);
    __syncthreads();   // chunk m's partials, the next decayed V and V / gates two ahead visible
  }

  if (nchunks > 0) {
    oprev = finish(nchunks - 1);
    store_out(nchunks - 1, oprev);
  }
  if (ht != nullptr) {
    float* htu = ht + ((int64_t)seq * H + hd) * K * V + (int64_t)(vt * VT + l32) * sl.cs;
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
      for (int a = 0; a < 16; ++a)
        htu[(int64_t)(k0w + 32 * rt + 16 * (a >> 3) + 8 * hf + (a & 7)) * sl.rs] = h[rt][a];
  }
}

template <int K, typename TOut>
hipError_t launch_k(const ChunkFwdParams& p, hipStream_t stream) {
  if (p.seqs.num_seqs == 0) return hipSuccess;
  const dim3 grid((unsigned)unit_grid(p.seqs.num_seqs, p.Hkv, p.H / p.Hkv, p.V / VT));
  const int per_row = p.seqs.T > 0 ? (p.seqs.T + C - 1) / C : 0;
  hipLaunchKernelGGL((chunk_fwd_bf16_wide_kernel<K, TOut>), grid, dim3(NT), 0, stream,
                     static_cast<const bf16*>(p.qfr), static_cast<const bf16*>(p.v), p.h0,
                     static_cast<TOut*>(p.o), p.ht, p.H, p.Hkv, p.V, p.sl, p.seqs, per_row, p.gates,
                     static_cast<const bf16*>(p.amat), static_cast<const bf16*>(p.ktf));
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
