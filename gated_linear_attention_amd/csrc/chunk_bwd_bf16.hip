// The chunked Simple GLA backward on the bf16 matrix cores, for bf16 q, k, v
// and dO with K in {64, 128, 256, 512}: the state pass (further below) and
// the per-(chunk, head) gradients (page
// "flash-linear-attention 中的 Simple GLA", section 三: the backward's
// q/k/gate and v gradient passes over the fp32 state trajectory; section 五:
// dq, dk, dv, dg).  The algebra is the fp32 gradient kernel's
// (chunk_bwd.hip), per chunk with b the chunk-local cumulative log2 gate,
// sc = scale 2^b, dv_j = 2^(b_last - b_j), h the state entering the chunk
// and dH the gradient of the state leaving it (both fp32 records of the
// state pass):
//   A  = scale (Q K^T) (.) M,   dA = scale (dO V^T) (.) M,  M_cj = 2^(b_c - b_j) (j <= c)
//   dQ = diag(sc) dO h^T + dA K
//   dK = dA^T Q + diag(dv) V dH^T
//   dV = A^T dO + diag(dv) K dH
// and the gate gradient from r_t = q_t . dq_t - k_t . dk_t plus, at the
// chunk's last token, its share of the state it hands on.
//
// q, k, v and dO are exact bf16 operands; h, dH, A and dA are split as
// bf16 hi + lo and each of their products issued twice.  Accumulation and
// every output are fp32.
//
// 8 waves (two per SIMD).  Wave w works on row tile rw = w % 4 (tokens
// [16 rw, +16)) and half kh = w / 4: A and dA column tiles {2 kh, 2 kh + 1},
// dQ and dK key tiles [kh KT/32, +KT/32), dV columns [16 kh, +16) of each
// 32-column V slice.  V is walked in 32-column slices, each loaded one slice
// ahead; operands reduced over tokens come from LDS through the transposing
// read ds_read_b64_tr_b16.
//
// Keys beyond 128 (K = 256, 512): every dQ and dK column depends on the keys
// only through A and through its own key column, so one workgroup per
// (chunk, head, 128-key tile) runs the same kernel on its key tile (dA is a
// reduction over V and each tile forms it itself) and leaves its share of
// the gate terms in a partial record; dV, which sums over all keys, comes
// from chunk_bwd_bf16_wide.hip, as does the gate gradient from the partials.
// The state pass splits the keys the same way: the rows of the state and of
// its gradient evolve independently.
#include <hip/hip_runtime.h>

#include "gate_scan.h"
#include "mfma_common.h"
#include "sgla_internal.h"
#include "unit_map.h"

namespace sgla {
namespace {

using namespace mf;

constexpr int C = kChunk;
constexpr int NTG = 512;        // threads (8 waves)
constexpr int VS = 32;          // V slice width
constexpr int LDS_ = VS + 8;    // slice row stride (elements): V, dO, h, dH
constexpr int LDA = C + 8;      // A / dA row stride (elements)

template <int K>
struct GradLayout {
  static constexpr int LDQ = K + 8;              // Q / K row stride (elements)
  static constexpr int OFF_Q = 0;
  static constexpr int OFF_K = OFF_Q + C * LDQ * 2;
  static constexpr int OFF_A = OFF_K + C * LDQ * 2;        // hi plane, then lo
  static constexpr int OFF_V = OFF_A + 2 * C * LDA * 2;
  static constexpr int OFF_O = OFF_V + C * LDS_ * 2;       // dO slice
  static constexpr int OFF_H = OFF_O + C * LDS_ * 2;       // h slice, hi then lo
  static constexpr int OFF_DH = OFF_H + 2 * K * LDS_ * 2;  // dH slice, hi then lo
  static constexpr int OFF_F = OFF_DH + 2 * K * LDS_ * 2;  // floats below
  static constexpr int NF = 3 * C + 4 * C + 8;             // sb sc dv | R[2] Ks[2] | frob[8]
  static constexpr int BYTES = OFF_F + NF * 4;
  static_assert(BYTES <= 160 * 1024, "LDS budget");
  static_assert(OFF_K % 16 == 0 && OFF_A % 16 == 0 && OFF_V % 16 == 0 && OFF_O % 16 == 0 &&
                    OFF_H % 16 == 0 && OFF_DH % 16 == 0 && OFF_F % 16 == 0,
                "16-byte aligned areas");
};

// bf16 hi / lo halves of four floats, packed two to a word
__device__ __forceinline__ void split4(f32x4 x, u32x2& hi, u32x2& lo) {
  uint32_t h0, l0, h1, l1;
  split2(x[0], x[1], h0, l0);
  split2(x[2], x[3], h1, l1);
  hi = u32x2{h0, h1};
  lo = u32x2{l0, l1};
}

// x written as its bf16 hi into plane[i] and lo into plane[i + lo_off]
__device__ __forceinline__ void put_split(bf16* plane, int i, int lo_off, float x) {
  const bf16 hi = (bf16)x;
  plane[i] = hi;
  plane[i + lo_off] = (bf16)(x - (float)hi);
}

// KT keys per workgroup.  WIDE = false: KT = K, the whole chunk's
// gradients.  WIDE = true: K > KT; workgroup (chunk, head, key tile kz) of
// map_unit writes dq and dk of keys [kz KT, +KT) and its gate partial record
// wpart[(chunk H + head) (K / KT) + kz] = {r_c (64), dv_c k_c . (V dH^T)_c (64),
// <dH, h> over its key rows}; A and dV are left to the wide dV kernel.
template <int KT, bool WIDE>
__global__ void __launch_bounds__(NTG)
chunk_bwd_grad_bf16_kernel(const bf16* __restrict__ q, const bf16* __restrict__ k,
                           const bf16* __restrict__ v, const bf16* __restrict__ dout,
                           const float* __restrict__ g, const float* __restrict__ g_gamma, float scale,
                           int32_t H, int32_t Hkv, int32_t K, int32_t V, SeqLayout seqs, int32_t chunks_per_row,
                           const float* __restrict__ hbuf, const float* __restrict__ dhbuf,
                           float* __restrict__ dq, float* __restrict__ dk, float* __restrict__ dv,
                           float* __restrict__ dg, float* __restrict__ gpart, float* __restrict__ wpart) {
  using L = GradLayout<KT>;
  constexpr int LDQ = L::LDQ;
  constexpr int NKT = KT / 16;         // 16-key tiles of dQ / dK
  constexpr int NKH = NKT / 2;         // per wave
  constexpr int KSTEP = KT / 32;       // 32-deep steps over the keys
  static_assert(NKH >= 2 && KSTEP >= 2, "KT");
  __shared__ __attribute__((aligned(16))) char smem[L::BYTES];
  bf16* const sQ = reinterpret_cast<bf16*>(smem + L::OFF_Q);
  bf16* const sK = reinterpret_cast<bf16*>(smem + L::OFF_K);
  bf16* const sA = reinterpret_cast<bf16*>(smem + L::OFF_A);
  bf16* const sV = reinterpret_cast<bf16*>(smem + L::OFF_V);
  bf16* const sO = reinterpret_cast<bf16*>(smem + L::OFF_O);
  bf16* const sH = reinterpret_cast<bf16*>(smem + L::OFF_H);
  bf16* const sdH = reinterpret_cast<bf16*>(smem + L::OFF_DH);
  float* const sb = reinterpret_cast<float*>(smem + L::OFF_F);
  float* const ssc = sb + C;
  float* const sdv = sb + 2 * C;
  float* const sR = sb + 3 * C;        // [2][C]
  float* const sKs = sb + 5 * C;       // [2][C]
  float* const sFrob = sb + 7 * C;     // [8]
  constexpr int ALO = C * LDA;         // offset of the lo planes
  constexpr int HLO = KT * LDS_;

  int gc, hd, kz = 0;
  if constexpr (WIDE) {
    // the key tiles of one (chunk, head) run on one XCD, whose L2 then
    // serves their repeated reads of V and dO
    const UnitMap um = map_unit((int32_t)blockIdx.x, K / KT, H, 1, seqs.num_chunks);
    if (!um.valid) return;
    gc = um.rank;
    hd = um.hk;
    kz = um.vt;
  } else {
    gc = blockIdx.x;
    hd = blockIdx.y;
  }
  const int kb = kz * KT;              // first key of the tile
  int64_t t0;
  int cl;
  if (seqs.chunk_table != nullptr) {
    const ChunkEntry e = seqs.chunk_table[gc];
    t0 = e.t0;
    cl = e.len;
  } else {
    const int row = gc / chunks_per_row;
    const int m = gc - row * chunks_per_row;
    t0 = (int64_t)row * seqs.T + (int64_t)m * seqs.chunk;
    cl = min(seqs.chunk, seqs.T - m * seqs.chunk);
  }
  const int tid = threadIdx.x, lane = tid & 63, g4 = lane >> 4, r = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index, uniform
  const int rw = w & 3, kh = w >> 2;
  const int kt0 = kh * NKH;
  const int hk = hd / (H / Hkv);   // kv head whose k and v rows this query head reads
  const int64_t RSV = (int64_t)H * V, RKV = (int64_t)Hkv * V;   // dout and v row strides
  const int64_t KV = (int64_t)K * V;
  const float* hu = hbuf + ((int64_t)gc * H + hd) * KV + (int64_t)kb * V;
  const float* dhu = dhbuf + ((int64_t)gc * H + hd) * KV + (int64_t)kb * V;

  // ---- Q and K rows of the key tile (zero past the chunk's end) and the gates
  {
    constexpr int PR = KT / 8;                // 16-byte pieces per row
    constexpr int NPC = C * PR / NTG;
    static_assert(NPC * NTG == C * PR, "staging split");
    uint4 qx[NPC], kx[NPC];
#pragma unroll
    for (int u = 0; u < NPC; ++u) {
      const int p = tid + NTG * u;
      const int c = p / PR, e = 8 * (p % PR);
      qx[u] = make_uint4(0u, 0u, 0u, 0u);
      kx[u] = make_uint4(0u, 0u, 0u, 0u);
      if (c < cl) {
        qx[u] = *reinterpret_cast<const uint4*>(q + ((t0 + c) * H + hd) * K + kb + e);
        kx[u] = *reinterpret_cast<const uint4*>(k + ((t0 + c) * Hkv + hk) * K + kb + e);
      }
    }
#pragma unroll
    for (int u = 0; u < NPC; ++u) {
      const int p = tid + NTG * u;
      *reinterpret_cast<uint4*>(sQ + (p / PR) * LDQ + 8 * (p % PR)) = qx[u];
      *reinterpret_cast<uint4*>(sK + (p / PR) * LDQ + 8 * (p % PR)) = kx[u];
    }
  }
  if (w == 0) {
    float b;
    if (g != nullptr) b = wave_cumsum_log2(lane < cl ? g[(t0 + lane) * H + hd] : 0.f);
    else if (g_gamma != nullptr) b = (float)min(lane + 1, cl) * (g_gamma[hd] * kRcpLn2f);
    else b = 0.f;
    const float blast = __shfl(b, C - 1, 64);
    sb[lane] = b;
    ssc[lane] = exp2f(b) * scale;
    sdv[lane] = exp2f(blast - b);
  }

  // ---- slice registers: V and dO as 4-element bf16 pieces, h and dH as
  //      4-float pieces, loaded one slice ahead --------------------------------
  constexpr int PVS = C * (VS / 4);
  constexpr int NVS = PVS / NTG;
  constexpr int PHS = KT * (VS / 4);
  constexpr int NHS = PHS / NTG;
  static_assert(NVS * NTG == PVS && NHS * NTG == PHS, "slice split");
  uint2 vx[NVS], ox[NVS];
  f32x4 hx[NHS], dhx[NHS];
  auto load_slice = [&](int vs) {
#pragma unroll
    for (int u = 0; u < NVS; ++u) {
      const int p = tid + NTG * u;
      const int row = p / (VS / 4), c4 = p % (VS / 4);
      vx[u] = make_uint2(0u, 0u);
      ox[u] = make_uint2(0u, 0u);
      if (row < cl) {
        const int64_t col = vs * VS + 4 * c4;
        vx[u] = *reinterpret_cast<const uint2*>(v + (t0 + row) * RKV + (int64_t)hk * V + col);
        ox[u] = *reinterpret_cast<const uint2*>(dout + (t0 + row) * RSV + (int64_t)hd * V + col);
      }
    }
#pragma unroll
    for (int u = 0; u < NHS; ++u) {
      const int p = tid + NTG * u;
      const int64_t off = (int64_t)(p / (VS / 4)) * V + vs * VS + 4 * (p % (VS / 4));
      hx[u] = *reinterpret_cast<const f32x4*>(hu + off);
      dhx[u] = *reinterpret_cast<const f32x4*>(dhu + off);
    }
  };
  float frob = 0.f;   // this thread's share of <dH, h> over the chunk record
  auto store_slice = [&]() {
#pragma unroll
    for (int u = 0; u < NVS; ++u) {
      const int p = tid + NTG * u;
      const int o = (p / (VS / 4)) * LDS_ + 4 * (p % (VS / 4));
      *reinterpret_cast<uint2*>(sV + o) = vx[u];
      *reinterpret_cast<uint2*>(sO + o) = ox[u];
    }
#pragma unroll
    for (int u = 0; u < NHS; ++u) {
      const int p = tid + NTG * u;
      const int o = (p / (VS / 4)) * LDS_ + 4 * (p % (VS / 4));
      u32x2 hi, lo;
      split4(hx[u], hi, lo);
      *reinterpret_cast<u32x2*>(sH + o) = hi;
      *reinterpret_cast<u32x2*>(sH + HLO + o) = lo;
      split4(dhx[u], hi, lo);
      *reinterpret_cast<u32x2*>(sdH + o) = hi;
      *reinterpret_cast<u32x2*>(sdH + HLO + o) = lo;
      const f32x4 x = hx[u], y = dhx[u];
      frob += x[0] * y[0] + x[1] * y[1] + x[2] * y[2] + x[3] * y[3];
    }
  };
  load_slice(0);
  __syncthreads();   // Q, K and the gates staged
  // the per-token factors this lane needs, read once: rows c = 16 rw + 4 g + i
  // and columns j = 16 (2 kh + t) + r of the A / dA tiles
  const f32x4 b_c = *reinterpret_cast<const f32x4*>(sb + 16 * rw + 4 * g4);
  const f32x4 sc_c = *reinterpret_cast<const f32x4*>(ssc + 16 * rw + 4 * g4);
  const f32x4 dv_c = *reinterpret_cast<const f32x4*>(sdv + 16 * rw + 4 * g4);
  const float b_j[2] = {sb[16 * (2 * kh) + r], sb[16 * (2 * kh + 1) + r]};

  // ---- A = scale (Q K^T) (.) M: row tile rw against column tiles 2 kh,
  //      2 kh + 1 (tiles above the diagonal come out as zeros) -----------------
  if constexpr (!WIDE) {
    f32x4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int s = 0; s < KSTEP; ++s) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(sQ + (16 * rw + r) * LDQ + 32 * s + 8 * g4);
#pragma unroll
      for (int t = 0; t < 2; ++t)
        acc[t] = mfma(a, *reinterpret_cast<const bf16x8*>(sK + (16 * (2 * kh + t) + r) * LDQ + 32 * s + 8 * g4),
                      acc[t]);
    }
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int j = 16 * (2 * kh + t) + r;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int c = 16 * rw + 4 * g4 + i;
        put_split(sA, c * LDA + j, ALO, j <= c ? acc[t][i] * exp2f(b_c[i] - b_j[t]) * scale : 0.f);
      }
    }
  }

  // ---- walk V in 32-column slices ----------------------------------------------
  f32x4 dAacc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
  f32x4 dQi[NKH], dKs[NKH];
#pragma unroll
  for (int t = 0; t < NKH; ++t) {
    dQi[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    dKs[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const int cs0 = rw >= 2 ? 1 : 0;   // first 32-token block with A[c][j] != 0 for j in tile rw
  for (int vs = 0; vs < V / VS; ++vs) {
    __syncthreads();   // previous slice's reads done (first pass: A published)
    store_slice();
    if (vs + 1 < V / VS) load_slice(vs + 1);
    __syncthreads();
    // dA += dO V^T, dQ_inter += dO h^T, dK_state += V dH^T over this slice
    {
      const bf16x8 ao = *reinterpret_cast<const bf16x8*>(sO + (16 * rw + r) * LDS_ + 8 * g4);
      const bf16x8 av = *reinterpret_cast<const bf16x8*>(sV + (16 * rw + r) * LDS_ + 8 * g4);
#pragma unroll
      for (int t = 0; t < 2; ++t)
        dAacc[t] = mfma(ao, *reinterpret_cast<const bf16x8*>(sV + (16 * (2 * kh + t) + r) * LDS_ + 8 * g4),
                        dAacc[t]);
#pragma unroll
      for (int t = 0; t < NKH; ++t) {
        const int o = (16 * (kt0 + t) + r) * LDS_ + 8 * g4;
        const bf16x8 hh = *reinterpret_cast<const bf16x8*>(sH + o);
        const bf16x8 hl = *reinterpret_cast<const bf16x8*>(sH + HLO + o);
        const bf16x8 dh = *reinterpret_cast<const bf16x8*>(sdH + o);
        const bf16x8 dl = *reinterpret_cast<const bf16x8*>(sdH + HLO + o);
        dQi[t] = mfma(ao, hh, dQi[t]);
        dKs[t] = mfma(av, dh, dKs[t]);
        dQi[t] = mfma(ao, hl, dQi[t]);
        dKs[t] = mfma(av, dl, dKs[t]);
      }
    }
    // dV rows [16 rw, +16), columns [16 kh, +16) of the slice
    if constexpr (!WIDE) {
      f32x4 in = {0.f, 0.f, 0.f, 0.f}, st = in;
      for (int cs = cs0; cs < 2; ++cs) {
        const int c0 = 32 * cs + 8 * g4;
        const bf16x8 ah = cat(tr_read(sA, LDA, c0, 16 * rw), tr_read(sA, LDA, c0 + 4, 16 * rw));
        const bf16x8 al = cat(tr_read(sA + ALO, LDA, c0, 16 * rw), tr_read(sA + ALO, LDA, c0 + 4, 16 * rw));
        const bf16x8 bo = cat(tr_read(sO, LDS_, c0, 16 * kh), tr_read(sO, LDS_, c0 + 4, 16 * kh));
        in = mfma(ah, bo, in);
        in = mfma(al, bo, in);
      }
#pragma unroll
      for (int s = 0; s < KSTEP; ++s) {
        const bf16x8 ak = *reinterpret_cast<const bf16x8*>(sK + (16 * rw + r) * LDQ + 32 * s + 8 * g4);
        const int k0 = 32 * s + 8 * g4;
        const bf16x8 bh = cat(tr_read(sdH, LDS_, k0, 16 * kh), tr_read(sdH, LDS_, k0 + 4, 16 * kh));
        const bf16x8 bl = cat(tr_read(sdH + HLO, LDS_, k0, 16 * kh), tr_read(sdH + HLO, LDS_, k0 + 4, 16 * kh));
        st = mfma(ak, bh, st);
        st = mfma(ak, bl, st);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = 16 * rw + 4 * g4 + i;
        if (j < cl) dv[((t0 + j) * H + hd) * (int64_t)V + vs * VS + 16 * kh + r] = in[i] + dv_c[i] * st[i];
      }
    }
  }
  __syncthreads();   // every read of A done

  // ---- dA masked and scaled, into the A planes -------------------------------
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int j = 16 * (2 * kh + t) + r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = 16 * rw + 4 * g4 + i;
      put_split(sA, c * LDA + j, ALO, j <= c ? dAacc[t][i] * exp2f(b_c[i] - b_j[t]) * scale : 0.f);
    }
  }
  // Frobenius product <dH, h> of the whole chunk record
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) frob += __shfl_xor(frob, d, 64);
  if (lane == 0) sFrob[w] = frob;
  __syncthreads();

  // ---- dQ = diag(sc) dQ_inter + dA K;  dK = dA^T Q + diag(dv) dK_state --------
  float rq[4] = {0.f, 0.f, 0.f, 0.f}, rk[4] = {0.f, 0.f, 0.f, 0.f}, ks4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int t = 0; t < NKH; ++t) {
    const int kt = kt0 + t;
    f32x4 aq = {0.f, 0.f, 0.f, 0.f}, ak = aq;
    // dA K: dA[c][j] = 0 for j > c, so tile rw needs token blocks j0 <= its rows
    for (int js = 0; js <= cs0; ++js) {
      const bf16* arow = sA + (16 * rw + r) * LDA + 32 * js + 8 * g4;
      const bf16x8 ah = *reinterpret_cast<const bf16x8*>(arow);
      const bf16x8 al = *reinterpret_cast<const bf16x8*>(arow + ALO);
      const int j0 = 32 * js + 8 * g4;
      const bf16x8 bk = cat(tr_read(sK, LDQ, j0, 16 * kt), tr_read(sK, LDQ, j0 + 4, 16 * kt));
      aq = mfma(ah, bk, aq);
      aq = mfma(al, bk, aq);
    }
    // dA^T Q: token blocks c0 >= the tile's rows
    for (int cs = cs0; cs < 2; ++cs) {
      const int c0 = 32 * cs + 8 * g4;
      const bf16x8 ah = cat(tr_read(sA, LDA, c0, 16 * rw), tr_read(sA, LDA, c0 + 4, 16 * rw));
      const bf16x8 al = cat(tr_read(sA + ALO, LDA, c0, 16 * rw), tr_read(sA + ALO, LDA, c0 + 4, 16 * rw));
      const bf16x8 bq = cat(tr_read(sQ, LDQ, c0, 16 * kt), tr_read(sQ, LDQ, c0 + 4, 16 * kt));
      ak = mfma(ah, bq, ak);
      ak = mfma(al, bq, ak);
    }
    const int col = 16 * kt + r;
    float qv[4], kv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      qv[i] = (float)sQ[(16 * rw + 4 * g4 + i) * LDQ + col];
      kv[i] = (float)sK[(16 * rw + 4 * g4 + i) * LDQ + col];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = 16 * rw + 4 * g4 + i;
      const float xq = sc_c[i] * dQi[t][i] + aq[i];
      const float xk = ak[i] + dv_c[i] * dKs[t][i];
      rq[i] += qv[i] * xq;
      rk[i] += kv[i] * xk;
      ks4[i] += kv[i] * dKs[t][i];
      if (c < cl) {
        dq[((t0 + c) * H + hd) * (int64_t)K + kb + col] = xq;
        dk[((t0 + c) * H + hd) * (int64_t)K + kb + col] = xk;
      }
    }
  }
  // row sums over the 16 lanes of a column group, one partial per key half
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int d = 8; d >= 1; d >>= 1) {
      rq[i] += __shfl_xor(rq[i], d, 64);
      rk[i] += __shfl_xor(rk[i], d, 64);
      ks4[i] += __shfl_xor(ks4[i], d, 64);
    }
    if (r == 0) {
      const int c = 16 * rw + 4 * g4 + i;
      sR[kh * C + c] = rq[i] - rk[i];
      sKs[kh * C + c] = dv_c[i] * ks4[i];
    }
  }
  __syncthreads();

  if constexpr (WIDE) {
    // the tile's gate terms, reduced over key tiles by the wide gate kernel
    if (w == 0) {
      float* rec = wpart + (((int64_t)gc * H + hd) * (K / KT) + kz) * kWidePart;
      rec[lane] = sR[lane] + sR[C + lane];
      rec[C + lane] = sKs[lane] + sKs[C + lane];
      if (lane == 0) {
        float frob_all = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) frob_all += sFrob[i];
        rec[2 * C] = frob_all;
      }
    }
    return;
  }
  // ---- gate gradient: reverse cumulative sum over the chunk ---------------
  if (w == 0) {
    float frob_all = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) frob_all += sFrob[i];
    // the chunk's share of the state it hands on, at its last real token
    double extra = (double)sKs[lane] + (double)sKs[C + lane];
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) extra += __shfl_xor(extra, d, 64);
    double x = lane < cl ? (double)sR[lane] + (double)sR[C + lane] : 0.0;
    if (lane == cl - 1) x += (double)exp2f(sb[C - 1]) * (double)frob_all + extra;
    // reverse inclusive scan: lane c gets x_c + ... + x_63
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const double y = __shfl_down(x, d, 64);
      if (lane + d < 64) x += y;
    }
    if (dg != nullptr && lane < cl) dg[(t0 + lane) * H + hd] = (float)x;
    if (gpart != nullptr) {
      double s = lane < cl ? x : 0.0;
#pragma unroll
      for (int d = 32; d >= 1; d >>= 1) s += __shfl_xor(s, d, 64);
      if (lane == 0) gpart[(int64_t)gc * H + hd] = (float)s;
    }
  }
}

// ---------------------------------------------------------------------------
// State pass on the bf16 matrix cores.  For each (sequence, head, 32-column
// V tile) one workgroup runs the forward recurrence h <- dall h + K^T diag(dv)
// V and stores the state entering every chunk; another runs the reverse
// recurrence dH <- dall dH + Q^T diag(sc) dO from dht and stores the gradient
// of the state leaving every chunk, then dh0.  K (Q) is an exact bf16
// operand; the weighted V (dO) is split into bf16 hi + lo planes once per
// chunk in LDS.  A workgroup covers KT state rows (key tile kz: rows
// [kz KT, +KT), KT = K up to 256) and 32 columns; 4 waves, wave w owns rows
// [w KT/4, +KT/4) of the tile as 16 x 16 fp32 accumulators.
// ---------------------------------------------------------------------------
constexpr int NTS = 256;        // state-pass threads (4 waves)
constexpr int LDY = VS + 8;     // V / dO tile row stride (elements)

template <int KT>
__global__ void __launch_bounds__(NTS)
chunk_bwd_state_bf16_kernel(const bf16* __restrict__ q, const bf16* __restrict__ k,
                            const bf16* __restrict__ v, const bf16* __restrict__ dout,
                            const float* __restrict__ g, const float* __restrict__ g_gamma,
                            const float* __restrict__ h0, const float* __restrict__ dht,
                            float* __restrict__ dh0, float scale, int32_t H, int32_t Hkv, int32_t K,
                            int32_t V, StateLayout sl, SeqLayout seqs, int32_t chunks_per_row,
                            float* __restrict__ hbuf, float* __restrict__ dhbuf) {
  constexpr int LDX = KT + 16;         // K / Q row stride (elements)
  constexpr int RT = KT / 64;          // 16-row state tiles per wave (KT/4 rows)
  constexpr int PRX = KT / 8;          // 16-byte pieces per K / Q row
  constexpr int NX = C * PRX / NTS;    // per thread
  constexpr int PY = C * (VS / 8);     // 16-byte pieces of the V / dO tile (256)
  static_assert(NX * NTS == C * PRX && PY == NTS && RT >= 1, "staging split");
  __shared__ __attribute__((aligned(16))) bf16 sX[C * LDX];      // K rows (forward) or Q rows (reverse)
  __shared__ __attribute__((aligned(16))) bf16 sY[C * LDY];      // V tile (forward) or dO tile (reverse)
  __shared__ __attribute__((aligned(16))) bf16 sYd[2 * C * LDY]; // weighted tile, hi then lo
  __shared__ float sW[C];              // 2^(b_last - b) (forward) or scale 2^b (reverse)
  __shared__ float sDall;

  // workgroups 2 u and 2 u + 1 run unit u's forward and reverse passes, so
  // the longest units start both at once
  const bool rev = (blockIdx.x & 1) != 0;
  const int bid = (int)(blockIdx.x >> 1);
  const int nvt = V / VS;
  const UnitMap um = map_unit(bid, nvt * (K / KT), H, 1, seqs.num_seqs);
  if (!um.valid) return;
  const int hd = um.hd, kz = um.vt / nvt, vt = um.vt - kz * nvt;
  const int hk = hd / (H / Hkv);   // kv head whose k and v rows this query head reads
  int64_t bos;
  int32_t len, seq, chunk0;
  if (seqs.seq_table != nullptr) {
    const SeqEntry e = seqs.seq_table[um.rank];
    bos = e.bos;
    len = e.len;
    seq = e.seq;
    chunk0 = e.chunk0;
  } else {
    bos = (int64_t)um.rank * seqs.T;
    len = seqs.T;
    seq = um.rank;
    chunk0 = um.rank * chunks_per_row;
  }
  const int nchunks = (len + seqs.chunk - 1) / seqs.chunk;
  const int tid = threadIdx.x, lane = tid & 63, g4 = lane >> 4, r = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index, uniform
  const int krow0 = kz * KT + w * (KT / 4);
  const int64_t KV = (int64_t)K * V;
  const int64_t ucol = (int64_t)vt * VS;

  // state tiles: hs[rt][ct][i] = S[krow0 + 16 rt + 4 g + i][ucol + 16 ct + r]
  f32x4 hs[RT][2];
  {
    const float* init = rev ? dht : h0;
    const float* iu = init != nullptr ? init + ((int64_t)seq * H + hd) * KV : nullptr;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int ct = 0; ct < 2; ++ct)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          hs[rt][ct][i] = iu != nullptr ? iu[(int64_t)(krow0 + 16 * rt + 4 * g4 + i) * sl.rs +
                                             (ucol + 16 * ct + r) * sl.cs]
                                        : 0.f;
  }

  // chunk m's rows and gate, loaded into registers one iteration ahead
  uint4 xx[NX], yx;
  float gx = 0.f;
  // reverse: q and dout rows of the query head; forward: k and v rows of its kv head
  const bf16* xsrc = (rev ? q + hd * K : k + hk * K) + kz * KT;
  const bf16* ysrc = rev ? dout + hd * V : v + hk * V;
  const int64_t xrs = (int64_t)(rev ? H : Hkv) * K, yrs = (int64_t)(rev ? H : Hkv) * V;
  auto load_chunk = [&](int it) {
    const int m = rev ? nchunks - 1 - it : it;
    const int64_t t0 = bos + (int64_t)m * seqs.chunk;
    const int cl = min(seqs.chunk, len - m * seqs.chunk);
#pragma unroll
    for (int u = 0; u < NX; ++u) {
      const int p = tid + NTS * u;
      const int c = p / PRX;
      xx[u] = make_uint4(0u, 0u, 0u, 0u);
      if (c < cl) xx[u] = *reinterpret_cast<const uint4*>(xsrc + (t0 + c) * xrs + 8 * (p % PRX));
    }
    {
      const int c = tid / (VS / 8);
      yx = make_uint4(0u, 0u, 0u, 0u);
      if (c < cl) yx = *reinterpret_cast<const uint4*>(ysrc + (t0 + c) * yrs + ucol + 8 * (tid % (VS / 8)));
    }
    if (w == 0 && g != nullptr) gx = lane < cl ? g[(t0 + lane) * H + hd] : 0.f;
  };
  if (nchunks > 0) load_chunk(0);
  for (int it = 0; it < nchunks; ++it) {
    const int m = rev ? nchunks - 1 - it : it;
    const int cl = min(seqs.chunk, len - m * seqs.chunk);
    // record: forward -> the state entering chunk m; reverse -> the gradient
    // of the state leaving chunk m
    float* rec = (rev ? dhbuf : hbuf) + ((int64_t)(chunk0 + m) * H + hd) * KV + ucol;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int ct = 0; ct < 2; ++ct)
#pragma unroll
        for (int i = 0; i < 4; ++i) rec[(int64_t)(krow0 + 16 * rt + 4 * g4 + i) * V + 16 * ct + r] = hs[rt][ct][i];
#pragma unroll
    for (int u = 0; u < NX; ++u) {
      const int p = tid + NTS * u;
      *reinterpret_cast<uint4*>(sX + (p / PRX) * LDX + 8 * (p % PRX)) = xx[u];
    }
    *reinterpret_cast<uint4*>(sY + (tid / (VS / 8)) * LDY + 8 * (tid % (VS / 8))) = yx;
    if (w == 0) {
      float b;
      if (g != nullptr) b = wave_cumsum_log2(gx);
      else if (g_gamma != nullptr) b = (float)min(lane + 1, cl) * (g_gamma[hd] * kRcpLn2f);
      else b = 0.f;
      const float blast = __shfl(b, C - 1, 64);
      sW[lane] = rev ? exp2f(b) * scale : exp2f(blast - b);
      if (lane == 0) sDall = exp2f(blast);
    }
    __syncthreads();   // rows, tile and weights staged
    // weighted tile, split: thread tid takes 8 columns of one token
    {
      const int c = tid / (VS / 8), c8 = 8 * (tid % (VS / 8));
      const u32x4 raw = *reinterpret_cast<const u32x4*>(sY + c * LDY + c8);
      const float wc = sW[c];
      float x[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[2 * e] = bf_lo(raw[e]) * wc;
        x[2 * e + 1] = bf_hi(raw[e]) * wc;
      }
      bf16x8 hi, lo;
      split8(x, hi, lo);
      *reinterpret_cast<bf16x8*>(sYd + c * LDY + c8) = hi;
      *reinterpret_cast<bf16x8*>(sYd + C * LDY + c * LDY + c8) = lo;
    }
    __syncthreads();   // weighted tile split
    // the next chunk's rows load from here (issued before the split they
    // delayed it, and with it every wave's first product: ~2 % of the pass)
    if (it + 1 < nchunks) load_chunk(it + 1);
    const float dall = sDall;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) hs[rt][ct] *= dall;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int c0 = 32 * s + 8 * g4;
      bf16x8 bh[2], bl[2];
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        bh[ct] = cat(tr_read(sYd, LDY, c0, 16 * ct), tr_read(sYd, LDY, c0 + 4, 16 * ct));
        bl[ct] = cat(tr_read(sYd + C * LDY, LDY, c0, 16 * ct), tr_read(sYd + C * LDY, LDY, c0 + 4, 16 * ct));
      }
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        // A operand: X^T[key krow0 + 16 rt + r][token c0 + e]
        const int xc = w * (KT / 4) + 16 * rt;   // the tile's key column in sX
        const bf16x8 a = cat(tr_read(sX, LDX, c0, xc), tr_read(sX, LDX, c0 + 4, xc));
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
          hs[rt][ct] = mfma(a, bh[ct], hs[rt][ct]);
          hs[rt][ct] = mfma(a, bl[ct], hs[rt][ct]);
        }
      }
    }
    __syncthreads();   // every read of this chunk's stage done
  }
  if (rev && dh0 != nullptr) {
    float* du = dh0 + ((int64_t)seq * H + hd) * KV;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int ct = 0; ct < 2; ++ct)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          du[(int64_t)(krow0 + 16 * rt + 4 * g4 + i) * sl.rs + (ucol + 16 * ct + r) * sl.cs] = hs[rt][ct][i];
  }
}

template <int KT, bool WIDE>
hipError_t launch_grad_k(const ChunkBwdParams& p, int32_t chunks_per_row, hipStream_t stream) {
  const dim3 grid = WIDE ? dim3((unsigned)unit_grid(p.seqs.num_chunks, p.H, 1, p.K / KT))
                         : dim3((unsigned)p.seqs.num_chunks, (unsigned)p.H);
  hipLaunchKernelGGL((chunk_bwd_grad_bf16_kernel<KT, WIDE>), grid, dim3(NTG), 0, stream,
                     static_cast<const bf16*>(p.q), static_cast<const bf16*>(p.k),
                     static_cast<const bf16*>(p.v), static_cast<const bf16*>(p.dout), p.g, p.g_gamma,
                     p.scale, p.H, p.Hkv, p.K, p.V, p.seqs, chunks_per_row, p.hbuf, p.dhbuf, p.dq, p.dk, p.dv,
                     p.dg, p.dg_gamma != nullptr ? p.gpart : nullptr, p.wpart);
  return hipGetLastError();
}

template <int KT>
hipError_t launch_state_k(const ChunkBwdParams& p, int32_t chunks_per_row, hipStream_t stream) {
  const int units = (int)unit_grid(p.seqs.num_seqs, p.H, 1, (p.V / VS) * (p.K / KT));
  hipLaunchKernelGGL((chunk_bwd_state_bf16_kernel<KT>), dim3((unsigned)(2 * units)), dim3(NTS), 0, stream,
                     static_cast<const bf16*>(p.q), static_cast<const bf16*>(p.k),
                     static_cast<const bf16*>(p.v), static_cast<const bf16*>(p.dout), p.g, p.g_gamma, p.h0,
                     p.dht, p.dh0, p.scale, p.H, p.Hkv, p.K, p.V, p.sl, p.seqs, chunks_per_row, p.hbuf,
                     p.dhbuf);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_chunk_bwd_state_bf16(const ChunkBwdParams& p, int32_t chunks_per_row, hipStream_t stream) {
  if (!bwd_bf16_grad(p.qkv_bf16 != 0, p.K) || p.V % VS != 0) return hipErrorInvalidValue;
  if (p.seqs.num_seqs == 0) return hipSuccess;
  switch (p.K) {
    case 64: return launch_state_k<64>(p, chunks_per_row, stream);
    case 128: return launch_state_k<128>(p, chunks_per_row, stream);
    default: return launch_state_k<256>(p, chunks_per_row, stream);   // K = 256, 512
  }
}

hipError_t launch_chunk_bwd_grad_bf16(const ChunkBwdParams& p, int32_t chunks_per_row, hipStream_t stream) {
  if (!bwd_bf16_grad(p.qkv_bf16 != 0, p.K) || p.V % VS != 0) return hipErrorInvalidValue;
  if (p.seqs.num_chunks == 0) return hipSuccess;
  switch (p.K) {
    case 64: return launch_grad_k<64, false>(p, chunks_per_row, stream);
    case 128: return launch_grad_k<128, false>(p, chunks_per_row, stream);
    default: {   // K = 256, 512: key tiles of 128, then dV and the gate gradient
      if (p.wpart == nullptr || p.V % kWideDvCols != 0) return hipErrorInvalidValue;
      hipError_t e = launch_grad_k<128, true>(p, chunks_per_row, stream);
      if (e == hipSuccess) e = launch_chunk_bwd_dv_wide(p, chunks_per_row, stream);
      if (e == hipSuccess) e = launch_chunk_bwd_gate_wide(p, chunks_per_row, stream);
      return e;
    }
  }
}

}  // namespace sgla
