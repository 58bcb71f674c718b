// Backward of the chunked Simple GLA forward (page "flash-linear-attention 中的
// Simple GLA", section 三: the backward reuses three common passes -- the
// state-gradient pass, the q/k/gate gradients and the v gradient -- computes
// the state trajectory in fp32 for gradient accuracy, and recovers the gate
// gradient with a reverse chunk-local cumulative sum; section 五: the tests
// check dq, dk, dv, dg and dh0).
//
// Loss gradients of  L = sum_t <do_t, o_t> + sum_n <dht_n, final_state_n>.
// Per chunk n of one (sequence, head), b the chunk-local cumulative log2 gate,
// sc_c = scale 2^b_c, dv_j = 2^(b_last - b_j), dall = 2^b_last, h_n the state
// entering the chunk and dH_n the gradient of the state after it:
//
//   state pass  (forward)  h_{n+1} = dall h_n + K^T diag(dv) V
//               (reverse)  dH_{n-1} = dall_n dH_n + Q_n^T diag(sc_n) dO_n,
//                          starting from dht; dh0 = the gradient of h_0
//   per chunk   A  = scale (Q K^T) (.) M,  M_cj = 2^(b_c - b_j) (j <= c)
//               dA = scale (dO V^T) (.) M
//               dQ = diag(sc) dO h_n^T + dA K
//               dK = dA^T Q + diag(dv) V dH_n^T
//               dV = A^T dO + diag(dv) K dH_n
//   gate        every term depends on the log gates only through differences
//               of running sums, so the gradient with respect to the running
//               sum at token t is  r_t = q_t . dq_t - k_t . dk_t, plus, at the
//               chunk's last token, the chunk's share of the state it hands
//               on: <dH_n, h_{n+1}> = dall <dH_n, h_n> + sum_j k_j . (dv_j V dH_n^T)_j.
//               dg is the reverse cumulative sum of r over the chunk; with
//               g_gamma its gradient is the sum of dg over every token.
//
// Grouped kv heads: query head h reads the k and v rows of kv head
// h / (H / Hkv); dk and dv come out per query head and kv_group_sum_kernel
// adds each group's query heads (the chain rule through the head repeat).
//
// The kernels below run every product on the fp32 matrix cores
// (v_mfma_f32_16x16x4_f32), so inputs are used exactly and states, gradients
// and accumulation are fp32; they serve float32 inputs and bf16 inputs with
// K in {16, 32}.  bf16 inputs with K in {64, 128, 256, 512} take the
// bf16-matrix-core passes of chunk_bwd_bf16.hip instead.
// Operand layout, per lane l with g = l / 16 and r = l % 16:
//   A operand A[m = r][k = g], B operand B[k = g][n = r],
//   result acc[i] = D[m = 4 g + i][n = r].
#include <hip/hip_runtime.h>

#include "gate_scan.h"
#include "row_stage.h"
#include "sgla_internal.h"
#include "unit_map.h"

namespace sgla {
namespace {

using stage::load4;
using stage::RowTile;

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int C = kChunk;
constexpr int NT = 256;           // threads (4 waves)
constexpr int VT = 32;            // V columns per state-pass workgroup and per slice
constexpr int LDT = VT + 4;       // row stride of 32-column tiles (floats)
constexpr int LDA = C + 4;        // row stride of the 64 x 64 A / dA tile
constexpr float kRcpLn2f = 1.44269504088896341f;

__device__ __forceinline__ f32x4 mfma4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// K rows x 32 columns of a [K][V] fp32 record, columns [c0, c0 + 32), by NTH
// threads.
template <int K, int NTH>
struct RecTile {
  static constexpr int P = K * (VT / 4);          // 16-byte pieces
  static constexpr int N = (P + NTH - 1) / NTH;   // per thread
  f32x4 x[N];
  __device__ __forceinline__ void load(const float* src, int64_t V, int64_t c0) {
#pragma unroll
    for (int u = 0; u < N; ++u) {
      const int i = threadIdx.x + u * NTH;
      x[u] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (P % NTH == 0 || i < P) x[u] = load4(src + (i / (VT / 4)) * V + c0 + 4 * (i % (VT / 4)));
    }
  }
  __device__ __forceinline__ void store(float* dst) const {
#pragma unroll
    for (int u = 0; u < N; ++u) {
      const int i = threadIdx.x + u * NTH;
      if (P % NTH == 0 || i < P)
        *reinterpret_cast<f32x4*>(dst + (i / (VT / 4)) * LDT + 4 * (i % (VT / 4))) = x[u];
    }
  }
};

// Where a (sequence, head) unit's tokens and chunk records are.
struct SeqInfo {
  int64_t bos;
  int32_t len, seq, chunk0;
};
__device__ __forceinline__ SeqInfo seq_info(const SeqLayout& seqs, int rank, int chunks_per_row) {
  SeqInfo s;
  if (seqs.seq_table != nullptr) {
    const SeqEntry e = seqs.seq_table[rank];
    s.bos = e.bos;
    s.len = e.len;
    s.seq = e.seq;
    s.chunk0 = e.chunk0;
  } else {
    s.bos = (int64_t)rank * seqs.T;
    s.len = seqs.T;
    s.seq = rank;
    s.chunk0 = rank * chunks_per_row;
  }
  return s;
}

// Chunk-local cumulative log2 gate of the chunk starting at token t0 with cl
// tokens, for lane = token offset; padding tokens add nothing.  Wave-wide.
// lo receives the rounding remainder of a per-token gate's running sum (0
// for the per-head decay), so differences of two running gates stay exact
// to fp32 after a very negative gate.
__device__ __forceinline__ float chunk_gate(const float* g, const float* g_gamma, int H, int hd,
                                            int64_t t0, int cl, float& lo) {
  const int lane = threadIdx.x & 63;
  lo = 0.f;
  if (g != nullptr) return wave_cumsum_log2_split(lane < cl ? g[(t0 + lane) * H + hd] : 0.f, lo);
  if (g_gamma != nullptr) return (float)min(lane + 1, cl) * (g_gamma[hd] * kRcpLn2f);
  return 0.f;
}

// ---------------------------------------------------------------------------
// State pass.  For each (sequence, head, 32-column V tile) one workgroup runs
// the forward recurrence and stores the state entering every chunk, and
// another runs the reverse recurrence of the state gradient and stores the
// gradient of the state leaving every chunk, then dh0.
// The K x 32 (gradient) state stays in MFMA accumulators: wave w owns 16 x 16
// tiles st = w + 4 s (rows 16 (st / 2), columns 16 (st % 2)).
// ---------------------------------------------------------------------------
template <int K, typename TIn>
__global__ void __launch_bounds__(NT)
chunk_bwd_state_kernel(const TIn* __restrict__ q, const TIn* __restrict__ k,
                       const TIn* __restrict__ v, const TIn* __restrict__ dout,
                       const float* __restrict__ g, const float* __restrict__ g_gamma,
                       const float* __restrict__ h0, const float* __restrict__ dht,
                       float* __restrict__ dh0, float scale, int32_t H, int32_t Hkv, int32_t V,
                       StateLayout sl, SeqLayout seqs,
                       int32_t chunks_per_row, float* __restrict__ hbuf, float* __restrict__ dhbuf) {
  constexpr int LDX = K + 4;
  constexpr int NST = (K / 16) * 2;
  constexpr int SPW = (NST + 3) / 4;
  __shared__ float sX[C * LDX];     // K rows (forward) or Q rows (reverse)
  __shared__ float sY[C * LDT];     // V tile (forward) or dO tile (reverse)
  __shared__ float sW[C];           // 2^(b_last - b) (forward) or scale 2^b (reverse)
  __shared__ float sDall;

  // workgroups 2 u and 2 u + 1 run unit u's forward and reverse passes, so
  // the longest units start both at once
  const bool rev = (blockIdx.x & 1) != 0;
  const int bid = (int)(blockIdx.x >> 1);
  const UnitMap um = map_unit(bid, V / VT, H, 1, seqs.num_seqs);
  if (!um.valid) return;
  const int hd = um.hd, vt = um.vt;
  const int hk = hd / (H / Hkv);   // kv head whose k and v rows this query head reads
  const SeqInfo si = seq_info(seqs, um.rank, chunks_per_row);
  const int nchunks = (si.len + seqs.chunk - 1) / seqs.chunk;
  const int tid = threadIdx.x, lane = tid & 63, g4 = lane >> 4, r = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index, uniform
  const int64_t KV = (int64_t)K * V;
  const int64_t ucol = vt * VT;

  f32x4 hs[SPW];
  {
    const float* init = rev ? dht : h0;
    const float* iu = init != nullptr ? init + ((int64_t)si.seq * H + hd) * KV : nullptr;
#pragma unroll
    for (int s = 0; s < SPW; ++s) {
      const int st = w + 4 * s;
      hs[s] = f32x4{0.f, 0.f, 0.f, 0.f};
      if ((NST % 4 == 0 || st < NST) && iu != nullptr) {
        const int kt = st >> 1, ctl = st & 1;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          hs[s][i] = iu[(int64_t)(16 * kt + 4 * g4 + i) * sl.rs + (ucol + 16 * ctl + r) * sl.cs];
      }
    }
  }

  // chunk m's rows and gate are loaded into registers one iteration ahead
  RowTile<K, NT, TIn> xt;
  RowTile<VT, NT, TIn> yt;
  float gx = 0.f;
  auto load_chunk = [&](int it) {
    const int m = rev ? nchunks - 1 - it : it;
    const int64_t t0 = si.bos + (int64_t)m * seqs.chunk;
    const int cl = min(seqs.chunk, si.len - m * seqs.chunk);
    xt.load(rev ? q + (t0 * H + hd) * K : k + (t0 * Hkv + hk) * K, (int64_t)(rev ? H : Hkv) * K, cl);
    yt.load(rev ? dout + (t0 * H + hd) * V + ucol : v + (t0 * Hkv + hk) * V + ucol,
            (int64_t)(rev ? H : Hkv) * V, cl);
    if (w == 0 && g != nullptr) gx = lane < cl ? g[(t0 + lane) * H + hd] : 0.f;
  };
  if (nchunks > 0) load_chunk(0);
  for (int it = 0; it < nchunks; ++it) {
    const int m = rev ? nchunks - 1 - it : it;
    const int cl = min(seqs.chunk, si.len - m * seqs.chunk);
    // record: forward -> the state entering chunk m; reverse -> the gradient
    // of the state leaving chunk m
    float* rec = (rev ? dhbuf : hbuf) + ((int64_t)(si.chunk0 + m) * H + hd) * KV + ucol;
#pragma unroll
    for (int s = 0; s < SPW; ++s) {
      const int st = w + 4 * s;
      if (NST % 4 == 0 || st < NST) {
        const int kt = st >> 1, ctl = st & 1;
#pragma unroll
        for (int i = 0; i < 4; ++i) rec[(int64_t)(16 * kt + 4 * g4 + i) * V + 16 * ctl + r] = hs[s][i];
      }
    }
    xt.store(sX, LDX);
    yt.store(sY, LDT);
    if (w == 0) {
      float b, bl = 0.f;
      if (g != nullptr) b = wave_cumsum_log2_split(gx, bl);
      else if (g_gamma != nullptr) b = (float)min(lane + 1, cl) * (g_gamma[hd] * kRcpLn2f);
      else b = 0.f;
      const float blast = __shfl(b, C - 1, 64), bllast = __shfl(bl, C - 1, 64);
      sW[lane] = rev ? exp2f(b) * scale : exp2f((blast - b) + (bllast - bl));
      if (lane == 0) sDall = exp2f(blast);
    }
    __syncthreads();
    if (it + 1 < nchunks) load_chunk(it + 1);
    const float dall = sDall;
#pragma unroll
    for (int s = 0; s < SPW; ++s) hs[s] *= dall;
    // the wave's tiles are independent accumulation chains: interleave them
#pragma unroll 4
    for (int cs = 0; cs < C / 4; ++cs) {
      const int c = 4 * cs + g4;
      const float wc = sW[c];
#pragma unroll
      for (int s = 0; s < SPW; ++s) {
        const int st = w + 4 * s;
        if (NST % 4 != 0 && st >= NST) continue;
        const int kt = st >> 1, ctl = st & 1;
        hs[s] = mfma4(sX[c * LDX + 16 * kt + r] * wc, sY[c * LDT + 16 * ctl + r], hs[s]);
      }
    }
    __syncthreads();
  }
  if (rev && dh0 != nullptr) {
    float* du = dh0 + ((int64_t)si.seq * H + hd) * KV;
#pragma unroll
    for (int s = 0; s < SPW; ++s) {
      const int st = w + 4 * s;
      if (NST % 4 == 0 || st < NST) {
        const int kt = st >> 1, ctl = st & 1;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          du[(int64_t)(16 * kt + 4 * g4 + i) * sl.rs + (ucol + 16 * ctl + r) * sl.cs] = hs[s][i];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Per-(chunk, head) gradients, 8 waves (two per SIMD).  Wave w works on row
// tile rw = w % 4 (rows [16 rw, +16) of A, dA, dQ, dK, dV) and column half
// kh = w / 4: A and dA column tiles {2 kh, 2 kh + 1}, dQ / dK column tiles
// [kh NKT / 2, +NKT / 2), dV columns [16 kh, +16) of each 32-column V slice.
// V is walked in 32-column slices, each loaded one slice ahead; A, then dA,
// live in LDS.
// ---------------------------------------------------------------------------
constexpr int NTG = 512;          // grad-kernel threads (8 waves)

template <int K, typename TIn>
__global__ void __launch_bounds__(NTG)
chunk_bwd_grad_kernel(const TIn* __restrict__ q, const TIn* __restrict__ k,
                      const TIn* __restrict__ v, const TIn* __restrict__ dout,
                      const float* __restrict__ g, const float* __restrict__ g_gamma, float scale,
                      int32_t H, int32_t Hkv, int32_t V, SeqLayout seqs, int32_t chunks_per_row,
                      const float* __restrict__ hbuf, const float* __restrict__ dhbuf,
                      float* __restrict__ dq, float* __restrict__ dk, float* __restrict__ dv,
                      float* __restrict__ dg, float* __restrict__ gpart) {
  constexpr int LDQ = K + 4;
  constexpr int NKT = K / 16;                   // 16-column tiles of dQ / dK
  constexpr int NKH = NKT >= 2 ? NKT / 2 : 1;   // per wave
  __shared__ float sQ[C * LDQ];
  __shared__ float sK[C * LDQ];
  __shared__ float sA[C * LDA];     // A during the slices, then dA
  __shared__ float sV[C * LDT];
  __shared__ float sdO[C * LDT];
  __shared__ float sH[K * LDT];
  __shared__ float sdH[K * LDT];
  __shared__ float sb[C], sbl[C], ssc[C], sdv[C];   // sb + sbl: the running log2 gate
  __shared__ float sR[2][C], sKs[2][C];
  __shared__ float sFrob[8];

  const int gc = blockIdx.x;
  const int hd = blockIdx.y;
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
  const bool has_k = NKT >= 2 || kh == 0;       // K = 16: one column tile, taken by kh = 0
  const int kt0 = kh * NKH;
  const int hk = hd / (H / Hkv);   // kv head whose k and v rows this query head reads
  const int64_t RSK = (int64_t)H * K, RSV = (int64_t)H * V;        // q and dout rows
  const int64_t RKK = (int64_t)Hkv * K, RKV = (int64_t)Hkv * V;    // k and v rows
  const int64_t KV = (int64_t)K * V;
  const float* hu = hbuf + ((int64_t)gc * H + hd) * KV;
  const float* dhu = dhbuf + ((int64_t)gc * H + hd) * KV;

  {
    RowTile<K, NTG, TIn> qt, kt;
    qt.load(q + (t0 * H + hd) * K, RSK, cl);
    kt.load(k + (t0 * Hkv + hk) * K, RKK, cl);
    qt.store(sQ, LDQ);
    kt.store(sK, LDQ);
  }
  if (w == 0) {
    float bl;
    const float b = chunk_gate(g, g_gamma, H, hd, t0, cl, bl);
    const float blast = __shfl(b, C - 1, 64), bllast = __shfl(bl, C - 1, 64);
    sb[lane] = b;
    sbl[lane] = bl;
    ssc[lane] = exp2f(b) * scale;
    sdv[lane] = exp2f((blast - b) + (bllast - bl));
  }
  // slice tiles, loaded one slice ahead of their use
  RowTile<VT, NTG, TIn> vtile, otile;
  RecTile<K, NTG> htile, dhtile;
  auto load_slice = [&](int vs) {
    vtile.load(v + (t0 * Hkv + hk) * V + vs * VT, RKV, cl);
    otile.load(dout + (t0 * H + hd) * V + vs * VT, RSV, cl);
    htile.load(hu, V, (int64_t)vs * VT);
    dhtile.load(dhu, V, (int64_t)vs * VT);
  };
  load_slice(0);
  __syncthreads();

  // ---- A = scale (Q K^T) (.) M: row tile rw against column tiles 2 kh, 2 kh + 1
  //      (upper tiles come out masked to zero) ------------------------------
  {
    f32x4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll 4
    for (int ks = 0; ks < K / 4; ++ks) {
      const float a = sQ[(16 * rw + r) * LDQ + 4 * ks + g4];
#pragma unroll
      for (int t = 0; t < 2; ++t) acc[t] = mfma4(a, sK[(16 * (2 * kh + t) + r) * LDQ + 4 * ks + g4], acc[t]);
    }
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int j = 16 * (2 * kh + t) + r;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int c = 16 * rw + 4 * g4 + i;
        sA[c * LDA + j] = j <= c ? acc[t][i] * exp2f((sb[c] - sb[j]) + (sbl[c] - sbl[j])) * scale : 0.f;
      }
    }
  }

  // ---- walk V in 32-column slices ---------------------------------------------
  f32x4 dAacc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
  f32x4 dQi[NKH], dKs[NKH];
#pragma unroll
  for (int t = 0; t < NKH; ++t) {
    dQi[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    dKs[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  float frob = 0.f;
  for (int vs = 0; vs < V / VT; ++vs) {
    __syncthreads();   // previous slice's reads done (first pass: A published)
    vtile.store(sV, LDT);
    otile.store(sdO, LDT);
    htile.store(sH);
    dhtile.store(sdH);
#pragma unroll
    for (int u = 0; u < RecTile<K, NTG>::N; ++u) {
      const f32x4 x = htile.x[u], y = dhtile.x[u];
      frob += x[0] * y[0] + x[1] * y[1] + x[2] * y[2] + x[3] * y[3];
    }
    if (vs + 1 < V / VT) load_slice(vs + 1);
    __syncthreads();
    // dA += dO V^T, dQ_inter += dO h^T, dK_state += V dH^T over this slice
#pragma unroll
    for (int s = 0; s < VT / 4; ++s) {
      const float ao = sdO[(16 * rw + r) * LDT + 4 * s + g4];
      const float av = sV[(16 * rw + r) * LDT + 4 * s + g4];
#pragma unroll
      for (int t = 0; t < 2; ++t) dAacc[t] = mfma4(ao, sV[(16 * (2 * kh + t) + r) * LDT + 4 * s + g4], dAacc[t]);
      if (has_k) {
#pragma unroll
        for (int t = 0; t < NKH; ++t) {
          dQi[t] = mfma4(ao, sH[(16 * (kt0 + t) + r) * LDT + 4 * s + g4], dQi[t]);
          dKs[t] = mfma4(av, sdH[(16 * (kt0 + t) + r) * LDT + 4 * s + g4], dKs[t]);
        }
      }
    }
    // dV: rows [16 rw, +16), columns [16 kh, +16) of the slice
    {
      f32x4 in = {0.f, 0.f, 0.f, 0.f}, st = in;
      for (int cs = 4 * rw; cs < C / 4; ++cs)   // A[c][j] = 0 for c < j
        in = mfma4(sA[(4 * cs + g4) * LDA + 16 * rw + r], sdO[(4 * cs + g4) * LDT + 16 * kh + r], in);
#pragma unroll 8
      for (int ks = 0; ks < K / 4; ++ks)
        st = mfma4(sK[(16 * rw + r) * LDQ + 4 * ks + g4], sdH[(4 * ks + g4) * LDT + 16 * kh + r], st);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = 16 * rw + 4 * g4 + i;
        if (j < cl) dv[((t0 + j) * H + hd) * (int64_t)V + vs * VT + 16 * kh + r] = in[i] + sdv[j] * st[i];
      }
    }
  }
  __syncthreads();   // every read of A is done

  // ---- dA masked and scaled, into the A buffer ------------------------------
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int j = 16 * (2 * kh + t) + r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = 16 * rw + 4 * g4 + i;
      sA[c * LDA + j] = j <= c ? dAacc[t][i] * exp2f((sb[c] - sb[j]) + (sbl[c] - sbl[j])) * scale : 0.f;
    }
  }
  // Frobenius product <dH, h> of the whole chunk record
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) frob += __shfl_xor(frob, d, 64);
  if (lane == 0) sFrob[w] = frob;
  __syncthreads();

  // ---- dQ = diag(sc) dQ_inter + dA K;  dK = dA^T Q + diag(dv) dK_state --------
  float rq[4] = {0.f, 0.f, 0.f, 0.f}, rk[4] = {0.f, 0.f, 0.f, 0.f}, ks4[4] = {0.f, 0.f, 0.f, 0.f};
  if (has_k) {
    constexpr int KP = NKH >= 2 ? 2 : 1;   // column tiles per pass (independent chains)
#pragma unroll
    for (int k0 = 0; k0 < NKH; k0 += KP) {
      f32x4 aq[KP], ak[KP];
#pragma unroll
      for (int u = 0; u < KP; ++u) aq[u] = ak[u] = f32x4{0.f, 0.f, 0.f, 0.f};
      for (int js = 0; js < 4 * (rw + 1); ++js) {   // dA[c][j] = 0 for j > c
        const float a = sA[(16 * rw + r) * LDA + 4 * js + g4];
#pragma unroll
        for (int u = 0; u < KP; ++u) aq[u] = mfma4(a, sK[(4 * js + g4) * LDQ + 16 * (kt0 + k0 + u) + r], aq[u]);
      }
      for (int cs = 4 * rw; cs < C / 4; ++cs) {
        const float a = sA[(4 * cs + g4) * LDA + 16 * rw + r];
#pragma unroll
        for (int u = 0; u < KP; ++u) ak[u] = mfma4(a, sQ[(4 * cs + g4) * LDQ + 16 * (kt0 + k0 + u) + r], ak[u]);
      }
#pragma unroll
      for (int u = 0; u < KP; ++u) {
        const int t = k0 + u;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int c = 16 * rw + 4 * g4 + i;
          const int col = 16 * (kt0 + t) + r;
          const float xq = ssc[c] * dQi[t][i] + aq[u][i];
          const float xk = ak[u][i] + sdv[c] * dKs[t][i];
          rq[i] += sQ[c * LDQ + col] * xq;
          rk[i] += sK[c * LDQ + col] * xk;
          ks4[i] += sK[c * LDQ + col] * dKs[t][i];
          if (c < cl) {
            dq[((t0 + c) * H + hd) * (int64_t)K + col] = xq;
            dk[((t0 + c) * H + hd) * (int64_t)K + col] = xk;
          }
        }
      }
    }
  }
  // row sums over the 16 lanes of a column group, one partial per column half
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
      sR[kh][c] = rq[i] - rk[i];
      sKs[kh][c] = sdv[c] * ks4[i];
    }
  }
  __syncthreads();

  // ---- gate gradient: reverse cumulative sum over the chunk ---------------
  if (w == 0) {
    float frob_all = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) frob_all += sFrob[i];
    // the chunk's share of the state it hands on, at its last real token
    double extra = (double)sKs[0][lane] + (double)sKs[1][lane];
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) extra += __shfl_xor(extra, d, 64);
    double x = lane < cl ? (double)sR[0][lane] + (double)sR[1][lane] : 0.0;
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

// dg_gamma[h] = sum over chunks of the per-(chunk, head) sums, in a fixed order.
__global__ void __launch_bounds__(NT)
chunk_bwd_gamma_kernel(const float* __restrict__ gpart, int32_t num_chunks, int32_t H,
                       float* __restrict__ dg_gamma) {
  __shared__ double part[NT];
  const int hd = blockIdx.x;
  double s = 0.0;
  for (int c = threadIdx.x; c < num_chunks; c += NT) s += (double)gpart[(int64_t)c * H + hd];
  part[threadIdx.x] = s;
  __syncthreads();
  for (int d = NT / 2; d >= 1; d >>= 1) {
    if ((int)threadIdx.x < d) part[threadIdx.x] += part[threadIdx.x + d];
    __syncthreads();
  }
  if (threadIdx.x == 0) dg_gamma[hd] = (float)part[0];
}

// Gradients of k and v with grouped kv heads: a kv head's row is read by its
// n_rep query heads, so its gradient is the sum of theirs (computed per query
// head by the kernels above).  One thread per 4 consecutive elements of a
// (token, kv head) row; the n_rep terms are added in query-head order.
__global__ void __launch_bounds__(256)
kv_group_sum_kernel(const float* __restrict__ src, float* __restrict__ dst, int64_t rows, int32_t n_rep,
                    int32_t D) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;   // float4 index into dst
  const int32_t d4 = D / 4;
  if (i >= rows * d4) return;
  const int64_t row = i / d4;                                   // token * Hkv + kv head
  const int32_t c = (int32_t)(i - row * d4);
  const f32x4* s = reinterpret_cast<const f32x4*>(src) + row * n_rep * d4 + c;
  f32x4 acc = s[0];
  for (int32_t j = 1; j < n_rep; ++j) acc += s[(int64_t)j * d4];
  reinterpret_cast<f32x4*>(dst)[i] = acc;
}

template <int K, typename TIn>
hipError_t launch_k(const ChunkBwdParams& p, int32_t per_row, hipStream_t stream) {
  const TIn* q = static_cast<const TIn*>(p.q);
  const TIn* k = static_cast<const TIn*>(p.k);
  const TIn* v = static_cast<const TIn*>(p.v);
  const TIn* dout = static_cast<const TIn*>(p.dout);
  if (p.seqs.num_seqs > 0) {
    const int units = (int)unit_grid(p.seqs.num_seqs, p.H, 1, p.V / VT);
    hipLaunchKernelGGL((chunk_bwd_state_kernel<K, TIn>), dim3((unsigned)(2 * units)), dim3(NT), 0, stream,
                       q, k, v, dout, p.g, p.g_gamma, p.h0, p.dht, p.dh0, p.scale, p.H, p.Hkv, p.V, p.sl,
                       p.seqs, per_row, p.hbuf, p.dhbuf);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (p.seqs.num_chunks > 0) {
    hipLaunchKernelGGL((chunk_bwd_grad_kernel<K, TIn>), dim3((unsigned)p.seqs.num_chunks, (unsigned)p.H),
                       dim3(NTG), 0, stream, q, k, v, dout, p.g, p.g_gamma, p.scale, p.H, p.Hkv, p.V, p.seqs,
                       per_row, p.hbuf, p.dhbuf, p.dq, p.dk, p.dv, p.dg,
                       p.dg_gamma != nullptr ? p.gpart : nullptr);
    return hipGetLastError();
  }
  return hipSuccess;
}

// The fp32-matrix-core passes: float32 inputs (K <= 128) and bf16 inputs
// with K in {16, 32}.
hipError_t launch_fp32_passes(const ChunkBwdParams& p, int32_t per_row, hipStream_t stream) {
  if (p.qkv_bf16) {
    switch (p.K) {
      case 16: return launch_k<16, __bf16>(p, per_row, stream);
      case 32: return launch_k<32, __bf16>(p, per_row, stream);
      default: return hipErrorInvalidValue;
    }
  }
  switch (p.K) {
    case 16: return launch_k<16, float>(p, per_row, stream);
    case 32: return launch_k<32, float>(p, per_row, stream);
    case 64: return launch_k<64, float>(p, per_row, stream);
    case 128: return launch_k<128, float>(p, per_row, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_kv_group_sum(const float* src, float* dst, int64_t tokens, int32_t H, int32_t Hkv,
                               int32_t D, hipStream_t stream) {
  const int64_t n4 = tokens * Hkv * (D / 4);
  if (n4 == 0) return hipSuccess;
  if (D % 4 != 0 || Hkv <= 0 || H % Hkv != 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(kv_group_sum_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, stream, src, dst,
                     tokens * Hkv, H / Hkv, D);
  return hipGetLastError();
}

hipError_t launch_chunk_bwd(const ChunkBwdParams& p, hipStream_t stream) {
  const int32_t per_row = p.seqs.T > 0 ? (p.seqs.T + p.seqs.chunk - 1) / p.seqs.chunk : 1;
  hipError_t e;
  if (bwd_bf16_grad(p.qkv_bf16 != 0, p.K)) {
    e = launch_chunk_bwd_state_bf16(p, per_row, stream);
    if (e == hipSuccess) e = launch_chunk_bwd_grad_bf16(p, per_row, stream);
  } else {
    e = launch_fp32_passes(p, per_row, stream);
  }
  if (e == hipSuccess && p.dg_gamma != nullptr) {
    hipLaunchKernelGGL(chunk_bwd_gamma_kernel, dim3((unsigned)p.H), dim3(NT), 0, stream, p.gpart,
                       p.seqs.num_chunks, p.H, p.dg_gamma);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace sgla
