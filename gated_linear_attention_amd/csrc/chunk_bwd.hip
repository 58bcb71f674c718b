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
// Every product runs on the fp32 matrix cores (v_mfma_f32_16x16x4_f32), so
// inputs are used exactly and states, gradients and accumulation are fp32.
// Operand layout, per lane l with g = l / 16 and r = l % 16:
//   A operand A[m = r][k = g], B operand B[k = g][n = r],
//   result acc[i] = D[m = 4 g + i][n = r].
#include <hip/hip_runtime.h>

#include "gate_scan.h"
#include "sgla_internal.h"
#include "unit_map.h"

namespace sgla {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int C = kChunk;
constexpr int NT = 256;           // threads (4 waves)
constexpr int VT = 32;            // V columns per state-pass workgroup and per slice
constexpr int LDT = VT + 4;       // row stride of 32-column tiles (floats)
constexpr int LDA = C + 4;        // row stride of the 64 x 64 A / dA tile
constexpr float kRcpLn2f = 1.44269504088896341f;

// Causal 16 x 16 tiles (c, j), j <= c, packed 4 bits each (c | j << 2); wave
// w takes entries w, w + 4, w + 8.
constexpr uint64_t kTiles = 0xFB73A62510ull;

__device__ __forceinline__ f32x4 mfma4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 load4(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
__device__ __forceinline__ f32x4 load4(const __bf16* p) {
  const uint2 u = *reinterpret_cast<const uint2*>(p);
  return f32x4{__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
               __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u)};
}

// rows [0, 64) x cols [0, W) of a token-major input (row stride RS elements)
// into LDS (row stride LD floats); rows at or past `rows` read as zero.
template <int W, typename T>
__device__ __forceinline__ void stage_rows(float* dst, int LD, const T* src, int64_t RS, int rows) {
  for (int i = threadIdx.x; i < C * (W / 4); i += NT) {
    const int c = i / (W / 4), c4 = i % (W / 4);
    f32x4 x = {0.f, 0.f, 0.f, 0.f};
    if (c < rows) x = load4(src + c * RS + 4 * c4);
    *reinterpret_cast<f32x4*>(dst + c * LD + 4 * c4) = x;
  }
}

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
__device__ __forceinline__ float chunk_gate(const float* g, const float* g_gamma, int H, int hd,
                                            int64_t t0, int cl) {
  const int lane = threadIdx.x & 63;
  if (g != nullptr) return wave_cumsum_log2(lane < cl ? g[(t0 + lane) * H + hd] : 0.f);
  if (g_gamma != nullptr) return (float)min(lane + 1, cl) * (g_gamma[hd] * kRcpLn2f);
  return 0.f;
}

// ---------------------------------------------------------------------------
// State pass.  Workgroups [0, half) run the forward recurrence of one
// (sequence, head, 32-column V tile) and store the state entering every
// chunk; workgroups [half, 2 half) run the reverse recurrence of the state
// gradient and store the gradient of the state leaving every chunk, then dh0.
// The K x 32 (gradient) state stays in MFMA accumulators: wave w owns 16 x 16
// tiles st = w + 4 s (rows 16 (st / 2), columns 16 (st % 2)).
// ---------------------------------------------------------------------------
template <int K, typename TIn>
__global__ void __launch_bounds__(NT)
chunk_bwd_state_kernel(const TIn* __restrict__ q, const TIn* __restrict__ k,
                       const TIn* __restrict__ v, const TIn* __restrict__ dout,
                       const float* __restrict__ g, const float* __restrict__ g_gamma,
                       const float* __restrict__ h0, const float* __restrict__ dht,
                       float* __restrict__ dh0, float scale, int32_t H, int32_t V, SeqLayout seqs,
                       int32_t chunks_per_row, float* __restrict__ hbuf, float* __restrict__ dhbuf,
                       int32_t half) {
  constexpr int LDX = K + 4;
  constexpr int NST = (K / 16) * 2;
  constexpr int SPW = (NST + 3) / 4;
  __shared__ float sX[C * LDX];     // K rows (forward) or Q rows (reverse)
  __shared__ float sY[C * LDT];     // V tile (forward) or dO tile (reverse)
  __shared__ float sW[C];           // 2^(b_last - b) (forward) or scale 2^b (reverse)
  __shared__ float sDall;

  const bool rev = (int)blockIdx.x >= half;
  const int bid = rev ? (int)blockIdx.x - half : (int)blockIdx.x;
  const UnitMap um = map_unit(bid, V / VT, H, 1, seqs.num_seqs);
  if (!um.valid) return;
  const int hd = um.hd, vt = um.vt;
  const SeqInfo si = seq_info(seqs, um.rank, chunks_per_row);
  const int nchunks = (si.len + C - 1) / C;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, g4 = lane >> 4, r = lane & 15;
  const int64_t KV = (int64_t)K * V;
  const int64_t ucol = vt * VT;

  f32x4 hs[SPW];
  {
    const float* init = rev ? dht : h0;
    const float* iu = init != nullptr ? init + ((int64_t)si.seq * H + hd) * KV + ucol : nullptr;
#pragma unroll
    for (int s = 0; s < SPW; ++s) {
      const int st = w + 4 * s;
      hs[s] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (st < NST && iu != nullptr) {
        const int kt = st >> 1, ctl = st & 1;
#pragma unroll
        for (int i = 0; i < 4; ++i) hs[s][i] = iu[(int64_t)(16 * kt + 4 * g4 + i) * V + 16 * ctl + r];
      }
    }
  }

  for (int it = 0; it < nchunks; ++it) {
    const int m = rev ? nchunks - 1 - it : it;
    const int64_t t0 = si.bos + (int64_t)m * C;
    const int cl = min(C, si.len - m * C);
    // record: forward -> the state entering chunk m; reverse -> the gradient
    // of the state leaving chunk m
    float* rec = (rev ? dhbuf : hbuf) + ((int64_t)(si.chunk0 + m) * H + hd) * KV + ucol;
#pragma unroll
    for (int s = 0; s < SPW; ++s) {
      const int st = w + 4 * s;
      if (st < NST) {
        const int kt = st >> 1, ctl = st & 1;
#pragma unroll
        for (int i = 0; i < 4; ++i) rec[(int64_t)(16 * kt + 4 * g4 + i) * V + 16 * ctl + r] = hs[s][i];
      }
    }
    if (rev) {
      stage_rows<K>(sX, LDX, q + (t0 * H + hd) * K, (int64_t)H * K, cl);
      stage_rows<VT>(sY, LDT, dout + (t0 * H + hd) * V + ucol, (int64_t)H * V, cl);
    } else {
      stage_rows<K>(sX, LDX, k + (t0 * H + hd) * K, (int64_t)H * K, cl);
      stage_rows<VT>(sY, LDT, v + (t0 * H + hd) * V + ucol, (int64_t)H * V, cl);
    }
    if (w == 0) {
      const float b = chunk_gate(g, g_gamma, H, hd, t0, cl);
      const float blast = __shfl(b, C - 1, 64);
      sW[lane] = rev ? exp2f(b) * scale : exp2f(blast - b);
      if (lane == 0) sDall = exp2f(blast);
    }
    __syncthreads();
    const float dall = sDall;
#pragma unroll
    for (int s = 0; s < SPW; ++s) {
      const int st = w + 4 * s;
      if (st >= NST) continue;
      const int kt = st >> 1, ctl = st & 1;
      f32x4 acc = hs[s] * dall;
#pragma unroll 8
      for (int cs = 0; cs < C / 4; ++cs) {
        const int c = 4 * cs + g4;
        acc = mfma4(sX[c * LDX + 16 * kt + r] * sW[c], sY[c * LDT + 16 * ctl + r], acc);
      }
      hs[s] = acc;
    }
    __syncthreads();
  }
  if (rev && dh0 != nullptr) {
    float* du = dh0 + ((int64_t)si.seq * H + hd) * KV + ucol;
#pragma unroll
    for (int s = 0; s < SPW; ++s) {
      const int st = w + 4 * s;
      if (st < NST) {
        const int kt = st >> 1, ctl = st & 1;
#pragma unroll
        for (int i = 0; i < 4; ++i) du[(int64_t)(16 * kt + 4 * g4 + i) * V + 16 * ctl + r] = hs[s][i];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Per-(chunk, head) gradients.  Wave w owns rows [16 w, +16) of dQ and dK (all
// K columns) and walks V in 32-column slices; dA and A live in LDS.
// ---------------------------------------------------------------------------
template <int K, typename TIn>
__global__ void __launch_bounds__(NT)
chunk_bwd_grad_kernel(const TIn* __restrict__ q, const TIn* __restrict__ k,
                      const TIn* __restrict__ v, const TIn* __restrict__ dout,
                      const float* __restrict__ g, const float* __restrict__ g_gamma, float scale,
                      int32_t H, int32_t V, SeqLayout seqs, int32_t chunks_per_row,
                      const float* __restrict__ hbuf, const float* __restrict__ dhbuf,
                      float* __restrict__ dq, float* __restrict__ dk, float* __restrict__ dv,
                      float* __restrict__ dg, float* __restrict__ gpart) {
  constexpr int LDQ = K + 4;
  constexpr int NKT = K / 16;       // 16-column tiles of dQ / dK per wave
  __shared__ float sQ[C * LDQ];
  __shared__ float sK[C * LDQ];
  __shared__ float sA[C * LDA];     // A during the slices, then dA
  __shared__ float sV[C * LDT];
  __shared__ float sdO[C * LDT];
  __shared__ float sH[K * LDT];
  __shared__ float sdH[K * LDT];
  __shared__ float sb[C], ssc[C], sdv[C];
  __shared__ float sR[C], sKs[C];
  __shared__ float sFrob[4];

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
    t0 = (int64_t)row * seqs.T + (int64_t)m * C;
    cl = min(C, seqs.T - m * C);
  }
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, g4 = lane >> 4, r = lane & 15;
  const int64_t RSK = (int64_t)H * K, RSV = (int64_t)H * V;
  const int64_t KV = (int64_t)K * V;
  const float* hu = hbuf + ((int64_t)gc * H + hd) * KV;
  const float* dhu = dhbuf + ((int64_t)gc * H + hd) * KV;

  stage_rows<K>(sQ, LDQ, q + (t0 * H + hd) * K, RSK, cl);
  stage_rows<K>(sK, LDQ, k + (t0 * H + hd) * K, RSK, cl);
  if (w == 0) {
    const float b = chunk_gate(g, g_gamma, H, hd, t0, cl);
    const float blast = __shfl(b, C - 1, 64);
    sb[lane] = b;
    ssc[lane] = exp2f(b) * scale;
    sdv[lane] = exp2f(blast - b);
  }
  // upper-triangle tiles of A / dA are never written: zero them once
  for (int i = tid; i < 6 * 256; i += NT) {
    const int tt = i >> 8, e = i & 255;
    const int ctile = tt < 3 ? 0 : (tt < 5 ? 1 : 2);
    const int jtile = tt < 3 ? tt + 1 : (tt < 5 ? tt - 1 : 3);
    sA[(16 * ctile + (e >> 4)) * LDA + 16 * jtile + (e & 15)] = 0.f;
  }
  __syncthreads();

  // ---- A = scale (Q K^T) (.) M, causal tiles --------------------------------
#pragma unroll
  for (int t = 0; t < 3; ++t) {
    const int ti = w + 4 * t;
    if (ti >= 10) continue;
    const int ctile = (int)(kTiles >> (4 * ti)) & 3, jtile = (int)(kTiles >> (4 * ti + 2)) & 3;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
    for (int ks = 0; ks < K / 4; ++ks)
      acc = mfma4(sQ[(16 * ctile + r) * LDQ + 4 * ks + g4], sK[(16 * jtile + r) * LDQ + 4 * ks + g4], acc);
    const int j = 16 * jtile + r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = 16 * ctile + 4 * g4 + i;
      sA[c * LDA + j] = j <= c ? acc[i] * exp2f(sb[c] - sb[j]) * scale : 0.f;
    }
  }

  // ---- walk V in 32-column slices ---------------------------------------------
  f32x4 dAacc[3];
  f32x4 dQi[NKT], dKs[NKT];
#pragma unroll
  for (int t = 0; t < 3; ++t) dAacc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int t = 0; t < NKT; ++t) {
    dQi[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    dKs[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  float frob = 0.f;
  for (int vs = 0; vs < V / VT; ++vs) {
    __syncthreads();   // previous slice's reads done (first pass: A and gates published)
    stage_rows<VT>(sV, LDT, v + (t0 * H + hd) * V + vs * VT, RSV, cl);
    stage_rows<VT>(sdO, LDT, dout + (t0 * H + hd) * V + vs * VT, RSV, cl);
    for (int i = tid; i < K * (VT / 4); i += NT) {
      const int row = i / (VT / 4), c4 = i % (VT / 4);
      const f32x4 x = load4(hu + (int64_t)row * V + vs * VT + 4 * c4);
      const f32x4 y = load4(dhu + (int64_t)row * V + vs * VT + 4 * c4);
      *reinterpret_cast<f32x4*>(sH + row * LDT + 4 * c4) = x;
      *reinterpret_cast<f32x4*>(sdH + row * LDT + 4 * c4) = y;
      frob += x[0] * y[0] + x[1] * y[1] + x[2] * y[2] + x[3] * y[3];
    }
    __syncthreads();
    // dA += dO V^T over this slice (causal tiles)
#pragma unroll
    for (int t = 0; t < 3; ++t) {
      const int ti = w + 4 * t;
      if (ti >= 10) continue;
      const int ctile = (int)(kTiles >> (4 * ti)) & 3, jtile = (int)(kTiles >> (4 * ti + 2)) & 3;
#pragma unroll
      for (int s = 0; s < VT / 4; ++s)
        dAacc[t] = mfma4(sdO[(16 * ctile + r) * LDT + 4 * s + g4], sV[(16 * jtile + r) * LDT + 4 * s + g4], dAacc[t]);
    }
    // dQ_inter += dO h^T and dK_state += V dH^T: rows of wave w
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt) {
#pragma unroll
      for (int s = 0; s < VT / 4; ++s) {
        dQi[kt] = mfma4(sdO[(16 * w + r) * LDT + 4 * s + g4], sH[(16 * kt + r) * LDT + 4 * s + g4], dQi[kt]);
        dKs[kt] = mfma4(sV[(16 * w + r) * LDT + 4 * s + g4], sdH[(16 * kt + r) * LDT + 4 * s + g4], dKs[kt]);
      }
    }
    // dV slice: rows [16 w, +16), columns 16 cv + r of the slice
#pragma unroll
    for (int cv = 0; cv < 2; ++cv) {
      f32x4 intra = {0.f, 0.f, 0.f, 0.f}, st = {0.f, 0.f, 0.f, 0.f};
      for (int cs = 4 * w; cs < C / 4; ++cs)   // A[c][j] = 0 for c < j
        intra = mfma4(sA[(4 * cs + g4) * LDA + 16 * w + r], sdO[(4 * cs + g4) * LDT + 16 * cv + r], intra);
#pragma unroll 8
      for (int ks = 0; ks < K / 4; ++ks)
        st = mfma4(sK[(16 * w + r) * LDQ + 4 * ks + g4], sdH[(4 * ks + g4) * LDT + 16 * cv + r], st);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = 16 * w + 4 * g4 + i;
        if (j < cl) dv[((t0 + j) * H + hd) * (int64_t)V + vs * VT + 16 * cv + r] = intra[i] + sdv[j] * st[i];
      }
    }
  }
  __syncthreads();   // every read of A is done

  // ---- dA masked and scaled, into the A buffer ------------------------------
#pragma unroll
  for (int t = 0; t < 3; ++t) {
    const int ti = w + 4 * t;
    if (ti >= 10) continue;
    const int ctile = (int)(kTiles >> (4 * ti)) & 3, jtile = (int)(kTiles >> (4 * ti + 2)) & 3;
    const int j = 16 * jtile + r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = 16 * ctile + 4 * g4 + i;
      sA[c * LDA + j] = j <= c ? dAacc[t][i] * exp2f(sb[c] - sb[j]) * scale : 0.f;
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
  for (int kt = 0; kt < NKT; ++kt) {
    f32x4 aq = {0.f, 0.f, 0.f, 0.f}, ak = {0.f, 0.f, 0.f, 0.f};
    for (int js = 0; js < 4 * (w + 1); ++js)   // dA[c][j] = 0 for j > c
      aq = mfma4(sA[(16 * w + r) * LDA + 4 * js + g4], sK[(4 * js + g4) * LDQ + 16 * kt + r], aq);
    for (int cs = 4 * w; cs < C / 4; ++cs)
      ak = mfma4(sA[(4 * cs + g4) * LDA + 16 * w + r], sQ[(4 * cs + g4) * LDQ + 16 * kt + r], ak);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = 16 * w + 4 * g4 + i;
      const int col = 16 * kt + r;
      const float xq = ssc[c] * dQi[kt][i] + aq[i];
      const float xk = ak[i] + sdv[c] * dKs[kt][i];
      rq[i] += sQ[c * LDQ + col] * xq;
      rk[i] += sK[c * LDQ + col] * xk;
      ks4[i] += sK[c * LDQ + col] * dKs[kt][i];
      if (c < cl) {
        dq[((t0 + c) * H + hd) * (int64_t)K + col] = xq;
        dk[((t0 + c) * H + hd) * (int64_t)K + col] = xk;
      }
    }
  }
  // row sums over the 16 lanes of a column group
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int d = 8; d >= 1; d >>= 1) {
      rq[i] += __shfl_xor(rq[i], d, 64);
      rk[i] += __shfl_xor(rk[i], d, 64);
      ks4[i] += __shfl_xor(ks4[i], d, 64);
    }
    if (r == 0) {
      const int c = 16 * w + 4 * g4 + i;
      sR[c] = rq[i] - rk[i];
      sKs[c] = sdv[c] * ks4[i];
    }
  }
  __syncthreads();

  // ---- gate gradient: reverse cumulative sum over the chunk ---------------
  if (w == 0) {
    const float frob_all = sFrob[0] + sFrob[1] + sFrob[2] + sFrob[3];
    // the chunk's share of the state it hands on, at its last real token
    double extra = (double)sKs[lane];
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) extra += __shfl_xor(extra, d, 64);
    double x = lane < cl ? (double)sR[lane] : 0.0;
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

template <int K, typename TIn>
hipError_t launch_k(const ChunkBwdParams& p, hipStream_t stream) {
  const int per_row = p.seqs.T > 0 ? (p.seqs.T + C - 1) / C : 1;
  const TIn* q = static_cast<const TIn*>(p.q);
  const TIn* k = static_cast<const TIn*>(p.k);
  const TIn* v = static_cast<const TIn*>(p.v);
  const TIn* dout = static_cast<const TIn*>(p.dout);
  if (p.seqs.num_seqs > 0) {
    const int half = (int)unit_grid(p.seqs.num_seqs, p.H, 1, p.V / VT);
    hipLaunchKernelGGL((chunk_bwd_state_kernel<K, TIn>), dim3((unsigned)(2 * half)), dim3(NT), 0, stream,
                       q, k, v, dout, p.g, p.g_gamma, p.h0, p.dht, p.dh0, p.scale, p.H, p.V, p.seqs,
                       per_row, p.hbuf, p.dhbuf, half);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (p.seqs.num_chunks > 0) {
    hipLaunchKernelGGL((chunk_bwd_grad_kernel<K, TIn>), dim3((unsigned)p.seqs.num_chunks, (unsigned)p.H),
                       dim3(NT), 0, stream, q, k, v, dout, p.g, p.g_gamma, p.scale, p.H, p.V, p.seqs,
                       per_row, p.hbuf, p.dhbuf, p.dq, p.dk, p.dv, p.dg,
                       p.dg_gamma != nullptr ? p.gpart : nullptr);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (p.dg_gamma != nullptr) {
    hipLaunchKernelGGL(chunk_bwd_gamma_kernel, dim3((unsigned)p.H), dim3(NT), 0, stream, p.gpart,
                       p.seqs.num_chunks, p.H, p.dg_gamma);
    return hipGetLastError();
  }
  return hipSuccess;
}

template <typename TIn>
hipError_t launch_in(const ChunkBwdParams& p, hipStream_t stream) {
  switch (p.K) {
    case 16: return launch_k<16, TIn>(p, stream);
    case 32: return launch_k<32, TIn>(p, stream);
    case 64: return launch_k<64, TIn>(p, stream);
    case 128: return launch_k<128, TIn>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_chunk_bwd(const ChunkBwdParams& p, hipStream_t stream) {
  return p.qkv_bf16 ? launch_in<__bf16>(p, stream) : launch_in<float>(p, stream);
}

}  // namespace sgla
