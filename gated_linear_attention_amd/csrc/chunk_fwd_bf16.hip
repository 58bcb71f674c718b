// Steps (2) and (3) of the chunked Simple GLA forward for bf16 q/k/v, fused in
// one kernel (page "flash-linear-attention 中的 Simple GLA", section 一: the
// chunk view with a decay-masked q k^T inside a chunk and a scalar-decayed
// state between chunks; section 三: the inter-chunk state pass and the output
// pass, which with a head-wise gate are plain matrix products).
//
// For chunk n of one (sequence, head), with b the chunk-local cumulative log2
// gate from step (1), b_last = b at the chunk's last token, and h_n the K x V
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
//   * one workgroup of 4 waves per (sequence, head, 64-wide V tile); the
//     workgroups of one (sequence, head) share an XCD so the second read of its
//     q and k rows is served by that XCD's L2;
//   * wave w owns state columns [16w, 16w + 16) of the tile for all K rows, in
//     MFMA accumulator registers (fp32), carried across chunks without ever
//     leaving the chip -- only the final state is written;
//   * each chunk's Q, K (64 x K) and V tile (64 x 64) are staged in LDS
//     row-major; the operands that need the token index contiguous per lane
//     (K^T and V as MFMA operands reduced over tokens) are fetched with the
//     gfx950 transposing LDS read ds_read_b64_tr_b16;
//   * the next chunk's rows are loaded into registers while the current chunk
//     computes (one chunk of latency hiding).
//
// Precision: the state, the accumulation and the output are fp32.  The three
// MFMA operands that are not exact bf16 inputs -- the decay-masked A, the
// state h used in Q h, and the decayed V used in the state update -- are split
// as x = hi + lo with hi = bf16(x), lo = bf16(x - hi), and each product is
// issued twice (hi and lo), keeping ~16 significant bits for those operands.
#include <hip/hip_runtime.h>

#include "sgla_internal.h"

#ifndef SGLA_TR_READ
#define SGLA_TR_READ 1
#endif

namespace sgla {
namespace {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

constexpr int C = kChunk;  // 64 tokens per chunk
constexpr int VT = 64;     // state / output columns per workgroup
constexpr int NTHREADS = 256;
constexpr int LDV = VT + 16;  // V tile row stride (elements)
constexpr int LDA = C + 8;    // A tile row stride (elements)
constexpr float kRcpLn2f = 1.44269504088896341f;

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 cat(bf16x4 a, bf16x4 b) {
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Transposed fragment read: lane r of each 16-lane group receives
// base[(row0 + e) * ld + col0 + r] for e = 0..3.  row0 and col0 must be the
// same for the 16 lanes of a group; addresses must be 8-byte aligned.
__device__ __forceinline__ bf16x4 tr_read(const bf16* base, int ld, int row0, int col0) {
  const int lane = threadIdx.x & 15;
#if SGLA_TR_READ
  const bf16* p = base + (row0 + (lane >> 2)) * ld + col0 + 4 * (lane & 3);
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p));
#else
  bf16x4 out;
#pragma unroll
  for (int e = 0; e < 4; ++e) out[e] = base[(row0 + e) * ld + col0 + lane];
  return out;
#endif
}

// x = hi + lo with hi, lo bf16 (round to nearest even on both roundings).
__device__ __forceinline__ void split8(const float (&x)[8], bf16x8& hi, bf16x8& lo) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const bf16 h = (bf16)x[e];
    hi[e] = h;
    lo[e] = (bf16)(x[e] - (float)h);
  }
}

template <int K>
struct Smem {
  static constexpr int LDQ = K + 8;
  static constexpr int LDK = K + 16;
  static constexpr int OFF_Q = 0;
  static constexpr int OFF_K = OFF_Q + C * LDQ * 2;
  static constexpr int OFF_V = OFF_K + C * LDK * 2;
  static constexpr int OFF_AH = OFF_V + C * LDV * 2;
  static constexpr int OFF_AL = OFF_AH + C * LDA * 2;
  static constexpr int OFF_G = OFF_AL + C * LDA * 2;
  static constexpr int BYTES = OFF_G + C * 4;
};

// Causal 16x16 tiles (c tile, j tile) of the 64 x 64 A matrix.
__constant__ int8_t kTileC[10] = {0, 1, 1, 2, 2, 2, 3, 3, 3, 3};
__constant__ int8_t kTileJ[10] = {0, 0, 1, 0, 1, 2, 0, 1, 2, 3};

template <int K, bool PREFETCH, typename TOut>
__global__ void __launch_bounds__(NTHREADS)
chunk_fwd_bf16_kernel(const bf16* __restrict__ q, const bf16* __restrict__ k,
                      const bf16* __restrict__ v, const float* __restrict__ gc,
                      const float* __restrict__ g_gamma, const float* __restrict__ h0,
                      TOut* __restrict__ o, float* __restrict__ ht, float scale, int32_t H,
                      int32_t V, SeqLayout seqs) {
  using S = Smem<K>;
  constexpr int LDQ = S::LDQ;
  constexpr int LDK = S::LDK;
  constexpr int SEG = K / 8;                 // 16-byte segments per q/k row
  constexpr int NQ = C * SEG / NTHREADS;     // q (and k) segments per thread
  constexpr int NV = C * (VT / 8) / NTHREADS;  // v segments per thread (2)
  constexpr int KT = K / 16;                 // 16-row state tiles per wave
  constexpr int KS = K / 32;                 // 32-deep k steps
  static_assert(NQ * NTHREADS == C * SEG, "K must be a multiple of 32");

  __shared__ __attribute__((aligned(16))) char smem[S::BYTES];
  bf16* sQ = reinterpret_cast<bf16*>(smem + S::OFF_Q);
  bf16* sK = reinterpret_cast<bf16*>(smem + S::OFF_K);
  bf16* sV = reinterpret_cast<bf16*>(smem + S::OFF_V);
  bf16* sAh = reinterpret_cast<bf16*>(smem + S::OFF_AH);
  bf16* sAl = reinterpret_cast<bf16*>(smem + S::OFF_AL);
  float* sG = reinterpret_cast<float*>(smem + S::OFF_G);

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
    bos = e.bos;
    len = e.len;
    seq = e.seq;
  } else {
    bos = (int64_t)rank * seqs.T;
    len = seqs.T;
    seq = rank;
  }
  const int nchunks = (len + C - 1) / C;

  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int lane = tid & 63;
  const int g4 = lane >> 4;   // 16-lane group 0..3
  const int r = lane & 15;
  const int vcol = vt * VT + 16 * w + r;   // this lane's state / output column
  const int64_t row_stride_qk = (int64_t)H * K;
  const int64_t row_stride_v = (int64_t)H * V;
  const float gam2 = g_gamma != nullptr ? g_gamma[hd] * kRcpLn2f : 0.f;

  // Upper-triangle A tiles are never written: zero both A buffers once.
  for (int i = tid; i < 2 * C * LDA / 8; i += NTHREADS)
    reinterpret_cast<uint4*>(sAh)[i] = make_uint4(0, 0, 0, 0);

  // ---- state in registers: h[kt][i] = state[16kt + 4g + i][vcol] ---------
  f32x4 h[KT];
  {
    const float* h0u = h0 != nullptr ? h0 + ((int64_t)seq * H + hd) * K * V : nullptr;
#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        h[kt][i] = h0u != nullptr ? h0u[(int64_t)(16 * kt + 4 * g4 + i) * V + vcol] : 0.f;
  }

  // ---- chunk staging registers -------------------------------------------
  uint4 pq[NQ], pk[NQ], pv[NV];
  float pg = 0.f;
  auto load_chunk = [&](int m) {
    const int64_t t0 = bos + (int64_t)m * C;
    const int cl = min(C, len - m * C);
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
      const int s = tid + i * NTHREADS;
      const int row = s / SEG, c8 = s % SEG;
      if (row < cl) {
        const int64_t off = (t0 + row) * row_stride_qk + (int64_t)hd * K + c8 * 8;
        pq[i] = *reinterpret_cast<const uint4*>(q + off);
        pk[i] = *reinterpret_cast<const uint4*>(k + off);
      } else {
        pq[i] = make_uint4(0, 0, 0, 0);
        pk[i] = make_uint4(0, 0, 0, 0);
      }
    }
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int s = tid + i * NTHREADS;
      const int row = s / (VT / 8), c8 = s % (VT / 8);
      if (row < cl) {
        const int64_t off = (t0 + row) * row_stride_v + (int64_t)hd * V + vt * VT + c8 * 8;
        pv[i] = *reinterpret_cast<const uint4*>(v + off);
      } else {
        pv[i] = make_uint4(0, 0, 0, 0);
      }
    }
    if (tid < C) {
      // rows past the chunk's end repeat the last gate value so that their
      // (zero) k and v rows get a finite decay factor
      const int c = min(tid, cl - 1);
      if (gc != nullptr) pg = gc[(t0 + c) * H + hd];
      else pg = (float)(c + 1) * gam2;
    }
  };
  auto store_chunk = [&]() {
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
      const int s = tid + i * NTHREADS;
      const int row = s / SEG, c8 = s % SEG;
      *reinterpret_cast<uint4*>(sQ + row * LDQ + c8 * 8) = pq[i];
      *reinterpret_cast<uint4*>(sK + row * LDK + c8 * 8) = pk[i];
    }
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int s = tid + i * NTHREADS;
      const int row = s / (VT / 8), c8 = s % (VT / 8);
      *reinterpret_cast<uint4*>(sV + row * LDV + c8 * 8) = pv[i];
    }
    if (tid < C) sG[tid] = pg;
  };

  if (nchunks > 0 && PREFETCH) load_chunk(0);

  for (int m = 0; m < nchunks; ++m) {
    if (!PREFETCH) load_chunk(m);
    store_chunk();
    __syncthreads();
    if (PREFETCH && m + 1 < nchunks) load_chunk(m + 1);
    const int64_t t0 = bos + (int64_t)m * C;
    const int cl = min(C, len - m * C);

    // ---- A = (Q K^T) (.) M, split into bf16 hi + lo, into LDS ------------
    for (int ti = w; ti < 10; ti += 4) {
      const int ct = kTileC[ti], jt = kTileJ[ti];
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(sK + (16 * jt + r) * LDK + 32 * s + 8 * g4);
        const bf16x8 b = *reinterpret_cast<const bf16x8*>(sQ + (16 * ct + r) * LDQ + 32 * s + 8 * g4);
        acc = mfma(a, b, acc);  // acc[i] = (q_c . k_j), c = 16ct + r, j = 16jt + 4g + i
      }
      const int c = 16 * ct + r;
      const float bc = sG[c];
      bf16x4 hi, lo;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = 16 * jt + 4 * g4 + i;
        const float x = (j <= c) ? acc[i] * exp2f(bc - sG[j]) : 0.f;
        const bf16 hv = (bf16)x;
        hi[i] = hv;
        lo[i] = (bf16)(x - (float)hv);
      }
      *reinterpret_cast<bf16x4*>(sAh + c * LDA + 16 * jt + 4 * g4) = hi;
      *reinterpret_cast<bf16x4*>(sAl + c * LDA + 16 * jt + 4 * g4) = lo;
    }
    __syncthreads();

    // ---- O = scale * (diag(2^b) Q h + A V) for this wave's 16 columns -----
    f32x4 oacc[4];
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) oacc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      // B operand from the state: k rows 32s + 4g + {0..3} and 32s + 16 + 4g + {0..3}
      float x[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[i] = h[2 * s][i];
        x[4 + i] = h[2 * s + 1][i];
      }
      bf16x8 bh, bl;
      split8(x, bh, bl);
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        const bf16* qrow = sQ + (16 * ct + r) * LDQ + 32 * s + 4 * g4;
        const bf16x8 a = cat(*reinterpret_cast<const bf16x4*>(qrow),
                             *reinterpret_cast<const bf16x4*>(qrow + 16));
        oacc[ct] = mfma(a, bh, oacc[ct]);
        oacc[ct] = mfma(a, bl, oacc[ct]);
      }
    }
#pragma unroll
    for (int ct = 0; ct < 4; ++ct)
#pragma unroll
      for (int i = 0; i < 4; ++i) oacc[ct][i] *= exp2f(sG[16 * ct + 4 * g4 + i]);

    // V tile fragments: vf[s][e] = V[32s + 8g + e][16w + r]
    bf16x8 vf[2];
#pragma unroll
    for (int s = 0; s < 2; ++s)
      vf[s] = cat(tr_read(sV, LDV, 32 * s + 8 * g4, 16 * w),
                  tr_read(sV, LDV, 32 * s + 8 * g4 + 4, 16 * w));
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      const int nsteps = ct < 2 ? 1 : 2;   // j < 32 suffices for c < 32
#pragma unroll
      for (int s = 0; s < nsteps; ++s) {
        const bf16x8 ah = *reinterpret_cast<const bf16x8*>(sAh + (16 * ct + r) * LDA + 32 * s + 8 * g4);
        const bf16x8 al = *reinterpret_cast<const bf16x8*>(sAl + (16 * ct + r) * LDA + 32 * s + 8 * g4);
        oacc[ct] = mfma(ah, vf[s], oacc[ct]);
        oacc[ct] = mfma(al, vf[s], oacc[ct]);
      }
    }
#pragma unroll
    for (int ct = 0; ct < 4; ++ct)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int c = 16 * ct + 4 * g4 + i;
        if (c < cl) o[((t0 + c) * H + hd) * (int64_t)V + vcol] = (TOut)(oacc[ct][i] * scale);
      }

    // ---- h <- 2^b_last h + K^T (diag(2^(b_last - b)) V) --------------------
    const float blast = sG[C - 1];
    const float dall = exp2f(blast);
#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i) h[kt][i] *= dall;
    bf16x8 vth[2], vtl[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      float x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = (float)vf[s][e] * exp2f(blast - sG[32 * s + 8 * g4 + e]);
      split8(x, vth[s], vtl[s]);
    }
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        // A operand: K^T[16kt + r][32s + 8g + e]
        const bf16x8 a = cat(tr_read(sK, LDK, 32 * s + 8 * g4, 16 * kt),
                             tr_read(sK, LDK, 32 * s + 8 * g4 + 4, 16 * kt));
        h[kt] = mfma(a, vth[s], h[kt]);
        h[kt] = mfma(a, vtl[s], h[kt]);
      }
    }
    __syncthreads();
  }

  if (ht != nullptr) {
    float* htu = ht + ((int64_t)seq * H + hd) * K * V;
#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i) htu[(int64_t)(16 * kt + 4 * g4 + i) * V + vcol] = h[kt][i];
  }
}

template <int K, bool PREFETCH, typename TOut>
hipError_t launch_k(const ChunkFwdParams& p, hipStream_t stream) {
  const int num_units = p.seqs.num_seqs * p.H;
  if (num_units == 0) return hipSuccess;
  const int nvt = p.V / VT;
  const int groups = (num_units + kXcds - 1) / kXcds;
  const dim3 grid((unsigned)(groups * kXcds * nvt));
  hipLaunchKernelGGL((chunk_fwd_bf16_kernel<K, PREFETCH, TOut>), grid, dim3(NTHREADS), 0, stream,
                     static_cast<const bf16*>(p.q), static_cast<const bf16*>(p.k),
                     static_cast<const bf16*>(p.v), p.gc, p.g_gamma, p.h0,
                     static_cast<TOut*>(p.o), p.ht, p.scale, p.H, p.V, p.seqs);
  return hipGetLastError();
}

template <typename TOut>
hipError_t launch_out(const ChunkFwdParams& p, hipStream_t stream) {
  switch (p.K) {
    case 64: return launch_k<64, true, TOut>(p, stream);
    case 128: return launch_k<128, true, TOut>(p, stream);
    case 256: return launch_k<256, true, TOut>(p, stream);
    case 512: return launch_k<512, false, TOut>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_chunk_fwd_bf16(const ChunkFwdParams& p, hipStream_t stream) {
  return p.o_bf16 ? launch_out<__bf16>(p, stream) : launch_out<float>(p, stream);
}

}  // namespace sgla
