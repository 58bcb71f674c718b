// The parts of the bf16 chunked Simple GLA backward that reduce over all
// keys when K is 256 or 512 (page "flash-linear-attention 中的 Simple GLA",
// section 三: the v gradient pass and the gate gradient recovered by a
// reverse cumulative sum; section 五: dv and dg).  Per chunk, with b the
// chunk-local cumulative log2 gate, dv_j = 2^(b_last - b_j) and dH the
// gradient of the state leaving the chunk (the state pass's fp32 record):
//   dV = A^T dO + diag(dv) K dH,   A = scale (Q K^T) (.) M,  M_cj = 2^(b_c - b_j) (j <= c)
// and, from the key-tile gate records of the dq/dk kernel,
//   dg_t = sum over s >= t in the chunk of r_s, plus at the chunk's last
//   token 2^b_last <dH, h> + sum_j dv_j k_j . (V dH^T)_j,
// which is the per-chunk algebra of the K <= 128 gradient kernel with the
// sums over keys split into tiles and added here in a fixed order.
//
// dV kernel: one workgroup per (chunk, head, 64-column V tile), 8 waves.
// Keys are walked in 64-key slices (each loaded into registers one slice
// ahead): Q K^T accumulates A while K dH accumulates the state term, so A
// costs one extra read of the Q rows rather than a workspace round trip.
// Wave w takes row tile rw = w % 4 (tokens [16 rw, +16)) and column tiles
// {2 kh, 2 kh + 1}, kh = w / 4, of both A and the dV tile.  dH is split
// into bf16 hi + lo planes and A likewise, each product issued twice.
#include <hip/hip_runtime.h>

#include "gate_scan.h"
#include "mfma_common.h"
#include "sgla_internal.h"
#include "unit_map.h"

namespace sgla {
namespace {

using namespace mf;

constexpr int C = kChunk;
constexpr int NT = 512;             // threads (8 waves)
constexpr int VW = kWideDvCols;     // V columns per workgroup
constexpr int KS = 64;              // keys per slice
constexpr int LDX = KS + 8;         // Q / K slice row stride (elements)
constexpr int LDD = VW + 8;         // dH slice and dO tile row stride (elements)
constexpr int LDA = C + 8;          // A row stride (elements)

struct DvLayout {
  static constexpr int OFF_Q = 0;
  static constexpr int OFF_K = OFF_Q + C * LDX * 2;
  static constexpr int OFF_DH = OFF_K + C * LDX * 2;        // hi plane, then lo
  static constexpr int OFF_A = OFF_DH + 2 * KS * LDD * 2;   // hi plane, then lo
  static constexpr int OFF_O = OFF_A + 2 * C * LDA * 2;
  static constexpr int OFF_F = OFF_O + C * LDD * 2;         // sb, sdv
  static constexpr int BYTES = OFF_F + 2 * C * 4;
  static_assert(BYTES <= 80 * 1024, "two workgroups per CU");
  static_assert(OFF_K % 16 == 0 && OFF_DH % 16 == 0 && OFF_A % 16 == 0 && OFF_O % 16 == 0 &&
                    OFF_F % 16 == 0,
                "16-byte aligned areas");
};

// x written as its bf16 hi into plane[i] and lo into plane[i + lo_off]
__device__ __forceinline__ void put_split(bf16* plane, int i, int lo_off, float x) {
  const bf16 hi = (bf16)x;
  plane[i] = hi;
  plane[i + lo_off] = (bf16)(x - (float)hi);
}

__device__ __forceinline__ void chunk_of(const SeqLayout& seqs, int gc, int chunks_per_row, int64_t& t0,
                                         int& cl) {
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
}

// Chunk-local cumulative log2 gate, lane = token offset (wave-wide); padding
// tokens add nothing.
__device__ __forceinline__ float chunk_gate_log2(const float* g, const float* g_gamma, int H, int hd, int64_t t0,
                                                 int cl) {
  const int lane = threadIdx.x & 63;
  if (g != nullptr) return wave_cumsum_log2(lane < cl ? g[(t0 + lane) * H + hd] : 0.f);
  if (g_gamma != nullptr) return (float)min(lane + 1, cl) * (g_gamma[hd] * kRcpLn2f);
  return 0.f;
}

__global__ void __launch_bounds__(NT)
chunk_bwd_dv_wide_kernel(const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ dout,
                         const float* __restrict__ g, const float* __restrict__ g_gamma, float scale, int32_t H,
                         int32_t Hkv, int32_t K, int32_t V, SeqLayout seqs, int32_t chunks_per_row,
                         const float* __restrict__ dhbuf, float* __restrict__ dv) {
  using L = DvLayout;
  __shared__ __attribute__((aligned(16))) char smem[L::BYTES];
  bf16* const sQ = reinterpret_cast<bf16*>(smem + L::OFF_Q);
  bf16* const sK = reinterpret_cast<bf16*>(smem + L::OFF_K);
  bf16* const sdH = reinterpret_cast<bf16*>(smem + L::OFF_DH);
  bf16* const sA = reinterpret_cast<bf16*>(smem + L::OFF_A);
  bf16* const sO = reinterpret_cast<bf16*>(smem + L::OFF_O);
  float* const sb = reinterpret_cast<float*>(smem + L::OFF_F);
  float* const sdv = sb + C;
  constexpr int DLO = KS * LDD;       // offset of the dH lo plane
  constexpr int ALO = C * LDA;        // offset of the A lo plane

  // the V tiles of one (chunk, head) run on one XCD, whose L2 then serves
  // their repeated reads of the Q and K rows
  const UnitMap um = map_unit((int32_t)blockIdx.x, V / VW, H, 1, seqs.num_chunks);
  if (!um.valid) return;
  const int gc = um.rank, hd = um.hk, vt = um.vt;
  int64_t t0;
  int cl;
  chunk_of(seqs, gc, chunks_per_row, t0, cl);
  const int tid = threadIdx.x, lane = tid & 63, g4 = lane >> 4, r = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index, uniform
  const int rw = w & 3, kh = w >> 2;
  const int hk = hd / (H / Hkv);   // kv head whose k rows this query head reads
  const int64_t col0 = (int64_t)vt * VW;
  const float* dhu = dhbuf + ((int64_t)gc * H + hd) * ((int64_t)K * V) + col0;

  // ---- the dO tile (zero past the chunk's end) and the gates ---------------
  {
    static_assert(C * (VW / 8) == NT, "one 16-byte piece per thread");
    const int c = tid / (VW / 8), e = 8 * (tid % (VW / 8));
    uint4 x = make_uint4(0u, 0u, 0u, 0u);
    if (c < cl) x = *reinterpret_cast<const uint4*>(dout + ((t0 + c) * H + hd) * V + col0 + e);
    *reinterpret_cast<uint4*>(sO + c * LDD + e) = x;
  }
  if (w == 0) {
    const float b = chunk_gate_log2(g, g_gamma, H, hd, t0, cl);
    sb[lane] = b;
    sdv[lane] = exp2f(__shfl(b, C - 1, 64) - b);
  }

  // ---- key slices: Q and K columns as bf16 pieces, dH rows as fp32 pieces
  static_assert(C * (KS / 8) == NT && (KS * VW / 4) == 2 * NT, "slice split");
  uint4 qx, kx;
  f32x4 dhx[2];
  auto load_slice = [&](int s) {
    const int c = tid / (KS / 8), e = 8 * (tid % (KS / 8));
    qx = make_uint4(0u, 0u, 0u, 0u);
    kx = qx;
    if (c < cl) {
      qx = *reinterpret_cast<const uint4*>(q + ((t0 + c) * H + hd) * K + s * KS + e);
      kx = *reinterpret_cast<const uint4*>(k + ((t0 + c) * Hkv + hk) * K + s * KS + e);
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int p = tid + NT * u;
      const int row = p / (VW / 4), c4 = p % (VW / 4);
      dhx[u] = *reinterpret_cast<const f32x4*>(dhu + (int64_t)(s * KS + row) * V + 4 * c4);
    }
  };
  auto store_slice = [&]() {
    const int c = tid / (KS / 8), e = 8 * (tid % (KS / 8));
    *reinterpret_cast<uint4*>(sQ + c * LDX + e) = qx;
    *reinterpret_cast<uint4*>(sK + c * LDX + e) = kx;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int p = tid + NT * u;
      const int o = (p / (VW / 4)) * LDD + 4 * (p % (VW / 4));
      const f32x4 x = dhx[u];
      uint32_t h0, l0, h1, l1;
      split2(x[0], x[1], h0, l0);
      split2(x[2], x[3], h1, l1);
      *reinterpret_cast<u32x2*>(sdH + o) = u32x2{h0, h1};
      *reinterpret_cast<u32x2*>(sdH + DLO + o) = u32x2{l0, l1};
    }
  };

  f32x4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};   // Q K^T
  f32x4 st[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};    // K dH
  const int nks = K / KS;
  load_slice(0);
  for (int s = 0; s < nks; ++s) {
    __syncthreads();   // previous slice's reads done
    store_slice();
    if (s + 1 < nks) load_slice(s + 1);
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < KS / 32; ++ks) {
      const bf16x8 aq = *reinterpret_cast<const bf16x8*>(sQ + (16 * rw + r) * LDX + 32 * ks + 8 * g4);
      const bf16x8 ak = *reinterpret_cast<const bf16x8*>(sK + (16 * rw + r) * LDX + 32 * ks + 8 * g4);
      const int k0 = 32 * ks + 8 * g4;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int ct = 16 * (2 * kh + t);
        acc[t] = mfma(aq, *reinterpret_cast<const bf16x8*>(sK + (ct + r) * LDX + 32 * ks + 8 * g4), acc[t]);
        const bf16x8 bh = cat(tr_read(sdH, LDD, k0, ct), tr_read(sdH, LDD, k0 + 4, ct));
        const bf16x8 bl = cat(tr_read(sdH + DLO, LDD, k0, ct), tr_read(sdH + DLO, LDD, k0 + 4, ct));
        st[t] = mfma(ak, bh, st[t]);
        st[t] = mfma(ak, bl, st[t]);
      }
    }
  }

  // ---- A masked and scaled, split into the A planes ---------------------------
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int j = 16 * (2 * kh + t) + r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = 16 * rw + 4 * g4 + i;
      put_split(sA, c * LDA + j, ALO, j <= c ? acc[t][i] * exp2f(sb[c] - sb[j]) * scale : 0.f);
    }
  }
  __syncthreads();

  // ---- dV = A^T dO + diag(dv) K dH: rows [16 rw, +16), columns 2 kh, 2 kh + 1
  f32x4 in[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
  const int cs0 = rw >= 2 ? 1 : 0;   // first 32-token block with A[c][j] != 0 for j in tile rw
  for (int cs = cs0; cs < 2; ++cs) {
    const int c0 = 32 * cs + 8 * g4;
    const bf16x8 ah = cat(tr_read(sA, LDA, c0, 16 * rw), tr_read(sA, LDA, c0 + 4, 16 * rw));
    const bf16x8 al = cat(tr_read(sA + ALO, LDA, c0, 16 * rw), tr_read(sA + ALO, LDA, c0 + 4, 16 * rw));
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int ct = 16 * (2 * kh + t);
      const bf16x8 bo = cat(tr_read(sO, LDD, c0, ct), tr_read(sO, LDD, c0 + 4, ct));
      in[t] = mfma(ah, bo, in[t]);
      in[t] = mfma(al, bo, in[t]);
    }
  }
#pragma unroll
  for (int t = 0; t < 2; ++t) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j = 16 * rw + 4 * g4 + i;
      if (j < cl) dv[((t0 + j) * H + hd) * (int64_t)V + col0 + 16 * (2 * kh + t) + r] = in[t][i] + sdv[j] * st[t][i];
    }
  }
}

// Gate gradient of one (chunk, head) per wave: the key-tile records added in
// tile order (in double), the chunk's share of the state it hands on at its
// last real token, then the reverse cumulative sum over the chunk.  With
// g_gamma, the per-chunk sum of dg goes to gpart.
__global__ void __launch_bounds__(256)
chunk_bwd_gate_wide_kernel(const float* __restrict__ g, const float* __restrict__ g_gamma, int32_t H,
                           int32_t nkt, SeqLayout seqs, int32_t chunks_per_row, const float* __restrict__ wpart,
                           float* __restrict__ dg, float* __restrict__ gpart) {
  const int lane = threadIdx.x & 63;
  const int task = (int)blockIdx.x * 4 + (int)(threadIdx.x >> 6);   // chunk * H + head
  if (task >= seqs.num_chunks * H) return;
  const int gc = task / H, hd = task - gc * H;
  int64_t t0;
  int cl;
  chunk_of(seqs, gc, chunks_per_row, t0, cl);
  const float blast = __shfl(chunk_gate_log2(g, g_gamma, H, hd, t0, cl), C - 1, 64);
  double x = 0.0, extra = 0.0, frob = 0.0;
  for (int kz = 0; kz < nkt; ++kz) {
    const float* rec = wpart + ((int64_t)task * nkt + kz) * kWidePart;
    x += (double)rec[lane];
    extra += (double)rec[C + lane];
    frob += (double)rec[2 * C];
  }
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) extra += __shfl_xor(extra, d, 64);
  if (lane >= cl) x = 0.0;
  if (lane == cl - 1) x += (double)exp2f(blast) * frob + extra;
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
    if (lane == 0) gpart[(int64_t)task] = (float)s;
  }
}

}  // namespace

hipError_t launch_chunk_bwd_dv_wide(const ChunkBwdParams& p, int32_t chunks_per_row, hipStream_t stream) {
  if (p.K % KS != 0 || p.V % VW != 0) return hipErrorInvalidValue;
  if (p.seqs.num_chunks == 0) return hipSuccess;
  hipLaunchKernelGGL(chunk_bwd_dv_wide_kernel, dim3((unsigned)unit_grid(p.seqs.num_chunks, p.H, 1, p.V / VW)),
                     dim3(NT), 0, stream, static_cast<const bf16*>(p.q), static_cast<const bf16*>(p.k),
                     static_cast<const bf16*>(p.dout), p.g, p.g_gamma, p.scale, p.H, p.Hkv, p.K, p.V, p.seqs,
                     chunks_per_row, p.dhbuf, p.dv);
  return hipGetLastError();
}

hipError_t launch_chunk_bwd_gate_wide(const ChunkBwdParams& p, int32_t chunks_per_row, hipStream_t stream) {
  const int64_t tasks = (int64_t)p.seqs.num_chunks * p.H;
  if (tasks == 0 || (p.dg == nullptr && p.dg_gamma == nullptr)) return hipSuccess;
  hipLaunchKernelGGL(chunk_bwd_gate_wide_kernel, dim3((unsigned)((tasks + 3) / 4)), dim3(256), 0, stream, p.g,
                     p.g_gamma, p.H, p.K / 128, p.seqs, chunks_per_row, p.wpart, p.dg,
                     p.dg_gamma != nullptr ? p.gpart : nullptr);
  return hipGetLastError();
}

}  // namespace sgla
