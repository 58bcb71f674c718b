// Entering states of the later segments of long sequences (bf16 q/k/v, K in
// {64, 128}), so that the segments of one sequence run their chunk chains in
// parallel (page "flash-linear-attention 中的 Simple GLA", section 一: the
// state after a stretch of tokens is the decayed state before it plus the
// stretch's own k v^T sum, the inter-chunk relation that section 三's state
// pass applies chunk by chunk -- here applied to blocks of chunks).
//
// For a block of whole chunks of one (sequence, head), with G the block's
// cumulative log2 gate (restarting at the block) and G_end its value at the
// block's last token:
//   U     = sum_t 2^(G_end - G_t) k_t v_t^T      (the block's state from zero)
//   a     = G_end                                (its total log2 decay)
// and across the blocks of a sequence, S_0 = initial state, S_{b+1} = 2^a_b
// S_b + U_b.  The entering state of segment s is S at the first block of s.
//
// Two launches:
//   segment_prepass_kernel -- one 4-wave workgroup per (block, head, 64-wide V
//     tile), a state-only chunk chain over the block: per chunk the update
//     U <- 2^b_last U + K^T (diag(2^(b_last - b)) V) of the chunk kernels, on
//     the bf16 matrix cores with the decayed V split into bf16 hi + lo (the
//     same precision as the forward's own state update), U in fp32 MFMA
//     accumulators; chunk staging double-buffered in LDS, loads two chunks
//     ahead.  Writes U and a.
//   segment_scan_kernel -- per (sequence, head, 1024 state elements), walks
//     the sequence's blocks in order and writes S into the entering-state
//     record a block ends on.
// When the segment, bin, block and scan tables fit one kernel-argument
// payload, the pre-pass carries them: its workgroup 0 writes them to the
// workspace (for the scan and the chunk kernel, which run after it) and every
// workgroup reads its block entry from the arguments, so no separate table
// launch is needed.
#include <hip/hip_runtime.h>

#include "gate_scan.h"
#include "mfma_common.h"
#include "sgla_internal.h"
#include "unit_map.h"

namespace sgla {
namespace {

using namespace mf;

constexpr int C = kChunk;
constexpr int VT = 64;            // state columns per workgroup (16 per wave)
constexpr int NT = 256;           // 4 waves
constexpr int LDV = VT + 16;      // V tile row stride (elements)

template <int K>
struct PreLayout {
  static constexpr int LDK = K + 16;
  static constexpr int SZ_K = C * LDK * 2;
  static constexpr int SZ_V = C * LDV * 2;
  static constexpr int SZ_D = C * 4;
  static constexpr int SZ_STAGE = SZ_K + SZ_V + SZ_D + 16;
  static constexpr int BYTES = 2 * SZ_STAGE;
};

// The tables travel in the arguments (INLINE) or sit in the workspace.
template <bool INLINE>
struct PreTables;
template <>
struct PreTables<false> {
  const BlockEntry* blocks;
};
template <>
struct PreTables<true> {
  TableWords words;   // the table region, from its first word
  uint32_t* dst;      // where the region goes in the workspace
  int32_t blk_word;   // first word of the block table within the region
};

template <int K, bool INLINE>
__global__ void __launch_bounds__(NT)
segment_prepass_kernel(const bf16* __restrict__ k, const bf16* __restrict__ v, const float* __restrict__ g,
                       const float* __restrict__ g_gamma, int32_t H, int32_t Hkv, int32_t V,
                       PreTables<INLINE> tables, int32_t num_blocks, float* __restrict__ urec,
                       float* __restrict__ ulog) {
  using L = PreLayout<K>;
  constexpr int SEG = K / 8;                 // 16-byte pieces per k row
  constexpr int NK = C * SEG / NT;           // k pieces per thread
  constexpr int NV = C * (VT / 8) / NT;      // v pieces per thread
  constexpr int KT = K / 16;                 // 16-row state tiles per wave
  static_assert(NK * NT == C * SEG && NV * NT == C * (VT / 8), "load split");
  __shared__ __attribute__((aligned(16))) char smem[L::BYTES];

  if constexpr (INLINE) {
    if (blockIdx.x == 0)
      for (int i = threadIdx.x; i < tables.words.count; i += NT) tables.dst[i] = tables.words.w[i];
  }
  const UnitMap um = map_unit(blockIdx.x, V / VT, Hkv, H / Hkv, num_blocks);
  if (!um.valid) return;
  const int rank = um.rank, hd = um.hd, hk = um.hk, vt = um.vt;
  BlockEntry be;
  if constexpr (INLINE) {
    const uint32_t* bw = tables.words.w + tables.blk_word + 4 * rank;
    be.t0 = (int32_t)bw[0];
    be.len = (int32_t)bw[1];
    be.out_rec = (int32_t)bw[2];
  } else {
    be = tables.blocks[rank];
  }
  const int64_t t0 = __builtin_amdgcn_readfirstlane(be.t0);
  const int32_t len = __builtin_amdgcn_readfirstlane(be.len);
  const int nchunks = (len + C - 1) / C;

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int g4 = lane >> 4;
  const int r = lane & 15;
  const int RSK = Hkv * K;
  const int RSV = Hkv * V;
  const bf16* kb = k + (t0 * Hkv + hk) * (int64_t)K;
  const bf16* vb = v + (t0 * Hkv + hk) * (int64_t)V + vt * VT;
  const float* gb = g != nullptr ? g + t0 * H + hd : nullptr;
  const float gam2 = g_gamma != nullptr
                         ? __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(
                                                         __builtin_bit_cast(int, g_gamma[hd]))) * kRcpLn2f
                         : 0.f;

  auto sK = [&](int p) { return reinterpret_cast<bf16*>(smem + p * L::SZ_STAGE); };
  auto sV = [&](int p) { return reinterpret_cast<bf16*>(smem + p * L::SZ_STAGE + L::SZ_K); };
  auto sD = [&](int p) { return reinterpret_cast<float*>(smem + p * L::SZ_STAGE + L::SZ_K + L::SZ_V); };
  auto sAll = [&](int p) {
    return reinterpret_cast<float*>(smem + p * L::SZ_STAGE + L::SZ_K + L::SZ_V + L::SZ_D);
  };

  struct Stage {
    u32x4 k[NK], v[NV];
    float g;
    int len;
  };
  auto load_chunk = [&](int m, Stage& st) {
    const int cl = max(0, min(C, len - m * C));
    st.len = cl;
    const int64_t tok = (int64_t)m * C;
    const auto rk = make_rsrc(kb + tok * RSK, (uint32_t)cl * RSK * 2);
    const auto rv = make_rsrc(vb + tok * RSV, (uint32_t)cl * RSV * 2);
#pragma unroll
    for (int i = 0; i < NK; ++i) {
      const int s = tid + i * NT;
      st.k[i] = __builtin_amdgcn_raw_buffer_load_b128(rk, ((s / SEG) * RSK + (s % SEG) * 8) * 2, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int s = tid + i * NT;
      st.v[i] = __builtin_amdgcn_raw_buffer_load_b128(rv, ((s / (VT / 8)) * RSV + (s % (VT / 8)) * 8) * 2, 0, 0);
    }
    st.g = 0.f;
    if (gb != nullptr) {
      const auto rg = make_rsrc(gb + tok * H, (uint32_t)cl * H * 4);
      st.g = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rg, (uint32_t)(lane * H * 4), 0, 0));
    }
  };
  double total = 0.0;   // the block's log2 decay (wave 0 keeps it)
  auto store_chunk = [&](int p, const Stage& st) {
    bf16* k_s = sK(p);
    bf16* v_s = sV(p);
#pragma unroll
    for (int i = 0; i < NK; ++i) {
      const int s = tid + i * NT;
      *reinterpret_cast<u32x4*>(k_s + (s / SEG) * L::LDK + (s % SEG) * 8) = st.k[i];
    }
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int s = tid + i * NT;
      *reinterpret_cast<u32x4*>(v_s + (s / (VT / 8)) * LDV + (s % (VT / 8)) * 8) = st.v[i];
    }
    if (w == 0) {
      // chunk-local cumulative log2 gate b (rows past the chunk's end add 0),
      // then 2^(b_last - b) per token and 2^b_last for the chunk
      const float b = gb != nullptr ? wave_cumsum_log2(st.g) : (float)min(lane + 1, st.len) * gam2;
      const float blast = __shfl(b, C - 1, 64);
      sD(p)[lane] = exp2_hw(blast - b);
      if (lane == 0) sAll(p)[0] = exp2_hw(blast);
      total += (double)blast;
    }
  };

  // U tiles of this wave: columns [16 w, 16 w + 16) of the V tile, all K rows;
  // u[kt][i] = U[16 kt + 4 g + i][16 w + r]
  f32x4 u[KT];
#pragma unroll
  for (int kt = 0; kt < KT; ++kt) u[kt] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto update = [&](int p) {
    const bf16* k_s = sK(p);
    const bf16* v_s = sV(p);
    const float* d_s = sD(p);
    const float dall = sAll(p)[0];
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) u[kt] *= dall;
    bf16x8 vth[2], vtl[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      // V[32 s + 8 g + e][16 w + r] times 2^(b_last - b) of its token
      const bf16x8 vf = cat(tr_read(v_s, LDV, 32 * s + 8 * g4, 16 * w), tr_read(v_s, LDV, 32 * s + 8 * g4 + 4, 16 * w));
      const f32x4 d0 = *reinterpret_cast<const f32x4*>(d_s + 32 * s + 8 * g4);
      const f32x4 d1 = *reinterpret_cast<const f32x4*>(d_s + 32 * s + 8 * g4 + 4);
      const u32x4 raw = __builtin_bit_cast(u32x4, vf);
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
#pragma unroll
    for (int s = 0; s < 2; ++s) {
#pragma unroll
      for (int k0 = 0; k0 < KT; k0 += 4) {
        bf16x8 a[4];
#pragma unroll
        for (int q = 0; q < 4; ++q)
          a[q] = cat(tr_read(k_s, L::LDK, 32 * s + 8 * g4, 16 * (k0 + q)),
                     tr_read(k_s, L::LDK, 32 * s + 8 * g4 + 4, 16 * (k0 + q)));
#pragma unroll
        for (int q = 0; q < 4; ++q) u[k0 + q] = mfma(a[q], vth[s], u[k0 + q]);
#pragma unroll
        for (int q = 0; q < 4; ++q) u[k0 + q] = mfma(a[q], vtl[s], u[k0 + q]);
      }
    }
  };

  Stage st0, st1;
  load_chunk(0, st0);
  load_chunk(1, st1);
  auto step = [&](const int m, const int p, Stage& st) {
    store_chunk(p, st);
    __syncthreads();   // chunk m staged; every read of this parity's previous chunk is done
    load_chunk(m + 2, st);
    update(p);
  };
  int m = 0;
  for (; m + 1 < nchunks; m += 2) {
    step(m, 0, st0);
    step(m + 1, 1, st1);
  }
  if (m < nchunks) step(m, 0, st0);

  float* ub = urec + ((int64_t)rank * H + hd) * K * V + vt * VT + 16 * w + r;
#pragma unroll
  for (int kt = 0; kt < KT; ++kt)
#pragma unroll
    for (int i = 0; i < 4; ++i) ub[(int64_t)(16 * kt + 4 * g4 + i) * V] = u[kt][i];
  if (vt == 0 && tid == 0) ulog[(int64_t)rank * H + hd] = (float)total;
}

// One thread per 4 consecutive elements of the [K][V] state of one (scanned
// sequence, head); a workgroup covers 1024 elements.
__global__ void __launch_bounds__(256)
segment_scan_kernel(const float* __restrict__ h0, int32_t H, int32_t K, int32_t V, StateLayout sl,
                    const BlockEntry* __restrict__ blocks, const ScanEntry* __restrict__ scans,
                    const float* __restrict__ urec, const float* __restrict__ ulog, float* __restrict__ sin) {
  const int parts = K * V / 1024;
  const int part = blockIdx.x % parts;
  const int hd = (blockIdx.x / parts) % H;
  const ScanEntry se = scans[blockIdx.x / parts / H];
  const int e = part * 1024 + threadIdx.x * 4;   // first of this thread's 4 elements
  const int row = e / V, col = e % V;
  const int64_t KV = (int64_t)K * V;
  f32x4 s = {0.f, 0.f, 0.f, 0.f};
  if (h0 != nullptr) {
    const float* hb = h0 + ((int64_t)se.seq * H + hd) * KV;
#pragma unroll
    for (int i = 0; i < 4; ++i) s[i] = hb[(int64_t)row * sl.rs + (int64_t)(col + i) * sl.cs];
  }
  for (int b = se.first_block; b < se.first_block + se.num_blocks; ++b) {
    const f32x4 ub = *reinterpret_cast<const f32x4*>(urec + ((int64_t)b * H + hd) * KV + e);
    const float a = exp2_hw(ulog[(int64_t)b * H + hd]);
    s = s * a + ub;
    const int rec = blocks[b].out_rec;
    if (rec >= 0) *reinterpret_cast<f32x4*>(sin + ((int64_t)rec * H + hd) * KV + e) = s;
  }
}

template <int K>
hipError_t launch_pre(const SegmentParams& p, hipStream_t stream) {
  const dim3 grid((unsigned)unit_grid(p.num_blocks, p.Hkv, p.H / p.Hkv, p.V / VT));
  const bf16* kp = static_cast<const bf16*>(p.k);
  const bf16* vp = static_cast<const bf16*>(p.v);
  if (p.inline_tables != nullptr) {
    PreTables<true> t;
    t.words = *p.inline_tables;
    t.dst = p.table_dst;
    t.blk_word = p.blk_word;
    hipLaunchKernelGGL((segment_prepass_kernel<K, true>), grid, dim3(NT), 0, stream, kp, vp, p.g, p.g_gamma, p.H,
                       p.Hkv, p.V, t, p.num_blocks, p.urec, p.ulog);
  } else {
    PreTables<false> t;
    t.blocks = p.blocks;
    hipLaunchKernelGGL((segment_prepass_kernel<K, false>), grid, dim3(NT), 0, stream, kp, vp, p.g, p.g_gamma,
                       p.H, p.Hkv, p.V, t, p.num_blocks, p.urec, p.ulog);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_segment_states(const SegmentParams& p, hipStream_t stream) {
  if (p.num_blocks == 0 || p.num_scans == 0) return hipSuccess;
  if (p.V % VT != 0 || (p.K * p.V) % 1024 != 0) return hipErrorInvalidValue;
  hipError_t e;
  switch (p.K) {
    case 64: e = launch_pre<64>(p, stream); break;
    case 128: e = launch_pre<128>(p, stream); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess) return e;
  const int parts = p.K * p.V / 1024;
  hipLaunchKernelGGL(segment_scan_kernel, dim3((unsigned)(p.num_scans * p.H * parts)), dim3(256), 0, stream,
                     p.h0, p.H, p.K, p.V, p.sl, p.blocks, p.scans, p.urec, p.ulog, p.sin);
  return hipGetLastError();
}

}  // namespace sgla
