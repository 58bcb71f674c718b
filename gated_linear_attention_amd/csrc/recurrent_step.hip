// Step (4): one decode token per sequence, updating the float32 state in place
// (page "flash-linear-attention 中的 Simple GLA", section 四: for single-token
// inference the layer switches from the chunk kernel to a fused recurrent
// kernel because a chunk launch for one token is slower; section 二: states
// are [N, H, K, V] with S[k][v]):
//
//     S <- exp(g) * S + k v^T ;    o = scale * S^T q   (post-update state),
//
// with g per (sequence, head), or a per-head constant g_gamma[h] (section 二),
// or no decay.  With grouped kv heads, query head h reads the k and v rows of
// kv head h / (H / Hkv) (page "relinear", its GQA target); state and gate stay
// per query head.
//
// The step is a pure read-modify-write stream over the state: 2 * K * V * 4
// bytes per (sequence, head) against 5 * K * V flops, so it is bound by HBM.
// One 256-thread workgroup owns one (sequence, head) state.  Each thread owns
// four adjacent v columns (16-byte accesses) and, when the rows split evenly
// into 4, 8 or 16 per row group, a contiguous block of k rows (row group rg
// owns rows [rg * rpt, +rpt)); otherwise every RG-th row.  Either way each
// load instruction of a wave covers whole contiguous state rows.  All rows of
// a batch are loaded before any is used so that many 16-byte loads are in
// flight per wave; the q-weighted column sums are then reduced across row
// groups through LDS.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "sgla_internal.h"

namespace sgla {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

template <typename T>
__device__ __forceinline__ float to_f32(T x);
template <>
__device__ __forceinline__ float to_f32<float>(float x) { return x; }
template <>
__device__ __forceinline__ float to_f32<__bf16>(__bf16 x) { return (float)x; }

template <int V, typename TIn, typename TOut>
__global__ void __launch_bounds__(256)
recurrent_step_kernel(const TIn* __restrict__ q, const TIn* __restrict__ k,
                      const TIn* __restrict__ v, const float* __restrict__ g,
                      const float* __restrict__ g_gamma, float* __restrict__ state,
                      TOut* __restrict__ o, float scale, int32_t H, int32_t Hkv, int32_t K) {
  constexpr int TPR = V / 4;          // threads per state row
  constexpr int RG = 256 / TPR;       // row groups
  constexpr int BATCH = 16;           // rows in flight per thread
  __shared__ float part[RG][V];

  const int64_t unit = blockIdx.x;    // n * H + h
  const uint32_t n = blockIdx.x / (uint32_t)H;
  const int h = (int)(blockIdx.x - n * (uint32_t)H);
  const int64_t ukv = (int64_t)n * Hkv + h / (H / Hkv);   // (sequence, kv head) row of k and v
  const int tid = threadIdx.x;
  const int cq = tid % TPR;
  const int rg = tid / TPR;
  const float gamma = expf(g != nullptr ? g[unit] : (g_gamma != nullptr ? g_gamma[h] : 0.f));
  const TIn* qu = q + unit * K;
  const TIn* ku = k + ukv * K;
  f32x4 vv;
  {
    const TIn* vu = v + ukv * V + 4 * cq;
    vv = f32x4{to_f32(vu[0]), to_f32(vu[1]), to_f32(vu[2]), to_f32(vu[3])};
  }
  f32x4* S = reinterpret_cast<f32x4*>(state + unit * (int64_t)K * V);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};

  const int rpt = K / RG;             // rows per row group when K % RG == 0
  // the usual case: row group rg owns the contiguous rows [rg * rpt, +rpt),
  // with rpt a compile-time count so nothing is predicated
  auto block_rows = [&](auto rows_c) {
    constexpr int R = decltype(rows_c)::value;
    const int r0 = rg * R;
    f32x4 s[R];
#pragma unroll
    for (int b = 0; b < R; ++b) s[b] = __builtin_nontemporal_load(&S[(int64_t)(r0 + b) * TPR + cq]);
    float kr[R], qr[R];
#pragma unroll
    for (int b = 0; b < R; ++b) {
      kr[b] = to_f32(ku[r0 + b]);
      qr[b] = to_f32(qu[r0 + b]);
    }
#pragma unroll
    for (int b = 0; b < R; ++b) {
      f32x4 x = s[b];
      x.x = fmaf(gamma, x.x, kr[b] * vv.x);
      x.y = fmaf(gamma, x.y, kr[b] * vv.y);
      x.z = fmaf(gamma, x.z, kr[b] * vv.z);
      x.w = fmaf(gamma, x.w, kr[b] * vv.w);
      __builtin_nontemporal_store(x, &S[(int64_t)(r0 + b) * TPR + cq]);
      acc.x = fmaf(x.x, qr[b], acc.x);
      acc.y = fmaf(x.y, qr[b], acc.y);
      acc.z = fmaf(x.z, qr[b], acc.z);
      acc.w = fmaf(x.w, qr[b], acc.w);
    }
  };
  const bool even = K % RG == 0;
  if (even && rpt == 16) {
    block_rows(std::integral_constant<int, 16>{});
  } else if (even && rpt == 8) {
    block_rows(std::integral_constant<int, 8>{});
  } else if (even && rpt == 4) {
    block_rows(std::integral_constant<int, 4>{});
  } else {
    // general K: row group rg owns rows rg, rg + RG, ...
    for (int r0 = rg; r0 < K; r0 += RG * BATCH) {
      f32x4 s[BATCH];
#pragma unroll
      for (int b = 0; b < BATCH; ++b) {
        const int r = r0 + b * RG;
        if (r < K) s[b] = __builtin_nontemporal_load(&S[(int64_t)r * TPR + cq]);
      }
#pragma unroll
      for (int b = 0; b < BATCH; ++b) {
        const int r = r0 + b * RG;
        if (r < K) {
          const float kr = to_f32(ku[r]);
          const float qr = to_f32(qu[r]);
          f32x4 x = s[b];
          x.x = fmaf(gamma, x.x, kr * vv.x);
          x.y = fmaf(gamma, x.y, kr * vv.y);
          x.z = fmaf(gamma, x.z, kr * vv.z);
          x.w = fmaf(gamma, x.w, kr * vv.w);
          __builtin_nontemporal_store(x, &S[(int64_t)r * TPR + cq]);
          acc.x = fmaf(x.x, qr, acc.x);
          acc.y = fmaf(x.y, qr, acc.y);
          acc.z = fmaf(x.z, qr, acc.z);
          acc.w = fmaf(x.w, qr, acc.w);
        }
      }
    }
  }
  static_assert(RG >= 2 && RG * TPR == 256, "V must be a power of two in [32, 512]");
  *reinterpret_cast<f32x4*>(&part[rg][4 * cq]) = acc;
  __syncthreads();
  for (int c = tid; c < V; c += 256) {
    float sum = 0.f;
#pragma unroll
    for (int i = 0; i < RG; ++i) sum += part[i][c];
    o[unit * V + c] = (TOut)(sum * scale);
  }
}

// The same step on the [V, K] state layout ([SG] 二, state_v_first): row v
// of a unit's state is S[.][v], K contiguous floats.  Each thread owns four
// adjacent keys (16-byte accesses) of every RG-th row, so each load of a wave
// covers whole contiguous rows; o[v] = scale * sum_k S[k][v] q[k] becomes a
// reduction along the row: over the row's lanes by a halving butterfly that
// reduces a thread's 16 rows together, and through LDS when a row spans two
// waves (K = 512).
template <int K, typename TIn, typename TOut>
__global__ void __launch_bounds__(256)
recurrent_step_vk_kernel(const TIn* __restrict__ q, const TIn* __restrict__ k,
                         const TIn* __restrict__ v, const float* __restrict__ g,
                         const float* __restrict__ g_gamma, float* __restrict__ state,
                         TOut* __restrict__ o, float scale, int32_t H, int32_t Hkv, int32_t V) {
  constexpr int TPR = K / 4;                  // threads per state row
  constexpr int RG = 256 / TPR;               // row groups
  constexpr int LW = TPR < 64 ? TPR : 64;     // lanes of a row within one wave
  constexpr int NSUB = TPR / LW;              // waves a row spans
  constexpr int BATCH = 16;                   // rows in flight per thread
  static_assert(RG >= 2 && RG * TPR == 256, "K must be a power of two in [32, 512]");
  __shared__ float part[1024 * NSUB];
  __shared__ float vsh[1024];         // the unit's v row (V <= 1024)

  const int64_t unit = blockIdx.x;    // n * H + h
  const uint32_t n = blockIdx.x / (uint32_t)H;
  const int h = (int)(blockIdx.x - n * (uint32_t)H);
  const int64_t ukv = (int64_t)n * Hkv + h / (H / Hkv);   // (sequence, kv head) row of k and v
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int cq = tid % TPR;
  const int rg = tid / TPR;
  const float gamma = expf(g != nullptr ? g[unit] : (g_gamma != nullptr ? g_gamma[h] : 0.f));
  f32x4 kk, qq;
  {
    const TIn* ku = k + ukv * K + 4 * cq;
    const TIn* qu = q + unit * K + 4 * cq;
    kk = f32x4{to_f32(ku[0]), to_f32(ku[1]), to_f32(ku[2]), to_f32(ku[3])};
    qq = f32x4{to_f32(qu[0]), to_f32(qu[1]), to_f32(qu[2]), to_f32(qu[3])};
  }
  const TIn* vu = v + ukv * V;
  f32x4* S = reinterpret_cast<f32x4*>(state + unit * (int64_t)K * V);
  const int rpt = V / RG;             // rows per row group (V % 32 == 0)
  auto load_batch = [&](int b0, f32x4 (&sv)[BATCH]) {
#pragma unroll
    for (int b = 0; b < BATCH; ++b)
      if (b0 + b < rpt) sv[b] = __builtin_nontemporal_load(&S[(int64_t)(rg + RG * (b0 + b)) * TPR + cq]);
  };
  // v goes through LDS once per workgroup (one load per element instead of
  // one per element and row group), staged while the first batch of state
  // rows is in flight
  f32x4 sv[BATCH];
  load_batch(0, sv);
  for (int c = tid; c < V; c += 256) vsh[c] = to_f32(vu[c]);
  __syncthreads();
  for (int b0 = 0; b0 < rpt; b0 += BATCH) {
    if (b0 > 0) load_batch(b0, sv);
    float vr[BATCH];
#pragma unroll
    for (int b = 0; b < BATCH; ++b)
      if (b0 + b < rpt) vr[b] = vsh[rg + RG * (b0 + b)];
    float pq[BATCH];
#pragma unroll
    for (int b = 0; b < BATCH; ++b) {
      pq[b] = 0.f;
      if (b0 + b < rpt) {                  // uniform over the workgroup
        const int row = rg + RG * (b0 + b);
        f32x4 x = sv[b];
        x.x = fmaf(gamma, x.x, vr[b] * kk.x);
        x.y = fmaf(gamma, x.y, vr[b] * kk.y);
        x.z = fmaf(gamma, x.z, vr[b] * kk.z);
        x.w = fmaf(gamma, x.w, vr[b] * kk.w);
        __builtin_nontemporal_store(x, &S[(int64_t)row * TPR + cq]);
        pq[b] = fmaf(x.x, qq.x, fmaf(x.y, qq.y, fmaf(x.z, qq.z, x.w * qq.w)));
      }
    }
    // sum each row's BATCH partials over the row's LW lanes: a butterfly that
    // halves the values a lane carries at every step (the lane keeps the upper
    // half when its mask bit is set), so a lane ends with the sums of `cnt`
    // consecutive rows starting at `bsel`; once one value is left the
    // remaining steps just add
    static_assert(BATCH == 16, "four halving stages");
    int bsel = 0;
    auto halve = [&](auto cnt_c, int m) {
      constexpr int HALF = decltype(cnt_c)::value / 2;
      const bool upper = (lane & m) != 0;
#pragma unroll
      for (int i = 0; i < HALF; ++i) {
        const float send = upper ? pq[i] : pq[i + HALF];
        const float keep = upper ? pq[i + HALF] : pq[i];
        pq[i] = keep + __shfl_xor(send, m, 64);
      }
      if (upper) bsel += HALF;
    };
    constexpr int M0 = LW / 2;
    if constexpr (M0 >= 1) halve(std::integral_constant<int, 16>{}, M0);
    if constexpr (M0 / 2 >= 1) halve(std::integral_constant<int, 8>{}, M0 / 2);
    if constexpr (M0 / 4 >= 1) halve(std::integral_constant<int, 4>{}, M0 / 4);
    if constexpr (M0 / 8 >= 1) halve(std::integral_constant<int, 2>{}, M0 / 8);
    constexpr int cnt = M0 >= 8 ? 1 : (M0 >= 4 ? 2 : (M0 >= 2 ? 4 : 8));   // values left per lane
    int addmask = 0;
#pragma unroll
    for (int m = M0 / 16; m >= 1; m >>= 1) {
      pq[0] += __shfl_xor(pq[0], m, 64);
      addmask |= m;
    }
    if ((lane & addmask) == 0) {
#pragma unroll
      for (int i = 0; i < BATCH; ++i) {
        if (i < cnt && b0 + bsel + i < rpt) {
          const int row = rg + RG * (b0 + bsel + i);
          part[row * NSUB + cq / LW] = pq[i];
        }
      }
    }
  }
  __syncthreads();
  for (int c = tid; c < V; c += 256) {
    float sum = 0.f;
#pragma unroll
    for (int i = 0; i < NSUB; ++i) sum += part[c * NSUB + i];
    o[unit * V + c] = (TOut)(sum * scale);
  }
}

template <int K, typename TIn, typename TOut>
hipError_t launch_vk(const StepParams& p, hipStream_t stream) {
  const int64_t units = (int64_t)p.N * p.H;
  if (units == 0) return hipSuccess;
  hipLaunchKernelGGL((recurrent_step_vk_kernel<K, TIn, TOut>), dim3((unsigned)units), dim3(256), 0,
                     stream, static_cast<const TIn*>(p.q), static_cast<const TIn*>(p.k),
                     static_cast<const TIn*>(p.v), p.g, p.g_gamma, p.state, static_cast<TOut*>(p.o),
                     p.scale, p.H, p.Hkv, p.V);
  return hipGetLastError();
}

template <int V, typename TIn, typename TOut>
hipError_t launch_v(const StepParams& p, hipStream_t stream) {
  const int64_t units = (int64_t)p.N * p.H;
  if (units == 0) return hipSuccess;
  hipLaunchKernelGGL((recurrent_step_kernel<V, TIn, TOut>), dim3((unsigned)units), dim3(256), 0,
                     stream, static_cast<const TIn*>(p.q), static_cast<const TIn*>(p.k),
                     static_cast<const TIn*>(p.v), p.g, p.g_gamma, p.state, static_cast<TOut*>(p.o),
                     p.scale, p.H, p.Hkv, p.K);
  return hipGetLastError();
}

template <typename TIn, typename TOut>
hipError_t launch_dtypes(const StepParams& p, hipStream_t stream) {
  if (p.state_v_first) {
    switch (p.K) {
      case 32: return launch_vk<32, TIn, TOut>(p, stream);
      case 64: return launch_vk<64, TIn, TOut>(p, stream);
      case 128: return launch_vk<128, TIn, TOut>(p, stream);
      case 256: return launch_vk<256, TIn, TOut>(p, stream);
      case 512: return launch_vk<512, TIn, TOut>(p, stream);
      default: return hipErrorInvalidValue;
    }
  }
  switch (p.V) {
    case 32: return launch_v<32, TIn, TOut>(p, stream);
    case 64: return launch_v<64, TIn, TOut>(p, stream);
    case 128: return launch_v<128, TIn, TOut>(p, stream);
    case 256: return launch_v<256, TIn, TOut>(p, stream);
    case 512: return launch_v<512, TIn, TOut>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_recurrent_step(const StepParams& p, hipStream_t stream) {
  if (p.qkv_bf16) {
    return p.o_bf16 ? launch_dtypes<__bf16, __bf16>(p, stream)
                    : launch_dtypes<__bf16, float>(p, stream);
  }
  return p.o_bf16 ? launch_dtypes<float, __bf16>(p, stream)
                  : launch_dtypes<float, float>(p, stream);
}

}  // namespace sgla
