// Step (1) of the chunked forward: chunk-local cumulative sum of the scalar
// log gates, pre-multiplied by 1/ln 2 so that every decay downstream is a
// hardware exp2 (page "flash-linear-attention 中的 Simple GLA", section 三:
// chunk_local_cumsum with the RCP_LN2 scale; the sum is per head and per chunk
// because the gate is one scalar per head).
//
// One 64-lane wavefront per (64-token block, head): lane c holds token c of
// the block, and a wave-level inclusive scan (log2(64) = 6 shuffle rounds)
// forms the prefix sums, restarting every chunk_size lanes (chunk_size a power
// of two <= 64; blocks start at sequence starts, so chunks do too).  The scan
// accumulates in float64 and rounds once to float32.
// The chunk kernels run the same scan in their chunk prologue; this kernel
// serves the standalone sgla_chunk_local_cumsum entry point.
#include <hip/hip_runtime.h>

#include "gate_scan.h"
#include "sgla_internal.h"

namespace sgla {
namespace {

__global__ void __launch_bounds__(256)
gate_cumsum_kernel(const float* __restrict__ g, float* __restrict__ gc, int32_t H,
                   SeqLayout seqs, int32_t chunk_size) {
  const int lane = threadIdx.x & 63;
  const int head = blockIdx.y * 4 + (threadIdx.x >> 6);
  if (head >= H) return;
  int64_t t0;
  int32_t len;
  if (seqs.chunk_table != nullptr) {
    const ChunkEntry ce = seqs.chunk_table[blockIdx.x];
    t0 = ce.t0;
    len = ce.len;
  } else {
    const int32_t per_row = (seqs.T + kChunk - 1) / kChunk;
    const int32_t b = blockIdx.x / per_row;
    const int32_t m = blockIdx.x - b * per_row;
    t0 = (int64_t)b * seqs.T + (int64_t)m * kChunk;
    len = min(kChunk, seqs.T - m * kChunk);
  }
  const bool active = lane < len;
  const float b = wave_segmented_cumsum_log2(active ? g[(t0 + lane) * H + head] : 0.f, chunk_size);
  if (active) gc[(t0 + lane) * H + head] = b;
}

}  // namespace

hipError_t launch_gate_cumsum(const float* g, float* gc, int32_t H, const SeqLayout& seqs,
                              int32_t chunk_size, hipStream_t stream) {
  if (seqs.num_chunks <= 0) return hipSuccess;
  if (chunk_size < 1 || chunk_size > kChunk || (chunk_size & (chunk_size - 1)) != 0) return hipErrorInvalidValue;
  dim3 grid(seqs.num_chunks, (H + 3) / 4);
  hipLaunchKernelGGL(gate_cumsum_kernel, grid, dim3(256), 0, stream, g, gc, H, seqs, chunk_size);
  return hipGetLastError();
}

}  // namespace sgla
