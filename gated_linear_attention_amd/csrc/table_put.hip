// Tables written into the workspace by kernels whose payload travels in the
// kernel arguments (the packed-sequence tables; the segment, block and scan
// tables of segmented chains).  The host builds the sequence table
// (longest sequence first); each launch carries up to kTablePut entries by
// value, so no host buffer has to outlive the call and nothing is copied
// from pageable memory.  The same launch expands every entry it carries into
// that sequence's rows of the chunk table (FlashAttention-style packing, page
// "flash-linear-attention 中的 Simple GLA", section 二: a sequence's chunks
// start at its first packed token, the last one may be partial).
#include <hip/hip_runtime.h>

#include "sgla_internal.h"

namespace sgla {
namespace {

// One workgroup per carried sequence: thread 0 stores the sequence entry,
// all threads stride over the sequence's chunk rows.
__global__ void __launch_bounds__(64)
table_put_kernel(TablePut put, SeqEntry* __restrict__ seq_table, ChunkEntry* __restrict__ chunk_table) {
  const int i = blockIdx.x;
  if (i >= put.count) return;
  const SeqEntry e = put.e[i];
  if (threadIdx.x == 0) seq_table[put.first + i] = e;
  if (chunk_table == nullptr) return;
  const int32_t cs = put.chunk;
  const int32_t nch = (e.len + cs - 1) / cs;
  for (int32_t c = threadIdx.x; c < nch; c += 64) {
    ChunkEntry ce;
    ce.t0 = e.bos + c * cs;
    ce.len = min(cs, e.len - c * cs);
    chunk_table[e.chunk0 + c] = ce;
  }
}

// Raw words: thread i of the launch writes word i of the payload.
__global__ void __launch_bounds__(256) table_words_kernel(TableWords put, uint32_t* __restrict__ dst) {
  for (int i = threadIdx.x; i < put.count; i += 256) dst[put.first + i] = put.w[i];
}

}  // namespace

hipError_t launch_table_words(const TableWords& put, uint32_t* dst, hipStream_t stream) {
  if (put.count <= 0) return hipSuccess;
  hipLaunchKernelGGL(table_words_kernel, dim3(1), dim3(256), 0, stream, put, dst);
  return hipGetLastError();
}

hipError_t launch_table_put(const TablePut& put, SeqEntry* seq_table, ChunkEntry* chunk_table,
                            hipStream_t stream) {
  if (put.count <= 0) return hipSuccess;
  hipLaunchKernelGGL(table_put_kernel, dim3((unsigned)put.count), dim3(64), 0, stream, put, seq_table,
                     chunk_table);
  return hipGetLastError();
}

}  // namespace sgla
