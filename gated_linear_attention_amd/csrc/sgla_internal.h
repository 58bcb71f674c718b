// Internal launch interface between the C-ABI layer (sgla_api.cpp) and the
// HIP kernels.  Not part of the public ABI.
#pragma once

#include <cstddef>
#include <cstdint>
#include <hip/hip_runtime_api.h>

#include "sgla.h"

namespace sgla {

// sgla_chunk_fwd with the validation, table upload and launches it performs
// (the C entry points call it with their own workspace).  With `acquire`
// given, the workspace pointer is obtained from it once every argument has
// passed validation (and only if the call needs workspace at all).
// chunk_fwd_workspace validates the arguments and returns the workspace
// bytes such a call needs (0 with *status != SGLA_OK on invalid arguments);
// report() records a message for sgla_last_error().
typedef sgla_status (*WorkspaceAcquire)(void** workspace);
sgla_status chunk_fwd_enqueue(const sgla_chunk_args* args, const void* q, const void* k, const void* v,
                              const float* g, const float* g_gamma, const float* initial_state,
                              const int64_t* cu_seqlens_host, void* o, float* final_state, void* workspace,
                              size_t workspace_bytes, hipStream_t stream, WorkspaceAcquire acquire);
size_t chunk_fwd_workspace(const sgla_chunk_args* args, const int64_t* cu_seqlens_host, sgla_status* status);
sgla_status report(sgla_status st, const char* msg);

constexpr int kChunk = 64;        // tokens per chunk
constexpr int kXcds = 8;          // MI355X: 8 XCDs, workgroups dealt round-robin

// Workgroups of the chunk kernels per (sequence, kv head) group and V tile
// count: kv groups are dealt to the XCDs round-robin, each group's n_rep
// query heads and nvt V tiles adjacent in dispatch order on its XCD.
inline int64_t unit_grid(int32_t num_seqs, int32_t Hkv, int32_t n_rep, int32_t nvt) {
  const int64_t groups = (int64_t)num_seqs * Hkv;
  return (groups + kXcds - 1) / kXcds * kXcds * n_rep * nvt;
}

// Per-sequence entry of the packed-input table, sorted longest first.
struct SeqEntry {
  int32_t bos;     // first packed token of the sequence
  int32_t len;     // tokens
  int32_t seq;     // index into initial_state / final_state
  int32_t chunk0;  // index of the sequence's first chunk in the chunk table
};

// Per-chunk entry used by the gate kernel for packed input.
struct ChunkEntry {
  int32_t t0;    // first packed token of the chunk
  int32_t len;   // tokens in the chunk (1..chunk of the grid, at most kChunk)
};

// Up to kTablePut sequence-table entries carried by value in the arguments
// of one table_put launch (2 KiB of payload); the launch writes them at rows
// [first, first + count) of the sequence table and expands each into its
// rows of the chunk table.
constexpr int kTablePut = 126;
struct TablePut {
  int32_t first;
  int32_t count;
  int32_t chunk;   // tokens per chunk row (kChunk, or the backward's chunk_size)
  int32_t pad;
  SeqEntry e[kTablePut];
};
hipError_t launch_table_put(const TablePut& put, SeqEntry* seq_table, ChunkEntry* chunk_table,
                            hipStream_t stream);

// Layout of a caller's [N, H, K, V] or [N, H, V, K] state ([SG] 二,
// state_v_first): element (k, v) of one (sequence, head) state sits at
// k * rs + v * cs.
struct StateLayout {
  int32_t rs;   // stride between key rows: V, or 1 for the [V, K] layout
  int32_t cs;   // stride between value columns: 1, or K for the [V, K] layout
};

// Description of the token ranges a launch covers.  Dense input: seq_table ==
// nullptr and every sequence b has bos = b * T, len = T.  Packed input: the
// table lives in device memory (workspace).
struct SeqLayout {
  int32_t num_seqs;          // N
  int32_t T;                 // dense: tokens per row
  const SeqEntry* seq_table; // packed only (device)
  const ChunkEntry* chunk_table; // packed only (device)
  int32_t num_chunks;        // total chunks over all sequences
  int32_t chunk;             // tokens per chunk of this grid: kChunk, or for the backward the
                             // requested chunk_size (16 or 32; such chunks run in 64-row tiles)
};

// Segments of long sequences (bf16 K <= 128 forward).  A sequence whose
// chain of 64-token chunks is long compared with the work the launch has for
// the rest of the GPU is cut at chunk boundaries into segments processed in
// parallel, each from its own initial state: segment 0 from the sequence's
// initial state, segment s > 0 from the state after segment s - 1.  Those
// entering states come from a state-only pass over the earlier segments
// (per block of chunks: the state each block adds from a zero start, and the
// block's total log2 decay) followed by a scan over the blocks.
struct SegEntry {
  int32_t bos;     // first packed token of the segment
  int32_t len;     // tokens
  int32_t seq;     // sequence index (initial_state / final_state row)
  int32_t init;    // -1: start from the sequence's initial state; else entering-state record
  int32_t last;    // 1: the sequence's last segment (writes final_state)
  int32_t pad[3];
};
// The segments one chunk workgroup processes in turn: rows [first, first +
// count) of the segment table.
struct BinEntry {
  int32_t first;
  int32_t count;
};
struct BlockEntry {
  int32_t t0;       // first packed token of the block
  int32_t len;      // tokens (a whole number of chunks, except a sequence's last)
  int32_t out_rec;  // after this block the scan writes entering-state record out_rec (-1: none)
  int32_t pad;
};
struct ScanEntry {
  int32_t seq;          // sequence index
  int32_t first_block;  // its blocks are [first_block, first_block + num_blocks)
  int32_t num_blocks;
  int32_t pad;
};

// Raw words carried by value in one table_words launch and written at
// dst[first, first + count).
constexpr int kTableWords = 500;
struct TableWords {
  int32_t first;
  int32_t count;
  uint32_t w[kTableWords];
};
hipError_t launch_table_words(const TableWords& put, uint32_t* dst, hipStream_t stream);

struct SegmentParams {
  const void* k;
  const void* v;
  const float* g;
  const float* g_gamma;
  const float* h0;            // [N, H, K, V] (layout sl) or nullptr
  int32_t H, Hkv, K, V;
  StateLayout sl;
  const BlockEntry* blocks;
  int32_t num_blocks;
  const ScanEntry* scans;
  int32_t num_scans;
  float* urec;                // [num_blocks, H, K, V]: state added by each block from a zero start
  float* ulog;                // [num_blocks, H]: each block's total log2 decay
  float* sin;                 // [records, H, K, V]: entering state of each later segment
  // the table region carried in the pre-pass arguments (written to table_dst
  // by its workgroup 0; blocks then read from word blk_word of the payload),
  // or nullptr when the tables are already in the workspace
  const TableWords* inline_tables = nullptr;
  uint32_t* table_dst = nullptr;
  int32_t blk_word = 0;
};
// state-only pass over the blocks, then the scan writing the entering states
hipError_t launch_segment_states(const SegmentParams& p, hipStream_t stream);

// Per-(chunk, head) outputs of the preparation kernel (wide-key bf16 path):
// kGateStride floats of gates [sc[64], dv[64], dall, pad] and a [2][64][64]
// bf16 hi/lo pair of the decay-masked, scaled q k^T, plus the chunk's Q and
// K^T, all in the MFMA operand order of the state/output kernel.
constexpr int kGateStride = 3 * kChunk;

struct ChunkPrepParams {
  const void* q;
  const void* k;
  const float* g;
  const float* g_gamma;
  float scale;
  int32_t H, Hkv, K;
  SeqLayout seqs;
  float* gates;              // [num_chunks, H, kGateStride]
  void* amat;                // [num_chunks, H, 2, 64, 64] bf16
  void* ktf;                 // [num_chunks, Hkv, K * 64] bf16, state-update operand order
  void* qfr;                 // [num_chunks, H, K * 64] bf16, q.h operand order
};

struct ChunkFwdParams {
  const void* q;
  const void* k;
  const void* v;
  const float* g;            // per-token natural-log gates [T_total, H], or nullptr
  const float* g_gamma;      // [H] natural-log decay, or nullptr
  const float* h0;           // [N, H, K, V] or nullptr
  void* o;
  float* ht;                 // [N, H, K, V] or nullptr
  float scale;
  int32_t H, Hkv, K, V;      // Hkv divides H: query head h reads kv head h / (H / Hkv)
  int32_t o_bf16;            // 1: o is bf16, 0: float32
  StateLayout sl;            // layout of h0 and ht
  SeqLayout seqs;
  const float* gates;        // wide-key path: preparation outputs (workspace)
  const void* amat;
  const void* ktf;
  const void* qfr;
  // segmented chains (bf16 K <= 128): one workgroup per bin of segments
  // instead of per sequence; nullptr = one workgroup per sequence
  const SegEntry* segs = nullptr;
  const BinEntry* bins = nullptr;
  int32_t num_bins = 0;
  const float* sin = nullptr;  // [records, H, K, V] entering states of later segments
};

// chunk_size: a power of two <= kChunk (the scan restarts inside each
// kChunk-token block of the layout)
hipError_t launch_gate_cumsum(const float* g, float* gc, int32_t H, const SeqLayout& seqs,
                              int32_t chunk_size, hipStream_t stream);

// bf16 q/k/v, MFMA path, whole key dimension per chunk step.  K in {64,128},
// V % 64 == 0; one workgroup per (sequence or segment, head, V tile of
// chunk_fwd_bf16_vtile(V) columns).
hipError_t launch_chunk_fwd_bf16(const ChunkFwdParams& p, hipStream_t stream);
int chunk_fwd_bf16_vtile(int32_t V);

// Wide-key bf16 path (K in {256,512}, V % 32 == 0): per-(chunk, head)
// preparation, then the state and output passes reading its results.
hipError_t launch_chunk_prep_bf16(const ChunkPrepParams& p, hipStream_t stream);
hipError_t launch_chunk_fwd_bf16_wide(const ChunkFwdParams& p, hipStream_t stream);

// Chunk sizes 16 and 32 (any supported dtype and K; V % 16 == 0): one
// generic kernel on the fp32 matrix cores.
hipError_t launch_chunk_fwd_small(const ChunkFwdParams& p, int chunk, bool qkv_bf16, hipStream_t stream);

// float32 q/k/v, VALU path.  K in {16,32,64,128}, V % 32 == 0.
hipError_t launch_chunk_fwd_f32(const ChunkFwdParams& p, hipStream_t stream);

// Backward: q, k, v, dout all bf16 or all float32; every gradient float32.
// K in {16, 32, 64, 128} (float32 or bf16) or {256, 512} (bf16, V % 64 ==
// 0), V % 32 == 0, any Hkv dividing H (k and v read by kv head, dk and dv
// written per query head for the group sum).
struct ChunkBwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* dout;
  const float* g;            // [T_total, H] or nullptr
  const float* g_gamma;      // [H] or nullptr
  const float* h0;           // [N, H, K, V] or nullptr
  const float* dht;          // [N, H, K, V] or nullptr
  float* dq;                 // [T_total, H, K]
  float* dk;                 // [T_total, H, K]: per query head (summed over kv groups afterwards)
  float* dv;                 // [T_total, H, V]: per query head
  float* dg;                 // [T_total, H] or nullptr
  float* dg_gamma;           // [H] or nullptr
  float* dh0;                // [N, H, K, V] or nullptr
  float scale;
  int32_t H, K, V;
  int32_t Hkv;               // kv heads of k and v (divides H); query head h reads kv head h / (H / Hkv)
  int32_t qkv_bf16;
  StateLayout sl;            // layout of h0, dht and dh0
  SeqLayout seqs;
  float* hbuf;               // workspace [num_chunks, H, K, V]: state entering each chunk
  float* dhbuf;              // workspace [num_chunks, H, K, V]: gradient of the state leaving it
  float* gpart;              // workspace [num_chunks, H]: per-chunk sums of dg (g_gamma)
  float* wpart;              // workspace [num_chunks, H, K / 128, kWidePart] for K > 128: per
                             // key tile gate terms (r_c, dv_c k_c . (V dH^T)_c, <dH, h>)
};

// Floats per key-tile gate record of the wide-key backward (64 + 64 + 1,
// padded), and the V columns per workgroup of its dV kernel.
constexpr int kWidePart = 132;
constexpr int kWideDvCols = 64;

hipError_t launch_chunk_bwd(const ChunkBwdParams& p, hipStream_t stream);
// dk [T_total, Hkv, K] (and dv likewise) = the sum of the n_rep = H / Hkv
// query-head gradients of each kv head, in query-head order
hipError_t launch_kv_group_sum(const float* src, float* dst, int64_t tokens, int32_t H, int32_t Hkv,
                               int32_t D, hipStream_t stream);

// The backward (state pass and per-chunk gradients) runs on the bf16 matrix
// cores (hi/lo splits of the fp32 operands) for bf16 inputs with K in {64,
// 128, 256, 512}; otherwise on the fp32 matrix cores.
inline bool bwd_bf16_grad(bool qkv_bf16, int32_t K) {
  return qkv_bf16 && (K == 64 || K == 128 || K == 256 || K == 512);
}
hipError_t launch_chunk_bwd_state_bf16(const ChunkBwdParams& p, int32_t chunks_per_row, hipStream_t stream);
hipError_t launch_chunk_bwd_grad_bf16(const ChunkBwdParams& p, int32_t chunks_per_row, hipStream_t stream);
// K > 128: dV over all keys, and the gate gradient from the key-tile records
hipError_t launch_chunk_bwd_dv_wide(const ChunkBwdParams& p, int32_t chunks_per_row, hipStream_t stream);
hipError_t launch_chunk_bwd_gate_wide(const ChunkBwdParams& p, int32_t chunks_per_row, hipStream_t stream);

// Elementwise-gate GLA forward: gk [T_total, H, K] float32 natural-log gates,
// one per key.  K in {16, 32, 64, 128}, V % 32 == 0.
struct GlaFwdParams {
  const void* q;
  const void* k;
  const void* v;
  const float* gk;
  const float* h0;
  void* o;
  float* ht;
  float scale;
  int32_t H, Hkv, K, V;
  int32_t qkv_bf16;
  int32_t o_bf16;
  StateLayout sl;
  SeqLayout seqs;
  float* amat;               // fp32 chain: workspace [num_chunks, H, 64, 64] decay-masked, scaled A
  // bf16 chain (gla_bf16_chain): per (chunk, query head) records written by
  // the preparation kernel, each a bf16 hi plane followed by its lo plane
  void* qk_hl;               // [num_chunks, H, 2 (q~, k~), 2, 64, K]
  void* a_hl;                // [num_chunks, H, 2, 64, 64]
  float* dl;                 // [num_chunks, H, K]: 2^(chunk's total log2 decay) per key
};

// The bf16 chain (bf16 matrix cores, hi/lo operands) serves bf16 inputs with
// K in {64, 128} and V a multiple of 64; everything else takes the fp32 chain.
inline bool gla_bf16_chain(bool qkv_bf16, int32_t K, int32_t V) {
  return qkv_bf16 && (K == 64 || K == 128) && V % 64 == 0;
}

hipError_t launch_gla_chunk_fwd(const GlaFwdParams& p, hipStream_t stream);
hipError_t launch_gla_chain_bf16(const GlaFwdParams& p, hipStream_t stream);

// Running normalizer (the ones column of the augmented value): den [T_total,
// H] = scale q . z, z [N, H, K] carried from z0 to zt.
struct NormalizerParams {
  const void* q;
  const void* k;
  const float* g;
  const float* g_gamma;
  const float* z0;           // [N, H, K] or nullptr
  float* den;                // [T_total, H]
  float* zt;                 // [N, H, K] or nullptr
  float scale;
  int32_t H, Hkv, K;
  int32_t qkv_bf16;
  SeqLayout seqs;
  float* zrec;               // workspace [num_chunks, H, K]: chunk sums, then z entering each chunk
  float* dlog;               // workspace [num_chunks, H]: each chunk's total log2 decay
};

struct StepNormalizerParams {
  const void* q;             // [N, H, K]
  const void* k;             // [N, Hkv, K]
  const float* g;            // [N, H] or nullptr
  const float* g_gamma;      // [H] or nullptr
  float* z;                  // [N, H, K], in place
  float* den;                // [N, H]
  float scale;
  int32_t N, H, Hkv, K;
  int32_t qkv_bf16;
};

hipError_t launch_chunk_normalizer(const NormalizerParams& p, hipStream_t stream);
hipError_t launch_step_normalizer(const StepNormalizerParams& p, hipStream_t stream);

// Parallel form: the decayed attention matrix of dense input written out,
// and o = A v.
struct ParallelParams {
  const void* q;             // [B, T, H, K] bf16 (launch_parallel_fwd) or float32 (launch_parallel_fwd_f32)
  const void* k;             // [B, T, Hkv, K], same dtype
  const void* v;             // [B, T, Hkv, V], same dtype
  const float* g;            // [B, T, H] or nullptr
  const float* g_gamma;      // [H] or nullptr
  void* o;                   // [B, T, H, V], float32 when o_f32 else bf16
  float* attn;               // [B, H, T, T] or nullptr
  float scale;
  int32_t B, T, H, Hkv, K, V;
  int32_t o_f32;
};

inline bool parallel_supported(int32_t K, int32_t V) {
  return (K == 64 || K == 128 || K == 256) && V >= 16 && V <= 256 && V % 16 == 0;
}

hipError_t launch_parallel_fwd(const ParallelParams& p, hipStream_t stream);

// float32 q, k, v: K and V multiples of 16 in [16, 256].
inline bool parallel_f32_supported(int32_t K, int32_t V) {
  return K >= 16 && K <= 256 && K % 16 == 0 && V >= 16 && V <= 256 && V % 16 == 0;
}

hipError_t launch_parallel_fwd_f32(const ParallelParams& p, hipStream_t stream);

struct StepParams {
  const void* q;
  const void* k;
  const void* v;
  const float* g;            // [N, H] or nullptr
  const float* g_gamma;      // [H] or nullptr
  float* state;              // [N, H, K, V], or [N, H, V, K] when state_v_first
  void* o;
  float scale;
  int32_t N, H, Hkv, K, V;
  int32_t state_v_first;
  int32_t qkv_bf16;
  int32_t o_bf16;
};

// V in {32,64,128,256,512}, 1 <= K <= 1024.
hipError_t launch_recurrent_step(const StepParams& p, hipStream_t stream);

}  // namespace sgla
