/*
 * sgla.h -- C ABI of libsgla, the gfx950 (MI355X) implementation of Simple GLA
 * (head-wise gated linear attention).
 *
 * Operator (page "flash-linear-attention 中的 Simple GLA", section 一): per
 * sequence and head, with a K x V state S,
 *
 *     S_t = exp(g_t) * S_{t-1} + k_t v_t^T,        o_t = scale * S_t^T q_t,
 *
 * where g_t is a scalar log gate per (token, head), or a per-head constant
 * log decay g_gamma[h] (section 二).  The output uses the state after token t.
 *
 * Conventions shared by every entry point:
 *   - All tensor arguments are DEVICE pointers to contiguous row-major memory
 *     allocated and owned by the caller.  The library never allocates, frees,
 *     retains a pointer past the call, or synchronizes the stream; all work
 *     is enqueued on the caller's `stream`.
 *   - Layouts follow section 二: q [B, T, H, K]; k [B, T, Hkv, K];
 *     v [B, T, Hkv, V]; o [B, T, H, V]; g [B, T, H]; g_gamma [H]; states
 *     [N, H, K, V] with S[k][v] (key index major), or [N, H, V, K] (value
 *     index major) when state_v_first is set (section 二: the [V, K] layout
 *     some backends keep; it applies to initial_state, final_state, dht, dh0
 *     and the decode state alike).  Hkv, the number of kv
 *     heads, divides H; query head h reads kv head h / (H / Hkv), the
 *     contiguous grouping of grouped-query attention (page "relinear", its
 *     GQA target, and the Simple GLA layer's num_kv_heads, section 四).  Every
 *     query head keeps its own gate and state.  Hkv == H is plain multi-head.  Packed (varlen) input has B == 1 and N sequences given by
 *     cu_seqlens[N + 1] (FlashAttention convention, section 二); dense input
 *     has N == B.
 *   - Gates, states and the state accumulation are float32.  q, k, v are all
 *     bf16 or all float32 (SGLA_BF16 / SGLA_F32); o is float32 or bf16.
 *   - Every argument check runs on the host before anything is enqueued.  On
 *     a non-OK status nothing has been written to any output, to the state or
 *     to the workspace, and sgla_last_error() describes the problem.  There is
 *     no fallback: an unsupported shape or dtype is an error, never a slower
 *     path.
 *   - A kernel launch failure reported by the runtime is returned as
 *     SGLA_ERR_HIP; asynchronous faults surface at the caller's next
 *     synchronization, as for any HIP work.
 */
#ifndef SGLA_H
#define SGLA_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SGLA_ABI_VERSION 5

typedef enum {
  SGLA_OK = 0,
  SGLA_ERR_INVALID_ARG = 1, /* NULL required pointer, both gates, bad scale, ... */
  SGLA_ERR_SHAPE = 2,       /* inconsistent sizes, malformed cu_seqlens, B != 1 with cu_seqlens */
  SGLA_ERR_DTYPE = 3,       /* dtype code not supported for this argument */
  SGLA_ERR_UNSUPPORTED = 4, /* valid request outside what the kernels implement */
  SGLA_ERR_WORKSPACE = 5,   /* workspace NULL or smaller than sgla_chunk_fwd_workspace_size */
  SGLA_ERR_HIP = 6          /* the HIP runtime rejected a launch or copy */
} sgla_status;

typedef enum { SGLA_BF16 = 1, SGLA_F32 = 2 } sgla_dtype;

typedef struct {
  int32_t B, T, H, K, V;      /* packed input: B == 1 and T = total tokens */
  int32_t num_seqs;           /* packed: number of sequences N; dense: ignored (N = B) */
  int32_t chunk_size;         /* tokens per chunk; 0 selects 64.  sgla_chunk_fwd,
                                 sgla_chunk_bwd, sgla_gla_chunk_fwd, sgla_chunk_normalizer:
                                 16, 32 or 64; sgla_chunk_local_cumsum: any power of two up to
                                 64 */
  int32_t qkv_dtype;          /* sgla_dtype of q, k and v */
  int32_t o_dtype;            /* sgla_dtype of o */
  float scale;                /* finite; callers wanting the default pass 1/sqrt(K) */
  int32_t output_final_state; /* nonzero: write final_state */
  int32_t num_kv_heads;       /* Hkv: heads of k and v; 0 means H.  Must divide H */
  int32_t state_v_first;      /* nonzero: every state argument is [N, H, V, K] */
} sgla_chunk_args;

/* ABI revision of the loaded library (SGLA_ABI_VERSION it was built with). */
int sgla_abi_version(void);

/* Message for the last non-OK status returned on the calling thread
 * (thread-local; empty string if none).  Valid until the next call on the
 * same thread. */
const char *sgla_last_error(void);

/*
 * Bytes of device workspace sgla_chunk_fwd needs for these arguments: for
 * packed input the sequence and chunk tables; for bf16 inputs with K = 256 or
 * 512 at chunk_size 64 also the per-(chunk, head) preparation records (gates, the masked
 * intra-chunk q k^T as bf16 hi/lo, and the chunk's q and k^T rearranged for
 * the state kernel: 128 K + 16 KiB + 768 bytes per 64-token chunk and query
 * head, plus 128 K bytes per 64-token chunk and kv head).
 * `cu_seqlens_host` is the same host array later passed to sgla_chunk_fwd, or
 * NULL for dense input.  Returns 0 if the arguments are invalid (the reason is
 * in sgla_last_error()); a valid call may also legitimately need 0 bytes only
 * when there is no token to process.
 */
size_t sgla_chunk_fwd_workspace_size(const sgla_chunk_args *args, const int64_t *cu_seqlens_host);

/*
 * Chunked Simple GLA forward (prefill), section 三's three steps on gfx950:
 *   (1) chunk-local cumulative sum of the log gates, pre-multiplied by 1/ln 2
 *       so decays are evaluated with exp2;
 *   (2) the inter-chunk state pass, h_{n+1} = 2^{b_last} h_n +
 *       (K_n * 2^{b_last - b})^T V_n, kept in an fp32 K x V state on chip;
 *   (3) the output pass, O_n = scale * [ (Q_n K_n^T (.) M_n) V_n +
 *       diag(2^b) Q_n h_n ], M_ij = 2^{b_i - b_j} for j <= i, else 0.
 * Steps (2) and (3) run fused in one kernel per (sequence, head, V tile).
 * For bf16 inputs with K = 256 or 512 a preparation kernel first computes,
 * once per (chunk, head), step (1), the masked scale * Q K^T of step (3) and
 * the operand rearrangements the fused kernel reads; the workspace carries
 * them between the two launches, so a call enqueues two kernels.
 *
 * Arguments (device pointers unless stated):
 *   q               [B, T, H, K] in qkv_dtype
 *   k               [B, T, Hkv, K] in qkv_dtype
 *   v               [B, T, Hkv, V] in qkv_dtype
 *   g               [B, T, H] float32 log gates, or NULL
 *   g_gamma         [H] float32 per-head log decay, or NULL.  At most one of
 *                   g / g_gamma may be given (section 二); neither means no
 *                   decay (plain causal linear attention).
 *   initial_state   [N, H, K, V] float32, or NULL for zeros.
 *   cu_seqlens_host HOST array [N + 1] of int64 token offsets for packed
 *                   input (cu[0] == 0, non-decreasing, cu[N] == T), or NULL
 *                   for dense input.  Sequences may have any length >= 0; a
 *                   zero-length sequence passes its initial state through.
 *   o               [B, T, H, V] output in o_dtype.
 *   final_state     [N, H, K, V] float32, written when output_final_state is
 *                   nonzero (may be NULL otherwise).  May alias initial_state
 *                   exactly (in-place state update); no other aliasing.
 *   workspace       device buffer of at least workspace_bytes >=
 *                   sgla_chunk_fwd_workspace_size(args, cu_seqlens_host).
 * Supported (any Hkv dividing H): K in {64, 128} with V a multiple of 64, or K in {256, 512}
 * with V a multiple of 32 (bf16 inputs);
 * K in {16, 32, 64, 128} and V a multiple of 32 (float32 inputs);
 * chunk_size 16, 32 or 64 (section 二: a power of two; section 五 tests 16,
 * 32 and 64).  64 runs the tuned kernels described above; 16 and 32 run one
 * generic kernel per (sequence, head, 16-column V tile) on the fp32 matrix
 * cores (float32 accuracy for either input dtype, a single launch, no
 * preparation records).  Other powers of two, and values that are not a
 * power of two, return SGLA_ERR_UNSUPPORTED.
 *
 * Packed input: the sequence and chunk tables are written into the
 * workspace by small kernels enqueued on `stream` ahead of the chunk
 * kernels; their contents travel in the kernel arguments, so
 * cu_seqlens_host may be freed or reused as soon as the call returns.
 */
sgla_status sgla_chunk_fwd(const sgla_chunk_args *args,
                           const void *q, const void *k, const void *v,
                           const float *g, const float *g_gamma,
                           const float *initial_state,
                           const int64_t *cu_seqlens_host,
                           void *o, float *final_state,
                           void *workspace, size_t workspace_bytes,
                           hipStream_t stream);

/*
 * sgla_chunk_fwd without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation.  Same arguments, semantics,
 * kernels and results as sgla_chunk_fwd; the scratch memory (the packed
 * sequence tables, and for bf16 K = 256 / 512 at chunk_size 64 the
 * preparation records) comes from a fixed device array inside the library,
 * sgla_chunk_fwd_noalloc_max_bytes() bytes (16 MiB) per GPU, held until the
 * process ends.  The call allocates nothing, frees nothing and does not
 * synchronize.
 *   - A request whose sgla_chunk_fwd_workspace_size exceeds that size
 *     returns SGLA_ERR_WORKSPACE before anything is enqueued.
 *   - The array is found for the current device; `stream` must belong to
 *     the current device.
 *   - Every call on one GPU shares that GPU's array and it keeps the last
 *     call's contents: calls that overlap on one GPU (different streams, or
 *     threads without ordering) race and must be serialized by the caller.
 *     Calls enqueued on one stream are ordered and safe.
 */
size_t sgla_chunk_fwd_noalloc_max_bytes(void);
sgla_status sgla_chunk_fwd_noalloc(const sgla_chunk_args *args,
                                   const void *q, const void *k, const void *v,
                                   const float *g, const float *g_gamma,
                                   const float *initial_state,
                                   const int64_t *cu_seqlens_host,
                                   void *o, float *final_state,
                                   hipStream_t stream);

/*
 * Bytes of device workspace sgla_chunk_bwd needs: the packed-sequence tables,
 * the fp32 state entering every chunk (of chunk_size tokens) and the fp32
 * gradient of the state leaving it (2 * 4 K V bytes per chunk and head), 4 bytes per
 * chunk and head for the g_gamma reduction, and with grouped kv heads (Hkv <
 * H) the per-query-head k and v gradients (4 (K + V) bytes per token and
 * query head).  Returns 0 on invalid arguments (reason in sgla_last_error()).
 */
size_t sgla_chunk_bwd_workspace_size(const sgla_chunk_args *args, const int64_t *cu_seqlens_host);

/*
 * Backward of sgla_chunk_fwd (section 三: the backward passes over the chunk
 * states in fp32 and recovers the gate gradient by a reverse chunk-local
 * cumulative sum; section 五 tests dq, dk, dv, dg and dh0).  Computes the
 * gradients of
 *     L = sum_t <dout_t, o_t> + sum_n <dht_n, final_state_n>
 * with respect to q, k, v, the gates and initial_state, for the forward with
 * the same arguments.  Three launches: a state pass (forward states and
 * reverse state gradients, one workgroup per (sequence, head, 32-column V
 * tile) each), a per-(chunk, head) gradient kernel, and with g_gamma a
 * per-head reduction; with grouped kv heads one more launch per gradient
 * sums the query heads of each kv group.  bf16 inputs with K in {64, 128} run both passes on
 * the bf16 matrix cores (the fp32 states, state gradients and intra-chunk
 * matrices split into bf16 hi + lo); other inputs on the fp32 matrix cores.
 *
 * Arguments (device pointers unless stated):
 *   args            as for sgla_chunk_fwd; o_dtype and output_final_state
 *                   are not read.
 *   q, k, v, g, g_gamma, initial_state, cu_seqlens_host
 *                   the forward's inputs (same layouts and rules).
 *   dout            [B, T, H, V] in qkv_dtype: gradient of o.
 *   dht             [N, H, K, V] float32 gradient of final_state, or NULL
 *                   (no loss on the final state).
 *   dq              [B, T, H, K] float32.
 *   dk, dv          [B, T, Hkv, K] and [B, T, Hkv, V] float32: with grouped
 *                   kv heads the gradient of a kv head's row is the sum over
 *                   the H / Hkv query heads that read it.
 *   dg              [B, T, H] float32; required when g is given, else unused.
 *   dg_gamma        [H] float32; required when g_gamma is given, else unused.
 *   dh0             [N, H, K, V] float32 gradient of initial_state, or NULL.
 *   workspace       >= sgla_chunk_bwd_workspace_size(args, cu_seqlens_host).
 * Outputs must not overlap inputs or each other.
 * Supported: K in {16, 32, 64, 128}, V a multiple of 32, bf16 or float32
 * inputs; K in {256, 512} with bf16 inputs and V a multiple of 64;
 * chunk_size 16, 32 or 64 (section 二; section 五 runs the gradients at all
 * three): the state records, the gate restarts and the per-chunk gradients
 * follow chunks of that size, each computed in a 64-row tile whose rows past
 * the chunk are zeros; any Hkv dividing H.  Other K, or K > 128 with float32
 * inputs, return SGLA_ERR_UNSUPPORTED.
 */
sgla_status sgla_chunk_bwd(const sgla_chunk_args *args,
                           const void *q, const void *k, const void *v,
                           const float *g, const float *g_gamma,
                           const float *initial_state,
                           const int64_t *cu_seqlens_host,
                           const void *dout, const float *dht,
                           float *dq, float *dk, float *dv, float *dg, float *dg_gamma,
                           float *dh0,
                           void *workspace, size_t workspace_bytes,
                           hipStream_t stream);

/*
 * Chunked forward of elementwise-gate GLA, the general form Simple GLA is the
 * head-wise special case of (section 一: the elementwise gate decays every
 * state element on its own; the relinear pages pass a gate vector over the
 * key dimension):
 *     S_t = diag(exp(gk_t)) S_{t-1} + k_t v_t^T ,   o_t = scale * S_t^T q_t
 * Arguments as for sgla_chunk_fwd, with gk in place of g / g_gamma:
 *   gk              [B, T, H, K] float32 log gates, one per key (required);
 *                   accurate for gk <= 0, the forget-gate range
 *   q [B, T, H, K]; k [B, T, Hkv, K]; v [B, T, Hkv, V]; o [B, T, H, V];
 *   initial_state / final_state [N, H, K, V] (or [N, H, V, K] with
 *   state_v_first); cu_seqlens_host as for sgla_chunk_fwd;
 *   workspace >= sgla_gla_chunk_fwd_workspace_size(args, cu) bytes (the
 *   packed-sequence table, then a 64 x 64 float32 matrix per (chunk, head),
 *   chunks of chunk_size tokens;
 *   0 when there are no tokens).
 * Two launches (per-chunk A in parallel over chunks, then the chunk chain),
 * all products on the fp32 matrix cores.  Supported: K in {16,
 * 32, 64, 128}, V a multiple of 32, bf16 or float32 inputs, chunk_size 16,
 * 32 or 64 (smaller chunks run as short chunks of the 64-row tiles).
 */
size_t sgla_gla_chunk_fwd_workspace_size(const sgla_chunk_args *args, const int64_t *cu_seqlens_host);
sgla_status sgla_gla_chunk_fwd(const sgla_chunk_args *args,
                               const void *q, const void *k, const void *v, const float *gk,
                               const float *initial_state, const int64_t *cu_seqlens_host,
                               void *o, float *final_state,
                               void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Running normalizer of normalized linear attention (page "relinear": the
 * output divided by q . z, which the pages obtain by appending a column of
 * ones to v -- its state column is z and its output the normalizer):
 *     z_t = exp(g_t) z_{t-1} + k_t ,    den_t = scale * q_t . z_t
 * per sequence and query head, computed on its own (no widening of V).
 * Together with sgla_chunk_fwd it gives o_t / den_t.
 *
 * Arguments (device pointers unless stated):
 *   args            B, T, H, K, num_seqs, chunk_size, qkv_dtype, scale,
 *                   num_kv_heads and output_final_state are read; V, o_dtype
 *                   and state_v_first are not.
 *   q               [B, T, H, K];  k [B, T, Hkv, K] in qkv_dtype
 *   g, g_gamma      as for sgla_chunk_fwd (at most one; neither = no decay)
 *   initial_z       [N, H, K] float32, or NULL for zeros
 *   cu_seqlens_host as for sgla_chunk_fwd
 *   den             [B, T, H] float32 output
 *   final_z         [N, H, K] float32, written when output_final_state is
 *                   nonzero (may alias initial_z exactly)
 *   workspace       >= sgla_chunk_normalizer_workspace_size(args, cu) bytes
 *                   (the packed-sequence table, then per (chunk, head) K + 1
 *                   floats of chunk records; 0 when there are no tokens)
 * Supported: K in {16, 32, 64, 128, 256}, bf16 or float32 inputs,
 * chunk_size 16, 32 or 64 (the chunk records follow chunks of that size).
 */
size_t sgla_chunk_normalizer_workspace_size(const sgla_chunk_args *args, const int64_t *cu_seqlens_host);
sgla_status sgla_chunk_normalizer(const sgla_chunk_args *args, const void *q, const void *k,
                                  const float *g, const float *g_gamma, const float *initial_z,
                                  const int64_t *cu_seqlens_host, float *den, float *final_z,
                                  void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * One decode step of the running normalizer, in place (the decode side of
 * sgla_chunk_normalizer, beside sgla_recurrent_step):
 *     z <- exp(g) z + k ;   den = scale * q . z
 *   q [N, H, K], k [N, Hkv, K] in qkv_dtype; g [N, H] or g_gamma [H] (at
 *   most one); z [N, H, K] float32 in place; den [N, H] float32.
 * Supported: 1 <= K <= 4096.
 */
sgla_status sgla_recurrent_step_normalizer(int32_t N, int32_t H, int32_t num_kv_heads, int32_t K,
                                           float scale, int32_t qkv_dtype,
                                           const void *q, const void *k,
                                           const float *g, const float *g_gamma,
                                           float *z, float *den, hipStream_t stream);

/*
 * Step (1) alone: chunk-local inclusive cumulative sum of g times 1/ln 2,
 * restarting at every chunk_size-token chunk of every sequence (section 三,
 * the chunk_local_cumsum call with the RCP_LN2 scale).  g and gc are device
 * [B, T, H] float32; cu_seqlens_host as for sgla_chunk_fwd.  `workspace`
 * (device) must hold sgla_chunk_fwd_workspace_size(args, cu_seqlens_host)
 * bytes when cu_seqlens_host is not NULL (it carries the sequence table) and
 * may be NULL otherwise.  Only B, T, H, num_seqs and chunk_size of `args` are
 * read; chunk_size may be any power of two up to 64 (section 五 tests
 * chunk sizes 16, 32 and 64).  Exposed for testing the step in isolation.
 */
sgla_status sgla_chunk_local_cumsum(const sgla_chunk_args *args, const float *g,
                                    const int64_t *cu_seqlens_host, float *gc,
                                    void *workspace, size_t workspace_bytes,
                                    hipStream_t stream);

/*
 * One decode step for N independent sequences x H heads (section 四: single
 * tokens take the fused recurrent path instead of a chunk launch), in place:
 *     S <- exp(g) * S + k v^T ;   o = scale * S^T q   (updated state)
 *   q       [N, H, K] in qkv_dtype
 *   k       [N, Hkv, K] in qkv_dtype;  v [N, Hkv, V] in qkv_dtype
 *           (num_kv_heads = Hkv divides H, 0 means H; query head h reads kv
 *           head h / (H / Hkv))
 *   g       [N, H] float32 log gate, or NULL
 *   g_gamma [H] float32 per-head log decay, or NULL.  At most one of g /
 *           g_gamma (section 二); neither means no decay.
 *   state   [N, H, K, V] float32, or [N, H, V, K] when state_v_first is
 *           nonzero, read and written in place
 *   o       [N, H, V] in o_dtype; must not alias the state
 * All pointers are device pointers.  Supported: [K, V] layout: 1 <= K <= 1024
 * and V in {32, 64, 128, 256, 512}; [V, K] layout: K in {32, 64, 128, 256,
 * 512} and V a multiple of 32 in [32, 1024].
 */
sgla_status sgla_recurrent_step(int32_t N, int32_t H, int32_t num_kv_heads, int32_t K, int32_t V,
                                float scale, int32_t qkv_dtype, int32_t o_dtype,
                                int32_t state_v_first,
                                const void *q, const void *k, const void *v,
                                const float *g, const float *g_gamma, float *state, void *o,
                                hipStream_t stream);

/*
 * Parallel form (section 二: the parallel entry writes out the decayed
 * attention matrix; section 五: its test checks that matrix).  Per batch row
 * b and query head h, with G_t = g_0 + ... + g_t the running log gate of the
 * row (g_t = g_gamma[h] for the per-head decay, 0 when neither is given):
 *     A[i][j] = scale * (q_i . k_j) * exp(G_i - G_j)   for j <= i, else 0
 *     o_i     = sum_j A[i][j] v_j
 * i.e. sgla_chunk_fwd's output from a zero initial state, computed as dense
 * causal attention with a decay mask instead of through chunk states.
 *
 * Arguments (device pointers):
 *   args     B, T, H, K, V, num_kv_heads, qkv_dtype, o_dtype and scale are
 *            read; num_seqs, chunk_size, output_final_state and
 *            state_v_first are not (dense input only, no initial or final
 *            state).
 *   q        [B, T, H, K];  k [B, T, Hkv, K];  v [B, T, Hkv, V]: all bf16 or
 *            all float32 (qkv_dtype)
 *   g        [B, T, H] float32 log gates, or NULL
 *   g_gamma  [H] float32 per-head log decay, or NULL (at most one of the two)
 *   o        [B, T, H, V] in o_dtype
 *   attn     [B, H, T, T] float32 written in full (zeros above the diagonal),
 *            or NULL to compute o only.  B * H * T * T * 4 bytes: the caller
 *            sizes T accordingly (T <= 4194304 when A is written).
 * All buffers 16-byte aligned; no output may alias an input.  No workspace,
 * one kernel launch.  Supported: bf16 q, k, v with K in {64, 128, 256} and V
 * a multiple of 16 in [16, 256] (bf16 matrix cores, A split into hi + lo);
 * float32 q, k, v with K and V multiples of 16 in [16, 256] (fp32 matrix
 * cores, decay exponents formed in float64).  Other shapes return
 * SGLA_ERR_UNSUPPORTED.
 */
sgla_status sgla_parallel_fwd(const sgla_chunk_args *args,
                              const void *q, const void *k, const void *v,
                              const float *g, const float *g_gamma,
                              void *o, float *attn, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* SGLA_H */
