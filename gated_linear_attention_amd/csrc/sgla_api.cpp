// C ABI of libsgla: argument validation, workspace sizing, packed-sequence
// tables and kernel launches.  Every check happens on the host before any
// work is enqueued, so a rejected call leaves outputs, state and workspace
// untouched (page "flash-linear-attention 中的 Simple GLA", section 二: g and
// g_gamma are exclusive, packed input needs B == 1 and one initial state per
// sequence, chunk_size is a power of two; errors are raised, never absorbed
// by a silent fallback).
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "sgla.h"
#include "sgla_internal.h"

namespace {

thread_local std::string g_last_error;

sgla_status fail(sgla_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

sgla_status ok() {
  g_last_error.clear();
  return SGLA_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

bool is_pow2(int32_t x) { return x > 0 && (x & (x - 1)) == 0; }

// Validated description of one chunk_fwd request.
struct Plan {
  int32_t N = 0;             // sequences
  int32_t Hkv = 0;           // kv heads (divides H)
  int64_t total_tokens = 0;  // B * T
  int32_t num_chunks = 0;
  bool packed = false;
  std::vector<sgla::SeqEntry> seqs;      // packed only, longest first
  int32_t chunk_size = 0;                // requested chunk size (power of two <= 64)
  int32_t grid_chunk = sgla::kChunk;     // tokens per chunk of the chunk tables: 64, or for the
                                         // backward the requested chunk size
  bool prep = false;                     // wide-key bf16 path: per-chunk preparation buffers
  size_t seq_off = 0, chunk_off = 0, gate_off = 0, amat_off = 0, kt_off = 0, q_off = 0, total_bytes = 0;
  // segmented chains (bf16 K <= 128 forward)
  bool seg = false;
  std::vector<sgla::SegEntry> segs;      // bin by bin
  std::vector<sgla::BinEntry> bins;      // most loaded first
  std::vector<sgla::BlockEntry> blocks;  // per scanned sequence, in token order
  std::vector<sgla::ScanEntry> scans;
  int32_t num_rec = 0;                   // entering-state records (segments after a sequence's first)
  size_t segt_off = 0, bint_off = 0, blkt_off = 0, scnt_off = 0, urec_off = 0, ulog_off = 0, sin_off = 0;
};

// Segmented chains.  The chunk kernel gives each workgroup slot a bin of
// units to run one after another; with one workgroup per (sequence, head, V
// tile) the longest sequence's chain bounds the launch.  A sequence longer
// than a chosen length T is cut at chunk boundaries into a leading remainder
// and pieces of exactly T chunks, and all pieces are packed into the bins
// (longest first onto the least loaded bin), which brings the bound towards
// (all chunks) / (bins) when the lengths are uneven or there are fewer
// sequences than bins.  Every chunk before a sequence's last piece costs one
// more pass over its k and v in the state-only pre-pass, charged here at
// kPrepassWeight of a chunk step spread over the whole GPU.
constexpr int64_t kSegSlots = 256;      // one chunk workgroup per CU of the 256
constexpr int64_t kMinSegChunks = 16;   // shortest T considered
constexpr double kPrepassWeight = 0.6;

struct BinPack {
  int64_t makespan = 0;               // chunks of the most loaded bin
  std::vector<int32_t> bin_of;        // per piece
};

// Longest-processing-time packing of piece lengths (chunks) into `bins`.
BinPack pack_bins(const std::vector<int64_t>& lens, int64_t bins) {
  BinPack bp;
  bp.bin_of.assign(lens.size(), 0);
  std::vector<int32_t> order(lens.size());
  for (size_t i = 0; i < lens.size(); ++i) order[i] = (int32_t)i;
  std::stable_sort(order.begin(), order.end(), [&](int32_t x, int32_t y) { return lens[x] > lens[y]; });
  // min-heap of (load, bin)
  std::vector<std::pair<int64_t, int32_t>> heap;
  for (int64_t b = 0; b < bins; ++b) heap.push_back({0, (int32_t)b});
  auto cmp = [](const std::pair<int64_t, int32_t>& x, const std::pair<int64_t, int32_t>& y) {
    return x.first != y.first ? x.first > y.first : x.second > y.second;
  };
  std::make_heap(heap.begin(), heap.end(), cmp);
  for (int32_t i : order) {
    std::pop_heap(heap.begin(), heap.end(), cmp);
    heap.back().first += std::max<int64_t>(lens[i], 1);
    bp.bin_of[i] = heap.back().second;
    bp.makespan = std::max(bp.makespan, heap.back().first);
    std::push_heap(heap.begin(), heap.end(), cmp);
  }
  return bp;
}

// Pieces of a sequence of c chunks at length T: the remainder first (if
// any), then pieces of T.  Returns their lengths in order.
std::vector<int64_t> pieces_of(int64_t c, int64_t T) {
  std::vector<int64_t> out;
  if (c <= T) {
    out.push_back(c);
    return out;
  }
  const int64_t k = (c + T - 1) / T;
  const int64_t first = c - (k - 1) * T;
  out.push_back(first);
  for (int64_t j = 1; j < k; ++j) out.push_back(T);
  return out;
}

void plan_segments(const sgla_chunk_args* a, const int64_t* cu, Plan* P) {
  const int64_t C = sgla::kChunk;
  const int32_t N = P->N;
  const int64_t units = (int64_t)a->H * (a->V / sgla::chunk_fwd_bf16_vtile(a->V));   // workgroups per piece
  const int64_t bins = std::max<int64_t>(1, kSegSlots / units);
  auto bos_of = [&](int32_t n) { return cu != nullptr ? cu[n] : (int64_t)n * a->T; };
  auto len_of = [&](int32_t n) { return cu != nullptr ? cu[n + 1] - cu[n] : (int64_t)a->T; };
  std::vector<int64_t> chunks(N);
  int64_t maxc = 0, total = 0;
  for (int32_t n = 0; n < N; ++n) {
    chunks[n] = (len_of(n) + C - 1) / C;
    maxc = std::max(maxc, chunks[n]);
    total += chunks[n];
  }
  if (maxc <= kMinSegChunks || N > 64 * bins) return;
  auto cost_at = [&](int64_t T, double* cost) {
    std::vector<int64_t> lens;
    int64_t pre = 0;
    for (int32_t n = 0; n < N; ++n) {
      const std::vector<int64_t> pc = pieces_of(chunks[n], T);
      lens.insert(lens.end(), pc.begin(), pc.end());
      pre += chunks[n] - pc.back();
    }
    *cost = (double)pack_bins(lens, bins).makespan + kPrepassWeight * (double)pre * (double)units / (double)kSegSlots;
  };
  double base;
  cost_at(maxc, &base);   // no piece cut
  double best = base;
  int64_t bestT = 0;
  const int64_t t_lo = std::max(kMinSegChunks, (total + bins - 1) / bins);
  // candidate lengths: the lower bound and the lengths that split the longest
  // sequence into k equal parts
  std::vector<int64_t> cand;
  for (int64_t t = t_lo; t < t_lo + 8 && t < maxc; ++t) cand.push_back(t);
  for (int64_t k = 2; k <= 64; ++k) {
    const int64_t t = (maxc + k - 1) / k;
    if (t >= t_lo && t < maxc) cand.push_back(t);
  }
  for (int64_t t : cand) {
    double cost;
    cost_at(t, &cost);
    if (cost < best * 0.97) {
      best = cost;
      bestT = t;
    }
  }
  if (bestT == 0) return;
  P->seg = true;
  std::vector<sgla::SegEntry> segs;
  std::vector<int64_t> seg_chunks;
  for (int32_t n = 0; n < N; ++n) {
    const int64_t bos = bos_of(n), len = len_of(n);
    const std::vector<int64_t> pc = pieces_of(chunks[n], bestT);
    const int64_t S = (int64_t)pc.size();
    int64_t start = 0;   // first chunk of the piece
    for (int64_t s = 0; s < S; ++s) {
      sgla::SegEntry e{};
      e.bos = (int32_t)(bos + start * C);
      e.len = (int32_t)std::min(len - start * C, pc[s] * C);
      e.seq = n;
      e.init = s == 0 ? -1 : P->num_rec + (int32_t)s - 1;
      e.last = s == S - 1 ? 1 : 0;
      segs.push_back(e);
      seg_chunks.push_back(pc[s]);
      start += pc[s];
    }
    if (S > 1) P->num_rec += (int32_t)S - 1;
  }
  // pre-pass blocks over every piece but a sequence's last: sized so the
  // pre-pass has about two workgroups per CU, 4 to 16 chunks each
  int64_t pre = 0;
  for (int32_t n = 0; n < N; ++n) pre += chunks[n] - pieces_of(chunks[n], bestT).back();
  const int64_t units_pre = (int64_t)a->H * (a->V / 64);
  const int64_t block_chunks =
      std::min<int64_t>(16, std::max<int64_t>(4, (pre * units_pre + 2 * kSegSlots - 1) / (2 * kSegSlots)));
  int32_t rec = 0;
  for (int32_t n = 0, i = 0; n < N; ++n) {
    const std::vector<int64_t> pc = pieces_of(chunks[n], bestT);
    const int32_t first_block = (int32_t)P->blocks.size();
    for (size_t s = 0; s + 1 < pc.size(); ++s) {
      const sgla::SegEntry& e = segs[i + s];
      const int64_t nb = (pc[s] + block_chunks - 1) / block_chunks;
      int64_t b0 = 0;
      for (int64_t b = 0; b < nb; ++b) {
        const int64_t bc = pc[s] / nb + (b < pc[s] % nb ? 1 : 0);
        sgla::BlockEntry be{};
        be.t0 = (int32_t)(e.bos + b0 * C);
        be.len = (int32_t)(bc * C);
        be.out_rec = b + 1 == nb ? rec + (int32_t)s : -1;
        P->blocks.push_back(be);
        b0 += bc;
      }
    }
    if (pc.size() > 1) {
      P->scans.push_back({n, first_block, (int32_t)P->blocks.size() - first_block, 0});
      rec += (int32_t)pc.size() - 1;
    }
    i += (int32_t)pc.size();
  }
  // pack, then lay the pieces out bin by bin, most loaded bin first
  const BinPack bp = pack_bins(seg_chunks, bins);
  std::vector<int64_t> load(bins, 0);
  std::vector<std::vector<int32_t>> members(bins);
  for (size_t i = 0; i < segs.size(); ++i) {
    load[bp.bin_of[i]] += seg_chunks[i];
    members[bp.bin_of[i]].push_back((int32_t)i);
  }
  std::vector<int32_t> border(bins);
  for (int64_t b = 0; b < bins; ++b) border[b] = (int32_t)b;
  std::stable_sort(border.begin(), border.end(), [&](int32_t x, int32_t y) { return load[x] > load[y]; });
  for (int32_t b : border) {
    if (members[b].empty()) continue;
    P->bins.push_back({(int32_t)P->segs.size(), (int32_t)members[b].size()});
    for (int32_t i : members[b]) P->segs.push_back(segs[i]);
  }
}

// chunk_grid: lay the chunk tables out at the requested chunk size (the
// backward, whose 64-row tiles take chunks of 16 or 32 tokens as short
// chunks); every other entry point keeps its 64-token grid.
sgla_status plan_shape(const sgla_chunk_args* a, const int64_t* cu, bool need_kv_support,
                       Plan* P, bool chunk_grid = false) {
  if (a == nullptr) return fail(SGLA_ERR_INVALID_ARG, "args is NULL");
  if (a->B < 0 || a->T < 0) return fail(SGLA_ERR_SHAPE, "B and T must be >= 0 (got B=%d T=%d)", a->B, a->T);
  if (a->H <= 0) return fail(SGLA_ERR_SHAPE, "H must be > 0 (got %d)", a->H);
  P->Hkv = a->num_kv_heads == 0 ? a->H : a->num_kv_heads;
  if (P->Hkv < 0 || a->H % P->Hkv != 0)
    return fail(SGLA_ERR_SHAPE, "num_kv_heads must divide H (got num_kv_heads=%d, H=%d)", a->num_kv_heads, a->H);
  const int32_t cs = a->chunk_size == 0 ? sgla::kChunk : a->chunk_size;
  if (!is_pow2(cs)) return fail(SGLA_ERR_UNSUPPORTED, "chunk_size must be a power of two (got %d)", cs);
  if (cs > sgla::kChunk)
    return fail(SGLA_ERR_UNSUPPORTED, "chunk_size %d is not implemented (at most 64)", cs);
  P->chunk_size = cs;
  P->grid_chunk = chunk_grid ? cs : sgla::kChunk;
  const int64_t gcs = P->grid_chunk;
  if (need_kv_support) {
    if (a->K <= 0 || a->V <= 0) return fail(SGLA_ERR_SHAPE, "K and V must be > 0");
    if (a->qkv_dtype == SGLA_BF16) {
      if (!(a->K == 64 || a->K == 128 || a->K == 256 || a->K == 512))
        return fail(SGLA_ERR_UNSUPPORTED, "bf16 inputs support K in {64,128,256,512} (got %d)", a->K);
      const int vmul = a->K >= 256 ? 32 : 64;
      if (a->V % vmul != 0)
        return fail(SGLA_ERR_UNSUPPORTED, "bf16 inputs with K=%d support V a multiple of %d (got %d)",
                    a->K, vmul, a->V);
    } else if (a->qkv_dtype == SGLA_F32) {
      if (!(a->K == 16 || a->K == 32 || a->K == 64 || a->K == 128))
        return fail(SGLA_ERR_UNSUPPORTED, "float32 inputs support K in {16,32,64,128} (got %d)", a->K);
      if (a->V % 32 != 0)
        return fail(SGLA_ERR_UNSUPPORTED, "float32 inputs support V a multiple of 32 (got %d)", a->V);
    } else {
      return fail(SGLA_ERR_DTYPE, "qkv_dtype must be SGLA_BF16 or SGLA_F32 (got %d)", a->qkv_dtype);
    }
    if (a->o_dtype != SGLA_BF16 && a->o_dtype != SGLA_F32)
      return fail(SGLA_ERR_DTYPE, "o_dtype must be SGLA_BF16 or SGLA_F32 (got %d)", a->o_dtype);
    if (!std::isfinite(a->scale)) return fail(SGLA_ERR_INVALID_ARG, "scale must be finite");
  }
  P->total_tokens = (int64_t)a->B * a->T;
  if (P->total_tokens > INT32_MAX)
    return fail(SGLA_ERR_UNSUPPORTED, "B*T = %lld tokens exceeds 2^31-1", (long long)P->total_tokens);
  if (cu != nullptr) {
    P->packed = true;
    if (a->B != 1) return fail(SGLA_ERR_SHAPE, "packed input (cu_seqlens given) requires B == 1 (got B=%d)", a->B);
    if (a->num_seqs < 1) return fail(SGLA_ERR_SHAPE, "num_seqs must be >= 1 with cu_seqlens (got %d)", a->num_seqs);
    P->N = a->num_seqs;
    if (cu[0] != 0) return fail(SGLA_ERR_SHAPE, "cu_seqlens[0] must be 0 (got %lld)", (long long)cu[0]);
    for (int32_t n = 0; n < P->N; ++n)
      if (cu[n + 1] < cu[n])
        return fail(SGLA_ERR_SHAPE, "cu_seqlens must be non-decreasing (cu[%d]=%lld > cu[%d]=%lld)", n,
                    (long long)cu[n], n + 1, (long long)cu[n + 1]);
    if (cu[P->N] != a->T)
      return fail(SGLA_ERR_SHAPE, "cu_seqlens[N] must equal T (got %lld, T=%d)", (long long)cu[P->N], a->T);
    P->seqs.resize(P->N);
    for (int32_t n = 0; n < P->N; ++n) {
      sgla::SeqEntry& e = P->seqs[n];
      e.bos = (int32_t)cu[n];
      e.len = (int32_t)(cu[n + 1] - cu[n]);
      e.seq = n;
      e.chunk0 = 0;
    }
    for (int32_t n = 1; n < P->N; ++n)
      P->seqs[n].chunk0 = P->seqs[n - 1].chunk0 + (int32_t)((P->seqs[n - 1].len + gcs - 1) / gcs);
    // longest sequences first: they bound the critical path
    std::stable_sort(P->seqs.begin(), P->seqs.end(),
                     [](const sgla::SeqEntry& x, const sgla::SeqEntry& y) { return x.len > y.len; });
    int64_t nch = 0;
    for (int32_t n = 0; n < P->N; ++n) nch += (cu[n + 1] - cu[n] + gcs - 1) / gcs;
    if (nch > INT32_MAX) return fail(SGLA_ERR_UNSUPPORTED, "%lld chunks exceed 2^31-1", (long long)nch);
    P->num_chunks = (int32_t)nch;
  } else {
    P->N = a->B;
    const int64_t nch = a->T > 0 ? (int64_t)a->B * ((a->T + gcs - 1) / gcs) : 0;
    if (nch > INT32_MAX) return fail(SGLA_ERR_UNSUPPORTED, "%lld chunks exceed 2^31-1", (long long)nch);
    P->num_chunks = (int32_t)nch;
  }
  // workgroup counts of the launches must fit a 32-bit grid
  if ((int64_t)P->num_chunks * a->H > INT32_MAX)
    return fail(SGLA_ERR_UNSUPPORTED, "%d chunks x %d heads exceeds 2^31-1 work units", P->num_chunks, a->H);
  P->prep = need_kv_support && a->qkv_dtype == SGLA_BF16 && a->K >= 256 && cs == sgla::kChunk;
  P->seq_off = 0;
  P->chunk_off = P->seq_off + align_up(P->seqs.size() * sizeof(sgla::SeqEntry), 256);
  P->gate_off = P->chunk_off + align_up((P->packed ? (size_t)P->num_chunks : 0) * sizeof(sgla::ChunkEntry), 256);
  P->amat_off = P->gate_off;
  if (P->prep) {
    const size_t tasks = (size_t)P->num_chunks * a->H;        // (chunk, query head)
    const size_t kv_tasks = (size_t)P->num_chunks * P->Hkv;   // (chunk, kv head)
    P->amat_off = P->gate_off + align_up(tasks * sgla::kGateStride * sizeof(float), 256);
    P->kt_off = P->amat_off + tasks * 2 * sgla::kChunk * sgla::kChunk * 2;
    P->q_off = P->kt_off + kv_tasks * (size_t)a->K * sgla::kChunk * 2;
    P->total_bytes = P->q_off + tasks * (size_t)a->K * sgla::kChunk * 2;
  } else {
    P->total_bytes = P->gate_off;
  }
  if (need_kv_support && a->qkv_dtype == SGLA_BF16 && a->K <= 128 && cs == sgla::kChunk && a->V % 64 == 0) {
    plan_segments(a, cu, P);
    if (P->seg) {
      const size_t KV = (size_t)a->K * a->V;
      P->segt_off = align_up(P->total_bytes, 256);
      P->bint_off = P->segt_off + align_up(P->segs.size() * sizeof(sgla::SegEntry), 256);
      P->blkt_off = P->bint_off + align_up(P->bins.size() * sizeof(sgla::BinEntry), 256);
      P->scnt_off = P->blkt_off + align_up(P->blocks.size() * sizeof(sgla::BlockEntry), 256);
      P->urec_off = P->scnt_off + align_up(P->scans.size() * sizeof(sgla::ScanEntry), 256);
      P->ulog_off = P->urec_off + align_up(P->blocks.size() * a->H * KV * sizeof(float), 256);
      P->sin_off = P->ulog_off + align_up(P->blocks.size() * a->H * sizeof(float), 256);
      P->total_bytes = P->sin_off + align_up((size_t)P->num_rec * a->H * KV * sizeof(float), 256);
    }
  }
  return SGLA_OK;
}

// The entry points whose kernels run any chunk grid in 64-row tiles (the
// backward, the elementwise-gate GLA, the normalizer): 16, 32 or 64.
sgla_status need_chunk_16_32_64(const Plan& P) {
  if (P.chunk_size != sgla::kChunk && P.chunk_size != 32 && P.chunk_size != 16)
    return fail(SGLA_ERR_UNSUPPORTED, "chunk_size %d is not implemented (16, 32 or 64)", P.chunk_size);
  return SGLA_OK;
}

// Backward request: the forward's shape rules, then the backward's own
// support set; workspace = tables, per-chunk states and state gradients,
// per-chunk gate sums, for K > 128 the key-tile gate records.
struct BwdPlan {
  Plan P;
  size_t h_off = 0, dh_off = 0, gpart_off = 0, wpart_off = 0, dkq_off = 0, dvq_off = 0, total_bytes = 0;
};

sgla_status plan_bwd(const sgla_chunk_args* a, const int64_t* cu, BwdPlan* B) {
  sgla_status st = plan_shape(a, cu, false, &B->P, true);
  if (st != SGLA_OK) return st;
  st = need_chunk_16_32_64(B->P);
  if (st != SGLA_OK) return st;
  if (a->qkv_dtype != SGLA_BF16 && a->qkv_dtype != SGLA_F32)
    return fail(SGLA_ERR_DTYPE, "qkv_dtype must be SGLA_BF16 or SGLA_F32 (got %d)", a->qkv_dtype);
  const bool wide = a->K == 256 || a->K == 512;
  if (!(a->K == 16 || a->K == 32 || a->K == 64 || a->K == 128 || wide))
    return fail(SGLA_ERR_UNSUPPORTED, "the backward supports K in {16,32,64,128,256,512} (got %d)", a->K);
  if (wide && a->qkv_dtype != SGLA_BF16)
    return fail(SGLA_ERR_UNSUPPORTED, "the backward supports K = %d for bf16 inputs only", a->K);
  if (a->V <= 0 || a->V % 32 != 0)
    return fail(SGLA_ERR_UNSUPPORTED, "the backward supports V a multiple of 32 (got %d)", a->V);
  if (wide && a->V % sgla::kWideDvCols != 0)
    return fail(SGLA_ERR_UNSUPPORTED, "the backward with K = %d supports V a multiple of %d (got %d)", a->K,
                sgla::kWideDvCols, a->V);
  if (!std::isfinite(a->scale)) return fail(SGLA_ERR_INVALID_ARG, "scale must be finite");
  const size_t tasks = (size_t)B->P.num_chunks * a->H;
  const size_t rec = tasks * (size_t)a->K * a->V * sizeof(float);
  B->h_off = align_up(B->P.total_bytes, 256);
  B->dh_off = B->h_off + align_up(rec, 256);
  B->gpart_off = B->dh_off + align_up(rec, 256);
  B->wpart_off = B->gpart_off + align_up(tasks * sizeof(float), 256);
  B->dkq_off = B->wpart_off;
  if (wide) B->dkq_off += align_up(tasks * (size_t)(a->K / 128) * sgla::kWidePart * sizeof(float), 256);
  B->total_bytes = B->dkq_off;
  if (B->P.Hkv != a->H) {
    // grouped kv heads: k and v gradients per query head, summed over each group
    const size_t th = (size_t)B->P.total_tokens * a->H;
    B->dvq_off = B->dkq_off + align_up(th * (size_t)a->K * sizeof(float), 256);
    B->total_bytes = B->dvq_off + align_up(th * (size_t)a->V * sizeof(float), 256);
  }
  return SGLA_OK;
}

sgla_status hip_fail(hipError_t e, const char* what) {
  return fail(SGLA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Write the packed-sequence tables into the workspace, stream-ordered: the
// sequence entries travel by value in the arguments of table_put launches
// (kTablePut per launch), which also expand each sequence into its chunk
// rows.  No host buffer outlives the call, nothing is copied from pageable
// memory and the host never waits.
sgla_status upload_tables(const Plan& P, char* ws, hipStream_t stream) {
  if (!P.packed) return SGLA_OK;
  auto* seq_table = reinterpret_cast<sgla::SeqEntry*>(ws + P.seq_off);
  auto* chunk_table = P.num_chunks == 0 ? nullptr : reinterpret_cast<sgla::ChunkEntry*>(ws + P.chunk_off);
  sgla::TablePut put;
  put.chunk = P.grid_chunk;
  put.pad = 0;
  for (size_t first = 0; first < P.seqs.size(); first += sgla::kTablePut) {
    const size_t n = std::min<size_t>(sgla::kTablePut, P.seqs.size() - first);
    put.first = (int32_t)first;
    put.count = (int32_t)n;
    std::memcpy(put.e, P.seqs.data() + first, n * sizeof(sgla::SeqEntry));
    const hipError_t e = sgla::launch_table_put(put, seq_table, chunk_table, stream);
    if (e != hipSuccess) return hip_fail(e, "writing the sequence and chunk tables");
  }
  return SGLA_OK;
}

// Copy a host table into the workspace through table_words launches (the
// payload travels in the launch arguments).
template <typename T>
sgla_status upload_words(const std::vector<T>& v, char* dst, hipStream_t stream) {
  static_assert(sizeof(T) % 4 == 0, "word-sized entries");
  const size_t words = v.size() * sizeof(T) / 4;
  const uint32_t* src = reinterpret_cast<const uint32_t*>(v.data());
  sgla::TableWords put;
  for (size_t first = 0; first < words; first += sgla::kTableWords) {
    const size_t n = std::min<size_t>(sgla::kTableWords, words - first);
    put.first = (int32_t)first;
    put.count = (int32_t)n;
    std::memcpy(put.w, src + first, n * 4);
    const hipError_t e = sgla::launch_table_words(put, reinterpret_cast<uint32_t*>(dst), stream);
    if (e != hipSuccess) return hip_fail(e, "writing the segment tables");
  }
  return SGLA_OK;
}

sgla::StateLayout state_layout(const sgla_chunk_args& a) {
  sgla::StateLayout s;
  s.rs = a.state_v_first ? 1 : a.V;
  s.cs = a.state_v_first ? a.K : 1;
  return s;
}

sgla::SeqLayout layout_of(const sgla_chunk_args* a, const Plan& P, char* ws) {
  sgla::SeqLayout L;
  L.num_seqs = P.N;
  L.T = a->T;
  L.seq_table = P.packed ? reinterpret_cast<const sgla::SeqEntry*>(ws + P.seq_off) : nullptr;
  L.chunk_table = P.packed ? reinterpret_cast<const sgla::ChunkEntry*>(ws + P.chunk_off) : nullptr;
  L.num_chunks = P.num_chunks;
  L.chunk = P.grid_chunk;
  return L;
}

}  // namespace

namespace sgla {

size_t chunk_fwd_workspace(const sgla_chunk_args* args, const int64_t* cu_seqlens_host, sgla_status* status) {
  Plan P;
  *status = plan_shape(args, cu_seqlens_host, true, &P);
  if (*status != SGLA_OK) return 0;
  if (P.chunk_size != kChunk && P.chunk_size != 32 && P.chunk_size != 16) {
    *status = fail(SGLA_ERR_UNSUPPORTED, "chunk_size %d is not implemented (16, 32 or 64)", P.chunk_size);
    return 0;
  }
  return P.total_bytes;
}

sgla_status report(sgla_status st, const char* msg) { return fail(st, "%s", msg); }

sgla_status chunk_fwd_enqueue(const sgla_chunk_args* args, const void* q, const void* k, const void* v,
                              const float* g, const float* g_gamma, const float* initial_state,
                              const int64_t* cu_seqlens_host, void* o, float* final_state, void* workspace,
                              size_t workspace_bytes, hipStream_t stream, WorkspaceAcquire acquire) {
  Plan P;
  sgla_status st = plan_shape(args, cu_seqlens_host, true, &P);
  if (st != SGLA_OK) return st;
  if (P.chunk_size != sgla::kChunk && P.chunk_size != 32 && P.chunk_size != 16)
    return fail(SGLA_ERR_UNSUPPORTED, "chunk_size %d is not implemented (16, 32 or 64)", P.chunk_size);
  const sgla_chunk_args& a = *args;
  if (g != nullptr && g_gamma != nullptr)
    return fail(SGLA_ERR_INVALID_ARG, "g and g_gamma are mutually exclusive; pass at most one");
  const bool any_tokens = P.total_tokens > 0;
  if (any_tokens && (q == nullptr || k == nullptr || v == nullptr || o == nullptr))
    return fail(SGLA_ERR_INVALID_ARG, "q, k, v and o must be non-NULL");
  if (a.output_final_state && final_state == nullptr)
    return fail(SGLA_ERR_INVALID_ARG, "output_final_state is set but final_state is NULL");
  if (any_tokens && !(aligned(q, 16) && aligned(k, 16) && aligned(v, 16) && aligned(o, 16)))
    return fail(SGLA_ERR_INVALID_ARG, "q, k, v and o must be 16-byte aligned");
  if ((g && !aligned(g, 4)) || (initial_state && !aligned(initial_state, 16)) ||
      (final_state && !aligned(final_state, 16)))
    return fail(SGLA_ERR_INVALID_ARG, "g and state pointers must be aligned");
  const size_t need = P.total_bytes;
  if (final_state != nullptr && initial_state != nullptr && final_state != initial_state) {
    const size_t sb = (size_t)P.N * a.H * a.K * a.V * sizeof(float);
    const char* f0 = reinterpret_cast<const char*>(final_state);
    const char* i0 = reinterpret_cast<const char*>(initial_state);
    if (f0 < i0 + sb && i0 < f0 + sb)
      return fail(SGLA_ERR_INVALID_ARG, "final_state partially overlaps initial_state (only exact aliasing is allowed)");
  }
  if (need > 0 && acquire != nullptr) {
    // every argument is valid: now obtain the library-owned scratch memory
    st = acquire(&workspace);
    if (st != SGLA_OK) return st;
  }
  if (need > 0 && (workspace == nullptr || workspace_bytes < need))
    return fail(SGLA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given%s", need, workspace_bytes,
                workspace == nullptr ? " (NULL)" : "");
  if (need > 0 && !aligned(workspace, 256)) return fail(SGLA_ERR_WORKSPACE, "workspace must be 256-byte aligned");

  char* ws = static_cast<char*>(workspace);
  if (!P.seg) {
    st = upload_tables(P, ws, stream);
    if (st != SGLA_OK) return st;
  }
  const sgla::SeqLayout L = layout_of(args, P, ws);

  sgla::ChunkFwdParams p;
  p.q = q;
  p.k = k;
  p.v = v;
  p.g = g;
  p.g_gamma = g_gamma;
  p.h0 = initial_state;
  p.o = o;
  p.ht = a.output_final_state ? final_state : nullptr;
  p.scale = a.scale;
  p.H = a.H;
  p.Hkv = P.Hkv;
  p.K = a.K;
  p.V = a.V;
  p.o_bf16 = a.o_dtype == SGLA_BF16;
  p.sl = state_layout(a);
  p.seqs = L;
  p.gates = P.prep ? reinterpret_cast<const float*>(ws + P.gate_off) : nullptr;
  p.amat = P.prep ? ws + P.amat_off : nullptr;
  p.ktf = P.prep ? ws + P.kt_off : nullptr;
  p.qfr = P.prep ? ws + P.q_off : nullptr;
  if (p.ht == nullptr && !any_tokens) return ok();
  hipError_t e;
  if (P.seg) {
    // segmented chains: tables, the later segments' entering states, then
    // one chunk workgroup per (segment, head, V tile)
    sgla::TableWords inline_words;
    bool tables_inline = false;
    {
      // the four tables are adjacent in the workspace: one region, uploaded
      // with as few launches as its size allows
      std::vector<uint32_t> region((P.urec_off - P.segt_off) / 4, 0u);
      auto put = [&](const void* src, size_t bytes, size_t off) {
        if (bytes > 0) std::memcpy(reinterpret_cast<char*>(region.data()) + (off - P.segt_off), src, bytes);
      };
      put(P.segs.data(), P.segs.size() * sizeof(sgla::SegEntry), P.segt_off);
      put(P.bins.data(), P.bins.size() * sizeof(sgla::BinEntry), P.bint_off);
      put(P.blocks.data(), P.blocks.size() * sizeof(sgla::BlockEntry), P.blkt_off);
      put(P.scans.data(), P.scans.size() * sizeof(sgla::ScanEntry), P.scnt_off);
      if (region.size() <= (size_t)sgla::kTableWords && !P.blocks.empty()) {
        // small: the pre-pass carries the region in its arguments
        inline_words.first = 0;
        inline_words.count = (int32_t)region.size();
        std::memcpy(inline_words.w, region.data(), region.size() * sizeof(uint32_t));
        tables_inline = true;
      } else {
        st = upload_words(region, ws + P.segt_off, stream);
        if (st != SGLA_OK) return st;
      }
    }
    sgla::SegmentParams sp;
    sp.k = k;
    sp.v = v;
    sp.g = g;
    sp.g_gamma = g_gamma;
    sp.h0 = initial_state;
    sp.H = a.H;
    sp.Hkv = P.Hkv;
    sp.K = a.K;
    sp.V = a.V;
    sp.sl = state_layout(a);
    sp.blocks = reinterpret_cast<const sgla::BlockEntry*>(ws + P.blkt_off);
    sp.num_blocks = (int32_t)P.blocks.size();
    sp.scans = reinterpret_cast<const sgla::ScanEntry*>(ws + P.scnt_off);
    sp.num_scans = (int32_t)P.scans.size();
    sp.urec = reinterpret_cast<float*>(ws + P.urec_off);
    sp.ulog = reinterpret_cast<float*>(ws + P.ulog_off);
    sp.sin = reinterpret_cast<float*>(ws + P.sin_off);
    if (tables_inline) {
      sp.inline_tables = &inline_words;
      sp.table_dst = reinterpret_cast<uint32_t*>(ws + P.segt_off);
      sp.blk_word = (int32_t)((P.blkt_off - P.segt_off) / 4);
    }
    e = sgla::launch_segment_states(sp, stream);
    if (e != hipSuccess) return hip_fail(e, "launching the segment state passes");
    p.segs = reinterpret_cast<const sgla::SegEntry*>(ws + P.segt_off);
    p.bins = reinterpret_cast<const sgla::BinEntry*>(ws + P.bint_off);
    p.num_bins = (int32_t)P.bins.size();
    p.sin = sp.sin;
  }
  if (P.chunk_size != sgla::kChunk) {
    e = sgla::launch_chunk_fwd_small(p, P.chunk_size, a.qkv_dtype == SGLA_BF16, stream);
  } else if (P.prep) {
    sgla::ChunkPrepParams pp;
    pp.q = q;
    pp.k = k;
    pp.g = g;
    pp.g_gamma = g_gamma;
    pp.scale = a.scale;
    pp.H = a.H;
    pp.Hkv = P.Hkv;
    pp.K = a.K;
    pp.seqs = L;
    pp.gates = reinterpret_cast<float*>(ws + P.gate_off);
    pp.amat = ws + P.amat_off;
    pp.ktf = ws + P.kt_off;
    pp.qfr = ws + P.q_off;
    e = sgla::launch_chunk_prep_bf16(pp, stream);
    if (e != hipSuccess) return hip_fail(e, "launching the chunk preparation kernel");
    e = sgla::launch_chunk_fwd_bf16_wide(p, stream);
  } else {
    e = a.qkv_dtype != SGLA_BF16 ? sgla::launch_chunk_fwd_f32(p, stream)
                                 : sgla::launch_chunk_fwd_bf16(p, stream);
  }
  if (e != hipSuccess) return hip_fail(e, "launching the chunk kernel");
  return ok();
}


}  // namespace sgla

extern "C" {

int sgla_abi_version(void) { return SGLA_ABI_VERSION; }

const char* sgla_last_error(void) { return g_last_error.c_str(); }

size_t sgla_chunk_fwd_workspace_size(const sgla_chunk_args* args, const int64_t* cu_seqlens_host) {
  // sized for any power-of-two chunk size: sgla_chunk_local_cumsum takes its
  // workspace from here too
  Plan P;
  if (plan_shape(args, cu_seqlens_host, true, &P) != SGLA_OK) return 0;
  g_last_error.clear();
  return P.total_bytes;
}

sgla_status sgla_chunk_fwd(const sgla_chunk_args* args, const void* q, const void* k, const void* v,
                           const float* g, const float* g_gamma, const float* initial_state,
                           const int64_t* cu_seqlens_host, void* o, float* final_state,
                           void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return sgla::chunk_fwd_enqueue(args, q, k, v, g, g_gamma, initial_state, cu_seqlens_host, o, final_state,
                                 workspace, workspace_bytes, stream, nullptr);
}

size_t sgla_chunk_bwd_workspace_size(const sgla_chunk_args* args, const int64_t* cu_seqlens_host) {
  BwdPlan B;
  if (plan_bwd(args, cu_seqlens_host, &B) != SGLA_OK) return 0;
  g_last_error.clear();
  return B.total_bytes;
}

sgla_status sgla_chunk_bwd(const sgla_chunk_args* args, const void* q, const void* k, const void* v,
                           const float* g, const float* g_gamma, const float* initial_state,
                           const int64_t* cu_seqlens_host, const void* dout, const float* dht,
                           float* dq, float* dk, float* dv, float* dg, float* dg_gamma, float* dh0,
                           void* workspace, size_t workspace_bytes, hipStream_t stream) {
  BwdPlan B;
  sgla_status st = plan_bwd(args, cu_seqlens_host, &B);
  if (st != SGLA_OK) return st;
  const Plan& P = B.P;
  const sgla_chunk_args& a = *args;
  if (g != nullptr && g_gamma != nullptr)
    return fail(SGLA_ERR_INVALID_ARG, "g and g_gamma are mutually exclusive; pass at most one");
  if (g != nullptr && dg == nullptr) return fail(SGLA_ERR_INVALID_ARG, "g is given but dg is NULL");
  if (g_gamma != nullptr && dg_gamma == nullptr)
    return fail(SGLA_ERR_INVALID_ARG, "g_gamma is given but dg_gamma is NULL");
  const bool any_tokens = P.total_tokens > 0;
  if (any_tokens && (q == nullptr || k == nullptr || v == nullptr || dout == nullptr || dq == nullptr ||
                     dk == nullptr || dv == nullptr))
    return fail(SGLA_ERR_INVALID_ARG, "q, k, v, dout, dq, dk and dv must be non-NULL");
  if (any_tokens && !(aligned(q, 16) && aligned(k, 16) && aligned(v, 16) && aligned(dout, 16) &&
                      aligned(dq, 16) && aligned(dk, 16) && aligned(dv, 16)))
    return fail(SGLA_ERR_INVALID_ARG, "q, k, v, dout, dq, dk and dv must be 16-byte aligned");
  if ((g && !aligned(g, 4)) || (dg && !aligned(dg, 4)) || (initial_state && !aligned(initial_state, 16)) ||
      (dht && !aligned(dht, 16)) || (dh0 && !aligned(dh0, 16)))
    return fail(SGLA_ERR_INVALID_ARG, "g, dg and state pointers must be aligned");
  const size_t need = B.total_bytes;
  if (need > 0 && (workspace == nullptr || workspace_bytes < need))
    return fail(SGLA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given%s", need, workspace_bytes,
                workspace == nullptr ? " (NULL)" : "");
  if (need > 0 && !aligned(workspace, 256)) return fail(SGLA_ERR_WORKSPACE, "workspace must be 256-byte aligned");

  char* ws = static_cast<char*>(workspace);
  st = upload_tables(P, ws, stream);
  if (st != SGLA_OK) return st;
  sgla::ChunkBwdParams p;
  p.q = q;
  p.k = k;
  p.v = v;
  p.dout = dout;
  p.g = g;
  p.g_gamma = g_gamma;
  p.h0 = initial_state;
  p.dht = dht;
  const bool grouped = P.Hkv != a.H;
  p.dq = dq;
  p.dk = grouped ? reinterpret_cast<float*>(ws + B.dkq_off) : dk;
  p.dv = grouped ? reinterpret_cast<float*>(ws + B.dvq_off) : dv;
  p.dg = g != nullptr ? dg : nullptr;
  p.dg_gamma = g_gamma != nullptr ? dg_gamma : nullptr;
  p.dh0 = dh0;
  p.scale = a.scale;
  p.H = a.H;
  p.Hkv = P.Hkv;
  p.K = a.K;
  p.V = a.V;
  p.qkv_bf16 = a.qkv_dtype == SGLA_BF16;
  p.sl = state_layout(a);
  p.seqs = layout_of(args, P, ws);
  p.hbuf = reinterpret_cast<float*>(ws + B.h_off);
  p.dhbuf = reinterpret_cast<float*>(ws + B.dh_off);
  p.gpart = reinterpret_cast<float*>(ws + B.gpart_off);
  p.wpart = a.K > 128 ? reinterpret_cast<float*>(ws + B.wpart_off) : nullptr;
  hipError_t e = sgla::launch_chunk_bwd(p, stream);
  if (e != hipSuccess) return hip_fail(e, "launching the backward kernels");
  if (grouped) {
    e = sgla::launch_kv_group_sum(p.dk, dk, P.total_tokens, a.H, P.Hkv, a.K, stream);
    if (e == hipSuccess) e = sgla::launch_kv_group_sum(p.dv, dv, P.total_tokens, a.H, P.Hkv, a.V, stream);
    if (e != hipSuccess) return hip_fail(e, "launching the kv-group gradient sum");
  }
  return ok();
}

// Elementwise-gate GLA workspace: the packed-sequence tables, then per
// (chunk, query head) the preparation kernel's records: the 64 x 64 float32
// A (fp32 chain), or bf16 hi/lo planes of q~, k~ and A plus K floats of decay
// (bf16 chain).
struct GlaPlan {
  size_t amat_off = 0, qk_off = 0, a_off = 0, dl_off = 0, total_bytes = 0;
};

GlaPlan plan_gla(const sgla_chunk_args* a, const Plan& P) {
  GlaPlan G;
  const size_t tasks = (size_t)P.num_chunks * a->H;
  const size_t C = sgla::kChunk;
  if (tasks == 0) {
    G.total_bytes = P.total_bytes;
    return G;
  }
  G.amat_off = G.qk_off = align_up(P.total_bytes, 256);
  if (sgla::gla_bf16_chain(a->qkv_dtype == SGLA_BF16, a->K, a->V)) {
    G.a_off = G.qk_off + tasks * 4 * C * (size_t)a->K * 2;
    G.dl_off = G.a_off + tasks * 2 * C * C * 2;
    G.total_bytes = G.dl_off + tasks * (size_t)a->K * sizeof(float);
  } else {
    G.total_bytes = G.amat_off + tasks * C * C * sizeof(float);
  }
  return G;
}

size_t sgla_gla_chunk_fwd_workspace_size(const sgla_chunk_args* args, const int64_t* cu_seqlens_host) {
  Plan P;
  if (plan_shape(args, cu_seqlens_host, false, &P, true) != SGLA_OK) return 0;
  g_last_error.clear();
  return plan_gla(args, P).total_bytes;
}

sgla_status sgla_gla_chunk_fwd(const sgla_chunk_args* args, const void* q, const void* k, const void* v,
                               const float* gk, const float* initial_state, const int64_t* cu_seqlens_host,
                               void* o, float* final_state, void* workspace, size_t workspace_bytes,
                               hipStream_t stream) {
  Plan P;
  sgla_status st = plan_shape(args, cu_seqlens_host, false, &P, true);
  if (st != SGLA_OK) return st;
  st = need_chunk_16_32_64(P);
  if (st != SGLA_OK) return st;
  const sgla_chunk_args& a = *args;
  if (a.qkv_dtype != SGLA_BF16 && a.qkv_dtype != SGLA_F32)
    return fail(SGLA_ERR_DTYPE, "qkv_dtype must be SGLA_BF16 or SGLA_F32 (got %d)", a.qkv_dtype);
  if (a.o_dtype != SGLA_BF16 && a.o_dtype != SGLA_F32)
    return fail(SGLA_ERR_DTYPE, "o_dtype must be SGLA_BF16 or SGLA_F32 (got %d)", a.o_dtype);
  if (!(a.K == 16 || a.K == 32 || a.K == 64 || a.K == 128))
    return fail(SGLA_ERR_UNSUPPORTED, "elementwise-gate GLA supports K in {16,32,64,128} (got %d)", a.K);
  if (a.V <= 0 || a.V % 32 != 0)
    return fail(SGLA_ERR_UNSUPPORTED, "elementwise-gate GLA supports V a multiple of 32 (got %d)", a.V);
  if (!std::isfinite(a.scale)) return fail(SGLA_ERR_INVALID_ARG, "scale must be finite");
  const bool any_tokens = P.total_tokens > 0;
  if (any_tokens && (q == nullptr || k == nullptr || v == nullptr || gk == nullptr || o == nullptr))
    return fail(SGLA_ERR_INVALID_ARG, "q, k, v, gk and o must be non-NULL");
  if (a.output_final_state && final_state == nullptr)
    return fail(SGLA_ERR_INVALID_ARG, "output_final_state is set but final_state is NULL");
  if (any_tokens && !(aligned(q, 16) && aligned(k, 16) && aligned(v, 16) && aligned(gk, 16) && aligned(o, 16)))
    return fail(SGLA_ERR_INVALID_ARG, "q, k, v, gk and o must be 16-byte aligned");
  const GlaPlan GP = plan_gla(args, P);
  const size_t need = GP.total_bytes;
  if (need > 0 && (workspace == nullptr || workspace_bytes < need))
    return fail(SGLA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, workspace_bytes);
  if (final_state != nullptr && initial_state != nullptr && final_state != initial_state) {
    const size_t sb = (size_t)P.N * a.H * a.K * a.V * sizeof(float);
    const char* f0 = reinterpret_cast<const char*>(final_state);
    const char* i0 = reinterpret_cast<const char*>(initial_state);
    if (f0 < i0 + sb && i0 < f0 + sb)
      return fail(SGLA_ERR_INVALID_ARG, "final_state partially overlaps initial_state (only exact aliasing is allowed)");
  }
  char* ws = static_cast<char*>(workspace);
  st = upload_tables(P, ws, stream);
  if (st != SGLA_OK) return st;
  sgla::GlaFwdParams p;
  p.q = q;
  p.k = k;
  p.v = v;
  p.gk = gk;
  p.h0 = initial_state;
  p.o = o;
  p.ht = a.output_final_state ? final_state : nullptr;
  p.scale = a.scale;
  p.H = a.H;
  p.Hkv = P.Hkv;
  p.K = a.K;
  p.V = a.V;
  p.qkv_bf16 = a.qkv_dtype == SGLA_BF16;
  p.o_bf16 = a.o_dtype == SGLA_BF16;
  p.sl = state_layout(a);
  p.seqs = layout_of(args, P, ws);
  const bool any_chunks = P.num_chunks > 0;
  const bool bf16_chain = sgla::gla_bf16_chain(p.qkv_bf16 != 0, a.K, a.V);
  p.amat = any_chunks && !bf16_chain ? reinterpret_cast<float*>(ws + GP.amat_off) : nullptr;
  p.qk_hl = any_chunks && bf16_chain ? ws + GP.qk_off : nullptr;
  p.a_hl = any_chunks && bf16_chain ? ws + GP.a_off : nullptr;
  p.dl = any_chunks && bf16_chain ? reinterpret_cast<float*>(ws + GP.dl_off) : nullptr;
  if (p.ht == nullptr && !any_tokens) return ok();
  hipError_t e = sgla::launch_gla_chunk_fwd(p, stream);
  if (e != hipSuccess) return hip_fail(e, "launching the elementwise-gate GLA kernel");
  return ok();
}

// Normalizer workspace: the packed-sequence tables, then per (chunk, head) a
// K-float z record and one log2 decay.
struct NormPlan {
  size_t zrec_off = 0, dlog_off = 0, total_bytes = 0;
};

NormPlan plan_norm(const sgla_chunk_args* a, const Plan& P) {
  NormPlan N;
  const size_t tasks = (size_t)P.num_chunks * a->H;
  N.zrec_off = align_up(P.total_bytes, 256);
  N.dlog_off = N.zrec_off + align_up(tasks * (size_t)a->K * sizeof(float), 256);
  N.total_bytes = tasks == 0 ? P.total_bytes : N.dlog_off + align_up(tasks * sizeof(float), 256);
  return N;
}

size_t sgla_chunk_normalizer_workspace_size(const sgla_chunk_args* args, const int64_t* cu_seqlens_host) {
  Plan P;
  if (plan_shape(args, cu_seqlens_host, false, &P, true) != SGLA_OK) return 0;
  if (args->K <= 0) return 0;
  g_last_error.clear();
  return plan_norm(args, P).total_bytes;
}

sgla_status sgla_chunk_normalizer(const sgla_chunk_args* args, const void* q, const void* k, const float* g,
                                  const float* g_gamma, const float* initial_z, const int64_t* cu_seqlens_host,
                                  float* den, float* final_z, void* workspace, size_t workspace_bytes,
                                  hipStream_t stream) {
  Plan P;
  sgla_status st = plan_shape(args, cu_seqlens_host, false, &P, true);
  if (st != SGLA_OK) return st;
  st = need_chunk_16_32_64(P);
  if (st != SGLA_OK) return st;
  const sgla_chunk_args& a = *args;
  if (a.qkv_dtype != SGLA_BF16 && a.qkv_dtype != SGLA_F32)
    return fail(SGLA_ERR_DTYPE, "qkv_dtype must be SGLA_BF16 or SGLA_F32 (got %d)", a.qkv_dtype);
  if (!(a.K == 16 || a.K == 32 || a.K == 64 || a.K == 128 || a.K == 256))
    return fail(SGLA_ERR_UNSUPPORTED, "the normalizer supports K in {16,32,64,128,256} (got %d)", a.K);
  if (!std::isfinite(a.scale)) return fail(SGLA_ERR_INVALID_ARG, "scale must be finite");
  if (g != nullptr && g_gamma != nullptr)
    return fail(SGLA_ERR_INVALID_ARG, "g and g_gamma are mutually exclusive; pass at most one");
  const bool any_tokens = P.total_tokens > 0;
  if (any_tokens && (q == nullptr || k == nullptr || den == nullptr))
    return fail(SGLA_ERR_INVALID_ARG, "q, k and den must be non-NULL");
  if (a.output_final_state && final_z == nullptr)
    return fail(SGLA_ERR_INVALID_ARG, "output_final_state is set but final_z is NULL");
  if (any_tokens && !(aligned(q, 16) && aligned(k, 16)))
    return fail(SGLA_ERR_INVALID_ARG, "q and k must be 16-byte aligned");
  const NormPlan NP = plan_norm(args, P);
  if (NP.total_bytes > 0 && (workspace == nullptr || workspace_bytes < NP.total_bytes))
    return fail(SGLA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", NP.total_bytes, workspace_bytes);
  char* ws = static_cast<char*>(workspace);
  st = upload_tables(P, ws, stream);
  if (st != SGLA_OK) return st;
  sgla::NormalizerParams p;
  p.q = q;
  p.k = k;
  p.g = g;
  p.g_gamma = g_gamma;
  p.z0 = initial_z;
  p.den = den;
  p.zt = a.output_final_state ? final_z : nullptr;
  p.scale = a.scale;
  p.H = a.H;
  p.Hkv = P.Hkv;
  p.K = a.K;
  p.qkv_bf16 = a.qkv_dtype == SGLA_BF16;
  p.seqs = layout_of(args, P, ws);
  p.zrec = P.num_chunks > 0 ? reinterpret_cast<float*>(ws + NP.zrec_off) : nullptr;
  p.dlog = P.num_chunks > 0 ? reinterpret_cast<float*>(ws + NP.dlog_off) : nullptr;
  hipError_t e = sgla::launch_chunk_normalizer(p, stream);
  if (e != hipSuccess) return hip_fail(e, "launching the normalizer kernel");
  return ok();
}

sgla_status sgla_recurrent_step_normalizer(int32_t N, int32_t H, int32_t num_kv_heads, int32_t K, float scale,
                                           int32_t qkv_dtype, const void* q, const void* k, const float* g,
                                           const float* g_gamma, float* z, float* den, hipStream_t stream) {
  if (N < 0 || H <= 0) return fail(SGLA_ERR_SHAPE, "N must be >= 0 and H > 0 (got N=%d H=%d)", N, H);
  const int32_t Hkv = num_kv_heads == 0 ? H : num_kv_heads;
  if (Hkv < 0 || H % Hkv != 0)
    return fail(SGLA_ERR_SHAPE, "num_kv_heads must divide H (got num_kv_heads=%d, H=%d)", num_kv_heads, H);
  if ((int64_t)N * H > INT32_MAX) return fail(SGLA_ERR_UNSUPPORTED, "N*H exceeds 2^31-1");
  if (K < 1 || K > 4096) return fail(SGLA_ERR_UNSUPPORTED, "the normalizer step supports 1 <= K <= 4096 (got %d)", K);
  if (qkv_dtype != SGLA_BF16 && qkv_dtype != SGLA_F32)
    return fail(SGLA_ERR_DTYPE, "qkv_dtype must be SGLA_BF16 or SGLA_F32 (got %d)", qkv_dtype);
  if (!std::isfinite(scale)) return fail(SGLA_ERR_INVALID_ARG, "scale must be finite");
  if (g != nullptr && g_gamma != nullptr)
    return fail(SGLA_ERR_INVALID_ARG, "g and g_gamma are mutually exclusive; pass at most one");
  if (N == 0) return ok();
  if (q == nullptr || k == nullptr || z == nullptr || den == nullptr)
    return fail(SGLA_ERR_INVALID_ARG, "q, k, z and den must be non-NULL");
  sgla::StepNormalizerParams p;
  p.q = q;
  p.k = k;
  p.g = g;
  p.g_gamma = g_gamma;
  p.z = z;
  p.den = den;
  p.scale = scale;
  p.N = N;
  p.H = H;
  p.Hkv = Hkv;
  p.K = K;
  p.qkv_bf16 = qkv_dtype == SGLA_BF16;
  hipError_t e = sgla::launch_step_normalizer(p, stream);
  if (e != hipSuccess) return hip_fail(e, "launching the normalizer step kernel");
  return ok();
}

sgla_status sgla_chunk_local_cumsum(const sgla_chunk_args* args, const float* g, const int64_t* cu_seqlens_host,
                                    float* gc, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  Plan P;
  sgla_status st = plan_shape(args, cu_seqlens_host, false, &P);
  if (st != SGLA_OK) return st;
  if (P.total_tokens > 0 && (g == nullptr || gc == nullptr))
    return fail(SGLA_ERR_INVALID_ARG, "g and gc must be non-NULL");
  if (P.packed && (workspace == nullptr || workspace_bytes < P.total_bytes))
    return fail(SGLA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", P.total_bytes, workspace_bytes);
  char* ws = static_cast<char*>(workspace);
  st = upload_tables(P, ws, stream);
  if (st != SGLA_OK) return st;
  const sgla::SeqLayout L = layout_of(args, P, ws);
  hipError_t e = sgla::launch_gate_cumsum(g, gc, args->H, L, P.chunk_size, stream);
  if (e != hipSuccess) return hip_fail(e, "launching the gate cumsum kernel");
  return ok();
}

sgla_status sgla_recurrent_step(int32_t N, int32_t H, int32_t num_kv_heads, int32_t K, int32_t V, float scale,
                                int32_t qkv_dtype, int32_t o_dtype, int32_t state_v_first,
                                const void* q, const void* k, const void* v,
                                const float* g, const float* g_gamma, float* state, void* o,
                                hipStream_t stream) {
  if (N < 0 || H <= 0) return fail(SGLA_ERR_SHAPE, "N must be >= 0 and H > 0 (got N=%d H=%d)", N, H);
  const int32_t Hkv = num_kv_heads == 0 ? H : num_kv_heads;
  if (Hkv < 0 || H % Hkv != 0)
    return fail(SGLA_ERR_SHAPE, "num_kv_heads must divide H (got num_kv_heads=%d, H=%d)", num_kv_heads, H);
  if ((int64_t)N * H > INT32_MAX)
    return fail(SGLA_ERR_UNSUPPORTED, "N*H = %lld exceeds 2^31-1", (long long)N * H);
  if (state_v_first) {
    if (!(K == 32 || K == 64 || K == 128 || K == 256 || K == 512))
      return fail(SGLA_ERR_UNSUPPORTED, "decode with the [V, K] state supports K in {32,64,128,256,512} (got %d)", K);
    if (V < 32 || V > 1024 || V % 32 != 0)
      return fail(SGLA_ERR_UNSUPPORTED, "decode with the [V, K] state supports V a multiple of 32 in [32, 1024] (got %d)", V);
  } else {
    if (K < 1 || K > 1024) return fail(SGLA_ERR_UNSUPPORTED, "decode supports 1 <= K <= 1024 (got %d)", K);
    if (!(V == 32 || V == 64 || V == 128 || V == 256 || V == 512))
      return fail(SGLA_ERR_UNSUPPORTED, "decode supports V in {32,64,128,256,512} (got %d)", V);
  }
  if (qkv_dtype != SGLA_BF16 && qkv_dtype != SGLA_F32)
    return fail(SGLA_ERR_DTYPE, "qkv_dtype must be SGLA_BF16 or SGLA_F32 (got %d)", qkv_dtype);
  if (o_dtype != SGLA_BF16 && o_dtype != SGLA_F32)
    return fail(SGLA_ERR_DTYPE, "o_dtype must be SGLA_BF16 or SGLA_F32 (got %d)", o_dtype);
  if (!std::isfinite(scale)) return fail(SGLA_ERR_INVALID_ARG, "scale must be finite");
  if (g != nullptr && g_gamma != nullptr)
    return fail(SGLA_ERR_INVALID_ARG, "g and g_gamma are mutually exclusive; pass at most one");
  if (N == 0) return ok();
  if (q == nullptr || k == nullptr || v == nullptr || state == nullptr || o == nullptr)
    return fail(SGLA_ERR_INVALID_ARG, "q, k, v, state and o must be non-NULL");
  if (!aligned(state, 16)) return fail(SGLA_ERR_INVALID_ARG, "state must be 16-byte aligned");
  const size_t osz = (size_t)N * H * V * (o_dtype == SGLA_BF16 ? 2 : 4);
  const size_t ssz = (size_t)N * H * K * V * sizeof(float);
  const char* oc = static_cast<const char*>(o);
  const char* sc = reinterpret_cast<const char*>(state);
  if (oc < sc + ssz && sc < oc + osz) return fail(SGLA_ERR_INVALID_ARG, "o must not alias the state");
  sgla::StepParams p;
  p.q = q;
  p.k = k;
  p.v = v;
  p.g = g;
  p.g_gamma = g_gamma;
  p.state = state;
  p.o = o;
  p.scale = scale;
  p.N = N;
  p.H = H;
  p.Hkv = Hkv;
  p.state_v_first = state_v_first != 0;
  p.K = K;
  p.V = V;
  p.qkv_bf16 = qkv_dtype == SGLA_BF16;
  p.o_bf16 = o_dtype == SGLA_BF16;
  hipError_t e = sgla::launch_recurrent_step(p, stream);
  if (e != hipSuccess) return hip_fail(e, "launching the decode kernel");
  return ok();
}

sgla_status sgla_parallel_fwd(const sgla_chunk_args* args, const void* q, const void* k, const void* v,
                              const float* g, const float* g_gamma, void* o, float* attn, hipStream_t stream) {
  if (args == nullptr) return fail(SGLA_ERR_INVALID_ARG, "args is NULL");
  const sgla_chunk_args& a = *args;
  if (a.B < 0 || a.T < 0) return fail(SGLA_ERR_SHAPE, "B and T must be >= 0 (got B=%d T=%d)", a.B, a.T);
  if (a.H <= 0) return fail(SGLA_ERR_SHAPE, "H must be > 0 (got %d)", a.H);
  const int32_t Hkv = a.num_kv_heads == 0 ? a.H : a.num_kv_heads;
  if (Hkv < 0 || a.H % Hkv != 0)
    return fail(SGLA_ERR_SHAPE, "num_kv_heads must divide H (got num_kv_heads=%d, H=%d)", a.num_kv_heads, a.H);
  if (a.K <= 0 || a.V <= 0) return fail(SGLA_ERR_SHAPE, "K and V must be > 0");
  if (a.qkv_dtype != SGLA_BF16 && a.qkv_dtype != SGLA_F32)
    return fail(SGLA_ERR_DTYPE, "qkv_dtype must be SGLA_BF16 or SGLA_F32 (got %d)", a.qkv_dtype);
  if (a.o_dtype != SGLA_BF16 && a.o_dtype != SGLA_F32)
    return fail(SGLA_ERR_DTYPE, "o_dtype must be SGLA_BF16 or SGLA_F32 (got %d)", a.o_dtype);
  const bool f32 = a.qkv_dtype == SGLA_F32;
  if (!f32 && !sgla::parallel_supported(a.K, a.V))
    return fail(SGLA_ERR_UNSUPPORTED,
                "the parallel form supports K in {64,128,256} and V a multiple of 16 in [16, 256] for bf16 "
                "inputs (got K=%d V=%d)",
                a.K, a.V);
  if (f32 && !sgla::parallel_f32_supported(a.K, a.V))
    return fail(SGLA_ERR_UNSUPPORTED,
                "the parallel form supports K and V multiples of 16 in [16, 256] for float32 inputs "
                "(got K=%d V=%d)",
                a.K, a.V);
  if (!std::isfinite(a.scale)) return fail(SGLA_ERR_INVALID_ARG, "scale must be finite");
  if (g != nullptr && g_gamma != nullptr)
    return fail(SGLA_ERR_INVALID_ARG, "g and g_gamma are mutually exclusive; pass at most one");
  if ((int64_t)a.B * a.T > INT32_MAX)
    return fail(SGLA_ERR_UNSUPPORTED, "B*T = %lld tokens exceeds 2^31-1", (long long)a.B * a.T);
  // one batch row of k or v (plus a tile of slack) is addressed with 32-bit byte offsets
  if (!f32 && ((int64_t)a.T + sgla::kChunk) * Hkv * std::max(a.K, a.V) * 2 > INT32_MAX)
    return fail(SGLA_ERR_UNSUPPORTED, "T x num_kv_heads x max(K, V) too large for the parallel form (T=%d)", a.T);
  // the rows of A one workgroup writes are addressed with 32-bit byte offsets
  // (128 rows of T floats); T beyond that would need petabytes of A anyway
  if (attn != nullptr && a.T > (1 << 22))
    return fail(SGLA_ERR_UNSUPPORTED, "writing A supports T <= 4194304 (got T=%d)", a.T);
  if (a.B == 0 || a.T == 0) return ok();
  const int32_t nT = (a.T + sgla::kChunk - 1) / sgla::kChunk;
  if (sgla::unit_grid(a.B, Hkv, a.H / Hkv, nT) > INT32_MAX)
    return fail(SGLA_ERR_UNSUPPORTED, "B x H x %d row tiles exceeds 2^31-1 workgroups", nT);
  if (q == nullptr || k == nullptr || v == nullptr || o == nullptr)
    return fail(SGLA_ERR_INVALID_ARG, "q, k, v and o must be non-NULL");
  if (!(aligned(q, 16) && aligned(k, 16) && aligned(v, 16) && aligned(o, 16)))
    return fail(SGLA_ERR_INVALID_ARG, "q, k, v and o must be 16-byte aligned");
  if (attn != nullptr && !aligned(attn, 16)) return fail(SGLA_ERR_INVALID_ARG, "attn must be 16-byte aligned");
  sgla::ParallelParams p;
  p.q = q;
  p.k = k;
  p.v = v;
  p.g = g;
  p.g_gamma = g_gamma;
  p.o = o;
  p.attn = attn;
  p.scale = a.scale;
  p.B = a.B;
  p.T = a.T;
  p.H = a.H;
  p.Hkv = Hkv;
  p.K = a.K;
  p.V = a.V;
  p.o_f32 = a.o_dtype == SGLA_F32;
  hipError_t e = f32 ? sgla::launch_parallel_fwd_f32(p, stream) : sgla::launch_parallel_fwd(p, stream);
  if (e != hipSuccess) return hip_fail(e, "launching the parallel-form kernel");
  return ok();
}

}  // extern "C"
