// sgla_chunk_fwd_noalloc: the chunked forward for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid allocation).  The scratch memory sgla_chunk_fwd takes
// as a caller workspace -- the packed-sequence tables and, for bf16 inputs
// with K = 256 or 512, the per-chunk preparation records -- lives instead in
// the fixed device array below, one copy per GPU, held until the process
// ends.  Requests that need more than the array holds are rejected before
// anything is enqueued.
//
// Every call on a GPU uses that GPU's one array: calls that overlap on one
// GPU (on different streams, or from different threads without ordering)
// race on it, and must be serialized by the caller.  Nothing in the array has
// to start at zero -- every byte a call reads was written earlier in the same
// call -- so it is never cleared.
#include <hip/hip_runtime.h>

#include <mutex>

#include "sgla.h"
#include "sgla_internal.h"

namespace {

constexpr size_t kScratchBytes = size_t(16) << 20;   // 16 MiB per GPU
constexpr int kMaxDevices = 64;

// The library's scratch memory.  In host code this name is only a stand-in
// for the symbol: its device address (one per GPU) comes from
// hipGetSymbolAddress and is the only form ever passed to kernels.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

// Device address of the current device's copy of `scratch`, looked up once
// per device with that device current.
sgla_status device_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return sgla::report(SGLA_ERR_HIP, hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return sgla::report(SGLA_ERR_UNSUPPORTED, "device index out of range");
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return sgla::report(SGLA_ERR_HIP, e != hipSuccess ? hipGetErrorString(e) : "no address for the scratch array");
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return SGLA_OK;
}

}  // namespace

extern "C" {

size_t sgla_chunk_fwd_noalloc_max_bytes(void) { return kScratchBytes; }

sgla_status sgla_chunk_fwd_noalloc(const sgla_chunk_args* args, const void* q, const void* k, const void* v,
                                   const float* g, const float* g_gamma, const float* initial_state,
                                   const int64_t* cu_seqlens_host, void* o, float* final_state,
                                   hipStream_t stream) {
  sgla_status st;
  const size_t need = sgla::chunk_fwd_workspace(args, cu_seqlens_host, &st);
  if (st != SGLA_OK) return st;
  if (need > kScratchBytes) {
    char msg[200];
    snprintf(msg, sizeof(msg),
             "this request needs %zu bytes of scratch memory; sgla_chunk_fwd_noalloc holds at most %zu "
             "(use sgla_chunk_fwd with a workspace)",
             need, kScratchBytes);
    return sgla::report(SGLA_ERR_WORKSPACE, msg);
  }
  // the scratch address is looked up only once every argument is valid
  return sgla::chunk_fwd_enqueue(args, q, k, v, g, g_gamma, initial_state, cu_seqlens_host, o, final_state,
                                 nullptr, kScratchBytes, stream, device_scratch);
}

}  // extern "C"
