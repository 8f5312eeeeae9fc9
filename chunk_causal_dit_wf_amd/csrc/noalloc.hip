// Allocation-free attention entry point: wf_chunk_attn_fwd with the split
// schedule's partial-result workspace taken from a file-scope device array
// instead of a caller buffer, for callers that cannot allocate device memory
// (code under graph capture, tight serving loops).
//
// The array lives in the library's code object: every GPU the library runs on
// holds one copy of WF_NOALLOC_SCRATCH_BYTES until the process ends.  Its
// device address differs per GPU and is taken once per device with
// hipGetSymbolAddress, with that device current; host code never uses the
// array's name as an address.  Every call on one GPU shares that GPU's array:
// calls that overlap on one GPU (different streams, or different host threads)
// race.  The attention kernels write every partial-result slot the merge
// kernel reads before it runs, so nothing has to start at zero.
#include <mutex>

#include "wf_internal.h"

namespace {

static_assert(WF_NOALLOC_SCRATCH_BYTES % 256 == 0, "scratch size must keep slots aligned");
__device__ __align__(256) unsigned char scratch[WF_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices];  // device address of `scratch` on each device (null until first use)

// Device address of the scratch array on the current device.
wf_status scratch_ptr(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return wf::set_error(WF_ERR_HIP, "hipGetDevice failed");
  if (dev < 0 || dev >= kMaxDevices) return wf::set_error(WF_ERR_UNSUPPORTED, "device index beyond 64");
  std::lock_guard<std::mutex> lk(g_mu);
  if (g_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return wf::set_error(WF_ERR_HIP, "hipGetSymbolAddress of the scratch array failed");
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return WF_OK;
}

}  // namespace

extern "C" wf_status wf_chunk_attn_fwd_noalloc(const wf_kv_cache* c, const void* q, int32_t q_dtype, void* o,
                                               float* lse, int32_t num_chunks, const int32_t* q_off,
                                               const int64_t* kv_begin, const int64_t* kv_end,
                                               float softmax_scale, void* stream) {
  void* ws = nullptr;
  wf_status s = scratch_ptr(&ws);
  if (s != WF_OK) return s;
  return wf::attn_fwd_impl(c, q, q_dtype, o, lse, num_chunks, q_off, kv_begin, kv_end, softmax_scale, ws,
                           WF_NOALLOC_SCRATCH_BYTES, true, stream);
}
