// noalloc.hip -- ttv_tree_attn_noalloc: ttv_tree_attn(_tuned) for callers that cannot
// allocate (code under HIP graph capture, tight serving loops, harnesses that
// forbid allocation).  The split-KV partials live in a file-scope device
// array instead of a caller's workspace; everything else is ttv_tree_attn's
// own host validation, launch plan and kernels.
#include <hip/hip_runtime.h>

#include <mutex>

#include "launch.h"
#include "ttv.h"

namespace ttv {
namespace {

static_assert(TTV_NOALLOC_SCRATCH_BYTES % 256 == 0, "scratch size");

// Each GPU the library runs on holds its own copy of this array until the
// process ends.  In host code `scratch` is only a host-side stand-in for the
// symbol: its device address comes from hipGetSymbolAddress, per device.
__device__ __align__(256) unsigned char scratch[TTV_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` per device (set once)

// The current device's copy of `scratch`, looked up on the first call made
// on that device (with it current) and kept.
hipError_t scratch_of_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace
}  // namespace ttv

extern "C" ttv_status ttv_tree_attn_noalloc(ttv_dtype dt, int32_t B, int32_t N, int32_t Hq,
                                            int32_t Hkv, int32_t D, float scale, const void* q,
                                            const void* k_cache, const void* v_cache,
                                            int32_t Lcap, const int32_t* cache_len,
                                            int32_t Lmax, const void* k_tree, const void* v_tree,
                                            const int32_t* parents, void* out, float* lse,
                                            uint64_t* anc_out, int32_t* depth_out,
                                            int32_t* dev_status, int32_t rows_per_block,
                                            int32_t chunk_keys, void* stream) {
  using namespace ttv;
  AttnPlan p;
  const ttv_status st = attn_prepare(dt, B, N, Hq, Hkv, D, scale, q, k_cache, v_cache, Lcap,
                                     cache_len, Lmax, k_tree, v_tree, parents, out,
                                     rows_per_block, chunk_keys, &p);
  if (st != TTV_OK) return st;
  if (p.ws_bytes > (size_t)TTV_NOALLOC_SCRATCH_BYTES) return TTV_E_SCRATCH;
  void* ws = nullptr;
  if (p.ws_bytes > 0 && scratch_of_current_device(&ws) != hipSuccess) return TTV_E_LAUNCH;
  // the partials need no initialisation: every one a combine reads was written
  // by this call's attention kernel
  return launch_attn(p, dt, B, N, Hq, Hkv, D, scale, q, k_cache, v_cache, Lcap, cache_len, Lmax,
                     k_tree, v_tree, parents, nullptr, out, lse, anc_out, depth_out, dev_status, ws,
                     static_cast<hipStream_t>(stream));
}
