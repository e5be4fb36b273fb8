// cb_blend_layer_static: cb_blend_layer for callers that cannot allocate device memory (code
// under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).  The
// workspace is a file-scope device array of kScratchBytes that every device the library runs
// on holds until the process ends; each device's copy sits at its own address, taken once per
// device with hipGetSymbolAddress and used instead of the array's name in host code.
#include <hip/hip_runtime.h>

#include <mutex>

#include "cb_host.h"

namespace {

constexpr size_t kScratchBytes = size_t(128) << 20;
constexpr int kMaxDevices = 64;

__device__ __align__(256) char scratch[kScratchBytes];

std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

// The device address of `device`'s copy of the array, looked up on the first call for that
// device with the device current (the caller's current device is restored).
cb_status scratch_on(int device, void** out) {
  std::lock_guard<std::mutex> lock(g_mu);
  if (device < 0 || device >= kMaxDevices) return cbi_fail(CB_EINVAL, "device %d outside [0, %d)", device, kMaxDevices);
  if (!g_scratch[device]) {
    int cur = 0;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return cbi_fail(CB_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (cur != device && (e = hipSetDevice(device)) != hipSuccess)
      return cbi_fail(CB_EHIP, "hipSetDevice(%d): %s", device, hipGetErrorString(e));
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != device) (void)hipSetDevice(cur);
    if (e != hipSuccess || !p)
      return cbi_fail(CB_EHIP, "hipGetSymbolAddress(scratch) on device %d: %s", device, hipGetErrorString(e));
    g_scratch[device] = p;
  }
  *out = g_scratch[device];
  return CB_OK;
}

}  // namespace

extern "C" cb_status cb_blend_layer_static(cb_ctx* c, int32_t layer, const float* hidden_sel, const void* x_sel,
                                           const void* kv_cached_k, const void* kv_cached_v, void* kv_fused_k,
                                           void* kv_fused_v, const int32_t* chunk_offsets_dev,
                                           const int32_t* chunk_offsets_host, int32_t n_chunks,
                                           const int32_t* sel_idx, int32_t n_sel, int32_t n_query, float ratio,
                                           int32_t* new_sel_idx, int32_t* new_sel_local, int32_t* n_new,
                                           void* out_sel, float* deviation) {
  if (!c) return cbi_fail(CB_EINVAL, "context is NULL");
  void* ws = nullptr;
  cb_status st = scratch_on(cbi_device(c), &ws);
  if (st) return st;
  // the workspace this call needs, when its sizes can be read (otherwise cb_blend_layer reports them)
  if (chunk_offsets_host && n_chunks >= 0 && n_sel >= 0 && n_query >= 0) {
    const long n_tok = (long)chunk_offsets_host[n_chunks] + n_query;
    if (n_tok <= cbi_desc(c)->max_tokens && n_sel <= n_tok) {
      size_t need = 0;
      st = cb_workspace_size(c, (int32_t)n_tok, n_sel, &need);
      if (st) return st;
      if (need > kScratchBytes)
        return cbi_fail(CB_ENOMEM, "cb_blend_layer_static: %d selected rows of a %ld-row prompt need %zu bytes of "
                        "workspace; the static scratch holds %zu (use cb_blend_layer with a workspace)",
                        n_sel, n_tok, need, kScratchBytes);
    }
  }
  return cb_blend_layer(c, layer, hidden_sel, x_sel, kv_cached_k, kv_cached_v, kv_fused_k, kv_fused_v,
                        chunk_offsets_dev, chunk_offsets_host, n_chunks, sel_idx, n_sel, n_query, ratio, new_sel_idx,
                        new_sel_local, n_new, out_sel, deviation, ws, kScratchBytes);
}
