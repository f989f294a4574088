// Decode without a workspace argument: the layer call's scratch lives in a
// file-scope device array, one per GPU, whose address is looked up once per
// device.  Nothing here allocates.
#include <mutex>

#include "internal.h"

namespace asr {

namespace {

constexpr size_t kScratchBytes = ASR_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

// The scratch.  In host code this name is only a stand-in for the symbol: host
// code passes the per-device address obtained from hipGetSymbolAddress.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

struct DeviceScratch {
  void *ptr = nullptr;
  bool cleared = false;
};
DeviceScratch g_scratch[kMaxDevices];
std::mutex g_mutex;

// counters of the workspace layout (one-dispatch counters and the per-(row, kv
// head) merge counters) start at zero; every call leaves them at zero again
__global__ void k_zero_words(uint32_t *p, uint32_t n) {
  for (uint32_t i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0u;
}

// the current device's scratch address; on the first call on a device also
// enqueue the clearing of its counters (a kernel, not a memset node, so the
// call stays safe to capture)
int device_scratch(hipStream_t stream, size_t counter_bytes, void **out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return ASR_EHIP;
  std::lock_guard<std::mutex> lock(g_mutex);
  DeviceScratch &d = g_scratch[dev];
  if (!d.ptr) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return ASR_EHIP;
    d.ptr = p;
  }
  if (!d.cleared) {
    const uint32_t words = (uint32_t)(counter_bytes / sizeof(uint32_t));
    hipLaunchKernelGGL(k_zero_words, dim3((words + 255) / 256), dim3(256), 0, stream, static_cast<uint32_t *>(d.ptr),
                       words);
    if (hipGetLastError() != hipSuccess) return ASR_EHIP;
    d.cleared = true;
  }
  *out = d.ptr;
  return ASR_OK;
}

}  // namespace

}  // namespace asr

using namespace asr;

extern "C" int asr_attn_layer_decode_noalloc(const asr_attn_config *cfg, const asr_attn_weights *w,
                                             const asr_kv_layer *kv, const void *x, const int32_t *slots,
                                             const int32_t *positions, int32_t B, const int32_t *host_lens,
                                             const void *residual, void *out, hipStream_t stream) {
  if (!cfg || !kv) return ASR_EINVAL;
  if (B < 0) return ASR_EINVAL;
  if (B == 0) return ASR_OK;
  const size_t need = asr_attn_workspace_bytes(cfg, B, kv->capacity);
  // an invalid config or capacity: run_layer reports why before it touches a workspace
  if (need == 0) return run_layer(cfg, w, kv, x, slots, positions, B, 1, host_lens, residual, out, nullptr, 0, stream);
  if (need > kScratchBytes) return ASR_ESCRATCH;
  // the counters come first in every layout, at offsets fixed for all shapes
  const WorkspaceLayout lay = workspace_layout(B, cfg->hidden, cfg->n_q_heads, cfg->n_kv_heads, kv->capacity);
  void *ws = nullptr;
  const int rc = device_scratch(stream, lay.rowtab, &ws);
  if (rc) return rc;
  return run_layer(cfg, w, kv, x, slots, positions, B, 1, host_lens, residual, out, ws, kScratchBytes, stream);
}
