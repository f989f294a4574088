// KV-cache transactions: bit-exact append of given rows, and crop of the
// committed lengths of many layers in one dispatch ("Can CTC make Qwen3-ASR
// faster?", section 03 "Greedy exactness": crop speculative KV state to the
// committed prefix; section 11 Phase D: transactional commit/crop of KV).
#include "device_common.h"
#include "internal.h"

namespace asr {

namespace {

struct AppendArgs {
  const uint4 *k_new, *v_new;  // [B][n][nkv][d] elements of `chunks` x 16 bytes per row (d = 128)
  const int32_t *slots;
  unsigned char *kc, *vc;
  int chunks;                  // 16-byte pieces per row: 16 (16-bit), 8 (E4M3 codes)
  int32_t *lens;
  uint32_t *status;
  int B, n, nkv, batch_cap, capacity;
  const int32_t *ptab;         // paged cache: [batch_cap][pps] page ids of psz rows, or null
  int pps, npages, psz;
};

__device__ __forceinline__ bool append_target(const AppendArgs &a, int b, int &slot, int &L) {
  slot = a.slots ? a.slots[b] : b;
  if (slot < 0 || slot >= a.batch_cap) return false;
  L = a.lens[slot];
  return L >= 0 && L + a.n <= a.capacity;
}

// `chunks` threads copy one row of K and of V (256 bytes of 16-bit elements or
// 128 bytes of E4M3 codes).
__global__ __launch_bounds__(256) void k_append_rows(AppendArgs a) {
  const size_t total_rows = (size_t)a.B * a.n * a.nkv;
  const size_t idx = ((size_t)blockIdx.x * 256 + threadIdx.x) / a.chunks;
  const int part = threadIdx.x % a.chunks;
  if (idx >= total_rows) return;
  const int g = (int)(idx % a.nkv);
  const size_t br = idx / a.nkv;
  const int r = (int)(br % a.n);
  const int b = (int)(br / a.n);
  int slot, L;
  if (!append_target(a, b, slot, L)) return;
  size_t dst_row = ((size_t)slot * a.nkv + g) * a.capacity + L + r;
  if (a.ptab) {
    // position L + r: row (L + r) % psz of its page; a page id outside the pool is not written
    const int t = L + r;
    const int page = a.ptab[(size_t)slot * a.pps + t / a.psz];
    if ((unsigned)page >= (unsigned)a.npages) {
      if (a.status && part == 0) atomicOr(a.status, (uint32_t)ASR_STATUS_BAD_PAGE);
      return;
    }
    dst_row = ((size_t)page * a.nkv + g) * a.psz + t % a.psz;
  }
  const size_t dst = dst_row * (size_t)a.chunks * 16;
  reinterpret_cast<uint4 *>(a.kc + dst)[part] = a.k_new[idx * a.chunks + part];
  reinterpret_cast<uint4 *>(a.vc + dst)[part] = a.v_new[idx * a.chunks + part];
}

// Runs after k_append_rows in stream order, so every row copy has read lens.
__global__ __launch_bounds__(256) void k_append_lens(AppendArgs a) {
  const int b = blockIdx.x * 256 + threadIdx.x;
  if (b >= a.B) return;
  int slot, L;
  if (append_target(a, b, slot, L)) {
    a.lens[slot] = L + a.n;
  } else if (a.status) {
    const bool slot_ok = (a.slots ? a.slots[b] : b) >= 0 && (a.slots ? a.slots[b] : b) < a.batch_cap;
    atomicOr(a.status, slot_ok ? (uint32_t)ASR_STATUS_CAPACITY : kStatusBadSlot);
  }
}

constexpr int kCropLayers = 64;

struct CropArgs {
  int32_t *lens[kCropLayers];
  uint32_t *status[kCropLayers];
  const int32_t *new_lens;
  int batch_cap;
};

__global__ __launch_bounds__(256) void k_crop(CropArgs a) {
  const int b = blockIdx.x * 256 + threadIdx.x;
  const int layer = blockIdx.y;
  if (b >= a.batch_cap) return;
  const int nl = a.new_lens[b];
  int32_t *lens = a.lens[layer];
  if (nl >= 0 && nl <= lens[b]) {
    lens[b] = nl;
  } else if (a.status[layer]) {
    atomicOr(a.status[layer], (uint32_t)ASR_STATUS_CROP_GROW);
  }
}

}  // namespace

hipError_t launch_kv_append(int dtype, const asr_kv_layer &kv, const void *k_new, const void *v_new,
                            const int32_t *slots, int B, int n, hipStream_t s) {
  AppendArgs a;   // a bit-exact copy: only the element size matters
  a.k_new = reinterpret_cast<const uint4 *>(k_new);
  a.v_new = reinterpret_cast<const uint4 *>(v_new);
  a.slots = slots;
  a.kc = reinterpret_cast<unsigned char *>(kv.k);
  a.vc = reinterpret_cast<unsigned char *>(kv.v);
  a.chunks = dtype == ASR_FP8_E4M3 ? 8 : 16;
  a.lens = kv.lens;
  a.status = kv.status;
  a.B = B;
  a.n = n;
  a.nkv = kv.n_kv_heads;
  a.batch_cap = kv.batch_cap;
  a.capacity = kv.capacity;
  a.ptab = kv.block_table;
  a.pps = kv.pages_per_seq;
  a.npages = kv.num_pages;
  a.psz = kv.page_size;
  const size_t rows = (size_t)B * n * kv.n_kv_heads;
  hipLaunchKernelGGL(k_append_rows, dim3((unsigned)((rows * a.chunks + 255) / 256)), dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_append_lens, dim3((B + 255) / 256), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_kv_crop(const asr_kv_layer *layers, int n_layers, const int32_t *new_lens, hipStream_t s) {
  for (int l0 = 0; l0 < n_layers; l0 += kCropLayers) {
    CropArgs a;
    const int nl = n_layers - l0 < kCropLayers ? n_layers - l0 : kCropLayers;
    for (int i = 0; i < kCropLayers; ++i) {
      a.lens[i] = i < nl ? layers[l0 + i].lens : nullptr;
      a.status[i] = i < nl ? layers[l0 + i].status : nullptr;
    }
    a.new_lens = new_lens;
    a.batch_cap = layers[0].batch_cap;
    hipLaunchKernelGGL(k_crop, dim3((a.batch_cap + 255) / 256, nl), dim3(256), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace asr
