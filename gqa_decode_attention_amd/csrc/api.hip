// C ABI of the attention-block library: validation, workspace layout,
// launch geometry.  Never allocates, never synchronises, never reads device
// memory back.
#include <math.h>
#include <stddef.h>
#include <stdlib.h>

#include "internal.h"

namespace asr {

namespace {

constexpr int kMaxRows = kMaxLayerRows;
constexpr int kMinShare = 64;    // least keys per wave share of the many-row attention
constexpr int kVectorRows = 4;   // up to this many rows the projections run as vector-ALU GEMVs
constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

int check_cfg(const asr_attn_config *c) {
  if (!c) return ASR_EINVAL;
  if (c->hidden <= 0 || c->n_q_heads <= 0 || c->n_kv_heads <= 0 || c->head_dim <= 0) return ASR_EINVAL;
  if (c->head_dim != kHeadDim) return ASR_EUNSUPPORTED;
  if (c->n_q_heads % c->n_kv_heads != 0) return ASR_EINVAL;
  const int group = c->n_q_heads / c->n_kv_heads;
  if (group != 1 && group != 2 && group != 4 && group != 8) return ASR_EUNSUPPORTED;
  if (c->hidden % 512 != 0 || c->hidden > 4096) return ASR_EUNSUPPORTED;
  const int qw = c->n_q_heads * kHeadDim;
  if (qw % 512 != 0 || qw > 4096) return ASR_EUNSUPPORTED;
  if (c->dtype != ASR_F16 && c->dtype != ASR_BF16) return ASR_EUNSUPPORTED;
  if (c->out_dtype != ASR_F32 && c->out_dtype != c->dtype) return ASR_EUNSUPPORTED;
  if (!(c->rms_eps >= 0.f) || !isfinite(c->rms_eps)) return ASR_EINVAL;
  if (!(c->rope_theta > 0.f) || !isfinite(c->rope_theta)) return ASR_EINVAL;
  if (c->kv_split != 0 && (c->kv_split % 16 != 0 || c->kv_split < kMinSplit || c->kv_split > kMaxSplit))
    return ASR_EINVAL;
  if (c->dispatch < ASR_DISPATCH_AUTO || c->dispatch > ASR_DISPATCH_FUSED) return ASR_EINVAL;
  return ASR_OK;
}

int check_kv(const asr_kv_layer *kv, const asr_attn_config *c) {
  if (!kv || !kv->k || !kv->v || !kv->lens) return ASR_EINVAL;
  if (kv->batch_cap <= 0 || kv->capacity <= 0) return ASR_EINVAL;
  if (kv->head_dim != kHeadDim) return ASR_EUNSUPPORTED;
  if (kv->dtype != ASR_F16 && kv->dtype != ASR_BF16) return ASR_EUNSUPPORTED;
  if (kv->n_kv_heads <= 0) return ASR_EINVAL;
  if (kv->capacity > kMaxChunks * kMaxSplit) return ASR_EUNSUPPORTED;
  if (c) {
    if (kv->n_kv_heads != c->n_kv_heads || kv->dtype != c->dtype) return ASR_EINVAL;
  }
  return ASR_OK;
}

// Workgroups per CU of the fused dispatch (a tuning knob; 1 by default).
int fused_blocks_per_cu() {
  const char *v = getenv("ASR_ATTN_FUSED_BLOCKS_PER_CU");
  const int n = v ? atoi(v) : 1;
  return n >= 1 && n <= 8 ? n : 1;
}

int device_cus() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    return 256;
  return cus;
}

// Smallest power-of-two chunk (>= the capacity-derived minimum) whose item
// count stays within a few items per CU.
int choose_split(const asr_attn_config *c, int capacity, int B, int n, const int32_t *host_lens, int cus) {
  int min_split = (capacity + kMaxChunks - 1) / kMaxChunks;
  min_split = (min_split + 15) / 16 * 16;
  if (min_split < kMinSplit) min_split = kMinSplit;
  if (c->kv_split) return c->kv_split;
  int split = kMinSplit;
  while (split < min_split) split *= 2;
  if ((long long)B * n <= kVectorRows) {
    // few rows: every o_proj workgroup merges all chunks of a row, so keep about
    // 8 chunks per row, and chunks of at least 64 keys (one step per wave)
    int nvis = 1;
    for (int b = 0; b < B; ++b) {
      const int L = host_lens ? host_lens[b] : capacity - n;
      if (L + n > nvis) nvis = L + n;
    }
    if (split < 64) split = 64;
    while (split < kMaxSplit && 8LL * split < nvis) split *= 2;
    return split;
  }
  // many rows: several items per CU amortise each item's fixed cost
  const long long target = 4LL * cus;
  for (; split < kMaxSplit; split *= 2) {
    long long items = 0;
    for (int b = 0; b < B; ++b) {
      const int L = host_lens ? host_lens[b] : capacity - n;
      for (int r = 0; r < n; ++r) items += (L + r + 1 + split - 1) / split;
    }
    items *= c->n_kv_heads;
    if (items <= target) break;
  }
  return split < kMaxSplit ? split : kMaxSplit;
}

int run_layer(const asr_attn_config *cfg, const asr_attn_weights *w, const asr_kv_layer *kv,
              const void *x, const int32_t *slots, const int32_t *positions, int B, int n,
              const int32_t *host_lens, const void *residual, void *out, void *ws, size_t ws_bytes,
              hipStream_t stream) {
  int rc = check_cfg(cfg);
  if (rc) return rc;
  if ((rc = check_kv(kv, cfg))) return rc;
  if (B < 0 || n < 1 || n > kMaxVerifyK) return ASR_EINVAL;
  if (B == 0) return ASR_OK;
  if (!w || !w->input_norm_w || !w->w_qkv || !w->q_norm_w || !w->k_norm_w || !w->w_o) return ASR_EINVAL;
  if (!x || !out) return ASR_EINVAL;
  if (!slots && B > kv->batch_cap) return ASR_EINVAL;
  if ((long long)B * n > kMaxRows) return ASR_EINVAL;
  const int rows = B * n;
  if (cfg->kv_split && (kv->capacity + cfg->kv_split - 1) / cfg->kv_split > kMaxChunks) return ASR_EINVAL;
  const WorkspaceLayout lay = workspace_layout(rows, cfg->hidden, cfg->n_q_heads, cfg->n_kv_heads, kv->capacity);
  if (!ws || ws_bytes < lay.total) return ASR_EWORKSPACE;
  if (host_lens) {
    for (int b = 0; b < B; ++b)
      if (host_lens[b] < 0 || (long long)host_lens[b] + n > kv->capacity) return ASR_ECAPACITY;
  }

  const int cus = device_cus();
  LayerArgs a;
  a.x = static_cast<const uint16_t *>(x);
  a.residual = static_cast<const uint16_t *>(residual);
  a.g_in = static_cast<const uint16_t *>(w->input_norm_w);
  a.w_qkv = static_cast<const uint16_t *>(w->w_qkv);
  a.g_q = static_cast<const uint16_t *>(w->q_norm_w);
  a.g_k = static_cast<const uint16_t *>(w->k_norm_w);
  a.w_o = static_cast<const uint16_t *>(w->w_o);
  a.slots = slots;
  a.positions = positions;
  a.kc = static_cast<uint16_t *>(kv->k);
  a.vc = static_cast<uint16_t *>(kv->v);
  a.lens = kv->lens;
  a.status = kv->status;
  a.out = out;
  char *base = static_cast<char *>(ws);
  a.qkv = reinterpret_cast<float *>(base + lay.qkv);
  a.ssq = reinterpret_cast<float *>(base + lay.ssq);
  a.att = reinterpret_cast<float *>(base + lay.att);
  a.att_hl = reinterpret_cast<uint16_t *>(base + lay.att_hl);
  a.part = reinterpret_cast<float *>(base + lay.part);
  a.flow = reinterpret_cast<uint32_t *>(base + lay.flow);
  a.mctr = reinterpret_cast<uint32_t *>(base + lay.mctr);
  a.rowtab = reinterpret_cast<int4 *>(base + lay.rowtab);
  a.B = B;
  a.n = n;
  a.rows = rows;
  a.H = cfg->hidden;
  a.nq = cfg->n_q_heads;
  a.nkv = cfg->n_kv_heads;
  a.group = cfg->n_q_heads / cfg->n_kv_heads;
  a.nqkv = (cfg->n_q_heads + 2 * cfg->n_kv_heads) * kHeadDim;
  a.batch_cap = kv->batch_cap;
  a.capacity = kv->capacity;
  a.split = choose_split(cfg, kv->capacity, B, n, host_lens, cus);
  a.eps = cfg->rms_eps;
  a.theta = cfg->rope_theta;
  a.out_f32 = cfg->out_dtype == ASR_F32;
  a.mfma = rows > kVectorRows;
  a.oproj_split = 0;

  // upper bound of attention work items; blocks stride over the real count.
  // nch_host: the most chunks of any row, by the host's view of the lengths
  long long bound = 0;
  a.nch_host = 1;
  for (int b = 0; b < B; ++b) {
    const int L = host_lens ? host_lens[b] : kv->capacity - n;
    for (int r = 0; r < n; ++r) {
      const int c = (L + r + 1 + a.split - 1) / a.split;
      bound += c;
      if (c > a.nch_host) a.nch_host = c;
    }
  }
  bound *= a.nkv;
  const long long cap_grid = 16LL * cus;
  int attn_grid = (int)(bound < 1 ? 1 : (bound > cap_grid ? cap_grid : bound));
  if (attn_waves_used(a)) {
    // many rows: one equal key share per wave of a resident grid; a (row, kv
    // head) spans at most capacity / share + 2 <= kMaxChunks shares
    attn_grid = attn_waves_grid(cfg->dtype, a.group, cus);
    if (attn_grid <= 0) return ASR_EHIP;
    int share = cfg->kv_split ? cfg->kv_split : kMinShare;
    const int least = (kv->capacity + kMaxChunks - 2) / (kMaxChunks - 1);
    a.split = share > least ? share : least;
  }

  bool fused = false;
  int fused_grid = 0;
  if (cfg->dispatch == ASR_DISPATCH_FUSED && rows <= kVectorRows && layer_fused_supported(a)) {
    fused_grid = fused_max_grid(cfg->dtype, a.H, layer_dyn_smem(a), cus);
    const long long want = (long long)cus * fused_blocks_per_cu();
    if (fused_grid > want) fused_grid = (int)want;
    fused = fused_grid > 0;
  }
  if (cfg->dispatch == ASR_DISPATCH_FUSED && !fused) return ASR_EUNSUPPORTED;
  // few rows with an fp32 output: o_proj in two head halves, each workgroup
  // reading half the chunk partials (the projection kernel zeroes the output)
  if (!fused && !a.mfma && a.out_f32 && a.nq % 8 == 0 && a.H % 64 == 0) a.oproj_split = 1;
  hipEvent_t *ev = cfg->phase_events;
  hipError_t e;
  if (fused) {
    e = launch_layer_fused(a, cfg->dtype, fused_grid, stream, ev);
  } else {
    e = launch_layer_multi(a, cfg->dtype, attn_grid, stream, ev);
  }
  return e == hipSuccess ? ASR_OK : ASR_EHIP;
}

}  // namespace

WorkspaceLayout workspace_layout(int rows, int H, int nq, int nkv, int capacity) {
  (void)H;
  (void)capacity;
  WorkspaceLayout l;
  const size_t nqkv = (size_t)(nq + 2 * nkv) * kHeadDim;
  size_t off = 0;
  l.flow = off;
  off = align_up(off + kFlowWords * sizeof(uint32_t));
  l.mctr = off;
  off = align_up(off + (size_t)rows * nkv * sizeof(uint32_t));
  l.rowtab = off;
  off = align_up(off + (size_t)rows * 4 * sizeof(int));
  l.qkv = off;
  off = align_up(off + (size_t)rows * nqkv * sizeof(float));
  l.ssq = off;
  off = align_up(off + (size_t)rows * (nq + nkv) * 8 * sizeof(float));
  l.att = off;
  off = align_up(off + (size_t)rows * nq * kHeadDim * sizeof(float));
  l.att_hl = off;
  off = align_up(off + (size_t)rows * 2 * nq * kHeadDim * sizeof(uint16_t));
  l.part = off;
  off = align_up(off + (size_t)rows * nq * kMaxChunks * kPartStride * sizeof(float));
  l.total = off;
  return l;
}

}  // namespace asr

using namespace asr;

extern "C" {

size_t asr_attn_workspace_bytes(const asr_attn_config *cfg, int32_t max_rows, int32_t capacity) {
  if (check_cfg(cfg) != ASR_OK || max_rows < 0 || max_rows > kMaxRows || capacity <= 0) return 0;
  if (capacity > kMaxChunks * kMaxSplit) return 0;
  return workspace_layout(max_rows, cfg->hidden, cfg->n_q_heads, cfg->n_kv_heads, capacity).total;
}

int asr_attn_layer_decode(const asr_attn_config *cfg, const asr_attn_weights *w, const asr_kv_layer *kv,
                          const void *x, const int32_t *slots, const int32_t *positions, int32_t B,
                          const int32_t *host_lens, const void *residual, void *out, void *workspace,
                          size_t ws_bytes, hipStream_t stream) {
  return run_layer(cfg, w, kv, x, slots, positions, B, 1, host_lens, residual, out, workspace, ws_bytes,
                   stream);
}

int asr_attn_layer_verify(const asr_attn_config *cfg, const asr_attn_weights *w, const asr_kv_layer *kv,
                          const void *x, const int32_t *slots, const int32_t *positions, int32_t B,
                          int32_t k, const int32_t *host_lens, const void *residual, void *out,
                          void *workspace, size_t ws_bytes, hipStream_t stream) {
  if (k < 1 || k > kMaxVerifyK) return ASR_EINVAL;
  return run_layer(cfg, w, kv, x, slots, positions, B, k, host_lens, residual, out, workspace, ws_bytes,
                   stream);
}

int asr_kv_append(const asr_kv_layer *kv, const void *k_new, const void *v_new, const int32_t *slots,
                  int32_t B, int32_t n, hipStream_t stream) {
  int rc = check_kv(kv, nullptr);
  if (rc) return rc;
  if (B < 0 || n < 0) return ASR_EINVAL;
  if (B == 0 || n == 0) return ASR_OK;
  if (!k_new || !v_new) return ASR_EINVAL;
  if (!slots && B > kv->batch_cap) return ASR_EINVAL;
  return launch_kv_append(kv->dtype, *kv, k_new, v_new, slots, B, n, stream) == hipSuccess ? ASR_OK : ASR_EHIP;
}

int asr_kv_crop(const asr_kv_layer *layers, int32_t n_layers, const int32_t *new_lens, hipStream_t stream) {
  if (n_layers < 0) return ASR_EINVAL;
  if (n_layers == 0) return ASR_OK;
  if (!layers || !new_lens) return ASR_EINVAL;
  for (int i = 0; i < n_layers; ++i) {
    if (!layers[i].lens || layers[i].batch_cap <= 0) return ASR_EINVAL;
    if (layers[i].batch_cap != layers[0].batch_cap) return ASR_EINVAL;
  }
  return launch_kv_crop(layers, n_layers, new_lens, stream) == hipSuccess ? ASR_OK : ASR_EHIP;
}

const char *asr_strerror(int code) {
  switch (code) {
    case ASR_OK: return "ok";
    case ASR_EINVAL: return "invalid argument";
    case ASR_EUNSUPPORTED: return "unsupported shape or type";
    case ASR_ECAPACITY: return "cache capacity exceeded (host lengths)";
    case ASR_EWORKSPACE: return "workspace missing or too small";
    case ASR_EHIP: return "HIP launch failed";
  }
  return "unknown error";
}

}  // extern "C"
