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
  const int32_t *ms = c->mrope_sections;
  if (ms[0] || ms[1] || ms[2]) {
    if (ms[0] < 0 || ms[1] < 0 || ms[2] < 0 || ms[0] + ms[1] + ms[2] != c->head_dim / 2) return ASR_EINVAL;
  }
  return ASR_OK;
}

int check_kv(const asr_kv_layer *kv, const asr_attn_config *c) {
  if (!kv || !kv->k || !kv->v || !kv->lens) return ASR_EINVAL;
  if (kv->batch_cap <= 0 || kv->capacity <= 0) return ASR_EINVAL;
  if (kv->head_dim != kHeadDim) return ASR_EUNSUPPORTED;
  if (kv->dtype != ASR_F16 && kv->dtype != ASR_BF16 && kv->dtype != ASR_FP8_E4M3) return ASR_EUNSUPPORTED;
  if (kv->dtype == ASR_FP8_E4M3 && (!kv->k_scale || !kv->v_scale)) return ASR_EINVAL;
  if (kv->n_kv_heads <= 0) return ASR_EINVAL;
  if (kv->capacity > kMaxChunks * kMaxSplit) return ASR_EUNSUPPORTED;
  if (kv->block_table) {
    // a paged pool: 16-bit elements, power-of-two pages of 16 .. 1024 rows
    const int P = kv->page_size;
    if (P < 16 || P > 1024 || (P & (P - 1)) != 0) return ASR_EUNSUPPORTED;
    if (kv->pages_per_seq <= 0 || kv->num_pages <= 0) return ASR_EINVAL;
    if ((long long)kv->pages_per_seq * P != kv->capacity) return ASR_EINVAL;
    if (kv->dtype == ASR_FP8_E4M3) return ASR_EUNSUPPORTED;
  }
  if (c) {
    if (kv->n_kv_heads != c->n_kv_heads) return ASR_EINVAL;
    if (kv->dtype != c->dtype && kv->dtype != ASR_FP8_E4M3) return ASR_EINVAL;
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
// Rows of sequence b: n, or its entry of a mixed call's block sizes.
struct SeqRows {
  const int32_t *nb;
  int n;
  int operator()(int b) const { return nb ? nb[b] : n; }
};

int choose_split(const asr_attn_config *c, int capacity, int B, SeqRows n, int rows, const int32_t *host_lens,
                 int cus) {
  int min_split = (capacity + kMaxChunks - 1) / kMaxChunks;
  min_split = (min_split + 15) / 16 * 16;
  if (min_split < kMinSplit) min_split = kMinSplit;
  if (c->kv_split) return c->kv_split;
  int split = kMinSplit;
  while (split < min_split) split *= 2;
  if (rows <= kVectorRows) {
    // few rows: every o_proj workgroup merges all chunks of a row, so keep about
    // 8 chunks per row, and chunks of at least 64 keys (one step per wave)
    int nvis = 1;
    for (int b = 0; b < B; ++b) {
      const int L = host_lens ? host_lens[b] : capacity - n(b);
      if (L + n(b) > nvis) nvis = L + n(b);
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
      const int L = host_lens ? host_lens[b] : capacity - n(b);
      for (int r = 0; r < n(b); ++r) items += (L + r + 1 + split - 1) / split;
    }
    items *= c->n_kv_heads;
    if (items <= target) break;
  }
  return split < kMaxSplit ? split : kMaxSplit;
}

}  // namespace

int run_layer(const asr_attn_config *cfg, const asr_attn_weights *w, const asr_kv_layer *kv,
              const void *x, const int32_t *slots, const int32_t *positions, int B, int n,
              const int32_t *host_lens, const void *residual, void *out, void *ws, size_t ws_bytes,
              hipStream_t stream, const int32_t *n_per_seq) {
  int rc = check_cfg(cfg);
  if (rc) return rc;
  if ((rc = check_kv(kv, cfg))) return rc;
  if (B < 0) return ASR_EINVAL;
  long long total = 0;
  if (n_per_seq) {
    // a mixed call: per-sequence block sizes, the host lays out the rows
    if (B > kVmMaxSeqs) return ASR_EINVAL;
    n = 1;
    bool uniform = true;
    for (int b = 0; b < B; ++b) {
      if (n_per_seq[b] < 1 || n_per_seq[b] > kMaxVerifyK) return ASR_EINVAL;
      total += n_per_seq[b];
      if (n_per_seq[b] > n) n = n_per_seq[b];
      uniform = uniform && n_per_seq[b] == n_per_seq[0];
    }
    if (uniform) n_per_seq = nullptr;   // one block size: the verify (k = 1: decode) call itself
  } else {
    if (n < 1 || n > kMaxVerifyK) return ASR_EINVAL;
    total = (long long)B * n;
  }
  if (B == 0) return ASR_OK;
  const SeqRows nb{n_per_seq, n};
  if (!w || !w->input_norm_w || !w->w_qkv || !w->q_norm_w || !w->k_norm_w || !w->w_o) return ASR_EINVAL;
  if (!x || !out) return ASR_EINVAL;
  if (!slots && B > kv->batch_cap) return ASR_EINVAL;
  if (total > kMaxRows) return ASR_EINVAL;
  const int rows = (int)total;
  if (cfg->kv_split && (kv->capacity + cfg->kv_split - 1) / cfg->kv_split > kMaxChunks) return ASR_EINVAL;
  const WorkspaceLayout lay = workspace_layout(rows, cfg->hidden, cfg->n_q_heads, cfg->n_kv_heads, kv->capacity);
  if (!ws || ws_bytes < lay.total) return ASR_EWORKSPACE;
  if (host_lens) {
    for (int b = 0; b < B; ++b)
      if (host_lens[b] < 0 || (long long)host_lens[b] + nb(b) > kv->capacity) return ASR_ECAPACITY;
  }
  if ((n_per_seq || kv->block_table) && cfg->dispatch == ASR_DISPATCH_FUSED) return ASR_EUNSUPPORTED;
  // mixed blocks run on the many-row kernels (matrix-core projections) whatever the row count

  const bool kv8 = kv->dtype == ASR_FP8_E4M3;
  if (kv8) {
    // FP8 caches: the many-row kernels (matrix-core projections, equal-share attention)
    const int group = cfg->n_q_heads / cfg->n_kv_heads;
    if ((rows <= kVectorRows && !n_per_seq) || (group != 2 && group != 4) || cfg->dispatch == ASR_DISPATCH_FUSED)
      return ASR_EUNSUPPORTED;
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
  a.ptab = kv->block_table;
  a.pps = kv->block_table ? kv->pages_per_seq : 0;
  a.npages = kv->block_table ? kv->num_pages : 0;
  a.psz = kv->block_table ? kv->page_size : 0;
  a.plog = 0;
  while (a.psz > (1 << a.plog)) ++a.plog;
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
  a.split = choose_split(cfg, kv->capacity, B, nb, rows, host_lens, cus);
  a.eps = cfg->rms_eps;
  a.theta = cfg->rope_theta;
  a.out_f32 = cfg->out_dtype == ASR_F32;
  // mixed blocks run on the many-row kernels whatever the row count
  a.mfma = rows > kVectorRows || n_per_seq != nullptr;
  a.oproj_split = 0;
  a.vm_items = 0;
  a.vm_nt = 1;
  a.kv8 = kv8;
  a.ksc = kv->k_scale;
  a.vsc = kv->v_scale;
  a.mrope = (cfg->mrope_sections[0] || cfg->mrope_sections[1] || cfg->mrope_sections[2]) ? 1 : 0;
  a.ms0 = cfg->mrope_sections[0];
  a.ms1 = cfg->mrope_sections[1];
  a.qo_n = n_per_seq ? 1 : 0;
  a.qo[0] = 0;
  if (n_per_seq)
    for (int b = 0; b < B; ++b) a.qo[b + 1] = a.qo[b] + n_per_seq[b];

  // upper bound of attention work items; blocks stride over the real count.
  // nch_host: the most chunks of any row, by the host's view of the lengths
  long long bound = 0;
  a.nch_host = 1;
  for (int b = 0; b < B; ++b) {
    const int L = host_lens ? host_lens[b] : kv->capacity - nb(b);
    for (int r = 0; r < nb(b); ++r) {
      const int c = (L + r + 1 + a.split - 1) / a.split;
      bound += c;
      if (c > a.nch_host) a.nch_host = c;
    }
  }
  bound *= a.nkv;
  const long long cap_grid = 16LL * cus;
  int attn_grid = (int)(bound < 1 ? 1 : (bound > cap_grid ? cap_grid : bound));
  if (attn_vmfma_used(a)) {
    // verify blocks on the matrix cores: items (sequence, kv head, chunk of
    // `split` keys, a multiple of the four waves' 32-key steps); at most
    // kMaxChunks chunks per sequence
    int split = 128;
    while (split < kMaxSplit && (long long)split * kMaxChunks < kv->capacity) split += 128;
    a.vm_nt = attn_vmfma_tiles(a.group, n);   // 16-row query tiles per (sequence, kv head)
    auto items = [&](int sp) {
      long long t = 0;
      for (int b = 0; b < B; ++b) {
        const int L = host_lens ? host_lens[b] : kv->capacity - n;
        t += (L + n + sp - 1) / sp;
      }
      return t * a.nkv * a.vm_nt;
    };
    const int grid = attn_vmfma_grid(cfg->dtype, a.group, n, B, cus);
    if (grid <= 0) return ASR_EHIP;
    if (!cfg->kv_split) {
      // the smallest chunk (in 128-key steps) whose items all fit the resident grid at
      // once: a second round of items would double the kernel's time
      while (split < kMaxSplit && items(split) > grid) split += 128;
    } else {
      split = cfg->kv_split < split ? split : (cfg->kv_split + 127) / 128 * 128;
    }
    a.split = split < kMaxSplit ? split : kMaxSplit;
    const long long want = items(a.split);
    attn_grid = (int)(want < 1 ? 1 : (want < grid ? want : grid));
    if (B <= kVmMaxSeqs) {   // the host lays the items out: the kernel starts without reading the lengths
      int run = 0;
      for (int b = 0; b < B; ++b) {
        a.vm_pre[b] = run;
        const int L = host_lens ? host_lens[b] : kv->capacity - n;
        run += (L + n + a.split - 1) / a.split * a.nkv * a.vm_nt;
      }
      a.vm_pre[B] = run;
      a.vm_items = run;
    }
  } else if (attn_waves_used(a)) {
    // many rows: one equal key share per wave of a resident grid; a (row, kv
    // head) spans at most capacity / share + 2 <= kMaxChunks shares
    attn_grid = attn_waves_grid(cfg->dtype, a.group, cus, n_per_seq != nullptr, kv->block_table != nullptr);
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

WorkspaceLayout workspace_layout(int rows, int H, int nq, int nkv, int capacity) {
  (void)H;
  (void)capacity;
  WorkspaceLayout l;
  const size_t nqkv = (size_t)(nq + 2 * nkv) * kHeadDim;
  size_t off = 0;
  l.flow = off;
  off = align_up(off + kFlowWords * sizeof(uint32_t));
  // the counters sit at the same offsets whatever the call's row count and
  // head count, so a workspace shared by calls of different shapes never finds
  // another call's data where its counters are (every call leaves them at zero)
  l.mctr = off;
  off = align_up(off + (size_t)kMaxRows * kMaxKvHeads * sizeof(uint32_t));
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

namespace asr {
namespace {

int check_mlp(const asr_mlp_config *c) {
  if (!c) return ASR_EINVAL;
  if (c->hidden <= 0 || c->intermediate <= 0) return ASR_EINVAL;
  if (c->hidden % 256 != 0 || c->hidden > 2048) return ASR_EUNSUPPORTED;
  if (c->intermediate % 256 != 0 || c->intermediate > 16384) return ASR_EUNSUPPORTED;
  if (c->dtype != ASR_F16 && c->dtype != ASR_BF16) return ASR_EUNSUPPORTED;
  if (c->in_dtype != ASR_F32 && c->in_dtype != c->dtype) return ASR_EUNSUPPORTED;
  if (c->out_dtype != ASR_F32 && c->out_dtype != c->dtype) return ASR_EUNSUPPORTED;
  if (!(c->rms_eps >= 0.f) || !isfinite(c->rms_eps)) return ASR_EINVAL;
  return ASR_OK;
}

size_t mlp_ws_bytes(const asr_mlp_config *c, int rows) {
  return align_up((size_t)2 * c->hidden * rows * sizeof(uint16_t)) +
         align_up((size_t)2 * c->intermediate * rows * sizeof(uint16_t));
}

int run_mlp(const asr_mlp_config *c, const asr_mlp_weights *w, const void *h, int rows, void *out, void *ws,
            size_t ws_bytes, hipStream_t stream) {
  int rc = check_mlp(c);
  if (rc) return rc;
  if (rows < 0 || rows > kMaxRows) return ASR_EINVAL;
  if (rows == 0) return ASR_OK;
  if (!w || !w->post_norm_w || !w->w_gate || !w->w_up || !w->w_down || !h || !out) return ASR_EINVAL;
  if (!ws || ws_bytes < mlp_ws_bytes(c, rows)) return ASR_EWORKSPACE;
  MlpArgs a;
  a.h = h;
  a.in_f32 = c->in_dtype == ASR_F32;
  a.g_post = static_cast<const uint16_t *>(w->post_norm_w);
  a.w_gate = static_cast<const uint16_t *>(w->w_gate);
  a.w_up = static_cast<const uint16_t *>(w->w_up);
  a.w_down = static_cast<const uint16_t *>(w->w_down);
  a.out = out;
  a.out_f32 = c->out_dtype == ASR_F32;
  a.y_hl = static_cast<uint16_t *>(ws);
  a.a_hl = reinterpret_cast<uint16_t *>(static_cast<char *>(ws) +
                                        align_up((size_t)2 * c->hidden * rows * sizeof(uint16_t)));
  a.rows = rows;
  a.H = c->hidden;
  a.I = c->intermediate;
  a.eps = c->rms_eps;
  return launch_mlp(a, c->dtype, stream, c->phase_events) == hipSuccess ? ASR_OK : ASR_EHIP;
}

// attention workspace, then h [rows][H] fp32, then the MLP's workspace
size_t layer_ws_bytes(const asr_attn_config *acfg, const asr_mlp_config *mcfg, int rows, int capacity) {
  const size_t att = asr_attn_workspace_bytes(acfg, rows, capacity);
  if (!att || check_mlp(mcfg) != ASR_OK || mcfg->hidden != acfg->hidden) return 0;
  return att + align_up((size_t)rows * acfg->hidden * sizeof(float)) + mlp_ws_bytes(mcfg, rows);
}

int run_decoder_layer(const asr_attn_config *acfg, const asr_attn_weights *aw, const asr_mlp_config *mcfg,
                      const asr_mlp_weights *mw, const asr_kv_layer *kv, const void *x, const int32_t *slots,
                      const int32_t *positions, int B, int n, const int32_t *host_lens, void *out, void *ws,
                      size_t ws_bytes, hipStream_t stream, const int32_t *n_per_seq = nullptr) {
  int rc = check_cfg(acfg);
  if (rc) return rc;
  if ((rc = check_mlp(mcfg))) return rc;
  if (mcfg->hidden != acfg->hidden || mcfg->dtype != acfg->dtype || mcfg->in_dtype != ASR_F32) return ASR_EINVAL;
  if (B < 0) return ASR_EINVAL;
  long long total = (long long)B * n;
  if (n_per_seq) {
    if (B > kVmMaxSeqs) return ASR_EINVAL;
    total = 0;
    for (int b = 0; b < B; ++b) {
      if (n_per_seq[b] < 1 || n_per_seq[b] > kMaxVerifyK) return ASR_EINVAL;
      total += n_per_seq[b];
    }
  } else if (n < 1 || n > kMaxVerifyK) {
    return ASR_EINVAL;
  }
  if (total > kMaxRows) return ASR_EINVAL;
  if (B == 0) return ASR_OK;
  if (!kv) return ASR_EINVAL;
  const int rows = (int)total;
  const size_t att = asr_attn_workspace_bytes(acfg, rows, kv->capacity);
  const size_t need = layer_ws_bytes(acfg, mcfg, rows, kv->capacity);
  if (!att || !need) return ASR_EINVAL;
  if (!ws || ws_bytes < need) return ASR_EWORKSPACE;
  asr_attn_config ac = *acfg;
  ac.out_dtype = ASR_F32;
  char *base = static_cast<char *>(ws);
  float *h = reinterpret_cast<float *>(base + att);
  char *mws = base + att + align_up((size_t)rows * acfg->hidden * sizeof(float));
  rc = run_layer(&ac, aw, kv, x, slots, positions, B, n, host_lens, x, h, ws, att, stream, n_per_seq);
  if (rc) return rc;
  return run_mlp(mcfg, mw, h, rows, out, mws, mlp_ws_bytes(mcfg, rows), stream);
}

int check_head(const asr_head_config *c) {
  if (!c) return ASR_EINVAL;
  if (c->hidden <= 0 || c->vocab <= 0) return ASR_EINVAL;
  if (c->hidden % 256 != 0 || c->hidden > 4096 || c->vocab % 16 != 0) return ASR_EUNSUPPORTED;
  if (c->dtype != ASR_F16 && c->dtype != ASR_BF16) return ASR_EUNSUPPORTED;
  if (c->in_dtype != ASR_F32 && c->in_dtype != c->dtype) return ASR_EUNSUPPORTED;
  if (!(c->rms_eps >= 0.f) || !isfinite(c->rms_eps)) return ASR_EINVAL;
  return ASR_OK;
}

int head_parts(const asr_head_config *c) { return (c->vocab + 127) / 128; }

size_t head_ws_bytes(const asr_head_config *c, int rows) {
  return align_up((size_t)2 * c->hidden * rows * sizeof(uint16_t)) +
         2 * align_up((size_t)head_parts(c) * rows * sizeof(float));
}

}  // namespace
}  // namespace asr

using namespace asr;

extern "C" {

int asr_embed(const void *table, int32_t vocab, int32_t hidden, int32_t dtype, const int32_t *ids, int32_t rows,
              void *x, hipStream_t stream) {
  if (rows < 0 || vocab <= 0 || hidden <= 0) return ASR_EINVAL;
  if (rows == 0) return ASR_OK;
  if (!table || !ids || !x) return ASR_EINVAL;
  if (hidden % 8 != 0) return ASR_EUNSUPPORTED;
  if (dtype != ASR_F16 && dtype != ASR_BF16) return ASR_EUNSUPPORTED;
  HeadArgs a{};
  a.table = static_cast<const uint16_t *>(table);
  a.ids_in = ids;
  a.x_out = x;
  a.rows = rows;
  a.H = hidden;
  a.V = vocab;
  return launch_embed(a, dtype, stream) == hipSuccess ? ASR_OK : ASR_EHIP;
}

size_t asr_lm_head_workspace_bytes(const asr_head_config *cfg, int32_t max_rows) {
  if (check_head(cfg) != ASR_OK || max_rows < 0 || max_rows > kMaxRows) return 0;
  return head_ws_bytes(cfg, max_rows);
}

int asr_lm_head_argmax(const asr_head_config *cfg, const void *final_norm_w, const void *w_lm, const void *h,
                       int32_t rows, int32_t *ids, float *max_logit, void *workspace, size_t ws_bytes,
                       hipStream_t stream) {
  int rc = check_head(cfg);
  if (rc) return rc;
  if (rows < 0 || rows > kMaxRows) return ASR_EINVAL;
  if (rows == 0) return ASR_OK;
  if (!final_norm_w || !w_lm || !h || !ids) return ASR_EINVAL;
  if (!workspace || ws_bytes < head_ws_bytes(cfg, rows)) return ASR_EWORKSPACE;
  char *base = static_cast<char *>(workspace);
  const size_t yb = align_up((size_t)2 * cfg->hidden * rows * sizeof(uint16_t));
  const size_t pb = align_up((size_t)head_parts(cfg) * rows * sizeof(float));
  MlpArgs n{};
  n.h = h;
  n.in_f32 = cfg->in_dtype == ASR_F32;
  n.g_post = static_cast<const uint16_t *>(final_norm_w);
  n.y_hl = reinterpret_cast<uint16_t *>(base);
  n.rows = rows;
  n.H = cfg->hidden;
  n.I = 0;
  n.eps = cfg->rms_eps;
  HeadArgs a{};
  a.w_lm = static_cast<const uint16_t *>(w_lm);
  a.y_hl = n.y_hl;
  a.part_v = reinterpret_cast<float *>(base + yb);
  a.part_i = reinterpret_cast<int *>(base + yb + pb);
  a.ids_out = ids;
  a.max_logit = max_logit;
  a.rows = rows;
  a.H = cfg->hidden;
  a.V = cfg->vocab;
  a.nparts = head_parts(cfg);
  return launch_head(n, a, cfg->dtype, stream) == hipSuccess ? ASR_OK : ASR_EHIP;
}

int asr_accept_greedy(const int32_t *draft, const int32_t *target, int32_t B, int32_t k, const int32_t *slots,
                      const int32_t *lens, int32_t batch_cap, int32_t *accepted, int32_t *next_token,
                      int32_t *new_lens, hipStream_t stream) {
  if (B < 0 || k < 1 || batch_cap <= 0) return ASR_EINVAL;
  if (B == 0) return ASR_OK;
  if (!draft || !target || !lens || !accepted || !next_token || !new_lens) return ASR_EINVAL;
  if (!slots && B > batch_cap) return ASR_EINVAL;
  AcceptArgs a{draft, target, slots, lens, accepted, next_token, new_lens, B, k, batch_cap, 0, {0}};
  return launch_accept(a, stream) == hipSuccess ? ASR_OK : ASR_EHIP;
}

int asr_accept_greedy_mixed(const int32_t *draft, const int32_t *target, int32_t B, const int32_t *n_per_seq,
                            const int32_t *slots, const int32_t *lens, int32_t batch_cap, int32_t *accepted,
                            int32_t *next_token, int32_t *new_lens, hipStream_t stream) {
  if (B < 0 || B > kVmMaxSeqs || batch_cap <= 0) return ASR_EINVAL;
  if (B == 0) return ASR_OK;
  if (!n_per_seq || !draft || !target || !lens || !accepted || !next_token || !new_lens) return ASR_EINVAL;
  if (!slots && B > batch_cap) return ASR_EINVAL;
  AcceptArgs a{draft, target, slots, lens, accepted, next_token, new_lens, B, 1, batch_cap, 1, {0}};
  for (int b = 0; b < B; ++b) {
    if (n_per_seq[b] < 1 || n_per_seq[b] > kMaxVerifyK) return ASR_EINVAL;
    a.qo[b + 1] = a.qo[b] + n_per_seq[b];
  }
  return launch_accept(a, stream) == hipSuccess ? ASR_OK : ASR_EHIP;
}

size_t asr_mlp_workspace_bytes(const asr_mlp_config *cfg, int32_t max_rows) {
  if (check_mlp(cfg) != ASR_OK || max_rows < 0 || max_rows > kMaxRows) return 0;
  return mlp_ws_bytes(cfg, max_rows);
}

int asr_mlp_layer(const asr_mlp_config *cfg, const asr_mlp_weights *w, const void *h, int32_t rows, void *out,
                  void *workspace, size_t ws_bytes, hipStream_t stream) {
  return run_mlp(cfg, w, h, rows, out, workspace, ws_bytes, stream);
}

size_t asr_decoder_layer_workspace_bytes(const asr_attn_config *acfg, const asr_mlp_config *mcfg, int32_t max_rows,
                                         int32_t capacity) {
  if (max_rows < 0 || max_rows > kMaxRows) return 0;
  return layer_ws_bytes(acfg, mcfg, max_rows, capacity);
}

int asr_decoder_layer_decode(const asr_attn_config *acfg, const asr_attn_weights *aw, const asr_mlp_config *mcfg,
                             const asr_mlp_weights *mw, const asr_kv_layer *kv, const void *x,
                             const int32_t *slots, const int32_t *positions, int32_t B,
                             const int32_t *host_lens, void *out, void *workspace, size_t ws_bytes,
                             hipStream_t stream) {
  return run_decoder_layer(acfg, aw, mcfg, mw, kv, x, slots, positions, B, 1, host_lens, out, workspace, ws_bytes,
                           stream);
}

int asr_decoder_layer_verify(const asr_attn_config *acfg, const asr_attn_weights *aw, const asr_mlp_config *mcfg,
                             const asr_mlp_weights *mw, const asr_kv_layer *kv, const void *x,
                             const int32_t *slots, const int32_t *positions, int32_t B, int32_t k,
                             const int32_t *host_lens, void *out, void *workspace, size_t ws_bytes,
                             hipStream_t stream) {
  if (k < 1 || k > kMaxVerifyK) return ASR_EINVAL;
  return run_decoder_layer(acfg, aw, mcfg, mw, kv, x, slots, positions, B, k, host_lens, out, workspace, ws_bytes,
                           stream);
}

int asr_decoder_layer_mixed(const asr_attn_config *acfg, const asr_attn_weights *aw, const asr_mlp_config *mcfg,
                            const asr_mlp_weights *mw, const asr_kv_layer *kv, const void *x,
                            const int32_t *slots, const int32_t *positions, int32_t B, const int32_t *n_per_seq,
                            const int32_t *host_lens, void *out, void *workspace, size_t ws_bytes,
                            hipStream_t stream) {
  if (B > 0 && !n_per_seq) return ASR_EINVAL;
  return run_decoder_layer(acfg, aw, mcfg, mw, kv, x, slots, positions, B, 1, host_lens, out, workspace, ws_bytes,
                           stream, n_per_seq);
}

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

int asr_attn_layer_mixed(const asr_attn_config *cfg, const asr_attn_weights *w, const asr_kv_layer *kv,
                         const void *x, const int32_t *slots, const int32_t *positions, int32_t B,
                         const int32_t *n_per_seq, const int32_t *host_lens, const void *residual, void *out,
                         void *workspace, size_t ws_bytes, hipStream_t stream) {
  if (B > 0 && !n_per_seq) return ASR_EINVAL;
  return run_layer(cfg, w, kv, x, slots, positions, B, 1, host_lens, residual, out, workspace, ws_bytes, stream,
                   n_per_seq);
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
    case ASR_ESCRATCH: return "call needs more scratch than the library's static scratch holds";
  }
  return "unknown error";
}

}  // extern "C"
