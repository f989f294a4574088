// Internal interface between the C ABI (api.hip) and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "asr_attn.h"

namespace asr {

constexpr int kHeadDim = 128;          // the only head size the kernels support
constexpr int kMaxChunks = 64;        // split-KV chunks per (row, kv head)
constexpr int kMinSplit = 16;         // keys per chunk, lower bound
constexpr int kMaxSplit = 1024;       // keys per chunk, upper bound
constexpr int kMaxVerifyK = 32;
constexpr int kMaxLayerRows = 2048;   // rows (B k) per layer call
constexpr int kVectorRows = 4;        // up to this many rows the projections run as vector-ALU GEMVs
constexpr int kMaxKvHeads = 32;       // n_q_heads * head_dim <= 4096 bounds both head counts
constexpr int kVmMaxSeqs = 64;        // sequences of a verify call whose work items the host lays out
constexpr int kFlowWords = 128;      // counters of the one-dispatch path (heads + 4 totals)
constexpr int kPartStride = 132;      // floats per (chunk, q head) partial: acc[128], m, l, pad
constexpr uint32_t kStatusBadSlot = ASR_STATUS_BAD_SLOT;  // slot index outside [0, batch_cap)
constexpr uint32_t kStatusBadPage = ASR_STATUS_BAD_PAGE;  // page id outside the paged cache's pool

// Everything a layer kernel needs, passed by value.
struct LayerArgs {
  // inputs
  const uint16_t *x;          // [rows][H]
  const uint16_t *residual;   // [rows][H] or null
  const uint16_t *g_in;       // [H]
  const uint16_t *w_qkv;      // [nqkv][H]
  const uint16_t *g_q;        // [d]
  const uint16_t *g_k;        // [d]
  const uint16_t *w_o;        // [H][nq d]
  const int32_t *slots;       // [B] or null
  const int32_t *positions;   // [B] or null
  // cache
  uint16_t *kc, *vc;          // [batch_cap][nkv][capacity][d], or paged: [npages][nkv][psz][d]
  int32_t *lens;              // [batch_cap]
  uint32_t *status;           // or null
  // paged cache (ptab not null): position t of slot s is row t % psz of page ptab[s * pps + t / psz]
  const int32_t *ptab;        // [batch_cap][pps]
  int pps, npages, psz, plog; // psz = 1 << plog
  // output
  void *out;                  // [rows][H] fp32 or 16-bit
  // workspace (zero-filled once by the caller; every call leaves the counters at zero)
  float *qkv;                 // [rows][nqkv] projection; q, k heads rotated and gained, not normalised
  float *ssq;                 // [rows][nq + nkv][8] partial sums of squares of the raw q, k heads
  float *att;                 // [rows][nq][d] merged attention output
  uint16_t *att_hl;           // [rows][2][nq d] the same as hi and lo 16-bit terms (MFMA o_proj)
  float *part;                // [rows][nkv][kMaxChunks][group][kPartStride]
  uint32_t *flow;             // [kFlowWords] counters of the one-dispatch path (zero between calls)
  uint32_t *mctr;             // [rows][nkv] finished chunks per (row, kv head)
  int4 *rowtab;               // [rows] {ok, L, slot, slot_ok} as seen before the call
  // shape
  int B, n, rows;             // sequences, rows per sequence (1 decode, k verify), B * n
  int H, nq, nkv, group, nqkv;
  int batch_cap, capacity;
  int split;                  // keys per chunk (few rows); least keys per wave share (many rows)
  int nch_host;               // chunks per row the launch was sized for (few rows)
  float eps, theta;
  int out_f32;
  int mfma;                   // projections on MFMA (more than a few rows)
  int oproj_split;            // few rows, fp32 out: o_proj in two head halves adding into the zeroed output
  // verify attention on the matrix cores: work items (sequence, kv head, chunk) laid out by the host
  // from its copy of the lengths (vm_items > 0; vm_pre[b] = first item of sequence b), else by the
  // device from the lengths (vm_items = 0)
  int vm_items;
  int vm_pre[kVmMaxSeqs + 1];
  // 16-row query tiles of a (sequence, kv head): one work item per (sequence, kv head, chunk, tile)
  int vm_nt;
  // FP8 (E4M3) cache: kc / vc hold one code per element; per-kv-head scales of K and V
  int kv8;
  const float *ksc, *vsc;
  // multi-section rotary: pairs [0, ms0) use position component 0, [ms0, ms0 + ms1) component 1,
  // the rest component 2 (positions [3][B]); mrope = 0: one position per row
  int mrope, ms0, ms1;
  // mixed blocks (qo_n = 1): sequence b owns rows [qo[b], qo[b + 1]) with qo[B] = rows, B <= kVmMaxSeqs,
  // and n is the largest block; qo_n = 0: every sequence owns n rows
  int qo_n;
  int qo[kVmMaxSeqs + 1];
};

// The rest of the decoder layer: post-attention RMSNorm, gated SiLU MLP, residual.
struct MlpArgs {
  const void *h;              // [rows][H] fp32 (in_f32) or 16-bit: the MLP's input and residual
  int in_f32;
  const uint16_t *g_post;     // [H]
  const uint16_t *w_gate;     // [I][H]
  const uint16_t *w_up;       // [I][H]
  const uint16_t *w_down;     // [H][I]
  void *out;                  // [rows][H] fp32 (out_f32) or 16-bit
  int out_f32;
  uint16_t *y_hl;             // workspace: [2][H / 32][rows][32] normalised input, hi and lo terms
  uint16_t *a_hl;             // workspace: [2][I / 32][rows][32] silu(gate) * up, hi and lo terms
  int rows, H, I;
  float eps;
};

hipError_t launch_mlp(const MlpArgs &a, int dtype, hipStream_t s, hipEvent_t *ev);

// The model head: embedding lookup, final norm + lm_head argmax.
struct HeadArgs {
  const uint16_t *table;      // [V][H] embedding (k_embed)
  const int32_t *ids_in;      // [rows] token ids (k_embed)
  void *x_out;                // [rows][H] 16-bit (k_embed)
  const uint16_t *w_lm;       // [V][H] lm_head
  const uint16_t *y_hl;       // [2][H / 32][rows][32] normalised rows (hi, lo)
  float *part_v;              // [nparts][rows] best logit of each block of 128 ids
  int *part_i;                // [nparts][rows] its id
  int32_t *ids_out;           // [rows] argmax ids
  float *max_logit;           // [rows] or null
  int rows, H, V, nparts;
};

// Strict greedy acceptance and the lengths to crop to.
struct AcceptArgs {
  const int32_t *draft, *target;  // [B][k], or the packed blocks of a mixed call
  const int32_t *slots;           // [B] or null
  const int32_t *lens;            // [batch_cap] lengths after the verify block
  int32_t *accepted, *next_token; // [B]
  int32_t *new_lens;              // [batch_cap]
  int B, k, batch_cap;
  // blocks of per-sequence sizes (qo_n = 1): sequence b's block is entries [qo[b], qo[b + 1])
  int qo_n;
  int qo[kVmMaxSeqs + 1];
};

hipError_t launch_embed(const HeadArgs &a, int dtype, hipStream_t s);
hipError_t launch_head(const MlpArgs &norm, const HeadArgs &h, int dtype, hipStream_t s);
hipError_t launch_accept(const AcceptArgs &a, hipStream_t s);

struct WorkspaceLayout {
  size_t flow, mctr, rowtab, qkv, ssq, att, att_hl, part, total;
};

WorkspaceLayout workspace_layout(int rows, int H, int nq, int nkv, int capacity);

// validation, workspace carving and launch of one layer call (decode: n = 1;
// verify: n = k; mixed: n_per_seq, a host array of B block sizes, with n unused);
// the workspace is any device buffer of ws_bytes
int run_layer(const asr_attn_config *cfg, const asr_attn_weights *w, const asr_kv_layer *kv, const void *x,
              const int32_t *slots, const int32_t *positions, int B, int n, const int32_t *host_lens,
              const void *residual, void *out, void *ws, size_t ws_bytes, hipStream_t stream,
              const int32_t *n_per_seq = nullptr);

// launchers; return hipSuccess or the launch error
hipError_t launch_layer_multi(const LayerArgs &a, int dtype, int attn_grid, hipStream_t s, hipEvent_t *ev);
bool layer_fused_supported(const LayerArgs &a);
hipError_t launch_layer_fused(const LayerArgs &a, int dtype, int grid, hipStream_t s, hipEvent_t *ev);
int fused_max_grid(int dtype, int H, size_t dyn_smem, int cus);
size_t layer_dyn_smem(const LayerArgs &a);
bool attn_waves_used(const LayerArgs &a);
bool attn_vmfma_used(const LayerArgs &a);
int attn_vmfma_grid(int dtype, int group, int n, int B, int cus);
int attn_vmfma_tiles(int group, int n);
int attn_waves_grid(int dtype, int group, int cus, bool mix, bool paged);
hipError_t launch_kv_append(int dtype, const asr_kv_layer &kv, const void *k_new, const void *v_new,
                            const int32_t *slots, int B, int n, hipStream_t s);
hipError_t launch_kv_crop(const asr_kv_layer *layers, int n_layers, const int32_t *new_lens,
                          hipStream_t s);

}  // namespace asr
