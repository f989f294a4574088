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
constexpr int kFlowWords = 128;      // counters of the one-dispatch path (heads + 4 totals)
constexpr int kPartStride = 132;      // floats per (chunk, q head) partial: acc[128], m, l, pad
constexpr uint32_t kStatusBadSlot = ASR_STATUS_BAD_SLOT;  // slot index outside [0, batch_cap)

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
  uint16_t *kc, *vc;          // [batch_cap][nkv][capacity][d]
  int32_t *lens;              // [batch_cap]
  uint32_t *status;           // or null
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
};

struct WorkspaceLayout {
  size_t flow, mctr, rowtab, qkv, ssq, att, att_hl, part, total;
};

WorkspaceLayout workspace_layout(int rows, int H, int nq, int nkv, int capacity);

// launchers; return hipSuccess or the launch error
hipError_t launch_layer_multi(const LayerArgs &a, int dtype, int attn_grid, hipStream_t s, hipEvent_t *ev);
bool layer_fused_supported(const LayerArgs &a);
hipError_t launch_layer_fused(const LayerArgs &a, int dtype, int grid, hipStream_t s, hipEvent_t *ev);
int fused_max_grid(int dtype, int H, size_t dyn_smem, int cus);
size_t layer_dyn_smem(const LayerArgs &a);
bool attn_waves_used(const LayerArgs &a);
int attn_waves_grid(int dtype, int group, int cus);
hipError_t launch_kv_append(int dtype, const asr_kv_layer &kv, const void *k_new, const void *v_new,
                            const int32_t *slots, int B, int n, hipStream_t s);
hipError_t launch_kv_crop(const asr_kv_layer *layers, int n_layers, const int32_t *new_lens,
                          hipStream_t s);

}  // namespace asr
