/*
 * asr_attn.h -- C ABI of the MI355X (gfx950) decoder attention block.
 *
 * One call runs one decoder layer's attention block for a set of rows:
 * input RMSNorm -> fused q/k/v projection -> per-head q/k RMSNorm -> rotary
 * -> KV-cache append -> grouped-query attention over the cache -> o_proj.
 * The operation list is the one "Qwen3-ASR -- Latency & Bottleneck Analysis"
 * gives for decoder attention in section 07 ("Why attention is 48.6% of
 * decode"), with the norms of "Norms are real money at this size" (same
 * section) and the fp32 rotary of the section 03 module table; there the
 * chain costs about ten tiny kernel launches per layer, here it is a single
 * library call.  Cache transactions are explicit calls (append, crop), as
 * "Can CTC make Qwen3-ASR faster?" asks for in section 06 (generate() hides
 * cache transactions) and section 11 Phase A/D (a loop that exposes one-token
 * decode and cache length; transactional commit/crop of KV).
 *
 * Conventions for every entry point
 *  - All tensor arguments are DEVICE pointers unless a comment says "host".
 *    The caller owns all memory.  The library never allocates, never
 *    synchronises the stream, never copies device data back to the host and
 *    keeps no pointer after it returns.  Work is enqueued on `stream` in
 *    stream order; calls are safe to capture in a HIP graph.
 *  - Return value: ASR_OK (0) or a negative ASR_E* code for a synchronous,
 *    host-side validation failure (nothing is enqueued then).  Conditions that
 *    only the device can see (a cache capacity overflow, a crop that would
 *    grow a length, a fused-dispatch synchronisation timeout) never fail
 *    silently: the affected rows' outputs are written as NaN where there are
 *    outputs, the affected lengths are left unchanged, and a bit is OR-ed into
 *    the layer's sticky `status` word (if non-NULL), which the caller reads at
 *    its own synchronisation points and clears itself.
 *  - Matrices are row-major [out][in] (the nn.Linear convention).
 *  - B = 0 is a no-op that returns ASR_OK.
 */
#ifndef ASR_ATTN_H
#define ASR_ATTN_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* element types */
enum { ASR_F16 = 0, ASR_BF16 = 1, ASR_F32 = 2 };

/* return codes */
enum {
  ASR_OK = 0,
  ASR_EINVAL = -1,        /* null pointer, negative size, inconsistent shapes, k out of range */
  ASR_EUNSUPPORTED = -2,  /* a shape or type the library has no kernel for (see asr_attn_config) */
  ASR_ECAPACITY = -3,     /* host_lens given and some lens + n > capacity */
  ASR_EWORKSPACE = -4,    /* workspace NULL or smaller than asr_attn_workspace_bytes() */
  ASR_EHIP = -5           /* the HIP runtime refused a launch */
};

/* bits of the sticky device status word */
enum {
  ASR_STATUS_CAPACITY = 1,     /* an append would pass the capacity: that sequence skipped */
  ASR_STATUS_CROP_GROW = 2,    /* a crop asked for a length < 0 or above the current one: ignored */
  ASR_STATUS_SYNC_TIMEOUT = 4, /* the fused dispatch gave up waiting for another workgroup */
  ASR_STATUS_BAD_SLOT = 8      /* a slot index outside [0, batch_cap): that row skipped */
};

/* how a layer call is dispatched */
enum {
  ASR_DISPATCH_AUTO = 0,   /* the library chooses (currently: one kernel per phase) */
  ASR_DISPATCH_MULTI = 1,  /* one kernel per phase, ordered by the stream */
  ASR_DISPATCH_FUSED = 2   /* one persistent kernel per layer call whose resident workgroups
                              order the phases through counters in the workspace (a phase waits
                              only for the producers it reads); hidden 1024 or 2048, 16 q heads,
                              8 kv heads, at most 4 rows (else ASR_EUNSUPPORTED); needs the whole
                              device (no concurrent kernels), else it may time out */
};

/*
 * Block shape and numerics.  Supported by the library: head_dim = 128;
 * n_q_heads a multiple of n_kv_heads with n_q_heads / n_kv_heads in
 * {1, 2, 4, 8}; n_q_heads * head_dim and hidden multiples of 512, at most
 * 4096; dtype ASR_F16 or ASR_BF16 (weights, x, residual and the KV cache);
 * out_dtype ASR_F32 or equal to dtype; at most 2048 rows per call (B for
 * decode, B * k for verify); cache capacity at most 65536.  The shapes of the
 * pages' model are hidden 1024 (or 2048), 16 q heads, 8 kv heads,
 * head_dim 128, eps 1e-6, rope_theta 1e6.  All arithmetic is fp32; 16-bit
 * operands of the matrix-core path are exact 16-bit data or two-term (hi + lo)
 * splits of fp32 values.
 */
typedef struct asr_attn_config {
  int32_t hidden;       /* H */
  int32_t n_q_heads;    /* nq */
  int32_t n_kv_heads;   /* nkv; q head i reads kv head i / (nq / nkv) */
  int32_t head_dim;     /* d */
  float rms_eps;        /* eps of all three RMSNorms: x * g / sqrt(mean(x^2) + eps) */
  float rope_theta;     /* rotary base: pair (t, t + d/2) turns by pos * theta^(-2t/d) */
  int32_t dtype;        /* ASR_F16 or ASR_BF16 */
  int32_t out_dtype;    /* ASR_F32 (recommended: carries the full-precision result) or dtype */
  int32_t kv_split;     /* keys per split-KV chunk: 0 = automatic, else a multiple of 16 in
                           [16, 1024] with capacity <= 64 * kv_split */
  int32_t dispatch;     /* ASR_DISPATCH_* */
  hipEvent_t *phase_events;  /* diagnostics, NULL normally: an array of 6 events (created by the
                                caller) that receive the start and end stamps of the projection,
                                attention and o_proj kernels, in that order, of the stream-ordered
                                dispatch; the fused dispatch stamps its one kernel into [0] and [5] */
} asr_attn_config;

/* One layer's weights (device pointers, elements of cfg.dtype). */
typedef struct asr_attn_weights {
  const void *input_norm_w;  /* [H] gain of the input RMSNorm */
  const void *w_qkv;         /* [(nq + 2 nkv) d][H]: q rows (head-major), then k rows, then v rows */
  const void *q_norm_w;      /* [d] gain of the per-head q RMSNorm (shared by all q heads) */
  const void *k_norm_w;      /* [d] gain of the per-head k RMSNorm */
  const void *w_o;           /* [H][nq d] output projection */
} asr_attn_weights;

/*
 * One layer's KV cache.  Each layer has its own lens: an append or a decode
 * on a layer advances only that layer's lengths.  Position t of sequence
 * slot s, kv head g lives at k[((s * n_kv_heads + g) * capacity + t) * head_dim].
 * Positions >= lens[s] hold no committed data and are never read.
 */
typedef struct asr_kv_layer {
  void *k;              /* [batch_cap][n_kv_heads][capacity][head_dim], elements of dtype */
  void *v;              /* same layout */
  int32_t *lens;        /* [batch_cap] committed length per slot (device) */
  uint32_t *status;     /* sticky ASR_STATUS_* word (device) or NULL */
  int32_t batch_cap;
  int32_t capacity;
  int32_t n_kv_heads;
  int32_t head_dim;
  int32_t dtype;        /* ASR_F16 or ASR_BF16 */
} asr_kv_layer;

/*
 * Workspace bytes needed by asr_attn_layer_decode / asr_attn_layer_verify for
 * up to `max_rows` rows (B for decode, B * k for verify) on caches of
 * `capacity` positions.  Returns 0 for an unsupported or invalid config.
 * The workspace is scratch owned by the caller; it must not be shared by
 * calls that may run concurrently.  It must be zero-filled before its first
 * use (it holds counters that every call leaves at zero again); after a call
 * that reported ASR_STATUS_SYNC_TIMEOUT it must be zero-filled again.
 */
size_t asr_attn_workspace_bytes(const asr_attn_config *cfg, int32_t max_rows, int32_t capacity);

/*
 * Single-token decode of B rows ("Qwen3-ASR -- Latency & Bottleneck
 * Analysis", section 03: one decoder step per generated token).  Row i works
 * on sequence slot s = slots[i] (slots NULL: s = i); the slots of one call
 * must be distinct.  With L = lens[s] on entry, the row's k and v are rounded
 * once to dtype and stored at position L, the row's q attends over positions
 * 0 .. L (its own key included), and lens[s] becomes L + 1.  Rotary uses
 * position positions[i] (positions NULL: L).
 *   x        [B][H] dtype          hidden states entering the block
 *   residual [B][H] dtype or NULL  added to the output when given
 *   out      [B][H] out_dtype      W_o * attention (+ residual)
 *   host_lens  HOST [B] or NULL: the caller's copy of lens[slots[i]], used only
 *            to size the launch and for the ASR_ECAPACITY check; the device
 *            lengths remain the truth.
 * out must not overlap x, residual, the cache or the workspace: with an fp32
 * out and a few rows it is zeroed by the call's first kernel and accumulated
 * by its last.
 */
int asr_attn_layer_decode(const asr_attn_config *cfg, const asr_attn_weights *w,
                          const asr_kv_layer *kv, const void *x, const int32_t *slots,
                          const int32_t *positions, int32_t B, const int32_t *host_lens,
                          const void *residual, void *out, void *workspace, size_t ws_bytes,
                          hipStream_t stream);

/*
 * k-token causal verification block ("Can CTC make Qwen3-ASR faster?",
 * section 03 and section 08 "Verifier, version 0": score k candidate
 * positions in one causal pass over the committed cache).  For sequence b
 * (slot s = slots[b], L = lens[s]) the k rows x[b][0..k-1] are appended at
 * L .. L + k - 1 and row r attends over positions 0 .. L + r: the committed
 * prefix and the candidates up to and including itself.  Rotary position of
 * row r is positions[b] + r (positions NULL: L + r).  lens[s] becomes L + k;
 * the caller then crops to the accepted prefix with asr_kv_crop.
 *   x, residual [B][k][H] dtype, out [B][k][H] out_dtype; 1 <= k <= 32.
 * With k = 1 this is the same computation as asr_attn_layer_decode.
 */
int asr_attn_layer_verify(const asr_attn_config *cfg, const asr_attn_weights *w,
                          const asr_kv_layer *kv, const void *x, const int32_t *slots,
                          const int32_t *positions, int32_t B, int32_t k,
                          const int32_t *host_lens, const void *residual, void *out,
                          void *workspace, size_t ws_bytes, hipStream_t stream);

/*
 * Bit-exact copy of given K/V rows into one layer's cache (a prefill filler).
 * k_new, v_new are [B][n][n_kv_heads][head_dim] elements of kv->dtype; the n
 * rows of sequence b go to positions lens[s] .. lens[s] + n - 1 of slot
 * s = slots[b] (NULL: b), then lens[s] grows by n.  A sequence whose rows
 * would pass the capacity is skipped (ASR_STATUS_CAPACITY).  Slots distinct.
 */
int asr_kv_append(const asr_kv_layer *kv, const void *k_new, const void *v_new,
                  const int32_t *slots, int32_t B, int32_t n, hipStream_t stream);

/*
 * Crop to the committed prefix ("Can CTC make Qwen3-ASR faster?", section 03
 * "Greedy exactness" and section 11 Phase D): for every one of the n_layers
 * layers (a HOST array of layer descriptors with equal batch_cap), set
 * lens[b] = new_lens[b] for every slot b < batch_cap, in one dispatch for up
 * to 64 layers.  Only shrinking or keeping is allowed: a slot whose new
 * length is negative or above its current length keeps it and the layer's
 * status gets ASR_STATUS_CROP_GROW.  Cached data are not touched; positions
 * past the new length are never read again, so a crop after a rejected
 * verify block leaves the layer exactly as if the rejected rows had never
 * been appended.
 *   new_lens [batch_cap] int32 (device)
 */
int asr_kv_crop(const asr_kv_layer *layers, int32_t n_layers, const int32_t *new_lens,
                hipStream_t stream);

/* Static text of an ASR_E* code. */
const char *asr_strerror(int code);

#ifdef __cplusplus
}
#endif

#endif /* ASR_ATTN_H */
