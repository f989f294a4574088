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
 *    keeps no pointer after it returns.  Its only state between calls is a
 *    per-process cache of kernel occupancies (computed on first use, the
 *    same value whichever thread stores it).  Work is enqueued on `stream` in
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

/* element types (ASR_FP8_E4M3: KV caches only) */
enum { ASR_F16 = 0, ASR_BF16 = 1, ASR_F32 = 2, ASR_FP8_E4M3 = 3 };

/* return codes */
enum {
  ASR_OK = 0,
  ASR_EINVAL = -1,        /* null pointer, negative size, inconsistent shapes, k out of range */
  ASR_EUNSUPPORTED = -2,  /* a shape or type the library has no kernel for (see asr_attn_config) */
  ASR_ECAPACITY = -3,     /* host_lens given and some lens + n > capacity */
  ASR_EWORKSPACE = -4,    /* workspace NULL or smaller than asr_attn_workspace_bytes() */
  ASR_EHIP = -5,          /* the HIP runtime refused a launch */
  ASR_ESCRATCH = -6       /* asr_attn_layer_decode_noalloc: the call needs more than
                             ASR_NOALLOC_SCRATCH_BYTES of scratch */
};

/* bits of the sticky device status word */
enum {
  ASR_STATUS_CAPACITY = 1,     /* an append would pass the capacity: that sequence skipped */
  ASR_STATUS_CROP_GROW = 2,    /* a crop asked for a length < 0 or above the current one: ignored */
  ASR_STATUS_SYNC_TIMEOUT = 4, /* the fused dispatch gave up waiting for another workgroup */
  ASR_STATUS_BAD_SLOT = 8,     /* a slot index outside [0, batch_cap): that row skipped */
  ASR_STATUS_BAD_PAGE = 16     /* a paged cache's block table names a page outside
                                  [0, num_pages) for a position a call needs */
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
  int32_t mrope_sections[3];  /* multi-section rotary ("MRoPE" of the Latency page's section 03
                                 table): all zero = one position per row; else s0 + s1 + s2 =
                                 head_dim / 2 and rotary pair t turns by position component 0 for
                                 t < s0, 1 for t < s0 + s1, 2 after; `positions` is then [3][B]
                                 (component c of sequence b at positions[c * B + b]; row r of a
                                 verify block adds r to every component; NULL: every component is
                                 the cache length) */
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
 *
 * An FP8 cache ("Baseten optimizes Qwen3-ASR 1.7B", section "KV cache
 * quantization": the cache in FP8, half the bytes each step reads, the
 * attention arithmetic at full precision) holds one E4M3 code per element
 * (1 sign, 4 exponent bits with bias 7, 3 mantissa bits, largest finite value
 * 448, no infinities) and one fp32 scale per kv head for K and for V: the
 * cached value of a code c of kv head g is k_scale[g] * value(c).  A row the
 * library appends is stored as the code nearest to value / scale, ties to the
 * even code, magnitudes past 448 saturating to 448.  The layer calls take an
 * FP8 cache for calls of more than 4 rows (B for decode, B * k for verify) with
 * 2 or 4 q heads per kv head and the stream-ordered dispatch; other calls on an
 * FP8 cache return ASR_EUNSUPPORTED.
 *
 * A paged cache (block_table not NULL) keeps K and V in one pool of fixed-size
 * pages shared by all slots, addressed through a page table per slot (the
 * cache of the vLLM engine that "Baseten optimizes Qwen3-ASR 1.7B", section
 * "Our optimized Qwen3-ASR stack", starts its serving stack from).  k and v
 * are then [num_pages][n_kv_heads][page_size][head_dim]; position t of slot s,
 * kv head g lives in page p = block_table[s * pages_per_seq + t / page_size]
 * at k[((p * n_kv_heads + g) * page_size + t % page_size) * head_dim].
 * capacity must equal pages_per_seq * page_size; page_size is a power of two
 * in [16, 1024]; 16-bit caches only.  Slots may name the same page (a shared
 * prompt prefix) as long as no call appends into a page that another slot
 * still reads.  The table is read by the kernels, never by the host: a page
 * id outside [0, num_pages) for a position a call needs sets
 * ASR_STATUS_BAD_PAGE, and that sequence's output rows, appended rows and
 * length are then unspecified (nothing outside the pool is read or written).
 * Layer calls on a paged cache take the kernels they take on a contiguous
 * cache, except that verify blocks attend on the vector units rather than the
 * matrix cores; the fused dispatch returns ASR_EUNSUPPORTED.
 */
typedef struct asr_kv_layer {
  void *k;              /* [batch_cap][n_kv_heads][capacity][head_dim], elements of dtype
                           (paged: [num_pages][n_kv_heads][page_size][head_dim]) */
  void *v;              /* same layout */
  int32_t *lens;        /* [batch_cap] committed length per slot (device) */
  uint32_t *status;     /* sticky ASR_STATUS_* word (device) or NULL */
  int32_t batch_cap;
  int32_t capacity;
  int32_t n_kv_heads;
  int32_t head_dim;
  int32_t dtype;        /* ASR_F16 or ASR_BF16 (the layer's dtype), or ASR_FP8_E4M3 */
  const float *k_scale; /* ASR_FP8_E4M3: [n_kv_heads] fp32 scales of K (device); else ignored */
  const float *v_scale; /* ASR_FP8_E4M3: [n_kv_heads] fp32 scales of V (device); else ignored */
  const int32_t *block_table; /* paged cache: [batch_cap][pages_per_seq] page ids (device);
                                 NULL: the contiguous layout above, and the fields below are ignored */
  int32_t page_size;    /* paged: positions per page */
  int32_t pages_per_seq;
  int32_t num_pages;    /* paged: pages in the pool */
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
 * Bytes of the library's static device scratch used by
 * asr_attn_layer_decode_noalloc: 40 MiB, which holds one decode call of up to
 * 64 rows at the pages' shapes (16 q / 8 kv heads: about 575 KB per row, most
 * of it split-KV partials).  Every GPU the entry point runs on holds one such
 * array from its first call until the process ends.
 */
#define ASR_NOALLOC_SCRATCH_BYTES (40u << 20)

/*
 * asr_attn_layer_decode without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  It computes exactly what
 * asr_attn_layer_decode computes, with the same kernels, using a file-scope
 * device array of ASR_NOALLOC_SCRATCH_BYTES as the workspace; it calls no
 * allocating routine.  The first call on a device looks up that device's
 * array and enqueues one small kernel that zeroes its counters.
 * Every call on one GPU shares that GPU's array: calls that may overlap on one
 * GPU (concurrent streams, threads) race and must be serialised by the caller.
 * Returns ASR_ESCRATCH (nothing enqueued) when the call's workspace
 * (asr_attn_workspace_bytes for B rows and the cache capacity) exceeds the
 * array, ASR_EHIP if the array's address cannot be obtained; otherwise as
 * asr_attn_layer_decode.
 */
int asr_attn_layer_decode_noalloc(const asr_attn_config *cfg, const asr_attn_weights *w,
                                  const asr_kv_layer *kv, const void *x, const int32_t *slots,
                                  const int32_t *positions, int32_t B, const int32_t *host_lens,
                                  const void *residual, void *out, hipStream_t stream);

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
 * Decode rows and verify blocks of different lengths in one call ("Can CTC
 * make Qwen3-ASR faster?", section 08 "Verifier, version 0": the block length
 * is chosen per sequence from the draft's confidence, so the sequences in
 * flight carry blocks of different k; a k of 1 is a plain decode step).
 * Sequence b owns n_per_seq[b] consecutive rows starting at row
 * n_per_seq[0] + ... + n_per_seq[b - 1]; with L = lens[s] its rows are appended
 * at L .. L + n_per_seq[b] - 1 and row r attends over positions 0 .. L + r, as
 * in asr_attn_layer_verify with k = n_per_seq[b].  lens[s] becomes
 * L + n_per_seq[b].  Rotary position of row r: positions[b] + r (NULL: L + r;
 * multi-section rotary: positions [3][B], component c of sequence b at
 * positions[c * B + b]).
 *   n_per_seq HOST [B] int32, each in 1 .. 32; B <= 64; rows = sum of n_per_seq <= 2048
 *   x, residual [rows][H] dtype, out [rows][H] out_dtype
 * It computes what one asr_attn_layer_verify call per sequence with its own k
 * computes (up to the order of fp32 sums: blocks of different sizes always
 * take the many-row kernels, whatever the row count).  Blocks all of one size
 * k are the asr_attn_layer_verify call with that k (k = 1: the decode call),
 * bit for bit.  Blocks of different sizes are not available with
 * ASR_DISPATCH_FUSED (ASR_EUNSUPPORTED); B > 64 or a block size outside
 * 1 .. 32: ASR_EINVAL.  Workspace: asr_attn_workspace_bytes for `rows` rows.
 */
int asr_attn_layer_mixed(const asr_attn_config *cfg, const asr_attn_weights *w,
                         const asr_kv_layer *kv, const void *x, const int32_t *slots,
                         const int32_t *positions, int32_t B, const int32_t *n_per_seq,
                         const int32_t *host_lens, const void *residual, void *out,
                         void *workspace, size_t ws_bytes, hipStream_t stream);

/*
 * Bit-exact copy of given K/V rows into one layer's cache: the prefill filler
 * ("Can CTC make Qwen3-ASR faster?", section 11 Phase D: build the prompt KV
 * once, then verify blocks against it; the faster-qwen-asr GB10 record's
 * configuration writes prefill straight into a static cache).
 * k_new, v_new are [B][n][n_kv_heads][head_dim] elements of kv->dtype (E4M3
 * codes for an FP8 cache: copied as they are, the scales do not enter); the n
 * rows of sequence b go to positions lens[s] .. lens[s] + n - 1 of slot
 * s = slots[b] (NULL: b), then lens[s] grows by n.  A sequence whose rows
 * would pass the capacity is skipped (ASR_STATUS_CAPACITY).  Slots distinct.
 * On a paged cache each row goes to the page its position maps to; a row
 * whose page id lies outside the pool is not stored (ASR_STATUS_BAD_PAGE).
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

/*
 * The rest of a decoder layer: post-attention RMSNorm, the gated SiLU MLP and
 * the residual ("Qwen3-ASR -- Latency & Bottleneck Analysis", section 03: the
 * decoder MLP, memory-bound at 529 MB per token over 28 layers; section 07
 * "Norms are real money at this size").  For each row,
 *   y   = h * post_norm_w / sqrt(mean(h^2) + rms_eps)
 *   out = h + W_down (silu(W_gate y) * (W_up y)),   silu(u) = u / (1 + e^-u)
 * All arithmetic is fp32; matrix-core operands that are fp32 values (y and
 * silu(gate) * up) are split into two 16-bit terms.  Supported: hidden and
 * intermediate multiples of 256 (hidden at most 2048, intermediate at most
 * 16384), dtype ASR_F16 or ASR_BF16, 1 to 2048 rows.
 */
typedef struct asr_mlp_config {
  int32_t hidden;        /* H */
  int32_t intermediate;  /* I */
  float rms_eps;
  int32_t dtype;         /* ASR_F16 or ASR_BF16: the weights */
  int32_t in_dtype;      /* h: ASR_F32 (the attention block's fp32 output) or dtype */
  int32_t out_dtype;     /* ASR_F32 or dtype */
  hipEvent_t *phase_events;  /* diagnostics, NULL normally: 4 caller-created events that receive the
                                start and end stamps of the normalising gate/up kernel, then of the
                                down kernel */
} asr_mlp_config;

/* One layer's MLP weights (device, elements of dtype, row-major [out][in]). */
typedef struct asr_mlp_weights {
  const void *post_norm_w;  /* [H] */
  const void *w_gate;       /* [I][H] */
  const void *w_up;         /* [I][H] */
  const void *w_down;       /* [H][I] */
} asr_mlp_weights;

/* Workspace bytes of asr_mlp_layer for up to max_rows rows (0: invalid config). */
size_t asr_mlp_workspace_bytes(const asr_mlp_config *cfg, int32_t max_rows);

/*
 * out[r] = h[r] + MLP(RMSNorm(h[r])) for rows r < rows.
 *   h   [rows][H] in_dtype (device), the residual stream after the attention block
 *   out [rows][H] out_dtype (device); must not overlap h or the workspace
 * The workspace needs no initialisation.  Returns ASR_OK or a host-side ASR_E*
 * code (nothing enqueued then).  rows = 0 is a no-op.
 */
int asr_mlp_layer(const asr_mlp_config *cfg, const asr_mlp_weights *w, const void *h, int32_t rows, void *out,
                  void *workspace, size_t ws_bytes, hipStream_t stream);

/*
 * Workspace bytes of asr_decoder_layer_decode / asr_decoder_layer_verify: the
 * attention block's workspace, the fp32 residual stream h, the MLP's workspace.
 */
size_t asr_decoder_layer_workspace_bytes(const asr_attn_config *acfg, const asr_mlp_config *mcfg, int32_t max_rows,
                                         int32_t capacity);

/*
 * One whole decoder layer for B one-token rows: h = x + attention(x) (the
 * attention block of asr_attn_layer_decode with the layer input as its
 * residual, kept in fp32 in the workspace), then out = h + MLP(RMSNorm(h)).
 * acfg->out_dtype is ignored (h is fp32); mcfg->in_dtype must be ASR_F32 and
 * mcfg->out_dtype gives out's type.  Arguments as asr_attn_layer_decode; the
 * workspace (asr_decoder_layer_workspace_bytes) must be zero-filled before
 * its first use, like the attention block's.
 */
int asr_decoder_layer_decode(const asr_attn_config *acfg, const asr_attn_weights *aw, const asr_mlp_config *mcfg,
                             const asr_mlp_weights *mw, const asr_kv_layer *kv, const void *x,
                             const int32_t *slots, const int32_t *positions, int32_t B,
                             const int32_t *host_lens, void *out, void *workspace, size_t ws_bytes,
                             hipStream_t stream);

/* The k-token verify block through a whole decoder layer: x, out [B][k][H]. */
int asr_decoder_layer_verify(const asr_attn_config *acfg, const asr_attn_weights *aw, const asr_mlp_config *mcfg,
                             const asr_mlp_weights *mw, const asr_kv_layer *kv, const void *x,
                             const int32_t *slots, const int32_t *positions, int32_t B, int32_t k,
                             const int32_t *host_lens, void *out, void *workspace, size_t ws_bytes,
                             hipStream_t stream);

/* Mixed decode rows and verify blocks (as asr_attn_layer_mixed) through a whole
   decoder layer: x, out [rows][H], rows = sum of n_per_seq. */
int asr_decoder_layer_mixed(const asr_attn_config *acfg, const asr_attn_weights *aw, const asr_mlp_config *mcfg,
                            const asr_mlp_weights *mw, const asr_kv_layer *kv, const void *x,
                            const int32_t *slots, const int32_t *positions, int32_t B, const int32_t *n_per_seq,
                            const int32_t *host_lens, void *out, void *workspace, size_t ws_bytes,
                            hipStream_t stream);

/*
 * The verify loop above the decoder ("Can CTC make Qwen3-ASR faster?", section
 * 11 Phase A: a loop exposing one-token decode and logits; verify_block returns
 * the target's argmax at every candidate position; section 03 "Greedy
 * exactness": accept the longest draft prefix equal to the target's argmax,
 * emit the target's token at the first mismatch, crop the speculative cache).
 *
 * A round starts from the last committed token p (its K/V not yet cached) and
 * a draft d[0..k-1]; the caller embeds the block [p, d[0], ..., d[k-2]] with
 * asr_embed, runs asr_decoder_layer_verify on every layer, takes the argmax of
 * every block row with asr_lm_head_argmax (row i verifies d[i]: the one-token
 * shift of section 11 step 3), then asr_accept_greedy gives the accepted count,
 * the next token and the lengths to crop every layer to with asr_kv_crop.
 */

/* x[r] = table[ids[r]] (16-bit rows of dtype); an id outside [0, vocab) gives a NaN row. */
int asr_embed(const void *table, int32_t vocab, int32_t hidden, int32_t dtype, const int32_t *ids, int32_t rows,
              void *x, hipStream_t stream);

/* Final RMSNorm and lm_head: vocab a multiple of 16, hidden a multiple of 256 (at most 4096). */
typedef struct asr_head_config {
  int32_t hidden;    /* H */
  int32_t vocab;     /* V */
  float rms_eps;
  int32_t dtype;     /* ASR_F16 or ASR_BF16: the weights */
  int32_t in_dtype;  /* h: ASR_F32 or dtype */
} asr_head_config;

/* Workspace bytes of asr_lm_head_argmax for up to max_rows rows (0: invalid config). */
size_t asr_lm_head_workspace_bytes(const asr_head_config *cfg, int32_t max_rows);

/*
 * ids[r] = argmax_v (W_lm RMSNorm(h[r]) * final_norm_w)[v], the smallest id
 * among equal maxima (-1 if no logit of the row is a number); max_logit[r]
 * (nullable) its logit.  Logits in fp32 on the matrix cores (W_lm exact, the
 * normalised row as two 16-bit terms).  final_norm_w [H], w_lm [V][H] of dtype;
 * h [rows][H] of in_dtype; ids, max_logit device arrays of rows entries.
 */
int asr_lm_head_argmax(const asr_head_config *cfg, const void *final_norm_w, const void *w_lm, const void *h,
                       int32_t rows, int32_t *ids, float *max_logit, void *workspace, size_t ws_bytes,
                       hipStream_t stream);

/*
 * Strict greedy acceptance for B sequences with k drafts each (device arrays):
 * draft, target [B][k] (target[b][i] = the target's argmax of block row i, which
 * verifies draft[b][i]).  accepted[b] = the longest prefix with draft = target;
 * next_token[b] = target[b][accepted] at a mismatch, else draft[b][k-1] (the
 * last committed token, which starts the next round); new_lens[batch_cap] =
 * lens (the lengths after the verify block) for every slot, minus the rejected
 * rows (k - accepted - 1 at a mismatch, none otherwise) for slots[b] (NULL: b).
 * All integer, on the device; then asr_kv_crop(layers, n, new_lens).
 */
int asr_accept_greedy(const int32_t *draft, const int32_t *target, int32_t B, int32_t k, const int32_t *slots,
                      const int32_t *lens, int32_t batch_cap, int32_t *accepted, int32_t *next_token,
                      int32_t *new_lens, hipStream_t stream);

/*
 * asr_accept_greedy for blocks of per-sequence sizes, as a mixed call lays them
 * out: draft and target hold sequence b's n_per_seq[b] entries after those of
 * sequences 0 .. b-1 (device arrays); n_per_seq is a HOST array of B sizes in
 * 1 .. 32, B <= 64.  Sequence b's results as asr_accept_greedy with k =
 * n_per_seq[b].
 */
int asr_accept_greedy_mixed(const int32_t *draft, const int32_t *target, int32_t B, const int32_t *n_per_seq,
                            const int32_t *slots, const int32_t *lens, int32_t batch_cap, int32_t *accepted,
                            int32_t *next_token, int32_t *new_lens, hipStream_t stream);

/*
 * The loop's block-length and draft-recycling policy ("Can CTC make Qwen3-ASR
 * faster?", section 07: adaptive block length and recycling of the aligned
 * suffix; section 08 "Verifier, version 0": at a mismatch recycle the draft
 * suffix that realigns after the correction, and choose the next k from the
 * draft's confidence, longer over low-entropy spans and shorter around
 * uncertain tokens).  Host functions on host arrays; neither changes what a
 * round commits, only how many rounds a transcript takes.
 *
 * asr_next_block_len: uncertainty[0..n-1] is the draft's uncertainty of each
 * token not yet verified (for example its frame entropy).  With j the first
 * index whose uncertainty is above threshold (n if none; NaN is never above),
 * the block ends at that token: k = j + 1, clamped to [k_min, k_max] and to n,
 * and at least 1 (no draft left: a greedy step).  Returns k, or ASR_EINVAL
 * (n < 0, a NULL array with n > 0, k_min < 1, k_max < k_min or k_max > 32).
 */
int32_t asr_next_block_len(const float *uncertainty, int32_t n, float threshold, int32_t k_min, int32_t k_max);

/*
 * asr_recycle_draft: the read position in draft[0..n-1] (host) for the next
 * round, after a round that verified the k tokens from position pos (tokens
 * past n were padding) and accepted `accepted` of them.  All accepted: pos + k.
 * Otherwise the target's correction replaces draft[pos + accepted]; if it equals
 * one of the next `window` tokens, the tokens before the first such match were
 * spurious and reading resumes just past the match; else, for a round that
 * failed at its first token (accepted = 0), if it equals one of the `window`
 * tokens before pos, the draft had dropped a token there and reading resumes
 * just past the nearest such match; else draft[pos + accepted] was a wrong
 * token in the right place and reading resumes after it.  Returns
 * the position, or ASR_EINVAL (n < 0, NULL draft with n > 0, pos < 0, k < 1,
 * accepted outside [0, k], window < 0).
 */
int32_t asr_recycle_draft(const int32_t *draft, int32_t n, int32_t pos, int32_t k, int32_t accepted,
                          int32_t correction, int32_t window);

/* Static text of an ASR_E* code. */
const char *asr_strerror(int code);

#ifdef __cplusplus
}
#endif

#endif /* ASR_ATTN_H */
