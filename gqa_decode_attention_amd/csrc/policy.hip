// Host-side policy of the verify loop: the next block length from the draft's
// per-token uncertainty, and the draft read position after a round ("Can CTC
// make Qwen3-ASR faster?", section 07 and section 08 "Verifier, version 0").
// Plain integer and comparison logic on host arrays: no device work.
#include <stddef.h>
#include <stdint.h>

#include "internal.h"

extern "C" {

int32_t asr_next_block_len(const float *uncertainty, int32_t n, float threshold, int32_t k_min, int32_t k_max) {
  if (n < 0 || (n > 0 && !uncertainty)) return ASR_EINVAL;
  if (k_min < 1 || k_max < k_min || k_max > asr::kMaxVerifyK) return ASR_EINVAL;
  // the block ends at the first token above the threshold (NaN is not above it)
  int32_t j = n;
  for (int32_t i = 0; i < n; ++i) {
    if (uncertainty[i] > threshold) {
      j = i;
      break;
    }
  }
  int32_t k = j + 1;
  if (k < k_min) k = k_min;
  if (k > k_max) k = k_max;
  if (k > n) k = n;      // never past the draft ...
  return k < 1 ? 1 : k;  // ... but at least one row: with no draft left, a greedy step
}

int32_t asr_recycle_draft(const int32_t *draft, int32_t n, int32_t pos, int32_t k, int32_t accepted,
                          int32_t correction, int32_t window) {
  if (n < 0 || (n > 0 && !draft) || pos < 0 || k < 1 || accepted < 0 || accepted > k || window < 0)
    return ASR_EINVAL;
  if (accepted == k) return pos + k;
  // the correction replaces draft[pos + accepted]; a match among the next `window`
  // tokens marks the ones before it as spurious, and reading resumes past it
  const int64_t miss = (int64_t)pos + accepted;
  int64_t last = miss + window;
  if (last > (int64_t)n - 1) last = (int64_t)n - 1;
  for (int64_t j = miss + 1; j <= last; ++j)
    if (draft[j] == correction) return (int32_t)(j + 1);
  // a round that failed at its first token: the previous realignment may have
  // skipped a token the draft had dropped; the nearest of the `window` tokens
  // before pos equal to the correction marks where the draft resumes
  if (accepted == 0) {
    int64_t hi = (int64_t)pos < (int64_t)n ? (int64_t)pos : (int64_t)n;
    const int64_t lo = (int64_t)pos - window > 0 ? (int64_t)pos - window : 0;
    for (int64_t j = hi - 1; j >= lo; --j)
      if (draft[j] == correction) return (int32_t)(j + 1);
  }
  return (int32_t)(miss + 1);
}

}  // extern "C"
