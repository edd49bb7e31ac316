// Device helpers shared by the attention kernels.
//
// Pages cited by tag and function: P1 "vllm_omni/experimental/ar_diffusion/kv_cache/paged_attention.py",
// P2 "tests/diffusion/ar_diffusion/test_paged_attention.py",
// P3 "vllm_omni/diffusion/attention/backends/utils/piecewise_attn.py",
// P4 "vllm_omni/diffusion/diffusion_kv/paged_attention_adapter.py".
#pragma once

#include <climits>

#include "pkv_internal.hpp"

namespace pkv {

// Exclusive key bound of query row g (key coordinates): FlashAttention's
// bottom-right convention for a causal segment [q_start, q_end) gives keys
// j <= g; a full segment gives keys j < kv_end (P3 module docstring and
// build_segments; P4 uses kv_end as the per-segment seq_len).
__device__ __forceinline__ int row_limit(const int32_t* __restrict__ seg, int s0, int s1, int g) {
  for (int k = s0; k < s1; ++k) {
    const int qs = seg[4 * k + 0];
    const int qe = seg[4 * k + 1];
    if (g >= qs && g < qe) return seg[4 * k + 3] == PKV_SEG_FULL ? seg[4 * k + 2] : g + 1;
  }
  return g + 1;  // not reached for validated segments (they tile the query)
}

// The segments of one sequence held in registers, so that every row limit a
// workgroup needs comes from one round of loads issued together (the walk
// above issues its loads one after another, each waiting for the last).
// Sequences with more than kSegCache segments fall back to the walk.
constexpr int kSegCache = 8;
struct SegCache {
  int n;  // segments s0 .. s1 - 1, or -1: too many (use row_limit)
  int qs[kSegCache], qe[kSegCache], kv[kSegCache];
};
__device__ __forceinline__ SegCache load_segments(const int32_t* __restrict__ seg, int s0, int s1) {
  SegCache c;
  c.n = (s1 - s0 <= kSegCache) ? s1 - s0 : -1;
  // Every load unconditional (slots past the sequence's segments re-read its
  // last one), so that all of them go out before the first result is used.
  const int last = s0 + max(min(s1 - s0, kSegCache) - 1, 0);
#pragma unroll
  for (int i = 0; i < kSegCache; ++i) {
    const int k = min(s0 + i, last);
    const int qs = seg[4 * k + 0], qe = seg[4 * k + 1], kv = seg[4 * k + 2], mode = seg[4 * k + 3];
    c.qs[i] = qs;
    c.qe[i] = i < c.n ? qe : INT32_MIN;
    c.kv[i] = mode == PKV_SEG_FULL ? kv : -1;  // -1: causal
  }
  return c;
}
__device__ __forceinline__ int row_limit(const SegCache& c, const int32_t* __restrict__ seg, int s0, int s1, int g) {
  if (c.n < 0) return row_limit(seg, s0, s1, g);
  int lim = g + 1;
#pragma unroll
  for (int i = 0; i < kSegCache; ++i)
    if (g >= c.qs[i] && g < c.qe[i] && c.kv[i] >= 0) lim = c.kv[i];
  return lim;
}

// Sequence owning global query token t: the last b with qsl[b] <= t.
__device__ __forceinline__ int seq_of_token(const int32_t* __restrict__ qsl, int num_seqs, int64_t t) {
  int lo = 0, hi = num_seqs - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (qsl[mid] <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}

}  // namespace pkv
