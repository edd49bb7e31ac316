// Device helpers shared by the attention kernels.
//
// Pages cited by tag and function: P1 "vllm_omni/experimental/ar_diffusion/kv_cache/paged_attention.py",
// P2 "tests/diffusion/ar_diffusion/test_paged_attention.py",
// P3 "vllm_omni/diffusion/attention/backends/utils/piecewise_attn.py",
// P4 "vllm_omni/diffusion/diffusion_kv/paged_attention_adapter.py".
#pragma once

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
