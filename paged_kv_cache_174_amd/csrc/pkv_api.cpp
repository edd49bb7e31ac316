// C-ABI front end of libpkv: argument validation, kernel selection and launch,
// and the host-side metadata helpers (slot mapping, visible-window table,
// piecewise segments, metadata validation).
//
// Pages cited by tag and function: P1 "vllm_omni/experimental/ar_diffusion/kv_cache/paged_attention.py",
// P2 "tests/diffusion/ar_diffusion/test_paged_attention.py",
// P3 "vllm_omni/diffusion/attention/backends/utils/piecewise_attn.py",
// P4 "vllm_omni/diffusion/diffusion_kv/paged_attention_adapter.py".
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "pkv_internal.hpp"

namespace pkv {

namespace {
thread_local char g_error[1024] = "";
thread_local char g_plan[256] = "";
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kMaxDevices = 64;
int g_cu_count[kMaxDevices] = {0};

int cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
  if (g_cu_count[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    g_cu_count[dev] = n;
  }
  return g_cu_count[dev];
}

int64_t dtype_size(int dt) { return dt == PKV_F32 ? 4 : dt == PKV_BF16 ? 2 : dt == PKV_FP8_E4M3 ? 1 : 0; }

int check_pools(const pkv_pools* p) {
  if (!p) return fail(PKV_EINVAL, "pools is NULL");
  if (!p->key || !p->value) return fail(PKV_EINVAL, "pool pointers must not be NULL");
  if (dtype_size(p->dtype) == 0) return fail(PKV_EINVAL, "unknown pool dtype %d", p->dtype);
  if (p->block_size != 16) return fail(PKV_EUNSUPPORTED, "block_size %d: the kernels page in 16-token blocks", p->block_size);
  if (p->num_blocks <= 0 || p->num_kv_heads <= 0 || p->head_dim <= 0)
    return fail(PKV_EINVAL, "pool sizes must be positive (blocks %lld, kv heads %d, head_dim %d)",
                static_cast<long long>(p->num_blocks), p->num_kv_heads, p->head_dim);
  if ((static_cast<int64_t>(p->num_kv_heads) * p->head_dim) % 16 != 0)
    return fail(PKV_EUNSUPPORTED, "num_kv_heads * head_dim must be a multiple of 16");
  if (p->dtype == PKV_FP8_E4M3) {
    if (!(p->k_scale > 0.f) || !(p->v_scale > 0.f) || !std::isfinite(p->k_scale) || !std::isfinite(p->v_scale))
      return fail(PKV_EINVAL, "fp8 pools need positive finite k_scale and v_scale");
  }
  return PKV_OK;
}

// Workspace bytes per query row and key split: the bf16 partial output
// (head_dim 128), then the fp32 (max, sum) pair, in two regions.
constexpr int64_t kPartialRowBytes = 128 * 2 + 2 * 4;

struct SplitPlan {
  int row_tiles;
  int splits;
  int split_len;
  bool short_rows;  // the short-query kernel (at most kShortRows rows per KV head)
  bool packed;      // short rows: the launch hands out real work first (see plan_short_packed)
  // Long bf16 kernel: 64-key tiles of each split, non-increasing (the last
  // split also runs on to max_seq_len).  Other kernels: split_len keys each.
  int tiles[kMaxSplits];
};

// Number of key splits for the MFMA kernel.  One workgroup occupies a CU, so
// the launch runs in ceil(workgroups / CUs) rounds of roughly equal
// workgroups; splitting the key range shortens each workgroup but costs the
// partial results' round trip through memory and a combine launch.  Pick the
// split count with the smallest modelled time, never cutting the key range
// below 512 keys and never needing more workspace than the caller gave.
// Short query chunks with the sequences' lengths known on the host: every
// (sequence, KV head) is cut into ceil(len / L) key ranges of L keys, and the
// launch hands these ranges out first, ahead of the empty ones, so that they
// spread over all CUs.  L (a multiple of the short kernel's 128-key step) is
// the one with the smallest modelled time: rounds of one workgroup per CU,
// each streaming its L keys at a measured per-CU rate after a fixed start-up
// cost, plus the partials' round trip.
constexpr int kMaxPackedSeqs = 64;  // the kernel finds its work by scanning the sequences
bool plan_short_packed(SplitPlan& p, int64_t num_q_tokens, int num_q_heads, int num_kv_heads, int num_seqs,
                       int max_seq_len, const int32_t* host_lens, size_t workspace_bytes, bool have_workspace,
                       int kv_elem_bytes) {
  if (!host_lens || num_seqs > kMaxPackedSeqs || !have_workspace) return false;
  const int cus = cu_count();
  const int64_t per_split_bytes = num_q_tokens * num_q_heads * kPartialRowBytes;
  constexpr double kCuBytesPerS = 20e9;  // K+V streamed by one short-kernel workgroup
  constexpr double kWgStart = 4e-6;      // s: start-up and epilogue of one workgroup
  constexpr double kPartialBw = 5.0e12;
  constexpr double kCombineLaunch = 3e-6;
  constexpr int kStep = 128;
  const double key_bytes = 2.0 * 128 * kv_elem_bytes;
  const int l_min = std::max(kStep, (max_seq_len + kMaxSplits - 1) / kMaxSplits);
  double best_t = 1e30;
  int best_l = 0;
  for (int L = (l_min + kStep - 1) / kStep * kStep; L <= kMaxSplitKeys - kStep; L += kStep) {
    const int splits = (max_seq_len + L - 1) / L;
    if (splits > 1 && workspace_bytes < static_cast<size_t>(per_split_bytes) * splits) {
      if (L >= max_seq_len) break;
      continue;
    }
    int64_t items = 0;
    for (int b = 0; b < num_seqs; ++b) items += (std::max(host_lens[b], 1) + L - 1) / L;
    items *= num_kv_heads;
    const double rounds = std::ceil(static_cast<double>(items) / cus);
    double t = rounds * (L * key_bytes / kCuBytesPerS + kWgStart);
    if (splits > 1) t += 2.0 * per_split_bytes * splits / kPartialBw + kCombineLaunch;
    if (t < best_t * 0.98) {
      best_t = t;
      best_l = L;
    }
    if (L >= max_seq_len) break;
  }
  if (best_l == 0) return false;
  p.split_len = best_l;
  p.splits = (max_seq_len + best_l - 1) / best_l;
  p.packed = p.splits > 1;
  for (int z = 0; z < p.splits && z < kMaxSplits; ++z) p.tiles[z] = best_l / kMfmaKeyTile;
  return true;
}

// The long bf16 kernel's launch, modelled.  XCD x runs the workgroups of the
// (sequence, KV head) groups x, x + 8, ..., split by split (see the kernel's
// work mapping).  A workgroup costs a fixed start-up and epilogue plus a time
// per 64-key tile (6 us and 1.5 us at the sustained clock, fitted to launches
// of the frame and 40-layer workloads).  How the XCD hands workgroups to its
// CUs is not documented, and measurements fit neither of two simple rules on
// every plan: the next workgroup to the first CU to come free, or workgroups
// dealt in turn to four groups of CUs, each taking its next one on its first
// free CU.  The model takes the later of the two finishing times, which ranked
// every measured plan in the right order.  With more than eight workgroups per
// CU the order hardly matters and the model is the fluid bound (the work
// spread evenly, plus half the longest workgroup).  Returns the busiest XCD's
// time.
double model_long_launch(const int* tiles, int splits, int64_t groups_per_xcd, int row_tiles, int cus_per_xcd) {
  constexpr double kTile = 1.5e-6, kWorkgroup = 6e-6;
  constexpr int kCuGroups = 4;
  const int cus = std::max(kCuGroups, cus_per_xcd);
  if (groups_per_xcd * row_tiles * splits > 8LL * cus) {
    double total = 0.0, longest = 0.0;
    for (int z = 0; z < splits; ++z) {
      const double cost = tiles[z] * kTile + kWorkgroup;
      total += cost * static_cast<double>(groups_per_xcd * row_tiles);
      longest = std::max(longest, cost);
    }
    return total / cus + 0.5 * longest;
  }
  auto later = [](double x, double y) { return x > y; };
  std::vector<double> any(static_cast<size_t>(cus), 0.0);  // min-heaps of CU free times
  std::vector<std::vector<double>> dealt(kCuGroups, std::vector<double>(static_cast<size_t>(cus / kCuGroups), 0.0));
  auto take = [&](std::vector<double>& h, double cost) {
    std::pop_heap(h.begin(), h.end(), later);
    h.back() += cost;
    std::push_heap(h.begin(), h.end(), later);
  };
  const int64_t per_split = groups_per_xcd * row_tiles;
  int64_t i = 0;
  for (int z = 0; z < splits; ++z) {
    const double cost = tiles[z] * kTile + kWorkgroup;
    for (int64_t k = 0; k < per_split; ++k, ++i) {
      take(any, cost);
      take(dealt[static_cast<size_t>(i % kCuGroups)], cost);
    }
  }
  double t = *std::max_element(any.begin(), any.end());
  for (const auto& h : dealt) t = std::max(t, *std::max_element(h.begin(), h.end()));
  return t;
}

// Key splits of the long bf16 kernel.  Candidates: for each split count, the
// first splits of A tiles each and a last one of the remaining tiles (1 to A),
// so that the short last split's workgroups fill in where the launch's last
// round would leave CUs idle (A swept in about a dozen steps for two to four
// splits; equal splits for more, where the rounds are already short).  Each is scored by model_long_launch plus the
// partials' round trip; a split must buy a clear gain.  plan_len is the
// longest sequence (the host lengths when given, else max_seq_len); the last
// split runs on to max_seq_len, and no split may span more keys than a
// workgroup's block-table slice holds.
void plan_long_splits(SplitPlan& p, int64_t num_q_tokens, int num_q_heads, int num_kv_heads, int num_seqs,
                      int max_seq_len, int plan_len, size_t workspace_bytes, bool have_workspace) {
  const int cus = cu_count();
  const int64_t groups_per_xcd = (static_cast<int64_t>(num_seqs) * num_kv_heads + 7) / 8;
  const int64_t per_split_bytes = num_q_tokens * num_q_heads * kPartialRowBytes;
  constexpr double kPartialBw = 5.0e12;    // B/s for writing and re-reading the partials
  constexpr double kCombineLaunch = 3e-6;  // s
  const int T = (plan_len + kMfmaKeyTile - 1) / kMfmaKeyTile;
  const int max_sp = std::max(1, std::min(kMaxSplits, std::min(T, plan_len / 512)));
  double best_t = 1e30;
  int best_sp = 0, best_a = T;
  for (int sp = 1; sp <= max_sp; ++sp) {
    if (sp > 1 && (!have_workspace || workspace_bytes < static_cast<size_t>(per_split_bytes) * sp)) break;
    const int a_lo = (T + sp - 1) / sp, a_hi = (sp == 1 || sp > 4) ? a_lo : (T - 1) / (sp - 1);
    const int step = std::max(1, (a_hi - a_lo) / 12);
    for (int A = a_lo; A <= a_hi; A += step) {
      int tiles[kMaxSplits];
      for (int z = 0; z + 1 < sp; ++z) tiles[z] = A;
      tiles[sp - 1] = T - (sp - 1) * A;
      if (tiles[sp - 1] < 1 || tiles[sp - 1] > A) continue;
      // The last split's range, [cut, max_seq_len), must fit the table slice.
      if (max_seq_len - (sp - 1) * A * kMfmaKeyTile > kMaxSplitKeys || A * kMfmaKeyTile > kMaxSplitKeys) continue;
      double t = model_long_launch(tiles, sp, groups_per_xcd, p.row_tiles, cus / 8);
      if (sp > 1) t += 2.0 * per_split_bytes * sp / kPartialBw + kCombineLaunch;
      if (t < best_t * (sp > best_sp ? 0.98 : 1.0) || best_sp == 0) {
        best_t = t;
        best_sp = sp;
        best_a = A;
      }
    }
  }
  if (best_sp == 0) {
    // Nothing fits (no workspace for the splits the table slice needs, or more
    // than kMaxSplits of them): the smallest split count that fits the slice,
    // which the caller then refuses for want of a workspace or as unsupported.
    p.splits = (max_seq_len + kMaxSplitKeys - 1) / kMaxSplitKeys;
    p.split_len = kMaxSplitKeys / kMfmaKeyTile * kMfmaKeyTile;
    for (int z = 0; z < std::min(p.splits, kMaxSplits); ++z) p.tiles[z] = p.split_len / kMfmaKeyTile;
    return;
  }
  p.splits = best_sp;
  for (int z = 0; z < best_sp; ++z) p.tiles[z] = z + 1 < best_sp ? best_a : std::max(1, T - (best_sp - 1) * best_a);
  p.split_len = best_a * kMfmaKeyTile;
}

// Plans are cached per thread (the same metadata serves every layer of a
// step, and the long kernel's search is not free).
struct PlanKey {
  int64_t num_q_tokens;
  int num_q_heads, num_kv_heads, num_seqs, max_query_len, max_seq_len, plan_len, kv_elem_bytes, cus;
  int64_t host_hash;
  size_t workspace_bytes;
  bool have_workspace;
  bool operator==(const PlanKey& o) const {
    return num_q_tokens == o.num_q_tokens && num_q_heads == o.num_q_heads && num_kv_heads == o.num_kv_heads &&
           num_seqs == o.num_seqs && max_query_len == o.max_query_len && max_seq_len == o.max_seq_len &&
           plan_len == o.plan_len && kv_elem_bytes == o.kv_elem_bytes && cus == o.cus && host_hash == o.host_hash &&
           workspace_bytes == o.workspace_bytes && have_workspace == o.have_workspace;
  }
};

SplitPlan plan_splits_uncached(int64_t num_q_tokens, int num_q_heads, int num_kv_heads, int num_seqs,
                               int max_query_len, int max_seq_len, size_t workspace_bytes, bool have_workspace,
                               const int32_t* host_lens, int kv_elem_bytes, int plan_len) {
  SplitPlan p{};
  const int group = num_q_heads / num_kv_heads;
  p.short_rows = static_cast<int64_t>(max_query_len) * group <= kShortRows;
  p.row_tiles = static_cast<int>((static_cast<int64_t>(max_query_len) * group + kMfmaRows - 1) / kMfmaRows);
  if (p.short_rows && plan_short_packed(p, num_q_tokens, num_q_heads, num_kv_heads, num_seqs, max_seq_len, host_lens,
                                        workspace_bytes, have_workspace, kv_elem_bytes))
    return p;
  if (!p.short_rows && kv_elem_bytes == 2) {
    plan_long_splits(p, num_q_tokens, num_q_heads, num_kv_heads, num_seqs, max_seq_len, plan_len, workspace_bytes,
                     have_workspace);
    return p;
  }
  const int64_t base = static_cast<int64_t>(num_seqs) * num_kv_heads * p.row_tiles;
  const int cus = cu_count();
  const int max_by_len = std::max(1, max_seq_len / 512);
  const int64_t per_split_bytes = num_q_tokens * num_q_heads * kPartialRowBytes;
  constexpr double kCuFlops = 4.9e12;     // sustained FLOP/s of one CU on this kernel (about half of peak)
  constexpr double kPartialBw = 5.0e12;   // B/s for writing and re-reading the partials
  constexpr double kCombineLaunch = 3e-6; // s
  constexpr double kShortStep = 1.4e-6;   // s per four-tile step of the short-query kernel
  // A split's block-table slice is staged in LDS, which bounds its length.
  const int min_splits = static_cast<int>((static_cast<int64_t>(max_seq_len) + kMaxSplitKeys - 1) / kMaxSplitKeys);
  int best = min_splits;
  double best_t = 1e30;
  for (int sp = min_splits; sp <= std::max(min_splits, std::min(kMaxSplits, max_by_len)); ++sp) {
    if (sp > 1 && (!have_workspace || workspace_bytes < static_cast<size_t>(per_split_bytes) * sp)) break;
    const int64_t keys = ((max_seq_len + sp - 1) / sp + kMfmaKeyTile - 1) / kMfmaKeyTile * kMfmaKeyTile;
    // The short-query kernel takes four key tiles per step (one per key group).
    const double wg_time = p.short_rows ? std::ceil(keys / (4.0 * kMfmaKeyTile)) * kShortStep
                                        : static_cast<double>(kMfmaRows) * keys * 128 * 4 / kCuFlops;
    const double rounds = std::ceil(static_cast<double>(base) * sp / cus);
    double t = rounds * wg_time;
    if (sp > 1) t += 2.0 * per_split_bytes * sp / kPartialBw + kCombineLaunch;
    if (t < best_t * 0.98) {  // a split must buy a clear gain
      best_t = t;
      best = sp;
    }
  }
  p.splits = best;
  const int per = (max_seq_len + best - 1) / best;
  p.split_len = ((per + kMfmaKeyTile - 1) / kMfmaKeyTile) * kMfmaKeyTile;
  if (p.split_len <= 0) p.split_len = kMfmaKeyTile;
  for (int z = 0; z < p.splits && z < kMaxSplits; ++z) p.tiles[z] = p.split_len / kMfmaKeyTile;
  return p;
}

SplitPlan plan_splits(int64_t num_q_tokens, int num_q_heads, int num_kv_heads, int num_seqs, int max_query_len,
                      int max_seq_len, size_t workspace_bytes, bool have_workspace, const int32_t* host_lens = nullptr,
                      int kv_elem_bytes = 2) {
  PlanKey k{};
  k.num_q_tokens = num_q_tokens;
  k.num_q_heads = num_q_heads;
  k.num_kv_heads = num_kv_heads;
  k.num_seqs = num_seqs;
  k.max_query_len = max_query_len;
  k.max_seq_len = max_seq_len;
  k.kv_elem_bytes = kv_elem_bytes;
  k.cus = cu_count();
  k.workspace_bytes = workspace_bytes;
  k.have_workspace = have_workspace;
  // The long kernel plans from the longest sequence; the short kernel's packing
  // uses every length.
  int plan_len = max_seq_len;
  if (host_lens) {
    int longest = 1;
    uint64_t h = 1469598103934665603ull;
    for (int b = 0; b < num_seqs; ++b) {
      longest = std::max(longest, host_lens[b]);
      h = (h ^ static_cast<uint32_t>(host_lens[b])) * 1099511628211ull;
    }
    plan_len = std::min(longest, max_seq_len);
    k.host_hash = static_cast<int64_t>(h);
  }
  k.plan_len = plan_len;
  constexpr int kCache = 8;
  thread_local PlanKey keys[kCache];
  thread_local SplitPlan plans[kCache];
  thread_local int used = 0, next = 0;
  for (int i = 0; i < used; ++i)
    if (keys[i] == k) return plans[i];
  const SplitPlan p = plan_splits_uncached(num_q_tokens, num_q_heads, num_kv_heads, num_seqs, max_query_len,
                                           max_seq_len, workspace_bytes, have_workspace, host_lens, kv_elem_bytes,
                                           plan_len);
  keys[next] = k;
  plans[next] = p;
  next = (next + 1) % kCache;
  used = std::min(used + 1, kCache);
  return p;
}


// ---- argument checks and launches shared by the separate calls and the fused one

int write_setup(const void* key, const void* value, int32_t src_dtype, int64_t num_tokens, const int64_t* slot_mapping,
                const pkv_pools* pools, WriteArgs& a, int& mode) {
  if (int rc = check_pools(pools)) return rc;
  if (num_tokens < 0) return fail(PKV_EINVAL, "num_tokens must be >= 0");
  a = WriteArgs{key, value, slot_mapping, pools->key, pools->value, num_tokens,
                static_cast<int64_t>(pools->num_kv_heads) * pools->head_dim, pools->k_inv_scale, pools->v_inv_scale};
  if (num_tokens == 0) return PKV_OK;
  if (!key || !value || !slot_mapping) return fail(PKV_EINVAL, "key, value and slot_mapping must not be NULL");
  if (src_dtype == PKV_F32 && pools->dtype == PKV_F32) mode = 0;
  else if (src_dtype == PKV_BF16 && pools->dtype == PKV_BF16) mode = 1;
  else if (src_dtype == PKV_BF16 && pools->dtype == PKV_FP8_E4M3) mode = 2;
  else return fail(PKV_EUNSUPPORTED, "no write from dtype %d into a dtype %d pool", src_dtype, pools->dtype);
  return PKV_OK;
}

int write_launch(const WriteArgs& a, int mode, hipStream_t st) {
  if (a.num_tokens == 0) return PKV_OK;
  if (hipError_t e = launch_write(a, mode, st); e != hipSuccess)
    return fail(PKV_EHIP, "write launch failed: %s", hipGetErrorString(e));
  return PKV_OK;
}

int gather_setup(const pkv_pools* pools, const int32_t* block_ids, int32_t n_blocks, int32_t first_block,
                 void* stage_key, void* stage_value, GatherArgs& a) {
  if (int rc = check_pools(pools)) return rc;
  if (n_blocks < 0 || first_block < 0 || first_block > n_blocks)
    return fail(PKV_EINVAL, "need 0 <= first_block <= n_blocks (got first_block %d, n_blocks %d)", first_block, n_blocks);
  a = GatherArgs{pools->key, pools->value, block_ids, stage_key, stage_value, first_block, n_blocks,
                 static_cast<int64_t>(pools->block_size) * pools->num_kv_heads * pools->head_dim * dtype_size(pools->dtype)};
  if (first_block == n_blocks) return PKV_OK;
  if (!block_ids || !stage_key || !stage_value) return fail(PKV_EINVAL, "block_ids and staging buffers must not be NULL");
  return PKV_OK;
}

int gather_launch(const GatherArgs& a, hipStream_t st) {
  if (a.first_block == a.n_blocks) return PKV_OK;
  if (hipError_t e = launch_gather(a, st); e != hipSuccess)
    return fail(PKV_EHIP, "gather launch failed: %s", hipGetErrorString(e));
  return PKV_OK;
}

}  // namespace

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_error, sizeof(g_error), fmt, ap);
  va_end(ap);
  return code;
}

// P1 video_block_table: index ranges that can hold a kept token are the
// sink's blocks and every block from the one holding the recent window's
// first position to the last written one; a block is read whole, so its
// length is min(B, end - first_position), and only the last block read may be
// partly written.
int window_read(BlockAt block_at, const void* ctx, int64_t history_tokens, int64_t query_tokens,
                int64_t sink_tokens, int64_t window_tokens, int32_t block_size, int32_t* out_table,
                int32_t capacity, int32_t* out_count, int32_t* out_kv_len, int64_t* reads) {
  if (!out_table || !out_count || !out_kv_len) return fail(PKV_EINVAL, "NULL pointer");
  if (block_size <= 0 || history_tokens < 0 || query_tokens <= 0 || sink_tokens < 0)
    return fail(PKV_EINVAL, "bad sizes");
  if (window_tokens < query_tokens)
    return fail(PKV_EINVAL, "the recent window (%lld) must hold the current chunk (%lld)",
                static_cast<long long>(window_tokens), static_cast<long long>(query_tokens));
  const int64_t B = block_size;
  const int64_t end = history_tokens + query_tokens;
  const int64_t need_blocks = (end + B - 1) / B;
  const int64_t sink_end = std::min(sink_tokens, end);
  const int64_t sink_blocks = (sink_end + B - 1) / B;
  const int64_t recent_start = std::max<int64_t>(end - window_tokens, 0);
  const int64_t recent_first = std::max(recent_start / B, sink_blocks);
  int32_t count = 0;
  int64_t kv_len = 0;
  int64_t prev_len = B;
  auto take = [&](int64_t i) -> int {
    const int32_t blk = block_at(ctx, i);
    ++*reads;
    if (blk < 0) return PKV_OK;  // evicted: nothing of it is read
    if (prev_len != B)
      return fail(PKV_EWINDOW, "block %d is partly written but block %d follows it", out_table[count - 1], blk);
    if (count >= capacity) return fail(PKV_ERANGE, "table capacity %d too small", capacity);
    const int64_t len = std::min<int64_t>(B, end - i * B);
    out_table[count++] = blk;
    kv_len += len;
    prev_len = len;
    return PKV_OK;
  };
  for (int64_t i = 0; i < sink_blocks; ++i)
    if (int rc = take(i)) return rc;
  for (int64_t i = recent_first; i < need_blocks; ++i)
    if (int rc = take(i)) return rc;
  if (count == 0) return fail(PKV_EINVAL, "the window holds no resident block");
  if (kv_len > INT32_MAX) return fail(PKV_ERANGE, "window longer than 2^31 tokens");
  *out_count = count;
  *out_kv_len = static_cast<int32_t>(kv_len);
  return PKV_OK;
}

}  // namespace pkv

using namespace pkv;

extern "C" {

const char* pkv_last_error(void) { return g_error; }

const char* pkv_last_attn_plan(void) { return g_plan; }

const char* pkv_version(void) { return "pkv 0.1.0 (gfx950)"; }

int pkv_paged_write(const void* key, const void* value, int32_t src_dtype, int64_t num_tokens,
                    const int64_t* slot_mapping, const pkv_pools* pools, void* stream) {
  g_error[0] = '\0';
  WriteArgs a{};
  int mode = 0;
  if (int rc = write_setup(key, value, src_dtype, num_tokens, slot_mapping, pools, a, mode)) return rc;
  return write_launch(a, mode, static_cast<hipStream_t>(stream));
}

int pkv_gather(const pkv_pools* pools, const int32_t* block_ids, int32_t n_blocks, int32_t first_block,
               void* stage_key, void* stage_value, void* stream) {
  g_error[0] = '\0';
  GatherArgs a{};
  if (int rc = gather_setup(pools, block_ids, n_blocks, first_block, stage_key, stage_value, a)) return rc;
  return gather_launch(a, static_cast<hipStream_t>(stream));
}

size_t pkv_paged_attn_workspace_size(int64_t num_q_tokens, int32_t num_q_heads, int32_t num_kv_heads,
                                     int32_t head_dim, int32_t num_seqs, int32_t max_query_len,
                                     int32_t max_seq_len) {
  if (num_q_tokens <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads ||
      (head_dim != 64 && head_dim != 128) ||
      num_seqs <= 0 || max_query_len <= 0 || max_seq_len <= 0)
    return 0;
  SplitPlan p = plan_splits(num_q_tokens, num_q_heads, num_kv_heads, num_seqs, max_query_len, max_seq_len,
                            static_cast<size_t>(-1), true);
  // Short query chunks may be planned from the sequences' own lengths, with
  // up to kMaxSplits splits (their rows are few).
  const int splits = p.short_rows ? std::max(p.splits, std::min(kMaxSplits, (max_seq_len + 127) / 128)) : p.splits;
  if (splits <= 1) return 0;
  return static_cast<size_t>(splits) * static_cast<size_t>(num_q_tokens) * num_q_heads * kPartialRowBytes;
}

}  // extern "C"

namespace {

constexpr unsigned kPhaseMain = 1u, kPhaseMerge = 2u;

// Everything an attention launch needs beyond the kernel arguments.
struct AttnLaunch {
  AttnArgs a{};
  SplitPlan p{};
  bool f32 = false;
  bool fp8 = false;
  int max_query_len = 0;
};

// Validates the attention arguments and plans the key splits; enqueues nothing.
// kpool / vpool are the K/V the kernel reads: the pools, or contiguous staging
// buffers when block_table is null.
int attn_setup(const void* q, int32_t q_dtype, int64_t num_q_tokens, int32_t num_q_heads, const pkv_pools* pools,
               const void* kpool, const void* vpool, const int32_t* block_table, int32_t table_width,
               const int32_t* query_start_loc, const int32_t* seq_lens, int32_t num_seqs, int32_t max_query_len,
               int32_t max_seq_len, const int32_t* segments, const int32_t* segment_start_loc,
               const int32_t* seq_order, const int32_t* query_pos, const int32_t* host_lens, float softmax_scale,
               void* out, void* workspace, size_t workspace_bytes, AttnLaunch& L) {
  if (int rc = check_pools(pools)) return rc;
  if (!q || !out || !query_start_loc || !seq_lens || !segments || !segment_start_loc)
    return fail(PKV_EINVAL, "q, out and every metadata pointer must be non-NULL");
  if (num_seqs <= 0) return fail(PKV_EINVAL, "num_seqs must be positive");
  if (num_q_tokens <= 0) return fail(PKV_EINVAL, "num_q_tokens must be positive");
  if (num_q_heads <= 0 || num_q_heads % pools->num_kv_heads)
    return fail(PKV_EINVAL, "num_q_heads (%d) must be a positive multiple of num_kv_heads (%d)", num_q_heads,
                pools->num_kv_heads);
  if (max_query_len <= 0 || max_seq_len <= 0 || max_query_len > max_seq_len)
    return fail(PKV_EINVAL, "need 0 < max_query_len <= max_seq_len (got %d, %d)", max_query_len, max_seq_len);
  if (block_table) {
    if (table_width <= 0) return fail(PKV_EINVAL, "table_width must be positive");
    if (static_cast<int64_t>(max_seq_len) > static_cast<int64_t>(table_width) * pools->block_size)
      return fail(PKV_EINVAL, "max_seq_len %d exceeds what a %d-entry block table can address", max_seq_len,
                  table_width);
  }
  if (!(softmax_scale > 0.f) || !std::isfinite(softmax_scale))
    return fail(PKV_EINVAL, "softmax_scale must be positive and finite");
  const bool f32 = pools->dtype == PKV_F32;
  if (f32 ? q_dtype != PKV_F32 : q_dtype != PKV_BF16)
    return fail(PKV_EINVAL, "query dtype %d does not go with pool dtype %d (f32 with f32, bf16 with bf16 or fp8)",
                q_dtype, pools->dtype);

  AttnArgs& a = L.a;
  a = AttnArgs{};
  a.q = q;
  a.out = out;
  a.kpool = kpool;
  a.vpool = vpool;
  a.block_table = block_table;
  a.qsl = query_start_loc;
  a.seq_lens = seq_lens;
  a.segments = segments;
  a.seg_loc = segment_start_loc;
  a.seq_order = seq_order;
  a.query_pos = query_pos;
  a.num_q_tokens = num_q_tokens;
  a.table_width = table_width;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = pools->num_kv_heads;
  a.group = num_q_heads / pools->num_kv_heads;
  a.head_dim = pools->head_dim;
  a.block_size = pools->block_size;
  const float k_scale = pools->dtype == PKV_FP8_E4M3 ? pools->k_scale : 1.f;
  a.v_scale = pools->dtype == PKV_FP8_E4M3 ? pools->v_scale : 1.f;
  a.scale_log2 = softmax_scale * k_scale * kLog2e;
  L.f32 = f32;
  L.fp8 = pools->dtype == PKV_FP8_E4M3;
  L.max_query_len = max_query_len;

  if (f32) {
    if (pools->head_dim != 64 && pools->head_dim != 128)
      return fail(PKV_EUNSUPPORTED, "f32 attention supports head_dim 64 and 128, not %d", pools->head_dim);
    a.num_splits = 1;
    a.row_tiles = 0;
    a.split_len = 0;
    L.p = SplitPlan{};
    L.p.splits = 1;
    std::snprintf(g_plan, sizeof(g_plan), "f32");
    return PKV_OK;
  }
  if (pools->head_dim != 64 && pools->head_dim != 128)
    return fail(PKV_EUNSUPPORTED, "bf16/fp8 attention supports head_dim 64 and 128, not %d", pools->head_dim);
  const SplitPlan p = plan_splits(num_q_tokens, num_q_heads, pools->num_kv_heads, num_seqs, max_query_len,
                                  max_seq_len, workspace_bytes, workspace != nullptr, host_lens,
                                  pools->dtype == PKV_FP8_E4M3 ? 1 : 2);
  if (p.splits > kMaxSplits)
    return fail(PKV_EUNSUPPORTED, "max_seq_len %d needs more than %d key splits", max_seq_len, kMaxSplits);
  if (p.splits > 1 &&
      (!workspace ||
       workspace_bytes < static_cast<size_t>(p.splits) * num_q_tokens * num_q_heads * kPartialRowBytes))
    return fail(PKV_EINVAL, "max_seq_len %d needs %d key splits and a workspace of pkv_paged_attn_workspace_size() bytes",
                max_seq_len, p.splits);
  L.p = p;
  a.row_tiles = p.row_tiles;
  a.num_splits = p.splits;
  a.split_len = p.split_len;
  a.packed = p.packed ? 1 : 0;
  for (int z = 0, cut = 0; z <= p.splits; ++z) {
    a.split_cut[z] = z == p.splits ? max_seq_len : std::min(cut, max_seq_len);
    if (z < p.splits) cut += p.tiles[z] * kMfmaKeyTile;
  }
  std::snprintf(g_plan, sizeof(g_plan), "%s splits=%d split_len=%d row_tiles=%d packed=%d",
                !L.fp8 && !p.short_rows ? "long" : p.short_rows ? "short" : "fp8", p.splits, p.split_len,
                p.row_tiles, p.packed ? 1 : 0);
  if (!L.fp8 && !p.short_rows && p.splits > 1) {
    for (int z = 1; z < p.splits; ++z) {
      const size_t n = std::strlen(g_plan);
      if (n + 16 >= sizeof(g_plan)) break;
      std::snprintf(g_plan + n, sizeof(g_plan) - n, z > 1 ? ",%d" : " cut=%d", a.split_cut[z]);
    }
  }
  if (p.splits > 1) {
    const int64_t rows = num_q_tokens * num_q_heads;
    a.ws_o = static_cast<float*>(workspace);
    a.ws_ml = reinterpret_cast<float*>(static_cast<char*>(workspace) + static_cast<int64_t>(p.splits) * rows * 128 * 2);
  }
  return PKV_OK;
}

// Launches the phases asked for: the attention kernel (kPhaseMain) and, when
// the keys are split, the merge of the partial results (kPhaseMerge).
int attn_launch(const AttnLaunch& L, unsigned phases, hipStream_t st) {
  if (L.f32) {
    if (phases & kPhaseMain) {
      if (hipError_t e = launch_attn_f32(L.a, L.max_query_len, st); e != hipSuccess)
        return fail(PKV_EHIP, "attention launch failed: %s", hipGetErrorString(e));
    }
    return PKV_OK;
  }
  if (phases & kPhaseMain) {
    // bf16 chunks of more than kShortRows rows per KV head: the one-wave-per-SIMD
    // kernel; fp8 pools and short chunks: the two-waves-per-SIMD kernels.
    const hipError_t e = (!L.fp8 && !L.p.short_rows) ? launch_attn_long(L.a, st)
                                                      : launch_attn_mfma(L.a, L.fp8, L.p.short_rows, st);
    if (e != hipSuccess)
      return fail(PKV_EHIP, "attention launch failed: %s", hipGetErrorString(e));
  }
  if ((phases & kPhaseMerge) && L.p.splits > 1) {
    if (hipError_t e = launch_attn_combine(L.a, st); e != hipSuccess)
      return fail(PKV_EHIP, "split combine launch failed: %s", hipGetErrorString(e));
  }
  return PKV_OK;
}

int paged_attn_impl(const void* q, int32_t q_dtype, int64_t num_q_tokens, int32_t num_q_heads,
                    const pkv_pools* pools, const int32_t* block_table, int32_t table_width,
                    const int32_t* query_start_loc, const int32_t* seq_lens, int32_t num_seqs,
                    int32_t max_query_len, int32_t max_seq_len, const int32_t* segments,
                    const int32_t* segment_start_loc, const int32_t* seq_order, const int32_t* host_seq_lens,
                    float softmax_scale, void* out, void* workspace, size_t workspace_bytes, void* stream,
                    unsigned phases) {
  g_error[0] = '\0';
  if (!block_table) return fail(PKV_EINVAL, "block_table must not be NULL");
  if (!pools) return fail(PKV_EINVAL, "pools is NULL");
  AttnLaunch L;
  if (int rc = attn_setup(q, q_dtype, num_q_tokens, num_q_heads, pools, pools->key, pools->value, block_table,
                          table_width, query_start_loc, seq_lens, num_seqs, max_query_len, max_seq_len, segments,
                          segment_start_loc, seq_order, nullptr, host_seq_lens, softmax_scale, out, workspace,
                          workspace_bytes, L))
    return rc;
  return attn_launch(L, phases, static_cast<hipStream_t>(stream));
}

}  // namespace

extern "C" {

#define PKV_ATTN_PARAMS                                                                                        \
  const void *q, int32_t q_dtype, int64_t num_q_tokens, int32_t num_q_heads, const pkv_pools *pools,          \
      const int32_t *block_table, int32_t table_width, const int32_t *query_start_loc, const int32_t *seq_lens, \
      int32_t num_seqs, int32_t max_query_len, int32_t max_seq_len, const int32_t *segments,                    \
      const int32_t *segment_start_loc, const int32_t *seq_order, const int32_t *host_seq_lens, float softmax_scale, \
      void *out, void *workspace, size_t workspace_bytes, void *stream
#define PKV_ATTN_ARGS                                                                                       \
  q, q_dtype, num_q_tokens, num_q_heads, pools, block_table, table_width, query_start_loc, seq_lens,         \
      num_seqs, max_query_len, max_seq_len, segments, segment_start_loc, seq_order, host_seq_lens, softmax_scale, \
      out, workspace, workspace_bytes, stream

int pkv_paged_attn(PKV_ATTN_PARAMS) { return paged_attn_impl(PKV_ATTN_ARGS, kPhaseMain | kPhaseMerge); }
int pkv_paged_attn_main(PKV_ATTN_PARAMS) { return paged_attn_impl(PKV_ATTN_ARGS, kPhaseMain); }
int pkv_paged_attn_merge(PKV_ATTN_PARAMS) { return paged_attn_impl(PKV_ATTN_ARGS, kPhaseMerge); }

#undef PKV_ATTN_PARAMS
#undef PKV_ATTN_ARGS

// P1 _paged_write_attn_impl (the per-layer op: slot writes of the current
// video and action K/V, then attention) and ar_diffusion_paged_attention's
// staged branch (_stage_window into caller-owned buffers, then attention over
// them as one contiguous run).
int pkv_paged_write_attn(const void* q, int32_t q_dtype, int64_t num_q_tokens, int32_t num_q_heads,
                         const void* key, const void* value, int32_t kv_dtype, int64_t num_tokens,
                         const int64_t* slot_mapping, const void* action_key, const void* action_value,
                         int64_t num_action_tokens, const int64_t* action_slot_mapping, const pkv_pools* pools,
                         const pkv_attn_meta* meta, const pkv_staging* staging, float softmax_scale, void* out,
                         void* workspace, size_t workspace_bytes, void* stream) {
  g_error[0] = '\0';
  if (!meta) return fail(PKV_EINVAL, "meta is NULL");
  if (!pools) return fail(PKV_EINVAL, "pools is NULL");
  if (!meta->block_table) return fail(PKV_EINVAL, "meta->block_table must not be NULL");
  WriteArgs wv{}, wa{};
  int mode_v = 0, mode_a = 0;
  if (int rc = write_setup(key, value, kv_dtype, num_tokens, slot_mapping, pools, wv, mode_v)) return rc;
  if (int rc = write_setup(action_key, action_value, kv_dtype, num_action_tokens, action_slot_mapping, pools, wa,
                           mode_a))
    return rc;
  GatherArgs ga{};
  const void* kread = pools->key;
  const void* vread = pools->value;
  const int32_t* table = meta->block_table;
  if (staging) {
    const int B = pools->block_size;
    if (meta->num_seqs != 1)
      return fail(PKV_EINVAL, "staged attention covers one sequence, not %d", meta->num_seqs);
    if (meta->max_seq_len <= 0 || meta->max_seq_len % B)
      return fail(PKV_EINVAL, "staged attention needs a block-aligned max_seq_len, got %d", meta->max_seq_len);
    const int32_t n_blocks = meta->max_seq_len / B;
    if (n_blocks > meta->table_width)
      return fail(PKV_EINVAL, "max_seq_len %d exceeds the %d-entry block table", meta->max_seq_len, meta->table_width);
    if (staging->capacity_tokens < meta->max_seq_len)
      return fail(PKV_EINVAL, "staging buffers hold %lld tokens but this call stages %d",
                  static_cast<long long>(staging->capacity_tokens), meta->max_seq_len);
    const int32_t first = staging->first_block;
    if (first != 0) {
      // Reuse: blocks [0, first) already hold this window; only the current
      // chunk's whole blocks are refreshed.
      const int64_t cur_blocks = num_tokens / B;
      if (num_tokens <= 0 || cur_blocks * B != num_tokens)
        return fail(PKV_EINVAL, "staged reuse needs a block-aligned current chunk, got %lld tokens",
                    static_cast<long long>(num_tokens));
      if (first < 0 || first + cur_blocks > n_blocks)
        return fail(PKV_EINVAL, "first_block %d + %lld current blocks exceeds the %d-block window", first,
                    static_cast<long long>(cur_blocks), n_blocks);
    }
    if (int rc = gather_setup(pools, meta->block_table, n_blocks, first, staging->stage_key, staging->stage_value, ga))
      return rc;
    kread = staging->stage_key;
    vread = staging->stage_value;
    table = nullptr;
  }
  AttnLaunch L;
  if (int rc = attn_setup(q, q_dtype, num_q_tokens, num_q_heads, pools, kread, vread, table, meta->table_width,
                          meta->query_start_loc, meta->seq_lens, meta->num_seqs, meta->max_query_len,
                          meta->max_seq_len, meta->segments, meta->segment_start_loc, meta->seq_order,
                          meta->query_pos, meta->host_seq_lens, softmax_scale,
                          out, workspace, workspace_bytes, L))
    return rc;
  // Everything is checked; enqueue in order on one stream.
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (int rc = write_launch(wv, mode_v, st)) return rc;
  if (int rc = write_launch(wa, mode_a, st)) return rc;
  if (staging) {
    if (int rc = gather_launch(ga, st)) return rc;
  }
  return attn_launch(L, kPhaseMain | kPhaseMerge, st);
}

// ------------------------------------------------------------------ host metadata

int pkv_slot_mapping(const int32_t* block_ids, int64_t num_block_ids, int64_t first_position, int64_t num_tokens,
                     int32_t block_size, int64_t* out_slots) {
  g_error[0] = '\0';
  if (block_size <= 0) return fail(PKV_EINVAL, "block_size must be positive");
  if (num_tokens < 0 || first_position < 0) return fail(PKV_EINVAL, "positions must be non-negative");
  if (num_tokens == 0) return PKV_OK;
  if (!block_ids || !out_slots) return fail(PKV_EINVAL, "NULL pointer");
  for (int64_t t = 0; t < num_tokens; ++t) {
    const int64_t p = first_position + t;
    const int64_t bi = p / block_size;
    if (bi >= num_block_ids) return fail(PKV_EINVAL, "position %lld needs block index %lld of %lld",
                                         static_cast<long long>(p), static_cast<long long>(bi),
                                         static_cast<long long>(num_block_ids));
    const int64_t blk = block_ids[bi];
    if (blk < 0) return fail(PKV_EINVAL, "position %lld falls in a non-resident block", static_cast<long long>(p));
    out_slots[t] = blk * block_size + p % block_size;
  }
  return PKV_OK;
}

int pkv_window_table(const int32_t* block_ids, int64_t num_block_ids, int64_t history_tokens, int64_t query_tokens,
                     int64_t sink_tokens, int64_t window_tokens, int32_t block_size, int32_t* out_table,
                     int32_t capacity, int32_t* out_count, int32_t* out_kv_len) {
  g_error[0] = '\0';
  if (!block_ids || !out_table || !out_count || !out_kv_len) return fail(PKV_EINVAL, "NULL pointer");
  if (block_size <= 0 || history_tokens < 0 || query_tokens <= 0) return fail(PKV_EINVAL, "bad sizes");
  const int64_t need_blocks = (history_tokens + query_tokens + block_size - 1) / block_size;
  if (num_block_ids < need_blocks)
    return fail(PKV_EINVAL, "%lld block ids given, %lld needed", static_cast<long long>(num_block_ids),
                static_cast<long long>(need_blocks));
  int64_t reads = 0;
  return window_read([](const void* ctx, int64_t i) { return static_cast<const int32_t*>(ctx)[i]; }, block_ids,
                     history_tokens, query_tokens, sink_tokens, window_tokens, block_size, out_table, capacity,
                     out_count, out_kv_len, &reads);
}

// P1 build_block_table: action K/V sits in scratch blocks listed after the
// video window, and the kernel reads table and length as one run.
int pkv_action_table(int32_t* table, int32_t capacity, int32_t* count, int32_t* kv_len,
                     const int32_t* action_block_ids, int32_t num_action_block_ids, int64_t action_tokens,
                     int32_t block_size) {
  g_error[0] = '\0';
  if (!table || !count || !kv_len) return fail(PKV_EINVAL, "NULL pointer");
  if (block_size <= 0 || action_tokens < 0 || *count < 0 || *kv_len < 0) return fail(PKV_EINVAL, "bad sizes");
  if (action_tokens == 0) return PKV_OK;
  // A video run that stops inside its last block would make the kernel read
  // that block's unwritten slots as the first action tokens.
  if (*kv_len % block_size)
    return fail(PKV_EINVAL,
                "action tokens cannot follow a partly written video block: the video run ends %d slots into its "
                "last block",
                *kv_len % block_size);
  const int64_t nb = (action_tokens + block_size - 1) / block_size;
  if (!action_block_ids || num_action_block_ids < nb)
    return fail(PKV_EINVAL, "%lld action tokens need %lld scratch blocks, got %d", static_cast<long long>(action_tokens),
                static_cast<long long>(nb), num_action_block_ids);
  if (*count + nb > capacity)
    return fail(PKV_ERANGE, "table capacity %d is too small for %lld entries", capacity,
                static_cast<long long>(*count + nb));
  for (int64_t i = 0; i < nb; ++i) {
    if (action_block_ids[i] < 0) return fail(PKV_EINVAL, "negative action block id");
    table[*count + i] = action_block_ids[i];
  }
  *count += static_cast<int32_t>(nb);
  *kv_len += static_cast<int32_t>(action_tokens);
  return PKV_OK;
}

int pkv_window_capacity(int64_t sink_tokens, int64_t window_tokens, int32_t chunk_size, int32_t block_size,
                        int64_t action_tokens, int64_t* out_blocks) {
  g_error[0] = '\0';
  if (!out_blocks) return fail(PKV_EINVAL, "NULL pointer");
  if (block_size <= 0 || chunk_size <= 0 || sink_tokens < 0 || window_tokens < 0 || action_tokens < 0)
    return fail(PKV_EINVAL, "bad sizes");
  int64_t g = chunk_size, r = block_size;  // gcd(chunk_size, block_size)
  while (r) {
    const int64_t t = g % r;
    g = r;
    r = t;
  }
  const int64_t lead = block_size - g;  // furthest a chunk boundary sits past a block edge
  const int64_t sink_blocks = (sink_tokens + block_size - 1) / block_size;
  const int64_t recent_blocks = (window_tokens + lead + block_size - 1) / block_size;
  const int64_t action_blocks = std::max<int64_t>(1, (action_tokens + block_size - 1) / block_size);
  *out_blocks = sink_blocks + recent_blocks + action_blocks;
  return PKV_OK;
}

int pkv_build_segments(const int32_t* full_spans, int32_t num_spans, int32_t query_offset, int32_t query_len,
                       int32_t* out_segments, int32_t capacity, int32_t* out_count) {
  g_error[0] = '\0';
  if (!out_segments || !out_count || (num_spans > 0 && !full_spans)) return fail(PKV_EINVAL, "NULL pointer");
  if (query_len <= 0 || query_offset < 0 || num_spans < 0) return fail(PKV_EINVAL, "bad query range or span count");
  int32_t prev_end = 0;
  for (int32_t k = 0; k < num_spans; ++k) {
    const int32_t a = full_spans[2 * k], b = full_spans[2 * k + 1];
    if (a < prev_end || a < 0 || a >= b)
      return fail(PKV_EINVAL, "full spans must be sorted, non-empty and non-overlapping (span %d = [%d, %d))", k, a, b);
    prev_end = b;
  }
  // The mask rule (P3 module docstring): a query row inside a full span
  // [a, b) attends K[:b]; every other row belongs to a causal segment [s, e)
  // that attends K[:e] bottom-right aligned.  Sweep the span edges that fall
  // strictly inside the query range: between two consecutive edges every row
  // has the same rule, and neighbouring pieces with the same rule (the rows
  // outside spans, or one span's rows) are one segment.
  const int32_t lo = query_offset, hi = query_offset + query_len;
  std::vector<int32_t> edges{lo, hi};
  for (int32_t k = 0; k < num_spans; ++k)
    for (int32_t e : {full_spans[2 * k], full_spans[2 * k + 1]})
      if (e > lo && e < hi) edges.push_back(e);
  std::sort(edges.begin(), edges.end());
  edges.erase(std::unique(edges.begin(), edges.end()), edges.end());
  int32_t n = 0;
  int32_t span = 0;  // first span that does not end at or before the current piece
  for (size_t i = 0; i + 1 < edges.size(); ++i) {
    const int32_t p0 = edges[i], p1 = edges[i + 1];
    while (span < num_spans && full_spans[2 * span + 1] <= p0) ++span;
    const bool full = span < num_spans && full_spans[2 * span] <= p0;
    const int32_t mode = full ? PKV_SEG_FULL : PKV_SEG_CAUSAL;
    const int32_t kv = full ? full_spans[2 * span + 1] : p1;
    int32_t* last = n > 0 ? out_segments + 4 * (n - 1) : nullptr;
    if (last && last[3] == mode && (mode == PKV_SEG_CAUSAL || last[2] == kv)) {
      last[1] = p1;
      if (mode == PKV_SEG_CAUSAL) last[2] = p1;
      continue;
    }
    if (n >= capacity) return fail(PKV_ERANGE, "segment capacity %d too small", capacity);
    int32_t* seg = out_segments + 4 * n++;
    seg[0] = p0;
    seg[1] = p1;
    seg[2] = kv;
    seg[3] = mode;
  }
  *out_count = n;
  return PKV_OK;
}

// P1 _prepare_history_staging, restated: a staged window may be kept when
// the buffers were last filled for the same request and nothing they hold
// has moved since -- the history (its length and the blocks the window lists
// for it), the staged extent and the chunk length -- and the chunk owns its
// blocks outright (it starts on a block edge and fills whole blocks).  Then
// only the chunk's blocks, after the history's, are gathered again.
int pkv_staging_decide(pkv_staging_state* st, int64_t session, const int32_t* table, int32_t table_len,
                       int64_t history_tokens, int64_t chunk_tokens, int32_t max_seq_len, int32_t block_size,
                       int64_t capacity_tokens, int32_t* out_reuse, int32_t* out_first_block) {
  g_error[0] = '\0';
  if (!st || !out_reuse || !out_first_block || (table_len > 0 && !table) ||
      (st->block_capacity > 0 && !st->history_blocks))
    return fail(PKV_EINVAL, "NULL pointer");
  if (session < 0 || table_len < 0 || history_tokens < 0 || chunk_tokens <= 0 || block_size <= 0 ||
      max_seq_len <= 0 || st->block_capacity < 0)
    return fail(PKV_EINVAL, "bad sizes");
  if (max_seq_len > capacity_tokens)
    return fail(PKV_ERANGE, "the staging buffers hold %lld tokens but this forward stages %d",
                static_cast<long long>(capacity_tokens), max_seq_len);
  const int64_t offset = history_tokens % block_size;  // where the chunk starts in its first block
  const int64_t chunk_blocks = (offset + chunk_tokens + block_size - 1) / block_size;
  if (chunk_blocks > table_len)
    return fail(PKV_EINVAL, "a %d-entry table cannot hold a chunk spanning %lld blocks", table_len,
                static_cast<long long>(chunk_blocks));
  const int32_t hist_blocks = table_len - static_cast<int32_t>(chunk_blocks);
  if (hist_blocks > st->block_capacity)
    return fail(PKV_ERANGE, "the visible history lists %d blocks; the state records at most %d", hist_blocks,
                st->block_capacity);
  const bool chunk_owns_blocks = offset == 0 && chunk_tokens % block_size == 0;
  const bool unchanged = st->session == session && st->history_tokens == history_tokens &&
                         st->chunk_tokens == chunk_tokens && st->max_seq_len == max_seq_len &&
                         st->num_history_blocks == hist_blocks &&
                         std::equal(table, table + hist_blocks, st->history_blocks);
  const bool reuse = chunk_owns_blocks && unchanged;
  st->session = session;
  st->history_tokens = history_tokens;
  st->chunk_tokens = chunk_tokens;
  st->max_seq_len = max_seq_len;
  st->num_history_blocks = hist_blocks;
  std::copy(table, table + hist_blocks, st->history_blocks);
  *out_reuse = reuse ? 1 : 0;
  *out_first_block = reuse ? hist_blocks : 0;
  return PKV_OK;
}

int pkv_validate_metadata_host(const int32_t* qsl, const int32_t* seq_lens, int32_t num_seqs,
                               const int32_t* block_table, int32_t table_width, int64_t num_blocks,
                               int32_t block_size, int32_t max_query_len, int32_t max_seq_len,
                               const int32_t* segments, const int32_t* seg_loc, const int32_t* query_pos) {
  g_error[0] = '\0';
  if (!qsl || !seq_lens || !block_table || !segments || !seg_loc) return fail(PKV_EINVAL, "NULL pointer");
  if (num_seqs <= 0 || table_width <= 0 || block_size <= 0) return fail(PKV_EINVAL, "bad sizes");
  if (qsl[0] != 0) return fail(PKV_EINVAL, "query_start_loc[0] must be 0");
  if (seg_loc[0] != 0) return fail(PKV_EINVAL, "segment_start_loc[0] must be 0");
  for (int32_t b = 0; b < num_seqs; ++b) {
    const int32_t q = qsl[b + 1] - qsl[b];
    const int32_t s = seq_lens[b];
    if (q < 1) return fail(PKV_EINVAL, "sequence %d: query length %d must be >= 1", b, q);
    if (s < q) return fail(PKV_EINVAL, "sequence %d: seq_len %d shorter than its query %d", b, s, q);
    if (q > max_query_len) return fail(PKV_EINVAL, "sequence %d: query length %d > max_query_len %d", b, q, max_query_len);
    if (s > max_seq_len) return fail(PKV_EINVAL, "sequence %d: seq_len %d > max_seq_len %d", b, s, max_seq_len);
    const int64_t nb = (static_cast<int64_t>(s) + block_size - 1) / block_size;
    if (nb > table_width) return fail(PKV_EINVAL, "sequence %d: %lld blocks do not fit a %d-wide table", b,
                                      static_cast<long long>(nb), table_width);
    for (int64_t i = 0; i < nb; ++i) {
      const int32_t blk = block_table[static_cast<int64_t>(b) * table_width + i];
      if (blk < 0 || blk >= num_blocks)
        return fail(PKV_EINVAL, "sequence %d: table entry %lld = %d outside the pool", b, static_cast<long long>(i), blk);
    }
    // The query rows sit at key positions [g0, g0 + q): the suffix, or a shard.
    const int32_t g0 = query_pos ? query_pos[b] : s - q;
    if (g0 < 0 || static_cast<int64_t>(g0) + q > s)
      return fail(PKV_EINVAL, "sequence %d: query rows [%d, %lld) lie outside its %d keys", b, g0,
                  static_cast<long long>(g0) + q, s);
    const int32_t s0 = seg_loc[b], s1 = seg_loc[b + 1];
    if (s1 <= s0) return fail(PKV_EINVAL, "sequence %d has no segments", b);
    int32_t cursor = g0;
    int32_t prev_limit = 0;  // key limit of the previous segment's last row
    for (int32_t k = s0; k < s1; ++k) {
      const int32_t qs = segments[4 * k], qe = segments[4 * k + 1], kv = segments[4 * k + 2], mode = segments[4 * k + 3];
      if (qs != cursor || qe <= qs) return fail(PKV_EINVAL, "sequence %d: segments must tile the query in order", b);
      if (mode == PKV_SEG_CAUSAL) {
        if (kv != qe) return fail(PKV_EINVAL, "sequence %d: a causal segment's kv_end must equal its q_end", b);
      } else if (mode == PKV_SEG_FULL) {
        if (kv < qe || kv > s) return fail(PKV_EINVAL, "sequence %d: a full segment's kv_end must lie in [q_end, seq_len]", b);
      } else {
        return fail(PKV_EINVAL, "sequence %d: unknown segment mode %d", b, mode);
      }
      // Row limits L(g): kv_end over a full segment, g + 1 down a causal
      // one.  The kernels bound a tile of rows by its last row's limit and
      // skip the mask below a wave's first row's, so L must not decrease.
      const int32_t first_limit = mode == PKV_SEG_FULL ? kv : qs + 1;
      if (k > s0 && first_limit < prev_limit)
        return fail(PKV_EINVAL,
                    "sequence %d: segment %d's rows see %d keys but the row before them sees %d; key limits must "
                    "not decrease down the query",
                    b, k - s0, first_limit, prev_limit);
      prev_limit = mode == PKV_SEG_FULL ? kv : qe;
      cursor = qe;
    }
    if (cursor != g0 + q)
      return fail(PKV_EINVAL, "sequence %d: segments end at %d, not at the query's end %d", b, cursor, g0 + q);
  }
  return PKV_OK;
}

}  // extern "C"
