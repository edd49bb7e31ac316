// Host-side window manager: the block allocator behind the paged K/V pools,
// per-request block tables in storage positions, chunk-granular eviction of
// tokens no future window reads, compaction of evicted gaps, scratch blocks
// for uncommitted chunks and action tokens, and the visible-window table of a
// prepared forward.
//
// The pages show the manager only through its callers and tests (P1
// ARDiffusionPagedForwardContext: ensure_video_slots, ensure_action_slots,
// video_block_table, max_video_blocks; P2: the eviction, compaction, reset and
// table-shape tests), so the rules below are re-derived from those:
//   * the chunk (one latent frame) is the eviction unit; the window keeps the
//     sink (sink_chunks chunks) and the most recent window_chunks chunks, the
//     current one included;
//   * after a commit ending at model position E, tokens in [S, E - W) snapped
//     down to a chunk boundary are dead (no later window reaches them); with
//     reset_at_boundary, the commit that completes an AR block of
//     chunks_per_block chunks kills every token past the sink;
//   * a block is freed when every token written in it is dead, except a partly
//     filled last block, which the next chunk continues;
//   * compaction drops whole runs of evicted blocks right after the sink's
//     blocks, a whole number of chunks and blocks at a time (a multiple of
//     lcm(block, chunk) tokens), so chunk boundaries and block offsets keep
//     their place: a storage position past the sink's blocks is its model
//     position minus the compacted tokens;
//   * reading the window looks up only the sink's blocks and those from the
//     recent window's start on (P2 bounds the lookups by max_video_blocks).
//
// Pages cited by tag and function: P1 "vllm_omni/experimental/ar_diffusion/kv_cache/paged_attention.py",
// P2 "tests/diffusion/ar_diffusion/test_paged_attention.py".
#include <algorithm>
#include <numeric>
#include <vector>

#include "pkv_internal.hpp"

using pkv::fail;

struct pkv_window_manager {
  struct Request {
    bool live = false;
    std::vector<int32_t> table;    // storage block index -> physical block, -1 once evicted
    std::vector<int32_t> scratch;  // blocks reserved for uncommitted chunks and action tokens
    int64_t computed = 0;          // committed tokens, storage positions
    int64_t compacted = 0;         // tokens dropped from the table by compaction
    int64_t chunks = 0;            // committed chunks
    // the prepared forward
    bool prepared = false;
    bool commit = false;
    int64_t tokens = 0;
    int64_t action = 0;
    std::vector<int32_t> cur;  // blocks of the current chunk from storage index computed / B on
  };
  pkv_window_config cfg{};
  std::vector<int32_t> free_blocks;  // a stack; block 0 is the null block and never handed out
  std::vector<Request> reqs;
};

namespace {

using Manager = pkv_window_manager;
using Request = pkv_window_manager::Request;

int64_t sink_tokens(const pkv_window_config& c) { return static_cast<int64_t>(c.sink_chunks) * c.chunk_size; }
int64_t window_tokens(const pkv_window_config& c) { return static_cast<int64_t>(c.window_chunks) * c.chunk_size; }
int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

Request* request(Manager* wm, int32_t id) {
  if (!wm || id < 0 || id >= static_cast<int32_t>(wm->reqs.size()) || !wm->reqs[id].live) return nullptr;
  return &wm->reqs[id];
}
const Request* request(const Manager* wm, int32_t id) { return request(const_cast<Manager*>(wm), id); }

// Frees the blocks whose written tokens are all dead after a commit, then
// drops whole lcm(block, chunk) runs of evicted entries after the sink.
void evict_and_compact(Manager* wm, Request& r) {
  const pkv_window_config& c = wm->cfg;
  const int64_t B = c.block_size, C = c.chunk_size;
  const int64_t S = sink_tokens(c), W = window_tokens(c);
  const int64_t E = r.computed + r.compacted;  // model position of the next token
  int64_t dead_end;                             // model positions [S, dead_end) are dead
  if (c.reset_at_boundary && c.chunks_per_block > 0 && r.chunks % c.chunks_per_block == 0) {
    dead_end = E;
  } else {
    const int64_t keep_from = E - W;  // no later window starts before this
    dead_end = keep_from > 0 ? (keep_from / C) * C : 0;
  }
  const int64_t sink_blocks = ceil_div(S, B);
  const int64_t written_blocks = ceil_div(r.computed, B);
  const bool partial_tail = r.computed % B != 0;
  for (int64_t k = sink_blocks; k < written_blocks; ++k) {
    if (r.table[k] < 0) continue;
    if (partial_tail && k == written_blocks - 1) continue;  // the next chunk continues it
    const int64_t first = k * B + r.compacted;              // model positions of its written tokens
    const int64_t last = std::min((k + 1) * B, r.computed) + r.compacted;
    if (first >= S && last <= dead_end) {
      wm->free_blocks.push_back(r.table[k]);
      r.table[k] = -1;
    }
  }
  if (!c.compact) return;
  const int64_t unit = std::lcm(B, C) / B;  // table entries per compaction step
  int64_t run = 0;
  while (sink_blocks + run < static_cast<int64_t>(r.table.size()) && r.table[sink_blocks + run] < 0) ++run;
  const int64_t drop = (run / unit) * unit;
  if (drop == 0) return;
  r.table.erase(r.table.begin() + sink_blocks, r.table.begin() + sink_blocks + drop);
  r.computed -= drop * B;
  r.compacted += drop * B;
}

struct ReadCtx {
  const Request* r;
  int64_t first_cur;  // storage block index of the current chunk's first block
};

int32_t block_of(const void* p, int64_t i) {
  const ReadCtx* x = static_cast<const ReadCtx*>(p);
  if (!x->r->commit && i >= x->first_cur) return x->r->cur[i - x->first_cur];
  return i < static_cast<int64_t>(x->r->table.size()) ? x->r->table[i] : -1;
}

}  // namespace

extern "C" {

int32_t pkv_wm_max_video_blocks(const pkv_window_config* c) {
  if (!c || c->block_size <= 0 || c->chunk_size <= 0 || c->sink_chunks < 0 || c->window_chunks <= 0) return -1;
  const int64_t B = c->block_size;
  // The sink ends at a fixed position; the recent range starts on a chunk
  // boundary, which sits at most B - gcd(chunk, B) tokens past a block edge
  // (P1 max_video_blocks).
  const int64_t slack = B - std::gcd(static_cast<int64_t>(c->chunk_size), B);
  return static_cast<int32_t>(ceil_div(sink_tokens(*c), B) + ceil_div(window_tokens(*c) + slack, B));
}

int pkv_wm_create(const pkv_window_config* cfg, pkv_window_manager** out) {
  if (!cfg || !out) return fail(PKV_EINVAL, "NULL pointer");
  if (cfg->block_size <= 0 || cfg->chunk_size <= 0 || cfg->sink_chunks < 0 || cfg->window_chunks <= 0 ||
      cfg->num_blocks < 2 || cfg->scratch_blocks < 0 || cfg->num_blocks > INT32_MAX ||
      (cfg->reset_at_boundary && cfg->chunks_per_block <= 0))
    return fail(PKV_EINVAL, "bad window manager configuration");
  auto* wm = new pkv_window_manager();
  wm->cfg = *cfg;
  wm->free_blocks.reserve(cfg->num_blocks - 1);
  for (int64_t b = cfg->num_blocks - 1; b >= 1; --b) wm->free_blocks.push_back(static_cast<int32_t>(b));
  *out = wm;
  return PKV_OK;
}

void pkv_wm_destroy(pkv_window_manager* wm) { delete wm; }

int pkv_wm_begin_request(pkv_window_manager* wm, int32_t* out_request) {
  if (!wm || !out_request) return fail(PKV_EINVAL, "NULL pointer");
  const int32_t need = wm->cfg.scratch_blocks;
  if (static_cast<int64_t>(wm->free_blocks.size()) < need)
    return fail(PKV_ERANGE, "%d scratch blocks requested, %zu free", need, wm->free_blocks.size());
  Request r;
  r.live = true;
  for (int32_t i = 0; i < need; ++i) {
    r.scratch.push_back(wm->free_blocks.back());
    wm->free_blocks.pop_back();
  }
  wm->reqs.push_back(std::move(r));
  *out_request = static_cast<int32_t>(wm->reqs.size() - 1);
  return PKV_OK;
}

int pkv_wm_end_request(pkv_window_manager* wm, int32_t id) {
  Request* r = request(wm, id);
  if (!r) return fail(PKV_EINVAL, "no live request %d", id);
  for (int32_t b : r->table)
    if (b >= 0) wm->free_blocks.push_back(b);
  for (int32_t b : r->scratch) wm->free_blocks.push_back(b);
  *r = Request();
  return PKV_OK;
}

int pkv_wm_prepare(pkv_window_manager* wm, int32_t id, int64_t tokens, int32_t commit, int64_t action_tokens,
                   int64_t* out_slots, int64_t* out_action_slots) {
  Request* r = request(wm, id);
  if (!r) return fail(PKV_EINVAL, "no live request %d", id);
  if (tokens <= 0 || action_tokens < 0) return fail(PKV_EINVAL, "bad token counts");
  if (!out_slots || (action_tokens && !out_action_slots)) return fail(PKV_EINVAL, "NULL pointer");
  const int64_t B = wm->cfg.block_size;
  const int64_t h = r->computed, offset = h % B;
  const int64_t first = h / B;
  const int64_t last = ceil_div(h + tokens, B);  // one past the chunk's last storage block index
  std::vector<int32_t> cur;
  int64_t scratch_used = 0;
  if (commit) {
    const int64_t fresh = last - std::max<int64_t>(first, static_cast<int64_t>(r->table.size()));
    if (fresh > static_cast<int64_t>(wm->free_blocks.size()))
      return fail(PKV_ERANGE, "the pool has %zu free blocks, the chunk needs %lld", wm->free_blocks.size(),
                  static_cast<long long>(fresh));
  } else {
    // An uncommitted chunk starts where the history stopped: its first tokens
    // fill the free slots of the history's last block, the rest go to scratch
    // blocks (P1 ensure_video_slots).
    scratch_used = last - first - (offset ? 1 : 0);
  }
  const int64_t action_blocks = ceil_div(action_tokens, B);
  if (scratch_used + action_blocks > static_cast<int64_t>(r->scratch.size()))
    return fail(PKV_ERANGE, "the request's %zu scratch blocks do not hold %lld + %lld blocks", r->scratch.size(),
                static_cast<long long>(scratch_used), static_cast<long long>(action_blocks));
  if (commit) {
    for (int64_t k = static_cast<int64_t>(r->table.size()); k < last; ++k) {
      r->table.push_back(wm->free_blocks.back());
      wm->free_blocks.pop_back();
    }
    for (int64_t t = 0; t < tokens; ++t) {
      const int64_t p = h + t;
      out_slots[t] = static_cast<int64_t>(r->table[p / B]) * B + p % B;
    }
  } else {
    if (offset) cur.push_back(r->table[first]);
    for (int64_t i = 0; i < scratch_used; ++i) cur.push_back(r->scratch[i]);
    for (int64_t t = 0; t < tokens; ++t) {
      const int64_t p = offset + t;  // position inside the chunk's run of blocks
      out_slots[t] = static_cast<int64_t>(cur[p / B]) * B + p % B;
    }
  }
  for (int64_t t = 0; t < action_tokens; ++t)
    out_action_slots[t] = static_cast<int64_t>(r->scratch[scratch_used + t / B]) * B + t % B;
  r->prepared = true;
  r->commit = commit != 0;
  r->tokens = tokens;
  r->action = action_tokens;
  r->cur = std::move(cur);
  // the action blocks follow the chunk's scratch blocks
  r->cur.insert(r->cur.end(), r->scratch.begin() + scratch_used, r->scratch.begin() + scratch_used + action_blocks);
  return PKV_OK;
}

int pkv_wm_window_table(const pkv_window_manager* wm, int32_t id, int32_t* out_table, int32_t capacity,
                        int32_t* out_count, int32_t* out_kv_len, int32_t* out_reads) {
  const Request* r = request(wm, id);
  if (!r) return fail(PKV_EINVAL, "no live request %d", id);
  if (!r->prepared) return fail(PKV_EINVAL, "request %d has no prepared forward", id);
  if (!out_table || !out_count || !out_kv_len) return fail(PKV_EINVAL, "NULL pointer");
  const int64_t B = wm->cfg.block_size;
  ReadCtx ctx{r, r->computed / B};
  int64_t reads = 0;
  if (int rc = pkv::window_read(block_of, &ctx, r->computed, r->tokens, sink_tokens(wm->cfg), window_tokens(wm->cfg),
                                wm->cfg.block_size, out_table, capacity, out_count, out_kv_len, &reads))
    return rc;
  if (r->action) {
    // Action K/V after the video run (P1 build_block_table).
    const int64_t scratch_used = r->commit ? 0 : static_cast<int64_t>(r->cur.size()) - ceil_div(r->action, B);
    const int32_t* act = (r->commit ? r->scratch.data() : r->cur.data() + scratch_used);
    if (int rc = pkv_action_table(out_table, capacity, out_count, out_kv_len, act,
                                  static_cast<int32_t>(ceil_div(r->action, B)), r->action, wm->cfg.block_size))
      return rc;
  }
  if (out_reads) *out_reads = static_cast<int32_t>(reads);
  return PKV_OK;
}

int pkv_wm_commit(pkv_window_manager* wm, int32_t id) {
  Request* r = request(wm, id);
  if (!r) return fail(PKV_EINVAL, "no live request %d", id);
  if (!r->prepared) return fail(PKV_EINVAL, "request %d has no prepared forward", id);
  r->prepared = false;
  if (!r->commit) return PKV_OK;  // an uncommitted forward leaves the request as it was
  r->computed += r->tokens;
  r->chunks += r->tokens / wm->cfg.chunk_size;
  evict_and_compact(wm, *r);
  return PKV_OK;
}

int pkv_wm_info(const pkv_window_manager* wm, int32_t id, int64_t* out) {
  const Request* r = request(wm, id);
  if (!r || !out) return fail(PKV_EINVAL, "no live request %d", id);
  int64_t nulls = 0;
  for (int32_t b : r->table) nulls += b < 0;
  out[0] = r->computed;
  out[1] = r->computed + r->compacted;
  out[2] = r->compacted;
  out[3] = static_cast<int64_t>(r->table.size());
  out[4] = static_cast<int64_t>(wm->free_blocks.size());
  out[5] = nulls;
  return PKV_OK;
}

int pkv_wm_block_table(const pkv_window_manager* wm, int32_t id, int32_t* out, int32_t capacity, int32_t* out_count) {
  const Request* r = request(wm, id);
  if (!r || !out || !out_count) return fail(PKV_EINVAL, "no live request %d", id);
  if (static_cast<int64_t>(r->table.size()) > capacity)
    return fail(PKV_ERANGE, "table of %zu entries, capacity %d", r->table.size(), capacity);
  std::copy(r->table.begin(), r->table.end(), out);
  *out_count = static_cast<int32_t>(r->table.size());
  return PKV_OK;
}

}  // extern "C"
