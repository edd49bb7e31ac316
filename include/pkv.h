/*
 * pkv -- paged K/V cache write, history-staging gather and paged self-attention
 * for autoregressive video diffusion, on AMD Instinct MI355X (gfx950).
 *
 * Source of the semantics: four vllm-omni pages, cited by tag and function:
 *   P1 "vllm_omni/experimental/ar_diffusion/kv_cache/paged_attention.py"
 *   P2 "tests/diffusion/ar_diffusion/test_paged_attention.py"
 *   P3 "vllm_omni/diffusion/attention/backends/utils/piecewise_attn.py"
 *   P4 "vllm_omni/diffusion/diffusion_kv/paged_attention_adapter.py"
 *
 * Conventions shared by every call
 * --------------------------------
 * - Pools are per layer, one for K and one for V, each
 *   [num_blocks * block_size, num_kv_heads, head_dim] row-major: a "slot" is one
 *   token row of num_kv_heads * head_dim contiguous elements, and block b holds
 *   slots [b * block_size, (b + 1) * block_size)  (P1 ARDiffusionPagedLayerInputs,
 *   P1 _paged_write_attn_impl: the flat pool is viewed as [blocks, block, heads, dim]).
 * - Activations are token-major [tokens, heads, head_dim], contiguous.
 * - Pointers named "device" must point to device memory of the current HIP
 *   device; pointers named "host" to host memory.  The caller owns every
 *   buffer; the library never allocates device memory behind the caller's back
 *   and never frees anything it was given.
 * - `stream` is a hipStream_t (NULL = the legacy default stream).  Device
 *   calls only enqueue work and return; ordering between a write and the
 *   attention that reads it comes from issuing both on one stream (P1 keeps
 *   write -> read ordering inside one op for the same reason).
 * - Return value: PKV_OK, or a negative pkv_status.  Argument errors are
 *   detected on the host before anything is enqueued; the message is then
 *   available from pkv_last_error() (thread-local).  Device-side metadata
 *   (slot mappings, block tables, seq_lens, segments) is trusted in the device
 *   calls, as FlashAttention trusts its seqused_k; pkv_validate_metadata_host
 *   checks host copies of it against the pages' rules.
 */
#ifndef PKV_H_
#define PKV_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PKV_F32 = 0,      /* IEEE binary32 */
  PKV_BF16 = 1,     /* bfloat16 */
  PKV_FP8_E4M3 = 2  /* OCP float8 e4m3fn, per-tensor scale (pools only) */
} pkv_dtype;

typedef enum {
  PKV_OK = 0,
  PKV_EINVAL = -1,        /* bad argument (message in pkv_last_error) */
  PKV_EUNSUPPORTED = -2,  /* valid request this build has no kernel for */
  PKV_EHIP = -3,          /* a HIP runtime call or kernel launch failed */
  PKV_ERANGE = -4,        /* an output buffer is too small */
  PKV_EWINDOW = -5        /* visible window would read past a partly written block */
} pkv_status;

typedef enum { PKV_SEG_CAUSAL = 0, PKV_SEG_FULL = 1 } pkv_seg_mode;

/* One layer's K and V pools (device memory owned by the caller). */
typedef struct {
  void* key;            /* device, [num_blocks * block_size, num_kv_heads, head_dim] */
  void* value;          /* device, same shape and dtype as key */
  int64_t num_blocks;
  int32_t block_size;   /* 16: the kernels page K/V in 16-token blocks (P1 supported_kernel_block_sizes) */
  int32_t num_kv_heads;
  int32_t head_dim;     /* 64 or 128 (64 runs through the 128-wide kernels with the upper half zero) */
  int32_t dtype;        /* pkv_dtype of the pools */
  float k_scale;        /* dequantisation multipliers: stored value * scale = real value (1 unless FP8) */
  float v_scale;
  float k_inv_scale;    /* quantisation multipliers used by pkv_paged_write for FP8 (1 unless FP8) */
  float v_inv_scale;
} pkv_pools;

/* ------------------------------------------------------------------ device calls */

/*
 * Slot-mapping scatter of the current chunk's K/V into the pools
 * (P1 _paged_write_attn_impl: each pool indexed by the slot mapping is
 * assigned the current K/V converted to the pool's dtype).
 *
 *   key, value    device, [num_tokens, num_kv_heads, head_dim] of src_dtype
 *   src_dtype     PKV_F32 into an F32 pool, PKV_BF16 into a BF16 or FP8_E4M3 pool
 *   slot_mapping  device int64 [num_tokens]; token t goes to slot slot_mapping[t]
 *
 * Same dtype: a bit-exact copy.  BF16 -> FP8_E4M3: fp32(x) * k_inv_scale (or
 * v_inv_scale) rounded once to fp32 (nearest-even), then to e4m3fn by
 * round-to-nearest-even with saturation to +-448; NaN stays NaN.
 * Preconditions (not checked on the device): slots unique and in
 * [0, num_blocks * block_size).  num_tokens == 0 is a no-op.
 */
int pkv_paged_write(const void* key, const void* value, int32_t src_dtype, int64_t num_tokens,
                    const int64_t* slot_mapping, const pkv_pools* pools, void* stream);

/*
 * History staging gather (P1 _stage_window): the staging buffers, seen as
 * [n_blocks, block_size, num_kv_heads, head_dim], receive pool block
 * block_ids[i] at block row i for first_block <= i < n_blocks.  Rows outside
 * [first_block * block_size, n_blocks * block_size) are not touched.
 * A bit-exact copy in the pool's dtype.
 *
 *   block_ids    device int32 [n_blocks]; entries must be in [0, num_blocks)
 *   stage_key    device, at least n_blocks * block_size token rows
 *   stage_value  device, same size
 * Errors: first_block < 0 or first_block > n_blocks -> PKV_EINVAL.
 * first_block == n_blocks is a no-op.
 */
int pkv_gather(const pkv_pools* pools, const int32_t* block_ids, int32_t n_blocks, int32_t first_block,
               void* stage_key, void* stage_value, void* stream);

/*
 * Varlen paged attention with a piecewise full/causal mask.
 *
 * Sequence b has query rows q[query_start_loc[b] : query_start_loc[b+1]] and
 * seq_lens[b] visible keys, read through block_table[b]: key j lives in slot
 * block_table[b][j / block_size] * block_size + j % block_size
 * (P1 _reference_paged_attention).  Only the first ceil(seq_lens[b] /
 * block_size) table entries are read.  The queries are the suffix of the
 * sequence: query row i sits at key position g = seq_lens[b] - q_len + i
 * (P3 piecewise_attn; P4 refuses rows that do not end at seq_len).
 *
 * Mask (P3 module docstring and build_segments): segments
 * [segment_start_loc[b], segment_start_loc[b+1]) of `segments`, each
 * {q_start, q_end, kv_end, mode} in key coordinates, tile
 * [seq_len - q_len, seq_len) in order.  A row g in a FULL segment sees keys
 * j < kv_end; in a CAUSAL segment keys j <= g (bottom-right alignment).
 * The AR default of P1 (causal=False) is one FULL segment with kv_end = seq_len.
 * Precondition: the per-row key limit L(g) (kv_end, or g + 1) never decreases
 * from one row to the next.  P3 build_segments' lists satisfy it (a FULL
 * segment reaches past its q_end only when it is the last one);
 * pkv_validate_metadata_host refuses lists that break it.
 *
 * GQA: query head h reads KV head h / (num_q_heads / num_kv_heads) (P4 requires
 * num_q_heads % num_kv_heads == 0).
 * out[t, h, :] = sum_j softmax_j(softmax_scale * q.k_j) v_j, accumulated in fp32
 * and rounded to q_dtype.
 *
 *   q                 device [num_q_tokens, num_q_heads, head_dim]; q_dtype PKV_F32 with
 *                     F32 pools, PKV_BF16 with BF16 or FP8_E4M3 pools
 *   block_table       device int32 [num_seqs, table_width]
 *   query_start_loc   device int32 [num_seqs + 1]; rows of q/out at or past
 *                     query_start_loc[num_seqs] belong to no sequence and are not written
 *   seq_lens          device int32 [num_seqs]
 *   max_query_len     host bound on every query length (grid sizing)
 *   max_seq_len       host bound on every seq_lens[b] (a capacity, P1 build_block_table)
 *   segments          device int32 [num_segments][4]
 *   segment_start_loc device int32 [num_seqs + 1] (CSR into segments)
 *   seq_order         device int32 [num_seqs], a permutation of 0 .. num_seqs - 1, or NULL:
 *                     the order in which the sequences' work is handed to the GPU.
 *                     Longest first (the ForwardPlan's choice) lets short sequences fill
 *                     in behind long ones; the result does not depend on it.
 *   host_seq_lens     host int32 [num_seqs] or NULL: the seq_lens values, as a planning
 *                     hint.  With short query chunks (at most 64 rows per KV head) the
 *                     library then cuts each sequence into key ranges by its own length and
 *                     hands the non-empty ranges out first, so they cover the CUs evenly.
 *                     The result is the same up to rounding whatever the hint (stale
 *                     hints, e.g. in a replayed graph, only cost speed).
 *   out               device, same shape and dtype as q
 *   workspace         device scratch for split-key partial results, or NULL;
 *                     pkv_paged_attn_workspace_size() gives the size that lets the
 *                     library use every split it would like.  With less (or none)
 *                     it uses fewer splits; the result is the same up to rounding.
 * Errors: PKV_EINVAL for inconsistent host arguments (head counts, dtypes,
 * null pointers, max_query_len > max_seq_len, ...); PKV_EUNSUPPORTED for a
 * head_dim or dtype pair without a kernel.
 */
int pkv_paged_attn(const void* q, int32_t q_dtype, int64_t num_q_tokens, int32_t num_q_heads,
                   const pkv_pools* pools, const int32_t* block_table, int32_t table_width,
                   const int32_t* query_start_loc, const int32_t* seq_lens, int32_t num_seqs,
                   int32_t max_query_len, int32_t max_seq_len, const int32_t* segments,
                   const int32_t* segment_start_loc, const int32_t* seq_order, const int32_t* host_seq_lens,
                   float softmax_scale, void* out, void* workspace, size_t workspace_bytes, void* stream);

/*
 * The two halves of pkv_paged_attn, with its arguments, meaning and errors:
 * pkv_paged_attn_main launches the attention kernel (which writes `out`
 * directly when the key range is not split, else one partial result per
 * split into `workspace`); pkv_paged_attn_merge then merges the partials into
 * `out` in split order, and does nothing when the keys were not split.  Both
 * plan the splits from the same arguments, so a caller passing identical
 * arguments to both, in that order on one stream, gets exactly
 * pkv_paged_attn's result.  They let a caller time or schedule the two
 * launches separately.
 */
int pkv_paged_attn_main(const void* q, int32_t q_dtype, int64_t num_q_tokens, int32_t num_q_heads,
                        const pkv_pools* pools, const int32_t* block_table, int32_t table_width,
                        const int32_t* query_start_loc, const int32_t* seq_lens, int32_t num_seqs,
                        int32_t max_query_len, int32_t max_seq_len, const int32_t* segments,
                        const int32_t* segment_start_loc, const int32_t* seq_order, const int32_t* host_seq_lens,
                        float softmax_scale, void* out, void* workspace, size_t workspace_bytes, void* stream);
int pkv_paged_attn_merge(const void* q, int32_t q_dtype, int64_t num_q_tokens, int32_t num_q_heads,
                         const pkv_pools* pools, const int32_t* block_table, int32_t table_width,
                         const int32_t* query_start_loc, const int32_t* seq_lens, int32_t num_seqs,
                         int32_t max_query_len, int32_t max_seq_len, const int32_t* segments,
                         const int32_t* segment_start_loc, const int32_t* seq_order, const int32_t* host_seq_lens,
                         float softmax_scale, void* out, void* workspace, size_t workspace_bytes, void* stream);

/*
 * pkv_paged_attn for callers that cannot allocate device memory: code under
 * HIP graph capture, serving loops and harnesses that forbid hipMalloc.  The
 * arguments, result and errors are pkv_paged_attn's, without the workspace:
 * the split-key partials go to a scratch array of PKV_NOALLOC_SCRATCH_BYTES
 * that the library holds on every device it runs on, for the life of the
 * process.  The call allocates and frees nothing.  It plans the splits
 * pkv_paged_attn plans with a workspace of pkv_paged_attn_workspace_size()
 * bytes, so the two give identical results.
 * Errors: PKV_ERANGE when pkv_paged_attn_workspace_size() exceeds
 * PKV_NOALLOC_SCRATCH_BYTES for these sizes (nothing is enqueued).
 * Every call on one device uses that device's one array and leaves its
 * contents behind (no part of it needs to start cleared: each partial the
 * merge reads is written by the same call): calls that may overlap on one
 * device, e.g. on two streams, race and must be serialised by the caller.
 */
#define PKV_NOALLOC_SCRATCH_BYTES (128u * 1024u * 1024u)
int pkv_paged_attn_noalloc(const void* q, int32_t q_dtype, int64_t num_q_tokens, int32_t num_q_heads,
                           const pkv_pools* pools, const int32_t* block_table, int32_t table_width,
                           const int32_t* query_start_loc, const int32_t* seq_lens, int32_t num_seqs,
                           int32_t max_query_len, int32_t max_seq_len, const int32_t* segments,
                           const int32_t* segment_start_loc, const int32_t* seq_order, const int32_t* host_seq_lens,
                           float softmax_scale, void* out, void* stream);

/*
 * Attention metadata of one forward, shared by every layer (P1
 * ARDiffusionPagedForwardContext.prepare builds it once per KV branch).  The
 * fields are pkv_paged_attn's arguments of the same names.  For capture in a
 * HIP graph keep table_width and max_seq_len fixed capacities (P1
 * build_block_table pads the table to a constant width and passes a constant
 * max_seq_len), so that only the device arrays' contents change between
 * forwards.
 */
typedef struct {
  const int32_t* block_table;        /* device int32 [num_seqs, table_width] */
  const int32_t* query_start_loc;    /* device int32 [num_seqs + 1] */
  const int32_t* seq_lens;           /* device int32 [num_seqs] */
  const int32_t* segments;           /* device int32 [num_segments][4] */
  const int32_t* segment_start_loc;  /* device int32 [num_seqs + 1] */
  const int32_t* seq_order;          /* device int32 [num_seqs] or NULL */
  const int32_t* host_seq_lens;      /* host int32 [num_seqs] or NULL: planning hint, as for pkv_paged_attn */
  const int32_t* query_pos;          /* device int32 [num_seqs] or NULL: key position of each sequence's
                                        first query row.  NULL places every query at the end of its keys
                                        (seq_len - q_len, the AR chunk).  Otherwise sequence b's rows sit at
                                        [query_pos[b], query_pos[b] + q_len) inside [0, seq_len): a local
                                        shard of a longer query (P3 piecewise_attn query_ranges), whose
                                        full segments may still reach past its own end (kv_end) */
  int32_t table_width;
  int32_t num_seqs;
  int32_t max_query_len;
  int32_t max_seq_len;
} pkv_attn_meta;

/*
 * Caller-owned contiguous staging of one sequence's visible window
 * (P1 _stage_window and the staged branch of ar_diffusion_paged_attention).
 */
typedef struct {
  void* stage_key;          /* device, capacity_tokens rows of num_kv_heads * head_dim pool elements */
  void* stage_value;        /* device, same size */
  int64_t capacity_tokens;  /* rows each buffer holds */
  int32_t first_block;      /* 0: restage the whole window; k > 0: block rows [0, k) already hold this
                               window (same history, P1 _prepare_history_staging) and only
                               [k, max_seq_len / block_size) are refreshed */
} pkv_staging;

/*
 * What one KV branch's staging buffers held after its last staged forward
 * (P1 history_staging_state), for pkv_staging_decide.  Caller-owned: set
 * session to -1 before the first use.  history_blocks is caller-owned storage
 * for block_capacity block ids (the most a visible history can list).
 */
typedef struct {
  int64_t session;             /* caller's id of the request staged last; -1: none */
  int64_t history_tokens;      /* its history length */
  int64_t chunk_tokens;        /* its current chunk's length */
  int32_t max_seq_len;         /* its staged extent */
  int32_t num_history_blocks;  /* its visible history's blocks, listed in history_blocks */
  int32_t* history_blocks;
  int32_t block_capacity;
} pkv_staging_state;

/*
 * Whether a forward may keep the rows its staging buffers already hold (P1
 * _prepare_history_staging): the staged history is still this forward's when
 * the last staged forward was for the same request (`session`, a caller id
 * >= 0), with the same history (length and visible blocks), extent
 * (max_seq_len) and chunk length, and the chunk starts on a block edge and
 * fills whole blocks (so no block holds both history and chunk rows).
 *   table          host, the forward's visible-window table (table_len entries,
 *                  as pkv_window_table builds it): the history's blocks, then the
 *                  blocks the current chunk touches
 *   capacity_tokens  rows the staging buffers hold
 * Writes *out_reuse (1 or 0) and *out_first_block: the pkv_staging.first_block
 * of this forward -- the visible history's block count when reusing, else 0
 * (restage everything).  The state then describes this forward.
 * Errors: PKV_ERANGE when max_seq_len > capacity_tokens (P1 raises) or the
 * history lists more blocks than state->block_capacity; PKV_EINVAL for bad
 * sizes or a table too short for the chunk.  The state is unchanged on error.
 */
int pkv_staging_decide(pkv_staging_state* state, int64_t session, const int32_t* table, int32_t table_len,
                       int64_t history_tokens, int64_t chunk_tokens, int32_t max_seq_len, int32_t block_size,
                       int64_t capacity_tokens, int32_t* out_reuse, int32_t* out_first_block);

/*
 * One layer of the per-layer op (P1 _paged_write_attn_impl): enqueues, in
 * order on `stream`,
 *   1. the slot writes of the current video K/V (as pkv_paged_write with
 *      key/value/kv_dtype/num_tokens/slot_mapping),
 *   2. the slot writes of the action K/V (the same with action_key,
 *      action_value, num_action_tokens, action_slot_mapping; skipped when
 *      num_action_tokens == 0, and the four may then be NULL/0),
 *   3. with staging != NULL: the gather of table row 0's blocks
 *      [first_block, max_seq_len / block_size) into the staging buffers (as
 *      pkv_gather), and attention over those buffers read as one contiguous
 *      run; with staging == NULL: attention over the pools through the table,
 *   4. the attention and split merge of pkv_paged_attn with meta's fields.
 * The call allocates nothing, synchronises nothing and launches a fixed
 * sequence of kernels for fixed host arguments, so it can be captured in a
 * HIP graph and replayed with new device contents.
 * Every argument is checked before anything is enqueued.  Errors: those of
 * pkv_paged_write, pkv_gather and pkv_paged_attn, and PKV_EINVAL for staged
 * calls with num_seqs != 1, a max_seq_len that is not a whole number of
 * blocks or exceeds table_width blocks or capacity_tokens, and, when
 * first_block > 0, a current chunk that is not a whole number of blocks or
 * first_block + its blocks > max_seq_len / block_size (P1 asserts both).
 */
int pkv_paged_write_attn(const void* q, int32_t q_dtype, int64_t num_q_tokens, int32_t num_q_heads,
                         const void* key, const void* value, int32_t kv_dtype, int64_t num_tokens,
                         const int64_t* slot_mapping, const void* action_key, const void* action_value,
                         int64_t num_action_tokens, const int64_t* action_slot_mapping, const pkv_pools* pools,
                         const pkv_attn_meta* meta, const pkv_staging* staging, float softmax_scale, void* out,
                         void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes pkv_paged_attn would like for these sizes on the current device. */
size_t pkv_paged_attn_workspace_size(int64_t num_q_tokens, int32_t num_q_heads, int32_t num_kv_heads,
                                     int32_t head_dim, int32_t num_seqs, int32_t max_query_len,
                                     int32_t max_seq_len);

/* ------------------------------------------------------------------ host metadata */

/*
 * Slot mapping (P1 ensure_video_slots / compute_slot_mapping): for the
 * num_tokens positions p = first_position + t,
 * out_slots[t] = block_ids[p / block_size] * block_size + p % block_size.
 * All arrays host.  Errors: a position whose block index is >= num_block_ids,
 * or a negative block id -> PKV_EINVAL.
 */
int pkv_slot_mapping(const int32_t* block_ids, int64_t num_block_ids, int64_t first_position,
                     int64_t num_tokens, int32_t block_size, int64_t* out_slots);

/*
 * Visible-window block table (P1 video_block_table).  block_ids[i] (host) is
 * the physical block holding positions [i * B, (i + 1) * B) of the sequence,
 * or a negative value for a block that is no longer resident.  Positions
 * [0, history_tokens + query_tokens) are written.  The window keeps the sink
 * [0, sink_tokens) and the most recent window_tokens positions (current chunk
 * included); every resident block holding a kept position is listed, in
 * position order, and read whole.  Writes the list to out_table (host,
 * capacity entries), its length to *out_count and the number of tokens the
 * kernel reads to *out_kv_len.
 * Errors: PKV_ERANGE if capacity is too small; PKV_EWINDOW if a partly written
 * block would be followed by another (P1 raises RuntimeError); PKV_EINVAL for
 * bad sizes (window_tokens < query_tokens, too few block ids, ...).
 */
int pkv_window_table(const int32_t* block_ids, int64_t num_block_ids, int64_t history_tokens,
                     int64_t query_tokens, int64_t sink_tokens, int64_t window_tokens, int32_t block_size,
                     int32_t* out_table, int32_t capacity, int32_t* out_count, int32_t* out_kv_len);

/*
 * Action tokens after the video window (P1 build_block_table and
 * ensure_action_slots): appends the scratch blocks holding action_tokens
 * action K/V rows (positions [0, action_tokens) of action_block_ids, host) to
 * a visible-window table (host, *count entries of capacity) and grows *count
 * by their number and *kv_len by action_tokens.  The kernel reads the table
 * as one run, so the video run must end on a block edge: *kv_len %
 * block_size != 0 with action tokens -> PKV_EINVAL (P1 raises ValueError).
 * action_tokens == 0 is a no-op.  Errors: PKV_EINVAL for too few or negative
 * ids; PKV_ERANGE if capacity is too small.
 */
int pkv_action_table(int32_t* table, int32_t capacity, int32_t* count, int32_t* kv_len,
                     const int32_t* action_block_ids, int32_t num_action_block_ids, int64_t action_tokens,
                     int32_t block_size);

/*
 * Fixed table capacity (P1 ARDiffusionPagedForwardContext.max_video_blocks
 * and build_block_table): the most table entries a visible window can span,
 * plus the action scratch blocks, so that the block table keeps one width and
 * max_seq_len one value (capacity * block_size) while the window fills.  The
 * sink [0, sink_tokens) and the recent window_tokens are rounded up to blocks
 * separately (each can straddle a block edge on its own); the recent range
 * starts at a whole number of chunks, so at most
 * block_size - gcd(chunk_size, block_size) tokens past a block edge, and
 * needs ceil((window_tokens + that) / block_size) blocks.  Action scratch
 * takes max(1, ceil(action_tokens / block_size)) blocks (P1 keeps one even
 * without actions).  *out_blocks receives the total.
 * Errors: PKV_EINVAL for block_size or chunk_size <= 0, negative token counts,
 * or a NULL out_blocks.
 */
int pkv_window_capacity(int64_t sink_tokens, int64_t window_tokens, int32_t chunk_size, int32_t block_size,
                        int64_t action_tokens, int64_t* out_blocks);

/*
 * Piecewise segments (P3 build_segments): full_spans (host, [num_spans][2],
 * half-open, key coordinates, sorted and disjoint) are clipped to the query
 * range [query_offset, query_offset + query_len); rows before a clipped span
 * that no span claimed become a CAUSAL segment, the clipped span a FULL
 * segment whose kv_end is the span's unclipped end, and the rest after the
 * last span a CAUSAL segment.  out_segments (host, [capacity][4]) receives
 * {q_start, q_end, kv_end, mode}; *out_count their number.
 * Errors: PKV_EINVAL for unsorted/overlapping/empty spans or query_len <= 0;
 * PKV_ERANGE if capacity is too small.
 */
int pkv_build_segments(const int32_t* full_spans, int32_t num_spans, int32_t query_offset, int32_t query_len,
                       int32_t* out_segments, int32_t capacity, int32_t* out_count);

/*
 * Checks host copies of the attention metadata against the rules the pages
 * enforce (P3 build_paged_piecewise_plan, P4 row and layout checks):
 * 1 <= q_len <= seq_len <= max_seq_len, q_len <= max_query_len, query_start_loc
 * starts at 0 and is non-decreasing, ceil(seq_len / block_size) <= table_width,
 * referenced table entries in [0, num_blocks), the query rows
 * [g0, g0 + q_len) inside [0, seq_len) with g0 = query_pos[b] (host, may be
 * NULL: g0 = seq_len - q_len), segments tiling [g0, g0 + q_len) in order with
 * causal kv_end == q_end, full kv_end in [q_end, seq_len], and row key limits
 * that never decrease from one segment to the next (the kernels' precondition,
 * see pkv_paged_attn).  Returns PKV_OK or PKV_EINVAL with a message.
 */
int pkv_validate_metadata_host(const int32_t* query_start_loc, const int32_t* seq_lens, int32_t num_seqs,
                               const int32_t* block_table, int32_t table_width, int64_t num_blocks,
                               int32_t block_size, int32_t max_query_len, int32_t max_seq_len,
                               const int32_t* segments, const int32_t* segment_start_loc,
                               const int32_t* query_pos);

/* ------------------------------------------------------------------ window manager */

/*
 * Host-side block manager behind the pools of one KV branch (P1
 * ARDiffusionPagedForwardContext with its cache manager; P2's eviction,
 * compaction, reset and table-shape tests).  Not thread-safe: one manager per
 * thread, or a lock around it.  Physical block 0 is the null block and is
 * never handed out, so tables padded with 0 never point at live data.
 *
 * Model positions count every token of a request from its start; storage
 * positions are what the block table indexes.  They agree on the sink's
 * blocks; past them a storage position is its model position minus the
 * tokens dropped by compaction, always a whole number of chunks and blocks.
 *
 * After a committing forward ends at model position E, the tokens in
 * [S, E - W) snapped down to a chunk boundary are dead (S = sink tokens, W =
 * the recent window's tokens); with reset_at_boundary the commit that
 * completes an AR block of chunks_per_block chunks kills every token past the
 * sink.  A block is freed once all its written tokens are dead, except a
 * partly written last block, which the next chunk continues.  Compaction
 * drops whole multiples of lcm(block_size, chunk_size) tokens of evicted
 * blocks right after the sink's blocks.
 */
typedef struct pkv_window_manager pkv_window_manager;

typedef struct {
  int64_t num_blocks;         /* physical blocks of the pools; block 0 is the null block */
  int32_t block_size;
  int32_t chunk_size;         /* tokens per chunk (one latent frame): the eviction unit */
  int32_t sink_chunks;        /* leading chunks the window always keeps */
  int32_t window_chunks;      /* most recent chunks kept, the current one included */
  int32_t chunks_per_block;   /* chunks per AR block: where reset_at_boundary acts */
  int32_t reset_at_boundary;  /* nonzero: an AR block's last commit keeps only the sink */
  int32_t scratch_blocks;     /* blocks reserved per request for uncommitted chunks and action tokens */
  int32_t compact;            /* nonzero: drop evicted gaps from the tables */
} pkv_window_config;

/* Most blocks a visible window spans (P1 max_video_blocks): the sink's blocks
   plus the recent range's, which starts on a chunk boundary at most
   block_size - gcd(chunk_size, block_size) tokens past a block edge.  The
   constant table width of the configuration (add the action capacity).
   -1 for a bad configuration. */
int32_t pkv_wm_max_video_blocks(const pkv_window_config* cfg);

/* Creates a manager (host memory only).  PKV_EINVAL for a bad configuration. */
int pkv_wm_create(const pkv_window_config* cfg, pkv_window_manager** out);
void pkv_wm_destroy(pkv_window_manager* wm);

/* Starts a request (one sequence of one KV branch) and reserves its scratch
   blocks; *out_request is its id.  PKV_ERANGE when the pool is short. */
int pkv_wm_begin_request(pkv_window_manager* wm, int32_t* out_request);
/* Returns every block of the request to the pool. */
int pkv_wm_end_request(pkv_window_manager* wm, int32_t request);

/*
 * Prepares a forward of `tokens` video tokens continuing the request's
 * history, plus `action_tokens` action tokens (P1 ensure_video_slots and
 * ensure_action_slots).  commit != 0: the tokens go to pool blocks after the
 * history (continuing its partly written last block) and pkv_wm_commit makes
 * them history.  commit == 0: they start in the free slots of the history's
 * last block and continue in scratch blocks, and the request is left as it
 * was.  Action tokens take scratch blocks after the chunk's.  Writes the
 * slots (host int64) of the video tokens to out_slots[tokens] and of the
 * action tokens to out_action_slots[action_tokens].  PKV_ERANGE when the pool
 * or the scratch blocks are short (nothing changes then).
 */
int pkv_wm_prepare(pkv_window_manager* wm, int32_t request, int64_t tokens, int32_t commit, int64_t action_tokens,
                   int64_t* out_slots, int64_t* out_action_slots);

/*
 * The visible-window block table of the prepared forward (P1
 * video_block_table then build_block_table): as pkv_window_table over the
 * request's storage positions, followed by the action blocks as
 * pkv_action_table appends them.  Writes the table (host) to out_table,
 * its length to *out_count, the tokens it holds to *out_kv_len, and the
 * number of table entries looked up to *out_reads (may be NULL), which
 * never exceeds pkv_wm_max_video_blocks.
 */
int pkv_wm_window_table(const pkv_window_manager* wm, int32_t request, int32_t* out_table, int32_t capacity,
                        int32_t* out_count, int32_t* out_kv_len, int32_t* out_reads);

/* Ends the prepared forward: a committing one becomes history, then eviction
   and compaction run; an uncommitted one is dropped. */
int pkv_wm_commit(pkv_window_manager* wm, int32_t request);

/* out[6] = {committed tokens (storage), committed tokens (model), compacted
   tokens, table entries, free pool blocks, evicted entries still in the table}. */
int pkv_wm_info(const pkv_window_manager* wm, int32_t request, int64_t* out);

/* The request's storage block table (host), -1 for an evicted block. */
int pkv_wm_block_table(const pkv_window_manager* wm, int32_t request, int32_t* out, int32_t capacity,
                       int32_t* out_count);

/* Thread-local description of the last error returned on this thread ("" if none). */
const char* pkv_last_error(void);

/* Thread-local description of the kernel plan the last attention call on this
   thread chose (after its checks passed): "long", "short" or "fp8" with the key
   splits and their length (for "long", the keys where splits 1, 2, ... start:
   the splits may differ in length), or "f32".  Diagnostic only: the format may
   change. */
const char* pkv_last_attn_plan(void);

/*
 * Measured peaks (diagnostics for stating fractions against what this GPU
 * sustains; not part of the attention path).  Both only enqueue work on
 * `stream`: the caller times it (events) and synchronises.
 *
 * pkv_probe_mfma: two workgroups of four waves per CU (two waves per SIMD),
 *   each wave issuing `iters` x 4 independent bf16 v_mfma_f32_32x32x16
 *   products.  *out_flop receives the floating-point operations the launch
 *   performs.  sink: device float scratch of at least 512 x (CU count) floats
 *   (the products' sums land there).
 * pkv_probe_stream: reads `bytes` (a multiple of 16) of device memory at `src`
 *   once, each workgroup its own contiguous chunk, 16 bytes per lane with eight
 *   loads in flight; sink: device scratch of at least 4 KB (written only in a
 *   case that never occurs in practice).
 * Errors: PKV_EINVAL for null pointers or sizes out of range, PKV_EHIP when no
 * device is current or the launch fails.
 */
int pkv_probe_mfma(int64_t iters, void* sink, int64_t sink_floats, int64_t* out_flop, void* stream);
int pkv_probe_stream(const void* src, int64_t bytes, void* sink, void* stream);

/* Library version string. */
const char* pkv_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H_ */
