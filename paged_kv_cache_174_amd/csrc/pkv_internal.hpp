// Internal declarations shared by the C-ABI front end (pkv_api.cpp) and the
// HIP kernels.  Not installed; the public interface is include/pkv.h.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "../../include/pkv.h"

namespace pkv {

// Records a printf-style message as the thread's last error and returns `code`.
int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));

// ----------------------------------------------------------------- host metadata

// Physical block at storage block index i of a sequence, negative when it is
// not resident.
typedef int32_t (*BlockAt)(const void* ctx, int64_t i);

// The visible-window read (pkv_window_table): the resident blocks holding a
// sink or recent-window position, in position order, and the tokens they hold.
// Only the sink's block indices and those from the recent window's start on
// are looked up; *reads counts the lookups.
int window_read(BlockAt block_at, const void* ctx, int64_t history_tokens, int64_t query_tokens,
                int64_t sink_tokens, int64_t window_tokens, int32_t block_size, int32_t* out_table,
                int32_t capacity, int32_t* out_count, int32_t* out_kv_len, int64_t* reads);

// ----------------------------------------------------------------- write / gather

struct WriteArgs {
  const void* key;
  const void* value;
  const int64_t* slots;
  void* kpool;
  void* vpool;
  int64_t num_tokens;
  int64_t row_elems;  // num_kv_heads * head_dim
  float k_inv_scale;
  float v_inv_scale;
};
// mode 0: 4-byte copy, 1: 2-byte copy, 2: bf16 -> e4m3 quantise
hipError_t launch_write(const WriteArgs& a, int mode, hipStream_t s);

struct GatherArgs {
  const void* kpool;
  const void* vpool;
  const int32_t* block_ids;
  void* kstage;
  void* vstage;
  int32_t first_block;
  int32_t n_blocks;
  int64_t block_bytes;  // block_size * num_kv_heads * head_dim * element size
};
hipError_t launch_gather(const GatherArgs& a, hipStream_t s);

// ----------------------------------------------------------------- attention

// Rows (query token x query head of one KV group) one MFMA workgroup covers.
constexpr int kMfmaRows = 256;
constexpr int kMfmaKeyTile = 64;
// Most key splits one attention call uses (the combine kernel holds one partial per split in registers).
constexpr int kMaxSplits = 16;

struct AttnArgs {
  const void* q;
  void* out;
  const void* kpool;
  const void* vpool;
  const int32_t* block_table;  // null: K/V are contiguous (logical block i is block i)
  const int32_t* qsl;
  const int32_t* seq_lens;
  const int32_t* segments;
  const int32_t* seg_loc;
  const int32_t* seq_order;  // dispatch order of the sequences, or null (natural order)
  const int32_t* query_pos;  // key position of each sequence's first query row, or null (the suffix)
  float* ws_o;   // split mode: [splits][rows][head_dim] bf16 partial outputs O / l
  float* ws_ml;  // [splits][rows][2] fp32 partial (max, sum), right after ws_o's bf16 rows
  int64_t num_q_tokens;
  int32_t table_width;
  int32_t num_seqs;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t group;      // num_q_heads / num_kv_heads
  int32_t head_dim;
  int32_t block_size;
  int32_t row_tiles;  // query-row tiles per (sequence, KV head)
  int32_t num_splits;
  int32_t split_len;  // keys per split, a multiple of the key tile (fp8 and short-row kernels)
  // Long bf16 kernel: split z covers keys [split_cut[z], split_cut[z + 1]);
  // the cuts are multiples of the key tile except the last, which is
  // max_seq_len, and the lengths never increase with z.
  int32_t split_cut[kMaxSplits + 1];
  int32_t packed;     // short rows: workgroups take the non-empty key ranges first
  float scale_log2;   // softmax_scale * k_scale * log2(e)
  float v_scale;
};

// Block-table entries one MFMA workgroup stages in LDS, so one key split spans at most
// kTableSlice * 16 keys (minus one block for a split that starts mid-block).
constexpr int kTableSlice = 4096;
constexpr int kMaxSplitKeys = (kTableSlice - 1) * 16;

// Rows (query tokens x query heads of one KV head) up to which the short-query
// kernel runs: two 32-row blocks, the keys split four ways inside the workgroup.
constexpr int kShortRows = 64;
// short_rows: every sequence has at most kShortRows rows per KV head (row_tiles == 1).
hipError_t launch_attn_mfma(const AttnArgs& a, bool kv_fp8, bool short_rows, hipStream_t s);
// bf16 K/V, more than kShortRows rows per KV head: four waves, one per SIMD (attn_long.hip).
hipError_t launch_attn_long(const AttnArgs& a, hipStream_t s);
hipError_t launch_attn_combine(const AttnArgs& a, hipStream_t s);
hipError_t launch_attn_f32(const AttnArgs& a, int max_query_len, hipStream_t s);

}  // namespace pkv
