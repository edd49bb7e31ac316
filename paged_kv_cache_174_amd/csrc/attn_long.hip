// Paged attention over long query chunks on the gfx950 matrix cores: bf16
// queries over bf16 K/V pools, head_dim 128.
//
// Work decomposition
//   A "row" is one (query token, query head) pair of a KV-head group, token
//   major, so the G = Hq / Hkv heads that share a K/V tile are computed from
//   one LDS copy of it (GQA).  A workgroup of four waves -- one per SIMD --
//   owns 256 consecutive rows of one (sequence, KV head) and, when the key
//   range is split, one range of keys (the host's split_cut; the ranges may
//   differ in length, longest first).  Each wave owns 64 rows as two halves
//   A and B of 32 rows, each one column block of the 32x32x16 bf16 MFMA.
//
// Why one wave per SIMD, two halves per wave
//   A SIMD overlaps a wave's own VALU work with that wave's MFMAs almost for
//   free (up to ~28 cycles of VALU beside each 32-cycle MFMA), while VALU
//   work of a second wave on the same SIMD slows an MFMA stream by about half.
//   So the softmax of one half runs inside the instruction stream that feeds
//   the other half's MFMAs.  Per 64-key tile t a wave runs two phases:
//     alpha(u): softmax of A(u)  beside  QK of B(u) and PV of B(u - 1)
//     beta(u):  softmax of B(u)  beside  QK of A(u + 1) and PV of A(u)
//   over 32-key sub-tiles u, 18 MFMAs per phase (8 QK, 8 PV, 2 row sums);
//   the K and V operand reads of a sub-tile feed both halves.
//
// Softmax without a per-tile maximum
//   Probabilities are exp2(s * c - m * c) with a running maximum m that is
//   fixed after each half's first 32 keys (their exact maximum): softmax is
//   exact for any common offset, so a stale m changes nothing but rounding,
//   and O and l are never rescaled in the loop.  Row sums are taken on the
//   matrix cores (a 16x16x32 MFMA of a 0/1 selector with P^T), i.e. of the
//   bf16-rounded probabilities that multiply V.  If a row's sum passes kFastSumLimit (2^64) or is not finite --
//   some later score rose more than 64 / c above the first keys' maximum --
//   the workgroup recomputes its key range exactly, tile by tile, with the
//   maximum moving per sub-tile and O and l rescaled.
//
// K/V tiles (64 keys) in LDS
//   Row-major bf16, one 256-byte row per key, 16-byte chunks XOR-permuted
//   (k_swz / v_swz) so the MFMA operand reads are free of bank conflicts.
//   Wave w copies the tile's 16-key block w straight from HBM into LDS
//   (buffer_load_dwordx4 ... lds, four rows per load) through the block-table
//   slice staged in LDS once per workgroup; the buffer descriptor's range
//   ends at the key limit, so keys past it arrive as zeros.  Four tile
//   buffers: the four phases after tile X - 3's barrier issue the wave's
//   eight loads of tile X (K rows 0-7, K 8-15, V 0-7, V 8-15 of its block),
//   into the buffer tile X - 4 left.  One barrier per tile, before the phase
//   that first reads the next tile.
//
// Epilogue: O / l rounded to bf16, staged through LDS and stored as whole
// 256-byte rows; with split keys the partial (O / l in bf16, (max, sum) in
// fp32) goes to the workspace for the merge kernel.
#include <type_traits>

#include "attn_common.hpp"
#include "mfma_util.hpp"

namespace pkv {

namespace {

using namespace mx;

constexpr int NW = 4;  // waves per workgroup, one per SIMD
constexpr int NT = 64 * NW;
constexpr int kHalfRows = 32;
constexpr int kWaveRows = 2 * kHalfRows;
static_assert(kMfmaRows == NW * kWaveRows, "rows per workgroup");
static_assert(kMfmaKeyTile == kTileKeys, "key tile");
constexpr int kBufs = 4;
// A row whose probability sum passes this (or is not a number) sends the
// workgroup to the exact rerun: some score rose more than 64 / (scale log2 e)
// above its first sub-tile's maximum, near the top of fp32's range.
constexpr float kFastSumLimit = 18446744073709551616.0f;  // 2^64
static_assert(NW * kWaveRows * kRowBytes <= kBufs * kTileBytes, "the epilogue stages every wave's rows in the K buffers");
static_assert(2 * kBufs * kTileBytes + kTableSlice * 4 <= 160 * 1024, "LDS budget of a gfx950 CU");

__shared__ __attribute__((aligned(16))) uint8_t s_k[kBufs][kTileBytes];
__shared__ __attribute__((aligned(16))) uint8_t s_v[kBufs][kTileBytes];
__shared__ int32_t s_tbl[kTableSlice];  // the workgroup's slice of its block-table row
__shared__ int32_t s_overflow[NW];      // per wave: some row's probability sum passed kFastSumLimit

// Fourth word of a raw buffer descriptor on gfx9 (32-bit data format).
constexpr int kBufferWord3 = 0x00020000;
// A lane offset past every descriptor's range (a K/V descriptor spans at most
// 16 rows of a few KB, the Q descriptor exactly this, with offsets below 65
// tokens of one chunk): the lane's 16 bytes arrive as zeros.
constexpr uint32_t kPastRange = 0x40000000u;

template <int B>
using Buf = std::integral_constant<int, B>;

// One 16-byte-per-lane direct load through a buffer descriptor into LDS:
// lane i's 16 bytes at byte offset off of the descriptor's range land at
// l + 16 i; offsets at or past the range read zeros.  Inline assembly, so
// the compiler adds no waits for it (the kernel waits with wait_vmcnt).  It
// carries the one wait state needed after M0 is written.  A vector-memory
// read of an SGPR also needs five after a VALU write of it (v_readfirstlane),
// which the compiler does not insert for inline assembly; the descriptors
// here are built on the scalar unit from values made wave-uniform long
// before, so no such write comes near a load (the kernel's assembly is
// checked for it).  Five wait states are twenty cycles of a wave's issue,
// which would be paid on every load.
__device__ __forceinline__ void dma16_buf(u32x4 r, uint32_t off, const void* l) {
  const uint32_t m0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_ptr)l));
  asm volatile("s_nop 0\nbuffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(off), "s"(r), "{m0}"(m0));
}
__global__ __attribute__((amdgpu_flat_work_group_size(NT, NT), amdgpu_waves_per_eu(1, 1))) void
attn_long_kernel(AttnArgs a) {
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l32 = lane & 31;
  const int h2 = lane >> 5;

  // ---- work item.  Workgroups are dealt to the 8 XCDs round-robin by id;
  // all workgroups of one (sequence, KV head) go to one XCD (they share its
  // L2 for the group's K/V), and consecutive groups to different XCDs.
  // Inside an XCD the items go out split by split -- every group's split 0,
  // then split 1, ... -- and within a split from the last row tile to the
  // first.  Split lengths never increase with z, and a later row tile never
  // sees fewer keys than an earlier one, so the longest items go first and the
  // short ones fill in behind them.
  const uint32_t xcd = blockIdx.x & 7u, pos = blockIdx.x >> 3;
  const uint32_t groups = static_cast<uint32_t>(a.num_seqs) * static_cast<uint32_t>(a.num_kv_heads);
  const uint32_t per_split = (groups + 7u) / 8u * static_cast<uint32_t>(a.row_tiles);
  const int z = static_cast<int>(pos / per_split);
  const uint32_t rem = pos % per_split;
  const uint32_t grp = xcd + 8u * (rem / static_cast<uint32_t>(a.row_tiles));
  if (grp >= groups) return;
  const int rt = a.row_tiles - 1 - static_cast<int>(rem % static_cast<uint32_t>(a.row_tiles));
  const int hk = static_cast<int>(grp % static_cast<uint32_t>(a.num_kv_heads));
  const int b_pos = static_cast<int>(grp / static_cast<uint32_t>(a.num_kv_heads));
  // ---- the workgroup's sequence and its metadata, in as few dependent
  // rounds of loads as possible (each is a trip to memory):
  //   1. the sequence id (seq_order) and, with at most 64 sequences, every
  //      sequence's entries (lane i loads sequence i's), read out of the
  //      lanes once the id is known;
  //   2. the sequence's segments, the block-table slice of the whole key
  //      range a split may cover (a bound that needs no segment) and Q;
  // all of it into registers and used up before the first direct-to-LDS
  // load goes out (the compiler waits for a load of its own with a vmcnt
  // that would also drain every direct load issued before the wait).
  // Round 1 goes to the vector memory unit as a whole (an opaque
  // lane offset keeps the sequence-id load there too): scalar loads share
  // one counter with the argument loads, and a wait for an argument pointer
  // would also wait for the id and put the per-lane loads in a round of
  // their own.
  int b, t0, t1, s, seg0, seg1, qpos;
  {
    int vzero = 0;
    asm volatile("" : "+v"(vzero));
    const int vb = a.seq_order ? a.seq_order[b_pos + vzero] : b_pos;
    if (a.num_seqs <= 64) {
      const int li = min(lane, a.num_seqs - 1);
      const int v_t0 = a.qsl[li], v_t1 = a.qsl[li + 1], v_s = a.seq_lens[li];
      const int v_g0 = a.seg_loc[li], v_g1 = a.seg_loc[li + 1];
      const int v_qp = a.query_pos ? a.query_pos[li] : 0;
      b = __builtin_amdgcn_readfirstlane(vb);
      t0 = __builtin_amdgcn_readlane(v_t0, b);
      t1 = __builtin_amdgcn_readlane(v_t1, b);
      s = __builtin_amdgcn_readlane(v_s, b);
      seg0 = __builtin_amdgcn_readlane(v_g0, b);
      seg1 = __builtin_amdgcn_readlane(v_g1, b);
      qpos = __builtin_amdgcn_readlane(v_qp, b);
    } else {
      b = __builtin_amdgcn_readfirstlane(vb);
      t0 = a.qsl[b];
      t1 = a.qsl[b + 1];
      s = a.seq_lens[b];
      seg0 = a.seg_loc[b];
      seg1 = a.seg_loc[b + 1];
      qpos = a.query_pos ? a.query_pos[b] : 0;
    }
  }
  const int G = a.group;
  const int q_len = t1 - t0;
  const int R = q_len * G;
  const int r0 = rt * kMfmaRows;
  const int gbase = a.query_pos ? qpos : s - q_len;  // key position of the first query row

  const int wr0 = r0 + kWaveRows * w;  // first row of this wave
  const bool active = wr0 < R;

  // ---- this lane's query row in each half
  bool valid[2];
  int tok[2], head[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int row = wr0 + kHalfRows * h + l32;
    valid[h] = row < R;
    tok[h] = valid[h] ? row / G : 0;
    head[h] = hk * G + (valid[h] ? row % G : 0);
  }

  if (r0 >= R) return;
  // Round 2.  Block-table slice (no table: the K/V buffers are one
  // contiguous run, logical block i is block i).
  const int k_begin = a.split_cut[z], k_stop = a.split_cut[z + 1];
  const int nblk = (s + 15) >> 4;
  const int blk_lo = k_begin >> 4;
  const int blk_cap = min(min((k_stop + 15) >> 4, nblk), blk_lo + kTableSlice);
  const int32_t* const table = a.block_table ? a.block_table + static_cast<int64_t>(b) * a.table_width : nullptr;
  const int tid = static_cast<int>(threadIdx.x);
  int te = blk_lo + tid;
  if (table && tid < blk_cap - blk_lo) te = table[blk_lo + tid];
  const SegCache segc = load_segments(a.segments, seg0, seg1);
  // Q by whole rows: load st brings rows 4 st + lane / 16 of the wave, 16
  // bytes (chunk lane % 16) per lane, so each load is 1 KB of consecutive
  // 256-byte rows.  (A load in the MFMA operand layout would take 32 bytes
  // of each of 32 rows, pieces whose address processing makes Q arrive
  // several times later than the table slice.)  Buffer loads, so that the
  // sixteen go out unconditionally, together with the table and segment
  // loads: rows past the chunk and chunks past head_dim get an offset past
  // the descriptor's range and read zeros.  head_dim 64 runs through the same
  // 128-wide kernel with head-dim [64, 128) of Q, K and V zero: it adds
  // nothing to a score, and the output's upper half is never stored.
  const int dh = a.head_dim;  // 64 or 128
  u32x4 qv[16];
  {
    const int tok_w0 = wr0 / G;
    const uint8_t* const qbase = static_cast<const uint8_t*>(a.q) +
                                 (static_cast<int64_t>(t0 + tok_w0) * a.num_q_heads + hk * G) * 2 * dh;
    const __amdgpu_buffer_rsrc_t qrs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(qbase), 0, static_cast<int>(kPastRange), kBufferWord3);
    // The lane's row of load st is head g of its token; roff is the row's
    // byte offset from qbase.
    const int head_b = 2 * dh, tok_b = a.num_q_heads * head_b;
    const int gr = wr0 + (lane >> 4);
    int g = gr % G;
    int roff = (gr / G - tok_w0) * tok_b + g * head_b;
    const int step_g = 4 % G, step_off = (4 / G) * tok_b + step_g * head_b, wrap_off = tok_b - G * head_b;
    const bool in_row = 16 * (lane & 15) < head_b;
#pragma unroll
    for (int st = 0; st < 16; ++st) {
      const bool ok = wr0 + 4 * st + (lane >> 4) < R && in_row;
      qv[st] = __builtin_amdgcn_raw_buffer_load_b128(qrs, ok ? roff + 16 * (lane & 15) : static_cast<int>(kPastRange), 0, 0);
      g += step_g;
      roff += step_off;
      if (g >= G) {
        g -= G;
        roff += wrap_off;
      }
    }
  }
  if (tid < blk_cap - blk_lo) s_tbl[tid] = te;
  for (int i = tid + NT; i < blk_cap - blk_lo; i += NT) s_tbl[i] = table ? table[blk_lo + i] : blk_lo + i;
  // Row limits are non-decreasing in the row's key position (the metadata
  // check enforces it), so the tile's last row bounds the workgroup's keys
  // and a wave's first row its mask-free prefix.
  const int wg_kmax = row_limit(segc, a.segments, seg0, seg1, gbase + (min(r0 + kMfmaRows, R) - 1) / G);
  const int k_end = min(k_stop, wg_kmax);
  const int64_t total_rows = a.num_q_tokens * a.num_q_heads;
  if (k_begin >= k_end) {
    // No key of this split is visible to any row of the tile: its partial is
    // empty (max -inf, sum 0), which the merge skips.
    if (a.num_splits > 1 && threadIdx.x < kMfmaRows) {
      const int row = r0 + static_cast<int>(threadIdx.x);
      if (row < R) {
        const int64_t orow = static_cast<int64_t>(t0 + row / G) * a.num_q_heads + hk * G + row % G;
        const f32x2 ml = {-INFINITY, 0.f};
        *reinterpret_cast<f32x2*>(a.ws_ml + (static_cast<int64_t>(z) * total_rows + orow) * 2) = ml;
      }
    }
    return;
  }
  const int wave_kmin = active ? row_limit(segc, a.segments, seg0, seg1, gbase + wr0 / G) : 0;
  int lrow[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) lrow[h] = valid[h] ? row_limit(segc, a.segments, seg0, seg1, gbase + tok[h]) : 0;
  const int blk_hi = min((k_end + 15) >> 4, nblk);

  // Q^T fragments for S^T = K Q^T: for k-step t the lane holds head-dim
  // [16 t + 8 h2, +8) of the wave's row 32 h + l32.  They go through LDS:
  // the wave's row r to tile row 16 w + r % 16 of K buffer r / 16 in the K
  // tile layout (where the wave later stages its own key block of tiles 0-3,
  // so no other wave writes there), and are read back like K's operands,
  // straight into AGPRs, which the QK products read them from (copied there
  // later, the register allocator spreads them over both register files and
  // moves them back in every phase).
  bf16x8 qf[2][8];
  {
#pragma unroll
    for (int st = 0; st < 16; ++st) {
      const int rr = 4 * (st & 3) + (lane >> 4);  // tile row - 16 w
      *reinterpret_cast<__attribute__((address_space(3))) u32x4*>(
          lds_addr(s_k[st >> 2]) + (16 * w + rr) * kRowBytes + 16 * ((lane & 15) ^ k_swz(rr))) = qv[st];
    }
    const int rq = l32 & 15;
    const uint32_t qrd = lds_addr(s_k[l32 >> 4]) + (16 * w + rq) * kRowBytes;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int t = 0; t < 8; ++t) qf[h][t] = *lds_at<bf16x8>(qrd + 2 * h * kTileBytes + 16 * ((2 * t + h2) ^ k_swz(rq)));
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int t = 0; t < 8; ++t) asm volatile("" : "+a"(qf[h][t]));
  }
  // The table slice is in LDS, and every wave has its Q fragments (a wave's
  // tile loads overwrite its Q rows).
  lds_barrier();
  // Keys at or past kv_lim are staged as zeros: past seq_len they do not
  // exist (their slots may hold anything), past the slice every row of the
  // workgroup masks them.
  const int kv_lim = min(s, blk_hi * 16);
  const int ntiles = (k_end - k_begin + kTileKeys - 1) / kTileKeys;

  // ---- staging geometry: wave w copies block w of each tile, rows
  // 16 w + 4 st + lane / 16 (st = 0..3), chunk position lane % 16.
  const int64_t row_bytes = static_cast<int64_t>(a.num_kv_heads) * dh * 2;
  const int64_t block_bytes = 16 * row_bytes;
  const uint8_t* kpool = static_cast<const uint8_t*>(a.kpool) + static_cast<int64_t>(hk) * dh * 2;
  const uint8_t* vpool = static_cast<const uint8_t*>(a.vpool) + static_cast<int64_t>(hk) * dh * 2;
  const int st_pos = lane & 15;
  const int st_sub = lane >> 4;
  // A chunk past head_dim gets an offset past the descriptor's range: it
  // arrives as zeros.
  uint32_t k_src_off[4], v_src_off[4];
#pragma unroll
  for (int st = 0; st < 4; ++st) {
    const int rb = 4 * st + st_sub;  // row inside the block (= tile row - 16 w)
    const int kc = st_pos ^ k_swz(rb), vc = st_pos ^ v_swz(rb);  // source chunks
    k_src_off[st] = 16 * kc < 2 * dh ? static_cast<uint32_t>(rb * row_bytes + 16 * kc) : kPastRange;
    v_src_off[st] = 16 * vc < 2 * dh ? static_cast<uint32_t>(rb * row_bytes + 16 * vc) : kPastRange;
  }
  // Direct loads through a buffer descriptor whose range ends at the last
  // key below kv_lim in this wave's block: rows past it are out of range and
  // arrive as zeros (past seq_len they do not exist and their slots may hold
  // anything; past the slice every row of the workgroup masks them), so a
  // value row that does not exist is 0, never garbage.  Base, range and the
  // lane offsets (k_src_off / v_src_off) need no vector arithmetic.
  // (A block past the slice only feeds rows past kv_lim, so any entry of the
  // slice serves; clamping keeps the lookup branch-free.)
  auto block_entry = [&](int kt) { return s_tbl[min((kt >> 4) + w - blk_lo, blk_hi - blk_lo - 1)]; };
  auto entry_base = [&](int e) { return static_cast<int64_t>(__builtin_amdgcn_readfirstlane(e)) * block_bytes; };
  auto block_base = [&](int kt) { return entry_base(block_entry(kt)); };
  // (The descriptor must live in SGPRs: its parts are made wave-uniform
  // explicitly, as the compiler cannot prove it for the range.)
  // The descriptor is built by scalar instructions only, whatever the
  // compiler does around it: base = pool + boff (stride 0), range = (rows of
  // the block below kv_lim) x row_bytes.  Its inputs are wave-uniform values
  // (a v_readfirstlane may make them; the scalar unit waits for those, the
  // direct load reads only what the scalar unit wrote).
  const int kv_lim_w = __builtin_amdgcn_readfirstlane(kv_lim - 16 * w);
  const int row_bytes32 = __builtin_amdgcn_readfirstlane(static_cast<int>(row_bytes));
  auto rsrc = [&](const uint8_t* pool, int64_t boff, int kt) {
    const uint64_t p = reinterpret_cast<uint64_t>(pool);
    const uint64_t o = static_cast<uint64_t>(boff);
    uint32_t lo, hi, bytes;
    asm("s_add_u32 %0, %3, %5\n"
        "s_addc_u32 %1, %4, %6\n"
        "s_and_b32 %1, %1, 0xffff\n"
        "s_sub_i32 %2, %7, %8\n"
        "s_max_i32 %2, %2, 0\n"
        "s_min_i32 %2, %2, 16\n"
        "s_mul_i32 %2, %2, %9"
        : "=&s"(lo), "=&s"(hi), "=&s"(bytes)
        : "s"(static_cast<uint32_t>(p)), "s"(static_cast<uint32_t>(p >> 32)), "s"(static_cast<uint32_t>(o)),
          "s"(static_cast<uint32_t>(o >> 32)), "s"(kv_lim_w), "s"(kt), "s"(row_bytes32)
        : "scc");
    const u32x4 d = {lo, hi, bytes, static_cast<uint32_t>(kBufferWord3)};
    return d;
  };
  // Row group st (four rows) of this wave's block into buffer B.
  auto load_k = [&](int kt, auto bufc, int64_t boff, int st) {
    constexpr int B = decltype(bufc)::value;
    dma16_buf(rsrc(kpool, boff, kt), k_src_off[st], s_k[B] + (16 * w + 4 * st) * kRowBytes);
  };
  auto load_v = [&](int kt, auto bufc, int64_t boff, int st) {
    constexpr int B = decltype(bufc)::value;
    dma16_buf(rsrc(vpool, boff, kt), v_src_off[st], s_v[B] + (16 * w + 4 * st) * kRowBytes);
  };

  // ---- MFMA operand addresses (bytes, buffer 0; buffer and key block are
  // constant offsets)
  uint32_t k_rd[8];  // K row 32 kb + l32, chunk 2 t + h2
#pragma unroll
  for (int t = 0; t < 8; ++t) k_rd[t] = lds_addr(s_k[0] + l32 * kRowBytes + 16 * ((2 * t + h2) ^ k_swz(l32)));
  // V^T via transposing reads: in each 16-lane group g, lane 4 j + q names the
  // 8-byte piece of V row 4 (g / 2) + j holding head-dim [16 (g % 2) + 4 q, +4)
  // of head-dim block db; the instruction hands lane i of the group element
  // i % 4 of the pieces named by lanes 4 j + i / 4, i.e. V[key(j)][d(lane)].
  uint32_t v_rd[4];
  {
    const int g = lane >> 4, j = (lane >> 2) & 3, q = lane & 3;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const int c = 4 * db + 2 * (g & 1) + (q >> 1);
      v_rd[db] = lds_addr(s_v[0] + (4 * (g >> 1) + j) * kRowBytes + 16 * (c ^ v_swz(j)) + 8 * (q & 1));
    }
  }
  auto k_frag = [&](uint32_t buf_off, int kb, int t) {
    return *lds_at<bf16x8>(k_rd[t] + buf_off + kb * 32 * kRowBytes);
  };
  auto v_frag = [&](uint32_t buf_off, int kb, int k16, int db) {
    const uint32_t base = v_rd[db] + buf_off + (32 * kb + 16 * k16) * kRowBytes;
    const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(lds_v4i16(base));
    const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(lds_v4i16(base + 8 * kRowBytes));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };

  const float sl = a.scale_log2;
  float m[2] = {-INFINITY, -INFINITY};
  float l[2] = {0.f, 0.f};
  f32x16 o[2][4];  // O^T of each half, head-dim blocks db = 0..3
  f32x16 sc[2];    // scores of each half for one 32-key sub-tile
  bf16x8 pb[2][2];  // probabilities of each half as PV operands, k16 = 0, 1
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[h][db][r] = 0.f;

  // Byte offset of key block kb (0, 1) of the tile buffer B.
  auto blk_off = [](int B, int kb) { return static_cast<uint32_t>(B * kTileBytes + kb * 32 * kRowBytes); };
  // S^T of half h for the 32-key sub-tile at byte offset off (exact step).
  auto qk_full = [&](int h, uint32_t off) __attribute__((always_inline)) {
#pragma unroll
    for (int r = 0; r < 16; ++r) sc[h][r] = 0.f;
#pragma unroll
    for (int t = 0; t < 8; ++t) sc[h] = mfma(k_frag(off, 0, t), qf[h][t], sc[h]);
  };
  // Keys j >= L(row) of half h get -inf.  Lane (l32, h2) holds key
  // kt + 8 (r / 4) + 4 h2 + r % 4 in element r, so one bound per lane is
  // compared with constants.
  auto mask = [&](int h, int kt) __attribute__((always_inline)) {
    const int lim = lrow[h] - kt - 4 * h2;
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (8 * (r >> 2) + (r & 3) >= lim) sc[h][r] = -INFINITY;
  };
  // Probabilities of half h at its running max, packed for PV; returns the
  // lane's partial row sum.
  auto exps = [&](int h) __attribute__((always_inline)) {
    const float mc = (m[h] == -INFINITY) ? 0.f : m[h] * sl;
    float ls[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k16 = 0; k16 < 2; ++k16) {
      u32x4 pk;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float p0 = __builtin_amdgcn_exp2f(fmaf(sc[h][8 * k16 + 2 * e], sl, -mc));
        const float p1 = __builtin_amdgcn_exp2f(fmaf(sc[h][8 * k16 + 2 * e + 1], sl, -mc));
        pk[e] = pack_bf16_rne(p0, p1);
        ls[e] = (ls[e] + p0) + p1;
      }
      pb[h][k16] = __builtin_bit_cast(bf16x8, pk);
    }
    return (ls[0] + ls[1]) + (ls[2] + ls[3]);
  };
  // First sub-tile of a half: its exact maximum is the running max m, fixed
  // for the rest of the fast loop (O is still zero, so nothing is rescaled).
  // mcs = m * scale * log2(e) is the shift of every later exponent.
  float mcs[2] = {0.f, 0.f};
  auto softmax_first = [&](int h, int kt) __attribute__((always_inline)) {
    if (kt + 32 > wave_kmin) mask(h, kt);
    float c4[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) c4[i] = fmaxf(fmaxf(fmaxf(sc[h][i], sc[h][i + 4]), sc[h][i + 8]), sc[h][i + 12]);
    m[h] = max_halves(fmaxf(fmaxf(c4[0], c4[1]), fmaxf(c4[2], c4[3])));
    mcs[h] = (m[h] == -INFINITY) ? 0.f : m[h] * sl;
    (void)exps(h);
  };

  auto kt_of = [&](int t) { return k_begin + t * kTileKeys; };

  // MFMA operands held in registers so that each K and V fragment is read
  // from LDS once per wave and serves both halves: kfr the K operands of one
  // sub-tile (k-steps 0..7), vfr[2] the V^T operands of two sub-tiles
  // ([k16][db]), alternating with the sub-tile's parity.
  bf16x8 kfr[8];
  bf16x8 vfr[2][2][4];
  // Row sums on the matrix cores, of the bf16 probabilities -- exactly the
  // weights that multiply V.  A PV operand pb (16 keys of 32 rows; lane l
  // holds row l % 32, keys 8 (l / 32) .. + 7) read as the B operand of the
  // 16x16x32 MFMA gives column n = l % 16 the lanes n, n + 16, n + 32, n + 48,
  // i.e. rows n and n + 16, each with both key halves.  The selector A takes
  // lane groups 0 and 2 (row n) into output rows 0..7 and groups 1 and 3
  // (row n + 16) into 8..15, so rs[h] += sel x pb puts row n's sum in lanes n
  // and n + 16 and row n + 16's in lanes n + 32 and n + 48, at half the
  // matrix work of a 32x32x16 product.
  f32x4 rs[2];
  bf16x8 sel;
  {
    const bool lower = (lane & 15) < 8, even_group = ((lane >> 4) & 1) == 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) sel[i] = static_cast<__bf16>(lower == even_group ? 1.0f : 0.0f);
  }
  // (opaque from here on: kept in registers rather than rebuilt in every phase)
  asm volatile("" : "+v"(sel));
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int r = 0; r < 4; ++r) rs[h][r] = 0.f;

  // One phase: 18 slots, each one MFMA plus at most ~28 cycles of other
  // issue (a 32-cycle MFMA hides that much of its own wave's work, a
  // 16-cycle row-sum MFMA about 12; a wave issues in order, so more, or an
  // instruction waiting on a result, idles the matrix pipe).  Two forms:
  //   alpha(u) (BETA false): slots 0-7 and 10-17 alternate QK B(u) (from kfr)
  //     and PV B(u - 1) (from vfr[VPV]); 8-9 B(u - 1)'s row sums; slots 0-7
  //     each read one V(u) operand (tile buffer BR, key block KR) into
  //     vfr[1 - VPV].
  //   beta(u) (BETA true): slots 0-7 PV A(u) (from vfr[VPV]), each reading
  //     one K operand of u + 1 (BR, KR) into kfr; 8-15 QK A(u + 1) from those
  //     operands; 16-17 A(u)'s row sums.
  // With SOFT the probabilities of the other half (HS) from its scores:
  // scale-and-shift of two scores in each of slots 0-7, their exponentials
  // in slots 8-15 and their bf16 packs in slots 10-17, each stage a slot or
  // more after the one it reads.  With LOAD 1 (K) or 2 (V), row groups ST0
  // and ST0 + 1 of this wave's block of tile t_load go into buffer BL in
  // slots 16 and 17 (boff: the block's byte offset, looked up before the
  // previous barrier).  sched_barrier keeps every slot in place.
  auto phase = [&](auto beta_c, auto br_c, auto kr_c, auto vpv_c, auto soft_c, auto load_c, auto st0_c, auto bl_c,
                   int t_load, int64_t boff) __attribute__((always_inline)) {
    constexpr bool BETA = decltype(beta_c)::value;
    constexpr int BR = decltype(br_c)::value, KR = decltype(kr_c)::value, VPV = decltype(vpv_c)::value;
    constexpr bool SOFT = decltype(soft_c)::value;
    constexpr int LOAD = decltype(load_c)::value, ST0 = decltype(st0_c)::value, BL = decltype(bl_c)::value;
    constexpr int HQ = BETA ? 0 : 1, HS = 1 - HQ, HP = HQ;
    const uint32_t roff = blk_off(BR, KR);
    const int kt_load = kt_of(t_load);
    u32x4 drs = {0u, 0u, 0u, 0u};
    if constexpr (LOAD != 0) drs = rsrc(LOAD == 1 ? kpool : vpool, boff, kt_load);
    float p[16];
    u32x4 pk[2];
#pragma unroll
    for (int r = 0; r < 16; ++r) sc[HQ][r] = 0.f;
#pragma unroll
    for (int j = 0; j < 18; ++j) {
      // the slot's MFMA
      if constexpr (!BETA) {
        if (j == 8 || j == 9) {
          rs[HP] = mfma16(sel, pb[HP][j - 8], rs[HP]);
        } else {
          const int jj = j < 8 ? j : j - 2;
          if ((jj & 1) == 0) {
            sc[HQ] = mfma(kfr[jj >> 1], qf[HQ][jj >> 1], sc[HQ]);
          } else {
            const int q = jj >> 1;  // PV operand (k16, db) = (q / 4, q % 4)
            o[HP][q & 3] = mfma(vfr[VPV][q >> 2][q & 3], pb[HP][q >> 2], o[HP][q & 3]);
          }
        }
      } else {
        if (j < 8) {
          o[HP][j & 3] = mfma(vfr[VPV][j >> 2][j & 3], pb[HP][j >> 2], o[HP][j & 3]);
        } else if (j < 16) {
          sc[HQ] = mfma(kfr[j - 8], qf[HQ][j - 8], sc[HQ]);
        } else {
          rs[HP] = mfma16(sel, pb[HP][j - 16], rs[HP]);
        }
      }
      // LDS operand reads
      if (j < 8) {
        if constexpr (!BETA) vfr[1 - VPV][j >> 2][j & 3] = v_frag(roff, 0, j >> 2, j & 3);
        else kfr[j] = k_frag(roff, 0, j);
      }
      // softmax of half HS
      if constexpr (SOFT) {
        if (j < 8) {
          p[2 * j] = fmaf(sc[HS][2 * j], sl, -mcs[HS]);
          p[2 * j + 1] = fmaf(sc[HS][2 * j + 1], sl, -mcs[HS]);
          asm volatile("" : "+v"(p[2 * j]), "+v"(p[2 * j + 1]));
        }
        if (j >= 8 && j < 16) {
          const int e = j - 8;
          p[2 * e] = __builtin_amdgcn_exp2f(p[2 * e]);
          p[2 * e + 1] = __builtin_amdgcn_exp2f(p[2 * e + 1]);
          asm volatile("" : "+v"(p[2 * e]), "+v"(p[2 * e + 1]));
        }
        if (j >= 10) {
          const int e = j - 10;  // scores 2 e, 2 e + 1: pair e % 4 of operand k16 = e / 4
          uint32_t x = pack_bf16_rne(p[2 * e], p[2 * e + 1]);
          asm volatile("" : "+v"(x));
          pk[e >> 2][e & 3] = x;
        }
      }
      if constexpr (LOAD != 0) {
        if (j >= 16) {
          const int st = ST0 + (j - 16);
          dma16_buf(drs, LOAD == 1 ? k_src_off[st] : v_src_off[st],
                    (LOAD == 1 ? s_k[BL] : s_v[BL]) + (16 * w + 4 * st) * kRowBytes);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (SOFT) {
#pragma unroll
      for (int k16 = 0; k16 < 2; ++k16) pb[HS][k16] = __builtin_bit_cast(bf16x8, pk[k16]);
    }
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using Soft = std::true_type;
  using NoSoft = std::false_type;
  using Alpha = std::false_type;
  using Beta = std::true_type;

  // The pipeline over 32-key sub-tiles u (tile u / 2, key block u % 2):
  //   alpha(u): softmax A(u) | QK B(u), PV B(u - 1); reads V(u)
  //   beta(u):  softmax B(u) | PV A(u), QK A(u + 1); reads K(u + 1)
  // Tile t runs alpha(2t), beta(2t), alpha(2t+1), then -- once every wave's
  // loads of tile t+1 have landed -- the barrier, then beta(2t+1), which
  // reads tile t+1.  Tile X's loads go out in the four phases after the
  // barrier of tile X - 3 (K row groups 0-1, K 2-3, V 0-1, V 2-3), into the
  // buffer tile X - 4 left: its last reads (V of its second sub-tile) ran in
  // alpha of that sub-tile, before the barrier of tile X - 3.  The QK of A
  // one past the last sub-tile reads a stale buffer and is never used.
  // Prologue: tiles 0, 1, 2 in full.
  {
    auto go = [&](int j, auto bufc) {
      const int kt = kt_of(j);
      const int64_t boff = block_base(kt);
#pragma unroll
      for (int st = 0; st < 4; ++st) load_k(kt, bufc, boff, st);
#pragma unroll
      for (int st = 0; st < 4; ++st) load_v(kt, bufc, boff, st);
    };
    go(0, Buf<0>{});
    go(1, Buf<1>{});
    go(2, Buf<2>{});
  }
  wait_vmcnt<16>();  // tile 0 landed
  lds_barrier();
  // A wave with no rows (the chunk's last row tile) only takes its share of
  // the loads and the barriers.
  auto idle_loads = [&](auto load_c, auto st0_c, auto buf_c, int t_load, int64_t boff) {
    constexpr int LOAD = decltype(load_c)::value, ST0 = decltype(st0_c)::value;
    const int kt = kt_of(t_load);
#pragma unroll
    for (int st = ST0; st < ST0 + 2; ++st) {
      if constexpr (LOAD == 1) load_k(kt, buf_c, boff, st);
      else load_v(kt, buf_c, boff, st);
    }
  };
  const int kt0 = kt_of(0);
  const bool edge0 = kt0 + 64 > wave_kmin;
  if (active) {
    qk_full(0, blk_off(0, 0));
    softmax_first(0, kt0);
    qk_full(1, blk_off(0, 0));
    softmax_first(1, kt0);
    // V(0) operands
#pragma unroll
    for (int k16 = 0; k16 < 2; ++k16)
#pragma unroll
      for (int db = 0; db < 4; ++db) vfr[0][k16][db] = v_frag(blk_off(0, 0), 0, k16, db);
    // beta(0) without a softmax: PV A(0), QK A(1) (K(1) read here)
    phase(Beta{}, Buf<0>{}, I1{}, I0{}, NoSoft{}, I0{}, I0{}, Buf<0>{}, 0, 0);
    // alpha(1): QK B(1), PV B(0); reads V(1)
    if (edge0) mask(0, kt0 + 32);
    phase(Alpha{}, Buf<0>{}, I1{}, I0{}, Soft{}, I0{}, I0{}, Buf<0>{}, 0, 0);
  }
  // Block of this wave's loads of tile 3 (the barrier's wait covers the LDS read).
  const int e3 = block_entry(kt_of(3));
  wait_vmcnt<8>();  // tile 1 landed
  lds_barrier();
  const int64_t boff_next = entry_base(e3);
  if (active) {
    // beta(1): PV A(1), QK A(2) (K(2) from tile 1); K rows 0-1 of tile 3
    if (edge0) mask(1, kt0 + 32);
    phase(Beta{}, Buf<1>{}, I0{}, I1{}, Soft{}, I1{}, I0{}, Buf<3>{}, 3, boff_next);
  } else {
    idle_loads(I1{}, I0{}, Buf<3>{}, 3, boff_next);
  }

  // Tile t >= 1 in buffer T = t % 4.
  // boff_load: block offset of this wave's loads of tile t + 2 (looked up
  // in the previous tile); the lookup for tile t + 3 goes before the barrier.
  int64_t boff_load = boff_next;
  // (Two copies of the loop, one for waves with rows and one for waves
  // without, so that no phase sits behind a branch; the mask checks are
  // expected false, which keeps the unmasked path straight-line.)
  auto tile = [&](auto tc, int t, auto act_c) __attribute__((always_inline)) {
    constexpr int T = decltype(tc)::value;
    constexpr bool ACT = decltype(act_c)::value;
    constexpr int Tp1 = (T + 1) % kBufs, Tp2 = (T + 2) % kBufs, Tp3 = (T + 3) % kBufs;
    const int kt = kt_of(t);
    const bool edge = kt + kTileKeys > wave_kmin;  // some row of the wave masks keys of this tile
    // Block of this wave's loads of tile t + 3, read from LDS here so that
    // its latency passes under the phases instead of in front of the barrier.
    const int e_next = block_entry(kt_of(t + 3));
    if constexpr (ACT) {
      // alpha(2t): QK B(2t), PV B(2t-1) [vfr 1]; reads V(2t) [T, 0] into vfr 0; K rows 2-3 of tile t+2
      if (__builtin_expect(edge, 0)) mask(0, kt);
      phase(Alpha{}, Buf<T>{}, I0{}, I1{}, Soft{}, I1{}, I2{}, Buf<Tp2>{}, t + 2, boff_load);
      // beta(2t): PV A(2t) [vfr 0], QK A(2t+1) (reads K(2t+1) [T, 1]); V rows 0-1 of tile t+2
      if (__builtin_expect(edge, 0)) mask(1, kt);
      phase(Beta{}, Buf<T>{}, I1{}, I0{}, Soft{}, I2{}, I0{}, Buf<Tp2>{}, t + 2, boff_load);
      // alpha(2t+1): QK B(2t+1), PV B(2t) [vfr 0]; reads V(2t+1) [T, 1] into vfr 1; V rows 2-3 of tile t+2
      if (__builtin_expect(edge, 0)) mask(0, kt + 32);
      phase(Alpha{}, Buf<T>{}, I1{}, I0{}, Soft{}, I2{}, I2{}, Buf<Tp2>{}, t + 2, boff_load);
    } else {
      (void)edge;
      idle_loads(I1{}, I2{}, Buf<Tp2>{}, t + 2, boff_load);
      idle_loads(I2{}, I0{}, Buf<Tp2>{}, t + 2, boff_load);
      idle_loads(I2{}, I2{}, Buf<Tp2>{}, t + 2, boff_load);
    }
    wait_vmcnt<8>();  // tile t + 1 landed (tile t + 2's eight loads may be in flight)
    lds_barrier();
    boff_load = entry_base(e_next);
    if constexpr (ACT) {
      // beta(2t+1): PV A(2t+1) [vfr 1], QK A(2t+2) (reads K(2t+2) [T+1, 0]); K rows 0-1 of tile t+3
      if (__builtin_expect(edge, 0)) mask(1, kt + 32);
      phase(Beta{}, Buf<Tp1>{}, I0{}, I1{}, Soft{}, I1{}, I0{}, Buf<Tp3>{}, t + 3, boff_load);
    } else {
      idle_loads(I1{}, I0{}, Buf<Tp3>{}, t + 3, boff_load);
    }
  };
  auto loop = [&](auto act_c) __attribute__((always_inline)) {
    for (int t = 1; t < ntiles; t += 4) {
      tile(Buf<1>{}, t, act_c);
      if (t + 1 < ntiles) tile(Buf<2>{}, t + 1, act_c);
      if (t + 2 < ntiles) tile(Buf<3>{}, t + 2, act_c);
      if (t + 3 < ntiles) tile(Buf<0>{}, t + 3, act_c);
    }
  };
  if (active) loop(std::true_type{});
  else loop(std::false_type{});
  // Drain: PV B of the last sub-tile (odd: vfr 1).  Every load (including
  // those of tiles past the range, which read zeros) has landed and every
  // wave has finished reading the tiles before the K buffers are reused for
  // the output rows.
  if (active) {
#pragma unroll
    for (int k16 = 0; k16 < 2; ++k16) {
#pragma unroll
      for (int db = 0; db < 4; ++db) o[1][db] = mfma(vfr[1][k16][db], pb[1][k16], o[1][db]);
      rs[1] = mfma16(sel, pb[1][k16], rs[1]);
    }
  }
  // Row sums into the lanes of their rows (lane l32 and l32 + 32 hold row l32).
  {
    const int src = l32 < 16 ? l32 : l32 + 16;
    l[0] = __shfl(rs[0][0], src, 64);
    l[1] = __shfl(rs[1][0], src, 64);
  }
  const bool overflow = __builtin_amdgcn_ballot_w64(active && !(fmaxf(l[0], l[1]) <= kFastSumLimit)) != 0;
  wait_vmcnt<0>();
  if (lane == 0) s_overflow[w] = overflow ? 1 : 0;
  lds_barrier();
  if (s_overflow[0] | s_overflow[1] | s_overflow[2] | s_overflow[3]) {
    // Exact rerun (some row's sum passed kFastSumLimit): tile by tile through
    // buffer 0, each sub-tile's maximum moving the running max and rescaling
    // O and l.
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      m[h] = -INFINITY;
      l[h] = 0.f;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[h][db][r] = 0.f;
    }
    for (int t = 0; t < ntiles; ++t) {
      const int kt = kt_of(t);
      const int64_t boff = block_base(kt);
#pragma unroll
      for (int st = 0; st < 4; ++st) load_k(kt, Buf<0>{}, boff, st);
#pragma unroll
      for (int st = 0; st < 4; ++st) load_v(kt, Buf<0>{}, boff, st);
      wait_vmcnt<0>();
      lds_barrier();
      if (active) {
        for (int sub = 0; sub < 2; ++sub) {
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            qk_full(h, blk_off(0, 0) + static_cast<uint32_t>(sub) * 32 * kRowBytes);
            const int ks = kt + 32 * sub;
            if (ks + 32 > wave_kmin) mask(h, ks);
            float c4[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) c4[i] = fmaxf(fmaxf(fmaxf(sc[h][i], sc[h][i + 4]), sc[h][i + 8]), sc[h][i + 12]);
            const float mx = max_halves(fmaxf(fmaxf(c4[0], c4[1]), fmaxf(c4[2], c4[3])));
            const float m_new = fmaxf(m[h], mx);
            const float alpha = (m[h] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((m[h] - m_new) * sl);
            l[h] *= alpha;
#pragma unroll
            for (int db = 0; db < 4; ++db)
#pragma unroll
              for (int r = 0; r < 16; ++r) o[h][db][r] *= alpha;
            m[h] = m_new;
            l[h] += exps(h);
            const uint32_t off = blk_off(0, 0) + static_cast<uint32_t>(sub) * 32 * kRowBytes;
#pragma unroll
            for (int k16 = 0; k16 < 2; ++k16)
#pragma unroll
              for (int db = 0; db < 4; ++db) o[h][db] = mfma(v_frag(off, 0, k16, db), pb[h][k16], o[h][db]);
          }
        }
      }
      lds_barrier();
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) l[h] = sum_halves(l[h]);  // lane partials -> the row's sum
  }

  // ---- epilogue: each wave rounds its 64 rows to bf16, writes them into its
  // own 16 KB of the K tile buffers (chunk c of row r at c ^ (r mod 16)) and
  // stores them back as whole 256-byte rows, four rows per instruction.
  const bool split = a.num_splits > 1;
  uint8_t* const reg = &s_k[0][0] + w * (kWaveRows * kRowBytes);
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const float lt = l[h];
    const float inv = split ? 1.0f / lt : a.v_scale / lt;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        u32x2 v;
        v[0] = pack_bf16_rne(o[h][db][4 * rq] * inv, o[h][db][4 * rq + 1] * inv);
        v[1] = pack_bf16_rne(o[h][db][4 * rq + 2] * inv, o[h][db][4 * rq + 3] * inv);
        *reinterpret_cast<u32x2*>(reg + (kHalfRows * h + l32) * kRowBytes + 16 * ((4 * db + rq) ^ (l32 & 15)) +
                                  8 * h2) = v;
      }
    if (split && h2 == 0 && valid[h]) {
      const int64_t orow_id = static_cast<int64_t>(t0 + tok[h]) * a.num_q_heads + head[h];
      const f32x2 ml = {m[h], lt};
      *reinterpret_cast<f32x2*>(a.ws_ml + (static_cast<int64_t>(z) * total_rows + orow_id) * 2) = ml;
    }
  }
  // (Partials keep 128-wide rows, the merge's layout; the output has head_dim.)
  __bf16* const dst = split ? reinterpret_cast<__bf16*>(a.ws_o) + static_cast<int64_t>(z) * total_rows * D
                            : static_cast<__bf16*>(a.out);
  const int dst_row = split ? D : dh;
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // this wave's LDS writes are done (lgkmcnt(0))
  asm volatile("" ::: "memory");
  if (!active) return;
  // Store k carries rows 4 k + lane / 16 of the wave, 16 bytes (chunk lane %
  // 16) per lane: all sixteen LDS reads go out first, then the sixteen
  // stores, through a buffer descriptor based at the wave's first row, so
  // that the per-row offsets are 32-bit and rows past the chunk (and chunks
  // past the row) are dropped by the range check instead of a branch.
  const int c = lane & 15;
  u32x4 ov[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const int rr = 4 * k + (lane >> 4);  // row of the wave, 0..63
    ov[k] = *lds_at<u32x4>(lds_addr(reg) + rr * kRowBytes + 16 * (c ^ (rr & 15)));
  }
  {
    const int tok_w0 = wr0 / G;
    const __amdgpu_buffer_rsrc_t ors = __builtin_amdgcn_make_buffer_rsrc(
        dst + (static_cast<int64_t>(t0 + tok_w0) * a.num_q_heads + hk * G) * dst_row, 0, static_cast<int>(kPastRange),
        kBufferWord3);
    // The lane's row of store k is head g of its token; roff is the row's
    // byte offset from the descriptor's base.
    const int head_b = 2 * dst_row, tok_b = a.num_q_heads * head_b;
    const int gr = wr0 + (lane >> 4);
    int g = gr % G;
    int roff = (gr / G - tok_w0) * tok_b + g * head_b;
    const int step_g = 4 % G, step_off = (4 / G) * tok_b + step_g * head_b, wrap_off = tok_b - G * head_b;
    const bool in_row = 16 * c < head_b;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const bool ok = wr0 + 4 * k + (lane >> 4) < R && in_row;
      __builtin_amdgcn_raw_buffer_store_b128(ov[k], ors, ok ? roff + 16 * c : static_cast<int>(kPastRange), 0, 0);
      g += step_g;
      roff += step_off;
      if (g >= G) {
        g -= G;
        roff += wrap_off;
      }
    }
  }
}

}  // namespace

hipError_t launch_attn_long(const AttnArgs& a, hipStream_t s) {
  // Groups (sequence, KV head) padded to a multiple of the 8 XCDs; see the
  // work-item mapping at the top of the kernel.
  const int64_t groups = static_cast<int64_t>(a.num_seqs) * a.num_kv_heads;
  const int64_t n = (groups + 7) / 8 * 8 * a.num_splits * a.row_tiles;
  if (n <= 0) return hipSuccess;
  if (n > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(attn_long_kernel, dim3(static_cast<unsigned>(n)), dim3(NT), 0, s, a);
  return hipGetLastError();
}

}  // namespace pkv
