// Paged attention on the gfx950 matrix cores, head_dim 128: bf16 queries over
// fp8 (OCP e4m3fn) K/V pools, and short query chunks (at most kShortRows rows
// per KV head) over bf16 or fp8 pools.  Longer chunks over bf16 pools run in
// attn_long.hip.
//
// Work decomposition
//   A "row" is one (query token, query head) pair of a KV-head group; a
//   sequence with q tokens and G = Hq / Hkv query heads per KV head has q * G
//   rows per KV head, ordered token-major, so the G heads that share a K/V
//   tile are computed from one LDS copy of it (GQA).  A workgroup of 8 waves
//   (two per SIMD) owns 256 consecutive rows of one (sequence, KV head) and,
//   when the key range is split, one range of keys; each wave owns 32 rows,
//   one 32-wide column block of the 32x32x16 bf16 MFMA.
//
// K/V tiles (64 keys) in LDS
//   Both K and V tiles are row-major bf16, one 256-byte row per key, with the
//   sixteen 16-byte chunks of a row permuted by an XOR of the row index so
//   that every read pattern below is free of bank conflicts (k_swz, v_swz).  A tile's four
//   16-token blocks are found through the block table (one entry per block,
//   staged in LDS once per workgroup; entries past ceil(seq_len / 16) are
//   never read).  Pools are copied straight from HBM into LDS with direct
//   global-to-LDS loads (the bf16 short-query path goes through registers);
//   fp8 tiles stay e4m3 in LDS (8 KB each of K and V per 64-key tile, half
//   the bf16 size) and are widened to bf16, exactly, after the LDS read.  Keys
//   outside the workgroup's range read a row of zeros, so a value row that
//   does not exist is 0, never garbage.
//
// Per tile, per wave
//   * S^T = K Q^T on the MFMA: the accumulator holds one query per lane and
//     16 keys per lane, so the row max / row sum need one cross-half swap
//     (v_permlane32_swap) instead of a 32-lane reduction;
//   * the piecewise mask is a per-row key bound L(g) (full segment: kv_end,
//     causal: g + 1), applied only on tiles that cross some row's bound;
//   * online softmax in the exp2 domain with a lazily moved running max;
//   * O^T += V^T P^T on the MFMA, the V^T operand read with the gfx950
//     transposing LDS read (ds_read_b64_tr_b16) from the row-major V tile,
//     P rounded to bf16 as the pages' own reference rounds probabilities to
//     the value dtype before the product.
//   The loop is software-pipelined over four LDS buffers: iteration t runs
//   QK for tile t + 1 next to the exponentials of tile t, then PV of tile t,
//   while tile t + 3 streams into LDS (staged by waves 0..3 for all eight).
//
// Epilogue: O / l rounded to bf16, stored from the accumulator layout.
//
// Split keys: with num_splits > 1 each workgroup writes a partial for its
// key range to the workspace -- its normalised output O / l in bf16 and
// (max, sum) in fp32 -- and a combine kernel merges the splits in a fixed
// order (deterministic, no atomics).
#include <type_traits>

#include "attn_common.hpp"
#include "mfma_util.hpp"

namespace pkv {

// Zeros that direct-to-LDS loads of keys outside the staged range read
// (static device storage starts zeroed and is never written).
__device__ __attribute__((aligned(16))) uint32_t g_zero_row[64 * 4];

namespace {

using namespace mx;

constexpr int KT = kMfmaKeyTile;  // keys per tile
constexpr int NW = 8;             // waves per workgroup (two per SIMD)
constexpr int NT = 64 * NW;
constexpr int kWaveRows = 32;     // query rows per wave: one 32-wide MFMA column block
static_assert(KT == kTileKeys, "tile size");
static_assert(kMfmaRows == NW * kWaveRows, "rows per workgroup");
constexpr float kRescaleLog2 = 8.0f;  // stale-max slack before O and l are rescaled
constexpr int kBufs = 4;             // LDS K/V tile buffers: tiles t, t + 1 read while t + 2, t + 3 arrive
constexpr int kLdsBytes = 2 * kBufs * kTileBytes + kTableSlice * 4;
static_assert(kLdsBytes <= 160 * 1024, "LDS budget of a gfx950 CU");
static_assert(NW * kWaveRows * kRowBytes <= kBufs * kTileBytes, "the epilogue stages every wave's rows in the K buffers");

// K and V tile buffers.  The direct-to-LDS loads that fill them are inline
// assembly the compiler does not see as LDS writes, so it adds no waits for
// them before reads of other buffers; the kernel orders them itself
// (wait_vmcnt, lds_barrier).
__shared__ __attribute__((aligned(16))) uint8_t s_k[kBufs][kTileBytes];
__shared__ __attribute__((aligned(16))) uint8_t s_v[kBufs][kTileBytes];
__shared__ int32_t s_tbl[kTableSlice];  // the workgroup's slice of its block-table row

template <int B>
__device__ __forceinline__ uint8_t* kbuf() { return s_k[B]; }
template <int B>
__device__ __forceinline__ uint8_t* vbuf() { return s_v[B]; }

template <int B>
using Buf = std::integral_constant<int, B>;

static_assert(kTableSlice * 16 >= kMaxSplitKeys, "table slice must cover a split");

// SHORT: at most 64 rows per (sequence, KV head) (short query chunks).  The
// eight waves then split the keys instead of the rows: wave w takes row block
// w % 2 (32 rows) and key group w / 2, i.e. tiles 4 i + w / 2 of iteration i,
// so every wave multiplies while the whole workgroup loads the next four tiles
// into registers; the four key groups' partial results are merged in LDS.
template <bool FP8, bool SHORT>
__global__ __attribute__((amdgpu_flat_work_group_size(NT, NT), amdgpu_waves_per_eu(2, 2))) void
attn_mfma_kernel(AttnArgs a) {
  static_assert(FP8 || SHORT, "bf16 pools with long chunks run in attn_long_kernel");
  int32_t* tbl = s_tbl;
  constexpr int ELSZ = FP8 ? 1 : 2;

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l32 = lane & 31;
  const int h2 = lane >> 5;

  // ---- work item.  Workgroups are dealt to the 8 XCDs round-robin by id
  // (id % 8), each XCD taking its share in id order.  A group is one
  // (sequence, KV head); all of a group's workgroups (key splits x row tiles)
  // go to one XCD, so they share its L2 for the group's K/V, and group g
  // (counted in dispatch order: sequences as seq_order lists them, KV heads
  // fastest) goes to XCD g % 8, which spreads every sequence over the XCDs
  // and keeps their loads balanced.
  int rt, z, hk, b;
  // (packed: the sequence's entries, read across the lanes with the item)
  int p_t0 = 0, p_t1 = 0, p_s = 0, p_g0 = 0, p_g1 = 0, p_qp = 0;
  if (SHORT && a.packed) {
    // Short query chunks planned from the sequences' lengths (one row tile):
    // the key ranges (sequence in seq_order, split z < ceil(seq_len /
    // split_len), KV head fastest) come first, then the empty ranges of every
    // sequence, which only record empty partials.  The host plans this only
    // for at most 64 sequences, so lane i holds sequence i's entries and
    // sequence position i's range count, and one round of loads finds the
    // workgroup's item (a scan and a ballot over the lanes).
    const int H = a.num_kv_heads;
    const int ns = a.num_seqs;
    const int64_t i = blockIdx.x;
    if (i >= static_cast<int64_t>(ns) * H * a.num_splits) return;
    const int li = min(lane, ns - 1);
    const int v_ord = a.seq_order ? a.seq_order[li] : li;
    const int v_len = a.seq_lens[li];
    const int v_t0 = a.qsl[li], v_t1 = a.qsl[li + 1];
    const int v_g0 = a.seg_loc[li], v_g1 = a.seg_loc[li + 1];
    const int v_qp = a.query_pos ? a.query_pos[li] : 0;
    const int len_bp = __shfl(v_len, v_ord, 64);  // length of the sequence at position lane
    const int n = lane < ns ? min(a.num_splits, (max(len_bp, 1) + a.split_len - 1) / a.split_len) : 0;
    // inclusive scans over the positions of the non-empty and the empty ranges
    int inc_full = n * H, inc_empty = lane < ns ? (a.num_splits - n) * H : 0;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int uf = __shfl_up(inc_full, d, 64), ue = __shfl_up(inc_empty, d, 64);
      if (lane >= d) {
        inc_full += uf;
        inc_empty += ue;
      }
    }
    const int total_full = __builtin_amdgcn_readlane(inc_full, 63);
    const bool empty_range = i >= total_full;
    const int64_t k = empty_range ? i - total_full : i;  // rank among its kind
    const int inc = empty_range ? inc_empty : inc_full;
    // position: the first lane whose inclusive count passes k
    const int bp = static_cast<int>(__builtin_popcountll(__builtin_amdgcn_ballot_w64(lane < ns && inc <= k)));
    const int before = bp > 0 ? __builtin_amdgcn_readlane(inc, bp - 1) : 0;
    const int n_bp = __builtin_amdgcn_readlane(n, bp);
    const int loc = static_cast<int>(k - before) + (empty_range ? n_bp * H : 0);
    b = __builtin_amdgcn_readlane(v_ord, bp);
    rt = 0;
    z = loc / H;
    hk = loc % H;
    p_t0 = __builtin_amdgcn_readlane(v_t0, b);
    p_t1 = __builtin_amdgcn_readlane(v_t1, b);
    p_s = __builtin_amdgcn_readlane(v_len, b);
    p_g0 = __builtin_amdgcn_readlane(v_g0, b);
    p_g1 = __builtin_amdgcn_readlane(v_g1, b);
    p_qp = __builtin_amdgcn_readlane(v_qp, b);
  } else {
    const uint32_t xcd = blockIdx.x & 7u, pos = blockIdx.x >> 3;
    const uint32_t per_group = static_cast<uint32_t>(a.num_splits) * static_cast<uint32_t>(a.row_tiles);
    const uint32_t grp = xcd + 8u * (pos / per_group);
    if (grp >= static_cast<uint32_t>(a.num_seqs) * static_cast<uint32_t>(a.num_kv_heads)) return;
    const uint32_t item = pos % per_group;
    // last row tile first: a later row tile never sees fewer keys, so the
    // longest items of a causal chunk go out first and the short ones fill in
    rt = a.row_tiles - 1 - static_cast<int>(item % static_cast<uint32_t>(a.row_tiles));
    z = static_cast<int>(item / static_cast<uint32_t>(a.row_tiles));
    hk = static_cast<int>(grp % static_cast<uint32_t>(a.num_kv_heads));
    const int b_pos = static_cast<int>(grp / static_cast<uint32_t>(a.num_kv_heads));
    b = a.seq_order ? a.seq_order[b_pos] : b_pos;
  }

  const int G = a.group;
  const bool pk = SHORT && a.packed;
  const int t0 = pk ? p_t0 : a.qsl[b];
  const int q_len = (pk ? p_t1 : a.qsl[b + 1]) - t0;
  const int s = pk ? p_s : a.seq_lens[b];
  const int R = q_len * G;
  const int r0 = rt * kMfmaRows;
  if (r0 >= R) return;
  const int seg0 = pk ? p_g0 : a.seg_loc[b], seg1 = pk ? p_g1 : a.seg_loc[b + 1];
  const SegCache segc = load_segments(a.segments, seg0, seg1);
  // key position of the first query row
  const int gbase = a.query_pos ? (pk ? p_qp : a.query_pos[b]) : s - q_len;
  // Row limits are non-decreasing in the row's key position, so the last row
  // bounds the workgroup's key range and the first row of a wave its mask-free prefix.
  const int wg_kmax = row_limit(segc, a.segments, seg0, seg1, gbase + (min(r0 + kMfmaRows, R) - 1) / G);
  const int k_begin = z * a.split_len;
  const int k_end = min(k_begin + a.split_len, wg_kmax);
  if (k_begin >= k_end) {
    // No key of this split is visible to any row of the tile: its partial is
    // empty (max -inf, sum 0), which the merge skips.
    if (a.num_splits > 1 && threadIdx.x < kMfmaRows) {
      const int row = r0 + static_cast<int>(threadIdx.x);
      if (row < R) {
        const int64_t orow = static_cast<int64_t>(t0 + row / G) * a.num_q_heads + hk * G + row % G;
        const int64_t total_rows = a.num_q_tokens * a.num_q_heads;
        const f32x2 ml = {-INFINITY, 0.f};
        *reinterpret_cast<f32x2*>(a.ws_ml + (static_cast<int64_t>(z) * total_rows + orow) * 2) = ml;
      }
    }
    return;
  }

  const int kg = SHORT ? (w >> 1) : 0;  // key group (SHORT)
  const int wr0 = SHORT ? kWaveRows * (w & 1) : r0 + kWaveRows * w;
  int wave_kmin = 0, wave_kmax = 0;
  if (wr0 < R) {
    wave_kmin = row_limit(segc, a.segments, seg0, seg1, gbase + wr0 / G);
    wave_kmax = row_limit(segc, a.segments, seg0, seg1, gbase + (min(wr0 + kWaveRows, R) - 1) / G);
  }

  // ---- this lane's query row
  const int row = wr0 + l32;
  const bool valid = row < R;
  const int tok = valid ? row / G : 0;
  const int head = hk * G + (valid ? row % G : 0);
  const int Lrow = valid ? row_limit(segc, a.segments, seg0, seg1, gbase + tok) : 0;

  // Q^T fragments for S^T = K Q^T: lane holds 8 consecutive head-dim values
  // [16 t + 8 h2, +8) of its query row for each of the 8 k-steps.
  // (fp8 pools: step t takes head-dim piece 4 (t / 2) + 2 h2 + t % 2 of 8
  // values instead, so that one 16-byte LDS read of K feeds two steps.)
  constexpr bool kF8Lds = FP8;  // fp8 K/V tiles are kept as fp8 in LDS
  // head_dim 64 runs through the same 128-wide kernel with head-dim
  // [64, 128) of Q, K and V zero: it adds nothing to a score, and the
  // output's upper half is never stored.
  const int dh = a.head_dim;  // 64 or 128
  bf16x8 qf[8];
  {
    const __bf16* qr = static_cast<const __bf16*>(a.q) +
                       (static_cast<int64_t>(t0 + tok) * a.num_q_heads + head) * dh;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int piece = kF8Lds ? 4 * (t >> 1) + 2 * h2 + (t & 1) : 2 * t + h2;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (valid && 8 * piece < dh) v = *reinterpret_cast<const u32x4*>(qr + 8 * piece);
      qf[t] = __builtin_bit_cast(bf16x8, v);
    }
  }
  // ---- block-table slice for this workgroup's keys (no table: the K/V
  // buffers are one contiguous run, logical block i is block i)
  const int nblk = (s + 15) >> 4;
  const int blk_lo = k_begin >> 4;
  const int blk_hi = min((k_end + 15) >> 4, nblk);
  if (a.block_table) {
    const int32_t* table = a.block_table + static_cast<int64_t>(b) * a.table_width;
    for (int i = threadIdx.x; i < blk_hi - blk_lo; i += NT) tbl[i] = table[blk_lo + i];
  } else {
    for (int i = threadIdx.x; i < blk_hi - blk_lo; i += NT) tbl[i] = blk_lo + i;
  }
  // Q and the table slice (loaded together, so their latencies overlap) have
  // landed before any K/V load is issued.  The compiler cannot see the
  // direct-to-LDS loads (inline assembly); without this wait it may guard a
  // later use of Q with a full vmcnt(0), which would drain the K/V prefetch.
  wait_vmcnt<0>();
  lds_barrier();
  // Keys at or past kv_lim are staged as zeros: past seq_len they do not exist,
  // and past the slice every row of the workgroup masks them anyway.
  const int kv_lim = min(s, blk_hi * 16);

  // ---- staging geometry (bf16): wave w stages tile rows [8 w, 8 w + 8) of
  // both the K and the V tile, four rows (one 1 KB direct load) per step; lane
  // i takes row 8 w + 4 step + i / 16 and LDS chunk position i % 16.
  const int64_t row_bytes = static_cast<int64_t>(a.num_kv_heads) * dh * ELSZ;
  const int64_t block_bytes = 16 * row_bytes;
  const uint8_t* kpool = static_cast<const uint8_t*>(a.kpool) + static_cast<int64_t>(hk) * dh * ELSZ;
  const uint8_t* vpool = static_cast<const uint8_t*>(a.vpool) + static_cast<int64_t>(hk) * dh * ELSZ;
  // Whether a 16-byte source chunk lies inside head_dim (chunks past it read zeros).
  const bool full_d = dh == D;
  auto in_d = [&](int chunk) { return 16 * chunk < dh * ELSZ; };
  const int st_pos = lane & 15;
  int st_row[2], k_src_off[2], v_src_off[2];
#pragma unroll
  for (int st = 0; st < 2; ++st) {
    st_row[st] = 8 * w + 4 * st + (lane >> 4);
    const int rb = st_row[st] & 15;  // row inside its 16-token block
    k_src_off[st] = static_cast<int>(rb * row_bytes) + (st_pos ^ k_swz(st_row[st])) * 8 * ELSZ;
    v_src_off[st] = static_cast<int>(rb * row_bytes) + (st_pos ^ v_swz(st_row[st])) * 8 * ELSZ;
  }

  // Block-table entry of the 16 keys whose rows wave ws stages for the tile
  // at key kt (rows 8 ws .. 8 ws + 7 lie in block ws / 2 of the tile).
  auto stage_entry = [&](int kt, int ws) {
    const int blk = (kt >> 4) + (ws >> 1);
    return (blk < blk_hi) ? tbl[blk - blk_lo] : 0;
  };
  // ---- MFMA operand addresses (bytes, without the buffer offset)
  // (buffer 0, or the key group's own buffer for SHORT)
  uint32_t k_rd[8];  // LDS address of K row 32 kb + l32, chunk 2 t + h2
#pragma unroll
  for (int t = 0; t < 8; ++t) k_rd[t] = lds_addr(s_k[kg] + l32 * kRowBytes + 16 * ((2 * t + h2) ^ k_swz(l32)));
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
      v_rd[db] = lds_addr(s_v[kg] + (4 * (g >> 1) + j) * kRowBytes + 16 * (c ^ v_swz(j)) + 8 * (q & 1));
    }
  }

  const float sl = a.scale_log2;
  float lt_merged = 0.f;  // SHORT: row sum after the key-group merge
  float m = -INFINITY;
  float l = 0.f;
  f32x16 o[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[db][r] = 0.f;

  auto qk = [&](auto bufc, f32x16 (&sacc)[2]) __attribute__((always_inline)) {
    constexpr int B = decltype(bufc)::value;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[kb][r] = 0.f;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x8 ka = *lds_at<bf16x8>(k_rd[t] + B * kTileBytes + kb * 32 * kRowBytes);
        sacc[kb] = mfma(ka, qf[t], sacc[kb]);
      }
    }
  };

  // Mask, running max (lazily moved) for tile kt.
  auto mask_and_rescale = [&](int kt, f32x16 (&sacc)[2]) __attribute__((always_inline)) {
    if (kt + KT > wave_kmin) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int j = kt + 32 * kb + 8 * (r >> 2) + 4 * h2 + (r & 3);
          if (j >= Lrow) sacc[kb][r] = -INFINITY;
        }
    }
    // Four independent chains of three-input maxima (v_max3_f32): 18
    // instructions for the 32 values, with four chains in flight.
    float c4[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float c = fmaxf(fmaxf(sacc[0][i], sacc[0][i + 4]), sacc[0][i + 8]);
      c = fmaxf(fmaxf(c, sacc[0][i + 12]), sacc[1][i]);
      c = fmaxf(fmaxf(c, sacc[1][i + 4]), sacc[1][i + 8]);
      c4[i] = fmaxf(c, sacc[1][i + 12]);
    }
    const float mx = max_halves(fmaxf(fmaxf(fmaxf(c4[0], c4[1]), c4[2]), c4[3]));
    // The running max only moves (and O, l are rescaled) when some row's tile
    // max exceeds it by more than 2^kRescaleLog2 in the exp2 domain.  Softmax
    // is exact for any common offset, so a stale max only lets probabilities
    // reach 2^kRescaleLog2 (well inside fp32/bf16 range) and leaves the result
    // unchanged up to rounding.
    const bool grow = (mx - m) * sl > kRescaleLog2;  // false for NaN (-inf - -inf)
    if (__builtin_amdgcn_ballot_w64(grow)) {
      const float m_new = fmaxf(m, mx);
      const float alpha = (m == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((m - m_new) * sl);
      l *= alpha;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
      m = m_new;
    }
  };

  // Probabilities of a tile, rounded to bf16, and their row sum.  The
  // exponentials overwrite S in place (all 32 first, then the packs and sums),
  // so the transcendental latency is covered without extra registers.
  auto probs = [&](f32x16 (&sacc)[2], bf16x8 (&pb)[2][2]) __attribute__((always_inline)) {
    const float mc = (m == -INFINITY) ? 0.f : m * sl;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[kb][r] = __builtin_amdgcn_exp2f(fmaf(sacc[kb][r], sl, -mc));
    float ls[4] = {0.f, 0.f, 0.f, 0.f};  // four independent partial sums
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int k16 = 0; k16 < 2; ++k16) {
        u32x4 pk;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p0 = sacc[kb][8 * k16 + 2 * e], p1 = sacc[kb][8 * k16 + 2 * e + 1];
          pk[e] = pack_bf16_rne(p0, p1);
          // The row sum adds the fp32 probabilities with plain adds.  (A bf16
          // dot instruction could add the rounded pair in one step, but it
          // issues to the matrix pipe and stalls the SIMD partner's MFMAs.)
          ls[e] = (ls[e] + p0) + p1;
        }
        pb[kb][k16] = __builtin_bit_cast(bf16x8, pk);
      }
    l += (ls[0] + ls[1]) + (ls[2] + ls[3]);
  };

  auto pv = [&](auto bufc, const bf16x8 (&pb)[2][2]) __attribute__((always_inline)) {
    constexpr int B = decltype(bufc)::value;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int k16 = 0; k16 < 2; ++k16)
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          const uint32_t base = v_rd[db] + B * kTileBytes + (32 * kb + 16 * k16) * kRowBytes;
          const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(lds_v4i16(base));
          const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(lds_v4i16(base + 8 * kRowBytes));
          const bf16x8 va = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
          o[db] = mfma(va, pb[kb][k16], o[db]);
        }
  };

  // ---- fp8 pools: tiles stay fp8 in LDS (8 KB of K and 8 KB of V per tile,
  // eight tiles in the 128 KB of tile buffers), filled by direct loads, and
  // are widened to bf16 as the MFMA operands are read.
  //   K: 128-byte rows, 16-byte chunk c of row r at position c ^ ((r / 2) % 8);
  //      lane (l32, h2) reads chunk 2 m + h2 of its row, the head-dim pieces
  //      of steps 2 m and 2 m + 1 (the order Q was loaded in).
  //   V: 128-byte rows, chunk c of row r at c ^ 2 (((r / 2) % 2) | ((r / 4) % 2 * 2));
  //      read with ds_read_b64_tr_b8: in each 16-lane group g, lane 8 hb + c
  //      receives byte c of the 8-byte pieces that lanes 2 j + hb (j = 0..7)
  //      name.  Lane 16 g + 2 j + hb names the row holding key
  //      8 (j / 4) + 4 (g / 2) + j % 4 of the 16-key chunk (the key order of
  //      P's MFMA operand) and head-dim piece 4 db + 2 (g % 2) + hb.
  // Both layouts are free of bank conflicts for these reads.
  uint8_t* const f8k_base = &s_k[0][0];
  uint8_t* const f8v_base = &s_v[0][0];
  constexpr int kF8Tile = 64 * D;  // bytes of one fp8 K (or V) tile
  auto f8_swz_k = [](int r) { return (r >> 1) & 7; };
  auto f8_swz_v = [](int r) { return 2 * (((r >> 1) & 1) | ((r >> 2) & 2)); };
  // direct loads: wave w fills rows 8 w .. 8 w + 7 of each tile, lane i
  // position i % 8 of row 8 w + i / 8
  const int dl_row = 8 * w + (lane >> 3), dl_pos = lane & 7;
  const uint32_t dl_k = static_cast<uint32_t>((dl_row & 15) * row_bytes + 16 * (dl_pos ^ f8_swz_k(dl_row)));
  const uint32_t dl_v = static_cast<uint32_t>((dl_row & 15) * row_bytes + 16 * (dl_pos ^ f8_swz_v(dl_row)));
  const uint8_t* f8_zero = reinterpret_cast<const uint8_t*>(g_zero_row) + 16 * dl_pos;
  // K operand addresses (buffer offset added per tile): chunk 2 m + h2 of row l32 (+ 32 kb)
  uint32_t k8_rd[4];
#pragma unroll
  for (int mm = 0; mm < 4; ++mm) k8_rd[mm] = lds_addr(f8k_base + l32 * D + 16 * ((2 * mm + h2) ^ f8_swz_k(l32)));
  uint32_t v8_rd[4];
  {
    const int g = lane >> 4, mpos = lane & 15, j = mpos >> 1, hb = mpos & 1;
    const int row = 8 * (j >> 2) + 4 * (g >> 1) + (j & 3);
    const int sq = f8_swz_v(row) >> 1;  // swizzle in units of 4 pieces
#pragma unroll
    for (int db = 0; db < 4; ++db)
      v8_rd[db] = lds_addr(f8v_base + row * D + 32 * (db ^ sq) + 8 * (2 * (g & 1) + hb));
  }
  // Direct loads of tile t (block-table entry e) into fp8 buffer buf: wave w
  // fills rows 8 w .. 8 w + 7; rows past kv_lim read zeros.
  // (ws = w, or w + 4 when waves 0..3 load for all eight: those rows sit 32
  // rows, two blocks, further on, at the same offsets inside their block)
  auto issue1 = [&](int buf, int t, int e, int ws) {
    const int kt = k_begin + t * KT;
    const int64_t boff = static_cast<int64_t>(__builtin_amdgcn_readfirstlane(e)) * block_bytes;
    uint8_t* kdst = f8k_base + buf * kF8Tile + 8 * ws * D;
    uint8_t* vdst = f8v_base + buf * kF8Tile + 8 * ws * D;
    if (full_d && kt + 8 * ws + 8 <= kv_lim) {  // all eight rows exist (uniform)
      dma16(kpool + boff, dl_k, kdst);
      dma16(vpool + boff, dl_v, vdst);
    } else {
      const bool ok = kt + dl_row + 8 * (ws - w) < kv_lim;
      const bool kok = ok && in_d(dl_pos ^ f8_swz_k(dl_row)), vok = ok && in_d(dl_pos ^ f8_swz_v(dl_row));
      dma16(kok ? kpool + boff + dl_k : f8_zero, kdst);
      dma16(vok ? vpool + boff + dl_v : f8_zero, vdst);
    }
  };
  auto qk8 = [&](int buf, f32x16 (&sacc)[2]) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[kb][r] = 0.f;
#pragma unroll
    for (int mm = 0; mm < 4; ++mm)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const u32x4 c = *lds_at<u32x4>(k8_rd[mm] + buf * kF8Tile + kb * 32 * D);
        const bf16x8 k0 = __builtin_bit_cast(bf16x8, e4m3x8_to_bf16x8(u32x2{c[0], c[1]}));
        const bf16x8 k1 = __builtin_bit_cast(bf16x8, e4m3x8_to_bf16x8(u32x2{c[2], c[3]}));
        sacc[kb] = mfma(k0, qf[2 * mm], sacc[kb]);
        sacc[kb] = mfma(k1, qf[2 * mm + 1], sacc[kb]);
      }
  };
  auto pv8 = [&](int buf, const bf16x8 (&pb)[2][2]) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int k16 = 0; k16 < 2; ++k16)
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          const uint32_t addr = v8_rd[db] + buf * kF8Tile + (32 * kb + 16 * k16) * D;
          const v2i32 c = __builtin_amdgcn_ds_read_tr8_b64_v2i32(lds_v2i32(addr));
          const bf16x8 va = __builtin_bit_cast(
              bf16x8, e4m3x8_to_bf16x8(u32x2{static_cast<uint32_t>(c[0]), static_cast<uint32_t>(c[1])}));
          o[db] = mfma(va, pb[kb][k16], o[db]);
        }
  };
  const int ntiles = (k_end - k_begin + KT - 1) / KT;
  auto kt_of = [&](int t) { return k_begin + t * KT; };

  if constexpr (kF8Lds && SHORT) {
    // ---- fp8 short path: 32-key tiles, four per step (one per key group),
    // in a ring of four steps of buffers.  Step i uses set i % 4; during step
    // i (after the barrier closing step i - 1) the loads of step i + 3 go into
    // the set of step i - 1.  Half a tile is one 16-key block of K and of V,
    // two direct loads each; waves w and w + 4 (w < 4) load the same half of
    // the tiles of key groups w / 2 and w / 2 + 2, and wave w issues both.
    constexpr int KT32 = 32;
    constexpr int kTile32 = KT32 * D;  // bytes of one fp8 K (or V) tile
    const int ntiles32 = (k_end - k_begin + KT32 - 1) / KT32;
    const int nsteps = (ntiles32 + 3) / 4;
    const int ld_part = w & 1;  // which 16-key block of the tile this wave loads
    // lane: row (ld_part * 16 + 8 * sub + lane / 8) of the tile, global chunk
    // (lane % 8) ^ swizzle of that row at LDS slot lane % 8
    const int ld_r8 = lane >> 3;
    uint32_t ld_k[2], ld_v[2];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      const int r = 16 * ld_part + 8 * sub + ld_r8;
      ld_k[sub] = static_cast<uint32_t>((r & 15) * row_bytes + 16 * (dl_pos ^ f8_swz_k(r)));
      ld_v[sub] = static_cast<uint32_t>((r & 15) * row_bytes + 16 * (dl_pos ^ f8_swz_v(r)));
    }
    auto tile_exists = [&](int step) { return 4 * step + kg < ntiles32; };  // kg == w / 2
    // Loads of step `step` for key group kgs (its tile, this wave's half).
    auto issue_step = [&](int step, int kgs) {
      if (!(4 * step + kgs < ntiles32)) return;
      const int set = step & 3;
      const int kt = k_begin + KT32 * (4 * step + kgs);
      const int blk = (kt >> 4) + ld_part;
      const int e = (blk < blk_hi) ? tbl[blk - blk_lo] : 0;
      const int64_t boff = static_cast<int64_t>(__builtin_amdgcn_readfirstlane(e)) * block_bytes;
      const int row0 = kt + 16 * ld_part;  // key of the first row this wave loads
      uint8_t* kdst = f8k_base + (4 * set + kgs) * kTile32 + 16 * ld_part * D;
      uint8_t* vdst = f8v_base + (4 * set + kgs) * kTile32 + 16 * ld_part * D;
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {
        if (full_d && row0 + 8 * sub + 8 <= kv_lim) {  // all eight rows exist (uniform)
          dma16(kpool + boff, ld_k[sub], kdst + 8 * sub * D);
          dma16(vpool + boff, ld_v[sub], vdst + 8 * sub * D);
        } else {  // rows past kv_lim, and chunks past head_dim, read zeros
          const int r = 16 * ld_part + 8 * sub + ld_r8;
          const bool ok = row0 + 8 * sub + ld_r8 < kv_lim;
          const bool kok = ok && in_d(dl_pos ^ f8_swz_k(r)), vok = ok && in_d(dl_pos ^ f8_swz_v(r));
          dma16(kok ? kpool + boff + ld_k[sub] : f8_zero, kdst + 8 * sub * D);
          dma16(vok ? vpool + boff + ld_v[sub] : f8_zero, vdst + 8 * sub * D);
        }
      }
    };
    // Waves 0..3 load for all eight: their own key group's tile and that of
    // wave w + 4 (key group kg + 2, the same half), at the end of their step,
    // where they would otherwise wait for their SIMD partners (a direct load
    // stalls the wave that issues it while the CU's earlier loads queue).
    const bool stager = w < 4;
    auto nloads = [&](int step) { return 4 * (4 * step + kg < ntiles32) + 4 * (4 * step + kg + 2 < ntiles32); };
    // Waits until a loading wave's loads of step `step` have landed, given
    // which later steps it has issued.
    auto wait_step = [&](int step, int issued_upto) {
      int later = 0;
      if (issued_upto >= step + 1) later += nloads(step + 1);
      if (issued_upto >= step + 2) later += nloads(step + 2);
      switch (later) {
        case 16: wait_vmcnt<16>(); break;
        case 12: wait_vmcnt<12>(); break;
        case 8: wait_vmcnt<8>(); break;
        case 4: wait_vmcnt<4>(); break;
        default: wait_vmcnt<0>(); break;
      }
    };
    if (stager) {
      for (int st0 = 0; st0 < 3; ++st0) {
        issue_step(st0, kg);
        issue_step(st0, kg + 2);
      }
      wait_step(0, 2);
    }
    lds_barrier();
    for (int step = 0; step < nsteps; ++step) {
      const int set = step & 3;
      const int kt = k_begin + KT32 * (4 * step + kg);
      if (tile_exists(step) && kt < wave_kmax) {
        const int buf = 4 * set + kg;
        f32x16 sc;
#pragma unroll
        for (int r = 0; r < 16; ++r) sc[r] = 0.f;
#pragma unroll
        for (int mm = 0; mm < 4; ++mm) {
          const u32x4 c = *lds_at<u32x4>(k8_rd[mm] + buf * kTile32);
          const bf16x8 k0 = __builtin_bit_cast(bf16x8, e4m3x8_to_bf16x8(u32x2{c[0], c[1]}));
          const bf16x8 k1 = __builtin_bit_cast(bf16x8, e4m3x8_to_bf16x8(u32x2{c[2], c[3]}));
          sc = mfma(k0, qf[2 * mm], sc);
          sc = mfma(k1, qf[2 * mm + 1], sc);
        }
        if (kt + KT32 > wave_kmin) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int j = kt + 8 * (r >> 2) + 4 * h2 + (r & 3);
            if (j >= Lrow) sc[r] = -INFINITY;
          }
        }
        float c4[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) c4[i] = fmaxf(fmaxf(fmaxf(sc[i], sc[i + 4]), sc[i + 8]), sc[i + 12]);
        const float mx = max_halves(fmaxf(fmaxf(fmaxf(c4[0], c4[1]), c4[2]), c4[3]));
        const bool grow = (mx - m) * sl > kRescaleLog2;  // false for NaN (-inf - -inf)
        if (__builtin_amdgcn_ballot_w64(grow)) {
          const float m_new = fmaxf(m, mx);
          const float alpha = (m == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((m - m_new) * sl);
          l *= alpha;
#pragma unroll
          for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
          m = m_new;
        }
        const float mc = (m == -INFINITY) ? 0.f : m * sl;
#pragma unroll
        for (int r = 0; r < 16; ++r) sc[r] = __builtin_amdgcn_exp2f(fmaf(sc[r], sl, -mc));
        float ls[4] = {0.f, 0.f, 0.f, 0.f};
        bf16x8 pb[2];
#pragma unroll
        for (int k16 = 0; k16 < 2; ++k16) {
          u32x4 pk;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            pk[e] = pack_bf16_rne(sc[8 * k16 + 2 * e], sc[8 * k16 + 2 * e + 1]);
            ls[e] = (ls[e] + sc[8 * k16 + 2 * e]) + sc[8 * k16 + 2 * e + 1];
          }
          pb[k16] = __builtin_bit_cast(bf16x8, pk);
        }
        l += (ls[0] + ls[1]) + (ls[2] + ls[3]);
#pragma unroll
        for (int k16 = 0; k16 < 2; ++k16)
#pragma unroll
          for (int db = 0; db < 4; ++db) {
            const uint32_t addr = v8_rd[db] + buf * kTile32 + 16 * k16 * D;
            const v2i32 c = __builtin_amdgcn_ds_read_tr8_b64_v2i32(lds_v2i32(addr));
            const bf16x8 va = __builtin_bit_cast(
                bf16x8, e4m3x8_to_bf16x8(u32x2{static_cast<uint32_t>(c[0]), static_cast<uint32_t>(c[1])}));
            o[db] = mfma(va, pb[k16], o[db]);
          }
      }
      if (stager) {
        // step + 3 goes into the set of step - 1, which every wave has left
        issue_step(step + 3, kg);
        issue_step(step + 3, kg + 2);
        wait_step(step + 1, step + 3);  // step + 1 has landed
      }
      lds_barrier();
    }
  } else if constexpr (SHORT) {
    // ---- bf16 short path: each wave multiplies tile 4 i + kg from buffer kg
    // while the workgroup loads tiles 4 i + 4 .. 4 i + 7 into registers (lane
    // i of wave w: chunk i % 16 of rows 8 w + 4 st + i / 16, at the positions
    // k_src_off / v_src_off name); after a barrier they are written into buffers 0..3.
    u32x4 rk[4][2], rv[4][2];
    auto load4 = [&](int t_first) {
      // All four block-table entries first: one LDS round trip, not four.
      int e[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) e[j] = (t_first + j < ntiles) ? stage_entry(kt_of(t_first + j), w) : 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int t = t_first + j;
        if (t >= ntiles) break;
        const int kt = kt_of(t);
        const int64_t boff = static_cast<int64_t>(__builtin_amdgcn_readfirstlane(e[j])) * block_bytes;
        const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          const bool ok = kt + st_row[st] < kv_lim;
          const bool kok = ok && in_d(st_pos ^ k_swz(st_row[st])), vok = ok && in_d(st_pos ^ v_swz(st_row[st]));
          rk[j][st] = kok ? *reinterpret_cast<const u32x4*>(kpool + boff + k_src_off[st]) : zero;
          rv[j][st] = vok ? *reinterpret_cast<const u32x4*>(vpool + boff + v_src_off[st]) : zero;
        }
      }
    };
    auto store4 = [&](int t_first) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (t_first + j >= ntiles) break;
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          const int dst = st_row[st] * kRowBytes + 16 * st_pos;
          *reinterpret_cast<u32x4*>(s_k[j] + dst) = rk[j][st];
          *reinterpret_cast<u32x4*>(s_v[j] + dst) = rv[j][st];
        }
      }
    };
    load4(0);
    store4(0);
    lds_barrier();
    f32x16 sacc[2];
    for (int t4 = 0; t4 < ntiles; t4 += 4) {
      load4(t4 + 4);
      const int t = t4 + kg;
      if (t < ntiles && kt_of(t) < wave_kmax) {
        qk(Buf<0>{}, sacc);
        mask_and_rescale(kt_of(t), sacc);
        bf16x8 pb[2][2];
        probs(sacc, pb);
        pv(Buf<0>{}, pb);
      }
      lds_barrier();
      store4(t4 + 4);
      lds_barrier();
    }
  } else if constexpr (FP8) {
    // ---- fp8 long chunks: tile t in fp8 buffer t % 8, loaded seven tiles
    // ahead.  Iteration t: mask / max of S(t); S(t+1) = K(t+1) Q^T next to the
    // exponentials of S(t); O += V(t) P(t); then waves 0..3 load tile t + 7
    // (all eight waves' rows, as in the bf16 loop) into buffer (t - 1) % 8,
    // whose last reader (V(t - 1)) finished before the barrier closing
    // iteration t - 1, and wait for tile t + 2, which iteration t + 1 reads
    // after the barrier.
    const bool stager = w < 4;
    auto wait_tiles = [&](int outstanding_tiles) {  // four loads per tile and loading wave
      switch (outstanding_tiles) {
        case 5: wait_vmcnt<20>(); break;
        case 4: wait_vmcnt<16>(); break;
        case 3: wait_vmcnt<12>(); break;
        case 2: wait_vmcnt<8>(); break;
        case 1: wait_vmcnt<4>(); break;
        default: wait_vmcnt<0>(); break;
      }
    };
    auto load_tile = [&](int buf, int t) {
      issue1(buf, t, stage_entry(kt_of(t), w), w);
      issue1(buf, t, stage_entry(kt_of(t), w + 4), w + 4);
    };
    if (stager) {
#pragma unroll
      for (int j = 0; j < 7; ++j)
        if (j < ntiles) load_tile(j, j);
      wait_tiles(max(0, min(ntiles, 7) - 2));  // tiles 0 and 1
    }
    lds_barrier();
    f32x16 sA[2], sB[2];
    qk8(0, sA);
    auto iteration = [&](auto bufc, int t, f32x16 (&s_cur)[2], f32x16 (&s_next)[2]) {
      constexpr int B = decltype(bufc)::value;
      if (kt_of(t) < wave_kmax) {
        mask_and_rescale(kt_of(t), s_cur);
        bf16x8 pb[2][2];
        qk8((B + 1) % 8, s_next);
        probs(s_cur, pb);
        pv8(B, pb);
      }
      if (stager) {
        if (t + 7 < ntiles) load_tile((B + 7) % 8, t + 7);
        wait_tiles(max(0, min(t + 7, ntiles - 1) - (t + 2)));
      }
      lds_barrier();
    };
    for (int t = 0; t < ntiles; t += 8) {
      iteration(Buf<0>{}, t, sA, sB);
      if (t + 1 < ntiles) iteration(Buf<1>{}, t + 1, sB, sA);
      if (t + 2 < ntiles) iteration(Buf<2>{}, t + 2, sA, sB);
      if (t + 3 < ntiles) iteration(Buf<3>{}, t + 3, sB, sA);
      if (t + 4 < ntiles) iteration(Buf<4>{}, t + 4, sA, sB);
      if (t + 5 < ntiles) iteration(Buf<5>{}, t + 5, sB, sA);
      if (t + 6 < ntiles) iteration(Buf<6>{}, t + 6, sA, sB);
      if (t + 7 < ntiles) iteration(Buf<7>{}, t + 7, sB, sA);
    }
  }

  if constexpr (SHORT) {
    // ---- merge the four key groups of each row block: common max, then
    // ((kg 0 + kg 2) + (kg 1 + kg 3)) in that order, through LDS.
    float lt_own = sum_halves(l);
    float* ml = reinterpret_cast<float*>(s_tbl);  // [wave][32 rows] running max
    if (h2 == 0) ml[w * 32 + l32] = m;
    lds_barrier();
    float M = -INFINITY;
#pragma unroll
    for (int g = 0; g < 4; ++g) M = fmaxf(M, ml[(2 * g + (w & 1)) * 32 + l32]);
    const float f = (m == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((m - M) * sl);
    lt_own *= f;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[db][r] *= f;
    // Region of a wave's O: 64 lanes x 64 floats, lane-interleaved f32x4.
    auto o_slot = [&](uint8_t* region, int db, int rq) {
      return reinterpret_cast<f32x4*>(region + ((db * 4 + rq) * 64 + lane) * 16);
    };
    float* lt_x = reinterpret_cast<float*>(s_tbl) + 512;  // [region][64 lanes]
    auto put = [&](uint8_t* region, int slot) {
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq)
          *o_slot(region, db, rq) = f32x4{o[db][4 * rq], o[db][4 * rq + 1], o[db][4 * rq + 2], o[db][4 * rq + 3]};
      lt_x[slot * 64 + lane] = lt_own;
    };
    auto add = [&](uint8_t* region, int slot) {
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          const f32x4 v = *o_slot(region, db, rq);
#pragma unroll
          for (int e = 0; e < 4; ++e) o[db][4 * rq + e] += v[e];
        }
      lt_own += lt_x[slot * 64 + lane];
    };
    // level 1: kg 2, 3 hand over to kg 0, 1 (regions in the K buffers)
    if (kg >= 2) put(s_k[w - 4], w - 4);
    lds_barrier();
    if (kg < 2) add(s_k[w], w);
    lds_barrier();
    // level 2: kg 1 hands over to kg 0 (regions in the V buffers)
    if (kg == 1) put(s_v[w - 2], 4 + (w - 2));
    lds_barrier();
    if (kg == 0) add(s_v[w], 4 + w);
    if (kg != 0) return;
    m = M;
    lt_merged = lt_own;
  }

  // ---- epilogue
  const float lt = SHORT ? lt_merged : sum_halves(l);
  const int64_t total_rows = a.num_q_tokens * a.num_q_heads;
  // Direct stores from the accumulator layout.  (Staging the rows through
  // LDS to store whole rows, as the bf16 long-chunk kernel does, changed the
  // fp8 long kernel's loop register allocation and cost 8% on long fp8
  // chunks; the short-query kernels store only two waves' rows.)
  if (!valid) return;
  const int64_t orow_id = static_cast<int64_t>(t0 + tok) * a.num_q_heads + head;
  if (a.num_splits > 1) {
    // The split's partial: its normalised output O / l (a weighted average of
    // V rows) rounded to bf16, and (max, sum) in fp32.  A row none of whose
    // keys lies in this split has max -inf and its O / l is never read.
    __bf16* wo = reinterpret_cast<__bf16*>(a.ws_o) + (static_cast<int64_t>(z) * total_rows + orow_id) * D;
    const float inv = 1.0f / lt;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        u32x2 v;
        v[0] = pack_bf16_rne(o[db][4 * rq] * inv, o[db][4 * rq + 1] * inv);
        v[1] = pack_bf16_rne(o[db][4 * rq + 2] * inv, o[db][4 * rq + 3] * inv);
        *reinterpret_cast<u32x2*>(wo + 32 * db + 8 * rq + 4 * h2) = v;
      }
    if (h2 == 0) {
      f32x2 ml = {m, lt};
      *reinterpret_cast<f32x2*>(a.ws_ml + (static_cast<int64_t>(z) * total_rows + orow_id) * 2) = ml;
    }
  } else {
    const float inv = a.v_scale / lt;
    __bf16* orow = static_cast<__bf16*>(a.out) + orow_id * dh;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        u32x2 v;
        v[0] = pack_bf16_rne(o[db][4 * rq] * inv, o[db][4 * rq + 1] * inv);
        v[1] = pack_bf16_rne(o[db][4 * rq + 2] * inv, o[db][4 * rq + 3] * inv);
        if (32 * db + 8 * rq + 4 * h2 < dh) *reinterpret_cast<u32x2*>(orow + 32 * db + 8 * rq + 4 * h2) = v;
      }
  }
}

// Merges the key splits of a row, in split order: 16 lanes per row, eight
// head-dim values (16 bytes of each bf16 partial) per lane, sixteen rows per
// workgroup.  Every split has a partial for every row (an empty one has max
// -inf and sum 0 and is skipped), so no sequence or mask metadata has to be
// looked up first.
constexpr int kCombineRows = 16;
template <int NZ>
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnArgs a) {
  const int sub = threadIdx.x & 15;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * kCombineRows + (threadIdx.x >> 4);
  const int64_t total_rows = a.num_q_tokens * a.num_q_heads;
  // Rows past the last sequence's queries belong to no sequence: no split
  // wrote a partial for them, and their output rows are left untouched.
  if (row >= min(total_rows, static_cast<int64_t>(a.qsl[a.num_seqs]) * a.num_q_heads)) return;
  const int nz = a.num_splits;
  // Every split's (max, sum) and numerator slice are loaded at once (one
  // round trip); an empty split (max -inf) wrote no numerator, so whatever
  // its slot holds is dropped by a select, never multiplied.
  f32x2 ml[NZ];
  u32x4 pv[NZ];
  const __bf16* wo = reinterpret_cast<const __bf16*>(a.ws_o);
#pragma unroll
  for (int zz = 0; zz < NZ; ++zz) {
    if (zz < nz) {
      ml[zz] = *reinterpret_cast<const f32x2*>(a.ws_ml + (zz * total_rows + row) * 2);
      pv[zz] = *reinterpret_cast<const u32x4*>(wo + (zz * total_rows + row) * D + 8 * sub);
    }
  }
  float M = -INFINITY;
#pragma unroll
  for (int zz = 0; zz < NZ; ++zz)
    if (zz < nz) M = fmaxf(M, ml[zz][0]);
  float den = 0.f;
  float num[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int zz = 0; zz < NZ; ++zz) {
    if (zz < nz) {
      const bool live = ml[zz][0] != -INFINITY;
      // weight of split zz: its sum of probabilities at the common max
      const float wz = live ? __builtin_amdgcn_exp2f((ml[zz][0] - M) * a.scale_log2) * ml[zz][1] : 0.f;
      den = live ? den + wz : den;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float lo = __uint_as_float(pv[zz][e] << 16), hi = __uint_as_float(pv[zz][e] & 0xFFFF0000u);
        num[2 * e] = live ? fmaf(wz, lo, num[2 * e]) : num[2 * e];
        num[2 * e + 1] = live ? fmaf(wz, hi, num[2 * e + 1]) : num[2 * e + 1];
      }
    }
  }
  const float inv = a.v_scale / den;
  u32x4 packed;
#pragma unroll
  for (int e = 0; e < 4; ++e) packed[e] = pack_bf16_rne(num[2 * e] * inv, num[2 * e + 1] * inv);
  if (8 * sub < a.head_dim) *reinterpret_cast<u32x4*>(static_cast<__bf16*>(a.out) + row * a.head_dim + 8 * sub) = packed;
}

}  // namespace

hipError_t launch_attn_mfma(const AttnArgs& a, bool kv_fp8, bool short_rows, hipStream_t s) {
  // Groups (sequence, KV head) padded to a multiple of the 8 XCDs; see the
  // work-item mapping at the top of the kernel.
  const int64_t groups = static_cast<int64_t>(a.num_seqs) * a.num_kv_heads;
  const int64_t n = (groups + 7) / 8 * 8 * a.num_splits * a.row_tiles;
  if (n <= 0) return hipSuccess;
  if (n > 0x7fffffff) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(n));
  if (short_rows) {
    if (a.row_tiles != 1) return hipErrorInvalidValue;
    if (kv_fp8) hipLaunchKernelGGL((attn_mfma_kernel<true, true>), grid, dim3(NT), 0, s, a);
    else hipLaunchKernelGGL((attn_mfma_kernel<false, true>), grid, dim3(NT), 0, s, a);
  } else {
    // (bf16 pools with long chunks run in attn_long_kernel)
    if (!kv_fp8) return hipErrorInvalidValue;
    hipLaunchKernelGGL((attn_mfma_kernel<true, false>), grid, dim3(NT), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_attn_combine(const AttnArgs& a, hipStream_t s) {
  const int64_t rows = a.num_q_tokens * a.num_q_heads;
  if (rows <= 0) return hipSuccess;
  // (one instantiation per bound on the split count: registers for unused
  // splits would lower the occupancy this latency-bound kernel relies on)
  const dim3 grid(static_cast<unsigned>((rows + kCombineRows - 1) / kCombineRows));
  if (a.num_splits <= 4) hipLaunchKernelGGL(attn_combine_kernel<4>, grid, dim3(256), 0, s, a);
  else if (a.num_splits <= 8) hipLaunchKernelGGL(attn_combine_kernel<8>, grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL(attn_combine_kernel<kMaxSplits>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace pkv
