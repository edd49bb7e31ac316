// Paged attention on the gfx950 matrix cores: bf16 queries over bf16 or fp8
// (OCP e4m3fn) K/V pools, head_dim 128.
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
//   never read).  bf16 pools are copied straight from HBM into LDS with
//   direct global-to-LDS loads; fp8 pools go through registers, where e4m3 is
//   widened to bf16 exactly.  Keys outside the workgroup's range read a row
//   of zeros, so a value row that does not exist is 0, never garbage.
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
//   while tile t + 3 streams into LDS.
//
// Split keys: with num_splits > 1 each workgroup writes unnormalised partial
// (O, max, sum) for its key range to the workspace and a combine kernel merges
// the splits in a fixed order (deterministic, no atomics).
#include <type_traits>

#include "attn_common.hpp"

namespace pkv {

// Zeros that direct-to-LDS loads of keys outside the staged range read
// (static device storage starts zeroed and is never written).
__device__ __attribute__((aligned(16))) uint32_t g_zero_row[64 * 4];

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lds_ptr;
typedef __attribute__((address_space(3))) v4i16* lds_v4i16_ptr;

constexpr int D = 128;
constexpr int KT = kMfmaKeyTile;  // keys per tile
constexpr int NW = 8;             // waves per workgroup (two per SIMD)
constexpr int NT = 64 * NW;
constexpr int kRowBytes = D * 2;            // one bf16 K or V row of an LDS tile
constexpr int kTileBytes = KT * kRowBytes;   // 16 KB
constexpr int kWaveRows = 32;     // query rows per wave: one 32-wide MFMA column block
static_assert(kMfmaRows == NW * kWaveRows, "rows per workgroup");
constexpr float kRescaleLog2 = 8.0f;  // stale-max slack before O and l are rescaled
constexpr int kBufs = 4;             // LDS K/V tile buffers: tiles t, t + 1 read while t + 2, t + 3 arrive
constexpr int kLdsBytes = 2 * kBufs * kTileBytes + kTableSlice * 4;
static_assert(kLdsBytes <= 160 * 1024, "LDS budget of a gfx950 CU");

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

// LDS byte address of p, hidden from the optimiser: addresses built as
// opaque base + constant keep the constant (buffer, key block) in the 16-bit
// offset field of the LDS instruction instead of an add per read.
__device__ __forceinline__ uint32_t lds_addr(const uint8_t* p) {
  uint32_t a = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_ptr)p));
  asm volatile("" : "+v"(a));
  return a;
}
template <typename T>
__device__ __forceinline__ const __attribute__((address_space(3))) T* lds_at(uint32_t a) {
  return (const __attribute__((address_space(3))) T*)(a);
}

template <int B>
using Buf = std::integral_constant<int, B>;

// One 16-byte-per-lane direct global-to-LDS load: lane i's 16 bytes from g
// land at l + 16 i (l is wave-uniform, passed in M0).  Issued as inline
// assembly so that the compiler does not add waits of its own for it: the
// kernel waits for these loads explicitly (wait_vmcnt) before the barrier
// that precedes their first reader.
__device__ __forceinline__ void dma16(const void* g, uint8_t* l) {
  const uint32_t m0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_ptr)l));
  asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(g), "{m0}"(m0));
}
// The same with a wave-uniform base address in SGPRs and a per-lane 32-bit
// byte offset, so the address takes no vector arithmetic.
__device__ __forceinline__ void dma16(const uint8_t* base, uint32_t off, uint8_t* l) {
  const uint32_t m0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_ptr)l));
  asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base), "{m0}"(m0));
}
static_assert(kTableSlice * 16 >= kMaxSplitKeys, "table slice must cover a split");

// Workgroup barrier for the K/V tile pipeline.  __syncthreads() -- and any
// release fence on LDS -- makes every wave wait for all of its outstanding
// vector-memory loads, including the direct-to-LDS loads of tiles that are
// only read iterations later, which would drain the prefetch at every tile.
// Here each wave waits for its own LDS stores (lgkmcnt) and, before calling
// this, for exactly the direct loads the next iteration reads (wait_vmcnt);
// the empty asm statements keep the compiler from moving memory accesses
// across the barrier.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt not waited on
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Chunk permutation of LDS tile rows.  The LDS serves 256 bytes per clock
// from 64 four-byte banks, and a 256-byte row maps onto all of them, so the
// 16-byte chunk c of row r is stored at position c ^ swz(r):
//   K: the MFMA reads one chunk from 16 consecutive rows per clock -> XOR with
//      r mod 16 puts them in 16 distinct positions;
//   V: a transposing read takes four consecutive rows x 64 bytes (four
//      chunks 4 k .. 4 k + 3) per clock -> XOR with 4 (r mod 4) moves each row
//      to its own 64-byte quarter.
__device__ __forceinline__ int k_swz(int r) { return r & 15; }
__device__ __forceinline__ int v_swz(int r) { return 4 * (r & 3); }

// Waits until at most N of this wave's vector-memory loads are outstanding
// (loads complete in order).  Direct-to-LDS loads are only counted here, so
// the consumer's barrier must be preceded by this wait.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Lanes l and l ^ 32 hold the two key halves of one query row in the S^T
// accumulator layout.  v_permlane32_swap exchanges the upper half of its first
// operand with the lower half of its second; with the same value in both, each
// lane ends up with its own value in one result and its partner's in the
// other, so max / sum over the pair are order-free functions of the two.
__device__ __forceinline__ float max_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Two floats known to be exact in bf16 (decoded e4m3 values) -> packed bf16 pair.
__device__ __forceinline__ uint32_t pack_exact_bf16(float lo, float hi) {
  return (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xFFFF0000u);
}

// Eight e4m3 codes -> eight bf16 (exact: every e4m3 value is a bf16 value),
// two codes per v_cvt_scalef32_pk_bf16_fp8 with scale 1.
__device__ __forceinline__ u32x4 e4m3x8_to_bf16x8(u32x2 c) {
  u32x4 r;
#pragma unroll
  for (int w = 0; w < 2; ++w) {
    r[2 * w] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[w], 1.0f, false));
    r[2 * w + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[w], 1.0f, true));
  }
  return r;
}

// Two floats -> packed bf16 pair, round to nearest even (one v_cvt_pk_bf16_f32;
// converting the two halves separately costs five instructions).
__device__ __forceinline__ uint32_t pack_bf16_rne(float lo, float hi) {
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// acc + lo + hi of a packed bf16 pair, accumulated in fp32.
__device__ __forceinline__ float add_bf16_pair(uint32_t pair, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pair),
                                         __builtin_bit_cast(bf16x2, 0x3F803F80u), acc, false);
}

// SHORT: at most 64 rows per (sequence, KV head) (short query chunks).  The
// eight waves then split the keys instead of the rows: wave w takes row block
// w % 2 (32 rows) and key group w / 2, i.e. tiles 4 i + w / 2 of iteration i,
// so every wave multiplies while the whole workgroup loads the next four tiles
// into registers; the four key groups' partial results are merged in LDS.
template <bool FP8, bool SHORT>
__global__ __attribute__((amdgpu_flat_work_group_size(NT, NT), amdgpu_waves_per_eu(2, 2))) void
attn_mfma_kernel(AttnArgs a) {
  int32_t* tbl = s_tbl;
  constexpr int ELSZ = FP8 ? 1 : 2;

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l32 = lane & 31;
  const int h2 = lane >> 5;

  // ---- work item: XCD-aware remap so that workgroups sharing K/V (same
  // sequence, KV head, key split) are dispatched to the same XCD and its L2.
  const uint32_t n = gridDim.x;
  const uint32_t id = blockIdx.x;
  const uint32_t xcd = id & 7u, k8 = id >> 3, q8 = n >> 3, r8 = n & 7u;
  const uint32_t logical = (xcd < r8) ? xcd * (q8 + 1) + k8 : r8 * (q8 + 1) + (xcd - r8) * q8 + k8;
  const int rt = static_cast<int>(logical % static_cast<uint32_t>(a.row_tiles));
  uint32_t rest = logical / static_cast<uint32_t>(a.row_tiles);
  const int z = static_cast<int>(rest % static_cast<uint32_t>(a.num_splits));
  rest /= static_cast<uint32_t>(a.num_splits);
  const int hk = static_cast<int>(rest % static_cast<uint32_t>(a.num_kv_heads));
  const int b = static_cast<int>(rest / static_cast<uint32_t>(a.num_kv_heads));

  const int G = a.group;
  const int t0 = a.qsl[b];
  const int q_len = a.qsl[b + 1] - t0;
  const int s = a.seq_lens[b];
  const int R = q_len * G;
  const int r0 = rt * kMfmaRows;
  if (r0 >= R) return;
  const int seg0 = a.seg_loc[b], seg1 = a.seg_loc[b + 1];
  const int gbase = s - q_len;
  // Row limits are non-decreasing in the row's key position, so the last row
  // bounds the workgroup's key range and the first row of a wave its mask-free prefix.
  const int wg_kmax = row_limit(a.segments, seg0, seg1, gbase + (min(r0 + kMfmaRows, R) - 1) / G);
  const int k_begin = z * a.split_len;
  const int k_end = min(k_begin + a.split_len, wg_kmax);
  if (k_begin >= k_end) return;

  const int kg = SHORT ? (w >> 1) : 0;  // key group (SHORT)
  const int wr0 = SHORT ? kWaveRows * (w & 1) : r0 + kWaveRows * w;
  int wave_kmin = 0, wave_kmax = 0;
  if (wr0 < R) {
    wave_kmin = row_limit(a.segments, seg0, seg1, gbase + wr0 / G);
    wave_kmax = row_limit(a.segments, seg0, seg1, gbase + (min(wr0 + kWaveRows, R) - 1) / G);
  }

  // ---- this lane's query row
  const int row = wr0 + l32;
  const bool valid = row < R;
  const int tok = valid ? row / G : 0;
  const int head = hk * G + (valid ? row % G : 0);
  const int Lrow = valid ? row_limit(a.segments, seg0, seg1, gbase + tok) : 0;

  // Q^T fragments for S^T = K Q^T: lane holds 8 consecutive head-dim values
  // [16 t + 8 h2, +8) of its query row for each of the 8 k-steps.
  bf16x8 qf[8];
  {
    const __bf16* qr = static_cast<const __bf16*>(a.q) +
                       (static_cast<int64_t>(t0 + tok) * a.num_q_heads + head) * D + 8 * h2;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (valid) v = *reinterpret_cast<const u32x4*>(qr + 16 * t);
      qf[t] = __builtin_bit_cast(bf16x8, v);
    }
  }
  // Q has landed before any K/V load is issued.  The compiler cannot see the
  // direct-to-LDS loads (inline assembly); without this wait it may guard a
  // later use of Q with a full vmcnt(0), which would drain the K/V prefetch.
  wait_vmcnt<0>();

  // ---- block-table slice for this workgroup's keys
  const int32_t* table = a.block_table + static_cast<int64_t>(b) * a.table_width;
  const int nblk = (s + 15) >> 4;
  const int blk_lo = k_begin >> 4;
  const int blk_hi = min((k_end + 15) >> 4, nblk);
  for (int i = threadIdx.x; i < blk_hi - blk_lo; i += NT) tbl[i] = table[blk_lo + i];
  lds_barrier();
  // Keys at or past kv_lim are staged as zeros: past seq_len they do not exist,
  // and past the slice every row of the workgroup masks them anyway.
  const int kv_lim = min(s, blk_hi * 16);

  // ---- staging geometry: wave w stages tile rows [8 w, 8 w + 8) of both the
  // K and the V tile, four rows (one 1 KB direct load) per step; lane i takes
  // row 8 w + 4 step + i / 16 and LDS chunk position i % 16.
  const int64_t row_bytes = static_cast<int64_t>(a.num_kv_heads) * D * ELSZ;
  const int64_t block_bytes = 16 * row_bytes;
  const uint8_t* kpool = static_cast<const uint8_t*>(a.kpool) + static_cast<int64_t>(hk) * D * ELSZ;
  const uint8_t* vpool = static_cast<const uint8_t*>(a.vpool) + static_cast<int64_t>(hk) * D * ELSZ;
  const int st_pos = lane & 15;
  int st_row[2], k_src_off[2], v_src_off[2];
#pragma unroll
  for (int st = 0; st < 2; ++st) {
    st_row[st] = 8 * w + 4 * st + (lane >> 4);
    const int rb = st_row[st] & 15;  // row inside its 16-token block
    k_src_off[st] = static_cast<int>(rb * row_bytes) + (st_pos ^ k_swz(st_row[st])) * 8 * ELSZ;
    v_src_off[st] = static_cast<int>(rb * row_bytes) + (st_pos ^ v_swz(st_row[st])) * 8 * ELSZ;
  }
  const uint8_t* zero_row = reinterpret_cast<const uint8_t*>(g_zero_row) + 16 * st_pos;

  // Issue the loads of the tile at key kt into LDS buffer buf (bf16: direct
  // to LDS; fp8: into registers, see fp8_store).
  u32x2 f8k[2], f8v[2];
  // Block-table entry of the 16 keys this wave stages for the tile at key kt.
  auto stage_entry = [&](int kt) {
    const int blk = (kt >> 4) + (w >> 1);
    return (blk < blk_hi) ? tbl[blk - blk_lo] : 0;
  };
  auto stage_load = [&](int kt, auto bufc, int e) {
    constexpr int B = decltype(bufc)::value;
    // The wave's eight rows lie in one 16-key block: its base address is
    // wave-uniform and lives in SGPRs.
    const int64_t boff = static_cast<int64_t>(__builtin_amdgcn_readfirstlane(e)) * block_bytes;
    const uint8_t* kb = kpool + boff;
    const uint8_t* vb = vpool + boff;
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      const int dst = (8 * w + 4 * st) * kRowBytes;
      if (kt + 8 * w + 4 * st + 4 <= kv_lim) {  // all four rows exist (uniform)
        if constexpr (FP8) {
          f8k[st] = *reinterpret_cast<const u32x2*>(kb + k_src_off[st]);
          f8v[st] = *reinterpret_cast<const u32x2*>(vb + v_src_off[st]);
        } else {
          dma16(kb, static_cast<uint32_t>(k_src_off[st]), kbuf<B>() + dst);
          dma16(vb, static_cast<uint32_t>(v_src_off[st]), vbuf<B>() + dst);
        }
      } else {  // the tile at the end of the staged keys: rows past kv_lim read zeros
        const bool ok = kt + st_row[st] < kv_lim;
        if constexpr (FP8) {
          f8k[st] = ok ? *reinterpret_cast<const u32x2*>(kb + k_src_off[st]) : u32x2{0u, 0u};
          f8v[st] = ok ? *reinterpret_cast<const u32x2*>(vb + v_src_off[st]) : u32x2{0u, 0u};
        } else {
          dma16(ok ? kb + k_src_off[st] : zero_row, kbuf<B>() + dst);
          dma16(ok ? vb + v_src_off[st] : zero_row, vbuf<B>() + dst);
        }
      }
    }
  };
  // fp8 only: widen the registers of the last stage_load into LDS buffer buf.
  auto fp8_store = [&](auto bufc) {
    constexpr int B = decltype(bufc)::value;
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      const int dst = st_row[st] * kRowBytes + 16 * st_pos;
      *reinterpret_cast<u32x4*>(kbuf<B>() + dst) = e4m3x8_to_bf16x8(f8k[st]);
      *reinterpret_cast<u32x4*>(vbuf<B>() + dst) = e4m3x8_to_bf16x8(f8v[st]);
    }
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

  auto qk = [&](auto bufc, f32x16 (&sacc)[2]) {
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
  auto mask_and_rescale = [&](int kt, f32x16 (&sacc)[2]) {
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
  auto probs = [&](f32x16 (&sacc)[2], bf16x8 (&pb)[2][2]) {
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
          pk[e] = pack_bf16_rne(sacc[kb][8 * k16 + 2 * e], sacc[kb][8 * k16 + 2 * e + 1]);
          // The row sum takes the bf16-rounded probabilities, the very
          // weights that multiply V, so the output's weights sum to one.
          ls[e] = add_bf16_pair(pk[e], ls[e]);
        }
        pb[kb][k16] = __builtin_bit_cast(bf16x8, pk);
      }
    l += (ls[0] + ls[1]) + (ls[2] + ls[3]);
  };

  auto pv = [&](auto bufc, const bf16x8 (&pb)[2][2]) {
    constexpr int B = decltype(bufc)::value;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int k16 = 0; k16 < 2; ++k16)
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          const uint32_t base = v_rd[db] + B * kTileBytes + (32 * kb + 16 * k16) * kRowBytes;
          const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_ptr)(base));
          const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_ptr)(base + 8 * kRowBytes));
          const bf16x8 va = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
          o[db] = mfma(va, pb[kb][k16], o[db]);
        }
  };

  if constexpr (SHORT) {
    // ---- iteration i: each wave multiplies tile 4 i + kg from buffer kg
    // while the workgroup loads tiles 4 i + 4 .. 4 i + 7 into registers; after
    // a barrier they are written (fp8 widened) into buffers 0..3.
    // Register staging, 16 bytes per lane per load.  bf16: lane i of wave w
    // holds chunk i % 16 of rows 8 w + 4 st + i / 16 (st = 0, 1), at the
    // positions stage_load uses.  fp8: one load per tile covers the wave's
    // eight rows, lane i holding codes [16 p, 16 p + 16) (p = i % 8) of row
    // 8 w + i / 8, i.e. chunks 2 p and 2 p + 1 once widened.
    constexpr int kLoads = FP8 ? 1 : 2;  // loads per tile per lane, for K and for V
    // fp8 tiles are loaded two steps ahead (two register sets); bf16 tiles,
    // twice the bytes, one step ahead.
    constexpr int kSets = FP8 ? 2 : 1;
    u32x4 rk[kSets][4][kLoads], rv[kSets][4][kLoads];
    const int f8_row = 8 * w + (lane >> 3), f8_pair = lane & 7;
    const int f8_src = (f8_row & 15) * static_cast<int>(row_bytes) + 16 * f8_pair;
    const int ntiles = (k_end - k_begin + KT - 1) / KT;
    auto kt_of = [&](int t) { return k_begin + t * KT; };
    auto load4 = [&](auto setc, int t_first) {
      constexpr int S = decltype(setc)::value;
      // All four block-table entries first: one LDS round trip, not four.
      int e[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) e[j] = (t_first + j < ntiles) ? stage_entry(kt_of(t_first + j)) : 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int t = t_first + j;
        if (t >= ntiles) break;
        const int kt = kt_of(t);
        const int64_t boff = static_cast<int64_t>(__builtin_amdgcn_readfirstlane(e[j])) * block_bytes;
        const u32x4 zero = {0u, 0u, 0u, 0u};
        if constexpr (FP8) {
          const bool ok = kt + f8_row < kv_lim;
          rk[S][j][0] = ok ? *reinterpret_cast<const u32x4*>(kpool + boff + f8_src) : zero;
          rv[S][j][0] = ok ? *reinterpret_cast<const u32x4*>(vpool + boff + f8_src) : zero;
        } else {
#pragma unroll
          for (int st = 0; st < 2; ++st) {
            const bool ok = kt + st_row[st] < kv_lim;
            rk[S][j][st] = ok ? *reinterpret_cast<const u32x4*>(kpool + boff + k_src_off[st]) : zero;
            rv[S][j][st] = ok ? *reinterpret_cast<const u32x4*>(vpool + boff + v_src_off[st]) : zero;
          }
        }
      }
    };
    auto store4 = [&](auto setc, int t_first) {
      constexpr int S = decltype(setc)::value;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (t_first + j >= ntiles) break;
        if constexpr (FP8) {
          const int row = f8_row * kRowBytes;
          const u32x4 klo = e4m3x8_to_bf16x8(u32x2{rk[S][j][0][0], rk[S][j][0][1]});
          const u32x4 khi = e4m3x8_to_bf16x8(u32x2{rk[S][j][0][2], rk[S][j][0][3]});
          const u32x4 vlo = e4m3x8_to_bf16x8(u32x2{rv[S][j][0][0], rv[S][j][0][1]});
          const u32x4 vhi = e4m3x8_to_bf16x8(u32x2{rv[S][j][0][2], rv[S][j][0][3]});
          *reinterpret_cast<u32x4*>(s_k[j] + row + 16 * ((2 * f8_pair) ^ k_swz(f8_row))) = klo;
          *reinterpret_cast<u32x4*>(s_k[j] + row + 16 * ((2 * f8_pair + 1) ^ k_swz(f8_row))) = khi;
          *reinterpret_cast<u32x4*>(s_v[j] + row + 16 * ((2 * f8_pair) ^ v_swz(f8_row))) = vlo;
          *reinterpret_cast<u32x4*>(s_v[j] + row + 16 * ((2 * f8_pair + 1) ^ v_swz(f8_row))) = vhi;
        } else {
#pragma unroll
          for (int st = 0; st < 2; ++st) {
            const int dst = st_row[st] * kRowBytes + 16 * st_pos;
            *reinterpret_cast<u32x4*>(s_k[j] + dst) = rk[S][j][st];
            *reinterpret_cast<u32x4*>(s_v[j] + dst) = rv[S][j][st];
          }
        }
      }
    };
    f32x16 sacc[2];
    auto step = [&](auto cur, int t4) {
      // Loads of the tiles two steps (fp8) or one step (bf16) ahead.
      constexpr int C = decltype(cur)::value;
      if constexpr (kSets == 2) load4(std::integral_constant<int, 1 - C>{}, t4 + 8);
      else load4(std::integral_constant<int, 0>{}, t4 + 4);
      const int t = t4 + kg;
      if (t < ntiles && kt_of(t) < wave_kmax) {
        qk(Buf<0>{}, sacc);
        mask_and_rescale(kt_of(t), sacc);
        bf16x8 pb[2][2];
        probs(sacc, pb);
        pv(Buf<0>{}, pb);
      }
      lds_barrier();
      if constexpr (kSets == 2) store4(std::integral_constant<int, C>{}, t4 + 4);
      else store4(std::integral_constant<int, 0>{}, t4 + 4);
      lds_barrier();
    };
    if constexpr (kSets == 2) {
      load4(std::integral_constant<int, 0>{}, 0);
      store4(std::integral_constant<int, 0>{}, 0);
      load4(std::integral_constant<int, 0>{}, 4);
      lds_barrier();
      // Step i keeps tiles 4 i + 4 .. + 7 in set i % 2 and loads 4 i + 8 .. into the other.
      for (int t4 = 0; t4 < ntiles; t4 += 8) {
        step(std::integral_constant<int, 0>{}, t4);
        if (t4 + 4 < ntiles) step(std::integral_constant<int, 1>{}, t4 + 4);
      }
    } else {
      load4(std::integral_constant<int, 0>{}, 0);
      store4(std::integral_constant<int, 0>{}, 0);
      lds_barrier();
      for (int t4 = 0; t4 < ntiles; t4 += 4) step(std::integral_constant<int, 0>{}, t4);
    }

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
  } else {
    // ---- software pipeline over tiles t = 0 .. n-1 (tile t: keys k_begin + 64 t,
    // LDS buffer t % 4).  Iteration t: mask / max of S(t); S(t+1) = K(t+1) Q^T
    // next to the exponentials of S(t); O += V(t) P(t); then the loads of tile
    // t + 3 are issued (bf16) or tile t + 2 is widened into LDS and tile t + 3
    // loaded into registers (fp8).  Buffer (t + 3) % 4 held tile t - 1, whose
    // last reader was iteration t - 1; the barrier closing iteration t makes
    // tile t + 2 visible to iteration t + 1.  S(t + 1) of the last tile reads a
    // stale buffer and is never used.
    const int ntiles = (k_end - k_begin + KT - 1) / KT;
    auto kt_of = [&](int t) { return k_begin + t * KT; };
    if constexpr (FP8) {
      stage_load(kt_of(0), Buf<0>{}, stage_entry(kt_of(0)));
      fp8_store(Buf<0>{});
      if (ntiles > 1) { stage_load(kt_of(1), Buf<1>{}, stage_entry(kt_of(1))); fp8_store(Buf<1>{}); }
      if (ntiles > 2) stage_load(kt_of(2), Buf<2>{}, stage_entry(kt_of(2)));
    } else {
      stage_load(kt_of(0), Buf<0>{}, stage_entry(kt_of(0)));
      if (ntiles > 1) stage_load(kt_of(1), Buf<1>{}, stage_entry(kt_of(1)));
      if (ntiles > 2) {
        stage_load(kt_of(2), Buf<2>{}, stage_entry(kt_of(2)));
        wait_vmcnt<4>();
      } else {
        wait_vmcnt<0>();
      }
    }
    int e_next = stage_entry(kt_of(3));  // entry for the tile staged in iteration 0
    lds_barrier();
    f32x16 sA[2], sB[2];
    qk(Buf<0>{}, sA);

    auto iteration = [&](auto bufc, int t, f32x16 (&s_cur)[2], f32x16 (&s_next)[2]) {
      constexpr int B = decltype(bufc)::value;
      const int kt = kt_of(t);
      // Tile t + 3 goes into buffer (t + 3) % 4, free since the barrier that
      // closed iteration t - 1; bf16 loads are issued first so that they
      // overlap this iteration's math.
      const int e_use = e_next;
      e_next = stage_entry(kt_of(t + 4));
      if constexpr (!FP8) {
        if (t + 3 < ntiles) stage_load(kt_of(t + 3), Buf<(B + 3) % kBufs>{}, e_use);
      }
      if (kt < wave_kmax) {
        mask_and_rescale(kt, s_cur);
        bf16x8 pb[2][2];
        qk(Buf<(B + 1) % kBufs>{}, s_next);
        probs(s_cur, pb);
        pv(bufc, pb);
      }
      if constexpr (FP8) {
        if (t + 2 < ntiles) fp8_store(Buf<(B + 2) % kBufs>{});
        if (t + 3 < ntiles) stage_load(kt_of(t + 3), Buf<(B + 3) % kBufs>{}, e_use);
      } else {
        // Tile t + 2 (issued one iteration ago) must have landed before the
        // barrier after which iteration t + 1 reads it.
        if (t + 3 < ntiles) wait_vmcnt<4>(); else wait_vmcnt<0>();
      }
      lds_barrier();
    };
    for (int t = 0; t < ntiles; t += kBufs) {
      iteration(Buf<0>{}, t, sA, sB);
      if (t + 1 < ntiles) iteration(Buf<1>{}, t + 1, sB, sA);
      if (t + 2 < ntiles) iteration(Buf<2>{}, t + 2, sA, sB);
      if (t + 3 < ntiles) iteration(Buf<3>{}, t + 3, sB, sA);
    }
  }

  // ---- epilogue
  const float lt = SHORT ? lt_merged : sum_halves(l);
  if (!valid) return;
  const int64_t total_rows = a.num_q_tokens * a.num_q_heads;
  const int64_t orow_id = static_cast<int64_t>(t0 + tok) * a.num_q_heads + head;
  if (a.num_splits > 1) {
    float* wo = a.ws_o + (static_cast<int64_t>(z) * total_rows + orow_id) * D;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        f32x4 v = {o[db][4 * rq], o[db][4 * rq + 1], o[db][4 * rq + 2], o[db][4 * rq + 3]};
        *reinterpret_cast<f32x4*>(wo + 32 * db + 8 * rq + 4 * h2) = v;
      }
    if (h2 == 0) {
      f32x2 ml = {m, lt};
      *reinterpret_cast<f32x2*>(a.ws_ml + (static_cast<int64_t>(z) * total_rows + orow_id) * 2) = ml;
    }
  } else {
    const float inv = a.v_scale / lt;
    __bf16* orow = static_cast<__bf16*>(a.out) + orow_id * D;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        u32x2 v;
        v[0] = pack_bf16_rne(o[db][4 * rq] * inv, o[db][4 * rq + 1] * inv);
        v[1] = pack_bf16_rne(o[db][4 * rq + 2] * inv, o[db][4 * rq + 3] * inv);
        *reinterpret_cast<u32x2*>(orow + 32 * db + 8 * rq + 4 * h2) = v;
      }
  }
}

// Merges the key splits of a row, in split order: 32 lanes per row, four
// head-dim values per lane, eight rows per workgroup.
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnArgs a) {
  const int sub = threadIdx.x & 31;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 8 + (threadIdx.x >> 5);
  const int64_t total_rows = a.num_q_tokens * a.num_q_heads;
  if (row >= total_rows) return;
  const int64_t t = row / a.num_q_heads;
  const int b = seq_of_token(a.qsl, a.num_seqs, t);
  const int t0 = a.qsl[b];
  const int q_len = a.qsl[b + 1] - t0;
  const int g = a.seq_lens[b] - q_len + static_cast<int>(t - t0);
  const int L = row_limit(a.segments, a.seg_loc[b], a.seg_loc[b + 1], g);
  const int nz = min(a.num_splits, (L + a.split_len - 1) / a.split_len);
  f32x2 ml[kMaxSplits];
  f32x4 ov[kMaxSplits];
  float M = -INFINITY;
#pragma unroll
  for (int zz = 0; zz < kMaxSplits; ++zz) {
    if (zz < nz) {
      ml[zz] = *reinterpret_cast<const f32x2*>(a.ws_ml + (zz * total_rows + row) * 2);
      ov[zz] = *reinterpret_cast<const f32x4*>(a.ws_o + (zz * total_rows + row) * D + 4 * sub);
      M = fmaxf(M, ml[zz][0]);
    }
  }
  float den = 0.f;
  f32x4 num = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int zz = 0; zz < kMaxSplits; ++zz) {
    if (zz < nz) {
      const float wz = __builtin_amdgcn_exp2f((ml[zz][0] - M) * a.scale_log2);
      den = fmaf(wz, ml[zz][1], den);
#pragma unroll
      for (int e = 0; e < 4; ++e) num[e] = fmaf(wz, ov[zz][e], num[e]);
    }
  }
  const float inv = a.v_scale / den;
  u32x2 packed;
  packed[0] = pack_bf16_rne(num[0] * inv, num[1] * inv);
  packed[1] = pack_bf16_rne(num[2] * inv, num[3] * inv);
  *reinterpret_cast<u32x2*>(static_cast<__bf16*>(a.out) + row * D + 4 * sub) = packed;
}

}  // namespace

hipError_t launch_attn_mfma(const AttnArgs& a, bool kv_fp8, bool short_rows, hipStream_t s) {
  const int64_t n = static_cast<int64_t>(a.num_seqs) * a.num_kv_heads * a.num_splits * a.row_tiles;
  if (n <= 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>(n));
  if (short_rows) {
    if (a.row_tiles != 1) return hipErrorInvalidValue;
    if (kv_fp8) hipLaunchKernelGGL((attn_mfma_kernel<true, true>), grid, dim3(NT), 0, s, a);
    else hipLaunchKernelGGL((attn_mfma_kernel<false, true>), grid, dim3(NT), 0, s, a);
  } else {
    if (kv_fp8) hipLaunchKernelGGL((attn_mfma_kernel<true, false>), grid, dim3(NT), 0, s, a);
    else hipLaunchKernelGGL((attn_mfma_kernel<false, false>), grid, dim3(NT), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_attn_combine(const AttnArgs& a, hipStream_t s) {
  const int64_t rows = a.num_q_tokens * a.num_q_heads;
  if (rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(attn_combine_kernel, dim3(static_cast<unsigned>((rows + 7) / 8)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace pkv
