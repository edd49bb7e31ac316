// Paged attention on the gfx950 matrix cores: bf16 queries over bf16 or fp8
// (OCP e4m3fn) K/V pools, head_dim 128.
//
// Work decomposition
//   A "row" is one (query token, query head) pair of a KV-head group; a
//   sequence with q tokens and G = Hq / Hkv query heads per KV head has q * G
//   rows per KV head, ordered token-major, so the G heads that share a K/V
//   tile are computed from one LDS copy of it (GQA).  A workgroup (4 waves)
//   owns 256 consecutive rows of one (sequence, KV head) and, when the key
//   range is split, one range of keys.  Each wave owns 64 rows, as two
//   32-wide column blocks of the 32x32x16 bf16 MFMA.
//
// Per 64-key tile
//   * the tile's four 16-token blocks are found through the block table (one
//     table entry per block; entries past ceil(seq_len / 16) are never read),
//     K rows land in LDS row-major, V rows transposed (head_dim-major) so the
//     P.V product can read 16-byte fragments; keys at or past seq_len are
//     written as zeros, never loaded;
//   * S^T = K Q^T on the MFMA: the accumulator puts one query per lane and 16
//     keys per lane in registers, so the row max / row sum need one cross-half
//     swap (v_permlane32_swap) instead of a 32-lane reduction;
//   * the piecewise mask is a per-row key bound L(g) (full segment: kv_end,
//     causal: g + 1), applied only on tiles that cross some row's bound;
//   * online softmax in the exp2 domain (scale * log2 e folded into one FMA);
//   * O^T += V^T P^T on the MFMA, with P rounded to bf16 as the pages' own
//     reference rounds probabilities to the value dtype before the product.
//   The next tile's global loads are issued before the current tile's math
//   (register prefetch), and LDS is double-buffered: one barrier per tile.
//
// Split keys: with num_splits > 1 each workgroup writes unnormalised partial
// (O, max, sum) for its key range to the workspace and a combine kernel merges
// the splits in a fixed order (deterministic, no atomics).
#include "attn_common.hpp"

namespace pkv {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int D = 128;
constexpr int KT = kMfmaKeyTile;  // keys per tile
constexpr int NW = 8;             // waves per workgroup (two per SIMD)
constexpr int NT = 64 * NW;
constexpr int KS = D + 8;    // K tile row stride in LDS (bf16): 272 B, breaks bank aliasing
constexpr int VS = KT + 8;   // V^T tile row stride in LDS (bf16): 144 B
constexpr int K_ELEMS = KT * KS;
constexpr int V_ELEMS = D * VS;
constexpr int BUF = K_ELEMS + V_ELEMS;
constexpr int kWaveRows = 32;     // query rows per wave: one 32-wide MFMA column block
static_assert(kMfmaRows == NW * kWaveRows, "rows per workgroup");
constexpr float kRescaleLog2 = 8.0f;  // stale-max slack before O and l are rescaled

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

// Eight e4m3 codes -> eight bf16 (exact: every e4m3 value is a bf16 value).
__device__ __forceinline__ u32x4 e4m3x8_to_bf16x8(u32x2 c) {
  u32x4 r;
#pragma unroll
  for (int w = 0; w < 2; ++w) {
    const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(c[w]), false);
    const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(c[w]), true);
    r[2 * w] = pack_exact_bf16(lo[0], lo[1]);
    r[2 * w + 1] = pack_exact_bf16(hi[0], hi[1]);
  }
  return r;
}

__device__ __forceinline__ uint32_t pack_bf16_rne(float lo, float hi) {
  const __bf16 a = static_cast<__bf16>(lo);
  const __bf16 b = static_cast<__bf16>(hi);
  return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, a)) |
         (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, b)) << 16);
}

template <bool FP8>
__global__ __attribute__((amdgpu_flat_work_group_size(NT, NT), amdgpu_waves_per_eu(2, 2))) void
attn_mfma_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) __bf16 lds[2 * BUF];
  constexpr int ELSZ = FP8 ? 1 : 2;
  using Chunk = typename std::conditional<FP8, u32x2, u32x4>::type;  // 8 head-dim elements

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

  const int wr0 = r0 + kWaveRows * w;
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

  // ---- K/V staging: waves 0-3 stage K, waves 4-7 stage V, 4 chunks per lane.
  const bool stage_k = w < 4;
  const int sw = w & 3;
  const int64_t row_elems = static_cast<int64_t>(a.num_kv_heads) * D;
  const uint8_t* src = static_cast<const uint8_t*>(stage_k ? a.kpool : a.vpool) + static_cast<int64_t>(hk) * D * ELSZ;
  const int32_t* table = a.block_table + static_cast<int64_t>(b) * a.table_width;
  const int nblk = (s + 15) >> 4;
  // K: wave sw stages keys [16 sw, 16 sw + 16) -- exactly tile block sw; lanes
  // 16 apart take consecutive keys, lanes within 16 the 16 head-dim chunks.
  // V: lane takes 4 consecutive keys 4 vkq + it of head-dim chunk v_chunk and
  // writes them transposed as one 8-byte run per head-dim element.
  const int vkq = lane & 15;
  const int key_of_it0 = stage_k ? 16 * sw + (lane >> 4) : 4 * vkq;  // key of chunk 0
  const int key_step = stage_k ? 4 : 1;
  const int chunk = stage_k ? (lane & 15) : 4 * sw + (lane >> 4);
  const int v_pos = 16 * (vkq >> 2) + 8 * (vkq & 1) + 4 * ((vkq >> 1) & 1);

  Chunk pre[4];
  auto load_tile = [&](int kt) {
    const int blk = (kt >> 4) + (stage_k ? sw : (vkq >> 2));  // one table entry per lane
    const int e = (blk < nblk) ? table[blk] : 0;
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int kk = key_of_it0 + key_step * it;
      const int64_t slot = static_cast<int64_t>(e) * 16 + (kk & 15);
      const uint8_t* p = src + (slot * row_elems + 8 * chunk) * ELSZ;
      Chunk zero = {};
      pre[it] = (kt + kk < s) ? *reinterpret_cast<const Chunk*>(p) : zero;
    }
  };

  auto store_tile = [&](int buf) {
    __bf16* Kl = lds + buf * BUF;
    __bf16* Vl = Kl + K_ELEMS;
    u32x4 v[4];
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      if constexpr (FP8) v[it] = e4m3x8_to_bf16x8(pre[it]); else v[it] = pre[it];
    }
    if (stage_k) {
#pragma unroll
      for (int it = 0; it < 4; ++it)
        *reinterpret_cast<u32x4*>(Kl + (key_of_it0 + 4 * it) * KS + 8 * chunk) = v[it];
    } else {
#pragma unroll
      for (int dd = 0; dd < 8; ++dd) {
        const int wd = dd >> 1;
        u32x2 x;
        if (dd & 1) {
          x[0] = (v[0][wd] >> 16) | (v[1][wd] & 0xFFFF0000u);
          x[1] = (v[2][wd] >> 16) | (v[3][wd] & 0xFFFF0000u);
        } else {
          x[0] = (v[0][wd] & 0xFFFFu) | (v[1][wd] << 16);
          x[1] = (v[2][wd] & 0xFFFFu) | (v[3][wd] << 16);
        }
        *reinterpret_cast<u32x2*>(Vl + (8 * chunk + dd) * VS + v_pos) = x;
      }
    }
  };

  const float sl = a.scale_log2;
  float m = -INFINITY;
  float l = 0.f;
  f32x16 o[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[db][r] = 0.f;

  auto compute = [&](int buf, int kt) {
    const __bf16* Kl = lds + buf * BUF;
    const __bf16* Vl = Kl + K_ELEMS;
    f32x16 sacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[kb][r] = 0.f;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x8 ka = *reinterpret_cast<const bf16x8*>(Kl + (32 * kb + l32) * KS + 16 * t + 8 * h2);
        sacc[kb] = mfma(ka, qf[t], sacc[kb]);
      }
    }
    if (kt + KT > wave_kmin) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int j = kt + 32 * kb + 8 * (r >> 2) + 4 * h2 + (r & 3);
          if (j >= Lrow) sacc[kb][r] = -INFINITY;
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][r]);
    mx = max_halves(mx);
    // Lazy rescaling: the running max only moves (and O, l are rescaled) when
    // some row's tile max exceeds it by more than 2^kRescaleLog2 in the exp2
    // domain.  Softmax is exact for any common offset, so a stale max only
    // lets probabilities reach 2^kRescaleLog2 (well inside fp32/bf16 range)
    // and leaves the result unchanged up to rounding.
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
    bf16x8 pb[2][2];
    float ls = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int k16 = 0; k16 < 2; ++k16) {
        u32x4 pk;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p0 = __builtin_amdgcn_exp2f(fmaf(sacc[kb][8 * k16 + 2 * e], sl, -mc));
          const float p1 = __builtin_amdgcn_exp2f(fmaf(sacc[kb][8 * k16 + 2 * e + 1], sl, -mc));
          ls += p0 + p1;
          pk[e] = pack_bf16_rne(p0, p1);
        }
        pb[kb][k16] = __builtin_bit_cast(bf16x8, pk);
      }
    l += ls;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int k16 = 0; k16 < 2; ++k16)
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          const bf16x8 va =
              *reinterpret_cast<const bf16x8*>(Vl + (32 * db + l32) * VS + 32 * kb + 16 * k16 + 8 * h2);
          o[db] = mfma(va, pb[kb][k16], o[db]);
        }
  };

  int buf = 0;
  load_tile(k_begin);
  for (int kt = k_begin; kt < k_end; kt += KT) {
    store_tile(buf);
    __syncthreads();
    if (kt + KT < k_end) load_tile(kt + KT);
    if (kt < wave_kmax) compute(buf, kt);
    buf ^= 1;
  }

  // ---- epilogue
  const float lt = sum_halves(l);
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

// Merges the key splits of one row per wave, in split order.
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  const int64_t total_rows = a.num_q_tokens * a.num_q_heads;
  if (row >= total_rows) return;
  const int64_t t = row / a.num_q_heads;
  const int b = seq_of_token(a.qsl, a.num_seqs, t);
  const int t0 = a.qsl[b];
  const int q_len = a.qsl[b + 1] - t0;
  const int g = a.seq_lens[b] - q_len + static_cast<int>(t - t0);
  const int L = row_limit(a.segments, a.seg_loc[b], a.seg_loc[b + 1], g);
  const int nz = min(a.num_splits, (L + a.split_len - 1) / a.split_len);
  float M = -INFINITY;
  for (int zz = 0; zz < nz; ++zz) M = fmaxf(M, a.ws_ml[(zz * total_rows + row) * 2]);
  float den = 0.f, n0 = 0.f, n1 = 0.f;
  for (int zz = 0; zz < nz; ++zz) {
    const f32x2 ml = *reinterpret_cast<const f32x2*>(a.ws_ml + (zz * total_rows + row) * 2);
    const float wz = __builtin_amdgcn_exp2f((ml[0] - M) * a.scale_log2);
    const f32x2 ov = *reinterpret_cast<const f32x2*>(a.ws_o + (zz * total_rows + row) * D + 2 * lane);
    den = fmaf(wz, ml[1], den);
    n0 = fmaf(wz, ov[0], n0);
    n1 = fmaf(wz, ov[1], n1);
  }
  const float inv = a.v_scale / den;
  uint32_t* orow = reinterpret_cast<uint32_t*>(static_cast<__bf16*>(a.out) + row * D);
  orow[lane] = pack_bf16_rne(n0 * inv, n1 * inv);
}

}  // namespace

hipError_t launch_attn_mfma(const AttnArgs& a, bool kv_fp8, hipStream_t s) {
  const int64_t n = static_cast<int64_t>(a.num_seqs) * a.num_kv_heads * a.num_splits * a.row_tiles;
  if (n <= 0) return hipSuccess;
  if (kv_fp8) {
    hipLaunchKernelGGL(attn_mfma_kernel<true>, dim3(static_cast<unsigned>(n)), dim3(NT), 0, s, a);
  } else {
    hipLaunchKernelGGL(attn_mfma_kernel<false>, dim3(static_cast<unsigned>(n)), dim3(NT), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_attn_combine(const AttnArgs& a, hipStream_t s) {
  const int64_t rows = a.num_q_tokens * a.num_q_heads;
  if (rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(attn_combine_kernel, dim3(static_cast<unsigned>((rows + 3) / 4)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace pkv
