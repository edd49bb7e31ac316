// fp32 paged attention (fp32 queries over fp32 pools).
//
// One wavefront per (query row, query head); the 64 lanes take 64 keys at a
// time for the logits and the head dimension for the weighted sum.  Softmax is
// the online (running max / running sum) form, exact fp32 throughout.  This is
// the path for full-precision pools; the bf16/fp8 pools use the MFMA kernel.
#include "attn_common.hpp"

namespace pkv {
namespace {

constexpr int kWaves = 4;

template <int D>
__global__ __launch_bounds__(64 * kWaves) void attn_f32_kernel(AttnArgs a) {
  constexpr int ND = D / 64;  // head-dim elements per lane
  __shared__ float qs[kWaves][D];
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int b = blockIdx.z;
  const int h = blockIdx.y;
  const int t0 = a.qsl[b];
  const int q_len = a.qsl[b + 1] - t0;
  const int i = blockIdx.x * kWaves + w;
  if (i >= q_len) return;  // whole wave leaves; no block-level barrier below
  const int s = a.seq_lens[b];
  const int g = (a.query_pos ? a.query_pos[b] : s - q_len) + i;  // the row's key position
  const int L = row_limit(a.segments, a.seg_loc[b], a.seg_loc[b + 1], g);
  const int hk = h / a.group;
  const int64_t row_elems = static_cast<int64_t>(a.num_kv_heads) * D;
  const float* q = static_cast<const float*>(a.q) + (static_cast<int64_t>(t0 + i) * a.num_q_heads + h) * D;
  const float* kp = static_cast<const float*>(a.kpool) + static_cast<int64_t>(hk) * D;
  const float* vp = static_cast<const float*>(a.vpool) + static_cast<int64_t>(hk) * D;
  // No table: the K/V buffers are one contiguous run (logical block i is block i).
  const int32_t* table = a.block_table ? a.block_table + static_cast<int64_t>(b) * a.table_width : nullptr;
  const int B = a.block_size;

  for (int d = lane; d < D; d += 64) qs[w][d] = q[d];
  __builtin_amdgcn_wave_barrier();  // the wave's own LDS writes precede its reads

  float m = -INFINITY, l = 0.f;
  float o[ND];
#pragma unroll
  for (int k = 0; k < ND; ++k) o[k] = 0.f;
  const float sc = a.scale_log2;  // softmax_scale * log2(e)

  for (int j0 = 0; j0 < L; j0 += 64) {
    const int j = j0 + lane;
    float z = -INFINITY;
    int64_t slot = 0;
    if (j < L) {
      slot = table ? static_cast<int64_t>(table[j / B]) * B + (j % B) : j;
      const float* kr = kp + slot * row_elems;
      float acc = 0.f;
      for (int d = 0; d < D; ++d) acc = fmaf(qs[w][d], kr[d], acc);
      z = acc;
    }
    float mx = z;
    for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
    const float m_new = fmaxf(m, mx);
    const float alpha = exp2f((m - m_new) * sc);  // m = -inf on the first tile -> 0
    const float p = (j < L) ? exp2f((z - m_new) * sc) : 0.f;
    float ps = p;
    for (int off = 32; off > 0; off >>= 1) ps += __shfl_xor(ps, off);
    l = l * alpha + ps;
    m = m_new;
#pragma unroll
    for (int k = 0; k < ND; ++k) o[k] *= alpha;
    const int n = min(64, L - j0);
    for (int jj = 0; jj < n; ++jj) {
      const float pj = __shfl(p, jj);
      const int64_t sj = __shfl(slot, jj);
      const float* vr = vp + sj * row_elems;
#pragma unroll
      for (int k = 0; k < ND; ++k) o[k] = fmaf(pj, vr[lane + 64 * k], o[k]);
    }
  }
  float* out = static_cast<float*>(a.out) + (static_cast<int64_t>(t0 + i) * a.num_q_heads + h) * D;
  const float inv = 1.f / l;
#pragma unroll
  for (int k = 0; k < ND; ++k) out[lane + 64 * k] = o[k] * inv;
}

}  // namespace

hipError_t launch_attn_f32(const AttnArgs& a, int max_query_len, hipStream_t s) {
  dim3 grid((max_query_len + kWaves - 1) / kWaves, a.num_q_heads, a.num_seqs);
  if (a.head_dim == 64) {
    hipLaunchKernelGGL(attn_f32_kernel<64>, grid, dim3(64 * kWaves), 0, s, a);
  } else {
    hipLaunchKernelGGL(attn_f32_kernel<128>, grid, dim3(64 * kWaves), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace pkv
