// Slot-mapping scatter (the paged K/V write) and the history-staging block
// gather.  Both are pure data movement, bound by HBM bandwidth: every thread
// moves 16-byte vectors, consecutive threads consecutive vectors of one token
// row (a pool slot is one contiguous row of num_kv_heads * head_dim elements).
#include "pkv_internal.hpp"

namespace pkv {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;

// fp32 -> OCP e4m3fn code: round to nearest, ties to even, saturate to +-448,
// keep the sign of zero, NaN -> NaN.  Done in integer arithmetic on the fp32
// bit pattern so the rounding is exactly the one stated, whatever the
// hardware conversion's mode bits are.
__device__ __forceinline__ uint32_t f32_to_e4m3(float x) {
  const uint32_t u = __float_as_uint(x);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7FFFFFFFu;
  if (a > 0x7F800000u) return sign | 0x7Fu;  // NaN
  if (a >= 0x43E00000u) return sign | 0x7Eu;  // >= 448 (and inf): saturate
  if (a < 0x3C800000u) {                      // below 2^-6: subnormal codes m * 2^-9
    // a * 2^9 is exact; rint rounds half to even; the result 8 is the
    // smallest normal (code 0x08), so no special case is needed.
    const float m = __builtin_rintf(__uint_as_float(a) * 512.0f);
    return sign | static_cast<uint32_t>(m);
  }
  // Normal: keep 3 mantissa bits with round-half-even on the 20 dropped bits;
  // a carry out of the mantissa correctly bumps the exponent.
  const uint32_t r = a + 0x7FFFFu + ((a >> 20) & 1u);
  return sign | ((r >> 20) - (120u << 3));
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// One token row per workgroup (grid-striding over rows), one 16-byte source
// vector per thread; blockIdx.y selects K (0) or V (1).  The row's slot is a
// wave-uniform load, and no per-element index division is needed.
template <int MODE>
__global__ __launch_bounds__(kThreads) void write_kernel(WriteArgs a, int vecs_per_row) {
  const bool is_v = blockIdx.y != 0;
  const uint8_t* __restrict__ src = static_cast<const uint8_t*>(is_v ? a.value : a.key);
  uint8_t* __restrict__ dst = static_cast<uint8_t*>(is_v ? a.vpool : a.kpool);
  const float inv = is_v ? a.v_inv_scale : a.k_inv_scale;
  // bytes of one row in the source and in the pool
  const int64_t src_row = static_cast<int64_t>(vecs_per_row) * 16;
  const int64_t dst_row = (MODE == 2) ? static_cast<int64_t>(vecs_per_row) * 8 : src_row;
  for (int64_t t = blockIdx.x; t < a.num_tokens; t += gridDim.x) {
    const int64_t slot = a.slots[t];
    const uint8_t* srow = src + t * src_row;
    uint8_t* drow = dst + slot * dst_row;
    for (int c = threadIdx.x; c < vecs_per_row; c += kThreads) {
      const u32x4 x = *reinterpret_cast<const u32x4*>(srow + 16 * c);
      if (MODE == 2) {
        uint32_t q[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          q[2 * i] = f32_to_e4m3(bf16_lo(x[i]) * inv);
          q[2 * i + 1] = f32_to_e4m3(bf16_hi(x[i]) * inv);
        }
        u32x2 y;
        y[0] = q[0] | (q[1] << 8) | (q[2] << 16) | (q[3] << 24);
        y[1] = q[4] | (q[5] << 8) | (q[6] << 16) | (q[7] << 24);
        *reinterpret_cast<u32x2*>(drow + 8 * c) = y;
      } else {
        *reinterpret_cast<u32x4*>(drow + 16 * c) = x;
      }
    }
  }
}

// One workgroup per (block row, K|V): copies block_bytes with 16-byte vectors.
__global__ __launch_bounds__(kThreads) void gather_kernel(GatherArgs a) {
  const int i = a.first_block + static_cast<int>(blockIdx.x);
  const bool is_v = blockIdx.y != 0;
  const int64_t blk = a.block_ids[i];
  const uint8_t* src = static_cast<const uint8_t*>(is_v ? a.vpool : a.kpool) + blk * a.block_bytes;
  uint8_t* dst = static_cast<uint8_t*>(is_v ? a.vstage : a.kstage) + static_cast<int64_t>(i) * a.block_bytes;
  const int64_t nvec = a.block_bytes / 16;
  for (int64_t v = threadIdx.x; v < nvec; v += kThreads) {
    reinterpret_cast<u32x4*>(dst)[v] = reinterpret_cast<const u32x4*>(src)[v];
  }
}

}  // namespace

hipError_t launch_write(const WriteArgs& a, int mode, hipStream_t s) {
  if (a.num_tokens == 0) return hipSuccess;
  const int64_t elem = (mode == 0) ? 4 : 2;  // source element size
  const int64_t vecs_per_row = a.row_elems * elem / 16;
  if (vecs_per_row <= 0 || vecs_per_row > (1 << 24)) return hipErrorInvalidValue;
  const int64_t blocks = a.num_tokens < 65535 ? a.num_tokens : 65535;  // grid-stride over rows beyond
  dim3 grid(static_cast<unsigned>(blocks), 2);
  const int vpr = static_cast<int>(vecs_per_row);
  switch (mode) {
    case 0: hipLaunchKernelGGL(write_kernel<0>, grid, dim3(kThreads), 0, s, a, vpr); break;
    case 1: hipLaunchKernelGGL(write_kernel<1>, grid, dim3(kThreads), 0, s, a, vpr); break;
    default: hipLaunchKernelGGL(write_kernel<2>, grid, dim3(kThreads), 0, s, a, vpr); break;
  }
  return hipGetLastError();
}

hipError_t launch_gather(const GatherArgs& a, hipStream_t s) {
  const int n = a.n_blocks - a.first_block;
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(gather_kernel, dim3(n, 2), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace pkv
