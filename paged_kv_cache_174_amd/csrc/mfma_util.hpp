// Device building blocks shared by the gfx950 attention kernels: operand
// types, direct global-to-LDS loads, the fence-free LDS barrier, exact
// vmcnt waits, the 32x32x16 bf16 MFMA, cross-half row reductions, bf16 and
// e4m3 conversions, and the LDS chunk permutations of the K/V tiles.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace pkv {
namespace mx {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef int v2i32 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void* lds_ptr;
typedef __attribute__((address_space(3))) v4i16* lds_v4i16_ptr;
typedef __attribute__((address_space(3))) v2i32* lds_v2i32_ptr;

constexpr int D = 128;                  // head_dim of the MFMA kernels
constexpr int kRowBytes = D * 2;        // one bf16 K or V row of an LDS tile
constexpr int kTileKeys = 64;           // keys per bf16 tile
constexpr int kTileBytes = kTileKeys * kRowBytes;  // 16 KB

// LDS byte address of p, hidden from the optimiser: addresses built as
// opaque base + constant keep the constant (buffer, key block) in the 16-bit
// offset field of the LDS instruction instead of an add per read.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  uint32_t a = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_ptr)p));
  asm volatile("" : "+v"(a));
  return a;
}
template <typename T>
__device__ __forceinline__ const __attribute__((address_space(3))) T* lds_at(uint32_t a) {
  return (const __attribute__((address_space(3))) T*)(static_cast<uintptr_t>(a));
}
__device__ __forceinline__ lds_v4i16_ptr lds_v4i16(uint32_t a) { return (lds_v4i16_ptr)(static_cast<uintptr_t>(a)); }
__device__ __forceinline__ lds_v2i32_ptr lds_v2i32(uint32_t a) { return (lds_v2i32_ptr)(static_cast<uintptr_t>(a)); }

// One 16-byte-per-lane direct global-to-LDS load: lane i's 16 bytes from g
// land at l + 16 i (l is wave-uniform, passed in M0).  Issued as inline
// assembly so that the compiler does not add waits of its own for it: the
// kernels wait for these loads explicitly (wait_vmcnt) before the barrier
// that precedes their first reader.
//
// The compiler does not look inside inline assembly for hazards, so the
// statement carries its own wait states: a vector memory instruction that
// reads an SGPR written by a VALU instruction (v_readfirstlane, which makes
// the wave-uniform bases and descriptors) needs five, and an LDS DMA needs
// one after M0 is written.  Without them the load may use a stale address.
#define PKV_VMEM_SGPR_WAIT "s_nop 4\n"
__device__ __forceinline__ void dma16(const void* g, const void* l) {
  const uint32_t m0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_ptr)l));
  asm volatile(PKV_VMEM_SGPR_WAIT "global_load_lds_dwordx4 %0, off" ::"v"(g), "{m0}"(m0));
}
// The same with a wave-uniform base address in SGPRs and a per-lane 32-bit
// byte offset, so the address takes no vector arithmetic.
__device__ __forceinline__ void dma16(const uint8_t* base, uint32_t off, const void* l) {
  const uint32_t m0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_ptr)l));
  asm volatile(PKV_VMEM_SGPR_WAIT "global_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base), "{m0}"(m0));
}

// Workgroup barrier for the K/V tile pipelines.  __syncthreads() -- and any
// release fence on LDS -- makes every wave wait for all of its outstanding
// vector-memory loads, including the direct-to-LDS loads of tiles that are
// only read iterations later, which would drain the prefetch at every tile.
// Here each wave waits for its own LDS accesses (lgkmcnt) and, before calling
// this, for exactly the direct loads the next phase reads (wait_vmcnt); the
// empty asm statements keep the compiler from moving memory accesses across
// the barrier.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt not waited on
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

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
// The 16x16x32 bf16 MFMA (half the matrix work of the 32x32x16 one).
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
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

// Chunk permutation of bf16 LDS tile rows.  The LDS serves 256 bytes per
// clock from 64 four-byte banks, and a 256-byte row maps onto all of them, so
// the 16-byte chunk c of row r is stored at position c ^ swz(r):
//   K: the MFMA reads one chunk from 16 consecutive rows per clock -> XOR with
//      r mod 16 puts them in 16 distinct positions;
//   V: a transposing read takes four consecutive rows x 64 bytes (four
//      chunks 4 k .. 4 k + 3) per clock -> XOR with 4 (r mod 4) moves each row
//      to its own 64-byte quarter.
__device__ __forceinline__ int k_swz(int r) { return r & 15; }
__device__ __forceinline__ int v_swz(int r) { return 4 * (r & 3); }

}  // namespace mx
}  // namespace pkv
