// common.hpp -- device helpers shared by the gfx950 attention kernels.
//
// MFMA operand/accumulator layouts used throughout (CDNA3/CDNA4 32x32 MFMA,
// checked on gfx950 with an in-bounds probe):
//   A (M x K): lane l holds row m = l % 32, a run of K-elements chosen by l / 32
//   B (K x N): lane l holds column n = l % 32, the same K-elements as A
//   D (M x N): lane l, accumulator register r holds
//              row m = 8 * (r / 4) + 4 * (l / 32) + (r % 4), column n = l % 32.
// Because A and B draw the same K-elements from the same lane, only the
// accumulator layout matters for correctness; the K order inside a lane is
// free as long as both operands use it.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ditattn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int kHeadDim = 128;
constexpr float kLog2e = 1.4426950408889634f;

#define DITATTN_LDS __attribute__((address_space(3)))

__device__ __forceinline__ int lane_id() { return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0)); }

// max / sum of x over lanes l and l ^ 32.
__device__ __forceinline__ float half_pair_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// max(a, b, c) in one v_max3_f32.  fmaxf on MFMA results makes the compiler
// canonicalize every operand first (one extra v_max per value); the scores
// here are never signalling NaNs, so the plain instruction is exact.
__device__ __forceinline__ float max3(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// Sum of n values as a balanced tree (independent adds instead of one chain).
template <int N>
__device__ __forceinline__ float tree_sum(const float* x) {
  if constexpr (N == 1) {
    return x[0];
  } else {
    return tree_sum<N / 2>(x) + tree_sum<N - N / 2>(x + N / 2);
  }
}

// ds_read_b64_tr_b16 issued as inline assembly, so the compiler does not
// treat it as aliasing in-flight global->LDS copies of the OTHER buffer and
// insert a vmcnt(0) before it.  The caller must run lds_wait() on the
// results before using them.  `addr` is an LDS byte address.
template <int OFFSET>
__device__ __forceinline__ u32x2 ds_read_tr16_b64(uint32_t addr) {
  u32x2 r;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFFSET) : "memory");
  return r;
}
// ds_read_b128 as inline assembly (see above); `addr` is an LDS byte address.
template <int OFFSET>
__device__ __forceinline__ u32x4 ds_read_b128(uint32_t addr) {
  u32x4 r;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFFSET) : "memory");
  return r;
}
// ds_read_b32 as inline assembly (see above); `addr` is an LDS byte address.
template <int OFFSET>
__device__ __forceinline__ uint32_t ds_read_b32(uint32_t addr) {
  uint32_t r;
  asm volatile("ds_read_b32 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFFSET) : "memory");
  return r;
}
// Wait until at most N LDS operations are outstanding; x depends on the wait.
template <int N>
__device__ __forceinline__ void lds_wait(u32x4& x) {
  static_assert(N >= 0 && N <= 15, "lgkmcnt is 4 bits");
  asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(x) : "i"(N));
}
template <int N>
__device__ __forceinline__ void lds_wait(uint32_t& x) {
  static_assert(N >= 0 && N <= 15, "lgkmcnt is 4 bits");
  asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(x) : "i"(N));
}
// Wait until at most N LDS operations are outstanding; a and b depend on the wait.
template <int N>
__device__ __forceinline__ void lds_wait(u32x4& a, u32x4& b) {
  static_assert(N >= 0 && N <= 15, "lgkmcnt is 4 bits");
  asm volatile("s_waitcnt lgkmcnt(%2)" : "+v"(a), "+v"(b) : "i"(N));
}
// Wait until at most N LDS operations are outstanding and make the given
// registers depend on the wait, so no consumer can be scheduled above it.
template <int N>
__device__ __forceinline__ void lds_wait(u32x2& a, u32x2& b, u32x2& c, u32x2& d, u32x2& e,
                                         u32x2& f, u32x2& g, u32x2& h) {
  static_assert(N >= 0 && N <= 15, "lgkmcnt is 4 bits");
  asm volatile("s_waitcnt lgkmcnt(%8)"
               : "+v"(a), "+v"(b), "+v"(c), "+v"(d), "+v"(e), "+v"(f), "+v"(g), "+v"(h)
               : "i"(N));
}

// Pin a value at this point of the program: the empty volatile asm "changes"
// it, so IR passes cannot sink the computation to a later use.
__device__ __forceinline__ void pin(float& x) { asm volatile("" : "+v"(x)); }
__device__ __forceinline__ void pin(bf16x8& x) { asm volatile("" : "+v"(x)); }
__device__ __forceinline__ void pin(f32x16& x) { asm volatile("" : "+v"(x)); }
__device__ __forceinline__ void pin(i32x16& x) { asm volatile("" : "+v"(x)); }

// Let the last MFMAs writing these accumulators retire before any VALU reads
// them (64 wait states, the full latency of a 16-pass MFMA).  The padding this
// compiler inserts after v_mfma_scale_f32_32x32x64_f8f6f4 is too short, and
// the first epilogue reads then see stale registers.  The accumulators are
// operands, so no read can be scheduled above the wait.
__device__ __forceinline__ void mfma_drain(f32x16& a, f32x16& b, f32x16& c, f32x16& d) {
  asm volatile("s_nop 15\n\ts_nop 15\n\ts_nop 15\n\ts_nop 15" : "+v"(a), "+v"(b), "+v"(c), "+v"(d));
}

__device__ __forceinline__ void mfma_drain(f32x16& a) {
  asm volatile("s_nop 15\n\ts_nop 15\n\ts_nop 15\n\ts_nop 15" : "+v"(a));
}

// Round two fp32 values to BF16 (nearest even) and pack them, low half first.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ f32x16 mfma_bf16_32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ i32x16 mfma_i8_32x32x32(i32x4 a, i32x4 b, i32x16 c) {
  return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c, 0, 0, 0);
}
// E8M0 block scale 2^0 (= 127) held in a VGPR.  Produced by an opaque move so
// the compiler keeps it as a live register operand: when the constant is
// passed directly, this compiler has been seen to reuse the scale register for
// other values in some code paths, which silently rescales rows of the result.
__device__ __forceinline__ int unit_e8m0_scale() {
  int s;
  asm volatile("v_mov_b32 %0, 0x7f" : "=v"(s));
  return s;
}
// FP8 (OCP e4m3) x FP8 -> FP32, 32x32x64, with the given E8M0 block scales
// (pass unit_e8m0_scale() for no scaling).
__device__ __forceinline__ f32x16 mfma_fp8_32x32x64(i32x8 a, i32x8 b, f32x16 c, int scale) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, scale, 0, scale);
}

// Workgroup index remapped so that consecutive logical tiles land on the same
// XCD: the dispatcher deals workgroups round-robin over the 8 XCDs, so
// physical block w runs on XCD w % 8.  Logical tiles [prefix(x), prefix(x+1))
// go to XCD x; tiles of one head then share that XCD's L2 for K/V.
__device__ __forceinline__ int xcd_remap(int w, int n) {
  const int x = w & 7, slot = w >> 3;
  const int q = n >> 3, rem = n & 7;
  return x * q + (x < rem ? x : rem) + slot;
}

}  // namespace ditattn
