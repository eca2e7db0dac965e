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
__device__ __forceinline__ void pin(f32x4& x) { asm volatile("" : "+v"(x)); }
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

__device__ __forceinline__ void mfma_drain(f32x4& a) {
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

// ---------------------------------------------------------------- split tail
// Both attention kernels can run a grid of one workgroup per compute unit: rounds of whole
// query tiles first, then the remaining (query tile, key tile) units cut into equal ranges,
// one per workgroup.  A piece that stops inside its query tile leaves FP32 partials in the
// workgroup's slot of a caller-owned workspace -- per thread of the 8-wave workgroup: its 64
// accumulator values, the running max m and the row sum l -- and raises the slot's flag to
// the call's epoch; the piece that ends at the tile's last key tile merges the partials of the
// lower-numbered workgroups that cover the rest of the tile, lowest first, and writes O.
enum { kSplitFull = 0, kSplitPartial = 1, kSplitOwner = 2 };
constexpr int kSplitSlotRows = 66;      // per thread: 64 accumulator values, m, l
constexpr int kSplitThreads = 512;      // threads of an attention workgroup (8 waves)
constexpr int kSplitRowBytes = kSplitThreads * 4;
// Partials and flags move with system-coherent accesses (sc0 sc1: through to the point of
// coherence of all XCDs, past both cache levels), ordered by vmcnt waits; no cache-wide
// write-back or invalidation, which would evict the K/V tiles the other workgroups stream.
constexpr int kSplitCoherent = 1 | 16;  // cache policy bits sc0, sc1

// Spin on a partial's ready flag (written by a lower-numbered workgroup, which never waits on
// this one); gives up after about a second so that every wave exits whatever happens.
__device__ __forceinline__ bool split_wait_flag(const uint32_t* flag, uint32_t epoch) {
  for (int it = 0; it < (1 << 21); ++it) {
    if (__hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM) == epoch) return true;
    __builtin_amdgcn_s_sleep(8);
  }
  return false;
}

// Workgroup g's slot: kSplitSlotRows rows of kSplitThreads floats (register-major, so every
// access is coalesced and a buffer access keeps the row offset in a scalar).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t split_slot(const float* part, int g) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)(part + (int64_t)g * kSplitSlotRows * kSplitThreads), (short)0,
                                           kSplitSlotRows * kSplitRowBytes, 0x00020000);
}

// This workgroup's partial (acc, m, l of every thread) to its slot, then its flag.
__device__ __forceinline__ void split_write_partial(float* part, uint32_t* flags, uint32_t epoch,
                                                    const f32x16 (&acc)[4], float m, float l) {
  const int tid = threadIdx.x;
  const __amdgpu_buffer_rsrc_t rs = split_slot(part, blockIdx.x);
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r)
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[dt][r]), rs, tid * 4, (16 * dt + r) * kSplitRowBytes,
                                            kSplitCoherent);
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(m), rs, tid * 4, 64 * kSplitRowBytes, kSplitCoherent);
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(l), rs, tid * 4, 65 * kSplitRowBytes, kSplitCoherent);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's stores have completed
  __syncthreads();
  if (tid == 0) __hip_atomic_store(flags + blockIdx.x, epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

// Merge the partials of workgroups p_lo .. p_hi (lowest first) into this thread's (acc, m, l),
// the blocked form's rescale by 2^(m_old - m_new); false when a piece never came.  A workgroup
// whose range of the tail_units units is empty (there are fewer units than workgroups) holds no
// piece and is skipped.
__device__ __forceinline__ bool split_merge(const float* part, const uint32_t* flags, uint32_t epoch, int p_lo,
                                            int p_hi, int64_t tail_units, f32x16 (&acc)[4], float& m, float& l) {
  __shared__ int ready_all;
  const int tid = threadIdx.x;
  const int G = gridDim.x;
  bool ok = true;
  for (int g = p_lo; g <= p_hi; ++g) {
    if (tail_units * g / G == tail_units * (g + 1) / G) continue;  // uniform
    if (tid == 0) ready_all = split_wait_flag(flags + g, epoch) ? 1 : 0;
    __syncthreads();
    ok = ok && ready_all != 0;
    const __amdgpu_buffer_rsrc_t rs = split_slot(part, g);
    const float mp = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, tid * 4, 64 * kSplitRowBytes, kSplitCoherent));
    const float lp = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, tid * 4, 65 * kSplitRowBytes, kSplitCoherent));
    const float mn = fmaxf(m, mp);
    const float sa = m == -INFINITY ? 0.0f : fast_exp2(m - mn);
    const float sb = mp == -INFINITY ? 0.0f : fast_exp2(mp - mn);
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        acc[dt][r] = acc[dt][r] * sa +
                     __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, tid * 4, (16 * dt + r) * kSplitRowBytes,
                                                                          kSplitCoherent)) * sb;
    l = l * sa + lp * sb;
    m = mn;
    __syncthreads();  // ready_all is rewritten for the next piece
  }
  return ok;
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

// The work items of split-tail workgroup blockIdx.x (every query tile has nk key tiles):
// rounds 0 .. rounds-1 give each workgroup whole query tiles; the rest, tail_units (query
// tile, key tile) units, is cut into equal ranges, range g to workgroup g.  A range's pieces
// run last first: the last one, when it stops inside a query tile, is that tile's partial; a
// piece that ends at its tile's last key tile owns the tile and merges the partials of the
// lower workgroups that cover the rest.  run(L, tb, te, mode, p_lo, p_hi) processes key tiles
// [tb, te) of query tile L (tb < 0: its whole key range).
template <typename Run>
__device__ __forceinline__ void split_tail_items(int rounds, int nk, int64_t tail_units, Run&& run) {
  const int G = gridDim.x, g = blockIdx.x;
  const int64_t T = tail_units;
  const int64_t s0 = T * g / G, e0 = T * (g + 1) / G;
  const int base = rounds * G;
  // work items: rounds 0 .. R-1, then the tail pieces from the last query tile down
  const int64_t u_hi = e0 > s0 ? (e0 - 1) / nk : 0, u_lo = s0 / nk;
  const int n_items = rounds + (e0 > s0 ? (int)(u_hi - u_lo + 1) : 0);
  for (int it = 0; it < n_items; ++it) {
    int L, tb = 0, te = nk, mode = kSplitFull, p_lo = 0, p_hi = -1;
    if (it < rounds) {
      L = it * G + xcd_remap(g, G);
    } else {
      const int64_t u = u_hi - (it - rounds);
      const int64_t ub = u * nk;
      tb = (int)((s0 > ub ? s0 : ub) - ub);
      te = (int)((e0 < ub + nk ? e0 : ub + nk) - ub);
      L = base + (int)u;
      if (te < nk) {
        mode = kSplitPartial;
      } else if (tb > 0) {
        mode = kSplitOwner;
        p_hi = g - 1;
        p_lo = g - 1;
        while (p_lo > 0 && T * p_lo / G > ub) --p_lo;  // the workgroup whose range holds ub
      }
    }
    run(L, tb, te, mode, p_lo, p_hi);
    __syncthreads();
  }
}

}  // namespace ditattn
