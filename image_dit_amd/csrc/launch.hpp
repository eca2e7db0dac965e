// launch.hpp -- host launchers behind the C ABI (private to libditattn).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cstddef>
#include <tuple>
#include <utility>

namespace ditattn {

// Arguments of the BF16 attention kernel.
struct Bf16Args {
  const void *q, *k, *v;  // BF16 [B, S_q, H, 128] and [B, S_kv, H_kv, 128] (k, v)
  void* o;                // BF16 [B, S_q, H, 128]
  int B, S_q, S_kv, H, H_kv;
  float c;                // float(double(scale) * log2(e)), computed once by the caller
  int wl, wr;             // key window (-1 = unbounded on that side)
  int num_qt, n_tiles, reverse;  // filled in by the launcher
  // split tail (sk_grid > 0): workspace flags and partial slots, per-call epoch
  int sk_grid, sk_rounds, sk_nk;
  int64_t sk_tail_units;
  uint32_t* ws_flag;
  float* ws_part;
  uint32_t epoch;
};

// Split-tail plan of an attention call (grid = 0: not split); bytes = workspace it needs.
// Both attention kernels tile alike (256 query rows, 64 keys, 8 waves), so one plan serves both.
struct SplitPlan {
  int grid, rounds, nk;
  int64_t tail_units;
  size_t flag_bytes, bytes;
};
SplitPlan split_tail_plan(int B, int S_q, int S_kv, int H, int wl, int wr);

hipError_t launch_attn_fwd_bf16(const Bf16Args& a, hipStream_t stream);

// Everything sage_prepare / sage_prepare_ex pass to the prepare kernels.
struct PrepareArgs {
  const void *q, *k, *v;  // BF16 [B, S_q, H, 128] and [B, S_kv, H_kv, 128]
  int8_t* q_i8;
  float* q_scale;
  int8_t* k_i8;
  float* k_scale;
  uint8_t* v_fp8;
  float* v_scale;
  int B, S_q, S_kv, H, H_kv;
  float c;                             // float(double(scale) * log2(e))
  const void *q_norm_w, *k_norm_w;     // BF16 [128] or nullptr
  float eps;
  const void *rope_cos, *rope_sin;     // BF16 [>= max(S_q, S_kv), rope_dim]
  int rope_dim;                        // 0 = no RoPE
  float* k_mean;                       // [B, H_kv, 128]: K smoothing on, or nullptr
  void* workspace;                     // >= sage_workspace_bytes(B, S_kv, H_kv) when k_mean
};

hipError_t launch_sage_prepare(const PrepareArgs& a, hipStream_t stream);

// Bytes of workspace the K-smoothing pass needs (fp64 partial channel sums).
size_t sage_workspace_bytes(int B, int S_kv, int H_kv);

hipError_t launch_qk_norm_rope(const void* x, void* out, int B, int S, int H, const void* norm_w,
                               float eps, const void* cos_t, const void* sin_t, int rope_dim,
                               hipStream_t stream);

// Arguments of the Sage attention kernel (tensors as written by the prepare stage).
struct SageArgs {
  const int8_t* q_i8;     // [B, H, S_q_pad, 128]
  const float* q_scale;   // [B, H, S_q_pad / 32]
  const int8_t* k_i8;     // [B, H_kv, S_kv_pad, 128]
  const float* k_scale;   // [B, H_kv, S_kv_pad / 32]
  const uint8_t* v_fp8;   // [B, H_kv, 128, S_kv_pad]
  const float* v_scale;   // [B, H_kv, 128]
  void* o;                // BF16 [B, S_q, H, 128]
  int B, S_q, S_kv, H, H_kv, S_q_pad, S_kv_pad;
  int wl, wr;             // key window (-1 = unbounded on that side)
  int num_qt, n_tiles, reverse;  // filled in by the launcher
  // split tail (sk_grid > 0): workspace flags and partial slots, per-call epoch
  int sk_grid, sk_rounds, sk_nk;
  int64_t sk_tail_units;
  uint32_t* ws_flag;
  float* ws_part;
  uint32_t epoch;
};

hipError_t launch_sage_attn_fwd(const SageArgs& a, hipStream_t stream);

namespace detail {
template <typename K, typename T, std::size_t... I>
hipError_t launch_args(K kernel, dim3 grid, dim3 block, hipStream_t stream, T& args,
                       std::index_sequence<I...>) {
  void* ptrs[] = {static_cast<void*>(&std::get<I>(args))...};
  return hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, ptrs, 0, stream);
}
}  // namespace detail

// Enqueue `kernel` with the arguments converted to its parameter types and
// return the status of this launch itself (hipGetLastError would also report
// an error left behind by an unrelated earlier call).
template <typename... P, typename... A>
hipError_t launch(void (*kernel)(P...), dim3 grid, dim3 block, hipStream_t stream, A... a) {
  static_assert(sizeof...(P) == sizeof...(A), "wrong number of kernel arguments");
  std::tuple<P...> args(static_cast<P>(a)...);
  return detail::launch_args(kernel, grid, block, stream, args, std::index_sequence_for<P...>{});
}

}  // namespace ditattn
