// launch.hpp -- host launchers behind the C ABI (private to libditattn).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cstddef>
#include <tuple>
#include <utility>

namespace ditattn {

// c = float(double(scale) * log2(e)) is computed once by the caller.
hipError_t launch_attn_fwd_bf16(const void* q, const void* k, const void* v, void* o, int B,
                                int S, int H, float c, hipStream_t stream);

hipError_t launch_sage_prepare(const void* q, const void* k, const void* v, int8_t* q_i8,
                               float* q_scale, int8_t* k_i8, float* k_scale, uint8_t* v_fp8,
                               float* v_scale, int B, int S, int H, int S_pad, float c,
                               hipStream_t stream);

hipError_t launch_sage_attn_fwd(const int8_t* q_i8, const float* q_scale, const int8_t* k_i8,
                                const float* k_scale, const uint8_t* v_fp8, const float* v_scale,
                                void* o, int B, int S, int H, int S_pad, hipStream_t stream);

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
