// launch.hpp -- host launchers behind the C ABI (private to libditattn).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ditattn {

// Query rows per workgroup of the BF16 and Sage kernels.
int bf16_tile_rows();
int sage_tile_rows();

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

}  // namespace ditattn
