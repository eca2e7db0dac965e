// abi.hip -- the C ABI of libditattn: argument checks, then one launch path.
//
// Every check runs before anything is enqueued, so an argument error leaves
// the outputs untouched.  Nothing here allocates, synchronizes or prints.
#include <math.h>
#include <stdint.h>

#include "../../include/ditattn.h"
#include "launch.hpp"

namespace {

constexpr double kLog2eD = 1.4426950408889634;

bool misaligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

bool overlaps(const void* a, int64_t na, const void* b, int64_t nb) {
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return a0 < b0 + static_cast<uintptr_t>(nb) && b0 < a0 + static_cast<uintptr_t>(na);
}

// Shared shape checks.  On success *elems = B * S * H * 128 and *s_pad = S_pad.
// The bounds are the ranges the kernels index in:
//   * B * H * S_pad <= INT32_MAX: tile, block and grid indices are int, and
//     every grid times its workgroup size stays below 2^32 work-items;
//   * H <= DITATTN_MAX_HEADS: the BF16 kernel addresses a K/V tile row as a
//     32-bit byte offset r * H * 256 with r < 64 (63 * 65536 * 256 < 2^32).
int check_shape(int B, int S, int H, int D, float scale, int64_t* elems, int* s_pad) {
  if (B < 1 || S < 1 || H < 1) return DITATTN_EINVAL;
  if (!isfinite(scale) || !(scale > 0.0f)) return DITATTN_EINVAL;
  if (D != 128) return DITATTN_EUNSUPPORTED;
  if (H > DITATTN_MAX_HEADS) return DITATTN_EOVERFLOW;
  if (S > (INT32_MAX - 255)) return DITATTN_EOVERFLOW;
  const int64_t sp = (static_cast<int64_t>(S) + 255) / 256 * 256;
  const int64_t bh = static_cast<int64_t>(B) * H;  // < 2^31 * 2^16: no int64 overflow
  if (bh * sp > INT32_MAX) return DITATTN_EOVERFLOW;
  *elems = bh * S * 128;
  *s_pad = static_cast<int>(sp);
  return DITATTN_OK;
}

float log2e_scale(float scale) { return static_cast<float>(static_cast<double>(scale) * kLog2eD); }

}  // namespace

extern "C" {

int ditattn_abi_version(void) { return DITATTN_ABI_VERSION; }

const char* ditattn_status_string(int status) {
  switch (status) {
    case DITATTN_OK: return "ok";
    case DITATTN_EINVAL: return "invalid argument (size < 1, null pointer, bad scale or aliased output)";
    case DITATTN_EUNSUPPORTED: return "unsupported head dim (only D = 128)";
    case DITATTN_EALIGN: return "pointer not 16-byte aligned";
    case DITATTN_EOVERFLOW: return "size exceeds what the kernels index";
    case DITATTN_EHIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

int ditattn_sage_padded_len(int S) {
  if (S < 1 || S > INT32_MAX - 255) return -1;
  return (S + 255) / 256 * 256;
}

int ditattn_check_shape(int entry, int B, int S, int H, int D, float scale) {
  int64_t elems;
  int s_pad;
  int st = check_shape(B, S, H, D, scale, &elems, &s_pad);
  if (st != DITATTN_OK) return st;
  switch (entry) {
    case DITATTN_ENTRY_ATTN_FWD_BF16:
    case DITATTN_ENTRY_SAGE_PREPARE: return DITATTN_OK;
    case DITATTN_ENTRY_SAGE_ATTN_FWD: return S > DITATTN_MAX_SEQ_SAGE ? DITATTN_EOVERFLOW : DITATTN_OK;
    default: return DITATTN_EINVAL;
  }
}

int attn_fwd_bf16(const void* q, const void* k, const void* v, void* o, int B, int S, int H,
                  int D, float scale, hipStream_t stream) {
  int64_t elems;
  int s_pad;
  int st = check_shape(B, S, H, D, scale, &elems, &s_pad);
  if (st != DITATTN_OK) return st;
  if (!q || !k || !v || !o) return DITATTN_EINVAL;
  if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(o)) return DITATTN_EALIGN;
  const int64_t bytes = elems * 2;
  if (overlaps(o, bytes, q, bytes) || overlaps(o, bytes, k, bytes) || overlaps(o, bytes, v, bytes))
    return DITATTN_EINVAL;
  if (ditattn::launch_attn_fwd_bf16(q, k, v, o, B, S, H, log2e_scale(scale), stream) != hipSuccess)
    return DITATTN_EHIP;
  return DITATTN_OK;
}

int sage_prepare(const void* q, const void* k, const void* v, int8_t* q_i8, float* q_scale,
                 int8_t* k_i8, float* k_scale, uint8_t* v_fp8, float* v_scale, int B, int S,
                 int H, int D, float scale, hipStream_t stream) {
  int64_t elems;
  int s_pad;
  int st = check_shape(B, S, H, D, scale, &elems, &s_pad);
  if (st != DITATTN_OK) return st;
  const void* ptrs[9] = {q, k, v, q_i8, q_scale, k_i8, k_scale, v_fp8, v_scale};
  for (const void* p : ptrs)
    if (!p) return DITATTN_EINVAL;
  for (const void* p : ptrs)
    if (misaligned(p)) return DITATTN_EALIGN;
  const int64_t bh = static_cast<int64_t>(B) * H;
  const int64_t in_bytes = elems * 2;
  const int64_t code_bytes = bh * s_pad * 128;
  const int64_t qk_scale_bytes = bh * (s_pad / 32) * 4;
  const int64_t v_scale_bytes = bh * 128 * 4;
  const void* outs[6] = {q_i8, q_scale, k_i8, k_scale, v_fp8, v_scale};
  const int64_t out_bytes[6] = {code_bytes, qk_scale_bytes, code_bytes, qk_scale_bytes, code_bytes, v_scale_bytes};
  const void* ins[3] = {q, k, v};
  for (int a = 0; a < 6; ++a) {
    for (int i = 0; i < 3; ++i)
      if (overlaps(outs[a], out_bytes[a], ins[i], in_bytes)) return DITATTN_EINVAL;
    for (int b2 = a + 1; b2 < 6; ++b2)
      if (overlaps(outs[a], out_bytes[a], outs[b2], out_bytes[b2])) return DITATTN_EINVAL;
  }
  if (ditattn::launch_sage_prepare(q, k, v, q_i8, q_scale, k_i8, k_scale, v_fp8, v_scale, B, S, H,
                                   s_pad, log2e_scale(scale), stream) != hipSuccess)
    return DITATTN_EHIP;
  return DITATTN_OK;
}

int sage_attn_fwd(const int8_t* q_i8, const float* q_scale, const int8_t* k_i8,
                  const float* k_scale, const uint8_t* v_fp8, const float* v_scale, void* o,
                  int B, int S, int H, int D, float scale, hipStream_t stream) {
  int64_t elems;
  int s_pad;
  int st = check_shape(B, S, H, D, scale, &elems, &s_pad);
  if (st != DITATTN_OK) return st;
  // the kernel addresses a V^T tile row as a 32-bit byte offset c * S_pad, c < 128
  if (S > DITATTN_MAX_SEQ_SAGE) return DITATTN_EOVERFLOW;
  const void* ptrs[7] = {q_i8, q_scale, k_i8, k_scale, v_fp8, v_scale, o};
  for (const void* p : ptrs)
    if (!p) return DITATTN_EINVAL;
  for (const void* p : ptrs)
    if (misaligned(p)) return DITATTN_EALIGN;
  const int64_t bh = static_cast<int64_t>(B) * H;
  const int64_t code_bytes = bh * s_pad * 128;
  const int64_t qk_scale_bytes = bh * (s_pad / 32) * 4;
  const int64_t v_scale_bytes = bh * 128 * 4;
  const void* ins[6] = {q_i8, q_scale, k_i8, k_scale, v_fp8, v_scale};
  const int64_t in_bytes[6] = {code_bytes, qk_scale_bytes, code_bytes, qk_scale_bytes, code_bytes, v_scale_bytes};
  for (int i = 0; i < 6; ++i)
    if (overlaps(o, elems * 2, ins[i], in_bytes[i])) return DITATTN_EINVAL;
  if (ditattn::launch_sage_attn_fwd(q_i8, q_scale, k_i8, k_scale, v_fp8, v_scale, o, B, S, H,
                                    s_pad, stream) != hipSuccess)
    return DITATTN_EHIP;
  return DITATTN_OK;
}

}  // extern "C"
