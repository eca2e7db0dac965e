// abi.hip -- the C ABI of libditattn: argument checks, then one launch path.
//
// Every check runs before anything is enqueued, so an argument error leaves
// the outputs untouched.  Nothing here allocates, synchronizes or prints.
#include <math.h>
#include <stdint.h>

#include <atomic>
#include <chrono>

#include "../../include/ditattn.h"
#include "launch.hpp"

// Device scratch of sage_prepare_ex_noalloc (the K-smoothing partial sums).  Each GPU
// the library runs on holds its own copy until the process ends.  In host code the
// name is only a stand-in: kernels get the device address from scratch_address().
static __device__ __align__(256) unsigned char scratch[DITATTN_STATIC_SCRATCH_BYTES];

namespace {

constexpr double kLog2eD = 1.4426950408889634;

bool misaligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

bool overlaps(const void* a, int64_t na, const void* b, int64_t nb) {
  if (!a || !b) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return a0 < b0 + static_cast<uintptr_t>(nb) && b0 < a0 + static_cast<uintptr_t>(na);
}

int64_t padded(int S) { return (static_cast<int64_t>(S) + 255) / 256 * 256; }

// Sizes of one attention problem: queries [B, S_q, H, D], keys/values [B, S_kv, H_kv, D].
// The bounds are the ranges the kernels index in:
//   * B * H * S_pad <= INT32_MAX on either side: tile, block and grid indices are
//     int, and every grid times its workgroup size stays below 2^32 work-items;
//   * H <= DITATTN_MAX_HEADS: the BF16 kernel addresses a K/V tile row as a
//     32-bit byte offset r * H_kv * 256 with r < 64 (63 * 65536 * 256 < 2^32).
int check_sizes(int B, int S_q, int S_kv, int H, int H_kv, int D, float scale) {
  if (B < 1 || S_q < 1 || S_kv < 1 || H < 1 || H_kv < 1) return DITATTN_EINVAL;
  if (!isfinite(scale) || !(scale > 0.0f)) return DITATTN_EINVAL;
  if (H % H_kv != 0) return DITATTN_EINVAL;
  if (D != 128) return DITATTN_EUNSUPPORTED;
  if (H > DITATTN_MAX_HEADS) return DITATTN_EOVERFLOW;
  if (S_q > INT32_MAX - 255 || S_kv > INT32_MAX - 255) return DITATTN_EOVERFLOW;
  if (static_cast<int64_t>(B) * H * padded(S_q) > INT32_MAX) return DITATTN_EOVERFLOW;
  if (static_cast<int64_t>(B) * H_kv * padded(S_kv) > INT32_MAX) return DITATTN_EOVERFLOW;
  return DITATTN_OK;
}

int check_shape(int entry, int B, int S, int H, int D, float scale) {
  const int st = check_sizes(B, S, S, H, H, D, scale);
  if (st != DITATTN_OK) return st;
  switch (entry) {
    case DITATTN_ENTRY_ATTN_FWD_BF16:
    case DITATTN_ENTRY_SAGE_PREPARE: return DITATTN_OK;
    // the Sage kernel addresses a V^T tile row as a 32-bit byte offset c * S_pad, c < 128
    case DITATTN_ENTRY_SAGE_ATTN_FWD: return S > DITATTN_MAX_SEQ_SAGE ? DITATTN_EOVERFLOW : DITATTN_OK;
    default: return DITATTN_EINVAL;
  }
}

// The optional Q/K row transform (RMSNorm weights, RoPE tables).
int check_xform(const void* norm_w0, const void* norm_w1, float eps, const void* cos_t,
                const void* sin_t, int rope_dim) {
  if (!isfinite(eps) || eps < 0.0f) return DITATTN_EINVAL;
  if (rope_dim != 0 && rope_dim != 32 && rope_dim != 64 && rope_dim != 96 && rope_dim != 128)
    return DITATTN_EUNSUPPORTED;
  if (rope_dim && (!cos_t || !sin_t)) return DITATTN_EINVAL;
  if (misaligned(norm_w0) || misaligned(norm_w1)) return DITATTN_EALIGN;
  if (rope_dim && (misaligned(cos_t) || misaligned(sin_t))) return DITATTN_EALIGN;
  return DITATTN_OK;
}

float log2e_scale(float scale) { return static_cast<float>(static_cast<double>(scale) * kLog2eD); }

// Per-call token of the split-tail flags: a flag counts as raised only when it holds this
// call's value, so the workspace needs no clearing between calls.  The numbering starts at a
// point drawn once per process (clock and address bits through a 64-bit mix), so flags a
// workspace still holds from another process's calls do not match this process's tokens.
uint32_t epoch_base() {
  uint64_t x = (uint64_t)std::chrono::steady_clock::now().time_since_epoch().count();
  x ^= (uint64_t)(uintptr_t)&x;  // stack address: differs between processes
  x += 0x9E3779B97F4A7C15ull;    // splitmix64 finalizer
  x = (x ^ (x >> 30)) * 0xBF58476D1CE4E5B9ull;
  x = (x ^ (x >> 27)) * 0x94D049BB133111EBull;
  return (uint32_t)(x ^ (x >> 31));
}
std::atomic<uint32_t> g_epoch{epoch_base()};
uint32_t next_epoch() {
  uint32_t e = g_epoch.fetch_add(1, std::memory_order_relaxed) + 1;
  if (e == 0) e = g_epoch.fetch_add(1, std::memory_order_relaxed) + 1;
  return e;
}

// Device address of `scratch` on the current device, looked up on the first call on each
// device and kept (the lookup allocates nothing; concurrent first calls store the same value).
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];

hipError_t scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return hipSuccess;
}

}  // namespace

extern "C" {

int ditattn_abi_version(void) { return DITATTN_ABI_VERSION; }

const char* ditattn_status_string(int status) {
  switch (status) {
    case DITATTN_OK: return "ok";
    case DITATTN_EINVAL:
      return "invalid argument (size < 1, null pointer, bad scale or eps, H not a multiple of H_kv, "
             "short workspace or aliased output)";
    case DITATTN_EUNSUPPORTED: return "unsupported head dim (only D = 128) or rope_dim (0, 32, 64, 96, 128)";
    case DITATTN_EALIGN: return "pointer not 16-byte aligned";
    case DITATTN_EOVERFLOW: return "size exceeds what the kernels index";
    case DITATTN_EHIP: return "HIP launch failed";
    case DITATTN_ENOSPACE: return "K smoothing needs more scratch than the static buffer holds (DITATTN_STATIC_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

int ditattn_sage_padded_len(int S) {
  if (S < 1 || S > INT32_MAX - 255) return -1;
  return (S + 255) / 256 * 256;
}

int ditattn_check_shape(int entry, int B, int S, int H, int D, float scale) {
  return check_shape(entry, B, S, H, D, scale);
}

size_t ditattn_sage_workspace_size(int B, int S_kv, int H_kv) {
  if (check_sizes(B, S_kv, S_kv, H_kv, H_kv, 128, 1.0f) != DITATTN_OK) return 0;
  return ditattn::sage_workspace_bytes(B, S_kv, H_kv);
}

int attn_fwd_bf16_ex(const void* q, const void* k, const void* v, void* o, int B, int S_q,
                     int S_kv, int H, int H_kv, int D, float scale, int window_left,
                     int window_right, hipStream_t stream) {
  int st = check_sizes(B, S_q, S_kv, H, H_kv, D, scale);
  if (st != DITATTN_OK) return st;
  if (window_left < -1 || window_right < -1) return DITATTN_EINVAL;
  if (!q || !k || !v || !o) return DITATTN_EINVAL;
  if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(o)) return DITATTN_EALIGN;
  const int64_t q_bytes = static_cast<int64_t>(B) * S_q * H * 256;
  const int64_t kv_bytes = static_cast<int64_t>(B) * S_kv * H_kv * 256;
  if (overlaps(o, q_bytes, q, q_bytes) || overlaps(o, q_bytes, k, kv_bytes) ||
      overlaps(o, q_bytes, v, kv_bytes))
    return DITATTN_EINVAL;
  ditattn::Bf16Args a{q, k, v, o, B, S_q, S_kv, H, H_kv, log2e_scale(scale), window_left,
                      window_right, 0, 0, 0};
  if (ditattn::launch_attn_fwd_bf16(a, stream) != hipSuccess) return DITATTN_EHIP;
  return DITATTN_OK;
}

size_t ditattn_bf16_workspace_size(int B, int S_q, int S_kv, int H, int H_kv, int window_left,
                                   int window_right) {
  if (check_sizes(B, S_q, S_kv, H, H_kv, 128, 1.0f) != DITATTN_OK) return 0;
  return ditattn::split_tail_plan(B, S_q, S_kv, H, window_left, window_right).bytes;
}

int attn_fwd_bf16_ws(const void* q, const void* k, const void* v, void* o, int B, int S_q,
                     int S_kv, int H, int H_kv, int D, float scale, int window_left,
                     int window_right, void* workspace, size_t workspace_bytes,
                     hipStream_t stream) {
  int st = check_sizes(B, S_q, S_kv, H, H_kv, D, scale);
  if (st != DITATTN_OK) return st;
  if (window_left < -1 || window_right < -1) return DITATTN_EINVAL;
  if (!q || !k || !v || !o) return DITATTN_EINVAL;
  if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(o)) return DITATTN_EALIGN;
  const int64_t q_bytes = static_cast<int64_t>(B) * S_q * H * 256;
  const int64_t kv_bytes = static_cast<int64_t>(B) * S_kv * H_kv * 256;
  if (overlaps(o, q_bytes, q, q_bytes) || overlaps(o, q_bytes, k, kv_bytes) ||
      overlaps(o, q_bytes, v, kv_bytes))
    return DITATTN_EINVAL;
  ditattn::Bf16Args a{q, k, v, o, B, S_q, S_kv, H, H_kv, log2e_scale(scale), window_left,
                      window_right, 0, 0, 0};
  const ditattn::SplitPlan plan = ditattn::split_tail_plan(B, S_q, S_kv, H, window_left, window_right);
  if (plan.grid > 0) {
    if (!workspace || workspace_bytes < plan.bytes) return DITATTN_EINVAL;
    if (misaligned(workspace)) return DITATTN_EALIGN;
    const int64_t wb = static_cast<int64_t>(plan.bytes);
    if (overlaps(workspace, wb, q, q_bytes) || overlaps(workspace, wb, k, kv_bytes) ||
        overlaps(workspace, wb, v, kv_bytes) || overlaps(workspace, wb, o, q_bytes))
      return DITATTN_EINVAL;
    a.sk_grid = plan.grid;
    a.sk_rounds = plan.rounds;
    a.sk_nk = plan.nk;
    a.sk_tail_units = plan.tail_units;
    a.ws_flag = static_cast<uint32_t*>(workspace);
    a.ws_part = reinterpret_cast<float*>(static_cast<char*>(workspace) + plan.flag_bytes);
    a.epoch = next_epoch();
  }
  if (ditattn::launch_attn_fwd_bf16(a, stream) != hipSuccess) return DITATTN_EHIP;
  return DITATTN_OK;
}

int attn_fwd_bf16(const void* q, const void* k, const void* v, void* o, int B, int S, int H,
                  int D, float scale, hipStream_t stream) {
  return attn_fwd_bf16_ex(q, k, v, o, B, S, S, H, H, D, scale, -1, -1, stream);
}

int sage_prepare_ex(const void* q, const void* k, const void* v, int8_t* q_i8, float* q_scale,
                    int8_t* k_i8, float* k_scale, uint8_t* v_fp8, float* v_scale, int B, int S_q,
                    int S_kv, int H, int H_kv, int D, float scale, const void* q_norm_w,
                    const void* k_norm_w, float norm_eps, const void* rope_cos,
                    const void* rope_sin, int rope_dim, float* k_mean, void* workspace,
                    size_t workspace_bytes, hipStream_t stream) {
  int st = check_sizes(B, S_q, S_kv, H, H_kv, D, scale);
  if (st != DITATTN_OK) return st;
  st = check_xform(q_norm_w, k_norm_w, norm_eps, rope_cos, rope_sin, rope_dim);
  if (st != DITATTN_OK) return st;
  const void* ptrs[9] = {q, k, v, q_i8, q_scale, k_i8, k_scale, v_fp8, v_scale};
  for (const void* p : ptrs)
    if (!p) return DITATTN_EINVAL;
  if (k_mean && !workspace) return DITATTN_EINVAL;
  for (const void* p : ptrs)
    if (misaligned(p)) return DITATTN_EALIGN;
  if (misaligned(k_mean) || misaligned(workspace)) return DITATTN_EALIGN;
  const size_t ws_need = k_mean ? ditattn::sage_workspace_bytes(B, S_kv, H_kv) : 0;
  if (k_mean && workspace_bytes < ws_need) return DITATTN_EINVAL;
  const int64_t sqp = padded(S_q), skp = padded(S_kv);
  const int64_t bhq = static_cast<int64_t>(B) * H, bhk = static_cast<int64_t>(B) * H_kv;
  const int64_t q_bytes = bhq * S_q * 256, kv_bytes = bhk * S_kv * 256;
  void* const outs[8] = {q_i8, q_scale, k_i8, k_scale, v_fp8, v_scale, k_mean, workspace};
  const int64_t out_bytes[8] = {bhq * sqp * 128, bhq * (sqp / 32) * 4, bhk * skp * 128,
                                bhk * (skp / 32) * 4, bhk * skp * 128, bhk * 128 * 4,
                                bhk * 128 * 4, static_cast<int64_t>(ws_need)};
  // the tables have a row per token position up to max(S_q, S_kv); a weight is 256 B
  const int64_t tab = static_cast<int64_t>(S_q > S_kv ? S_q : S_kv) * rope_dim * 2;
  const void* ins[7] = {q, k, v, q_norm_w, k_norm_w, rope_dim ? rope_cos : nullptr,
                        rope_dim ? rope_sin : nullptr};
  const int64_t in_bytes[7] = {q_bytes, kv_bytes, kv_bytes, 256, 256, tab, tab};
  for (int a = 0; a < 8; ++a) {
    for (int i = 0; i < 7; ++i)
      if (overlaps(outs[a], out_bytes[a], ins[i], in_bytes[i])) return DITATTN_EINVAL;
    for (int b2 = a + 1; b2 < 8; ++b2)
      if (overlaps(outs[a], out_bytes[a], outs[b2], out_bytes[b2])) return DITATTN_EINVAL;
  }
  ditattn::PrepareArgs a{q, k, v, q_i8, q_scale, k_i8, k_scale, v_fp8, v_scale,
                         B, S_q, S_kv, H, H_kv, log2e_scale(scale), q_norm_w, k_norm_w, norm_eps,
                         rope_dim ? rope_cos : nullptr, rope_dim ? rope_sin : nullptr, rope_dim,
                         k_mean, workspace};
  if (ditattn::launch_sage_prepare(a, stream) != hipSuccess) return DITATTN_EHIP;
  return DITATTN_OK;
}

int sage_prepare_ex_noalloc(const void* q, const void* k, const void* v, int8_t* q_i8,
                            float* q_scale, int8_t* k_i8, float* k_scale, uint8_t* v_fp8,
                            float* v_scale, int B, int S_q, int S_kv, int H, int H_kv, int D,
                            float scale, const void* q_norm_w, const void* k_norm_w,
                            float norm_eps, const void* rope_cos, const void* rope_sin,
                            int rope_dim, float* k_mean, hipStream_t stream) {
  void* ws = nullptr;
  size_t ws_bytes = 0;
  if (k_mean) {
    // the size check touches no GPU; the shapes themselves are checked by sage_prepare_ex
    const int st = check_sizes(B, S_q, S_kv, H, H_kv, D, scale);
    if (st != DITATTN_OK) return st;
    if (ditattn::sage_workspace_bytes(B, S_kv, H_kv) > DITATTN_STATIC_SCRATCH_BYTES)
      return DITATTN_ENOSPACE;
    if (scratch_address(&ws) != hipSuccess) return DITATTN_EHIP;
    ws_bytes = DITATTN_STATIC_SCRATCH_BYTES;
  }
  return sage_prepare_ex(q, k, v, q_i8, q_scale, k_i8, k_scale, v_fp8, v_scale, B, S_q, S_kv, H,
                         H_kv, D, scale, q_norm_w, k_norm_w, norm_eps, rope_cos, rope_sin,
                         rope_dim, k_mean, ws, ws_bytes, stream);
}

int sage_prepare(const void* q, const void* k, const void* v, int8_t* q_i8, float* q_scale,
                 int8_t* k_i8, float* k_scale, uint8_t* v_fp8, float* v_scale, int B, int S,
                 int H, int D, float scale, hipStream_t stream) {
  return sage_prepare_ex(q, k, v, q_i8, q_scale, k_i8, k_scale, v_fp8, v_scale, B, S, S, H, H, D,
                         scale, nullptr, nullptr, 0.0f, nullptr, nullptr, 0, nullptr, nullptr, 0,
                         stream);
}

int qk_norm_rope_bf16(const void* x, void* out, int B, int S, int H, int D, const void* norm_w,
                      float norm_eps, const void* rope_cos, const void* rope_sin, int rope_dim,
                      hipStream_t stream) {
  int st = check_sizes(B, S, S, H, H, D, 1.0f);
  if (st != DITATTN_OK) return st;
  st = check_xform(norm_w, nullptr, norm_eps, rope_cos, rope_sin, rope_dim);
  if (st != DITATTN_OK) return st;
  if (!x || !out) return DITATTN_EINVAL;
  if (misaligned(x) || misaligned(out)) return DITATTN_EALIGN;
  const int64_t bytes = static_cast<int64_t>(B) * S * H * 256;
  const int64_t tab = static_cast<int64_t>(S) * rope_dim * 2;
  // in place (out == x) is allowed: every row fragment is read before the same lane
  // writes it; any other overlap is not
  if (out != x && overlaps(out, bytes, x, bytes)) return DITATTN_EINVAL;
  if (overlaps(out, bytes, norm_w, 256) || (rope_dim && (overlaps(out, bytes, rope_cos, tab) ||
                                                         overlaps(out, bytes, rope_sin, tab))))
    return DITATTN_EINVAL;
  if (ditattn::launch_qk_norm_rope(x, out, B, S, H, norm_w, norm_eps, rope_dim ? rope_cos : nullptr,
                                   rope_dim ? rope_sin : nullptr, rope_dim, stream) != hipSuccess)
    return DITATTN_EHIP;
  return DITATTN_OK;
}

}  // extern "C"

namespace {
// Argument checks shared by the Sage attention entry points; fills `a` when they pass.
int sage_attn_args(const int8_t* q_i8, const float* q_scale, const int8_t* k_i8, const float* k_scale,
                   const uint8_t* v_fp8, const float* v_scale, void* o, int B, int S_q, int S_kv, int H,
                   int H_kv, int D, float scale, int window_left, int window_right, ditattn::SageArgs& a,
                   int64_t& o_bytes) {
  int st = check_sizes(B, S_q, S_kv, H, H_kv, D, scale);
  if (st != DITATTN_OK) return st;
  if (window_left < -1 || window_right < -1) return DITATTN_EINVAL;
  // the kernel addresses a V^T tile row as a 32-bit byte offset c * S_kv_pad, c < 128
  if (S_kv > DITATTN_MAX_SEQ_SAGE) return DITATTN_EOVERFLOW;
  const void* ptrs[7] = {q_i8, q_scale, k_i8, k_scale, v_fp8, v_scale, o};
  for (const void* p : ptrs)
    if (!p) return DITATTN_EINVAL;
  for (const void* p : ptrs)
    if (misaligned(p)) return DITATTN_EALIGN;
  const int64_t sqp = padded(S_q), skp = padded(S_kv);
  const int64_t bhq = static_cast<int64_t>(B) * H, bhk = static_cast<int64_t>(B) * H_kv;
  const void* ins[6] = {q_i8, q_scale, k_i8, k_scale, v_fp8, v_scale};
  const int64_t in_bytes[6] = {bhq * sqp * 128, bhq * (sqp / 32) * 4, bhk * skp * 128,
                               bhk * (skp / 32) * 4, bhk * skp * 128, bhk * 128 * 4};
  o_bytes = bhq * S_q * 256;
  for (int i = 0; i < 6; ++i)
    if (overlaps(o, o_bytes, ins[i], in_bytes[i])) return DITATTN_EINVAL;
  a = ditattn::SageArgs{q_i8, q_scale, k_i8, k_scale, v_fp8, v_scale, o, B, S_q, S_kv, H, H_kv,
                        static_cast<int>(sqp), static_cast<int>(skp), window_left, window_right,
                        0, 0, 0};
  return DITATTN_OK;
}
}  // namespace

extern "C" {

int sage_attn_fwd_ex(const int8_t* q_i8, const float* q_scale, const int8_t* k_i8,
                     const float* k_scale, const uint8_t* v_fp8, const float* v_scale, void* o,
                     int B, int S_q, int S_kv, int H, int H_kv, int D, float scale,
                     int window_left, int window_right, hipStream_t stream) {
  ditattn::SageArgs a{};
  int64_t o_bytes = 0;
  const int st = sage_attn_args(q_i8, q_scale, k_i8, k_scale, v_fp8, v_scale, o, B, S_q, S_kv, H, H_kv, D,
                                scale, window_left, window_right, a, o_bytes);
  if (st != DITATTN_OK) return st;
  if (ditattn::launch_sage_attn_fwd(a, stream) != hipSuccess) return DITATTN_EHIP;
  return DITATTN_OK;
}

size_t ditattn_sage_attn_workspace_size(int B, int S_q, int S_kv, int H, int H_kv, int window_left,
                                        int window_right) {
  if (check_sizes(B, S_q, S_kv, H, H_kv, 128, 1.0f) != DITATTN_OK) return 0;
  return ditattn::split_tail_plan(B, S_q, S_kv, H, window_left, window_right).bytes;
}

int sage_attn_fwd_ws(const int8_t* q_i8, const float* q_scale, const int8_t* k_i8,
                     const float* k_scale, const uint8_t* v_fp8, const float* v_scale, void* o,
                     int B, int S_q, int S_kv, int H, int H_kv, int D, float scale,
                     int window_left, int window_right, void* workspace, size_t workspace_bytes,
                     hipStream_t stream) {
  ditattn::SageArgs a{};
  int64_t o_bytes = 0;
  const int st = sage_attn_args(q_i8, q_scale, k_i8, k_scale, v_fp8, v_scale, o, B, S_q, S_kv, H, H_kv, D,
                                scale, window_left, window_right, a, o_bytes);
  if (st != DITATTN_OK) return st;
  const ditattn::SplitPlan plan = ditattn::split_tail_plan(B, S_q, S_kv, H, window_left, window_right);
  if (plan.grid > 0) {
    if (!workspace || workspace_bytes < plan.bytes) return DITATTN_EINVAL;
    if (misaligned(workspace)) return DITATTN_EALIGN;
    const int64_t wb = static_cast<int64_t>(plan.bytes);
    const int64_t sqp = padded(S_q), skp = padded(S_kv);
    const int64_t bhq = static_cast<int64_t>(B) * H, bhk = static_cast<int64_t>(B) * H_kv;
    const void* all[7] = {q_i8, q_scale, k_i8, k_scale, v_fp8, v_scale, o};
    const int64_t all_bytes[7] = {bhq * sqp * 128, bhq * (sqp / 32) * 4, bhk * skp * 128,
                                  bhk * (skp / 32) * 4, bhk * skp * 128, bhk * 128 * 4, o_bytes};
    for (int i = 0; i < 7; ++i)
      if (overlaps(workspace, wb, all[i], all_bytes[i])) return DITATTN_EINVAL;
    a.sk_grid = plan.grid;
    a.sk_rounds = plan.rounds;
    a.sk_nk = plan.nk;
    a.sk_tail_units = plan.tail_units;
    a.ws_flag = static_cast<uint32_t*>(workspace);
    a.ws_part = reinterpret_cast<float*>(static_cast<char*>(workspace) + plan.flag_bytes);
    a.epoch = next_epoch();
  }
  if (ditattn::launch_sage_attn_fwd(a, stream) != hipSuccess) return DITATTN_EHIP;
  return DITATTN_OK;
}

int sage_attn_fwd(const int8_t* q_i8, const float* q_scale, const int8_t* k_i8,
                  const float* k_scale, const uint8_t* v_fp8, const float* v_scale, void* o,
                  int B, int S, int H, int D, float scale, hipStream_t stream) {
  return sage_attn_fwd_ex(q_i8, q_scale, k_i8, k_scale, v_fp8, v_scale, o, B, S, S, H, H, D, scale,
                          -1, -1, stream);
}

}  // extern "C"
