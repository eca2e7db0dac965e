/*
 * ditattn.h -- C ABI of the MI355X (gfx950) DiT flash self-attention library
 * (libditattn.so).
 *
 * Non-causal self-attention forward at head dim 128, as used by diffusion
 * transformers, in two modes:
 *   - BF16: both GEMMs in BF16 on MFMA, FP32 accumulation, online softmax.
 *   - Sage: a prepare stage quantizes Q/K to INT8 and V to FP8 e4m3; Q.K^T
 *     then runs on INT8 MFMA and P.V on FP8 MFMA, FP32 accumulation.
 *
 * Sources of the operations (page title, section):
 *   [FA]   "Kernel acceleration: attention, compilation and fusion",
 *          section "Attention: from O(N^2) memory to blocks": attention
 *          computed block by block with a running max and sum (online
 *          softmax), never writing the N x N score matrix.
 *   [SAGE] "gfx1201_sage_prepare / gfx1201_sage_attention" (aiter PR 6390),
 *          sections "Technical Details" and the two commit messages: the
 *          prepare stage and the quantized forward, non-causal, head dim 128,
 *          no mask or varlen, BF16 in and out, forward only.
 *   [RDNA] "RDNAttention" README, sections "Overview" and "Quick start": the
 *          layer above the kernels only passes the addresses of tensors that
 *          already live on the GPU; it copies nothing and opens no GPU context
 *          of its own.
 *
 * Conventions shared by every entry point
 *   - Pointers are DEVICE pointers owned by the caller.  The library
 *     allocates nothing, keeps no state between calls and is thread-safe.
 *   - Tensors are contiguous.  BF16 tensors q, k, v, o are [B, S, H, D]
 *     (token-major, head next, channel fastest), 2 bytes per element.
 *   - D must be 128.  B, S, H must be >= 1.  Size limits (larger shapes
 *     return DITATTN_EOVERFLOW before anything is enqueued):
 *       H <= DITATTN_MAX_HEADS, B * H * S_pad <= INT32_MAX, and for
 *       sage_attn_fwd also S <= DITATTN_MAX_SEQ_SAGE.
 *   - Every pointer must be 16-byte aligned.
 *   - Each call only enqueues work on `stream` (0 = the null stream) and
 *     returns; results are valid once the stream has reached that point.
 *     Nothing synchronizes the device.
 *   - Errors are returned, never raised, printed or aborted on.  Arguments are
 *     checked before anything is enqueued: an argument error leaves every
 *     output untouched.  DITATTN_EHIP reports a failed launch (the HIP error
 *     is cleared with hipGetLastError; outputs are then undefined).
 *   - Padded length: S_pad = ditattn_sage_padded_len(S) = S rounded up to a
 *     multiple of 256.
 */
#ifndef DITATTN_H
#define DITATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Same definition as the HIP runtime's, so both headers can be included. */
struct ihipStream_t;
typedef struct ihipStream_t* hipStream_t;

#define DITATTN_ABI_VERSION 2

/* Size limits (see the conventions above). */
#define DITATTN_MAX_HEADS 65536
#define DITATTN_MAX_SEQ_SAGE (1 << 25)
/* Size of the library's static device scratch (sage_prepare_ex_noalloc). */
#define DITATTN_STATIC_SCRATCH_BYTES (16u << 20)

/* Status codes. */
#define DITATTN_OK 0
#define DITATTN_EINVAL (-1)       /* a size < 1, null pointer, scale not finite or <= 0, bad eps,
                                     H not a multiple of H_kv, short workspace, output aliasing an input */
#define DITATTN_EUNSUPPORTED (-2) /* D != 128, rope_dim not 0/32/64/96/128 */
#define DITATTN_EALIGN (-3)       /* a pointer is not 16-byte aligned */
#define DITATTN_EOVERFLOW (-4)    /* a byte size or the grid exceeds what the kernels index */
#define DITATTN_EHIP (-5)         /* the HIP runtime rejected a launch */
#define DITATTN_ENOSPACE (-6)     /* sage_prepare_ex_noalloc: scratch needed > DITATTN_STATIC_SCRATCH_BYTES */

/* DITATTN_ABI_VERSION of the loaded library. */
int ditattn_abi_version(void);

/* Static, never-NULL description of a status code. */
const char* ditattn_status_string(int status);

/* S rounded up to a multiple of 256 (the token length of prepared tensors);
 * -1 if S < 1 or the result overflows int. */
int ditattn_sage_padded_len(int S);

/* Entry points, for ditattn_check_shape. */
#define DITATTN_ENTRY_ATTN_FWD_BF16 0
#define DITATTN_ENTRY_SAGE_PREPARE 1
#define DITATTN_ENTRY_SAGE_ATTN_FWD 2

/* The status the given entry point returns for these sizes and scale before
 * it looks at any pointer (DITATTN_OK, DITATTN_EINVAL, DITATTN_EUNSUPPORTED or
 * DITATTN_EOVERFLOW); DITATTN_EINVAL for an unknown entry.  Touches no GPU. */
int ditattn_check_shape(int entry, int B, int S, int H, int D, float scale);

/*
 * attn_fwd_bf16 -- o = softmax(q k^T * scale) v per (batch, head), non-causal.
 * [FA] (tiled online softmax); [SAGE] "Technical Details" (shape contract:
 * BF16 [B, S, H, 128] in and out, non-causal, no mask).
 *   q, k, v : const BF16 [B, S, H, 128]
 *   o       : BF16 [B, S, H, 128], written in full; must not overlap q, k or v
 *   scale   : softmax scale (e.g. 1/sqrt(128)), finite and > 0
 * Softmax runs in FP32 in base 2 (scores times scale * log2(e)); P is rounded
 * to BF16 for the second GEMM; the row sum uses the FP32 values.
 */
int attn_fwd_bf16(const void* q, const void* k, const void* v, void* o, int B, int S, int H,
                  int D, float scale, hipStream_t stream);

/*
 * attn_fwd_bf16_ex -- attn_fwd_bf16 for cross-attention, grouped-query heads and
 * a key window ("RDNAttention" README, "Features": cross-attention and decode
 * with seq_len != key_seq_len, GQA/MQA, causal masking, one- or two-sided
 * sliding window).
 *   q, o    : BF16 [B, S_q, H, 128];  k, v : BF16 [B, S_kv, H_kv, 128]
 *   H must be a multiple of H_kv; query head h reads key/value head h / (H / H_kv).
 *   Query i sees key j when lo(i) <= j <= hi(i), with off = S_kv - S_q (queries
 *   aligned to the END of the keys, so a decode step S_q = 1 sees every key):
 *     lo(i) = i + off - window_left   (no lower bound when window_left == -1)
 *     hi(i) = i + off + window_right  (no upper bound when window_right == -1)
 *   (-1, -1) is full attention, (-1, 0) causal, (w, 0) a one-sided and (w, w)
 *   a two-sided sliding window.  Other negative values are DITATTN_EINVAL.
 *   A query row that sees no key is written as zeros.
 * attn_fwd_bf16(...) equals attn_fwd_bf16_ex(..., S, S, H, H, ..., -1, -1, ...).
 */
int attn_fwd_bf16_ex(const void* q, const void* k, const void* v, void* o, int B, int S_q,
                     int S_kv, int H, int H_kv, int D, float scale, int window_left,
                     int window_right, hipStream_t stream);

/*
 * sage_prepare -- quantize BF16 Q, K, V for sage_attn_fwd.  [SAGE] first
 * commit and "Technical Details" (Q/K to INT8 with one FP32 scale per
 * (batch, head, 32-row block), Q carrying scale * log2(e); V to FP8 e4m3
 * with one FP32 scale per channel, transposed to [B, H, 128, S_pad]).
 *   q, k, v  : const BF16 [B, S, H, 128]
 *   q_i8     : int8  [B, H, S_pad, 128]  Q codes
 *   q_scale  : float [B, H, S_pad / 32]  one scale per 32-row block
 *   k_i8     : int8  [B, H, S_pad, 128]  K codes
 *   k_scale  : float [B, H, S_pad / 32]
 *   v_fp8    : uint8 [B, H, 128, S_pad]  V codes, OCP FP8 E4M3 (e4m3fn) bytes
 *   v_scale  : float [B, H, 128]         one scale per (b, h, channel)
 *   scale    : the softmax scale the attention will use, finite and > 0
 * Arithmetic (IEEE fp32, round to nearest even throughout):
 *   c = float(double(scale) * log2(e));  Q values y = float(q) * c, K values y = float(k)
 *   per 32-row block: s = max|y| / 127, code = clamp(rint(y / s), -127, 127)
 *   per V channel over the S real tokens: sv = max|v| / 448, code = e4m3(v / sv)
 *   an all-zero block or channel gets scale 0 and codes 0; pad rows, pad
 *   columns (tokens S..S_pad-1) and pad blocks are written as 0.
 * Outputs must not overlap each other or the inputs.  v_scale doubles as the
 * absmax scratch while the call runs.
 */
int sage_prepare(const void* q, const void* k, const void* v, int8_t* q_i8, float* q_scale,
                 int8_t* k_i8, float* k_scale, uint8_t* v_fp8, float* v_scale, int B, int S,
                 int H, int D, float scale, hipStream_t stream);

/*
 * sage_prepare_ex -- sage_prepare with the optional Q/K row transform, K
 * smoothing and cross-attention / grouped-query shapes.
 *
 * Shapes: q is BF16 [B, S_q, H, 128]; k, v are BF16 [B, S_kv, H_kv, 128] with
 * H a multiple of H_kv.  Outputs as sage_prepare with S_q for the Q side and
 * S_kv, H_kv for the K and V sides: q_i8 [B, H, S_q_pad, 128], q_scale
 * [B, H, S_q_pad / 32], k_i8 [B, H_kv, S_kv_pad, 128], k_scale
 * [B, H_kv, S_kv_pad / 32], v_fp8 [B, H_kv, 128, S_kv_pad], v_scale [B, H_kv, 128].
 *
 * Row transform ([SAGE] first commit and "Technical Details": optional QK
 * RMSNorm and rotate-half RoPE, rounded like the eager PyTorch BF16
 * sequence), applied to each 128-channel Q and K row before quantization:
 *   q_norm_w, k_norm_w : BF16 [128] RMSNorm weights, or NULL (no RMSNorm on that side)
 *       n = bf16(x * r), r = 1 / sqrt(sum(x^2) / 128 + norm_eps) in fp32 (the sum
 *       a pairwise tree over the channels in index order), y = bf16(n * w)
 *   rope_dim : 0 (no RoPE), 32, 64, 96 or 128
 *   rope_cos, rope_sin : BF16 [>= max(S_q, S_kv), rope_dim], row = token position
 *       out[c] = bf16(bf16(y[c] * cos[c]) + bf16(rot[c] * sin[c])) for c < rope_dim,
 *       rot[c] = -y[c + rope_dim/2] below rope_dim/2, y[c - rope_dim/2] above
 *   norm_eps : finite, >= 0
 * RMSNorm comes first, then RoPE, then (for Q) the multiply by scale * log2(e).
 * The result equals qk_norm_rope_bf16 followed by sage_prepare, bit for bit.
 *
 * K smoothing ("Kernel acceleration: attention, compilation and fusion",
 * section "SageAttention: quantizing attention too": subtracting K's mean over
 * the tokens before quantizing leaves attention unchanged, since it shifts every
 * score of a query row by the same amount):
 *   k_mean : fp32 [B, H_kv, 128] output, or NULL (no smoothing).  When given,
 *       k_mean = fp32(sum_j y_j / S_kv) with the sum over the (transformed) K
 *       values in fp64, and K is quantized as fp32(y) - k_mean.
 *   workspace, workspace_bytes : device scratch of at least
 *       ditattn_sage_workspace_size(B, S_kv, H_kv) bytes when k_mean is given
 *       (ignored otherwise); contents on entry do not matter.
 * The fp64 channel sums are exact (so the mean is independent of the
 * summation order) when the values of a channel span less than
 * 2^(45 - ceil(log2 S_kv)) in magnitude.
 * Outputs, k_mean and workspace must not overlap each other or any input.
 */
int sage_prepare_ex(const void* q, const void* k, const void* v, int8_t* q_i8, float* q_scale,
                    int8_t* k_i8, float* k_scale, uint8_t* v_fp8, float* v_scale, int B, int S_q,
                    int S_kv, int H, int H_kv, int D, float scale, const void* q_norm_w,
                    const void* k_norm_w, float norm_eps, const void* rope_cos,
                    const void* rope_sin, int rope_dim, float* k_mean, void* workspace,
                    size_t workspace_bytes, hipStream_t stream);

/*
 * sage_prepare_ex_noalloc -- sage_prepare_ex without the workspace arguments, for
 * callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc).  It allocates nothing: K
 * smoothing (k_mean != NULL) uses a static device buffer of the library,
 * DITATTN_STATIC_SCRATCH_BYTES per GPU, and returns DITATTN_ENOSPACE before
 * anything is enqueued when ditattn_sage_workspace_size(B, S_kv, H_kv) exceeds
 * it.  The buffer's contents on entry do not matter (every value read is
 * written earlier in the same call).  Every call on one GPU shares that GPU's
 * buffer: calls that may overlap on one GPU (other streams, other threads) race.
 * The buffer's device address is looked up on the first smoothing call on each
 * device; make that first call outside graph capture.  Results are bit for bit
 * those of sage_prepare_ex.
 */
int sage_prepare_ex_noalloc(const void* q, const void* k, const void* v, int8_t* q_i8,
                            float* q_scale, int8_t* k_i8, float* k_scale, uint8_t* v_fp8,
                            float* v_scale, int B, int S_q, int S_kv, int H, int H_kv, int D,
                            float scale, const void* q_norm_w, const void* k_norm_w,
                            float norm_eps, const void* rope_cos, const void* rope_sin,
                            int rope_dim, float* k_mean, hipStream_t stream);

/*
 * attn_fwd_bf16_ws -- attn_fwd_bf16_ex with a workspace that lets the last, partial
 * round of query tiles be split over every compute unit.  Same operation ("Kernel
 * acceleration: attention, compilation and fusion", section "Attention: from O(N^2)
 * memory to blocks": the blocked form with running max and sum), same arguments,
 * checks and status codes as attn_fwd_bf16_ex, plus:
 *   workspace        device pointer, 16-byte aligned, overlapping no tensor, at least
 *                    ditattn_bf16_workspace_size(...) bytes (owned by the caller and
 *                    zero-filled before its first use, the fill complete or ordered
 *                    before the call on its stream; later calls need no clearing);
 *                    may be NULL when that size is 0
 *   workspace_bytes  its size; too small -> DITATTN_EINVAL before anything is enqueued
 * When the size is 0 (key window on, fewer than three whole rounds of query tiles, one
 * key tile per query tile, or a last round that is already 95 % full) the call is
 * attn_fwd_bf16_ex.  Otherwise the grid is one workgroup per compute unit: whole query
 * tiles first, then equal ranges of (query tile, key tile) units; a query tile split over
 * several workgroups is merged, in a fixed order, by the one holding its last key tile
 * from FP32 partials (m, l, O) the others leave in the workspace.  The result meets the
 * same accuracy as attn_fwd_bf16_ex's (it differs from it by the rounding of P to BF16,
 * taken relative to each piece's own running max) and is run-to-run deterministic.  One
 * workspace serves one call at a time.  A workgroup waits only for partials of lower-numbered
 * workgroups, and for at most about a second: with the GPU to itself the whole grid (one
 * workgroup per compute unit) is resident and the waits are short; kernels running at the
 * same time on other streams can hold compute units and delay the pieces, and a partial that
 * does not come within the bound leaves its rows NaN instead of hanging the GPU.
 */
int attn_fwd_bf16_ws(const void* q, const void* k, const void* v, void* o, int B, int S_q,
                     int S_kv, int H, int H_kv, int D, float scale, int window_left,
                     int window_right, void* workspace, size_t workspace_bytes,
                     hipStream_t stream);

/* Workspace bytes attn_fwd_bf16_ws needs on the current device (0: no split; also 0 for
 * sizes the library rejects). */
size_t ditattn_bf16_workspace_size(int B, int S_q, int S_kv, int H, int H_kv, int window_left,
                                   int window_right);

/* Workspace bytes sage_prepare_ex needs for K smoothing at these sizes (0 for
 * sizes it rejects).  Touches no GPU. */
size_t ditattn_sage_workspace_size(int B, int S_kv, int H_kv);

/*
 * qk_norm_rope_bf16 -- the row transform of sage_prepare_ex alone, BF16 in and
 * out: out = RoPE(RMSNorm(x)) per [b, s, h] row with the same arithmetic and
 * arguments (norm_w NULL: no RMSNorm; rope_dim 0: no RoPE; tables
 * [>= S, rope_dim]).  x, out: BF16 [B, S, H, 128]; out == x (in place) is
 * allowed, any other overlap is not.
 */
int qk_norm_rope_bf16(const void* x, void* out, int B, int S, int H, int D, const void* norm_w,
                      float norm_eps, const void* rope_cos, const void* rope_sin, int rope_dim,
                      hipStream_t stream);

/*
 * sage_attn_fwd -- the quantized forward on tensors written by sage_prepare
 * (the kernel alone on prepared tensors).  [SAGE] second commit: Q K^T on
 * INT8 MFMA, P V on FP8 MFMA, FP32 accumulation, online softmax, BF16 out.
 *   q_i8, q_scale, k_i8, k_scale, v_fp8, v_scale : as written by sage_prepare
 *                                                 for the same B, S, H
 *   o      : BF16 [B, S, H, 128], written in full; must not overlap the inputs
 *   scale  : checked (finite, > 0) but otherwise unused: sage_prepare already
 *            folded scale * log2(e) into q_scale.
 * Scores s = int32(q_code . k_code) * q_scale * k_scale are in base-2 units.
 * Keys j >= S are masked.  P is rounded to FP8 e4m3 as p * 2^8 and the row sum
 * l is taken over the same FP8 values; o = acc * v_scale / l.
 * Any magnitude: a workgroup whose q_scale * k_scale exceeds 2^-8 on some tile
 * (|q| and |k| in the tens and beyond) makes P's codes from the exact score
 * rather than the one-FMA form, whose rounding would grow with the scales; the
 * output stays finite while 2^29 * q_scale * k_scale is a finite fp32 value.
 */
int sage_attn_fwd(const int8_t* q_i8, const float* q_scale, const int8_t* k_i8,
                  const float* k_scale, const uint8_t* v_fp8, const float* v_scale, void* o,
                  int B, int S, int H, int D, float scale, hipStream_t stream);

/*
 * sage_attn_fwd_ex -- sage_attn_fwd on tensors written by sage_prepare_ex, with the
 * shapes and key window of attn_fwd_bf16_ex (same arguments and meaning):
 *   q_i8 [B, H, S_q_pad, 128], q_scale [B, H, S_q_pad / 32], k_i8 [B, H_kv, S_kv_pad, 128],
 *   k_scale [B, H_kv, S_kv_pad / 32], v_fp8 [B, H_kv, 128, S_kv_pad], v_scale [B, H_kv, 128],
 *   o BF16 [B, S_q, H, 128].  S_kv <= DITATTN_MAX_SEQ_SAGE.
 * sage_attn_fwd(...) equals sage_attn_fwd_ex(..., S, S, H, H, ..., -1, -1, ...).
 */
int sage_attn_fwd_ex(const int8_t* q_i8, const float* q_scale, const int8_t* k_i8,
                     const float* k_scale, const uint8_t* v_fp8, const float* v_scale, void* o,
                     int B, int S_q, int S_kv, int H, int H_kv, int D, float scale,
                     int window_left, int window_right, hipStream_t stream);

/*
 * sage_attn_fwd_ws -- sage_attn_fwd_ex with a workspace that lets the last, partial round
 * of query tiles be split over every compute unit, as attn_fwd_bf16_ws does for the BF16
 * path (same plan: both kernels tile queries by 256 rows and keys by 64).  Same operation,
 * arguments, checks and status codes as sage_attn_fwd_ex, plus:
 *   workspace        device pointer, 16-byte aligned, overlapping no tensor, at least
 *                    ditattn_sage_attn_workspace_size(...) bytes (owned by the caller and
 *                    zero-filled before its first use, the fill complete or ordered
 *                    before the call on its stream; later calls need no clearing);
 *                    may be NULL when that size is 0
 *   workspace_bytes  its size; too small -> DITATTN_EINVAL before anything is enqueued
 * When the size is 0 (key window on, fewer than three whole rounds of query tiles, one
 * key tile per query tile, or a last round that is already 95 % full) the call is
 * sage_attn_fwd_ex.  Otherwise a query tile split over several workgroups is merged, in a
 * fixed order, from FP32 partials (m, l, acc) by the workgroup holding its last key tile.
 * The result meets sage_attn_fwd_ex's accuracy (it differs from it by P's FP8 rounding,
 * taken relative to each piece's own running max) and is run-to-run deterministic.  One
 * workspace serves one call at a time.  Waits for partials are bounded as in
 * attn_fwd_bf16_ws (NaN rows instead of a hang).
 */
int sage_attn_fwd_ws(const int8_t* q_i8, const float* q_scale, const int8_t* k_i8,
                     const float* k_scale, const uint8_t* v_fp8, const float* v_scale, void* o,
                     int B, int S_q, int S_kv, int H, int H_kv, int D, float scale,
                     int window_left, int window_right, void* workspace, size_t workspace_bytes,
                     hipStream_t stream);

/* Workspace bytes sage_attn_fwd_ws needs on the current device (0: no split; also 0 for
 * sizes the library rejects).  Equal to ditattn_bf16_workspace_size for the same shape. */
size_t ditattn_sage_attn_workspace_size(int B, int S_q, int S_kv, int H, int H_kv, int window_left,
                                        int window_right);

#ifdef __cplusplus
}
#endif

#endif /* DITATTN_H */
