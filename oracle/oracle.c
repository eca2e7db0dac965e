/*
 * oracle.c -- plain CPU oracle for the DiT flash self-attention path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may call, link or
 * load this file.  Only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg use it, through oracle/__init__.py.  It shares no code,
 * header, table or constant with the HIP library: it is written from the
 * pages, independently of the kernels.
 *
 * What it computes
 * ----------------
 *  1. Exact attention in fp64 (both modes are gated against it).
 *     "Kernel acceleration: attention, compilation and fusion", section
 *     "Attention: from O(N^2) memory to blocks": the naive form materialises
 *     the scores q.k^T * scale, takes a row softmax and multiplies by V.
 *     oracle_softmax_row + oracle_attn_rows follow that form one query row at
 *     a time.  oracle_attn_blocked follows the blocked form of the same
 *     section (running max m, running sum l, accumulator acc, rescaled by
 *     exp(m - m_new) per key block); it is kept only to cross-check the naive
 *     form.
 *  2. The SageAttention-style quantizer, bit-exact, in IEEE fp32.
 *     "gfx1201_sage_prepare / gfx1201_sage_attention" (aiter PR 6390),
 *     section "Technical Details", first commit: Q/K -> INT8 with one FP32
 *     scale per (batch, head, 32-row block), Q carrying
 *     softmax_scale * log2(e); V -> FP8 e4m3, transposed to [B, H, 128, S_pad],
 *     one FP32 scale per channel.
 *     Readings where the page is silent (each one is listed with its reason in
 *     the design notes):
 *       - Q is multiplied by c = float(double(scale) * log2(e)) in fp32 first,
 *         then quantized (the configuration text says "Q pre-multiplied").
 *       - block scale s = absmax / 127 (fp32 division), codes
 *         clamp(rint(x / s), -127, 127) with fp32 division and
 *         round-half-to-even; an all-zero block has s = 0 and codes 0.
 *       - V scale sv = absmax / 448 per (b, h, channel) over the S real
 *         tokens; codes = e4m3fn(v / sv) (OCP E4M3, bias 7, no infinities,
 *         max 448), round to nearest, ties to even, saturating at 448.
 *       - code layouts: Q/K [B, H, S_pad, 128], scales [B, H, S_pad / 32];
 *         V codes [B, H, 128, S_pad], V scales [B, H, 128].  Pad rows, pad
 *         columns and pad blocks are 0.
 *
 *  1b. Exact attention for cross-attention (S_q != S_kv), grouped-query heads
 *     (H a multiple of H_kv) and a key window per query ("RDNAttention"
 *     README, "Features"): oracle_attn_rows_ex, same naive form, with each
 *     query row restricted to the keys it sees (queries aligned to the end of
 *     the keys); a row that sees no key is 0 by definition.
 *  3. The optional Q/K row transform of the prepare stage (same page, first
 *     commit and "Technical Details": RMSNorm and rotate-half RoPE with
 *     rope_dim 32/64/96/128, rounded like the eager PyTorch BF16 sequence).
 *     Readings (the page names the rounding rule, not the formulas):
 *       - RMSNorm normalizes each (b, s, h) row over its D channels, as the
 *         per-head QK norm of a DiT does:
 *           ms = (sum of fp32(x)^2 over the row) / D           (fp32)
 *           r  = 1 / sqrt(ms + eps)     (correctly rounded sqrt, then division)
 *           n  = bf16(fp32(x) * r);     y = bf16(fp32(n) * fp32(w))
 *         The sum of squares is taken as a pairwise tree over the channels in
 *         index order ((x0^2 + x1^2) + (x2^2 + x3^2)) + ...; eager PyTorch
 *         leaves its reduction order unspecified.
 *       - RoPE rotates the first rope_dim channels with BF16 tables
 *         cos, sin [S_tab, rope_dim] indexed by the row's token position:
 *           out[c] = bf16( bf16(y[c] * cos[c]) + bf16(rot[c] * sin[c]) ),
 *           rot[c] = -y[c + rope_dim/2] (c < rope_dim/2), y[c - rope_dim/2] (else);
 *         channels c >= rope_dim pass through.  Each BF16 product or sum is
 *         an fp32 operation rounded to BF16 (round to nearest even), which is
 *         how eager PyTorch evaluates BF16 tensor arithmetic.
 *       - RMSNorm (when enabled) comes first, then RoPE, then the quantizer.
 *  4. Attention of the quantized operands, in fp64 (same page, commit text of
 *     gfx1201_sage_attention: Q K^T on the INT8 codes, P V on the FP8 V codes,
 *     FP32 scales, online softmax; Q's scale carries softmax_scale * log2(e),
 *     so the softmax is taken in base 2).  It is what the Sage attention
 *     computes when only its inputs are rounded: its distance to (1) is the
 *     quantizer's error, a kernel's distance to it is the kernel's own
 *     (chiefly the rounding of P to FP8).
 *
 * Inputs are BF16 bit patterns (uint16) in [B, S, H, D] order.  Build with
 * plain gcc, -O2 -ffp-contract=off, no fast-math: the quantizer must round
 * every fp32 operation exactly as IEEE 754 says.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_OK 0
#define ORACLE_EINVAL (-1)
#define ORACLE_ENOMEM (-2)
#define ORACLE_ENONFINITE (-3)

/* BF16 is the top half of an fp32 word; widening is exact. */
static float bf16_to_f32(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return f;
}

static int64_t idx_bshd(int64_t b, int64_t i, int64_t h, int64_t d, int S, int H, int D) {
  return ((b * S + i) * H + h) * D + d;
}

int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* ------------------------------------------------------------------------ */
/* 1. Exact attention                                                         */
/* ------------------------------------------------------------------------ */

/*
 * Softmax probabilities of one query row (b, h, i):
 *   s_j = (sum_d q_d k_jd) * scale  for every key j < S,
 *   p_j = exp(s_j - max_j s_j) / sum_j exp(s_j - max_j s_j).
 * Natural exp on purpose: the kernels use exp2 with log2(e) folded into the
 * scores, which is the same function; the oracle keeps the textbook form.
 * p must hold S doubles.  Returns ORACLE_ENONFINITE if an input is not finite.
 */
int oracle_softmax_row(const uint16_t* q, const uint16_t* k, int B, int S, int H, int D,
                       float scale, int b, int h, int i, double* p) {
  if (b < 0 || b >= B || h < 0 || h >= H || i < 0 || i >= S || S <= 0 || D <= 0)
    return ORACLE_EINVAL;
  const double sc = (double)scale;
  double smax = -INFINITY;
  for (int j = 0; j < S; ++j) {
    double dot = 0.0;
    for (int d = 0; d < D; ++d)
      dot += (double)bf16_to_f32(q[idx_bshd(b, i, h, d, S, H, D)]) *
             (double)bf16_to_f32(k[idx_bshd(b, j, h, d, S, H, D)]);
    double s = dot * sc;
    if (!isfinite(s)) return ORACLE_ENONFINITE;
    p[j] = s;
    if (s > smax) smax = s;
  }
  double l = 0.0;
  for (int j = 0; j < S; ++j) {
    p[j] = exp(p[j] - smax);
    l += p[j];
  }
  for (int j = 0; j < S; ++j) p[j] /= l;
  return ORACLE_OK;
}

/*
 * Exact attention output for a list of query rows.
 * rows: nrows triples (b, h, i); out: nrows x D doubles,
 *   out[r][d] = sum_j p_j v_jd   with p from oracle_softmax_row.
 * Rows are independent; OpenMP spreads them over the host cores
 * (nthreads <= 0 means the OpenMP default).
 */
int oracle_attn_rows(const uint16_t* q, const uint16_t* k, const uint16_t* v, int B, int S,
                     int H, int D, float scale, const int64_t* rows, int64_t nrows,
                     double* out, int nthreads) {
  if (B <= 0 || S <= 0 || H <= 0 || D <= 0 || nrows < 0) return ORACLE_EINVAL;
  for (int64_t r = 0; r < nrows; ++r) {
    if (rows[3 * r] < 0 || rows[3 * r] >= B || rows[3 * r + 1] < 0 || rows[3 * r + 1] >= H ||
        rows[3 * r + 2] < 0 || rows[3 * r + 2] >= S)
      return ORACLE_EINVAL;
  }
#ifdef _OPENMP
  const int nt = nthreads > 0 ? nthreads : omp_get_max_threads();  /* this call only */
#else
  (void)nthreads;
#endif
  int status = ORACLE_OK;
#pragma omp parallel num_threads(nt)
  {
    double* p = (double*)malloc(sizeof(double) * (size_t)S);
    if (!p) {
#pragma omp atomic write
      status = ORACLE_ENOMEM;
    }
#pragma omp for schedule(dynamic, 4)
    for (int64_t r = 0; r < nrows; ++r) {
      if (!p) continue;
      const int b = (int)rows[3 * r], h = (int)rows[3 * r + 1], i = (int)rows[3 * r + 2];
      int st = oracle_softmax_row(q, k, B, S, H, D, scale, b, h, i, p);
      if (st != ORACLE_OK) {
#pragma omp atomic write
        status = st;
        continue;
      }
      for (int d = 0; d < D; ++d) out[r * D + d] = 0.0;
      for (int j = 0; j < S; ++j)
        for (int d = 0; d < D; ++d)
          out[r * D + d] += p[j] * (double)bf16_to_f32(v[idx_bshd(b, j, h, d, S, H, D)]);
    }
    free(p);
  }
  return status;
}

/*
 * Blocked attention with an online softmax, all rows, fp64.  Per query block
 * of bq rows and per key block of bk keys, for every row:
 *   m_new = max(m, max_j s_j)          (m starts at -inf)
 *   p_j   = exp(s_j - m_new)
 *   l     = l * exp(m - m_new) + sum_j p_j        (l starts at 0)
 *   acc   = acc * exp(m - m_new) + sum_j p_j v_j  (acc starts at 0)
 *   m     = m_new
 * and finally out = acc / l.  out is [B, S, H, D] doubles.
 * Kept to cross-check oracle_attn_rows; it is not what the gates compare to.
 */
int oracle_attn_blocked(const uint16_t* q, const uint16_t* k, const uint16_t* v, int B, int S,
                        int H, int D, float scale, int bq, int bk, double* out) {
  if (B <= 0 || S <= 0 || H <= 0 || D <= 0 || bq <= 0 || bk <= 0) return ORACLE_EINVAL;
  const double sc = (double)scale;
  double* m = (double*)malloc(sizeof(double) * (size_t)bq);
  double* l = (double*)malloc(sizeof(double) * (size_t)bq);
  double* acc = (double*)malloc(sizeof(double) * (size_t)bq * (size_t)D);
  double* s = (double*)malloc(sizeof(double) * (size_t)bq * (size_t)bk);
  if (!m || !l || !acc || !s) {
    free(m); free(l); free(acc); free(s);
    return ORACLE_ENOMEM;
  }
  for (int b = 0; b < B; ++b)
    for (int h = 0; h < H; ++h)
      for (int i0 = 0; i0 < S; i0 += bq) {
        const int ni = (S - i0 < bq) ? S - i0 : bq;
        for (int r = 0; r < ni; ++r) {
          m[r] = -INFINITY;
          l[r] = 0.0;
          for (int d = 0; d < D; ++d) acc[r * D + d] = 0.0;
        }
        for (int j0 = 0; j0 < S; j0 += bk) {
          const int nj = (S - j0 < bk) ? S - j0 : bk;
          for (int r = 0; r < ni; ++r) {
            double bmax = -INFINITY;
            for (int c = 0; c < nj; ++c) {
              double dot = 0.0;
              for (int d = 0; d < D; ++d)
                dot += (double)bf16_to_f32(q[idx_bshd(b, i0 + r, h, d, S, H, D)]) *
                       (double)bf16_to_f32(k[idx_bshd(b, j0 + c, h, d, S, H, D)]);
              s[r * bk + c] = dot * sc;
              if (s[r * bk + c] > bmax) bmax = s[r * bk + c];
            }
            const double m_new = (m[r] > bmax) ? m[r] : bmax;
            const double alpha = exp(m[r] - m_new); /* exp(-inf) = 0 on the first block */
            double psum = 0.0;
            for (int d = 0; d < D; ++d) acc[r * D + d] *= alpha;
            for (int c = 0; c < nj; ++c) {
              const double p = exp(s[r * bk + c] - m_new);
              psum += p;
              for (int d = 0; d < D; ++d)
                acc[r * D + d] += p * (double)bf16_to_f32(v[idx_bshd(b, j0 + c, h, d, S, H, D)]);
            }
            l[r] = l[r] * alpha + psum;
            m[r] = m_new;
          }
        }
        for (int r = 0; r < ni; ++r)
          for (int d = 0; d < D; ++d)
            out[idx_bshd(b, i0 + r, h, d, S, H, D)] = acc[r * D + d] / l[r];
      }
  free(m); free(l); free(acc); free(s);
  return ORACLE_OK;
}

/* ------------------------------------------------------------------------ */
/* 2. Quantizer                                                               */
/* ------------------------------------------------------------------------ */

/*
 * OCP FP8 E4M3 ("e4m3fn"): 1 sign bit, 4 exponent bits with bias 7,
 * 3 mantissa bits, no infinities, the all-ones pattern is NaN.
 * Value of a magnitude code 0..126 (0x7F is NaN):
 *   exponent field 0:      m * 2^-9                (subnormal)
 *   exponent field e > 0:  (1 + m/8) * 2^(e - 7) = (8 + m) * 2^(e - 10)
 */
double oracle_e4m3_decode(uint8_t code) {
  const int mag = code & 0x7F;
  if (mag == 0x7F) return NAN;
  const int e = mag >> 3, m = mag & 7;
  const double a = (e == 0) ? ldexp((double)m, -9) : ldexp((double)(8 + m), e - 10);
  return (code & 0x80) ? -a : a;
}

/*
 * Round a finite fp32 value to the nearest E4M3 value, ties to the code whose
 * mantissa LSB is 0 (ties to even), saturating at +-448.  The definition is
 * taken literally: the magnitude codes 0..126 are sorted by value, so a
 * binary search finds the two neighbours of |x| and the nearer one wins.
 * The sign bit is copied from x (so -0.0 and tiny negatives give 0x80).
 */
static double e4m3_mag[127]; /* e4m3_mag[c] = oracle_e4m3_decode(c), filled once */
static int e4m3_ready = 0;

static void e4m3_fill(void) {
#pragma omp critical(oracle_e4m3_table)
  {
    if (!e4m3_ready) {
      for (int c = 0; c < 127; ++c) e4m3_mag[c] = oracle_e4m3_decode((uint8_t)c);
#pragma omp flush
      e4m3_ready = 1;
    }
  }
}

uint8_t oracle_e4m3_encode(float x) {
  if (!e4m3_ready) e4m3_fill();
  const uint8_t sign = signbit(x) ? 0x80 : 0x00;
  const double a = fabs((double)x);
  if (a >= 448.0) return sign | 0x7E;
  int lo = 0, hi = 126; /* invariant: value(lo) <= a < value(hi) */
  while (hi - lo > 1) {
    const int mid = (lo + hi) / 2;
    if (e4m3_mag[mid] <= a) lo = mid; else hi = mid;
  }
  const double dlo = a - e4m3_mag[lo];
  const double dhi = e4m3_mag[hi] - a;
  int code;
  if (dlo < dhi) code = lo;
  else if (dhi < dlo) code = hi;
  else code = (lo & 1) ? hi : lo;
  return sign | (uint8_t)code;
}

int oracle_sage_padded_len(int S) { return (S + 255) / 256 * 256; }

/*
 * Q or K block quantization.  x: BF16 [B, S, H, D]; mult: c for Q, 1.0f for K
 * (multiplying by 1.0f is exact, so K is quantized as it stands).
 * For every (b, h, blk) with rows i in [32 blk, min(32 blk + 32, S)):
 *   y    = fp32(x) * mult            (one fp32 multiply)
 *   amax = max |y|
 *   s    = amax / 127                (fp32 division)
 *   code = clamp(rint(y / s), -127, 127), or 0 when s == 0
 * codes: int8 [B, H, S_pad, D]; scales: fp32 [B, H, S_pad / 32].
 */
int oracle_quant_qk_mean(const uint16_t* x, int B, int S, int H, int D, float mult, int S_pad,
                         const float* mean, int8_t* codes, float* scales);

int oracle_quant_qk(const uint16_t* x, int B, int S, int H, int D, float mult, int S_pad,
                    int8_t* codes, float* scales) {
  return oracle_quant_qk_mean(x, B, S, H, D, mult, S_pad, NULL, codes, scales);
}

/*
 * As oracle_quant_qk, with y = (fp32(x) - mean[b, h, d]) * mult when mean is not
 * NULL (mean: fp32 [B, H, D]; the subtraction is one fp32 operation).  This is
 * the smoothed K of the prepare stage ("Kernel acceleration: attention,
 * compilation and fusion", section "SageAttention: quantizing attention too":
 * K minus its mean over the tokens gives the same attention).
 */
int oracle_quant_qk_mean(const uint16_t* x, int B, int S, int H, int D, float mult, int S_pad,
                         const float* mean, int8_t* codes, float* scales) {
  if (B <= 0 || S <= 0 || H <= 0 || D <= 0 || S_pad < S || S_pad % 32 != 0) return ORACLE_EINVAL;
  const int nblk = S_pad / 32;
  int status = ORACLE_OK;
  /* blocks are independent; spread them over the host cores */
#pragma omp parallel for collapse(3) schedule(static)
  for (int b = 0; b < B; ++b)
    for (int h = 0; h < H; ++h)
      for (int blk = 0; blk < nblk; ++blk) {
        const int i0 = blk * 32;
        const int i1 = (i0 + 32 < S) ? i0 + 32 : S;
        const float* mu = mean ? mean + ((int64_t)b * H + h) * D : NULL;
        float amax = 0.0f;
        for (int i = i0; i < i1; ++i)
          for (int d = 0; d < D; ++d) {
            float y = bf16_to_f32(x[idx_bshd(b, i, h, d, S, H, D)]);
            if (mu) y = y - mu[d];
            y = y * mult;
            if (!isfinite(y)) {
#pragma omp atomic write
              status = ORACLE_ENONFINITE;
            }
            const float ay = fabsf(y);
            if (ay > amax) amax = ay;
          }
        const float s = amax / 127.0f;
        scales[((int64_t)b * H + h) * nblk + blk] = s;
        for (int i = i0; i < i0 + 32; ++i)
          for (int d = 0; d < D; ++d) {
            int8_t code = 0;
            if (i < i1 && s != 0.0f) {
              float y = bf16_to_f32(x[idx_bshd(b, i, h, d, S, H, D)]);
              if (mu) y = y - mu[d];
              y = y * mult;
              float r = rintf(y / s);
              if (r > 127.0f) r = 127.0f;
              if (r < -127.0f) r = -127.0f;
              code = (int8_t)r;
            }
            codes[(((int64_t)b * H + h) * S_pad + i) * D + d] = code;
          }
      }
  return status;
}

/*
 * V per-channel quantization and transpose.  v: BF16 [B, S, H, D].
 * For every (b, h, ch):
 *   amax = max_{j < S} |fp32(v_j)|,  sv = amax / 448  (fp32 division)
 *   code[b, h, ch, j] = e4m3(fp32(v_j) / sv) for j < S (0 when sv == 0),
 *   code = 0 for the pad columns S <= j < S_pad.
 * codes: uint8 [B, H, D, S_pad]; scales: fp32 [B, H, D].
 */
int oracle_quant_v(const uint16_t* v, int B, int S, int H, int D, int S_pad, uint8_t* codes,
                   float* scales) {
  if (B <= 0 || S <= 0 || H <= 0 || D <= 0 || S_pad < S) return ORACLE_EINVAL;
  int status = ORACLE_OK;
  e4m3_fill();
  /* channels are independent; spread them over the host cores */
#pragma omp parallel for collapse(3) schedule(static)
  for (int b = 0; b < B; ++b)
    for (int h = 0; h < H; ++h)
      for (int ch = 0; ch < D; ++ch) {
        float amax = 0.0f;
        for (int j = 0; j < S; ++j) {
          const float y = bf16_to_f32(v[idx_bshd(b, j, h, ch, S, H, D)]);
          if (!isfinite(y)) {
#pragma omp atomic write
            status = ORACLE_ENONFINITE;
          }
          if (fabsf(y) > amax) amax = fabsf(y);
        }
        const float sv = amax / 448.0f;
        scales[((int64_t)b * H + h) * D + ch] = sv;
        uint8_t* row = codes + (((int64_t)b * H + h) * D + ch) * S_pad;
        for (int j = 0; j < S_pad; ++j) {
          uint8_t code = 0;
          if (j < S && sv != 0.0f) code = oracle_e4m3_encode(bf16_to_f32(v[idx_bshd(b, j, h, ch, S, H, D)]) / sv);
          row[j] = code;
        }
      }
  return status;
}

/* ------------------------------------------------------------------------ */
/* 3. Q/K row transform: RMSNorm and rotate-half RoPE (BF16 rounding)        */
/* ------------------------------------------------------------------------ */

/* fp32 -> BF16, round to nearest, ties to even (inputs are finite). */
uint16_t oracle_f32_to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  const uint32_t lsb = (u >> 16) & 1u;
  return (uint16_t)((u + 0x7FFFu + lsb) >> 16);
}

static float bf16r(float f) { return bf16_to_f32(oracle_f32_to_bf16(f)); }

/* Sum of v[0..n) as a pairwise tree in index order (n a power of two). */
static float pairwise_sum(const float* v, int n) {
  if (n == 1) return v[0];
  return pairwise_sum(v, n / 2) + pairwise_sum(v + n / 2, n / 2);
}

/*
 * out = RoPE(RMSNorm(x)) per row, both optional (see the readings at the top).
 *   x, out   : BF16 [B, S, H, D] (may not alias)
 *   norm_w   : BF16 [D] or NULL (no RMSNorm); eps its epsilon
 *   cos_t, sin_t : BF16 [>= S, rope_dim] or NULL when rope_dim == 0
 *   rope_dim : 0 (no RoPE) or an even number <= D
 * D must be a power of two <= 128.
 */
int oracle_qk_norm_rope(const uint16_t* x, int B, int S, int H, int D, const uint16_t* norm_w,
                        float eps, const uint16_t* cos_t, const uint16_t* sin_t, int rope_dim,
                        uint16_t* out) {
  if (B <= 0 || S <= 0 || H <= 0 || D <= 0 || D > 128 || (D & (D - 1)) != 0) return ORACLE_EINVAL;
  if (rope_dim < 0 || rope_dim > D || (rope_dim & 1) || (rope_dim && (!cos_t || !sin_t)))
    return ORACLE_EINVAL;
  const int half = rope_dim / 2;
#pragma omp parallel for collapse(3) schedule(static)
  for (int b = 0; b < B; ++b)
    for (int i = 0; i < S; ++i)
      for (int h = 0; h < H; ++h) {
        float y[128], sq[128];
        for (int d = 0; d < D; ++d) y[d] = bf16_to_f32(x[idx_bshd(b, i, h, d, S, H, D)]);
        if (norm_w) {
          for (int d = 0; d < D; ++d) sq[d] = y[d] * y[d];
          const float ms = pairwise_sum(sq, D) / (float)D;
          const float r = 1.0f / sqrtf(ms + eps);
          for (int d = 0; d < D; ++d) y[d] = bf16r(bf16r(y[d] * r) * bf16_to_f32(norm_w[d]));
        }
        if (rope_dim) {
          float z[128];
          for (int c = 0; c < rope_dim; ++c) {
            const float cs = bf16_to_f32(cos_t[(int64_t)i * rope_dim + c]);
            const float sn = bf16_to_f32(sin_t[(int64_t)i * rope_dim + c]);
            const float rot = (c < half) ? -y[c + half] : y[c - half];
            z[c] = bf16r(bf16r(y[c] * cs) + bf16r(rot * sn));
          }
          for (int c = 0; c < rope_dim; ++c) y[c] = z[c];
        }
        for (int d = 0; d < D; ++d) out[idx_bshd(b, i, h, d, S, H, D)] = oracle_f32_to_bf16(y[d]);
      }
  return ORACLE_OK;
}

/*
 * Channel means for K smoothing: mean[b, h, d] = fp32( (sum over j < S of
 * fp64(x[b, j, h, d])) / S ), the sum taken in token order in fp64 and the
 * quotient rounded to fp32.  mean: fp32 [B, H, D].
 */
int oracle_channel_mean(const uint16_t* x, int B, int S, int H, int D, float* mean) {
  if (B <= 0 || S <= 0 || H <= 0 || D <= 0) return ORACLE_EINVAL;
#pragma omp parallel for collapse(3) schedule(static)
  for (int b = 0; b < B; ++b)
    for (int h = 0; h < H; ++h)
      for (int d = 0; d < D; ++d) {
        double s = 0.0;
        for (int j = 0; j < S; ++j) s += (double)bf16_to_f32(x[idx_bshd(b, j, h, d, S, H, D)]);
        mean[((int64_t)b * H + h) * D + d] = (float)(s / (double)S);
      }
  return ORACLE_OK;
}

/* ------------------------------------------------------------------------ */
/* 1b. Exact attention with a key window, S_q != S_kv and grouped heads       */
/* ------------------------------------------------------------------------ */

/*
 * q: BF16 [B, S_q, H, D]; k, v: BF16 [B, S_kv, H_kv, D]; query head h reads
 * key/value head h / (H / H_kv).  Query i sees key j when lo <= j <= hi with
 * off = S_kv - S_q, lo = i + off - wl (wl >= 0; no bound when wl < 0) and
 * hi = i + off + wr (wr >= 0; no bound when wr < 0).  Over the visible keys:
 *   s_j = (sum_d q_d k_jd) * scale,  p_j = exp(s_j - max s) / sum exp(s - max s),
 *   out_d = sum_j p_j v_jd;  out = 0 when no key is visible.
 * rows: nrows triples (b, h, i); out: nrows x D doubles.
 */
int oracle_attn_rows_ex(const uint16_t* q, const uint16_t* k, const uint16_t* v, int B, int S_q,
                        int S_kv, int H, int H_kv, int D, float scale, int wl, int wr,
                        const int64_t* rows, int64_t nrows, double* out, int nthreads) {
  if (B <= 0 || S_q <= 0 || S_kv <= 0 || H <= 0 || H_kv <= 0 || D <= 0 || nrows < 0 || H % H_kv)
    return ORACLE_EINVAL;
  for (int64_t r = 0; r < nrows; ++r)
    if (rows[3 * r] < 0 || rows[3 * r] >= B || rows[3 * r + 1] < 0 || rows[3 * r + 1] >= H ||
        rows[3 * r + 2] < 0 || rows[3 * r + 2] >= S_q)
      return ORACLE_EINVAL;
#ifdef _OPENMP
  const int nt = nthreads > 0 ? nthreads : omp_get_max_threads();  /* this call only */
#else
  (void)nthreads;
#endif
  const int G = H / H_kv;
  const double sc = (double)scale;
  int status = ORACLE_OK;
#pragma omp parallel num_threads(nt)
  {
    double* s = (double*)malloc(sizeof(double) * (size_t)S_kv);
    if (!s) {
#pragma omp atomic write
      status = ORACLE_ENOMEM;
    }
#pragma omp for schedule(dynamic, 4)
    for (int64_t r = 0; r < nrows; ++r) {
      if (!s) continue;
      const int64_t b = rows[3 * r], h = rows[3 * r + 1], i = rows[3 * r + 2];
      const int64_t hk = h / G;
      const int64_t off = (int64_t)S_kv - S_q;
      int64_t lo = 0, hi = S_kv - 1;
      if (wl >= 0 && i + off - wl > lo) lo = i + off - wl;
      if (wr >= 0 && i + off + wr < hi) hi = i + off + wr;
      for (int d = 0; d < D; ++d) out[r * D + d] = 0.0;
      if (lo > hi) continue; /* no visible key */
      double smax = -INFINITY;
      for (int64_t j = lo; j <= hi; ++j) {
        double dot = 0.0;
        for (int d = 0; d < D; ++d)
          dot += (double)bf16_to_f32(q[((b * S_q + i) * H + h) * D + d]) *
                 (double)bf16_to_f32(k[((b * S_kv + j) * H_kv + hk) * D + d]);
        s[j] = dot * sc;
        if (s[j] > smax) smax = s[j];
      }
      double l = 0.0;
      for (int64_t j = lo; j <= hi; ++j) {
        s[j] = exp(s[j] - smax);
        l += s[j];
      }
      for (int64_t j = lo; j <= hi; ++j)
        for (int d = 0; d < D; ++d)
          out[r * D + d] += (s[j] / l) * (double)bf16_to_f32(v[((b * S_kv + j) * H_kv + hk) * D + d]);
    }
    free(s);
  }
  return status;
}

/* ------------------------------------------------------------------------ */
/* 4. Attention of the quantized operands                                     */
/* ------------------------------------------------------------------------ */
/*
 * For each row (b, h, i) of rows (nrows triples), with the codes and scales in
 * the layouts oracle_quant_qk and oracle_quant_v write: Q [B, H, S_q_pad, D],
 * K [B, H_kv, S_kv_pad, D], V [B, H_kv, D, S_kv_pad]; query head h reads key /
 * value head h / (H / H_kv), and sees key j when lo(i) <= j <= hi(i) with the
 * window of oracle_attn_rows_ex (lo = i + S_kv - S_q - wl, hi = i + S_kv - S_q + wr,
 * a negative bound meaning none on that side):
 *   x_j = (sum_d qc[b,h,i,d] * kc[b,hk,j,d]) * qs[b,h,i/32] * ks[b,hk,j/32]
 *   p_j = 2^(x_j - max x)   over the keys the query sees
 *   out[r][d] = vs[b,hk,d] * (sum_j p_j * e4m3(vc[b,hk,d,j])) / (sum_j p_j),
 * or 0 for a row that sees no key.  The dot products of codes are exact
 * integers; the rest is fp64.
 */
int oracle_sage_attn_rows_ex(const int8_t* qc, const float* qs, const int8_t* kc, const float* ks,
                             const uint8_t* vc, const float* vs, int B, int S_q, int S_kv, int H,
                             int H_kv, int D, int S_q_pad, int S_kv_pad, int wl, int wr,
                             const int64_t* rows, int64_t nrows, double* out, int nthreads) {
  if (B <= 0 || S_q <= 0 || S_kv <= 0 || H <= 0 || H_kv <= 0 || H % H_kv != 0 || D <= 0 ||
      S_q_pad < S_q || S_kv_pad < S_kv || S_q_pad % 32 != 0 || S_kv_pad % 32 != 0 || nrows < 0)
    return ORACLE_EINVAL;
  for (int64_t r = 0; r < nrows; ++r) {
    if (rows[3 * r] < 0 || rows[3 * r] >= B || rows[3 * r + 1] < 0 || rows[3 * r + 1] >= H ||
        rows[3 * r + 2] < 0 || rows[3 * r + 2] >= S_q)
      return ORACLE_EINVAL;
  }
#ifdef _OPENMP
  const int nt = nthreads > 0 ? nthreads : omp_get_max_threads();  /* this call only */
#else
  (void)nthreads;
#endif
  const int group = H / H_kv;
  int status = ORACLE_OK;
#pragma omp parallel num_threads(nt)
  {
    double* x = (double*)malloc(sizeof(double) * (size_t)S_kv);
    if (!x) {
#pragma omp atomic write
      status = ORACLE_ENOMEM;
    }
#pragma omp for schedule(dynamic, 4)
    for (int64_t r = 0; r < nrows; ++r) {
      if (!x) continue;
      const int64_t b = rows[3 * r], h = rows[3 * r + 1], i = rows[3 * r + 2];
      const int64_t bh = b * H + h, bk = b * H_kv + h / group;
      const int64_t c = i + S_kv - S_q;
      const int64_t lo = wl >= 0 ? (c - wl > 0 ? c - wl : 0) : 0;
      const int64_t hi = wr >= 0 ? (c + wr < S_kv - 1 ? c + wr : S_kv - 1) : S_kv - 1;
      if (lo > hi) {
        for (int d = 0; d < D; ++d) out[r * D + d] = 0.0;
        continue;
      }
      const int8_t* qrow = qc + (bh * S_q_pad + i) * D;
      const double q_s = (double)qs[bh * (S_q_pad / 32) + i / 32];
      double xmax = -INFINITY;
      for (int64_t j = lo; j <= hi; ++j) {
        const int8_t* krow = kc + (bk * S_kv_pad + j) * D;
        int64_t dot = 0;
        for (int d = 0; d < D; ++d) dot += (int64_t)qrow[d] * (int64_t)krow[d];
        x[j] = (double)dot * q_s * (double)ks[bk * (S_kv_pad / 32) + j / 32];
        if (x[j] > xmax) xmax = x[j];
      }
      double l = 0.0;
      for (int64_t j = lo; j <= hi; ++j) {
        x[j] = exp2(x[j] - xmax);
        l += x[j];
      }
      for (int d = 0; d < D; ++d) {
        const uint8_t* vrow = vc + (bk * D + d) * S_kv_pad;
        double acc = 0.0;
        for (int64_t j = lo; j <= hi; ++j) acc += x[j] * oracle_e4m3_decode(vrow[j]);
        out[r * D + d] = (double)vs[bk * D + d] * acc / l;
      }
    }
    free(x);
  }
  return status;
}

/* Self-attention without a window: oracle_sage_attn_rows_ex with S_q = S_kv = S, H_kv = H. */
int oracle_sage_attn_rows(const int8_t* qc, const float* qs, const int8_t* kc, const float* ks,
                          const uint8_t* vc, const float* vs, int B, int S, int H, int D,
                          int S_pad, const int64_t* rows, int64_t nrows, double* out,
                          int nthreads) {
  return oracle_sage_attn_rows_ex(qc, qs, kc, ks, vc, vs, B, S, S, H, H, D, S_pad, S_pad, -1, -1,
                                  rows, nrows, out, nthreads);
}
