// prepare.hip -- Sage prepare stage for gfx950: BF16 Q/K -> INT8 codes with
// one FP32 scale per (b, h, 32-row block), V -> FP8 e4m3 codes with one FP32
// scale per (b, h, channel), transposed to [B, H, 128, S_pad].
//
// Operation: "gfx1201_sage_prepare / gfx1201_sage_attention" (aiter PR 6390),
// first commit and "Technical Details".  Q carries softmax_scale * log2(e):
// it is multiplied by c = float(double(scale) * log2(e)) in fp32 before it is
// quantized.  Scales are absmax / 127 (Q, K) and absmax / 448 (V, the largest
// finite e4m3 value); codes round to nearest even; an all-zero block or
// channel gets scale 0 and codes 0; pad rows, pad tokens and pad blocks are 0.
//
// All of it is HBM-bound, so the kernels are shaped for coalescing:
//   quant_qk   one wave per (b, h, 32-row block) of Q or K: 32 rows x 256 B in,
//              4 KB of codes out (contiguous), one scale.
//   v_absmax   per (b, token range, 512 channels): running |v| maxima in
//              registers, combined across the 4 waves in LDS, then one
//              atomicMax per channel on the fp32 bit pattern (order free: max
//              of non-negative floats = max of their bit patterns).
//   v_quant    per (b, h, 128-token chunk): quantize, transpose through LDS,
//              write 128 channel rows of 128 B; the chunk-0 workgroup of each
//              (b, h) also writes the final v_scale = absmax / 448.
// The V absmax accumulator is the v_scale buffer itself.  While it holds a
// running maximum, bit 31 of each word is set (quant_qk, which runs first,
// initializes it to 0x80000000, i.e. a maximum of +0 with the flag); the
// finished scale absmax / 448 is a non-negative float, bit 31 clear.  A
// v_quant workgroup that reads a word of its (b, h) either finds the flagged
// maximum and divides it by 448 itself or finds the finished scale written by
// the chunk-0 workgroup: both give the same value, so the write needs no
// ordering against the other workgroups' reads and no fourth launch.
// Division and rounding are IEEE fp32 (the library is built with correctly
// rounded division), so the codes are bit-identical to a scalar CPU quantizer.
#include "common.hpp"
#include "launch.hpp"

namespace ditattn {
namespace prep {

constexpr uint32_t kAmaxFlag = 0x80000000u;  // bit 31 marks a running absmax word

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// y / s rounded to nearest, as the correctly rounded division, from inv = 1 / s (itself
// correctly rounded, computed once per scale): q0 = y * inv is within one ulp of y / s,
// the residual y - q0 s is exact in one FMA, and q0 + r * inv then rounds to y / s
// (Markstein's theorem on division by FMA).  It needs the residual not to underflow:
// callers use it for 2^-60 <= s <= 2^100 (fast_div_ok) and divide otherwise.  The sign
// is copied from y so that y = -0 gives -0 as the division does.  Checked against the
// division on the GPU for every float32 quotient of magnitude 2^-12 .. 1024 and 64
// divisors between 2^-63 and 2^120.
__device__ __forceinline__ bool fast_div_ok(float s) { return s >= 0x1p-60f && s <= 0x1p100f; }
__device__ __forceinline__ float div_by_recip(float y, float s, float inv) {
  const float q0 = y * inv;
  const float r = fmaf(-q0, s, y);
  return __builtin_copysignf(fmaf(r, inv, q0), y);
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x = fmaxf(x, __shfl_xor(x, off, 64));
  return x;
}

// ---------------------------------------------------------------- Q/K row transform
// Optional RMSNorm and rotate-half RoPE of a Q or K row before it is quantized,
// rounded like the eager BF16 sequence: n = bf16(x * r) with r = 1 / sqrt(mean(x^2) + eps),
// y = bf16(n * w); then out = bf16(bf16(y * cos) + bf16(rot(y) * sin)) on the first
// rope_dim channels, rot(y)[c] = -y[c + rope_dim/2] below rope_dim/2, y[c - rope_dim/2] above.
// The sum of squares is a pairwise tree over the channels in index order.
struct RowXform {
  const uint16_t* norm_w;  // BF16 [128] RMSNorm weight, or nullptr (no RMSNorm)
  float eps;
  const uint16_t* cos_t;   // BF16 [S_tab, rope_dim], row = token position
  const uint16_t* sin_t;
  int rope_dim;            // 0 (no RoPE), 32, 64, 96 or 128
};

__device__ __forceinline__ float round_bf16(float x) { return (float)(__bf16)x; }

__device__ __forceinline__ void unpack_bf16x8(const uint4& raw, float (&y)[8]) {
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    y[2 * e] = bf16_bits_to_f32(w[e] & 0xFFFFu);
    y[2 * e + 1] = bf16_bits_to_f32(w[e] >> 16);
  }
}

// y: channels 8 * chunk + 0..7 of one row at token position `tok`; the 16 lanes with
// the same lane >> 4 hold the 16 fragments of that row.  Every lane of the wave
// calls this together (it shuffles); rows with valid == false come out as zeros.
__device__ __forceinline__ void xform_fragment(float (&y)[8], int chunk, int tok, bool valid,
                                               const RowXform& t) {
#pragma clang fp contract(off)
  if (t.norm_w) {
    float sq[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) sq[e] = y[e] * y[e];
    float s = ((sq[0] + sq[1]) + (sq[2] + sq[3])) + ((sq[4] + sq[5]) + (sq[6] + sq[7]));
#pragma unroll
    for (int off = 1; off <= 8; off <<= 1) s = s + __shfl_xor(s, off, 64);
    const float r = 1.0f / sqrtf(s / 128.0f + t.eps);
    float w[8];
    unpack_bf16x8(*(const uint4*)(t.norm_w + 8 * chunk), w);
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] = round_bf16(round_bf16(y[e] * r) * w[e]);
  }
  if (t.rope_dim) {
    const int lane = threadIdx.x & 63;
    const bool rot_lane = 8 * chunk < t.rope_dim;
    const bool lower = 16 * chunk < t.rope_dim;   // channel < rope_dim / 2
    const int hc = t.rope_dim >> 4;               // rope_dim / 2 in 8-channel chunks
    const int src = rot_lane ? (lower ? lane + hc : lane - hc) : lane;
    float part[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) part[e] = __shfl(y[e], src, 64);
    if (rot_lane && valid) {
      float cs[8], sn[8];
      const int64_t o = (int64_t)tok * t.rope_dim + 8 * chunk;
      unpack_bf16x8(*(const uint4*)(t.cos_t + o), cs);
      unpack_bf16x8(*(const uint4*)(t.sin_t + o), sn);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float rot = lower ? -part[e] : part[e];
        y[e] = round_bf16(round_bf16(y[e] * cs[e]) + round_bf16(rot * sn[e]));
      }
    }
  }
  if (!valid) {
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] = 0.0f;
  }
}

// ---------------------------------------------------------------- Q and K
// One side (Q or K) of the quantizer.
struct QuantSide {
  const uint16_t* x;  // BF16 [B, S, H, 128]
  int8_t* codes;      // [B, H, S_pad, 128]
  float* scales;      // [B, H, S_pad / 32]
  const float* mean;  // [B, H, 128] subtracted (fp32) after the transform, or nullptr
  int S, H, nblk, units;
  float mult;         // c = scale * log2(e) for Q, 1 for K (x * 1.0f is exact)
  RowXform xf;
};

// grid.x: ceil(max(units) / 4) workgroups of 4 waves; grid.y: 0 = Q, 1 = K.
// One wave per (b, h, 32-row block): 32 rows x 256 B in, 4 KB of codes out, one scale.
template <bool XF>
__global__ void __launch_bounds__(256)
quant_qk_kernel(QuantSide qs, QuantSide ks, uint32_t* __restrict__ amax_bits, int n_amax) {
  // initialize the V absmax accumulator (flagged +0) for v_absmax_kernel, which runs
  // later on the stream; the first ceil(n_amax / 256) workgroups of the Q half do it
  {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (blockIdx.y == 0 && i < n_amax) amax_bits[i] = kAmaxFlag;
  }
  const QuantSide& a = blockIdx.y == 0 ? qs : ks;
  const int unit = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (unit >= a.units) return;  // whole waves leave together
  const int lane = threadIdx.x & 63;
  const int blk = unit % a.nblk;
  const int bh = unit / a.nblk;
  const int b = bh / a.H, h = bh - b * a.H;
  const int64_t tok = (int64_t)a.H * kHeadDim;
  const uint16_t* src = a.x + ((int64_t)b * a.S * a.H + h) * kHeadDim;

  // lane owns 8 channels (chunk lane & 15) of rows (lane >> 4) + 4 p, p = 0..7
  const int chunk = lane & 15;
  float y[8][8];
  float mean[8];
  if (a.mean) {
    const float* m = a.mean + (int64_t)bh * kHeadDim + 8 * chunk;
#pragma unroll
    for (int e = 0; e < 8; ++e) mean[e] = m[e];
  }
  float amax = 0.0f;
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    const int i = blk * 32 + (lane >> 4) + 4 * p;
    uint4 raw = uint4{0, 0, 0, 0};
    if (i < a.S) raw = *(const uint4*)(src + i * tok + 8 * chunk);
    unpack_bf16x8(raw, y[p]);
    if constexpr (XF) xform_fragment(y[p], chunk, i, i < a.S, a.xf);
    if (a.mean && i < a.S) {
#pragma unroll
      for (int e = 0; e < 8; ++e) y[p][e] = y[p][e] - mean[e];
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      y[p][e] = y[p][e] * a.mult;
      amax = fmaxf(amax, fabsf(y[p][e]));
    }
  }
  amax = wave_max(amax);
  const float s = amax / 127.0f;
  const bool fast = fast_div_ok(s);
  const float inv = 1.0f / s;
  int8_t* dst = a.codes + ((int64_t)bh * a.nblk * 32 + blk * 32) * kHeadDim;
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    const int r = (lane >> 4) + 4 * p;
    uint32_t packed[2] = {0u, 0u};
    if (fast) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float qv = rintf(div_by_recip(y[p][e], s, inv));
        qv = fminf(fmaxf(qv, -127.0f), 127.0f);
        packed[e >> 2] |= ((uint32_t)(int)qv & 0xFFu) << (8 * (e & 3));
      }
    } else if (s != 0.0f) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float qv = rintf(y[p][e] / s);
        qv = fminf(fmaxf(qv, -127.0f), 127.0f);
        packed[e >> 2] |= ((uint32_t)(int)qv & 0xFFu) << (8 * (e & 3));
      }
    }
    *(uint2*)(dst + r * kHeadDim + 8 * chunk) = uint2{packed[0], packed[1]};
  }
  if (lane == 0) a.scales[(int64_t)bh * a.nblk + blk] = s;
}

// ---------------------------------------------------------------- transform alone
// out = transform(x), BF16 [B, S, H, 128] -> BF16; same lanes as quant_qk_kernel.
__global__ void __launch_bounds__(256)
xform_kernel(const uint16_t* __restrict__ x, uint16_t* __restrict__ out, int S, int H, int nblk,
             int units, RowXform xf) {
  const int unit = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (unit >= units) return;
  const int lane = threadIdx.x & 63;
  const int blk = unit % nblk;
  const int bh = unit / nblk;
  const int b = bh / H, h = bh - b * H;
  const int64_t tok = (int64_t)H * kHeadDim;
  const int64_t base = ((int64_t)b * S * H + h) * kHeadDim;
  const int chunk = lane & 15;
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    const int i = blk * 32 + (lane >> 4) + 4 * p;
    uint4 raw = uint4{0, 0, 0, 0};
    if (i < S) raw = *(const uint4*)(x + base + i * tok + 8 * chunk);
    float y[8];
    unpack_bf16x8(raw, y);
    xform_fragment(y, chunk, i, i < S, xf);
    if (i < S) {
      uint32_t w[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t lo = __builtin_bit_cast(uint16_t, (__bf16)y[2 * e]);
        const uint32_t hi = __builtin_bit_cast(uint16_t, (__bf16)y[2 * e + 1]);
        w[e] = lo | (hi << 16);
      }
      *(uint4*)(out + base + i * tok + 8 * chunk) = uint4{w[0], w[1], w[2], w[3]};
    }
  }
}

// ---------------------------------------------------------------- K channel means (smoothing)
// Per-(b, h, channel) mean of the (transformed) K values over the S tokens:
// mean = fp32(fp64 sum / S).  k_colsum_kernel writes fp64 partial sums per token
// range (no atomics, fixed order) to the workspace [B, nchunk, H, 128]; k_mean_kernel
// adds them up in a fixed order.  Both sums are exact, hence order free, whenever the
// values of a channel span less than 2^(45 - log2 S) in magnitude.
// Grid and lanes as v_absmax_kernel: a workgroup covers 4 heads (64 lanes x 16 B) of
// one token range; the 16 lanes of one head row sit together, as the transform needs.
template <bool XF>
__global__ void __launch_bounds__(256)
k_colsum_kernel(const uint16_t* __restrict__ k, double* __restrict__ partial, int S, int H,
                int tok_per_wg, int nchunk, int colblk, RowXform xf) {
  __shared__ double red[4][64][8];
  const int rng = blockIdx.x % nchunk;
  const int bc = blockIdx.x / nchunk;
  const int b = bc / colblk, cb = bc - b * colblk;
  const int ncol = H * 16;
  const int col = cb * 64 + (threadIdx.x & 63);
  const bool col_ok = col < ncol;  // a whole head (16 lanes) is in or out
  const int wv = threadIdx.x >> 6;
  const int chunk = threadIdx.x & 15;
  const int j0 = rng * tok_per_wg;
  const int j1 = min(j0 + tok_per_wg, S);
  const int64_t tok = (int64_t)H * kHeadDim;
  const uint16_t* src = k + (int64_t)b * S * tok + 8 * (int64_t)(col_ok ? col : 0);
  double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int j = j0 + wv; j < j1; j += 4) {  // wave-uniform trip count
    uint4 raw = uint4{0, 0, 0, 0};
    if (col_ok) raw = *(const uint4*)(src + j * tok);
    float y[8];
    unpack_bf16x8(raw, y);
    if constexpr (XF) xform_fragment(y, chunk, j, col_ok, xf);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] += (double)y[e];
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) red[wv][threadIdx.x & 63][e] = acc[e];
  __syncthreads();
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int idx = threadIdx.x + 256 * r;
    const int c = idx >> 3, e = idx & 7;
    const int gcol = cb * 64 + c;
    if (gcol < ncol)
      partial[((int64_t)b * nchunk + rng) * H * kHeadDim + 8 * gcol + e] =
          (red[0][c][e] + red[1][c][e]) + (red[2][c][e] + red[3][c][e]);
  }
}

// grid: ceil(B * H * 128 / 16) workgroups of 256 threads, 16 consecutive (b, h, channel)
// outputs each (so a load instruction reads 16 full 128-B lines): thread t adds the ranges
// t / 16, t / 16 + 16, ... of output t % 16, then the 16 sums of an output are added in a
// fixed order.  A single thread walking all ranges waits out one dependent load per range
// (about 150 of them at 4608 tokens); the sums are exact, so their order is free.
__global__ void __launch_bounds__(256)
k_mean_kernel(const double* __restrict__ partial, float* __restrict__ k_mean, int S, int H,
              int nchunk, int n) {
  __shared__ double red[16][17];
  const int o = threadIdx.x & 15, cl = threadIdx.x >> 4;
  const int idx = blockIdx.x * 16 + o;
  double s = 0.0;
  if (idx < n) {
    const int hc = H * kHeadDim;
    const int b = idx / hc, r = idx - b * hc;
    const double* p = partial + (int64_t)b * nchunk * hc + r;
#pragma unroll 4
    for (int c = cl; c < nchunk; c += 16) s += p[(int64_t)c * hc];
  }
  red[cl][o] = s;
  __syncthreads();
  if (cl == 0 && idx < n) {
    double t = 0.0;
#pragma unroll
    for (int c = 0; c < 16; ++c) t += red[c][o];
    k_mean[idx] = (float)(t / (double)S);
  }
}

// ---------------------------------------------------------------- V absmax
// grid: B * colblk * nchunk workgroups of 256 threads (nchunk = ceil(S / tok_per_wg),
// colblk = ceil(H * 16 / 64)), workgroup x = (b * colblk + cb) * nchunk + chunk.
// Thread t owns chunk column cb * 64 + (t & 63) (8 channels) and tokens
// j0 + (t >> 6) + 4 k: a wave reads 1 KB of one token row.  The 4 waves combine
// their maxima in LDS, then one atomicMax per channel on the fp32 bit pattern
// of |v|.  amax_bits: [B, H, 128], initialized by quant_qk_kernel, which runs first.
__global__ void __launch_bounds__(256)
v_absmax_kernel(const uint16_t* __restrict__ v, uint32_t* __restrict__ amax_bits, int S, int H,
                int tok_per_wg, int nchunk, int colblk) {
  __shared__ uint32_t red[4][64][8];
  const int chunk = blockIdx.x % nchunk;
  const int bc = blockIdx.x / nchunk;
  const int b = bc / colblk, cb = bc - b * colblk;
  const int ncol = H * 16;  // 16-byte chunks per token row (all heads)
  const int col = cb * 64 + (threadIdx.x & 63);
  const int wv = threadIdx.x >> 6;
  const int j0 = chunk * tok_per_wg;
  const int j1 = min(j0 + tok_per_wg, S);
  const int64_t tok = (int64_t)H * kHeadDim;
  uint32_t mx[8] = {0, 0, 0, 0, 0, 0, 0, 0};  // |v| as bf16 magnitude bits
  if (col < ncol) {
    const uint16_t* src = v + (int64_t)b * S * tok + 8 * col;
    for (int j = j0 + wv; j < j1; j += 16) {
      uint4 raw[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) raw[u] = (j + 4 * u < j1) ? *(const uint4*)(src + (j + 4 * u) * tok) : uint4{0, 0, 0, 0};
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const uint32_t w[4] = {raw[u].x, raw[u].y, raw[u].z, raw[u].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          mx[2 * e] = max(mx[2 * e], w[e] & 0x7FFFu);
          mx[2 * e + 1] = max(mx[2 * e + 1], (w[e] >> 16) & 0x7FFFu);
        }
      }
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) red[wv][threadIdx.x & 63][e] = mx[e];
  __syncthreads();
  // 64 columns x 8 channels = 512 maxima, two per thread
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int idx = threadIdx.x + 256 * k;
    const int c = idx >> 3, e = idx & 7;
    const uint32_t m4 = max(max(red[0][c][e], red[1][c][e]), max(red[2][c][e], red[3][c][e]));
    const int gcol = cb * 64 + c;
    // bf16 magnitude bits << 16 = fp32 bits of |v|; finite magnitudes order like integers
    if (gcol < ncol && m4 != 0u) atomicMax(amax_bits + (int64_t)b * H * kHeadDim + 8 * gcol + e, (m4 << 16) | kAmaxFlag);
  }
}

// ---------------------------------------------------------------- V quantize + transpose
constexpr int kVTok = 128;          // tokens per v_quant workgroup
constexpr int kVRowB = kVTok + 8;   // LDS row stride in bytes (channel rows)

// grid: B * H * (S_pad / kVTok) workgroups, x = bh * (S_pad / kVTok) + token chunk.
// Thread t: chunk t & 15 (8 channels), tokens 8 * (t >> 4) + 0..7.
// amax_bits doubles as the v_scale output (see the top of this file).
__global__ void __launch_bounds__(256)
v_quant_kernel(const uint16_t* __restrict__ v, uint32_t* __restrict__ amax_bits,
               uint8_t* __restrict__ v_fp8, int S, int H, int S_pad) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[kHeadDim * kVRowB];
  const int nch = S_pad / kVTok;
  const int bh = blockIdx.x / nch;
  const int tchunk = blockIdx.x - bh * nch;
  const int b = bh / H, h = bh - b * H;
  const int j0 = tchunk * kVTok;
  const int chunk = threadIdx.x & 15, tg = threadIdx.x >> 4;
  const int64_t tok = (int64_t)H * kHeadDim;
  const uint16_t* src = v + ((int64_t)b * S * H + h) * kHeadDim;

  float sv[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const uint32_t w = amax_bits[(int64_t)bh * kHeadDim + 8 * chunk + e];
    sv[e] = (w & kAmaxFlag) ? __uint_as_float(w & ~kAmaxFlag) / 448.0f : __uint_as_float(w);
  }

  float x[8][8];  // [token][channel]
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int j = j0 + 8 * tg + u;
    uint4 raw = uint4{0, 0, 0, 0};
    if (j < S) raw = *(const uint4*)(src + j * tok + 8 * chunk);
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[u][2 * e] = bf16_bits_to_f32(w[e] & 0xFFFFu);
      x[u][2 * e + 1] = bf16_bits_to_f32(w[e] >> 16);
    }
  }
  bool fast = true;
  float inv[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    fast = fast && fast_div_ok(sv[e]);
    inv[e] = 1.0f / sv[e];
  }
  // x / v_scale, 0 for tokens >= S (their codes are the zero padding)
  if (fast) {
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int e = 0; e < 8; ++e) x[u][e] = div_by_recip(x[u][e], sv[e], inv[e]);
  } else {
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int e = 0; e < 8; ++e) x[u][e] = sv[e] != 0.0f ? x[u][e] / sv[e] : 0.0f;
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {  // channel 8 * chunk + e, tokens 8 tg + 0..7
    uint32_t word[2];
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      float a[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int j = j0 + 8 * tg + 4 * half + u;
        a[u] = j < S ? x[4 * half + u][e] : 0.0f;
      }
      int wv = __builtin_amdgcn_cvt_pk_fp8_f32(a[0], a[1], 0, false);
      wv = __builtin_amdgcn_cvt_pk_fp8_f32(a[2], a[3], wv, true);
      word[half] = (uint32_t)wv;
    }
    *(uint2*)(lds + (8 * chunk + e) * kVRowB + 8 * tg) = uint2{word[0], word[1]};
  }
  __syncthreads();
  // the chunk-0 workgroup publishes the finished scales (threads 0..15 own all 128 channels)
  if (tchunk == 0 && threadIdx.x < 16) {
#pragma unroll
    for (int e = 0; e < 8; ++e) amax_bits[(int64_t)bh * kHeadDim + 8 * chunk + e] = __float_as_uint(sv[e]);
  }
  // 128 channel rows x 128 B; 8 bytes per thread per step, 16 threads per row
  uint8_t* dst = v_fp8 + (int64_t)bh * kHeadDim * S_pad + j0;
#pragma unroll
  for (int step = 0; step < 8; ++step) {
    const int idx = step * 256 + threadIdx.x;
    const int row = idx >> 4, part = idx & 15;
    *(uint2*)(dst + (int64_t)row * S_pad + 8 * part) = *(const uint2*)(lds + row * kVRowB + 8 * part);
  }
}

}  // namespace prep

namespace {

// Token ranges of v_absmax_kernel and k_colsum_kernel: about 1000 workgroups
// whatever the shape, ranges a multiple of 16 tokens.
struct Chunking {
  int tok_per_wg, nchunk, colblk;
};
Chunking chunking(int B, int S, int H) {
  Chunking c;
  c.colblk = (H * 16 + 63) / 64;
  int t = (int)(((int64_t)S * c.colblk * B + 1023) / 1024);
  t = (t + 15) / 16 * 16;
  c.tok_per_wg = t < 16 ? 16 : t;
  c.nchunk = (S + c.tok_per_wg - 1) / c.tok_per_wg;
  return c;
}

prep::RowXform row_xform(const void* norm_w, float eps, const void* cos_t, const void* sin_t,
                         int rope_dim) {
  return prep::RowXform{(const uint16_t*)norm_w, eps, (const uint16_t*)cos_t, (const uint16_t*)sin_t,
                        rope_dim};
}

}  // namespace

size_t sage_workspace_bytes(int B, int S_kv, int H_kv) {
  const Chunking ch = chunking(B, S_kv, H_kv);
  return (size_t)B * ch.nchunk * H_kv * kHeadDim * sizeof(double);
}

hipError_t launch_sage_prepare(const PrepareArgs& a, hipStream_t stream) {
  const int S_q_pad = (a.S_q + 255) / 256 * 256, S_kv_pad = (a.S_kv + 255) / 256 * 256;
  const bool xq = a.q_norm_w || a.rope_dim, xk = a.k_norm_w || a.rope_dim;
  uint32_t* amax_bits = reinterpret_cast<uint32_t*>(a.v_scale);
  const Chunking ch = chunking(a.B, a.S_kv, a.H_kv);
  hipError_t e;
  if (a.k_mean) {  // K smoothing: channel means of the (transformed) K first
    double* partial = reinterpret_cast<double*>(a.workspace);
    const prep::RowXform kx = row_xform(a.k_norm_w, a.eps, a.rope_cos, a.rope_sin, a.rope_dim);
    const dim3 grid(a.B * ch.colblk * ch.nchunk);
    e = xk ? launch(prep::k_colsum_kernel<true>, grid, dim3(256), stream, (const uint16_t*)a.k, partial,
                    a.S_kv, a.H_kv, ch.tok_per_wg, ch.nchunk, ch.colblk, kx)
           : launch(prep::k_colsum_kernel<false>, grid, dim3(256), stream, (const uint16_t*)a.k, partial,
                    a.S_kv, a.H_kv, ch.tok_per_wg, ch.nchunk, ch.colblk, kx);
    if (e != hipSuccess) return e;
    const int n = a.B * a.H_kv * kHeadDim;
    e = launch(prep::k_mean_kernel, dim3((n + 15) / 16), dim3(256), stream, (const double*)partial,
               a.k_mean, a.S_kv, a.H_kv, ch.nchunk, n);
    if (e != hipSuccess) return e;
  }
  prep::QuantSide qs{(const uint16_t*)a.q, a.q_i8, a.q_scale, nullptr, a.S_q, a.H, S_q_pad / 32,
                     a.B * a.H * (S_q_pad / 32), a.c,
                     row_xform(a.q_norm_w, a.eps, a.rope_cos, a.rope_sin, a.rope_dim)};
  prep::QuantSide ks{(const uint16_t*)a.k, a.k_i8, a.k_scale, a.k_mean, a.S_kv, a.H_kv, S_kv_pad / 32,
                     a.B * a.H_kv * (S_kv_pad / 32), 1.0f,
                     row_xform(a.k_norm_w, a.eps, a.rope_cos, a.rope_sin, a.rope_dim)};
  const int units = qs.units > ks.units ? qs.units : ks.units;
  const int n_amax = a.B * a.H_kv * kHeadDim;  // <= 64 * qs.units: the Q half covers it
  const dim3 qgrid((units + 3) / 4, 2);
  e = (xq || xk) ? launch(prep::quant_qk_kernel<true>, qgrid, dim3(256), stream, qs, ks, amax_bits, n_amax)
                 : launch(prep::quant_qk_kernel<false>, qgrid, dim3(256), stream, qs, ks, amax_bits, n_amax);
  if (e != hipSuccess) return e;
  e = launch(prep::v_absmax_kernel, dim3(a.B * ch.colblk * ch.nchunk), dim3(256), stream,
             (const uint16_t*)a.v, amax_bits, a.S_kv, a.H_kv, ch.tok_per_wg, ch.nchunk, ch.colblk);
  if (e != hipSuccess) return e;
  return launch(prep::v_quant_kernel, dim3(a.B * a.H_kv * (S_kv_pad / prep::kVTok)), dim3(256), stream,
                (const uint16_t*)a.v, amax_bits, a.v_fp8, a.S_kv, a.H_kv, S_kv_pad);
}

hipError_t launch_qk_norm_rope(const void* x, void* out, int B, int S, int H, const void* norm_w,
                               float eps, const void* cos_t, const void* sin_t, int rope_dim,
                               hipStream_t stream) {
  const int nblk = (S + 31) / 32;
  const int units = B * H * nblk;
  return launch(prep::xform_kernel, dim3((units + 3) / 4), dim3(256), stream, (const uint16_t*)x,
                (uint16_t*)out, S, H, nblk, units, row_xform(norm_w, eps, cos_t, sin_t, rope_dim));
}

}  // namespace ditattn
