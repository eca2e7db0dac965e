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

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x = fmaxf(x, __shfl_xor(x, off, 64));
  return x;
}

// ---------------------------------------------------------------- Q and K
// grid.x: ceil(B * H * nblk / 4) workgroups of 4 waves; grid.y: 0 = Q, 1 = K.
__global__ void __launch_bounds__(256)
quant_qk_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                int8_t* __restrict__ q_i8, float* __restrict__ q_scale, int8_t* __restrict__ k_i8,
                float* __restrict__ k_scale, int S, int H, int nblk, int units, float c,
                uint32_t* __restrict__ amax_bits, int n_amax) {
  // initialize the V absmax accumulator (flagged +0) for v_absmax_kernel, which runs
  // next on the stream; the first ceil(n_amax / 256) workgroups of the Q half do it
  {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (blockIdx.y == 0 && i < n_amax) amax_bits[i] = kAmaxFlag;
  }

  const bool is_q = blockIdx.y == 0;
  const uint16_t* x = is_q ? q : k;
  int8_t* codes = is_q ? q_i8 : k_i8;
  float* scales = is_q ? q_scale : k_scale;
  const float mult = is_q ? c : 1.0f;  // x * 1.0f is exact

  const int unit = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (unit >= units) return;
  const int lane = threadIdx.x & 63;
  const int blk = unit % nblk;
  const int bh = unit / nblk;
  const int b = bh / H, h = bh - b * H;
  const int64_t tok = (int64_t)H * kHeadDim;
  const uint16_t* src = x + ((int64_t)b * S * H + h) * kHeadDim;

  // lane owns 8 channels (chunk lane & 15) of rows (lane >> 4) + 4 p, p = 0..7
  const int chunk = lane & 15;
  float y[8][8];
  float amax = 0.0f;
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    const int i = blk * 32 + (lane >> 4) + 4 * p;
    uint4 raw = uint4{0, 0, 0, 0};
    if (i < S) raw = *(const uint4*)(src + i * tok + 8 * chunk);
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      y[p][2 * e] = bf16_bits_to_f32(w[e] & 0xFFFFu) * mult;
      y[p][2 * e + 1] = bf16_bits_to_f32(w[e] >> 16) * mult;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(y[p][e]));
  }
  amax = wave_max(amax);
  const float s = amax / 127.0f;
  int8_t* dst = codes + ((int64_t)bh * nblk * 32 + blk * 32) * kHeadDim;
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    const int r = (lane >> 4) + 4 * p;
    uint32_t packed[2] = {0u, 0u};
    if (s != 0.0f) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float qv = rintf(y[p][e] / s);
        qv = fminf(fmaxf(qv, -127.0f), 127.0f);
        packed[e >> 2] |= ((uint32_t)(int)qv & 0xFFu) << (8 * (e & 3));
      }
    }
    *(uint2*)(dst + r * kHeadDim + 8 * chunk) = uint2{packed[0], packed[1]};
  }
  if (lane == 0) scales[(int64_t)bh * nblk + blk] = s;
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
#pragma unroll
  for (int e = 0; e < 8; ++e) {  // channel 8 * chunk + e, tokens 8 tg + 0..7
    uint32_t word[2];
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      float a[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int j = j0 + 8 * tg + 4 * half + u;
        a[u] = (j < S && sv[e] != 0.0f) ? x[4 * half + u][e] / sv[e] : 0.0f;
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

hipError_t launch_sage_prepare(const void* q, const void* k, const void* v, int8_t* q_i8,
                               float* q_scale, int8_t* k_i8, float* k_scale, uint8_t* v_fp8,
                               float* v_scale, int B, int S, int H, int S_pad, float c,
                               hipStream_t stream) {
  const int nblk = S_pad / 32;
  const int units = B * H * nblk;
  const int nscale = B * H * kHeadDim;  // <= units: the Q half of quant_qk covers it
  uint32_t* amax_bits = reinterpret_cast<uint32_t*>(v_scale);
  hipError_t e = launch(prep::quant_qk_kernel, dim3((units + 3) / 4, 2), dim3(256), stream,
                        (const uint16_t*)q, (const uint16_t*)k, q_i8, q_scale, k_i8, k_scale, S, H,
                        nblk, units, c, amax_bits, nscale);
  if (e != hipSuccess) return e;
  // V absmax: about 1000 workgroups whatever the shape, token ranges a multiple of 16
  const int colblk = (H * 16 + 63) / 64;
  int tok_per_wg = (int)(((int64_t)S * colblk * B + 1023) / 1024);
  tok_per_wg = (tok_per_wg + 15) / 16 * 16;
  if (tok_per_wg < 16) tok_per_wg = 16;
  const int nchunk = (S + tok_per_wg - 1) / tok_per_wg;
  e = launch(prep::v_absmax_kernel, dim3(B * colblk * nchunk), dim3(256), stream, (const uint16_t*)v,
             amax_bits, S, H, tok_per_wg, nchunk, colblk);
  if (e != hipSuccess) return e;
  return launch(prep::v_quant_kernel, dim3(B * H * (S_pad / prep::kVTok)), dim3(256), stream,
                (const uint16_t*)v, amax_bits, v_fp8, S, H, S_pad);
}

}  // namespace ditattn
