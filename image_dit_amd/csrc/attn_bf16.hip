// attn_bf16.hip -- BF16 flash self-attention forward for gfx950 (MI355X).
//
// Operation: "Kernel acceleration: attention, compilation and fusion",
// section "Attention: from O(N^2) memory to blocks" -- attention computed one
// key block at a time with a running row max m, running row sum l and an
// accumulator rescaled by exp(m_old - m_new), so the S x S scores never leave
// the chip.  Shape contract (BF16 [B, S, H, 128] in and out, non-causal) from
// "gfx1201_sage_prepare / gfx1201_sage_attention", "Technical Details".
//
// gfx950 mapping
//   * Work unit: one workgroup per (b, h, BQ-row query tile); 4 waves, each
//     owning 32 * QG query rows.  Workgroups are remapped so one head's tiles
//     share an XCD (and its L2) while they stream the same K/V.
//   * Scores are computed transposed, S^T = K Q^T, on
//     v_mfma_f32_32x32x16_bf16: A = 32 keys x 16 channels read from LDS,
//     B = 16 channels x 32 queries kept in registers for the whole loop.  In
//     the accumulator every lane then owns ONE query row (column l % 32) and 16
//     of its keys, so row max / row sum are per-lane loops plus one
//     permlane32_swap with the other half-wave.
//   * O^T = V^T P^T on the same MFMA: the accumulator registers of S^T, rounded
//     to BF16, are exactly the B operand (same lane = same query, same keys),
//     so P never goes through LDS.  The A operand V^T (channels x keys) is read
//     from the row-major V tile with ds_read_b64_tr_b16, which transposes 16-bit
//     elements inside groups of 16 lanes.
//   * K/V tiles of BK = 64 keys are double-buffered in LDS (one barrier per
//     tile).  Rows are 256 B, unpadded, with 16-byte chunks XOR-swizzled per row
//     so that both the MFMA-operand reads and the transposed reads are free of
//     bank conflicts.
//   * Softmax in base 2: x = s * c with c = scale * log2(e); exp2 on v_exp_f32.
//     The running max is only raised when a row's tile max exceeds it by more
//     than kLazyThresh (in log2 units): P values up to 2^kLazyThresh are
//     harmless in BF16/FP32, and the O rescale (64 multiplies per lane and
//     query group) is skipped on almost every tile.  The result is the same
//     math: every p and l use the same stale max, which cancels in acc / l.
//   * Ragged tail: key rows >= S are zero-filled in LDS and their scores set to
//     -inf; query rows >= S are computed on zeros and not stored.
#include <type_traits>

#include "common.hpp"

namespace ditattn {
namespace bf16attn {

// Tuning knobs (compile-time; defaults are the measured choice).
#ifndef DITATTN_BF16_OCC
#define DITATTN_BF16_OCC 1  // workgroups per CU the register budget is sized for
#endif
#ifndef DITATTN_BF16_QG
#define DITATTN_BF16_QG 1   // 32-row query groups per wave
#endif

#ifndef DITATTN_BF16_NW
#define DITATTN_BF16_NW 8   // waves per workgroup (all share one K/V tile); 2 per SIMD
#endif
#ifndef DITATTN_BF16_NSTAGE
#define DITATTN_BF16_NSTAGE 2  // K/V tiles resident in LDS (copies run NSTAGE - 1 tiles ahead)
#endif

constexpr int BK = 64;      // keys per K/V tile
constexpr int NW = DITATTN_BF16_NW;
constexpr int RPW = BK / NW;   // tile rows each wave copies
constexpr int NCP = RPW / 4;   // 1 KB copy instructions per wave per tile (K or V)
constexpr int NSTAGE = DITATTN_BF16_NSTAGE;
static_assert(NSTAGE >= 2 && NSTAGE <= 4, "LDS holds at most 4 stages of 32 KB");
constexpr int ROW_CHUNKS = 16;  // 16-byte chunks per 128-channel BF16 row
constexpr float kLazyThresh = 8.0f;


// Byte layout of the LDS ring: [buf][K | V][64 rows x 256 B].
constexpr int TILE_BYTES = BK * 256;
constexpr int BUF_BYTES = 2 * TILE_BYTES;

template <int QG>
__global__ void __launch_bounds__(NW * 64, DITATTN_BF16_OCC)
attn_fwd_bf16_kernel(const __bf16* __restrict__ q, const __bf16* __restrict__ k,
                     const __bf16* __restrict__ v, __bf16* __restrict__ o, int S, int H, float c,
                     int num_qt, int n_tiles) {
  constexpr int BQ = NW * QG * 32;
  __shared__ __attribute__((aligned(16))) char lds[NSTAGE * BUF_BYTES];

  const int L = xcd_remap(blockIdx.x, n_tiles);
  const int bh = L / num_qt;
  const int qt = L - bh * num_qt;
  const int b = bh / H, h = bh - b * H;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l = tid & 63, hl = l >> 5, ln = l & 31;
  const int64_t tok = (int64_t)H * kHeadDim;  // elements between consecutive tokens
  const uint32_t tok_bytes = (uint32_t)(tok * 2);
  const int64_t base = ((int64_t)b * S * H + h) * kHeadDim;
  const __bf16* qbh = q + base;
  const char* kbh = (const char*)(k + base);
  const char* vbh = (const char*)(v + base);
  __bf16* obh = o + base;

  // Q^T operand, resident for the whole key loop: Q[q0 + 32 g + ln][16 ks + 8 hl + 0..7].
  const int q0 = qt * BQ + wave * QG * 32;
  bf16x8 qf[QG][8];
#pragma unroll
  for (int g = 0; g < QG; ++g) {
    const int i = q0 + 32 * g + ln;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      if (i < S) qf[g][ks] = *(const bf16x8*)(qbh + i * tok + 16 * ks + 8 * hl);
      else qf[g][ks] = bf16x8{};
    }
  }

  f32x16 acc[QG][4];
  float m[QG], lsum[QG];
#pragma unroll
  for (int g = 0; g < QG; ++g) {
    m[g] = -INFINITY;
    lsum[g] = 0.0f;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) acc[g][dt] = f32x16{};
  }

  // ---- global -> LDS (direct).  Wave w, instruction n writes LDS rows RPW w + 4 n + l / 16,
  // physical chunk l % 16; the lane fetches the logical chunk that lands there.
  const int p_chunk = l & 15;
  uint32_t koff[NCP], voff[NCP];  // this lane's source offsets in a full tile
#pragma unroll
  for (int n = 0; n < NCP; ++n) {
    const int r = RPW * wave + 4 * n + (l >> 4);
    koff[n] = r * tok_bytes + 16u * (uint32_t)(p_chunk ^ (r & 15));
    voff[n] = r * tok_bytes + 16u * (uint32_t)(p_chunk ^ ((r & 3) << 2));
  }
  auto issue_tile = [&](int t, int buf, bool clamp) {
    const int j0 = t * BK;
    const char* kt = kbh + (int64_t)j0 * tok * 2;
    const char* vt = vbh + (int64_t)j0 * tok * 2;
#pragma unroll
    for (int n = 0; n < NCP; ++n) {
      uint32_t ko = koff[n], vo = voff[n];
      if (clamp) {  // rows past the end repeat the last real key
        const int r = RPW * wave + 4 * n + (l >> 4);
        const int rr = (j0 + r >= S) ? S - 1 - j0 : r;
        ko = rr * tok_bytes + 16u * (uint32_t)(p_chunk ^ (r & 15));
        vo = rr * tok_bytes + 16u * (uint32_t)(p_chunk ^ ((r & 3) << 2));
      }
      char* kdst = lds + buf * BUF_BYTES + (RPW * wave + 4 * n) * 256;
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(kt + ko),
                                       (DITATTN_LDS void*)kdst, 16, 0, 0);
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(vt + vo),
                                       (DITATTN_LDS void*)(kdst + TILE_BYTES), 16, 0, 0);
    }
  };

  // ---- per-lane LDS read offsets (bytes, relative to the tile), constant over the loop
  // K (A operand of S^T): row 32 tt + ln, logical chunk 2 ks + hl, physical chunk ^ (row & 15).
  uint32_t kofs[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) kofs[ks] = ln * 256 + 16 * ((2 * ks + hl) ^ (ln & 15));
  // V (A operand of O^T, transposed read): lane j of its 16-lane group addresses
  // row 16 cc + 8 E + 4 hl + j / 4, columns 32 dt + 16 (group & 1) + 4 (j & 3) .. + 3.
  uint32_t vofs[4];
  {
    const int grp = l >> 4, j = l & 15, qrow = j >> 2;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      const int col = 32 * dt + 16 * (grp & 1) + 4 * (j & 3);
      vofs[dt] = (4 * hl + qrow) * 256 + 16 * ((col >> 3) ^ (qrow << 2)) + (col & 7) * 2;
    }
  }

  const int n_kt = (S + BK - 1) / BK;
  const bool ragged = (S % BK) != 0;

  // One key tile: S^T = K Q^T, online softmax, O^T += V^T P^T.
  // One key tile from LDS buffer `buf` (a constant in the main loop, a runtime
  // value for the last tile, which always goes through one code path so that
  // nothing is merged between its last MFMA and the epilogue).
  auto tile = [&](auto buf_v, auto tail_c, int t) {
    constexpr bool tail = decltype(tail_c)::value;
    const int buf = buf_v;
    const char* kb = lds + buf * BUF_BYTES;
    const char* vb = kb + TILE_BYTES;

    f32x16 s[2][QG];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int g = 0; g < QG; ++g) s[tt][g] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const bf16x8 kf = *(const DITATTN_LDS bf16x8*)((const DITATTN_LDS char*)kb + kofs[ks] + tt * 32 * 256);
#pragma unroll
        for (int g = 0; g < QG; ++g) s[tt][g] = mfma_bf16_32x32x16(kf, qf[g][ks], s[tt][g]);
      }
    }
    if constexpr (tail) {
      if (ragged) {
        const int j0 = t * BK;
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int j = j0 + 32 * tt + 8 * (r >> 2) + 4 * hl + (r & 3);
#pragma unroll
            for (int g = 0; g < QG; ++g)
              if (j >= S) s[tt][g][r] = -INFINITY;
          }
      }
    }

    bf16x8 pf[QG][4];
#pragma unroll
    for (int g = 0; g < QG; ++g) {
      float mx = fmaxf(s[0][g][0], s[1][g][0]);
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = max3(mx, s[0][g][r], s[1][g][r]);
      mx = half_pair_max(mx) * c;
      // raise the running max only when it grew by more than the threshold
      if (__builtin_amdgcn_ballot_w64(mx > m[g] + kLazyThresh) != 0) {
        const float m_new = fmaxf(m[g], mx);
        const float alpha = fast_exp2(m[g] - m_new);
        m[g] = m_new;
        lsum[g] *= alpha;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) acc[g][dt] *= alpha;
      }
      const float mneg = -m[g];
      float p[32];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int r = 0; r < 16; ++r) p[16 * tt + r] = fast_exp2(fmaf(s[tt][g][r], c, mneg));
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) {
        bf16x8 pv;
#pragma unroll
        for (int e = 0; e < 8; ++e) pv[e] = (__bf16)p[8 * cc + e];
        pf[g][cc] = pv;
      }
      lsum[g] += tree_sum<32>(p);
    }

    // V^T fragments, one 16-key chunk at a time (4 channel tiles x 2 transposed
    // reads), double-buffered so the next chunk's reads overlap this chunk's MFMAs.
    const uint32_t vaddr = (uint32_t)(uintptr_t)(const DITATTN_LDS char*)vb;
    u32x2 fa[4][2], fb[4][2];
    auto vread = [&](auto cc_c, u32x2 (&f)[4][2]) {
      constexpr int cc = decltype(cc_c)::value;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        f[dt][0] = ds_read_tr16_b64<(16 * cc) * 256>(vaddr + vofs[dt]);
        f[dt][1] = ds_read_tr16_b64<(16 * cc + 8) * 256>(vaddr + vofs[dt]);
      }
    };
    auto pv_chunk = [&](auto cc_c, u32x2 (&f)[4][2]) {
      constexpr int cc = decltype(cc_c)::value;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        const bf16x8 va = __builtin_bit_cast(bf16x8, u32x4{f[dt][0][0], f[dt][0][1], f[dt][1][0], f[dt][1][1]});
#pragma unroll
        for (int g = 0; g < QG; ++g) acc[g][dt] = mfma_bf16_32x32x16(va, pf[g][cc], acc[g][dt]);
      }
    };
    using C0 = std::integral_constant<int, 0>;
    using C1 = std::integral_constant<int, 1>;
    using C2 = std::integral_constant<int, 2>;
    using C3 = std::integral_constant<int, 3>;
    vread(C0{}, fa);
    vread(C1{}, fb);
    lds_wait<8>(fa[0][0], fa[0][1], fa[1][0], fa[1][1], fa[2][0], fa[2][1], fa[3][0], fa[3][1]);
    pv_chunk(C0{}, fa);
    vread(C2{}, fa);
    lds_wait<8>(fb[0][0], fb[0][1], fb[1][0], fb[1][1], fb[2][0], fb[2][1], fb[3][0], fb[3][1]);
    pv_chunk(C1{}, fb);
    vread(C3{}, fb);
    lds_wait<8>(fa[0][0], fa[0][1], fa[1][0], fa[1][1], fa[2][0], fa[2][1], fa[3][0], fa[3][1]);
    pv_chunk(C2{}, fa);
    lds_wait<0>(fb[0][0], fb[0][1], fb[1][0], fb[1][1], fb[2][0], fb[2][1], fb[3][0], fb[3][1]);
    pv_chunk(C3{}, fb);
  };

  using Full = std::integral_constant<bool, false>;
  using Last = std::integral_constant<bool, true>;
  const int n_main = n_kt - 1;  // tiles before the last one
  constexpr int kCopies = 2 * NCP;  // copy instructions per wave per tile

  // Prologue: tiles 0 .. NSTAGE-2 in flight, wait for all of them once.
#pragma unroll
  for (int p = 0; p < NSTAGE - 1; ++p)
    if (p < n_kt) issue_tile(p, p, p == n_kt - 1);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  // Iteration t: refill the stage freed by tile t-1 with tile t+NSTAGE-1, compute
  // tile t, then wait until this wave's copies of tile t+1 have landed.
  auto step = [&](auto buf_c, int t) {
    constexpr int buf = decltype(buf_c)::value;
    const int nxt = t + NSTAGE - 1;
    const bool refill = nxt < n_kt;
    if (refill) issue_tile(nxt, (buf + NSTAGE - 1) % NSTAGE, nxt == n_kt - 1);
    tile(buf_c, Full{}, t);
    if (refill) {
      asm volatile("s_waitcnt vmcnt(%0)" ::"i"((NSTAGE - 2) * kCopies) : "memory");
    } else {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    __syncthreads();
  };
  // NSTAGE tiles per trip so the stage offsets are immediates; the trip is
  // left as soon as only the last tile remains.
  int t = 0;
  while (true) {
    if (t >= n_main) break;
    step(std::integral_constant<int, 0>{}, t++);
    if (t >= n_main) break;
    step(std::integral_constant<int, 1>{}, t++);
    if constexpr (NSTAGE > 2) {
      if (t >= n_main) break;
      step(std::integral_constant<int, 2 % NSTAGE>{}, t++);
    }
    if constexpr (NSTAGE > 3) {
      if (t >= n_main) break;
      step(std::integral_constant<int, 3 % NSTAGE>{}, t++);
    }
  }
  tile(t % NSTAGE, Last{}, t);  // the last tile (masked when S is ragged)

  // ---- epilogue: O = acc / l, BF16, rows < S
#pragma unroll
  for (int g = 0; g < QG; ++g) mfma_drain(acc[g][0], acc[g][1], acc[g][2], acc[g][3]);
#pragma unroll
  for (int g = 0; g < QG; ++g) {
    const float inv = 1.0f / half_pair_sum(lsum[g]);
    const int i = q0 + 32 * g + ln;
    if (i < S) {
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          const int d = 32 * dt + 8 * rq + 4 * hl;
          bf16x4 ov;
#pragma unroll
          for (int e = 0; e < 4; ++e) ov[e] = (__bf16)(acc[g][dt][4 * rq + e] * inv);
          *(bf16x4*)(obh + i * tok + d) = ov;
        }
    }
  }
}

}  // namespace bf16attn

// Query rows per workgroup of the launched configuration.
constexpr int kBf16QG = DITATTN_BF16_QG;
constexpr int kBf16BQ = bf16attn::NW * kBf16QG * 32;

int bf16_tile_rows() { return kBf16BQ; }

hipError_t launch_attn_fwd_bf16(const void* q, const void* k, const void* v, void* o, int B,
                                int S, int H, float c, hipStream_t stream) {
  const int num_qt = (S + kBf16BQ - 1) / kBf16BQ;
  const int n_tiles = B * H * num_qt;
  hipLaunchKernelGGL(bf16attn::attn_fwd_bf16_kernel<kBf16QG>, dim3(n_tiles), dim3(bf16attn::NW * 64),
                     0, stream, (const __bf16*)q, (const __bf16*)k, (const __bf16*)v, (__bf16*)o, S,
                     H, c, num_qt, n_tiles);
  return hipGetLastError();
}

}  // namespace ditattn
