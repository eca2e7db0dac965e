// attn_sage.hip -- Sage attention forward for gfx950 on tensors written by
// sage_prepare / sage_prepare_ex: Q K^T on INT8 MFMA, P V on FP8 (OCP e4m3)
// MFMA, FP32 accumulation, online softmax in base 2, BF16 output.
//
// Operation: "gfx1201_sage_prepare / gfx1201_sage_attention" (aiter PR 6390),
// second commit and "Technical Details": the kernel alone on prepared tensors,
// head dim 128.  Online softmax as in "Kernel acceleration: attention,
// compilation and fusion", section "Attention: from O(N^2) memory to blocks".
// Beyond the page's non-causal self-attention: S_q != S_kv (cross-attention),
// H a multiple of H_kv (grouped-query heads) and an optional key window per
// query (causal and sliding-window masks), as listed in the "Features" table of
// the "RDNAttention" README.
//
// gfx950 mapping
//   * Workgroup = 8 waves x 32 query rows (BQ = 256) of one (b, h), all reading
//     the same K/V tiles of BK = 64 keys from LDS, copied global -> LDS
//     directly through a three-stage ring.  XCD-aware tile order.
//   * S^T = K Q^T on v_mfma_i32_32x32x32_i8 (exact int32: |acc| <= 128 * 127^2
//     < 2^21).  Q codes stay in registers.  Key rows are fed to the A operand in
//     an order that gives each half-wave 32 consecutive keys, i.e. one 32-row K
//     block and one k_scale: a lane's scores are x = acc * s with
//     s = q_scale * k_scale, already in base-2 units.  The accumulators start
//     at the bit pattern of 1/(2 pi), so an int32 sum read
//     as fp32 is exactly 1/(2 pi) + score * 2^-26: the row max is taken on those
//     bit patterns, and the base-2 argument x = score * s - m + 8 of p * 2^8 is
//     one FMA on them, no conversion.
//   * P's e4m3 codes come from x directly, with no exponential: inside one
//     octave the e4m3 values are evenly spaced, 2^(E-7) (1 + M/8), so the code
//     8 E + M = 8 (x + 7), rounded, is the e4m3 number with exponent floor(x)
//     and mantissa frac(x) in eighths: 2^x with its in-octave factor 2^f taken
//     as 1 + f (at most 6.2 % high).  One FMA makes 8 x + 56 less a centring
//     offset of 0.35 code steps and one v_cvt_pk_u8_f32 rounds it into its
//     byte (clamped at 0: p * 2^8 below 2^-7 becomes 0).  Two vector
//     instructions per score instead of FMA, exp2 and half an FP8 packing;
//     the relative L2 error of O against exact attention rises from about
//     0.042 to 0.045 (gate 0.05).  That FMA cancels a constant that grows with
//     the scales; a workgroup whose q_scale * k_scale exceeds 2^-8 on some tile
//     (|q|, |k| in the tens and beyond) takes the score out of the pattern
//     first and clamps the argument at 126 (code 127 is NaN).
//   * Matrix phase reads are issued as explicit LDS instructions ahead of the
//     MFMAs that take them: four K fragments, the tile's k_scale pair and two
//     V^T fragments at the start of the phase, then one K fragment (later two
//     V^T fragments) after each MFMA.  Each MFMA waits only for its own operands
//     (LDS reads return in issue order), so the phase pays about one LDS latency
//     instead of one per fragment, as the compiler's own placement did.
//   * P V on v_mfma_scale_f32_32x32x64_f8f6f4 (e4m3 operands, unit block
//     scales): A = V^T tile (channels x 64 keys) from LDS, B = P from registers
//     (the S^T accumulator of a lane already holds the B operand's keys).
//   * P is stored as p * 2^8 in e4m3; the running max is raised lazily (only
//     when a row's tile max exceeds it by more than 0.8 in base-2 units), so
//     p * 2^8 <= 2^8.8 = 445.7 < 448.  The row sum l comes from one more FP8
//     MFMA with the same P: the matrix unit has slack here and the vector unit
//     has none, and numerator and denominator then use the same rounded P.  It
//     is a 16x16x128 product (half the cycles of a 32x32x64 one) that reads P in
//     place as its B operand, with a constant 0 / 1 A operand that sums, for each
//     output row block, the two lane groups holding one query's keys; every lane
//     gets its own query's l (exact sums of e4m3 values).  O = acc * v_scale / l.
//   * Two wave groups ping-pong on each SIMD (waves w and w + 4 share one):
//     one group's matrix phase (the row sums of the previous tile's P while
//     the first K fragments are read, K Q^T of this tile, then P V of the
//     previous one; the last phase takes the row sums after its P V) runs under
//     the other group's softmax (mask and row max of the new scores, then the
//     P codes).  Both phases are issue-bound: a single
//     wave issues at most one vector instruction every few cycles and reads
//     LDS at roughly 1 KB per 40 cycles, so each phase is bound by one wave's
//     issue and LDS rates, not by the vector unit's width.  Only one wave per
//     SIMD uses the matrix core at a time: splitting P V into the softmax
//     phase was measured slower (the two waves' MFMA chains then collide).
//   * Masks: keys j >= S_kv (zero codes, which would score 0) and keys outside
//     a query's window get p = 0.  Only tiles that cross a mask boundary for
//     some row of the workgroup take the masked path; a row with no visible
//     key writes zeros.
//   * Split tail (sage_attn_fwd_split_kernel, entry point sage_attn_fwd_ws): the
//     same body run over the work items of split_tail_items (common.hpp), one
//     workgroup per CU, when the last round of query tiles is partial: pieces
//     of a query tile leave FP32 (acc, m, l) partials that the piece holding
//     the tile's last key tile merges.  It keeps the mask and row max at the end
//     of the matrix phase (in the softmax phase they cost it 2 spilled VGPRs).
#include <stdint.h>

#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace ditattn {
namespace sageattn {

constexpr int BK = 64;
constexpr int NW = 8;
constexpr int BQ = NW * 32;
constexpr float kPScaleLog2 = 8.0f;  // P is stored as p * 2^8
// The running max is raised only when a row's tile max exceeds it by more than
// this (base-2 units).  P then stays <= 2^0.8, so p * 2^8 <= 445.7 fits e4m3.
constexpr float kLazyThresh = 0.8f;
// e4m3 code of p * 2^8 = 2^x: 8 (x + 7) (eight codes per octave, exponent bias 7), less 0.35 of a
// code step, which centres the error of the in-octave factor 1 + f against 2^f (0 to +0.69 steps).
constexpr float kCodeSlope = 8.0f;
constexpr float kCodeOffset = 56.0f - 0.35f;
// Largest 8 s (code steps per int32 score unit times 2^26) for which the one-FMA code argument is
// exact to about a fiftieth of a code step: kSeed * kFastS8 * 2^-24 = 0.02.
constexpr float kFastS8 = 0x1p21f;
// K Q^T accumulator seed: the bit pattern of 1/(2 pi) (0x3E22F983).  Its mantissa field, 2293123,
// stays inside [0, 2^23) after adding any score (|score| <= 128 * 127^2 = 2064512): the int32
// sum read as fp32 is exactly kSeed + score * 2^-26.
constexpr uint32_t kSeedBits = 0x3E22F983u;
constexpr float kSeed = __builtin_bit_cast(float, kSeedBits);
constexpr float kScoreUnit = 0x1p26f;  // a seeded score moves in steps of 2^-26

// LDS tiles (bytes):  K: 64 key rows x 128 B, 16-B chunk c of row r stored at c ^ ((r >> 1) & 7).
//                     V^T: 128 channel rows x 64 B, chunk c of row r at c ^ ((r >> 2) & 3).
constexpr int KT_BYTES = BK * 128;
constexpr int VT_BYTES = 128 * BK;
constexpr int NSTAGE = 3;  // copy ring depth
constexpr int K_STAGE0 = 0;
constexpr int V_STAGE0 = NSTAGE * KT_BYTES;
constexpr int KS_STAGE0 = NSTAGE * (KT_BYTES + VT_BYTES);  // the tile's two k_scale values, 16 B per stage

// Accumulator row m of sub-tile tt holds key 32 * ((m >> 2) & 1) + 16 tt + 4 (m >> 3) + (m & 3)
// of the 64-key tile.  Then register r of a lane in half hl holds key 32 hl + 16 tt + r: P's
// 32 FP8 bytes of a lane are 32 consecutive keys and V^T is read with two 16-byte loads.
__device__ __forceinline__ int key_of_row(int m, int tt) { return 32 * ((m >> 2) & 1) + 16 * tt + 4 * (m >> 3) + (m & 3); }

// half_pair_max for values that are never NaN: one v_max_f32, without the canonicalizing
// moves fmaxf adds.
__device__ __forceinline__ float half_pair_max_nc(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  float y;
  asm("v_max_f32 %0, %1, %2" : "=v"(y) : "v"(__uint_as_float(r[0])), "v"(__uint_as_float(r[1])));
  return y;
}

// First and last key query row i sees (an empty range when hi < lo).
__device__ __forceinline__ int key_lo(const SageArgs& a, int i) {
  if (a.wl < 0) return 0;
  const int64_t lo = (int64_t)i + a.S_kv - a.S_q - a.wl;
  return (int)(lo < 0 ? 0 : (lo > a.S_kv ? a.S_kv : lo));
}
__device__ __forceinline__ int key_hi(const SageArgs& a, int i) {
  if (a.wr < 0) return a.S_kv - 1;
  const int64_t hi = (int64_t)i + a.S_kv - a.S_q + a.wr;
  return (int)(hi < -1 ? -1 : (hi > a.S_kv - 1 ? a.S_kv - 1 : hi));
}

static_assert(NW * 64 == kSplitThreads && BQ == 256 && BK == 64,
              "the split-tail plan and slots assume the BF16 kernel's tiling");

template <bool SK>
__device__ __forceinline__ void sage_body(const SageArgs& a) {
  __shared__ __attribute__((aligned(16))) char lds[NSTAGE * (KT_BYTES + VT_BYTES) + NSTAGE * 16];  // 48 KB
  __shared__ int large_w[NW];  // per wave: the large-scale code path is needed
  __shared__ __attribute__((aligned(16))) float vsc_lds[kHeadDim];  // this tile's v_scale

  // One query tile L: the key tiles its window covers (tb < 0), or the tiles [tb, te) of a split
  // tail, ending by mode: kSplitFull writes O, kSplitPartial writes (acc, m, l) to the
  // workgroup's slot and raises its flag, kSplitOwner first merges the slots of workgroups
  // p_lo .. p_hi, then writes O.
  auto run = [&](int L, int tb, int te, int mode, int p_lo, int p_hi) __attribute__((always_inline)) {
  const int bh = L / a.num_qt;
  int qt = L - bh * a.num_qt;
  if (a.reverse) qt = a.num_qt - 1 - qt;  // longest key ranges first (causal)
  const int b = bh / a.H, h = bh - b * a.H;
  const int bhk = b * a.H_kv + h / (a.H / a.H_kv);
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l = tid & 63, hl = l >> 5, ln = l & 31;
  const int nblk_q = a.S_q_pad / 32, nblk_k = a.S_kv_pad / 32;

  const int8_t* qbh = a.q_i8 + (int64_t)bh * a.S_q_pad * kHeadDim;
  const char* kbh = (const char*)(a.k_i8 + (int64_t)bhk * a.S_kv_pad * kHeadDim);
  const char* vbh = (const char*)(a.v_fp8 + (int64_t)bhk * kHeadDim * a.S_kv_pad);
  const float* ksc = a.k_scale + (int64_t)bhk * nblk_k;

  // Q codes (B operand), resident: Q[q0 + ln][32 ks + 16 hl + 0..15].  Rows < S_q_pad always.
  const int q0 = qt * BQ + wave * 32;
  const int qi = q0 + ln;  // this lane's query row
  i32x4 qf[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) qf[ks] = *(const i32x4*)(qbh + (int64_t)qi * kHeadDim + 32 * ks + 16 * hl);
  // q_scale * 2^26: s_tile below is then one product (the power of two is exact)
  const float sq = a.q_scale[(int64_t)bh * nblk_q + q0 / 32] * kScoreUnit;

  // ---- key range.  Query i sees keys j with lo(i) <= j <= hi(i): lo = i + off - wl (wl >= 0),
  // hi = i + off + wr (wr >= 0), off = S_kv - S_q, both clamped to [0, S_kv - 1] (computed in
  // 64 bits).  The workgroup visits the tiles holding a key that one of its rows < S_q sees.
  const int i_first = qt * BQ, i_last = min(qt * BQ + BQ - 1, a.S_q - 1);
  const int lo_i = key_lo(a, qi), hi_i = key_hi(a, qi);
  const int lo_first = key_lo(a, i_first), lo_last = key_lo(a, i_last);
  const int hi_first = key_hi(a, i_first), hi_last = key_hi(a, i_last);
  const int t0 = tb >= 0 ? tb : lo_first / BK;
  const int t1 = tb >= 0 ? te : (hi_last >= 0 ? hi_last / BK + 1 : 0);
  const int n = t1 - t0;  // tiles this workgroup visits (uniform)
  // a tile needs no mask when every key of it is visible to every row of the workgroup
  auto masked_tile = [&](int t) __attribute__((always_inline)) { return t * BK < lo_last || t * BK + BK - 1 > hi_first; };

  f32x16 acc[4];  // O^T: channels 32 dt + (accumulator row), this lane's query
  f32x4 lacc;     // row sum l of this lane's query (in each of the four)
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) acc[dt] = f32x16{};
  lacc = f32x4{};
  float m = -INFINITY;
  // Kept with m (which changes only when the running max is raised): m + kLazyThresh, and the
  // code offset kCodeOffset + 8 (8 - m) (kCodeOffset while a row has no visible key, m = -inf).
  float m_thr = -INFINITY, mneg = kCodeOffset;
  const int unit_scale = unit_e8m0_scale();
  // Row sums on one 16x16x128 FP8 MFMA that reads P in place as its B operand: lane L is then
  // column L % 16 and holds 32 of the 128 k values, its k group L / 16 (the same grouping for A).
  // Query q < 16 sits in lanes q (keys 0-31) and q + 32 (keys 32-63), k groups 0 and 2; query
  // 16 + q in lanes 16 + q and 48 + q, groups 1 and 3.  Output row block i / 4 lands in lanes
  // 16 (i / 4) .. + 15, whose query is q for even blocks and 16 + q for odd ones, so A row i is
  // e4m3 1.0 on the k groups of the matching parity and 0 elsewhere: lane L of A (row L % 16,
  // group L / 16) holds ones when (L / 16) % 2 == (L % 16 / 4) % 2.
  const int rsel = ((l >> 4) & 1) == ((l >> 2) & 1) ? 0x38383838 : 0;
  i32x8 lsel = {rsel, rsel, rsel, rsel, rsel, rsel, rsel, rsel};
  asm volatile("" : "+v"(lsel));  // kept in registers (else rebuilt before every row-sum MFMA)

  if (n > 0) {
    // ---- global -> LDS (direct); every lane fetches the chunk that lands in its LDS slot.
    // K: wave w fills rows 8 w .. 8 w + 7 (1 KB), lane -> row 8 w + l / 8, slot l % 8.
    // V^T: wave w fills channel rows 16 w .. 16 w + 15, lane -> row 16 w + l / 4, slot l % 4.
    // Tiles never reach past S_kv_pad, where the codes are zero.
    const int kr = 8 * wave + (l >> 3), vr = 16 * wave + (l >> 2);
    const uint32_t kgo = kr * 128 + 16 * ((l & 7) ^ ((kr >> 1) & 7));
    const uint32_t vgo = vr * a.S_kv_pad + 16 * ((l & 3) ^ ((vr >> 2) & 3));
    // The k_scale values of the tile's two 32-key blocks travel with its K rows (lanes 0, 1 of
    // wave 0), so the softmax reads them from LDS instead of waiting on a global load.
    auto issue_k = [&](int t, int stage) __attribute__((always_inline)) {
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(kbh + (int64_t)t * BK * kHeadDim + kgo),
                                       (DITATTN_LDS void*)(lds + K_STAGE0 + stage * KT_BYTES + wave * 1024), 16, 0, 0);
      if (wave == 0 && l < 2)
        __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(ksc + 2 * t + l),
                                         (DITATTN_LDS void*)(lds + KS_STAGE0 + stage * 16), 4, 0, 0);
    };
    auto issue_v = [&](int t, int stage) __attribute__((always_inline)) {
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(vbh + t * BK + vgo),
                                       (DITATTN_LDS void*)(lds + V_STAGE0 + stage * VT_BYTES + wave * 1024), 16, 0, 0);
    };

    // ---- per-lane LDS read offsets
    // K (A operand): row key_of_row(ln, tt) (tt = 1 adds 16 rows, same swizzle), logical chunk 2 ks + hl.
    uint32_t kofs[4];
    {
      const int row = key_of_row(ln, 0);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) kofs[ks] = row * 128 + 16 * ((2 * ks + hl) ^ ((row >> 1) & 7));
    }
    // V^T (A operand of P V): channel row 32 dt + ln (dt adds 32 rows = 2 KB, same swizzle),
    // keys 32 hl + 0..31 = logical chunks 2 hl, 2 hl + 1.
    uint32_t vofs[2];
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2) vofs[c2] = ln * 64 + 16 * ((2 * hl + c2) ^ ((ln >> 2) & 3));

    // The K Q^T accumulators start at kSeedBits, so the scores need no int -> fp32
    // conversion (see the softmax).
    i32x16 seed;
#pragma unroll
    for (int r = 0; r < 16; ++r) seed[r] = (int)kSeedBits;
    // Kept in registers for the whole loop: left as a constant, the compiler rebuilds it from
    // scalar registers before every tile's first MFMAs (eight 64-bit moves per tile).
    asm volatile("" : "+v"(seed));
    i32x16 si[2];  // biased int32 scores of the latest tile, one 32-key sub-tile each
    i32x8 pf;      // P of the latest softmax (e4m3, p * 2^8)
    float s_tile;  // q_scale * k_scale * 2^26 of the half-wave's 32-key block in that tile
    float mx_tile;  // row max (scaled, log2 units) of the latest K Q^T, -inf where all hidden
    constexpr int kMasked = INT32_MIN;  // no real score gets there: |acc| <= 128 * 127^2
    // ---- mask and row max of the scores of tile t (in si), into mx_tile.  The plain kernel takes
    // them at the start of the softmax phase (its matrix phase is the longer one); the split-tail
    // kernel keeps them at the end of the matrix phase, as its work-item plan needs the registers
    // the other placement takes.
    auto row_max = [&](int t) __attribute__((always_inline)) {
      if (masked_tile(t)) {
        // keys t * BK + 32 hl + e, e = 16 tt + r, visible for e in [elo, ehi]
        const int elo = lo_i - (t * BK + 32 * hl), ehi = hi_i - (t * BK + 32 * hl);
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int e = 16 * tt + r;
            si[tt][r] = (e < elo || e > ehi) ? kMasked : si[tt][r];
          }
      }
      // row max on the biased int32 patterns (positive floats order like their bits), as a
      // tree of v_max3_i32 for a short dependency chain
      int m8[11];
#pragma unroll
      for (int j = 0; j < 10; ++j) {
        const int e = 3 * j;
        m8[j] = max(max(si[e >> 4][e & 15], si[(e + 1) >> 4][(e + 1) & 15]), si[(e + 2) >> 4][(e + 2) & 15]);
      }
      m8[10] = max(si[1][14], si[1][15]);
      const int mi = max(max(max(max(m8[0], m8[1]), m8[2]), max(max(m8[3], m8[4]), m8[5])),
                         max(max(max(m8[6], m8[7]), m8[8]), max(m8[9], m8[10])));
      // s >= 0: scaling keeps the max; a half-wave with every key hidden contributes -inf
      const float mh = mi == kMasked ? -INFINITY : (__int_as_float(mi) - kSeed) * s_tile;
      mx_tile = half_pair_max_nc(mh);
    };

    // ---- matrix phase: the row sums of P (1 MFMA, first: it needs no LDS data), S^T = K Q^T
    // for K stage KS (8 MFMA), then O^T += V^T P^T for V stage VS (4 MFMA).  The last matrix
    // phase (P V only) takes the row sums after the P V products.
    auto mphase = [&](auto vs_c, auto ks_c, auto pv_c, auto qk_c, int t) __attribute__((always_inline)) {
      constexpr int VS = decltype(vs_c)::value, KS = decltype(ks_c)::value;
      constexpr bool PV = decltype(pv_c)::value, QK = decltype(qk_c)::value;
      constexpr int KB = K_STAGE0 + KS * KT_BYTES, VB = V_STAGE0 + VS * VT_BYTES, SB = KS_STAGE0 + KS * 16;
      const uint32_t lds0 = (uint32_t)(uintptr_t)(const DITATTN_LDS char*)lds;
      // Fragment reads: K fragment j = 2 ks + tt (sub-tile tt adds 16 rows = 2 KB), the tile's
      // k_scale pair (read with the K rows: the stage is refilled one window later, while the
      // other group may still be in this tile's softmax), V^T fragment j = 2 dt + c2 (dt adds
      // 32 channel rows = 2 KB).  Four K fragments are in flight ahead of the MFMA that takes
      // them and the V^T reads follow as the K registers free up; each MFMA waits only for its
      // own operands (LDS reads return in issue order), so the phase pays about one LDS latency.
      u32x4 kf[8], vf[8];
      uint32_t ksb = 0;
      auto kread = [&](auto j_c) __attribute__((always_inline)) {
        constexpr int j = decltype(j_c)::value;
        kf[j] = ds_read_b128<KB + (j & 1) * 2048>(lds0 + kofs[j >> 1]);
      };
      auto vread = [&](auto j_c) __attribute__((always_inline)) {
        constexpr int j = decltype(j_c)::value;
        vf[j] = ds_read_b128<VB + (j >> 1) * 2048>(lds0 + vofs[j & 1]);
      };
      using J0 = std::integral_constant<int, 0>;
      using J1 = std::integral_constant<int, 1>;
      using J2 = std::integral_constant<int, 2>;
      using J3 = std::integral_constant<int, 3>;
      using J4 = std::integral_constant<int, 4>;
      using J5 = std::integral_constant<int, 5>;
      using J6 = std::integral_constant<int, 6>;
      using J7 = std::integral_constant<int, 7>;
      // Issue order with both parts: K0 K1 K2 K3 S V0 V1, then after MFMA j: K(j+4) (j < 4),
      // V2 V3 (j = 4), V4 V5 (j = 5), V6 V7 (j = 6).  Without P V: K0..K3 S, then K(j+4).
      // Position of each read in that order, and the reads issued before the wait for K j:
      constexpr int kpos_pv[8] = {0, 1, 2, 3, 7, 8, 9, 10}, kpos_qk[8] = {0, 1, 2, 3, 5, 6, 7, 8};
      constexpr int before_pv[8] = {7, 8, 9, 10, 11, 13, 15, 17}, before_qk[8] = {5, 6, 7, 8, 9, 9, 9, 9};
      constexpr int vpos[8] = {5, 6, 11, 12, 13, 14, 15, 16};
      if constexpr (QK) {
        kread(J0{}); kread(J1{}); kread(J2{}); kread(J3{});
        ksb = ds_read_b32<SB>(lds0 + 4 * hl);
        if constexpr (PV) {
          vread(J0{}); vread(J1{});
          // the row sums need only P: they run while the first K fragment is on its way
          lacc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(lsel, pf, lacc, 0, 0, 0, unit_scale, 0, unit_scale);
          __builtin_amdgcn_sched_barrier(0);
        }
        auto qk = [&](auto j_c) __attribute__((always_inline)) {
          constexpr int j = decltype(j_c)::value;
          constexpr int later = PV ? before_pv[j] - kpos_pv[j] - 1 : before_qk[j] - kpos_qk[j] - 1;
          lds_wait<later>(kf[j]);
          si[j & 1] = mfma_i8_32x32x32(__builtin_bit_cast(i32x4, kf[j]), qf[j >> 1], j < 2 ? seed : si[j & 1]);
          if constexpr (j < 4) {
            kread(std::integral_constant<int, j + 4>{});
          } else if constexpr (PV) {
            if constexpr (j == 4) { vread(J2{}); vread(J3{}); }
            if constexpr (j == 5) { vread(J4{}); vread(J5{}); }
            if constexpr (j == 6) { vread(J6{}); vread(J7{}); }
          }
          // keep each MFMA between its wait and the next one
          __builtin_amdgcn_sched_barrier(0);
        };
        qk(J0{}); qk(J1{}); qk(J2{}); qk(J3{}); qk(J4{}); qk(J5{}); qk(J6{}); qk(J7{});
        lds_wait<PV ? 17 - 4 - 1 : 9 - 4 - 1>(ksb);
        s_tile = sq * __uint_as_float(ksb);
      } else if constexpr (PV) {
        vread(J0{}); vread(J1{}); vread(J2{}); vread(J3{}); vread(J4{}); vread(J5{}); vread(J6{}); vread(J7{});
      }
      if constexpr (PV) {
        auto pv = [&](auto dt_c) __attribute__((always_inline)) {
          constexpr int dt = decltype(dt_c)::value;
          constexpr int later = QK ? 17 - vpos[2 * dt + 1] - 1 : 6 - 2 * dt;
          lds_wait<later>(vf[2 * dt], vf[2 * dt + 1]);
          const i32x8 va = __builtin_shufflevector(__builtin_bit_cast(i32x4, vf[2 * dt]),
                                                   __builtin_bit_cast(i32x4, vf[2 * dt + 1]), 0, 1, 2, 3, 4, 5, 6, 7);
          acc[dt] = mfma_fp8_32x32x64(va, pf, acc[dt], unit_scale);
          __builtin_amdgcn_sched_barrier(0);
        };
        pv(J0{}); pv(J1{}); pv(J2{}); pv(J3{});
        // after the last tile the row sums come last: the epilogue reads the P V accumulators
        // right after the drain, and this product keeps the matrix unit between the two
        if constexpr (!QK)
          lacc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(lsel, pf, lacc, 0, 0, 0, unit_scale, 0, unit_scale);
      }
      if constexpr (QK && SK) {
        row_max(t);
        pin(si[0]);
        pin(si[1]);
        pin(mx_tile);
      }
      if constexpr (PV) {
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) pin(acc[dt]);
        pin(lacc);
      }
    };

    // ---- softmax of the scores of tile t (in si): lazily raised running max, P -> e4m3.
    // One body for every tile (two copies of it make the compiler double-allocate the
    // accumulators); a tile crossing a mask boundary only takes two small branches: its
    // hidden scores become INT32_MIN before the row max, and their P codes become 0.
    auto softmax = [&](int t, auto large_c) __attribute__((always_inline)) {
      constexpr bool kLarge = decltype(large_c)::value;
      if constexpr (!SK) row_max(t);
      const float s = s_tile;
      const bool masked = masked_tile(t);  // uniform
      const float mx = mx_tile;
      if (__builtin_amdgcn_ballot_w64(mx > m_thr) != 0) {
        const float m_new = fmaxf(m, mx);
        const float alpha = m_new == m ? 1.0f : fast_exp2(m - m_new);
        m = m_new;
        m_thr = m + kLazyThresh;
        mneg = m == -INFINITY ? kCodeOffset : fmaf(kCodeSlope, kPScaleLog2 - m, kCodeOffset);
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) acc[dt] *= alpha;
        lacc *= alpha;
      }
      // The code argument 8 x + kCodeOffset as ONE fma on the seeded pattern A = kSeed + score *
      // 2^-26, with s = q_scale * k_scale * 2^26 in base-2 units: A * 8 s + (mneg - kSeed * 8 s).
      // That constant is rounded at about kSeed * 8 s * 2^-24, a fiftieth of a code step while
      // 8 s <= kFastS8 (every tile of inputs of ordinary magnitude).  For larger scales (|q| and |k|
      // in the tens and beyond) a wave takes the score out of the pattern first, A - kSeed, which
      // is exact (both share one exponent), and clamps the code argument at 126, so the codes stay
      // right and never reach 127 (NaN) whatever the magnitude or the running max.
      const float s8 = kCodeSlope * s;
      // P (B operand, 32 e4m3 bytes): byte e = key 32 hl + e.  v_cvt_pk_u8_f32 rounds to the
      // nearest integer and clamps to [0, 255]; y <= 8 * 8.8 + 56 - 0.35 < 126.5 (and the large-scale
      // path clamps at 126), so the largest code is 126 (448) and never 127 (NaN).  Every byte of
      // the old word is overwritten.  Each path packs its own codes, so only P's eight registers
      // meet after the branch.
      auto codes = [&](auto large_c) __attribute__((always_inline)) {
        constexpr bool large = decltype(large_c)::value;
        const float cst = fmaf(-kSeed, s8, mneg);
        float y[32];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float A = __int_as_float(si[tt][r]);
            y[16 * tt + r] = large ? fminf(fmaf(A - kSeed, s8, mneg), 126.0f) : fmaf(A, s8, cst);
          }
        if (masked) {
#pragma unroll
          for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int r = 0; r < 16; ++r) y[16 * tt + r] = si[tt][r] == kMasked ? -1.0f : y[16 * tt + r];
        }
#pragma unroll
        for (int w = 0; w < 8; ++w) {
          uint32_t word = __builtin_amdgcn_cvt_pk_u8_f32(y[4 * w], 0, (uint32_t)pf[w]);
          word = __builtin_amdgcn_cvt_pk_u8_f32(y[4 * w + 1], 1, word);
          word = __builtin_amdgcn_cvt_pk_u8_f32(y[4 * w + 2], 2, word);
          word = __builtin_amdgcn_cvt_pk_u8_f32(y[4 * w + 3], 3, word);
          pf[w] = (int)word;
        }
      };
      codes(std::integral_constant<bool, kLarge>{});
      // keep the softmax in its phase: without the pin the compiler sinks the
      // code conversions past the barrier, next to the P V products that consume them
      asm volatile("" : "+v"(pf));
    };

    // ---- ping-pong over key tiles t0 .. t1 - 1 (local index p = t - t0), as in the BF16
    // kernel.  Waves w and w + 4 share a SIMD.  Every wave runs
    //   M(0) | V(0) | M(1) | V(1) | ... | M(n)
    // with a barrier after each phase, where M(p) = [P V of tile p-1, K Q^T of tile p] and
    // V(p) = softmax of tile p; group B (waves 4-7) starts one barrier late, so on each SIMD
    // one wave's matrix phase overlaps the other's softmax.  Barrier k: group A has finished
    // phase k-1 of its sequence, group B phase k-2.  K(p+1) and V(p) are copied in the window
    // between barriers 2p and 2p+2, each group its own rows (issued at the window's start,
    // awaited at its end): the stages they overwrite (K(p-1), V(p-2)) were last read in
    // M(p-1), which both groups finished by barrier 2p, and their first readers (M(p+1) of
    // group A) start at barrier 2p+2.
    const bool grp_a = wave < NW / 2;
    // copy(q) = K(q+2) and V(q+1), where they exist, into stages (q+2) % 3 and (q+1) % 3
    auto copy = [&](int q) __attribute__((always_inline)) {
      if (q + 2 < n) issue_k(t0 + q + 2, (q + 2) % NSTAGE);
      if (q + 1 < n) issue_v(t0 + q + 1, (q + 1) % NSTAGE);
    };
    // wait until the copies of the previous window have landed; the current window's (one
    // K and one V instruction per wave, plus a scale load on wave 0) may stay in flight
    auto prev_landed = [&](int q) __attribute__((always_inline)) {
      if (q + 2 < n) asm volatile("s_waitcnt vmcnt(2)" ::: "memory");
      else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    };
    // s_barrier without the release fence of __syncthreads(), which would also wait for the
    // copies in flight; LDS reads before it have all been consumed.
    auto barrier = [&]() __attribute__((always_inline)) { asm volatile("s_barrier" ::: "memory"); };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using T = std::true_type;
    using F = std::false_type;
    // ---- ping-pong over key tiles t0 .. t1 - 1 (local index p).  Waves w and w + 4 share a
    // SIMD.  Every wave runs  M(0) | V(0) | M(1) | V(1) | ... | M(n)  with a barrier after each
    // phase, M(p) = [P V of tile p-1, K Q^T of tile p], V(p) = softmax of tile p; group B
    // (waves 4-7) starts one barrier late, so on each SIMD one wave's matrix phase overlaps
    // the other's softmax.  Barrier k: group A has finished phase k-1, group B phase k-2.
    // Three-stage copy ring: window q (barriers 2q .. 2q+2) copies K(q+2) and V(q+1), each
    // group its own rows at the start of its M(q); they must land by barrier 2q+4, where
    // group A's M(q+2) first reads them, and each group waits for them at the end of its last
    // phase before that barrier (one full window after the issue).  The stages they refill
    // held K(q-1) and V(q-2), last read in M(q-1), finished by both groups at barrier 2q.
    // The k_scale pair of a tile is read in the M phase with its K rows.
    auto period = [&](auto st_c, int p, auto large_c) __attribute__((always_inline)) {  // 1 <= p <= n - 1
      constexpr int st = decltype(st_c)::value;  // p % 3
      using KS = std::integral_constant<int, st>;
      using VS = std::integral_constant<int, (st + NSTAGE - 1) % NSTAGE>;
      copy(p);
      mphase(VS{}, KS{}, T{}, T{}, t0 + p);
      if (!grp_a) prev_landed(p);
      barrier();
      softmax(t0 + p, large_c);
      if (grp_a) prev_landed(p);
      barrier();
    };

    issue_k(t0, 0);
    if (n > 1) issue_k(t0 + 1, 1);
    issue_v(t0, 0);
    // The code path of the softmax (below) is chosen once per workgroup and query tile (or piece
    // of one), from the largest k_scale of the key blocks it visits, loaded under the first
    // copies: the large-scale path only where a wave's 8 s could exceed kFastS8 on some tile.
    // Choosing it per tile instead cost 2 to 4 %: its code in the loop changed how the compiler
    // laid out the fast one.
    {
      // this tile's v_scale to LDS under the same wait: read in the epilogue from global memory,
      // its latency came once per query tile after the key loop (+0.8 % at FLUX-1024)
      f32x4 vs4 = {0.0f, 0.0f, 0.0f, 0.0f};
      if (tid < kHeadDim / 4) vs4 = *(const f32x4*)(a.v_scale + (int64_t)bhk * kHeadDim + 4 * tid);
      float kmax = 0.0f;
      const int b0 = 2 * t0, b1 = min(2 * t1, nblk_k);
#pragma unroll 4
      for (int i = b0 + tid; i < b1; i += NW * 64) kmax = fmaxf(kmax, ksc[i]);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      if (tid < kHeadDim / 4) *(f32x4*)(vsc_lds + 4 * tid) = vs4;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) kmax = fmaxf(kmax, __shfl_xor(kmax, off, 64));
      if (l == 0) large_w[wave] = kCodeSlope * sq * kmax > kFastS8 ? 1 : 0;
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the flag is in LDS before the barrier
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    barrier();  // barrier 0
    if (!grp_a) barrier();  // group B's leading barrier (barrier 1 for group A)
    bool large = false;
    {
#pragma unroll
      for (int w = 0; w < NW; ++w) large = large || large_w[w] != 0;
    }
    auto key_loop = [&](auto large_c) __attribute__((always_inline)) {
      // period 0: no P V yet, no window before it to wait for
      copy(0);
      mphase(I0{}, I0{}, F{}, T{}, t0);
      barrier();
      softmax(t0, large_c);
      barrier();
      int p = 1;
      for (; p + 2 < n; p += 3) {  // three periods per trip: stage offsets are immediates
        period(I1{}, p, large_c);
        period(I2{}, p + 1, large_c);
        period(I0{}, p + 2, large_c);
      }
      if (p < n) {
        period(I1{}, p, large_c);
        ++p;
      }
      if (p < n) {
        period(I2{}, p, large_c);
        ++p;
      }
      // M(n): P V of the last tile (n - 1) from V stage (n - 1) % 3
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      const int vs_last = (n - 1) % NSTAGE;
      if (vs_last == 0) mphase(I0{}, I0{}, T{}, F{}, 0);
      else if (vs_last == 1) mphase(I1{}, I0{}, T{}, F{}, 0);
      else mphase(I2{}, I0{}, T{}, F{}, 0);
    };
    if (large) key_loop(std::true_type{});
    else key_loop(std::false_type{});
    if (grp_a) barrier();  // matches group B's leading barrier
  }

  // ---- epilogue: O[i][d] = acc * v_scale[d] / l (0 for a row with no visible key)
  // Twice the drain of a 16-pass MFMA: a partial piece stores these registers at once, and a
  // single drain right after the last P V product let it store stale values (the split-tail
  // test at 4608 x 1000 tokens with grouped heads then differed from run to run).
  mfma_drain(acc[0], acc[1], acc[2], acc[3]);
  mfma_drain(acc[0], acc[1], acc[2], acc[3]);
  mfma_drain(lacc);
  float lsum = lacc[0];
  if (mode == kSplitPartial) {
    split_write_partial(a.ws_part, a.ws_flag, a.epoch, acc, m, lsum);
    return;
  }
  bool ok = true;
  if (mode == kSplitOwner) ok = split_merge(a.ws_part, a.ws_flag, a.epoch, p_lo, p_hi, a.sk_tail_units, acc, m, lsum);
  // (NaN if a piece never came)
  const float inv = !ok ? __builtin_nanf("") : (lsum > 0.0f ? 1.0f / lsum : 0.0f);
  if (qi < a.S_q) {
    // the lane's channel offset, opaque here: hoisted out of the split kernel's loop over work
    // items, its 64-bit output address stayed live across the key loop and spilled
    int hl_e = hl;
    asm volatile("" : "+v"(hl_e));
    __bf16* orow = (__bf16*)a.o + (((int64_t)b * a.S_q + qi) * a.H + h) * kHeadDim;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const int d = 32 * dt + 8 * rq + 4 * hl_e;
        const f32x4 s4 = *(const f32x4*)(vsc_lds + d);
        bf16x4 ov;
#pragma unroll
        for (int e = 0; e < 4; ++e) ov[e] = (__bf16)(acc[dt][4 * rq + e] * s4[e] * inv);
        *(bf16x4*)(orow + d) = ov;
      }
  }
  };  // run

  if constexpr (!SK) run(xcd_remap(blockIdx.x, a.n_tiles), -1, -1, kSplitFull, 0, -1);
  else split_tail_items(a.sk_rounds, a.sk_nk, a.sk_tail_units, run);
}

__global__ void __launch_bounds__(NW * 64, 1) sage_attn_fwd_kernel(SageArgs a) { sage_body<false>(a); }
__global__ void __launch_bounds__(NW * 64, 1) sage_attn_fwd_split_kernel(SageArgs a) { sage_body<true>(a); }

}  // namespace sageattn

hipError_t launch_sage_attn_fwd(const SageArgs& a0, hipStream_t stream) {
  SageArgs a = a0;
  a.num_qt = (a.S_q + sageattn::BQ - 1) / sageattn::BQ;
  a.n_tiles = a.B * a.H * a.num_qt;
  a.reverse = a.wr >= 0 ? 1 : 0;  // a key range that ends at the query: later tiles see more keys
  if (a.sk_grid > 0)
    return launch(sageattn::sage_attn_fwd_split_kernel, dim3(a.sk_grid), dim3(sageattn::NW * 64), stream, a);
  return launch(sageattn::sage_attn_fwd_kernel, dim3(a.n_tiles), dim3(sageattn::NW * 64), stream, a);
}

}  // namespace ditattn

