// attn_bf16.hip -- BF16 flash attention forward for gfx950 (MI355X).
//
// Operation: "Kernel acceleration: attention, compilation and fusion",
// section "Attention: from O(N^2) memory to blocks" -- attention computed one
// key block at a time with a running row max m, running row sum l and an
// accumulator rescaled by exp(m_old - m_new), so the S_q x S_kv scores never
// leave the chip.  Shape contract (BF16 [B, S, H, 128] in and out) from
// "gfx1201_sage_prepare / gfx1201_sage_attention", "Technical Details";
// cross-attention (S_q != S_kv), grouped-query heads (H_kv | H) and key
// windows (causal / sliding, bottom-right aligned) generalise it.
//
// gfx950 mapping
//   * Work unit: one workgroup of 8 waves per (b, h, 256-row query tile), each
//     wave owning 32 query rows.  Workgroups are remapped so one head's tiles
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
//   * K/V tiles of 64 keys are double-buffered in LDS.  Rows are 256 B,
//     unpadded, with 16-byte chunks XOR-swizzled per row so that both the
//     MFMA-operand reads and the transposed reads are free of bank conflicts.
//   * Ping-pong: waves w and w + 4 share a SIMD and run the same phase sequence
//     one barrier apart, so one wave's matrix phase (P V of the previous tile,
//     K Q^T of this one: 32 MFMA) overlaps the other's softmax (VALU).
//   * Copies: only the first four waves copy, eight 1 KB buffer_load ... lds
//     per wave per tile, one after every second MFMA of their matrix phase, so
//     the address unit (about 64 B per clock per CU) drains while the matrix
//     core works instead of stalling every wave at the same barrier.  The
//     buffer resource ends after the last key: rows past it in a ragged last
//     tile read as zeros, and their scores are masked to -inf.
//   * Softmax in base 2: x = s * c with c = scale * log2(e); exp2 on v_exp_f32.
//     The running max is only raised when a row's tile max exceeds it by more
//     than kLazyThresh (in log2 units): P values up to 2^kLazyThresh are
//     harmless in BF16/FP32, and the O rescale (64 multiplies per lane) is
//     skipped on almost every tile.  Every p and l use the same stale max,
//     which cancels in acc / l.
//   * Query rows >= S_q are computed on zeros and not stored; rows that see no
//     key (an empty window) are written as zeros.
#include <atomic>
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace ditattn {
namespace bf16attn {

// Tuning knobs (compile-time; defaults are the measured choice).
#ifndef DITATTN_BF16_OCC
#define DITATTN_BF16_OCC 1  // workgroups per CU the register budget is sized for
#endif

#ifndef DITATTN_BF16_NW
#define DITATTN_BF16_NW 8   // waves per workgroup (all share one K/V tile); 2 per SIMD
#endif

constexpr int BK = 64;      // keys per K/V tile
constexpr int NW = DITATTN_BF16_NW;
static_assert(NW == 8, "the ping-pong pairs waves w and w + 4 on one SIMD");
constexpr float kLazyThresh = 8.0f;


// LDS: two K stages then two V stages, each 64 rows x 256 B.
constexpr int TILE_BYTES = BK * 256;
constexpr int K_STAGE0 = 0;
constexpr int V_STAGE0 = 2 * TILE_BYTES;

// First and last key query row i sees (an empty range when hi < lo): lo = i + off - wl
// (wl >= 0), hi = i + off + wr (wr >= 0), off = S_kv - S_q, clamped to the keys, in 64 bits.
__device__ __forceinline__ int key_lo(const Bf16Args& a, int i) {
  if (a.wl < 0) return 0;
  const int64_t lo = (int64_t)i + a.S_kv - a.S_q - a.wl;
  return (int)(lo < 0 ? 0 : (lo > a.S_kv ? a.S_kv : lo));
}
__device__ __forceinline__ int key_hi(const Bf16Args& a, int i) {
  if (a.wr < 0) return a.S_kv - 1;
  const int64_t hi = (int64_t)i + a.S_kv - a.S_q + a.wr;
  return (int)(hi < -1 ? -1 : (hi > a.S_kv - 1 ? a.S_kv - 1 : hi));
}

static_assert(NW * 64 == kSplitThreads, "split-tail slots hold one row per thread");

template <bool SK>
__device__ __forceinline__ void attn_body(const Bf16Args& a) {
  constexpr int BQ = NW * 32;
  __shared__ __attribute__((aligned(16))) char lds[4 * TILE_BYTES];  // K stage 0, 1, V stage 0, 1

  // One query tile L: the key tiles its window covers (tb < 0), or the tiles [tb, te) of a split
  // tail, ending by mode: kSplitFull writes O, kSplitPartial writes (acc, m, l) to the
  // workgroup's slot and raises its flag, kSplitOwner first merges the slots of workgroups
  // p_lo .. p_hi, then writes O.
  auto run = [&](int L, int tb, int te, int mode, int p_lo, int p_hi) {
  const int bh = L / a.num_qt;
  int qt = L - bh * a.num_qt;
  if (a.reverse) qt = a.num_qt - 1 - qt;  // longest key ranges first (causal)
  const int b = bh / a.H, h = bh - b * a.H;
  const int hk = h / (a.H / a.H_kv);  // key/value head of this query head
  const float c = a.c;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l = tid & 63, hl = l >> 5, ln = l & 31;
  const int64_t tok = (int64_t)a.H * kHeadDim;       // elements between consecutive Q/O tokens
  const int64_t tok_kv = (int64_t)a.H_kv * kHeadDim;  // ... and K/V tokens
  const uint32_t tok_bytes = (uint32_t)(tok_kv * 2);
  const int64_t base = ((int64_t)b * a.S_q * a.H + h) * kHeadDim;
  const int64_t base_kv = ((int64_t)b * a.S_kv * a.H_kv + hk) * kHeadDim;
  const __bf16* qbh = (const __bf16*)a.q + base;
  const char* kbh = (const char*)((const __bf16*)a.k + base_kv);
  const char* vbh = (const char*)((const __bf16*)a.v + base_kv);
  __bf16* obh = (__bf16*)a.o + base;

  // Q^T operand, resident for the whole key loop: Q[q0 + ln][16 ks + 8 hl + 0..7].
  const int q0 = qt * BQ + wave * 32;
  const int qi = q0 + ln;  // this lane's query row
  bf16x8 qf[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    if (qi < a.S_q) qf[ks] = *(const bf16x8*)(qbh + qi * tok + 16 * ks + 8 * hl);
    else qf[ks] = bf16x8{};
  }

  // ---- key range: the workgroup visits the tiles holding a key one of its rows < S_q sees;
  // a tile needs no mask when every key of it is visible to every row of the workgroup.
  const int i_first = qt * BQ, i_last = min(qt * BQ + BQ - 1, a.S_q - 1);
  const int lo_i = key_lo(a, qi), hi_i = key_hi(a, qi);
  const int lo_last = key_lo(a, i_last), hi_first = key_hi(a, i_first);
  const int hi_last = key_hi(a, i_last);
  const int t0 = tb >= 0 ? tb : key_lo(a, i_first) / BK;
  const int t1 = tb >= 0 ? te : (hi_last >= 0 ? hi_last / BK + 1 : 0);
  const int n = t1 - t0;  // tiles this run visits (uniform)
  auto masked_tile = [&](int t) { return t * BK < lo_last || t * BK + BK - 1 > hi_first; };

  f32x16 acc[4];  // O^T: channels 32 dt + (accumulator row), this lane's query
  float m = -INFINITY, lsum = 0.0f;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) acc[dt] = f32x16{};

  // ---- global -> LDS (direct).  Instruction n of a copying wave writes LDS rows
  // 16 w + 4 n + l / 16, physical chunk l % 16; the lane fetches the logical chunk
  // that lands there.
  const int p_chunk = l & 15;
  // Group-A copies: wave w (< NW / 2) copies rows 16 w .. 16 w + 15 of each tile, four
  // 1 KB instructions, instruction n covering rows 16 w + 4 n + l / 16.
  uint32_t akoff[4], avoff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 16 * (wave & 3) + 4 * i + (l >> 4);
    akoff[i] = r * tok_bytes + 16u * (uint32_t)(p_chunk ^ (r & 15));
    avoff[i] = r * tok_bytes + 16u * (uint32_t)(p_chunk ^ ((r & 3) << 2));
  }
  // One period's copies: K(q+1) and V(q) (local tile indices), where they exist.
  struct CopyPlan {
    __amdgpu_buffer_rsrc_t rk, rv;  // K(q+1) and V(q)
    int kdst, vdst;                 // LDS byte offsets of this wave's first rows
    bool k_ok, v_ok;
  };
  auto plan = [&](int q) {
    CopyPlan c;
    auto rsrc = [&](const char* src, int tl) {
      const int j0 = (t0 + tl) * BK;
      const int rows = min(a.S_kv - j0, BK);
      return __builtin_amdgcn_make_buffer_rsrc((void*)(src + (int64_t)j0 * tok_kv * 2), (short)0,
                                               (rows - 1) * (int)tok_bytes + 256, 0x00020000);
    };
    c.k_ok = q + 1 < n;
    c.v_ok = q >= 0 && q < n;
    c.rk = rsrc(kbh, c.k_ok ? q + 1 : 0);
    c.rv = rsrc(vbh, c.v_ok ? q : 0);
    c.kdst = K_STAGE0 + ((q + 1) & 1) * TILE_BYTES + 16 * (wave & 3) * 256;
    c.vdst = V_STAGE0 + (q & 1) * TILE_BYTES + 16 * (wave & 3) * 256;
    return c;
  };
  // instruction j (0..7) of a copy plan: j < 4 -> part j of K(q+1), else part j - 4 of V(q)
  auto copy_part = [&](const CopyPlan& c, int j) {
    const int i = j & 3;
    if (j < 4) {
      if (c.k_ok)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(c.rk, (DITATTN_LDS void*)(lds + c.kdst + 4 * i * 256), 16, akoff[i], 0, 0, 0);
    } else {
      if (c.v_ok)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(c.rv, (DITATTN_LDS void*)(lds + c.vdst + 4 * i * 256), 16, avoff[i], 0, 0, 0);
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

  // ---- matrix phase: O^T += V^T P^T for the keys of V stage VS (16 MFMA, 32
  // transposed reads) and/or S^T = K Q^T for the keys of K stage KS (16 MFMA, 16
  // reads), as one explicitly pipelined stream: V fragments one 16-key chunk
  // ahead, K fragments three channel steps ahead, and the first K reads issued
  // under the last P V chunks.  Waits count outstanding LDS reads (returned in order).
  f32x16 sc[2];  // scores of the latest tile, one 32-key sub-tile each
  bf16x8 pf[4];  // P of the latest softmax, one 16-key chunk each
  auto mphase = [&](auto vs_c, auto ks_c, auto pv_c, auto qk_c, int cq) {
    const bool cp = cq >= 0;
    const CopyPlan cpl = plan(cp ? cq : 0);
    constexpr int VS = decltype(vs_c)::value, KS = decltype(ks_c)::value;
    constexpr bool PV = decltype(pv_c)::value, QK = decltype(qk_c)::value;
    constexpr int VB = V_STAGE0 + VS * TILE_BYTES, KB = K_STAGE0 + KS * TILE_BYTES;
    const uint32_t lds0 = (uint32_t)(uintptr_t)(const DITATTN_LDS char*)lds;
    u32x4 kf[8][2];
    auto kread = [&](auto s_c) {
      constexpr int st = decltype(s_c)::value;
      if constexpr (st < 8) {
        kf[st][0] = ds_read_b128<KB>(lds0 + kofs[st]);
        kf[st][1] = ds_read_b128<KB + 32 * 256>(lds0 + kofs[st]);
      }
    };
    using C0 = std::integral_constant<int, 0>;
    using C1 = std::integral_constant<int, 1>;
    using C2 = std::integral_constant<int, 2>;
    using C3 = std::integral_constant<int, 3>;
    if constexpr (PV) {
      u32x2 fa[4][2], fb[4][2];
      auto vread = [&](auto cc_c, u32x2 (&f)[4][2]) {
        constexpr int cc = decltype(cc_c)::value;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          f[dt][0] = ds_read_tr16_b64<VB + (16 * cc) * 256>(lds0 + vofs[dt]);
          f[dt][1] = ds_read_tr16_b64<VB + (16 * cc + 8) * 256>(lds0 + vofs[dt]);
        }
      };
      auto chunk = [&](auto cc_c, u32x2 (&f)[4][2]) {
        constexpr int cc = decltype(cc_c)::value;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          const bf16x8 va = __builtin_bit_cast(bf16x8, u32x4{f[dt][0][0], f[dt][0][1], f[dt][1][0], f[dt][1][1]});
          acc[dt] = mfma_bf16_32x32x16(va, pf[cc], acc[dt]);
          if (dt & 1) {
            if (cp) copy_part(cpl, 2 * cc + (dt >> 1));
          }
        }
      };
      vread(C0{}, fa);
      vread(C1{}, fb);
      lds_wait<8>(fa[0][0], fa[0][1], fa[1][0], fa[1][1], fa[2][0], fa[2][1], fa[3][0], fa[3][1]);
      chunk(C0{}, fa);
      vread(C2{}, fa);
      lds_wait<8>(fb[0][0], fb[0][1], fb[1][0], fb[1][1], fb[2][0], fb[2][1], fb[3][0], fb[3][1]);
      chunk(C1{}, fb);
      vread(C3{}, fb);
      lds_wait<8>(fa[0][0], fa[0][1], fa[1][0], fa[1][1], fa[2][0], fa[2][1], fa[3][0], fa[3][1]);
      chunk(C2{}, fa);
      if constexpr (QK) {
        kread(C0{});
        kread(C1{});
        kread(C2{});
        lds_wait<6>(fb[0][0], fb[0][1], fb[1][0], fb[1][1], fb[2][0], fb[2][1], fb[3][0], fb[3][1]);
      } else {
        lds_wait<0>(fb[0][0], fb[0][1], fb[1][0], fb[1][1], fb[2][0], fb[2][1], fb[3][0], fb[3][1]);
      }
      chunk(C3{}, fb);
    } else if constexpr (QK) {
      kread(C0{});
      kread(C1{});
      kread(C2{});
    }
    if constexpr (QK) {
      sc[0] = f32x16{};
      sc[1] = f32x16{};
      auto step = [&](auto s_c) {
        constexpr int st = decltype(s_c)::value;
        constexpr int later = 2 * ((st + 2 < 7 ? st + 2 : 7) - st);  // reads issued after step st's
        lds_wait<later>(kf[st][0], kf[st][1]);
        sc[0] = mfma_bf16_32x32x16(__builtin_bit_cast(bf16x8, kf[st][0]), qf[st], sc[0]);
        sc[1] = mfma_bf16_32x32x16(__builtin_bit_cast(bf16x8, kf[st][1]), qf[st], sc[1]);
        if constexpr (!PV) {
          if (cp) copy_part(cpl, st);
        }
        kread(std::integral_constant<int, st + 3>{});
      };
      step(C0{});
      step(C1{});
      step(C2{});
      step(C3{});
      step(std::integral_constant<int, 4>{});
      step(std::integral_constant<int, 5>{});
      step(std::integral_constant<int, 6>{});
      step(std::integral_constant<int, 7>{});
      pin(sc[0]);
      pin(sc[1]);
    }
    if constexpr (PV) {
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) pin(acc[dt]);
    }
  };
  // softmax of the scores of tile t (in sc): mask the keys this lane's query does not
  // see (tiles crossing a mask boundary only), raise the running max lazily (rescaling
  // acc and l, whose last update is complete), P -> BF16.
  auto softmax = [&](int t) {
    if (masked_tile(t)) {
      // key t * BK + 32 tt + 8 (r / 4) + 4 hl + r % 4 is visible for offsets
      // 32 tt + 8 (r / 4) + r % 4 in [elo, ehi]; the opaque moves keep the compares here
      // instead of hoisted out of the key loop
      int elo = lo_i - t * BK - 4 * hl, ehi = hi_i - t * BK - 4 * hl;
      asm volatile("" : "+v"(elo), "+v"(ehi));
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int e = 32 * tt + 8 * (r >> 2) + (r & 3);
          if (e < elo || e > ehi) sc[tt][r] = -INFINITY;
        }
    }
    float mx = fmaxf(sc[0][0], sc[1][0]);
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = max3(mx, sc[0][r], sc[1][r]);
    mx = half_pair_max(mx) * c;
    if (__builtin_amdgcn_ballot_w64(mx > m + kLazyThresh) != 0) {
      const float m_new = fmaxf(m, mx);
      const float alpha = m_new == m ? 1.0f : fast_exp2(m - m_new);
      m = m_new;
      lsum *= alpha;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) acc[dt] *= alpha;
    }
    const float mneg = m == -INFINITY ? 0.0f : -m;  // rows with no visible key yet
    float p[32];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int r = 0; r < 16; ++r) p[16 * tt + r] = fast_exp2(fmaf(sc[tt][r], c, mneg));
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) {
      bf16x8 v8;
#pragma unroll
      for (int e = 0; e < 8; ++e) v8[e] = (__bf16)p[8 * cc + e];
      pf[cc] = v8;
    }
    lsum += tree_sum<32>(p);
    // keep the softmax in its phase: without the pins the compiler sinks the
    // exponentials past the barrier, next to the P V products that consume them
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) pin(pf[cc]);
    pin(lsum);
  };

  // ---- ping-pong over key tiles.  Waves w and w + 4 share a SIMD.  Every wave runs
  // the same sequence  M(0) | V(0) | M(1) | V(1) | ... | M(n)  with a barrier after
  // each phase, where M(p) = [P V of tile p-1, K Q^T of tile p] (32 MFMA) and
  // V(p) = softmax of tile p (VALU).  Group B (waves 4-7) starts one barrier late,
  // so on each SIMD one wave's matrix phase overlaps the other's softmax.
  // Barrier k: group A has finished phase k-1 of its sequence, group B phase k-2.
  // Group A copies K(q+1) and V(q) during its M(q) (after barrier 2q) and waits for
  // them at the end of its V(q) (before barrier 2q+2): the stages they overwrite
  // (K(q-1), V(q-2)) were last read in M(q-1), which both groups finished by barrier
  // 2q, and their first readers (M(q+1) of group A) start at barrier 2q+2.
  const bool grp_a = wave < NW / 2;
  auto copies_landed = [&]() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); };
  // s_barrier without the release fence of __syncthreads(), which would also wait
  // for the copies in flight; LDS reads before it have all been consumed.
  auto barrier = [&]() { asm volatile("s_barrier" ::: "memory"); };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using T = std::true_type;
  using F = std::false_type;
  // one period p (1 <= p <= n - 1) with compile-time K stage par = p & 1
  auto period = [&](auto par_c, int p) {
    constexpr int par = decltype(par_c)::value;
    using KS = std::integral_constant<int, par>;
    using VS = std::integral_constant<int, par ^ 1>;
    mphase(VS{}, KS{}, T{}, T{}, grp_a ? p : -1);
    barrier();
    softmax(t0 + p);
    if (grp_a) copies_landed();
    barrier();
  };

  if (n > 0) {  // uniform: every wave of the workgroup takes the same path
  if (grp_a) {  // K(0)
    const CopyPlan c0 = plan(-1);
#pragma unroll
    for (int j = 0; j < 4; ++j) copy_part(c0, j);
    copies_landed();
  }
  barrier();  // barrier 0
  if (!grp_a) {
    barrier();  // group B's leading barrier (barrier 1 for group A)
  }
  // period 0: no P V yet
  mphase(I0{}, I0{}, F{}, T{}, grp_a ? 0 : -1);
  barrier();
  softmax(t0);
  if (grp_a) copies_landed();
  barrier();
  int p = 1;
  for (; p + 1 < n; p += 2) {  // two periods per trip: stage offsets are immediates
    period(I1{}, p);
    period(I0{}, p + 1);
  }
  if (p < n) {  // p odd
    period(I1{}, p);
    ++p;
  }
  // M(n): P V of the last tile only
  if (p & 1) mphase(I0{}, I0{}, T{}, F{}, -1);
  else mphase(I1{}, I0{}, T{}, F{}, -1);
  if (grp_a) barrier();  // matches group B's leading barrier
  }

  // ---- epilogue
  mfma_drain(acc[0], acc[1], acc[2], acc[3]);
  if (mode == kSplitPartial) {
    split_write_partial(a.ws_part, a.ws_flag, a.epoch, acc, m, lsum);
    return;
  }
  bool ok = true;
  if (mode == kSplitOwner) ok = split_merge(a.ws_part, a.ws_flag, a.epoch, p_lo, p_hi, a.sk_tail_units, acc, m, lsum);
  // O = acc / l, BF16, rows < S_q (0 for a row with no visible key; NaN if a piece never came)
  const float lt = half_pair_sum(lsum);
  const float inv = !ok ? __builtin_nanf("") : (lt > 0.0f ? 1.0f / lt : 0.0f);
  if (qi < a.S_q) {
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const int d = 32 * dt + 8 * rq + 4 * hl;
        bf16x4 ov;
#pragma unroll
        for (int e = 0; e < 4; ++e) ov[e] = (__bf16)(acc[dt][4 * rq + e] * inv);
        *(bf16x4*)(obh + qi * tok + d) = ov;
      }
  }
  };  // run

  if constexpr (!SK) run(xcd_remap(blockIdx.x, a.n_tiles), -1, -1, kSplitFull, 0, -1);
  else split_tail_items(a.sk_rounds, a.sk_nk, a.sk_tail_units, run);
}

__global__ void __launch_bounds__(NW * 64, DITATTN_BF16_OCC) attn_fwd_bf16_kernel(Bf16Args a) {
  attn_body<false>(a);
}
__global__ void __launch_bounds__(NW * 64, DITATTN_BF16_OCC) attn_fwd_bf16_split_kernel(Bf16Args a) {
  attn_body<true>(a);
}

}  // namespace bf16attn

// Query rows per workgroup of the launched configuration.
constexpr int kBf16BQ = bf16attn::NW * 32;

namespace {
// Compute units of the current device (the split-tail grid), looked up once per device.
int cu_count() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int c = cached[dev].load(std::memory_order_relaxed);
  if (c == 0) {
    if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    cached[dev].store(c, std::memory_order_relaxed);
  }
  return c;
}
}  // namespace

// Split-tail plan of either attention kernel (both tile queries by 256 rows and keys by 64):
// used when the key windows are off, there are at least three whole rounds of query tiles and
// the last round would leave more than 5 % of the CU-rounds idle.  With
// fewer whole rounds the tail's pieces, start-ups and merges cost more than the idle CUs of a
// plain last round (measured: the board's clock rises while they idle).
SplitPlan split_tail_plan(int B, int S_q, int S_kv, int H, int wl, int wr) {
  SplitPlan p{};
  const int G = cu_count();
  const int64_t U = (int64_t)B * H * ((S_q + kBf16BQ - 1) / kBf16BQ);
  const int nk = (S_kv + bf16attn::BK - 1) / bf16attn::BK;
  if (G <= 0 || wl >= 0 || wr >= 0 || U < 3 * (int64_t)G || nk < 2) return p;
  const int64_t rounds = (U + G - 1) / G;
  if ((double)U / (double)(rounds * G) >= 0.95) return p;
  p.grid = G;
  p.rounds = (int)(U / G);
  p.nk = nk;
  p.tail_units = (U - (int64_t)p.rounds * G) * nk;
  p.flag_bytes = ((size_t)G * 4 + 255) / 256 * 256;
  p.bytes = p.flag_bytes + (size_t)G * kSplitSlotRows * kSplitThreads * sizeof(float);
  return p;
}

hipError_t launch_attn_fwd_bf16(const Bf16Args& a0, hipStream_t stream) {
  Bf16Args a = a0;
  a.num_qt = (a.S_q + kBf16BQ - 1) / kBf16BQ;
  a.n_tiles = a.B * a.H * a.num_qt;
  a.reverse = a.wr >= 0 ? 1 : 0;  // a key range that ends at the query: later tiles see more keys
  if (a.sk_grid > 0)
    return launch(bf16attn::attn_fwd_bf16_split_kernel, dim3(a.sk_grid), dim3(bf16attn::NW * 64), stream, a);
  return launch(bf16attn::attn_fwd_bf16_kernel, dim3(a.n_tiles), dim3(bf16attn::NW * 64), stream, a);
}

}  // namespace ditattn
