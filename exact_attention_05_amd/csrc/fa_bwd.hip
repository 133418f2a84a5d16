// Backward pass of exact attention on gfx950, by recomputation: the
// probabilities are rebuilt block by block from Q, K and the saved row
// log-sum-exp instead of being stored ("Apa itu FlashAttention", section
// "Cara kerja teknik Tiling dan Recomputation"; "Flash Attention Nedir?",
// section "Recomputation").  With P_ij = exp(scale q_i.k_j - LSE_i):
//
//   D_i = sum_c dO_ic O_ic            (stage 1, from the saved output)
//   dV  = P^T dO,  dP = dO V^T,  dS = P o (dP - D)
//   dK  = scale dS^T Q                (stage 2, one workgroup per key block)
//   dQ  = scale dS K                  (stage 3, one workgroup per query block)
//
// Stages 2 and 3 both recompute S and dP, so no atomics are needed and the
// result is bitwise repeatable.  Stage 1 also stores LSE_i * log2(e) next to
// D_i in the workspace, so the later stages exponentiate base 2 with a single
// fused multiply-add and can copy both rows straight into LDS.
//
// bf16 stage 2 (dK, dV): 4 waves (one per SIMD, 512 registers each; 2 for
// causal and sliding-window passes and nearly empty grids); each wave owns
// 32 keys and keeps their K and V rows in registers as matrix-core
// B operands for the whole pass.  Query stages of 64 rows (Q, dO, and the two
// row vectors) stream through double-buffered LDS by direct global -> LDS
// copies.  S = Q K^T and dP = dO V^T land in the accumulator layout with one
// key per lane, which is the B-operand layout needed for dV^T += dO^T P and
// dK^T += Q^T dS; the dO^T and Q^T A operands come from the same LDS tiles
// through the transposing read.  Each stage is two 32-query sub-blocks, and
// the unmasked stages run software-pipelined: the S and dP products of one
// sub-block issue while the vector unit turns the previous sub-block's
// probabilities into bf16 dS, and the dV and dK products of a sub-block
// overlap the next one's exponentials; operand fragments are read from LDS
// four products ahead.  Stages that need a mask (causal diagonal, window
// edges, ragged ends) take a plain, unpipelined path.  With shared K/V heads
// each workgroup takes one query head of the group (a "run") and writes
// float32 partial dK, dV; a reduction kernel adds the runs in a fixed order.
// Runs of several heads, summed inside the workgroup, are used only when
// the partials of one-head runs would not fit the workspace limit.
//
// bf16 stage 3 (dQ): mirrors the forward kernel.  8 waves (4 with a sliding
// window) own 32 queries each and keep Q and dO in registers; key blocks of 64 rows (K, V) stream
// through LDS.  S^T = K Q^T and dP^T = V dO^T put one query per lane, so
// LSE_i and D_i are one register each, and dQ^T += K^T dS^T reads K^T
// through the transposing read.  Key blocks that need no mask for any row of
// the workgroup run through a separate code path, two at a time with fixed
// LDS buffers.  At d = 128 with 256-row workgroups the two waves of each
// SIMD run half a step apart instead (bwd_dq_bf16_pp_kernel): one wave's
// products (dQ of the previous key block, S and dP of this one) beside the
// other wave's exponentials.
//
// Masks: the query offset and sliding window of the extended entry points
// (see Band) decide which query stages or key blocks a workgroup visits at
// all and which of those need a per-element mask.
#include "fa_internal.hpp"
#include "fa_device.hpp"
#include "fa_tiles.hpp"

#include <cmath>
#include <type_traits>

namespace fa {
namespace {

using F = std::false_type;
using T = std::true_type;
template <int B>
using Buf = std::integral_constant<int, B>;

// ------------------------------------------------------------ stage 1

template <int D, typename TT>
__global__ __launch_bounds__(256) void bwd_preprocess_kernel(const TT* __restrict__ o,
                                                            const TT* __restrict__ dO,
                                                            const float* __restrict__ lse,
                                                            float* __restrict__ delta,
                                                            float* __restrict__ lse2,
                                                            long rows) {
  constexpr int kVec = 16 / sizeof(TT);       // elements per 16-byte load
  constexpr int kLanesPerRow = D / kVec;      // 4 .. 32
  constexpr int kRowsPerBlock = 256 / kLanesPerRow;
  const int tid = threadIdx.x;
  const long row = (long)blockIdx.x * kRowsPerBlock + tid / kLanesPerRow;
  const int part = tid % kLanesPerRow;
  float acc = 0.f;
  if (row < rows) {
    const TT* op = o + row * D + part * kVec;
    const TT* gp = dO + row * D + part * kVec;
    if constexpr (sizeof(TT) == 2) {
      const bf16x8 x = *reinterpret_cast<const bf16x8*>(op);
      const bf16x8 y = *reinterpret_cast<const bf16x8*>(gp);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc = fmaf((float)x[e], (float)y[e], acc);
    } else {
      const f32x4 x = *reinterpret_cast<const f32x4*>(op);
      const f32x4 y = *reinterpret_cast<const f32x4*>(gp);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc = fmaf(x[e], y[e], acc);
    }
  }
#pragma unroll
  for (int off = kLanesPerRow / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
  if (row < rows && part == 0) {
    delta[row] = acc;
    lse2[row] = lse[row] * kLog2e;
  }
}

// ------------------------------------------------------ stage 2 (bf16)

template <int D, int WAVES>
struct DkdvCfg {
  static constexpr int kWaves = WAVES;           // one per SIMD, 512 registers each: 4, or 2
  static constexpr int kThreads = kWaves * 64;
  static constexpr int kBK = kWaves * 32;        // keys per workgroup, 32 per wave
  static constexpr int kBQ = 64;                 // queries per streamed stage
  static constexpr int kDC = D / 16;
  static constexpr int kDB = D / 32;
  static constexpr int kS1 = kDC;                // steps of region 1 (Q / dO row fragments)
  static constexpr int kS2 = 2 * kDB;            // steps of region 2 (dO^T / Q^T fragments)
  static constexpr int kAhead = 4;               // fragments read ahead of their products
  static constexpr int kRing = kAhead + 1;
  using QT = Tile<D, kBQ>;                       // one Q or dO stage in LDS
  static constexpr int kRowVecBytes = kBQ * 4;   // one stage of LSE2 or D
};

// MODE 0: one query head per workgroup, no sharing (group 1), final dK/dV;
// MODE 1: one query head of a shared K/V head, float32 partials;
// MODE 2: a run of several query heads of a shared K/V head.
template <int D, bool CAUSAL, int MODE, int WAVES>
__global__ __launch_bounds__(WAVES * 64) void bwd_dkdv_bf16_kernel(BwdArgs a, int n_ktiles) {
  using C = DkdvCfg<D, WAVES>;
  constexpr bool GROUPED = MODE == 2;
  // Query heads per K/V head, a compile-time 1 without sharing.
  const int group = MODE == 0 ? 1 : a.group;
  __shared__ __attribute__((aligned(1024))) char sq[2][C::QT::kBytes];
  __shared__ __attribute__((aligned(1024))) char sdo[2][C::QT::kBytes];
  __shared__ __attribute__((aligned(16))) float slse[2][C::kBQ];
  __shared__ __attribute__((aligned(16))) float sdel[2][C::kBQ];

  // One workgroup per (key tile, batch * K/V head); with shared K/V heads it
  // sums dK and dV over the query heads of its group.
  // Work item (key tile, K/V head, run of `run` consecutive query heads of
  // its group); without shared heads one run of one head.
  const int slices = MODE == 0 ? 1 : a.slices;
  const int run = GROUPED ? group / slices : 1;
  int hs, kt;
  if (CAUSAL) {
    // the first key tiles are seen by the most queries: they go first
    costliest_first(blockIdx.x, gridDim.x, n_ktiles, hs, kt);
  } else {
    const int work = xcd_remap(blockIdx.x, gridDim.x);
    hs = work / n_ktiles;
    kt = work - hs * n_ktiles;
  }
  const int bhkv = hs / slices;
  const int sl = hs - bhkv * slices;
  const int h_kv = a.H / group;
  const int bh0 = (bhkv / h_kv) * a.H + (bhkv % h_kv) * group + sl * run;  // first query head

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  const int n_q = a.n_q, n_k = a.n_k;
  const float sl2 = a.scale_log2;
  const int k0 = kt * C::kBK;
  const int key = k0 + wave * 32 + l32;  // this lane's key (a column of S)

  // Query-side rows of the current query head (advanced per head below).
  const __bf16* qp = static_cast<const __bf16*>(a.q) + (size_t)bh0 * n_q * D;
  const __bf16* dop = static_cast<const __bf16*>(a.dO) + (size_t)bh0 * n_q * D;
  const float* lsep = a.lse2 + (size_t)bh0 * n_q;
  const float* delp = a.delta + (size_t)bh0 * n_q;
  const __bf16* kp = static_cast<const __bf16*>(a.k) + (size_t)bhkv * n_k * D;
  const __bf16* vp = static_cast<const __bf16*>(a.v) + (size_t)bhkv * n_k * D;

  // The lane's K and V rows stay in registers as the B operands of
  // S = Q K^T and dP = dO V^T.
  bf16x8 kf[C::kDC], vf[C::kDC];
#pragma unroll
  for (int c = 0; c < C::kDC; ++c) {
    kf[c] = key < n_k ? *reinterpret_cast<const bf16x8*>(kp + (size_t)key * D + 16 * c + 8 * hi)
                      : bf16x8{};
    vf[c] = key < n_k ? *reinterpret_cast<const bf16x8*>(vp + (size_t)key * D + 16 * c + 8 * hi)
                      : bf16x8{};
    // moved into AGPRs once: the products read them there
    asm volatile("" : "+a"(kf[c]));
    asm volatile("" : "+a"(vf[c]));
  }

  // Query stages holding rows that see some key of this workgroup.
  const Band band = band_of(a, CAUSAL);
  int qvlo, qvspan;  // rows that see this lane's key: [qvlo, qvlo + qvspan]
  band.query_range(key, qvlo, qvspan);
  const int k1 = min(n_k, k0 + C::kBK);
  const int q_first = band.q_lo(k0), q_last = band.q_hi(k1);
  const int qb_first = q_first / C::kBQ;
  const int nblocks = q_last > q_first ? (q_last + C::kBQ - 1) / C::kBQ - qb_first : 0;

  TileDma<D, C::kBQ, C::kWaves> dma;
  dma.init(wave, lane);
  TileLane<D, C::kBQ> tqt;
  tqt.init(lane);
  const uint32_t sq_addr = lds_address(&sq[0][0]);
  const uint32_t sdo_addr = lds_address(&sdo[0][0]);
  const uint32_t slse_addr = lds_address(&slse[0][0]);
  const uint32_t sdel_addr = lds_address(&sdel[0][0]);
  auto load_block = [&](int b, int buf) __attribute__((always_inline)) {
    const int q0 = (qb_first + b) * C::kBQ;
    const int valid = n_q - q0;
    dma.load(qp + (size_t)q0 * D, valid, sq_addr + buf * C::QT::kBytes);
    dma.load(dop + (size_t)q0 * D, valid, sdo_addr + buf * C::QT::kBytes);
    // The two row vectors, 16 lanes x 16 bytes each, copied by the last two
    // waves.  Lane j copies entries 4j .. 4j+3 when entry 4j exists; the up
    // to three entries read past the last query lie in the next row vector
    // or in the workspace's slack (their rows are masked).  Lanes whose
    // entries are all past the end copy entries 0 .. 3 instead.
    if (wave >= C::kWaves - 2 && lane < C::kBQ / 4) {
      const float* src = (wave == C::kWaves - 1 ? lsep : delp) + q0;
      const uint32_t dst = (wave == C::kWaves - 1 ? slse_addr : sdel_addr) + buf * C::kRowVecBytes;
      lds_dma16(dst, src, (uint32_t)((4 * lane < valid ? 4 * lane : 0) * 4));
    }
  };

  // Register files: the dK, dV accumulators (compiler-placed products) and
  // the K, V operands in AGPRs for the whole pass; S and dP, which the vector
  // code reads, in vector registers (products written as inline assembly,
  // see mfma_bf16_v).
  f32x16 dk[C::kDB], dv[C::kDB];
#pragma unroll
  for (int db = 0; db < C::kDB; ++db) { dk[db] = f32x16{}; dv[db] = f32x16{}; }
  f32x16 s, dp;             // S and dP of the current 32-query sub-block
  f32x4 lv[4], dl[4];       // LSE2 and D of the lane's 16 query rows of that sub-block
  float ex[16], dd[16];     // its probabilities and dP - D (element i: row 8(i/4) + 4 hi + i%4)
  u32x4 pb[2], dsb[2];      // P and dS of the previous sub-block as bf16 pairs
#pragma unroll
  for (int i = 0; i < 16; ++i) { ex[i] = 0.f; dd[i] = 0.f; }
  bf16x8 fa[C::kRing], fb[C::kRing];

  // Probability step for element i of the current sub-block (section
  // "Recomputation": P = exp(scale S - LSE), and dP - D for dS = P o (dP - D)).
  // With MASK, hidden pairs (query past n_q, key past n_k, key after query
  // when causal) get P = 0 and dP - D = 0: a row past n_q reads its LSE and D
  // from whatever follows the last row vector (the next head's rows, or
  // workspace slack that nothing writes), so neither may reach dS, not even
  // as 0 * (dP - D), which is NaN when that slack holds NaN bits.
  auto stage_a = [&](auto mask_tag, int i, int qrow0) __attribute__((always_inline)) {
    const int g4 = i >> 2, e = i & 3;
    float p = fast_exp2(fmaf(s[i], sl2, -lv[g4][e]));
    float r = dp[i] - dl[g4][e];
    if constexpr (decltype(mask_tag)::value) {
      if (!Band::in_range(qrow0 + 4 * hi - qvlo + 8 * g4 + e, 0, qvspan)) {
        p = 0.f;
        r = 0.f;
      }
    }
    ex[i] = p;
    dd[i] = r;
    pin(ex[i]);
    pin(dd[i]);
  };
  // dS for key pair pr (elements 2 pr, 2 pr + 1) and both rounded to bf16 in
  // the order of the B operand of dV^T += dO^T P and dK^T += Q^T dS.
  auto stage_b = [&](int pr) __attribute__((always_inline)) {
    const float d0 = ex[2 * pr] * dd[2 * pr], d1 = ex[2 * pr + 1] * dd[2 * pr + 1];
    uint32_t wp = pack_bf16x2(ex[2 * pr], ex[2 * pr + 1]);
    uint32_t wd = pack_bf16x2(d0, d1);
    pin(wp);
    pin(wd);
    pb[pr >> 2][pr & 3] = wp;
    dsb[pr >> 2][pr & 3] = wd;
  };
  auto step_order = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);       // fragment reads
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);       // product
    __builtin_amdgcn_sched_group_barrier(0x2 | 0x400, 4, 0); // vector work
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);       // product
    __builtin_amdgcn_sched_group_barrier(0x2 | 0x400, 64, 0);
    __builtin_amdgcn_sched_barrier(0);
  };

  // Iteration over one 32-query sub-block (rows R0 of stage buffer BUF),
  // software-pipelined with the sub-block before it (rows RP of buffer BP):
  //   region 1: S, dP of this sub-block   with dS and bf16 rounding of the previous
  //   region 2: dV, dK of the previous one with P, dP - D of this one
  // qrow0 is the absolute index of row R0.  FIRST: there is no previous
  // sub-block (the first iteration of a pass); region 2 then has no products,
  // so nothing reads the other buffer, which may hold no data yet (stale LDS
  // bits times a zero probability could be 0 * NaN).
  auto iteration = [&](auto mask_tag, auto buf_tag, auto r0_tag, auto bp_tag, auto rp_tag, auto first_tag,
                       int qrow0) __attribute__((always_inline)) {
    constexpr int BUF = decltype(buf_tag)::value, R0 = decltype(r0_tag)::value;
    constexpr int BP = decltype(bp_tag)::value, RP = decltype(rp_tag)::value;
    constexpr bool FIRST = decltype(first_tag)::value;
    const char* qt = sq[BUF];
    const char* gt = sdo[BUF];
    static_for<0, (C::kS1 < C::kAhead ? C::kS1 : C::kAhead)>([&](auto i) __attribute__((always_inline)) {
      fa[decltype(i)::value] = tqt.read_rows(qt, R0, decltype(i)::value);
      fb[decltype(i)::value] = tqt.read_rows(gt, R0, decltype(i)::value);
    });
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      lv[g4] = *reinterpret_cast<const f32x4*>(&slse[BUF][R0 + 8 * g4 + 4 * hi]);
      dl[g4] = *reinterpret_cast<const f32x4*>(&sdel[BUF][R0 + 8 * g4 + 4 * hi]);
    }
    static_for<0, C::kS1>([&](auto c_tag) __attribute__((always_inline)) {
      constexpr int c = decltype(c_tag)::value;
      if constexpr (c + C::kAhead < C::kS1) {
        fa[(c + C::kAhead) % C::kRing] = tqt.read_rows(qt, R0, c + C::kAhead);
        fb[(c + C::kAhead) % C::kRing] = tqt.read_rows(gt, R0, c + C::kAhead);
      }
      if constexpr (c == 0) {
        s = mfma_bf16_v0(fa[0], kf[0]);
        dp = mfma_bf16_v0(fb[0], vf[0]);
      } else {
        mfma_bf16_v(s, fa[c % C::kRing], kf[c]);
        mfma_bf16_v(dp, fb[c % C::kRing], vf[c]);
      }
      static_for<c * 8 / C::kS1, (c + 1) * 8 / C::kS1>([&](auto pr) __attribute__((always_inline)) {
        stage_b(decltype(pr)::value);
      });
      if constexpr (c == C::kS1 - 1 && !FIRST) {
        static_for<0, (C::kS2 < C::kAhead ? C::kS2 : C::kAhead)>([&](auto i) __attribute__((always_inline)) {
          constexpr int f = decltype(i)::value;
          fa[f] = tqt.read_cols_tr(sdo[BP], RP + 16 * (f / C::kDB), 32 * (f % C::kDB));
          fb[f] = tqt.read_cols_tr(sq[BP], RP + 16 * (f / C::kDB), 32 * (f % C::kDB));
        });
      }
      step_order();
    });
    static_for<0, C::kS2>([&](auto f_tag) __attribute__((always_inline)) {
      constexpr int f = decltype(f_tag)::value;
      constexpr int c2 = f / C::kDB, db = f % C::kDB;
      if constexpr (!FIRST) {
        if constexpr (f + C::kAhead < C::kS2) {
          constexpr int g = f + C::kAhead;
          fa[g % C::kRing] = tqt.read_cols_tr(sdo[BP], RP + 16 * (g / C::kDB), 32 * (g % C::kDB));
          fb[g % C::kRing] = tqt.read_cols_tr(sq[BP], RP + 16 * (g / C::kDB), 32 * (g % C::kDB));
        }
        dv[db] = mfma_bf16(fa[f % C::kRing], bf16x8_of(pb[c2]), dv[db]);
        dk[db] = mfma_bf16(fb[f % C::kRing], bf16x8_of(dsb[c2]), dk[db]);
      }
      if constexpr (f == 0) fence_results(s, dp);  // S and dP are read from here on
      static_for<f * 16 / C::kS2, (f + 1) * 16 / C::kS2>([&](auto i) __attribute__((always_inline)) {
        stage_a(mask_tag, decltype(i)::value, qrow0);
      });
      step_order();
    });
  };

  // One 64-query stage in buffer BUF: its two sub-blocks, the first paired
  // with the second sub-block of the previous stage (buffer BUF ^ 1).  The
  // stage was copied during the previous stage; after the first sub-block
  // every wave is past the previous stage, whose buffer then takes the next.
  // FIRST: the first stage of a pass (its first sub-block has no
  // predecessor).
  auto do_stage = [&](auto mask_tag, auto buf_tag, int b, auto first_tag) __attribute__((always_inline)) {
    constexpr int BUF = decltype(buf_tag)::value;
    using IB = std::integral_constant<int, BUF>;
    using IP = std::integral_constant<int, BUF ^ 1>;
    using R0 = std::integral_constant<int, 0>;
    using R32 = std::integral_constant<int, 32>;
    const int qrow0 = (qb_first + b) * C::kBQ;
    wait_lds_dma();
    phase_barrier();
    iteration(mask_tag, IB{}, R0{}, IP{}, R32{}, first_tag, qrow0);
    phase_barrier();
    if (b + 1 < nblocks) load_block(b + 1, BUF ^ 1);
    iteration(mask_tag, IB{}, R32{}, IB{}, R0{}, F{}, qrow0 + 32);
  };

  // Stages [b_lo, b_hi) need no mask: every row sees every key of the
  // workgroup below n_k.  The others -- causal diagonal, window edges, a
  // ragged last stage -- are masked.  Keys past n_k need no mask: their K and
  // V rows are zero, a product keeps each key's column apart, and their dK
  // and dV are never stored.
  int b_lo, b_hi;
  {
    const int full_lo = band.q_full_lo(k1), full_hi = min(n_q, band.q_full_hi(k0));
    b_lo = min(nblocks, max(0, (full_lo - qb_first * C::kBQ + C::kBQ - 1) / C::kBQ));
    b_hi = max(b_lo, min(nblocks, (full_hi - qb_first * C::kBQ) / C::kBQ));
  }

  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;
  const bool any_masked = b_lo > 0 || b_hi < nblocks;

  // A masked stage, without the pipeline (they are few: the causal diagonal
  // and ragged ends): per sub-block S and dP, masked P and dS, then the dV
  // and dK products.  The next stage is started at once, since nothing here
  // reads the other buffer.
  // Query rows that see some key of this wave (none past n_k): a masked
  // sub-block outside them is skipped.
  const int kw0 = k0 + wave * 32;
  const int wq_lo = kw0 < n_k ? band.q_lo(kw0) : 0;
  const int wq_hi = kw0 < n_k ? band.q_hi(min(n_k, kw0 + 32)) : 0;
  auto masked_stage = [&](int b) __attribute__((always_inline)) {
    const int buf = b & 1;
    wait_lds_dma();
    phase_barrier();
    if (b + 1 < nblocks) load_block(b + 1, buf ^ 1);
    const char* qt = sq[buf];
    const char* gt = sdo[buf];
#pragma unroll 1
    for (int r0 = 0; r0 < C::kBQ; r0 += 32) {
      const int qs = (qb_first + b) * C::kBQ + r0;
      if (qs + 32 <= wq_lo || qs >= wq_hi) continue;  // no row here sees a key of this wave
      s = mfma_bf16_v0(tqt.read_rows(qt, r0, 0), kf[0]);
      dp = mfma_bf16_v0(tqt.read_rows(gt, r0, 0), vf[0]);
#pragma unroll
      for (int c = 1; c < C::kDC; ++c) {
        mfma_bf16_v(s, tqt.read_rows(qt, r0, c), kf[c]);
        mfma_bf16_v(dp, tqt.read_rows(gt, r0, c), vf[c]);
      }
      fence_results(s, dp);
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        lv[g4] = *reinterpret_cast<const f32x4*>(&slse[buf][r0 + 8 * g4 + 4 * hi]);
        dl[g4] = *reinterpret_cast<const f32x4*>(&sdel[buf][r0 + 8 * g4 + 4 * hi]);
      }
      const int qrow0 = (qb_first + b) * C::kBQ + r0;
      static_for<0, 16>([&](auto i) __attribute__((always_inline)) { stage_a(T{}, decltype(i)::value, qrow0); });
      static_for<0, 8>([&](auto pr) __attribute__((always_inline)) { stage_b(decltype(pr)::value); });
#pragma unroll
      for (int f = 0; f < C::kS2; ++f) {
        const int c2 = f / C::kDB, db = f % C::kDB;
        dv[db] = mfma_bf16(tqt.read_cols_tr(gt, r0 + 16 * c2, 32 * db), bf16x8_of(pb[c2]), dv[db]);
        dk[db] = mfma_bf16(tqt.read_cols_tr(qt, r0 + 16 * c2, 32 * db), bf16x8_of(dsb[c2]), dk[db]);
      }
    }
  };

  // dS of the last pipelined sub-block (rows 32..63 of buffer BUF), then
  // its dV and dK products.
  auto finish = [&](auto buf_tag) __attribute__((always_inline)) {
    constexpr int BUF = decltype(buf_tag)::value;
    static_for<0, 8>([&](auto pr) __attribute__((always_inline)) { stage_b(decltype(pr)::value); });
#pragma unroll
    for (int f = 0; f < C::kS2; ++f) {
      const int c2 = f / C::kDB, db = f % C::kDB;
      dv[db] = mfma_bf16(tqt.read_cols_tr(sdo[BUF], 32 + 16 * c2, 32 * db), bf16x8_of(pb[c2]), dv[db]);
      dk[db] = mfma_bf16(tqt.read_cols_tr(sq[BUF], 32 + 16 * c2, 32 * db), bf16x8_of(dsb[c2]), dk[db]);
    }
  };

  // One pass over the query stages of one query head.
  auto one_head = [&]() __attribute__((always_inline)) {
      load_block(0, 0);
      int b = 0;
      if (any_masked)
        for (; b < b_lo; ++b) masked_stage(b);
      // Unmasked stages [b, b_hi) through the pipeline, in pairs with fixed
      // buffers; its state starts empty (zero probabilities for the "previous"
      // sub-block of the first iteration).
      if (b < b_hi) {
  #pragma unroll
        for (int i = 0; i < 16; ++i) { ex[i] = 0.f; dd[i] = 0.f; }
        if (b & 1) do_stage(F{}, B1{}, b, T{});
        else do_stage(F{}, B0{}, b, T{});
        ++b;
        if (b < b_hi && (b & 1)) {
          do_stage(F{}, B1{}, b, F{});
          ++b;
        }
        for (; b + 1 < b_hi; b += 2) {
          do_stage(F{}, B0{}, b, F{});
          do_stage(F{}, B1{}, b + 1, F{});
        }
        if (b < b_hi) {
          do_stage(F{}, B0{}, b, F{});
          ++b;
        }
        if ((b - 1) & 1) finish(B1{});
        else finish(B0{});
      }
      if (any_masked)
        for (; b < nblocks; ++b) masked_stage(b);
  };
  if constexpr (!GROUPED) {
    if (nblocks > 0) one_head();
  } else {
    for (int g = 0; g < run && nblocks > 0; ++g) {
      if (g > 0) {
        qp += (size_t)n_q * D;
        dop += (size_t)n_q * D;
        lsep += n_q;
        delp += n_q;
        // Every wave is past the previous head's last reads of buffer 0.
        phase_barrier();
      }
      one_head();
    }
  }

  if (MODE == 1 || (MODE == 2 && slices > 1)) {
    // float32 partial sums of this run, added up by the reduction
    if (key < n_k) {
      const size_t off = (((size_t)sl * (a.BH / group) + bhkv) * n_k + key) * D;
#pragma unroll
      for (int db = 0; db < C::kDB; ++db)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          f32x4 rk, rv;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            rk[e] = dk[db][4 * g4 + e] * a.scale;
            rv[e] = dv[db][4 * g4 + e];
          }
          *reinterpret_cast<f32x4*>(a.part_dk + off + 32 * db + 8 * g4 + 4 * hi) = rk;
          *reinterpret_cast<f32x4*>(a.part_dv + off + 32 * db + 8 * g4 + 4 * hi) = rv;
        }
    }
    return;
  }
  if (key < n_k) {
    __bf16* dkp = static_cast<__bf16*>(a.dk) + ((size_t)bhkv * n_k + key) * D;
    __bf16* dvp = static_cast<__bf16*>(a.dv) + ((size_t)bhkv * n_k + key) * D;
#pragma unroll
    for (int db = 0; db < C::kDB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        bf16x4 rk, rv;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          rk[e] = (__bf16)(dk[db][4 * g4 + e] * a.scale);
          rv[e] = (__bf16)dv[db][4 * g4 + e];
        }
        *reinterpret_cast<bf16x4*>(dkp + 32 * db + 8 * g4 + 4 * hi) = rk;
        *reinterpret_cast<bf16x4*>(dvp + 32 * db + 8 * g4 + 4 * hi) = rv;
      }
  }
}

// ------------------------------------------------------ stage 3 (bf16)

template <int D, int WAVES>
struct DqCfg {
  static constexpr int kWaves = WAVES;           // 8: two per SIMD; 4 with a sliding window
  static constexpr int kThreads = kWaves * 64;
  static constexpr int kBM = kWaves * 32;        // queries per workgroup, 32 per wave
  static constexpr int kBN = 64;                 // keys per block
  static constexpr int kKB = kBN / 32;
  static constexpr int kDC = D / 16;
  static constexpr int kDB = D / 32;
  using KV = Tile<D, kBN>;
};

template <int D, bool CAUSAL, int WAVES>
__global__ __launch_bounds__(WAVES * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bwd_dq_bf16_kernel(BwdArgs a, int n_qtiles) {
  using C = DqCfg<D, WAVES>;
  __shared__ __attribute__((aligned(1024))) char sk[2][C::KV::kBytes];
  __shared__ __attribute__((aligned(1024))) char sv[2][C::KV::kBytes];

  int bh, qt;
  if (CAUSAL) {
    // the last query tiles see the most keys: they go first
    costliest_first(blockIdx.x, gridDim.x, n_qtiles, bh, qt);
    qt = n_qtiles - 1 - qt;
  } else {
    const int work = xcd_remap(blockIdx.x, gridDim.x);
    bh = work / n_qtiles;
    qt = work - bh * n_qtiles;
  }

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  const int n_q = a.n_q, n_k = a.n_k;
  const float sl2 = a.scale_log2;
  const int q0 = qt * C::kBM;
  const int qw = q0 + wave * 32;
  const int qi = qw + l32;  // this lane's query (column of S^T)

  const __bf16* qp = static_cast<const __bf16*>(a.q) + (size_t)bh * n_q * D;
  const __bf16* dop = static_cast<const __bf16*>(a.dO) + (size_t)bh * n_q * D;
  const int kvh = kv_head_index(bh, a.H, a.group);
  const __bf16* kp = static_cast<const __bf16*>(a.k) + (size_t)kvh * n_k * D;
  const __bf16* vp = static_cast<const __bf16*>(a.v) + (size_t)kvh * n_k * D;

  bf16x8 qf[C::kDC], gf[C::kDC];
#pragma unroll
  for (int c = 0; c < C::kDC; ++c) {
    if (qi < n_q) {
      qf[c] = *reinterpret_cast<const bf16x8*>(qp + (size_t)qi * D + 16 * c + 8 * hi);
      gf[c] = *reinterpret_cast<const bf16x8*>(dop + (size_t)qi * D + 16 * c + 8 * hi);
    } else {
      qf[c] = bf16x8{};
      gf[c] = bf16x8{};
    }
  }
  // Rows past n_q have zero Q and dO, so their (unstored) dQ stays finite.
  const float lse2 = (qi < n_q) ? a.lse2[(size_t)bh * n_q + qi] : 0.f;
  const float dlt = (qi < n_q) ? a.delta[(size_t)bh * n_q + qi] : 0.f;

  // Key blocks [t_lo, t_hi) hold keys some row of the workgroup sees;
  // blocks [f_lo, f_hi) need no mask for any row.
  const Band band = band_of(a, CAUSAL);
  const int q_end = min(n_q, q0 + C::kBM);
  const int t_lo = band.key_lo(q0) / C::kBN;
  const int t_hi = max(t_lo, (band.key_hi(q_end) + C::kBN - 1) / C::kBN);
  const int f_lo = min(t_hi, max(t_lo, (band.key_full_lo(q_end) + C::kBN - 1) / C::kBN));
  const int f_hi = max(f_lo, min(t_hi, band.key_full_hi(q0) / C::kBN));
  int vlo, vspan;  // keys this lane's query sees: [vlo, vlo + vspan]
  band.key_range(qi, vlo, vspan);

  TileDma<D, C::kBN, C::kWaves> dma;
  dma.init(wave, lane);
  TileLane<D, C::kBN> tkv;
  tkv.init(lane);
  const uint32_t sk_addr = lds_address(&sk[0][0]);
  const uint32_t sv_addr = lds_address(&sv[0][0]);
  auto load_tile = [&](int t, int buf) {
    const int k0 = t * C::kBN;
    dma.load(kp + (size_t)k0 * D, n_k - k0, sk_addr + buf * C::KV::kBytes);
    dma.load(vp + (size_t)k0 * D, n_k - k0, sv_addr + buf * C::KV::kBytes);
  };

  f32x16 dq[C::kDB];
#pragma unroll
  for (int db = 0; db < C::kDB; ++db) dq[db] = f32x16{};
  // dP^T accumulates from -D (one query per lane), so the products give
  // dP - D for dS = P o (dP - D) directly.
  f32x16 neg_d;
#pragma unroll
  for (int i = 0; i < 16; ++i) neg_d[i] = -dlt;

  auto block = [&](auto mask_tag, auto buf_tag, int t) {
    constexpr bool MASK = decltype(mask_tag)::value;
    constexpr int BUFC = decltype(buf_tag)::value;
    const int buf = BUFC >= 0 ? BUFC : (t & 1);
    wait_lds_dma();
    __syncthreads();
    if (t + 1 < t_hi) load_tile(t + 1, buf ^ 1);
    const char* ks = sk[buf];
    const char* vs = sv[buf];
    const int k0 = t * C::kBN;
#pragma unroll
    for (int kb = 0; kb < C::kKB; ++kb) {
      // every key of the sub-block hidden from this wave
      if (MASK && (k0 + kb * 32 >= band.key_hi(qw + 32) || k0 + kb * 32 + 32 <= band.key_lo(qw))) continue;
      f32x16 s = f32x16{}, dp = neg_d;
#pragma unroll
      for (int c = 0; c < C::kDC; ++c) {
        s = mfma_bf16(tkv.read_rows(ks, kb * 32, c), qf[c], s);
        dp = mfma_bf16(tkv.read_rows(vs, kb * 32, c), gf[c], dp);
      }
      u32x4 dsb[2];
#pragma unroll
      for (int i = 0; i < 16; i += 2) {
        float p0 = fast_exp2(fmaf(s[i], sl2, -lse2));
        float p1 = fast_exp2(fmaf(s[i + 1], sl2, -lse2));
        if constexpr (MASK) {
          const int rel = k0 + kb * 32 + 4 * hi - vlo + 8 * (i >> 2) + (i & 3);  // key - vlo
          if (!Band::in_range(rel, 0, vspan)) p0 = 0.f;
          if (!Band::in_range(rel + 1, 0, vspan)) p1 = 0.f;
        }
        dsb[i >> 3][(i & 7) >> 1] = pack_bf16x2(p0 * dp[i], p1 * dp[i + 1]);
      }
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
        for (int db = 0; db < C::kDB; ++db)
          dq[db] = mfma_bf16(tkv.read_cols_tr(ks, kb * 32 + 16 * c2, 32 * db),
                             bf16x8_of(dsb[c2]), dq[db]);
    }
  };

  // Unmasked blocks two at a time with fixed buffers (block t in buffer
  // t % 2), the others masked.
  if (t_lo < t_hi) load_tile(t_lo, t_lo & 1);
  int t = t_lo;
  for (; t < f_lo; ++t) block(T{}, Buf<-1>{}, t);
  if (t < f_hi && (t & 1)) {
    block(F{}, Buf<-1>{}, t);
    ++t;
  }
  for (; t + 1 < f_hi; t += 2) {
    block(F{}, Buf<0>{}, t);
    block(F{}, Buf<1>{}, t + 1);
  }
  for (; t < f_hi; ++t) block(F{}, Buf<-1>{}, t);
  for (; t < t_hi; ++t) block(T{}, Buf<-1>{}, t);

  if (qi < n_q) {
    __bf16* dqp = static_cast<__bf16*>(a.dq) + ((size_t)bh * n_q + qi) * D;
#pragma unroll
    for (int db = 0; db < C::kDB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        bf16x4 r;
#pragma unroll
        for (int e = 0; e < 4; ++e) r[e] = (__bf16)(dq[db][4 * g4 + e] * a.scale);
        *reinterpret_cast<bf16x4*>(dqp + 32 * db + 8 * g4 + 4 * hi) = r;
      }
  }
}

// bf16 stage 3 at d = 128, the two waves of each SIMD half a step apart
// (as the forward's ping-pong kernel): a wave's step i is
//   phase A(i): dQ^T += K^T dS^T of block f_lo + i - 1 (if i > 0), then
//               S^T = K Q^T and dP^T = V dO^T of block f_lo + i (if i < n)
//   phase B(i): P = exp2(scale_log2 S - LSE2), dS = P o (dP - D), bf16
// so that one wave's vector work runs beside the other wave's products.
// Phase A reads two K blocks (K^T of the previous block for dQ, K rows of
// this one for S): K blocks take four LDS buffers (three would do; four
// keep the buffer indices compile-time constants in a loop unrolled by
// four), V blocks two.  Waves 4-7
// run one barrier behind and issue the copies in their phase B: in B(i) K
// and V of block f_lo + i + 2, into the buffers of blocks f_lo + i - 1 (K,
// last read in A(i)) and f_lo + i (V, last read in A(i)); they wait for the
// copies before the barrier in the middle of their next step, which
// precedes the first read.  Blocks that need a mask (before f_lo: window
// edges; from f_hi on: causal diagonal, key tail) take the plain path.
// The same products as bwd_dq_bf16_kernel, except that dP is accumulated
// from zero and D subtracted in phase B (a tile of -D as the products'
// starting value would hold 16 more registers), so the two kernels' dQ may
// differ in the last bf16 bit.  c3 dQ 331.9 -> 321.8 us, causal B=2 H=16
// 176.4 -> 172.6 us, n = 8192 1290.5 -> 1240.3 us (same box).
template <int D, bool CAUSAL>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bwd_dq_bf16_pp_kernel(BwdArgs a, int n_qtiles) {
  using C = DqCfg<D, 8>;
  constexpr int kKBufs = 4;
  __shared__ __attribute__((aligned(1024))) char sv[2][C::KV::kBytes];
  __shared__ __attribute__((aligned(1024))) char sk[kKBufs][C::KV::kBytes];

  int bh, qt;
  if (CAUSAL) {
    costliest_first(blockIdx.x, gridDim.x, n_qtiles, bh, qt);
    qt = n_qtiles - 1 - qt;
  } else {
    const int work = xcd_remap(blockIdx.x, gridDim.x);
    bh = work / n_qtiles;
    qt = work - bh * n_qtiles;
  }

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;  // 0: waves 0-3, 1: waves 4-7, one half-step behind
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  const int n_q = a.n_q, n_k = a.n_k;
  const float sl2 = a.scale_log2;
  const int q0 = qt * C::kBM;
  const int qw = q0 + wave * 32;
  const int qi = qw + l32;  // this lane's query (column of S^T)

  const __bf16* qp = static_cast<const __bf16*>(a.q) + (size_t)bh * n_q * D;
  const __bf16* dop = static_cast<const __bf16*>(a.dO) + (size_t)bh * n_q * D;
  const int kvh = kv_head_index(bh, a.H, a.group);
  const __bf16* kp = static_cast<const __bf16*>(a.k) + (size_t)kvh * n_k * D;
  const __bf16* vp = static_cast<const __bf16*>(a.v) + (size_t)kvh * n_k * D;

  bf16x8 qf[C::kDC], gf[C::kDC];
#pragma unroll
  for (int c = 0; c < C::kDC; ++c) {
    if (qi < n_q) {
      qf[c] = *reinterpret_cast<const bf16x8*>(qp + (size_t)qi * D + 16 * c + 8 * hi);
      gf[c] = *reinterpret_cast<const bf16x8*>(dop + (size_t)qi * D + 16 * c + 8 * hi);
    } else {
      qf[c] = bf16x8{};
      gf[c] = bf16x8{};
    }
  }
  // Rows past n_q have zero Q and dO, so their (unstored) dQ stays finite.
  const float lse2 = (qi < n_q) ? a.lse2[(size_t)bh * n_q + qi] : 0.f;
  const float dlt = (qi < n_q) ? a.delta[(size_t)bh * n_q + qi] : 0.f;

  const Band band = band_of(a, CAUSAL);
  const int q_end = min(n_q, q0 + C::kBM);
  const int t_lo = band.key_lo(q0) / C::kBN;
  const int t_hi = max(t_lo, (band.key_hi(q_end) + C::kBN - 1) / C::kBN);
  const int f_lo = min(t_hi, max(t_lo, (band.key_full_lo(q_end) + C::kBN - 1) / C::kBN));
  const int f_hi = max(f_lo, min(t_hi, band.key_full_hi(q0) / C::kBN));
  const int n = f_hi - f_lo;  // blocks of the ping-pong
  int vlo, vspan;  // keys this lane's query sees: [vlo, vlo + vspan]
  band.key_range(qi, vlo, vspan);

  TileDma<D, C::kBN, C::kWaves> dma;
  dma.init(wave, lane);
  TileDma<D, C::kBN, 4> dma4;
  dma4.init(wave & 3, lane);
  TileLane<D, C::kBN> tkv;
  tkv.init(lane);
  const uint32_t sk_addr = lds_address(&sk[0][0]);
  const uint32_t sv_addr = lds_address(&sv[0][0]);
  // Block t: K in buffer (t - f_lo) mod 3, V in buffer (t - f_lo) mod 2.
  auto kbufof = [&](int t) { return (t - f_lo) & (kKBufs - 1); };
  auto vbufof = [&](int t) { return (t - f_lo) & 1; };
  auto load_tile = [&](int t) {
    const int k0 = t * C::kBN;
    dma.load(kp + (size_t)k0 * D, n_k - k0, sk_addr + kbufof(t) * C::KV::kBytes);
    dma.load(vp + (size_t)k0 * D, n_k - k0, sv_addr + vbufof(t) * C::KV::kBytes);
  };

  f32x16 dq[C::kDB];
#pragma unroll
  for (int db = 0; db < C::kDB; ++db) dq[db] = f32x16{};

  // A masked block (plain path): wait for block t, barrier, start the copy
  // of block t + 1, then S, dP, masked dS and dQ for both 32-key halves.
  // dP^T accumulates from -D, so the products give dP - D directly.
  auto masked_block = [&](int t) {
    wait_lds_dma();
    __syncthreads();
    if (t + 1 < t_hi) load_tile(t + 1);
    const char* ks = sk[kbufof(t)];
    const char* vs = sv[vbufof(t)];
    const int k0 = t * C::kBN;
#pragma unroll
    for (int kb = 0; kb < C::kKB; ++kb) {
      // every key of the sub-block hidden from this wave
      if (k0 + kb * 32 >= band.key_hi(qw + 32) || k0 + kb * 32 + 32 <= band.key_lo(qw)) continue;
      f32x16 s = f32x16{}, dp;
#pragma unroll
      for (int i = 0; i < 16; ++i) dp[i] = -dlt;
#pragma unroll
      for (int c = 0; c < C::kDC; ++c) {
        s = mfma_bf16(tkv.read_rows(ks, kb * 32, c), qf[c], s);
        dp = mfma_bf16(tkv.read_rows(vs, kb * 32, c), gf[c], dp);
      }
      u32x4 dsb[2];
#pragma unroll
      for (int i = 0; i < 16; i += 2) {
        float p0 = fast_exp2(fmaf(s[i], sl2, -lse2));
        float p1 = fast_exp2(fmaf(s[i + 1], sl2, -lse2));
        const int rel = k0 + kb * 32 + 4 * hi - vlo + 8 * (i >> 2) + (i & 3);  // key - vlo
        if (!Band::in_range(rel, 0, vspan)) p0 = 0.f;
        if (!Band::in_range(rel + 1, 0, vspan)) p1 = 0.f;
        dsb[i >> 3][(i & 7) >> 1] = pack_bf16x2(p0 * dp[i], p1 * dp[i + 1]);
      }
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
        for (int db = 0; db < C::kDB; ++db)
          dq[db] = mfma_bf16(tkv.read_cols_tr(ks, kb * 32 + 16 * c2, 32 * db), bf16x8_of(dsb[c2]), dq[db]);
    }
  };

  if (t_lo < t_hi) load_tile(t_lo);
  int t = t_lo;
  for (; t < f_lo; ++t) masked_block(t);  // up to block f_lo's copy

  if (n > 0) {
    f32x16 s[C::kKB], dp[C::kKB];  // S^T and dP^T of the wave's current block
    u32x4 dsb[C::kKB][2];          // its dS as bf16 pairs
    // Phase A as one stream of product steps: steps 0-15 the dQ products of
    // the previous block (two transposing K reads each), then for c = 0..7
    // the S and dP products of both 32-key halves (one K or V row read
    // each).  Operand reads run kAhead steps ahead through a ring.
    constexpr int kDq = 2 * C::kKB * C::kDB;   // 16
    constexpr int kSd = 2 * C::kKB * C::kDC;   // 32
    constexpr int kAhead = 4;
    // kc_tag: K buffer of this step's block (the previous block's is the
    // one before it, mod 4), V buffer kc mod 2; compile-time in the unrolled
    // loop, run-time in the last few steps.
    auto phase_a = [&](auto kc_tag, auto dq_tag, auto sd_tag) __attribute__((always_inline)) {
      constexpr bool DQ = decltype(dq_tag)::value, SD = decltype(sd_tag)::value;
      constexpr int J0 = DQ ? 0 : kDq, J1 = SD ? kDq + kSd : kDq;
      const int kc = value_of(kc_tag);
      const char* kprev = sk[(kc + kKBufs - 1) & (kKBufs - 1)];  // K of the previous block (dQ)
      const char* kcur = sk[kc];                                 // K and V of this block (S, dP)
      const char* vcur = sv[kc & 1];
      auto read = [&](auto j_tag) __attribute__((always_inline)) -> bf16x8 {
        constexpr int J = decltype(j_tag)::value;
        if constexpr (J < kDq) {
          constexpr int kb = J / (2 * C::kDB), c2 = (J / C::kDB) % 2, db = J % C::kDB;
          return tkv.read_cols_tr(kprev, kb * 32 + 16 * c2, 32 * db);
        } else {
          constexpr int c = (J - kDq) / (2 * C::kKB), kb = ((J - kDq) / 2) % C::kKB, v = (J - kDq) % 2;
          return tkv.read_rows(v ? vcur : kcur, kb * 32, c);
        }
      };
      auto product = [&](auto j_tag, const bf16x8& op) __attribute__((always_inline)) {
        constexpr int J = decltype(j_tag)::value;
        if constexpr (J < kDq) {
          constexpr int kb = J / (2 * C::kDB), c2 = (J / C::kDB) % 2, db = J % C::kDB;
          dq[db] = mfma_bf16(op, bf16x8_of(dsb[kb][c2]), dq[db]);
        } else {
          constexpr int c = (J - kDq) / (2 * C::kKB), kb = ((J - kDq) / 2) % C::kKB, v = (J - kDq) % 2;
          if constexpr (v == 0)
            s[kb] = mfma_bf16(op, qf[c], c == 0 ? f32x16{} : s[kb]);
          else
            dp[kb] = mfma_bf16(op, gf[c], c == 0 ? f32x16{} : dp[kb]);
        }
      };
      bf16x8 ring[kAhead];
      phase_barrier();
      // The product phase issues at raised wave priority, so that on each
      // SIMD its products and operand reads go ahead of the other wave's
      // vector work (c3 dQ 318.7 -> 315.2 us, bitwise the same results).
      __builtin_amdgcn_s_setprio(1);
      static_for<J0, (J0 + kAhead < J1 ? J0 + kAhead : J1)>([&](auto j) __attribute__((always_inline)) {
        ring[(decltype(j)::value - J0) % kAhead] = read(j);
      });
      __builtin_amdgcn_sched_barrier(0);
      static_for<J0, J1>([&](auto j) __attribute__((always_inline)) {
        constexpr int J = decltype(j)::value;
        product(j, ring[(J - J0) % kAhead]);
        if constexpr (J + kAhead < J1) ring[(J - J0) % kAhead] = read(std::integral_constant<int, J + kAhead>{});
        __builtin_amdgcn_sched_barrier(0);  // each product with the read kAhead steps ahead
      });
      __builtin_amdgcn_s_setprio(0);
    };
    // Phase B: dS = P o (dP - D) of both halves, rounded to bf16 pairs.
    auto phase_b = [&]() __attribute__((always_inline)) {
#pragma unroll
      for (int kb = 0; kb < C::kKB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; i += 2) {
          const float p0 = fast_exp2(fmaf(s[kb][i], sl2, -lse2));
          const float p1 = fast_exp2(fmaf(s[kb][i + 1], sl2, -lse2));
          dsb[kb][i >> 3][(i & 7) >> 1] = pack_bf16x2(p0 * (dp[kb][i] - dlt), p1 * (dp[kb][i + 1] - dlt));
        }
    };
    auto step = [&](auto kc_tag, auto dq_tag, auto sd_tag, int i) __attribute__((always_inline)) {
      phase_a(kc_tag, dq_tag, sd_tag);
      if (grp == 1) wait_lds_dma();
      phase_barrier();
      if (grp == 1) {
        const int tn = f_lo + i + 2;
        if (tn <= f_hi && tn < t_hi) {
          const int k0 = tn * C::kBN;
          dma4.load(kp + (size_t)k0 * D, n_k - k0, sk_addr + kbufof(tn) * C::KV::kBytes);
          dma4.load(vp + (size_t)k0 * D, n_k - k0, sv_addr + vbufof(tn) * C::KV::kBytes);
        }
      }
      if constexpr (decltype(sd_tag)::value) phase_b();
    };
    // Block f_lo was started by the previous block or the first copy; every
    // wave waits for its part before the ping-pong starts, and waves 4-7
    // start block f_lo + 1 (read first at step 1).
    wait_lds_dma();
    if (grp == 1) {
      if (f_lo + 1 <= f_hi && f_lo + 1 < t_hi) {
        const int k0 = (f_lo + 1) * C::kBN;
        dma4.load(kp + (size_t)k0 * D, n_k - k0, sk_addr + kbufof(f_lo + 1) * C::KV::kBytes);
        dma4.load(vp + (size_t)k0 * D, n_k - k0, sv_addr + vbufof(f_lo + 1) * C::KV::kBytes);
      }
      phase_barrier();
    }
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using I3 = std::integral_constant<int, 3>;
    step(I0{}, F{}, T{}, 0);  // S and dP of block f_lo only
    int i = 1;
    for (; i + 3 < n; i += 4) {
      step(I1{}, T{}, T{}, i);
      step(I2{}, T{}, T{}, i + 1);
      step(I3{}, T{}, T{}, i + 2);
      step(I0{}, T{}, T{}, i + 3);
    }
    for (; i < n; ++i) step(i & (kKBufs - 1), T{}, T{}, i);
    step(n & (kKBufs - 1), T{}, F{}, n);  // the last dQ products only
    if (grp == 0) phase_barrier();
    t = f_hi;
  }
  // After the ping-pong: block f_hi's K and V were started at step n - 2
  // (or before the first step when n = 1; nothing beyond); the masked blocks
  // continue with one block of look-ahead.
  for (; t < t_hi; ++t) masked_block(t);

  if (qi < n_q) {
    __bf16* dqp = static_cast<__bf16*>(a.dq) + ((size_t)bh * n_q + qi) * D;
#pragma unroll
    for (int db = 0; db < C::kDB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        bf16x4 r;
#pragma unroll
        for (int e = 0; e < 4; ++e) r[e] = (__bf16)(dq[db][4 * g4 + e] * a.scale);
        *reinterpret_cast<bf16x4*>(dqp + 32 * db + 8 * g4 + 4 * hi) = r;
      }
  }
}

// ------------------------------------------------------ fp32 stages 2, 3
//
// Same dataflow on the 32x32x2 f32 matrix cores: operands are single floats
// (lane l supplies row/col l%32 at k = l/32), so every operand comes from
// LDS with plain 4-byte reads and no transposing read is needed.

template <int D>
struct F32BwdCfg {
  static constexpr int kWaves = 4;
  static constexpr int kThreads = kWaves * 64;
  static constexpr int kBlk = kWaves * 32;       // rows owned per workgroup
  static constexpr int kBS = 32;                 // streamed rows per block
  static constexpr int kDB = D / 32;
  static constexpr int kStride = D + 8;          // floats
  static constexpr int kChunks = D / 4;
  static constexpr int kLoads = kBS * kChunks / kThreads;
  static_assert(kLoads * kThreads == kBS * kChunks, "tile load split");
};

// Stage 2, fp32: wave owns 32 keys; streams 32-query blocks of Q and dO.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) void bwd_dkdv_f32_kernel(BwdArgs a, int n_ktiles) {
  using C = F32BwdCfg<D>;
  __shared__ __attribute__((aligned(16))) float sq[2][C::kBS * C::kStride];
  __shared__ __attribute__((aligned(16))) float sdo[2][C::kBS * C::kStride];
  __shared__ float slse[2][C::kBS];
  __shared__ float sdel[2][C::kBS];

  // One workgroup per (key tile, batch * K/V head), summing over the query
  // heads that share the K/V head.
  // Work item (key tile, K/V head, run of `run` consecutive query heads).
  const int run = a.group / a.slices;
  int hs, kt;
  if (CAUSAL) {
    // the first key tiles are seen by the most queries: they go first
    costliest_first(blockIdx.x, gridDim.x, n_ktiles, hs, kt);
  } else {
    const int work = xcd_remap(blockIdx.x, gridDim.x);
    hs = work / n_ktiles;
    kt = work - hs * n_ktiles;
  }
  const int bhkv = hs / a.slices;
  const int sl = hs - bhkv * a.slices;
  const int h_kv = a.H / a.group;
  const int bh0 = (bhkv / h_kv) * a.H + (bhkv % h_kv) * a.group + sl * run;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  const int n_q = a.n_q, n_k = a.n_k;
  const int k0 = kt * C::kBlk;
  const int kw = k0 + wave * 32;
  const int key = kw + l32;

  const float* qp = nullptr;
  const float* dop = nullptr;
  const float* lsep = nullptr;
  const float* delp = nullptr;
  const float* kp = static_cast<const float*>(a.k) + (size_t)bhkv * n_k * D;
  const float* vp = static_cast<const float*>(a.v) + (size_t)bhkv * n_k * D;

  // K and V rows of this lane's key, as B operands (d = 2c + hi).
  float kreg[D / 2], vreg[D / 2];
#pragma unroll
  for (int c = 0; c < D / 2; ++c) {
    kreg[c] = (key < n_k) ? kp[(size_t)key * D + 2 * c + hi] : 0.f;
    vreg[c] = (key < n_k) ? vp[(size_t)key * D + 2 * c + hi] : 0.f;
  }

  const Band band = band_of(a, CAUSAL);
  const int k1 = min(n_k, k0 + C::kBlk);
  const int q_first = band.q_lo(k0), q_last = band.q_hi(k1);
  const int qb_first = q_first / C::kBS;
  const int nblocks = q_last > q_first ? (q_last + C::kBS - 1) / C::kBS - qb_first : 0;
  const int wq_lo = band.q_lo(kw), wq_hi = band.q_hi(min(n_k, kw + 32));  // rows seeing this wave's keys

  f32x4 qst[C::kLoads], dost[C::kLoads];
  float lse_st = 0.f, del_st = 0.f;
  auto gload = [&](int b) {
    const int qbase = (qb_first + b) * C::kBS;
#pragma unroll
    for (int i = 0; i < C::kLoads; ++i) {
      const int idx = tid + i * C::kThreads;
      const int row = idx / C::kChunks;
      const int ch = idx - row * C::kChunks;
      const int qi = qbase + row;
      if (qi < n_q) {
        qst[i] = *reinterpret_cast<const f32x4*>(qp + (size_t)qi * D + ch * 4);
        dost[i] = *reinterpret_cast<const f32x4*>(dop + (size_t)qi * D + ch * 4);
      } else {
        qst[i] = f32x4{};
        dost[i] = f32x4{};
      }
    }
    if (tid < C::kBS) {
      const int qi = qbase + tid;
      lse_st = (qi < n_q) ? lsep[qi] : 0.f;
      del_st = (qi < n_q) ? delp[qi] : 0.f;
    }
  };
  auto swrite = [&](int buf) {
#pragma unroll
    for (int i = 0; i < C::kLoads; ++i) {
      const int idx = tid + i * C::kThreads;
      const int row = idx / C::kChunks;
      const int ch = idx - row * C::kChunks;
      *reinterpret_cast<f32x4*>(&sq[buf][row * C::kStride + ch * 4]) = qst[i];
      *reinterpret_cast<f32x4*>(&sdo[buf][row * C::kStride + ch * 4]) = dost[i];
    }
    if (tid < C::kBS) {
      slse[buf][tid] = lse_st;
      sdel[buf][tid] = del_st;
    }
  };

  f32x16 dk[C::kDB], dv[C::kDB];
#pragma unroll
  for (int db = 0; db < C::kDB; ++db) { dk[db] = f32x16{}; dv[db] = f32x16{}; }

  for (int g = 0; g < run; ++g) {
  const size_t bh = (size_t)(bh0 + g);
  qp = static_cast<const float*>(a.q) + bh * n_q * D;
  dop = static_cast<const float*>(a.dO) + bh * n_q * D;
  lsep = a.lse2 + bh * n_q;
  delp = a.delta + bh * n_q;
  if (nblocks > 0) {
    gload(0);
    swrite(0);
  }
  __syncthreads();

  for (int b = 0; b < nblocks; ++b) {
    const int buf = b & 1;
    if (b + 1 < nblocks) gload(b + 1);
    const int qbase = (qb_first + b) * C::kBS;
    if (kw < n_k && qbase < wq_hi && qbase + C::kBS > wq_lo) {
      // S = Q K^T and dP = dO V^T: A = Q/dO rows (query l%32, d = 2c + hi),
      // B = K/V rows (key l%32, d = 2c + hi).
      f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int c = 0; c < D / 2; ++c) {
        s = mfma_f32(sq[buf][l32 * C::kStride + 2 * c + hi], kreg[c], s);
        dp = mfma_f32(sdo[buf][l32 * C::kStride + 2 * c + hi], vreg[c], dp);
      }
      f32x16 p, ds;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int r = 8 * (i >> 2) + 4 * hi + (i & 3);
        const int qi = qbase + r;
        float pv = fast_exp2(fmaf(s[i], a.scale_log2, -slse[buf][r]));
        const bool hide = qi >= n_q || band.hidden(qi, key);
        pv = hide ? 0.f : pv;
        p[i] = pv;
        ds[i] = pv * (dp[i] - sdel[buf][r]);
      }
      // dV^T[d][key] += dO^T P: A = dO^T (row d, k = query), B = P (k = query).
      // The block's 32 query rows are summed from zero and the block sum is
      // then added to the running total: a key's gradient over many query
      // rows (600 rows on 5 keys: values near 15) otherwise carries the
      // rounding of every addition into a large running sum, about
      // sqrt(n_q) half-ulps of the result.  One set of block sums serves dV,
      // then dK (two sets would spill at d = 128).
      f32x16 bs[C::kDB];
#pragma unroll
      for (int db = 0; db < C::kDB; ++db) bs[db] = f32x16{};
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int r = 8 * (i >> 2) + 4 * hi + (i & 3);
#pragma unroll
        for (int db = 0; db < C::kDB; ++db)
          bs[db] = mfma_f32(sdo[buf][r * C::kStride + 32 * db + l32], p[i], bs[db]);
      }
      settle_acc(bs);
#pragma unroll
      for (int db = 0; db < C::kDB; ++db) {
        dv[db] += bs[db];
        bs[db] = f32x16{};
      }
      // dK^T[d][key] += Q^T dS, the same way.
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int r = 8 * (i >> 2) + 4 * hi + (i & 3);
#pragma unroll
        for (int db = 0; db < C::kDB; ++db)
          bs[db] = mfma_f32(sq[buf][r * C::kStride + 32 * db + l32], ds[i], bs[db]);
      }
      settle_acc(bs);
#pragma unroll
      for (int db = 0; db < C::kDB; ++db) dk[db] += bs[db];
    }
    if (b + 1 < nblocks) swrite(buf ^ 1);
    __syncthreads();
  }
  }  // query heads of the group

  if (key < n_k) {
    // with several runs, float32 partial sums added up by the reduction
    const bool part = a.slices > 1;
    const size_t off = part ? (((size_t)sl * (a.BH / a.group) + bhkv) * n_k + key) * D
                            : ((size_t)bhkv * n_k + key) * D;
    float* dkp = (part ? a.part_dk : static_cast<float*>(a.dk)) + off;
    float* dvp = (part ? a.part_dv : static_cast<float*>(a.dv)) + off;
#pragma unroll
    for (int db = 0; db < C::kDB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        f32x4 rk, rv;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          rk[e] = dk[db][4 * g4 + e] * a.scale;
          rv[e] = dv[db][4 * g4 + e];
        }
        *reinterpret_cast<f32x4*>(dkp + 32 * db + 8 * g4 + 4 * hi) = rk;
        *reinterpret_cast<f32x4*>(dvp + 32 * db + 8 * g4 + 4 * hi) = rv;
      }
  }
}

// Stage 3, fp32: wave owns 32 queries; streams 32-key blocks of K and V.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) void bwd_dq_f32_kernel(BwdArgs a, int n_qtiles) {
  using C = F32BwdCfg<D>;
  __shared__ __attribute__((aligned(16))) float sk[2][C::kBS * C::kStride];
  __shared__ __attribute__((aligned(16))) float sv[2][C::kBS * C::kStride];

  int bh, qt;
  if (CAUSAL) {
    // the last query tiles see the most keys: they go first
    costliest_first(blockIdx.x, gridDim.x, n_qtiles, bh, qt);
    qt = n_qtiles - 1 - qt;
  } else {
    const int work = xcd_remap(blockIdx.x, gridDim.x);
    bh = work / n_qtiles;
    qt = work - bh * n_qtiles;
  }
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  const int n_q = a.n_q, n_k = a.n_k;
  const int q0 = qt * C::kBlk;
  const int qw = q0 + wave * 32;
  const int qi = qw + l32;

  const float* qp = static_cast<const float*>(a.q) + (size_t)bh * n_q * D;
  const float* dop = static_cast<const float*>(a.dO) + (size_t)bh * n_q * D;
  const int kvh = kv_head_index(bh, a.H, a.group);
  const float* kp = static_cast<const float*>(a.k) + (size_t)kvh * n_k * D;
  const float* vp = static_cast<const float*>(a.v) + (size_t)kvh * n_k * D;

  // Q and dO rows of this lane's query, as B operands (d = 2c + hi).
  float qreg[D / 2], greg[D / 2];
#pragma unroll
  for (int c = 0; c < D / 2; ++c) {
    qreg[c] = (qi < n_q) ? qp[(size_t)qi * D + 2 * c + hi] : 0.f;
    greg[c] = (qi < n_q) ? dop[(size_t)qi * D + 2 * c + hi] : 0.f;
  }
  const float lse2 = (qi < n_q) ? a.lse2[(size_t)bh * n_q + qi] : 0.f;
  const float dlt = (qi < n_q) ? a.delta[(size_t)bh * n_q + qi] : 0.f;

  const Band band = band_of(a, CAUSAL);
  const int q_end = min(n_q, q0 + C::kBlk);
  const int t_lo = band.key_lo(q0) / C::kBS;
  const int t_hi = max(t_lo, (band.key_hi(q_end) + C::kBS - 1) / C::kBS);
  const int wk_lo = band.key_lo(qw), wk_hi = band.key_hi(qw + 32);  // keys this wave sees

  f32x4 kst[C::kLoads], vst[C::kLoads];
  auto gload = [&](int t) {
#pragma unroll
    for (int i = 0; i < C::kLoads; ++i) {
      const int idx = tid + i * C::kThreads;
      const int row = idx / C::kChunks;
      const int ch = idx - row * C::kChunks;
      const int kj = t * C::kBS + row;
      if (kj < n_k) {
        kst[i] = *reinterpret_cast<const f32x4*>(kp + (size_t)kj * D + ch * 4);
        vst[i] = *reinterpret_cast<const f32x4*>(vp + (size_t)kj * D + ch * 4);
      } else {
        kst[i] = f32x4{};
        vst[i] = f32x4{};
      }
    }
  };
  auto swrite = [&](int buf) {
#pragma unroll
    for (int i = 0; i < C::kLoads; ++i) {
      const int idx = tid + i * C::kThreads;
      const int row = idx / C::kChunks;
      const int ch = idx - row * C::kChunks;
      *reinterpret_cast<f32x4*>(&sk[buf][row * C::kStride + ch * 4]) = kst[i];
      *reinterpret_cast<f32x4*>(&sv[buf][row * C::kStride + ch * 4]) = vst[i];
    }
  };

  f32x16 dq[C::kDB];
#pragma unroll
  for (int db = 0; db < C::kDB; ++db) dq[db] = f32x16{};

  if (t_lo < t_hi) {
    gload(t_lo);
    swrite(t_lo & 1);
  }
  __syncthreads();

  for (int t = t_lo; t < t_hi; ++t) {
    const int buf = t & 1;
    if (t + 1 < t_hi) gload(t + 1);
    const int k0 = t * C::kBS;
    if (k0 < wk_hi && k0 + C::kBS > wk_lo) {
      // S^T = K Q^T, dP^T = V dO^T (one query per lane).
      f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int c = 0; c < D / 2; ++c) {
        s = mfma_f32(sk[buf][l32 * C::kStride + 2 * c + hi], qreg[c], s);
        dp = mfma_f32(sv[buf][l32 * C::kStride + 2 * c + hi], greg[c], dp);
      }
      f32x16 ds;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int kj = k0 + 8 * (i >> 2) + 4 * hi + (i & 3);
        float pv = fast_exp2(fmaf(s[i], a.scale_log2, -lse2));
        const bool hide = qi >= n_q || band.hidden(qi, kj);
        pv = hide ? 0.f : pv;
        ds[i] = pv * (dp[i] - dlt);
      }
      // dQ^T[d][q] += K^T dS^T: A = K^T (row d, k = key), B = dS^T.
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int r = 8 * (i >> 2) + 4 * hi + (i & 3);
#pragma unroll
        for (int db = 0; db < C::kDB; ++db)
          dq[db] = mfma_f32(sk[buf][r * C::kStride + 32 * db + l32], ds[i], dq[db]);
      }
      settle_acc(dq);
    }
    if (t + 1 < t_hi) swrite(buf ^ 1);
    __syncthreads();
  }

  if (qi < n_q) {
    float* dqp = static_cast<float*>(a.dq) + ((size_t)bh * n_q + qi) * D;
#pragma unroll
    for (int db = 0; db < C::kDB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        f32x4 r;
#pragma unroll
        for (int e = 0; e < 4; ++e) r[e] = dq[db][4 * g4 + e] * a.scale;
        *reinterpret_cast<f32x4*>(dqp + 32 * db + 8 * g4 + 4 * hi) = r;
      }
  }
}

// ---------------------------------------------------------- launchers

hipError_t launch_raw(const void* kernel, int grid, int block, void** params, hipStream_t s) {
  return hipLaunchKernel(kernel, dim3(grid), dim3(block), params, 0, s);
}

template <int D, bool CAUSAL, int WAVES>
hipError_t dkdv_bf16_w(const BwdArgs& a, hipStream_t s) {
  using C = DkdvCfg<D, WAVES>;
  const int n_ktiles = (a.n_k + C::kBK - 1) / C::kBK;
  BwdArgs args = a;
  int nt = n_ktiles;
  void* params[] = {&args, &nt};
  // runs of one query head need no head loop (and its registers)
  const void* kernel =
      a.group == 1 ? reinterpret_cast<const void*>(bwd_dkdv_bf16_kernel<D, CAUSAL, 0, WAVES>)
      : a.group == a.slices ? reinterpret_cast<const void*>(bwd_dkdv_bf16_kernel<D, CAUSAL, 1, WAVES>)
                            : reinterpret_cast<const void*>(bwd_dkdv_bf16_kernel<D, CAUSAL, 2, WAVES>);
  return launch_raw(kernel, n_ktiles * (a.BH / a.group) * a.slices, C::kThreads, params, s);
}

// 64-key workgroups (two waves) balance a causal pass better — its first key
// tiles see the most queries — visit fewer masked stages under a sliding
// window, and fill a chip that 128-key workgroups would leave half idle;
// on full passes that fill the chip they stream each query stage through
// LDS for half as many keys and lose 2-3 %.  Measured at d=128 (outputs
// bitwise equal): causal B=1 H=32 n=1024 39.1 -> 37.5 us, n=4096 280.2 ->
// 277.6 us, n=16384 4162 -> 4099 us, B=4 n=4096 1244 -> 1190 us; whole
// backward at B=1 H=32 n=4096 with a window of 256, 191.9 -> 179.3 us; full
// B=1 H=4 n=4096 (128 workgroups) 107.7 -> 98.4 us, H=32 512.1 -> 522.6 us.
constexpr long long kDkdvIdleHalfWgs = 128;
template <int D, bool CAUSAL>
hipError_t dkdv_bf16_t(const BwdArgs& a, hipStream_t s) {
  using C4 = DkdvCfg<D, 4>;
  if constexpr (CAUSAL) {
    return dkdv_bf16_w<D, true, 2>(a, s);  // causal passes always take two waves
  } else {
    const long long wgs = (long long)((a.n_k + C4::kBK - 1) / C4::kBK) * (a.BH / a.group) * a.slices;
    const bool narrow = a.window >= 0 || wgs <= kDkdvIdleHalfWgs;
    return narrow ? dkdv_bf16_w<D, false, 2>(a, s) : dkdv_bf16_w<D, false, 4>(a, s);
  }
}

template <int D, bool CAUSAL>
hipError_t dq_bf16_pp(const BwdArgs& a, hipStream_t s) {
  using C = DqCfg<D, 8>;
  const int n_qtiles = (a.n_q + C::kBM - 1) / C::kBM;
  BwdArgs args = a;
  int nt = n_qtiles;
  void* params[] = {&args, &nt};
  return launch_raw(reinterpret_cast<const void*>(bwd_dq_bf16_pp_kernel<D, CAUSAL>), n_qtiles * a.BH,
                    C::kThreads, params, s);
}

template <int D, bool CAUSAL, int WAVES>
hipError_t dq_bf16_w(const BwdArgs& a, hipStream_t s) {
  using C = DqCfg<D, WAVES>;
  const int n_qtiles = (a.n_q + C::kBM - 1) / C::kBM;
  BwdArgs args = a;
  int nt = n_qtiles;
  void* params[] = {&args, &nt};
  return launch_raw(reinterpret_cast<const void*>(bwd_dq_bf16_kernel<D, CAUSAL, WAVES>),
                    n_qtiles * a.BH, C::kThreads, params, s);
}

// With a sliding window a 256-row workgroup visits about window + 256 keys
// while each of its waves needs window + 32: 128-row workgroups waste less.
// A causal pass with fewer than two 256-row workgroups per compute unit of
// the 256-CU chip is set by its longest tile: 128-row workgroups balance
// better there.  Without the mask they pay off when 256-row workgroups
// would leave at least half the compute units idle, and for heads of up to
// 1024 rows (less padding, twice the workgroups: B=16 H=32 d=128 n=512
// 141.7 -> 121.5 us, n=1024 416.5 -> 393.1 us; but B=1 H=32 n=2048 94.1 ->
// 97.1 us and n=4096 338 -> 353 us).
constexpr long long kDqCausalBalanceWgs = 512;
constexpr long long kDqIdleHalfWgs = 128;
constexpr int kDqShortRows = 1024;
template <int D, bool CAUSAL>
hipError_t dq_bf16_t(const BwdArgs& a, hipStream_t s) {
  const long long wide_wgs = (long long)a.BH * ((a.n_q + DqCfg<D, 8>::kBM - 1) / DqCfg<D, 8>::kBM);
  const bool narrow = a.n_q <= kDqShortRows || a.window >= 0 ||
                      (CAUSAL ? wide_wgs < kDqCausalBalanceWgs : wide_wgs <= kDqIdleHalfWgs);
  if (narrow) return dq_bf16_w<D, CAUSAL, 4>(a, s);
  // 256-row workgroups at d = 128 take the ping-pong kernel; at d <= 64 the
  // 8-wave kernel is kept.
  if constexpr (D == 128) return dq_bf16_pp<D, CAUSAL>(a, s);
  else return dq_bf16_w<D, CAUSAL, 8>(a, s);
}

template <int D, bool CAUSAL>
hipError_t dkdv_f32_t(const BwdArgs& a, hipStream_t s) {
  const int n_ktiles = (a.n_k + F32BwdCfg<D>::kBlk - 1) / F32BwdCfg<D>::kBlk;
  BwdArgs args = a;
  int nt = n_ktiles;
  void* params[] = {&args, &nt};
  return launch_raw(reinterpret_cast<const void*>(bwd_dkdv_f32_kernel<D, CAUSAL>),
                    n_ktiles * (a.BH / a.group) * a.slices, F32BwdCfg<D>::kThreads, params, s);
}

template <int D, bool CAUSAL>
hipError_t dq_f32_t(const BwdArgs& a, hipStream_t s) {
  const int n_qtiles = (a.n_q + F32BwdCfg<D>::kBlk - 1) / F32BwdCfg<D>::kBlk;
  BwdArgs args = a;
  int nt = n_qtiles;
  void* params[] = {&args, &nt};
  return launch_raw(reinterpret_cast<const void*>(bwd_dq_f32_kernel<D, CAUSAL>),
                    n_qtiles * a.BH, F32BwdCfg<D>::kThreads, params, s);
}

template <int D, typename TT>
hipError_t preprocess_t(const BwdArgs& a, hipStream_t s) {
  constexpr int kRowsPerBlock = 256 / (D / (16 / sizeof(TT)));
  const long rows = (long)a.BH * a.n_q;
  const long grid = (rows + kRowsPerBlock - 1) / kRowsPerBlock;
  const TT* o = static_cast<const TT*>(a.o);
  const TT* g = static_cast<const TT*>(a.dO);
  const float* lse = a.lse;
  float* delta = a.delta;
  float* lse2 = a.lse2;
  long r = rows;
  void* params[] = {&o, &g, &lse, &delta, &lse2, &r};
  return hipLaunchKernel(reinterpret_cast<const void*>(bwd_preprocess_kernel<D, TT>),
                         dim3((unsigned)grid), dim3(256), params, 0, s);
}

// dK, dV = sum over the runs of the float32 partials, in run order (so the
// result does not depend on scheduling); four values per thread.
template <typename TO>
__global__ __launch_bounds__(256) void bwd_reduce_slices_kernel(BwdArgs a, long long n4) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= n4) return;
  const size_t per = (size_t)n4 * 4;  // floats per run
  f32x4 sk = f32x4{}, sv = f32x4{};
  for (int r = 0; r < a.slices; ++r) {
    sk += *reinterpret_cast<const f32x4*>(a.part_dk + r * per + 4 * i);
    sv += *reinterpret_cast<const f32x4*>(a.part_dv + r * per + 4 * i);
  }
  TO* dk = static_cast<TO*>(a.dk) + 4 * i;
  TO* dv = static_cast<TO*>(a.dv) + 4 * i;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    dk[e] = (TO)sk[e];
    dv[e] = (TO)sv[e];
  }
}

#define FA_DISPATCH_D(fn, d, causal, a, s)                                          \
  switch (d) {                                                                      \
    case 32: return causal ? fn<32, true>(a, s) : fn<32, false>(a, s);              \
    case 64: return causal ? fn<64, true>(a, s) : fn<64, false>(a, s);              \
    case 128: return causal ? fn<128, true>(a, s) : fn<128, false>(a, s);           \
    default: return hipErrorInvalidValue;                                           \
  }

}  // namespace

hipError_t launch_bwd_preprocess(const BwdArgs& a, int d, bool bf16, hipStream_t s) {
  switch (d) {
    case 32: return bf16 ? preprocess_t<32, __bf16>(a, s) : preprocess_t<32, float>(a, s);
    case 64: return bf16 ? preprocess_t<64, __bf16>(a, s) : preprocess_t<64, float>(a, s);
    case 128: return bf16 ? preprocess_t<128, __bf16>(a, s) : preprocess_t<128, float>(a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_bwd_dkdv_bf16(const BwdArgs& a, int d, bool causal, hipStream_t s) {
  FA_DISPATCH_D(dkdv_bf16_t, d, causal, a, s)
}
hipError_t launch_bwd_dq_bf16(const BwdArgs& a, int d, bool causal, hipStream_t s) {
  FA_DISPATCH_D(dq_bf16_t, d, causal, a, s)
}
hipError_t launch_bwd_dkdv_f32(const BwdArgs& a, int d, bool causal, hipStream_t s) {
  FA_DISPATCH_D(dkdv_f32_t, d, causal, a, s)
}
hipError_t launch_bwd_dq_f32(const BwdArgs& a, int d, bool causal, hipStream_t s) {
  FA_DISPATCH_D(dq_f32_t, d, causal, a, s)
}
hipError_t launch_bwd_reduce_slices(const BwdArgs& a, int d, bool bf16, hipStream_t s) {
  BwdArgs args = a;
  long long n4 = (long long)(a.BH / a.group) * a.n_k * d / 4;
  void* params[] = {&args, &n4};
  const int grid = (int)((n4 + 255) / 256);
  return launch_raw(bf16 ? reinterpret_cast<const void*>(bwd_reduce_slices_kernel<__bf16>)
                         : reinterpret_cast<const void*>(bwd_reduce_slices_kernel<float>),
                    grid, 256, params, s);
}

}  // namespace fa
