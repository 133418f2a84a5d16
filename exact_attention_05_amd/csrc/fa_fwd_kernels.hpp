// Forward-pass kernels of exact attention on gfx950: O = softmax(scale Q K^T [+ M]) V
// and the per-row natural-log LSE, one key block at a time with an online
// softmax ("Attention Mechanism: Revolusi Representasi Sequence", section 13,
// running max m and running sum l; the old output is rescaled by
// exp(m_old - m_new) and normalised once at the end).  No score or
// probability block ever leaves the chip.
//
// bf16 kernel (the hot path)
// --------------------------
// A workgroup is 8 waves (two per SIMD; 4 waves for heads of at most 512
// query rows) and owns 32 consecutive query rows of one (batch, head) per
// wave.  Key and value blocks of 64 rows stream
// through double-buffered LDS by direct global -> LDS copies: the copies of
// block t+1 (in the pipelined path: K of block t+2, V of block t+1) are in
// flight while block t is computed, and one barrier per block separates the
// two buffers.  LDS addresses are a per-lane constant XOR the operand's
// chunk offset (TileLane).
//
// The wave computes the transposed score tile S^T = K Q^T on the
// 32x32x16 bf16 matrix cores, with K read from LDS as the A operand and Q
// held in registers as the B operand for the whole pass.  In the S^T
// accumulator layout a lane holds one query column and 16 keys, so a row
// maximum needs only the lane's own values plus one swap with the other half
// of the wave, and the row sum needs no cross-lane step until the end.
// The probabilities are rounded to bf16 and used directly, from registers,
// as the B operand of O^T += V^T P^T; the V^T operand comes from LDS through
// the transposing read ds_read_b64_tr_b16.  Exponentials are base 2 with
// scale * log2(e) folded into one fused multiply-add.
//
// Grid: one workgroup per (query tile, batch*head), remapped so that the
// workgroups of one head run on the same XCD and share its L2; with the
// causal mask the longest query tiles are issued first.  A workgroup visits
// only the key blocks some of its rows see (causal mask, query offset,
// sliding window; see Band).  Blocks that every row sees entirely run
// through an unmasked, software-pipelined path (fixed LDS buffers, two
// blocks per loop turn): the score products of block t+1 are issued in the
// same instruction stream as the exponentials of block t, and those blocks
// skip the block maximum unless the probabilities grow too large.
//
// At d = 128 the 8-wave workgroups run the ping-pong variant of this kernel
// (fwd_bf16_pp_kernel): the two waves of each SIMD alternate between the
// matrix products of a block and the softmax of the next one, half a step
// apart, so that one wave's vector work runs beside the other's products
// (same arithmetic in the same order: bitwise the same results).
//
// fp32 kernel
// -----------
// Same dataflow with float32 operands on the 32x32x2 f32 matrix cores,
// 4 waves x 32 query rows and 32-key blocks; probabilities stay in fp32.
//
// The kernels and their launch rules live in this header so that two
// translation units instantiate them: fa_fwd.hip the plain forward pass and
// fa_fwd_merge.hip the variant whose epilogue merges into a prior result.
#pragma once

#include "fa_internal.hpp"
#include "fa_device.hpp"
#include "fa_tiles.hpp"

#include <cmath>
#include <type_traits>

namespace fa {
namespace fwdk {

template <int D, int WAVES>
struct Bf16FwdCfg {
  static constexpr int kWaves = WAVES;             // 8: two per SIMD; 4 for short rows
  static constexpr int kThreads = kWaves * 64;
  static constexpr int kBM = kWaves * 32;          // query rows per workgroup, 32 per wave
  static constexpr int kBN = 64;                   // keys per block
  static constexpr int kKB = kBN / 32;             // 32-key sub-blocks
  static constexpr int kDC = D / 16;               // 16-wide chunks of the head dim
  static constexpr int kDB = D / 32;               // 32-row blocks of O^T
  using KV = Tile<D, kBN>;                         // one K or V block in LDS
};

// Largest amount by which a row's scores may exceed the reference maximum
// used for its exponentials, in log2 units: probabilities stay below 2^8, so
// the reference (and the rescaling of the output) only changes when a block
// raises the row maximum by more than this.
constexpr float kLazyRescale = 8.0f;
// Largest sum of one lane's probabilities in a block accepted without
// looking at the block maximum.  Below it every probability is at most
// 2^16, so the fp32 output and row sum cannot overflow; a block whose
// maximum stays within kLazyRescale of the reference never exceeds it
// (32 values of at most 2^8), so passing it always moves the reference.
constexpr float kFastSum = 65536.0f;

// Epilogue of one query row, merged into a prior result over other keys
// ("Attention Mechanism", section 13: the running output is rescaled by the
// exponential of the change of reference, here applied to two whole
// results; section 16 "Ring Attention": one step of attention over keys
// held by several workers).  The lane holds the row's unnormalised output
// oacc (column 32 db + 8 g4 + 4 hi + e of element 4 g4 + e of oacc[db]), the
// reference maximum m in log2 units and the row sum lt (both halves added).
// This call's result is O_n = oacc / lt with LSE_n = m + log2 lt (log2
// units); the prior is (O_p, LSE_p).  With M = max(LSE_p, LSE_n),
//   w_p = 2^(LSE_p - M),  w_n = 2^(m - M)  (so w_n oacc = 2^(LSE_n - M) O_n),
//   S = w_p + w_n lt,  O = (w_p O_p + w_n oacc) / S,  LSE = M + log2 S.
// A side without keys (LSE = -inf, or lt = 0) has weight 0 and its O is not
// read; a row without keys on either side gets O = 0 and LSE = -inf.  Each
// lane reads the prior at exactly the places it writes, so o may be o_prior.
template <int KDB>
__device__ __forceinline__ void merge_store(const FwdArgs& a, size_t row, int hi, const f32x16 (&oacc)[KDB],
                                            float m, float lt) {
  constexpr int D = 32 * KDB;
  const float lp = a.lse_prior[row] * kLog2e;
  const float ln = lt > 0.f ? m + fast_log2(lt) : -INFINITY;
  const float mx = fmaxf(lp, ln);
  const bool none = mx == -INFINITY;
  const float ref = none ? 0.f : mx;
  const float wp = lp == -INFINITY ? 0.f : fast_exp2(lp - ref);
  const float wn = lt > 0.f ? fast_exp2(m - ref) : 0.f;
  const float sum = wp + wn * lt;
  const float inv = sum > 0.f ? 1.f / sum : 0.f;
  const float cp = wp * inv, cn = wn * inv;
#pragma unroll
  for (int db = 0; db < KDB; ++db)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const size_t off = row * D + 32 * db + 8 * g4 + 4 * hi;
      f32x4 prev = f32x4{};
      if (wp > 0.f) {
        if (a.prior_f32) {
          prev = *reinterpret_cast<const f32x4*>(static_cast<const float*>(a.o_prior) + off);
        } else {
          const bf16x4 b = *reinterpret_cast<const bf16x4*>(static_cast<const __bf16*>(a.o_prior) + off);
#pragma unroll
          for (int e = 0; e < 4; ++e) prev[e] = (float)b[e];
        }
      }
      f32x4 r;
#pragma unroll
      for (int e = 0; e < 4; ++e) r[e] = cp * prev[e] + cn * oacc[db][4 * g4 + e];
      if (a.out_f32) {
        *reinterpret_cast<f32x4*>(static_cast<float*>(a.o) + off) = r;
      } else {
        bf16x4 b;
#pragma unroll
        for (int e = 0; e < 4; ++e) b[e] = (__bf16)r[e];
        *reinterpret_cast<bf16x4*>(static_cast<__bf16*>(a.o) + off) = b;
      }
    }
  if (hi == 0) a.lse[row] = none ? -INFINITY : (ref + fast_log2(sum)) * kLn2;
}

template <int D, bool CAUSAL, int WAVES, bool MERGE>
__global__ __launch_bounds__(WAVES * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fwd_bf16_kernel(FwdArgs a, int n_qtiles) {
  using C = Bf16FwdCfg<D, WAVES>;
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
  const int q0 = qt * C::kBM;
  const int qw = q0 + wave * 32;
  const int qi = qw + l32;  // this lane's query (column of S^T)
  const int n_q = a.n_q, n_k = a.n_k;
  const float sl2 = a.scale_log2;

  const __bf16* qp = static_cast<const __bf16*>(a.q) + (size_t)bh * n_q * D;
  const int kvh = kv_head_index(bh, a.H, a.group);
  const __bf16* kp = static_cast<const __bf16*>(a.k) + (size_t)kvh * n_k * D;
  const __bf16* vp = static_cast<const __bf16*>(a.v) + (size_t)kvh * n_k * D;

  // Q fragments: B operand of S^T = K Q^T, kept for the whole pass.
  bf16x8 qf[C::kDC];
#pragma unroll
  for (int c = 0; c < C::kDC; ++c) {
    if (qi < n_q)
      qf[c] = *reinterpret_cast<const bf16x8*>(qp + (size_t)qi * D + 16 * c + 8 * hi);
    else
      qf[c] = bf16x8{};
  }

  // Key blocks [t_lo, t_hi) hold keys some row of the workgroup sees;
  // blocks [f_lo, f_hi) inside them need no mask for any row.
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
  TileLane<D, C::kBN> tl;
  tl.init(lane);
  const uint32_t sk_addr = lds_address(&sk[0][0]);
  const uint32_t sv_addr = lds_address(&sv[0][0]);
  auto load_tile = [&](int t, int buf) {
    const int k0 = t * C::kBN;
    dma.load(kp + (size_t)k0 * D, n_k - k0, sk_addr + buf * C::KV::kBytes);
    dma.load(vp + (size_t)k0 * D, n_k - k0, sv_addr + buf * C::KV::kBytes);
  };

  f32x16 oacc[C::kDB];
#pragma unroll
  for (int db = 0; db < C::kDB; ++db) oacc[db] = f32x16{};
  float m = -INFINITY, l = 0.f;

  // One key block: wait for it, start the next block's copy, then
  // S^T = K Q^T, softmax, O^T += V^T P^T.  MASK selects the variant with the
  // causal / key-tail mask; BUF (0, 1, or -1 for "t % 2 at run time") names
  // the LDS buffer, so that with a fixed buffer every LDS address is a
  // per-lane register plus an immediate.
  auto block = [&](auto mask_tag, auto buf_tag, int t) {
    constexpr bool MASK = decltype(mask_tag)::value;
    constexpr int BUFC = decltype(buf_tag)::value;
    const int buf = BUFC >= 0 ? BUFC : (t & 1);
    // Block t is complete in LDS once every wave's own loads have landed;
    // after the barrier nobody reads buffer buf ^ 1 any more.
    wait_lds_dma();
    __syncthreads();
    if (t + 1 < t_hi) load_tile(t + 1, buf ^ 1);
    const char* ks = sk[buf];
    const char* vs = sv[buf];
    const int k0 = t * C::kBN;
    // A masked block whose keys none of this wave's rows sees (the causal
    // diagonal above the wave, a window edge) changes nothing for it.
    if (MASK && (qw >= n_q || band.key_hi(qw + 32) <= k0 || band.key_lo(qw) >= k0 + C::kBN)) return;

    f32x16 s[C::kKB];
    auto scores = [&]() __attribute__((always_inline)) {
      // S^T = K Q^T for kBN keys x 32 queries.
#pragma unroll
      for (int kb = 0; kb < C::kKB; ++kb) s[kb] = f32x16{};
#pragma unroll
      for (int c = 0; c < C::kDC; ++c) {
#pragma unroll
        for (int kb = 0; kb < C::kKB; ++kb) {
          s[kb] = mfma_bf16(tl.read_rows(ks, kb * 32, c), qf[c], s[kb]);
        }
      }
    };
    // Row maximum of the block (raw scores), then the lazy reference update.
    auto raise_ref = [&]() __attribute__((always_inline)) {
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < C::kKB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; i += 2) mx = fmaxf(mx, fmaxf(s[kb][i], s[kb][i + 1]));
      mx = max_halves(mx);
      const float mt = (mx == -INFINITY) ? -INFINITY : mx * sl2;
      if (__builtin_amdgcn_ballot_w64(mt > m + kLazyRescale) != 0) {
        const float m_new = fmaxf(m, mt);
        const float ref = (m_new == -INFINITY) ? 0.f : m_new;
        const float alpha = fast_exp2(m - ref);
        l *= alpha;
#pragma unroll
        for (int db = 0; db < C::kDB; ++db) oacc[db] *= alpha;
        m = m_new;
      }
    };
    // P = exp2(scale_log2 * S - ref), rounded to bf16 as the B operand of
    // the P V product; returns the lane's sum of the unrounded values (the
    // LSE needs them: a sum of bf16-rounded terms is off by up to 2^-9).
    u32x4 pw[C::kKB][2];
    auto probs = [&]() __attribute__((always_inline)) -> float {
      const float ref = (m == -INFINITY) ? 0.f : m;
      float rs0 = 0.f, rs1 = 0.f;
#pragma unroll
      for (int kb = 0; kb < C::kKB; ++kb)
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2) {
#pragma unroll
          for (int e = 0; e < 8; e += 2) {
            float p0 = fast_exp2(fmaf(s[kb][8 * c2 + e], sl2, -ref));
            float p1 = fast_exp2(fmaf(s[kb][8 * c2 + e + 1], sl2, -ref));
            if constexpr (MASK) {
              // exp2(-inf) is 0 already unless the scale is 0.
              if (s[kb][8 * c2 + e] == -INFINITY) p0 = 0.f;
              if (s[kb][8 * c2 + e + 1] == -INFINITY) p1 = 0.f;
            }
            pw[kb][c2][e >> 1] = pack_bf16x2(p0, p1);
            rs0 += p0;
            rs1 += p1;
          }
        }
      return rs0 + rs1;
    };

    scores();
    float rs;
    if constexpr (MASK) {
      // Hidden entries (key past the end, after the query when causal,
      // outside the window) leave the maximum alone and get probability 0.
      const int rel = k0 + 4 * hi - vlo;  // key - vlo of element 0
#pragma unroll
      for (int kb = 0; kb < C::kKB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (!Band::in_range(rel + kb * 32 + 8 * (i >> 2) + (i & 3), 0, vspan)) s[kb][i] = -INFINITY;
      raise_ref();
      rs = probs();
    } else {
      // Without a mask the block maximum is needed only when the reference
      // must move: exponentiate against the current one, and only if some
      // lane's sum passes kFastSum (so might a probability) or a row has no
      // reference yet, recompute the scores, raise the reference and redo.
      rs = probs();
      if (__builtin_amdgcn_ballot_w64(!(rs <= kFastSum) || m == -INFINITY) != 0) {
        scores();
        raise_ref();
        rs = probs();
      }
    }
    l += rs;

    // O^T += V^T P^T, 16 keys per matrix-core step.
#pragma unroll
    for (int kb = 0; kb < C::kKB; ++kb)
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
        for (int db = 0; db < C::kDB; ++db)
          oacc[db] = mfma_bf16(tl.read_cols_tr(vs, kb * 32 + 16 * c2, 32 * db),
                               bf16x8_of(pw[kb][c2]), oacc[db]);
  };

  // Blocks that need no mask for any row of the workgroup go two at a time
  // with fixed buffers (block t in buffer t % 2); the others (window edges,
  // key tail, causal diagonal) masked.
  using F = std::false_type;
  using T = std::true_type;
  using BR = std::integral_constant<int, -1>;
  // When the first two blocks are both unmasked (the pipeline starts at
  // once), both buffers are free and both blocks' copies go out together, so
  // the workgroup waits for memory once before it starts.  (Workgroups that
  // start on masked blocks, window edges, keep one block of look-ahead:
  // measured faster there.)
  const bool early = f_lo == t_lo && t_lo + 1 < f_hi;
  if (t_lo < t_hi) load_tile(t_lo, t_lo & 1);
  if (early) load_tile(t_lo + 1, (t_lo + 1) & 1);
  int t = t_lo;
  for (; t < f_lo; ++t) block(T{}, BR{}, t);

  // Unmasked blocks, software-pipelined inside each wave: iteration t
  // issues the score products of block t+1 while the vector unit
  // exponentiates block t, then adds block t's P V.  K runs one block ahead
  // of V through the same two buffers (K_t, V_t in buffer t % 2): at
  // iteration t's barrier K_{t+1} and V_t have landed, and the copies of
  // K_{t+2} and V_{t+1} start.
  if (f_lo < f_hi) {
    f32x16 sc[C::kKB], sn[C::kKB];
    auto pscores = [&](const char* ks, f32x16 (&s)[C::kKB]) __attribute__((always_inline)) {
#pragma unroll
      for (int kb = 0; kb < C::kKB; ++kb) s[kb] = f32x16{};
#pragma unroll
      for (int c = 0; c < C::kDC; ++c)
#pragma unroll
        for (int kb = 0; kb < C::kKB; ++kb)
          s[kb] = mfma_bf16(tl.read_rows(ks, kb * 32, c), qf[c], s[kb]);
    };
    auto pprobs = [&](u32x4 (&pw)[C::kKB][2]) __attribute__((always_inline)) -> float {
      const float ref = (m == -INFINITY) ? 0.f : m;
      float rs0 = 0.f, rs1 = 0.f;
#pragma unroll
      for (int kb = 0; kb < C::kKB; ++kb)
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
          for (int e = 0; e < 8; e += 2) {
            const float p0 = fast_exp2(fmaf(sc[kb][8 * c2 + e], sl2, -ref));
            const float p1 = fast_exp2(fmaf(sc[kb][8 * c2 + e + 1], sl2, -ref));
            pw[kb][c2][e >> 1] = pack_bf16x2(p0, p1);
            rs0 += p0;
            rs1 += p1;
          }
      return rs0 + rs1;
    };
    auto praise = [&]() __attribute__((always_inline)) {
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < C::kKB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; i += 2) mx = fmaxf(mx, fmaxf(sc[kb][i], sc[kb][i + 1]));
      mx = max_halves(mx);
      const float mt = mx * sl2;
      if (__builtin_amdgcn_ballot_w64(mt > m + kLazyRescale) != 0) {
        const float m_new = fmaxf(m, mt);
        const float alpha = fast_exp2(m - m_new);
        l *= alpha;
#pragma unroll
        for (int db = 0; db < C::kDB; ++db) oacc[db] *= alpha;
        m = m_new;
      }
    };
    auto iter = [&](auto buf_tag, auto next_tag, int t) __attribute__((always_inline)) {
      constexpr int B = decltype(buf_tag)::value;
      constexpr bool NEXT = decltype(next_tag)::value;
      wait_lds_dma();
      __syncthreads();
      if (NEXT && t + 2 < t_hi) {
        const int k2 = (t + 2) * C::kBN;
        dma.load(kp + (size_t)k2 * D, n_k - k2, sk_addr + B * C::KV::kBytes);
      }
      if (t + 1 < t_hi && !(early && t == f_lo)) {
        const int k1 = (t + 1) * C::kBN;
        dma.load(vp + (size_t)k1 * D, n_k - k1, sv_addr + (B ^ 1) * C::KV::kBytes);
      }
      if constexpr (NEXT) pscores(sk[B ^ 1], sn);
      u32x4 pw[C::kKB][2];
      float rs = pprobs(pw);
      if (__builtin_amdgcn_ballot_w64(!(rs <= kFastSum) || m == -INFINITY) != 0) {
        praise();
        rs = pprobs(pw);
      }
      l += rs;
#pragma unroll
      for (int kb = 0; kb < C::kKB; ++kb)
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
          for (int db = 0; db < C::kDB; ++db)
            oacc[db] = mfma_bf16(tl.read_cols_tr(sv[B], kb * 32 + 16 * c2, 32 * db),
                                 bf16x8_of(pw[kb][c2]), oacc[db]);
      if constexpr (NEXT) {
#pragma unroll
        for (int kb = 0; kb < C::kKB; ++kb) sc[kb] = sn[kb];
      }
    };
    // Prologue: K_{f_lo} and V_{f_lo} were started by the previous block (or
    // the first load); start K_{f_lo + 1} (unless started with them) and
    // compute block f_lo's scores.
    if (early) wait_lds_dma_but<2 * decltype(dma)::kMine>();  // block f_lo + 1 may still be in flight
    else wait_lds_dma();
    __syncthreads();
    if (f_lo + 1 < t_hi && !early) {
      const int k1 = (f_lo + 1) * C::kBN;
      dma.load(kp + (size_t)k1 * D, n_k - k1, sk_addr + ((f_lo + 1) & 1) * C::KV::kBytes);
    }
    pscores(sk[f_lo & 1], sc);
    using B0 = std::integral_constant<int, 0>;
    using B1 = std::integral_constant<int, 1>;
    if (t < f_hi - 1 && (t & 1)) {
      iter(B1{}, T{}, t);
      ++t;
    }
    for (; t + 1 < f_hi - 1; t += 2) {
      iter(B0{}, T{}, t);
      iter(B1{}, T{}, t + 1);
    }
    if (t < f_hi - 1) {
      iter(B0{}, T{}, t);
      ++t;
    }
    if (t & 1) iter(B1{}, F{}, t); else iter(B0{}, F{}, t);
    ++t;
  }
  for (; t < t_hi; ++t) block(T{}, BR{}, t);

  // Epilogue: normalise, store O (bf16) and LSE (natural log).  A row that
  // sees no key at all gets O = 0 and LSE = -inf.  MERGE: combined with the
  // prior result of the row instead.
  const float lt = sum_halves(l);
  if constexpr (MERGE) {
    if (qi < n_q) merge_store(a, (size_t)bh * n_q + qi, hi, oacc, m, lt);
    return;
  }
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  if (qi < n_q) {
    __bf16* op = static_cast<__bf16*>(a.o) + ((size_t)bh * n_q + qi) * D;
#pragma unroll
    for (int db = 0; db < C::kDB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        bf16x4 r;
#pragma unroll
        for (int e = 0; e < 4; ++e) r[e] = (__bf16)(oacc[db][4 * g4 + e] * inv);
        *reinterpret_cast<bf16x4*>(op + 32 * db + 8 * g4 + 4 * hi) = r;
      }
    if (hi == 0) a.lse[(size_t)bh * n_q + qi] = (m + fast_log2(lt)) * kLn2;
  }
}

// Ping-pong variant of the 8-wave kernel for the blocks every row sees.  The
// two waves that share a SIMD (wave w and wave w + 4) work one half-step
// apart: while one issues the matrix products of a block (the P V product
// of block t - 1 and the scores of block t, 32 products), the other runs the
// softmax of its scores (about 110 vector instructions), so the matrix cores
// and the vector unit of each SIMD are busy at the same time; a workgroup
// barrier separates the half-steps.  A wave's own work alternates
//   phase A(i): O^T += V_{t-1}^T P_{t-1}^T (if i > 0) and S_t = K_t Q^T
//               (t = f_lo + i, if i < n)
//   phase B(i): P_t = exp2(scale_log2 S_t - ref), row sums, bf16 P_t
// for i = 0 .. n (n unmasked blocks).  Both groups run the same code, step
// i = [barrier, A(i), barrier, B(i)]; waves 4-7 pass one extra barrier
// first (barriers rendezvous by count), which puts them one half-step
// behind, and waves 0-3 one extra at the end.  K and V blocks use two LDS
// buffers each (block f_lo + i in buffer i mod 2, a compile-time index in
// the loop, unrolled by two).  Waves 4-7 issue the copies, in their vector
// phase: issuing a direct copy costs its wave about 50 cycles, which in a
// product phase delays all 32 products (c3: 239 -> 226 us against copies
// issued by waves 0-3 at the start of their product phase).  Blocks that
// need a mask (before f_lo: window edges; from f_hi on: causal diagonal, key
// tail) take the plain path.
template <int D, bool CAUSAL, bool MERGE>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fwd_bf16_pp_kernel(FwdArgs a, int n_qtiles) {
  using C = Bf16FwdCfg<D, 8>;
  using F = std::false_type;
  using T = std::true_type;
  __shared__ __attribute__((aligned(1024))) char sk[2][C::KV::kBytes];
  __shared__ __attribute__((aligned(1024))) char sv[2][C::KV::kBytes];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;  // 0: waves 0-3, 1: waves 4-7, one half-step behind
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  const int n_q = a.n_q, n_k = a.n_k;
  const float sl2 = a.scale_log2;
  const Band band = band_of(a, CAUSAL);

  TileDma<D, C::kBN, C::kWaves> dma;
  dma.init(wave, lane);
  TileDma<D, C::kBN, 4> dma4;
  dma4.init(wave & 3, lane);
  TileLane<D, C::kBN> tl;
  tl.init(lane);
  const uint32_t sk_addr = lds_address(&sk[0][0]);
  const uint32_t sv_addr = lds_address(&sv[0][0]);

  // Tile w of the launch (a query tile of one head) and its key blocks:
  // [t_lo, t_hi) visited, [f_lo, f_hi) unmasked (the ping-pong).  Without
  // the causal mask a workgroup may take several tiles (w, w + gridDim.x,
  // ...: a grid of one workgroup per compute unit), the next tile's Q and
  // first K/V block loading while the current tile's output is written.
  struct TileW {
    int bh, q0, t_lo, t_hi, f_lo, f_hi;
    const __bf16 *qp, *kp, *vp;
  };
  auto tile_of = [&](int w) {
    TileW tw;
    int qt;
    if (CAUSAL) {
      costliest_first(w, n_qtiles * a.BH, n_qtiles, tw.bh, qt);
      qt = n_qtiles - 1 - qt;
    } else {
      const int work = xcd_remap(w, n_qtiles * a.BH);
      tw.bh = work / n_qtiles;
      qt = work - tw.bh * n_qtiles;
    }
    tw.q0 = qt * C::kBM;
    const int q_end = min(n_q, tw.q0 + C::kBM);
    tw.t_lo = band.key_lo(tw.q0) / C::kBN;
    tw.t_hi = max(tw.t_lo, (band.key_hi(q_end) + C::kBN - 1) / C::kBN);
    tw.f_lo = min(tw.t_hi, max(tw.t_lo, (band.key_full_lo(q_end) + C::kBN - 1) / C::kBN));
    tw.f_hi = max(tw.f_lo, min(tw.t_hi, band.key_full_hi(tw.q0) / C::kBN));
    tw.qp = static_cast<const __bf16*>(a.q) + (size_t)tw.bh * n_q * D;
    const int kvh = kv_head_index(tw.bh, a.H, a.group);
    tw.kp = static_cast<const __bf16*>(a.k) + (size_t)kvh * n_k * D;
    tw.vp = static_cast<const __bf16*>(a.v) + (size_t)kvh * n_k * D;
    return tw;
  };
  // Block t of tile tw lives in buffer (t - tw.f_lo) mod 2.
  auto load_tile_of = [&](const TileW& tw, int t) {
    const int k0 = t * C::kBN;
    const int buf = (t - tw.f_lo) & 1;
    dma.load(tw.kp + (size_t)k0 * D, n_k - k0, sk_addr + buf * C::KV::kBytes);
    dma.load(tw.vp + (size_t)k0 * D, n_k - k0, sv_addr + buf * C::KV::kBytes);
  };
  bf16x8 qf[C::kDC];
  auto load_q = [&](const TileW& tw) {
    const int row = tw.q0 + wave * 32 + l32;
#pragma unroll
    for (int c = 0; c < C::kDC; ++c) {
      if (row < n_q)
        qf[c] = *reinterpret_cast<const bf16x8*>(tw.qp + (size_t)row * D + 16 * c + 8 * hi);
      else
        qf[c] = bf16x8{};
    }
  };

  const int total = n_qtiles * a.BH;
  TileW tw = tile_of(blockIdx.x);
  load_q(tw);
  if (tw.t_lo < tw.t_hi) load_tile_of(tw, tw.t_lo);
  for (int w = blockIdx.x; w < total; w += gridDim.x) {
  const int bh = tw.bh, q0 = tw.q0;
  const int t_lo = tw.t_lo, t_hi = tw.t_hi, f_lo = tw.f_lo, f_hi = tw.f_hi;
  const __bf16* const kp = tw.kp;
  const __bf16* const vp = tw.vp;
  const int qw = q0 + wave * 32;
  const int qi = qw + l32;
  const int n = f_hi - f_lo;  // blocks of the ping-pong
  int vlo, vspan;
  band.key_range(qi, vlo, vspan);
  auto bufof = [&](int t) { return (t - f_lo) & 1; };
  auto load_tile = [&](int t) { load_tile_of(tw, t); };

  f32x16 oacc[C::kDB];
#pragma unroll
  for (int db = 0; db < C::kDB; ++db) oacc[db] = f32x16{};
  float m = -INFINITY, l = 0.f;

  // A masked block (plain path, run-time buffer): wait for block t, barrier,
  // start the copy of block t + 1 (next_ok: it is not copied yet), then
  // S^T = K Q^T, masked online softmax with the block maximum, O^T += V^T P^T.
  auto masked_block = [&](int t, bool next_ok) {
    wait_lds_dma();
    __syncthreads();
    if (next_ok && t + 1 < t_hi) load_tile(t + 1);
    const int buf = bufof(t);
    const char* ks = sk[buf];
    const char* vs = sv[buf];
    const int k0 = t * C::kBN;
    if (qw >= n_q || band.key_hi(qw + 32) <= k0 || band.key_lo(qw) >= k0 + C::kBN) return;
    f32x16 s[C::kKB];
#pragma unroll
    for (int kb = 0; kb < C::kKB; ++kb) s[kb] = f32x16{};
#pragma unroll
    for (int c = 0; c < C::kDC; ++c)
#pragma unroll
      for (int kb = 0; kb < C::kKB; ++kb) s[kb] = mfma_bf16(tl.read_rows(ks, kb * 32, c), qf[c], s[kb]);
    const int rel = k0 + 4 * hi - vlo;
#pragma unroll
    for (int kb = 0; kb < C::kKB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (!Band::in_range(rel + kb * 32 + 8 * (i >> 2) + (i & 3), 0, vspan)) s[kb][i] = -INFINITY;
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < C::kKB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; i += 2) mx = fmaxf(mx, fmaxf(s[kb][i], s[kb][i + 1]));
    mx = max_halves(mx);
    const float mt = (mx == -INFINITY) ? -INFINITY : mx * sl2;
    if (__builtin_amdgcn_ballot_w64(mt > m + kLazyRescale) != 0) {
      const float m_new = fmaxf(m, mt);
      const float ref = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = fast_exp2(m - ref);
      l *= alpha;
#pragma unroll
      for (int db = 0; db < C::kDB; ++db) oacc[db] *= alpha;
      m = m_new;
    }
    const float ref = (m == -INFINITY) ? 0.f : m;
    u32x4 pw[C::kKB][2];
    float rs0 = 0.f, rs1 = 0.f;
#pragma unroll
    for (int kb = 0; kb < C::kKB; ++kb)
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          float p0 = fast_exp2(fmaf(s[kb][8 * c2 + e], sl2, -ref));
          float p1 = fast_exp2(fmaf(s[kb][8 * c2 + e + 1], sl2, -ref));
          if (s[kb][8 * c2 + e] == -INFINITY) p0 = 0.f;
          if (s[kb][8 * c2 + e + 1] == -INFINITY) p1 = 0.f;
          pw[kb][c2][e >> 1] = pack_bf16x2(p0, p1);
          rs0 += p0;
          rs1 += p1;
        }
    l += rs0 + rs1;
#pragma unroll
    for (int kb = 0; kb < C::kKB; ++kb)
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
        for (int db = 0; db < C::kDB; ++db)
          oacc[db] = mfma_bf16(tl.read_cols_tr(vs, kb * 32 + 16 * c2, 32 * db), bf16x8_of(pw[kb][c2]), oacc[db]);
  };

  int t = t_lo;  // block t_lo's copy was started with the tile's Q load
  for (; t < f_lo; ++t) masked_block(t, true);  // up to block f_lo's copy

  if (n > 0) {
    f32x16 sc[C::kKB];          // scores of the wave's current block
    u32x4 pw[C::kKB][2];        // its probabilities as bf16 pairs
    // Phase A as one stream of product steps: steps 0-15 the P V products
    // (two transposing reads each), steps 16-31 the score products (one K
    // row read each); P V first, so that the previous block's bf16 P is dead
    // before the new scores are written.  Operand reads run kAhead steps
    // ahead of their products through a ring, hand-scheduled (the scheduler
    // would otherwise issue all 48 reads first and run out of registers).
    constexpr int kHalf = C::kDC * C::kKB;
    constexpr int kAhead = 6;
    auto phase_a = [&](auto kb_tag, auto vb_tag, auto pv_tag, auto s_tag) __attribute__((always_inline)) {
      constexpr int KB = decltype(kb_tag)::value, VB = decltype(vb_tag)::value;
      constexpr bool PV = decltype(pv_tag)::value, SC = decltype(s_tag)::value;
      constexpr int J0 = PV ? 0 : kHalf, J1 = SC ? 2 * kHalf : kHalf;
      auto read = [&](auto j_tag) __attribute__((always_inline)) -> bf16x8 {
        constexpr int J = decltype(j_tag)::value;
        if constexpr (J >= kHalf) {
          constexpr int c = (J - kHalf) / C::kKB, kb = (J - kHalf) % C::kKB;
          return tl.read_rows(sk[KB], kb * 32, c);
        } else {
          constexpr int kb = J / (2 * C::kDB), c2 = (J / C::kDB) % 2, db = J % C::kDB;
          return tl.read_cols_tr(sv[VB], kb * 32 + 16 * c2, 32 * db);
        }
      };
      auto product = [&](auto j_tag, const bf16x8& op) __attribute__((always_inline)) {
        constexpr int J = decltype(j_tag)::value;
        if constexpr (J >= kHalf) {
          constexpr int c = (J - kHalf) / C::kKB, kb = (J - kHalf) % C::kKB;
          sc[kb] = mfma_bf16(op, qf[c], c == 0 ? f32x16{} : sc[kb]);
        } else {
          constexpr int kb = J / (2 * C::kDB), c2 = (J / C::kDB) % 2, db = J % C::kDB;
          oacc[db] = mfma_bf16(op, bf16x8_of(pw[kb][c2]), oacc[db]);
        }
      };
      bf16x8 ring[kAhead];
      phase_barrier();
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
    };
    auto probs = [&]() __attribute__((always_inline)) -> float {
      const float ref = (m == -INFINITY) ? 0.f : m;
      float rs0 = 0.f, rs1 = 0.f;
#pragma unroll
      for (int kb = 0; kb < C::kKB; ++kb)
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
          for (int e = 0; e < 8; e += 2) {
            const float p0 = fast_exp2(fmaf(sc[kb][8 * c2 + e], sl2, -ref));
            const float p1 = fast_exp2(fmaf(sc[kb][8 * c2 + e + 1], sl2, -ref));
            pw[kb][c2][e >> 1] = pack_bf16x2(p0, p1);
            rs0 += p0;
            rs1 += p1;
          }
      return rs0 + rs1;
    };
    // Phase B: the softmax of the wave's scores against the running
    // reference; only when a probability might pass 2^16 or a row has no
    // reference yet is the block maximum taken (lazy rescale, as above).
    auto phase_b = [&]() __attribute__((always_inline)) {
      float rs = probs();
      if (__builtin_amdgcn_ballot_w64(!(rs <= kFastSum) || m == -INFINITY) != 0) {
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < C::kKB; ++kb)
#pragma unroll
          for (int e = 0; e < 16; e += 2) mx = fmaxf(mx, fmaxf(sc[kb][e], sc[kb][e + 1]));
        mx = max_halves(mx);
        const float mt = mx * sl2;
        if (__builtin_amdgcn_ballot_w64(mt > m + kLazyRescale) != 0) {
          const float m_new = fmaxf(m, mt);
          const float alpha = fast_exp2(m - m_new);
          l *= alpha;
#pragma unroll
          for (int db = 0; db < C::kDB; ++db) oacc[db] *= alpha;
          m = m_new;
        }
        rs = probs();
      }
      l += rs;
    };
    // Copies by waves 4-7 in their phase B (vector work, while waves 0-3
    // run products): in B(i) (which starts at the barrier that ends every
    // read of blocks f_lo + i and f_lo + i - 1) K of block f_lo + i + 2 (up
    // to f_hi) and V of f_lo + i + 1 (up to f_hi), both first read two
    // half-steps later; waves 4-7 wait for them before the barrier in the
    // middle of their next step, which precedes the first read.
    auto step = [&](auto p_tag, auto pv_tag, auto s_tag, int i) __attribute__((always_inline)) {
      constexpr int P = decltype(p_tag)::value;  // i mod 2
      phase_a(std::integral_constant<int, P>{}, std::integral_constant<int, P ^ 1>{}, pv_tag, s_tag);
      if (grp == 1) wait_lds_dma();
      phase_barrier();
      if (grp == 1) {
        const int tk = f_lo + i + 2, tv = f_lo + i + 1;
        if (tk <= f_hi && tk < t_hi) {
          const int k0 = tk * C::kBN;
          dma4.load(kp + (size_t)k0 * D, n_k - k0, sk_addr + P * C::KV::kBytes);
        }
        if (tv <= f_hi && tv < t_hi) {
          const int k0 = tv * C::kBN;
          dma4.load(vp + (size_t)k0 * D, n_k - k0, sv_addr + (P ^ 1) * C::KV::kBytes);
        }
      }
      if constexpr (decltype(s_tag)::value) phase_b();
    };
    using Z = std::integral_constant<int, 0>;
    using O = std::integral_constant<int, 1>;
    // Block f_lo (K and V) was started by the previous block or the first
    // copy; every wave waits for its part before the ping-pong starts, and
    // waves 4-7 start K of block f_lo + 1 (read first at step 1).
    wait_lds_dma();
    if (grp == 1) {
      if (f_lo + 1 <= f_hi && f_lo + 1 < t_hi) {
        const int k0 = (f_lo + 1) * C::kBN;
        dma4.load(kp + (size_t)k0 * D, n_k - k0, sk_addr + C::KV::kBytes);
      }
      phase_barrier();
    }
    step(Z{}, F{}, T{}, 0);  // scores of block f_lo only
    int i = 1;
    for (; i + 1 < n; i += 2) {
      step(O{}, T{}, T{}, i);
      step(Z{}, T{}, T{}, i + 1);
    }
    if (i < n) {
      step(O{}, T{}, T{}, i);
      ++i;
    }
    // i == n: the last P V product only
    if (n & 1) step(O{}, T{}, F{}, n);
    else step(Z{}, T{}, F{}, n);
    if (grp == 0) phase_barrier();
    t = f_hi;
  }
  // After the ping-pong: block f_hi's K was started at step n - 1 and its V
  // at step n (nothing beyond); the masked blocks continue with one block of
  // look-ahead.
  for (; t < t_hi; ++t) masked_block(t, true);

  // The next tile's Q and first K/V block, once every wave is done with
  // this tile's (Q is in registers: this wave's last product has issued;
  // the barrier covers the LDS buffers).
  if (w + (int)gridDim.x < total) {
    __syncthreads();
    tw = tile_of(w + gridDim.x);
    load_q(tw);
    if (tw.t_lo < tw.t_hi) load_tile_of(tw, tw.t_lo);
  }

  const float lt = sum_halves(l);
  if constexpr (MERGE) {
    if (qi < n_q) merge_store(a, (size_t)bh * n_q + qi, hi, oacc, m, lt);
    continue;
  }
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  if (qi < n_q) {
    __bf16* op = static_cast<__bf16*>(a.o) + ((size_t)bh * n_q + qi) * D;
#pragma unroll
    for (int db = 0; db < C::kDB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        bf16x4 r;
#pragma unroll
        for (int e = 0; e < 4; ++e) r[e] = (__bf16)(oacc[db][4 * g4 + e] * inv);
        *reinterpret_cast<bf16x4*>(op + 32 * db + 8 * g4 + 4 * hi) = r;
      }
    if (hi == 0) a.lse[(size_t)bh * n_q + qi] = (m + fast_log2(lt)) * kLn2;
  }
  }
}

// ------------------------------------------------------------------ fp32

// Online-softmax update of one 32-query block held as S^T fragments
// s[kb] (kb = 32-key sub-block), updating the reference maximum every block.
// Turns s into unnormalised probabilities exp2(scale_log2 * s - m_new),
// updates the running max m and the lane's partial running sum l, and
// returns the rescale factor for the old output.  With MASK, hidden entries
// (hide bit set) are left out of the max and get probability 0 (this also
// covers scale == 0, where -inf * 0 would be NaN).
template <int KB, bool MASK>
__device__ __forceinline__ float softmax_block(f32x16 (&s)[KB], float& m, float& l,
                                               float scale_log2, const uint32_t* hide) {
  float mx = -INFINITY;
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (MASK && ((hide[kb] >> i) & 1u)) continue;
      mx = fmaxf(mx, s[kb][i]);
    }
  mx = max_halves(mx);
  const float mt = (mx == -INFINITY) ? -INFINITY : mx * scale_log2;
  const float m_new = fmaxf(m, mt);
  const float ref = (m_new == -INFINITY) ? 0.f : m_new;
  const float alpha = fast_exp2(m - ref);
  float rs = 0.f;
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float p = fast_exp2(fmaf(s[kb][i], scale_log2, -ref));
      if (MASK && ((hide[kb] >> i) & 1u)) p = 0.f;
      s[kb][i] = p;
      rs += p;
    }
  l = alpha * l + rs;
  m = m_new;
  return alpha;
}

template <int D>
struct F32FwdCfg {
  static constexpr int kWaves = 4;
  static constexpr int kThreads = kWaves * 64;
  static constexpr int kBM = kWaves * 32;          // one 32-row block per wave
  static constexpr int kBN = 32;
  static constexpr int kDB = D / 32;
  static constexpr int kKStride = D + 2;           // floats
  static constexpr int kVStride = D + 8;
  static constexpr int kChunks = D / 4;            // 16-byte chunks per row
  static constexpr int kLoads = kBN * kChunks / kThreads;
  static_assert(kLoads * kThreads == kBN * kChunks, "tile load split");
};

template <int D, bool CAUSAL, bool MERGE>
__global__ __launch_bounds__(256) void fwd_f32_kernel(FwdArgs a, int n_qtiles) {
  using C = F32FwdCfg<D>;
  __shared__ __attribute__((aligned(16))) float sk[2][C::kBN * C::kKStride];
  __shared__ __attribute__((aligned(16))) float sv[2][C::kBN * C::kVStride];

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
  const int q0 = qt * C::kBM;
  const int qw = q0 + wave * 32;
  const int n_q = a.n_q, n_k = a.n_k;

  const float* qp = static_cast<const float*>(a.q) + (size_t)bh * n_q * D;
  const int kvh = kv_head_index(bh, a.H, a.group);
  const float* kp = static_cast<const float*>(a.k) + (size_t)kvh * n_k * D;
  const float* vp = static_cast<const float*>(a.v) + (size_t)kvh * n_k * D;

  const int qi = qw + l32;
  float qf[D / 2];
#pragma unroll
  for (int c = 0; c < D / 2; ++c) qf[c] = (qi < n_q) ? qp[(size_t)qi * D + 2 * c + hi] : 0.f;

  const Band band = band_of(a, CAUSAL);
  const int q_end = min(n_q, q0 + C::kBM);
  const int t_lo = band.key_lo(q0) / C::kBN;
  const int t_hi = max(t_lo, (band.key_hi(q_end) + C::kBN - 1) / C::kBN);
  int vlo, vspan;  // keys this lane's query sees: [vlo, vlo + vspan]
  band.key_range(qi, vlo, vspan);
  // Keys every row of this wave sees.
  const int wfull_lo = band.key_full_lo(qw + 32), wfull_hi = band.key_full_hi(qw);

  // The 16-byte row chunks are stored unaligned into the padded K rows
  // (pitch D + 2), so K goes through LDS as float2 pairs.
  f32x4 kst[C::kLoads], vst[C::kLoads];
  auto gload = [&](int t) {
#pragma unroll
    for (int i = 0; i < C::kLoads; ++i) {
      const int idx = tid + i * C::kThreads;
      const int row = idx / C::kChunks;
      const int ch = idx - row * C::kChunks;
      const int key = t * C::kBN + row;
      if (key < n_k) {
        kst[i] = *reinterpret_cast<const f32x4*>(kp + (size_t)key * D + ch * 4);
        vst[i] = *reinterpret_cast<const f32x4*>(vp + (size_t)key * D + ch * 4);
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
      float* kd = &sk[buf][row * C::kKStride + ch * 4];
      kd[0] = kst[i][0]; kd[1] = kst[i][1]; kd[2] = kst[i][2]; kd[3] = kst[i][3];
      *reinterpret_cast<f32x4*>(&sv[buf][row * C::kVStride + ch * 4]) = vst[i];
    }
  };

  f32x16 oacc[C::kDB];
#pragma unroll
  for (int db = 0; db < C::kDB; ++db) oacc[db] = f32x16{};
  float m = -INFINITY, l = 0.f;

  if (t_lo < t_hi) {
    gload(t_lo);
    swrite(t_lo & 1);
  }
  __syncthreads();

  for (int t = t_lo; t < t_hi; ++t) {
    const int buf = t & 1;
    if (t + 1 < t_hi) gload(t + 1);
    const int k0 = t * C::kBN;

    f32x16 s[1];
    s[0] = f32x16{};
#pragma unroll
    for (int c = 0; c < D / 2; ++c)
      s[0] = mfma_f32(sk[buf][l32 * C::kKStride + 2 * c + hi], qf[c], s[0]);

    const bool need_mask = k0 < wfull_lo || k0 + C::kBN > wfull_hi;
    float alpha;
    if (need_mask) {
      uint32_t bits = 0;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const bool h = !Band::in_range(k0 + 4 * hi - vlo + 8 * (i >> 2) + (i & 3), 0, vspan);
        bits |= (h ? 1u : 0u) << i;
      }
      alpha = softmax_block<1, true>(s, m, l, a.scale_log2, &bits);
    } else {
      alpha = softmax_block<1, false>(s, m, l, a.scale_log2, nullptr);
    }
#pragma unroll
    for (int db = 0; db < C::kDB; ++db) oacc[db] *= alpha;

    // O^T += V^T P^T: accumulator element i of this lane is the probability
    // of key 8*(i/4) + 4*hi + (i%4), which is exactly the B operand slot.
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int key = 8 * (i >> 2) + 4 * hi + (i & 3);
#pragma unroll
      for (int db = 0; db < C::kDB; ++db)
        oacc[db] = mfma_f32(sv[buf][key * C::kVStride + 32 * db + l32], s[0][i], oacc[db]);
    }
    settle_acc(oacc);

    if (t + 1 < t_hi) swrite(buf ^ 1);
    __syncthreads();
  }

  const float lt = sum_halves(l);
  if constexpr (MERGE) {
    if (qi < n_q) merge_store(a, (size_t)bh * n_q + qi, hi, oacc, m, lt);
    return;
  }
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  if (qi < n_q) {
    float* op = static_cast<float*>(a.o) + ((size_t)bh * n_q + qi) * D;
#pragma unroll
    for (int db = 0; db < C::kDB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        f32x4 r;
#pragma unroll
        for (int e = 0; e < 4; ++e) r[e] = oacc[db][4 * g4 + e] * inv;
        *reinterpret_cast<f32x4*>(op + 32 * db + 8 * g4 + 4 * hi) = r;
      }
    if (hi == 0) a.lse[(size_t)bh * n_q + qi] = (m + fast_log2(lt)) * kLn2;
  }
}

// Key-split float32 forward, for shapes whose query rows are too few to fill
// the GPU with 128-row workgroups but which have many keys (one head of a few
// thousand rows).  The four waves of a workgroup share one 32-row block and
// take its 32-key steps w, w + 4, w + 8, ...: each through its own LDS tile
// and with no workgroup barrier in the loop (the next step's rows load into
// registers while the current one is used), with the products and the
// online softmax of fwd_f32_kernel.  At the end the waves' partial results
// over their key subsets merge through LDS exactly as the online softmax
// merges blocks ("Attention Mechanism: Revolusi Representasi Sequence",
// section 13): weights exp2(m_w - max_w m_w) on each wave's O and l.
template <int D>
struct F32SplitCfg {
  static constexpr int kWaves = 4;
  static constexpr int kThreads = kWaves * 64;
  static constexpr int kBN = 32;                       // keys per wave step
  static constexpr int kDB = D / 32;
  static constexpr int kKStride = D + 2;               // floats (as fwd_f32_kernel)
  static constexpr int kVStride = D + 8;
  static constexpr int kChunks = D / 4;                // 16-byte chunks per row
  static constexpr int kLoads = kBN * kChunks / 64;    // per lane, one wave loading a step
  static constexpr int kTile = kBN * (kKStride + kVStride);  // floats per wave
  static constexpr int kOPitch = D + 1;                // merge rows (conflict-free columns)
  static constexpr int kMerge = kWaves * 32 * kOPitch + 2 * kWaves * 32;
  static constexpr int kSmem = kWaves * kTile > kMerge ? kWaves * kTile : kMerge;
  static constexpr int kColsPerThread = D * 32 / kThreads;  // merge: 8 threads per row
  static_assert(kLoads * 64 == kBN * kChunks, "step load split");
  static_assert(kColsPerThread * kThreads == D * 32, "merge split");
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) void fwd_f32_split_kernel(FwdArgs a, int n_rb) {
  using C = F32SplitCfg<D>;
  __shared__ __attribute__((aligned(16))) float smem[C::kSmem];

  const int work = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = work / n_rb;
  const int q0 = (work - bh * n_rb) * 32;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  const int n_q = a.n_q, n_k = a.n_k;
  float* const sk = smem + wave * C::kTile;
  float* const sv = sk + C::kBN * C::kKStride;

  const float* qp = static_cast<const float*>(a.q) + (size_t)bh * n_q * D;
  const int kvh = kv_head_index(bh, a.H, a.group);
  const float* kp = static_cast<const float*>(a.k) + (size_t)kvh * n_k * D;
  const float* vp = static_cast<const float*>(a.v) + (size_t)kvh * n_k * D;

  const int qi = q0 + l32;
  float qf[D / 2];
#pragma unroll
  for (int c = 0; c < D / 2; ++c) qf[c] = (qi < n_q) ? qp[(size_t)qi * D + 2 * c + hi] : 0.f;

  const Band band = band_of(a, CAUSAL);
  const int q_end = min(n_q, q0 + 32);
  const int t_lo = band.key_lo(q0) / C::kBN;
  const int t_hi = max(t_lo, (band.key_hi(q_end) + C::kBN - 1) / C::kBN);
  int vlo, vspan;  // keys this lane's query sees: [vlo, vlo + vspan]
  band.key_range(qi, vlo, vspan);
  const int wfull_lo = band.key_full_lo(q0 + 32), wfull_hi = band.key_full_hi(q0);

  f32x4 kst[C::kLoads], vst[C::kLoads];
  auto gload = [&](int t) {
#pragma unroll
    for (int i = 0; i < C::kLoads; ++i) {
      const int idx = lane + i * 64;
      const int row = idx / C::kChunks;
      const int ch = idx - row * C::kChunks;
      const int key = t * C::kBN + row;
      if (key < n_k) {
        kst[i] = *reinterpret_cast<const f32x4*>(kp + (size_t)key * D + ch * 4);
        vst[i] = *reinterpret_cast<const f32x4*>(vp + (size_t)key * D + ch * 4);
      } else {
        kst[i] = f32x4{};
        vst[i] = f32x4{};
      }
    }
  };
  // The wave's own tile: its LDS accesses run in program order, so the
  // previous step's reads are done before these writes land.
  auto swrite = [&]() {
#pragma unroll
    for (int i = 0; i < C::kLoads; ++i) {
      const int idx = lane + i * 64;
      const int row = idx / C::kChunks;
      const int ch = idx - row * C::kChunks;
      float* kd = &sk[row * C::kKStride + ch * 4];
      kd[0] = kst[i][0]; kd[1] = kst[i][1]; kd[2] = kst[i][2]; kd[3] = kst[i][3];
      *reinterpret_cast<f32x4*>(&sv[row * C::kVStride + ch * 4]) = vst[i];
    }
  };

  f32x16 oacc[C::kDB];
#pragma unroll
  for (int db = 0; db < C::kDB; ++db) oacc[db] = f32x16{};
  float m = -INFINITY, l = 0.f;

  int t = t_lo + wave;
  if (t < t_hi) gload(t);
  for (; t < t_hi; t += C::kWaves) {
    swrite();
    if (t + C::kWaves < t_hi) gload(t + C::kWaves);
    const int k0 = t * C::kBN;

    f32x16 s[1];
    s[0] = f32x16{};
#pragma unroll
    for (int c = 0; c < D / 2; ++c) s[0] = mfma_f32(sk[l32 * C::kKStride + 2 * c + hi], qf[c], s[0]);

    const bool need_mask = k0 < wfull_lo || k0 + C::kBN > wfull_hi;
    float alpha;
    if (need_mask) {
      uint32_t bits = 0;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const bool h = !Band::in_range(k0 + 4 * hi - vlo + 8 * (i >> 2) + (i & 3), 0, vspan);
        bits |= (h ? 1u : 0u) << i;
      }
      alpha = softmax_block<1, true>(s, m, l, a.scale_log2, &bits);
    } else {
      alpha = softmax_block<1, false>(s, m, l, a.scale_log2, nullptr);
    }
#pragma unroll
    for (int db = 0; db < C::kDB; ++db) oacc[db] *= alpha;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int key = 8 * (i >> 2) + 4 * hi + (i & 3);
#pragma unroll
      for (int db = 0; db < C::kDB; ++db)
        oacc[db] = mfma_f32(sv[key * C::kVStride + 32 * db + l32], s[0][i], oacc[db]);
    }
    settle_acc(oacc);
  }

  // Merge: each wave's O (rows = queries), m and l; then 8 threads per row
  // combine the waves.  A wave with no step has m = -inf, l = 0, O = 0.
  __syncthreads();
  float* const mo = smem;
  float* const mm = smem + C::kWaves * 32 * C::kOPitch;
  float* const ml = mm + C::kWaves * 32;
  const float lt = sum_halves(l);
#pragma unroll
  for (int db = 0; db < C::kDB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i)
      mo[(wave * 32 + l32) * C::kOPitch + 32 * db + 8 * (i >> 2) + 4 * hi + (i & 3)] = oacc[db][i];
  if (hi == 0) {
    mm[wave * 32 + l32] = m;
    ml[wave * 32 + l32] = lt;
  }
  __syncthreads();
  const int r = tid / (C::kThreads / 32);
  const int col0 = (tid % (C::kThreads / 32)) * C::kColsPerThread;
  float mx = -INFINITY;
#pragma unroll
  for (int w = 0; w < C::kWaves; ++w) mx = fmaxf(mx, mm[w * 32 + r]);
  float wgt[C::kWaves];
  float lsum = 0.f;
#pragma unroll
  for (int w = 0; w < C::kWaves; ++w) {
    const float mw = mm[w * 32 + r];
    wgt[w] = mw == -INFINITY ? 0.f : fast_exp2(mw - mx);
    lsum += wgt[w] * ml[w * 32 + r];
  }
  const int row = q0 + r;
  if (row < n_q) {
    const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
    float* op = static_cast<float*>(a.o) + ((size_t)bh * n_q + row) * D + col0;
#pragma unroll
    for (int c4 = 0; c4 < C::kColsPerThread; c4 += 4) {
      f32x4 res;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float acc = 0.f;
#pragma unroll
        for (int w = 0; w < C::kWaves; ++w) acc = fmaf(wgt[w], mo[(w * 32 + r) * C::kOPitch + col0 + c4 + e], acc);
        res[e] = acc * inv;
      }
      *reinterpret_cast<f32x4*>(op + c4) = res;
    }
    if (col0 == 0) a.lse[(size_t)bh * n_q + row] = lsum > 0.f ? (mx + fast_log2(lsum)) * kLn2 : -INFINITY;
  }
}

// The same with 16-row blocks on the 16x16x4 float32 products, for shapes
// whose 32-row blocks still leave compute units idle (one head of 4096 rows:
// 128 blocks of 32 for 256 compute units).  S^T = K Q^T per 16 keys: lane l
// holds keys 4(l/16) + i, i = 0..3, of query l % 16.  In O^T += V^T P^T the
// key dimension of product i is laid out so that lane group g = l / 16
// contracts key 4g + i: the lane's own probability i is then its B operand,
// and V is read at that key.  Rows of the LDS tiles are D + 4 floats apart,
// so that the four lane groups' reads fall into different banks.  W waves
// split the keys: 4, or 8 (two per SIMD, so that one wave's products run
// beside the other's softmax and loads) where they fit in registers and LDS
// (d <= 64: 175 registers, 136 KiB) and every wave gets several key steps.
template <int D, int W>
struct F32Split16Cfg {
  static constexpr int kWaves = W;
  static constexpr int kThreads = kWaves * 64;
  static constexpr int kBN = 32;                       // keys per wave step (two 16-key sub-blocks)
  static constexpr int kDB = D / 16;                   // 16-row blocks of O^T
  static constexpr int kPitch = D + 4;                 // floats per K or V row in LDS
  static constexpr int kChunks = D / 4;
  static constexpr int kLoads = kBN * kChunks / 64;
  static constexpr int kTile = 2 * kBN * kPitch;       // K then V, floats per wave
  static constexpr int kOPitch = D + 1;
  static constexpr int kMerge = kWaves * 16 * kOPitch + 2 * kWaves * 16;
  static constexpr int kSmem = kWaves * kTile > kMerge ? kWaves * kTile : kMerge;
  static constexpr int kColsPerThread = D / 16;        // merge: 16 threads per row
  static_assert(kLoads * 64 == kBN * kChunks, "step load split");
};

template <int D, bool CAUSAL, int W>
__global__ __launch_bounds__(W * 64) void fwd_f32_split16_kernel(FwdArgs a, int n_rb) {
  using C = F32Split16Cfg<D, W>;
  static_assert(W == 4 || (W == 8 && D <= 64), "eight waves only where their tiles fit in LDS");
  __shared__ __attribute__((aligned(16))) float smem[C::kSmem];

  const int work = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = work / n_rb;
  const int q0 = (work - bh * n_rb) * 16;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l16 = lane & 15;
  const int g = lane >> 4;
  const int n_q = a.n_q, n_k = a.n_k;
  float* const sk = smem + wave * C::kTile;
  float* const sv = sk + C::kBN * C::kPitch;

  const float* qp = static_cast<const float*>(a.q) + (size_t)bh * n_q * D;
  const int kvh = kv_head_index(bh, a.H, a.group);
  const float* kp = static_cast<const float*>(a.k) + (size_t)kvh * n_k * D;
  const float* vp = static_cast<const float*>(a.v) + (size_t)kvh * n_k * D;

  const int qi = q0 + l16;
  float qf[D / 4];
#pragma unroll
  for (int c = 0; c < D / 4; ++c) qf[c] = (qi < n_q) ? qp[(size_t)qi * D + 4 * c + g] : 0.f;

  const Band band = band_of(a, CAUSAL);
  const int q_end = min(n_q, q0 + 16);
  const int t_lo = band.key_lo(q0) / C::kBN;
  const int t_hi = max(t_lo, (band.key_hi(q_end) + C::kBN - 1) / C::kBN);
  int vlo, vspan;  // keys this lane's query sees: [vlo, vlo + vspan]
  band.key_range(qi, vlo, vspan);
  const int wfull_lo = band.key_full_lo(q0 + 16), wfull_hi = band.key_full_hi(q0);
  const float sl2 = a.scale_log2;

  f32x4 kst[C::kLoads], vst[C::kLoads];
  auto gload = [&](int t) {
#pragma unroll
    for (int i = 0; i < C::kLoads; ++i) {
      const int idx = lane + i * 64;
      const int row = idx / C::kChunks;
      const int ch = idx - row * C::kChunks;
      const int key = t * C::kBN + row;
      if (key < n_k) {
        kst[i] = *reinterpret_cast<const f32x4*>(kp + (size_t)key * D + ch * 4);
        vst[i] = *reinterpret_cast<const f32x4*>(vp + (size_t)key * D + ch * 4);
      } else {
        kst[i] = f32x4{};
        vst[i] = f32x4{};
      }
    }
  };
  // The wave's own tile: its LDS accesses run in program order.
  auto swrite = [&]() {
#pragma unroll
    for (int i = 0; i < C::kLoads; ++i) {
      const int idx = lane + i * 64;
      const int row = idx / C::kChunks;
      const int ch = idx - row * C::kChunks;
      *reinterpret_cast<f32x4*>(&sk[row * C::kPitch + ch * 4]) = kst[i];
      *reinterpret_cast<f32x4*>(&sv[row * C::kPitch + ch * 4]) = vst[i];
    }
  };

  f32x4 oacc[C::kDB];
#pragma unroll
  for (int db = 0; db < C::kDB; ++db) oacc[db] = f32x4{};
  float m = -INFINITY, l = 0.f;  // running maximum (log2 units) and this lane's partial sum

  int t = t_lo + wave;
  if (t < t_hi) gload(t);
  for (; t < t_hi; t += C::kWaves) {
    swrite();
    if (t + C::kWaves < t_hi) gload(t + C::kWaves);
    const int k0 = t * C::kBN;

    f32x4 s[2];
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      s[sb] = f32x4{};
#pragma unroll
      for (int c = 0; c < D / 4; ++c) s[sb] = mfma_f32_16(sk[(16 * sb + l16) * C::kPitch + 4 * c + g], qf[c], s[sb]);
    }
    const bool need_mask = k0 < wfull_lo || k0 + C::kBN > wfull_hi;
    if (need_mask) {
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (!Band::in_range(k0 + 16 * sb + 4 * g + i - vlo, 0, vspan)) s[sb][i] = -INFINITY;
    }
    // Online softmax over the step's 32 keys: the lane's 8 values, then the
    // four lane groups of the query.
    float mx = -INFINITY;
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
      for (int i = 0; i < 4; ++i) mx = fmaxf(mx, s[sb][i]);
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mt = (mx == -INFINITY) ? -INFINITY : mx * sl2;
    const float m_new = fmaxf(m, mt);
    const float ref = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = fast_exp2(m - ref);
    float p[2][4];
    float rs = 0.f;
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float pv = fast_exp2(fmaf(s[sb][i], sl2, -ref));
        if (need_mask && s[sb][i] == -INFINITY) pv = 0.f;
        p[sb][i] = pv;
        rs += pv;
      }
    l = alpha * l + rs;
    m = m_new;
#pragma unroll
    for (int db = 0; db < C::kDB; ++db) oacc[db] *= alpha;
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int db = 0; db < C::kDB; ++db)
          oacc[db] = mfma_f32_16(sv[(16 * sb + 4 * g + i) * C::kPitch + 16 * db + l16], p[sb][i], oacc[db]);
  }

  // Merge: each wave's O (rows = queries), m and l (summed over the four
  // lane groups); then 16 threads per row (the first 256) combine the waves.
  __syncthreads();
  float* const mo = smem;
  float* const mm = smem + C::kWaves * 16 * C::kOPitch;
  float* const ml = mm + C::kWaves * 16;
  float lt = l + __shfl_xor(l, 16);
  lt += __shfl_xor(lt, 32);
#pragma unroll
  for (int db = 0; db < C::kDB; ++db)
#pragma unroll
    for (int j = 0; j < 4; ++j) mo[(wave * 16 + l16) * C::kOPitch + 16 * db + 4 * g + j] = oacc[db][j];
  if (g == 0) {
    mm[wave * 16 + l16] = m;
    ml[wave * 16 + l16] = lt;
  }
  __syncthreads();
  if (tid >= 256) return;
  const int r = tid / 16;
  const int col0 = (tid % 16) * C::kColsPerThread;
  float mq = -INFINITY;
#pragma unroll
  for (int w = 0; w < C::kWaves; ++w) mq = fmaxf(mq, mm[w * 16 + r]);
  float wgt[C::kWaves];
  float lsum = 0.f;
#pragma unroll
  for (int w = 0; w < C::kWaves; ++w) {
    const float mw = mm[w * 16 + r];
    wgt[w] = mw == -INFINITY ? 0.f : fast_exp2(mw - mq);
    lsum += wgt[w] * ml[w * 16 + r];
  }
  const int row = q0 + r;
  if (row < n_q) {
    const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
    float* op = static_cast<float*>(a.o) + ((size_t)bh * n_q + row) * D + col0;
#pragma unroll
    for (int c = 0; c < C::kColsPerThread; ++c) {
      float acc = 0.f;
#pragma unroll
      for (int w = 0; w < C::kWaves; ++w) acc = fmaf(wgt[w], mo[(w * 16 + r) * C::kOPitch + col0 + c], acc);
      op[c] = acc * inv;
    }
    if (col0 == 0) a.lse[(size_t)bh * n_q + row] = lsum > 0.f ? (mq + fast_log2(lsum)) * kLn2 : -INFINITY;
  }
}

template <typename Kernel>
hipError_t launch(Kernel kernel, int grid, int block, const FwdArgs& a, int n_qtiles,
                  hipStream_t stream) {
  FwdArgs args = a;
  int nq = n_qtiles;
  void* params[] = {&args, &nq};
  return hipLaunchKernel(reinterpret_cast<const void*>(kernel), dim3(grid), dim3(block), params, 0,
                         stream);
}

template <int D, bool CAUSAL, int WAVES, bool MERGE>
hipError_t fwd_bf16_w(const FwdArgs& a, hipStream_t stream) {
  using C = Bf16FwdCfg<D, WAVES>;
  const int n_qtiles = (a.n_q + C::kBM - 1) / C::kBM;
  return launch(fwd_bf16_kernel<D, CAUSAL, WAVES, MERGE>, n_qtiles * a.BH, C::kThreads, a, n_qtiles, stream);
}

// Up to this many query rows per head, 128-row workgroups (4 waves) beat the
// 256-row ones: less padding and twice the workgroups in flight (measured at
// B=16, H=32, d=128: 17.7 vs 23.4 us at n=128, 96.6 vs 109 us at n=512, equal
// at n=1024, 3 % slower at n=4096).  With a sliding window a 256-row
// workgroup visits about window + 256 keys while each wave needs window + 32,
// so windows take 128-row workgroups at any length (H=32, n=4096, d=128:
// causal w=512 65.6 -> 56.1 us, w=2048 127 -> 116 us).
constexpr int kShortRows = 512;
// A causal pass gives its workgroups unequal work (the last query tiles see
// the most keys).  With fewer than two 256-row workgroups per compute unit of
// the 256-CU chip the longest tile sets the time, and 128-row workgroups
// balance better (B=1, H=32, d=128 causal: n=1024 31.5 -> 22.4 us, n=2048
// 58.1 -> 46.3 us, n=3072 86.9 -> 85.5 us; n=4096, 512 workgroups, equal).
// Without the mask they pay off only when 256-row workgroups would leave at
// least half the compute units idle (B=1, d=128: H=32 n=1024 33.1 -> 24.5
// us, H=8 n=4096 101 -> 74 us; but H=32 n=1536, 192 workgroups, 48.7 ->
// 51.0 us).
constexpr long long kCausalBalanceWgs = 512;
constexpr long long kIdleHalfWgs = 128;

template <int D, bool CAUSAL, bool MERGE>
hipError_t fwd_bf16_pp(const FwdArgs& a, hipStream_t stream) {
  using C = Bf16FwdCfg<D, 8>;
  const int n_qtiles = (a.n_q + C::kBM - 1) / C::kBM;
  const int total = n_qtiles * a.BH;
  // Without the mask every tile costs the same: one workgroup per compute
  // unit (one fills it) walks tiles w, w + grid, ..., each loading the next
  // tile while it writes the current one.  Causal tiles differ in cost and
  // keep one workgroup each, dispatched costliest first.
  int grid = total;
  if (!CAUSAL) {
    const int cus = compute_units(stream);
    if (cus > 0 && total > cus) grid = cus;
  }
  return launch(fwd_bf16_pp_kernel<D, CAUSAL, MERGE>, grid, C::kThreads, a, n_qtiles, stream);
}

template <int D, bool CAUSAL, bool MERGE>
hipError_t fwd_bf16_t(const FwdArgs& a, hipStream_t stream) {
  const long long wide_wgs = (long long)a.BH * ((a.n_q + Bf16FwdCfg<D, 8>::kBM - 1) / Bf16FwdCfg<D, 8>::kBM);
  const bool narrow = a.n_q <= kShortRows || a.window >= 0 ||
                      (CAUSAL ? wide_wgs < kCausalBalanceWgs : wide_wgs <= kIdleHalfWgs);
  if (narrow) return fwd_bf16_w<D, CAUSAL, 4, MERGE>(a, stream);
  // 256-row workgroups at d = 128 take the ping-pong kernel (bitwise the same
  // results; c3 243 -> 231 us, causal 133 -> 128 us, n = 8192 918 -> 870 us
  // on one box); at d = 64 it measured slower (147 -> 150 us) and d <= 64
  // keeps the plain 8-wave kernel.
  if constexpr (D == 128) return fwd_bf16_pp<D, CAUSAL, MERGE>(a, stream);
  else return fwd_bf16_w<D, CAUSAL, 8, MERGE>(a, stream);
}

template <int D, bool CAUSAL>
hipError_t fwd_f32_split_t(const FwdArgs& a, hipStream_t stream) {
  const int n_rb = (a.n_q + 31) / 32;
  return launch(fwd_f32_split_kernel<D, CAUSAL>, n_rb * a.BH, F32SplitCfg<D>::kThreads, a, n_rb, stream);
}

// Eight waves from this many keys on (four 32-key steps per wave); below it
// half of them would have one step or none.  Measured on MI355X, 4 -> 8
// waves: c2 fp32 (n = 4096, d = 64) 77.5 -> 60.7 us, d = 32 44.3 -> 33.7
// us, H=2 n=2048 d=64 40.8 -> 33.9 us; c1 (128 keys) 4.8 -> 5.7 us.
constexpr int kSplit16WideKeys = 1024;

template <int D, bool CAUSAL>
hipError_t fwd_f32_split16_t(const FwdArgs& a, hipStream_t stream) {
  const int n_rb = (a.n_q + 15) / 16;
  if constexpr (D <= 64) {
    if (a.n_k >= kSplit16WideKeys)
      return launch(fwd_f32_split16_kernel<D, CAUSAL, 8>, n_rb * a.BH, F32Split16Cfg<D, 8>::kThreads, a, n_rb,
                    stream);
  }
  return launch(fwd_f32_split16_kernel<D, CAUSAL, 4>, n_rb * a.BH, F32Split16Cfg<D, 4>::kThreads, a, n_rb, stream);
}

template <int D, bool CAUSAL, bool MERGE>
hipError_t fwd_f32_t(const FwdArgs& a, hipStream_t stream) {
  const int n_qtiles = (a.n_q + F32FwdCfg<D>::kBM - 1) / F32FwdCfg<D>::kBM;
  return launch(fwd_f32_kernel<D, CAUSAL, MERGE>, n_qtiles * a.BH, F32FwdCfg<D>::kThreads, a, n_qtiles,
                stream);
}

}  // namespace fwdk
}  // namespace fa
