// Forward pass of exact attention on gfx950: O = softmax(scale Q K^T [+ M]) V
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
// fp32 kernel
// -----------
// Same dataflow with float32 operands on the 32x32x2 f32 matrix cores,
// 4 waves x 32 query rows and 32-key blocks; probabilities stay in fp32.
#include "fa_internal.hpp"
#include "fa_device.hpp"
#include "fa_tiles.hpp"

#include <cmath>
#include <type_traits>

namespace fa {
namespace {

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

template <int D, bool CAUSAL, int WAVES>
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
  // sees no key at all gets O = 0 and LSE = -inf.
  const float lt = sum_halves(l);
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

template <int D, bool CAUSAL>
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

template <typename Kernel>
hipError_t launch(Kernel kernel, int grid, int block, const FwdArgs& a, int n_qtiles,
                  hipStream_t stream) {
  FwdArgs args = a;
  int nq = n_qtiles;
  void* params[] = {&args, &nq};
  return hipLaunchKernel(reinterpret_cast<const void*>(kernel), dim3(grid), dim3(block), params, 0,
                         stream);
}

template <int D, bool CAUSAL, int WAVES>
hipError_t fwd_bf16_w(const FwdArgs& a, hipStream_t stream) {
  using C = Bf16FwdCfg<D, WAVES>;
  const int n_qtiles = (a.n_q + C::kBM - 1) / C::kBM;
  return launch(fwd_bf16_kernel<D, CAUSAL, WAVES>, n_qtiles * a.BH, C::kThreads, a, n_qtiles, stream);
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

template <int D, bool CAUSAL>
hipError_t fwd_bf16_t(const FwdArgs& a, hipStream_t stream) {
  const long long wide_wgs = (long long)a.BH * ((a.n_q + Bf16FwdCfg<D, 8>::kBM - 1) / Bf16FwdCfg<D, 8>::kBM);
  const bool narrow = a.n_q <= kShortRows || a.window >= 0 ||
                      (CAUSAL ? wide_wgs < kCausalBalanceWgs : wide_wgs <= kIdleHalfWgs);
  return narrow ? fwd_bf16_w<D, CAUSAL, 4>(a, stream) : fwd_bf16_w<D, CAUSAL, 8>(a, stream);
}

template <int D, bool CAUSAL>
hipError_t fwd_f32_t(const FwdArgs& a, hipStream_t stream) {
  const int n_qtiles = (a.n_q + F32FwdCfg<D>::kBM - 1) / F32FwdCfg<D>::kBM;
  return launch(fwd_f32_kernel<D, CAUSAL>, n_qtiles * a.BH, F32FwdCfg<D>::kThreads, a, n_qtiles,
                stream);
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdArgs& a, int d, bool causal, hipStream_t stream) {
  switch (d) {
    case 32: return causal ? fwd_bf16_t<32, true>(a, stream) : fwd_bf16_t<32, false>(a, stream);
    case 64: return causal ? fwd_bf16_t<64, true>(a, stream) : fwd_bf16_t<64, false>(a, stream);
    case 128: return causal ? fwd_bf16_t<128, true>(a, stream) : fwd_bf16_t<128, false>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_fwd_f32(const FwdArgs& a, int d, bool causal, hipStream_t stream) {
  switch (d) {
    case 32: return causal ? fwd_f32_t<32, true>(a, stream) : fwd_f32_t<32, false>(a, stream);
    case 64: return causal ? fwd_f32_t<64, true>(a, stream) : fwd_f32_t<64, false>(a, stream);
    case 128: return causal ? fwd_f32_t<128, true>(a, stream) : fwd_f32_t<128, false>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fa
