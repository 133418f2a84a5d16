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
// result is bitwise repeatable.
//
// Stage 2 (dK, dV): each wave owns 32 keys and keeps their K and V rows in
// registers as matrix-core B operands for the whole pass.  Query blocks of
// 64 rows (Q, dO, LSE, D) stream through double-buffered LDS.  S = Q K^T and
// dP = dO V^T land in the accumulator layout with one key per lane, which is
// the B-operand layout needed for dV^T += dO^T P and dK^T += Q^T dS; the
// dO^T and Q^T A operands come from LDS through ds_read_b64_tr_b16.
//
// Stage 3 (dQ): mirrors the forward kernel.  Each wave owns 32 queries and
// keeps Q and dO in registers; key blocks of 64 rows (K, V) stream through
// LDS.  S^T = K Q^T and dP^T = V dO^T put one query per lane, so LSE_i and
// D_i are one register each, and dQ^T += K^T dS^T takes K^T through the
// transposing LDS read.
#include "fa_internal.hpp"
#include "fa_device.hpp"

#include <cmath>

namespace fa {
namespace {

// ------------------------------------------------------------ stage 1

template <int D, typename T>
__global__ __launch_bounds__(256) void bwd_preprocess_kernel(const T* __restrict__ o,
                                                            const T* __restrict__ dO,
                                                            float* __restrict__ delta,
                                                            long rows) {
  constexpr int kVec = 16 / sizeof(T);        // elements per 16-byte load
  constexpr int kLanesPerRow = D / kVec;      // 4 .. 32
  constexpr int kRowsPerBlock = 256 / kLanesPerRow;
  const int tid = threadIdx.x;
  const long row = (long)blockIdx.x * kRowsPerBlock + tid / kLanesPerRow;
  const int part = tid % kLanesPerRow;
  float acc = 0.f;
  if (row < rows) {
    const T* op = o + row * D + part * kVec;
    const T* gp = dO + row * D + part * kVec;
    if constexpr (sizeof(T) == 2) {
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
  if (row < rows && part == 0) delta[row] = acc;
}

// ------------------------------------------------------ stage 2 (bf16)

template <int D>
struct DkdvCfg {
  static constexpr int kWaves = 4;
  static constexpr int kThreads = kWaves * 64;
  static constexpr int kBK = kWaves * 32;        // keys per workgroup
  static constexpr int kBQ = 64;                 // queries per block
  static constexpr int kQS = kBQ / 32;           // 32-query sub-blocks
  static constexpr int kDC = D / 16;
  static constexpr int kDB = D / 32;
  static constexpr int kStride = D + 16;         // LDS pitch (elements) of Q and dO
  static constexpr int kChunks = D / 8;
  static constexpr int kLoads = kBQ * kChunks / kThreads;
  static_assert(kLoads * kThreads == kBQ * kChunks, "tile load split");
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) void bwd_dkdv_bf16_kernel(BwdArgs a, int n_ktiles) {
  using C = DkdvCfg<D>;
  __shared__ __attribute__((aligned(16))) __bf16 sq[2][C::kBQ * C::kStride];
  __shared__ __attribute__((aligned(16))) __bf16 sdo[2][C::kBQ * C::kStride];
  __shared__ __attribute__((aligned(16))) float slse[2][C::kBQ];
  __shared__ __attribute__((aligned(16))) float sdel[2][C::kBQ];

  const int work = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = work / n_ktiles;
  const int kt = work - bh * n_ktiles;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  const int n_q = a.n_q, n_k = a.n_k;
  const int k0 = kt * C::kBK;
  const int key = k0 + wave * 32 + l32;  // this lane's key (column of S)

  const __bf16* qp = static_cast<const __bf16*>(a.q) + (size_t)bh * n_q * D;
  const __bf16* dop = static_cast<const __bf16*>(a.dO) + (size_t)bh * n_q * D;
  const __bf16* kp = static_cast<const __bf16*>(a.k) + (size_t)bh * n_k * D;
  const __bf16* vp = static_cast<const __bf16*>(a.v) + (size_t)bh * n_k * D;
  const float* lsep = a.lse + (size_t)bh * n_q;
  const float* delp = a.delta + (size_t)bh * n_q;

  bf16x8 kf[C::kDC], vf[C::kDC];
#pragma unroll
  for (int c = 0; c < C::kDC; ++c) {
    if (key < n_k) {
      kf[c] = *reinterpret_cast<const bf16x8*>(kp + (size_t)key * D + 16 * c + 8 * hi);
      vf[c] = *reinterpret_cast<const bf16x8*>(vp + (size_t)key * D + 16 * c + 8 * hi);
    } else {
      kf[c] = bf16x8{};
      vf[c] = bf16x8{};
    }
  }

  // Query blocks that can see any key of this workgroup.
  const int qb_first = CAUSAL ? (k0 / C::kBQ) : 0;
  const int qb_end = (n_q + C::kBQ - 1) / C::kBQ;
  const int nblocks = (CAUSAL && k0 >= n_q) ? 0 : max(0, qb_end - qb_first);

  u32x4 qst[C::kLoads], dost[C::kLoads];
  float lse_st = 0.f, del_st = 0.f;
  auto gload = [&](int b) {
    const int qbase = (qb_first + b) * C::kBQ;
#pragma unroll
    for (int i = 0; i < C::kLoads; ++i) {
      const int idx = tid + i * C::kThreads;
      const int row = idx / C::kChunks;
      const int ch = idx - row * C::kChunks;
      const int qi = qbase + row;
      if (qi < n_q) {
        qst[i] = *reinterpret_cast<const u32x4*>(qp + (size_t)qi * D + ch * 8);
        dost[i] = *reinterpret_cast<const u32x4*>(dop + (size_t)qi * D + ch * 8);
      } else {
        qst[i] = u32x4{0u, 0u, 0u, 0u};
        dost[i] = u32x4{0u, 0u, 0u, 0u};
      }
    }
    if (tid < C::kBQ) {
      const int qi = qbase + tid;
      lse_st = (qi < n_q) ? lsep[qi] * kLog2e : 0.f;
      del_st = (qi < n_q) ? delp[qi] : 0.f;
    }
  };
  auto swrite = [&](int buf) {
#pragma unroll
    for (int i = 0; i < C::kLoads; ++i) {
      const int idx = tid + i * C::kThreads;
      const int row = idx / C::kChunks;
      const int ch = idx - row * C::kChunks;
      *reinterpret_cast<u32x4*>(&sq[buf][row * C::kStride + ch * 8]) = qst[i];
      *reinterpret_cast<u32x4*>(&sdo[buf][row * C::kStride + ch * 8]) = dost[i];
    }
    if (tid < C::kBQ) {
      slse[buf][tid] = lse_st;
      sdel[buf][tid] = del_st;
    }
  };

  f32x16 dk[C::kDB], dv[C::kDB];
#pragma unroll
  for (int db = 0; db < C::kDB; ++db) { dk[db] = f32x16{}; dv[db] = f32x16{}; }

  const int grp = lane >> 4;
  const int tr_row = (lane & 15) >> 2;
  const int tr_col = 16 * (grp & 1) + 4 * (lane & 3);

  if (nblocks > 0) {
    gload(0);
    swrite(0);
  }
  __syncthreads();

  for (int b = 0; b < nblocks; ++b) {
    const int buf = b & 1;
    if (b + 1 < nblocks) gload(b + 1);
    const int qbase = (qb_first + b) * C::kBQ;

#pragma unroll
    for (int qs = 0; qs < C::kQS; ++qs) {
      const int qrow0 = qbase + qs * 32;
      // Skip sub-blocks entirely above this wave's keys (all hidden).
      if (CAUSAL && qrow0 + 31 < k0 + wave * 32) continue;
      f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int c = 0; c < C::kDC; ++c) {
        const int off = (qs * 32 + l32) * C::kStride + 16 * c + 8 * hi;
        const bf16x8 qa = *reinterpret_cast<const bf16x8*>(&sq[buf][off]);
        const bf16x8 ga = *reinterpret_cast<const bf16x8*>(&sdo[buf][off]);
        s = mfma_bf16(qa, kf[c], s);
        dp = mfma_bf16(ga, vf[c], dp);
      }
      // P and dS; element i is query row qrow0 + 8*(i/4) + 4*hi + (i%4).
      f32x16 p, ds;
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int r0 = qs * 32 + 8 * g4 + 4 * hi;
        const f32x4 lv = *reinterpret_cast<const f32x4*>(&slse[buf][r0]);
        const f32x4 dv4 = *reinterpret_cast<const f32x4*>(&sdel[buf][r0]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = 4 * g4 + e;
          const int qi = qbase + r0 + e;
          float pv = fast_exp2(fmaf(s[i], a.scale_log2, -lv[e]));
          const bool hide = qi >= n_q || key >= n_k || (CAUSAL && key > qi);
          pv = hide ? 0.f : pv;
          p[i] = pv;
          ds[i] = pv * (dp[i] - dv4[e]);
        }
      }
      // dV^T += dO^T P and dK^T += Q^T dS, 16 queries per step.
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2) {
        bf16x8 pb, dsb;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          pb[e] = (__bf16)p[8 * c2 + e];
          dsb[e] = (__bf16)ds[8 * c2 + e];
        }
        const int ra = qs * 32 + 16 * c2 + 4 * hi + tr_row;
#pragma unroll
        for (int db = 0; db < C::kDB; ++db) {
          const int col = 32 * db + tr_col;
          const bf16x4 ga = lds_read_tr16(&sdo[buf][ra * C::kStride + col]);
          const bf16x4 gb = lds_read_tr16(&sdo[buf][(ra + 8) * C::kStride + col]);
          const bf16x8 gop = {ga[0], ga[1], ga[2], ga[3], gb[0], gb[1], gb[2], gb[3]};
          dv[db] = mfma_bf16(gop, pb, dv[db]);
          const bf16x4 qa = lds_read_tr16(&sq[buf][ra * C::kStride + col]);
          const bf16x4 qb2 = lds_read_tr16(&sq[buf][(ra + 8) * C::kStride + col]);
          const bf16x8 qop = {qa[0], qa[1], qa[2], qa[3], qb2[0], qb2[1], qb2[2], qb2[3]};
          dk[db] = mfma_bf16(qop, dsb, dk[db]);
        }
      }
    }

    if (b + 1 < nblocks) swrite(buf ^ 1);
    __syncthreads();
  }

  if (key < n_k) {
    __bf16* dkp = static_cast<__bf16*>(a.dk) + ((size_t)bh * n_k + key) * D;
    __bf16* dvp = static_cast<__bf16*>(a.dv) + ((size_t)bh * n_k + key) * D;
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

template <int D>
struct DqCfg {
  static constexpr int kWaves = 4;
  static constexpr int kThreads = kWaves * 64;
  static constexpr int kBM = kWaves * 32;        // queries per workgroup
  static constexpr int kBN = 64;                 // keys per block
  static constexpr int kKB = kBN / 32;
  static constexpr int kDC = D / 16;
  static constexpr int kDB = D / 32;
  static constexpr int kStride = D + 16;
  static constexpr int kChunks = D / 8;
  static constexpr int kLoads = kBN * kChunks / kThreads;
  static_assert(kLoads * kThreads == kBN * kChunks, "tile load split");
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) void bwd_dq_bf16_kernel(BwdArgs a, int n_qtiles) {
  using C = DqCfg<D>;
  __shared__ __attribute__((aligned(16))) __bf16 sk[2][C::kBN * C::kStride];
  __shared__ __attribute__((aligned(16))) __bf16 sv[2][C::kBN * C::kStride];

  const int work = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = work / n_qtiles;
  int qt = work - bh * n_qtiles;
  if (CAUSAL) qt = n_qtiles - 1 - qt;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  const int n_q = a.n_q, n_k = a.n_k;
  const int q0 = qt * C::kBM;
  const int qw = q0 + wave * 32;
  const int qi = qw + l32;  // this lane's query (column of S^T)

  const __bf16* qp = static_cast<const __bf16*>(a.q) + (size_t)bh * n_q * D;
  const __bf16* dop = static_cast<const __bf16*>(a.dO) + (size_t)bh * n_q * D;
  const __bf16* kp = static_cast<const __bf16*>(a.k) + (size_t)bh * n_k * D;
  const __bf16* vp = static_cast<const __bf16*>(a.v) + (size_t)bh * n_k * D;

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
  const float lse2 = (qi < n_q) ? a.lse[(size_t)bh * n_q + qi] * kLog2e : 0.f;
  const float dlt = (qi < n_q) ? a.delta[(size_t)bh * n_q + qi] : 0.f;

  const int q_end = min(n_q, q0 + C::kBM);
  const int k_end = CAUSAL ? min(n_k, q_end) : n_k;
  const int ntiles = (k_end + C::kBN - 1) / C::kBN;

  u32x4 kst[C::kLoads], vst[C::kLoads];
  auto gload = [&](int t) {
#pragma unroll
    for (int i = 0; i < C::kLoads; ++i) {
      const int idx = tid + i * C::kThreads;
      const int row = idx / C::kChunks;
      const int ch = idx - row * C::kChunks;
      const int kj = t * C::kBN + row;
      if (kj < n_k) {
        kst[i] = *reinterpret_cast<const u32x4*>(kp + (size_t)kj * D + ch * 8);
        vst[i] = *reinterpret_cast<const u32x4*>(vp + (size_t)kj * D + ch * 8);
      } else {
        kst[i] = u32x4{0u, 0u, 0u, 0u};
        vst[i] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  };
  auto swrite = [&](int buf) {
#pragma unroll
    for (int i = 0; i < C::kLoads; ++i) {
      const int idx = tid + i * C::kThreads;
      const int row = idx / C::kChunks;
      const int ch = idx - row * C::kChunks;
      *reinterpret_cast<u32x4*>(&sk[buf][row * C::kStride + ch * 8]) = kst[i];
      *reinterpret_cast<u32x4*>(&sv[buf][row * C::kStride + ch * 8]) = vst[i];
    }
  };

  f32x16 dq[C::kDB];
#pragma unroll
  for (int db = 0; db < C::kDB; ++db) dq[db] = f32x16{};

  const int grp = lane >> 4;
  const int tr_row = (lane & 15) >> 2;
  const int tr_col = 16 * (grp & 1) + 4 * (lane & 3);

  gload(0);
  swrite(0);
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    if (t + 1 < ntiles) gload(t + 1);
    const int k0 = t * C::kBN;
#pragma unroll
    for (int kb = 0; kb < C::kKB; ++kb) {
      if (CAUSAL && k0 + kb * 32 > qw + 31) continue;  // all keys hidden from this wave
      f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int c = 0; c < C::kDC; ++c) {
        const int off = (kb * 32 + l32) * C::kStride + 16 * c + 8 * hi;
        const bf16x8 ka = *reinterpret_cast<const bf16x8*>(&sk[buf][off]);
        const bf16x8 va = *reinterpret_cast<const bf16x8*>(&sv[buf][off]);
        s = mfma_bf16(ka, qf[c], s);
        dp = mfma_bf16(va, gf[c], dp);
      }
      f32x16 ds;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int kj = k0 + kb * 32 + 8 * (i >> 2) + 4 * hi + (i & 3);
        float pv = fast_exp2(fmaf(s[i], a.scale_log2, -lse2));
        const bool hide = qi >= n_q || kj >= n_k || (CAUSAL && kj > qi);
        pv = hide ? 0.f : pv;
        ds[i] = pv * (dp[i] - dlt);
      }
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2) {
        bf16x8 dsb;
#pragma unroll
        for (int e = 0; e < 8; ++e) dsb[e] = (__bf16)ds[8 * c2 + e];
        const int ra = kb * 32 + 16 * c2 + 4 * hi + tr_row;
#pragma unroll
        for (int db = 0; db < C::kDB; ++db) {
          const int col = 32 * db + tr_col;
          const bf16x4 x = lds_read_tr16(&sk[buf][ra * C::kStride + col]);
          const bf16x4 y = lds_read_tr16(&sk[buf][(ra + 8) * C::kStride + col]);
          const bf16x8 kop = {x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
          dq[db] = mfma_bf16(kop, dsb, dq[db]);
        }
      }
    }
    if (t + 1 < ntiles) swrite(buf ^ 1);
    __syncthreads();
  }

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

  const int work = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = work / n_ktiles;
  const int kt = work - bh * n_ktiles;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  const int n_q = a.n_q, n_k = a.n_k;
  const int k0 = kt * C::kBlk;
  const int kw = k0 + wave * 32;
  const int key = kw + l32;

  const float* qp = static_cast<const float*>(a.q) + (size_t)bh * n_q * D;
  const float* dop = static_cast<const float*>(a.dO) + (size_t)bh * n_q * D;
  const float* kp = static_cast<const float*>(a.k) + (size_t)bh * n_k * D;
  const float* vp = static_cast<const float*>(a.v) + (size_t)bh * n_k * D;
  const float* lsep = a.lse + (size_t)bh * n_q;
  const float* delp = a.delta + (size_t)bh * n_q;

  // K and V rows of this lane's key, as B operands (d = 2c + hi).
  float kreg[D / 2], vreg[D / 2];
#pragma unroll
  for (int c = 0; c < D / 2; ++c) {
    kreg[c] = (key < n_k) ? kp[(size_t)key * D + 2 * c + hi] : 0.f;
    vreg[c] = (key < n_k) ? vp[(size_t)key * D + 2 * c + hi] : 0.f;
  }

  const int qb_first = CAUSAL ? (k0 / C::kBS) : 0;
  const int qb_end = (n_q + C::kBS - 1) / C::kBS;
  const int nblocks = (CAUSAL && k0 >= n_q) ? 0 : max(0, qb_end - qb_first);

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
      lse_st = (qi < n_q) ? lsep[qi] * kLog2e : 0.f;
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

  if (nblocks > 0) {
    gload(0);
    swrite(0);
  }
  __syncthreads();

  for (int b = 0; b < nblocks; ++b) {
    const int buf = b & 1;
    if (b + 1 < nblocks) gload(b + 1);
    const int qbase = (qb_first + b) * C::kBS;
    if (!(CAUSAL && qbase + 31 < kw)) {
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
        const bool hide = qi >= n_q || key >= n_k || (CAUSAL && key > qi);
        pv = hide ? 0.f : pv;
        p[i] = pv;
        ds[i] = pv * (dp[i] - sdel[buf][r]);
      }
      // dV^T[d][key] += dO^T P: A = dO^T (row d, k = query), B = P (k = query).
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int r = 8 * (i >> 2) + 4 * hi + (i & 3);
#pragma unroll
        for (int db = 0; db < C::kDB; ++db) {
          dv[db] = mfma_f32(sdo[buf][r * C::kStride + 32 * db + l32], p[i], dv[db]);
          dk[db] = mfma_f32(sq[buf][r * C::kStride + 32 * db + l32], ds[i], dk[db]);
        }
      }
    }
    if (b + 1 < nblocks) swrite(buf ^ 1);
    __syncthreads();
  }

  if (key < n_k) {
    float* dkp = static_cast<float*>(a.dk) + ((size_t)bh * n_k + key) * D;
    float* dvp = static_cast<float*>(a.dv) + ((size_t)bh * n_k + key) * D;
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

  const int work = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = work / n_qtiles;
  int qt = work - bh * n_qtiles;
  if (CAUSAL) qt = n_qtiles - 1 - qt;
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
  const float* kp = static_cast<const float*>(a.k) + (size_t)bh * n_k * D;
  const float* vp = static_cast<const float*>(a.v) + (size_t)bh * n_k * D;

  // Q and dO rows of this lane's query, as B operands (d = 2c + hi).
  float qreg[D / 2], greg[D / 2];
#pragma unroll
  for (int c = 0; c < D / 2; ++c) {
    qreg[c] = (qi < n_q) ? qp[(size_t)qi * D + 2 * c + hi] : 0.f;
    greg[c] = (qi < n_q) ? dop[(size_t)qi * D + 2 * c + hi] : 0.f;
  }
  const float lse2 = (qi < n_q) ? a.lse[(size_t)bh * n_q + qi] * kLog2e : 0.f;
  const float dlt = (qi < n_q) ? a.delta[(size_t)bh * n_q + qi] : 0.f;

  const int q_end = min(n_q, q0 + C::kBlk);
  const int k_end = CAUSAL ? min(n_k, q_end) : n_k;
  const int ntiles = (k_end + C::kBS - 1) / C::kBS;

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

  gload(0);
  swrite(0);
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    if (t + 1 < ntiles) gload(t + 1);
    const int k0 = t * C::kBS;
    if (!(CAUSAL && k0 > qw + 31)) {
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
        const bool hide = qi >= n_q || kj >= n_k || (CAUSAL && kj > qi);
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
    }
    if (t + 1 < ntiles) swrite(buf ^ 1);
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

template <int D, bool CAUSAL>
hipError_t dkdv_bf16_t(const BwdArgs& a, hipStream_t s) {
  const int n_ktiles = (a.n_k + DkdvCfg<D>::kBK - 1) / DkdvCfg<D>::kBK;
  BwdArgs args = a;
  int nt = n_ktiles;
  void* params[] = {&args, &nt};
  return launch_raw(reinterpret_cast<const void*>(bwd_dkdv_bf16_kernel<D, CAUSAL>),
                    n_ktiles * a.BH, 256, params, s);
}

template <int D, bool CAUSAL>
hipError_t dq_bf16_t(const BwdArgs& a, hipStream_t s) {
  const int n_qtiles = (a.n_q + DqCfg<D>::kBM - 1) / DqCfg<D>::kBM;
  BwdArgs args = a;
  int nt = n_qtiles;
  void* params[] = {&args, &nt};
  return launch_raw(reinterpret_cast<const void*>(bwd_dq_bf16_kernel<D, CAUSAL>),
                    n_qtiles * a.BH, 256, params, s);
}

template <int D, bool CAUSAL>
hipError_t dkdv_f32_t(const BwdArgs& a, hipStream_t s) {
  const int n_ktiles = (a.n_k + F32BwdCfg<D>::kBlk - 1) / F32BwdCfg<D>::kBlk;
  BwdArgs args = a;
  int nt = n_ktiles;
  void* params[] = {&args, &nt};
  return launch_raw(reinterpret_cast<const void*>(bwd_dkdv_f32_kernel<D, CAUSAL>),
                    n_ktiles * a.BH, 256, params, s);
}

template <int D, bool CAUSAL>
hipError_t dq_f32_t(const BwdArgs& a, hipStream_t s) {
  const int n_qtiles = (a.n_q + F32BwdCfg<D>::kBlk - 1) / F32BwdCfg<D>::kBlk;
  BwdArgs args = a;
  int nt = n_qtiles;
  void* params[] = {&args, &nt};
  return launch_raw(reinterpret_cast<const void*>(bwd_dq_f32_kernel<D, CAUSAL>),
                    n_qtiles * a.BH, 256, params, s);
}

template <int D, typename T>
hipError_t preprocess_t(const BwdArgs& a, hipStream_t s) {
  constexpr int kRowsPerBlock = 256 / (D / (16 / sizeof(T)));
  const long rows = (long)a.BH * a.n_q;
  const long grid = (rows + kRowsPerBlock - 1) / kRowsPerBlock;
  const T* o = static_cast<const T*>(a.o);
  const T* g = static_cast<const T*>(a.dO);
  float* delta = a.delta;
  long r = rows;
  void* params[] = {&o, &g, &delta, &r};
  return hipLaunchKernel(reinterpret_cast<const void*>(bwd_preprocess_kernel<D, T>),
                         dim3((unsigned)grid), dim3(256), params, 0, s);
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

}  // namespace fa
