// Split-KV attention for decoding, and the merge of attention results over
// disjoint key sets.
//
// Decoding ("Attention Mechanism: Revolusi Representasi Sequence", section 8,
// "Key-Value (KV) Cache"): every generation step attends a handful of new
// query rows to all cached keys.  The work is one pass over K and V, so HBM
// bandwidth sets the time, not the matrix cores.  To keep enough workgroups
// in flight the key axis is cut into chunks ("split-KV"): a workgroup attends
// its query rows to one chunk and leaves the chunk's normalised output and
// LSE, and the merge combines the chunks exactly, weighting chunk p by
// exp(LSE_p - LSE) -- the online softmax's rescaling (same page, section 13)
// applied to whole chunks.  The merge alone is also the one-GPU piece of ring
// attention (same page, section 16): attention over a sequence whose keys are
// spread over several workers is the merge of each worker's (O, LSE).
//
// Decoding kernel (bf16)
// ----------------------
// The group * n_q query rows that share one K/V head (section 12, grouped
// K/V heads) are packed into 32-row blocks, so each K/V step is read once for
// the whole group.  A workgroup is W waves (4, or 8 for small grids at
// d <= 64) and owns one (batch, K/V head, row block, chunk); wave w takes the
// chunk's 32-key steps w, w+W, w+2W, ...
// and runs on its own, without workgroup barriers: the K and V rows of its
// next step load into registers while the current step, already written to
// the wave's own swizzled LDS tiles, is used with the forward pass's scheme
// (deeper register rings measured no faster: 101 us at three steps ahead
// against 98 us at one on the 32K-context workload): S^T = K Q^T
// on the 32x32x16 bf16 matrix cores (Q in registers), an online softmax per
// query column whose reference maximum moves only when a step raises it by
// more than 2^8 (the output is rescaled then, not at every step), O^T +=
// V^T P^T with V^T from the transposing LDS read.  At
// the end the waves' (m, l, O) are merged through LDS: the same
// rescaling, by exp2(m_w - max_w m_w).
//
// Merge kernel
// ------------
// D/4 threads per output row, four columns each; the part weights come from
// one pass over the parts' LSE values.
#include "fa_internal.hpp"
#include "fa_device.hpp"
#include "fa_tiles.hpp"

#include <cmath>

namespace fa {
namespace {

// Largest amount (log2 units) by which a row's scores may exceed the
// reference maximum its probabilities are taken against: they stay below
// 2^8, and their sums over any key range fit a float with room to spare.
constexpr float kLazyRescale = 8.0f;

template <int D, int W>
struct DecCfg {
  static constexpr int kWaves = W;
  static constexpr int kThreads = kWaves * 64;
  static constexpr int kSub = 32;              // keys per wave step
  static constexpr int kDepth = 1;             // steps loading while one is computed
  static constexpr int kDC = D / 16;           // 16-wide chunks of the head dim
  static constexpr int kDB = D / 32;           // 32-row blocks of O^T
  static constexpr int kPer = D / 8;           // output columns per thread at the end
  using T = Tile<D, kSub>;                     // one wave's K or V step in LDS
  static constexpr int kLd = T::kBytes / (64 * 16);  // 16-byte loads per lane per tile
  static_assert(kLd * 64 * 16 == T::kBytes, "whole 16-byte loads per lane");
  // Merge scratch: m and l per wave and query, then every wave's O^T.
  static constexpr int kScratchFloats = 2 * kWaves * 32 + kWaves * D * 32;
  static constexpr int kSmemBytes = kWaves * 2 * T::kBytes > kScratchFloats * 4
                                        ? kWaves * 2 * T::kBytes : kScratchFloats * 4;
};

template <int D, bool CAUSAL, int W>
__global__ __launch_bounds__(W * 64) void decode_bf16_kernel(DecArgs a) {
  using C = DecCfg<D, W>;
  using T = typename C::T;
  // Per wave: its K step then its V step; reused for the merge at the end.
  __shared__ __attribute__((aligned(1024))) char smem[C::kSmemBytes];

  int work = xcd_remap(blockIdx.x, gridDim.x);
  const int rb = work % a.n_rb;
  work /= a.n_rb;
  const int split = work % a.n_splits;
  work /= a.n_splits;
  const int b = work / a.h_kv;
  const int kvh = work - b * a.h_kv;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  const int n_q = a.n_q, n_k = a.n_k;
  const float sl2 = a.scale_log2;

  // This lane's packed query row: the column of S^T it holds.
  const int r = rb * 32 + l32;
  const bool rvalid = r < a.rows;
  const int qi = rvalid ? r % n_q : 0;
  const int hq = kvh * a.group + (rvalid ? r / n_q : 0);
  const __bf16* qp = static_cast<const __bf16*>(a.q) + (((size_t)b * a.H + hq) * n_q + qi) * D;
  const size_t kv_base = ((size_t)b * a.h_kv + kvh) * (size_t)n_k * D;
  const __bf16* kp = static_cast<const __bf16*>(a.k) + kv_base;
  const __bf16* vp = static_cast<const __bf16*>(a.v) + kv_base;

  bf16x8 qf[C::kDC];
#pragma unroll
  for (int c = 0; c < C::kDC; ++c)
    qf[c] = rvalid ? *reinterpret_cast<const bf16x8*>(qp + 16 * c + 8 * hi) : bf16x8{};

  // Rows (within a head) that the block holds: one run r0 % n_q .. (r1-1) %
  // n_q, or every row when the block wraps past a head.
  const int r0 = rb * 32, r1 = min(a.rows, r0 + 32);
  int i_lo = 0, i_hi = n_q;
  if (r1 - r0 < n_q && r0 % n_q <= (r1 - 1) % n_q) {
    i_lo = r0 % n_q;
    i_hi = (r1 - 1) % n_q + 1;
  }
  const Band band{n_q, n_k, a.q_offset, a.window, CAUSAL};
  // 32-key steps of this chunk that some row sees; the keys every row sees
  // (steps inside them need no mask).  Wave w takes steps w, w + 4, ...
  const int ks = split * a.chunk;
  const int ke = min(n_k, ks + a.chunk);
  const int key_lo = max(ks, band.key_lo(i_lo));
  const int key_hi = min(ke, band.key_hi(i_hi));
  const int s_lo = key_lo / C::kSub;
  const int s_hi = key_hi > key_lo ? (key_hi + C::kSub - 1) / C::kSub : s_lo;
  const int n_steps = max(0, (s_hi - s_lo - wave + C::kWaves - 1) / C::kWaves);
  const int full_lo = band.key_full_lo(i_hi);
  const int full_hi = band.key_full_hi(i_lo);
  int vlo, vspan;  // keys this lane's query sees: [vlo, vlo + vspan]
  band.key_range(qi, vlo, vspan);

  // Global -> register loads of one step (row-major 16-byte pieces, each
  // lane's piece at the same place in every row group), then register -> LDS
  // into the swizzled tile layout.  Rows past n_k repeat row n_k - 1.
  u32x4 kst[C::kDepth][C::kLd], vst[C::kDepth][C::kLd];
  auto load = [&](int j, auto slot) __attribute__((always_inline)) {
    constexpr int S = decltype(slot)::value;
    const int k0 = (s_lo + wave + C::kWaves * j) * C::kSub;
#pragma unroll
    for (int i = 0; i < C::kLd; ++i) {
      const int idx = lane + 64 * i;
      const int row = idx / T::kChunks;
      const int ch = idx - row * T::kChunks;
      const size_t off = (size_t)min(k0 + row, n_k - 1) * D + ch * 8;
      kst[S][i] = *reinterpret_cast<const u32x4*>(kp + off);
      vst[S][i] = *reinterpret_cast<const u32x4*>(vp + off);
    }
  };
  char* const kt = smem + wave * 2 * T::kBytes;
  char* const vt = kt + T::kBytes;
  TileLane<D, C::kSub> tl;
  tl.init(lane);
  auto stage = [&](auto slot) __attribute__((always_inline)) {
    constexpr int S = decltype(slot)::value;
#pragma unroll
    for (int i = 0; i < C::kLd; ++i) {
      const int idx = lane + 64 * i;
      const int row = idx / T::kChunks;
      const int ch = idx - row * T::kChunks;
      *reinterpret_cast<u32x4*>(kt + T::offset(row, ch)) = kst[S][i];
      *reinterpret_cast<u32x4*>(vt + T::offset(row, ch)) = vst[S][i];
    }
  };

  f32x16 oacc[C::kDB];
#pragma unroll
  for (int db = 0; db < C::kDB; ++db) oacc[db] = f32x16{};
  float m = -INFINITY, l = 0.f;  // running maximum (log2 units) and sum of this lane's query

  // One step: S^T = K Q^T for 32 keys, online softmax, O^T += V^T P^T.
  auto compute = [&](int j) __attribute__((always_inline)) {
    const int k0 = (s_lo + wave + C::kWaves * j) * C::kSub;
    const bool masked = k0 < full_lo || k0 + C::kSub > full_hi;
    f32x16 s = f32x16{};
#pragma unroll
    for (int c = 0; c < C::kDC; ++c) s = mfma_bf16(tl.read_rows(kt, 0, c), qf[c], s);
    if (masked) {
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (!Band::in_range(k0 + 4 * hi - vlo + 8 * (i >> 2) + (i & 3), 0, vspan)) s[i] = -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; i += 2) mx = fmaxf(mx, fmaxf(s[i], s[i + 1]));
    mx = max_halves(mx);
    const float mt = mx == -INFINITY ? -INFINITY : mx * sl2;
    // The reference maximum m moves only when a step raises some row's
    // maximum by more than kLazyRescale (log2 units), and then for every row
    // of the wave; otherwise the probabilities are taken against the old
    // reference (at most 2^kLazyRescale each) and the output is not
    // rescaled.  Exact in real arithmetic: O and l share the reference.
    if (__builtin_amdgcn_ballot_w64(mt > m + kLazyRescale) != 0) {
      const float m_new = fmaxf(m, mt);
      const float alpha = fast_exp2(m - (m_new == -INFINITY ? 0.f : m_new));  // 0 while the row saw nothing
      l *= alpha;
#pragma unroll
      for (int db = 0; db < C::kDB; ++db) oacc[db] *= alpha;
      m = m_new;
    }
    const float ref = m == -INFINITY ? 0.f : m;
    // P = exp2(scale_log2 * S - ref) as bf16 pairs, in the order of the
    // transposing V read (element i is key 8(i/4) + 4(l/32) + i%4).
    u32x4 pw[2];
    float rs = 0.f;
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        float p0 = fast_exp2(fmaf(s[8 * c2 + e], sl2, -ref));
        float p1 = fast_exp2(fmaf(s[8 * c2 + e + 1], sl2, -ref));
        if (masked) {
          if (s[8 * c2 + e] == -INFINITY) p0 = 0.f;
          if (s[8 * c2 + e + 1] == -INFINITY) p1 = 0.f;
        }
        pw[c2][e >> 1] = pack_bf16x2(p0, p1);
        rs += p0 + p1;
      }
    l += rs;
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
      for (int db = 0; db < C::kDB; ++db)
        oacc[db] = mfma_bf16(tl.read_cols_tr(vt, 16 * c2, 32 * db), bf16x8_of(pw[c2]), oacc[db]);
  };

  // The wave's steps through a ring of kDepth register sets: step j is
  // staged into LDS and computed while steps j+1 .. j+kDepth are loading.
  // Every ring slot is refilled at every turn -- past the last step with the
  // last step again (an L2 hit) -- so that the number of loads issued after
  // any step's loads is the same on every path and the compiler's wait before
  // staging a step covers only that step's loads.
  if (n_steps > 0) {
    static_for<0, C::kDepth>([&](auto u) __attribute__((always_inline)) {
      load(min((int)decltype(u)::value, n_steps - 1), u);
    });
    for (int j0 = 0; j0 < n_steps; j0 += C::kDepth) {
      static_for<0, C::kDepth>([&](auto u) __attribute__((always_inline)) {
        const int j = j0 + decltype(u)::value;
        const bool live = j < n_steps;
        if (live) stage(u);
        load(min(j + C::kDepth, n_steps - 1), u);
        if (live) compute(j);
      });
    }
  }

  settle_acc(oacc);  // the loop's last products, before the merge reads them

  // Merge the four waves: each scales its O^T by exp2(m_w - M), M the
  // largest m_w of the query, and the sums add up.
  const float lt = sum_halves(l);
  __syncthreads();  // every wave is done with its K/V tiles
  float* sm = reinterpret_cast<float*>(smem);  // [wave][32] m
  float* sl = sm + C::kWaves * 32;             // [wave][32] l
  float* so = sl + C::kWaves * 32;             // [wave][d][32] O^T
  if (hi == 0) {
    sm[wave * 32 + l32] = m;
    sl[wave * 32 + l32] = lt;
  }
  __syncthreads();
  {
    float mq = -INFINITY;
#pragma unroll
    for (int w = 0; w < C::kWaves; ++w) mq = fmaxf(mq, sm[w * 32 + l32]);
    const float f = fast_exp2(m - (mq == -INFINITY ? 0.f : mq));
#pragma unroll
    for (int db = 0; db < C::kDB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int d = 32 * db + 8 * (i >> 2) + 4 * hi + (i & 3);
        so[(wave * D + d) * 32 + l32] = oacc[db][i] * f;
      }
  }
  __syncthreads();

  // Thread (q = tid % 32, columns d0 .. d0 + kPer - 1) of packed row q.
  if (tid >= 256) return;  // the output: 8 threads per row, D / 8 columns each
  const int q = tid & 31;
  const int d0 = (tid >> 5) * C::kPer;
  float mq = -INFINITY;
#pragma unroll
  for (int w = 0; w < C::kWaves; ++w) mq = fmaxf(mq, sm[w * 32 + q]);
  const float ref = mq == -INFINITY ? 0.f : mq;
  float lq = 0.f;
#pragma unroll
  for (int w = 0; w < C::kWaves; ++w) lq += sl[w * 32 + q] * fast_exp2(sm[w * 32 + q] - ref);
  float acc[C::kPer];
#pragma unroll
  for (int j = 0; j < C::kPer; ++j) {
    float x = 0.f;
#pragma unroll
    for (int w = 0; w < C::kWaves; ++w) x += so[(w * D + d0 + j) * 32 + q];
    acc[j] = x;
  }
  const int rq = rb * 32 + q;
  if (rq >= a.rows) return;
  const float inv = lq > 0.f ? 1.f / lq : 0.f;
  const float lse_q = lq > 0.f ? (mq + fast_log2(lq)) * kLn2 : -INFINITY;
  const size_t row = ((size_t)b * a.H + kvh * a.group + rq / n_q) * n_q + rq % n_q;
  if (a.n_splits == 1) {
    __bf16* op = static_cast<__bf16*>(a.o) + row * D + d0;
    if constexpr (C::kPer % 8 == 0) {
#pragma unroll
      for (int j = 0; j < C::kPer; j += 8) {
        float v8[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v8[e] = acc[j + e] * inv;
        *reinterpret_cast<bf16x8*>(op + j) = to_bf16x8(v8);
      }
    } else {
      bf16x4 v4;
#pragma unroll
      for (int e = 0; e < 4; ++e) v4[e] = (__bf16)(acc[e] * inv);
      *reinterpret_cast<bf16x4*>(op) = v4;
    }
    if (d0 == 0) a.lse[row] = lse_q;
  } else {
    const size_t total = (size_t)a.B * a.H * n_q;
    float* pp = a.part_o + ((size_t)split * total + row) * D + d0;
#pragma unroll
    for (int j = 0; j < C::kPer; j += 4) {
      f32x4 v4;
#pragma unroll
      for (int e = 0; e < 4; ++e) v4[e] = acc[j + e] * inv;
      *reinterpret_cast<f32x4*>(pp + j) = v4;
    }
    if (d0 == 0) a.part_lse[(size_t)split * total + row] = lse_q;
  }
}

// ------------------------------------------------------------------ merge

template <typename T>
struct Vec4;
template <>
struct Vec4<float> {
  __device__ static __forceinline__ f32x4 load(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
  __device__ static __forceinline__ void store(float* p, const f32x4& v) { *reinterpret_cast<f32x4*>(p) = v; }
};
template <>
struct Vec4<__bf16> {
  __device__ static __forceinline__ f32x4 load(const __bf16* p) {
    const bf16x4 x = *reinterpret_cast<const bf16x4*>(p);
    return f32x4{(float)x[0], (float)x[1], (float)x[2], (float)x[3]};
  }
  __device__ static __forceinline__ void store(__bf16* p, const f32x4& v) {
    *reinterpret_cast<bf16x4*>(p) = bf16x4{(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
  }
};

// One 16-byte load of a part: 4 float32 or 8 bfloat16 values of a row.
template <typename T>
struct Part16 {
  static constexpr int kCols = 16 / (int)sizeof(T);
  __device__ static __forceinline__ void load(const T* p, float (&x)[kCols]) {
#pragma unroll
    for (int j = 0; j < kCols; j += 4) {
      const f32x4 v = Vec4<T>::load(p + j);
#pragma unroll
      for (int e = 0; e < 4; ++e) x[j + e] = v[e];
    }
  }
};

template <int D, typename TI, typename TO>
__global__ __launch_bounds__(256) void lse_merge_kernel(MergeArgs a) {
  constexpr int kCols = Part16<TI>::kCols;  // columns per thread: one 16-byte load per part
  constexpr int kTpr = D / kCols;           // threads per row
  constexpr int kRows = 256 / kTpr;         // rows per workgroup
  const long long row = (long long)blockIdx.x * kRows + threadIdx.x / kTpr;
  if (row >= a.rows) return;
  const int c = (threadIdx.x % kTpr) * kCols;
  const TI* op = static_cast<const TI*>(a.o_parts);
  const float* lp = a.lse_parts;

  // Parts in groups of kU, so that a group's loads are in flight together.
  constexpr int kU = 8;
  float mx = -INFINITY;
  for (int p0 = 0; p0 < a.n_parts; p0 += kU) {
    float lv[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u)
      lv[u] = p0 + u < a.n_parts ? lp[(size_t)(p0 + u) * a.rows + row] : -INFINITY;
#pragma unroll
    for (int u = 0; u < kU; ++u) mx = fmaxf(mx, lv[u]);
  }
  const float ref = mx == -INFINITY ? 0.f : mx;
  float acc[kCols];
#pragma unroll
  for (int j = 0; j < kCols; ++j) acc[j] = 0.f;
  float s = 0.f;
  for (int p0 = 0; p0 < a.n_parts; p0 += kU) {
    float w[kU];
    float x[kU][kCols];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const bool in = p0 + u < a.n_parts;
      const size_t pr = (size_t)(in ? p0 + u : p0) * a.rows + row;
      w[u] = in ? fast_exp2((lp[pr] - ref) * kLog2e) : 0.f;  // 0 for a part without keys
      Part16<TI>::load(op + pr * D + c, x[u]);
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
#pragma unroll
      for (int j = 0; j < kCols; ++j) acc[j] += w[u] * x[u][j];
      s += w[u];
    }
  }
  const float inv = s > 0.f ? 1.f / s : 0.f;
  TO* dst = static_cast<TO*>(a.o) + (size_t)row * D + c;
#pragma unroll
  for (int j = 0; j < kCols; j += 4)
    Vec4<TO>::store(dst + j, f32x4{acc[j] * inv, acc[j + 1] * inv, acc[j + 2] * inv, acc[j + 3] * inv});
  if (c == 0) a.lse[row] = s > 0.f ? ref + fast_log2(s) * kLn2 : -INFINITY;
}

template <int D, bool CAUSAL, int W>
hipError_t decode_w(const DecArgs& a, int grid, hipStream_t stream) {
  DecArgs args = a;
  void* params[] = {&args};
  return hipLaunchKernel(reinterpret_cast<const void*>(decode_bf16_kernel<D, CAUSAL, W>), dim3(grid),
                         dim3(DecCfg<D, W>::kThreads), params, 0, stream);
}

// Eight waves per workgroup (two per SIMD, each taking every eighth key step)
// when the grid has at most one workgroup per compute unit and d <= 64 (at
// d = 128 eight waves would spill): one wave per SIMD runs each step's
// dependent chain alone, a second one overlaps it.  Measured on MI355X (bf16
// forward, one chunk): B=1 H=1 n=4096 d=64 33.1 -> 23.7 us, d=32 25.2 -> 17.6
// us, H=2 2048 x 8192 keys 61.6 -> 42.2 us; with 512 workgroups (H=4
// n=4096) 43.3 -> 46.5 us, where four waves stay.
template <int D, bool CAUSAL>
hipError_t decode_t(const DecArgs& a, hipStream_t stream) {
  const int grid = a.B * a.h_kv * a.n_splits * a.n_rb;
  if constexpr (D <= 64) {
    const int cus = compute_units(stream);
    if (cus > 0 && grid <= cus) return decode_w<D, CAUSAL, 8>(a, grid, stream);
  }
  return decode_w<D, CAUSAL, 4>(a, grid, stream);
}

template <int D, typename TI, typename TO>
hipError_t merge_t(const MergeArgs& a, hipStream_t stream) {
  MergeArgs args = a;
  void* params[] = {&args};
  constexpr int kRows = 256 / (D / Part16<TI>::kCols);
  const int grid = (int)((a.rows + kRows - 1) / kRows);
  return hipLaunchKernel(reinterpret_cast<const void*>(lse_merge_kernel<D, TI, TO>), dim3(grid), dim3(256),
                         params, 0, stream);
}

template <int D>
hipError_t merge_d(const MergeArgs& a, bool in_bf16, bool out_bf16, hipStream_t s) {
  if (in_bf16) return out_bf16 ? merge_t<D, __bf16, __bf16>(a, s) : merge_t<D, __bf16, float>(a, s);
  return out_bf16 ? merge_t<D, float, __bf16>(a, s) : merge_t<D, float, float>(a, s);
}

}  // namespace

hipError_t launch_lse_merge(const MergeArgs& a, int d, bool in_bf16, bool out_bf16, hipStream_t s) {
  switch (d) {
    case 32: return merge_d<32>(a, in_bf16, out_bf16, s);
    case 64: return merge_d<64>(a, in_bf16, out_bf16, s);
    case 128: return merge_d<128>(a, in_bf16, out_bf16, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_decode_bf16(const DecArgs& a, int d, bool causal, hipStream_t s) {
  hipError_t e;
  switch (d) {
    case 32: e = causal ? decode_t<32, true>(a, s) : decode_t<32, false>(a, s); break;
    case 64: e = causal ? decode_t<64, true>(a, s) : decode_t<64, false>(a, s); break;
    case 128: e = causal ? decode_t<128, true>(a, s) : decode_t<128, false>(a, s); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess || a.n_splits == 1) return e;
  MergeArgs m;
  m.o_parts = a.part_o;
  m.lse_parts = a.part_lse;
  m.o = a.o;
  m.lse = a.lse;
  m.rows = (long long)a.B * a.H * a.n_q;
  m.n_parts = a.n_splits;
  return launch_lse_merge(m, d, false, true, s);
}

}  // namespace fa
