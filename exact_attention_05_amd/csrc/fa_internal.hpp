// Internal kernel parameters and launchers shared by the C ABI and the
// kernel translation units.  Not part of the public interface.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace fa {

// Arguments of one forward launch.  All tensors contiguous (B,H,n,d).
struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int BH;           // B * H (query heads)
  int H;            // query heads per batch entry
  int group;        // query heads per K/V head (H / H_kv); 1 without sharing
  int n_q;
  int n_k;
  int q_offset;     // absolute position of query row 0 against key 0 (see Band)
  int window;       // sliding-window half-width, or -1 for none (see Band)
  float scale;      // softmax scale on q . k
  float scale_log2; // scale * log2(e): scores are exponentiated base 2
  // Merge launches only: the rows' prior result over other keys, o_prior
  // (B,H,n_q,d) and its natural-log lse_prior (B,H,n_q); o and lse receive
  // the result over both key sets.  prior_f32 / out_f32: o_prior / o hold
  // float32 (else bf16; the fp32 kernel takes float32 only).
  const void* o_prior;
  const float* lse_prior;
  int prior_f32;
  int out_f32;
};

// Arguments of the backward stages.
struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dO;
  const float* lse;  // (B,H,n_q) natural-log LSE saved by the forward pass
  float* delta;     // workspace: (B,H,n_q) float32 row sums of dO * O
  float* lse2;      // workspace: (B,H,n_q) float32 LSE * log2(e)
  void* dq;
  void* dk;         // (B,H_kv,n_k,d), like k
  void* dv;
  int BH;           // B * H (query heads)
  int H;            // query heads per batch entry
  int group;        // query heads per K/V head (H / H_kv)
  int n_q;
  int n_k;
  int q_offset;
  int window;
  float scale;
  float scale_log2;
  // Shared K/V heads: the group's query heads are split into `slices`
  // consecutive runs, one dK/dV workgroup per (key tile, K/V head, run); with
  // more than one run each writes float32 partial sums (slices, B*H_kv, n_k, d)
  // that a reduction adds up in a fixed order.
  int slices;
  float* part_dk;
  float* part_dv;
};

// (batch, K/V head) index of the query head bh = b * H + h.  Query heads are
// grouped consecutively: heads h = j * group .. j * group + group - 1 share
// K/V head j ("Attention Mechanism", section 12 "GQA vs MQA").
__host__ __device__ inline int kv_head_index(int bh, int H, int group) {
  if (group == 1) return bh;
  return (bh / H) * (H / group) + (bh % H) / group;
}

// Which keys a query row sees.  Query row i sits at absolute position
// p = i + q_offset on the key axis (q_offset = 0: the top-left alignment of
// the causal mask, "Attention Mechanism", section 4.4); key j is hidden when
// j >= n_k, when causal and j > p, or, with a sliding window of half-width
// w >= 0, when |p - j| > w (same page, section 4.5 "Sparse Attention", the
// window of the +-w neighbours).  The helpers give half-open index ranges.
struct Band {
  int n_q, n_k, q_offset, window;
  bool causal;

  __host__ __device__ bool hidden(int q, int key) const {
    const int p = q + q_offset;
    return key >= n_k || (causal && key > p) || (window >= 0 && (key < p - window || key > p + window));
  }
  // Keys seen by some row of [r0, r1) (r0 < r1).
  __host__ __device__ int key_lo(int r0) const {
    return window < 0 ? 0 : max(0, r0 + q_offset - window);
  }
  __host__ __device__ int key_hi(int r1) const {
    int h = n_k;
    if (causal) h = min(h, r1 + q_offset);
    if (window >= 0) h = min(h, r1 + q_offset + window);
    return max(h, 0);
  }
  // Keys seen by every row of [r0, r1) (possibly an empty range).
  __host__ __device__ int key_full_lo(int r1) const {
    return window < 0 ? 0 : max(0, r1 - 1 + q_offset - window);
  }
  __host__ __device__ int key_full_hi(int r0) const {
    int h = n_k;
    if (causal) h = min(h, r0 + q_offset + 1);
    if (window >= 0) h = min(h, r0 + q_offset + window + 1);
    return max(h, 0);
  }
  // The keys row q sees as one interval [lo, lo + span]: key is visible iff
  // (unsigned)(key - lo) <= (unsigned)span -- one subtraction and one
  // comparison per element in the kernels.  A row that sees nothing gets
  // lo = 2^30, span = 0 (every index here is below 2^30).
  __host__ __device__ void key_range(int q, int& lo, int& span) const {
    const int p = q + q_offset;
    int l = 0, h = n_k - 1;
    if (causal) h = min(h, p);
    if (window >= 0) {
      l = max(l, p - window);
      h = min(h, p + window);
    }
    lo = h < l ? (1 << 30) : l;
    span = h < l ? 0 : h - l;
  }
  // The rows that see key as one interval, the same way (a key past n_k is
  // seen by none).
  __host__ __device__ void query_range(int key, int& lo, int& span) const {
    int l = 0, h = n_q - 1;
    if (causal) l = max(l, key - q_offset);
    if (window >= 0) {
      l = max(l, key - q_offset - window);
      h = min(h, key - q_offset + window);
    }
    if (key >= n_k) h = -1;
    lo = h < l ? (1 << 30) : l;
    span = h < l ? 0 : h - l;
  }
  __host__ __device__ static bool in_range(int x, int lo, int span) {
    return (unsigned)(x - lo) <= (unsigned)span;
  }
  // Query rows that see some key of [k0, k1) (k0 < k1 <= n_k).
  __host__ __device__ int q_lo(int k0) const {
    int l = 0;
    if (causal) l = max(l, k0 - q_offset);
    if (window >= 0) l = max(l, k0 - q_offset - window);
    return min(l, n_q);
  }
  __host__ __device__ int q_hi(int k1) const {
    int h = n_q;
    if (window >= 0) h = min(h, k1 - 1 - q_offset + window + 1);
    return max(h, 0);
  }
  // Query rows that see every key of [k0, k1) (possibly an empty range).
  __host__ __device__ int q_full_lo(int k1) const {
    int l = 0;
    if (causal) l = max(l, k1 - 1 - q_offset);
    if (window >= 0) l = max(l, k1 - 1 - q_offset - window);
    return min(l, n_q);
  }
  __host__ __device__ int q_full_hi(int k0) const {
    int h = n_q;
    if (window >= 0) h = min(h, k0 - q_offset + window + 1);
    return max(h, 0);
  }
};

template <typename Args>
__host__ __device__ inline Band band_of(const Args& a, bool causal) {
  return Band{a.n_q, a.n_k, a.q_offset, a.window, causal};
}

// Arguments of one split-KV decoding launch (bf16).  The group * n_q query
// rows that share a K/V head are packed: packed row r is row r % n_q of query
// head kv * group + r / n_q.  The keys are cut into n_splits chunks of `chunk`
// keys (a multiple of the key block); each (batch, K/V head, row block,
// chunk) workgroup leaves a partial result that the merge combines, unless
// n_splits == 1, when it writes O and LSE itself.
struct DecArgs {
  const void* q;     // (B,H,n_q,d)
  const void* k;     // (B,H_kv,n_k,d)
  const void* v;
  void* o;           // (B,H,n_q,d) bf16
  float* lse;        // (B,H,n_q)
  float* part_o;     // (n_splits, B*H*n_q, d) float32 partial outputs
  float* part_lse;   // (n_splits, B*H*n_q) float32 partial LSE
  int B;
  int H;             // query heads per batch entry
  int group;         // query heads per K/V head
  int h_kv;          // K/V heads per batch entry
  int n_q;
  int n_k;
  int q_offset;
  int window;
  int rows;          // group * n_q packed rows per (batch, K/V head)
  int n_rb;          // 32-row blocks of packed rows
  int n_splits;
  int chunk;         // keys per split
  float scale_log2;
};

// Arguments of the LSE merge of n_parts partial results over disjoint key
// sets: parts (n_parts, rows, d) and (n_parts, rows) -> (rows, d), (rows).
struct MergeArgs {
  const void* o_parts;
  const float* lse_parts;
  void* o;
  float* lse;
  long long rows;
  int n_parts;
};

// Each launcher enqueues its kernel(s) on `stream` and returns the HIP status
// of the launch.  Shapes were validated by the caller.
// Compute units of the device that `stream` runs on (0 if unknown); cached
// per device.
int compute_units(hipStream_t stream);

hipError_t launch_fwd_bf16(const FwdArgs& a, int d, bool causal, hipStream_t stream);
hipError_t launch_fwd_f32(const FwdArgs& a, int d, bool causal, hipStream_t stream);
// Float32 forward with the keys of each 32-row block split over the four
// waves of a workgroup (for shapes with few query rows and many keys).
hipError_t launch_fwd_f32_split(const FwdArgs& a, int d, bool causal, hipStream_t stream);
// The same with 16-row blocks (16x16x4 products), for still fewer rows.
hipError_t launch_fwd_f32_split16(const FwdArgs& a, int d, bool causal, hipStream_t stream);
// The same passes with the epilogue merging into a.o_prior, a.lse_prior.
hipError_t launch_fwd_merge_bf16(const FwdArgs& a, int d, bool causal, hipStream_t stream);
hipError_t launch_fwd_merge_f32(const FwdArgs& a, int d, bool causal, hipStream_t stream);

hipError_t launch_bwd_preprocess(const BwdArgs& a, int d, bool bf16, hipStream_t stream);
hipError_t launch_bwd_dkdv_bf16(const BwdArgs& a, int d, bool causal, hipStream_t stream);
hipError_t launch_bwd_dq_bf16(const BwdArgs& a, int d, bool causal, hipStream_t stream);
hipError_t launch_bwd_dkdv_f32(const BwdArgs& a, int d, bool causal, hipStream_t stream);
hipError_t launch_bwd_dq_f32(const BwdArgs& a, int d, bool causal, hipStream_t stream);
// dK, dV (the input dtype) = the sum over the slices of the float32 partials.
hipError_t launch_bwd_reduce_slices(const BwdArgs& a, int d, bool bf16, hipStream_t stream);

// Key block of the decoding kernel: chunks are whole multiples of it.
constexpr int kDecodeBlock = 128;
hipError_t launch_decode_bf16(const DecArgs& a, int d, bool causal, hipStream_t stream);
// in_bf16 / out_bf16: bf16 (else float32) partial and merged outputs.
hipError_t launch_lse_merge(const MergeArgs& a, int d, bool in_bf16, bool out_bf16, hipStream_t stream);

}  // namespace fa
