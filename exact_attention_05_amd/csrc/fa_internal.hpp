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
  float scale;      // softmax scale on q . k
  float scale_log2; // scale * log2(e): scores are exponentiated base 2
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
  float scale;
  float scale_log2;
};

// (batch, K/V head) index of the query head bh = b * H + h.  Query heads are
// grouped consecutively: heads h = j * group .. j * group + group - 1 share
// K/V head j ("Attention Mechanism", section 12 "GQA vs MQA").
__host__ __device__ inline int kv_head_index(int bh, int H, int group) {
  if (group == 1) return bh;
  return (bh / H) * (H / group) + (bh % H) / group;
}

// Each launcher enqueues its kernel(s) on `stream` and returns the HIP status
// of the launch.  Shapes were validated by the caller.
hipError_t launch_fwd_bf16(const FwdArgs& a, int d, bool causal, hipStream_t stream);
hipError_t launch_fwd_f32(const FwdArgs& a, int d, bool causal, hipStream_t stream);

hipError_t launch_bwd_preprocess(const BwdArgs& a, int d, bool bf16, hipStream_t stream);
hipError_t launch_bwd_dkdv_bf16(const BwdArgs& a, int d, bool causal, hipStream_t stream);
hipError_t launch_bwd_dq_bf16(const BwdArgs& a, int d, bool causal, hipStream_t stream);
hipError_t launch_bwd_dkdv_f32(const BwdArgs& a, int d, bool causal, hipStream_t stream);
hipError_t launch_bwd_dq_f32(const BwdArgs& a, int d, bool causal, hipStream_t stream);

}  // namespace fa
