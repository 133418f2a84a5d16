// Forward pass of exact attention on gfx950 merged into a prior result over
// other keys (the kernels are in fa_fwd_kernels.hpp; the merge is their
// epilogue, merge_store).
#include "fa_fwd_kernels.hpp"

namespace fa {

using fwdk::fwd_bf16_t;
using fwdk::fwd_f32_t;

hipError_t launch_fwd_merge_bf16(const FwdArgs& a, int d, bool causal, hipStream_t stream) {
  switch (d) {
    case 32: return causal ? fwd_bf16_t<32, true, true>(a, stream) : fwd_bf16_t<32, false, true>(a, stream);
    case 64: return causal ? fwd_bf16_t<64, true, true>(a, stream) : fwd_bf16_t<64, false, true>(a, stream);
    case 128: return causal ? fwd_bf16_t<128, true, true>(a, stream) : fwd_bf16_t<128, false, true>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_fwd_merge_f32(const FwdArgs& a, int d, bool causal, hipStream_t stream) {
  switch (d) {
    case 32: return causal ? fwd_f32_t<32, true, true>(a, stream) : fwd_f32_t<32, false, true>(a, stream);
    case 64: return causal ? fwd_f32_t<64, true, true>(a, stream) : fwd_f32_t<64, false, true>(a, stream);
    case 128: return causal ? fwd_f32_t<128, true, true>(a, stream) : fwd_f32_t<128, false, true>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fa
