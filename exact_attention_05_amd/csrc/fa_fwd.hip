// Forward pass of exact attention on gfx950 (the kernels are in
// fa_fwd_kernels.hpp): the plain launches, O and LSE written directly.
#include "fa_fwd_kernels.hpp"

namespace fa {

using fwdk::fwd_bf16_t;
using fwdk::fwd_f32_t;
using fwdk::fwd_f32_split_t;
using fwdk::fwd_f32_split16_t;

hipError_t launch_fwd_bf16(const FwdArgs& a, int d, bool causal, hipStream_t stream) {
  switch (d) {
    case 32: return causal ? fwd_bf16_t<32, true, false>(a, stream) : fwd_bf16_t<32, false, false>(a, stream);
    case 64: return causal ? fwd_bf16_t<64, true, false>(a, stream) : fwd_bf16_t<64, false, false>(a, stream);
    case 128: return causal ? fwd_bf16_t<128, true, false>(a, stream) : fwd_bf16_t<128, false, false>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_fwd_f32_split(const FwdArgs& a, int d, bool causal, hipStream_t stream) {
  switch (d) {
    case 32: return causal ? fwd_f32_split_t<32, true>(a, stream) : fwd_f32_split_t<32, false>(a, stream);
    case 64: return causal ? fwd_f32_split_t<64, true>(a, stream) : fwd_f32_split_t<64, false>(a, stream);
    case 128: return causal ? fwd_f32_split_t<128, true>(a, stream) : fwd_f32_split_t<128, false>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_fwd_f32_split16(const FwdArgs& a, int d, bool causal, hipStream_t stream) {
  switch (d) {
    case 32: return causal ? fwd_f32_split16_t<32, true>(a, stream) : fwd_f32_split16_t<32, false>(a, stream);
    case 64: return causal ? fwd_f32_split16_t<64, true>(a, stream) : fwd_f32_split16_t<64, false>(a, stream);
    case 128: return causal ? fwd_f32_split16_t<128, true>(a, stream) : fwd_f32_split16_t<128, false>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_fwd_f32(const FwdArgs& a, int d, bool causal, hipStream_t stream) {
  switch (d) {
    case 32: return causal ? fwd_f32_t<32, true, false>(a, stream) : fwd_f32_t<32, false, false>(a, stream);
    case 64: return causal ? fwd_f32_t<64, true, false>(a, stream) : fwd_f32_t<64, false, false>(a, stream);
    case 128: return causal ? fwd_f32_t<128, true, false>(a, stream) : fwd_f32_t<128, false, false>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fa
