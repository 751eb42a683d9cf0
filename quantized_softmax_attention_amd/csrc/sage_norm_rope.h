// sage_norm_rope.h -- parameters of the RMSNorm + RoPE step that precedes
// quantisation (sage_qk_norm_rope, sage_quantize_qkv_rope), shared by the
// quantiser kernels and the C ABI layer.
#pragma once

namespace sage {

// RMSNorm weights and rotary table applied to Q and K before quantisation.
struct NormRope {
    const float *gamma_q, *gamma_k;   // [D] each
    const float *rope;                // [N, D/2, 2]: (cos, sin) per token and channel pair
    float eps;
};

}  // namespace sage
