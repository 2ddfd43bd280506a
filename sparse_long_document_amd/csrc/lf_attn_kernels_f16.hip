// The forward kernel for f16 inputs: the same source as the bf16 kernel,
// compiled with f16 as its 16-bit element type (v_mfma_f32_32x32x16_f16,
// v_dot2_f32_f16, f16 probabilities and outputs).
#define LF_HALF_F16 1
#include "lf_attn_kernels.hip"
