// The f16 forward kernel at head dim 128 (lf_attn_kernels.hip with LF_KD =
// 128 and LF_HALF_F16).
#define LF_KD 128
#define LF_HALF_F16 1
#include "lf_attn_kernels.hip"
