// The f16 forward kernel at head dim 32 (lf_attn_kernels.hip with LF_KD =
// 32 and LF_HALF_F16).
#define LF_KD 32
#define LF_HALF_F16 1
#include "lf_attn_kernels.hip"
