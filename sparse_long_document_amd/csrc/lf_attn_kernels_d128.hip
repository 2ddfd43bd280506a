// The forward kernels (bf16 and fp32) at head dim 128: the same source as
// the head-dim-64 kernels, compiled with LF_KD = 128.
#define LF_KD 128
#include "lf_attn_kernels.hip"
