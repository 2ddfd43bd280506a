// The forward kernels (bf16 and fp32) at head dim 32: the same source as
// the head-dim-64 kernels, compiled with LF_KD = 32.
#define LF_KD 32
#include "lf_attn_kernels.hip"
