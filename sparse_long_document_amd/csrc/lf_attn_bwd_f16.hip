// The backward kernels with f16 elements: the same source, built with
// _Float16 as its 16-bit element type.
#define LF_HALF_F16 1
#include "lf_attn_bwd.hip"
