// Vector decode kernel, paged KV cache: the instantiations of gqa_valu.hip
// for this addressing mode, in a translation unit of their own.
#define ATTN_VALU_MODE 2
#include "gqa_valu.hip"
