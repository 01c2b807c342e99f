// The decode megakernel for FP4 weights: mk_kernel.hip compiled with MK_WFMT = 2
// (LM head, Wqkv, Wo and expert gate/up/down as OCP E2M1 codes, two a byte,
// with one fp32 scale per row; exported as mk_megakernel_fp4 /
// mkk_launch_step_fp4).
#define MK_WFMT 2
#include "mk_kernel.hip"
