// The decode megakernel for FP8 weights: mk_kernel.hip compiled with MK_WFMT = 1
// (LM head, Wqkv, Wo and expert gate/up/down as OCP E4M3 codes with one fp32
// scale per row; exported as mk_megakernel_fp8 / mkk_launch_step_fp8).
#define MK_WFMT 1
#include "mk_kernel.hip"
