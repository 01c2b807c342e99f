// The decode megakernel for the sequential block with bf16 weights: mk_kernel.hip
// compiled with MK_SEQ = 1 (the MoE path normalizes x + this layer's Wo rows
// with its own gain; exported as mk_megakernel_seq / mkk_launch_step_seq).
#define MK_SEQ 1
#include "mk_kernel.hip"
