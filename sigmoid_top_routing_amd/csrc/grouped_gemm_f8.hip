// grouped_gemm_f8.hip -- the block-FP8 instantiations of the persistent
// grouped GEMM (grouped_gemm.hip), in a compilation unit of their own: it is
// built with the MFMAs' VGPR form (-mllvm -amdgpu-mfma-vgpr-form), which
// keeps the 128 accumulators of a lane in VGPRs, where the rescale at each
// K-block boundary multiplies them in place. The bf16 kernels, whose
// 256-row tiles hold 256 accumulators per lane, stay in the other unit with
// AGPR accumulators.
#define MOE_GROUPED_F8_UNIT 1
#include "grouped_gemm.hip"
