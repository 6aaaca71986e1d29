// grouped_gemm_f4.hip -- the NVFP4 and MXFP4 instantiations of the
// persistent grouped GEMM (grouped_gemm.hip), in a compilation unit of their
// own, built like the bf16 unit (AGPR accumulators), so that the units
// compile side by side.
#define MOE_GROUPED_F4_UNIT 1
#include "grouped_gemm.hip"
