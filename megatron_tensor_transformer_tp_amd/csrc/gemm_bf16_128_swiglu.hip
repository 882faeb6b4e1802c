// bf16 GEMM instantiation of the SwiGLU column layer: both projections in one
// product (paired gate / value weight tiles), SiLU(gate) * value in the
// epilogue; 128 x 128 tiles (64 features; 4 waves, two workgroups per CU), global->LDS copy kernel.
#include "gemm_bf16_dma.h"

namespace tpk {

template hipError_t launch_gemm_bf16_t_cfg<128, 128, false, true, EPI_SWIGLU, false>(
    const uint16_t*, int64_t, const uint16_t*, int64_t, int, int, int, const Epilogue&, hipStream_t);

}  // namespace tpk
