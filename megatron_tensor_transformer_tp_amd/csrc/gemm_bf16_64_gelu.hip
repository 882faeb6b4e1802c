// bf16 GEMM instantiations: 64x128 tiles (products with too few 128x128 tiles to fill the CUs), GeLU epilogue (column-parallel layer).
#include "gemm_bf16_dma.h"

namespace tpk {

template hipError_t launch_gemm_bf16_cfg<64, 128, EPI_GELU, true>(const uint16_t*, int64_t, const uint16_t*, int64_t, int, int, int, const Epilogue&, hipStream_t);

template hipError_t launch_gemm_bf16_cfg<64, 128, EPI_GELU, false>(const uint16_t*, int64_t, const uint16_t*, int64_t, int, int, int, const Epilogue&, hipStream_t);

}  // namespace tpk
