// bf16 GEMM instantiations: 64x128 tiles (products with too few 128x128 tiles to fill the CUs), plain / bias / residual epilogue (row-parallel layer).
#include "gemm_bf16_dma.h"

namespace tpk {

template hipError_t launch_gemm_bf16_cfg<64, 128, EPI_LINEAR, true>(const uint16_t*, int64_t, const uint16_t*, int64_t, int, int, int, const Epilogue&, hipStream_t);

template hipError_t launch_gemm_bf16_cfg<64, 128, EPI_LINEAR, false>(const uint16_t*, int64_t, const uint16_t*, int64_t, int, int, int, const Epilogue&, hipStream_t);

template hipError_t launch_gemm_bf16_cfg<64, 128, EPI_QKV_F16, false>(const uint16_t*, int64_t, const uint16_t*, int64_t, int, int, int, const Epilogue&, hipStream_t);

}  // namespace tpk
