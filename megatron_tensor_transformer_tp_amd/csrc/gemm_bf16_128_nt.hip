// bf16 GEMM instantiations with k-major flags A false, B false (A [M, K], B given as [N, K]: dH = dZ B_i^T with the GeLU-backward epilogue, dX = dY A_i^T):
// 128x128 tiles (4 waves, two workgroups per CU), global->LDS copy kernel (ragged M, N and K included).
#include "gemm_bf16_dma.h"

namespace tpk {

template hipError_t launch_gemm_bf16_t_cfg<128, 128, false, false, EPI_GELU_BWD, false>(const uint16_t*, int64_t, const uint16_t*, int64_t, int, int, int, const Epilogue&, hipStream_t);

template hipError_t launch_gemm_bf16_t_cfg<128, 128, false, false, EPI_LINEAR, true>(const uint16_t*, int64_t, const uint16_t*, int64_t, int, int, int, const Epilogue&, hipStream_t);

template hipError_t launch_gemm_bf16_t_cfg<128, 128, false, false, EPI_LINEAR, false>(const uint16_t*, int64_t, const uint16_t*, int64_t, int, int, int, const Epilogue&, hipStream_t);

}  // namespace tpk
