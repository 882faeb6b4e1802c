// bf16 GEMM instantiations with k-major flags A true, B true (A given as [K, M], B [K, N]: the weight gradients H^T dZ and X^T dY):
// 128x128 tiles (4 waves, two workgroups per CU), global->LDS copy kernel (ragged M, N and K included).
#include "gemm_bf16_dma.h"

namespace tpk {

template hipError_t launch_gemm_bf16_t_cfg<128, 128, true, true, EPI_LINEAR, true>(const uint16_t*, int64_t, const uint16_t*, int64_t, int, int, int, const Epilogue&, hipStream_t);

template hipError_t launch_gemm_bf16_t_cfg<128, 128, true, true, EPI_LINEAR, false>(const uint16_t*, int64_t, const uint16_t*, int64_t, int, int, int, const Epilogue&, hipStream_t);

}  // namespace tpk
