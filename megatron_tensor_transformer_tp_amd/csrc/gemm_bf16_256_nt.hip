// bf16 GEMM instantiations with k-major flags A false, B false (A [M, K], B given as [N, K]: dH = dZ B_i^T with the GeLU-backward epilogue, dX = dY A_i^T):
// 256x256 tiles, global->LDS copy kernel (ragged M, N and K included).
#include "gemm_bf16_dma.h"

namespace tpk {

template <bool A_KMAJOR, bool B_KMAJOR, int EPI, bool OUT_F32>
hipError_t launch_gemm_bf16_t_cfg(const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb,
                                  int M, int N, int K, const Epilogue& ep, hipStream_t stream) {
  return gemm_detail::launch_tile_dma<256, 256, 2, 4, 4, A_KMAJOR, B_KMAJOR, EPI, OUT_F32>(
      A, lda, B, ldb, M, N, K, ep, stream);
}

template hipError_t launch_gemm_bf16_t_cfg<false, false, EPI_GELU_BWD, false>(const uint16_t*, int64_t, const uint16_t*, int64_t, int, int, int, const Epilogue&, hipStream_t);

template hipError_t launch_gemm_bf16_t_cfg<false, false, EPI_LINEAR, true>(const uint16_t*, int64_t, const uint16_t*, int64_t, int, int, int, const Epilogue&, hipStream_t);

template hipError_t launch_gemm_bf16_t_cfg<false, false, EPI_LINEAR, false>(const uint16_t*, int64_t, const uint16_t*, int64_t, int, int, int, const Epilogue&, hipStream_t);

}  // namespace tpk
