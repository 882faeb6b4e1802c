// bf16 GEMM instantiation of the SwiGLU column layer: both projections in one
// product (paired gate / value weight tiles), SiLU(gate) * value in the
// epilogue; 256 x 256 tiles (128 features), global->LDS copy kernel.
#include "gemm_bf16_dma.h"

namespace tpk {

template <bool A_KMAJOR, bool B_KMAJOR, int EPI, bool OUT_F32>
hipError_t launch_gemm_bf16_t_cfg(const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb,
                                  int M, int N, int K, const Epilogue& ep, hipStream_t stream) {
  return gemm_detail::launch_tile_dma<256, 256, 2, 4, 4, A_KMAJOR, B_KMAJOR, EPI, OUT_F32>(
      A, lda, B, ldb, M, N, K, ep, stream);
}

template hipError_t launch_gemm_bf16_t_cfg<false, true, EPI_SWIGLU, false>(
    const uint16_t*, int64_t, const uint16_t*, int64_t, int, int, int, const Epilogue&, hipStream_t);

}  // namespace tpk
