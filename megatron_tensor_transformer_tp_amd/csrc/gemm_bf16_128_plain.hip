// bf16 GEMM instantiations: 128x128 tiles, plain / bias / residual epilogue (row-parallel layer).
#include "gemm_bf16_impl.h"

namespace tpk {

template <int BM, int BN, int EPI, bool OUT_F32>
hipError_t launch_gemm_bf16_cfg(const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb,
                                int M, int N, int K, const Epilogue& ep, hipStream_t stream) {
  return gemm_detail::launch_tile<BM, BN, 2, 2, EPI, OUT_F32>(A, lda, B, ldb, M, N, K, ep, stream);
}

template hipError_t launch_gemm_bf16_cfg<128, 128, EPI_LINEAR, true>(const uint16_t*, int64_t, const uint16_t*, int64_t, int, int, int, const Epilogue&, hipStream_t);

template hipError_t launch_gemm_bf16_cfg<128, 128, EPI_LINEAR, false>(const uint16_t*, int64_t, const uint16_t*, int64_t, int, int, int, const Epilogue&, hipStream_t);

}  // namespace tpk
