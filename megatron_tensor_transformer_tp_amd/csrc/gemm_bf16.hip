// Dispatch of the bf16 GEMM to its tile shape and epilogue instantiation.
#include "gemm_bf16_impl.h"

namespace tpk {

namespace {
template <int BM, int BN>
hipError_t launch_epi(const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb, int M, int N,
                      int K, const Epilogue& ep, hipStream_t stream) {
  if (ep.gelu)
    return ep.out_f32 ? launch_gemm_bf16_cfg<BM, BN, true, true>(A, lda, B, ldb, M, N, K, ep, stream)
                      : launch_gemm_bf16_cfg<BM, BN, true, false>(A, lda, B, ldb, M, N, K, ep, stream);
  return ep.out_f32 ? launch_gemm_bf16_cfg<BM, BN, false, true>(A, lda, B, ldb, M, N, K, ep, stream)
                    : launch_gemm_bf16_cfg<BM, BN, false, false>(A, lda, B, ldb, M, N, K, ep, stream);
}
}  // namespace

hipError_t launch_gemm_bf16(const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb,
                            int64_t M, int64_t N, int64_t K, const Epilogue& ep,
                            hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  const int64_t tiles256 = ((M + 255) / 256) * ((N + 255) / 256);
  // Large problems: 256x256 tiles (one workgroup per CU, 144 KiB LDS).
  // Smaller ones: 128x128 tiles so that the 256 CUs still get work.
  if (tiles256 >= 256)
    return launch_epi<256, 256>(A, lda, B, ldb, static_cast<int>(M), static_cast<int>(N),
                                static_cast<int>(K), ep, stream);
  return launch_epi<128, 128>(A, lda, B, ldb, static_cast<int>(M), static_cast<int>(N),
                              static_cast<int>(K), ep, stream);
}

}  // namespace tpk
