// Dispatch of the bf16 GEMM to its tile shape and epilogue instantiation.
#include "gemm_bf16_impl.h"

namespace tpk {

namespace {
template <int BM, int BN>
hipError_t launch_epi(const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb, int M, int N,
                      int K, const Epilogue& ep, hipStream_t stream) {
  if (ep.kind == EPI_GELU)
    return ep.out_f32 ? launch_gemm_bf16_cfg<BM, BN, EPI_GELU, true>(A, lda, B, ldb, M, N, K, ep, stream)
                      : launch_gemm_bf16_cfg<BM, BN, EPI_GELU, false>(A, lda, B, ldb, M, N, K, ep, stream);
  if (ep.kind == EPI_QKV_F16)
    return ep.out_f32 ? hipErrorInvalidValue
                      : launch_gemm_bf16_cfg<BM, BN, EPI_QKV_F16, false>(A, lda, B, ldb, M, N, K, ep, stream);
  if (ep.kind != EPI_LINEAR) return hipErrorInvalidValue;
  return ep.out_f32 ? launch_gemm_bf16_cfg<BM, BN, EPI_LINEAR, true>(A, lda, B, ldb, M, N, K, ep, stream)
                    : launch_gemm_bf16_cfg<BM, BN, EPI_LINEAR, false>(A, lda, B, ldb, M, N, K, ep, stream);
}
}  // namespace

hipError_t launch_gemm_bf16(const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb,
                            int64_t M, int64_t N, int64_t K, const Epilogue& ep,
                            hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  const int64_t tiles256 = ((M + 255) / 256) * ((N + 255) / 256);
  // Large problems: 256x256 tiles (one workgroup per CU); a single round of
  // at least 192 of them (3/4 of the CUs at full per-tile speed) still beats
  // 128x128 tiles (measured on the 4096 x 3072 x 8192 attention projection).
  // Smaller ones: 128x128 tiles so that the 256 CUs still get work.
  if (tiles256 >= 192)
    return launch_epi<256, 256>(A, lda, B, ldb, static_cast<int>(M), static_cast<int>(N),
                                static_cast<int>(K), ep, stream);
  return launch_epi<128, 128>(A, lda, B, ldb, static_cast<int>(M), static_cast<int>(N),
                              static_cast<int>(K), ep, stream);
}

hipError_t launch_gemm_bf16_t(const uint16_t* A, int64_t lda, bool a_kmajor, const uint16_t* B,
                              int64_t ldb, bool b_kmajor, int64_t M, int64_t N, int64_t K,
                              const Epilogue& ep, hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  if (K <= 0) return hipErrorInvalidValue;
  const int m = static_cast<int>(M), n = static_cast<int>(N), k = static_cast<int>(K);
  if (!a_kmajor && b_kmajor) {
    if (ep.kind == EPI_GELU_BWD) return hipErrorInvalidValue;
    return launch_gemm_bf16(A, lda, B, ldb, M, N, K, ep, stream);
  }
  if (!a_kmajor && !b_kmajor) {
    if (ep.kind == EPI_GELU_BWD && !ep.out_f32)
      return launch_gemm_bf16_t_cfg<false, false, EPI_GELU_BWD, false>(A, lda, B, ldb, m, n, k, ep, stream);
    if (ep.kind == EPI_LINEAR)
      return ep.out_f32 ? launch_gemm_bf16_t_cfg<false, false, EPI_LINEAR, true>(A, lda, B, ldb, m, n, k, ep, stream)
                        : launch_gemm_bf16_t_cfg<false, false, EPI_LINEAR, false>(A, lda, B, ldb, m, n, k, ep, stream);
    return hipErrorInvalidValue;
  }
  if (a_kmajor && b_kmajor && ep.kind == EPI_LINEAR)
    return ep.out_f32 ? launch_gemm_bf16_t_cfg<true, true, EPI_LINEAR, true>(A, lda, B, ldb, m, n, k, ep, stream)
                      : launch_gemm_bf16_t_cfg<true, true, EPI_LINEAR, false>(A, lda, B, ldb, m, n, k, ep, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_gemm_bf16_swiglu(const uint16_t* A, int64_t lda, const uint16_t* Bg,
                                   const uint16_t* Bu, int64_t ldb, int64_t M, int64_t F,
                                   int64_t K, uint16_t* out, int64_t ldo, hipStream_t stream) {
  if (M == 0 || F == 0) return hipSuccess;
  if (K <= 0 || F % 8 != 0) return hipErrorInvalidValue;
  Epilogue ep{nullptr, nullptr, 0, out, ldo, false, EPI_SWIGLU};
  ep.b2 = Bu;
  // the product runs over the 2F interleaved gate / value columns
  return launch_gemm_bf16_t_cfg<false, true, EPI_SWIGLU, false>(
      A, lda, Bg, ldb, static_cast<int>(M), static_cast<int>(2 * F), static_cast<int>(K), ep, stream);
}

}  // namespace tpk
