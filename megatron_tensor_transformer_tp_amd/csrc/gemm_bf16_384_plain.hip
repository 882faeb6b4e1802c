// bf16 GEMM instantiations: 128x384 tiles, plain / bias / residual and packed-QKV epilogues.
// One round of these fills the 256 CUs where 256x256 tiles would leave a
// quarter of them idle (e.g. the 4096 x 3072 attention projection: 256 tiles
// instead of 192).
#include "gemm_bf16_dma.h"

namespace tpk {

template <int BM, int BN, int EPI, bool OUT_F32>
hipError_t launch_gemm_bf16_cfg(const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb,
                                int M, int N, int K, const Epilogue& ep, hipStream_t stream) {
  // global->LDS copy kernel: 8 waves (2 per SIMD) of 64 x 96, 4 LDS stages of
  // 32 KiB
  return gemm_detail::launch_tile_dma<BM, BN, 2, 4, 4, false, true, EPI, OUT_F32>(
      A, lda, B, ldb, M, N, K, ep, stream);
}

template hipError_t launch_gemm_bf16_cfg<128, 384, EPI_LINEAR, true>(const uint16_t*, int64_t, const uint16_t*, int64_t, int, int, int, const Epilogue&, hipStream_t);

template hipError_t launch_gemm_bf16_cfg<128, 384, EPI_LINEAR, false>(const uint16_t*, int64_t, const uint16_t*, int64_t, int, int, int, const Epilogue&, hipStream_t);

template hipError_t launch_gemm_bf16_cfg<128, 384, EPI_QKV_F16, false>(const uint16_t*, int64_t, const uint16_t*, int64_t, int, int, int, const Epilogue&, hipStream_t);

}  // namespace tpk
