// bf16 GEMM instantiations: 128x384 tiles, GeLU epilogue (column-parallel layer).
// One round of these fills the 256 CUs where 256x256 tiles would leave a
// quarter of them idle (e.g. the 4096 x 3072 attention projection: 256 tiles
// instead of 192).
#include "gemm_bf16_dma.h"

namespace tpk {

template hipError_t launch_gemm_bf16_cfg<128, 384, EPI_GELU, true>(const uint16_t*, int64_t, const uint16_t*, int64_t, int, int, int, const Epilogue&, hipStream_t);

template hipError_t launch_gemm_bf16_cfg<128, 384, EPI_GELU, false>(const uint16_t*, int64_t, const uint16_t*, int64_t, int, int, int, const Epilogue&, hipStream_t);

}  // namespace tpk
