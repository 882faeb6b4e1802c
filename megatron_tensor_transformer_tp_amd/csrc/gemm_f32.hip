// fp32 GEMM with fp32 FMA accumulation and the same fused epilogue as the
// bf16 path (bias, GeLU, residual).  This is the fp32 variant of the column-
// and row-parallel linears (列并行 tutorial, 数学基础 and MLP 应用); no value
// is rounded below fp32 anywhere.
//
// A [M, K] row-major (lda), B [K, N] row-major (ldb).  64 x 64 output tile
// per 256-thread workgroup, BK = 16, each thread a 4 x 4 block; both operand
// tiles staged in LDS k-major (sA[k][m], sB[k][n]) so the inner product
// reads are broadcast-friendly.  Edges are masked (zero-filled loads,
// predicated stores), so any M, N, K >= 1 works.
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "kernels.h"

namespace tpk {
namespace {

constexpr int kBM = 64, kBN = 64, kBKf = 16;

template <bool GELU>
__global__ __launch_bounds__(256) void gemm_f32_kernel(const float* __restrict__ A, int64_t lda,
                                                       const float* __restrict__ B, int64_t ldb,
                                                       int M, int N, int K,
                                                       const float* __restrict__ bias,
                                                       const float* __restrict__ residual,
                                                       int64_t ldr, float* __restrict__ out,
                                                       int64_t ldo) {
  __shared__ float sA[kBKf][kBM + 4];
  __shared__ float sB[kBKf][kBN + 4];
  const int tid = threadIdx.x;
  const int tx = tid & 15, ty = tid >> 4;
  const int m0 = blockIdx.y * kBM, n0 = blockIdx.x * kBN;

  float acc[4][4];
  for (int i = 0; i < 4; ++i)
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.0f;

  for (int k0 = 0; k0 < K; k0 += kBKf) {
    for (int r = 0; r < 4; ++r) {
      const int idx = tid + 256 * r;
      const int row = idx >> 4, kk = idx & 15;  // A: 64 rows x 16 k
      const int gm = m0 + row, gk = k0 + kk;
      sA[kk][row] = (gm < M && gk < K) ? A[static_cast<int64_t>(gm) * lda + gk] : 0.0f;
      const int kb = idx >> 6, col = idx & 63;  // B: 16 k x 64 cols
      const int gkb = k0 + kb, gn = n0 + col;
      sB[kb][col] = (gkb < K && gn < N) ? B[static_cast<int64_t>(gkb) * ldb + gn] : 0.0f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kBKf; ++kk) {
      float a[4], b[4];
      for (int i = 0; i < 4; ++i) a[i] = sA[kk][ty * 4 + i];
      for (int j = 0; j < 4; ++j) b[j] = sB[kk][tx * 4 + j];
      for (int i = 0; i < 4; ++i)
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }

  for (int i = 0; i < 4; ++i) {
    const int m = m0 + ty * 4 + i;
    if (m >= M) continue;
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + tx * 4 + j;
      if (n >= N) continue;
      float v = acc[i][j];
      if (bias != nullptr) v += bias[n];
      if (GELU) v = gelu_f32(v);
      if (residual != nullptr) v += residual[static_cast<int64_t>(m) * ldr + n];
      out[static_cast<int64_t>(m) * ldo + n] = v;
    }
  }
}

}  // namespace

hipError_t launch_gemm_f32(const float* A, int64_t lda, const float* B, int64_t ldb, int64_t M,
                           int64_t N, int64_t K, const Epilogue& ep, hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>((N + kBN - 1) / kBN),
                  static_cast<unsigned>((M + kBM - 1) / kBM));
  const float* bias = static_cast<const float*>(ep.bias);
  const float* res = static_cast<const float*>(ep.residual);
  float* out = static_cast<float*>(ep.out);
  if (ep.gelu)
    hipLaunchKernelGGL(gemm_f32_kernel<true>, grid, dim3(256), 0, stream, A, lda, B, ldb,
                       static_cast<int>(M), static_cast<int>(N), static_cast<int>(K), bias, res,
                       ep.ldr, out, ep.ldo);
  else
    hipLaunchKernelGGL(gemm_f32_kernel<false>, grid, dim3(256), 0, stream, A, lda, B, ldb,
                       static_cast<int>(M), static_cast<int>(N), static_cast<int>(K), bias, res,
                       ep.ldr, out, ep.ldo);
  return hipGetLastError();
}

}  // namespace tpk
