// fp32 GEMM with fp32 FMA accumulation and the same fused epilogues as the
// bf16 path (bias, GeLU with optional pre-activation save, residual, GeLU
// backward).  This is the fp32 variant of the column- and row-parallel
// linears (列并行 tutorial, 数学基础 and MLP 应用) and of their backward
// products (Megatron expert interview Level 2, M025 and M026); no value is
// rounded below fp32 anywhere.
//
// A is [M, K] row-major, or [K, M] if a_kmajor; B is [K, N] row-major if
// b_kmajor, else [N, K].  T x T output tile per 256-thread workgroup
// (T = 64: each thread a 4 x 4 block; T = 32 for products with fewer than
// four 64 x 64 tiles per CU, each thread a 2 x 2 block, so that a CU holds
// enough waves to hide the load latency), BK = 16; both operand tiles
// staged in LDS k-major (sA[k][m], sB[k][n]) so the inner product reads are
// broadcast-friendly.  Edges are masked (zero-filled loads, predicated
// stores), so any M, N, K >= 1 works.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "device_common.h"
#include "kernels.h"

namespace tpk {
namespace {

constexpr int kBKf = 16;

template <int EPI, int T>
__global__ __launch_bounds__(256) void gemm_f32_kernel(const float* __restrict__ A, int64_t lda,
                                                       bool a_kmajor, const float* __restrict__ B,
                                                       int64_t ldb, bool b_kmajor, int M, int N,
                                                       int K, const Epilogue ep) {
  constexpr int R = T / 16;                 // rows (and columns) per thread
  __shared__ float sA[kBKf][T + 4];
  __shared__ float sB[kBKf][T + 4];
  const int tid = threadIdx.x;
  const int tx = tid & 15, ty = tid >> 4;
  const int m0 = blockIdx.x * T, n0 = blockIdx.y * T;   // M tiles on x: no 65535 limit

  float acc[R][R];
  for (int i = 0; i < R; ++i)
    for (int j = 0; j < R; ++j) acc[i][j] = 0.0f;

  for (int k0 = 0; k0 < K; k0 += kBKf) {
    for (int r = 0; r < R; ++r) {
      const int idx = tid + 256 * r;
      const int row = idx >> 4, kk = idx & 15;  // A: T rows x 16 k
      const int gm = m0 + row, gk = k0 + kk;
      sA[kk][row] = (gm < M && gk < K)
                        ? A[a_kmajor ? static_cast<int64_t>(gk) * lda + gm
                                     : static_cast<int64_t>(gm) * lda + gk]
                        : 0.0f;
      const int kb = idx / T, col = idx % T;    // B: 16 k x T cols
      const int gkb = k0 + kb, gn = n0 + col;
      sB[kb][col] = (gkb < K && gn < N)
                        ? B[b_kmajor ? static_cast<int64_t>(gkb) * ldb + gn
                                     : static_cast<int64_t>(gn) * ldb + gkb]
                        : 0.0f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kBKf; ++kk) {
      float a[R], b[R];
      for (int i = 0; i < R; ++i) a[i] = sA[kk][ty * R + i];
      for (int j = 0; j < R; ++j) b[j] = sB[kk][tx * R + j];
      for (int i = 0; i < R; ++i)
        for (int j = 0; j < R; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }

  const float* bias = static_cast<const float*>(ep.bias);
  const float* residual = static_cast<const float*>(ep.residual);
  const float* aux = static_cast<const float*>(ep.aux);
  float* out = static_cast<float*>(ep.out);
  float* pre = static_cast<float*>(ep.pre);
  float* out2 = static_cast<float*>(ep.out2);
  for (int i = 0; i < R; ++i) {
    const int m = m0 + ty * R + i;
    if (m >= M) continue;
    for (int j = 0; j < R; ++j) {
      const int n = n0 + tx * R + j;
      if (n >= N) continue;
      const int64_t o = static_cast<int64_t>(m) * ep.ldo + n;
      float v = acc[i][j];
      if constexpr (EPI == EPI_GELU_BWD) {
        const float y = aux[static_cast<int64_t>(m) * ep.ldaux + n];
        v *= gelu_grad_f32(y);
        out2[o] = gelu_f32(y);
      } else {
        if (bias != nullptr) v += bias[n];
        if constexpr (EPI == EPI_GELU) {
          if (pre != nullptr) pre[o] = v;
          v = gelu_f32(v);
        }
        if (residual != nullptr) v += residual[static_cast<int64_t>(m) * ep.ldr + n];
      }
      out[o] = v;
    }
  }
}

}  // namespace

hipError_t launch_gemm_f32(const float* A, int64_t lda, bool a_kmajor, const float* B, int64_t ldb,
                           bool b_kmajor, int64_t M, int64_t N, int64_t K, const Epilogue& ep,
                           hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  auto launch = [&](auto tile) {
    constexpr int T = decltype(tile)::value;
    const int64_t tiles_n = (N + T - 1) / T;
    if (tiles_n > 65535) return hipErrorInvalidValue;     // grid y limit
    const dim3 grid(static_cast<unsigned>((M + T - 1) / T), static_cast<unsigned>(tiles_n));
    const int m = static_cast<int>(M), n = static_cast<int>(N), k = static_cast<int>(K);
    switch (ep.kind) {
      case EPI_LINEAR:
        hipLaunchKernelGGL((gemm_f32_kernel<EPI_LINEAR, T>), grid, dim3(256), 0, stream, A, lda,
                           a_kmajor, B, ldb, b_kmajor, m, n, k, ep);
        break;
      case EPI_GELU:
        hipLaunchKernelGGL((gemm_f32_kernel<EPI_GELU, T>), grid, dim3(256), 0, stream, A, lda,
                           a_kmajor, B, ldb, b_kmajor, m, n, k, ep);
        break;
      case EPI_GELU_BWD:
        hipLaunchKernelGGL((gemm_f32_kernel<EPI_GELU_BWD, T>), grid, dim3(256), 0, stream, A, lda,
                           a_kmajor, B, ldb, b_kmajor, m, n, k, ep);
        break;
      default:
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
  };
  const int64_t tiles64 = ((M + 63) / 64) * ((N + 63) / 64);
  if (tiles64 < 4 * device_cus()) return launch(std::integral_constant<int, 32>{});
  return launch(std::integral_constant<int, 64>{});
}

}  // namespace tpk
