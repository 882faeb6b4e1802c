// Column sums out[n] = sum_m in[m, n] for the bias gradients of the MLP shard
// backward (the output-bias and first-layer-bias terms of the chain rule in
// Megatron expert interview Level 2, M025/M026: a bias added to every token
// row receives the sum of that row-wise gradient over tokens).
//
// HBM-bound (algorithmic bytes = M * N * element size + 4 N).  Two passes,
// no atomics, so the result is deterministic: pass 1 sums 256-row chunks
// (thread = column, consecutive threads on consecutive columns, so each wave
// reads contiguous row segments) into partial[chunk][n]; pass 2 adds the
// chunks in order.
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "kernels.h"

namespace tpk {
namespace {

constexpr int kRows = 256;
constexpr int kCols = 256;

template <typename T>
__device__ __forceinline__ float load_f(const T* p);
template <>
__device__ __forceinline__ float load_f<float>(const float* p) { return *p; }
template <>
__device__ __forceinline__ float load_f<uint16_t>(const uint16_t* p) { return bf16_to_f32(*p); }

template <typename T>
__global__ __launch_bounds__(kCols) void colsum_chunk_kernel(const T* __restrict__ in, int64_t ld,
                                                            int M, int N,
                                                            float* __restrict__ partial) {
  const int n = blockIdx.y * kCols + threadIdx.x;
  if (n >= N) return;
  const int r0 = blockIdx.x * kRows;
  const int r1 = min(M, r0 + kRows);
  float s = 0.0f;
  for (int r = r0; r < r1; ++r) s += load_f(in + static_cast<int64_t>(r) * ld + n);
  partial[static_cast<int64_t>(blockIdx.x) * N + n] = s;
}

__global__ __launch_bounds__(kCols) void colsum_finish_kernel(const float* __restrict__ partial,
                                                             int chunks, int N,
                                                             float* __restrict__ out) {
  const int n = blockIdx.x * kCols + threadIdx.x;
  if (n >= N) return;
  float s = 0.0f;
  for (int c = 0; c < chunks; ++c) s += partial[static_cast<int64_t>(c) * N + n];
  out[n] = s;
}

template <typename T>
__global__ __launch_bounds__(256) void zero_2d_kernel(T* __restrict__ p, int64_t rows, int cols,
                                                     int64_t ld) {
  const int64_t total = rows * cols;
  for (int64_t i = blockIdx.x * 256ll + threadIdx.x; i < total; i += 256ll * gridDim.x)
    p[(i / cols) * ld + i % cols] = T(0);
}

}  // namespace

hipError_t launch_zero_2d(void* p, int64_t rows, int64_t cols, int64_t ld, int elt_bytes,
                          hipStream_t stream) {
  if (rows == 0 || cols == 0) return hipSuccess;
  const int64_t total = rows * cols;
  const int64_t want = (total + 255) / 256;
  const unsigned blocks = static_cast<unsigned>(want < 4096 ? want : 4096);
  if (elt_bytes == 2)
    hipLaunchKernelGGL(zero_2d_kernel<uint16_t>, dim3(blocks), dim3(256), 0, stream,
                       static_cast<uint16_t*>(p), rows, static_cast<int>(cols), ld);
  else
    hipLaunchKernelGGL(zero_2d_kernel<float>, dim3(blocks), dim3(256), 0, stream,
                       static_cast<float*>(p), rows, static_cast<int>(cols), ld);
  return hipGetLastError();
}

int64_t colsum_partial_floats(int64_t M, int64_t N) { return ((M + kRows - 1) / kRows) * N; }

hipError_t launch_colsum(const void* in, int64_t ld, int in_dt, int64_t M, int64_t N, float* out,
                         float* partial, hipStream_t stream) {
  if (N == 0) return hipSuccess;
  const int chunks = static_cast<int>((M + kRows - 1) / kRows);
  const unsigned col_blocks = static_cast<unsigned>((N + kCols - 1) / kCols);
  if (col_blocks > 65535) return hipErrorInvalidValue;   // grid y limit
  if (chunks > 0) {
    // row chunks on x (no 65535 limit), column blocks on y
    const dim3 grid(static_cast<unsigned>(chunks), col_blocks);
    if (in_dt == 1)
      hipLaunchKernelGGL(colsum_chunk_kernel<uint16_t>, grid, dim3(kCols), 0, stream,
                         static_cast<const uint16_t*>(in), ld, static_cast<int>(M),
                         static_cast<int>(N), partial);
    else
      hipLaunchKernelGGL(colsum_chunk_kernel<float>, grid, dim3(kCols), 0, stream,
                         static_cast<const float*>(in), ld, static_cast<int>(M),
                         static_cast<int>(N), partial);
  }
  hipLaunchKernelGGL(colsum_finish_kernel, dim3(col_blocks), dim3(kCols), 0, stream, partial,
                     chunks, static_cast<int>(N), out);
  return hipGetLastError();
}

}  // namespace tpk
