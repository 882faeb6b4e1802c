// Column sums out[n] = sum_m in[m, n] for the bias gradients of the MLP shard
// backward (the output-bias and first-layer-bias terms of the chain rule in
// Megatron expert interview Level 2, M025/M026: a bias added to every token
// row receives the sum of that row-wise gradient over tokens).
//
// HBM-bound (algorithmic bytes = M * N * element size + 4 N).  Two passes,
// no atomics, so the result is deterministic: pass 1 sums 64-row chunks into
// partial[chunk][n] (each thread owns 16 bytes of one row's columns, 8 bf16
// or 4 fp32, with eight rows' loads in flight per step; consecutive threads
// on consecutive column groups, so each wave reads a contiguous 1 KiB row
// segment); pass 2 adds the chunks in a fixed order (eight interleaved
// subsets per column, each with four running sums, then combined in order).
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "kernels.h"

namespace tpk {
namespace {

constexpr int kRows = 64;        // rows per pass-1 chunk
constexpr int kThreads = 256;
constexpr int kUnroll = 8;       // rows loaded per step

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// The 16 bytes at p as floats: 8 bf16 or 4 fp32 values.
template <typename T>
__device__ __forceinline__ void add_vec(const u32x4_t& w, float (&acc)[16 / sizeof(T)]) {
  if constexpr (sizeof(T) == 2) {
    static_for<4>([&](auto Q) __attribute__((always_inline)) {
      constexpr int q = Q;
      acc[2 * q] += __uint_as_float(w[q] << 16);
      acc[2 * q + 1] += __uint_as_float(w[q] & 0xFFFF0000u);
    });
  } else {
    static_for<4>([&](auto Q) __attribute__((always_inline)) {
      constexpr int q = Q;
      acc[q] += __uint_as_float(w[q]);
    });
  }
}

// Pass 1: partial[chunk][n] = sum over the chunk's rows of in[m, n].  Block
// (x = chunk, y = column block of kThreads * VEC columns); N % VEC == 0, ld %
// VEC == 0 and a 16-byte aligned base.
template <typename T>
__global__ __launch_bounds__(kThreads) void colsum_chunk_kernel(const T* __restrict__ in, int64_t ld,
                                                                int M, int N,
                                                                float* __restrict__ partial) {
  constexpr int VEC = 16 / sizeof(T);
  const int c0 = (blockIdx.y * kThreads + threadIdx.x) * VEC;
  if (c0 >= N) return;
  const int r0 = blockIdx.x * kRows;
  const int r1 = min(M, r0 + kRows);
  float acc[VEC];
  static_for<VEC>([&](auto V) __attribute__((always_inline)) { acc[V] = 0.0f; });
  const T* base = in + c0;
  int r = r0;
  for (; r + kUnroll <= r1; r += kUnroll) {
    u32x4_t w[kUnroll];
    static_for<kUnroll>([&](auto U) __attribute__((always_inline)) {
      w[U] = *reinterpret_cast<const u32x4_t*>(base + static_cast<int64_t>(r + U) * ld);
    });
    static_for<kUnroll>([&](auto U) __attribute__((always_inline)) { add_vec<T>(w[U], acc); });
  }
  for (; r < r1; ++r) add_vec<T>(*reinterpret_cast<const u32x4_t*>(base + static_cast<int64_t>(r) * ld), acc);
  float* dst = partial + static_cast<int64_t>(blockIdx.x) * N + c0;
  static_for<VEC / 4>([&](auto Q) __attribute__((always_inline)) {
    typedef float f32x4_t __attribute__((ext_vector_type(4)));
    *reinterpret_cast<f32x4_t*>(dst + 4 * Q) =
        f32x4_t{acc[4 * Q], acc[4 * Q + 1], acc[4 * Q + 2], acc[4 * Q + 3]};
  });
}

// Pass 2: out[n] = sum over chunks of partial[chunk][n]; 32 columns per
// block, eight threads per column each summing an interleaved chunk subset
// with four independent running sums, combined in a fixed order through LDS.
constexpr int kFinCols = 32, kFinGroups = kThreads / kFinCols;
__global__ __launch_bounds__(kThreads) void colsum_finish_kernel(const float* __restrict__ partial,
                                                                 int chunks, int N,
                                                                 float* __restrict__ out) {
  __shared__ float red[kFinGroups][kFinCols];
  const int col = threadIdx.x % kFinCols, g = threadIdx.x / kFinCols;
  const int n = blockIdx.x * kFinCols + col;
  float s[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  if (n < N) {
    int c = g;
    for (; c + 3 * kFinGroups < chunks; c += 4 * kFinGroups) {
      static_for<4>([&](auto U) __attribute__((always_inline)) {
        s[U] += partial[static_cast<int64_t>(c + U * kFinGroups) * N + n];
      });
    }
    for (; c < chunks; c += kFinGroups) s[0] += partial[static_cast<int64_t>(c) * N + n];
  }
  red[g][col] = (s[0] + s[1]) + (s[2] + s[3]);
  __syncthreads();
  if (g == 0 && n < N) {
    float t = 0.0f;
    static_for<kFinGroups>([&](auto G) __attribute__((always_inline)) { t += red[G][col]; });
    out[n] = t;
  }
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
  const int vec = in_dt == 1 ? 8 : 4;                  // columns per thread (16 bytes)
  if (N % vec != 0 || ld % vec != 0 || (reinterpret_cast<uintptr_t>(in) & 15) != 0)
    return hipErrorInvalidValue;
  const int64_t chunks = (M + kRows - 1) / kRows;
  const int64_t col_blocks = (N / vec + kThreads - 1) / kThreads;
  if (col_blocks > 65535 || chunks > INT32_MAX) return hipErrorInvalidValue;   // grid limits
  if (chunks > 0) {
    // row chunks on x (no 65535 limit), column blocks on y
    const dim3 grid(static_cast<unsigned>(chunks), static_cast<unsigned>(col_blocks));
    if (in_dt == 1)
      hipLaunchKernelGGL(colsum_chunk_kernel<uint16_t>, grid, dim3(kThreads), 0, stream,
                         static_cast<const uint16_t*>(in), ld, static_cast<int>(M),
                         static_cast<int>(N), partial);
    else
      hipLaunchKernelGGL(colsum_chunk_kernel<float>, grid, dim3(kThreads), 0, stream,
                         static_cast<const float*>(in), ld, static_cast<int>(M),
                         static_cast<int>(N), partial);
  }
  hipLaunchKernelGGL(colsum_finish_kernel, dim3(static_cast<unsigned>((N + kFinCols - 1) / kFinCols)), dim3(kThreads),
                     0, stream, partial, static_cast<int>(chunks), static_cast<int>(N), out);
  return hipGetLastError();
}

}  // namespace tpk
