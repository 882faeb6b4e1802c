// Split-K for products with few tiles (the MLP shard at small token
// counts): the bf16 GEMM kernel runs ksplit sets of workgroups, set s
// taking k-slice s of K / ksplit and writing its fp32 partial product to
// slab s (gemm_bf16_dma.h); this kernel then sums the slabs in slice order
// (so the result does not depend on scheduling) and applies the epilogue
// the unsplit product would have: EPI_GELU (bias, saved pre-activation,
// GeLU) or EPI_LINEAR (bias, residual), bf16 or fp32 out.
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "gemm_bf16_impl.h"
#include "kernels.h"

namespace tpk {
namespace {

typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ void load4_bf16(const uint16_t* p, float (&v)[4]) {
  const u32x2_t w = *reinterpret_cast<const u32x2_t*>(p);
  v[0] = __uint_as_float(w[0] << 16);
  v[1] = __uint_as_float(w[0] & 0xFFFF0000u);
  v[2] = __uint_as_float(w[1] << 16);
  v[3] = __uint_as_float(w[1] & 0xFFFF0000u);
}

__device__ __forceinline__ void store4(void* out, bool f32, int64_t off, const float (&v)[4]) {
  if (f32) {
    *reinterpret_cast<f32x4_t*>(static_cast<float*>(out) + off) = f32x4_t{v[0], v[1], v[2], v[3]};
  } else {
    *reinterpret_cast<u32x2_t*>(static_cast<uint16_t*>(out) + off) =
        u32x2_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
  }
}

// One thread per 4 consecutive columns of one row; KS slabs.
template <int EPI, int KS>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ part,
                                                             int64_t slab, int64_t M, int64_t N,
                                                             const Epilogue ep) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t qn = N / 4;
  if (i >= M * qn) return;
  const int64_t m = i / qn, n = (i - m * qn) * 4;
  const float* p = part + m * N + n;
  // Every slab's load is issued before the first add (one memory round
  // trip instead of one per slab); the sum runs in slice order.
  f32x4_t x[KS];
  static_for<KS>([&](auto S) { x[S] = *reinterpret_cast<const f32x4_t*>(p + S * slab); });
  f32x4_t acc = x[0];
  static_for<KS - 1>([&](auto S) { acc += x[S + 1]; });
  float v[4] = {acc[0], acc[1], acc[2], acc[3]};
  if (ep.bias != nullptr) {
    float b[4];
    load4_bf16(static_cast<const uint16_t*>(ep.bias) + n, b);
    static_for<4>([&](auto R) { v[R] += b[R]; });
  }
  const int64_t off = m * ep.ldo + n;
  if constexpr (EPI == EPI_GELU) {
    if (ep.pre != nullptr) store4(ep.pre, ep.out_f32, off, v);
    static_for<4>([&](auto R) { v[R] = gelu_f32(v[R]); });
  } else {
    if (ep.residual != nullptr) {
      float r[4];
      load4_bf16(static_cast<const uint16_t*>(ep.residual) + m * ep.ldr + n, r);
      static_for<4>([&](auto R) { v[R] += r[R]; });
    }
  }
  store4(ep.out, ep.out_f32, off, v);
}

}  // namespace

namespace {
// Rows of the split products' tiles: 64 x 128 up to 128 rows, 128 x 128 above.
int splitk_tile_rows(int64_t M) { return M <= 128 ? 64 : 128; }
}  // namespace

int splitk_factor(int64_t M, int64_t N, int64_t K) {
  if (M > kSplitKMaxRows) return 1;
  const int64_t bm = splitk_tile_rows(M);
  const int64_t tiles = ((M + bm - 1) / bm) * ((N + 127) / 128);
  const int64_t cus = device_cus();
  int ks = 1;
  while (ks < kSplitKMax && tiles * ks * 2 <= cus && K % (64 * ks * 2) == 0) ks *= 2;
  return ks;
}

hipError_t launch_gemm_bf16_splitk(const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb,
                                   int64_t M, int64_t N, int64_t K, int ksplit, float* part,
                                   hipStream_t stream) {
  Epilogue ep{nullptr, nullptr, 0, part, N, true, EPI_LINEAR};
  ep.ksplit = ksplit;
  ep.slab = M * N;
  if (splitk_tile_rows(M) == 128)
    return launch_gemm_bf16_cfg<128, 128, EPI_LINEAR, true>(A, lda, B, ldb, static_cast<int>(M),
                                                            static_cast<int>(N), static_cast<int>(K),
                                                            ep, stream);
  return launch_gemm_bf16_cfg<64, 128, EPI_LINEAR, true>(A, lda, B, ldb, static_cast<int>(M),
                                                         static_cast<int>(N), static_cast<int>(K), ep,
                                                         stream);
}

hipError_t launch_splitk_reduce(const float* part, int ksplit, int64_t M, int64_t N,
                                const Epilogue& ep, hipStream_t stream) {
  if (M == 0) return hipSuccess;
  if (N % 4 != 0 || (ep.kind != EPI_GELU && ep.kind != EPI_LINEAR)) return hipErrorInvalidValue;
  const int64_t threads = M * (N / 4);
  const dim3 grid(static_cast<unsigned>((threads + 255) / 256));
  auto launch = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, grid, dim3(256), 0, stream, part, M * N, M, N, ep);
    return hipGetLastError();
  };
  const bool gelu = ep.kind == EPI_GELU;
  switch (ksplit) {
    case 2: return gelu ? launch(splitk_reduce_kernel<EPI_GELU, 2>) : launch(splitk_reduce_kernel<EPI_LINEAR, 2>);
    case 4: return gelu ? launch(splitk_reduce_kernel<EPI_GELU, 4>) : launch(splitk_reduce_kernel<EPI_LINEAR, 4>);
    case 8: return gelu ? launch(splitk_reduce_kernel<EPI_GELU, 8>) : launch(splitk_reduce_kernel<EPI_LINEAR, 8>);
    default: return hipErrorInvalidValue;   // splitk_factor gives 2, 4 or 8 when it splits
  }
}

}  // namespace tpk
