// Standalone elementwise GeLU, out = in * Phi(in) (列并行 tutorial, MLP 应用):
// the unfused form of the activation between the column- and row-parallel
// layers.  HBM-bound: each element is read once and written once.  Threads
// handle 8 consecutive elements with vector loads/stores (16 B of bf16 or
// 2 x 16 B of fp32); a scalar loop covers the tail.  The grid is sized to a
// few waves of workgroups per CU and strides over the array.
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "kernels.h"

namespace tpk {
namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

template <typename T>
struct Io;

template <>
struct Io<float> {
  static __device__ __forceinline__ void load8(const float* p, float v[8]) {
    const f32x4_t a = *reinterpret_cast<const f32x4_t*>(p);
    const f32x4_t b = *reinterpret_cast<const f32x4_t*>(p + 4);
    for (int i = 0; i < 4; ++i) { v[i] = a[i]; v[4 + i] = b[i]; }
  }
  static __device__ __forceinline__ void store8(float* p, const float v[8]) {
    *reinterpret_cast<f32x4_t*>(p) = f32x4_t{v[0], v[1], v[2], v[3]};
    *reinterpret_cast<f32x4_t*>(p + 4) = f32x4_t{v[4], v[5], v[6], v[7]};
  }
  static __device__ __forceinline__ float load1(const float* p) { return *p; }
  static __device__ __forceinline__ void store1(float* p, float v) { *p = v; }
};

template <>
struct Io<uint16_t> {
  static __device__ __forceinline__ void load8(const uint16_t* p, float v[8]) {
    const u32x4_t a = *reinterpret_cast<const u32x4_t*>(p);
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(a[i] << 16);
      v[2 * i + 1] = __uint_as_float(a[i] & 0xFFFF0000u);
    }
  }
  static __device__ __forceinline__ void store8(uint16_t* p, const float v[8]) {
    *reinterpret_cast<u32x4_t*>(p) = u32x4_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                                             pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7])};
  }
  static __device__ __forceinline__ float load1(const uint16_t* p) { return bf16_to_f32(*p); }
  static __device__ __forceinline__ void store1(uint16_t* p, float v) { *p = f32_to_bf16(v); }
};

template <typename InT, typename OutT>
__global__ __launch_bounds__(256) void gelu_kernel(const InT* in, OutT* out, int64_t n) {
  const int64_t nvec = n / 8;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t v = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; v < nvec;
       v += stride) {
    float x[8];
    Io<InT>::load8(in + v * 8, x);
    for (int i = 0; i < 8; ++i) x[i] = gelu_f32(x[i]);
    Io<OutT>::store8(out + v * 8, x);
  }
  if (blockIdx.x == 0) {
    for (int64_t k = nvec * 8 + threadIdx.x; k < n; k += blockDim.x)
      Io<OutT>::store1(out + k, gelu_f32(Io<InT>::load1(in + k)));
  }
}

template <typename InT, typename OutT>
hipError_t launch_typed(const void* in, void* out, int64_t n, hipStream_t stream) {
  const int64_t nvec = n / 8;
  int64_t blocks = (nvec + 255) / 256;
  if (blocks > 256 * 16) blocks = 256 * 16;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL((gelu_kernel<InT, OutT>), dim3(static_cast<unsigned>(blocks)), dim3(256), 0,
                     stream, static_cast<const InT*>(in), static_cast<OutT*>(out), n);
  return hipGetLastError();
}

// fp32 SwiGLU combine for the fp32 path (the bf16 path fuses it into the
// GEMM epilogue): h = SiLU(g) * u, grid-stride, one element per step.
__global__ __launch_bounds__(256) void swiglu_combine_kernel(const float* __restrict__ g,
                                                             const float* __restrict__ u,
                                                             float* __restrict__ h, int64_t n) {
  for (int64_t k = blockIdx.x * 256ll + threadIdx.x; k < n; k += 256ll * gridDim.x)
    h[k] = silu_f32(g[k]) * u[k];
}

}  // namespace

hipError_t launch_swiglu_combine_f32(const float* g, const float* u, float* h, int64_t n,
                                     hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const int64_t want = (n + 255) / 256;
  hipLaunchKernelGGL(swiglu_combine_kernel, dim3(static_cast<unsigned>(want < 4096 ? want : 4096)),
                     dim3(256), 0, stream, g, u, h, n);
  return hipGetLastError();
}

hipError_t launch_gelu(const void* in, void* out, int64_t n, int in_dt, int out_dt,
                       hipStream_t stream) {
  if (n == 0) return hipSuccess;
  if (in_dt == 0 && out_dt == 0) return launch_typed<float, float>(in, out, n, stream);
  if (in_dt == 0 && out_dt == 1) return launch_typed<float, uint16_t>(in, out, n, stream);
  if (in_dt == 1 && out_dt == 0) return launch_typed<uint16_t, float>(in, out, n, stream);
  return launch_typed<uint16_t, uint16_t>(in, out, n, stream);
}

}  // namespace tpk
