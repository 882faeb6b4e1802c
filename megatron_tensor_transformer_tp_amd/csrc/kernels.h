// Internal launcher interface between the C-ABI front end (tp_shard_abi.cpp)
// and the gfx950 kernels.  Arguments are already validated when these run.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tpk {

// Epilogue applied to the fp32 accumulator of C = A B, element (m, n):
//   v = acc + bias[n]            (bias: input dtype, or null)
//   v = GeLU(v)                  (if gelu)
//   v = v + residual[m, n]       (residual: input dtype, row stride ldr, or null)
//   out[m, n] = v                (fp32, or bf16 rounded to nearest-even)
struct Epilogue {
  const void* bias;
  const void* residual;
  int64_t ldr;
  void* out;
  int64_t ldo;
  bool out_f32;
  bool gelu;
};

// bf16 x bf16 -> fp32 accumulate, MFMA.  A [M, K] row-major (lda), B [K, N]
// row-major (ldb).  Requires N % 8 == 0, K % 8 == 0, lda/ldb/ldr/ldo % 8 == 0
// (ldo % 4 for fp32 out), 16-byte aligned pointers.
hipError_t launch_gemm_bf16(const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb,
                            int64_t M, int64_t N, int64_t K, const Epilogue& ep,
                            hipStream_t stream);

// fp32 x fp32 -> fp32 FMA.  Same layout rules with 4-element alignment.
hipError_t launch_gemm_f32(const float* A, int64_t lda, const float* B, int64_t ldb,
                           int64_t M, int64_t N, int64_t K, const Epilogue& ep,
                           hipStream_t stream);

// out[k] = GeLU(in[k]), dtypes 0 = f32, 1 = bf16.
hipError_t launch_gelu(const void* in, void* out, int64_t n, int in_dt, int out_dt,
                       hipStream_t stream);

}  // namespace tpk
