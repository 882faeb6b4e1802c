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
//   out_lo[m, n] = v - out[m, n] (bf16 out only, if out_lo is set: v as the
//                                 pair hi + lo, ~16 significant bits)
struct Epilogue {
  const void* bias;
  const void* residual;
  int64_t ldr;
  void* out;
  int64_t ldo;
  bool out_f32;
  bool gelu;
  void* out_lo = nullptr;
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

// Head-local attention: qkv_hi/qkv_lo [batch*seq, ld_qkv] bf16 pair holding
// the rank's packed projection (per head [q | k | v], head_dim columns each);
// o [batch*seq, ld_o] bf16, head j at columns j*head_dim.  head_dim == 128,
// seq % 128 == 0.
hipError_t launch_attention(const uint16_t* qkv_hi, const uint16_t* qkv_lo, int64_t ld_qkv,
                            uint16_t* o, int64_t ld_o, int batch, int seq, int heads,
                            int head_dim, bool causal, hipStream_t stream);

// out[k] = GeLU(in[k]), dtypes 0 = f32, 1 = bf16.
hipError_t launch_gelu(const void* in, void* out, int64_t n, int in_dt, int out_dt,
                       hipStream_t stream);

}  // namespace tpk
