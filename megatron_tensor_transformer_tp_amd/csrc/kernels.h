// Internal launcher interface between the C-ABI front end (tp_shard_abi.cpp)
// and the gfx950 kernels.  Arguments are already validated when these run.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tpk {

// Epilogue kinds (compile-time in the kernels).
enum EpilogueKind : int {
  EPI_LINEAR = 0,    // v = acc + bias[n]; v += residual[m, n]
  EPI_GELU = 1,      // y = acc + bias[n]; pre[m, n] = y (if pre); v = GeLU(y)
  EPI_GELU_BWD = 2,  // y = aux[m, n]; v = acc * GeLU'(y); out2[m, n] = GeLU(y)
  EPI_SWIGLU = 3,    // gate and value columns of one feature: out = SiLU(g) * u
  EPI_QKV_F16 = 4,   // packed [q | k | v] projection: q, k columns as fp16(v * 2^-8),
                     // v columns as bf16 (128-column parts, bf16 out only)
};

// Scale of the fp16 Q and K columns written by EPI_QKV_F16 (their product
// carries kQkScale^2, removed again in the softmax scale).
constexpr float kQkScale = 1.0f / 256.0f;
constexpr int kQkvPart = 128;

// Epilogue applied to the fp32 accumulator of C = A B, element (m, n), then
//   out[m, n] = v                (fp32, or bf16 rounded to nearest-even)
// bias: input dtype or null; residual: input dtype, row stride ldr, or null
// (EPI_LINEAR only); pre and out2 share out's dtype and row stride ldo; aux
// is in the input dtype with row stride ldaux.
struct Epilogue {
  const void* bias;
  const void* residual;
  int64_t ldr;
  void* out;
  int64_t ldo;
  bool out_f32;
  int kind;
  void* pre = nullptr;
  const void* aux = nullptr;
  int64_t ldaux = 0;
  void* out2 = nullptr;
  const void* b2 = nullptr;   // EPI_SWIGLU: the value projection (B is the gate)
  // split-K (EPI_LINEAR, fp32 out, no bias or residual): ksplit workgroup
  // sets each take K / ksplit of the k range (K % (64 ksplit) == 0) and
  // write their partial product to out + s * slab (elements)
  int ksplit = 1;
  int64_t slab = 0;
};

// Compute units of the current device (cached per device; 256 on a whole
// MI355X).  The GEMM kernels size their grids by it.
int64_t device_cus();

// Split-K for products of few tiles (splitk.hip): at most kSplitKMaxRows
// rows, at most kSplitKMax k-slices.  splitk_factor: the slices for an
// M x N x K product on this device (1: do not split; a power of two whose
// tiles (64 x 128 up to 128 rows, 128 x 128 above) times slices fill at most
// the CUs, with K % (64 ks) == 0).
// launch_gemm_bf16_splitk: part[s][M][N] fp32 = A[:, kslice s] B[kslice s, :]
// (A [M, K] k-contiguous, B [K, N] k-major, as launch_gemm_bf16);
// launch_splitk_reduce: out = epilogue(sum over s of part[s]) in slice order,
// ep as for the unsplit product (EPI_GELU or EPI_LINEAR, bf16 bias and
// residual).
constexpr int64_t kSplitKMaxRows = 512;
constexpr int kSplitKMax = 8;
inline int64_t splitk_part_floats(int64_t rows, int64_t width) { return kSplitKMax * rows * width; }
int splitk_factor(int64_t M, int64_t N, int64_t K);
hipError_t launch_gemm_bf16_splitk(const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb,
                                   int64_t M, int64_t N, int64_t K, int ksplit, float* part,
                                   hipStream_t stream);
hipError_t launch_splitk_reduce(const float* part, int ksplit, int64_t M, int64_t N,
                                const Epilogue& ep, hipStream_t stream);

// bf16 x bf16 -> fp32 accumulate, MFMA.  A [M, K] row-major (lda), B [K, N]
// row-major (ldb).  Any M, N and K >= 1 with N % 8 == 0, K % 8 == 0,
// lda/ldb/ldr/ldo % 8 == 0 (ldo % 4 for fp32 out), 16-byte aligned pointers
// (else hipErrorInvalidValue where checked).  EPI_LINEAR / EPI_GELU /
// EPI_QKV_F16.
hipError_t launch_gemm_bf16(const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb,
                            int64_t M, int64_t N, int64_t K, const Epilogue& ep,
                            hipStream_t stream);

// The same product with either operand stored k-major or not:
//   a_kmajor: A given as [K, M] row-major (lda >= M), i.e. the product uses Aᵀ of it;
//   b_kmajor: B given as [K, N] row-major (the usual form); false: B given as
//             [N, K] row-major (ldb >= K).
// Any M, N and K >= 1 with the dimension that is contiguous in memory a
// multiple of 8 for each operand (K for a k-contiguous one, M or N for a
// k-major one), alignment as above.  Layout pairs and epilogues: (false,
// true) as launch_gemm_bf16; (false, false) EPI_LINEAR and bf16 EPI_GELU_BWD;
// (true, true) EPI_LINEAR (else hipErrorInvalidValue).
hipError_t launch_gemm_bf16_t(const uint16_t* A, int64_t lda, bool a_kmajor, const uint16_t* B,
                              int64_t ldb, bool b_kmajor, int64_t M, int64_t N, int64_t K,
                              const Epilogue& ep, hipStream_t stream);

// SwiGLU column layer: out[m, j] = SiLU((A Bg)[m, j]) * (A Bu)[m, j], j < F,
// A [M, K] row-major, Bg and Bu [K, F] row-major with the same ldb, out bf16
// [M, F] (ldo).  One product over both projections: any M, F % 8 == 0,
// K % 8 == 0, K >= 1 (else hipErrorInvalidValue).
hipError_t launch_gemm_bf16_swiglu(const uint16_t* A, int64_t lda, const uint16_t* Bg,
                                   const uint16_t* Bu, int64_t ldb, int64_t M, int64_t F,
                                   int64_t K, uint16_t* out, int64_t ldo, hipStream_t stream);

// fp32 SwiGLU combine: h[k] = SiLU(g[k]) * u[k], k < n.
hipError_t launch_swiglu_combine_f32(const float* g, const float* u, float* h, int64_t n,
                                     hipStream_t stream);

// fp32 x fp32 -> fp32 FMA, any shape.  Same layout flags as launch_gemm_bf16_t
// (a_kmajor: A given [K, M]; b_kmajor: B given [K, N], else [N, K]); every
// epilogue kind.
hipError_t launch_gemm_f32(const float* A, int64_t lda, bool a_kmajor, const float* B, int64_t ldb,
                           bool b_kmajor, int64_t M, int64_t N, int64_t K, const Epilogue& ep,
                           hipStream_t stream);

// Column sums out[n] = sum_m in[m, n] (fp32 accumulation, in fp32 or bf16 by
// in_dt 0/1, row stride ld), in two passes over 64-row chunks (deterministic):
// partial needs colsum_partial_floats(M, N) floats of scratch.  N and ld are
// multiples of 16 bytes' worth of elements, in 16-byte aligned (else
// hipErrorInvalidValue).
int64_t colsum_partial_floats(int64_t M, int64_t N);
hipError_t launch_colsum(const void* in, int64_t ld, int in_dt, int64_t M, int64_t N, float* out,
                         float* partial, hipStream_t stream);

// p[r, c] = 0 for r < rows, c < cols, row stride ld elements of elt_bytes
// (2 or 4) bytes: a kernel, not a memset, so that it may sit in a captured
// graph.
hipError_t launch_zero_2d(void* p, int64_t rows, int64_t cols, int64_t ld, int elt_bytes,
                          hipStream_t stream);

// Head-local attention: qkv [batch*seq, ld_qkv] holding the rank's packed
// projection as written by EPI_QKV_F16 (per head [q | k | v], head_dim
// columns each; q and k fp16 scaled by kQkScale, v bf16); o [batch*seq,
// ld_o] bf16, head j at columns j*head_dim.  head_dim == 128, seq >= 32.
// part (attn_part_floats floats) and arrivals (attn_arrival_ints ints), or
// null: scratch for causal grids whose rows are split over two workgroups.
hipError_t launch_attention(const uint16_t* qkv, int64_t ld_qkv, uint16_t* o, int64_t ld_o,
                            int batch, int seq, int heads, int head_dim, bool causal, float* part,
                            int* arrivals, hipStream_t stream);
inline int64_t attn_part_floats(int64_t tokens, int64_t heads) { return 2 * tokens * heads * 130; }
inline int64_t attn_arrival_ints(int64_t batch, int64_t seq, int64_t heads) {
  return batch * heads * ((seq + 127) / 128);
}

// Sequence-parallel reduce-scatter on one device: out[m, :] = sum_{j < t}
// parts.p[j][row0 + m, :] (+ bias) (+ residual[m, :]) for m < rows; partials
// fp32 [*, hidden] contiguous; bias / residual in in_dt, out in out_dt
// (0 = f32, 1 = bf16); hidden % 4 == 0, 16-byte aligned pointers.
constexpr int kSpMaxParts = 16;
struct SpPartials {
  const float* p[kSpMaxParts];
};
hipError_t launch_sp_reduce(const SpPartials& parts, int t, int64_t row0, int64_t rows,
                            int64_t hidden, const void* bias, const void* residual, int in_dt,
                            void* out, int out_dt, hipStream_t stream);

// out[k] = GeLU(in[k]), dtypes 0 = f32, 1 = bf16.
hipError_t launch_gelu(const void* in, void* out, int64_t n, int in_dt, int out_dt,
                       hipStream_t stream);

}  // namespace tpk
