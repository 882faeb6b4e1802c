// C-ABI front end: argument validation and kernel dispatch for the
// tensor-parallel shard entry points declared in include/tp_shard.h.
//
// Every check runs before anything is enqueued, and no check touches the HIP
// runtime, so the error paths work (and are tested) on a machine with no GPU.
// The shard width is derived here from the logical ffn (or heads) and t,
// rejecting splits that do not divide (列并行 tutorial, 切分原理; Megatron
// expert interview Level 2, M031).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <climits>

#include "../../include/tp_shard.h"
#include "abi_internal.h"
#include "kernels.h"

namespace {

constexpr int kVersion = 100;  // 0.1.0

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool dtype_known(int dt) { return dt == TP_F32 || dt == TP_BF16; }

int64_t elem_bytes(tp_dtype dt) { return dt == TP_BF16 ? 2 : 4; }

// Row widths / leading dimensions must be a multiple of this many elements so
// that every 16-byte vector access stays inside one row and aligned.
int64_t elem_align(tp_dtype dt) { return dt == TP_BF16 ? 8 : 4; }

// bf16 -> bf16, bf16 -> f32 and f32 -> f32 are the GEMM pairs.
bool gemm_pair_ok(int in_dt, int out_dt) {
  return (in_dt == TP_BF16 && (out_dt == TP_BF16 || out_dt == TP_F32)) ||
         (in_dt == TP_F32 && out_dt == TP_F32);
}

tp_status check_split(int64_t split, int t, int rank, int64_t* width) {
  if (t < 1 || rank < 0 || rank >= t) return TP_ERR_BAD_RANK;
  if (split < 1) return TP_ERR_INVALID_ARG;
  if (split % t != 0) return TP_ERR_NOT_DIVISIBLE;
  *width = split / t;
  return TP_OK;
}

// A required row-major operand of `width` elements per row.
tp_status check_matrix(const void* p, int64_t ld, int64_t width, tp_dtype dt) {
  if (p == nullptr) return TP_ERR_INVALID_ARG;
  if (ld < width) return TP_ERR_INVALID_ARG;
  if (!aligned16(p) || ld % elem_align(dt) != 0 || width % elem_align(dt) != 0)
    return TP_ERR_MISALIGNED;
  return TP_OK;
}

tp_status check_optional_vec(const void* p) {
  if (p != nullptr && !aligned16(p)) return TP_ERR_MISALIGNED;
  return TP_OK;
}

// Dimensions are handled as 32-bit ints inside the kernels, with room for a
// tile's worth of index arithmetic past the end.
bool fits_int32(int64_t v) { return v <= (int64_t{1} << 30); }

tp_status from_hip(hipError_t e) { return e == hipSuccess ? TP_OK : TP_ERR_HIP; }

#define TP_TRY(expr)                  \
  do {                                \
    const tp_status s_ = (expr);      \
    if (s_ != TP_OK) return s_;       \
  } while (0)

// Launch C[M, N] = A[M, K] B[K, N] with the given epilogue in dtype `in_dt`.
tp_status run_gemm(tp_dtype in_dt, const void* a, int64_t lda, const void* b, int64_t ldb,
                   int64_t M, int64_t N, int64_t K, const tpk::Epilogue& ep, hipStream_t stream) {
  if (in_dt == TP_BF16)
    return from_hip(tpk::launch_gemm_bf16(static_cast<const uint16_t*>(a), lda,
                                          static_cast<const uint16_t*>(b), ldb, M, N, K, ep,
                                          stream));
  return from_hip(tpk::launch_gemm_f32(static_cast<const float*>(a), lda, false,
                                       static_cast<const float*>(b), ldb, true, M, N, K, ep,
                                       stream));
}

// The same with k-major flags (A given [K, M] if a_kmajor; B given [K, N] if
// b_kmajor, else [N, K]).
tp_status run_gemm_t(tp_dtype in_dt, const void* a, int64_t lda, bool a_kmajor, const void* b,
                     int64_t ldb, bool b_kmajor, int64_t M, int64_t N, int64_t K,
                     const tpk::Epilogue& ep, hipStream_t stream) {
  if (in_dt == TP_BF16)
    return from_hip(tpk::launch_gemm_bf16_t(static_cast<const uint16_t*>(a), lda, a_kmajor,
                                            static_cast<const uint16_t*>(b), ldb, b_kmajor, M, N,
                                            K, ep, stream));
  return from_hip(tpk::launch_gemm_f32(static_cast<const float*>(a), lda, a_kmajor,
                                       static_cast<const float*>(b), ldb, b_kmajor, M, N, K, ep,
                                       stream));
}

size_t round256(size_t v) { return (v + 255) & ~static_cast<size_t>(255); }

}  // namespace

namespace tpabi {

tp_status mlp_fwd_validate(const void* x, const void* a_i, int64_t lda, const void* b_i,
                           const void* bias_a_i, const void* bias_b, const void* residual,
                           const void* z_i, const void* y_save, int64_t tokens, int64_t hidden,
                           int64_t ffn, int t, int rank, tp_dtype in_dt, tp_dtype out_dt,
                           int64_t* f_out) {
  if (!dtype_known(in_dt) || !dtype_known(out_dt) || !gemm_pair_ok(in_dt, out_dt))
    return TP_ERR_DTYPE;
  if (tokens < 0 || hidden < 1) return TP_ERR_INVALID_ARG;
  int64_t f = 0;
  TP_TRY(check_split(ffn, t, rank, &f));
  if (!fits_int32(tokens) || !fits_int32(hidden) || !fits_int32(f)) return TP_ERR_UNSUPPORTED;
  *f_out = f;
  if (tokens == 0) return TP_OK;
  TP_TRY(check_matrix(x, hidden, hidden, in_dt));
  TP_TRY(check_matrix(a_i, lda, f, in_dt));
  TP_TRY(check_matrix(b_i, hidden, hidden, in_dt));
  TP_TRY(check_matrix(z_i, hidden, hidden, out_dt));
  if (y_save != nullptr) TP_TRY(check_matrix(y_save, f, f, in_dt));
  TP_TRY(check_optional_vec(bias_a_i));
  const bool owner = rank == 0;
  TP_TRY(check_optional_vec(owner ? bias_b : nullptr));
  TP_TRY(check_optional_vec(owner ? residual : nullptr));
  return TP_OK;
}

tp_status mlp_fwd_enqueue(const void* x, const void* a_i, int64_t lda, const void* b_i,
                          const void* bias_a_i, const void* bias_use, const void* res_use,
                          void* z_i, void* y_save, void* h, float* part, int64_t tokens,
                          int64_t hidden, int64_t f, tp_dtype in_dt, tp_dtype out_dt, hipStream_t s) {
  // Few tokens: each product has few tiles and most CUs would sit idle
  // while it streams its weights, so its k range is split (fp32 partial
  // products in `part`, summed in slice order by a kernel that applies the
  // epilogue; the part buffer serves the two products one after the other).
  const int ks1 = in_dt == TP_BF16 && part != nullptr ? tpk::splitk_factor(tokens, f, hidden) : 1;
  const int ks2 = in_dt == TP_BF16 && part != nullptr ? tpk::splitk_factor(tokens, hidden, f) : 1;
  // Column-parallel GEMM with GeLU fused into its epilogue: H_i = GeLU(X A_i + a_i)
  // stored once in h (bf16 for bf16 inputs, fp32 for fp32); the
  // pre-activation also goes to y_save when asked for.
  tpk::Epilogue ep1{bias_a_i, nullptr, 0, h, f, in_dt == TP_F32, tpk::EPI_GELU};
  ep1.pre = y_save;
  if (ks1 > 1) {
    TP_TRY(from_hip(tpk::launch_gemm_bf16_splitk(static_cast<const uint16_t*>(x), hidden,
                                                 static_cast<const uint16_t*>(a_i), lda, tokens, f,
                                                 hidden, ks1, part, s)));
    TP_TRY(from_hip(tpk::launch_splitk_reduce(part, ks1, tokens, f, ep1, s)));
  } else {
    TP_TRY(run_gemm(in_dt, x, hidden, a_i, lda, tokens, f, hidden, ep1, s));
  }
  // Row-parallel GEMM: Z_i = H_i B_i (+ b + R on rank 0).
  tpk::Epilogue ep2{bias_use, res_use, hidden, z_i, hidden, out_dt == TP_F32, tpk::EPI_LINEAR};
  if (ks2 > 1) {
    TP_TRY(from_hip(tpk::launch_gemm_bf16_splitk(static_cast<const uint16_t*>(h), f,
                                                 static_cast<const uint16_t*>(b_i), hidden, tokens,
                                                 hidden, f, ks2, part, s)));
    return from_hip(tpk::launch_splitk_reduce(part, ks2, tokens, hidden, ep2, s));
  }
  return run_gemm(in_dt, h, f, b_i, hidden, tokens, hidden, f, ep2, s);
}

}  // namespace tpabi

extern "C" {

const char* tp_status_string(tp_status s) {
  switch (s) {
    case TP_OK: return "TP_OK";
    case TP_ERR_INVALID_ARG: return "TP_ERR_INVALID_ARG: null pointer, negative size or ld < width";
    case TP_ERR_NOT_DIVISIBLE: return "TP_ERR_NOT_DIVISIBLE: split dimension not divisible by t";
    case TP_ERR_BAD_RANK: return "TP_ERR_BAD_RANK: t < 1 or rank outside [0, t)";
    case TP_ERR_DTYPE: return "TP_ERR_DTYPE: unsupported dtype combination";
    case TP_ERR_MISALIGNED: return "TP_ERR_MISALIGNED: pointer, width or leading dimension misaligned";
    case TP_ERR_WORKSPACE: return "TP_ERR_WORKSPACE: workspace missing or too small";
    case TP_ERR_UNSUPPORTED: return "TP_ERR_UNSUPPORTED: request outside what the kernels implement";
    case TP_ERR_HIP: return "TP_ERR_HIP: a HIP launch failed";
  }
  return "TP_ERR_UNKNOWN";
}

int tp_version(void) { return kVersion; }

tp_status tp_column_linear(const void* x, int64_t ldx, const void* a_i, int64_t lda,
                           const void* bias_i, void* y_i, int64_t ldy, int64_t tokens,
                           int64_t hidden, int64_t ffn, int t, int rank, tp_dtype in_dt,
                           tp_dtype out_dt, int apply_gelu, void* stream) {
  if (!dtype_known(in_dt) || !dtype_known(out_dt) || !gemm_pair_ok(in_dt, out_dt))
    return TP_ERR_DTYPE;
  if (tokens < 0 || hidden < 1 || (apply_gelu != 0 && apply_gelu != 1)) return TP_ERR_INVALID_ARG;
  int64_t f = 0;
  TP_TRY(check_split(ffn, t, rank, &f));
  if (!fits_int32(tokens) || !fits_int32(hidden) || !fits_int32(f)) return TP_ERR_UNSUPPORTED;
  if (tokens == 0) return TP_OK;
  TP_TRY(check_matrix(x, ldx, hidden, in_dt));
  TP_TRY(check_matrix(a_i, lda, f, in_dt));
  TP_TRY(check_matrix(y_i, ldy, f, out_dt));
  TP_TRY(check_optional_vec(bias_i));
  tpk::Epilogue ep{bias_i, nullptr, 0, y_i, ldy, out_dt == TP_F32,
                   apply_gelu == 1 ? tpk::EPI_GELU : tpk::EPI_LINEAR};
  return run_gemm(in_dt, x, ldx, a_i, lda, tokens, f, hidden, ep,
                  static_cast<hipStream_t>(stream));
}

tp_status tp_gelu(const void* in, void* out, int64_t n, tp_dtype in_dt, tp_dtype out_dt,
                  void* stream) {
  if (!dtype_known(in_dt) || !dtype_known(out_dt)) return TP_ERR_DTYPE;
  if (n < 0) return TP_ERR_INVALID_ARG;
  if (n == 0) return TP_OK;
  if (in == nullptr || out == nullptr) return TP_ERR_INVALID_ARG;
  if (!aligned16(in) || !aligned16(out)) return TP_ERR_MISALIGNED;
  // exact aliasing is allowed when the element sizes match; partial overlap is not
  const uintptr_t ib = reinterpret_cast<uintptr_t>(in), ob = reinterpret_cast<uintptr_t>(out);
  const uintptr_t ie = ib + static_cast<uintptr_t>(n) * elem_bytes(in_dt);
  const uintptr_t oe = ob + static_cast<uintptr_t>(n) * elem_bytes(out_dt);
  const bool overlap = ib < oe && ob < ie;
  if (overlap && !(ib == ob && in_dt == out_dt)) return TP_ERR_INVALID_ARG;
  return from_hip(tpk::launch_gelu(in, out, n, in_dt, out_dt, static_cast<hipStream_t>(stream)));
}

tp_status tp_row_linear(const void* h_i, int64_t ldh, const void* b_i, int64_t ldb,
                        const void* bias, const void* residual, int64_t ldr, void* z_i,
                        int64_t ldz, int64_t tokens, int64_t ffn, int64_t hidden, int t,
                        int rank, tp_dtype in_dt, tp_dtype out_dt, void* stream) {
  if (!dtype_known(in_dt) || !dtype_known(out_dt) || !gemm_pair_ok(in_dt, out_dt))
    return TP_ERR_DTYPE;
  if (tokens < 0 || hidden < 1) return TP_ERR_INVALID_ARG;
  int64_t f = 0;
  TP_TRY(check_split(ffn, t, rank, &f));
  if (!fits_int32(tokens) || !fits_int32(hidden) || !fits_int32(f)) return TP_ERR_UNSUPPORTED;
  if (tokens == 0) return TP_OK;
  TP_TRY(check_matrix(h_i, ldh, f, in_dt));
  TP_TRY(check_matrix(b_i, ldb, hidden, in_dt));
  TP_TRY(check_matrix(z_i, ldz, hidden, out_dt));
  const bool owner = rank == 0;  // bias and residual belong to the summed output
  const void* bias_use = owner ? bias : nullptr;
  const void* res_use = owner ? residual : nullptr;
  TP_TRY(check_optional_vec(bias_use));
  if (res_use != nullptr) TP_TRY(check_matrix(res_use, ldr, hidden, in_dt));
  tpk::Epilogue ep{bias_use, res_use, ldr, z_i, ldz, out_dt == TP_F32, tpk::EPI_LINEAR};
  return run_gemm(in_dt, h_i, ldh, b_i, ldb, tokens, hidden, f, ep,
                  static_cast<hipStream_t>(stream));
}

namespace {
// Workspace of tp_mlp_shard_fwd: H_i [tokens, f] (in_dt), then, for bf16
// calls of at most kSplitKMaxRows tokens, the split-K partial products.
struct MlpFwdWorkspace {
  size_t h_bytes, part_bytes, total;
};
MlpFwdWorkspace mlp_fwd_workspace(int64_t tokens, int64_t hidden, int64_t f, tp_dtype in_dt) {
  const size_t hb = round256(static_cast<size_t>(tokens) * static_cast<size_t>(f) *
                             static_cast<size_t>(elem_bytes(in_dt)));
  const bool split = in_dt == TP_BF16 && tokens > 0 && tokens <= tpk::kSplitKMaxRows;
  const size_t pb = split ? round256(static_cast<size_t>(tpk::splitk_part_floats(
                                         tokens, f > hidden ? f : hidden)) * 4)
                          : 0;
  return {hb, pb, hb + pb};
}
}  // namespace

size_t tp_mlp_shard_workspace_bytes(int64_t tokens, int64_t hidden, int64_t ffn, int t,
                                    tp_dtype in_dt) {
  if (!dtype_known(in_dt) || tokens < 0 || hidden < 1) return 0;
  int64_t f = 0;
  if (check_split(ffn, t, 0, &f) != TP_OK) return 0;
  return mlp_fwd_workspace(tokens, hidden, f, in_dt).total;
}

tp_status tp_mlp_shard_fwd(const void* x, const void* a_i, int64_t lda, const void* b_i,
                           const void* bias_a_i, const void* bias_b, const void* residual,
                           void* z_i, void* y_save, void* workspace, size_t workspace_bytes,
                           int64_t tokens,
                           int64_t hidden, int64_t ffn, int t, int rank, tp_dtype in_dt,
                           tp_dtype out_dt, void* stream) {
  int64_t f = 0;
  TP_TRY(tpabi::mlp_fwd_validate(x, a_i, lda, b_i, bias_a_i, bias_b, residual, z_i, y_save, tokens,
                                 hidden, ffn, t, rank, in_dt, out_dt, &f));
  if (tokens == 0) return TP_OK;
  const MlpFwdWorkspace ws = mlp_fwd_workspace(tokens, hidden, f, in_dt);
  if (workspace == nullptr || workspace_bytes < ws.total) return TP_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return TP_ERR_MISALIGNED;
  float* part = ws.part_bytes
                    ? reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + ws.h_bytes)
                    : nullptr;
  return tpabi::mlp_fwd_enqueue(x, a_i, lda, b_i, bias_a_i, rank == 0 ? bias_b : nullptr,
                                rank == 0 ? residual : nullptr, z_i, y_save, workspace, part,
                                tokens, hidden, f, in_dt, out_dt, static_cast<hipStream_t>(stream));
}


size_t tp_mlp_swiglu_shard_workspace_bytes(int64_t tokens, int64_t hidden, int64_t ffn, int t,
                                           tp_dtype in_dt) {
  if (!dtype_known(in_dt) || tokens < 0 || hidden < 1) return 0;
  int64_t f = 0;
  if (check_split(ffn, t, 0, &f) != TP_OK) return 0;
  const size_t act = round256(static_cast<size_t>(tokens) * static_cast<size_t>(f) *
                              static_cast<size_t>(elem_bytes(in_dt)));
  return in_dt == TP_BF16 ? act : 3 * act;   // fp32: gate, value, product
}

tp_status tp_mlp_swiglu_shard_fwd(const void* x, const void* wg_i, const void* wu_i, int64_t lda,
                                  const void* b_i, const void* bias_b, const void* residual,
                                  void* z_i, void* workspace, size_t workspace_bytes,
                                  int64_t tokens, int64_t hidden, int64_t ffn, int t, int rank,
                                  tp_dtype in_dt, tp_dtype out_dt, void* stream) {
  if (!dtype_known(in_dt) || !dtype_known(out_dt) || !gemm_pair_ok(in_dt, out_dt))
    return TP_ERR_DTYPE;
  if (tokens < 0 || hidden < 1) return TP_ERR_INVALID_ARG;
  int64_t f = 0;
  TP_TRY(check_split(ffn, t, rank, &f));
  if (!fits_int32(tokens) || !fits_int32(hidden) || !fits_int32(2 * f)) return TP_ERR_UNSUPPORTED;
  if (tokens == 0) return TP_OK;
  TP_TRY(check_matrix(x, hidden, hidden, in_dt));
  TP_TRY(check_matrix(wg_i, lda, f, in_dt));
  TP_TRY(check_matrix(wu_i, lda, f, in_dt));
  TP_TRY(check_matrix(b_i, hidden, hidden, in_dt));
  TP_TRY(check_matrix(z_i, hidden, hidden, out_dt));
  const bool owner = rank == 0;
  const void* bias_use = owner ? bias_b : nullptr;
  const void* res_use = owner ? residual : nullptr;
  TP_TRY(check_optional_vec(bias_use));
  TP_TRY(check_optional_vec(res_use));
  const size_t need = tp_mlp_swiglu_shard_workspace_bytes(tokens, hidden, ffn, t, in_dt);
  if (workspace == nullptr || workspace_bytes < need) return TP_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return TP_ERR_MISALIGNED;

  hipStream_t s = static_cast<hipStream_t>(stream);
  uint8_t* w = static_cast<uint8_t*>(workspace);
  void* h = w;
  if (in_dt == TP_BF16) {
    // Both gated projections in one product, H_i = SiLU(X Wg_i) * (X Wu_i)
    // formed in the epilogue (one bf16 HBM round trip of H_i).
    TP_TRY(from_hip(tpk::launch_gemm_bf16_swiglu(
        static_cast<const uint16_t*>(x), hidden, static_cast<const uint16_t*>(wg_i),
        static_cast<const uint16_t*>(wu_i), lda, tokens, f, hidden, static_cast<uint16_t*>(h), f, s)));
  } else {
    const size_t act = round256(static_cast<size_t>(tokens) * static_cast<size_t>(f) * 4);
    float* g = reinterpret_cast<float*>(w + act);
    float* u = reinterpret_cast<float*>(w + 2 * act);
    tpk::Epilogue eg{nullptr, nullptr, 0, g, f, true, tpk::EPI_LINEAR};
    TP_TRY(run_gemm(in_dt, x, hidden, wg_i, lda, tokens, f, hidden, eg, s));
    tpk::Epilogue eu{nullptr, nullptr, 0, u, f, true, tpk::EPI_LINEAR};
    TP_TRY(run_gemm(in_dt, x, hidden, wu_i, lda, tokens, f, hidden, eu, s));
    TP_TRY(from_hip(tpk::launch_swiglu_combine_f32(g, u, static_cast<float*>(h), tokens * f, s)));
  }
  // Row-parallel GEMM: Z_i = H_i B_i (+ b + R on rank 0).
  tpk::Epilogue e2{bias_use, res_use, hidden, z_i, hidden, out_dt == TP_F32, tpk::EPI_LINEAR};
  return run_gemm(in_dt, h, f, b_i, hidden, tokens, hidden, f, e2, s);
}

namespace {
// Workspace of tp_mlp_shard_bwd: dY_i, H_i [tokens, f] (in_dt), then the
// column-sum partials (fp32) of the bias gradients.
struct MlpBwdWorkspace {
  size_t dy, h, partial, total;
};
MlpBwdWorkspace mlp_bwd_workspace(int64_t tokens, int64_t hidden, int64_t f, tp_dtype in_dt) {
  const size_t act = round256(static_cast<size_t>(tokens) * static_cast<size_t>(f) *
                              static_cast<size_t>(elem_bytes(in_dt)));
  const int64_t cols = f > hidden ? f : hidden;
  const size_t part = round256(static_cast<size_t>(tpk::colsum_partial_floats(tokens, cols)) * 4);
  return {act, act, part, 2 * act + part};
}
}  // namespace

size_t tp_mlp_shard_bwd_workspace_bytes(int64_t tokens, int64_t hidden, int64_t ffn, int t,
                                        tp_dtype in_dt) {
  if (!dtype_known(in_dt) || tokens < 0 || hidden < 1) return 0;
  int64_t f = 0;
  if (check_split(ffn, t, 0, &f) != TP_OK) return 0;
  return mlp_bwd_workspace(tokens, hidden, f, in_dt).total;
}

tp_status tp_mlp_shard_bwd(const void* x, const void* a_i, int64_t lda, const void* b_i,
                           const void* y_i, const void* dz, void* dx_i, void* da_i, void* db_i,
                           void* dbias_a_i, void* dbias_b, void* workspace,
                           size_t workspace_bytes, int64_t tokens, int64_t hidden, int64_t ffn,
                           int t, int rank, tp_dtype in_dt, tp_dtype grad_dt, void* stream) {
  if (!dtype_known(in_dt) || !dtype_known(grad_dt) || !gemm_pair_ok(in_dt, grad_dt))
    return TP_ERR_DTYPE;
  if (tokens < 0 || hidden < 1) return TP_ERR_INVALID_ARG;
  int64_t f = 0;
  TP_TRY(check_split(ffn, t, rank, &f));
  if (!fits_int32(tokens) || !fits_int32(hidden) || !fits_int32(f)) return TP_ERR_UNSUPPORTED;
  // operands that are read (tokens == 0 reads none of the token-indexed ones)
  TP_TRY(check_matrix(a_i, lda, f, in_dt));
  TP_TRY(check_matrix(b_i, hidden, hidden, in_dt));
  TP_TRY(check_matrix(da_i, lda, f, grad_dt));
  TP_TRY(check_matrix(db_i, hidden, hidden, grad_dt));
  TP_TRY(check_optional_vec(dbias_a_i));
  TP_TRY(check_optional_vec(dbias_b));
  if (tokens > 0) {
    TP_TRY(check_matrix(x, hidden, hidden, in_dt));
    TP_TRY(check_matrix(y_i, f, f, in_dt));
    TP_TRY(check_matrix(dz, hidden, hidden, in_dt));
    TP_TRY(check_matrix(dx_i, hidden, hidden, grad_dt));
  }
  const MlpBwdWorkspace ws = mlp_bwd_workspace(tokens, hidden, f, in_dt);
  if (workspace == nullptr || workspace_bytes < ws.total) return TP_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return TP_ERR_MISALIGNED;

  hipStream_t s = static_cast<hipStream_t>(stream);
  const int geb = static_cast<int>(elem_bytes(grad_dt));
  const bool g32 = grad_dt == TP_F32;
  if (tokens == 0) {
    // sums over no tokens: zero weight and bias gradients
    TP_TRY(from_hip(tpk::launch_zero_2d(da_i, hidden, f, lda, geb, s)));
    TP_TRY(from_hip(tpk::launch_zero_2d(db_i, f, hidden, hidden, geb, s)));
    if (dbias_a_i != nullptr) TP_TRY(from_hip(tpk::launch_zero_2d(dbias_a_i, 1, f, f, 4, s)));
    if (dbias_b != nullptr) TP_TRY(from_hip(tpk::launch_zero_2d(dbias_b, 1, hidden, hidden, 4, s)));
    return TP_OK;
  }
  uint8_t* w = static_cast<uint8_t*>(workspace);
  void* dy = w;
  void* h = w + ws.dy;
  float* partial = reinterpret_cast<float*>(w + ws.dy + ws.h);
  const bool in32 = in_dt == TP_F32;
  // 1. dH_i = dz B_i^T (B_i is [f, hidden]: the product reads it as [N, K]),
  //    with dY_i = dH_i * GeLU'(Y_i) and H_i = GeLU(Y_i) in the epilogue.
  tpk::Epilogue e1{nullptr, nullptr, 0, dy, f, in32, tpk::EPI_GELU_BWD};
  e1.aux = y_i;
  e1.ldaux = f;
  e1.out2 = h;
  TP_TRY(run_gemm_t(in_dt, dz, hidden, false, b_i, hidden, false, tokens, f, hidden, e1, s));
  // 2. db_i = H_i^T dz: A = H_i read as [K = tokens, M = f].
  tpk::Epilogue e2{nullptr, nullptr, 0, db_i, hidden, g32, tpk::EPI_LINEAR};
  TP_TRY(run_gemm_t(in_dt, h, f, true, dz, hidden, true, f, hidden, tokens, e2, s));
  // 3. da_i = X^T dY_i: A = X read as [K = tokens, M = hidden].
  tpk::Epilogue e3{nullptr, nullptr, 0, da_i, lda, g32, tpk::EPI_LINEAR};
  TP_TRY(run_gemm_t(in_dt, x, hidden, true, dy, f, true, hidden, f, tokens, e3, s));
  // 4. dx_i = dY_i A_i^T (A_i is [hidden, f]: read as [N, K]).
  tpk::Epilogue e4{nullptr, nullptr, 0, dx_i, hidden, g32, tpk::EPI_LINEAR};
  TP_TRY(run_gemm_t(in_dt, dy, f, false, a_i, lda, false, tokens, hidden, f, e4, s));
  // 5. bias gradients: column sums over the tokens.
  const int dt = in_dt == TP_BF16 ? 1 : 0;
  if (dbias_a_i != nullptr)
    TP_TRY(from_hip(tpk::launch_colsum(dy, f, dt, tokens, f, static_cast<float*>(dbias_a_i),
                                       partial, s)));
  if (dbias_b != nullptr)
    TP_TRY(from_hip(tpk::launch_colsum(dz, hidden, dt, tokens, hidden,
                                       static_cast<float*>(dbias_b), partial, s)));
  return TP_OK;
}

namespace {
// Workspace of tp_attn_shard_fwd: the rank's packed QKV projection [tokens,
// 3*hl*d] (q, k columns fp16 scaled, v columns bf16), the attention output
// [tokens, hl*d] bf16, then, for grids small enough that their rows may be
// split over two workgroups (at most kAttnSplitMaxRows query blocks: twice
// the CUs of a whole MI355X), the split's partial states and arrival
// counters; larger grids never split and get none (at most ~68 MB).
constexpr int64_t kAttnSplitMaxRows = 512;
struct AttnWorkspace {
  size_t qkv_bytes, o_bytes, part_bytes, arrival_bytes, total;
};
AttnWorkspace attn_workspace(int64_t batch, int64_t seq, int64_t hl, int64_t head_dim) {
  const int64_t tokens = batch * seq;
  const size_t qkv = round256(static_cast<size_t>(tokens) * 3 * hl * head_dim * 2);
  const size_t o = round256(static_cast<size_t>(tokens) * hl * head_dim * 2);
  const int64_t rows = tpk::attn_arrival_ints(batch, seq, hl);   // query blocks
  const bool may_split = rows <= kAttnSplitMaxRows;
  const size_t part = may_split ? round256(static_cast<size_t>(tpk::attn_part_floats(tokens, hl)) * 4) : 0;
  const size_t arr = may_split ? round256(static_cast<size_t>(rows) * 4) : 0;
  return {qkv, o, part, arr, qkv + o + part + arr};
}
}  // namespace

size_t tp_attn_shard_workspace_bytes(int64_t batch, int64_t seq, int64_t hidden, int64_t heads,
                                     int64_t head_dim, int t, tp_dtype in_dt) {
  if (in_dt != TP_BF16 || batch < 0 || seq < 0 || hidden < 1 || head_dim < 1) return 0;
  int64_t hl = 0;
  if (check_split(heads, t, 0, &hl) != TP_OK || hidden != heads * head_dim) return 0;
  return attn_workspace(batch, seq, hl, head_dim).total;
}

tp_status tp_attn_shard_fwd(const void* x, const void* wqkv_i, const void* wo_i, void* out_i,
                            void* workspace, size_t workspace_bytes, int64_t batch, int64_t seq,
                            int64_t hidden, int64_t heads, int64_t head_dim, int causal, int t,
                            int rank, tp_dtype in_dt, tp_dtype out_dt, void* stream) {
  if (!dtype_known(in_dt) || !dtype_known(out_dt) || in_dt != TP_BF16) return TP_ERR_DTYPE;
  if (batch < 0 || seq < 0 || hidden < 1 || head_dim < 1 || (causal != 0 && causal != 1))
    return TP_ERR_INVALID_ARG;
  int64_t hl = 0;  // heads per rank
  TP_TRY(check_split(heads, t, rank, &hl));
  if (hidden != heads * head_dim) return TP_ERR_INVALID_ARG;
  if (hidden % 8 != 0) return TP_ERR_MISALIGNED;
  const int64_t tokens = batch * seq;
  if (head_dim != 128 || (tokens > 0 && seq < 32)) return TP_ERR_UNSUPPORTED;
  if (!fits_int32(tokens) || !fits_int32(hidden) || !fits_int32(3 * hl * head_dim))
    return TP_ERR_UNSUPPORTED;
  if (tokens == 0) return TP_OK;
  const int64_t dl = hl * head_dim;  // local attention width
  TP_TRY(check_matrix(x, hidden, hidden, in_dt));
  TP_TRY(check_matrix(wqkv_i, 3 * dl, 3 * dl, in_dt));
  TP_TRY(check_matrix(wo_i, hidden, hidden, in_dt));
  TP_TRY(check_matrix(out_i, hidden, hidden, out_dt));
  const AttnWorkspace ws = attn_workspace(batch, seq, hl, head_dim);
  if (workspace == nullptr || workspace_bytes < ws.total) return TP_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return TP_ERR_MISALIGNED;

  hipStream_t s = static_cast<hipStream_t>(stream);
  uint8_t* w = static_cast<uint8_t*>(workspace);
  uint16_t* qkv = reinterpret_cast<uint16_t*>(w);
  uint16_t* o = reinterpret_cast<uint16_t*>(w + ws.qkv_bytes);
  float* part = ws.part_bytes ? reinterpret_cast<float*>(w + ws.qkv_bytes + ws.o_bytes) : nullptr;
  int* arrivals =
      ws.arrival_bytes ? reinterpret_cast<int*>(w + ws.qkv_bytes + ws.o_bytes + ws.part_bytes) : nullptr;
  // 1. Column-parallel packed QKV projection of the rank's heads; Q and K
  //    leave the fp32 accumulator as scaled fp16 (11 significant bits for
  //    Q K^T), V as bf16.
  tpk::Epilogue ep1{nullptr, nullptr, 0, qkv, 3 * dl, false, tpk::EPI_QKV_F16};
  TP_TRY(run_gemm(in_dt, x, hidden, wqkv_i, 3 * dl, tokens, 3 * dl, hidden, ep1, s));
  // 2. softmax(Q K^T / sqrt(d)) V per local head.
  TP_TRY(from_hip(tpk::launch_attention(qkv, 3 * dl, o, dl, static_cast<int>(batch),
                                        static_cast<int>(seq), static_cast<int>(hl),
                                        static_cast<int>(head_dim), causal == 1, part, arrivals,
                                        s)));
  // 3. Row-parallel output projection: the rank's full-hidden partial.
  tpk::Epilogue ep3{nullptr, nullptr, 0, out_i, hidden, out_dt == TP_F32, tpk::EPI_LINEAR};
  return run_gemm(in_dt, o, dl, wo_i, hidden, tokens, hidden, dl, ep3, s);
}

tp_status tp_sp_reduce_scatter(const void* const* partials, int t, int rank, const void* bias,
                               const void* residual_r, void* out_r, int64_t tokens,
                               int64_t hidden, tp_dtype in_dt, tp_dtype out_dt, void* stream) {
  if (!dtype_known(in_dt) || !dtype_known(out_dt)) return TP_ERR_DTYPE;
  if (t < 1 || rank < 0 || rank >= t) return TP_ERR_BAD_RANK;
  if (t > tpk::kSpMaxParts) return TP_ERR_UNSUPPORTED;
  if (tokens < 0 || hidden < 1 || partials == nullptr) return TP_ERR_INVALID_ARG;
  if (tokens % t != 0) return TP_ERR_NOT_DIVISIBLE;
  if (hidden % 4 != 0) return TP_ERR_MISALIGNED;
  if (!fits_int32(hidden)) return TP_ERR_UNSUPPORTED;
  if (tokens == 0) return TP_OK;
  tpk::SpPartials parts{};
  for (int j = 0; j < t; ++j) {
    if (partials[j] == nullptr) return TP_ERR_INVALID_ARG;
    if (!aligned16(partials[j])) return TP_ERR_MISALIGNED;
    parts.p[j] = static_cast<const float*>(partials[j]);
  }
  if (out_r == nullptr) return TP_ERR_INVALID_ARG;
  if (!aligned16(out_r)) return TP_ERR_MISALIGNED;
  TP_TRY(check_optional_vec(bias));
  TP_TRY(check_optional_vec(residual_r));
  const int64_t rows = tokens / t;
  return from_hip(tpk::launch_sp_reduce(parts, t, rank * rows, rows, hidden, bias, residual_r,
                                        in_dt == TP_BF16 ? 1 : 0, out_r, out_dt == TP_BF16 ? 1 : 0,
                                        static_cast<hipStream_t>(stream)));
}

}  // extern "C"
