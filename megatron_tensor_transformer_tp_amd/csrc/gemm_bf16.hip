// Dispatch of the bf16 GEMM to its tile shape and epilogue instantiation.
#include <atomic>

#include "gemm_bf16_impl.h"

namespace tpk {

namespace {
template <int BM, int BN>
hipError_t launch_epi(const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb, int M, int N,
                      int K, const Epilogue& ep, hipStream_t stream) {
  if (ep.kind == EPI_GELU)
    return ep.out_f32 ? launch_gemm_bf16_cfg<BM, BN, EPI_GELU, true>(A, lda, B, ldb, M, N, K, ep, stream)
                      : launch_gemm_bf16_cfg<BM, BN, EPI_GELU, false>(A, lda, B, ldb, M, N, K, ep, stream);
  if (ep.kind == EPI_QKV_F16)
    return ep.out_f32 ? hipErrorInvalidValue
                      : launch_gemm_bf16_cfg<BM, BN, EPI_QKV_F16, false>(A, lda, B, ldb, M, N, K, ep, stream);
  if (ep.kind != EPI_LINEAR) return hipErrorInvalidValue;
  return ep.out_f32 ? launch_gemm_bf16_cfg<BM, BN, EPI_LINEAR, true>(A, lda, B, ldb, M, N, K, ep, stream)
                    : launch_gemm_bf16_cfg<BM, BN, EPI_LINEAR, false>(A, lda, B, ldb, M, N, K, ep, stream);
}
}  // namespace

// Compute units of the current device (cached per device, safe to call
// from several threads; 256 on a whole MI355X, fewer on a partition).
int64_t device_cus() {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cus[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
  int n = cus[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cus[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// Tile shape by an estimate of the launch time in units of one 256 x 256
// tile's time, from the tile counts (one workgroup per CU for 256 x 256 and
// 128 x 384, two for 128 x 128) and relative per-CU throughputs measured on
// the 4096 x 8192 x {3072, 1536} products (128 x 384: 0.84, 128 x 128: 0.82
// of the 256 x 256 rate; a last 128 x 128 round with one workgroup per CU
// costs 0.73 of a full one).
// The forward's linears also have 64 x 128 tiles (two workgroups per CU,
// 0.456 of the 256 x 256 rate per CU: fitted to the 2048 x 1024 x 4096 row
// product, 128 x 128 tiles on half the CUs 31.5 us, 64 x 128 on all 28.4),
// which win only where 128 x 128 tiles leave CUs idle.  Without the
// forward-only shapes (forward false) the choice is between 256 x 256 and
// 128 x 128; r128 is the 128 x 128 tile's per-CU rate relative to the
// 256 x 256 tile's.
static int gemm_tile_choice(int64_t M, int64_t N, bool forward = true, double r128 = 0.82) {
  const int64_t kCUs = device_cus();
  auto tiles = [&](int64_t bm, int64_t bn) { return ((M + bm - 1) / bm) * ((N + bn - 1) / bn); };
  // rounds of two workgroups per CU, a last round with at most one per CU
  // costing 0.73 of a full one, in units of one 256 x 256 tile's time
  auto cost2 = [&](int64_t t, double area, double rate) {
    const int64_t rem = t % (2 * kCUs);
    return (static_cast<double>(t / (2 * kCUs)) + (rem == 0 ? 0.0 : rem <= kCUs ? 0.73 : 1.0)) * 2.0 *
           area / (256.0 * 256.0) / rate;
  };
  const int64_t t256 = tiles(256, 256), t384 = tiles(128, 384);
  const double c256 = static_cast<double>((t256 + kCUs - 1) / kCUs);
  const double c384 = forward ? static_cast<double>((t384 + kCUs - 1) / kCUs) * (128.0 * 384.0) /
                                    (256.0 * 256.0) / 0.84
                              : 1e300;
  const double c128 = cost2(tiles(128, 128), 128.0 * 128.0, r128);
  const double c64 = forward ? cost2(tiles(64, 128), 64.0 * 128.0, 0.456) : 1e300;
  if (c256 <= c384 && c256 <= c128 && c256 <= c64) return 256;
  if (c384 <= c128 && c384 <= c64) return 384;
  return c128 <= c64 ? 128 : 64;
}

hipError_t launch_gemm_bf16(const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb,
                            int64_t M, int64_t N, int64_t K, const Epilogue& ep,
                            hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  const int m = static_cast<int>(M), n = static_cast<int>(N), k = static_cast<int>(K);
  switch (gemm_tile_choice(M, N)) {
    case 256: return launch_epi<256, 256>(A, lda, B, ldb, m, n, k, ep, stream);
    case 384: return launch_epi<128, 384>(A, lda, B, ldb, m, n, k, ep, stream);
    case 128: return launch_epi<128, 128>(A, lda, B, ldb, m, n, k, ep, stream);
    default: return launch_epi<64, 128>(A, lda, B, ldb, m, n, k, ep, stream);
  }
}

namespace {
template <int BM, int BN>
hipError_t launch_t_tile(const uint16_t* A, int64_t lda, bool a_kmajor, const uint16_t* B,
                         int64_t ldb, bool b_kmajor, int m, int n, int k, const Epilogue& ep,
                         hipStream_t stream) {
  if (!a_kmajor && !b_kmajor) {
    if (ep.kind == EPI_GELU_BWD && !ep.out_f32)
      return launch_gemm_bf16_t_cfg<BM, BN, false, false, EPI_GELU_BWD, false>(A, lda, B, ldb, m, n, k, ep, stream);
    if (ep.kind == EPI_LINEAR)
      return ep.out_f32
                 ? launch_gemm_bf16_t_cfg<BM, BN, false, false, EPI_LINEAR, true>(A, lda, B, ldb, m, n, k, ep, stream)
                 : launch_gemm_bf16_t_cfg<BM, BN, false, false, EPI_LINEAR, false>(A, lda, B, ldb, m, n, k, ep, stream);
    return hipErrorInvalidValue;
  }
  if (a_kmajor && b_kmajor && ep.kind == EPI_LINEAR)
    return ep.out_f32
               ? launch_gemm_bf16_t_cfg<BM, BN, true, true, EPI_LINEAR, true>(A, lda, B, ldb, m, n, k, ep, stream)
               : launch_gemm_bf16_t_cfg<BM, BN, true, true, EPI_LINEAR, false>(A, lda, B, ldb, m, n, k, ep, stream);
  return hipErrorInvalidValue;
}
}  // namespace

// The backward's layouts (both operands k-contiguous or both k-major) on
// 256 x 256 or 128 x 128 tiles by the same estimate as the forward (small
// weight gradients, e.g. 4096 x 1376, fill a fraction of the CUs with
// 256 x 256 tiles).
hipError_t launch_gemm_bf16_t(const uint16_t* A, int64_t lda, bool a_kmajor, const uint16_t* B,
                              int64_t ldb, bool b_kmajor, int64_t M, int64_t N, int64_t K,
                              const Epilogue& ep, hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  if (K <= 0) return hipErrorInvalidValue;
  const int m = static_cast<int>(M), n = static_cast<int>(N), k = static_cast<int>(K);
  if (!a_kmajor && b_kmajor) {
    if (ep.kind == EPI_GELU_BWD) return hipErrorInvalidValue;
    return launch_gemm_bf16(A, lda, B, ldb, M, N, K, ep, stream);
  }
  if (a_kmajor != b_kmajor) return hipErrorInvalidValue;
  if (gemm_tile_choice(M, N, false) == 256)
    return launch_t_tile<256, 256>(A, lda, a_kmajor, B, ldb, b_kmajor, m, n, k, ep, stream);
  return launch_t_tile<128, 128>(A, lda, a_kmajor, B, ldb, b_kmajor, m, n, k, ep, stream);
}

hipError_t launch_gemm_bf16_swiglu(const uint16_t* A, int64_t lda, const uint16_t* Bg,
                                   const uint16_t* Bu, int64_t ldb, int64_t M, int64_t F,
                                   int64_t K, uint16_t* out, int64_t ldo, hipStream_t stream) {
  if (M == 0 || F == 0) return hipSuccess;
  if (K <= 0 || F % 8 != 0) return hipErrorInvalidValue;
  Epilogue ep{nullptr, nullptr, 0, out, ldo, false, EPI_SWIGLU};
  ep.b2 = Bu;
  // the product runs over the 2F interleaved gate / value columns; its
  // 128 x 128 tiles run at 0.63 of the 256 x 256 rate per CU (measured at
  // M 8192, K 4096, 2F 2752: 3 rounds of 128 x 128 tiles took 1.19 times
  // the 2 rounds of 256 x 256 tiles)
  const int m = static_cast<int>(M), n = static_cast<int>(2 * F), k = static_cast<int>(K);
  if (gemm_tile_choice(M, 2 * F, false, 0.63) == 256)
    return launch_gemm_bf16_t_cfg<256, 256, false, true, EPI_SWIGLU, false>(A, lda, Bg, ldb, m, n, k, ep, stream);
  return launch_gemm_bf16_t_cfg<128, 128, false, true, EPI_SWIGLU, false>(A, lda, Bg, ldb, m, n, k, ep, stream);
}

}  // namespace tpk
