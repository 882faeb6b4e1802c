// tp_mlp_shard_fwd_noalloc: the MLP shard forward for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc).  It is tp_mlp_shard_fwd with the GeLU
// intermediate H_i kept in a fixed device array of this library instead of
// a caller workspace; nothing here allocates or frees.
//
//   * `scratch` is a file-scope __device__ array of TP_NOALLOC_SCRATCH_BYTES.
//     Each GPU the library runs on holds its own copy until the process
//     ends.  In host code the name `scratch` is only a host-side stand-in, so
//     the array's device address is looked up once per device with
//     hipGetSymbolAddress (that device current) and only that address is
//     handed to kernels.
//   * The MLP is row-independent, so tokens are processed in row chunks
//     whose H_i fits the array (a multiple of 256 rows when more than one
//     chunk is needed): any token count works, and the shard width is
//     bounded instead (at least 256 rows of H_i must fit).
//   * H_i is written in full by each chunk's first GEMM before its second
//     GEMM reads it, so nothing needs clearing between calls.  All calls on
//     one GPU share its array: calls that overlap on one GPU (other streams,
//     other threads) race on it.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "../../include/tp_shard.h"
#include "abi_internal.h"

namespace {

constexpr size_t kScratchBytes = TP_NOALLOC_SCRATCH_BYTES;
constexpr int64_t kChunkRows = 256;   // the row granularity of the GEMM tiles
constexpr int kMaxDevices = 64;

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of the current device's copy of `scratch` (looked up on
// the first call on that device, then cached).
tp_status scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return TP_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return TP_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return TP_OK;
}

}  // namespace

extern "C" {

tp_status tp_mlp_shard_fwd_noalloc(const void* x, const void* a_i, int64_t lda, const void* b_i,
                                   const void* bias_a_i, const void* bias_b, const void* residual,
                                   void* z_i, void* y_save, int64_t tokens, int64_t hidden,
                                   int64_t ffn, int t, int rank, tp_dtype in_dt, tp_dtype out_dt,
                                   void* stream) {
  int64_t f = 0;
  const tp_status v = tpabi::mlp_fwd_validate(x, a_i, lda, b_i, bias_a_i, bias_b, residual, z_i,
                                              y_save, tokens, hidden, ffn, t, rank, in_dt, out_dt, &f);
  if (v != TP_OK) return v;
  if (tokens == 0) return TP_OK;
  const int64_t ie = in_dt == TP_BF16 ? 2 : 4;
  const int64_t oe = out_dt == TP_BF16 ? 2 : 4;
  const int64_t fit = static_cast<int64_t>(kScratchBytes) / (f * ie);   // rows of H_i the array holds
  if (fit < (tokens < kChunkRows ? tokens : kChunkRows)) return TP_ERR_WORKSPACE;
  const int64_t chunk = tokens <= fit ? tokens : fit / kChunkRows * kChunkRows;
  void* h = nullptr;
  const tp_status sa = scratch_address(&h);
  if (sa != TP_OK) return sa;

  const bool owner = rank == 0;
  const char* xb = static_cast<const char*>(x);
  const char* rb = static_cast<const char*>(owner ? residual : nullptr);
  char* zb = static_cast<char*>(z_i);
  char* yb = static_cast<char*>(y_save);
  hipStream_t s = static_cast<hipStream_t>(stream);
  for (int64_t m0 = 0; m0 < tokens; m0 += chunk) {
    const int64_t rows = tokens - m0 < chunk ? tokens - m0 : chunk;
    const tp_status e = tpabi::mlp_fwd_enqueue(
        xb + m0 * hidden * ie, a_i, lda, b_i, bias_a_i, owner ? bias_b : nullptr,
        rb == nullptr ? nullptr : rb + m0 * hidden * ie, zb + m0 * hidden * oe,
        yb == nullptr ? nullptr : yb + m0 * f * ie, h, nullptr, rows, hidden, f, in_dt, out_dt, s);
    if (e != TP_OK) return e;
  }
  return TP_OK;
}

}  // extern "C"
