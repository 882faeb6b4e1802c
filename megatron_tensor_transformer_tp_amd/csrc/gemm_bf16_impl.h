// bf16 GEMM with fp32 accumulation on gfx950 matrix cores: the pieces shared
// by the kernel (gemm_bf16_dma.h) and its instantiation units
// (gemm_bf16_*.hip, one per tile shape and operand layout, so that they
// compile in parallel): workgroup -> tile maps, scheduling helpers and the
// fused epilogues.
//
//   C[M, N] = A[M, K] . B[K, N]      bf16 operands, fp32 accumulators
//
// The column-parallel linear of a tensor-parallel MLP calls it with
// A = X [tokens, hidden], B = A_i [hidden, f] and the GeLU epilogue; the
// row-parallel linear with A = H_i [tokens, f], B = B_i [f, hidden] and the
// bias/residual epilogue (列并行 tutorial, 数学基础 and MLP 应用; Megatron
// expert interview Level 2, M025/M026).
//
//   * Operand roles inside the MFMA (v_mfma_f32_16x16x32_bf16, or
//     v_mfma_f32_32x32x16_bf16) are swapped (the B fragment is the MFMA's
//     first operand, the A fragment the second), so each lane ends up owning
//     4 CONSECUTIVE output columns of one row: the epilogue stores 16-byte
//     fp32 or 8-byte bf16 vectors.
//   * Workgroup -> tile mapping is XCD-aware: consecutive workgroup ids are
//     dealt round-robin to the 8 XCDs, so ids are first regrouped so that
//     each XCD owns a contiguous range of logical tiles, then tiles are
//     ordered in groups of 8 tile-rows so that concurrently running tiles
//     on one XCD share A row-panels and B column-panels in its L2.
#pragma once

#include <hip/hip_runtime.h>

#include <type_traits>

#include "device_common.h"
#include "kernels.h"

namespace tpk {
namespace gemm_detail {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kBKd = 32;         // k-tile of the global->LDS copy kernel
constexpr int kXcds = 8;
constexpr int kGroupM = 8;

__device__ __forceinline__ void tile_coords(int bid, int nblk, int tiles_m, int tiles_n,
                                            int& tm, int& tn) {
  int pid = bid;
  if (nblk % kXcds == 0) pid = (bid % kXcds) * (nblk / kXcds) + bid / kXcds;
  const int width = kGroupM * tiles_n;
  const int group = pid / width;
  const int first_m = group * kGroupM;
  const int gsize = min(tiles_m - first_m, kGroupM);
  const int in_group = pid - group * width;
  tm = first_m + in_group % gsize;
  tn = in_group / gsize;
}

// Round-synchronous order for one-tile-per-CU grids: workgroup b runs on
// XCD b % 8 as that XCD's (b / 8)-th tile; an XCD's tiles come in rounds of
// 32 (one per CU of the XCD), and round r of all XCDs covers one compact
// block of (256 / tiles_n) x tiles_n tiles, XCD x taking a 4 x 8 sub-block.
// The operand panels live in one round (A rows of the block + all of B) fit
// in the last-level (MALL) cache, while each XCD's L2 still sees only 4 + 8
// panels per round.  Applies when tiles_n is 8, 16 or 32 and tiles_m a
// multiple of 256 / tiles_n; returns false otherwise.
__device__ __forceinline__ bool tile_coords_rounds(int bid, int nblk, int tiles_m, int tiles_n,
                                                   int& tm, int& tn) {
  if (tiles_n != 8 && tiles_n != 16 && tiles_n != 32) return false;
  const int rows = 256 / tiles_n;                // tile-rows per round block
  if (nblk != tiles_m * tiles_n || tiles_m % rows != 0) return false;
  const int xcd = bid % kXcds, k = bid / kXcds;
  const int round = k / 32, s = k % 32;
  const int xr = rows / 4;                       // XCD sub-blocks stacked vertically
  tm = round * rows + (xcd % xr) * 4 + (s % 4);
  tn = (xcd / xr) * 8 + s / 4;
  return true;
}

// Scheduling fence between the k-substeps of the main loop: nothing moves
// across it, so the LDS reads issued in substep s for substep s+1 stay ahead
// of the MFMAs of substep s (the default scheduler would sink them next to
// their uses and expose the LDS latency to the matrix pipe).
__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

// Within a substep, an explicit interleave: each MFMA is followed by one of
// the LDS fragment reads for the next substep (sched_group_barrier masks).
constexpr int kSchedMfma = 0x008;
constexpr int kSchedDsRead = 0x100;

template <int MASK, int N>
__device__ __forceinline__ void sched_group() {
  __builtin_amdgcn_sched_group_barrier(MASK, N, 0);
}

// Epilogue shared by the GEMM kernels.  acc[j][i][4g + r] is C[m][n] with
//   m = m_lane + i*32 + row_of(g),  n = n_lane + j*32 + col_of(g) + r,
// i.e. each lane owns 4 consecutive columns per (i, j, g): one 16-byte fp32
// or 8-byte bf16 store.  32 x 32 x 16 MFMA blocks: row_of(g) = 0,
// col_of(g) = 8g (lanes l and l + 32 hold columns 4 apart), m_lane = .. + l % 32.
// 16 x 16 x 32 MFMA blocks (MF16, four per 32 x 32 block, sub-block g at
// rows 16 (g / 2), columns 16 (g % 2)): m_lane = .. + l % 16 and
// n_lane = .. + 4 (l / 16).  EPI selects the epilogue kind at compile time; the
// optional inputs (bias, residual) are uniform, so each combination's body is
// instantiated once and selected with one branch (the GeLU kinds never take
// a residual).
__device__ __forceinline__ void load_bf16x4(const uint16_t* p, float (&v)[4]) {
  const u32x2_t w = *reinterpret_cast<const u32x2_t*>(p);
  v[0] = __uint_as_float(w[0] << 16);
  v[1] = __uint_as_float(w[0] & 0xFFFF0000u);
  v[2] = __uint_as_float(w[1] << 16);
  v[3] = __uint_as_float(w[1] & 0xFFFF0000u);
}

template <bool OUT_F32>
__device__ __forceinline__ void store_x4(void* base, int64_t off, const float (&v)[4]) {
  if constexpr (OUT_F32) {
    typedef float f32x4_t __attribute__((ext_vector_type(4)));
    *reinterpret_cast<f32x4_t*>(static_cast<float*>(base) + off) = f32x4_t{v[0], v[1], v[2], v[3]};
  } else {
    *reinterpret_cast<u32x2_t*>(static_cast<uint16_t*>(base) + off) =
        u32x2_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
  }
}

template <bool MF16>
__device__ __forceinline__ constexpr int row_of(int g) { return MF16 ? 16 * (g >> 1) : 0; }
template <bool MF16>
__device__ __forceinline__ constexpr int col_of(int g) { return MF16 ? 16 * (g & 1) : 8 * g; }

template <int TM, int TN, bool MASKED, int EPI, bool OUT_F32, bool MF16 = false>
__device__ __forceinline__ void store_tile(const f32x16_t (&acc)[TN][TM], int m_lane, int n_lane,
                                           int M, int N, const Epilogue& ep) {
  const uint16_t* __restrict__ bias = static_cast<const uint16_t*>(ep.bias);
  const uint16_t* __restrict__ residual = static_cast<const uint16_t*>(ep.residual);
  const uint16_t* __restrict__ aux = static_cast<const uint16_t*>(ep.aux);
  auto epilogue = [&](auto has_bias, auto has_res, auto has_extra) __attribute__((always_inline)) {
    constexpr bool kBias = decltype(has_bias)::value;
    constexpr bool kRes = decltype(has_res)::value;
    constexpr bool kExtra = decltype(has_extra)::value;   // pre (GeLU)
    static_for<TM>([&](auto I) __attribute__((always_inline)) {
      const int m_i = m_lane + I * 32;
      if (!MF16 && MASKED && m_i >= M) return;
      static_for<TN>([&](auto J) __attribute__((always_inline)) {
        static_for<4>([&](auto G) __attribute__((always_inline)) {
          constexpr int col = J * 32 + col_of<MF16>(G);
          const int m = m_i + row_of<MF16>(G);
          if (MASKED && ((MF16 && m >= M) || n_lane + col >= N)) return;
          const int64_t row_out = static_cast<int64_t>(m) * ep.ldo + n_lane;
          const int64_t row_res = kRes ? static_cast<int64_t>(m) * ep.ldr + n_lane : 0;
          const int64_t row_aux = EPI == EPI_GELU_BWD ? static_cast<int64_t>(m) * ep.ldaux + n_lane : 0;
          float v[4];
          static_for<4>([&](auto R) __attribute__((always_inline)) { v[R] = acc[J][I][4 * G + R]; });
          if constexpr (EPI == EPI_QKV_F16) {
            static_assert(!OUT_F32, "the packed projection is 16-bit");
            // this store's columns (MF16: 16 at a 16-aligned offset; 8 at an
            // 8-aligned one otherwise) lie in one 128-column part, so the
            // part is wave-uniform
            if (__builtin_amdgcn_readfirstlane(((n_lane + col) / kQkvPart) % 3) < 2) {
              typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
              const f16x2_t a = {static_cast<_Float16>(v[0] * kQkScale), static_cast<_Float16>(v[1] * kQkScale)};
              const f16x2_t b = {static_cast<_Float16>(v[2] * kQkScale), static_cast<_Float16>(v[3] * kQkScale)};
              *reinterpret_cast<u32x2_t*>(static_cast<uint16_t*>(ep.out) + row_out + col) =
                  u32x2_t{__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b)};
              return;
            }
          } else if constexpr (EPI == EPI_GELU_BWD) {
            float y[4], h[4];
            load_bf16x4(aux + row_aux + col, y);
            static_for<4>([&](auto R) __attribute__((always_inline)) {
              v[R] *= gelu_grad_f32(y[R]);
              h[R] = gelu_f32(y[R]);
            });
            store_x4<OUT_F32>(ep.out2, row_out + col, h);
          } else {
            if constexpr (kBias) {
              float b[4];
              load_bf16x4(bias + n_lane + col, b);
              static_for<4>([&](auto R) __attribute__((always_inline)) { v[R] += b[R]; });
            }
            if constexpr (EPI == EPI_GELU) {
              if constexpr (kExtra) store_x4<OUT_F32>(ep.pre, row_out + col, v);
              static_for<4>([&](auto R) __attribute__((always_inline)) { v[R] = gelu_f32(v[R]); });
            }
            if constexpr (kRes) {
              float r[4];
              load_bf16x4(residual + row_res + col, r);
              static_for<4>([&](auto R) __attribute__((always_inline)) { v[R] += r[R]; });
            }
          }
          store_x4<OUT_F32>(ep.out, row_out + col, v);
        });
        // keep the accumulator reads of one 32x32 block next to its stores
        // (hoisting all of them ahead of the stores would spill)
        sched_fence();
      });
    });
  };
  using T = std::true_type;
  using F = std::false_type;
  if constexpr (EPI == EPI_GELU_BWD && !MASKED) {
    // All of the tile's saved pre-activations are loaded first (one memory
    // latency per tile instead of one per 32 x 32 block), then one sweep
    // forms acc * GeLU'(y) and GeLU(y).
    u32x2_t yv[TM][TN][4];
    static_for<TM>([&](auto I) __attribute__((always_inline)) {
      static_for<TN>([&](auto J) __attribute__((always_inline)) {
        static_for<4>([&](auto G) __attribute__((always_inline)) {
          const int64_t row_aux =
              static_cast<int64_t>(m_lane + I * 32 + row_of<MF16>(G)) * ep.ldaux + n_lane;
          yv[I][J][G] = *reinterpret_cast<const u32x2_t*>(aux + row_aux + J * 32 + col_of<MF16>(G));
        });
      });
    });
    static_for<TM>([&](auto I) __attribute__((always_inline)) {
      static_for<TN>([&](auto J) __attribute__((always_inline)) {
        static_for<4>([&](auto G) __attribute__((always_inline)) {
          const int64_t row_out =
              static_cast<int64_t>(m_lane + I * 32 + row_of<MF16>(G)) * ep.ldo + n_lane;
          const float y[4] = {__uint_as_float(yv[I][J][G][0] << 16),
                              __uint_as_float(yv[I][J][G][0] & 0xFFFF0000u),
                              __uint_as_float(yv[I][J][G][1] << 16),
                              __uint_as_float(yv[I][J][G][1] & 0xFFFF0000u)};
          float v[4], h[4];
          static_for<4>([&](auto R) __attribute__((always_inline)) {
            v[R] = acc[J][I][4 * G + R] * gelu_grad_f32(y[R]);
            h[R] = gelu_f32(y[R]);
          });
          store_x4<OUT_F32>(ep.out, row_out + J * 32 + col_of<MF16>(G), v);
          store_x4<OUT_F32>(ep.out2, row_out + J * 32 + col_of<MF16>(G), h);
        });
        sched_fence();
      });
    });
  } else if constexpr (EPI == EPI_GELU_BWD || EPI == EPI_QKV_F16) {
    epilogue(F{}, F{}, F{});
  } else if constexpr (EPI == EPI_GELU) {
    if (bias != nullptr) {
      if (ep.pre != nullptr) epilogue(T{}, F{}, T{}); else epilogue(T{}, F{}, F{});
    } else {
      if (ep.pre != nullptr) epilogue(F{}, F{}, T{}); else epilogue(F{}, F{}, F{});
    }
  } else if (bias != nullptr) {
    if (residual != nullptr) epilogue(T{}, T{}, F{}); else epilogue(T{}, F{}, F{});
  } else {
    if (residual != nullptr) epilogue(F{}, T{}, F{}); else epilogue(F{}, F{}, F{});
  }
}

// Interleave for one k-substep: kM MFMAs; before MFMA i the scheduler is asked
// for the next substep's LDS fragment reads (front-loaded, kR in total).
template <int kM, int kR>
__device__ __forceinline__ void interleave_substep() {
  static_for<kM>([&](auto I) __attribute__((always_inline)) {
    constexpr int i = I;
    sched_group<kSchedMfma, 1>();
    constexpr int r = (i == kM - 1) ? (kR > i ? kR - i : 0) : (i < kR ? 1 : 0);
    if constexpr (r > 0) sched_group<kSchedDsRead, r>();
  });
}

}  // namespace gemm_detail

// One explicit instantiation set per (tile shape, epilogue kind, output type).
// Both launchers are defined once, in gemm_bf16_dma.h; each gemm_bf16_*.hip
// unit instantiates its share of them (so that the units compile in
// parallel), and callers that see only these declarations link to those
// instantiations.
template <int BM, int BN, int EPI, bool OUT_F32>
hipError_t launch_gemm_bf16_cfg(const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb,
                                int M, int N, int K, const Epilogue& ep, hipStream_t stream);

// Products with k-major flags (256 x 256 or 128 x 128 tiles, copy kernel);
// instantiated in the gemm_bf16_{256,128}_{nt,tn,swiglu}.hip units.
template <int BM, int BN, bool A_KMAJOR, bool B_KMAJOR, int EPI, bool OUT_F32>
hipError_t launch_gemm_bf16_t_cfg(const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb,
                                  int M, int N, int K, const Epilogue& ep, hipStream_t stream);

}  // namespace tpk
