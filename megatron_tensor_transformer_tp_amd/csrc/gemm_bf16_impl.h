// bf16 GEMM with fp32 accumulation on gfx950 matrix cores, with the
// column-/row-parallel epilogues fused in (kernel template; the launch
// configurations are instantiated in gemm_bf16_*.hip, one translation unit
// per tile shape and output type, so that they compile in parallel).
//
//   C[M, N] = A[M, K] . B[K, N]      A, B row-major bf16, C fp32 accumulators
//
// The column-parallel linear of a tensor-parallel MLP calls it with
// A = X [tokens, hidden], B = A_i [hidden, f] and the GeLU epilogue; the
// row-parallel linear with A = H_i [tokens, f], B = B_i [f, hidden] and the
// bias/residual epilogue (列并行 tutorial, 数学基础 and MLP 应用; Megatron
// expert interview Level 2, M025/M026).
//
// Design (gfx950, 256 CUs in 8 XCDs, 160 KiB LDS per CU, wave64):
//   * Workgroup = 4 waves (256 threads) computing a BM x BN tile, BK = 64.
//     The 4 waves form a 2 x 2 grid; each owns a (BM/2) x (BN/2) sub-tile as
//     a grid of 32x32 MFMA blocks (v_mfma_f32_32x32x16_bf16).
//   * Operand roles inside the MFMA are swapped (the weight fragment is the
//     MFMA's first operand, the activation fragment the second), so each lane
//     ends up owning 4 CONSECUTIVE output columns of one row: the epilogue
//     stores 16-byte fp32 or 8-byte bf16 vectors.
//   * Both operands are staged in LDS as [row][k] with k contiguous and a
//     row pitch of 72 elements (144 B = 9 x 16 B).  An MFMA fragment is one
//     16-byte ds_read per lane; 16 lanes reading 16 consecutive rows at the
//     same k hit 16 distinct 16-byte bank groups.
//   * The row-major weight tile [BK, BN] has n contiguous in memory but the
//     MFMA wants k contiguous per lane: each loader thread fetches an 8x8
//     block (8 rows of 16 B) and transposes it in registers with v_perm_b32
//     before the 16-byte LDS stores.
//   * Two LDS stages (2 x (BM + BN) x 144 B; 144 KiB for 256 x 256) and a
//     register prefetch of the next k-tile: global loads for k-tile t+1 are
//     in flight while the MFMAs consume k-tile t; one barrier per k-tile.
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

constexpr int kBK = 64;
constexpr int kPitch = kBK + 8;  // LDS row pitch in bf16 elements (144 B)
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

__device__ __forceinline__ u32x4_t zero4() { return u32x4_t{0u, 0u, 0u, 0u}; }

// Scheduling fence between the k-substeps of the main loop: nothing moves
// across it, so the LDS reads issued in substep s for substep s+1 stay ahead
// of the MFMAs of substep s (the default scheduler would sink them next to
// their uses and expose the LDS latency to the matrix pipe).
__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

// Within a substep, an explicit interleave: each MFMA is followed by one of
// the substep's memory operations, LDS reads for the next substep first.
constexpr int kSchedValu = 0x002;
constexpr int kSchedMfma = 0x008;
constexpr int kSchedVmemRead = 0x020;
constexpr int kSchedDsRead = 0x100;
constexpr int kSchedDsWrite = 0x200;

template <int MASK, int N>
__device__ __forceinline__ void sched_group() {
  __builtin_amdgcn_sched_group_barrier(MASK, N, 0);
}

// Epilogue shared by the GEMM kernels.  acc[j][i][4g + r] is C[m][n] with
//   m = m_lane + i*32,  n = n_lane + j*32 + 8g + r,
// i.e. each lane owns 4 consecutive columns per (i, j, g): one 16-byte fp32
// or 8-byte bf16 store.  EPI selects the epilogue kind at compile time; the
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

template <int TM, int TN, bool MASKED, int EPI, bool OUT_F32>
__device__ __forceinline__ void store_tile(const f32x16_t (&acc)[TN][TM], int m_lane, int n_lane,
                                           int M, int N, const Epilogue& ep) {
  const uint16_t* __restrict__ bias = static_cast<const uint16_t*>(ep.bias);
  const uint16_t* __restrict__ residual = static_cast<const uint16_t*>(ep.residual);
  const uint16_t* __restrict__ aux = static_cast<const uint16_t*>(ep.aux);
  uint16_t* __restrict__ out_lo = static_cast<uint16_t*>(ep.out_lo);
  auto epilogue = [&](auto has_bias, auto has_res, auto has_extra) __attribute__((always_inline)) {
    constexpr bool kBias = decltype(has_bias)::value;
    constexpr bool kRes = decltype(has_res)::value;
    constexpr bool kExtra = decltype(has_extra)::value;   // pre (GeLU) or out_lo (linear)
    static_for<TM>([&](auto I) __attribute__((always_inline)) {
      const int m = m_lane + I * 32;
      if (MASKED && m >= M) return;
      const int64_t row_out = static_cast<int64_t>(m) * ep.ldo + n_lane;
      const int64_t row_res = kRes ? static_cast<int64_t>(m) * ep.ldr + n_lane : 0;
      const int64_t row_aux = EPI == EPI_GELU_BWD ? static_cast<int64_t>(m) * ep.ldaux + n_lane : 0;
      static_for<TN>([&](auto J) __attribute__((always_inline)) {
        static_for<4>([&](auto G) __attribute__((always_inline)) {
          constexpr int col = J * 32 + G * 8;
          if (MASKED && n_lane + col >= N) return;
          float v[4];
          static_for<4>([&](auto R) __attribute__((always_inline)) { v[R] = acc[J][I][4 * G + R]; });
          if constexpr (EPI == EPI_QKV_F16) {
            static_assert(!OUT_F32, "the packed projection is 16-bit");
            // every wave's columns lie in one 128-column part (wave widths 64
            // or 128 at 64-aligned offsets), so the part is wave-uniform
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
          if constexpr (EPI == EPI_LINEAR && kExtra && !OUT_F32) {
            float lo[4];
            static_for<2>([&](auto P) __attribute__((always_inline)) {
              const uint32_t hi = pack_bf16x2(v[2 * P], v[2 * P + 1]);
              lo[2 * P] = v[2 * P] - __uint_as_float(hi << 16);
              lo[2 * P + 1] = v[2 * P + 1] - __uint_as_float(hi & 0xFFFF0000u);
            });
            store_x4<false>(out_lo, row_out + col, lo);
          }
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
      const int64_t row_aux = static_cast<int64_t>(m_lane + I * 32) * ep.ldaux + n_lane;
      static_for<TN>([&](auto J) __attribute__((always_inline)) {
        static_for<4>([&](auto G) __attribute__((always_inline)) {
          yv[I][J][G] = *reinterpret_cast<const u32x2_t*>(aux + row_aux + J * 32 + G * 8);
        });
      });
    });
    static_for<TM>([&](auto I) __attribute__((always_inline)) {
      const int64_t row_out = static_cast<int64_t>(m_lane + I * 32) * ep.ldo + n_lane;
      static_for<TN>([&](auto J) __attribute__((always_inline)) {
        static_for<4>([&](auto G) __attribute__((always_inline)) {
          const float y[4] = {__uint_as_float(yv[I][J][G][0] << 16),
                              __uint_as_float(yv[I][J][G][0] & 0xFFFF0000u),
                              __uint_as_float(yv[I][J][G][1] << 16),
                              __uint_as_float(yv[I][J][G][1] & 0xFFFF0000u)};
          float v[4], h[4];
          static_for<4>([&](auto R) __attribute__((always_inline)) {
            v[R] = acc[J][I][4 * G + R] * gelu_grad_f32(y[R]);
            h[R] = gelu_f32(y[R]);
          });
          store_x4<OUT_F32>(ep.out, row_out + J * 32 + G * 8, v);
          store_x4<OUT_F32>(ep.out2, row_out + J * 32 + G * 8, h);
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
  } else if (out_lo != nullptr) {
    epilogue(F{}, F{}, T{});
  } else if (bias != nullptr) {
    if (residual != nullptr) epilogue(T{}, T{}, F{}); else epilogue(T{}, F{}, F{});
  } else {
    if (residual != nullptr) epilogue(F{}, T{}, F{}); else epilogue(F{}, F{}, F{});
  }
}

// Interleave for one k-substep: kM MFMAs; before MFMA i the scheduler is asked
// for the substep's next LDS fragment reads (front-loaded, kR in total), and a
// proportional share of its VALU ops (kP), LDS stores (kW) and global loads (kV).
template <int kM, int kR, int kP, int kW, int kV>
__device__ __forceinline__ void interleave_substep() {
  static_for<kM>([&](auto I) __attribute__((always_inline)) {
    constexpr int i = I;
    sched_group<kSchedMfma, 1>();
    constexpr int r = (i == kM - 1) ? (kR > i ? kR - i : 0) : (i < kR ? 1 : 0);
    if constexpr (r > 0) sched_group<kSchedDsRead, r>();
    constexpr int p = (i + 1) * kP / kM - i * kP / kM;
    if constexpr (p > 0) sched_group<kSchedValu, p>();
    constexpr int w = (i + 1) * kW / kM - i * kW / kM;
    if constexpr (w > 0) sched_group<kSchedDsWrite, w>();
    constexpr int v = (i + 1) * kV / kM - i * kV / kM;
    if constexpr (v > 0) sched_group<kSchedVmemRead, v>();
  });
}

// BM x BN tile per workgroup of WGM x WGN waves; each wave owns a
// (BM/WGM) x (BN/WGN) sub-tile of 32x32 MFMA blocks.
template <int BM, int BN, int WGM, int WGN, bool MASKED, int EPI, bool OUT_F32>
__global__ __launch_bounds__(64 * WGM * WGN) void gemm_bf16_kernel(
    const uint16_t* __restrict__ A, int64_t lda, const uint16_t* __restrict__ B, int64_t ldb,
    int M, int N, int K, const Epilogue ep) {
  constexpr int NT = 64 * WGM * WGN;
  constexpr int WM = BM / WGM, WN = BN / WGN;
  constexpr int TM = WM / 32, TN = WN / 32;
  constexpr int A_CHUNKS = BM * kBK / 8 / NT;  // 16-byte chunks of the A tile per thread
  constexpr int RB = kBK * BN / 8 / NT;        // k-rows of the B tile per thread (x 8 columns)
  constexpr int KG = kBK / RB;                 // k-groups of RB rows
  static_assert(A_CHUNKS >= 1 && (RB == 2 || RB == 4 || RB == 8) && KG * (BN / 8) == NT,
                "tile / thread shape");

  __shared__ __attribute__((aligned(16))) uint16_t sA[2][BM * kPitch];
  __shared__ __attribute__((aligned(16))) uint16_t sB[2][BN * kPitch];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: lives in an SGPR
  const int wm = wave / WGN, wn = wave % WGN;

  int tm, tn;
  tile_coords(blockIdx.x, gridDim.x, (M + BM - 1) / BM, (N + BN - 1) / BN, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int nk = (K + kBK - 1) / kBK;

  // A loader: chunk i of thread t is row i*(NT/8) + t/8, k-chunk t%8.
  const int a_row = tid >> 3, a_kc = tid & 7;
  // B loader: thread t covers k-rows (t%KG)*RB .. +RB-1 of columns (t/KG)*8 .. +7.
  const int b_kb = tid % KG, b_nb = tid / KG;

  u32x4_t ra[A_CHUNKS];
  u32x4_t rb[RB];

  auto load_a = [&](int kt) __attribute__((always_inline)) {
    const int k0 = kt * kBK;
    static_for<A_CHUNKS>([&](auto I) __attribute__((always_inline)) {
      const int gm = m0 + I * (NT / 8) + a_row, gk = k0 + a_kc * 8;
      if (!MASKED || (gm < M && gk < K))
        ra[I] = *reinterpret_cast<const u32x4_t*>(A + static_cast<int64_t>(gm) * lda + gk);
      else
        ra[I] = zero4();
    });
  };
  auto load_b = [&](int kt) __attribute__((always_inline)) {
    const int k0 = kt * kBK;
    static_for<RB>([&](auto J) __attribute__((always_inline)) {
      const int gk = k0 + b_kb * RB + J, gn = n0 + b_nb * 8;
      if (!MASKED || (gk < K && gn < N))
        rb[J] = *reinterpret_cast<const u32x4_t*>(B + static_cast<int64_t>(gk) * ldb + gn);
      else
        rb[J] = zero4();
    });
  };
  auto store_a = [&](int buf) __attribute__((always_inline)) {
    static_for<A_CHUNKS>([&](auto I) __attribute__((always_inline)) {
      *reinterpret_cast<u32x4_t*>(&sA[buf][(I * (NT / 8) + a_row) * kPitch + a_kc * 8]) = ra[I];
    });
  };
  auto store_b = [&](int buf) __attribute__((always_inline)) {
    // rb[j] holds B[k0 + kb*RB + j][n0 + nb*8 .. +7]; column e of this RB x 8
    // block becomes RB consecutive k values of LDS row n = nb*8 + e.
    static_for<8>([&](auto E) __attribute__((always_inline)) {
      constexpr int q = E >> 1;
      constexpr uint32_t sel = (E & 1) ? 0x07060302u : 0x05040100u;
      uint16_t* dst = &sB[buf][(b_nb * 8 + E) * kPitch + b_kb * RB];
      if constexpr (RB == 8) {
        u32x4_t t;
        t[0] = __builtin_amdgcn_perm(rb[1][q], rb[0][q], sel);
        t[1] = __builtin_amdgcn_perm(rb[3][q], rb[2][q], sel);
        t[2] = __builtin_amdgcn_perm(rb[5][q], rb[4][q], sel);
        t[3] = __builtin_amdgcn_perm(rb[7][q], rb[6][q], sel);
        *reinterpret_cast<u32x4_t*>(dst) = t;
      } else if constexpr (RB == 4) {
        u32x2_t t;
        t[0] = __builtin_amdgcn_perm(rb[1][q], rb[0][q], sel);
        t[1] = __builtin_amdgcn_perm(rb[3][q], rb[2][q], sel);
        *reinterpret_cast<u32x2_t*>(dst) = t;
      } else {
        *reinterpret_cast<uint32_t*>(dst) = __builtin_amdgcn_perm(rb[1][q], rb[0][q], sel);
      }
    });
  };

  // MFMA operand fragments, double-buffered by k-substep parity.
  const int frag_row = lane & 31;
  const int frag_k = (lane >> 5) * 8;
  const int a_frag = (wm * WM + frag_row) * kPitch + frag_k;
  const int b_frag = (wn * WN + frag_row) * kPitch + frag_k;
  bf16x8_t af0[TM], bf0[TN], af1[TM], bf1[TN];
  auto read_frags = [&](int buf, int s, bf16x8_t(&af)[TM], bf16x8_t(&bf)[TN])
      __attribute__((always_inline)) {
    const uint16_t* a_s = sA[buf] + a_frag + s * 16;
    const uint16_t* b_s = sB[buf] + b_frag + s * 16;
    static_for<TM>([&](auto I) __attribute__((always_inline)) {
      af[I] = *reinterpret_cast<const bf16x8_t*>(a_s + I * 32 * kPitch);
    });
    static_for<TN>([&](auto J) __attribute__((always_inline)) {
      bf[J] = *reinterpret_cast<const bf16x8_t*>(b_s + J * 32 * kPitch);
    });
  };

  f32x16_t acc[TN][TM];
  static_for<TN>([&](auto J) __attribute__((always_inline)) {
    static_for<TM>([&](auto I) __attribute__((always_inline)) {
      acc[J][I] = (f32x16_t)(0.0f);
    });
  });
  auto mfmas = [&](const bf16x8_t(&af)[TM], const bf16x8_t(&bf)[TN]) __attribute__((always_inline)) {
    static_for<TN>([&](auto J) __attribute__((always_inline)) {
      static_for<TM>([&](auto I) __attribute__((always_inline)) {
        acc[J][I] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bf[J], af[I], acc[J][I], 0, 0, 0);
      });
    });
  };

  // Software pipeline over k-tiles (4 k-substeps of 16 each).  In iteration kt
  // the registers ra/rb hold k-tile kt+1 (loaded one iteration earlier):
  //   s0: LDS-store A of tile kt+1 into the other stage, issue global loads of
  //       A for tile kt+2, read fragments of s1, MFMAs of s0
  //   s1: same for B (with the in-register transposes), fragments of s2, MFMAs of s1
  //   s2: fragments of s3, MFMAs of s2
  //   s3: barrier (tile kt+1 complete in the other stage, all reads of this
  //       stage done), fragments of tile kt+1 s0, MFMAs of s3
  // The prefetch index is clamped to the last tile, so the loop body has no
  // branches; the clamped loads re-read a tile that is never consumed.
  load_a(0);
  load_b(0);
  store_a(0);
  store_b(0);
  const int k_second = nk > 1 ? 1 : 0;
  load_a(k_second);
  load_b(k_second);
  __syncthreads();
  read_frags(0, 0, af0, bf0);

  constexpr int kFrags = TM + TN;
  constexpr int kMfma = TM * TN;
  constexpr int kPermsB = 8 * (RB / 2);
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1, nxt = cur ^ 1;
    const int kpre = min(kt + 2, nk - 1);
    // s0
    read_frags(cur, 1, af1, bf1);
    store_a(nxt);
    load_a(kpre);
    mfmas(af0, bf0);
    interleave_substep<kMfma, kFrags, 0, A_CHUNKS, A_CHUNKS>();
    sched_fence();
    // s1
    read_frags(cur, 2, af0, bf0);
    store_b(nxt);
    load_b(kpre);
    mfmas(af1, bf1);
    interleave_substep<kMfma, kFrags, kPermsB, 8, RB>();
    sched_fence();
    // s2
    read_frags(cur, 3, af1, bf1);
    mfmas(af0, bf0);
    interleave_substep<kMfma, kFrags, 0, 0, 0>();
    sched_fence();
    // s3: tile kt+1 is complete in the other stage after the barrier
    __syncthreads();
    read_frags(nxt, 0, af0, bf0);
    mfmas(af1, bf1);
    interleave_substep<kMfma, kFrags, 0, 0, 0>();
    sched_fence();
  }

  store_tile<TM, TN, MASKED, EPI, OUT_F32>(acc, m0 + wm * WM + (lane & 31), n0 + wn * WN + (lane >> 5) * 4,
                                          M, N, ep);
}

template <int BM, int BN, int WGM, int WGN, int EPI, bool OUT_F32>
hipError_t launch_tile(const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb, int M,
                       int N, int K, const Epilogue& ep, hipStream_t stream) {
  const int tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  const bool masked = (M % BM) || (N % BN) || (K % kBK);
  const dim3 block(64 * WGM * WGN);
  if (masked)
    hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, WGM, WGN, true, EPI, OUT_F32>), dim3(tiles), block,
                       0, stream, A, lda, B, ldb, M, N, K, ep);
  else
    hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, WGM, WGN, false, EPI, OUT_F32>), dim3(tiles), block,
                       0, stream, A, lda, B, ldb, M, N, K, ep);
  return hipGetLastError();
}

}  // namespace gemm_detail

// One explicit instantiation set per (tile shape, epilogue kind, output type);
// defined in the gemm_bf16_*.hip translation units.
template <int BM, int BN, int EPI, bool OUT_F32>
hipError_t launch_gemm_bf16_cfg(const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb,
                                int M, int N, int K, const Epilogue& ep, hipStream_t stream);

// Tile-aligned products with k-major flags (256 x 256 tiles, copy kernel);
// defined in the gemm_bf16_256_*.hip translation units.
template <bool A_KMAJOR, bool B_KMAJOR, int EPI, bool OUT_F32>
hipError_t launch_gemm_bf16_t_cfg(const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb,
                                  int M, int N, int K, const Epilogue& ep, hipStream_t stream);

}  // namespace tpk
