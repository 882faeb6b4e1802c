// bf16 GEMM, C[M,N] = A[M,K] . B[K,N], fp32 accumulation on the gfx950 matrix
// cores, with both operand tiles brought into LDS by the asynchronous
// global->LDS copy (global_load_lds_dwordx4) instead of through registers.
// Each operand is stored either with k contiguous ("row-major in k": A as
// [M, K], B as [N, K]) or k-major (A as [K, M], B as [K, N]); the two LDS
// layouts below serve either operand.
//
//   * k-tiles of 32, STAGES LDS stages of (BM + BN) x 64 B (32 KiB each for
//     256 x 256): tiles kt+1 .. kt+STAGES-1 are in flight while tile kt is
//     multiplied (4 stages measured faster than 5 at the headline shapes).
//   * Each copy instruction moves 1 KiB: lane t's 16 bytes land at
//     LDS base + 16 t.  The lane -> global address map applies the LDS swizzle,
//     so the bytes of a 16-byte chunk are never split.
//   * k-contiguous operand (activations in the forward): rows of 64 B = 4
//     chunks; logical chunk c of row r sits at chunk c ^ ((r >> 2) & 3).  An
//     MFMA fragment (16 consecutive rows, one chunk each) is one ds_read_b128
//     per lane and touches 16 distinct 16-byte bank groups.
//   * k-major operand (weights [in, out] in the forward): k-rows of R*2
//     bytes as in memory; logical chunk c of k-row r sits at chunk
//     c ^ ((r & 3) << 2) (with the 16 x 16 x 32 MFMA also ^ 2 for k-rows with
//     bit 3 set).  The MFMA wants 8 consecutive k per lane for one row:
//     ds_read_b64_tr_b16 gives it directly (within each 16-lane group, lane
//     4r+c points at 4 consecutive elements of k-row r, and lane i receives
//     column i of the resulting 4 x 16 block), two reads per fragment; the
//     four k-rows of one read fall in four different 64-byte bank windows.
//   * The MFMA is v_mfma_f32_16x16x32_bf16 (one per 16 x 16 output block and
//     k-tile, MF16) or v_mfma_f32_32x32x16_bf16 (two k-substeps per k-tile);
//     all launchers use the former, which the power-capped part runs faster
//     (see kMf16 at the end of this file).
//   * Synchronisation is explicit: before the barrier that publishes tile
//     kt+1 each wave waits (s_waitcnt vmcnt) only for its own copies of that
//     tile, never for the younger tiles in flight; the barrier is a bare
//     s_barrier with a compiler memory clobber (a workgroup fence would make
//     the compiler drain every outstanding copy).
//   * A k-contiguous B with K % 64 == 0 (the backward's products against a
//     weight stored [N, K]) is copied two k-tiles at a time into pair stages
//     of 128-byte rows (OperandPairTile), so that each copy instruction
//     reads whole cache lines; A keeps single stages.
//   * The grid is one round of resident workgroups; each loops over the tiles
//     a one-tile-per-workgroup grid would give it, in the same order, and
//     starts the next tile's first k-tiles before the current epilogue when
//     the epilogue leaves their stages alone.
//   * Ragged shapes: the copy cannot zero-fill, so every copy source is
//     clamped into the operand instead.  Rows (k-contiguous) or 8-column
//     chunks (k-major) past M or N re-read the last valid one; their products
//     reach only outputs that the masked epilogue of an edge tile does not
//     store.  A K that is not a multiple of 32 (KTAIL) leaves fewer than 32
//     valid k, [klast, K), in the last k-tile (klast = 32 (nk - 1)): that
//     tile is copied from the window of the last 32 k,
//     [K - 32, K) (one uniform offset on every lane's source, so the tail
//     holds no per-lane registers), and its fragments are zeroed outside the
//     k not yet accumulated, [klast, K), before the last MFMAs.  With
//     K < 32 the window is [0, 32) and each lane's k (k-contiguous: its
//     8-k chunk; k-major: its k-row) is clamped to the last valid one.
//     Requirements: 16-byte aligned bases and leading dimensions, a
//     k-contiguous operand's K and a k-major operand's row length multiples
//     of 8.
#pragma once

#include "gemm_bf16_impl.h"

namespace tpk {
namespace gemm_detail {

typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef short i16x8_t __attribute__((ext_vector_type(8)));
#define TPK_LDS(T, p) ((__attribute__((address_space(3))) T*)(p))

// One operand's share of a k-tile: R rows (M or N) x kBKd k, copied by NW
// waves (Q copies of 1 KiB each per wave).  MF16: the fragments are read for
// the 16 x 16 x 32 MFMA (see frag16), and a k-major tile's swizzle also
// flips chunk bit 1 on k-rows with bit 3 set.
template <int R, int NW, bool KMAJOR, bool KTAIL, bool MF16 = false>
struct OperandTile {
  static constexpr int kBytes = R * kBKd * 2;
  static constexpr int Q = kBytes / 1024 / NW;
  static constexpr int CB = R / 8;     // 16-byte chunks per k-row (k-major)
  static_assert(Q * NW * 1024 == kBytes && (!KMAJOR || CB >= 16), "operand tile shape");

  // Physical chunk of logical chunk c of k-row r (an involution, so it also
  // maps a physical chunk back to its logical one).  The frag16 reads of one
  // instruction cover k-rows 8g + 0..3 of the four 16-lane groups g; bit 3 of
  // the k-row puts groups 0 / 1 (and 2 / 3), which share a cycle, in
  // different 16-byte bank groups.
  static __device__ __forceinline__ int kswz(int r) {
    return ((r & 3) << 2) ^ (MF16 ? ((r >> 3) & 1) << 1 : 0);
  }

  const uint16_t* src[Q];   // sources of k-tile 0
  int64_t step;             // elements per k-tile
  int64_t unit;             // elements per k
  int kbase;                // KTAIL: first k of the last k-tile's window

  __device__ __forceinline__ void set_steps(int64_t ld, int K) {
    unit = KMAJOR ? ld : 1;
    step = kBKd * unit;
    kbase = max(K - kBKd, 0);
  }

  // Per-lane copy sources for the rows [r0, r0 + R) of an operand with `rows`
  // rows (k-contiguous: rows of [rows, K]; k-major: columns of [K, rows],
  // rows % 8 == 0), clamped to the last row / chunk, and with KTAIL to the
  // last valid k (which changes nothing unless K < 32).
  __device__ __forceinline__ void init(const uint16_t* base, int64_t ld, int r0, int rows, int K,
                                       int wave, int lane) {
    static_for<Q>([&](auto I) __attribute__((always_inline)) {
      const int slot = (wave * Q + I) * 64 + lane;
      if constexpr (!KMAJOR) {
        const int row = slot >> 2, kin = 8 * ((slot & 3) ^ ((row >> 2) & 3));
        src[I] = base + static_cast<int64_t>(min(r0 + row, rows - 1)) * ld +
                 (KTAIL ? min(kin, K - 8) : kin);
      } else {
        const int krow = slot / CB, c = (slot % CB) ^ kswz(krow);
        src[I] = base + min(r0 + 8 * c, rows - 8) +
                 static_cast<int64_t>(KTAIL ? min(krow, K - 1) : krow) * ld;
      }
    });
    set_steps(ld, K);
  }

  // SwiGLU form of a k-major weight tile: LDS columns in 32-column blocks
  // alternating between the gate projection (even blocks) and the value
  // projection (odd blocks) of the same 32 features, so an MFMA wave whose
  // 64 columns start on an even block holds gate and value of 32 features.
  // Features [f0, f0 + R/2) of both projections (same ld) of `feats`
  // features, clamped to the last 8-feature chunk.
  __device__ __forceinline__ void init_dual(const uint16_t* gate, const uint16_t* value, int64_t ld,
                                            int f0, int feats, int K, int wave, int lane) {
    static_assert(KMAJOR, "the paired tile is a weight ([K, N]) tile");
    static_for<Q>([&](auto I) __attribute__((always_inline)) {
      const int slot = (wave * Q + I) * 64 + lane;
      const int krow = slot / CB, c = (slot % CB) ^ kswz(krow);
      const int blk = c >> 2;
      const uint16_t* p = ((blk & 1) ? value : gate) +
                          min(f0 + (blk >> 1) * 32 + (c & 3) * 8, feats - 8);
      src[I] = p + static_cast<int64_t>(KTAIL ? min(krow, K - 1) : krow) * ld;
    });
    set_steps(ld, K);
  }

  // Copies of k-tile kc into the LDS region at byte address `lds`.  KTAIL:
  // k-tile kc < nk - 1 starts at 32 kc < kbase, and the last one (kc =
  // nk - 1, 32 kc >= kbase) is the window at kbase, so a uniform min picks
  // the place without a branch.
  __device__ __forceinline__ void issue(int kc, uint32_t lds, int wave) const {
    const int64_t off = KTAIL ? min(kc * kBKd, kbase) * unit : kc * step;   // uniform
    static_for<Q>([&](auto I) __attribute__((always_inline)) {
      copy_to_lds(src[I] + off, lds + (wave * Q + I) * 1024);
    });
  }

  // MFMA fragment of 32 rows starting at row0 (a multiple of 32), k-substep
  // s (k = 16 s .. 16 s + 15): lane l gets row row0 + l % 32, k 16 s + 8 (l / 32) .. +7.
  __device__ __forceinline__ bf16x8_t frag(const uint8_t* st, int row0, int s, int lane) const {
    if constexpr (!KMAJOR) {
      const int chunk = (2 * s + (lane >> 5)) ^ ((lane >> 2) & 3);
      return *TPK_LDS(const bf16x8_t, st + (row0 + (lane & 31)) * 64 + chunk * 16);
    } else {
      const int gi = lane & 15;
      const int row_lane = (lane >> 5) * 8 + (gi >> 2);
      const int chunk = ((row0 >> 3) + ((lane >> 4) & 1) * 2 + ((gi & 3) >> 1)) ^ ((gi >> 2) << 2);
      const int within = (gi & 1) * 8;
      i16x4_t h[2];
      static_for<2>([&](auto H) __attribute__((always_inline)) {
        const int krow = s * 16 + H * 4 + row_lane;
        h[H] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            TPK_LDS(i16x4_t, st + krow * (R * 2) + chunk * 16 + within));
      });
      const i16x8_t v = {h[0][0], h[0][1], h[0][2], h[0][3], h[1][0], h[1][1], h[1][2], h[1][3]};
      return __builtin_bit_cast(bf16x8_t, v);
    }
  }

  // Fragment of the 16 x 16 x 32 MFMA: 16 rows starting at row0 (a multiple
  // of 16), the k-tile's 32 k; lane l gets row row0 + l % 16, k 8 (l / 16) ..
  // +7.  k-contiguous: one ds_read_b128 (the 16 lanes of one k-chunk fall in
  // distinct bank groups).  k-major: two transposed reads; in each 16-lane
  // group g, lane 4r + c points at 4 consecutive rows of k-row 8g + 4H + r.
  __device__ __forceinline__ bf16x8_t frag16(const uint8_t* st, int row0, int lane) const {
    if constexpr (!KMAJOR) {
      const int chunk = (lane >> 4) ^ ((lane >> 2) & 3);
      return *TPK_LDS(const bf16x8_t, st + (row0 + (lane & 15)) * 64 + chunk * 16);
    } else {
      const int gi = lane & 15;
      const int within = (gi & 1) * 8;
      i16x4_t h[2];
      static_for<2>([&](auto H) __attribute__((always_inline)) {
        const int krow = 8 * (lane >> 4) + H * 4 + (gi >> 2);
        const int chunk = ((row0 >> 3) + ((gi & 3) >> 1)) ^ kswz(krow);
        h[H] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            TPK_LDS(i16x4_t, st + krow * (R * 2) + chunk * 16 + within));
      });
      const i16x8_t v = {h[0][0], h[0][1], h[0][2], h[0][3], h[1][0], h[1][1], h[1][2], h[1][3]};
      return __builtin_bit_cast(bf16x8_t, v);
    }
  }
};

// A k-contiguous operand copied two k-tiles at a time: R rows of 64 k, 128
// bytes each, so every copy instruction reads 8 whole 128-byte lines (a
// single k-tile's 64-byte row pieces cost the texture addresser about twice
// as much per byte, which limits a product whose operands are both
// k-contiguous).  Logical chunk c (8 k) of row r sits at chunk
// c ^ ((r >> 1) & 7): the 16 rows read by 16 consecutive lanes of a fragment
// fall in distinct 16-byte bank groups.  K % 64 == 0 (no partial tiles).
template <int R, int NW>
struct OperandPairTile {
  static constexpr int kBytes = R * 2 * kBKd * 2;
  static constexpr int Q = kBytes / 1024 / NW;
  static_assert(Q * NW * 1024 == kBytes, "pair tile shape");

  const uint16_t* src[Q];   // sources of k-tiles 0 and 1

  // Rows [r0, r0 + R) of an operand [rows, K] (row stride ld), clamped to
  // the last row.
  __device__ __forceinline__ void init(const uint16_t* base, int64_t ld, int r0, int rows, int wave,
                                       int lane) {
    static_for<Q>([&](auto I) __attribute__((always_inline)) {
      const int slot = (wave * Q + I) * 64 + lane;
      const int row = slot >> 3, kin = 8 * ((slot & 7) ^ ((row >> 1) & 7));
      src[I] = base + static_cast<int64_t>(min(r0 + row, rows - 1)) * ld + kin;
    });
  }

  // Copies of k-tiles 2j and 2j + 1 into the LDS region at byte address lds.
  __device__ __forceinline__ void issue(int j, uint32_t lds, int wave) const {
    static_for<Q>([&](auto I) __attribute__((always_inline)) {
      copy_to_lds(src[I] + static_cast<int64_t>(j) * (2 * kBKd), lds + (wave * Q + I) * 1024);
    });
  }

  // MFMA fragment of 32 rows starting at row0 (a multiple of 32) from the
  // k-tile half h of the pair, k-substep s: lane l gets row row0 + l % 32,
  // k 16 s + 8 (l / 32) .. +7 of that k-tile.
  __device__ __forceinline__ bf16x8_t frag(const uint8_t* st, int row0, int h, int s, int lane) const {
    const int r = lane & 31;
    const int chunk = (4 * h + 2 * s + (lane >> 5)) ^ ((r >> 1) & 7);
    return *TPK_LDS(const bf16x8_t, st + (row0 + r) * 128 + chunk * 16);
  }

  // The 16 x 16 x 32 MFMA's fragment from k-tile half h: 16 rows from row0
  // (a multiple of 16), lane l gets row row0 + l % 16, k 8 (l / 16) .. +7.
  __device__ __forceinline__ bf16x8_t frag16(const uint8_t* st, int row0, int h, int lane) const {
    const int r = lane & 15;
    const int chunk = (4 * h + (lane >> 4)) ^ ((r >> 1) & 7);
    return *TPK_LDS(const bf16x8_t, st + (row0 + r) * 128 + chunk * 16);
  }
};

// SwiGLU epilogue: acc[0] holds the gate and acc[1] the value of the same 32
// features (see OperandTile::init_dual); out[m, n] = SiLU(gate) * value for
// m < M and n < F (F % 4 == 0).
// (Element mapping of acc as for store_tile; gate and value sub-blocks sit
// at the same place in acc[0] and acc[1].)
template <int TM, bool MASKED, bool OUT_F32, bool MF16>
__device__ __forceinline__ void store_swiglu(const f32x16_t (&acc)[2][TM], int m_lane, int n_lane,
                                             int M, int F, const Epilogue& ep) {
  static_for<TM>([&](auto I) __attribute__((always_inline)) {
    const int m_i = m_lane + I * 32;
    if (!MF16 && MASKED && m_i >= M) return;
    static_for<4>([&](auto G) __attribute__((always_inline)) {
      const int m = m_i + row_of<MF16>(G);
      constexpr int col = col_of<MF16>(G);
      if (MASKED && ((MF16 && m >= M) || n_lane + col >= F)) return;
      float h[4];
      static_for<4>([&](auto R) __attribute__((always_inline)) {
        h[R] = silu_f32(acc[0][I][4 * G + R]) * acc[1][I][4 * G + R];
      });
      store_x4<OUT_F32>(ep.out, static_cast<int64_t>(m) * ep.ldo + n_lane + col, h);
    });
    sched_fence();
  });
}

// fp32 linear epilogue (bias and residual optional) of an interior tile,
// restaged through LDS: the MFMA layout gives each lane 4 columns of one row,
// so a direct store instruction writes 16-byte pieces of 32 different rows
// (32 cache lines).  Here each wave writes one 32-row slab of its
// accumulators into its own LDS region of kStagedSlabBytes, reads it back
// row by row and stores whole row segments: WN/4 lanes per row, each
// instruction covering 64*16/(WN*4) rows of WN*4 contiguous bytes.  The
// 16-byte chunk c of slab row r sits at chunk c ^ (r & 15) (for W = 64: the
// 16 rows written by 16 consecutive lanes, and the 16 chunks of one row read
// by 16 consecutive lanes, fall in distinct bank groups).  The stores carry
// the non-temporal hint.  The caller guarantees that nothing else reads or
// writes the region meanwhile.
template <int TN>
constexpr int kStagedSlabBytes = 32 * TN * 32 * 4;
template <int TM, int TN, bool MF16>
__device__ __forceinline__ void store_linear_f32_staged(const f32x16_t (&acc)[TN][TM], uint8_t* lds,
                                                        int lane, int m_w, int n_w,
                                                        const Epilogue& ep) {
  typedef float f32x4_t __attribute__((ext_vector_type(4)));
  constexpr int W = TN * 32;            // columns of the wave's sub-tile
  constexpr int PITCH = W * 4;          // bytes per staged row
  constexpr int CPR = W / 4;            // 16-byte chunks per row
  constexpr int SWZ = (CPR < 16 ? CPR : 16) - 1;
  constexpr int LPR = CPR;              // lanes per row
  constexpr int RPI = 64 / LPR;         // rows per store instruction
  static_assert(LPR * RPI == 64 && 32 % RPI == 0 && (CPR & (CPR - 1)) == 0,
                "whole rows per store instruction");
  const uint16_t* __restrict__ bias = static_cast<const uint16_t*>(ep.bias);
  const uint16_t* __restrict__ residual = static_cast<const uint16_t*>(ep.residual);
  const int col = (lane % LPR) * 4, rsub = lane / LPR;
  auto body = [&](auto has_bias, auto has_res) __attribute__((always_inline)) {
    constexpr bool kBias = decltype(has_bias)::value;
    constexpr bool kRes = decltype(has_res)::value;
    float b[4] = {0.f, 0.f, 0.f, 0.f};
    if constexpr (kBias) load_bf16x4(bias + n_w + col, b);
    static_for<TM>([&](auto I) __attribute__((always_inline)) {
      static_for<TN>([&](auto J) __attribute__((always_inline)) {
        static_for<4>([&](auto G) __attribute__((always_inline)) {
          const f32x4_t v = {acc[J][I][4 * G], acc[J][I][4 * G + 1], acc[J][I][4 * G + 2],
                             acc[J][I][4 * G + 3]};
          // slab row and 16-byte column chunk of this lane's 4 values
          const int r = MF16 ? row_of<true>(G) + (lane & 15) : lane & 31;
          const int c = MF16 ? J * 8 + col_of<true>(G) / 4 + (lane >> 4) : J * 8 + G * 2 + (lane >> 5);
          *TPK_LDS(f32x4_t, lds + r * PITCH + ((c ^ (r & SWZ)) * 16)) = v;
        });
      });
      static_for<32 / RPI>([&](auto Q) __attribute__((always_inline)) {
        const int r = Q * RPI + rsub;
        const f32x4_t v = *TPK_LDS(const f32x4_t, lds + r * PITCH + (((col >> 2) ^ (r & SWZ)) * 16));
        const int64_t m = m_w + I * 32 + r;
        float o[4] = {v[0] + b[0], v[1] + b[1], v[2] + b[2], v[3] + b[3]};
        if constexpr (kRes) {
          float rr[4];
          load_bf16x4(residual + m * ep.ldr + n_w + col, rr);
          static_for<4>([&](auto R) __attribute__((always_inline)) { o[R] += rr[R]; });
        }
        // non-temporal: the output is not read again, and its 64 MB per round
        // (row GEMM) would otherwise evict the next round's operand panels
        // from L2 (+2.6-3.8% on the 8-round fp32 products; whole-line stores
        // only: the scattered direct stores lose with this hint)
        __builtin_nontemporal_store(f32x4_t{o[0], o[1], o[2], o[3]},
                                    reinterpret_cast<f32x4_t*>(static_cast<float*>(ep.out) +
                                                               m * ep.ldo + n_w + col));
      });
    });
  };
  using T = std::true_type;
  using F = std::false_type;
  if (bias != nullptr) {
    if (residual != nullptr) body(T{}, T{}); else body(T{}, F{});
  } else {
    if (residual != nullptr) body(F{}, T{}); else body(F{}, F{});
  }
}

// Keeps the bf16 elements e of a fragment (e counted from the fragment's
// first k, 0 .. 7) with lo <= e < hi and zeroes the others.
__device__ __forceinline__ bf16x8_t keep_range(bf16x8_t v, int lo, int hi) {
  u32x4_t w = __builtin_bit_cast(u32x4_t, v);
  static_for<4>([&](auto D) __attribute__((always_inline)) {
    constexpr int e = 2 * D;
    const uint32_t m = (lo <= e && e < hi ? 0x0000FFFFu : 0u) |
                       (lo <= e + 1 && e + 1 < hi ? 0xFFFF0000u : 0u);
    w[int(D)] &= m;
  });
  return __builtin_bit_cast(bf16x8_t, w);
}

// LDS of one workgroup.  Single k-tile stages: A's STAGES stages of
// BM x 64 bytes, then B's of BN x 64 bytes, so that each operand's stages lie
// in one 64 KiB window and a fragment's LDS address is one register plus an
// immediate offset (the LDS read's 16-bit field) for every stage (stages of
// A and B interleaved put the last ones past 64 KiB, and a k-major operand,
// whose fragments each need an address register of their own, then needs a
// set per stage).  With the fp32 restaging (linear fp32 epilogue, wave widths
// whose rows split evenly over the 64 lanes) the slabs sit in A's last stage,
// B's last stage and the bytes past the stages, so that the next tile's
// first STAGES-1 k-tiles can be in flight during the epilogue.  PAIR 1 (B
// k-contiguous) or 2 (A k-contiguous), K % 64 == 0: STAGES single stages of
// the other operand (rows x 64 bytes), then kPairs stages of the paired
// operand holding two k-tiles each (rows x 128 bytes); the slabs reuse the
// stage area, so with them the next tile starts after the epilogue.
template <int BM, int BN, int WGM, int WGN, int STAGES, int EPI, bool OUT_F32, int PAIR>
struct DmaLayout {
  static constexpr int kWaves = WGM * WGN;
  static constexpr int kTN = BN / WGN / 32;
  static constexpr int kABytes = BM * kBKd * 2;
  static constexpr int kBBytes = BN * kBKd * 2;
  static constexpr int kStage = (BM + BN) * kBKd * 2;
  static constexpr int kPairs = 3;
  static constexpr int kPairBytes = (PAIR == 2 ? BM : BN) * 2 * kBKd * 2;
  static constexpr int kPairAt = STAGES * (PAIR == 2 ? kBBytes : kABytes);
  static constexpr int kBAt = STAGES * kABytes;   // PAIR 0: B's first stage
  static constexpr bool kStaged = EPI == EPI_LINEAR && OUT_F32 && 64 % (BN / WGN / 4) == 0;
  static constexpr bool kPrefetch = PAIR == 0 || !kStaged;   // next tile's copies during the epilogue
  static constexpr int kSlab = kStagedSlabBytes<kTN>;
  static constexpr int kSlabsInA = PAIR ? 0 : kABytes / kSlab;   // in A's last stage
  static constexpr int kSlabsInB = PAIR ? 0 : kBBytes / kSlab;   // in B's last stage
  static constexpr int kStageBytes = PAIR ? kPairAt + kPairs * kPairBytes : STAGES * kStage;
  static constexpr int kSlabsPast = kWaves - kSlabsInA - kSlabsInB;
  static constexpr int kStagingEnd =
      PAIR ? kWaves * kSlab : kStageBytes + (kSlabsPast > 0 ? kSlabsPast : 0) * kSlab;
  static constexpr int kLdsBytes =
      kStaged && kStagingEnd > kStageBytes ? kStagingEnd : kStageBytes;
  // LDS byte offset of wave w's staging slab
  static __device__ __forceinline__ int slab_at(int w) {
    if (PAIR) return w * kSlab;
    if (w < kSlabsInA) return (STAGES - 1) * kABytes + w * kSlab;
    if (w < kSlabsInA + kSlabsInB) return kBAt + (STAGES - 1) * kBBytes + (w - kSlabsInA) * kSlab;
    return kStageBytes + (w - kSlabsInA - kSlabsInB) * kSlab;
  }
  static constexpr int kPerCu = 160 * 1024 / kLdsBytes;   // resident workgroups per CU
  static_assert(kLdsBytes <= 160 * 1024, "LDS");
};

// LDS places of one k-tile in the main loop: single stage, pair stage and
// half of the pair; KNOWN: the k-tile's parity is a compile-time EVEN.
template <bool KNOWN, bool EVEN>
struct KPlace {
  static constexpr bool kParityKnown = KNOWN;
  static constexpr bool kEven = EVEN;
  int a, p, h;
};

template <int BM, int BN, int WGM, int WGN, int STAGES, bool A_KMAJOR, bool B_KMAJOR, int EPI,
          bool OUT_F32, bool KTAIL, int PAIR, bool MF16>
// at least two waves per SIMD (256 x 256: 8 waves of one workgroup; 128 x
// 128: 4 waves each of two workgroups), so at most 256 registers per wave
__global__ __launch_bounds__(64 * WGM * WGN, 2) void gemm_bf16_dma_kernel(
    const uint16_t* __restrict__ A_in, int64_t lda, const uint16_t* __restrict__ B_in, int64_t ldb,
    int M, int N, int K_in, const Epilogue ep_in) {
  // split-K: workgroup set blockIdx.y takes k-slice blockIdx.y of K /
  // gridDim.y and writes its partial product to its own output slab (one
  // set, the whole product, when gridDim.y is 1)
  const int ks = blockIdx.y;
  const int K = K_in / static_cast<int>(gridDim.y);
  const int64_t k0 = static_cast<int64_t>(ks) * K;
  const uint16_t* __restrict__ A = A_in + (A_KMAJOR ? k0 * lda : k0);
  const uint16_t* __restrict__ B = B_in + (B_KMAJOR ? k0 * ldb : k0);
  Epilogue ep = ep_in;
  ep.out = static_cast<float*>(ep_in.out) + ks * ep_in.slab;
  constexpr int NW = WGM * WGN;
  constexpr int WM = BM / WGM, WN = BN / WGN;
  constexpr int TM = WM / 32, TN = WN / 32;
  static_assert(WM % 32 == 0 && WN % 32 == 0, "wave sub-tiles of whole 32 x 32 MFMA blocks");
  static_assert(PAIR == 0 || (!KTAIL && (EPI != EPI_SWIGLU || PAIR == 2) && STAGES == 4 &&
                              (PAIR == 1 ? !B_KMAJOR : PAIR == 2 && !A_KMAJOR)),
                "paired stages: a k-contiguous operand (SwiGLU: A), whole 64-k pairs, 4 single stages");
  static_assert(!MF16 || TM % 2 == 0, "MF16: the k-tile's MFMAs in two halves of whole 32-row blocks");
  using TileA = OperandTile<BM, NW, A_KMAJOR, KTAIL, MF16>;
  using TileB = OperandTile<BN, NW, B_KMAJOR, KTAIL, MF16>;
  using TileP = OperandPairTile<PAIR == 2 ? BM : BN, NW>;
  constexpr int A_BYTES = TileA::kBytes;
  constexpr int B_BYTES = TileB::kBytes;
  constexpr int QS = PAIR == 2 ? TileB::Q : TileA::Q;   // copies per wave of the single operand
  constexpr int STAGE = A_BYTES + TileB::kBytes;
  constexpr int L = TileA::Q + TileB::Q;   // copies per wave per k-tile (single stages)
  static_assert(STAGES >= 3 && STAGES * STAGE <= 160 * 1024, "LDS stages");

  using Layout = DmaLayout<BM, BN, WGM, WGN, STAGES, EPI, OUT_F32, PAIR>;
  static_assert(Layout::kStage == STAGE && Layout::kABytes == A_BYTES &&
                Layout::kPairBytes == TileP::kBytes, "stage sizes");
  constexpr bool kStaged = Layout::kStaged;
  constexpr bool kPrefetch = Layout::kPrefetch;
  constexpr int kPairs = Layout::kPairs;
  constexpr int kPairAt = Layout::kPairAt;
  constexpr int kPairBytes = Layout::kPairBytes;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[Layout::kLdsBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: lives in an SGPR
  const int wm = wave / WGN, wn = wave % WGN;

  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  const int ntiles = tiles_m * tiles_n;
  const int nk = (K + kBKd - 1) / kBKd;
  const int npairs = nk / 2;   // PAIR: nk is even

  // Workgroup b computes tiles b, b + gridDim.x, ...; tile t takes the place
  // workgroup t of a one-tile-per-workgroup grid would (XCD t % 8, round
  // order), so a grid of whole rounds changes no tile's neighbours.
  TileA ta;
  TileB tb;
  TileP tp;
  int m0, n0;
  auto setup = [&](int t) __attribute__((always_inline)) {
    int tm, tn;
    if (!(BM == 256 && BN == 256 && tile_coords_rounds(t, ntiles, tiles_m, tiles_n, tm, tn)))
      tile_coords(t, ntiles, tiles_m, tiles_n, tm, tn);
    m0 = tm * BM;
    n0 = tn * BN;
    if constexpr (PAIR == 2)
      tp.init(A, lda, m0, M, wave, lane);
    else
      ta.init(A, lda, m0, M, K, wave, lane);
    if constexpr (PAIR == 1)
      tp.init(B, ldb, n0, N, wave, lane);
    else if constexpr (EPI == EPI_SWIGLU)
      tb.init_dual(B, static_cast<const uint16_t*>(ep.b2), ldb, n0 / 2, N / 2, K, wave, lane);
    else
      tb.init(B, ldb, n0, N, K, wave, lane);
  };

  // LDS places of k-tile kt: a single-stage operand in its stage
  // kt % STAGES, the paired one in pair stage (kt / 2) % kPairs, half kt % 2.
  const uint32_t smem_base = lds_address(smem);
  auto a_at = [](int ss, int sp) {
    return PAIR == 2 ? kPairAt + sp * kPairBytes : ss * A_BYTES;
  };
  auto b_at = [](int ss, int sp) {
    return PAIR == 1 ? kPairAt + sp * kPairBytes : PAIR == 2 ? ss * B_BYTES : Layout::kBAt + ss * B_BYTES;
  };
  // Copies of k-tile kt of a single-stage operand (clamped to the last
  // tile), and of pair j of the paired one (clamped to the last pair).
  auto issue_a = [&](int kt) __attribute__((always_inline)) {
    ta.issue(min(kt, nk - 1), smem_base + a_at(kt % STAGES, 0), wave);
  };
  auto issue_b = [&](int kt) __attribute__((always_inline)) {
    tb.issue(min(kt, nk - 1), smem_base + b_at(kt % STAGES, 0), wave);
  };
  auto issue_single = [&](int kt) __attribute__((always_inline)) {
    if constexpr (PAIR == 2) issue_b(kt); else issue_a(kt);
  };
  auto issue_pair = [&](int j) __attribute__((always_inline)) {
    const int sp = j % kPairs;
    tp.issue(min(j, npairs - 1), smem_base + (PAIR == 2 ? a_at(0, sp) : b_at(0, sp)), wave);
  };
  // The first k-tiles of the current tile, and the vmcnt that says k-tile 0
  // has landed.  Single stages: k-tiles 0 .. STAGES-2.  Pairs: single 0,
  // pair 0, single 1, single 2, pair 1 (k-tiles 0 .. 3 of the paired operand).
  auto prologue = [&]() __attribute__((always_inline)) {
    if constexpr (PAIR != 0) {
      issue_single(0);
      issue_pair(0);
      issue_single(1);
      issue_single(2);
      issue_pair(1);
    } else {
      static_for<STAGES - 1>([&](auto T) __attribute__((always_inline)) {
        issue_a(T);
        issue_b(T);
      });
    }
  };
  constexpr int kFirstWait = PAIR ? 2 * QS + TileP::Q : (STAGES - 2) * L;
  // "k-tile kt+1 has landed" inside the main loop.  Single stages: every
  // iteration issues L copies per wave (past the end they re-read the last
  // tile into a stage never read again), so only tiles kt+2 .. kt+STAGES-2
  // may be in flight.  Pairs: iteration kt issues the single operand's
  // k-tile kt+3 and, for even kt, the pair of k-tiles kt+4, kt+5 (into the
  // pair stage k-tiles kt-2, kt-1 left); k-tile kt+1 of the single operand
  // was issued in iteration kt-2 and its pair earlier, and after it exactly
  // one single k-tile and one pair have been issued.
  constexpr int kLoopWait = PAIR ? QS + TileP::Q : (STAGES - 3) * L;

  // The lane index of the fragment reads, renewed (opaquely) for every tile:
  // their loop-invariant LDS addresses are then computed per tile instead of
  // being hoisted out of the tile loop and held live through the epilogue.
  int flane = lane;
  bf16x8_t af0[TM], bf0[TN], af1[TM], bf1[TN];
  // Fragments of substep s of the k-tile whose A sits at LDS offset ao and
  // whose B sits at offset bo (half h of a pair).
  auto frags = [&](int ao, int bo, int h, int s, bf16x8_t(&af)[TM], bf16x8_t(&bf)[TN])
      __attribute__((always_inline)) {
    static_for<TM>([&](auto I) __attribute__((always_inline)) {
      if constexpr (PAIR == 2)
        af[I] = tp.frag(smem + ao, wm * WM + I * 32, h, s, flane);
      else
        af[I] = ta.frag(smem + ao, wm * WM + I * 32, s, flane);
    });
    static_for<TN>([&](auto J) __attribute__((always_inline)) {
      if constexpr (PAIR == 1)
        bf[J] = tp.frag(smem + bo, wn * WN + J * 32, h, s, flane);
      else
        bf[J] = tb.frag(smem + bo, wn * WN + J * 32, s, flane);
    });
  };
  auto read_frags = [&](int kt, int s, bf16x8_t(&af)[TM], bf16x8_t(&bf)[TN])
      __attribute__((always_inline)) {
    frags(a_at(kt % STAGES, (kt / 2) % kPairs), b_at(kt % STAGES, (kt / 2) % kPairs), kt & 1, s, af,
          bf);
  };

  f32x16_t acc[TN][TM];
  auto mfmas = [&](const bf16x8_t(&af)[TM], const bf16x8_t(&bf)[TN]) __attribute__((always_inline)) {
    static_for<TN>([&](auto J) __attribute__((always_inline)) {
      static_for<TM>([&](auto I) __attribute__((always_inline)) {
        acc[J][I] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bf[J], af[I], acc[J][I], 0, 0, 0);
      });
    });
  };

  constexpr int kFrags = TM + 2 * TN;
  constexpr int kMfma = TM * TN;

  // MF16 (v_mfma_f32_16x16x32_bf16, one MFMA per 16 x 16 sub-block and
  // k-tile; the smaller accumulator moves fewer register bytes per FLOP,
  // which the power-capped part turns into clock).  A k-tile's MFMAs run in
  // two halves by rows: half h takes the wave's rows h WM/2 .. +WM/2 as TM
  // fragments of 16 rows (af0 / af1), against the 2 TN fragments of 16
  // columns of B (bq), which both halves share.  Sub-block (a, b) of 32 x 32
  // block (J, I) is acc[J][I][4 (2a + b) .. +3].
  bf16x8_t bq[2 * TN];
  auto a_frags16 = [&](int ao, int h, int half, bf16x8_t(&af)[TM]) __attribute__((always_inline)) {
    static_for<TM>([&](auto I) __attribute__((always_inline)) {
      const int row0 = wm * WM + half * (WM / 2) + I * 16;
      if constexpr (PAIR == 2)
        af[I] = tp.frag16(smem + ao, row0, h, flane);
      else
        af[I] = ta.frag16(smem + ao, row0, flane);
    });
  };
  auto b_frag16 = [&](int bo, int h, int j) __attribute__((always_inline)) {
    const int col0 = wn * WN + j * 16;
    if constexpr (PAIR == 1)
      return tp.frag16(smem + bo, col0, h, flane);
    else
      return tb.frag16(smem + bo, col0, flane);
  };
  auto read_a16 = [&](int kt, int half, bf16x8_t(&af)[TM]) __attribute__((always_inline)) {
    a_frags16(a_at(kt % STAGES, (kt / 2) % kPairs), kt & 1, half, af);
  };
  auto read_b16 = [&](int kt) __attribute__((always_inline)) {
    static_for<2 * TN>([&](auto J) __attribute__((always_inline)) {
      bq[J] = b_frag16(b_at(kt % STAGES, (kt / 2) % kPairs), kt & 1, J);
    });
  };
  // The MFMAs of B fragment j against half `half`'s A fragments.
  auto mfmas16_col = [&](const bf16x8_t(&af)[TM], auto HALF, auto JJ) __attribute__((always_inline)) {
    constexpr int j = decltype(JJ)::value, J = j / 2, b = j % 2;
    static_for<TM>([&](auto II) __attribute__((always_inline)) {
      constexpr int i = decltype(II)::value;
      constexpr int I = decltype(HALF)::value * (TM / 2) + i / 2, q = 2 * (i % 2) + b;
      typedef float f32x4_t __attribute__((ext_vector_type(4)));
      f32x4_t c = {acc[J][I][4 * q], acc[J][I][4 * q + 1], acc[J][I][4 * q + 2], acc[J][I][4 * q + 3]};
      c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bq[j], af[i], c, 0, 0, 0);
      acc[J][I][4 * q] = c[0];
      acc[J][I][4 * q + 1] = c[1];
      acc[J][I][4 * q + 2] = c[2];
      acc[J][I][4 * q + 3] = c[3];
    });
  };
  auto mfmas16 = [&](const bf16x8_t(&af)[TM], auto HALF) __attribute__((always_inline)) {
    static_for<2 * TN>([&](auto JJ) __attribute__((always_inline)) { mfmas16_col(af, HALF, JJ); });
  };

  // One k-tile: substep 0 of tile kt (fragments of substep 1 load under its
  // MFMAs), then substep 1: publish tile kt+1, start the copies that reuse
  // the places of tile kt-1 (every wave finished reading them before this
  // barrier), fragments of tile kt+1.  `sel(d)` gives the (single stage, pair
  // stage, half) of tile kt + d: compile-time values in the unrolled loop, so
  // every LDS address is a loop-invariant register plus an immediate offset
  // and the stage arithmetic disappears (+4-6% on the headline shapes).
  // The copies of iteration kt, into the places k-tile kt-1 (and for pairs
  // kt-2, kt-1) left: every wave finished reading them before this
  // iteration's barrier.
  auto issue_copies = [&](int kt, auto sel) __attribute__((always_inline)) {
    constexpr bool kEvenKnown = decltype(sel(0))::kParityKnown;
    const int kn = kt + STAGES - 1;
    if constexpr (PAIR != 2)
      ta.issue(min(kn, nk - 1), smem_base + a_at(sel(STAGES - 1).a, 0), wave);
    if constexpr (PAIR != 0) {
      // the pair of k-tiles kt+4, kt+5 goes where kt-2, kt-1 were
      const int sp = sel(4).p;
      const uint32_t pair_lds = smem_base + (PAIR == 2 ? a_at(0, sp) : b_at(0, sp));
      if constexpr (PAIR == 2)
        tb.issue(min(kn, nk - 1), smem_base + b_at(sel(STAGES - 1).a, 0), wave);
      if constexpr (kEvenKnown) {
        if constexpr (decltype(sel(0))::kEven) tp.issue(min(kt / 2 + 2, npairs - 1), pair_lds, wave);
      } else {
        if ((kt & 1) == 0) tp.issue(min(kt / 2 + 2, npairs - 1), pair_lds, wave);
      }
    } else {
      tb.issue(min(kn, nk - 1), smem_base + b_at(sel(STAGES - 1).a, 0), wave);
    }
  };
  auto ktile = [&](int kt, auto sel) __attribute__((always_inline)) {
    frags(a_at(sel(0).a, sel(0).p), b_at(sel(0).a, sel(0).p), sel(0).h, 1, af1, bf1);
    mfmas(af0, bf0);
    interleave_substep<kMfma, kFrags>();
    sched_fence();
    wait_vmcnt<kLoopWait>();
    lds_barrier();
    issue_copies(kt, sel);
    frags(a_at(sel(1).a, sel(1).p), b_at(sel(1).a, sel(1).p), sel(1).h, 0, af0, bf0);
    mfmas(af1, bf1);
    interleave_substep<kMfma, kFrags>();
    sched_fence();
  };
  // MF16 k-tile: half 0 (A rows half 0 against bq) with A half 1 of kt
  // loading under it; publish k-tile kt+1 and start the copies; half 1 with
  // A half 0 of kt+1 loading, and each B fragment of kt+1 read into bq[j]
  // right after the last MFMA of kt that uses bq[j] (the fences keep each
  // read below those MFMAs, so it can take their register: the B fragments
  // are not double-buffered).
  auto ktile16 = [&](int kt, auto sel) __attribute__((always_inline)) {
    using H0 = std::integral_constant<int, 0>;
    using H1 = std::integral_constant<int, 1>;
    a_frags16(a_at(sel(0).a, sel(0).p), sel(0).h, 1, af1);
    mfmas16(af0, H0{});
    interleave_substep<2 * TN * TM, TM>();
    sched_fence();
    wait_vmcnt<kLoopWait>();
    lds_barrier();
    issue_copies(kt, sel);
    a_frags16(a_at(sel(1).a, sel(1).p), sel(1).h, 0, af0);
    static_for<2 * TN>([&](auto JJ) __attribute__((always_inline)) {
      mfmas16_col(af1, H1{}, JJ);
      sched_fence();
      bq[decltype(JJ)::value] = b_frag16(b_at(sel(1).a, sel(1).p), sel(1).h, decltype(JJ)::value);
    });
    sched_fence();
  };
  // Places of tile kt + d: compile-time from the position U in the unrolled
  // cycle (a multiple of the cycle is a multiple of STAGES, of 2 and of
  // 2 kPairs), or computed at run time.
  constexpr int kCycle = PAIR ? 12 : STAGES;
  static_assert(!PAIR || (kCycle % STAGES == 0 && kCycle % (2 * kPairs) == 0), "unroll cycle");

  int tile = blockIdx.x;
  setup(tile);
  prologue();
  wait_vmcnt<kFirstWait>();
  for (;;) {
    // k-tile 0 of the current tile has landed (each wave waited for its own copies)
    flane = lane;
    asm volatile("" : "+v"(flane));
    lds_barrier();
    if constexpr (MF16) {
      read_a16(0, 0, af0);
      read_b16(0);
    } else {
      read_frags(0, 0, af0, bf0);
    }
    static_for<TN>([&](auto J) __attribute__((always_inline)) {
      static_for<TM>([&](auto I) __attribute__((always_inline)) { acc[J][I] = (f32x16_t)(0.0f); });
    });
    int kt = 0;
    for (; kt + kCycle <= nk - 1; kt += kCycle) {
      static_for<kCycle>([&](auto U) __attribute__((always_inline)) {
        auto sel = [](int d) {
          constexpr int u = decltype(U)::value;
          return KPlace<true, u % 2 == 0>{(u + d) % STAGES, ((u + d) / 2) % kPairs, (u + d) & 1};
        };
        if constexpr (MF16) ktile16(kt + decltype(U)::value, sel); else ktile(kt + decltype(U)::value, sel);
      });
    }
    for (; kt < nk - 1; ++kt) {
      auto sel = [kt](int d) {
        return KPlace<false, false>{(kt + d) % STAGES, ((kt + d) / 2) % kPairs, (kt + d) & 1};
      };
      if constexpr (MF16) ktile16(kt, sel); else ktile(kt, sel);
    }
    if constexpr (MF16) {
      // the last k-tile: its A half 0 is in af0 and its B in bq
      read_a16(nk - 1, 1, af1);
      if constexpr (KTAIL) {
        // the window holds k kbase .. kbase + 31, of which [klast, K) are
        // still to be added; lane l's fragments hold window places
        // 8 (l / 16) .. +7
        const int kbase = max(K - kBKd, 0), klast = (nk - 1) * kBKd;
        const int k_lane = 8 * (flane >> 4);
        const int lo = klast - kbase - k_lane, hi = K - kbase - k_lane;
        static_for<TM>([&](auto I) __attribute__((always_inline)) {
          af0[I] = keep_range(af0[I], lo, hi);
          af1[I] = keep_range(af1[I], lo, hi);
        });
        static_for<2 * TN>([&](auto J) __attribute__((always_inline)) {
          bq[J] = keep_range(bq[J], lo, hi);
        });
      }
      mfmas16(af0, std::integral_constant<int, 0>{});
      mfmas16(af1, std::integral_constant<int, 1>{});
    } else {
      // the last k-tile (its substep-0 fragments are in af0 / bf0)
      read_frags(nk - 1, 1, af1, bf1);
      if constexpr (KTAIL) {
        // window places as above; lane l's fragments of substep s hold
        // places 16 s + 8 (l / 32) .. +7
        const int kbase = max(K - kBKd, 0), klast = (nk - 1) * kBKd;
        const int k_lane = 8 * (flane >> 5);
        const int lo = klast - kbase - k_lane, hi = K - kbase - k_lane;
        static_for<TM>([&](auto I) __attribute__((always_inline)) {
          af0[I] = keep_range(af0[I], lo, hi);
          af1[I] = keep_range(af1[I], lo - 16, hi - 16);
        });
        static_for<TN>([&](auto J) __attribute__((always_inline)) {
          bf0[J] = keep_range(bf0[J], lo, hi);
          bf1[J] = keep_range(bf1[J], lo - 16, hi - 16);
        });
      }
      mfmas(af0, bf0);
      mfmas(af1, bf1);
    }

    // Every stage is free once each wave's copies have landed (the clamped
    // re-reads past the last k-tile included) and its fragment reads have
    // returned, and all waves have passed the barrier after that.  With
    // single stages the next tile's first STAGES-1 k-tiles are then started
    // before this tile's epilogue, which they overlap.
    const int cm0 = m0, cn0 = n0;
    const int next = tile + static_cast<int>(gridDim.x);
    const bool more = next < ntiles;   // workgroup-uniform
    wait_vmcnt<0>();
    if (more || kStaged) {
      sched_fence();
      __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
      lds_barrier();
    }
    if constexpr (kPrefetch) {
      if (more) {
        setup(next);
        prologue();
      }
    }

    // The epilogue's per-lane addresses are loop-invariant; computed from an
    // opaque copy of the lane index they are not hoisted out of the tile
    // loop, where they would stay live through the main loop.
    int elane = lane;
    asm volatile("" : "+v"(elane));
    const bool edge = cm0 + BM > M || cn0 + BN > N;   // workgroup-uniform
    // the lane's row and first column in the accumulator layout
    const int m_lane = cm0 + wm * WM + (MF16 ? elane & 15 : elane & 31);
    const int n_quad = MF16 ? (elane >> 4) * 4 : (elane >> 5) * 4;
    if constexpr (EPI == EPI_SWIGLU) {
      static_assert(TN == 2, "gate and value blocks per wave");
      const int n_lane = cn0 / 2 + wn * (WN / 2) + n_quad;
      if (edge)
        store_swiglu<TM, true, OUT_F32, MF16>(acc, m_lane, n_lane, M, N / 2, ep);
      else
        store_swiglu<TM, false, OUT_F32, MF16>(acc, m_lane, n_lane, M, N / 2, ep);
    } else {
      bool stored = false;
      if constexpr (kStaged) {
        if (!edge) {
          store_linear_f32_staged<TM, TN, MF16>(acc, smem + Layout::slab_at(wave),
                                                elane, cm0 + wm * WM, cn0 + wn * WN, ep);
          stored = true;
        }
      }
      if (!stored) {
        const int n_lane = cn0 + wn * WN + n_quad;
        if (edge)
          store_tile<TM, TN, true, EPI, OUT_F32, MF16>(acc, m_lane, n_lane, M, N, ep);
        else
          store_tile<TM, TN, false, EPI, OUT_F32, MF16>(acc, m_lane, n_lane, M, N, ep);
      }
    }
    if (!more) break;
    // The copy sources are rebuilt from an opaque copy of the tile index, so
    // that the ones used for the prefetch above are not kept live across
    // the epilogue.
    tile = next;
    asm volatile("" : "+s"(tile));
    setup(tile);
    if constexpr (kPrefetch) {
      // the next tile's first k-tile (and everything before it) has landed;
      // waiting for the epilogue's stores as well keeps the count simple
      sched_fence();
      wait_vmcnt<0>();
    } else {
      if constexpr (kStaged) {
        // every wave is done with the slabs before the copies overwrite them
        sched_fence();
        __builtin_amdgcn_s_waitcnt(0xC07F);
        lds_barrier();
      }
      prologue();
      wait_vmcnt<kFirstWait>();
    }
  }
}

// Any M, N >= 1 and K >= 1 within the requirements above (the shape ones
// are checked here; the caller guarantees alignment).
template <int BM, int BN, int WGM, int WGN, int STAGES, bool A_KMAJOR, bool B_KMAJOR, int EPI,
          bool OUT_F32, bool MF16>
hipError_t launch_tile_dma(const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb, int M,
                           int N, int K, const Epilogue& ep, hipStream_t stream) {
  const int b_rows = EPI == EPI_SWIGLU ? N / 2 : N;   // paired tiles: features
  if (M <= 0 || N <= 0 || K <= 0 || ((!A_KMAJOR || !B_KMAJOR) && K % 8 != 0) ||
      (A_KMAJOR && M % 8 != 0) || (B_KMAJOR && b_rows % 8 != 0) ||
      (EPI == EPI_SWIGLU && N % 2 != 0))
    return hipErrorInvalidValue;
  const int64_t tiles = ((static_cast<int64_t>(M) + BM - 1) / BM) * ((static_cast<int64_t>(N) + BN - 1) / BN);
  if (tiles > INT32_MAX) return hipErrorInvalidValue;     // tile indices are ints
  // split-K: whole 64-k pairs per slice, partial products only
  const int ks = ep.ksplit > 1 ? ep.ksplit : 1;
  if (ks > 1 && (EPI != EPI_LINEAR || !OUT_F32 || ep.bias != nullptr || ep.residual != nullptr ||
                 K % (2 * kBKd * ks) != 0 || ks > 65535))
    return hipErrorInvalidValue;
  const int kslice = K / ks;
  // one round of resident workgroups (whole XCD rounds: a multiple of 8),
  // each looping over its tiles
  auto launch = [&](auto ktail, auto pair) {
    constexpr bool kTail = decltype(ktail)::value;
    constexpr int kPair = decltype(pair)::value;
    using Layout = DmaLayout<BM, BN, WGM, WGN, STAGES, EPI, OUT_F32, kPair>;
    int64_t cap = device_cus() * Layout::kPerCu / 8 * 8;
    if (cap < 8) cap = 8;
    const unsigned grid = static_cast<unsigned>(tiles < cap ? tiles : cap);
    hipLaunchKernelGGL(
        (gemm_bf16_dma_kernel<BM, BN, WGM, WGN, STAGES, A_KMAJOR, B_KMAJOR, EPI, OUT_F32, kTail, kPair,
                              MF16>),
        dim3(grid, ks), dim3(64 * WGM * WGN), 0, stream, A, lda, B, ldb, M, N, K, ep);
  };
  using T = std::true_type;
  using F = std::false_type;
  using P0 = std::integral_constant<int, 0>;
  if (kslice % kBKd != 0) {
    launch(T{}, P0{});
  } else {
    // Whole 64-k pairs of a k-contiguous operand: a k-contiguous B takes the
    // paired stages, else a k-contiguous A does (each copy instruction then
    // reads whole 128-byte lines, which the copy path turns into fewer
    // addresser cycles per byte: 256 x 256 headline products 1.7-3.8% faster)
    constexpr int kPair = STAGES != 4                      ? 0
                          : !B_KMAJOR && EPI != EPI_SWIGLU  ? 1
                          : !A_KMAJOR                       ? 2
                                                            : 0;
    if constexpr (kPair != 0) {
      if (kslice % (2 * kBKd) == 0) {
        launch(F{}, std::integral_constant<int, kPair>{});
        return hipGetLastError();
      }
    }
    launch(F{}, P0{});
  }
  return hipGetLastError();
}

#undef TPK_LDS

}  // namespace gemm_detail

// The launchers declared in gemm_bf16_impl.h, defined once here; each
// gemm_bf16_*.hip unit only instantiates its share of them.  256 x 256 and
// 128 x 384 tiles run 8 waves (2 per SIMD: 256 x 256 as 2 x 4 waves of
// 128 x 64, 128 x 384 as 2 x 4 of 64 x 96), 128 x 128 tiles 4 waves of
// 64 x 64 and 64 x 128 tiles 1 x 4 waves of 64 x 32 (two workgroups per
// CU); 4 LDS stages throughout.
// Every tile multiplies with v_mfma_f32_16x16x32_bf16 (MF16): on this
// power-capped part it sustains 12-19% more FLOP/s than v_mfma_f32_32x32x16
// with random operands (fewer accumulator register bytes per FLOP), and the
// GEMMs run 4-8% faster with bit-identical results.  The 32 x 32 x 16
// schedule (MF16 false) is kept beside it as the measured reference.
constexpr bool kMf16 = true;

template <int BM, int BN, int EPI, bool OUT_F32>
hipError_t launch_gemm_bf16_cfg(const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb,
                                int M, int N, int K, const Epilogue& ep, hipStream_t stream) {
  constexpr int kWgm = BM == 64 ? 1 : 2;
  constexpr int kWgn = BM == 128 && BN == 128 ? 2 : 4;
  return gemm_detail::launch_tile_dma<BM, BN, kWgm, kWgn, 4, false, true, EPI, OUT_F32, kMf16>(
      A, lda, B, ldb, M, N, K, ep, stream);
}

template <int BM, int BN, bool A_KMAJOR, bool B_KMAJOR, int EPI, bool OUT_F32>
hipError_t launch_gemm_bf16_t_cfg(const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb,
                                  int M, int N, int K, const Epilogue& ep, hipStream_t stream) {
  static_assert((BM == 256 && BN == 256) || (BM == 128 && BN == 128), "tile shapes");
  constexpr int kWgn = BM == 128 ? 2 : 4;
  return gemm_detail::launch_tile_dma<BM, BN, 2, kWgn, 4, A_KMAJOR, B_KMAJOR, EPI, OUT_F32, kMf16>(
      A, lda, B, ldb, M, N, K, ep, stream);
}

}  // namespace tpk
