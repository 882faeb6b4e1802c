// Head-local attention of one tensor-parallel rank: for each local head j,
// O_j = softmax(Q_j K_j^T / sqrt(d)) V_j over the rank's heads only (Tencent
// Hunyuan AI-Infra interview write-up, attention paragraph; Megatron expert
// interview Level 2, M028: heads split over ranks, no communication inside
// attention because the softmax reduces over keys).
//
// Input: the packed QKV projection of the rank, per token row laid out per
// local head as [q | k | v] (head_dim columns each), with the q and k
// columns in fp16 scaled by 2^-8 and the v columns in bf16: Q K^T runs on
// the fp16 MFMA (11 significant bits; with logits of std ~3 a bf16 Q/K
// would alone cost ~5e-3 relative error in the output), the 2^16 going back
// in the softmax scale.  The scale keeps |q|, |k| in [2^-6, 2^24) at full
// fp16 precision.
// Output: O [tokens, heads_local * head_dim] bf16, head j in columns j*d.
//
// Flash-style, gfx950:
//   * workgroup = one (batch, head, 128-query block) and 8 waves in two
//     groups of 4: wave w owns queries 32 (w % 4) .. +31 of the block, and
//     group g = w / 4 takes the 32-key blocks with index = g (mod 2).  Each
//     wave keeps its own online-softmax state; the two groups' states are
//     merged through LDS at the end (max, rescale, add);
//   * each wave software-pipelines its blocks: one iteration computes the
//     scores of its next block (MFMA) while the same wave forms the softmax
//     weights of the current block (VALU), then O += P V of the current
//     block (MFMA) while it takes the max of the next block; the wave raises
//     its issue priority (s_setprio) for the first of the two phases;
//   * grid ids are ordered head-fastest, so with 8 local heads each XCD
//     serves one head and its K/V stay in that XCD's L2; causal grids run
//     the query blocks from the last (longest row) to the first;
//   * K and V of a 32-key block (16 KiB) arrive by global->LDS copies (saddr
//     form: uniform base + 32-bit lane offset); 8 LDS stages, 4 per group:
//     the current block, the next block, one in flight and one being issued;
//     the loop is unrolled by 4 so that every LDS fragment address is a
//     loop-invariant register plus an immediate offset;
//   * S^T = K Q^T with v_mfma_f32_32x32x16_f16, K fragments from LDS (one
//     ds_read_b128, rows XOR-swizzled by row % 16, read one d-step ahead),
//     Q fragments held in registers; each lane owns one query and 16 of the
//     block's 32 keys, so the row max needs one exchange with lane ^ 32,
//     done by v_permlane32_swap in the VALU (no LDS round trip);
//   * O^T = V^T P^T: each lane keeps 64 of its query's output dimensions, so
//     the rescale is lane-local; V^T fragments come straight from the
//     row-major V block with ds_read_b64_tr_b16 (rows XOR-swizzled by
//     4 * (row % 4)); P is rounded to bf16 (RNE) for the MFMA; the key order
//     inside a 16-key MFMA step is permuted identically in P and V;
//   * exp via v_exp_f32 of fma(score, log2(e) / sqrt(d) * scale, -max) (the
//     max taken on the raw scores); the running max starts at a
//     large finite negative value, so fully masked (causal) entries give
//     exp = 0 and never NaN; it is raised lazily (only when a block's max
//     exceeds it by more than 8 in log2 units, decided per wave), so the
//     64-register output rescale is rare;
//   * causal: only the key blocks that cross the diagonal of a wave's 32
//     queries run the mask comparisons (a wave-uniform test of the block's
//     last key against the wave's first query);
//   * grids of at most half as many query blocks as CUs with 1024 keys or
//     more (causal: one per CU with 4096 keys or more) split each row's key
//     iterations over two workgroups; each
//     publishes its unnormalised partial state with device-scope stores and
//     counts itself in; the second to arrive merges the two (symmetric in
//     the halves, so the bits do not depend on the order of arrival);
//   * any sequence of at least 32 tokens: a partial last key block is read
//     as the window of the last 32 keys (a uniform offset) with its keys
//     before the block masked, an odd block count is padded by a fully
//     masked block, and queries past the end load the last query's row and
//     store nothing.
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "kernels.h"

namespace tpk {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef short i16x8_t __attribute__((ext_vector_type(8)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
#define TPK_LDS(T, p) ((__attribute__((address_space(3))) T*)(p))

constexpr int kD = 128;                 // head_dim
constexpr int kBQ = 128;                // queries per workgroup
constexpr int kBKV = 32;                // keys per block
constexpr int kStages = 8;
constexpr int kCycle = kStages / 2;      // iterations per stage cycle (per group half)
constexpr int kArr = kBKV * kD * 2;     // one array (K or V) of a block: 8 KiB
constexpr int kStage = 2 * kArr;        // 16 KiB
constexpr int kWaves = 8;
constexpr int kCopies = 2 * kStage / 1024 / kWaves;  // two blocks per iteration: 4 per wave
constexpr int kCopiesPerBlock = kStage / 1024;       // 16
constexpr float kNegBig = -1.0e30f;
// log2 units by which the running max may lag the true one before the
// output accumulator is rescaled (so the softmax weights stay <= 2^8).
constexpr float kRescaleSlack = 8.0f;
static_assert(kStages * kStage <= 160 * 1024, "LDS");
static_assert(kWaves / 2 * 64 * 66 * 4 <= kStages * kStage, "merge area");
static_assert(kQkvPart == kD, "q / k / v parts of head_dim columns");
// Split causal rows: values per (token, head) partial state (the
// unnormalised output, then the running max and the weight sum), stored
// value-major, part[half][head][value][token], so that a store or load of
// one value by a wave covers consecutive tokens.
constexpr int kPartValues = kD + 2;
static_assert(kPartValues == 130, "attn_part_floats");
// shortest sequence whose rows are split (each half then has at least one
// iteration, and the split pays for its extra launch)
constexpr int kSplitMinSeq = 1024;
// shortest sequence whose causal rows are split in a grid of one query
// block per CU
constexpr int kSplitCausalFullSeq = 4096;

// One global->LDS copy with a uniform base (SGPR pair) and a per-lane 32-bit
// byte offset: lane t's 16 bytes land at LDS byte address lds_addr + 16 t
// (lds_addr bound to M0 as an input, written by the compiler).
__device__ __forceinline__ void copy_to_lds_off(const void* base, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" : : "v"(voff), "s"(base), "{m0}"(lds_addr));
}

// The values of lanes l % 32 and l % 32 + 32 (lane l and its partner l ^ 32),
// in that order in every lane.  v_permlane32_swap with both operands v
// exchanges lanes 32..63 of the first with lanes 0..31 of the second
// (measured), leaving lane l's pair in the two results.
struct LanePair {
  float lo, hi;
};
__device__ __forceinline__ LanePair lane_pair(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return {__uint_as_float(r[0]), __uint_as_float(r[1])};
}

// RAGGED: seq is not a multiple of 128 (partial query and key blocks); the
// other instantiation carries none of the code for them.  SPLIT: two
// workgroups per query block, each taking one half of the row's key
// iterations; each publishes its partial state (unnormalised output, max,
// weight sum) in `part`, counts itself in `arrivals` (zeroed before the
// launch), and the second to arrive merges the two and stores O.
template <bool CAUSAL, bool RAGGED, bool SPLIT>
__global__ __launch_bounds__(512) void attn_fwd_kernel(const uint16_t* __restrict__ qkv,
                                                       int64_t ld_qkv, uint16_t* __restrict__ o,
                                                       int64_t ld_o, int seq, int heads,
                                                       float scale_log2, float* __restrict__ part,
                                                       int* __restrict__ arrivals) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kStages * kStage];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int group = wave >> 2;             // which half of the key blocks
  const int nqb = RAGGED ? (seq + kBQ - 1) / kBQ : seq / kBQ;
  const int id = blockIdx.x;
  const int head = id % heads;
  // causal rows grow with the query block: the longest are dispatched
  // first (query block slowest, descending), so that when the grid takes
  // several rounds the shorter ones fill in behind them; the two halves of
  // a split row are neighbours (same head, so the same XCD with 8 heads)
  const int nsplit = SPLIT ? 2 : 1;
  const int batch = static_cast<int>(gridDim.x) / (heads * nqb * nsplit);
  const int rest = SPLIT ? id / heads / 2 : id / heads;
  const int half_id = SPLIT ? (id / heads) % 2 : 0;
  const int qb = CAUSAL ? nqb - 1 - rest / batch : rest % nqb;
  const int b = CAUSAL ? rest % batch : rest / nqb;

  const int64_t row0 = static_cast<int64_t>(b) * seq;   // first token row of this batch
  const int col_q = head * 3 * kD, col_k = col_q + kD, col_v = col_q + 2 * kD;
  const int h = lane >> 5;                 // which half of the keys / dims this lane holds
  const int query = qb * kBQ + (wave & 3) * 32 + (lane & 31);
  const int wave_q0 = qb * kBQ + (wave & 3) * 32;   // the wave's first query (uniform)

  // Q fragments (B operand of S^T = K Q^T): lane holds Q[query][16t + 8h .. +7]
  // (a query past the end of the sequence, in the last block, reads the last
  // one's and is never stored).
  f16x8_t qf[8];
  {
    const int64_t qoff = (row0 + (RAGGED ? min(query, seq - 1) : query)) * ld_qkv + col_q + 8 * h;
    static_for<8>([&](auto T) __attribute__((always_inline)) {
      qf[T] = *reinterpret_cast<const f16x8_t*>(qkv + qoff + 16 * T);
    });
  }

  // Copies of one iteration: two blocks x (K, V) x 8 KiB = 32 copy
  // instructions of 1 KiB, 4 per wave; copy q moves 4 key rows of one array.
  // Lane -> (row, physical chunk), the array's swizzle undone on the global
  // side; the per-lane part is a byte offset from the block's first row.
  uint32_t coff[kCopies];
  static_for<kCopies>([&](auto Q) __attribute__((always_inline)) {
    const int rem = (wave * kCopies + Q) % kCopiesPerBlock;
    const int arr = rem / 8;                   // 0: K, 1: V
    const int slot = (rem % 8) * 64 + lane;
    const int row = slot >> 4, p = slot & 15;
    const int c = arr == 0 ? (p ^ (row & 15)) : (p ^ ((row & 3) << 2));
    coff[Q] = static_cast<uint32_t>((row * ld_qkv + (arr == 0 ? col_k : col_v) + 8 * c) * 2);
  });
  const int64_t block_step = static_cast<int64_t>(kBKV) * ld_qkv;
  const uint32_t smem_base = lds_address(smem);
  // Key blocks: a sequence that is not a multiple of 32 ends in a partial
  // block, which is copied from the window of the last 32 keys, [seq - 32,
  // seq), its keys before 32 kb (the previous block's) masked; an odd block
  // count gets a phantom last block (a copy of the last real one, every key
  // masked) so that both groups run the same iterations.
  const int nblk_all = RAGGED ? (seq + kBKV - 1) / kBKV : seq / kBKV;
  const int nblk = CAUSAL ? min(nblk_all, (qb + 1) * (kBQ / kBKV)) : nblk_all;
  const int nit_row = RAGGED ? (nblk + 1) / 2 : nblk / 2;
  // this workgroup's iterations: all of the row's, or one half of them
  // (the first half rounded up); blk0 is its first key block
  const int nit_first = (nit_row + 1) / 2;
  const int nit = SPLIT ? (half_id == 0 ? nit_first : nit_row - nit_first) : nit_row;
  const int blk0 = SPLIT && half_id == 1 ? 2 * nit_first : 0;
  // first key of block kb's window
  auto key_base = [seq](int kb) { return RAGGED ? min(kb * kBKV, seq - kBKV) : kb * kBKV; };

  // LDS placement: block j sits in its group's half of the stages (j % 2)
  // at its iteration's place in a kCycle-iteration cycle ((j / 2) % kCycle),
  //   stage(j) = (j % 2) * kCycle * kStage + ((j / 2) % kCycle) * kStage,
  // so with the loop unrolled by kCycle every fragment address is a per-lane
  // register (holding the group's base) plus a compile-time offset that the
  // LDS instruction's immediate field carries.
  auto stage_off = [](int j) { return (j % 2) * kCycle * kStage + ((j / 2) % kCycle) * kStage; };

  // Copies of blocks blk0 + 2 it and blk0 + 2 it + 1 (clamped to the last
  // block) into the stages of local blocks 2 it, 2 it + 1.
  auto issue = [&](int it) __attribute__((always_inline)) {
    static_for<kCopies>([&](auto Q) __attribute__((always_inline)) {
      const int q = wave * kCopies + Q;
      const int j = 2 * it + q / kCopiesPerBlock;
      const int kc = min(blk0 + j, nblk - 1);
      const int rem = q % kCopiesPerBlock;
      const uint16_t* base = RAGGED ? qkv + (row0 + key_base(kc)) * ld_qkv
                                    : qkv + row0 * ld_qkv + kc * block_step;
      copy_to_lds_off(base, coff[Q], smem_base + stage_off(j) + (rem / 8) * kArr + (rem % 8) * 1024);
    });
  };

  // Per-lane fragment offsets within the group's stages.
  const int k_row = lane & 31;
  const int k_sw = lane & 15;                  // row % 16 for the K swizzle
  const int gi = lane & 15;
  const int v_row = 4 * h + (gi >> 2);         // + 16u (+8 for the second read)
  const int v_sw = (gi >> 2) << 2;             // 4 * (row % 4)
  const int v_chunk = 2 * ((lane >> 4) & 1) + ((gi & 3) >> 1);  // + 4*dt
  const int v_within = (gi & 1) * 8;
  const int grp_off = group * kCycle * kStage;
  int k_off[8], v_off[4];
  static_for<8>([&](auto T) __attribute__((always_inline)) {
    k_off[T] = grp_off + k_row * (kD * 2) + (((2 * T + h) ^ k_sw) * 16);
  });
  static_for<4>([&](auto DT) __attribute__((always_inline)) {
    v_off[DT] = grp_off + kArr + v_row * (kD * 2) + (((4 * DT + v_chunk) ^ v_sw) * 16) + v_within;
  });

  f32x16_t acc_o[4];
  static_for<4>([&](auto DT) __attribute__((always_inline)) { acc_o[DT] = (f32x16_t)(0.0f); });
  float m_run = kNegBig, l_run = 0.0f;

  // S^T of one 32-key block from the stage at `so` (8 MFMAs, the K fragment
  // of d-step T+1 read ahead of the MFMA of d-step T).
  auto qk = [&](int so) __attribute__((always_inline)) {
    f32x16_t sv = (f32x16_t)(0.0f);
    f16x8_t kf[2];
    kf[0] = *TPK_LDS(const f16x8_t, smem + k_off[0] + so);
    static_for<8>([&](auto T) __attribute__((always_inline)) {
      constexpr int cur = T & 1;
      if constexpr (T < 7) kf[cur ^ 1] = *TPK_LDS(const f16x8_t, smem + k_off[T + 1] + so);
      sv = __builtin_amdgcn_mfma_f32_32x32x16_f16(kf[cur], qf[T], sv, 0, 0, 0);
    });
    return sv;
  };

  // Masks and the block's max (log2 units; this lane: its query and 16 of
  // the 32 keys, S^T rows 8 (R / 4) + 4 h + R % 4 of the block's window).
  // A key is masked when it is later than the query (causal; only a block
  // whose last key is later than the wave's first query can hold such a
  // key, so the others skip the comparisons in a wave-uniform branch) or,
  // in a partial or phantom block (a workgroup-uniform branch), when it
  // precedes the block (already counted).  The max is taken on the raw
  // scores: it commutes with the positive scale, which enters the exponent
  // through one fma.
  auto block_max = [&](f32x16_t& sv, int kb) __attribute__((always_inline)) {
    // window place of element R: 4 h + c(R), c(R) = 8 (R / 4) + R % 4
    const int kbase = key_base(kb);
    const int lo = kb * kBKV - kbase;   // places before lo: already counted (uniform)
    if constexpr (CAUSAL && RAGGED) {
      // the same comparison as a threshold on c(R) (fewer registers here)
      if (kbase + kBKV - 1 > wave_q0) {
        const int hi = query - kbase - 4 * h;
        static_for<16>([&](auto R) __attribute__((always_inline)) {
          if (8 * (R / 4) + (R % 4) > hi) sv[int(R)] = -__builtin_inff();
        });
      }
    } else if constexpr (CAUSAL) {
      if (kbase + kBKV - 1 > wave_q0) {
        static_for<16>([&](auto R) __attribute__((always_inline)) {
          const int key = kbase + 8 * (R / 4) + 4 * h + (R % 4);
          if (key > query) sv[int(R)] = -__builtin_inff();
        });
      }
    }
    if (RAGGED && lo > 0) {
      const int lo_h = lo - 4 * h;
      static_for<16>([&](auto R) __attribute__((always_inline)) {
        if (8 * (R / 4) + (R % 4) < lo_h) sv[int(R)] = -__builtin_inff();
      });
    }
    float mraw = kNegBig;
    static_for<16>([&](auto R) __attribute__((always_inline)) { mraw = fmaxf(mraw, sv[int(R)]); });
    const LanePair mp = lane_pair(mraw);
    return fmaxf(mp.lo, mp.hi) * scale_log2;
  };

  // The running max is raised (and the accumulator rescaled) only when a
  // block's max exceeds it by more than kRescaleSlack, decided for the whole
  // wave at once; otherwise the weights may grow up to 2^kRescaleSlack.
  auto raise_max = [&](float mx) __attribute__((always_inline)) {
    if (__any(mx > m_run + kRescaleSlack)) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
      static_for<4>([&](auto DT) __attribute__((always_inline)) { acc_o[DT] *= alpha; });
    }
  };

  // Softmax weights of a masked block against the running max, their sum,
  // and P^T fragments: step u covers keys 16u .. 16u+15; half h holds keys
  // {4h..4h+3, 8+4h..8+4h+3} of the step, V^T uses the same order.
  auto weights = [&](const f32x16_t& sv, bf16x8_t (&pf)[2]) __attribute__((always_inline)) {
    float p[16];
    static_for<16>([&](auto R) __attribute__((always_inline)) {
      p[R] = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[int(R)], scale_log2, -m_run));
    });
    static_for<16>([&](auto R) __attribute__((always_inline)) { l_run += p[R]; });
    static_for<2>([&](auto U2) __attribute__((always_inline)) {
      i16x8_t w;
      static_for<4>([&](auto R) __attribute__((always_inline)) {
        w[int(R)] = __builtin_bit_cast(short, static_cast<__bf16>(p[8 * U2 + R]));
        w[4 + int(R)] = __builtin_bit_cast(short, static_cast<__bf16>(p[8 * U2 + 4 + R]));
      });
      pf[U2] = __builtin_bit_cast(bf16x8_t, w);
    });
  };

  // O^T += V^T P^T from the stage at `so`, the V^T fragments of the next 32
  // dims loading under the MFMAs of the current ones.
  auto pv = [&](const bf16x8_t (&pf)[2], int so) __attribute__((always_inline)) {
    i16x4_t vf[2][2][2];
    auto load_v = [&](auto DT, auto BUF) __attribute__((always_inline)) {
      static_for<2>([&](auto U2) __attribute__((always_inline)) {
        vf[BUF][U2][0] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            TPK_LDS(i16x4_t, smem + v_off[DT] + so + (16 * U2) * (kD * 2)));
        vf[BUF][U2][1] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            TPK_LDS(i16x4_t, smem + v_off[DT] + so + (16 * U2 + 8) * (kD * 2)));
      });
    };
    load_v(std::integral_constant<int, 0>{}, std::integral_constant<int, 0>{});
    static_for<4>([&](auto DT) __attribute__((always_inline)) {
      constexpr int cur = DT & 1;
      if constexpr (DT < 3) load_v(std::integral_constant<int, DT + 1>{}, std::integral_constant<int, cur ^ 1>{});
      static_for<2>([&](auto U2) __attribute__((always_inline)) {
        const i16x8_t w = {vf[cur][U2][0][0], vf[cur][U2][0][1], vf[cur][U2][0][2], vf[cur][U2][0][3],
                           vf[cur][U2][1][0], vf[cur][U2][1][1], vf[cur][U2][1][2], vf[cur][U2][1][3]};
        acc_o[DT] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, w), pf[U2],
                                                             acc_o[DT], 0, 0, 0);
      });
    });
  };

  // Software pipeline over this wave's blocks b = 2 it + group: iteration it
  // runs S of block b+2 (the next one) under the softmax weights of block b,
  // then P V of block b under the max of block b+2; the running max is raised
  // for block b+2 after P V of block b.  Per block the arithmetic and its
  // order are those of the plain sequence max -> raise -> weights -> P V.
  // Copies: iteration it needs blocks 2 it (+ group) and 2 it + 2 (+ group)
  // resident and issues blocks 2 it + 6, 2 it + 7 into the stages of blocks
  // 2 it - 2, 2 it - 1 (read for the last time in iteration it - 1).
  issue(0);
  issue(1);
  issue(2);
  wait_vmcnt<2 * kCopies>();
  lds_barrier();
  // scores of the current and the next block, alternating roles by step
  // parity (the unroll factor is even), so no copy passes them on
  f32x16_t s_buf[2];
  s_buf[0] = qk(0);                             // block group: stage offset 0 in the group's half
  raise_max(block_max(s_buf[0], blk0 + group));

  auto step = [&](int it, auto U) __attribute__((always_inline)) {
    constexpr int ust = U * kStage;                        // block 2 it + group
    constexpr int nst = ((U + 1) % kCycle) * kStage;       // block 2 it + 2 + group
    // Nothing of the previous iteration (its MFMAs and their LDS waits)
    // moves past the barrier; blocks 2 it + 2, 2 it + 3 have landed.
    __builtin_amdgcn_sched_barrier(0);
    wait_vmcnt<kCopies>();
    lds_barrier();
    issue(it + 3);
    constexpr int C = U & 1, N = C ^ 1;                     // current / next score buffer
    bf16x8_t pf[2];
    __builtin_amdgcn_s_setprio(1);
    s_buf[N] = qk(nst);
    weights(s_buf[C], pf);
    __builtin_amdgcn_s_setprio(0);
    __builtin_amdgcn_sched_barrier(0);
    pv(pf, ust);
    const float mx = block_max(s_buf[N], blk0 + 2 * it + 2 + group);
    if (it + 1 < nit) raise_max(mx);
  };
  static_assert(kCycle % 2 == 0, "score buffers alternate within one unrolled group");
  for (int it = 0; it < nit; it += kCycle) {
    step(it, std::integral_constant<int, 0>{});
    if (it + 1 < nit) step(it + 1, std::integral_constant<int, 1>{});
    if (it + 2 < nit) step(it + 2, std::integral_constant<int, 2>{});
    if (it + 3 < nit) step(it + 3, std::integral_constant<int, 3>{});
  }
  // Merge the two groups: group 1 publishes (m, l, acc) through LDS (the
  // stages are free once every wave's copies have landed and its last
  // fragment reads have returned), group 0 combines with its partner wave
  // w + 4 (same queries, same lane layout) and stores.
  __builtin_amdgcn_sched_barrier(0);
  wait_vmcnt<0>();
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
  lds_barrier();
  float* mrg = reinterpret_cast<float*>(smem) + ((wave & 3) * 64 + lane) * 66;
  if (group == 1) {
    mrg[0] = m_run;
    mrg[1] = l_run;
    static_for<4>([&](auto DT) __attribute__((always_inline)) {
      static_for<16>([&](auto R) __attribute__((always_inline)) { mrg[2 + 16 * DT + R] = acc_o[DT][int(R)]; });
    });
  }
  // the barrier does not wait for LDS writes: each wave waits for its own
  // first, so the other groups' reads after it see them (whatever SIMD
  // the writing wave runs on)
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
  lds_barrier();
  if constexpr (!SPLIT) {
    if (group == 0) {
      const float m1 = mrg[0], l1 = mrg[1];
      const float m = fmaxf(m_run, m1);
      const float a0 = __builtin_amdgcn_exp2f(m_run - m), a1 = __builtin_amdgcn_exp2f(m1 - m);
      const float l_lane = l_run * a0 + l1 * a1;
      const LanePair lp = lane_pair(l_lane);
      const float l_tot = lp.lo + lp.hi;
      const float inv = 1.0f / l_tot;
      uint16_t* orow = o + (row0 + query) * ld_o + head * kD + 4 * h;
      if (!RAGGED || query < seq) static_for<4>([&](auto DT) __attribute__((always_inline)) {
        float v[16];
        static_for<16>([&](auto R) __attribute__((always_inline)) {
          v[R] = (acc_o[DT][int(R)] * a0 + mrg[2 + 16 * DT + R] * a1) * inv;
        });
        // O[query][dt*32 + 8g + 4h + r]: 4 consecutive dims per store
        static_for<4>([&](auto G) __attribute__((always_inline)) {
          const u32x2_t w = {pack_bf16x2(v[4 * G], v[4 * G + 1]), pack_bf16x2(v[4 * G + 2], v[4 * G + 3])};
          *reinterpret_cast<u32x2_t*>(orow + DT * 32 + 8 * G) = w;
        });
      });
    }
  } else {
    // This half's state (group 0 merges its two groups without
    // normalising) goes to `part` (value-major), by device-scope
    // atomic stores (written where every XCD sees them, so no cache
    // write-back or invalidation is needed); once they have completed, one
    // thread counts the workgroup in; the second of the row's two
    // workgroups to arrive reads the other half's state by device-scope
    // atomic loads and stores O = (O_a w_a + O_b w_b) / (l_a w_a + l_b w_b),
    // w = 2^(m - max), symmetric in the halves, so the result does not
    // depend on which of the two arrives last.
    const int64_t tokens = static_cast<int64_t>(batch) * seq;
    const int64_t token = row0 + query;
    float m = 0.0f, l_tot = 0.0f;
    const bool live = !RAGGED || query < seq;
    if (group == 0) {
      const float m1 = mrg[0], l1 = mrg[1];
      m = fmaxf(m_run, m1);
      const float a0 = __builtin_amdgcn_exp2f(m_run - m), a1 = __builtin_amdgcn_exp2f(m1 - m);
      const LanePair lp = lane_pair(l_run * a0 + l1 * a1);
      l_tot = lp.lo + lp.hi;
      static_for<4>([&](auto DT) __attribute__((always_inline)) {
        static_for<16>([&](auto R) __attribute__((always_inline)) {
          acc_o[DT][int(R)] = acc_o[DT][int(R)] * a0 + mrg[2 + 16 * DT + R] * a1;
        });
      });
      if (live) {
        float* pr = part + (static_cast<int64_t>(half_id) * heads + head) * kPartValues * tokens + token;
        static_for<4>([&](auto DT) __attribute__((always_inline)) {
          static_for<16>([&](auto R) __attribute__((always_inline)) {
            __hip_atomic_store(pr + (DT * 32 + 8 * (R / 4) + 4 * h + R % 4) * tokens, acc_o[DT][int(R)],
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          });
        });
        if (h == 0) {
          __hip_atomic_store(pr + kD * tokens, m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          __hip_atomic_store(pr + (kD + 1) * tokens, l_tot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
      wait_vmcnt<0>();
    }
    int* flag = reinterpret_cast<int*>(smem + kStages * kStage - 16);   // past the merge area
    lds_barrier();
    if (threadIdx.x == 0) *flag = atomicAdd(arrivals + (static_cast<int64_t>(b) * nqb + qb) * heads + head, 1);
    __builtin_amdgcn_s_waitcnt(0xC07F);   // the flag's LDS write, before the barrier
    lds_barrier();
    if (*flag == 1 && group == 0) {
      if (live) {
        // products rounded apart (no fused multiply-add): each sum is then
        // the same whichever half merges
#pragma clang fp contract(off)
        const float* po = part + (static_cast<int64_t>(1 - half_id) * heads + head) * kPartValues * tokens + token;
        // every load issued before the first use: one round trip to where
        // the device-scope stores landed, not one per group of four
        float xo[4][16];
        const float mo = __hip_atomic_load(po + kD * tokens, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const float lo = __hip_atomic_load(po + (kD + 1) * tokens, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        static_for<4>([&](auto DT) __attribute__((always_inline)) {
          static_for<16>([&](auto R) __attribute__((always_inline)) {
            xo[DT][R] = __hip_atomic_load(po + (DT * 32 + 8 * (R / 4) + 4 * h + R % 4) * tokens,
                                          __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          });
        });
        __builtin_amdgcn_sched_barrier(0);
        const float mm = fmaxf(m, mo);
        const float w0 = __builtin_amdgcn_exp2f(m - mm), w1 = __builtin_amdgcn_exp2f(mo - mm);
        const float inv = 1.0f / (l_tot * w0 + lo * w1);
        uint16_t* orow = o + (row0 + query) * ld_o + head * kD + 4 * h;
        static_for<4>([&](auto DT) __attribute__((always_inline)) {
          static_for<4>([&](auto G) __attribute__((always_inline)) {
            float v[4];
            static_for<4>([&](auto R) __attribute__((always_inline)) {
              v[R] = (acc_o[DT][4 * G + R] * w0 + xo[DT][4 * G + R] * w1) * inv;
            });
            const u32x2_t w = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
            *reinterpret_cast<u32x2_t*>(orow + DT * 32 + 8 * G) = w;
          });
        });
      }
    }
  }
}

// Zeroes the arrival counters of a split launch (a kernel, so that the
// launch sequence can be captured in a graph).
__global__ __launch_bounds__(256) void attn_clear_kernel(int* __restrict__ p, int64_t n) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i < n) p[i] = 0;
}

}  // namespace

hipError_t launch_attention(const uint16_t* qkv, int64_t ld_qkv, uint16_t* o, int64_t ld_o,
                            int batch, int seq, int heads, int head_dim, bool causal, float* part,
                            int* arrivals, hipStream_t stream) {
  if (batch == 0 || seq == 0) return hipSuccess;
  // per-lane copy offsets are 32-bit byte offsets within one key block
  if (static_cast<int64_t>(kBKV) * ld_qkv * 2 >= (int64_t{1} << 31)) return hipErrorInvalidValue;
  if (head_dim != kD || seq < kBKV) return hipErrorInvalidValue;
  // log2(e) / sqrt(d), times 1 / kQkScale^2 for the scaled fp16 Q and K
  const float scale_log2 = 1.4426950408889634f / __builtin_sqrtf(static_cast<float>(head_dim)) /
                           (kQkScale * kQkScale);
  const int64_t rows = static_cast<int64_t>(batch) * heads * ((seq + kBQ - 1) / kBQ);
  // A grid of at most half as many query blocks as CUs leaves CUs idle:
  // its rows are split over two workgroups each.  Measured (kernel alone,
  // non-causal / causal): 128 query blocks at seq 2048 9% / 20% faster, at
  // seq 4096 16% / 30%, 64 at seq 8192 25% / 37%, 64 at seq 1024 2-4% /
  // 5-7%, but 64 at seq 512 11-14% slower (the counter-clearing launch and
  // the workgroups' start take what the split saves).  Fuller grids lose
  // under the power cap (one query block per CU: non-causal 19-33% slower,
  // causal at seq 2048 10% slower), except causal ones at seq 4096 and
  // more, whose unequal rows make the split pay (8 heads x seq 4096: 11%,
  // 4 heads x seq 8192: 22% faster); grids of two rounds or more lose.
  const int64_t cus = device_cus();
  const bool split = part != nullptr && arrivals != nullptr &&
                     ((seq >= kSplitMinSeq && 2 * rows <= cus) ||
                      (causal && seq >= kSplitCausalFullSeq && rows <= cus));
  if (split) {
    hipLaunchKernelGGL(attn_clear_kernel, dim3(static_cast<unsigned>((rows + 255) / 256)), dim3(256), 0,
                       stream, arrivals, rows);
  }
  const dim3 grid(static_cast<unsigned>(rows * (split ? 2 : 1)));
  auto go = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, grid, dim3(64 * kWaves), 0, stream, qkv, ld_qkv, o, ld_o, seq, heads,
                       scale_log2, part, arrivals);
  };
  const bool ragged = seq % kBQ != 0;
  if (causal && split)
    ragged ? go(attn_fwd_kernel<true, true, true>) : go(attn_fwd_kernel<true, false, true>);
  else if (causal)
    ragged ? go(attn_fwd_kernel<true, true, false>) : go(attn_fwd_kernel<true, false, false>);
  else if (split)
    ragged ? go(attn_fwd_kernel<false, true, true>) : go(attn_fwd_kernel<false, false, true>);
  else
    ragged ? go(attn_fwd_kernel<false, true, false>) : go(attn_fwd_kernel<false, false, false>);
  return hipGetLastError();
}

}  // namespace tpk
