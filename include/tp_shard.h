/*
 * tp_shard.h -- C ABI of the tensor-parallel MLP / attention shard library
 * (one rank's share of a Megatron-style Transformer block, gfx950 / MI355X).
 *
 * Notation.  X [M, h] is the input (M = tokens = seq x batch, h = hidden),
 * A [h, F] and B [F, h] are the two MLP weights (F = ffn width, 4h in the
 * standard block), t is the tensor-parallel degree and f = F / t the shard
 * width.  Rank r owns the contiguous index block S_r = [r*f, (r+1)*f): columns
 * S_r of A (A_r, [h, f]) and rows S_r of B (B_r, [f, h]).
 *
 * Passages defining the operations (page titles as printed on the pages):
 *   - Column-parallel linear: W split by output columns, X replicated, each
 *     rank produces its column block of the output with no communication.
 *     Tencent Hunyuan AI-Infra interview write-up, 参考解析 (first paragraph);
 *     列并行 tutorial (aiqz.cc), 切分原理 and 数学基础; Megatron expert
 *     interview Level 2 (blog.cptz.space), M025.
 *   - GeLU(z) = z * Phi(z), elementwise, valid on each column block:
 *     列并行 tutorial, MLP 应用.
 *   - Row-parallel linear: W split by input rows, the input split on its last
 *     dimension, each rank produces a full-hidden partial that the ranks sum:
 *     Megatron Level 2, M026; distributed-parallelism overview
 *     (talentme.airsota.com), 考点 2.
 *   - MLP shard = column layer -> GeLU -> row layer with no exchange between
 *     them: Tencent write-up, FFN paragraph; 列并行 tutorial, MLP 应用;
 *     Megatron Level 2, M027.
 *   - Attention shard: heads split over ranks, packed QKV interleaved per
 *     head, local softmax(Q K^T / sqrt(d)) V, row-parallel output projection:
 *     Tencent write-up, attention paragraph; Megatron Level 2, M028.
 *   - SwiGLU variant: the gated activation acts on paired local shards of
 *     the two projections (Megatron Level 2, M027, M031).
 *   - Backward: for the column layer the weight gradient X^T dY_i is local
 *     and the input-gradient contributions dY_i A_i^T are summed over the
 *     ranks (Megatron Level 2, M025); for the row layer the input gradient
 *     dZ B_i^T is already the rank's input-block gradient and the weight
 *     gradient is local (Megatron Level 2, M026).
 *   - Sequence-parallel boundary: the row-parallel partials are summed by a
 *     Reduce-Scatter that leaves each rank its sequence shard [s/t, b, h],
 *     on which per-token work (bias, residual) runs locally: Megatron
 *     Level 2, M034.
 *   - Shapes that do not divide are rejected, never padded: 列并行 tutorial,
 *     切分原理; Megatron Level 2, M031.
 *
 * What this interface adds to the method's five operations (column linear,
 * GeLU, row linear, MLP shard, attention shard, each taking shard shapes, t
 * and rank), and why:
 *   - Leading dimensions (ldx, lda, ldy, ldh, ldb, ldr, ldz): a rank's weight
 *     block may be a column-block VIEW of the full weight (lda = F), and
 *     activations may be row-strided views; the pages' shapes are the
 *     logical ones.
 *   - y_save (tp_mlp_shard_fwd): the pre-activation the backward needs.
 *   - Workspace arguments and their *_workspace_bytes queries: the library
 *     never allocates, so the caller hands in the scratch for H_i (the
 *     intermediate's one HBM round trip) and the attention's Q/K/V/O.
 *   - tp_mlp_shard_bwd, tp_mlp_swiglu_shard_fwd, tp_sp_reduce_scatter: the
 *     backward, the gated variant and the sequence-parallel boundary that the
 *     pages name beside the forward MLP (passages at each declaration).
 *   - tp_status_string, tp_version: error text and versioning.
 *
 * Conventions shared by every entry point.
 *   - Tensor pointers are DEVICE pointers owned by the caller.  The library
 *     never allocates, frees or synchronises; it enqueues kernels on
 *     `stream` (a hipStream_t passed as void*, NULL = the default stream) and
 *     returns.  Outputs are valid once the caller synchronises that stream.
 *   - Matrices are row-major with an explicit leading dimension in ELEMENTS
 *     (ld >= row width).  bf16 data is the 16-bit bfloat16 bit pattern.
 *   - The caller passes the LOGICAL (unsharded) ffn / heads plus t and rank;
 *     the library derives the shard width itself, so the divisibility check
 *     is always live.  Weight pointers point AT the rank's shard (the library
 *     never offsets by rank); rank decides who adds the output bias and the
 *     residual (rank 0 only, so that the sum of the partials is the layer).
 *   - Alignment: every pointer 16-byte aligned; row widths and leading
 *     dimensions a multiple of 8 elements (bf16) or 4 elements (fp32).
 *     Any tokens >= 0 is accepted (tokens == 0 enqueues nothing).
 *   - Errors: every argument is checked before anything is enqueued; on an
 *     error nothing is enqueued and a tp_status code is returned.  A failed
 *     launch returns TP_ERR_HIP.  Nothing is printed, no exception crosses
 *     the ABI.  Calls are stateless and thread-safe; calls that write the
 *     same output buffer concurrently race, as with any kernel.
 *   - Sizes: tokens, hidden and each shard width up to 2^30 (larger ones
 *     return TP_ERR_UNSUPPORTED); a product whose tile count or fp32 grid
 *     exceeds the launch limits fails with TP_ERR_HIP before it runs.
 *   - Numerics: bf16 inputs are multiplied with fp32 accumulation (MFMA);
 *     fp32 inputs with fp32 FMA.  GeLU is applied to the fp32 accumulator;
 *     a bf16 output is rounded to nearest-even.  Inputs must be finite.
 */
#ifndef TP_SHARD_H_
#define TP_SHARD_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  TP_OK = 0,
  TP_ERR_INVALID_ARG = 1,   /* null pointer, negative size, ld < width, bad flag */
  TP_ERR_NOT_DIVISIBLE = 2, /* ffn (or heads) not divisible by t                  */
  TP_ERR_BAD_RANK = 3,      /* rank outside [0, t) or t < 1                       */
  TP_ERR_DTYPE = 4,         /* unsupported dtype or dtype combination             */
  TP_ERR_MISALIGNED = 5,    /* pointer / width / leading dimension misaligned     */
  TP_ERR_WORKSPACE = 6,     /* workspace missing or smaller than required         */
  TP_ERR_UNSUPPORTED = 7,   /* valid request outside what the kernels implement   */
  TP_ERR_HIP = 8            /* a HIP launch failed                                */
} tp_status;

typedef enum { TP_F32 = 0, TP_BF16 = 1 } tp_dtype;

/* Human-readable name of a status code (static string, never NULL). */
const char* tp_status_string(tp_status s);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int tp_version(void);

/*
 * Column-parallel linear: Y_i = X A_i (+ a_i), then GeLU if apply_gelu.
 * Passages: 列并行 tutorial, 切分原理 and 数学基础 (W split by output
 * columns, X replicated, Y = [X W^(1) | ... | X W^(p)]); Megatron Level 2,
 * M025 (W_i [h, 4h/t], output [s, b, 4h/t] with no gather when the next op
 * consumes the shard).
 *   x      [tokens, hidden], ld ldx          (in_dt)
 *   a_i    [hidden, f], ld lda, f = ffn / t  (in_dt) -- the rank's column block
 *   bias_i [f] or NULL                       (in_dt) -- the rank's block of a
 *   y_i    [tokens, f], ld ldy               (out_dt)
 * dtype pairs (in -> out): bf16 -> bf16, bf16 -> f32, f32 -> f32.
 */
tp_status tp_column_linear(const void* x, int64_t ldx, const void* a_i, int64_t lda,
                           const void* bias_i, void* y_i, int64_t ldy,
                           int64_t tokens, int64_t hidden, int64_t ffn, int t, int rank,
                           tp_dtype in_dt, tp_dtype out_dt, int apply_gelu, void* stream);

/*
 * Elementwise exact GeLU, out[k] = in[k] * Phi(in[k]), k < n.  Passage:
 * 列并行 tutorial, MLP 应用 (GeLU(z) = z Phi(z), Phi the standard normal CDF;
 * being elementwise it acts on each column block with no communication).  in and out may
 * alias exactly (in place) when in_dt == out_dt; partial overlap is not
 * allowed.  dtype pairs: any of f32/bf16 -> f32/bf16.  n >= 0; pointers
 * 16-byte aligned.
 */
tp_status tp_gelu(const void* in, void* out, int64_t n, tp_dtype in_dt, tp_dtype out_dt,
                  void* stream);

/*
 * Row-parallel linear: Z_i = H_i B_i, plus (rank 0 only) bias and residual.
 * Passages: Megatron Level 2, M026 (W split by input rows, the input split
 * on its last dimension, each rank's output a full-shape partial that the
 * ranks sum); distributed-parallelism overview, 考点 2 (Z = Z_1 + Z_2 by one
 * All-Reduce); the bias placed once outside the partials: Megatron Level 2,
 * M025 (the bias boundary).
 *   h_i      [tokens, f], ld ldh, f = ffn / t (in_dt) -- the rank's input block
 *   b_i      [f, hidden], ld ldb              (in_dt) -- the rank's row block
 *   bias     [hidden] or NULL                 (in_dt) -- added by rank 0 only
 *   residual [tokens, hidden], ld ldr, or NULL (in_dt) -- added by rank 0 only
 *   z_i      [tokens, hidden], ld ldz         (out_dt) -- full-hidden partial
 * dtype pairs: bf16 -> f32 (partial for t > 1), bf16 -> bf16, f32 -> f32.
 * On ranks != 0 bias and residual are ignored (they may be NULL).
 */
tp_status tp_row_linear(const void* h_i, int64_t ldh, const void* b_i, int64_t ldb,
                        const void* bias, const void* residual, int64_t ldr,
                        void* z_i, int64_t ldz,
                        int64_t tokens, int64_t ffn, int64_t hidden, int t, int rank,
                        tp_dtype in_dt, tp_dtype out_dt, void* stream);

/*
 * Bytes of workspace tp_mlp_shard_fwd needs (this interface's addition: the
 * library does not allocate): the GeLU intermediate
 * H_i [tokens, f] in in_dt (bf16 for bf16 inputs, f32 for f32), rounded up to
 * 256 bytes, and for bf16 calls of at most 512 tokens the split-K partial
 * products that follow it (8 * tokens * max(f, hidden) floats).  Returns 0
 * for invalid arguments (and for tokens == 0).
 */
size_t tp_mlp_shard_workspace_bytes(int64_t tokens, int64_t hidden, int64_t ffn, int t,
                                    tp_dtype in_dt);

/*
 * One rank's MLP shard: Z_i = GeLU(X A_i + a_i) B_i (+ b + R on rank 0).
 * Passages: Tencent write-up, FFN paragraph (column layer, GeLU, row layer,
 * one All-Reduce at the end); 列并行 tutorial, MLP 应用 (no All-Gather
 * between the layers: f/g fusion); Megatron Level 2, M027; overview page,
 * 第三章 (contiguous column slices of the first weight and row slices of the
 * second with the same indices).
 *   x         [tokens, hidden] contiguous (ld = hidden)  (in_dt)
 *   a_i       [hidden, f], ld lda                          (in_dt)
 *   b_i       [f, hidden] contiguous (ld = hidden)         (in_dt)
 *   bias_a_i  [f] or NULL (the rank's block of a)          (in_dt)
 *   bias_b    [hidden] or NULL (rank 0 only)               (in_dt)
 *   residual  [tokens, hidden] contiguous or NULL (rank 0) (in_dt)
 *   z_i       [tokens, hidden] contiguous                  (out_dt)
 *   y_save    [tokens, f] contiguous, or NULL: if given, also receives the
 *             pre-activation Y_i = X A_i + a_i (in_dt), which
 *             tp_mlp_shard_bwd takes as its saved activation
 *   workspace >= tp_mlp_shard_workspace_bytes(...), 256-byte aligned; it
 *             holds H_i between the two GEMMs (one HBM round trip) and is
 *             scratch: its contents after the call are unspecified.
 * dtype pairs: bf16 -> f32, bf16 -> bf16, f32 -> f32.
 * With bf16 inputs and at most 512 tokens, a product of few tiles splits
 * its k range over several workgroup sets (fp32 partial products summed in
 * a fixed order), so the result is reproducible but not bitwise the tiled
 * product's.
 */
tp_status tp_mlp_shard_fwd(const void* x, const void* a_i, int64_t lda, const void* b_i,
                           const void* bias_a_i, const void* bias_b, const void* residual,
                           void* z_i, void* y_save, void* workspace, size_t workspace_bytes,
                           int64_t tokens, int64_t hidden, int64_t ffn, int t, int rank,
                           tp_dtype in_dt, tp_dtype out_dt, void* stream);

/*
 * Size of the library's fixed device array used by tp_mlp_shard_fwd_noalloc
 * (one copy per GPU the library runs on, held until the process ends).
 */
#define TP_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/*
 * tp_mlp_shard_fwd for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same arguments, results and errors without the workspace; the GeLU
 * intermediate H_i lives in the library's own TP_NOALLOC_SCRATCH_BYTES device
 * array.  Nothing is allocated, freed or synchronised.
 *   Tokens are processed in row chunks whose H_i fits the array, so any
 *   tokens works; the shard width is limited instead: if fewer than
 *   min(tokens, 256) rows of H_i fit (f * element size > 256 KiB, i.e.
 *   f > 131072 in bf16 or 65536 in fp32) the call returns TP_ERR_WORKSPACE.
 *   The array's address on the current device is looked up on the first
 *   call on that device (the stream must belong to the current device); a
 *   failed lookup returns TP_ERR_HIP.
 *   Every call on one GPU shares that GPU's array: calls that overlap on one
 *   GPU (on other streams or threads) race and must be serialised by the
 *   caller.  Nothing in the array needs to start zeroed.
 *   The products always run tiled (no split-K), so below 513 tokens the
 *   results agree with tp_mlp_shard_fwd's to the rounding of the sums, not
 *   bit for bit.
 */
tp_status tp_mlp_shard_fwd_noalloc(const void* x, const void* a_i, int64_t lda, const void* b_i,
                                   const void* bias_a_i, const void* bias_b, const void* residual,
                                   void* z_i, void* y_save, int64_t tokens, int64_t hidden,
                                   int64_t ffn, int t, int rank, tp_dtype in_dt, tp_dtype out_dt,
                                   void* stream);

/*
 * Bytes of workspace tp_mlp_swiglu_shard_fwd needs (the library does not
 * allocate): H_i [tokens, f] in in_dt
 * (fp32 inputs: also the two gated projections), rounded up to 256 bytes;
 * 0 if invalid.
 */
size_t tp_mlp_swiglu_shard_workspace_bytes(int64_t tokens, int64_t hidden, int64_t ffn, int t,
                                           tp_dtype in_dt);

/*
 * One rank's SwiGLU MLP shard (the gated variant of the MLP; Megatron
 * Level 2, M027: the gate acts on paired local shards, no other rank is
 * needed; M031: both projections are split, each must divide):
 *   H_i = SiLU(X Wg_i) * (X Wu_i),  SiLU(z) = z / (1 + exp(-z)),
 *   Z_i = H_i B_i (+ b + R on rank 0).
 *   x         [tokens, hidden] contiguous                  (in_dt)
 *   wg_i      [hidden, f], ld lda: the rank's column block of the gate
 *             projection                                   (in_dt)
 *   wu_i      [hidden, f], ld lda: the SAME columns of the value
 *             projection                                   (in_dt)
 *   b_i       [f, hidden] contiguous                       (in_dt)
 *   bias_b, residual, z_i, workspace: as for tp_mlp_shard_fwd.
 * f = ffn / t with ffn the width of each projection.  Any tokens; widths,
 * leading dimensions, alignment and dtype pairs as for tp_mlp_shard_fwd.
 */
tp_status tp_mlp_swiglu_shard_fwd(const void* x, const void* wg_i, const void* wu_i, int64_t lda,
                                  const void* b_i, const void* bias_b, const void* residual,
                                  void* z_i, void* workspace, size_t workspace_bytes,
                                  int64_t tokens, int64_t hidden, int64_t ffn, int t, int rank,
                                  tp_dtype in_dt, tp_dtype out_dt, void* stream);

/*
 * Bytes of workspace tp_mlp_shard_bwd needs (the library does not
 * allocate): dY_i and H_i [tokens, f] in
 * in_dt plus the column-sum partials of the bias gradients, each part
 * rounded up to 256 bytes.  Returns 0 for invalid arguments.
 */
size_t tp_mlp_shard_bwd_workspace_bytes(int64_t tokens, int64_t hidden, int64_t ffn, int t,
                                        tp_dtype in_dt);

/*
 * Backward of one rank's MLP shard (the adjoint of tp_mlp_shard_fwd).
 * Passages: Megatron Level 2, M025 (column layer: dW_i = X^T dY_i local, the
 * input-gradient contributions SUM-reduced over the ranks) and M026 (row
 * layer: dX_i = dY W_i^T is already the input block's gradient, dW_i local);
 * the GeLU derivative is the product rule on z Phi(z) (列并行 tutorial,
 * MLP 应用, for the definition).  dz is
 * dL/dZ of the summed output Z = sum over ranks of Z_r (the same tensor on
 * every rank); y_i is the rank's saved pre-activation Y_i = X A_i + a_i.
 *   dY_i      = (dz B_i^T) * GeLU'(Y_i), GeLU'(y) = Phi(y) + y phi(y)
 *   db_i      = GeLU(Y_i)^T dz   [f, hidden]      the rank's row block of dB
 *   da_i      = X^T dY_i         [hidden, f]      the rank's column block of dA
 *   dx_i      = dY_i A_i^T       [tokens, hidden] the rank's contribution:
 *                                the sum over ranks is dX (the All-Reduce)
 *   dbias_a_i = sum over tokens of dY_i  [f]      (f32; skipped if NULL)
 *   dbias_b   = sum over tokens of dz    [hidden] (f32; skipped if NULL; the
 *                                same on every rank)
 * The residual's gradient is dz itself.
 *   x [tokens, hidden], b_i [f, hidden], y_i [tokens, f], dz [tokens, hidden]
 *   contiguous, a_i [hidden, f] ld lda: in_dt.
 *   dx_i [tokens, hidden] and db_i [f, hidden] contiguous, da_i [hidden, f]
 *   with the same ld lda as a_i: grad_dt.
 *   workspace >= tp_mlp_shard_bwd_workspace_bytes(...), 256-byte aligned,
 *   scratch.
 * dtype pairs (in_dt -> grad_dt): bf16 -> f32, bf16 -> bf16, f32 -> f32.
 * Any tokens; widths, leading dimensions and alignment as for
 * tp_mlp_shard_fwd.  tokens == 0 gives zero weight and bias gradients.  dY_i and H_i are rounded to in_dt (bf16: nearest-even)
 * before the weight- and input-gradient products.
 */
tp_status tp_mlp_shard_bwd(const void* x, const void* a_i, int64_t lda, const void* b_i,
                           const void* y_i, const void* dz, void* dx_i, void* da_i, void* db_i,
                           void* dbias_a_i, void* dbias_b, void* workspace,
                           size_t workspace_bytes, int64_t tokens, int64_t hidden, int64_t ffn,
                           int t, int rank, tp_dtype in_dt, tp_dtype grad_dt, void* stream);

/*
 * Bytes of workspace tp_attn_shard_fwd needs (the library does not
 * allocate): Q, K, V of the local heads, the local attention output, and,
 * for grids of at most 512 query blocks of 128 (batch * hl * ceil(seq /
 * 128)), the partial softmax states and counters of launches that split
 * each query block's keys over two workgroups (2 * batch * seq * hl * 130
 * floats, at most ~68 MB); rounded up to 256 bytes; 0 if invalid.
 */
size_t tp_attn_shard_workspace_bytes(int64_t batch, int64_t seq, int64_t hidden, int64_t heads,
                                     int64_t head_dim, int t, tp_dtype in_dt);

/*
 * One rank's head-local attention shard.  Passages: Tencent write-up,
 * attention paragraph (QKV column-split by heads with each head's q, k, v
 * kept together in an interleaved packed weight, local softmax(Q K^T / sqrt
 * d) V, row-parallel output projection, one All-Reduce); Megatron Level 2,
 * M028 (heads / t heads per rank; the softmax reduces over keys, not heads,
 * so no exchange is needed inside attention).
 *   x       [batch, seq, hidden] contiguous                     (in_dt)
 *   wqkv_i  [hidden, 3 * hl * head_dim] contiguous, hl = heads / t: the
 *           rank's column block of the packed QKV weight, laid out per local
 *           head as [q | k | v] blocks of head_dim columns each  (in_dt)
 *   wo_i    [hl * head_dim, hidden] contiguous: the rank's row block of the
 *           output projection                                   (in_dt)
 *   out_i   [batch, seq, hidden] contiguous full-hidden partial (out_dt)
 *   causal  0: every query sees every key; 1: key j <= query i only.
 * Per local head j: O_j = softmax(Q_j K_j^T / sqrt(head_dim)) V_j;
 * out_i = [O_0 | ... | O_{hl-1}] wo_i.  hidden == heads * head_dim.
 * dtype pairs: bf16 -> f32, bf16 -> bf16.  head_dim must be 128 and, unless
 * batch or seq is 0 (nothing to do), seq at least 32 (TP_ERR_UNSUPPORTED
 * otherwise); any such seq, not only multiples of the kernel's blocks.
 * Q and K enter Q K^T as
 * fp16 (11 significant bits) scaled by 2^-8, so |q|, |k| must stay below
 * 2^24: a larger value overflows to infinity, and the rows of every query
 * whose scores it reaches come out non-finite (Inf / NaN), never finite and
 * wrong; V, the softmax weights and O are bf16 operands; every product
 * accumulates in fp32.
 */
tp_status tp_attn_shard_fwd(const void* x, const void* wqkv_i, const void* wo_i, void* out_i,
                            void* workspace, size_t workspace_bytes,
                            int64_t batch, int64_t seq, int64_t hidden, int64_t heads,
                            int64_t head_dim, int causal, int t, int rank,
                            tp_dtype in_dt, tp_dtype out_dt, void* stream);

/*
 * Sequence-parallel boundary on one device: the SUM Reduce-Scatter half of
 * the exchange, fused with the shard's bias and residual.  Passages: Megatron
 * Level 2, M026 and M034 (with sequence parallelism the partials' All-Reduce
 * becomes a Reduce-Scatter that leaves each rank [s/t, b, h]; the per-token
 * work then runs on that shard).  Rank `rank`
 * receives its sequence shard of the summed output,
 *   out_r[m, :] = sum_{j < t} Z_j[rank*M/t + m, :] + bias + residual_r[m, :],
 * m < M/t, M = tokens (rows ordered sequence-major, so the shard is the
 * contiguous row block [rank*M/t, (rank+1)*M/t)).
 *   partials    HOST array of t DEVICE pointers; partials[j] is rank j's
 *               partial Z_j [tokens, hidden] contiguous, fp32
 *   bias        [hidden] or NULL                         (in_dt)
 *   residual_r  [tokens/t, hidden] contiguous or NULL: the rank's rows of
 *               the (sequence-sharded) residual stream   (in_dt)
 *   out_r       [tokens/t, hidden] contiguous            (out_dt)
 * The partials are summed in rank order in fp32 (deterministic).
 * tokens % t != 0 -> TP_ERR_NOT_DIVISIBLE; t > 16 -> TP_ERR_UNSUPPORTED;
 * hidden must be a multiple of 4.  in_dt, out_dt: f32 or bf16 (any pair).
 */
tp_status tp_sp_reduce_scatter(const void* const* partials, int t, int rank, const void* bias,
                               const void* residual_r, void* out_r, int64_t tokens,
                               int64_t hidden, tp_dtype in_dt, tp_dtype out_dt, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* TP_SHARD_H_ */
