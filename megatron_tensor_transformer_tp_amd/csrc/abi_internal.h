// Pieces of the C-ABI front end shared between its source files: the MLP
// shard forward split into its argument validation and its launches, so that
// the no-allocation variant (noalloc.hip) validates exactly as
// tp_mlp_shard_fwd does before it enqueues anything.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/tp_shard.h"

namespace tpabi {

// Every check of tp_mlp_shard_fwd except the workspace's; *f_out = ffn / t.
// Touches no HIP state.
tp_status mlp_fwd_validate(const void* x, const void* a_i, int64_t lda, const void* b_i,
                           const void* bias_a_i, const void* bias_b, const void* residual,
                           const void* z_i, const void* y_save, int64_t tokens, int64_t hidden,
                           int64_t ffn, int t, int rank, tp_dtype in_dt, tp_dtype out_dt,
                           int64_t* f_out);

// The two GEMMs of the shard over `tokens` rows, H_i in h ([tokens, f], row
// stride f, in_dt); bias_use / res_use already resolved for the rank
// (NULL unless rank 0).  part: room for splitk_part_floats(tokens,
// max(f, hidden)) floats, or NULL: with it, products of few tiles (bf16, at
// most kSplitKMaxRows tokens) run split-K.  Arguments validated.
tp_status mlp_fwd_enqueue(const void* x, const void* a_i, int64_t lda, const void* b_i,
                          const void* bias_a_i, const void* bias_use, const void* res_use,
                          void* z_i, void* y_save, void* h, float* part, int64_t tokens,
                          int64_t hidden, int64_t f, tp_dtype in_dt, tp_dtype out_dt, hipStream_t s);

}  // namespace tpabi
