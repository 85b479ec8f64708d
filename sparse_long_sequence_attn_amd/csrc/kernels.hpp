// Host-side launchers of the library's kernels (defined in attn_kernel.hip
// and merge_kernel.hip). All launches are asynchronous on the given stream.
#pragma once

#include "da_bwd.hpp"
#include "da_common.hpp"

namespace da {

// Query rows per attention workgroup for nw waves (4 or 1) and the dtype.
int attn_tile_rows(bool bf16, int nw);

// The fused gather / QK^T / online softmax / PV kernel over every tile of
// every pattern in `a`. nw is 4 (256-row bf16 / 128-row fp32 tiles, 64-key
// LDS tiles) or 1 (32-row tiles, 32-key LDS tiles, for short segments).
hipError_t launch_attention(const AttnArgs& a, bool bf16, int nw, bool causal, bool final_out,
                            int64_t grid, hipStream_t st);
// The one-wave attention kernel with the module's qk_norm applied to q and k
// as they are loaded (a.qkn, a.qkn_eps set; one pattern, segments of at most
// 32 gathered rows, final outputs).
// One-pass forward (bf16): grid = kXcds * ceil(B H nwin / kXcds) * L * nblk.
hipError_t launch_onepass(const OnePassArgs& a, bool causal, int64_t grid, hipStream_t st);
hipError_t launch_attention_qkn(const AttnArgs& a, bool bf16, bool causal, int64_t grid,
                                hipStream_t st);

// Log-sum-exp merge of the per-pattern partials into out and lse.
hipError_t launch_merge(const MergeArgs& a, bool bf16, hipStream_t st);

// Backward pass (bwd_kernel.hip): D = dout . out per row; dK and dV per
// key tile; dQ per query tile (tiles of 128 gathered rows, the attention
// launch's tile order, nw = 4); the partial sums and zero rows.
hipError_t launch_bwd_prep(const BwdRowArgs& a, bool bf16, hipStream_t st);
hipError_t launch_bwd_kv(const BwdArgs& a, bool bf16, bool causal, int64_t grid, hipStream_t st);
hipError_t launch_bwd_q(const BwdArgs& a, bool bf16, bool causal, int64_t grid, hipStream_t st);
// Segments of at most 32 gathered rows (the plan's one-wave case): dq, dk,
// dv and D in one kernel, one wave per unit.
hipError_t launch_bwd_short(const BwdArgs& a, bool bf16, bool causal, int64_t grid,
                            hipStream_t st);
hipError_t launch_bwd_merge(const BwdRowArgs& a, bool bf16, hipStream_t st);
// Fused qk_norm backward: the short-segment kernel's per-unit gain/bias
// gradient partials [2][units][2 kDh] folded (fixed order) into
// [2][qkn_groups(units)][2 kDh], then summed by launch_qk_norm_reduce.
int64_t qkn_groups(int64_t units);
hipError_t launch_qkn_fold(const float* part, int64_t units, float* folded, hipStream_t st);
hipError_t launch_qk_norm_reduce(const float* partials, int64_t nblk, float* dparams,
                                 hipStream_t st);

// qk_norm (qknorm_kernel.hip): blocks per tensor for `rows` rows; forward;
// backward (row gradients, per-block partials of the gain and bias
// gradients, then their fixed-order sum).
int64_t qk_norm_blocks(int64_t rows);
hipError_t launch_qk_norm_fwd(const QkNormArgs& a, bool bf16, hipStream_t st);
hipError_t launch_qk_norm_bwd(const QkNormArgs& a, bool bf16, hipStream_t st);

// Test hooks: dump the gather map / the inverse (coverage) map of one
// pattern for one head, computed with the kernels' own index functions.
hipError_t launch_gather_map(const PatDev& p, int32_t h, int64_t* out, hipStream_t st);
hipError_t launch_coverage_map(const PatDev& p, int32_t h, int64_t N, int64_t* out,
                               hipStream_t st);

}  // namespace da
