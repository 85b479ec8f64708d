/*
 * dilated_attn.h — C ABI of the MI355X (gfx950) dilated-attention forward and
 * backward passes.
 *
 * The operation (sources: "LONGNET: Scaling Transformer to 1 billion tokens"
 * blog, sections "LongNet's attention allocation principle" and the
 * multi-head paragraph after it; "LongNet论文精读" page, section
 * "Dilated Attention的工作原理", steps 1-4; dakule.com news page, sections
 * "如何做到？" and "实验评估"):
 *
 *   For every pattern (w, r): w' = min(w, N); the sequence is cut into N/w'
 *   segments of w' tokens. Head h gathers, inside each segment, the rows at
 *   offsets (h mod r) + m*r < w' (m = 0 .. L-1, L = ceil((w' - h mod r) / r)),
 *   runs softmax attention among them (causal over the gathered order when
 *   asked), and scatters the result back to those rows. The per-pattern
 *   results O_i with log-sum-exp lse_i of each row are then merged:
 *       LSE = log(sum_i exp(lse_i)),  out = sum_i exp(lse_i - LSE) * O_i
 *   over the patterns that gather the row; rows no pattern gathers get
 *   out = 0 and lse = -inf. The pages do not print the merge weights; this
 *   weighting by each pattern's softmax denominator is the reading this
 *   library implements.
 *
 * Layout (all row-major, contiguous):
 *   q, k, v, out : [B, N, H, Dh], one element type for all four
 *                  (DA_F32: float, DA_BF16: bfloat16), dim = H * Dh.
 *   lse          : [B, H, N] float, natural logarithm.
 * Scores are scale * (q . k); scale <= 0 selects 1/sqrt(Dh).
 *
 * Memory and ownership: every pointer except `patterns` (host) and the
 * stream handle is DEVICE memory owned by the caller. The library allocates
 * nothing and keeps no pointer after a call returns. Its only mutable global
 * state is the per-GPU device array behind dilated_attn_fwd_noalloc (see
 * there); every other call may run concurrently with others on different
 * streams as long as they do not share output or workspace buffers.
 *
 * Asynchrony: compute calls enqueue kernels on `stream` (a hipStream_t; NULL
 * is the default stream) and return without synchronising. Faults during
 * execution surface at the caller's next synchronisation.
 *
 * Errors: every call validates all arguments before launching anything.
 * A non-zero return other than DA_ERR_LAUNCH means nothing was launched and
 * nothing was written. DA_ERR_LAUNCH (the runtime rejected a launch) can
 * follow kernels of the same call that were already enqueued on the stream
 * (an attention launch before a failed merge launch, earlier backward
 * stages); the outputs are then undefined.
 *
 * Inputs are not checked for finiteness. Elements of q, k, v are expected
 * to be finite: a NaN or infinity reaches the rows whose softmax it enters
 * with unspecified values (the kernels take maxima without NaN ordering).
 */
#ifndef DILATED_ATTN_H
#define DILATED_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DA_VERSION 1
#define DA_MAX_PATTERNS 8
#define DA_HEAD_DIM 64

/* One (segment length, dilation rate) pattern. w >= 1, r >= 1 and
 * r <= min(w, N); N must be a multiple of min(w, N). */
typedef struct {
  int32_t w;
  int32_t r;
} da_pattern;

enum { DA_F32 = 0, DA_BF16 = 1 };

enum {
  DA_OK = 0,
  DA_ERR_NULL = -1,      /* a required pointer is NULL                          */
  DA_ERR_SHAPE = -2,     /* B, N or H negative, N not a multiple of min(w, N),  */
                         /* or sizes beyond the supported range: N * H and     */
                         /* B below 2^31 and 2^16, and one segment plus 128    */
                         /* dilated rows, (min(w,N) + 128 r) * H * Dh * element */
                         /* size, below 2^31 bytes                             */
  DA_ERR_PATTERN = -3,   /* n_patterns outside 1..DA_MAX_PATTERNS, w < 1,       */
                         /* r < 1 or r > min(w, N)                              */
  DA_ERR_DTYPE = -4,     /* dtype is not DA_F32 or DA_BF16                      */
  DA_ERR_HEADDIM = -5,   /* Dh != DA_HEAD_DIM                                   */
  DA_ERR_WORKSPACE = -6, /* workspace NULL or smaller than required             */
  DA_ERR_ALIGN = -7,     /* q, k, v, out not 16-byte, lse not 4-byte, or        */
                         /* workspace not 256-byte aligned                      */
  DA_ERR_ALIAS = -8,     /* out, lse or workspace overlaps an input or another  */
                         /* output                                              */
  DA_ERR_ARG = -9,       /* other invalid scalar (scale not finite, causal not  */
                         /* 0/1, capacity too small)                            */
  DA_ERR_LAUNCH = -10    /* the HIP runtime rejected a kernel launch            */
};

/* Bytes of device workspace dilated_attn_fwd needs for this problem (0 for
 * a single pattern, whose kernel writes out and lse directly). For two or
 * more patterns it holds each pattern's per-row partial output (float, Dh
 * per gathered row) and log-sum-exp before the merge: the per-pattern
 * results of the mixture of dilated patterns (dakule.com news page, "如何
 * 做到？"; LONGNET blog, "LongNet's attention allocation principle") that
 * the merge weighs by their softmax denominators. Writes *bytes and returns
 * DA_OK, or an error code for invalid arguments. */
int dilated_attn_workspace_bytes(int64_t B, int64_t N, int32_t H, int32_t Dh,
                                 const da_pattern* patterns, int32_t n_patterns, int32_t dtype,
                                 size_t* bytes);

/* The whole forward pass (LONGNET blog, "LongNet's attention allocation
 * principle" and the multi-head paragraph after it; "LongNet论文精读" page,
 * "Dilated Attention的工作原理", steps 1-4: segment, gather every r-th row
 * from the head's offset, dense attention inside each sparsified segment,
 * scatter back; dakule.com news page, "实验评估", for the mixture of
 * patterns): dilated attention for every pattern, then the log-sum-exp
 * merge. Writes every element of out and lse. causal is 0 or 1.
 * workspace: device memory of at least dilated_attn_workspace_bytes() bytes,
 * 256-byte aligned (may be NULL when that size is 0); its contents on entry
 * are ignored. Returns DA_OK or a DA_ERR_* code. */
int dilated_attn_fwd(const void* q, const void* k, const void* v, void* out, float* lse,
                     int64_t B, int64_t N, int32_t H, int32_t Dh, const da_pattern* patterns,
                     int32_t n_patterns, int32_t causal, int32_t dtype, float scale,
                     void* workspace, size_t workspace_bytes, void* stream);

/* The two stages of dilated_attn_fwd, exposed separately so a caller can
 * time each kernel with events between them. Same arguments and checks as
 * dilated_attn_fwd; calling _attention then _merge on one stream with the
 * same arguments is exactly dilated_attn_fwd.
 *  _attention: one launch covering every pattern. It writes out and lse for
 *              every row that exactly one pattern gathers (with a single
 *              pattern also 0 / -inf for the rows it does not gather), and
 *              workspace partials for rows that several patterns gather.
 *  _merge:     combines the workspace partials into out and lse for rows
 *              two or more patterns gather, and writes 0 / -inf for rows no
 *              pattern gathers; does nothing for a single pattern. */
int dilated_attn_fwd_attention(const void* q, const void* k, const void* v, void* out, float* lse,
                               int64_t B, int64_t N, int32_t H, int32_t Dh,
                               const da_pattern* patterns, int32_t n_patterns, int32_t causal,
                               int32_t dtype, float scale, void* workspace,
                               size_t workspace_bytes, void* stream);
int dilated_attn_fwd_merge(const void* q, const void* k, const void* v, void* out, float* lse,
                           int64_t B, int64_t N, int32_t H, int32_t Dh,
                           const da_pattern* patterns, int32_t n_patterns, int32_t causal,
                           int32_t dtype, float scale, void* workspace, size_t workspace_bytes,
                           void* stream);

/* ------------------------------------------------------------------ backward
 *
 * Gradients of sum(dout * out) with respect to q, k and v, for training
 * (LongNet package README, "Key Advantages": training runs and the
 * distributed trainer; LONGNET blog, "Token expansion reaches 1 billion+").
 * With the merge above, a row's output is one softmax over the multiset of
 * (pattern, key) pairs its covering patterns give it, so with the merged
 * lse and D = dout . out of each row:
 *     P = exp(scale q.k - lse),  dS = P (dout . v - D),
 *     dq = scale sum dS k,  dk = scale sum dS q,  dv = sum P dout,
 * summed over every (pattern, segment) that gathers both rows. Rows no
 * pattern gathers get zero gradients.
 *
 * Inputs: q, k, v as given to dilated_attn_fwd; out and lse as it returned
 * them (same patterns, causal flag and scale); dout [B, N, H, Dh] in the
 * element type of q. Outputs: dq, dk, dv [B, N, H, Dh] in that element type,
 * every element written. Same alignment rules as the forward pass (the
 * tensors 16-byte, lse 4-byte, workspace 256-byte aligned). dq, dk, dv and
 * the workspace must not overlap each other or any input (DA_ERR_ALIAS);
 * inputs may overlap each other. The workspace is required (it holds D, and
 * the partials of rows several patterns gather; when every segment gathers
 * at most 32 rows D stays in registers and only the partials use it) and its
 * contents on entry are ignored. */

/* Bytes of device workspace dilated_attn_bwd needs: one float per row for D
 * and, for two or more patterns, the per-pattern partial dq, dk, dv rows of
 * rows several patterns gather, in the gradients' dtype (so the size depends
 * on dtype). Writes *bytes and returns DA_OK, or an error code for invalid
 * arguments. */
int dilated_attn_bwd_workspace_bytes(int64_t B, int64_t N, int32_t H, int32_t Dh,
                                     const da_pattern* patterns, int32_t n_patterns,
                                     int32_t dtype, size_t* bytes);

/* The whole backward pass. Returns DA_OK or a DA_ERR_* code. */
int dilated_attn_bwd(const void* q, const void* k, const void* v, const void* out,
                     const float* lse, const void* dout, void* dq, void* dk, void* dv, int64_t B,
                     int64_t N, int32_t H, int32_t Dh, const da_pattern* patterns,
                     int32_t n_patterns, int32_t causal, int32_t dtype, float scale,
                     void* workspace, size_t workspace_bytes, void* stream);

/* Stages of dilated_attn_bwd, for timing each kernel. Launched in this
 * order on one stream, all four are exactly dilated_attn_bwd:
 *  DA_BWD_PREP:  D = dout . out of every row into the workspace;
 *  DA_BWD_KV:    dk and dv of every row one pattern gathers, workspace
 *                partials of rows several patterns gather (needs D);
 *  DA_BWD_Q:     the same for dq (needs D);
 *  DA_BWD_MERGE: sums the partials of rows several patterns gather and
 *                writes zeros to rows no pattern gathers.
 * When every pattern's segments gather at most 32 rows (ceil(min(w, N) / r)
 * <= 32 for all patterns), DA_BWD_KV runs one kernel that forms D itself and
 * writes dq, dk and dv (or their partials); DA_BWD_PREP and DA_BWD_Q then
 * launch nothing.
 * stages is a non-empty OR of these flags (else DA_ERR_ARG); the other
 * arguments and checks are those of dilated_attn_bwd. */
enum { DA_BWD_PREP = 1, DA_BWD_KV = 2, DA_BWD_Q = 4, DA_BWD_MERGE = 8, DA_BWD_ALL = 15 };
int dilated_attn_bwd_stages(int32_t stages, const void* q, const void* k, const void* v,
                            const void* out, const float* lse, const void* dout, void* dq,
                            void* dk, void* dv, int64_t B, int64_t N, int32_t H, int32_t Dh,
                            const da_pattern* patterns, int32_t n_patterns, int32_t causal,
                            int32_t dtype, float scale, void* workspace, size_t workspace_bytes,
                            void* stream);

/* ------------------------------------------------------------------ qk_norm
 *
 * The DilatedAttention module's optional query-key normalisation (LongNet
 * package README, DilatedAttention parameter qk_norm): every row of
 * Dh = DA_HEAD_DIM query values and every row of key values is layer-
 * normalised, y = (x - mean) / sqrt(var + eps) * gain + bias, with the
 * biased variance over the row and one gain and bias vector (Dh values
 * each) per tensor, shared by all heads.
 *
 * xq, xk, yq, yk, dyq, dyk, dxq, dxk: rows x Dh contiguous device arrays
 * (e.g. [B, N, H, Dh], rows = B * N * H) of `dtype`; gains and biases: Dh
 * values of `dtype`. All 16-byte aligned. Outputs must not overlap any
 * input or each other (DA_ERR_ALIAS). eps must be finite and > 0
 * (DA_ERR_ARG). rows = 0 is a no-op. */
int dilated_attn_qk_norm_fwd(const void* xq, const void* xk, const void* gain_q,
                             const void* bias_q, const void* gain_k, const void* bias_k, void* yq,
                             void* yk, int64_t rows, int32_t Dh, int32_t dtype, float eps,
                             void* stream);

/* Device workspace bytes dilated_attn_qk_norm_bwd needs for `rows` rows
 * (per-block partial sums of the gain and bias gradients). */
int dilated_attn_qk_norm_workspace_bytes(int64_t rows, size_t* bytes);

/* Backward of dilated_attn_qk_norm_fwd: dxq, dxk (rows x Dh, dtype) and
 * dparams, a device float array [2][2][Dh]: [0][0] dgain_q, [0][1] dbias_q,
 * [1][0] dgain_k, [1][1] dbias_k (4-byte aligned, every element written).
 * The row statistics are recomputed from xq and xk. workspace: at least
 * dilated_attn_qk_norm_workspace_bytes(rows), 256-byte aligned. The sums
 * over rows are taken in a fixed order: results are deterministic. */
int dilated_attn_qk_norm_bwd(const void* xq, const void* xk, const void* dyq, const void* dyk,
                             const void* gain_q, const void* gain_k, void* dxq, void* dxk,
                             float* dparams, int64_t rows, int32_t Dh, int32_t dtype, float eps,
                             void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------ qk_norm fused
 *
 * The DilatedAttention module with qk_norm (LongNet package README,
 * DilatedAttention parameters) in one pass per direction, for one pattern
 * whose segments gather at most 32 rows (ceil(min(w, N) / r) <= 32, e.g. the
 * README's usage example): q = qk_norm(xq), k = qk_norm(xk) as defined for
 * dilated_attn_qk_norm_fwd are formed inside the attention kernels as rows
 * are loaded and never stored. Any other pattern list returns
 * DA_ERR_PATTERN; the separate dilated_attn_qk_norm_* and dilated_attn_*
 * calls compute the same values there.
 *
 * xq, xk, v as q, k, v of dilated_attn_fwd (the un-normalised rows), except
 * that row_stride gives the elements between consecutive positions of each
 * (0: H * Dh, the dense [B, N, H, Dh] layout; otherwise at least H * Dh, the
 * rows 16-byte aligned, DA_ERR_ARG / DA_ERR_ALIGN): xq, xk, v may then be
 * the three parts of one [B, N, 3, H, Dh] buffer, as one projection GEMM
 * writes them (row_stride 3 H Dh). out and lse keep their dense layouts.
 * Gains and biases: Dh values of dtype, 16-byte aligned, not overlapping any
 * output; eps finite and > 0 (DA_ERR_ARG). No workspace. Other arguments,
 * checks and outputs as dilated_attn_fwd. */
int dilated_attn_fwd_qknorm(const void* xq, const void* xk, const void* v, const void* gain_q,
                            const void* bias_q, const void* gain_k, const void* bias_k,
                            float eps, void* out, float* lse, int64_t B, int64_t N, int32_t H,
                            int32_t Dh, int64_t row_stride, const da_pattern* patterns,
                            int32_t n_patterns, int32_t causal, int32_t dtype, float scale,
                            void* stream);

/* Device workspace bytes of dilated_attn_bwd_qknorm (the backward's own,
 * plus per-(batch, head, segment) partial sums of the gain and bias
 * gradients). DA_ERR_PATTERN where the fused form does not apply. */
int dilated_attn_bwd_qknorm_workspace_bytes(int64_t B, int64_t N, int32_t H, int32_t Dh,
                                            const da_pattern* patterns, int32_t n_patterns,
                                            int32_t dtype, size_t* bytes);

/* Backward of dilated_attn_fwd_qknorm: dxq, dxk (gradients with respect to
 * the un-normalised rows, of dtype), dv, all three in the layout row_stride
 * gives xq, xk, v (they may interleave in one buffer; rows of one must not
 * touch rows of another, DA_ERR_ALIAS), and dparams, a device
 * float array [2][2][Dh] as for dilated_attn_qk_norm_bwd (gain_q, bias_q,
 * gain_k, bias_k gradients), all written. out and lse as dilated_attn_fwd_qknorm
 * returned them. The gain and bias gradients are summed in a fixed order
 * (no atomics). Other arguments, checks and rules as dilated_attn_bwd; dparams
 * must not overlap any other buffer (DA_ERR_ALIAS). */
int dilated_attn_bwd_qknorm(const void* xq, const void* xk, const void* v, const void* gain_q,
                            const void* bias_q, const void* gain_k, const void* bias_k,
                            float eps, const void* out, const float* lse, const void* dout,
                            void* dxq, void* dxk, void* dv, float* dparams, int64_t B, int64_t N,
                            int32_t H, int32_t Dh, int64_t row_stride, const da_pattern* patterns,
                            int32_t n_patterns, int32_t causal, int32_t dtype, float scale,
                            void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------ one pass
 *
 * The forward of dilated_attn_fwd in a single launch, with no workspace and
 * no merge pass (bf16 only; DA_ERR_DTYPE for fp32). Each row's merged
 * output is one softmax over every (pattern, key) pair its covering
 * patterns give it (the LSE merge of the per-pattern results, reading of
 * the LONGNET blog's "Dilated Attention" mixture and the dakule.com news
 * article's pattern list), so a workgroup streams the keys of every pattern
 * that covers its rows through one online softmax and writes final rows.
 * Rows are grouped by position residue mod L = lcm(r) inside windows of
 * W = gcd(min(w, N)) positions, which every pattern covers all or none of.
 * DA_ERR_PATTERN when L > W. Arguments, checks and outputs as
 * dilated_attn_fwd without the workspace; results equal dilated_attn_fwd's
 * up to rounding order. */
int dilated_attn_fwd_onepass(const void* q, const void* k, const void* v, void* out, float* lse,
                             int64_t B, int64_t N, int32_t H, int32_t Dh,
                             const da_pattern* patterns, int32_t n_patterns, int32_t causal,
                             int32_t dtype, float scale, void* stream);

/* ------------------------------------------------------------------ no allocation
 *
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the whole
 * forward pass of dilated_attn_fwd with the workspace taken from a
 * file-scope device array of DA_NOALLOC_MAX_WORKSPACE_BYTES bytes inside
 * the library instead of a caller buffer. The array exists once per GPU the
 * library runs on and is held until the process ends; its address is looked
 * up once per device (hipGetSymbolAddress). The call allocates nothing.
 * Problems whose dilated_attn_workspace_bytes() exceeds the array return
 * DA_ERR_WORKSPACE before anything is launched; DA_ERR_LAUNCH also covers a
 * failed address lookup. All calls on one GPU share that GPU's array and
 * nothing in it needs clearing between calls, but calls that overlap in
 * time on one GPU (different streams, or host threads) race on it: the
 * caller must order them. Arguments, other checks and outputs as
 * dilated_attn_fwd without the workspace; results are bit-identical to it. */
#define DA_NOALLOC_MAX_WORKSPACE_BYTES ((size_t)64 << 20)
int dilated_attn_fwd_noalloc(const void* q, const void* k, const void* v, void* out, float* lse,
                             int64_t B, int64_t N, int32_t H, int32_t Dh,
                             const da_pattern* patterns, int32_t n_patterns, int32_t causal,
                             int32_t dtype, float scale, void* stream);

/* Test hook: the gather map the kernels use (LONGNET blog, "LongNet's
 * attention allocation principle" and the multi-head paragraph after it:
 * segments of w tokens, every r-th token from the head's offset; "LongNet
 * 论文精读" page, "Dilated Attention的工作原理", steps 1-2), written by a
 * device kernel through the same index function as the attention kernel.
 * shape: host int64[2], may be NULL; receives the map's shape
 * {N / min(w, N), ceil(min(w, N) / r)} (segments, rows per segment of a head
 * with offset 0). dev_out: device int64 array of that shape, segment-major;
 * entry [s][m] is the sequence position of gathered row m of segment s for
 * head h, or -1 where m >= L(h). cap is dev_out's length in elements and must
 * be at least shape[0] * shape[1]. With dev_out NULL the call only fills
 * shape (which must then be non-NULL) and launches nothing. */
int dilated_attn_gather_map(int64_t N, int32_t H, da_pattern pattern, int32_t h, int64_t* dev_out,
                            int64_t cap, int64_t* shape, void* stream);

/* Test hook: the inverse map the merge kernel uses. dev_out: device int64
 * [N]; entry t is s * ceil(min(w, N) / r) + m when position t is gathered
 * row m of segment s for head h, else -1. cap must be at least N. */
int dilated_attn_coverage_map(int64_t N, int32_t H, da_pattern pattern, int32_t h,
                              int64_t* dev_out, int64_t cap, void* stream);

/* Static description of an error code (never NULL). */
const char* dilated_attn_strerror(int code);

/* DA_VERSION of the built library. */
int dilated_attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DILATED_ATTN_H */
