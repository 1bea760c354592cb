/*
 * moe.h -- C ABI of libmoe.so, the MI355X (gfx950) MoE expert-FFN path.
 *
 * The operations follow four pages on the subject:
 *   [TE-MoE]   TransformerEngine pull request "[JAX] Add an MoE Block (Layer)
 *              that compound router, permutation, groupedGEMM and
 *              communication": the block's sequence diagram (route -> dispatch
 *              -> grouped GEMM x3 -> combine, and the mirrored backward), the
 *              review of _combine_bwd, the align_size receive-buffer bound and
 *              the commit notes on the SwiGLU projection outputs.
 *   [MT-Chunk] MaxText pull request "Overlap moe comms with collective
 *              matmul": gmm/tgmm with in-place partial-sum accumulation,
 *              tgmm zero-initialised empty groups, the gmm backward rule.
 *   [MT-GG]    MaxText pull request "[Draft] Integrate TE/JAX GroupedGEMM for
 *              MoE": grouped vs batched GEMM, token dropping (Tests).
 *   [MT-ES]    MaxText pull request "Onboard explicit sharding to deepseek":
 *              gate projection shape and the expert weight layouts.
 *
 * Conventions shared by every call
 *   - Every data pointer is a DEVICE pointer owned by the caller.  The library
 *     never allocates, frees or synchronises and keeps no state between calls.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Each
 *     call enqueues its kernels on it and returns; results are valid in stream
 *     order.
 *   - Return value: MOE_OK (0), or a negative MOE_ERR_* when the host-side
 *     argument check fails (nothing is launched in that case) or a launch
 *     fails.  moe_status_string() gives the text.  No call aborts or throws.
 *   - Data errors only the device can see (an expert id outside [0, E), group
 *     sizes that are negative or overrun the buffer) never cause an
 *     out-of-bounds access: the offending item is skipped and a MOE_DERR_* bit
 *     is OR-ed into the caller's int32 word `err` (may be NULL).
 *   - dtype codes: MOE_F32 or MOE_BF16 for activations and weights.  Expert
 *     ids, group sizes and row maps are int32; logits and routing weights
 *     are float32.  Lengths are int64.  Leading dimensions (ld_*) and strides
 *     are in elements.  All matrices are row-major.
 *   - Slot s = t*K + j is token t's j-th routing choice.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  MOE_OK = 0,
  MOE_ERR_ARG = -1,         /* bad size, null pointer, misaligned pointer/stride */
  MOE_ERR_DTYPE = -2,       /* unsupported dtype or dtype combination */
  MOE_ERR_CAPACITY = -3,    /* a buffer is smaller than the static bound */
  MOE_ERR_LAUNCH = -4,      /* the HIP runtime refused a launch */
  MOE_ERR_WORKSPACE = -5    /* workspace too small or misaligned */
};

enum { MOE_F32 = 0, MOE_BF16 = 1 };
enum { MOE_SOFTMAX = 0, MOE_SIGMOID = 1 };
/* How a per-expert routing bias enters: added to the logits (selection and
 * weights), or added to the scores for the selection only. */
enum { MOE_BIAS_LOGIT = 0, MOE_BIAS_SELECT = 1 };
/* FP8 formats (OCP): E4M3FN (bias 7, fmax 448) and E5M2 (bias 15, fmax 57344) */
enum { MOE_FP8_E4M3 = 0, MOE_FP8_E5M2 = 1 };

/* bits OR-ed into the device error word */
enum {
  MOE_DERR_EXPERT_ID = 1,   /* an expert id outside [0, E): that slot was dropped */
  MOE_DERR_GROUP_SIZES = 2, /* negative group size or sum(group_sizes) > rows: clipped */
  MOE_DERR_ROWS = 4         /* permuted rows exceed the output buffer: clipped */
};

const char* moe_status_string(int status);
int moe_abi_version(void);  /* bumped on any signature change */

/* -------------------------------------------------------------- routing
 * moe_route: top-K routing [TE-MoE, Description/Changes: fused top-K with
 * optional grouped/sigmoid scoring; MaxText DeepSeek-V3 router:
 * pre_bias_logits, n_routing_groups / topk_routing_group].
 *   Scores: MOE_SOFTMAX p = softmax over all E of z; MOE_SIGMOID
 *   p = 1/(1+e^-z); z = logits + bias (bias_mode MOE_BIAS_LOGIT; -inf
 *   switches an expert off) or z = logits (MOE_BIAS_SELECT).
 *   Selection key, float32: z (MOE_BIAS_LOGIT) or p + bias (MOE_BIAS_SELECT:
 *   the bias moves only the selection).  Experts are ranked by key
 *   descending; an equal key ranks the lower id first; topk_ids[t, j] is the
 *   j-th ranked expert.
 *   Grouped selection (n_groups > 1, E % n_groups == 0, n_groups <= 64,
 *   1 <= topk_groups <= n_groups, K <= topk_groups * E / n_groups): experts
 *   [g E/n_groups, (g+1) E/n_groups) form group g, scored by the sum of its
 *   two largest keys (float32; its only key if groups have one expert); the
 *   topk_groups best groups (ties: lower g) keep their experts as
 *   candidates.  n_groups <= 1: no grouping (topk_groups ignored).
 *   topk_w[t, j] = p of the j-th expert, divided by the sum over the K
 *   selected when renorm != 0.
 *   logits [T, E] f32, bias [E] f32 or NULL, topk_ids [T, K] i32,
 *   topk_w [T, K] f32.  Requires 1 <= K <= E <= 1024, K <= 64.
 */
int moe_route(const float* logits, const float* bias, int bias_mode, int n_groups,
              int topk_groups, int64_t T, int E, int K, int score, int renorm, int32_t* topk_ids,
              float* topk_w, void* stream);

/* moe_route_bwd: d_logits [T, E] (fully written) from d_topk_w [T, K], with
 * the selection topk_ids held fixed (the gate-kernel gradient path of the
 * [TE-MoE] block backward).  Same logits/bias/bias_mode/score/renorm as the
 * forward (a MOE_BIAS_SELECT bias does not enter the weights, so it has no
 * gradient path).  d_logits is stored in dlogits_dtype (MOE_F32, or
 * MOE_BF16 to feed a bf16 router-GEMM backward); the arithmetic is float32.
 *   softmax+renorm: dz_ej = w_j (dw_j - sum_i w_i dw_i), others 0
 *   softmax:        dz_e  = p_e ([e = e_j] dw_j - sum_i p_ei dw_i), all e
 *   sigmoid+renorm: dz_ej = s_j(1-s_j)(dw_j - sum_i w_i dw_i) / sum_i s_i
 *   sigmoid:        dz_ej = dw_j s_j (1 - s_j)
 */
int moe_route_bwd(const float* logits, const float* bias, int bias_mode, const int32_t* topk_ids,
                  const float* d_topk_w, int64_t T, int E, int K, int score, int renorm,
                  void* d_logits, int dlogits_dtype, void* stream);

/* Workspace bytes moe_aux_loss needs (256-byte aligned device memory). */
size_t moe_aux_loss_workspace(int64_t T, int E);

/* moe_aux_loss: the auxiliary load-balancing loss [TE-MoE, Description:
 * optional auxiliary load-balancing loss]:
 *   f_e = (selected slots of expert e in topk_ids) / (T K)
 *   P_e = (1/T) sum_t p_te,  p = softmax of the logits over the E experts,
 *         or for MOE_SIGMOID the sigmoids of the logits normalised to sum 1
 *   loss = alpha * E * sum_e f_e P_e   (one float32, device)
 * expert_counts [E] (T K f_e) and expert_probs [E] (P_e) are written when
 * not NULL; the backward needs the counts.  Sums are taken in a fixed order
 * (deterministic).  T >= 1.
 */
int moe_aux_loss(const float* logits, const int32_t* topk_ids, int64_t T, int E, int K, int score,
                 float alpha, float* loss, int32_t* expert_counts, float* expert_probs,
                 void* workspace, size_t ws_bytes, void* stream);

/* moe_aux_loss_bwd: d_logits (+)= d loss / d logits with the counts held
 * fixed (f carries no gradient):
 *   softmax: (alpha E / T) p_tk (f_k - sum_e f_e p_te)
 *   sigmoid: (alpha E / T) s_tk (1 - s_tk) / S_t (f_k - sum_e f_e p_te)
 * accumulate != 0 adds into d_logits (e.g. after moe_route_bwd).
 */
int moe_aux_loss_bwd(const float* logits, const int32_t* expert_counts, int64_t T, int E, int K,
                     int score, float alpha, void* d_logits, int dlogits_dtype, int accumulate,
                     void* stream);

/* -------------------------------------------------------------- permutation
 * moe_rows_bound: the static row count of the expert-sorted buffers:
 *   capacity_layout: E*capacity;  align > 0: T*K + E*(align-1) (the
 *   worst-case receive-buffer bound for align_size > 0 in the [TE-MoE]
 *   review);  otherwise T*K.  Returns -1 on bad arguments.
 */
int64_t moe_rows_bound(int64_t T, int K, int E, int align, int capacity, int capacity_layout);

/* Workspace bytes moe_permute needs (256-byte aligned device memory). */
size_t moe_permute_workspace(int64_t T, int K, int E);

/* moe_permute: group the routed slots by expert (the [TE-MoE] "global
 * permute" with group_sizes and align_size; token dropping in router order
 * as in the [MT-GG] Tests).
 *   Router order is ascending slot s.  With capacity C > 0 a slot is kept iff
 *   fewer than C earlier slots chose the same expert.  counts[e] = kept slots
 *   of e.  group_sizes[e] = counts[e] rounded up to a multiple of align
 *   (align > 0; 0 stays 0), or C for every expert in capacity_layout.
 *   group_offsets[e] = sum of earlier group sizes, group_offsets[E] = total.
 *   Inside a group the kept slots are in ascending s (stable), followed by
 *   the group's padding rows.
 *   row_of_slot[s] = destination row, -1 if dropped.  slot_of_row[r] = source
 *   slot, -1 for padding rows (including every row >= group_offsets[E]).
 *   x_sorted[r] = x[slot_of_row[r] / K], zero for padding rows.
 *   x [T, D] and x_sorted [rows, D] in `dtype`; rows >= moe_rows_bound(...).
 *   x_sorted may be NULL (index maps only).  Requires E <= 1024, K <= 64.
 */
int moe_permute(const void* x, int dtype, int64_t T, int64_t D, const int32_t* topk_ids, int K,
                int E, int align, int capacity, int capacity_layout, void* x_sorted, int64_t rows,
                int32_t* counts, int32_t* group_sizes, int32_t* group_offsets,
                int32_t* row_of_slot, int32_t* slot_of_row, void* workspace, size_t ws_bytes,
                int32_t* err, void* stream);

/* Scratch words (int32) of moe_permute_noalloc: 262144 (1 MiB per GPU). */
#define MOE_PERMUTE_NOALLOC_SCRATCH_WORDS 262144

/* moe_permute_noalloc: moe_permute without a workspace argument, for callers
 * that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc).  Same arguments, results
 * and errors as moe_permute; it calls no allocating routine.  Its per-block
 * expert counts live in a static device array of the library (one per GPU,
 * held until the process ends), so it supports
 * moe_permute_workspace(T, K, E) <= 4 * MOE_PERMUTE_NOALLOC_SCRATCH_WORDS
 * bytes (ceil(T K / 1024) * E <= 262144; e.g. T K <= 1M slots with E = 256)
 * and returns MOE_ERR_WORKSPACE beyond that.  Every call on one GPU shares
 * that array: calls that may overlap on one GPU (different streams without
 * ordering, several host threads) race and must be serialised by the
 * caller.  No entry needs to start at zero (each call writes every entry
 * it reads).
 */
int moe_permute_noalloc(const void* x, int dtype, int64_t T, int64_t D, const int32_t* topk_ids,
                        int K, int E, int align, int capacity, int capacity_layout,
                        void* x_sorted, int64_t rows, int32_t* counts, int32_t* group_sizes,
                        int32_t* group_offsets, int32_t* row_of_slot, int32_t* slot_of_row,
                        int32_t* err, void* stream);

/* moe_permute_bwd: d_x[t] (+)= sum_j d_x_sorted[row_of_slot[t*K+j]] over kept
 * slots (adjoint of the row gather; the dispatch backward of [TE-MoE]).
 * accumulate != 0 adds into d_x.  d_x_sorted [rows, D], d_x [T, D], both in
 * `dtype`; sums are taken in float32.
 */
int moe_permute_bwd(const void* d_x_sorted, int dtype, int64_t T, int64_t D, int K, int64_t rows,
                    const int32_t* row_of_slot, void* d_x, int accumulate, void* stream);

/* ------------------------------------------------------------ grouped GEMMs
 * moe_gmm: grouped GEMM [MT-Chunk; TE-MoE grouped_gemm].
 *   For group g with rows [o_g, o_g + n_g), o_g = sum_{g'<g} n_g':
 *     out[o_g + i, :] (+)= lhs[o_g + i, :Kdim] . B_g
 *   where B_g = rhs + g*rhs_group_stride viewed as [Kdim, N] with row stride
 *   ld_rhs (trans_rhs = 0), or as [N, Kdim] with row stride ld_rhs and used
 *   transposed (trans_rhs = 1).
 *   lhs: [M_lhs, Kdim] with row stride ld_lhs; out: [M_out, N] with row stride
 *   ld_out, M_out <= M_lhs (lhs may be padded to a row tile while the output
 *   is not).  accumulate != 0: out += product (in-place partial sum); rows
 *   >= sum(group_sizes) are left untouched.  accumulate == 0: out = product;
 *   rows in [sum(group_sizes), M_out) are zero-filled.
 *   in_dtype is the dtype of lhs and rhs; MOE_BF16 runs on bf16 MFMA with
 *   float32 accumulation; MOE_F32 runs in float32 FMA.  out_dtype is
 *   MOE_F32 or MOE_BF16 (rounded to nearest even).
 *   valid_rows (device, [G], may be NULL): the caller asserts that lhs rows
 *   [valid_rows[g], group_sizes[g]) of group g are zero (moe_permute's
 *   counts: align_size / capacity padding rows); those rows are not read and
 *   their products are written as zero.  NULL reads every row.
 *   bias (device, may be NULL): [G, N] row-major in in_dtype, the per-expert
 *   MLP bias of the [MT-Chunk] chunked layer (its w0/w1/wo bias arguments;
 *   Testing: MLP bias with the chunked layer).  bias[g] is added to every
 *   output row of group g, after the product and any partial sum; under
 *   partial sums pass it with one of the calls only.
 *   Requires Kdim, N, ld_* and strides to be multiples of 8 and 16-byte
 *   aligned pointers.  G <= 1024.  If sum(group_sizes) > M_out the groups are
 *   clipped at M_out and MOE_DERR_GROUP_SIZES is raised.
 */
int moe_gmm(const void* lhs, int64_t M_lhs, int64_t ld_lhs, const void* rhs, int64_t ld_rhs,
            int64_t rhs_group_stride, int trans_rhs, const int32_t* group_sizes,
            const int32_t* valid_rows, int G, int64_t Kdim, int64_t N, int in_dtype,
            const void* bias, void* out, int64_t M_out, int64_t ld_out, int out_dtype,
            int accumulate, int32_t* err, void* stream);

/* moe_gmm_swiglu: the up-projection with a fused weight and the SwiGLU
 * activation in its epilogue (the fused gate/up weight of [TE-MoE]; the
 * gate_proj_out / up_proj_out pair its commit notes name; SwiGLU as in
 * moe_swiglu).  rhs + g*rhs_group_stride is wi[g] = [wi_0[g] | wi_1[g]]
 * viewed as [Kdim, 2F] with row stride ld_rhs (gate columns 0..F-1, up
 * columns F..2F-1).  For each group (rows as moe_gmm's):
 *     h[o_g + i, :]   = lhs[o_g + i, :Kdim] . wi[g] (+ bias[g])   [rows, 2F]
 *     act[o_g + i, :] = silu(h[.., :F]) * h[.., F:]                [rows, F]
 *   with act computed from the bf16-rounded h, so the result equals
 *   moe_gmm into h followed by moe_swiglu on its halves, bit for bit.
 *   h (may be NULL: not written) keeps the pre-activation values the
 *   backward needs; row stride ld_h >= 2F.  act has row stride ld_act >= F.
 *   Rows in [sum(group_sizes), M_out) of h and act are zero-filled.
 *   valid_rows and bias as in moe_gmm (bias [G, 2F]).  bf16 only; F a
 *   multiple of 128; Kdim, ld_* and strides multiples of 8; 16-byte aligned
 *   pointers; G <= 1024.  No partial sums (chunked up-projections use
 *   moe_gmm, then moe_swiglu).
 */
int moe_gmm_swiglu(const void* lhs, int64_t M_lhs, int64_t ld_lhs, const void* rhs, int64_t ld_rhs,
                   int64_t rhs_group_stride, const int32_t* group_sizes, const int32_t* valid_rows,
                   int G, int64_t Kdim, int64_t F, int in_dtype, const void* bias, void* h,
                   int64_t ld_h, void* act, int64_t ld_act, int64_t M_out, int32_t* err,
                   void* stream);

/* moe_gmm_swiglu_bwd: the d_act GEMM of the backward with the SwiGLU
 * backward in its epilogue (the gradient counterpart of moe_gmm_swiglu).
 * For each group (rows as moe_gmm's), with wo[g] = rhs + g*rhs_group_stride
 * viewed as [F, Kdim] (row stride ld_rhs) and used transposed:
 *     d_act = bf16(lhs[o_g + i, :Kdim] . wo[g]^T)                    [rows, F]
 *     d_h0 = d_act * h1 * s * (1 + h0 * (1 - s)),  d_h1 = d_act * h0 * s,
 *   s = sigmoid(h0), from the forward's h0, h1 (row stride ld_h), written to
 *   d_h0, d_h1 (row stride ld_dh; both may be halves of one [rows, 2F]
 *   buffer).  Equal, bit for bit, to moe_gmm(trans_rhs) into a bf16 d_act
 *   followed by moe_swiglu_bwd.  Rows in [sum(group_sizes), M_out) of d_h0
 *   and d_h1 are zero-filled.  valid_rows as in moe_gmm.  bf16 only (lhs,
 *   rhs, h0, h1, d_h0, d_h1);
 *   F > 128 and Kdim > 32 (smaller shapes use the two calls); F, Kdim, ld_*
 *   and strides multiples of 8; 16-byte aligned pointers; G <= 1024.
 */
int moe_gmm_swiglu_bwd(const void* lhs, int64_t M_lhs, int64_t ld_lhs, const void* rhs,
                       int64_t ld_rhs, int64_t rhs_group_stride, const int32_t* group_sizes,
                       const int32_t* valid_rows, int G, int64_t Kdim, int64_t F, int in_dtype,
                       const void* h0, const void* h1, int64_t ld_h, void* d_h0, void* d_h1,
                       int64_t ld_dh, int64_t M_out, int32_t* err, void* stream);

/* moe_tgmm: transposed grouped GEMM [MT-Chunk: tgmm, output
 * (num_local_groups, in_size, out_size), zero-initialised empty groups].
 *   out[g] (+)= lhs[rows of g, :Kdim]^T . rhs[rows of g, :N]   -> [Kdim, N]
 *   lhs [M, Kdim] row stride ld_lhs; rhs [M, N] row stride ld_rhs; out[g]
 *   at out + g*out_group_stride with row stride ld_out.  An empty group's
 *   block is zero (accumulate == 0) or left unchanged (accumulate != 0).
 *   valid_rows (device, [G], may be NULL): the caller asserts that rows
 *   [valid_rows[g], group_sizes[g]) of group g are zero in lhs or in rhs;
 *   the contraction then stops after the first valid_rows[g] rows of the
 *   group (moe_permute's counts: the align_size / capacity padding rows
 *   carry zeros).  NULL contracts over every row of each group.
 *   Same dtype and alignment rules as moe_gmm.
 */
int moe_tgmm(const void* lhs, int64_t ld_lhs, const void* rhs, int64_t ld_rhs,
             const int32_t* group_sizes, const int32_t* valid_rows, int G, int64_t M,
             int64_t Kdim, int64_t N, int in_dtype, void* out, int64_t ld_out,
             int64_t out_group_stride, int out_dtype, int accumulate, int32_t* err,
             void* stream);

/* Workspace bytes moe_router_bwd needs (256-byte aligned device memory). */
size_t moe_router_bwd_workspace(int64_t T, int64_t D, int E);

/* moe_router_bwd: backward of the router GEMM logits = x . Wg (the gate
 * projection of the [TE-MoE] block; [MT-ES] review: [B, S, E] ->
 * [B, S, num_exp]), with the float32 d_logits of moe_route_bwd /
 * moe_aux_loss_bwd:
 *     d_Wg  = x^T . d_logits               [D, E] float32, fully written
 *     dx  (+)= d_logits . Wg^T             [T, D] in dx_dtype
 *   x [T, D] and Wg [D, E] contiguous bf16; d_logits [T, E] contiguous
 *   float32; dx contiguous, added to when accumulate_dx != 0 (the token
 *   gradient of the expert path is already there).  The products are those
 *   of float32 arithmetic: d_logits is split exactly into three bf16 planes
 *   (hi + mid + lo == d_logits) that the bf16 MFMA GEMMs contract with x and
 *   with three copies of Wg, accumulating in float32; d_Wg's per-block
 *   partial sums are added in a fixed order (deterministic).  Requires
 *   D a multiple of 8, 1 <= E <= 1024, 16-byte aligned x, Wg, dx.
 */
int moe_router_bwd(const void* x, const void* Wg, const float* d_logits, int64_t T, int64_t D,
                   int E, float* d_Wg, void* dx, int dx_dtype, int accumulate_dx,
                   void* workspace, size_t ws_bytes, int32_t* err, void* stream);

/* Workspace bytes moe_group_sum needs: (ceil(M / 256) + G) * N float32
 * partial rows (16-byte aligned device memory). */
size_t moe_group_sum_workspace(int64_t M, int G, int64_t N);

/* moe_group_sum: per-group column sums, the gradient of a per-expert MLP
 * bias [MT-Chunk chunked layer with MLP bias]:
 *   out[g, :] (+)= sum of rows [o_g, o_g + n_g) of in,  o_g = sum_{g'<g} n_g'
 *   in [M, N] with row stride ld_in, in in_dtype; out [G, N] row-major in
 *   out_dtype (MOE_F32 or MOE_BF16).  Sums are float32 in a fixed order
 *   (deterministic).  An empty group gives zero (accumulate == 0) or leaves
 *   out[g] unchanged (accumulate != 0).  valid_rows (device, [G], may be
 *   NULL): rows past valid_rows[g] in group g are zero and are skipped (as
 *   in moe_tgmm).  N and ld_in multiples of 8, 16-byte aligned pointers,
 *   G <= 1024; sum(group_sizes) > M raises MOE_DERR_GROUP_SIZES.
 */
int moe_group_sum(const void* in, int64_t ld_in, int in_dtype, const int32_t* group_sizes,
                  const int32_t* valid_rows, int G, int64_t M, int64_t N, void* out, int out_dtype,
                  int accumulate, void* workspace, size_t ws_bytes, int32_t* err, void* stream);

/* ------------------------------------------------------------------- FP8
 * The quantization=fp8 recipe of [MT-GG] (current-tensor scaling, e4m3 in
 * the forward, e5m2 in the backward, two quantized copies of each operand)
 * with the per-expert weight amax of [TE-MoE] commit notes.  moe_tgmm_fp8
 * takes both operands contraction-contiguous (the quantizer writes the
 * transposed copies of activations and gradients); moe_gmm_fp8 reads its
 * weight operand in either orientation, so one row-wise copy of a weight
 * serves the forward and the d_lhs product.  FP8 buffers are bytes; strides
 * in bytes (= elements).
 */

/* Workspace bytes of moe_fp8_amax_scale (16-byte aligned device memory). */
size_t moe_fp8_scale_workspace(int64_t rows, int64_t cols, int G);

/* moe_fp8_amax_scale: current scaling of x [rows, cols] (row stride ld,
 * dtype MOE_BF16 or MOE_F32) split into G equal blocks of rows / G rows (G = 1:
 * the whole tensor; G = E over a weight viewed as [E * a, b]: per expert).
 * Writes scales [3 G] float32: amax[g] = max |x| of block g, scale[g] =
 * fmax / amax[g] (1 if amax is 0), scale_inv[g] = 1 / scale[g] (correctly
 * rounded float32 divisions).  Requires rows % G == 0, cols and ld
 * multiples of 8.  Deterministic.
 */
int moe_fp8_amax_scale(const void* x, int64_t ld, int dtype, int64_t rows, int64_t cols, int G,
                       int fmt, float* scales, void* workspace, size_t ws_bytes, void* stream);

/* Column count P of a transposed copy in the padded layout: 64 * (ceil(rows /
 * 64) + G - 1) bounds the sum over groups of their rows rounded up to 64. */
int64_t moe_fp8_padded_rows(int64_t rows, int G);

/* moe_fp8_quantize: q = fp8(float32(x) * scale), the float32 product rounded
 * to the nearest FP8 value (ties to even), magnitudes above fmax saturated to
 * fmax, the sign kept.  x [rows, cols] (row stride ld) is split into groups
 * of group_sizes[g] consecutive rows (device, [G], G <= 1024); scale is
 * scale[g] (per_group != 0) or scale[0].
 *   q (may be NULL): row-wise copy [rows, cols], row stride ld_q; only rows
 *     inside groups are written.
 *   qt (may be NULL): transposed copy.  qt_group_stride == 0: one [cols, P]
 *     matrix (row stride ld_qt >= moe_fp8_padded_rows(rows, G)); group g's
 *     rows start at column 64 * sum_{g'<g} ceil(n_g' / 64) and the columns up
 *     to the group's next multiple of 64 are zero (the layout moe_tgmm_fp8
 *     reads).  qt_group_stride > 0: group g at qt + g * qt_group_stride as
 *     [cols, n_g] with row stride ld_qt (>= n_g); only the group's rows are
 *     written (a per-expert transposed weight copy).
 *   cols, ld, ld_q multiples of 8; ld_qt, qt_group_stride multiples of 16;
 *   16-byte aligned pointers.
 */
int moe_fp8_quantize(const void* x, int64_t ld, int dtype, int64_t rows, int64_t cols,
                     const int32_t* group_sizes, int G, const float* scale, int per_group, int fmt,
                     void* q, int64_t ld_q, void* qt, int64_t ld_qt, int64_t qt_group_stride,
                     int32_t* err, void* stream);

/* moe_gmm_fp8: grouped GEMM on FP8 operands (the semantics of moe_gmm):
 *   out[o_g + i, :] (+)= sa * sb[g] * lhs[o_g + i, :Kdim] . B_g (+ bias[g])
 *   lhs [M_lhs, Kdim] FP8 (lhs_fmt, row stride ld_lhs), sa = lhs_scale_inv[0];
 *   trans_rhs = 1: B_g^T = rhs + g * rhs_group_stride as [N, Kdim] (row stride
 *   ld_rhs >= Kdim); trans_rhs = 0: B_g as [Kdim, N] (row stride ld_rhs >= N,
 *   each row spanning ld_rhs bytes: the chunk holding column N - 1 is read
 *   whole), both in rhs_fmt; sb = rhs_scale_inv (device, [G]: per expert).  So
 *   one row-wise copy of a [K, N] weight serves both the forward (trans_rhs =
 *   0) and the d_lhs product (trans_rhs = 1).  Products are exact and
 *   accumulated in float32 by v_mfma_f32_32x32x64_f8f6f4; the scales are
 *   applied to the float32 sums.  valid_rows, bias: as in moe_gmm.  Output rows
 *   and accumulate as in moe_gmm.  Kdim, ld_lhs, ld_rhs, rhs_group_stride
 *   multiples of 16; N, ld_out multiples of 8; G <= 1000.
 */
int moe_gmm_fp8(const void* lhs, int64_t M_lhs, int64_t ld_lhs, int lhs_fmt,
                const float* lhs_scale_inv, const void* rhs, int64_t ld_rhs,
                int64_t rhs_group_stride, int trans_rhs, int rhs_fmt,
                const float* rhs_scale_inv,
                const int32_t* group_sizes, const int32_t* valid_rows, int G, int64_t Kdim,
                int64_t N, const void* bias,
                void* out, int64_t M_out, int64_t ld_out, int out_dtype, int accumulate,
                int32_t* err, void* stream);

/* moe_tgmm_fp8: transposed grouped GEMM on transposed FP8 copies in the
 * padded layout of moe_fp8_quantize (qt_group_stride == 0), for groups
 * group_sizes [G] of the M grouped rows:
 *   out[g] (+)= sa * sb * lhs_t[:Kdim, cols of g] . rhs_t[:N, cols of g]^T
 *   -> [Kdim, N] at out + g * out_group_stride (row stride ld_out).
 *   sa = lhs_scale_inv[0], sb = rhs_scale_inv[0].  The contraction covers
 *   each group's rows rounded up to 64 (zeros past its end), or valid_rows[g]
 *   rounded up to 64 when valid_rows (device, [G]) is given (rows past it are
 *   zero, as in moe_tgmm).  Empty groups: zero, or unchanged when
 *   accumulating.  ld_lhs, ld_rhs >= moe_fp8_padded_rows(M, G), multiples of
 *   16; G <= 1000.
 */
int moe_tgmm_fp8(const void* lhs_t, int64_t ld_lhs, int lhs_fmt, const float* lhs_scale_inv,
                 const void* rhs_t, int64_t ld_rhs, int rhs_fmt, const float* rhs_scale_inv,
                 const int32_t* group_sizes, const int32_t* valid_rows, int G, int64_t M,
                 int64_t Kdim, int64_t N, void* out, int64_t ld_out, int64_t out_group_stride,
                 int out_dtype, int accumulate, int32_t* err, void* stream);

/* -------------------------------------------------------------------- SwiGLU
 * moe_swiglu: act = silu(h0) * h1, silu(z) = z / (1 + e^-z), computed in
 * float32 (gate_proj_out / up_proj_out of the [TE-MoE] SwiGLU FFN).
 * h0, h1 [rows, F] in h_dtype with row stride ld_h >= F (two column halves
 * of one [rows, 2F] product of a fused [wi_0 | wi_1] weight: h1 = h0 + F,
 * ld_h = 2F); act [rows, F] contiguous in act_dtype.  F and ld_h multiples
 * of 8, rows * F / 8 < 2^31.
 */
int moe_swiglu(const void* h0, const void* h1, int h_dtype, int64_t rows, int64_t F,
               int64_t ld_h, void* act, int act_dtype, void* stream);

/* moe_swiglu_bwd: d_h0 = d_act*h1*s*(1 + h0*(1 - s)), d_h1 = d_act*silu(h0),
 * s = sigmoid(h0).  h0, h1 in h_dtype with row stride ld_h; d_act [rows, F]
 * contiguous in d_dtype; d_h0, d_h1 in d_dtype with row stride ld_dh (the
 * halves of a [rows, 2F] gradient with ld_dh = 2F in the fused layout).
 */
int moe_swiglu_bwd(const void* h0, const void* h1, int h_dtype, int64_t ld_h, const void* d_act,
                   int64_t rows, int64_t F, void* d_h0, void* d_h1, int64_t ld_dh, int d_dtype,
                   void* stream);

/* ------------------------------------------------------------------ combine
 * moe_combine: y[t] = sum_j topk_w[t, j] * y_sorted[row_of_slot[t*K+j]] over
 * kept slots, summed in float32 (the combine einsum "BKE,BK -> BE" of
 * [TE-MoE]).  y_sorted [rows, D], y [T, D] in `dtype`.
 */
int moe_combine(const void* y_sorted, int dtype, int64_t T, int64_t D, int K, int64_t rows,
                const int32_t* row_of_slot, const float* topk_w, void* y, void* stream);

/* moe_combine_bwd: the hand-derived combine backward of [TE-MoE]:
 *   d_y_sorted[r] = topk_w[s] * d_y[s / K] for r = row_of_slot[s];
 *   rows no slot maps to (slot_of_row[r] = -1) are written as zero;
 *   d_topk_w[s] = <d_y[s / K], y_sorted[row_of_slot[s]]> (float32 sum),
 *   0 for a dropped slot.
 *   d_y [T, D], y_sorted and d_y_sorted [rows, D] in `dtype`.
 */
int moe_combine_bwd(const void* d_y, const void* y_sorted, int dtype, int64_t T, int64_t D, int K,
                    int64_t rows, const int32_t* row_of_slot, const int32_t* slot_of_row,
                    const float* topk_w, void* d_y_sorted, float* d_topk_w, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H */
