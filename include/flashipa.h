/*
 * flashipa.h -- C ABI of the MI355X (gfx950) FlashIPA forward library.
 *
 * The library computes the aggregation core of monomer-style Invariant Point
 * Attention exactly as the "Invariant point attention (IPA)" problem page
 * (biotorch) states it in "Required behavior", with the pair representation
 * given as rank-R factors z_ij = sum_r zl_ir * zr_jr and a per-head pair bias
 * sum_c w_pair[h,c] z_ij[c] (FlashIPA rebuttal, paperhub page, answers to Q4
 * and Q5).  The whole logit -- scalar term, pair bias and the expanded squared
 * point distance (FlashIPA verdict page, key_machinery) -- is evaluated as one
 * inner product of lifted query and key rows inside a fused attention kernel,
 * so no [B,H,N,N] logit, bias, attention or pair tensor ever exists in memory.
 *
 * Three calls make one forward:
 *   ipa_lift      frames -> global points, point weight, lifted Q/K/V rows
 *   ipa_flash_fwd fused masked online-softmax attention over lifted rows
 *   ipa_epilogue  inverse frame transform, pair expansion, point lengths,
 *                 head-major feature concat and the output projection
 * Their buffers: the lifted workspace (ipa_lifted_bytes; written by
 * ipa_lift, read by ipa_flash_fwd), the attention output o and lse (written
 * by ipa_flash_fwd, read by ipa_epilogue) and the epilogue's workspace
 * (ipa_epilogue_workspace_bytes), all caller-owned.
 *
 * Conventions shared by every call
 *  - All device pointers refer to memory of the current HIP device; tensors
 *    are dense, row-major (C order) with the layouts stated below.
 *  - Floating inputs all have the dtype named in ipa_shape.dtype (IEEE fp32,
 *    or bfloat16 stored as 16-bit words).  Masks are bytes (0 = invalid,
 *    nonzero = valid).  Outputs are fp32.
 *  - Every device pointer must be 16-byte aligned.
 *  - Ownership: the caller allocates and frees every buffer.  The library
 *    never allocates, frees, retains a pointer after returning, or
 *    synchronises; all work is enqueued on `stream` (a hipStream_t, NULL for
 *    the default stream) and completes in stream order.
 *  - Errors: each call validates its arguments on the host and returns
 *    IPA_OK or an ipa_status code without enqueuing anything; kernel launch
 *    failures are reported as IPA_ERR_LAUNCH.  Finite inputs are a
 *    precondition and are not checked.
 *  - Tracing: every call that enqueues work is bracketed by a roctx range
 *    named after the call (rocprofv3 --marker-trace).
 *  - Debugging: with the environment variable FLASHIPA_DEBUG set to a
 *    non-zero value (read once per process), every call also waits for its
 *    kernels and returns IPA_ERR_LAUNCH, naming the call on stderr, when one
 *    of them failed.  Calls then synchronise their stream, so this mode is
 *    not for graph capture or timing.
 */
#ifndef FLASHIPA_H
#define FLASHIPA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  IPA_OK = 0,
  IPA_ERR_NULL = 1,        /* a required pointer is NULL */
  IPA_ERR_SHAPE = 2,       /* a dimension is <= 0, or eps <= 0 */
  IPA_ERR_UNSUPPORTED = 3, /* dims beyond the compiled kernel limits, or unknown dtype */
  IPA_ERR_ALIGN = 4,       /* a pointer is not 16-byte aligned */
  IPA_ERR_LAUNCH = 5,      /* a kernel launch failed (hipGetLastError) */
  IPA_ERR_DEVICE = 6,      /* HIP runtime / device query failed */
  IPA_ERR_SCRATCH = 7      /* ipa_forward_noalloc: the shape needs more than its static scratch */
} ipa_status;

typedef enum { IPA_F32 = 0, IPA_BF16 = 1 } ipa_dtype;

/* Problem sizes, all positive (IPA page, "Required behavior").
 *   B batch, N residues, H heads, D scalar q/k width, Dv scalar value width,
 *   P query/key points per head, Q value points per head, Cz pair channels,
 *   R factor rank, Cout output width.  F = H*(Dv+4Q+Cz).
 * dtype: IPA_F32 runs the fp32 path (fp32 storage and fp32 arithmetic
 * throughout); IPA_BF16 runs the matrix-core path (bf16/fp16 MFMA operands,
 * fp32 accumulation, see ipa_flash_fwd).
 * eps: added under the output point-length square root only. */
typedef struct {
  int64_t B, N, H, D, Dv, P, Q, Cz, R, Cout;
  int32_t dtype;
  float eps;
} ipa_shape;

/* Inputs of ipa_lift (IPA page, "Required behavior"; factors per the
 * FlashIPA rebuttal, Q4/Q5).  Layouts:
 *   q, k              [B,N,H,D]      projected scalar queries / keys
 *   v                 [B,N,H,Dv]     projected scalar values
 *   q_points,k_points [B,N,H,P,3]    LOCAL query / key points
 *   v_points          [B,N,H,Q,3]    LOCAL value points
 *   rotation          [B,N,3,3]      R_i, column-vector convention
 *                                     T_i(x) = R_i @ x + t_i
 *   translation       [B,N,3]        t_i
 *   point_weight_raw  [H]            softplus is applied inside
 *   w_pair            [H,Cz]         per-head pair-bias weights:
 *                                     pair_bias_ijh = sum_c w_pair[h,c] z_ij[c]
 *   zl, zr            [B,N,R,Cz]     pair factors, z_ij[c] = sum_r zl[i,r,c] zr[j,r,c]
 *   mask              [B,N] bytes    residue mask
 *   pair_mask         [B,N,N] bytes  or NULL (all valid); key j is permitted
 *                                     for query i iff mask_i && mask_j && pair_mask_ij */
typedef struct {
  const void* q;
  const void* k;
  const void* v;
  const void* q_points;
  const void* k_points;
  const void* v_points;
  const void* rotation;
  const void* translation;
  const void* point_weight_raw;
  const void* w_pair;
  const void* zl;
  const void* zr;
  const uint8_t* mask;
  const uint8_t* pair_mask;
} ipa_lift_in;

/* Inputs of ipa_epilogue besides the attention output.  Layouts:
 *   zl [B,N,R,Cz], rotation [B,N,3,3], translation [B,N,3],
 *   w_out [F,Cout] (update = features @ w_out + b_out), b_out [Cout]. */
typedef struct {
  const void* zl;
  const void* rotation;
  const void* translation;
  const void* w_out;
  const void* b_out;
} ipa_epi_in;

/* Size in bytes of the opaque "lifted" workspace that ipa_lift fills and
 * ipa_flash_fwd reads (lifted query rows, key/value tiles, per-tile
 * centroids, point weights, packed masks, and the partial results of the
 * fused kernel's key ranges when it splits them).  with_pair_mask != 0 reserves
 * room for a bit-packed pair mask (B*N*ceil(N/64)*8 bytes, the only part
 * that grows as N^2/8); pass 0 when ipa_lift will get pair_mask == NULL.
 * Returns 0 for an invalid or unsupported shape. */
size_t ipa_lifted_bytes(const ipa_shape* s, int with_pair_mask);

/* Width of one (residue, head) row of the attention output O:
 * Dv + R*Cz + 3*Q. */
int64_t ipa_o_width(const ipa_shape* s);

/* Kernel 1 (lift).  Applies the frames to every point (T_i(x) = R_i x + t_i),
 * forms the per-head point weight gamma_h = 1/2 softplus(w_h) sqrt(2/(27P)),
 * and writes the lifted rows whose inner products give
 *   L_ijh = q.k/sqrt(3D) + pair_bias_ijh/sqrt(3) - gamma_h sum_p |T_i q_p - T_j k_p|^2
 * (IPA page, "Required behavior"; lifting per the FlashIPA verdict page,
 * key_machinery).  Distances are expanded about a per-key-tile centroid so
 * that the expanded form keeps its accuracy for long chains.
 * `lifted` (lifted_bytes bytes, at least ipa_lifted_bytes(s, pair_mask != NULL))
 * is overwritten; IPA_ERR_SHAPE if it is too small. */
ipa_status ipa_lift(const ipa_shape* s, const ipa_lift_in* in, void* lifted, size_t lifted_bytes,
                    void* stream);

/* Kernel 2 (fused attention).  For every (b, h, i), masked stable softmax
 * over the permitted keys j of L_ijh (IPA page: key j permitted iff
 * mask_i && mask_j && pair_mask_ij; an empty neighbourhood gives an all-zero
 * attention row) followed by the aggregations, written per (b, i, h) as
 *   o[b,i,h, 0:Dv]              sum_j a_hij v_jh
 *   o[b,i,h, Dv:Dv+R*Cz]        sum_j a_hij zr_j          (layout [R,Cz])
 *   o[b,i,h, Dv+R*Cz: +3Q]      sum_j a_hij T_j(v_points_jhq)   (global, [Q,3])
 * o is [B,N,H,ipa_o_width(s)] fp32; rows with an empty neighbourhood are 0.
 * lse [B,H,N] fp32 receives log sum_j exp(L_ijh) over permitted keys
 * (natural log; -inf for an empty neighbourhood), so that the attention row
 * is a_hij = exp(L_ijh - lse_hi).
 * `lifted` must come from ipa_lift with the same shape, mask and pair_mask.
 * bf16 path: bf16 MFMA for the scalar and pair columns, fp16 hi/lo split
 * MFMA for the centred point columns, fp32 softmax and accumulation.  Its
 * shapes: D <= 16, Dv <= 31, P <= 5, Q <= 9, R*Cz <= 192 (else
 * IPA_ERR_UNSUPPORTED from ipa_lifted_bytes and the calls).  Its range: the
 * point term of a query against the centroid of a key tile, minus the row's
 * running maximum (the maximum over the permitted keys of the tiles seen so
 * far; zero before the first tile with a permitted key), is held in fp16
 * parts and must stay within 16 * 65504 in log2 units, i.e. gamma_h
 * sum_p |T_i q_p - c_t|^2 below about 7e5 at a row's first tile with a
 * permitted key; beyond that it is clamped (finite results, no NaN). */
ipa_status ipa_flash_fwd(const ipa_shape* s, const void* lifted, float* o, float* lse, void* stream);

/* Comparison only: the pages' own stacked point layout (FlashIPA rebuttal,
 * Q3: the point term as stacked vectors of five columns per point fed to
 * the same attention kernel).  Identical to ipa_lift / ipa_flash_fwd except
 * that the point term of L_ijh is evaluated as the inner product of
 *   query [T_i q_p (3) | |T_i q_p|^2 | 1]  and
 *   key   [2 gamma_h T_j k_p (3) | -gamma_h | -gamma_h |T_j k_p|^2]
 * per point, in bf16 and in global coordinates (two bf16 K-steps instead of
 * three fp16 hi/lo K-steps about centroids).  The squared norms of global
 * coordinates are then rounded to 8 significant bits, so on chains far from
 * the origin the logits, and with them o and lse, carry errors far beyond
 * the bf16 path's tolerance; these calls exist to measure that error and
 * the layout's speed beside the standard path, not to replace it.  The
 * lifted buffer (ipa_lifted_bytes_stacked bytes) is only valid for
 * ipa_flash_fwd_stacked; o and lse have the layouts of ipa_flash_fwd and
 * may be passed to ipa_epilogue.  Shapes: bf16 only, D <= 16, Dv <= 31,
 * P = 4, Q <= 9, 64 < R*Cz <= 128, D, Dv and Cz multiples of 8 (else
 * IPA_ERR_UNSUPPORTED, or 0 bytes). */
size_t ipa_lifted_bytes_stacked(const ipa_shape* s, int with_pair_mask);
ipa_status ipa_lift_stacked(const ipa_shape* s, const ipa_lift_in* in, void* lifted, size_t lifted_bytes,
                            void* stream);
ipa_status ipa_flash_fwd_stacked(const ipa_shape* s, const void* lifted, float* o, float* lse, void* stream);

/* Bytes of the epilogue's own workspace for this shape (the output
 * projection packed for the matrix-core product: per head or transposed,
 * bf16); at least 16.  0 for an invalid shape or one the epilogue does not
 * support. */
size_t ipa_epilogue_workspace_bytes(const ipa_shape* s);

/* Kernel 3 (epilogue).  Per residue i: local_points = R_i^T (g - t_i) for
 * every head and value point, lengths sqrt(|local|^2 + eps), pair features
 * o_pair = sum_r zl_ir * o_zr_r, head-major concat
 * [scalar (H,Dv) | x (H,Q) | y | z | length (H,Q) | pair (H,Cz)], and
 * update = features @ w_out + b_out; everything zero for an empty
 * neighbourhood (IPA page, "Required behavior").
 *   workspace    caller-owned, workspace_bytes >= ipa_epilogue_workspace_bytes(s);
 *                overwritten with w_out packed for the product (may be NULL
 *                on the fp32 path, which packs nothing).  The lifted rows of
 *                ipa_lift are not an argument: the epilogue reads only o, lse
 *                and the inputs below.
 *   o, lse       from ipa_flash_fwd
 *   update       [B,N,Cout] fp32 (written)
 *   local_points [B,N,H,Q,3] fp32 (written)
 * IPA_ERR_UNSUPPORTED if the feature row F does not fit the kernel's LDS
 * staging (bf16 path: F <= 2544; fp32 path: F <= 2559); IPA_ERR_SHAPE if
 * the workspace is too small. */
ipa_status ipa_epilogue(const ipa_shape* s, void* workspace, size_t workspace_bytes, const float* o, const float* lse,
                        const ipa_epi_in* in, float* update, float* local_points, void* stream);

/* The whole forward (ipa_lift, ipa_flash_fwd, ipa_epilogue) in one call
 * that allocates nothing, for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation.  Inputs and outputs as for the three calls (in, epi, update
 * [B,N,Cout] fp32, local_points [B,N,H,Q,3] fp32); every other buffer (the
 * lifted rows, o, lse, the packed output projection) lives in a static
 * device array of 128 MiB per GPU, held from the library's first use on that
 * GPU until the process ends.  The shape must fit in it:
 *   align256(ipa_lifted_bytes(s, pm)) + align256(4 B N H ipa_o_width(s))
 *     + align256(4 B H N) + ipa_epilogue_workspace_bytes(s) <= 128 MiB
 * (B=8, N=256: 18 MiB; B=1, N=2048: 61 MiB, at H=8 and the standard
 * widths), else
 * IPA_ERR_SCRATCH before anything is enqueued.  Results are those of the
 * three calls.  Every call on a GPU shares that GPU's array: calls that
 * overlap on one GPU (other streams, other host threads) race.  Other errors
 * as for the three calls; IPA_ERR_DEVICE if the array's device address
 * cannot be found. */
ipa_status ipa_forward_noalloc(const ipa_shape* s, const ipa_lift_in* in, const ipa_epi_in* epi, float* update,
                               float* local_points, void* stream);

/* Diagnostic (tests only): the logits the fused kernel uses, for query rows
 * row0 .. row0+nrows-1 of (b, h), recomputed from the lifted rows with the
 * fused kernel's operand rounding, in natural-log units; -inf where the key is
 * not permitted.  out is [nrows, N] fp32. */
ipa_status ipa_logit_rows(const ipa_shape* s, const void* lifted, int64_t b, int64_t h, int64_t row0,
                          int64_t nrows, float* out, void* stream);

/* ------------------------------------------------------------------------
 * Backward pass (fp32)
 *
 * Gradients of  <update, d_update> + <local_points, d_local_points>  with
 * respect to every input of the forward defined above (IPA page, "Required
 * behavior"; its starter code states that the suite grades gradients).
 * Readings: rotation is differentiated as a free 3x3 matrix (the formula
 * uses R and R^T linearly); masks are not differentiable; an empty
 * neighbourhood passes no gradient.  The computation is fp32 throughout
 * (vector ALU): it recomputes the attention core (output and log-sum-exp)
 * from the inputs, runs the epilogue's backward, two passes over the key
 * and query pairs with recomputed probabilities (FlashAttention style, no
 * [B,H,N,N] array), and maps the row gradients back to the inputs.
 *
 * s->dtype names the inputs' type as for the forward (IPA_F32 or IPA_BF16;
 * bf16 inputs are widened to fp32 copies in the workspace first, so the
 * gradients are those at the bf16 values, computed in fp32).  Limits: P <= 5, D + R*Cz <= 256,
 * Dv + R*Cz + 3Q <= 256.  in / epi are the forward's input structs (the
 * pair mask may be NULL); d_update [B,N,Cout] and d_local [B,N,H,Q,3] are
 * fp32.  Every gradient pointer of ipa_grads is required; each array has its
 * input's shape and is fully written.  The workspace (ipa_backward_workspace_bytes,
 * O(B H N (D + R Cz + Dv + 3Q) + B N H (Dv + 4Q + Cz)) bytes) is caller-owned
 * and overwritten.  Errors as for ipa_lift (IPA_ERR_SHAPE also for a
 * workspace that is too small); nothing is enqueued on error. */
typedef struct {
  float* q;
  float* k;
  float* v;
  float* q_points;
  float* k_points;
  float* v_points;
  float* rotation;
  float* translation;
  float* point_weight_raw;
  float* w_pair;
  float* zl;
  float* zr;
  float* w_out;
  float* b_out;
} ipa_grads;

/* Bytes of the workspace ipa_backward needs for this shape, 0 when the
 * shape is invalid or beyond the limits above. */
size_t ipa_backward_workspace_bytes(const ipa_shape* s);

ipa_status ipa_backward(const ipa_shape* s, const ipa_lift_in* in, const ipa_epi_in* epi, const float* d_update,
                        const float* d_local, void* workspace, size_t workspace_bytes, ipa_grads* grads,
                        void* stream);

/* ------------------------------------------------------------------------
 * k-nearest-neighbour distogram (pair-feature preprocessing)
 *
 * FlashIPA rebuttal, paperhub page, answer to Q6: per residue only the
 * distances to its k nearest neighbours are kept, as a (B, L, k, n_bins)
 * distogram rather than (B, L, L, n_bins), the neighbours being found from
 * the full L x L distance matrix; the answer also allows computing them
 * block-wise in a streaming fashion, which is what this call does: no L x L
 * array exists, memory is O(L k).
 *
 * Definition (the page leaves the arithmetic open; this is the reading):
 *  - the position of residue i is its frame translation t_i (fp32);
 *  - d2(i,j) = ((dx*dx + dy*dy) + dz*dz) in fp32 with dx = t_j.x - t_i.x
 *    etc., every operation rounded to nearest, no fused multiply-add;
 *    the distance is the correctly rounded fp32 square root of d2;
 *  - the candidates of a valid residue i are the valid residues j != i of
 *    the same sample, ordered by d2, equal d2 by the lower j first; the
 *    first k are kept (slot 0 = nearest);
 *  - bins: w = fl32(dmax / nbins); bin = floor(fl32(d / w)), and any d
 *    with fl32(d / w) >= nbins is in bin nbins-1.
 * Slots beyond the number of candidates, and every slot of an invalid
 * residue, hold index -1, distance +inf and an all-zero one-hot row.
 * The result is exact: the same bits as the definition above, whatever the
 * data (ties, duplicate positions, masks).  Finite coordinates are a
 * precondition. */
typedef struct {
  int64_t B, N;        /* samples, residues per sample (both > 0) */
  int64_t k;           /* neighbours kept per residue, 1 .. 64 */
  int64_t nbins;       /* distance bins, 1 .. 4096 */
  float dmax;          /* > 0 and finite: the bins split [0, dmax) evenly */
  int32_t dgram_dtype; /* IPA_F32 or IPA_BF16: element type of dgram */
} ipa_knn_shape;

/* translation [B,N,3] fp32 (the same array ipa_lift takes), mask [B,N]
 * bytes or NULL (all valid).  Outputs, all written in full:
 *   nn_index [B,N,k] int32   neighbour indices within the sample (required)
 *   nn_dist  [B,N,k] fp32    their distances (NULL to skip)
 *   dgram    [B,N,k,nbins]   one-hot bins, 1.0 / 0.0 in dgram_dtype (NULL
 *                            to skip)
 * Returns IPA_ERR_NULL (translation or nn_index NULL), IPA_ERR_SHAPE
 * (B, N <= 0, k or nbins out of range, dmax not positive and finite),
 * IPA_ERR_UNSUPPORTED (unknown dgram_dtype), IPA_ERR_ALIGN (a pointer not
 * 16-byte aligned) before enqueuing anything, or IPA_ERR_LAUNCH. */
ipa_status ipa_knn_distogram(const ipa_knn_shape* s, const float* translation, const uint8_t* mask,
                             int32_t* nn_index, float* nn_dist, void* dgram, void* stream);

/* ------------------------------------------------------------------
 * Attention with a low-rank bias (FlashBias: Fast Computation of Attention
 * with Bias, atlas.scime.ai summary, Problem and Approach).  A dense bias
 * b_ij = phi_q(i) . phi_k(j) is given by its two factor tensors, which are
 * concatenated onto the queries and keys, so the [N, M] bias is never formed:
 *
 *   L_ij  = scale q_i . k_j + phi_q(i) . phi_k(j)      (natural-log units)
 *   O_i   = sum_j softmax_j(L_ij) v_j,  lse_i = log sum_j exp(L_ij)
 *
 * over the permitted keys j of the same sample: key_mask[b, j] != 0 (all
 * when key_mask is NULL) and, when causal, j <= i.  A row with no permitted
 * key gets O_i = 0 and lse_i = -inf.
 *
 * Arithmetic: bf16 matrix-core operands with fp32 accumulation.  The q.k
 * part uses bf16 q scale log2(e) and bf16 k; every factor product is taken
 * as hi.hi + hi.lo + lo.hi of bf16 hi/lo pairs (~16 significant bits per
 * factor, so large exact factors such as ALiBi positions stay exact to
 * ~1e-5 relative); probabilities are rounded to bf16 against bf16 values;
 * softmax statistics in fp32.  fp32 q, k, v are rounded to bf16 in the same
 * way; fp32 factors keep the ~16 bits of their hi/lo pairs. 
 * ------------------------------------------------------------------ */
typedef struct {
  int64_t B, N, M, H; /* samples (<= 65535), queries, keys, heads (<= 65535); all >= 1 */
  int64_t D;          /* q / k width (>= 1) */
  int64_t Dv;         /* value width, 1 .. 256 */
  int64_t R;          /* bias rank (>= 0); D + 3 R <= 256 */
  int32_t dtype;      /* IPA_F32 or IPA_BF16: q, k, v */
  int32_t phi_dtype;  /* IPA_F32 or IPA_BF16: phi_q, phi_k (fp32 keeps exact factors exact) */
  int32_t causal;     /* nonzero: key j permitted for query i only if j <= i (needs N == M) */
  float scale;        /* multiplies q . k (finite), e.g. 1/sqrt(D) */
} ipa_bias_shape;

/* Workspace bytes ipa_bias_attention needs for this shape (lifted rows,
 * transposed value tiles and mask words, O(B H (N + M)(D + 3R + Dv))); 0 if
 * the shape is invalid or beyond the compiled limits. */
size_t ipa_bias_workspace_bytes(const ipa_bias_shape* s);

/* Inputs (device pointers, row-major, all 16-byte aligned):
 *   q [B,N,H,D], k [B,M,H,D], v [B,M,H,Dv]          in s->dtype
 *   phi_q [B,N,H,R], phi_k [B,M,H,R]                in s->phi_dtype (may be NULL if R == 0)
 *   key_mask [B,M] bytes, or NULL (every key permitted)
 * Outputs (written in full): o [B,N,H,Dv] fp32, lse [B,H,N] fp32.
 * workspace: device memory of at least ipa_bias_workspace_bytes(s) bytes,
 * owned by the caller, overwritten.  Enqueued on `stream` (hipStream_t, NULL
 * for the default stream); no allocation, no synchronisation.
 * Returns IPA_ERR_NULL (a required pointer NULL), IPA_ERR_SHAPE (a dimension
 * out of range, scale not finite, causal with N != M, B H max(N, M) beyond
 * ~6.7e7, workspace too small),
 * IPA_ERR_UNSUPPORTED (unknown dtype or phi_dtype, D + 3R > 256 or Dv > 256), IPA_ERR_ALIGN
 * before enqueuing anything, or IPA_ERR_LAUNCH. */
ipa_status ipa_bias_attention(const ipa_bias_shape* s, const void* q, const void* k, const void* v,
                              const void* phi_q, const void* phi_k, const uint8_t* key_mask, float* o, float* lse,
                              void* workspace, size_t workspace_bytes, void* stream);

/* Human-readable name of a status code (static string). */
const char* ipa_status_string(int status);

/* Library version string (static). */
const char* ipa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FLASHIPA_H */
