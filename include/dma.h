/*
 * dma.h - C ABI of the MI355X (gfx950) Dynamic Mask Attention forward.
 *
 * The method is the one of the Hugging Face blog "Trainable Dynamic Mask
 * Sparse Attention" (cited here as "the DMA blog"):
 *   1. dynamic weights  delta = exp(tau(v Delta) x A), tau = softplus
 *      (section "Dynamic Sparse Mask Generation", delta equation);
 *   2. keep mask        m_t = f(top_w(delta + m_c^t)): query position p keeps
 *      the w causally valid keys j <= p with the largest delta, equal delta
 *      going to the lower key index, and f puts -inf on every other key
 *      (section "Mask Combination with Causal Constraints");
 *   3. attention        o_t = softmax(q_t k^T / sqrt(d_h) o m_t) v, read as
 *      adding delta to the scaled scores of kept keys; masked keys get weight
 *      exactly 0, so their work is skipped (section "Efficient Sparse
 *      Attention Computation" and its "Forward Pass Safety" item).
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are device memory owned by the caller.  The library
 *     allocates nothing and keeps no state besides its loaded code objects.
 *   - `stream` is a hipStream_t (NULL = the null stream).  Calls only enqueue
 *     work on it; outputs are ready once the stream reaches them.
 *   - Every argument is validated on the host before anything is enqueued.
 *     On any error nothing is launched or written and a status is returned.
 *     A launch failure reported by the runtime maps to DMA_ERR_HIP.
 *   - Sizes and strides are in elements.  Empty work (B == 0, or no query
 *     rows, or no keys for dma_weights) returns DMA_OK without launching.
 *   - Shapes use B batch, Hq query heads, Hkv key/value heads (Hq % Hkv == 0,
 *     query head hq reads kv head hq / (Hq/Hkv)), Sq query rows, Sk key rows,
 *     D head size (64 or 128), w keys kept per query row (w >= 1); query row
 *     i sits at absolute position p = q_offset + i, with q_offset + Sq <= Sk.
 *   - Calls are reentrant; calls on one stream run in order.
 */
#ifndef DMA_H
#define DMA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DMA_OK = 0,
  DMA_ERR_INVALID_ARG = 1, /* null pointer, bad size, bad stride or alignment */
  DMA_ERR_UNSUPPORTED = 2, /* a legal shape this build does not handle */
  DMA_ERR_WORKSPACE = 3,   /* workspace or list capacity too small */
  DMA_ERR_HIP = 4          /* the HIP runtime reported an error */
} dma_status;

typedef enum { DMA_F32 = 0, DMA_BF16 = 1 } dma_dtype;

/* Build limits. */
#define DMA_MAX_SK (1 << 20) /* keys per sequence */
#define DMA_BLOCK_Q 64       /* query rows per tile (Bq) */
#define DMA_BLOCK_K 64       /* keys per key tile (Bk) */

/* Human-readable name of a status code (static storage). */
const char* dma_status_string(dma_status s);

/* ABI version; bumped whenever a signature or a layout below changes. */
int dma_abi_version(void);

/* Tile sizes fixed by this build: Bq query rows per tile, Bk keys per key tile. */
void dma_tile_sizes(int32_t* Bq, int32_t* Bk);

/*
 * Mask produced by dma_topk_mask and consumed by dma_attn_fwd.  Sizes come
 * from dma_mask_dims.  Query rows are cut into n_tiles = ceil(Sq / Bq) tiles
 * per (b, kv head); tile index g = (b*Hkv + h)*n_tiles + t covers query rows
 * [t*Bq, min(Sq, (t+1)*Bq)).
 *
 *   evict  int32 [B*Hkv*Sk]  eviction row of each key (written when Sq > 1):
 *          key j is kept by exactly the query positions p with j <= p < evict[j]
 *          (positions over the whole sequence 0..Sk-1; evict[j] == j for a key
 *          no position keeps, evict[j] == Sk for a key kept to the end).  This interval form is exact because delta has
 *          no query index, so a key once dropped never returns.
 *   u_idx  int32 [n_tiles_total * u_stride]  the union U_g of the keep sets of
 *          the tile's rows, as two ascending runs: first the u_nfull[g] keys
 *          every row of the tile keeps, then the keys only some rows keep.
 *   u_cnt, u_nfull  int32 [n_tiles_total]   |U_g| and the length of the first run.
 *   u_dmax float [n_tiles_total]   largest delta over U_g.
 *   kt_idx int32 [n_tiles_total * kt_stride]  ascending key-tile indices kt with
 *          [kt*Bk, (kt+1)*Bk) holding at least one key of U_g (the block-skip
 *          list: every other key tile is skipped).  May be NULL (not written).
 *   kt_cnt int32 [n_tiles_total]   length of that list (NULL iff kt_idx is NULL).
 *   u_dlo  float [n_tiles_total]   largest delta over the keys before the tile's
 *          first row (j < q_offset + t*Bq; -inf when there are none).  Row p's
 *          largest kept delta is the prefix maximum of delta over keys 0..p
 *          (a row always keeps its best key); the attention derives it from
 *          u_dlo and the tile's own keys.  May be NULL for dma_topk_mask
 *          (then not written); the bf16 prefill attention requires it.
 *   u_dval float [n_tiles_total * u_stride]   with Sq == 1 only: delta of each
 *          key of u_idx, at the same positions.  May be NULL (not written).
 *          When set, the one-row mask calls write it and the one-row attention
 *          reads it instead of gathering delta at the listed keys (one
 *          contiguous read of w values instead of one scattered read per key,
 *          which touches nearly every line of the delta row).
 * With Sq == 1 (one decode row) evict and u_dlo are not read or written and
 * may be NULL.  With Sq > 1 u_dval is not read or written.
 */
typedef struct {
  int32_t* evict;
  int32_t* u_idx;
  int32_t* u_cnt;
  int32_t* u_nfull;
  float* u_dmax;
  int32_t* kt_idx;
  int32_t* kt_cnt;
  float* u_dlo;
  float* u_dval;
} dma_mask;

typedef struct {
  int64_t n_tiles;       /* tiles per (b, kv head): ceil(Sq / Bq) */
  int64_t n_tiles_total; /* B * Hkv * n_tiles */
  int64_t u_stride;      /* min(Sk, w + Bq - 1): largest possible |U_g| */
  int64_t kt_stride;     /* ceil(Sk / Bk) */
  int64_t evict_elems;   /* B*Hkv*Sk, or 0 when Sq == 1 */
  int64_t u_elems;       /* n_tiles_total * u_stride */
  int64_t kt_elems;      /* n_tiles_total * kt_stride */
} dma_mask_dims;

/* Sizes of the mask arrays for a call of dma_topk_mask with these arguments. */
dma_status dma_mask_dims_for(int64_t B, int64_t Hkv, int64_t Sq, int64_t Sk, int64_t q_offset,
                             int64_t w, dma_mask_dims* out);

/* Workspace bytes dma_topk_mask needs for these arguments (0 when Sq <= 1). */
size_t dma_topk_workspace_bytes(int64_t B, int64_t Hkv, int64_t Sq, int64_t Sk, int64_t w);

/* Workspace bytes dma_attn_fwd needs (split partials of the one-row path; 0
 * when Sq > 1). */
size_t dma_attn_workspace_bytes(int64_t B, int64_t Hq, int64_t Sq, int64_t D, int64_t w);

/*
 * Step 1: dynamic weights (DMA blog, delta equation).
 *   pre[b,j,h]   = sum_{c < Hkv*D} V[b,j,c] * Delta[c,h]   (c = kv_head*D + channel)
 *   delta[b,h,j] = exp(softplus(pre[b,j,h]) * A[h])
 * V       [B, Sk, Hkv, D] of type vt (F32 or BF16); element (b,j,c) at
 *         b*v_stride_b + j*v_stride_s + c, i.e. each key's Hkv*D values are
 *         contiguous.  16-byte aligned base and strides.
 * Delta   float [Hkv*D, Hkv] row-major.   A float [Hkv].
 * delta   float [B, Hkv, Sk] contiguous (output).
 * Arithmetic: fp32 accumulation, fp32 softplus/exp.  Limits: Hkv*D <= 2048.
 */
dma_status dma_weights(const void* V, dma_dtype vt, int64_t B, int64_t Sk, int64_t Hkv, int64_t D,
                       int64_t v_stride_b, int64_t v_stride_s, const float* Delta, const float* A,
                       float* delta, void* stream);

/*
 * Step 2: causal top-w keep mask and block-skip lists (DMA blog, m_t
 * equation), for query positions q_offset .. q_offset+Sq-1 over keys 0..Sk-1.
 * delta  float [B, Hkv, Sk] (from dma_weights or any other source; NaN is
 *        not allowed).  Ordering is exact: larger delta wins, equal delta
 *        (IEEE equality, so -0 equals +0) goes to the lower key index.
 * out    arrays sized by dma_mask_dims_for (kt_idx/kt_cnt may be NULL).
 * ws     dma_topk_workspace_bytes(...) bytes of device scratch (16-byte aligned),
 *        may be NULL when that is 0.  Its contents are undefined afterwards.
 * Results are integer and deterministic: bit-identical on every run.
 */
dma_status dma_topk_mask(const float* delta, int64_t B, int64_t Hkv, int64_t Sq, int64_t Sk,
                         int64_t q_offset, int64_t w, const dma_mask* out, void* ws,
                         size_t ws_bytes, void* stream);

/*
 * dma_topk_mask for callers that cannot allocate device memory (code under
 * graph capture, serving loops that forbid allocation): the same call and
 * results, without the ws arguments.  The workspace is a static device
 * array of DMA_TOPK_SCRATCH_BYTES that the library holds on each GPU it runs
 * on until the process ends; this call allocates nothing.  Calls whose
 * dma_topk_workspace_bytes(...) exceeds it return DMA_ERR_WORKSPACE (the
 * 16K-token prefill needs ~8 MiB, the 64K one ~50 MiB).  Every call on a GPU
 * shares that GPU's array, so calls that overlap in time on one GPU (other
 * streams, other threads) race; calls on one stream run in order.
 */
#define DMA_TOPK_SCRATCH_BYTES ((size_t)64 << 20)
dma_status dma_topk_mask_noalloc(const float* delta, int64_t B, int64_t Hkv, int64_t Sq,
                                 int64_t Sk, int64_t q_offset, int64_t w, const dma_mask* out,
                                 void* stream);

/*
 * Step 2, one decode step (DMA blog, m_t equation; the keep set of position
 * p is the top w of keys 0..p).  Keep sets nest, so keep(p) is the top w of
 * keep(p-1) plus key p: key p enters exactly when it beats the worst kept key
 * (smaller delta, or equal delta and higher index), which it replaces.
 * delta  float [B, Hkv, Sk]; key p = Sk-1 is the new key.
 * mask   on entry the one-row lists of position Sk-2 over keys 0..Sk-2, as
 *        written by dma_topk_mask(delta, B, Hkv, 1, Sk-1, Sk-2, w) or by a
 *        previous call of this function; on return those of position Sk-1,
 *        identical to what dma_topk_mask(delta, B, Hkv, 1, Sk, Sk-1, w) writes.
 *        u_idx [B*Hkv, w], u_cnt, u_nfull, u_dmax [B*Hkv]; kt_idx and kt_cnt
 *        must be NULL (key-tile lists are not maintained).
 * Requires Sk-1 >= w (the list is full, stride w) and w <= 32768; sequences
 * whose list does not hold w keys are left unchanged.  Updated in place on
 * the stream; O(w) work per sequence instead of a selection over all Sk keys.
 */
dma_status dma_decode_keep_append(const float* delta, int64_t B, int64_t Hkv, int64_t Sk,
                                  int64_t w, const dma_mask* mask, void* stream);

/*
 * Step 3: masked attention (DMA blog, o_t equation with additive mask).
 *   For query row i of head hq (position p = q_offset + i, kv head h):
 *   s_j = scale * (q . k_j) + delta[b,h,j] over the keys j row p keeps,
 *   O[b,i,hq,:] = sum_j softmax(s)_j v_j,   lse[b,hq,i] = log sum_j exp(s_j).
 * Q [B,Sq,Hq,D], K and V [B,Sk,Hkv,D] of type t; q_strides / kv_strides give
 * the element strides of the b, s and head dimensions (the D values of a
 * head are contiguous; K and V share strides); 16-byte aligned.
 * delta, mask: from steps 1 and 2 for the same (B, Hkv, Sq, Sk, q_offset, w).
 * scale  <= 0 selects 1/sqrt(D).
 * O      [B,Sq,Hq,D] contiguous, type t (output).   lse float [B,Hq,Sq] or NULL.
 *        bf16 prefill: with lse requested the logits are rounded exactly as
 *        dma_attn_bwd recomputes them (O, lse and the gradients then agree to
 *        the last bit in nearly one-hot rows, and O equals dma_attn_fwd_train's);
 *        with lse NULL the score scale is applied inside the exponent, which
 *        is faster.  The two O can differ in the last bit of bf16; both are
 *        within the stated tolerance of the exact result.
 * ws     dma_attn_workspace_bytes(...) bytes (NULL allowed when 0).
 * Arithmetic: BF16 inputs use bf16 MFMA products with fp32 accumulation and
 * an fp32 online softmax; F32 inputs are computed in fp32 throughout.
 * BF16 with Sq > 1 reads mask->u_dlo (required).
 * Limits: BF16 with Sq > 1 needs D == 128, the rows of one (batch, kv
 * head) within 4 GiB: (Sk-1)*kv_strides[1]*2 + 256 <= 2^32, a key row
 * stride under 16 MiB (kv_strides[1]*2 < 2^24) and Sk <= 2^24; otherwise
 * DMA_ERR_UNSUPPORTED.  With Sq == 1 any strides are accepted: key rows
 * further apart than that are gathered with 64-bit offsets by the (slower)
 * vector kernel instead of the matrix-core one.
 */
dma_status dma_attn_fwd(const void* Q, const void* K, const void* V, dma_dtype t, int64_t B,
                        int64_t Sq, int64_t Sk, int64_t Hq, int64_t Hkv, int64_t D,
                        const int64_t q_strides[3], const int64_t kv_strides[3], int64_t q_offset,
                        int64_t w, const float* delta, const dma_mask* mask, float scale, void* O,
                        float* lse, void* ws, size_t ws_bytes, void* stream);

/*
 * Step 3 for training: dma_attn_fwd (bf16, D == 128, Sq > 1, no workspace)
 * that also writes O_res [B,Sq,Hq,D] bf16, the rounding residual of O (the
 * fp32 result minus the stored bf16 O).  O + O_res carries O to ~2^-18, which
 * dma_attn_bwd needs for dO . O where the attention is nearly one-hot (there
 * the exact gradient is a small difference that bf16 O alone would swamp).
 * lse is required.
 */
dma_status dma_attn_fwd_train(const void* Q, const void* K, const void* V, dma_dtype t,
                              int64_t B, int64_t Sq, int64_t Sk, int64_t Hq, int64_t Hkv,
                              int64_t D, const int64_t q_strides[3],
                              const int64_t kv_strides[3], int64_t q_offset, int64_t w,
                              const float* delta, const dma_mask* mask, float scale, void* O,
                              float* lse, void* O_res, void* stream);

/* Workspace bytes dma_weights_bwd needs: the pre-activation gradient [B,Sk,Hkv]. */
size_t dma_weights_bwd_workspace_bytes(int64_t B, int64_t Sk, int64_t Hkv);

/*
 * Backward of step 1 (DMA blog, delta equation), given ddelta = dL/ddelta:
 *   dpre[b,j,h]  = ddelta * delta * A[h] * sigmoid(pre)   (softplus' = sigmoid)
 *   dA[h]        = sum_{b,j} ddelta * delta * softplus(pre)
 *   dDelta[c,h]  = sum_{b,j} V[b,j,c] * dpre[b,j,h]
 *   dV[b,j,c]   += sum_h dpre[b,j,h] * Delta[c,h]
 * pre is recomputed from V and Delta as in dma_weights (exact bf16 products).
 * V, Delta, A, strides as dma_weights (BF16 only); ddelta float [B,Hkv,Sk];
 * dV float [B,Sk,Hkv*D] contiguous, accumulated into (pass the attention's
 * dV); dDelta float [Hkv*D,Hkv] and dA float [Hkv] overwritten.
 * ws: dma_weights_bwd_workspace_bytes bytes (16-byte aligned).
 * dDelta and dA are sums of per-workgroup partials added atomically, so their
 * last bits may differ from run to run.
 */
dma_status dma_weights_bwd(const void* V, dma_dtype vt, int64_t B, int64_t Sk, int64_t Hkv,
                           int64_t D, int64_t v_stride_b, int64_t v_stride_s, const float* Delta,
                           const float* A, const float* ddelta, float* dV, float* dDelta,
                           float* dA, void* ws, size_t ws_bytes, void* stream);

/* Workspace bytes dma_attn_bwd needs (0 when Sq <= 1). */
size_t dma_attn_bwd_workspace_bytes(int64_t B, int64_t Hq, int64_t Hkv, int64_t Sq, int64_t Sk,
                                    int64_t w);

/*
 * Backward of step 3 (DMA blog, o_t equation; masked keys get exactly zero
 * gradient, section "Efficient Sparse Attention Computation", "Backward Pass
 * Safety").  Gradients of L = sum(dO * O) with the keep sets held fixed:
 *   P_ij = exp(s_ij - lse_i),  dS_ij = P_ij (dO_i . v_j - dO_i . O_i)
 *   dQ_i = scale sum_j dS_ij k_j       dK_j = scale sum_i dS_ij q_i
 *   dV_j = sum_i P_ij dO_i             ddelta[b,h,j] = sum_i dS_ij
 * (i over the query rows and the Hq/Hkv query heads of kv head h).
 * Arguments as dma_attn_fwd, plus: O and lse the outputs of the forward
 * (lse required); O_res the residual from dma_attn_fwd_train, or NULL (then
 * dO . O uses the bf16 O alone); dO [B,Sq,Hq,D] contiguous, type t.  Outputs, float,
 * contiguous, overwritten: dQ [B,Sq,Hq,D], dK and dV [B,Sk,Hkv,D], ddelta
 * [B,Hkv,Sk] (add the weights backward's dV separately).  ws:
 * dma_attn_bwd_workspace_bytes bytes, 256-byte aligned.
 * Arithmetic: bf16 MFMA products with fp32 accumulation; the per-row
 * partial sums of dK/dV/ddelta are added in fp32.  Limits: BF16, D == 128,
 * Sq > 1; query, dO and key rows within 4 GiB of their (b, h) base.
 */
dma_status dma_attn_bwd(const void* Q, const void* K, const void* V, dma_dtype t, int64_t B,
                        int64_t Sq, int64_t Sk, int64_t Hq, int64_t Hkv, int64_t D,
                        const int64_t q_strides[3], const int64_t kv_strides[3], int64_t q_offset,
                        int64_t w, const float* delta, const dma_mask* mask, float scale,
                        const void* O, const void* O_res, const float* lse, const void* dO,
                        float* dQ, float* dK, float* dV, float* ddelta, void* ws,
                        size_t ws_bytes, void* stream);

/*
 * Steps 0 and 1 fused (DMA blog, section "Dynamic Sparse Mask Generation":
 * delta is computed from the value matrix): the value projection with the
 * dynamic weights formed in its epilogue.
 *   V[b,j,n]     = sum_{k < Cin} X[b,j,k] * Wv[k,n],  n < Hkv*D   (fp32 sums,
 *                  stored as bf16)
 *   delta[b,h,j] = exp(softplus(sum_n V[b,j,n] * Delta[n,h]) * A[h]) over the
 *                  stored bf16 V, i.e. dma_weights on the V written here (the
 *                  products are exact as there; the fp32 sums run in another
 *                  order).
 * X      bf16 [B, Sk, Cin], element (b,j,k) at b*x_stride_b + j*x_stride_s + k.
 * Wv     bf16 [Cin, Hkv*D] row-major (the projection's weight, input-major).
 * V      bf16 [B, Sk, Hkv, D] (output), element (b,j,n) at b*v_stride_b +
 *        j*v_stride_s + n.
 * Delta, A, delta as in dma_weights.  delta NULL: the projection alone
 *        (Delta and A are not read, no workspace is needed).
 * ws     dma_vproj_workspace_bytes(B, Sk, Hkv, D) bytes (16-byte aligned),
 *        contents undefined afterwards.
 * Limits: Cin a positive multiple of 64; Hkv*D a multiple of 256 and at most
 * 2048; Hkv <= 8 when delta is computed; B*Sk < 2^31; bases and strides
 * 16-byte aligned.  Otherwise DMA_ERR_UNSUPPORTED / DMA_ERR_INVALID_ARG.
 */
size_t dma_vproj_workspace_bytes(int64_t B, int64_t Sk, int64_t Hkv, int64_t D);
dma_status dma_vproj_weights(const void* X, int64_t B, int64_t Sk, int64_t Cin,
                             int64_t x_stride_b, int64_t x_stride_s, const void* Wv, int64_t Hkv,
                             int64_t D, void* V, int64_t v_stride_b, int64_t v_stride_s,
                             const float* Delta, const float* A, float* delta, void* ws,
                             size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DMA_H */
