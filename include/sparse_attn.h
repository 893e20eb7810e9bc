/*
 * sparse_attn.h -- C ABI of the MI355X (gfx950) hybrid block-sparse attention
 * library for video diffusion transformers.
 *
 * The path (all steps are GPU kernels of this library):
 *   reorder      row-major video tokens -> cube-major blocks of 64 tokens
 *   pool         per-block mean of Q and K over the block's real tokens
 *   block_scores S = Qbar Kbar^T * scale (float32 scores from three-term
 *                bf16 splits on the path; a float64 form beside it)
 *   select       per query block: hybrid Top-k U Top-p kept-block list
 *   fwd          block-sparse attention over the kept blocks -> O, LSE
 *                (fwd_tokens: the same, writing token order -- unreorder fused)
 *   coarse       block-level attention on pooled Q, K, V (coarse branch)
 *   router       fine-grained router scores (sub-cube pooling, G x G pooling)
 *   bwd          gradients of the block-sparse attention (dQ, dK, dV)
 *   quality      retained pooled mass, retained attention mass, L1 error,
 *                ideal block scores and the recall of kept lists
 *   attention    the whole path in one call, overlapped over two streams
 *   groups       asymmetric blocks: masks and forward for query blocks of
 *                2 or 4 cubes against single-cube key blocks
 *   sequence     per-sequence Top-K: one block budget per head
 *   unreorder    cube-major O (and LSE) -> row-major tokens
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every tensor pointer is a DEVICE pointer that the caller allocated; the
 *   library never allocates, frees or keeps caller-visible memory.  Scratch
 *   memory comes in through a caller-provided `workspace` (device pointer,
 *   256-byte aligned) whose size the *_workspace_bytes() functions report.
 * - `stream` is a hipStream_t (NULL = the default stream).  All work is
 *   enqueued asynchronously on it; nothing synchronises the host.
 * - Tensors are dense and row-major with the shapes given at each function;
 *   bf16 tensors must be 16-byte aligned, float64 8-byte, int32/float 4-byte.
 * - A token grid of frames x height x width is flattened row-major,
 *   n = t*height*width + h*width + w ("N" = real tokens).  Cube-major tensors
 *   hold nblk blocks of 64 slots ("n_pad" = 64*nblk); block
 *   (bt, bh, bw) is number (bt*Nh + bh)*Nw + bw and its slot for the token at
 *   offset (tt, hh, ww) inside the cube is (tt*cube_h + hh)*cube_w + ww.
 *   A grid side that is not a multiple of the cube side is padded up; pad
 *   slots are never treated as tokens (pooling skips them, attention masks
 *   them as keys and writes O = 0, LSE = -inf for them as queries).  Pad slots
 *   must hold finite values (reorder writes zeros there).
 * - Every cube-major tensor is [batch, heads, nblk, 64*head_dim] bf16: block
 *   b of a head occupies 64*d contiguous elements.  Inside a block the
 *   element order depends on the tensor (d = head_dim, s = slot, c = dim):
 *     SA_LAYOUT_QK (queries, keys): element (s, c) is at
 *        ((s/32)*(d/16) + c/16)*512 + ((c/8)%2)*256 + (s%32)*8 + c%8
 *     SA_LAYOUT_V (values): element (s, c) is at
 *        ((c/32)*4 + s/16)*512 + ((s/8)%2)*256 + (c%32)*8 + s%8
 *     slot-major (attention output O): element (s, c) is at s*d + c
 *   The first two are the operand order of the 32x32x16 bf16 matrix-core
 *   instruction, so the attention kernel loads every operand as whole,
 *   contiguous kilobytes.  sparse_attn_reorder writes them; nothing else in
 *   the caller needs to know them.
 * - Return value: SA_OK (0) or a negative SA_ERR_* code.  On an argument error
 *   nothing is launched and no output is touched; sparse_attn_last_error()
 *   gives a message (per calling thread).  A failed launch returns
 *   SA_ERR_HIP.  Faults inside kernels surface at the caller's next
 *   synchronisation, as for any HIP work.
 * - Functions keep no caller-visible state between calls and are safe to
 *   call from several host threads.  (sparse_attn_attention on two streams
 *   reuses HIP events it creates, one pool per host thread and device.)
 *
 * Citations name the pages this library follows by title and section:
 *   [SA2]  "SpargeAttention2: Trainable Sparse Attention via Hybrid Top-k+Top-p
 *          Masking and Distillation" (summary page)
 *   [VSA]  "VSA: Faster Video Diffusion with Trainable Sparse Attention"
 *          (summary page)
 *   [VSA2] "Improving Video Sparse Attention with Fine-grained Router and
 *          Sparse Rebasing"
 */
#ifndef SPARSE_ATTN_H
#define SPARSE_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element order of a cube-major tensor written by sparse_attn_reorder. */
enum { SA_LAYOUT_QK = 0, SA_LAYOUT_V = 1 };

enum {
  SA_OK = 0,
  SA_ERR_INVALID_ARG = -1, /* null/misaligned pointer, bad size or parameter */
  SA_ERR_UNSUPPORTED = -2, /* valid but outside what the kernels implement */
  SA_ERR_CAPACITY = -3,    /* workspace or LUT capacity too small */
  SA_ERR_HIP = -4          /* a HIP launch or runtime call failed */
};

/* Shape of one attention call.  [VSA] "Cube Partitioning and Token
 * Re-Indexing": cubes of cube_t x cube_h x cube_w tokens (default 4x4x4).
 * cube_t*cube_h*cube_w must be 64 (the block size of every kernel).
 * head_dim must be 64 or 128; batch*heads at most 65535; nblk at most 2^24
 * and batch*heads*nblk below 2^31 (SA_ERR_UNSUPPORTED otherwise). */
typedef struct sa_geom {
  int32_t batch;
  int32_t heads;
  int32_t frames;   /* latent frames T */
  int32_t height;   /* latent rows */
  int32_t width;    /* latent columns */
  int32_t head_dim; /* d */
  int32_t cube_t;
  int32_t cube_h;
  int32_t cube_w;
} sa_geom;

/* Host only.  Block count nblk = ceil(T/ct)*ceil(H/ch)*ceil(W/cw), real
 * tokens N and padded tokens n_pad = 64*nblk of one (batch, head).
 * Padding per side follows [VSA2] section 2.2, "Kernel Implementation".
 * Any output pointer may be NULL. */
int32_t sparse_attn_geometry(const sa_geom* g, int32_t* nblk, int64_t* n_real,
                             int64_t* n_pad);

/* Host only.  Top-k count ceil(k_frac * nblk) of [SA2] "The Hybrid Top-k+Top-p
 * Masking Rule", clamped to [0, nblk]; an excess below 1e-9 from binary
 * rounding of k_frac*nblk does not round up.  Returns the count, or
 * SA_ERR_INVALID_ARG for nblk < 0 or a non-finite k_frac. */
int32_t sparse_attn_ceil_k(double k_frac, int32_t nblk);

/* Cube re-indexing, [VSA] "Cube Partitioning and Token Re-Indexing"; [VSA2]
 * section 2.2 "Permutation".
 *   x      [batch, heads, N, head_dim] bf16, row-major tokens         (input)
 *   xc     [batch, heads, n_pad, head_dim] bf16, cube-major           (output)
 *   layout SA_LAYOUT_QK for queries and keys, SA_LAYOUT_V for values
 * Pad slots of xc are written with zeros.  x and xc must not overlap. */
int32_t sparse_attn_reorder(const void* x, void* xc, int32_t layout,
                            const sa_geom* g, void* stream);

/* sparse_attn_reorder fused with the block means of sparse_attn_pool:
 * [VSA] "Cube Partitioning and Token Re-Indexing"; [SA2] "Block-Pooled
 * Attention for Efficient Mask Construction" step 2 (queries, keys); [VSA]
 * "The Coarse Stage" (pooled values for the coarse output).
 *   x      [batch, heads, N, head_dim] bf16, row-major tokens         (input)
 *   xc     [batch, heads, n_pad, head_dim] bf16 in `layout`           (output)
 *   layout SA_LAYOUT_QK or SA_LAYOUT_V
 *   xbar   [batch, heads, nblk, head_dim] float64 block means         (output)
 * xc is bit-identical to sparse_attn_reorder's and xbar to sparse_attn_pool's
 * output for the same tokens; pooling then costs no second read of xc. */
int32_t sparse_attn_reorder_pool(const void* x, void* xc, int32_t layout,
                                 double* xbar, const sa_geom* g, void* stream);

/* The three re-indexings of one attention call in one launch: queries and
 * keys to SA_LAYOUT_QK with their block means (sparse_attn_reorder_pool) and
 * values to SA_LAYOUT_V (sparse_attn_reorder).  [VSA] "Cube Partitioning and
 * Token Re-Indexing"; [SA2] "Block-Pooled Attention for Efficient Mask
 * Construction" step 2.
 *   q, k, v    [batch, heads, N, head_dim] bf16, row-major tokens     (inputs)
 *   qc, kc     [batch, heads, n_pad, head_dim] bf16, SA_LAYOUT_QK     (outputs)
 *   vc         [batch, heads, n_pad, head_dim] bf16, SA_LAYOUT_V      (output)
 *   qbar, kbar [batch, heads, nblk, head_dim] float64 block means     (outputs)
 * Every output is bit-identical to that of the separate calls; one launch
 * instead of three saves two kernel boundaries.  No output may overlap an
 * input. */
int32_t sparse_attn_reorder_qkv(const void* q, const void* k, const void* v,
                                void* qc, void* kc, void* vc, double* qbar,
                                double* kbar, const sa_geom* g, void* stream);

/* Inverse re-indexing of the attention output (pad slots dropped): the
 * inverse permutation of [VSA2] section 2.2 "Permutation", applied once at
 * the end of the attention; [VSA] "Cube Partitioning and Token Re-Indexing".
 *   oc    [batch, heads, n_pad, head_dim] bf16, slot-major  (input)
 *   o     [batch, heads, N, head_dim] bf16       (output)
 *   lse_c [batch, heads, n_pad] float32          (input, may be NULL)
 *   lse   [batch, heads, N] float32              (output, NULL iff lse_c is)
 */
int32_t sparse_attn_unreorder(const void* oc, void* o, const float* lse_c,
                              float* lse, const sa_geom* g, void* stream);

/* Mean pooling of each block's real tokens, [SA2] "Block-Pooled Attention for
 * Efficient Mask Construction" step 2; [VSA] "The Coarse Stage".
 *   qc, kc     [batch, heads, n_pad, head_dim] bf16, SA_LAYOUT_QK  (inputs)
 *   qbar, kbar [batch, heads, nblk, head_dim] float64              (outputs)
 * Sums are taken in float64 (exact for bf16 inputs) and divided by the block's
 * real-token count. */
int32_t sparse_attn_pool(const void* qc, const void* kc, double* qbar,
                         double* kbar, const sa_geom* g, void* stream);

/* Pooled block scores S = Qbar Kbar^T * scale, [SA2] "Block-Pooled Attention
 * for Efficient Mask Construction" step 3, in float64 on the matrix cores.
 *   qbar, kbar [batch, heads, nblk, head_dim] float64   (inputs)
 *   scores     [batch, heads, nblk, nblk] float64       (output)
 * scale <= 0 selects 1/sqrt(head_dim). */
int32_t sparse_attn_block_scores(const double* qbar, const double* kbar,
                                 double* scores, double scale,
                                 const sa_geom* g, void* stream);

/* The same block scores written as float32, computed on the bf16 matrix
 * cores: each float64 mean is split into three bf16 terms (the remainder is
 * below 2^-24 of the mean), the six term products that reach float32
 * accuracy are summed in float32 (the largest apart from the five smaller),
 * and the two sums are added and scaled in float64 before one rounding to
 * float32.  The page fixes no precision for this step; the error is a few
 * 1e-7 of a row's largest |score|, inside the 1e-6 relative margin at which
 * two scores count as tied for the selection.  Half the bytes of the float64
 * form.
 *   qbar, kbar [batch, heads, nblk, head_dim] float64, 16-byte aligned (inputs)
 *   scores     [batch, heads, nblk, nblk] float32       (output) */
int32_t sparse_attn_block_scores_f32(const double* qbar, const double* kbar,
                                     float* scores, double scale,
                                     const sa_geom* g, void* stream);

/* Coarse branch output, [VSA] "The Coarse Stage" ([VSA2] section 2.2):
 * attention at block granularity on the pooled tokens,
 *   oc[i] = sum_j softmax(scores[i, :])_j * vbar[j],
 * in float64; row i is the coarse output of every real token of block i (the
 * gate that would mix it with the fine output needs trained weights and is
 * not part of the library).
 *   scores [batch, heads, nblk, nblk] float64 (sparse_attn_block_scores)  (input)
 *   vbar   [batch, heads, nblk, head_dim] float64 pooled values
 *          (sparse_attn_reorder_pool with SA_LAYOUT_V)                     (input)
 *   oc     [batch, heads, nblk, head_dim] float64                          (output)
 * oc must not overlap the inputs. */
int32_t sparse_attn_coarse(const double* scores, const double* vbar, double* oc,
                           const sa_geom* g, void* stream);

/* Fine-grained router, [VSA2] section 2.2 (router equations, Figure 2,
 * "Kernel Implementation"): Q and K pooled over sub-cubes of rt x rh x rw
 * tokens (G = 64 / (rt*rh*rw) sub-cubes per cube; the sub-cube must tile the
 * cube), the router softmax over every sub-cube key of the head, and a G x G
 * aggregation into block scores P_r.  Readings of the aggregation: sum over
 * the key sub-cubes of a block, mean over the query sub-cubes, so each row of
 * P_r sums to 1; sub-cubes holding only pad slots take no part.
 *
 * sparse_attn_router_pool: sub-cube means of a QK-layout tensor.
 *   xc [batch, heads, n_pad, head_dim] bf16, SA_LAYOUT_QK            (input)
 *   xr [batch, heads, nblk*G, head_dim] float64, row blk*G + a       (output)
 *      (sub-cube a row-major over the cube's sub-cube grid; an all-pad
 *      sub-cube gets zeros)
 * sparse_attn_router_scores: log P_r, float64, without materialising the
 * router softmax.
 *   qr, kr [batch, heads, nblk*G, head_dim] float64                  (inputs)
 *   scores [batch, heads, nblk, nblk] float64 = log P_r               (output)
 *   scale <= 0 selects 1/sqrt(head_dim).
 *   workspace NULL: the page's two passes over the sub-cube scores (the row
 *     log-sum-exp first, then the softmax and the aggregation), no scratch.
 *   workspace non-NULL (device, 256-byte aligned, workspace_bytes of it):
 *     one pass.  Each row's mass on each key block is kept in the workspace,
 *     relative to the row's running maximum, and rescaled by the row's
 *     log-sum-exp once the sweep has ended, so the scores and their
 *     exponentials are computed once.  Same values up to rounding.
 *     sparse_attn_router_workspace_bytes gives the size for every head at
 *     once; a smaller workspace runs the heads in chunks of what it holds,
 *     and one smaller than a single head's share is SA_ERR_CAPACITY.  Calls
 *     that overlap must not share a workspace.
 * The scores go to sparse_attn_select unchanged: their row softmax is P_r. */
int32_t sparse_attn_router_pool(const void* xc, double* xr, const sa_geom* g,
                                int32_t rt, int32_t rh, int32_t rw, void* stream);
int32_t sparse_attn_router_scores(const double* qr, const double* kr,
                                  double* scores, double scale,
                                  const sa_geom* g, int32_t rt, int32_t rh,
                                  int32_t rw, void* workspace,
                                  size_t workspace_bytes, void* stream);

/* sparse_attn_router_scores in float32: the sub-cube means rounded to
 * float32, the sub-cube scores (with a workspace: summed in float32 from
 * exact three-term bf16 splits of those means on the bf16 matrix cores;
 * without one: on the float32 matrix cores) and their exponentials in
 * float32, the row log-sum-exp accumulated in float64, and log P_r written as
 * float32 for sparse_attn_select_f32.  Checked against the float64 lists of
 * the oracle outside near ties.  Workspace as above (its size for
 * score_bytes 4).
 *   scores [batch, heads, nblk, nblk] float32 = log P_r               (output) */
int32_t sparse_attn_router_scores_f32(const double* qr, const double* kr,
                                      float* scores, double scale, const sa_geom* g,
                                      int32_t rt, int32_t rh, int32_t rw,
                                      void* workspace, size_t workspace_bytes,
                                      void* stream);

/* Bytes of workspace for the one-pass router over every (batch, head):
 * score_bytes 8 for sparse_attn_router_scores, 4 for the float32 form (0 for
 * an invalid geometry, sub-cube or score_bytes).  At 720p with 2x2x2
 * sub-cubes that is about 150 MB (float64) or 84 MB (float32) per head. */
size_t sparse_attn_router_workspace_bytes(const sa_geom* g, int32_t rt,
                                          int32_t rh, int32_t rw,
                                          int32_t score_bytes);

/* ---- the whole path in one call ------------------------------------------
 * Buffers of sparse_attn_attention (device pointers the caller allocated). */
typedef struct sa_path_buffers {
  const void* q;        /* [batch, heads, N, head_dim] bf16, row-major tokens (inputs) */
  const void* k;
  const void* v;
  void* qc;             /* [batch, heads, n_pad, head_dim] bf16, cube-major operands (written) */
  void* kc;
  void* vc;
  double* qbar;         /* [batch, heads, nblk, head_dim] float64 block means (written),
                           16-byte aligned (as kbar) */
  double* kbar;
  void* scores;         /* workspace of batch*heads*nblk*nblk*8 bytes, 8-byte aligned; holds
                           the float32 pooled scores [batch, heads, nblk, nblk] in its first
                           half on return (as sparse_attn_block_scores_f32 writes them; with
                           row_budget its start is then reused for the forward's
                           count-balanced row order, see sparse_attn_fwd) */
  int32_t* lut;         /* [batch, heads, nblk, cap] kept lists (written) */
  int32_t* counts;      /* [batch, heads, nblk] */
  int32_t cap;
  const int32_t* row_budget; /* [batch, heads, nblk] or NULL, as for sparse_attn_select */
  void* oc;             /* [batch, heads, n_pad, head_dim] bf16 slot-major output (written), or
                           NULL together with lse_c: the forward then writes o and lse in token
                           order directly and the slot-major copy (which sparse_attn_bwd_delta
                           and sparse_attn_bwd take) is not produced */
  float* lse_c;         /* [batch, heads, n_pad] (written), or NULL with oc */
  void* o;              /* [batch, heads, N, head_dim] bf16 output in token order (written) */
  float* lse;           /* [batch, heads, N] (written) */
} sa_path_buffers;

/* The mask phase of sparse_attn_attention alone: re-indexing of Q, K (block
 * means on the way) and V, block scores and selection ([VSA] "Cube
 * Partitioning and Token Re-Indexing"; [SA2] "Block-Pooled Attention for
 * Efficient Mask Construction" and "The Hybrid Top-k+Top-p Masking Rule").
 * Writes qc, kc, vc, qbar, kbar, scores, lut and counts of `buffers`; oc,
 * lse_c, o and lse are not used and may be NULL.  With aux_stream NULL (or
 * equal to stream) the kernels run in order on `stream`.  Otherwise the
 * batch*heads rows are cut into up to 4 parts: `stream` re-indexes the first
 * part's queries and keys and then builds each part's mask as soon as its
 * inputs are ready, while aux_stream re-indexes the other parts' queries and
 * keys and then the values (the re-indexing is bound by HBM, the scores and
 * selection by compute, so the two overlap).  `stream` waits for aux_stream's
 * last work, so completion is observed on `stream`.  The results are the same
 * either way.  Allocation, synchronisation and graph capture as for
 * sparse_attn_attention. */
int32_t sparse_attn_mask_path(const sa_path_buffers* buffers, const sa_geom* g,
                              double k_frac, double p, void* stream,
                              void* aux_stream);

/* reorder_pool(Q), reorder_pool(K), reorder(V), block_scores, select, fwd,
 * unreorder -- the path of [SA2] Algorithm 1 and [VSA]'s two stages -- in one
 * call.  Block scores use 1/sqrt(head_dim); `scale` (<= 0: 1/sqrt(head_dim))
 * is the attention scale.  With aux_stream NULL (or equal to stream) the
 * kernels run in order on `stream`.  Otherwise two streams share the work:
 * the mask phase runs as in sparse_attn_mask_path (the rows in up to 4 parts,
 * masks on `stream` beside the re-indexing on aux_stream); the forward then
 * runs on aux_stream in chunks of head_chunk
 * batch*heads rows (head_chunk >= batch*heads: one chunk), and `stream`
 * re-indexes each chunk's output while the next chunk's forward runs (with
 * buffers->oc NULL the forward writes token order itself and `stream` only
 * waits for each chunk).  The last work on `stream` waits for the last
 * forward chunk, so completion is observed on `stream`.  The results are the
 * same either way.  Both streams must belong to the current device.
 *
 * The call neither allocates nor synchronises the host, so it can be captured
 * in a HIP graph on `stream`.  aux_stream forks from the capture through the
 * call's events and joins it again before the call returns.  The first call
 * on a host thread creates those events; making one call before capturing
 * keeps their creation out of the captured region. */
int32_t sparse_attn_attention(const sa_path_buffers* buffers, const sa_geom* g,
                              double k_frac, double p, float scale,
                              int32_t head_chunk, void* stream,
                              void* aux_stream);

/* ---- backward pass of the block-sparse attention ------------------------
 * [SA2] "Why this implementation is trainable": gradients flow through the
 * kept blocks (the mask carries none).  For query block i and its kept key
 * blocks, with P recomputed from the forward's LSE:
 *   D = rowsum(dO * O), dP = dO V^T, dS = P * (dP - D),
 *   dV += P^T dO, dK += scale dS^T Q, dQ += scale dS K.
 * The caller runs sparse_attn_bwd_delta, sparse_attn_transpose_lut and then
 * sparse_attn_bwd.  dQ is accumulated per query block along the kept list,
 * dK and dV per key block along the transposed list, without atomics, so the
 * results are deterministic. */

/* D = rowsum(dO * O) per slot.
 *   oc     [batch, heads, n_pad, head_dim] bf16, slot-major (sparse_attn_fwd) (input)
 *   do_qk  [batch, heads, n_pad, head_dim] bf16 dO in SA_LAYOUT_QK          (input)
 *   delta  [batch, heads, n_pad] float32                                  (output) */
int32_t sparse_attn_bwd_delta(const void* oc, const void* do_qk, float* delta,
                              const sa_geom* g, void* stream);

/* Bytes of workspace sparse_attn_transpose_lut needs (a bitmap of
 * nblk x ceil(nblk/32) words per head).  0 on an invalid geometry. */
size_t sparse_attn_transpose_workspace_bytes(const sa_geom* g);

/* Transposed kept lists: for every key block j, the query blocks whose list
 * holds j, in ascending order.
 *   lut, counts, cap      forward lists as sparse_attn_select writes them (inputs)
 *   lut_t [batch, heads, nblk, cap_t] int32, counts_t [batch, heads, nblk] (outputs)
 * cap_t must be >= nblk (SA_ERR_CAPACITY otherwise); the workspace is
 * cleared by the call itself. */
int32_t sparse_attn_transpose_lut(const int32_t* lut, const int32_t* counts,
                                  int32_t cap, int32_t* lut_t, int32_t* counts_t,
                                  int32_t cap_t, const sa_geom* g,
                                  void* workspace, size_t workspace_bytes,
                                  void* stream);

/* Operands of sparse_attn_bwd (device pointers).  Tensors are cube-major
 * [batch, heads, n_pad, head_dim] bf16 in the layout named. */
typedef struct sa_bwd_args {
  const void* q;         /* queries, SA_LAYOUT_QK */
  const void* k;         /* keys, SA_LAYOUT_QK */
  const void* v_qk;      /* values, SA_LAYOUT_QK */
  const void* k_v;       /* keys, SA_LAYOUT_V */
  const void* do_qk;     /* output gradient, SA_LAYOUT_QK */
  const float* lse;      /* [batch, heads, n_pad] natural-log LSE of sparse_attn_fwd (16-byte aligned) */
  const float* delta;    /* [batch, heads, n_pad] from sparse_attn_bwd_delta (16-byte aligned) */
  const int32_t* lut;    /* forward lists [batch, heads, nblk, cap] */
  const int32_t* counts;
  int32_t cap;
  const int32_t* lut_t;  /* transposed lists [batch, heads, nblk, cap_t] */
  const int32_t* counts_t;
  int32_t cap_t;
} sa_bwd_args;

/* Gradients of sparse_attn_fwd's O with respect to Q, K and V.
 *   dq, dk, dv [batch, heads, n_pad, head_dim] bf16, slot-major like oc
 *   (pad slots get zeros; sparse_attn_unreorder brings them to token order)
 * scale must be the forward's (<= 0 selects 1/sqrt(head_dim)). */
int32_t sparse_attn_bwd(const sa_bwd_args* args, const sa_geom* g, float scale,
                        void* dq, void* dk, void* dv, void* stream);

/* ---- mask-quality diagnostics --------------------------------------------
 * [SA2] "The Sparse Attention Error Decomposition" (Eq. 8's tau, Table 1's L1
 * error); [VSA] on the attention mass the selected cubes capture.
 *
 * sparse_attn_pooled_mass: per row, the mass the kept blocks hold in the row
 * softmax of `scores` (block scores or router scores), float64.
 *   scores [batch, heads, nblk, nblk] float64; lut, counts, cap as selected
 *   mass   [batch, heads, nblk] float64                                (output)
 * sparse_attn_mask_error: from a sparse forward (lists) and a dense one
 * (every block kept, e.g. sparse_attn_select with p = 1):
 *   lse_s, lse_d [batch, heads, n_pad] float32 (inputs)
 *   oc_s, oc_d   [batch, heads, n_pad, head_dim] bf16 slot-major (inputs)
 *   tau    [batch, heads, n_pad] float32 = exp(lse_s - lse_d), the dense
 *          softmax mass on the kept real keys (0 on pad slots)       (output)
 *   rel_l1 [batch, heads, nblk] float32 = sum|o_s - o_d| / sum|o_d| over the
 *          block's real queries                                        (output) */
int32_t sparse_attn_pooled_mass(const double* scores, const int32_t* lut,
                                const int32_t* counts, int32_t cap,
                                const sa_geom* g, double* mass, void* stream);
int32_t sparse_attn_mask_error(const float* lse_s, const float* lse_d,
                               const void* oc_s, const void* oc_d,
                               const sa_geom* g, float* tau, float* rel_l1,
                               void* stream);

/* sparse_attn_mask_error plus the two terms of [SA2] Eq. 8 ("The Sparse
 * Attention Error Decomposition"), o - o_s = (p(1 - m) + (1 - 1/tau)(p m))V:
 * per query the dropped term (p(1 - m))V = o_d - tau o_s and the
 * renormalisation term (1 - 1/tau)(p m)V = (tau - 1) o_s, each summed in L1
 * over the block's real queries and the head_dim channels and divided by
 * sum |o_d| (0 for a block whose dense output is all zero).
 *   inputs, tau, rel_l1 as for sparse_attn_mask_error
 *   rel_drop, rel_ren [batch, heads, nblk] float32                     (outputs) */
int32_t sparse_attn_mask_error_terms(const float* lse_s, const float* lse_d,
                                     const void* oc_s, const void* oc_d,
                                     const sa_geom* g, float* tau,
                                     float* rel_l1, float* rel_drop,
                                     float* rel_ren, void* stream);

/* Hybrid Top-k U Top-p selection, [SA2] "The Hybrid Top-k+Top-p Masking Rule"
 * (Eq. 9), producing index lists as [VSA] "Kernel Implementation" describes
 * (contiguous block ids, not a binary mask).
 * Per row i (one query block of one batch/head), with the row's softmax P:
 *   order = block ids by score descending, lower id first on equal scores;
 *   kc    = row_budget ? row_budget[row] (clamped to [0, nblk])
 *                      : sparse_attn_ceil_k(k_frac, nblk);
 *   pc    = shortest prefix of `order` whose probability sum reaches p
 *           (p <= 0: 0; p >= 1: nblk);
 *   kept  = the first max(kc, pc) ids of `order`, written in ascending id.
 *   scores [batch, heads, nblk, nblk] float64                 (input)
 *   row_budget [batch, heads, nblk] int32 or NULL; when given, p must be 0
 *   lut    [batch, heads, nblk, cap] int32: row r's ids in lut[r*cap ...]
 *   counts [batch, heads, nblk] int32: number of ids in each row
 * cap must be >= nblk when p > 0 or row_budget is given, else >= kc.
 * Entries of lut beyond a row's count are left as they were.
 * Probability mass is accumulated in 2^-40 fixed point from float32
 * exponentials, so the result is deterministic; a row whose decision hinges on
 * a cumulative sum within ~1e-7 of p may differ from an exact evaluation.
 * nblk must be <= 4096. */
int32_t sparse_attn_select(const double* scores, const sa_geom* g,
                           double k_frac, double p, const int32_t* row_budget,
                           int32_t* lut, int32_t* counts, int32_t cap,
                           void* stream);

/* sparse_attn_select on float32 scores (sparse_attn_block_scores_f32): each
 * score is widened exactly to float64 when loaded, so the lists are those
 * sparse_attn_select gives for the same values; same arguments and errors.
 *   scores [batch, heads, nblk, nblk] float32                 (input) */
int32_t sparse_attn_select_f32(const float* scores, const sa_geom* g,
                               double k_frac, double p, const int32_t* row_budget,
                               int32_t* lut, int32_t* counts, int32_t cap,
                               void* stream);

/* Bytes of workspace sparse_attn_build_mask needs (Qbar and Kbar in float64,
 * then room for the scores at 8 bytes each, each region 256-byte aligned).
 * 0 on an invalid geometry. */
size_t sparse_attn_mask_workspace_bytes(const sa_geom* g);

/* pool + block_scores_f32 + select_f32 in one call (scale 1/sqrt(head_dim)):
 * float64 block means, float32 scores (the same lists as the float64 scores
 * outside near ties; the whole-path calls use the same kernels).  block must
 * be 64.  Arguments as for those functions; the intermediates live in
 * `workspace` (>= sparse_attn_mask_workspace_bytes, else SA_ERR_CAPACITY). */
int32_t sparse_attn_build_mask(const void* qc, const void* kc,
                               const sa_geom* g, int32_t block, double k_frac,
                               double p, const int32_t* row_budget,
                               int32_t* lut, int32_t* counts, int32_t cap,
                               void* workspace, size_t workspace_bytes,
                               void* stream);

/* sparse_attn_build_mask for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same arguments without the workspace, the same lists and
 * counts.  The float64 block means and float32 scores live in a device array
 * of the library, fixed at sparse_attn_build_mask_noalloc_scratch_bytes()
 * (64 MiB) per GPU and held until the process ends; the (batch, head) rows are
 * taken in chunks that fit it, one after another on `stream`.  One (batch,
 * head) needs 2*round256(nblk*head_dim*8) + round256(nblk*nblk*4) bytes; above
 * the array's size (nblk above about 3,800 at head_dim 128) the call returns
 * SA_ERR_CAPACITY and launches nothing.  The call allocates and frees
 * nothing.  Calls on one GPU share the array: calls that overlap (other
 * streams, other host threads) race and must be ordered by the caller. */
size_t sparse_attn_build_mask_noalloc_scratch_bytes(void);
int32_t sparse_attn_build_mask_noalloc(const void* qc, const void* kc,
                                       const sa_geom* g, int32_t block,
                                       double k_frac, double p,
                                       const int32_t* row_budget,
                                       int32_t* lut, int32_t* counts,
                                       int32_t cap, void* stream);

/* Bytes of workspace sparse_attn_fwd and sparse_attn_fwd_tokens use for the
 * count-balanced order of their rows (one int32 per workgroup). */
size_t sparse_attn_fwd_workspace_bytes(const sa_geom* g);

/* Block-sparse attention forward, [SA2] "Kernel Implementation of the
 * Hybrid-Masked Block-Sparse Attention" (Algorithm 1) and the renormalised
 * output of "The Sparse Attention Error Decomposition"; [VSA] "The Fine
 * Stage".  For every real query token of query block i, over the real keys
 * of the blocks lut[row][0 .. counts[row]-1]:
 *   O   = sum_j softmax_j(scale * q.k_j) v_j
 *   LSE = ln sum_j exp(scale * q.k_j)
 *   qc, kc     [batch, heads, n_pad, head_dim] bf16, SA_LAYOUT_QK  (inputs)
 *   vc         [batch, heads, n_pad, head_dim] bf16, SA_LAYOUT_V   (input)
 *   lut, counts as written by sparse_attn_select; at most cap ids per row are
 *               read, ids outside [0, nblk) are skipped
 *   oc    [batch, heads, n_pad, head_dim] bf16, slot-major        (output)
 *   lse_c [batch, heads, n_pad] float32, natural log              (output)
 * Rows with count 0 and pad query slots get O = 0, LSE = -inf.  Products run
 * in bf16 on the matrix cores with float32 accumulation and an online
 * softmax in float32.  scale <= 0 selects 1/sqrt(head_dim).
 * One workgroup per query block; the rows go to the 8 XCDs in sweeps of
 * neighbouring query blocks (four XCDs per head), so blocks with overlapping
 * lists share K/V in an XCD's L2.  When a head's K/V is 32 MiB or more
 * (nblk >= 1024 at head_dim 128), groups of four neighbouring query blocks
 * whose lists are dense (summed count at least nblk per block / 4) run
 * instead in a second kernel whose four wavefronts walk the union of their
 * lists together, each K/V tile copied once into an LDS ring (direct
 * global-to-LDS loads) and read from there by every wavefront whose list
 * holds it, in the same order: the results are the same bytes, with a
 * quarter or less of the tile traffic.  With workspace NULL that sweep order is
 * used as is, which balances rows of similar list lengths.  With a workspace
 * (>= sparse_attn_fwd_workspace_bytes, else SA_ERR_CAPACITY) a small kernel
 * first writes a count-balanced order into it: each quarter-head run of the
 * sweep whose longest list is above twice the run's mean is reordered
 * longest list first, so rows of very different lengths (per-row budgets)
 * end together.  The results are identical either way.  The call rewrites
 * the workspace before the forward reads it (no memset), so it can be
 * captured in a HIP graph; calls that overlap must not share a workspace. */
int32_t sparse_attn_fwd(const void* qc, const void* kc, const void* vc,
                        const int32_t* lut, const int32_t* counts, int32_t cap,
                        const sa_geom* g, float scale, void* oc, float* lse_c,
                        void* workspace, size_t workspace_bytes, void* stream);

/* The same forward with the inverse re-indexing ([VSA2] section 2.2,
 * "Permutation") fused into its epilogue: O and LSE go straight to token
 * order, as sparse_attn_unreorder would leave them, and no slot-major copy
 * is written (the backward needs that copy: use sparse_attn_fwd there).
 *   qc, kc, vc, lut, counts, cap, scale as for sparse_attn_fwd     (inputs)
 *   o    [batch, heads, N, head_dim] bf16, token order            (output)
 *   lse  [batch, heads, N] float32, natural log                   (output)
 *   workspace, workspace_bytes  the count-balanced row order, as for
 *        sparse_attn_fwd (NULL: the sweep order; the same results)
 * Bit-identical to sparse_attn_fwd followed by sparse_attn_unreorder. */
int32_t sparse_attn_fwd_tokens(const void* qc, const void* kc, const void* vc,
                               const int32_t* lut, const int32_t* counts,
                               int32_t cap, const sa_geom* g, float scale,
                               void* o, float* lse, void* workspace,
                               size_t workspace_bytes, void* stream);

/* Ideal block scores ([VSA2] section 2.2: MeanPool of the full attention
 * matrix, the target a router approximates): mass[i][j] = the full softmax
 * mass that block i's real queries put on block j's real keys, averaged over
 * those queries (rows sum to 1), recomputed from a dense run's LSE.
 *   qc, kc [batch, heads, n_pad, head_dim] bf16, SA_LAYOUT_QK        (inputs)
 *   lse_d  [batch, heads, n_pad] float32, natural-log LSE of sparse_attn_fwd
 *          with every block kept (pad slots -inf)                     (input)
 *   mass   [batch, heads, nblk, nblk] float64                         (output)
 * scale <= 0 selects 1/sqrt(head_dim) and must match the dense run's. */
int32_t sparse_attn_ideal_block_mass(const void* qc, const void* kc,
                                     const float* lse_d, const sa_geom* g,
                                     float scale, double* mass, void* stream);

/* Recall of kept lists against the ideal block scores: per row, the share of
 * the counts[row] blocks with the largest mass (lower id first on equal
 * values) that the row's list holds; 1 for an empty list.
 *   mass [batch, heads, nblk, nblk] float64; lut, counts, cap as selected,
 *   with counts <= cap                                                (inputs)
 *   recall [batch, heads, nblk] float64                               (output)
 * workspace >= sparse_attn_recall_workspace_bytes (the top lists, [batch,
 * heads, nblk, nblk] int32, and their counts), else SA_ERR_CAPACITY; nblk at
 * most 4096 (SA_ERR_UNSUPPORTED). */
size_t sparse_attn_recall_workspace_bytes(const sa_geom* g);
int32_t sparse_attn_mask_recall(const double* mass, const int32_t* lut,
                                const int32_t* counts, int32_t cap,
                                const sa_geom* g, double* recall,
                                void* workspace, size_t workspace_bytes,
                                void* stream);

/* ---- asymmetric blocks: query blocks of qgroup cubes --------------------
 * [SA2] "Block-Pooled Attention for Efficient Mask Construction": query
 * blocks of b_q tokens against key blocks of b_kv tokens (b_q = 128,
 * b_kv = 64 there).  In the cube-major order a query block is qgroup
 * consecutive cubes (qgroup 2: 128 query slots; 1, 2 or 4 accepted, else
 * SA_ERR_INVALID_ARG); key blocks stay single cubes.  A head has
 * nq = ceil(nblk / qgroup) query blocks.
 *
 * Bytes of workspace sparse_attn_build_mask_groups needs: group means of Q
 * [batch, heads, nq, head_dim], block means of K [batch, heads, nblk,
 * head_dim] and scores [batch, heads, nq, nblk], float64, in that order,
 * each region 256-byte aligned.  0 on an invalid geometry or qgroup. */
size_t sparse_attn_mask_groups_workspace_bytes(const sa_geom* g, int32_t qgroup);

/* Mask of the asymmetric blocks: Q pooled over each query block's real
 * tokens, K per cube, scores Qbar Kbar^T / sqrt(head_dim) [nq x nblk] per
 * head, then the hybrid rule on every query block's row with
 * kc = ceil(k_frac * nblk) (sparse_attn_ceil_k of nblk).
 *   qc, kc  [batch, heads, n_pad, head_dim] bf16, SA_LAYOUT_QK   (inputs)
 *   lut     [batch, heads, nq, cap] int32, counts [batch, heads, nq] (outputs)
 * cap as for sparse_attn_select; workspace >= the size above (else
 * SA_ERR_CAPACITY). */
int32_t sparse_attn_build_mask_groups(const void* qc, const void* kc,
                                      const sa_geom* g, int32_t qgroup,
                                      double k_frac, double p, int32_t* lut,
                                      int32_t* counts, int32_t cap,
                                      void* workspace, size_t workspace_bytes,
                                      void* stream);

/* sparse_attn_fwd with one kept list per query block of qgroup cubes: cube i
 * of a head attends through list row i / qgroup of lut [batch, heads, nq,
 * cap] and counts [batch, heads, nq].  Outputs as sparse_attn_fwd; qgroup 1
 * is sparse_attn_fwd itself. */
int32_t sparse_attn_fwd_groups(const void* qc, const void* kc, const void* vc,
                               const int32_t* lut, const int32_t* counts,
                               int32_t cap, int32_t qgroup, const sa_geom* g,
                               float scale, void* oc, float* lse_c,
                               void* stream);

/* ---- per-sequence Top-K -------------------------------------------------
 * [VSA2] section 1 and its ablation of the TopK scope: one budget per head
 * instead of per query block.  The budget is what per-row Top-k would keep,
 * T = nblk * ceil(k_frac * nblk) (sparse_attn_ceil_k); the T largest entries of
 * the head's row-softmax block probabilities (row i of softmax(scores)) win,
 * equal probabilities going to the lower row-major index first; row i keeps
 * its c_i = (entries of row i that won) top-scoring blocks, ascending ids, as
 * sparse_attn_select with row_budget c would.  A row may keep no block.
 *   scores [batch, heads, nblk, nblk] float64 (block or router scores) (input)
 *   lut [batch, heads, nblk, cap], counts [batch, heads, nblk]       (outputs)
 * cap must be >= nblk (SA_ERR_CAPACITY); workspace (>= the size below, else
 * SA_ERR_CAPACITY) holds row log-sum-exps, radix-select state and the counts.
 * nblk is at most 4096 (SA_ERR_UNSUPPORTED). */
size_t sparse_attn_sequence_workspace_bytes(const sa_geom* g);
int32_t sparse_attn_select_per_sequence(const double* scores, const sa_geom* g,
                                        double k_frac, int32_t* lut,
                                        int32_t* counts, int32_t cap,
                                        void* workspace, size_t workspace_bytes,
                                        void* stream);

/* Message describing the calling thread's last error ("" if none). */
const char* sparse_attn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* SPARSE_ATTN_H */
