/*
 * sdpa.h - C ABI of the MI355X (gfx950) fused scaled-dot-product attention library.
 *
 * The library computes, on one GPU:
 *   forward   O = softmax(scale * Q K^T + mask) V, and the per-row log-sum-exp
 *             LSE_i = log sum_j exp(scale * q_i . k_j) over the visible keys
 *             (natural log, scores include the scale);
 *   backward  dQ, dK, dV of a loss through O and LSE, recomputing P from LSE;
 *   merge     the LSE merge of two partial results over disjoint (or not) key sets,
 *             forward and backward.
 * Sources: "[PyTorch] fused CUDNN attention kernel not properly handling strides"
 * (TransformerEngine issue 1195: q/k/v as strided views of a packed tensor, qkv_format,
 * window_size, softmax_scale, GQA groups), "Add support for cuDNN FusedAttention + THD +
 * CP" (TransformerEngine issue 885: THD with cu_seqlens), "Significant Accuracy
 * Difference between Compiled and Eager Flex Attention" (PyTorch issue 135161:
 * return_lse, the merge_attn helper, the sliding-window masks, true fp32).
 *
 * Conventions shared by every call
 * --------------------------------
 * - Tensors are described by a base pointer and per-dimension strides counted in
 *   ELEMENTS, given in the logical order of the descriptor's layout:
 *     BSHD (b, s, h, d)   SBHD (s, b, h, d)   BHSD (b, h, s, d)   THD (t, h, d)
 *   The last (d) stride must be 1.  No other stride is assumed: q, k and v may be views
 *   of one packed [s, b, hq + 2 hk, d] buffer (base pointers offset by whole heads,
 *   strides (hq+2hk)*d, ..., d, 1).  Packed layouts are not separate tags: pass the three
 *   views.  Nothing is ever made contiguous or copied behind the caller's back.
 * - Row statistics (LSE, dLSE) are fp32 [b, h, s] for BSHD/SBHD/BHSD and [h, t] for THD,
 *   again with element strides in that order (stride[2] unused for THD).
 * - Input strides may be 0 (broadcast) or overlap (q/k/v from one buffer).  Outputs must
 *   not map two elements to one address, must not overlap each other and must not overlap
 *   any input.  Outputs that are disjoint head ranges of one packed buffer are accepted.
 * - Every call validates completely before launching; on any error it returns a non-zero
 *   status, writes nothing and leaves a message for sdpa_last_error().
 * - Compute calls are asynchronous on the given HIP stream (a hipStream_t; NULL = the
 *   default stream).  They never synchronise the device.  All buffers, the workspace
 *   included, belong to the caller and must stay alive until the stream reaches the work.
 *   The library allocates no device memory and holds no mutable global state apart from
 *   the per-thread last-error message.
 */
#ifndef SDPA_MI355X_H
#define SDPA_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SDPA_VERSION 5

/* Status codes returned by every entry point. */
enum sdpa_status {
  SDPA_OK = 0,
  SDPA_ERR_NULL = 1,        /* a required pointer is NULL                                */
  SDPA_ERR_SHAPE = 2,       /* a size is negative, zero where it may not be, or too large */
  SDPA_ERR_STRIDE = 3,      /* d-stride != 1, negative stride, or an output self-overlaps */
  SDPA_ERR_ALIGN = 4,       /* a pointer is not aligned to its element size              */
  SDPA_ERR_ALIAS = 5,       /* outputs overlap each other or an input                    */
  SDPA_ERR_UNSUPPORTED = 6, /* dtype / head_dim / layout combination not built           */
  SDPA_ERR_WORKSPACE = 7,   /* workspace missing or too small                            */
  SDPA_ERR_HIP = 8,         /* a HIP launch failed; the HIP message is in last_error     */
  SDPA_ERR_ARG = 9          /* an enum or option is out of range                         */
};

enum sdpa_layout { SDPA_LAYOUT_BSHD = 0, SDPA_LAYOUT_SBHD = 1, SDPA_LAYOUT_BHSD = 2, SDPA_LAYOUT_THD = 3 };
/* SDPA_DTYPE_FP8_E4M3: q, k, v as OCP E4M3 codes (1 sign, 4 exponent bits with bias 7, 3
 * mantissa bits, no infinities), forward only, through sdpa_fwd_fp8; O is bf16. */
enum sdpa_dtype { SDPA_DTYPE_F16 = 0, SDPA_DTYPE_BF16 = 1, SDPA_DTYPE_F32 = 2, SDPA_DTYPE_FP8_E4M3 = 3 };
/* Where the diagonal of a window sits when seqlen_q != seqlen_k: query i is aligned with
 * key i (TOP_LEFT) or with key i + seqlen_k - seqlen_q (BOTTOM_RIGHT).  Per sequence for THD. */
enum sdpa_diag_align { SDPA_ALIGN_TOP_LEFT = 0, SDPA_ALIGN_BOTTOM_RIGHT = 1 };

/* A q/k/v/o/dO/dq/dk/dv tensor: element (i0,i1,i2,i3) of the layout's logical order lives at
 * data + sum(i_n * stride[n]) elements.  For THD only stride[0..2] are read. */
typedef struct sdpa_tensor {
  void* data;
  int64_t stride[4];
} sdpa_tensor_t;

/* An fp32 row statistic (LSE or dLSE): [b,h,s] or, for THD, [h,t]. */
typedef struct sdpa_rowstat {
  float* data;
  int64_t stride[3];
} sdpa_rowstat_t;

/* Problem description shared by q, k, v, o, dO, dq, dk, dv of one call.
 *
 * batch       number of sequences (THD: entries of cu_seqlens minus one).
 * seqlen_q/k  sequence lengths (THD: the maxima over the batch; rows beyond a sequence's
 *             own length are never touched).
 * heads_q/kv  query and key/value heads; heads_q must be a multiple of heads_kv (GQA/MQA):
 *             q head h reads kv head h / (heads_q / heads_kv).
 * head_dim    D, shared by q, k, v; 32, 64 or 128.
 * cu_seqlens_q/k  THD only: DEVICE int32[batch+1], non-decreasing, starting at 0; may be the
 *             same pointer.  Entries are clamped to [0, total] on the device so a bad array
 *             cannot cause out-of-bounds access (it gives wrong rows instead).
 * total_q/k   THD only: number of packed rows of q and of k/v (= cu_seqlens[batch]).
 * softmax_scale  multiplies Q K^T; required, no default.
 * window_left/right  key j is visible to query i iff
 *             (window_left == -1 or j >= i + off - window_left) and
 *             (window_right == -1 or j <= i + off + window_right),
 *             off = 0 (TOP_LEFT) or seqlen_k - seqlen_q (BOTTOM_RIGHT).  -1 is unbounded,
 *             (-1,-1) no mask, (-1,0) causal, (128,0) a 129-key causal band.  Any other
 *             value, negative ones included, is an offset bound: (-1,-129) keeps only keys
 *             at least 129 behind the query.  A query with no visible key gets O = 0 and
 *             LSE = -inf and contributes no gradient.
 * diag_align  enum sdpa_diag_align.
 * cu_seqlens_q_padded / cu_seqlens_k_padded  THD only, optional (NULL: sequences packed
 *             back to back): DEVICE int32[batch+1], the packed row where each sequence starts
 *             ("Add support for cuDNN FusedAttention + THD + CP", TransformerEngine issue
 *             885: THD tensors with unused rows between packed sequences).  Sequence b occupies
 *             rows [padded[b], padded[b] + (cu_seqlens[b+1] - cu_seqlens[b])); the rows after
 *             it up to padded[b+1] are padding: never read as keys and never written (O, LSE,
 *             dQ, dK and dV of padding rows keep their contents; dLSE/Delta of them are not
 *             used).  Entries are clamped to [0, total] on the device.
 * block_mask  optional (NULL: none): a block-sparse element mask, see sdpa_block_mask_t.
 *             Key j is then visible to query i iff the window admits it AND the mask bit
 *             (i, j) is set.  BSHD, SBHD and BHSD only.
 * Size limit (ERR_UNSUPPORTED, before any launch): query rows times heads_q plus key rows
 * times heads_kv, rows padded to multiples of 128 per sequence (THD: total plus 128 per
 * sequence), must stay below 2^30, since a kernel launch counts its work-items in 32 bits
 * (with 64 heads, 2^23 query and key rows each are refused). */
/* Block-sparse mask (FlexAttention's BlockMask model: "Significant Accuracy Difference
 * between Compiled and Eager Flex Attention", PyTorch issue 135161, builds its masks with
 * create_block_mask from predicates over (q_idx, kv_idx) and passes them as block_mask=).
 * The (seqlen_q, seqlen_k) plane is cut into SDPA_MASK_BLOCK x SDPA_MASK_BLOCK blocks.  A
 * block with no visible pair is skipped, a block whose every pair is visible is computed
 * without an element test, any other block tests the element bits.  The result equals plain
 * attention under the element mask; the block table only saves work.
 *
 * batch, heads  extents of the mask: 1 (one mask for every batch entry / every q head) or
 *               desc->batch / desc->heads_q.  Plane (b, h) of the mask is
 *               (batch == 1 ? 0 : b) * heads + (heads == 1 ? 0 : h).
 * bits          DEVICE uint64 [batch][heads][seqlen_q][words], words = ceil(seqlen_k / 64),
 *               rows contiguous: bit j of word w of row i set <=> key 64 w + j is visible to
 *               query i.  Bits of keys >= seqlen_k are ignored.  Written by the caller.
 * kv_count      DEVICE int32 [batch][heads][nqb], nqb = ceil(seqlen_q / SDPA_MASK_BLOCK).
 * kv_list       DEVICE int32 [batch][heads][nqb][nkb], nkb = ceil(seqlen_k / SDPA_MASK_BLOCK):
 *               row qb lists, in increasing kb, 2 kb + 1 for each partial block and 2 kb for
 *               each full block; entries past kv_count are unspecified.
 * q_count       DEVICE int32 [batch][heads][nkb].
 * q_list        DEVICE int32 [batch][heads][nkb][nqb]: the same blocks by column, in
 *               increasing qb (2 qb + partial).
 * The four table arrays are written by sdpa_block_mask_build from `bits` and read by
 * sdpa_fwd / sdpa_bwd; all five buffers belong to the caller.  The attention calls trust
 * the table: it must have been built from these bits for the same seqlen_q / seqlen_k, on
 * the same stream (or after it).  Block-list entries are clamped to the plane on the device.
 * Limits (ERR_UNSUPPORTED otherwise): seqlen_q and seqlen_k at most 512 blocks (65536);
 * fp16/bf16 need 16-byte aligned rows of q, k, v, o (and dO, dq, dk, dv for the backward)
 * with k/v (and q/dO) row strides >= head_dim; the fp16/bf16 backward needs head_dim >= 64
 * and, for per-head masks, (heads_q / heads_kv) * ceil(seqlen_q / 128) <= 512.  fp32 takes
 * any strides.  Not with sdpa_cp_fwd / sdpa_cp_bwd. */
#define SDPA_MASK_BLOCK 128
typedef struct sdpa_block_mask {
  int32_t batch;
  int32_t heads;
  const uint64_t* bits;
  int32_t* kv_count;
  int32_t* kv_list;
  int32_t* q_count;
  int32_t* q_list;
} sdpa_block_mask_t;

typedef struct sdpa_desc {
  int32_t layout;
  int32_t dtype;
  int32_t batch;
  int32_t seqlen_q;
  int32_t seqlen_k;
  int32_t heads_q;
  int32_t heads_kv;
  int32_t head_dim;
  const int32_t* cu_seqlens_q;
  const int32_t* cu_seqlens_k;
  int64_t total_q;
  int64_t total_k;
  float softmax_scale;
  int32_t window_left;
  int32_t window_right;
  int32_t diag_align;
  const int32_t* cu_seqlens_q_padded;
  const int32_t* cu_seqlens_k_padded;
  const sdpa_block_mask_t* block_mask;
} sdpa_desc_t;

/* Merge description: rows of x are [layout order] tensors of `heads` heads of head_dim,
 * lse is the matching row statistic.  THD uses `total` rows and ignores seqlen; with
 * cu_seqlens (THD only, optional, DEVICE int32[batch+1]) only the rows of the batch sequences
 * are merged: sequence b's rows start at cu_seqlens_padded[b] (DEVICE int32[batch+1], or
 * cu_seqlens[b] when NULL) and number cu_seqlens[b+1] - cu_seqlens[b]; other rows are not
 * touched.  Entries are clamped to [0, total] on the device. */
typedef struct sdpa_merge_desc {
  int32_t layout;
  int32_t dtype;
  int32_t batch;
  int32_t seqlen;
  int32_t heads;
  int32_t head_dim;
  int64_t total;
  const int32_t* cu_seqlens;
  const int32_t* cu_seqlens_padded;
} sdpa_merge_desc_t;

/* Library version (SDPA_VERSION of the build). */
int sdpa_version(void);

/* Message for the last failing call on this host thread ("" if none).  The string is
 * owned by the library and valid until the next call on the same thread. */
const char* sdpa_last_error(void);

/* Forward workspace size in bytes for `desc` (0 unless layout is THD, where it holds the
 * longest-first work list built from cu_seqlens).  Host only. */
int sdpa_fwd_workspace_size(const sdpa_desc_t* desc, size_t* bytes);

/* Host-only dry run of sdpa_fwd's validation: same arguments, no launch, no device access. */
int sdpa_fwd_validate(const sdpa_desc_t* desc, const sdpa_tensor_t* q, const sdpa_tensor_t* k,
                      const sdpa_tensor_t* v, const sdpa_tensor_t* o, const sdpa_rowstat_t* lse,
                      size_t workspace_bytes);

/* Forward (fused, online softmax; TransformerEngine issue 1195 repro calls, PyTorch issue
 * 135161 return_lse=True).  Reads q, k, v; writes o (same dtype and logical shape as q) and
 * lse (fp32).  `lse->data` may be NULL to skip writing LSE. */
int sdpa_fwd(const sdpa_desc_t* desc, const sdpa_tensor_t* q, const sdpa_tensor_t* k,
             const sdpa_tensor_t* v, const sdpa_tensor_t* o, const sdpa_rowstat_t* lse,
             void* workspace, size_t workspace_bytes, void* stream);

/* FP8 forward ("[PyTorch] fused CUDNN attention kernel not properly handling strides",
 * TransformerEngine issue 1195: its fused attention call carries an FP8 recipe,
 * DelayedScaling, whose tensors are 8-bit codes with one fp32 scale per tensor).
 * desc->dtype must be SDPA_DTYPE_FP8_E4M3: q, k, v hold E4M3 codes (strides in elements =
 * bytes), o is bf16 with q's logical shape (its own strides, in bf16 elements), lse fp32.
 * descale_q/k/v: DEVICE pointers to one fp32 each (NULL = 1.0); element values are
 * code * descale.  Computes O = softmax(scale * Q K^T + mask) V on those values with both
 * products on FP8 matrix cores; P is rounded to E4M3 after scaling by 2^8 (the row sum and
 * the LSE use the unrounded fp32 P).  head_dim 64 or 128; q, k, v and o rows 16-byte aligned
 * with k and v row strides >= head_dim (ERR_UNSUPPORTED otherwise); no block_mask.  The
 * workspace is sdpa_fwd_workspace_size's.  Other calls reject SDPA_DTYPE_FP8_E4M3. */
int sdpa_fwd_fp8_validate(const sdpa_desc_t* desc, const sdpa_tensor_t* q, const sdpa_tensor_t* k,
                          const sdpa_tensor_t* v, const sdpa_tensor_t* o, const sdpa_rowstat_t* lse,
                          size_t workspace_bytes);
int sdpa_fwd_fp8(const sdpa_desc_t* desc, const sdpa_tensor_t* q, const sdpa_tensor_t* k,
                 const sdpa_tensor_t* v, const float* descale_q, const float* descale_k,
                 const float* descale_v, const sdpa_tensor_t* o, const sdpa_rowstat_t* lse,
                 void* workspace, size_t workspace_bytes, void* stream);

/* Backward workspace size in bytes: fp32 Delta_i = dO_i . O_i - dLSE_i and fp32
 * LSE_i * log2(e) for every q row, plus the THD work lists, plus under GQA on small grids
 * (16-bit inputs, head_dim 64 or 128, no block mask, at most 8 work blocks per compute unit
 * of the current device) the fp32 partial dK/dV sums of the two halves of every 64-key block
 * (1 KiB x head_dim per block) and one counter per block, plus for THD on large grids (16-bit,
 * head_dim 64 or 128, no block mask, more than 12 work blocks per compute unit) up to 32 MiB
 * of fp32 partial dK/dV sums for the longest key tiles, which may run as two halves.  That
 * last room is optional: given a workspace without it, sdpa_bwd splits no key tile (the
 * results then differ only in the order of their fp32 sums).  Host only; query it with the
 * device that will run the call current. */
int sdpa_bwd_workspace_size(const sdpa_desc_t* desc, size_t* bytes);

/* Host-only dry run of sdpa_bwd's validation. */
int sdpa_bwd_validate(const sdpa_desc_t* desc, const sdpa_tensor_t* q, const sdpa_tensor_t* k,
                      const sdpa_tensor_t* v, const sdpa_tensor_t* o, const sdpa_rowstat_t* lse,
                      const sdpa_tensor_t* dout, const sdpa_rowstat_t* dlse,
                      const sdpa_tensor_t* dq, const sdpa_tensor_t* dk, const sdpa_tensor_t* dv,
                      size_t workspace_bytes);

/* Backward from the saved LSE (PyTorch issue 135161: gradients through O and through the
 * returned LSE).  Reads q, k, v, o, lse (from sdpa_fwd), dout and optionally dlse
 * (dlse == NULL or dlse->data == NULL means dL/dLSE = 0).  Writes dq (q's shape), dk and dv
 * (k's shape; summed over the q heads of each group).  No atomic accumulation: every output
 * element has one writer (under GQA on small grids the second of a block's two halves to
 * finish, found with one atomic counter per block, adds the first half's partial sums in
 * fp32; under THD on large grids the two halves of a long key tile write their fp32 sums to
 * slots of their own and a following launch adds them; neither result depends on which half
 * finishes first).  accumulate = 0 overwrites, 1 adds to the existing contents (to sum the
 * gradients of several partial attentions into one buffer). */
int sdpa_bwd(const sdpa_desc_t* desc, const sdpa_tensor_t* q, const sdpa_tensor_t* k,
             const sdpa_tensor_t* v, const sdpa_tensor_t* o, const sdpa_rowstat_t* lse,
             const sdpa_tensor_t* dout, const sdpa_rowstat_t* dlse, const sdpa_tensor_t* dq,
             const sdpa_tensor_t* dk, const sdpa_tensor_t* dv, int accumulate, void* workspace,
             size_t workspace_bytes, void* stream);

/* sdpa_bwd for callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): the same kernels, with the workspace
 * taken from a static device buffer of sdpa_bwd_noalloc_max_workspace() bytes (64 MiB) that
 * each GPU holds until the process ends, instead of the caller's.  Arguments, results and
 * errors as sdpa_bwd; a problem whose workspace, less the optional room for split key tiles,
 * exceeds the buffer returns ERR_WORKSPACE before anything runs.  Allocates nothing (no hipMalloc / hipFree).  Every
 * call on one GPU shares that GPU's buffer: calls that overlap on one GPU (other streams or
 * host threads) race and must be serialised by the caller; calls on one stream are ordered.
 * The buffer needs no clearing: each call's kernels write what they later read. */
size_t sdpa_bwd_noalloc_max_workspace(void);
int sdpa_bwd_noalloc(const sdpa_desc_t* desc, const sdpa_tensor_t* q, const sdpa_tensor_t* k,
                     const sdpa_tensor_t* v, const sdpa_tensor_t* o, const sdpa_rowstat_t* lse,
                     const sdpa_tensor_t* dout, const sdpa_rowstat_t* dlse,
                     const sdpa_tensor_t* dq, const sdpa_tensor_t* dk, const sdpa_tensor_t* dv,
                     int accumulate, void* stream);

/* Builds the block table of `mask` (kv_count, kv_list, q_count, q_list) from its bits on
 * `stream`: every block of the (seqlen_q, seqlen_k) plane is classified over its pairs
 * inside the plane (the last block row and column may be short).  Asynchronous; reads only
 * bits, writes only the four table arrays.  Errors: NULL pointers (ERR_NULL), batch or heads
 * < 1, seqlen_q or seqlen_k < 1 or > 2^28 - 1 (ERR_SHAPE). */
int sdpa_block_mask_build(const sdpa_block_mask_t* mask, int32_t seqlen_q, int32_t seqlen_k,
                          void* stream);

/* Host-only dry runs of the merge calls. */
int sdpa_merge_fwd_validate(const sdpa_merge_desc_t* desc, const sdpa_tensor_t* x_a,
                            const sdpa_rowstat_t* lse_a, const sdpa_tensor_t* x_b,
                            const sdpa_rowstat_t* lse_b, const sdpa_tensor_t* x,
                            const sdpa_rowstat_t* lse);
int sdpa_merge_bwd_validate(const sdpa_merge_desc_t* desc, const sdpa_tensor_t* x_a,
                            const sdpa_rowstat_t* lse_a, const sdpa_tensor_t* x_b,
                            const sdpa_rowstat_t* lse_b, const sdpa_tensor_t* g,
                            const sdpa_rowstat_t* g_lse, const sdpa_tensor_t* dx_a,
                            const sdpa_rowstat_t* dlse_a, const sdpa_tensor_t* dx_b,
                            const sdpa_rowstat_t* dlse_b);

/* LSE merge of two partials (PyTorch issue 135161, merge_attn): per row,
 * m = max(lse_a, lse_b), w = exp(lse - m), x = (x_a w_a + x_b w_b) / (w_a + w_b),
 * lse = m + log(w_a + w_b); two -inf rows give (0, -inf).  Computed in fp32, x rounded to
 * the dtype.  `lse->data` may be NULL to skip it. */
int sdpa_merge_fwd(const sdpa_merge_desc_t* desc, const sdpa_tensor_t* x_a,
                   const sdpa_rowstat_t* lse_a, const sdpa_tensor_t* x_b,
                   const sdpa_rowstat_t* lse_b, const sdpa_tensor_t* x,
                   const sdpa_rowstat_t* lse, void* stream);

/* Backward of the merge for upstream g = dL/dx and g_lse = dL/dlse (NULL = 0), with
 * alpha = w_a / (w_a + w_b), beta = w_b / (w_a + w_b):
 *   dx_a = alpha g,  dx_b = beta g,
 *   dlse_a = alpha beta sum_d g (x_a - x_b) + alpha g_lse,  dlse_b symmetric.
 * Recomputes alpha and beta from lse_a and lse_b (no saved output needed). */
int sdpa_merge_bwd(const sdpa_merge_desc_t* desc, const sdpa_tensor_t* x_a,
                   const sdpa_rowstat_t* lse_a, const sdpa_tensor_t* x_b,
                   const sdpa_rowstat_t* lse_b, const sdpa_tensor_t* g,
                   const sdpa_rowstat_t* g_lse, const sdpa_tensor_t* dx_a,
                   const sdpa_rowstat_t* dlse_a, const sdpa_tensor_t* dx_b,
                   const sdpa_rowstat_t* dlse_b, void* stream);

/* Context-parallel ring attention, emulated on one GPU ("Add support for cuDNN
 * FusedAttention + THD + CP", TransformerEngine issue 885: each sequence is split into
 * 2*cp chunks, rank r holds chunks r and 2*cp-1-r for load balance, K/V chunk pairs move
 * around a ring, and the ring's result does not depend on the order of its hops).
 *
 * `desc` describes the whole sequence: layout BSHD, SBHD or BHSD (not THD), seqlen_q ==
 * seqlen_k a positive multiple of 2*cp, window (-1,0) (causal) or (-1,-1) (no mask); the
 * other fields and all tensors are exactly those of sdpa_fwd / sdpa_bwd on the whole
 * sequence, and the results equal theirs up to rounding.  cp in [1, 64].  hop_order: NULL
 * (ring order) or a permutation of 0..cp-1; at hop h rank r works on the K/V of rank
 * (r - hop_order[h]) mod cp.
 *
 * Forward: for each rank and each of its q chunks i, every K/V chunk c the hops bring is a
 * pair that is full (c < i), causal with the diagonal at the chunk start (c == i) or
 * skipped (c > i; causal only).  Each pair runs sdpa_fwd on the chunk views and its
 * (O, LSE) is folded into the running result with sdpa_merge_fwd, in hop order.  `lse`
 * must be given.  Backward: every pair runs sdpa_bwd with the final O and LSE of its rows
 * (so its P and Delta equal full attention's); each chunk's diagonal pair writes dq, dk,
 * dv first, every other pair adds to them in hop order.
 * Workspace: sdpa_cp_workspace_size bytes, caller-owned, used by both calls.  Errors:
 * validation of the whole problem runs before any launch; an error from a later launch
 * returns that launch's status (earlier launches of the call may have run). */
int sdpa_cp_workspace_size(const sdpa_desc_t* desc, int cp, size_t* bytes);
int sdpa_cp_fwd(const sdpa_desc_t* desc, int cp, const int32_t* hop_order, const sdpa_tensor_t* q,
                const sdpa_tensor_t* k, const sdpa_tensor_t* v, const sdpa_tensor_t* o,
                const sdpa_rowstat_t* lse, void* workspace, size_t workspace_bytes, void* stream);
int sdpa_cp_bwd(const sdpa_desc_t* desc, int cp, const int32_t* hop_order, const sdpa_tensor_t* q,
                const sdpa_tensor_t* k, const sdpa_tensor_t* v, const sdpa_tensor_t* o,
                const sdpa_rowstat_t* lse, const sdpa_tensor_t* dout, const sdpa_rowstat_t* dlse,
                const sdpa_tensor_t* dq, const sdpa_tensor_t* dk, const sdpa_tensor_t* dv,
                void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SDPA_MI355X_H */
