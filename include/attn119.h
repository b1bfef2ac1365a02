/*
 * attn119 -- fused exact-attention forward pass for AMD Instinct MI355X (gfx950).
 *
 * C ABI of libattn119.so.  Plain pointers and sizes only; every device pointer is
 * memory the caller allocated (hipMalloc or a framework allocator) on the current
 * HIP device.  The library allocates nothing and keeps no state between calls.
 *
 * The operation (pages, cited by title and section):
 *   "FlashAttention 4: Γρηγορότερη και Αποδοτική σε Μνήμη Προσοχή για LLMs"
 *   (el.linux-konsole.com), section "Εισαγωγή": attention multiplies the queries
 *   by the keys, normalises with a softmax, multiplies by the values; section
 *   "Γιατί οι πυρήνες προσοχής ...": the score matrix is processed in tiles on
 *   chip and only a running maximum and sum are kept per query row; section
 *   "Έξυπνος επανακανονισμός Softmax ...": the accumulator is rescaled only when
 *   the running maximum grows by a significant amount.
 *   "PyTorchs FlexAttention mit FlashAttention-4 ist ein Game-Changer" (liora.io),
 *   opening section: the ALiBi, sliding-window, document-mask and soft-capping
 *   variants; section "Aktuelle Einschränkungen": block sparsity.
 *   "FlashAttention-3: Rekordverdächtige Geschwindigkeit und Präzision bei
 *   AI-Modellen" (ctol-digital.de), section "Analyse": FP8 inputs with block
 *   quantisation.
 *
 * For every batch b, head h and query row q (0-based), with s = (Q[q].K[k])*scale:
 *   ATTN_SOFTCAP:  s <- softcap * tanh(s / softcap)          (on the scaled score)
 *   ATTN_ALIBI:    s <- s - slope[h] * |q - k|               (= slope*(k - q) for k <= q)
 *   visible(q,k) = [k <= q if ATTN_CAUSAL] and [|q - k| <= window-1 if ATTN_WINDOW]
 *                  and [doc_id[b][q] == doc_id[b][k] if ATTN_DOCUMENT]
 *   O[q]   = sum_k softmax_k(s) V[k] over visible k          (bf16 output)
 *   LSE[q] = ln sum_k exp(s) over visible k                  (fp32 output)
 * Every valid mask keeps the diagonal, so no row is ever empty.
 *
 * Layouts (all contiguous, row-major, innermost index last):
 *   q, k, v : [B][H][N][d] of bf16, or of OCP E4M3FN bytes (ATTN_FP8_E4M3)
 *   o       : [B][H][N][d] bf16 (round to nearest even)
 *   lse     : [B][H][N] fp32, natural log
 *   doc_id  : [B][N] int32, non-decreasing along N (documents are contiguous runs)
 *   alibi_slopes : [H] fp32, or NULL for 2^(-8(h+1)/H), h = 0..H-1
 *   fp8 scales   : [B][H][ceil(N/128)] fp32; value = code * scale of its 128-row block
 * d must be 64 or 128; any N >= 1 is accepted.  Device pointers must be 16-byte
 * aligned.
 *
 * Errors: every entry point validates its host-visible arguments and returns a
 * negative attn_status *before* launching anything.  Launch failures are reported
 * as ATTN_ERR_HIP.  Faults inside kernels surface at the caller's next
 * synchronisation.  No exception crosses the ABI.  All calls are thread-safe.
 */
#ifndef ATTN119_H_
#define ATTN119_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum attn_status {
  ATTN_OK = 0,
  ATTN_ERR_INVALID_ARG = -1,   /* null pointer, bad size, bad scalar */
  ATTN_ERR_UNSUPPORTED = -2,   /* d not in {64,128}, unknown dtype / flag / pv mode */
  ATTN_ERR_BAD_BLOCKMAP = -3,  /* blockmap missing or of the wrong size for (B, N, mask) */
  ATTN_ERR_HIP = -4,           /* a HIP runtime call or kernel launch failed */
  ATTN_ERR_BAD_DOC_ID = -5     /* doc_id decreases somewhere (attn_blockmap_status) */
} attn_status;

typedef enum attn_dtype { ATTN_BF16 = 0, ATTN_FP8_E4M3 = 1 } attn_dtype;

/* attn_mask.flags bits */
enum {
  ATTN_CAUSAL = 1,
  ATTN_WINDOW = 2,
  ATTN_DOCUMENT = 4,
  ATTN_ALIBI = 8,
  ATTN_SOFTCAP = 16
};

/* attn_fp8.pv_mode */
enum {
  ATTN_PV_F16 = 0,  /* V codes widened exactly to fp16, P (in units of the V block scale over
                       the head's largest V block scale, <= 2^tau) rounded to fp16, fp16 MFMA
                       with fp32 accumulation */
  ATTN_PV_E4M3 = 1, /* P rounded to e4m3 and multiplied with the V codes on the f8f6f4 MFMA
                       (FlashAttention-3's all-FP8 product, "FlashAttention-3: ..." (ctol-
                       digital.de), "Analyse"): a measured mode, its error reported, not
                       gated.  Needs qk_mode ATTN_QK_E4M3, d = 128 and no mask or modifier
                       (else ATTN_ERR_UNSUPPORTED).  O is normalised by the sum of the rounded P */
  ATTN_PV_FP4 = 2   /* P rounded to FP4 (E2M1) with one E8M0 scale per 32 keys of a row (the
                       smallest power of two that holds their largest value without clipping),
                       straight from the exponentials, on the scaled f8f6f4 MFMA with the V
                       codes: the "Direct-P" of "Hardware-Aware FP4 FlashAttention-4"
                       (gist.science) for non-causal inference, a measured mode with the same
                       conditions as ATTN_PV_E4M3 */
};

/* attn_fp8.qk_mode */
enum {
  ATTN_QK_BF16 = 0, /* Q and K codes widened exactly to bf16, bf16 MFMA with fp32 accumulation:
                       scores exact to fp32 rounding (the accurate mode) */
  ATTN_QK_E4M3 = 1  /* Q.K^T on the e4m3 MFMA (twice the bf16 rate), P.V as ATTN_PV_F16.
                       gfx950's f8f6f4 MFMA truncates its 64-term sums at about 2^-14 of the
                       largest product (measured), so a score dominated by a few large
                       products (outlier features) carries an error of that size relative
                       to them: on four x20 channels the LSE error at |LSE| ~ 600 is ~0.07
                       without and ~3e-3 with incoherent processing (attn_fp8_quantize's
                       rotation of Q and K), O within 6e-2 beyond bf16 rounding with it.
                       A measured mode: the accurate one is ATTN_QK_BF16 */
};

/*
 * Mask and score modifiers.  The struct is read during the call only; the device
 * arrays it points to must stay valid until the enqueued work completes.
 *   window : visible keys per query side including itself (>= 1) when ATTN_WINDOW;
 *            with ATTN_CAUSAL exactly `window` keys q-window+1 .. q are visible.
 *   softcap: cap > 0 when ATTN_SOFTCAP.
 */
typedef struct attn_mask {
  uint32_t flags;
  int32_t window;
  float softcap;
  const int32_t* doc_id;     /* device [B][N], required iff ATTN_DOCUMENT */
  const float* alibi_slopes; /* device [H] or NULL (default slopes) */
} attn_mask;

/* FP8 inputs: per (b, h, 128-row block) scales of q, k and v (device, > 0). */
typedef struct attn_fp8 {
  const float* q_scale;
  const float* k_scale;
  const float* v_scale;
  int32_t pv_mode; /* ATTN_PV_* */
  int32_t qk_mode; /* ATTN_QK_* */
} attn_fp8;

/*
 * Block map (block sparsity).  A workspace in caller-owned device memory that
 * classifies every 128-query x 128-key block as EMPTY (0), PARTIAL (1) or FULL (2)
 * and lists the non-empty key blocks of each query block, so that the forward pass
 * never touches an EMPTY block and evaluates the mask only inside PARTIAL ones.
 * Needed whenever flags contain ATTN_CAUSAL, ATTN_WINDOW or ATTN_DOCUMENT.
 *
 * Byte layout (nqb = nkb = ceil(N/128); every section starts 256-byte aligned,
 * offsets as returned by attn_blockmap_layout_of):
 *   header   : attn_blockmap_header
 *   cls      : uint8  [B][nqb][nkb]     block class
 *   counts   : int32  [B][nqb][2]       number of FULL, number of PARTIAL blocks
 *   idx      : int32  [B][nqb][2][nkb]  ascending FULL kb, then -1; ascending PARTIAL kb, then -1
 *   row_lo   : int32  [B][N]            smallest visible key of each query
 *   row_hi   : int32  [B][N]            largest visible key of each query
 *   col_lo   : int32  [B][N]            smallest query that sees each key
 *   col_hi   : int32  [B][N]            largest query that sees each key
 *   pairs    : int64  [B][nqb]          visible (q, k) pairs of each query block
 *   status   : int32  [B][nqb]          1 if doc_id[b] decreases from a row of this block to
 *                                       the next row (packed batches: or the share of the
 *                                       sequence offsets this block checks is out of order),
 *                                       else 0 (a batch row with any 1 is invalid)
 *   order    : int32  [B * nqb]         work order of the forward pass (this library's
 *                                       scheduling choice; it never changes a result): with
 *                                       ATTN_DOCUMENT the entries e = b * nqb + qb sorted by
 *                                       decreasing work order_full_cost * #FULL +
 *                                       order_partial_cost * #PARTIAL (weights in the
 *                                       header), equal work in increasing e; without it the
 *                                       identity 0 .. B*nqb-1
 *
 * The compact form (attn_blockmap_compact_bytes, _layout_of, _build_compact; also the map
 * inside the workspace of a packed batch, attn_varlen_prepare) has header.compact = 1 and
 * the sections above without cls and idx, so that it grows as O(N) rather than
 * O(B N^2 / 128^2) (its layout has cls = idx = 0).  Every call that takes a block map
 * takes either form and tells them apart by the byte count (the general form is always
 * larger).  No kernel needs those two sections: every query row's visible
 * keys form one interval [row_lo, row_hi] whose ends never decrease from row to row (and
 * likewise every key's rows [col_lo, col_hi]), so a query block's non-empty and FULL key
 * blocks follow from the intervals of its first and last rows, and a key block's query
 * blocks from those of its first and last keys.
 */
typedef struct attn_blockmap_header {
  uint32_t magic; /* 0x39313141 */
  int32_t B, N, nqb, nkb;
  uint32_t flags; /* mask flags restricted to CAUSAL|WINDOW|DOCUMENT */
  int32_t window;
  int32_t order_full_cost;    /* work of a FULL key block in the work order */
  int32_t order_partial_cost; /* work of a PARTIAL key block in the work order */
  int32_t compact;            /* 0: the layout above; 1: the compact form (packed batches) */
  int32_t reserved[6];
} attn_blockmap_header;

typedef struct attn_blockmap_layout {
  size_t cls, counts, idx, row_lo, row_hi, col_lo, col_hi, pairs, status, order, total;
} attn_blockmap_layout;

/* Size in bytes of the block-map workspace for (B, N, mask).  Host only. */
attn_status attn_blockmap_bytes(int32_t B, int32_t N, const attn_mask* mask, size_t* bytes);

/* Byte offset of every section of the block-map workspace.  Host only. */
attn_status attn_blockmap_layout_of(int32_t B, int32_t N, attn_blockmap_layout* layout);

/* The same three for the compact form (no cls and idx sections: O(B N) bytes); its
 * sections hold the same values as the general form's. */
attn_status attn_blockmap_compact_bytes(int32_t B, int32_t N, const attn_mask* mask, size_t* bytes);
attn_status attn_blockmap_compact_layout_of(int32_t B, int32_t N, attn_blockmap_layout* layout);
attn_status attn_blockmap_build_compact(int32_t B, int32_t N, const attn_mask* mask, void* map, size_t bytes,
                                        void* stream);

/*
 * Builds the block map for (B, N, mask) into `map` (device, `bytes` bytes, as
 * returned by attn_blockmap_bytes) on `stream` (a hipStream_t; NULL = default
 * stream).  Asynchronous; deterministic; the result is byte-identical for equal
 * inputs.  A decreasing doc_id is recorded in the status section (see
 * attn_blockmap_status) and makes attn_fwd write NaN to O and LSE of the batch row.
 */
attn_status attn_blockmap_build(int32_t B, int32_t N, const attn_mask* mask, void* map, size_t bytes,
                                void* stream);

/*
 * Synchronises `stream`, then reads the map's status section: ATTN_OK or
 * ATTN_ERR_BAD_DOC_ID.  `bytes` is the map's size (attn_blockmap_bytes; for the compact
 * form of a packed batch attn_varlen_layout_of's total, or the whole workspace's
 * attn_varlen_workspace_bytes).
 */
attn_status attn_blockmap_status(const void* map, size_t bytes, void* stream);

/*
 * Host-side validation of an attn_fwd call (no HIP call, usable without a GPU):
 * the same arguments as attn_fwd minus the stream.
 */
attn_status attn_check_args(const void* q, const void* k, const void* v, void* o, float* lse,
                            int32_t B, int32_t H, int32_t N, int32_t d, float scale, int32_t dtype,
                            const attn_mask* mask, const void* blockmap, size_t blockmap_bytes,
                            const attn_fp8* fp8, float rescale_tau);

/*
 * Enqueues the forward pass on `stream` (a hipStream_t; NULL = default stream) and
 * returns after the launch.
 *   scale        : > 0 and finite (typically 1/sqrt(d)).
 *   dtype        : ATTN_BF16 or ATTN_FP8_E4M3 (then `fp8` is required).
 *   mask         : NULL for plain attention.
 *   blockmap     : built by attn_blockmap_build for the same (B, N, mask).  Required
 *                  with DOCUMENT.  With CAUSAL and/or WINDOW alone it may be
 *                  NULL: every row then sees one interval of keys whose ends grow with
 *                  the row, and the kernel derives the same block lists and row
 *                  intervals from the flags (bit-identical results, no map launch).
 *                  Ignored without a positional mask.
 *   rescale_tau  : online-softmax rescale threshold in log2 units, 0 <= tau <= 8:
 *                  the running maximum used as the exponent offset is replaced only
 *                  when a row's maximum exceeds it by more than tau.  The result
 *                  does not depend on tau beyond rounding.
 * Reads q, k, v (and the scales, doc ids, slopes, map); writes every element of
 * o and lse.  Deterministic: equal inputs give bit-identical outputs.
 */
attn_status attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int32_t B,
                     int32_t H, int32_t N, int32_t d, float scale, int32_t dtype, const attn_mask* mask,
                     const void* blockmap, size_t blockmap_bytes, const attn_fp8* fp8,
                     float rescale_tau, void* stream);

/*
 * Grouped-query attention (GQA; MQA with H_kv = 1), the case the page "FlashAttention 4:
 * ... για LLMs" (el.linux-konsole.com) lists among FA4's gaps in its section
 * "Συμβατότητα και τρέχουσα κατάσταση": several query heads share one key/value head.
 * The same pass with H query heads and H_kv key/value heads, H_kv >= 1 dividing H;
 * query head h reads key/value head h / (H / H_kv).
 *   q, o : [B][H][N][d];  lse: [B][H][N];  k, v: [B][H_kv][N][d].
 *   fp8  : q_scale [B][H][ceil(N/128)], k_scale and v_scale [B][H_kv][ceil(N/128)].
 *   alibi_slopes: per query head, [H].
 * attn_check_args / attn_fwd are the case H_kv = H.  Errors: ATTN_ERR_INVALID_ARG when
 * H_kv < 1 or H_kv does not divide H, otherwise as attn_check_args / attn_fwd.
 */
attn_status attn_check_args_gqa(const void* q, const void* k, const void* v, void* o, float* lse,
                                int32_t B, int32_t H, int32_t H_kv, int32_t N, int32_t d, float scale,
                                int32_t dtype, const attn_mask* mask, const void* blockmap,
                                size_t blockmap_bytes, const attn_fp8* fp8, float rescale_tau);
attn_status attn_fwd_gqa(const void* q, const void* k, const void* v, void* o, float* lse, int32_t B,
                         int32_t H, int32_t H_kv, int32_t N, int32_t d, float scale, int32_t dtype,
                         const attn_mask* mask, const void* blockmap, size_t blockmap_bytes,
                         const attn_fp8* fp8, float rescale_tau, void* stream);

/*
 * The forward pass of attn_fwd_gqa that also counts, for every query row, its rescale
 * events: the steps (64 keys each) in which the row's running maximum exceeded the offset
 * in use by more than rescale_tau, so that the offset was replaced and the accumulator
 * rescaled (the first step with a visible key always counts).  The measurement behind the
 * page "FlashAttention 4: ... για LLMs" (el.linux-konsole.com), section "Έξυπνος
 * επανακανονισμός Softmax ...": rescaling only on a significant growth of the maximum
 * makes rescales rare.  The count depends on the kernel's step order (for a query block:
 * its PARTIAL key blocks ascending, then its FULL ones ascending; without a positional
 * mask and N a multiple of 128, all key blocks ascending).
 *   counts: device int32 [B][H][N], 4-byte aligned; every row is written.
 * bf16 inputs only (a separate instantiation of the kernels, so the counter costs the
 * other kernels nothing).  O and LSE are those of attn_fwd_gqa.  Errors as attn_fwd_gqa,
 * plus ATTN_ERR_INVALID_ARG for a null or misaligned counts and ATTN_ERR_UNSUPPORTED for
 * fp8 inputs.
 */
attn_status attn_fwd_rescale_counts(const void* q, const void* k, const void* v, void* o, float* lse,
                                    int32_t* counts, int32_t B, int32_t H, int32_t H_kv, int32_t N, int32_t d,
                                    float scale, int32_t dtype, const attn_mask* mask, const void* blockmap,
                                    size_t blockmap_bytes, const attn_fp8* fp8, float rescale_tau, void* stream);

/*
 * Variable-length batches (varlen): sequences of different lengths packed one after
 * another without padding, the other gap the page "FlashAttention 4: ... για LLMs"
 * (el.linux-konsole.com) names in its section "Συμβατότητα και τρέχουσα κατάσταση".
 * Each sequence attends only to itself, so a packed batch is the pass with B = 1,
 * N = total and the document mask whose documents are the sequences; the mask's
 * other flags (ATTN_CAUSAL, ATTN_WINDOW, ATTN_ALIBI, ATTN_SOFTCAP) act inside each
 * sequence exactly as on a separate batch row (positions are only ever compared
 * within one sequence, and differences of packed positions equal differences of
 * positions in the sequence).  ATTN_DOCUMENT itself is not accepted (INVALID_ARG).
 *   cu_seqlens: device int32 [nseq + 1], non-decreasing, cu_seqlens[0] = 0,
 *               cu_seqlens[nseq] = total; sequence i is tokens cu_seqlens[i] ..
 *               cu_seqlens[i+1]-1 (empty sequences allowed).  An offset array that
 *               breaks this (a decrease, a first entry other than 0, a last entry other
 *               than total) is reported by attn_blockmap_status(workspace,
 *               attn_varlen_workspace_bytes(total, mask)) as ATTN_ERR_BAD_DOC_ID, and O
 *               and LSE are then NaN.
 *   q, o : [H][total][d];  k, v : [H_kv][total][d];  lse : [H][total]   (B = 1 layout)
 *   fp8 scales: q_scale [H][ceil(total/128)], k_scale and v_scale [H_kv][ceil(total/128)],
 *               one scale per 128 tokens of the packed stream.
 *   workspace : caller-owned device memory of attn_varlen_workspace_bytes, 16-byte
 *               aligned: the compact block map of (1, total) (offsets from
 *               attn_varlen_layout_of), then the int32 sequence id of every token at
 *               the layout's total; O(total) bytes.  attn_varlen_prepare fills it once per batch; any number
 *               of attn_fwd_varlen calls (say, one per layer) then read it.
 * Errors as attn_check_args_gqa; a workspace of the wrong size is ATTN_ERR_BAD_BLOCKMAP.
 */
attn_status attn_varlen_workspace_bytes(int32_t total, const attn_mask* mask, size_t* bytes);
/* Byte offsets of the compact block map's sections in the workspace (cls = idx = 0: absent;
 * total: the map's size, where the sequence ids start).  Host only. */
attn_status attn_varlen_layout_of(int32_t total, attn_blockmap_layout* layout);
attn_status attn_varlen_prepare(const int32_t* cu_seqlens, int32_t nseq, int32_t total, const attn_mask* mask,
                                void* workspace, size_t bytes, void* stream);
attn_status attn_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse, int32_t H,
                            int32_t H_kv, int32_t total, int32_t d, float scale, int32_t dtype,
                            const attn_mask* mask, const void* workspace, size_t bytes, const attn_fp8* fp8,
                            float rescale_tau, void* stream);

/*
 * FP8 block quantisation on the device, with optional incoherent processing: the step
 * before an ATTN_FP8_E4M3 call.  The FlashAttention-3 news (ctol-digital.de), section
 * "Analyse", names block quantisation and a processing step against outlier features
 * (read as incoherent processing: Q and K multiplied by one random orthogonal matrix,
 * which keeps Q.K^T).  For every (b, h, 128-row block) of x:
 *   y = x, or with rotate_signs: y = (x * signs) H, H the Sylvester Walsh-Hadamard
 *       matrix of order d, computed in fp32 by the fast transform (strides 1, 2, ...,
 *       d/2), signs[j] = -1 when bit j % 32 of rotate_signs[j / 32] is set, else +1;
 *   s = fp32(max|y| / 448), 1 for an all-zero block;
 *   codes = the OCP e4m3fn value nearest to y / s, ties to even, saturated at +-448
 *       (computed as fp32(y * fp32(448 / max|y|)), with every e4m3 tie that product
 *       comes close to resolved from the exact residual: without rotation the codes
 *       are exactly those of x / s);
 *   scales[b][h][block] = s, or with rotation fp32(s * fp32(1/sqrt(d))) (1 for an
 *       all-zero block), so that code * scale approximates x R with R = D H / sqrt(d)
 *       orthogonal; the fp32 transform rounds, so rotated codes can differ from those of
 *       the exact x R by one step where y / s lies within that rounding of a tie.
 * Give Q and K the same signs (and V none) to keep Q.K^T and the output unchanged.
 *   x      : device bf16 [B][H][N][d];  codes: device uint8 [B][H][N][d];
 *   scales : device fp32 [B][H][ceil(N/128)];  d = 64 or 128;
 *   rotate_signs: HOST array of d/32 words, read during the call, or NULL (no rotation).
 * x and codes 16-byte aligned.  Errors: ATTN_ERR_INVALID_ARG (null or misaligned
 * pointer, B, H or N < 1), ATTN_ERR_UNSUPPORTED (d), ATTN_ERR_HIP (launch).
 */
attn_status attn_fp8_quantize(const void* x, void* codes, float* scales, int32_t B, int32_t H, int32_t N,
                              int32_t d, const uint32_t* rotate_signs, void* stream);

/*
 * Backward pass (bf16): the gradients of L = sum(O * dO) for the same mask, modifiers
 * and grouped heads as the forward call -- the piece the page "FlashAttention 4: ...
 * για LLMs" (el.linux-konsole.com) lists as missing from FA4 in its sections "Κύρια
 * Συμπεράσματα" and "Συμβατότητα και τρέχουσα κατάσταση".  With P = exp(s - LSE):
 *   dV = P^T dO,  dP = dO V^T,  D = rowsum(dO * O),  dS = P * (dP - D),
 *   dR = dS * ds/dr (ds/dr = scale, or scale * (1 - tanh^2) under ATTN_SOFTCAP),
 *   dQ = dR K,  dK = dR^T Q;  dK and dV summed over the query heads sharing them.
 *   q, o, dout, dq : bf16 [B][H][N][d];  k, v, dk, dv : bf16 [B][H_kv][N][d];
 *   lse  : fp32 [B][H][N], the forward call's output for the same q, k, v;
 *   delta: fp32 [B][H][N] caller-owned scratch, overwritten with D;
 *   mask, blockmap: as for the forward call (a document mask needs the block map, in
 *           either form; causal and window masks may pass none: the kernels then take
 *           the key intervals from the flags).
 * Deterministic (no atomics): equal inputs give equal bits.  Errors as attn_check_args_gqa,
 * plus ATTN_ERR_INVALID_ARG for a null or misaligned dout, dq, dk, dv (16 B) or delta (4 B).
 * attn_bwd is the case H_kv = H.
 */
attn_status attn_bwd_gqa(const void* q, const void* k, const void* v, const void* o, const float* lse,
                         const void* dout, void* dq, void* dk, void* dv, float* delta, int32_t B, int32_t H,
                         int32_t H_kv, int32_t N, int32_t d, float scale, const attn_mask* mask,
                         const void* blockmap, size_t blockmap_bytes, void* stream);
attn_status attn_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
                     void* dq, void* dk, void* dv, float* delta, int32_t B, int32_t H, int32_t N, int32_t d,
                     float scale, const attn_mask* mask, const void* blockmap, size_t blockmap_bytes,
                     void* stream);

/*
 * The backward pass of a packed variable-length batch (the gradients of attn_fwd_varlen,
 * bf16 inputs): every sequence attends only to itself, so it is attn_bwd_gqa with B = 1,
 * N = total and the sequences as documents, walking the workspace's compact block map
 * (prepared by attn_varlen_prepare for the same offsets and mask; the backward kernels
 * take every block range from the map's row and column intervals, so the workspace stays
 * O(total)).
 *   q, o, dout, dq : bf16 [H][total][d];  k, v, dk, dv : bf16 [H_kv][total][d];
 *   lse, delta     : fp32 [H][total] (lse from attn_fwd_varlen, delta overwritten with D).
 * Errors as attn_bwd_gqa; a workspace of the wrong size is ATTN_ERR_BAD_BLOCKMAP.
 */
attn_status attn_bwd_varlen(const void* q, const void* k, const void* v, const void* o, const float* lse,
                            const void* dout, void* dq, void* dk, void* dv, float* delta, int32_t H, int32_t H_kv,
                            int32_t total, int32_t d, float scale, const attn_mask* mask, const void* workspace,
                            size_t bytes, void* stream);

/*
 * The backward pass of attn_bwd_gqa without the delta workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the row sums D go to a scratch array inside the library, one per GPU,
 * of at most 4,194,304 rows (16 MiB, held by each GPU the library runs on until the process
 * ends).  This call allocates nothing.  Every call on one GPU shares that GPU's array, so
 * calls that overlap on one GPU (on different streams, or from different threads) race;
 * serialise them.  Arguments, results and errors as attn_bwd_gqa without delta, plus
 * ATTN_ERR_INVALID_ARG when B * H * N exceeds 4,194,304.  dq, dk, dv are bit-identical to
 * attn_bwd_gqa's for the same inputs.
 */
attn_status attn_bwd_gqa_noalloc(const void* q, const void* k, const void* v, const void* o, const float* lse,
                                 const void* dout, void* dq, void* dk, void* dv, int32_t B, int32_t H, int32_t H_kv,
                                 int32_t N, int32_t d, float scale, const attn_mask* mask, const void* blockmap,
                                 size_t blockmap_bytes, void* stream);

/*
 * Name of the compiled kernel variant attn_fwd selects for these arguments, e.g.
 * "bf16 d128 masked softcap" (host logic only, no HIP call, usable without a GPU);
 * NULL when the combination is unsupported.  The string is static.  A "masked"
 * variant reads the block map; it is chosen exactly when the mask has CAUSAL,
 * WINDOW or DOCUMENT.
 */
const char* attn_fwd_kernel_name(int32_t d, int32_t dtype, const attn_mask* mask, const attn_fp8* fp8);

/* Static description of a status code. */
const char* attn_status_str(int32_t status);

#ifdef __cplusplus
}
#endif

#endif /* ATTN119_H_ */
