/*
 * psq.h -- packed-sequence (THD) varlen-attention metadata on MI355X (gfx950).
 *
 * A C ABI over hand-written HIP kernels.  Three operations, one per page of
 * the method:
 *
 *   psq_params_from_doc_ids  document map -> cu_seqlens, max_seqlen
 *       NeMo AutoModel API, nemo_automodel.components.datasets.packed_seq:
 *       packed_seq_params_from_doc_ids and PackedSeqParams.
 *   psq_process_thd          length tables (or a document map) -> THD
 *       metadata, layout padding mask, and the BSHD -> THD collapse copies
 *       NeMo AutoModel 0.5 API, nemo_automodel.components.distributed.
 *       thd_utils: process_input_for_thd and _thd_padding_mask.
 *   psq_pack_rows            the squeeze of padded sources into fixed-capacity
 *       packs, last padded boundary folded to capacity
 *       "Who packs the sequences: the loader, or the trainer?", What the data
 *       looks like at each hop (Trainer packs, Loader packs).
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Pointers are DEVICE pointers unless a parameter says "host".  The caller
 *    owns and allocates every buffer, including the workspace; the library
 *    allocates nothing and keeps no state between calls.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).  No
 *    call synchronizes: outputs and *status are valid once the stream reaches
 *    the work.  Calls that overlap in time must use distinct workspaces.
 *  - Return value: PSQ_OK, or a PSQ_ERR_* code for errors found on the host
 *    from the arguments alone.  Nothing is enqueued when an error is returned.
 *  - Data-dependent errors (found by the kernels) are bits OR-ed into the
 *    device word *status (0 = success).  Output contents are unspecified
 *    when *status != 0, but every kernel stays inside the buffers described
 *    below whatever the data.
 *  - Workspace: query its size with the matching *_workspace() call, then
 *    zero-fill it once (psq_workspace_init, or any zero fill) before its
 *    first use.  Every call leaves the workspace zero-filled again when it
 *    completes, so the zero fill is needed only once per allocation.
 *  - Boundary arrays (cu_seqlens*) are int32; entries past the valid count
 *    are left unspecified.  Masks are uint8 0/1 (byte-identical to a torch
 *    bool tensor).
 */
#ifndef PSQ_H
#define PSQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* element types of integer inputs */
#define PSQ_I32 0
#define PSQ_I64 1

/* host-side return codes */
#define PSQ_OK            0
#define PSQ_ERR_ARG       1   /* null required pointer, bad enum, bad size   */
#define PSQ_ERR_OVERFLOW  2   /* a size does not fit int32 boundaries        */
#define PSQ_ERR_WORKSPACE 3   /* workspace missing or smaller than required  */
#define PSQ_ERR_HIP       4   /* the HIP runtime refused a launch            */

/* data-dependent status bits (device word *status) */
#define PSQ_DATA_BAD_LENGTH      1   /* negative length, or real > padded     */
#define PSQ_DATA_TABLE_MISMATCH  2   /* sentinel slots differ between tables  */
#define PSQ_DATA_ROW_OVERFLOW    4   /* a row's padded lengths exceed S       */
#define PSQ_DATA_EMPTY_ROW       8   /* a row holds no sequence               */
#define PSQ_DATA_PACK_OVERFLOW  16   /* a pack's padded sources exceed it     */
#define PSQ_DATA_EMPTY_PACK     32   /* a pack has no member                  */
#define PSQ_DATA_BAD_INDEX      64   /* member, pack or source out of range   */
#define PSQ_DATA_WORKSPACE     128   /* workspace was not zero-filled (a
                                        bounded wait or a bound check failed) */

/* layouts accepted by psq_process_thd */
#define PSQ_LAYOUT_SEQ_LENS 0
#define PSQ_LAYOUT_DOC_IDS  1

/* maximum number of copies one psq_process_thd call carries */
#define PSQ_MAX_COPIES 8

/* Text for a host return code (PSQ_ERR_*) or, with is_status != 0, for a
 * set of data status bits.  The string is static; never free it. */
const char *psq_status_string(int code, int is_status);

/* Zero-fill a workspace of `bytes` bytes on `stream` (a fill kernel, so it
 * may be recorded into a HIP graph).  Returns PSQ_OK or PSQ_ERR_*. */
int psq_workspace_init(void *workspace, size_t bytes, void *stream);

/* ------------------------------------------------------------------------
 * psq_params_from_doc_ids
 *
 * NeMo AutoModel API, packed_seq: packed_seq_params_from_doc_ids.  Segments
 * are the maximal runs of one document index inside a row; a segment always
 * starts at a row start; runs of the padding index 0 are segments too, so
 * the segments tile the flattened B*S axis.
 *
 *   doc_ids       [B, S] row-major, element type doc_dtype (PSQ_I32/PSQ_I64).
 *                 Values are only compared; 0 marks padding for the mask.
 *   cu_seqlens    int32, capacity B*S+1.  On completion cu_seqlens[0..n]
 *                 holds the segment starts followed by B*S.
 *   num_segments  int32 scalar n.
 *   max_seqlen    int32 scalar: the longest segment (padding runs count).
 *   padding_mask  uint8 [B*S] (1 where doc_ids == 0), or NULL to skip it.
 *   status        int32 scalar (only PSQ_DATA_WORKSPACE can occur), or NULL.
 *   workspace     device scratch of psq_params_from_doc_ids_workspace(B, S)
 *                 bytes, zero-filled before first use.
 * Host errors: PSQ_ERR_ARG (null pointer, B or S < 0, bad dtype),
 * PSQ_ERR_OVERFLOW (B*S >= 2^31), PSQ_ERR_WORKSPACE.
 * ---------------------------------------------------------------------- */
size_t psq_params_from_doc_ids_workspace(int64_t B, int64_t S);
int psq_params_from_doc_ids(const void *doc_ids, int doc_dtype, int64_t B, int64_t S,
                            int32_t *cu_seqlens, int32_t *num_segments,
                            int32_t *max_seqlen, uint8_t *padding_mask,
                            int32_t *status, void *workspace, size_t workspace_bytes,
                            void *stream);

/* One byte copy of the BSHD -> THD collapse: `rows` rows of `row_bytes`
 * bytes, read at a stride of src_row_stride_bytes, written densely.  A
 * contiguous tensor is one row (or rows with stride == row_bytes).  src and
 * dst must not overlap. */
typedef struct psq_copy {
    const void *src;
    void *dst;
    int64_t rows;
    int64_t row_bytes;
    int64_t src_row_stride_bytes;
} psq_copy;

/* Where the THD layout comes from (host struct). */
typedef struct psq_thd_layout {
    int kind;                     /* PSQ_LAYOUT_SEQ_LENS or PSQ_LAYOUT_DOC_IDS  */
    /* PSQ_LAYOUT_SEQ_LENS */
    const void *seq_lens;         /* [B, P] real lengths, lens_dtype           */
    const void *seq_lens_padded;  /* [B, P] reserved slot counts, or NULL      */
    int lens_dtype;               /* PSQ_I32 or PSQ_I64                        */
    int64_t P;                    /* table width (max sequences per row)       */
    int64_t pad_value;            /* unused-slot sentinel (the pages: -1000)   */
    /* PSQ_LAYOUT_DOC_IDS */
    const void *doc_ids;          /* [B, S] document map, doc_dtype            */
    int doc_dtype;
} psq_thd_layout;

/* ------------------------------------------------------------------------
 * psq_process_thd
 *
 * NeMo AutoModel 0.5 API, thd_utils: process_input_for_thd with
 * _thd_padding_mask.  Table layout (PSQ_LAYOUT_SEQ_LENS): entries equal to
 * pad_value are dropped; the remaining sequences, in row-major order, give
 *   cu_seqlens        = [0] + cumsum(real)                  (attention)
 *   cu_seqlens_padded = [0] + cumsum(padded')               (physical)
 * where padded' is the padded length, except that each row's trailing pad
 * (S minus the row's padded sum) is folded into the row's last sequence so
 * that row r's physical boundaries end at (r+1)*S.  Without seq_lens_padded,
 * padded = real.  padding_mask[t] = 1 unless t lies in the first real_i slots
 * of sequence i's physical range.  Trailing-pad absorption (one context-
 * parallel rank): when every interior entry of cu_seqlens equals the
 * physical one and cu_seqlens[n] < B*S, cu_seqlens[n] becomes B*S.  Then
 * pad_between_seqs = (cu_seqlens != cu_seqlens_padded anywhere) and
 * max_seqlen = max_i(cu_seqlens[i+1] - cu_seqlens[i]), after absorption.
 * Document-map layout (PSQ_LAYOUT_DOC_IDS): cu_seqlens and max_seqlen as in
 * psq_params_from_doc_ids, cu_seqlens_padded = cu_seqlens,
 * pad_between_seqs = 0, padding_mask = (doc_ids == 0).
 *
 *   layout            host struct above.  Tables must be [B, P] row-major.
 *   cu_seqlens        int32, capacity B*P+1 (doc map: B*S+1).
 *   cu_seqlens_padded int32, same capacity, or NULL.
 *   num_seqs, max_seqlen, pad_between_seqs   int32 scalars.
 *   padding_mask      uint8 [B*S], or NULL.
 *   copies            host array of n_copies (<= PSQ_MAX_COPIES) collapses.
 *   status            int32 scalar, required (data errors above).
 *   workspace         psq_process_thd_workspace(layout, B, S) bytes.
 * Host errors: PSQ_ERR_ARG (null pointer, negative size, bad kind/dtype,
 * n_copies out of range, a copy with a null pointer or overlapping src/dst),
 * PSQ_ERR_OVERFLOW (B*S or B*P+1 >= 2^31), PSQ_ERR_WORKSPACE.
 * ---------------------------------------------------------------------- */
size_t psq_process_thd_workspace(const psq_thd_layout *layout, int64_t B, int64_t S);
int psq_process_thd(const psq_thd_layout *layout, int64_t B, int64_t S,
                    int32_t *cu_seqlens, int32_t *cu_seqlens_padded,
                    int32_t *num_seqs, int32_t *max_seqlen, int32_t *pad_between_seqs,
                    uint8_t *padding_mask, const psq_copy *copies, int n_copies,
                    int32_t *status, void *workspace, size_t workspace_bytes,
                    void *stream);

/* ------------------------------------------------------------------------
 * psq_pack_rows
 *
 * "Who packs the sequences: the loader, or the trainer?", Trainer packs and
 * Loader packs.  Source i is src_tokens[src_offsets[i] .. +real_len[i]).
 * Its padded length is ceil(real_len[i] / pad_to) * pad_to.  The members of
 * pack p are pack_order[pack_start[p] .. pack_start[p+1]) (or those indices
 * themselves when pack_order is NULL); they are laid end to end at their
 * padded lengths in row p of `packed`, every other slot of the row holds
 * pad_token, and token_mask is 1 exactly on the real tokens.  Per pack,
 *   cu_seqlens        = [0] + cumsum(real)
 *   cu_seqlens_padded = [0] + cumsum(padded), whose last entry becomes
 *                       `capacity` when fold != 0 (the loader's shape).
 * Both are stored as one flat CSR array: pack p's k_p+1 entries start at
 * index pack_start[p] + p (total pack_start[P] + P entries).
 *
 *   src_tokens     int64 [src_len].
 *   src_offsets    int64 [N] element offsets.   real_len  int32 [N].
 *   pack_order     int32 [N] or NULL.           pack_start int64 [P+1].
 *   packed         int64 [P, capacity].         token_mask uint8 [P, capacity].
 *   cu_seqlens, cu_seqlens_padded   int32, capacity N+P.
 *   status         int32 scalar, required.
 *   workspace      psq_pack_rows_workspace(N, P, capacity) bytes.
 * Data errors: PACK_OVERFLOW, EMPTY_PACK, BAD_INDEX (pack_start outside
 * [0, N] or decreasing, a member index outside [0, N), a source outside
 * src_tokens), BAD_LENGTH (real_len < 0).
 * Host errors: PSQ_ERR_ARG (null pointer, negative size, pad_to < 1,
 * capacity < 1 or > 2^30), PSQ_ERR_OVERFLOW (N+P >= 2^31),
 * PSQ_ERR_WORKSPACE.
 * ---------------------------------------------------------------------- */
size_t psq_pack_rows_workspace(int64_t N, int64_t P, int32_t capacity);
int psq_pack_rows(const int64_t *src_tokens, int64_t src_len, const int64_t *src_offsets,
                  const int32_t *real_len, int64_t N, int32_t pad_to,
                  const int32_t *pack_order, const int64_t *pack_start, int64_t P,
                  int32_t capacity, int fold, int64_t pad_token,
                  int64_t *packed, uint8_t *token_mask,
                  int32_t *cu_seqlens, int32_t *cu_seqlens_padded, int32_t *status,
                  void *workspace, size_t workspace_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* PSQ_H */
