/*
 * psq.h -- packed-sequence (THD) varlen-attention metadata on MI355X (gfx950).
 *
 * A C ABI over hand-written HIP kernels.  The operations follow the pages'
 * functions one for one:
 *
 *   psq_params_from_doc_ids  document map -> cu_seqlens, max_seqlen
 *       NeMo AutoModel API, nemo_automodel.components.datasets.packed_seq:
 *       packed_seq_params_from_doc_ids and PackedSeqParams.
 *   psq_process_thd          length tables (or a document map) -> THD
 *       metadata, layout padding mask, and the BSHD -> THD collapse copies
 *       NeMo AutoModel 0.5 API, nemo_automodel.components.distributed.
 *       thd_utils: process_input_for_thd and _thd_padding_mask.
 *   psq_split_thd            the same for equal row groups, results stacked
 *       (split_batch_into_thd_chunks, same page).
 *   psq_padding_mask_from_token_ids   the metadata-free padding mask,
 *       which fails when the pad id also occurs among the content ids
 *       (thd_padding_mask_from_token_ids, same page).
 *   psq_pack_rows            the squeeze of padded sources into fixed-capacity
 *       packs, last padded boundary folded to capacity
 *       "Who packs the sequences: the loader, or the trainer?", What the data
 *       looks like at each hop (Trainer packs, Loader packs).
 *   psq_pack_padded_rows     the trainer's squeeze straight from the padded
 *       [N, W] rectangle (same page, Trainer packs).
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Pointers are DEVICE pointers unless a parameter says "host".  The caller
 *    owns and allocates every buffer, including the workspace; the library
 *    allocates nothing and keeps no state between calls (one exception:
 *    psq_params_from_doc_ids_noalloc's per-GPU scratch).
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).  No
 *    call synchronizes: outputs and *status are valid once the stream reaches
 *    the work.  Calls that overlap in time must use distinct workspaces.
 *  - Return value: PSQ_OK, or a PSQ_ERR_* code.  PSQ_ERR_ARG, _OVERFLOW and
 *    _WORKSPACE are found on the host from the arguments alone, before
 *    anything is enqueued.  PSQ_ERR_HIP means the runtime refused a launch;
 *    launches of the same call issued before it may already be enqueued.
 *  - Calls enqueue kernels only (no memset, no allocation), so they may be
 *    captured in a HIP graph and replayed.
 *  - Data-dependent errors (found by the kernels) are bits OR-ed into the
 *    device word *status (0 = success).  Output contents are unspecified
 *    when *status != 0, but every kernel stays inside the buffers described
 *    below whatever the data.
 *  - Workspace: query its size with the matching *_workspace() call; the
 *    pointer must be 16-byte aligned (any device allocation is).  Zero-fill
 *    it once (psq_workspace_init, or any zero fill) before its first use.
 *    Every call leaves the parts it relies on zero-filled again when it
 *    completes, so the zero fill is needed only once per allocation and one
 *    workspace can serve every call on a stream.  (The document-map calls
 *    keep records and state in bytes 256 .. 49664, which no other call
 *    reads; there they leave data that the next document-map call expects.)
 *    A call whose *status holds PSQ_DATA_WORKSPACE may leave records behind
 *    (a bounded wait gave up while other workgroups still ran): zero-fill
 *    the workspace again, after the stream has drained, before reusing it.
 *    A query returns 0 for sizes its call would reject (PSQ_ERR_ARG or
 *    PSQ_ERR_OVERFLOW).
 *  - Grids: one HIP launch runs fewer than 2^32 threads.  Sizes that would
 *    need more in a call's metadata launch are PSQ_ERR_OVERFLOW; the limits
 *    are given with each call and lie far beyond the memory one GPU holds
 *    for any but degenerate shapes (millions of one-token rows, tens of
 *    millions of tiny packs).
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
#define PSQ_ERR_OVERFLOW  2   /* a size does not fit int32 boundaries, or a
                                 call's copies do not fit one launch grid    */
#define PSQ_ERR_WORKSPACE 3   /* workspace missing, smaller than required or
                                 not 16-byte aligned                         */
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
                                        bounded wait or a bound check failed;
                                        for a document map: the map changed
                                        during the call) */
#define PSQ_DATA_PAD_IS_CONTENT 256  /* the pad id occurs before the pad tail */

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
 *   status        int32 scalar, or NULL.  Set to 0: a map has no invalid
 *                 values.  PSQ_DATA_WORKSPACE reports a failed bound check,
 *                 possible only when the map changes during the call.
 *   workspace     device scratch of psq_params_from_doc_ids_workspace(B, S)
 *                 bytes (at most 49664 for any size), 16-byte aligned,
 *                 zero-filled once like every workspace.
 * Each workgroup reduces a chunk (or a range of chunks) to a record
 * (boundary count, first and last boundary, longest inner segment) and
 * starts its boundaries at the sum of the counts before it.  A map of at
 * most 4096 positions is one workgroup.  Maps of up to 2^22 positions take
 * one launch over at most 256 chunks of 1024 to 16384 positions (the
 * smallest that fits), each workgroup reading the earlier workgroups'
 * records as they are published; larger maps take two launches over chunks
 * of 4096 (records, then boundaries).
 * Host errors: PSQ_ERR_ARG (null pointer, B or S < 0, bad dtype),
 * PSQ_ERR_OVERFLOW (B*S >= 2^31), PSQ_ERR_WORKSPACE.
 * ---------------------------------------------------------------------- */
size_t psq_params_from_doc_ids_workspace(int64_t B, int64_t S);
int psq_params_from_doc_ids(const void *doc_ids, int doc_dtype, int64_t B, int64_t S,
                            int32_t *cu_seqlens, int32_t *num_segments,
                            int32_t *max_seqlen, uint8_t *padding_mask,
                            int32_t *status, void *workspace, size_t workspace_bytes,
                            void *stream);

/* ------------------------------------------------------------------------
 * psq_params_from_doc_ids_noalloc
 *
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  The same
 * operation, arguments and outputs as psq_params_from_doc_ids, without the
 * workspace: the library uses its own file-scope device scratch of
 * PSQ_NOALLOC_SCRATCH_BYTES bytes instead, one copy per GPU, held until the
 * process ends.  The current device's copy is used (hipGetDevice), so
 * `stream` must belong to the current device.  The call allocates nothing;
 * its first call on a device also enqueues one fill kernel on `stream` that
 * zero-fills that device's scratch.  Every size psq_params_from_doc_ids
 * accepts fits the scratch (the largest document-map workspace); a larger
 * need would return PSQ_ERR_OVERFLOW.  Each call leaves the scratch ready
 * for the next one.  Calls that overlap in time on one GPU (several streams
 * or host threads) share the scratch and race: order them on one stream.
 * The caller cannot zero-fill the scratch again: should a call report
 * PSQ_DATA_WORKSPACE from a bounded wait that gave up (a dispatched
 * workgroup made no progress for seconds), stop using this call on that GPU
 * and use psq_params_from_doc_ids with a freshly zero-filled workspace.
 * Host errors: as psq_params_from_doc_ids (without PSQ_ERR_WORKSPACE), and
 * PSQ_ERR_HIP when the scratch's device address cannot be looked up.
 * ---------------------------------------------------------------------- */
#define PSQ_NOALLOC_SCRATCH_BYTES 49664
int psq_params_from_doc_ids_noalloc(const void *doc_ids, int doc_dtype, int64_t B, int64_t S,
                                    int32_t *cu_seqlens, int32_t *num_segments,
                                    int32_t *max_seqlen, uint8_t *padding_mask,
                                    int32_t *status, void *stream);

/* One byte copy of the BSHD -> THD collapse: `rows` rows of `row_bytes`
 * bytes, read at a stride of src_row_stride_bytes and written at a stride of
 * dst_row_stride_bytes (0 = row_bytes, i.e. densely).  A contiguous tensor
 * is one row (or rows with both strides == row_bytes).  Strides are at least
 * row_bytes; src and dst must not overlap (checked over their whole spans).
 * The copies of one call run concurrently with each other and with the
 * call's metadata work: the bytes a copy writes must not be read or written
 * by another copy or be any other buffer of the call (not checked; several
 * copies may write interleaved rows of one buffer, and read one source). */
typedef struct psq_copy {
    const void *src;
    void *dst;
    int64_t rows;
    int64_t row_bytes;
    int64_t src_row_stride_bytes;
    int64_t dst_row_stride_bytes;
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
 * n_copies out of range, a copy with a null pointer, a stride below its row
 * or overlapping src/dst), PSQ_ERR_OVERFLOW (B*S or B*P+1 >= 2^31, copies
 * of 2^31 units of one size or more, or, for the table layout above 4096
 * table entries, 256 * B * ceil(S / 4096) threads plus the copy units of
 * 16 bytes reaching 2^32), PSQ_ERR_WORKSPACE.
 * ---------------------------------------------------------------------- */
size_t psq_process_thd_workspace(const psq_thd_layout *layout, int64_t B, int64_t S);
int psq_process_thd(const psq_thd_layout *layout, int64_t B, int64_t S,
                    int32_t *cu_seqlens, int32_t *cu_seqlens_padded,
                    int32_t *num_seqs, int32_t *max_seqlen, int32_t *pad_between_seqs,
                    uint8_t *padding_mask, const psq_copy *copies, int n_copies,
                    int32_t *status, void *workspace, size_t workspace_bytes,
                    void *stream);

/* ------------------------------------------------------------------------
 * psq_split_thd
 *
 * NeMo AutoModel 0.5 API, thd_utils: split_batch_into_thd_chunks.  The B rows
 * are cut into num_chunks equal groups of Bc = B / num_chunks consecutive
 * rows; each group is one psq_process_thd call on a batch of Bc rows (its own
 * boundaries starting at 0, its own absorption, scalars and mask), and the
 * results are stacked.  Table layout only (PSQ_LAYOUT_SEQ_LENS).
 *
 *   cu_seqlens        int32, capacity num_chunks * (Bc*P+1).  On completion
 *                     the first num_chunks * L entries hold a row-major
 *                     [num_chunks, L] array, L = *cu_width = the longest
 *                     group's n+1; a shorter group's row is filled up to L
 *                     with layout->pad_value.
 *   cu_seqlens_padded the same for the physical boundaries, or NULL.
 *   cu_width          int32 scalar L (0 when *status != 0).
 *   num_seqs, max_seqlen, pad_between_seqs   int32 [num_chunks].
 *   padding_mask      uint8 [B*S] (= [num_chunks, Bc*S]), or NULL.
 *   copies            as in psq_process_thd; a [B,S,...] tensor stacked per
 *                     group is the same bytes as its flattening, and the
 *                     destination row stride of a copy allows the mRoPE
 *                     [n, B, S] -> [num_chunks, n, 1, Bc*S] reordering.
 *   status            int32 scalar, required (OR over the groups).
 *   workspace         psq_split_thd_workspace(layout, B, S, num_chunks) bytes.
 * Host errors: as psq_process_thd, plus PSQ_ERR_ARG when num_chunks < 1,
 * num_chunks does not divide B, the layout is not a table layout, or
 * pad_value does not fit int32 (it fills int32 rows).
 * ---------------------------------------------------------------------- */
size_t psq_split_thd_workspace(const psq_thd_layout *layout, int64_t B, int64_t S,
                               int64_t num_chunks);
int psq_split_thd(const psq_thd_layout *layout, int64_t B, int64_t S, int64_t num_chunks,
                  int32_t *cu_seqlens, int32_t *cu_seqlens_padded, int32_t *cu_width,
                  int32_t *num_seqs, int32_t *max_seqlen, int32_t *pad_between_seqs,
                  uint8_t *padding_mask, const psq_copy *copies, int n_copies,
                  int32_t *status, void *workspace, size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------------
 * psq_padding_mask_from_token_ids
 *
 * NeMo AutoModel 0.5 API, thd_utils: thd_padding_mask_from_token_ids, for
 * callers without pack metadata.  padding_mask[t] = (input_ids[t] == pad_id).
 * That comparison is a correct mask only when the pad slots form a right-
 * padded tail, so the call checks exactly that and sets
 * PSQ_DATA_PAD_IS_CONTENT in *status when some pad slot comes before a
 * non-pad slot (the pad id then also stands for content tokens).
 *
 *   input_ids     [T], element type ids_dtype (PSQ_I32 or PSQ_I64).  With
 *                 int32 ids, a pad_id outside the int32 range matches none.
 *   padding_mask  uint8 [T], required.
 *   num_content   int32 scalar: index of the first pad slot (T when there is
 *                 none), i.e. the content length; or NULL.
 *   status        int32 scalar, required.
 *   workspace     psq_padding_mask_from_token_ids_workspace(T) bytes.
 * Host errors: PSQ_ERR_ARG (null pointer, T < 0, bad dtype),
 * PSQ_ERR_OVERFLOW (T >= 2^31), PSQ_ERR_WORKSPACE.
 * ---------------------------------------------------------------------- */
size_t psq_padding_mask_from_token_ids_workspace(int64_t T);
int psq_padding_mask_from_token_ids(const void *input_ids, int ids_dtype, int64_t T,
                                    int64_t pad_id, uint8_t *padding_mask,
                                    int32_t *num_content, int32_t *status, void *workspace,
                                    size_t workspace_bytes, void *stream);

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
 * src_tokens), BAD_LENGTH (real_len < 0).  With pack_order, the members
 * are pack_start[P] entries of it and the CSR holds pack_start[P] + P.
 * Host errors: PSQ_ERR_ARG (null pointer, negative size, pad_to < 1,
 * capacity < 1 or > 2^30), PSQ_ERR_OVERFLOW (N+P >= 2^31, or
 * P * ceil(capacity / 896) >= 2^26 workgroups of 64 threads),
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

/* ------------------------------------------------------------------------
 * psq_pack_padded_rows
 *
 * "Who packs the sequences: the loader, or the trainer?", Trainer packs: the
 * batch reaches the worker as a padded rectangle input_ids [N, W] with
 * input_lengths, the bins are chosen on the host, and the squeeze lays each
 * bin's rows end to end.  Exactly psq_pack_rows with source i = row i
 * (offset i*W); the row width of the output (`capacity`) is the caller's,
 * the trainer taking the widest bin's padded sum, with fold = 0.
 *
 *   rows           int64 [N, W] row-major.       real_len int32 [N].
 *   pack_order     int32 [N] or NULL.            pack_start int64 [P+1].
 *   packed, token_mask, cu_seqlens, cu_seqlens_padded, status   as in
 *                  psq_pack_rows.
 *   workspace      psq_pack_rows_workspace(N, P, capacity) bytes.
 * Data errors: as psq_pack_rows; BAD_LENGTH also for a member whose length
 * exceeds W (such a member counts as empty toward its pack's fill).
 * Host errors: as psq_pack_rows, plus PSQ_ERR_ARG for W < 0 and
 * PSQ_ERR_OVERFLOW when N*W >= 2^62.
 * ---------------------------------------------------------------------- */
int psq_pack_padded_rows(const int64_t *rows, int64_t W, const int32_t *real_len, int64_t N,
                         int32_t pad_to, const int32_t *pack_order, const int64_t *pack_start,
                         int64_t P, int32_t capacity, int fold, int64_t pad_token,
                         int64_t *packed, uint8_t *token_mask, int32_t *cu_seqlens,
                         int32_t *cu_seqlens_padded, int32_t *status, void *workspace,
                         size_t workspace_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* PSQ_H */
