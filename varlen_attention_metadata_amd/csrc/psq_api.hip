// psq_api.hip -- the C ABI declared in include/psq.h: host-side argument
// validation, workspace sizing and kernel dispatch.  Every check here runs
// before the first HIP call, so a rejected call enqueues nothing.
#include <string.h>

#include <algorithm>

#include "psq.h"
#include "psq_copy.hpp"
#include "psq_internal.hpp"

namespace {

constexpr int64_t kI32Limit = (int64_t)1 << 31;

bool valid_dtype(int d) { return d == PSQ_I32 || d == PSQ_I64; }

bool overlaps(const void *a, int64_t na, const void *b, int64_t nb) {
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return na > 0 && nb > 0 && x < y + (uintptr_t)nb && y < x + (uintptr_t)na;
}

int check_copies(const psq_copy *copies, int n_copies) {
    if (n_copies < 0 || n_copies > PSQ_MAX_COPIES) return PSQ_ERR_ARG;
    if (n_copies > 0 && copies == nullptr) return PSQ_ERR_ARG;
    for (int i = 0; i < n_copies; ++i) {
        const psq_copy &c = copies[i];
        if (c.rows < 0 || c.row_bytes < 0) return PSQ_ERR_ARG;
        if (c.rows == 0 || c.row_bytes == 0) continue;
        if (c.src == nullptr || c.dst == nullptr) return PSQ_ERR_ARG;
        if (c.rows > 1 && c.src_row_stride_bytes < c.row_bytes) return PSQ_ERR_ARG;
        if (c.dst_row_stride_bytes < 0 ||
            (c.rows > 1 && c.dst_row_stride_bytes != 0 && c.dst_row_stride_bytes < c.row_bytes))
            return PSQ_ERR_ARG;
        const int64_t dst_stride = c.dst_row_stride_bytes ? c.dst_row_stride_bytes : c.row_bytes;
        const int64_t widest = std::max(std::max(dst_stride, c.src_row_stride_bytes), c.row_bytes);
        if (c.rows > (INT64_MAX - c.row_bytes) / widest) return PSQ_ERR_OVERFLOW;
        const int64_t dst_span = (c.rows - 1) * dst_stride + c.row_bytes;
        const int64_t src_span = (c.rows - 1) * c.src_row_stride_bytes + c.row_bytes;
        if (overlaps(c.src, src_span, c.dst, dst_span)) return PSQ_ERR_ARG;
    }
    if (!psq::copies_fit(copies, n_copies)) return PSQ_ERR_OVERFLOW;
    return PSQ_OK;
}

int from_hip(hipError_t e) { return e == hipSuccess ? PSQ_OK : PSQ_ERR_HIP; }

// A workspace is usable when present, large enough and 16-byte aligned (its
// records are read as 16-byte vectors, its counters as 64-bit atomics).
bool workspace_ok(const void *workspace, size_t bytes, size_t need) {
    return workspace != nullptr && bytes >= need && ((uintptr_t)workspace % 16) == 0;
}

}  // namespace

extern "C" {

const char *psq_status_string(int code, int is_status) {
    if (!is_status) {
        switch (code) {
            case PSQ_OK: return "ok";
            case PSQ_ERR_ARG: return "invalid argument (null pointer, negative size, bad enum)";
            case PSQ_ERR_OVERFLOW: return "size does not fit int32 boundary arrays";
            case PSQ_ERR_WORKSPACE: return "workspace missing, too small or not 16-byte aligned";
            case PSQ_ERR_HIP: return "HIP runtime error while enqueuing";
            default: return "unknown error code";
        }
    }
    // data status bits: name the lowest set bit (callers see all bits too)
    if (code == 0) return "ok";
    if (code & PSQ_DATA_BAD_LENGTH) return "negative length, or real length above padded length";
    if (code & PSQ_DATA_TABLE_MISMATCH) return "seq_lens and seq_lens_padded mark different unused slots";
    if (code & PSQ_DATA_ROW_OVERFLOW) return "a row's padded lengths exceed the row length";
    if (code & PSQ_DATA_EMPTY_ROW) return "a row holds no sequence";
    if (code & PSQ_DATA_PACK_OVERFLOW) return "a pack's padded sources exceed its capacity";
    if (code & PSQ_DATA_EMPTY_PACK) return "a pack has no member";
    if (code & PSQ_DATA_BAD_INDEX) return "member, pack or source index out of range";
    if (code & PSQ_DATA_WORKSPACE) return "workspace was not zero-filled before use";
    if (code & PSQ_DATA_PAD_IS_CONTENT)
        return "the pad id appears among the content tokens (its slots do not form one run "
               "ending the stream)";
    return "unknown status bits";
}

int psq_workspace_init(void *workspace, size_t bytes, void *stream) {
    if (bytes > 0 && workspace == nullptr) return PSQ_ERR_ARG;
    return from_hip(psq::launch_zero_fill(workspace, bytes, (hipStream_t)stream));
}

size_t psq_params_from_doc_ids_workspace(int64_t B, int64_t S) {
    if (B < 0 || S < 0) return 0;
    if (S > 0 && B > (kI32Limit - 1) / S) return 0;
    return psq::doc_segments_workspace(B, S);
}

int psq_params_from_doc_ids(const void *doc_ids, int doc_dtype, int64_t B, int64_t S,
                            int32_t *cu_seqlens, int32_t *num_segments, int32_t *max_seqlen,
                            uint8_t *padding_mask, int32_t *status, void *workspace,
                            size_t workspace_bytes, void *stream) {
    if (B < 0 || S < 0 || !valid_dtype(doc_dtype)) return PSQ_ERR_ARG;
    if (S > 0 && B > (kI32Limit - 1) / S) return PSQ_ERR_OVERFLOW;
    if (cu_seqlens == nullptr || num_segments == nullptr || max_seqlen == nullptr)
        return PSQ_ERR_ARG;
    if (B * S > 0 && doc_ids == nullptr) return PSQ_ERR_ARG;
    if (!workspace_ok(workspace, workspace_bytes, psq::doc_segments_workspace(B, S)))
        return PSQ_ERR_WORKSPACE;
    return from_hip(psq::launch_doc_segments(doc_ids, doc_dtype, B, S, cu_seqlens, nullptr,
                                             num_segments, max_seqlen, padding_mask, status,
                                             nullptr, workspace, nullptr, 0,
                                             (hipStream_t)stream));
}

size_t psq_process_thd_workspace(const psq_thd_layout *layout, int64_t B, int64_t S) {
    if (layout == nullptr || B < 0 || S < 0) return 0;
    if (S > 0 && B > (kI32Limit - 1) / S) return 0;
    if (layout->kind == PSQ_LAYOUT_DOC_IDS) return psq::doc_segments_workspace(B, S);
    if (layout->kind != PSQ_LAYOUT_SEQ_LENS || layout->P < 0) return 0;
    if (layout->P > 0 && B > (kI32Limit - 2) / layout->P) return 0;
    return psq::thd_tables_workspace(B, layout->P, 1);
}

int psq_process_thd(const psq_thd_layout *layout, int64_t B, int64_t S, int32_t *cu_seqlens,
                    int32_t *cu_seqlens_padded, int32_t *num_seqs, int32_t *max_seqlen,
                    int32_t *pad_between_seqs, uint8_t *padding_mask, const psq_copy *copies,
                    int n_copies, int32_t *status, void *workspace, size_t workspace_bytes,
                    void *stream) {
    if (layout == nullptr || B < 0 || S < 0) return PSQ_ERR_ARG;
    if (S > 0 && B > (kI32Limit - 1) / S) return PSQ_ERR_OVERFLOW;
    if (cu_seqlens == nullptr || num_seqs == nullptr || max_seqlen == nullptr ||
        pad_between_seqs == nullptr || status == nullptr)
        return PSQ_ERR_ARG;
    const int cc = check_copies(copies, n_copies);
    if (cc != PSQ_OK) return cc;
    const hipStream_t st = (hipStream_t)stream;

    if (layout->kind == PSQ_LAYOUT_DOC_IDS) {
        if (!valid_dtype(layout->doc_dtype)) return PSQ_ERR_ARG;
        if (B * S > 0 && layout->doc_ids == nullptr) return PSQ_ERR_ARG;
        if (!workspace_ok(workspace, workspace_bytes, psq::doc_segments_workspace(B, S)))
            return PSQ_ERR_WORKSPACE;
        return from_hip(psq::launch_doc_segments(layout->doc_ids, layout->doc_dtype, B, S,
                                                 cu_seqlens, cu_seqlens_padded, num_seqs,
                                                 max_seqlen, padding_mask, status,
                                                 pad_between_seqs, workspace, copies,
                                                 n_copies, st));
    }
    if (layout->kind != PSQ_LAYOUT_SEQ_LENS) return PSQ_ERR_ARG;
    if (!valid_dtype(layout->lens_dtype) || layout->P < 0) return PSQ_ERR_ARG;
    // bound B*P before forming it: with S = 0 the row-length check leaves B unbounded
    if (layout->P > 0 && B > (kI32Limit - 2) / layout->P) return PSQ_ERR_OVERFLOW;
    if (B * layout->P > 0 && layout->seq_lens == nullptr) return PSQ_ERR_ARG;
    if (!psq::thd_tables_grid_fits(B, layout->P, S, 1, copies, n_copies))
        return PSQ_ERR_OVERFLOW;
    if (!workspace_ok(workspace, workspace_bytes, psq::thd_tables_workspace(B, layout->P, 1)))
        return PSQ_ERR_WORKSPACE;
    return from_hip(psq::launch_thd_tables(layout->seq_lens, layout->seq_lens_padded,
                                           layout->lens_dtype, B, layout->P, S, 1,
                                           layout->pad_value, cu_seqlens, cu_seqlens_padded,
                                           num_seqs, max_seqlen, pad_between_seqs, nullptr,
                                           padding_mask, status, workspace, copies, n_copies,
                                           st));
}

size_t psq_split_thd_workspace(const psq_thd_layout *layout, int64_t B, int64_t S,
                               int64_t num_chunks) {
    if (layout == nullptr || B < 0 || S < 0 || num_chunks < 1 || B % num_chunks != 0 ||
        layout->kind != PSQ_LAYOUT_SEQ_LENS || layout->P < 0)
        return 0;
    if (S > 0 && B > (kI32Limit - 1) / S) return 0;
    if (num_chunks > kI32Limit) return 0;
    if (layout->P > 0 && B > (kI32Limit - 2 - num_chunks) / layout->P) return 0;
    return psq::thd_tables_workspace(B, layout->P, num_chunks);
}

int psq_split_thd(const psq_thd_layout *layout, int64_t B, int64_t S, int64_t num_chunks,
                  int32_t *cu_seqlens, int32_t *cu_seqlens_padded, int32_t *cu_width,
                  int32_t *num_seqs, int32_t *max_seqlen, int32_t *pad_between_seqs,
                  uint8_t *padding_mask, const psq_copy *copies, int n_copies,
                  int32_t *status, void *workspace, size_t workspace_bytes, void *stream) {
    if (layout == nullptr || B < 0 || S < 0) return PSQ_ERR_ARG;
    if (num_chunks < 1 || B % num_chunks != 0) return PSQ_ERR_ARG;
    if (layout->kind != PSQ_LAYOUT_SEQ_LENS) return PSQ_ERR_ARG;
    // the sentinel also fills the stacked int32 boundary rows
    if (layout->pad_value < INT32_MIN || layout->pad_value > INT32_MAX) return PSQ_ERR_ARG;
    if (S > 0 && B > (kI32Limit - 1) / S) return PSQ_ERR_OVERFLOW;
    if (cu_seqlens == nullptr || cu_width == nullptr || num_seqs == nullptr ||
        max_seqlen == nullptr || pad_between_seqs == nullptr || status == nullptr)
        return PSQ_ERR_ARG;
    const int cc = check_copies(copies, n_copies);
    if (cc != PSQ_OK) return cc;
    if (!valid_dtype(layout->lens_dtype) || layout->P < 0) return PSQ_ERR_ARG;
    // every staged / stacked boundary array holds at most B*P + num_chunks entries
    // (checked before B*P is formed, which S = 0 would leave unbounded)
    if (num_chunks > kI32Limit) return PSQ_ERR_OVERFLOW;
    if (layout->P > 0 && B > (kI32Limit - 2 - num_chunks) / layout->P) return PSQ_ERR_OVERFLOW;
    if (B * layout->P > 0 && layout->seq_lens == nullptr) return PSQ_ERR_ARG;
    if (!psq::thd_tables_grid_fits(B, layout->P, S, num_chunks, copies, n_copies))
        return PSQ_ERR_OVERFLOW;
    if (!workspace_ok(workspace, workspace_bytes,
                      psq::thd_tables_workspace(B, layout->P, num_chunks)))
        return PSQ_ERR_WORKSPACE;
    return from_hip(psq::launch_thd_tables(layout->seq_lens, layout->seq_lens_padded,
                                           layout->lens_dtype, B, layout->P, S, num_chunks,
                                           layout->pad_value, cu_seqlens, cu_seqlens_padded,
                                           num_seqs, max_seqlen, pad_between_seqs, cu_width,
                                           padding_mask, status, workspace, copies, n_copies,
                                           (hipStream_t)stream));
}

size_t psq_padding_mask_from_token_ids_workspace(int64_t T) {
    (void)T;
    return psq::pad_ids_workspace();
}

int psq_padding_mask_from_token_ids(const void *input_ids, int ids_dtype, int64_t T,
                                    int64_t pad_id, uint8_t *padding_mask,
                                    int32_t *num_content, int32_t *status, void *workspace,
                                    size_t workspace_bytes, void *stream) {
    if (T < 0 || !valid_dtype(ids_dtype)) return PSQ_ERR_ARG;
    if (T >= kI32Limit) return PSQ_ERR_OVERFLOW;
    if (status == nullptr) return PSQ_ERR_ARG;
    if (T > 0 && (input_ids == nullptr || padding_mask == nullptr)) return PSQ_ERR_ARG;
    if (!workspace_ok(workspace, workspace_bytes, psq::pad_ids_workspace()))
        return PSQ_ERR_WORKSPACE;
    return from_hip(psq::launch_pad_ids(input_ids, ids_dtype, T, pad_id, padding_mask,
                                        num_content, status, workspace, (hipStream_t)stream));
}

size_t psq_pack_rows_workspace(int64_t N, int64_t P, int32_t capacity) {
    (void)N;
    (void)P;
    (void)capacity;
    return psq::pack_rows_workspace();
}

int psq_pack_rows(const int64_t *src_tokens, int64_t src_len, const int64_t *src_offsets,
                  const int32_t *real_len, int64_t N, int32_t pad_to, const int32_t *pack_order,
                  const int64_t *pack_start, int64_t P, int32_t capacity, int fold,
                  int64_t pad_token, int64_t *packed, uint8_t *token_mask, int32_t *cu_seqlens,
                  int32_t *cu_seqlens_padded, int32_t *status, void *workspace,
                  size_t workspace_bytes, void *stream) {
    if (N < 0 || P < 0 || src_len < 0 || pad_to < 1 || capacity < 1) return PSQ_ERR_ARG;
    if (capacity > (1 << 30)) return PSQ_ERR_ARG;
    if (N >= kI32Limit || P >= kI32Limit - N) return PSQ_ERR_OVERFLOW;   // N + P, unformed
    if (pack_start == nullptr || status == nullptr) return PSQ_ERR_ARG;
    if (P > 0 && (packed == nullptr || token_mask == nullptr || cu_seqlens == nullptr ||
                  cu_seqlens_padded == nullptr))
        return PSQ_ERR_ARG;
    if (!psq::pack_rows_grid_fits(P, capacity)) return PSQ_ERR_OVERFLOW;
    if (N > 0 && (src_offsets == nullptr || real_len == nullptr)) return PSQ_ERR_ARG;
    if (src_len > 0 && src_tokens == nullptr) return PSQ_ERR_ARG;
    if (!workspace_ok(workspace, workspace_bytes, psq::pack_rows_workspace()))
        return PSQ_ERR_WORKSPACE;
    return from_hip(psq::launch_pack_rows(src_tokens, src_len, src_offsets, 0, real_len, N,
                                          pad_to, pack_order, pack_start, P, capacity, fold,
                                          pad_token, packed, token_mask, cu_seqlens,
                                          cu_seqlens_padded, status, workspace,
                                          (hipStream_t)stream));
}

int psq_pack_padded_rows(const int64_t *rows, int64_t W, const int32_t *real_len, int64_t N,
                         int32_t pad_to, const int32_t *pack_order, const int64_t *pack_start,
                         int64_t P, int32_t capacity, int fold, int64_t pad_token,
                         int64_t *packed, uint8_t *token_mask, int32_t *cu_seqlens,
                         int32_t *cu_seqlens_padded, int32_t *status, void *workspace,
                         size_t workspace_bytes, void *stream) {
    if (N < 0 || P < 0 || W < 0 || pad_to < 1 || capacity < 1) return PSQ_ERR_ARG;
    if (capacity > (1 << 30)) return PSQ_ERR_ARG;
    if (N >= kI32Limit || P >= kI32Limit - N) return PSQ_ERR_OVERFLOW;   // N + P, unformed
    if (W > 0 && N > ((int64_t)1 << 62) / W) return PSQ_ERR_OVERFLOW;
    if (pack_start == nullptr || status == nullptr) return PSQ_ERR_ARG;
    if (P > 0 && (packed == nullptr || token_mask == nullptr || cu_seqlens == nullptr ||
                  cu_seqlens_padded == nullptr))
        return PSQ_ERR_ARG;
    if (!psq::pack_rows_grid_fits(P, capacity)) return PSQ_ERR_OVERFLOW;
    if (N > 0 && real_len == nullptr) return PSQ_ERR_ARG;
    if (N * W > 0 && rows == nullptr) return PSQ_ERR_ARG;
    if (!workspace_ok(workspace, workspace_bytes, psq::pack_rows_workspace()))
        return PSQ_ERR_WORKSPACE;
    return from_hip(psq::launch_pack_rows(rows, N * W, nullptr, W, real_len, N, pad_to,
                                          pack_order, pack_start, P, capacity, fold, pad_token,
                                          packed, token_mask, cu_seqlens, cu_seqlens_padded,
                                          status, workspace, (hipStream_t)stream));
}

}  // extern "C"
