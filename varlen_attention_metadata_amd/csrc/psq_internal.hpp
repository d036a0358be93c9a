// psq_internal.hpp -- launchers shared between the host API and the kernel
// translation units.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "psq.h"

namespace psq {

// One HIP launch runs at most 2^32 - 1 threads along x.
constexpr uint64_t kMaxGridThreads = 0xffffffffull;

// k_segments.hip -- document map -> segment boundaries (then the collapse copies).
size_t doc_segments_workspace(int64_t B, int64_t S);
hipError_t launch_doc_segments(const void *doc, int doc_dtype, int64_t B, int64_t S,
                               int32_t *cu, int32_t *cu2, int32_t *num_segments,
                               int32_t *max_seqlen, uint8_t *mask, int32_t *status,
                               int32_t *pad_between, void *workspace, const psq_copy *copies,
                               int n_copies, hipStream_t stream);

// k_thd.hip -- length tables -> THD metadata and layout mask (+ fused copies),
// for G equal row groups (G == 1: one process_input_for_thd call).
size_t thd_tables_workspace(int64_t B, int64_t P, int64_t G);
// Whether every grid of the call fits kMaxGridThreads (sizes already bounded
// by the int32 checks of the API).
bool thd_tables_grid_fits(int64_t B, int64_t P, int64_t S, int64_t G, const psq_copy *copies,
                          int n_copies);
hipError_t launch_thd_tables(const void *L, const void *Lp, int lens_dtype, int64_t B,
                             int64_t P, int64_t S, int64_t G, int64_t pad_value, int32_t *cu,
                             int32_t *cp, int32_t *num_seqs, int32_t *max_seqlen,
                             int32_t *pad_between, int32_t *cu_width, uint8_t *mask,
                             int32_t *status, void *workspace, const psq_copy *copies,
                             int n_copies, hipStream_t stream);

// k_copy.hip -- batched byte copies (the BSHD -> THD collapse).
hipError_t launch_copies(const psq_copy *copies, int n_copies, hipStream_t stream);
hipError_t launch_zero_fill(void *ptr, size_t bytes, hipStream_t stream);

// k_pack.hip -- the squeeze into fixed-capacity packs.
size_t pack_rows_workspace();
bool pack_rows_grid_fits(int64_t P, int32_t C);
hipError_t launch_pack_rows(const int64_t *src, int64_t src_len, const int64_t *src_off,
                            int64_t src_stride, const int32_t *real_len, int64_t N, int32_t q,
                            const int32_t *order, const int64_t *pack_start, int64_t P,
                            int32_t C, int fold, int64_t pad_token, int64_t *packed,
                            uint8_t *tmask, int32_t *cu, int32_t *cp, int32_t *status,
                            void *workspace, hipStream_t stream);

// k_padids.hip -- the metadata-free padding mask from token ids.
size_t pad_ids_workspace();
hipError_t launch_pad_ids(const void *ids, int ids_dtype, int64_t T, int64_t pad,
                          uint8_t *mask, int32_t *num_content, int32_t *status,
                          void *workspace, hipStream_t stream);

inline size_t round_up(size_t x, size_t m) { return (x + m - 1) / m * m; }

}  // namespace psq
