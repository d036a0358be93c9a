// psq_copy.hpp -- the BSHD -> THD collapse as batched byte copies: device
// code shared by the copy-only launch and the fused metadata+copy launches.
//
// NeMo AutoModel 0.5 API, nemo_automodel.components.distributed.thd_utils:
// process_input_for_thd collapses the batch axis of input_ids / labels /
// position_ids ([B,S] -> [T], [B,S,H] -> [T,H], mRoPE [n,B,S] -> [n,1,T]);
// the bytes are unchanged, so each collapse is a copy into the caller's
// THD buffer.
//
// Each copy is cut into units of g bytes, g the largest of 16/8/4/1 dividing
// both addresses, the row length and both row strides.  A workgroup moves
// 256 threads x 1 unit (4 KiB at g = 16): on MI355X many short workgroups
// streamed faster than fewer long ones with several loads in flight per
// thread (8 GiB copies: 6.4 TB/s at 4 KiB per workgroup, 5.5 TB/s at 16 KiB,
// 5.0 TB/s at 32 KiB).  Loads are non-temporal (the source is read once);
// stores are plain, which measured faster than non-temporal stores.
#pragma once

#include "psq.h"
#include "psq_device.hpp"

namespace psq {

constexpr int kCopyThreads = 256;
constexpr int kCopyUnroll = 1;
constexpr int64_t kCopyUnitsPerGroup = (int64_t)kCopyThreads * kCopyUnroll;

struct CopyJob {
    const uint8_t *src;
    uint8_t *dst;
    int64_t units;           // total units of this copy
    int64_t units_per_row;   // units in one row
    int64_t src_stride;      // bytes between source rows
    int64_t dst_stride;      // bytes between destination rows
    int64_t group_begin;     // first workgroup of this copy
    int32_t shift;           // log2 of the unit size
    int32_t dense;           // 1: rows are back to back on both sides
};

struct CopyBatch {
    CopyJob job[PSQ_MAX_COPIES];
    int32_t n;
};

template <typename U, bool kDense>
__device__ __forceinline__ void copy_units(const CopyJob &jb, int64_t u0) {
    const U *__restrict__ s = (const U *)jb.src;
    U *__restrict__ d = (U *)jb.dst;
    if (kDense && u0 + kCopyUnitsPerGroup <= jb.units) {
        U v[kCopyUnroll];
#pragma unroll
        for (int k = 0; k < kCopyUnroll; ++k)
            v[k] = __builtin_nontemporal_load(s + u0 + (int64_t)k * kCopyThreads + threadIdx.x);
#pragma unroll
        for (int k = 0; k < kCopyUnroll; ++k)
            d[u0 + (int64_t)k * kCopyThreads + threadIdx.x] = v[k];
        return;
    }
    // ragged tail or strided rows: one unit at a time (kept register-light,
    // since a kernel's register budget is the maximum over all its paths)
    const int64_t stride_units = jb.src_stride >> jb.shift;
    const int64_t dst_stride_units = jb.dst_stride >> jb.shift;
    for (int k = 0; k < kCopyUnroll; ++k) {
        const int64_t u = u0 + (int64_t)k * kCopyThreads + threadIdx.x;
        if (u >= jb.units) break;
        int64_t at = u, to = u;
        if (!kDense) {
            const int64_t row = u / jb.units_per_row;
            const int64_t col = u - row * jb.units_per_row;
            at = row * stride_units + col;
            to = row * dst_stride_units + col;
        }
        d[to] = __builtin_nontemporal_load(s + at);
    }
}

// Workgroup g of a batch: the jobs sit back to back in the grid.
template <typename U, bool kDense>
__device__ __forceinline__ void copy_group(const CopyBatch &batch, int64_t g) {
    int i = 0;
    while (i + 1 < batch.n && g >= batch.job[i + 1].group_begin) ++i;
    const CopyJob &jb = batch.job[i];
    copy_units<U, kDense>(jb, (g - jb.group_begin) * kCopyUnitsPerGroup);
}

// Host side: the copies of one call grouped by kernel variant (unit shift
// 4/3/2/0 x dense/strided).  Variant 0 (16-byte, dense) is the one the
// fused metadata+copy launches carry; any other variant is launched alone.
struct CopyPlan {
    CopyBatch batch[8];
    int64_t groups[8];
    int shift[8];
    int dense[8];
};

// Destination row stride of a copy (0 in the struct means dense rows).
inline int64_t copy_dst_stride(const psq_copy &c) {
    return c.dst_row_stride_bytes != 0 ? c.dst_row_stride_bytes : c.row_bytes;
}

inline int copy_unit_shift(const psq_copy &c) {
    const uint64_t bits = (uint64_t)(uintptr_t)c.src | (uint64_t)(uintptr_t)c.dst |
                          (uint64_t)c.row_bytes |
                          (c.rows > 1 ? (uint64_t)c.src_row_stride_bytes |
                                            (uint64_t)copy_dst_stride(c)
                                      : 0ull);
    if ((bits & 15) == 0) return 4;
    if ((bits & 7) == 0) return 3;
    if ((bits & 3) == 0) return 2;
    return 0;
}

inline void plan_copies(const psq_copy *copies, int n_copies, CopyPlan *plan) {
    for (int v = 0; v < 8; ++v) {
        const int want_shift = (v >> 1) == 0 ? 4 : (v >> 1) == 1 ? 3 : (v >> 1) == 2 ? 2 : 0;
        const int want_dense = (v & 1) == 0;
        CopyBatch &batch = plan->batch[v];
        batch = CopyBatch{};
        int64_t groups = 0;
        int n = 0;
        for (int i = 0; i < n_copies; ++i) {
            const psq_copy &c = copies[i];
            const int64_t bytes = c.rows * c.row_bytes;
            if (bytes == 0) continue;
            const int shift = copy_unit_shift(c);
            const int dense = (c.rows <= 1 || (c.src_row_stride_bytes == c.row_bytes &&
                                               copy_dst_stride(c) == c.row_bytes))
                                  ? 1
                                  : 0;
            if (shift != want_shift || dense != want_dense) continue;
            CopyJob &jb = batch.job[n++];
            jb.shift = shift;
            jb.src = (const uint8_t *)c.src;
            jb.dst = (uint8_t *)c.dst;
            jb.units = bytes >> shift;
            jb.units_per_row = c.row_bytes >> shift;
            jb.src_stride = c.src_row_stride_bytes;
            jb.dst_stride = copy_dst_stride(c);
            jb.dense = dense;
            jb.group_begin = groups;
            groups += (jb.units + kCopyUnitsPerGroup - 1) / kCopyUnitsPerGroup;
        }
        batch.n = n;
        plan->groups[v] = groups;
        plan->shift[v] = want_shift;
        plan->dense[v] = want_dense;
    }
}

// Launch every variant of the plan from `first_variant` on, alone.
hipError_t launch_copy_plan(const CopyPlan &plan, int first_variant, hipStream_t stream);

}  // namespace psq
