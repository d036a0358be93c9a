// psq_copy.hpp -- the BSHD -> THD collapse as batched byte copies: device
// code shared by the copy-only launch and the fused metadata+copy launch of
// the length-table path.
//
// NeMo AutoModel 0.5 API, nemo_automodel.components.distributed.thd_utils:
// process_input_for_thd collapses the batch axis of input_ids / labels /
// position_ids ([B,S] -> [T], [B,S,H] -> [T,H], mRoPE [n,B,S] -> [n,1,T]);
// the bytes are unchanged, so each collapse is a copy into the caller's
// THD buffer.
//
// Each copy is cut into units of g bytes, g the largest of 16/8/4/1 dividing
// both addresses, the row length and both row strides.  A standalone copy
// workgroup is one wave moving one unit per lane (1 KiB at g = 16): on
// MI355X many short workgroups streamed faster than fewer long ones with
// several loads in flight per thread (8 GiB copies: 6.55 TB/s at 1 KiB per
// one-wave workgroup, 6.4 TB/s at 4 KiB per 256-thread workgroup, 5.5 TB/s
// at 16 KiB, 5.0 TB/s at 32 KiB).  Loads and stores are non-temporal (every
// byte is moved once): with one-wave workgroups the non-temporal stores took
// the 8 GiB stage collapse from 6.48 to 6.55-6.59 TB/s.
#pragma once

#include "psq.h"
#include "psq_device.hpp"

namespace psq {

// Threads of a standalone copy workgroup.  A fused launch carries its copy
// workgroups at its own block size (kT below): one unit per thread.
constexpr int kCopyThreads = 64;

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

// Units u0 .. u0+kT-1 of one copy, one per thread of a kT-thread workgroup.
template <int kT, typename U, bool kDense>
__device__ __forceinline__ void copy_units(const CopyJob &jb, int64_t u0) {
    const U *__restrict__ s = (const U *)jb.src;
    U *__restrict__ d = (U *)jb.dst;
    const int64_t u = u0 + threadIdx.x;
    if (kDense && u0 + kT <= jb.units) {
        if constexpr (sizeof(U) == 16)
            store_stream(d + u, __builtin_nontemporal_load(s + u));
        else
            __builtin_nontemporal_store(__builtin_nontemporal_load(s + u), d + u);
        return;
    }
    // ragged tail or strided rows (kept register-light, since a kernel's
    // register budget is the maximum over all its paths)
    if (u >= jb.units) return;
    int64_t at = u, to = u;
    if (!kDense) {
        const int64_t row = u / jb.units_per_row;
        const int64_t col = u - row * jb.units_per_row;
        at = row * (jb.src_stride >> jb.shift) + col;
        to = row * (jb.dst_stride >> jb.shift) + col;
    }
    __builtin_nontemporal_store(__builtin_nontemporal_load(s + at), d + to);
}

// Workgroup g of a batch planned at kT units per workgroup: the jobs sit
// back to back in the grid.
template <int kT, typename U, bool kDense>
__device__ __forceinline__ void copy_group(const CopyBatch &batch, int64_t g) {
    int i = 0;
    while (i + 1 < batch.n && g >= batch.job[i + 1].group_begin) ++i;
    const CopyJob &jb = batch.job[i];
    copy_units<kT, U, kDense>(jb, (g - jb.group_begin) * kT);
}

// Largest unit count of one call per kernel variant: the grid of a launch is
// counted in 32-bit work-items, one per unit.
constexpr int64_t kMaxCopyUnits = (int64_t)1 << 31;

// Host side: the copies of one call grouped by kernel variant (unit shift
// 4/3/2/0 x dense/strided).  Variant 0 (16-byte, dense) is planned at
// `fused_threads` units per workgroup -- the block size of the launch that
// carries it; every other variant is launched alone, at kCopyThreads.
struct CopyPlan {
    CopyBatch batch[8];
    int64_t groups[8];
    int shift[8];
    int dense[8];
    int threads[8];
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

// True when every variant of these copies fits one launch.
inline bool copies_fit(const psq_copy *copies, int n_copies) {
    int64_t units[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int i = 0; i < n_copies; ++i) {
        const psq_copy &c = copies[i];
        if (c.rows <= 0 || c.row_bytes <= 0) continue;
        if (c.rows > INT64_MAX / c.row_bytes) return false;
        const int shift = copy_unit_shift(c);
        const int v = (shift == 4 ? 0 : shift == 3 ? 1 : shift == 2 ? 2 : 3);
        const int64_t u = (c.rows * c.row_bytes) >> shift;
        if (u >= kMaxCopyUnits) return false;
        units[v] += u;
        if (units[v] >= kMaxCopyUnits) return false;
    }
    return true;
}

inline void plan_copies(const psq_copy *copies, int n_copies, CopyPlan *plan,
                        int fused_threads) {
    for (int v = 0; v < 8; ++v) {
        const int64_t per_group = v == 0 ? fused_threads : kCopyThreads;
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
            groups += (jb.units + per_group - 1) / per_group;
        }
        batch.n = n;
        plan->groups[v] = groups;
        plan->shift[v] = want_shift;
        plan->dense[v] = want_dense;
        plan->threads[v] = (int)per_group;
    }
}

// Launch every variant of the plan from `first_variant` on, alone (variant 0
// only when it was planned at kCopyThreads).
hipError_t launch_copy_plan(const CopyPlan &plan, int first_variant, hipStream_t stream);

}  // namespace psq
