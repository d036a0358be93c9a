// k_copy.hip -- the BSHD -> THD collapse as batched byte copies.
//
// NeMo AutoModel 0.5 API, nemo_automodel.components.distributed.thd_utils:
// process_input_for_thd collapses the batch axis of input_ids / labels /
// position_ids ([B,S] -> [T], [B,S,H] -> [T,H], mRoPE [n,B,S] -> [n,1,T]);
// the bytes are unchanged, so each collapse is a copy into the caller's
// THD buffer.
//
// Each copy is cut into units of g bytes, g the largest of 16/8/4/1 dividing
// both addresses, the row length and the source stride; copies that share a
// unit width and density go out as one launch (normally every copy of a call
// is 16-byte and dense: one launch).  A workgroup moves 256 threads x 8 units
// (32 KiB at g = 16) with every load issued before the first store, and
// both loads and stores are non-temporal: the data is touched exactly once,
// so it should not displace anything in L2 or the MALL.
#include "psq_device.hpp"
#include "psq_internal.hpp"

namespace psq {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 8;
constexpr int64_t kUnitsPerGroup = (int64_t)kThreads * kUnroll;

struct CopyJob {
    const uint8_t *src;
    uint8_t *dst;
    int64_t units;           // total units of this copy
    int64_t units_per_row;   // units in one row
    int64_t src_stride;      // bytes between source rows (== row bytes: dense)
    int64_t group_begin;     // first workgroup of this copy
    int32_t shift;           // log2 of the unit size
    int32_t dense;           // 1: rows are back to back in the source
};

struct CopyBatch {
    CopyJob job[PSQ_MAX_COPIES];
    int32_t n;
};

template <typename U, bool kDense>
__device__ __forceinline__ void copy_units(const CopyJob &jb, int64_t u0) {
    const U *__restrict__ s = (const U *)jb.src;
    U *__restrict__ d = (U *)jb.dst;
    if (kDense && u0 + kUnitsPerGroup <= jb.units) {
        U v[kUnroll];
#pragma unroll
        for (int k = 0; k < kUnroll; ++k)
            v[k] = __builtin_nontemporal_load(s + u0 + (int64_t)k * kThreads + threadIdx.x);
#pragma unroll
        for (int k = 0; k < kUnroll; ++k)
            __builtin_nontemporal_store(v[k], d + u0 + (int64_t)k * kThreads + threadIdx.x);
        return;
    }
    // ragged tail or strided rows: one unit at a time (kept register-light,
    // since the kernel's register budget is the maximum over all its paths)
    const int64_t stride_units = jb.src_stride >> jb.shift;
    for (int k = 0; k < kUnroll; ++k) {
        const int64_t u = u0 + (int64_t)k * kThreads + threadIdx.x;
        if (u >= jb.units) break;
        int64_t at = u;
        if (!kDense) {
            const int64_t row = u / jb.units_per_row;
            at = row * stride_units + (u - row * jb.units_per_row);
        }
        __builtin_nontemporal_store(__builtin_nontemporal_load(s + at), d + u);
    }
}

// One launch covers every job of one (unit width, density) variant; the
// jobs of the batch sit back to back in the grid.
template <typename U, bool kDense>
__global__ __launch_bounds__(kThreads) void k_copies(CopyBatch batch) {
    const int64_t g = blockIdx.x;
    int i = 0;
    while (i + 1 < batch.n && g >= batch.job[i + 1].group_begin) ++i;
    const CopyJob &jb = batch.job[i];
    copy_units<U, kDense>(jb, (g - jb.group_begin) * kUnitsPerGroup);
}

__global__ __launch_bounds__(kThreads) void k_zero_fill(uint8_t *__restrict__ p, uint64_t bytes) {
    const uint64_t n16 = ((uintptr_t)p % 16) == 0 ? bytes / 16 : 0;
    const uint64_t stride = (uint64_t)gridDim.x * kThreads;
    for (uint64_t i = (uint64_t)blockIdx.x * kThreads + threadIdx.x; i < n16; i += stride)
        ((u32x4 *)p)[i] = u32x4{0u, 0u, 0u, 0u};
    if (blockIdx.x == 0) {
        for (uint64_t b = n16 * 16 + threadIdx.x; b < bytes; b += kThreads) p[b] = 0;
    }
}

int unit_shift(const psq_copy &c) {
    const uint64_t bits = (uint64_t)(uintptr_t)c.src | (uint64_t)(uintptr_t)c.dst |
                          (uint64_t)c.row_bytes |
                          (c.rows > 1 ? (uint64_t)c.src_row_stride_bytes : 0ull);
    if ((bits & 15) == 0) return 4;
    if ((bits & 7) == 0) return 3;
    if ((bits & 3) == 0) return 2;
    return 0;
}

}  // namespace

hipError_t launch_copies(const psq_copy *copies, int n_copies, hipStream_t stream) {
    // group the copies by kernel variant: unit shift (4, 3, 2, 0) x density
    for (int variant = 0; variant < 8; ++variant) {
        const int want_shift = (variant >> 1) == 0 ? 4 : (variant >> 1) == 1 ? 3 : (variant >> 1) == 2 ? 2 : 0;
        const int want_dense = variant & 1;
        CopyBatch batch{};
        int64_t groups = 0;
        int n = 0;
        for (int i = 0; i < n_copies; ++i) {
            const psq_copy &c = copies[i];
            const int64_t bytes = c.rows * c.row_bytes;
            if (bytes == 0) continue;
            const int shift = unit_shift(c);
            const int dense = (c.rows <= 1 || c.src_row_stride_bytes == c.row_bytes) ? 1 : 0;
            if (shift != want_shift || dense != want_dense) continue;
            CopyJob &jb = batch.job[n++];
            jb.shift = shift;
            jb.src = (const uint8_t *)c.src;
            jb.dst = (uint8_t *)c.dst;
            jb.units = bytes >> shift;
            jb.units_per_row = c.row_bytes >> shift;
            jb.src_stride = c.src_row_stride_bytes;
            jb.dense = dense;
            jb.group_begin = groups;
            groups += (jb.units + kUnitsPerGroup - 1) / kUnitsPerGroup;
        }
        batch.n = n;
        if (n == 0) continue;
        const dim3 grid((uint32_t)groups), block(kThreads);
#define PSQ_COPY_LAUNCH(U)                                                                   \
    if (want_dense)                                                                          \
        hipLaunchKernelGGL((k_copies<U, true>), grid, block, 0, stream, batch);              \
    else                                                                                     \
        hipLaunchKernelGGL((k_copies<U, false>), grid, block, 0, stream, batch);
        switch (want_shift) {
            case 4: PSQ_COPY_LAUNCH(u32x4) break;
            case 3: PSQ_COPY_LAUNCH(u32x2) break;
            case 2: PSQ_COPY_LAUNCH(uint32_t) break;
            default: PSQ_COPY_LAUNCH(uint8_t) break;
        }
#undef PSQ_COPY_LAUNCH
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_zero_fill(void *ptr, size_t bytes, hipStream_t stream) {
    if (bytes == 0) return hipSuccess;
    uint64_t groups = (bytes / 16 + kThreads - 1) / kThreads;
    if (groups < 1) groups = 1;
    if (groups > 4096) groups = 4096;
    hipLaunchKernelGGL(k_zero_fill, dim3((uint32_t)groups), dim3(kThreads), 0, stream,
                       (uint8_t *)ptr, (uint64_t)bytes);
    return hipGetLastError();
}

}  // namespace psq
