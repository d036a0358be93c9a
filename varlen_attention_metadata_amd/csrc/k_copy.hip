// k_copy.hip -- copy-only launches of the THD collapse, and the workspace
// zero fill.  The copy device code lives in psq_copy.hpp, shared with the
// fused metadata+copy launch of the length-table path.
#include "psq_copy.hpp"
#include "psq_internal.hpp"

namespace psq {
namespace {

template <typename U, bool kDense>
__global__ __launch_bounds__(kCopyThreads) void k_copies(CopyBatch batch) {
    copy_group<kCopyThreads, U, kDense>(batch, blockIdx.x);
}

__global__ __launch_bounds__(kCopyThreads) void k_zero_fill(uint8_t *__restrict__ p, uint64_t bytes) {
    const uint64_t n16 = ((uintptr_t)p % 16) == 0 ? bytes / 16 : 0;
    const uint64_t stride = (uint64_t)gridDim.x * kCopyThreads;
    for (uint64_t i = (uint64_t)blockIdx.x * kCopyThreads + threadIdx.x; i < n16; i += stride)
        ((u32x4 *)p)[i] = u32x4{0u, 0u, 0u, 0u};
    if (blockIdx.x == 0) {
        for (uint64_t b = n16 * 16 + threadIdx.x; b < bytes; b += kCopyThreads) p[b] = 0;
    }
}

}  // namespace

hipError_t launch_copy_plan(const CopyPlan &plan, int first_variant, hipStream_t stream) {
    for (int v = first_variant; v < 8; ++v) {
        if (plan.groups[v] == 0) continue;
        if (plan.threads[v] != kCopyThreads) return hipErrorInvalidValue;
        const dim3 grid((uint32_t)plan.groups[v]), block(kCopyThreads);
        const CopyBatch &b = plan.batch[v];
#define PSQ_COPY_LAUNCH(U)                                                                   \
    if (plan.dense[v])                                                                       \
        hipLaunchKernelGGL((k_copies<U, true>), grid, block, 0, stream, b);                  \
    else                                                                                     \
        hipLaunchKernelGGL((k_copies<U, false>), grid, block, 0, stream, b);
        switch (plan.shift[v]) {
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

hipError_t launch_copies(const psq_copy *copies, int n_copies, hipStream_t stream) {
    CopyPlan plan;
    plan_copies(copies, n_copies, &plan, kCopyThreads);
    return launch_copy_plan(plan, 0, stream);
}

hipError_t launch_zero_fill(void *ptr, size_t bytes, hipStream_t stream) {
    if (bytes == 0) return hipSuccess;
    uint64_t groups = (bytes / 16 + kCopyThreads - 1) / kCopyThreads;
    if (groups < 1) groups = 1;
    if (groups > 4096) groups = 4096;
    hipLaunchKernelGGL(k_zero_fill, dim3((uint32_t)groups), dim3(kCopyThreads), 0, stream,
                       (uint8_t *)ptr, (uint64_t)bytes);
    return hipGetLastError();
}

}  // namespace psq
