// psq_noalloc.hip -- psq_params_from_doc_ids_noalloc: the document-map call
// for callers that cannot allocate device memory (code under HIP graph
// capture, tight serving loops, harnesses that forbid hipMalloc).
//
// It runs the kernels of psq_params_from_doc_ids, with the workspace taken
// from `scratch`, a file-scope device array.  Every GPU the library runs on
// holds its own copy of the array until the process ends.  In host code the
// array's name only stands in for the symbol: the device address of each
// GPU's copy comes from hipGetSymbolAddress, looked up once per device (with
// that device current) on the first call there, and only that address is
// ever handed to a kernel.
//
// The kernels keep their records (at most 1024 of 16 bytes, whatever the
// map's size) and the small maps' protocol state in the scratch.  The state
// must start zero-filled, so the first call on a device enqueues one fill
// kernel on its stream before its own kernels; every call then leaves the
// scratch ready for the next.  Calls that overlap in time on one GPU (two
// streams, two host threads) share the array and race.
#include <hip/hip_runtime.h>

#include <mutex>

#include "psq.h"
#include "psq_device.hpp"
#include "psq_internal.hpp"

namespace {

constexpr size_t kScratchBytes = PSQ_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes >= psq::kWsDocEnd,
              "the scratch holds the largest document-map workspace");

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void *g_scratch[kMaxDevices];   // per device: the device address of `scratch`

// The current device's copy of `scratch`; on the first call on a device,
// its address is looked up and a zero fill is enqueued on `stream`.  Returns
// PSQ_OK or PSQ_ERR_HIP.
int scratch_address(hipStream_t stream, void **out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return PSQ_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_mutex);
    if (g_scratch[dev] == nullptr) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
            return PSQ_ERR_HIP;
        if (psq::launch_zero_fill(p, kScratchBytes, stream) != hipSuccess) return PSQ_ERR_HIP;
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return PSQ_OK;
}

}  // namespace

extern "C" int psq_params_from_doc_ids_noalloc(const void *doc_ids, int doc_dtype, int64_t B,
                                               int64_t S, int32_t *cu_seqlens,
                                               int32_t *num_segments, int32_t *max_seqlen,
                                               uint8_t *padding_mask, int32_t *status,
                                               void *stream) {
    constexpr int64_t kI32Limit = (int64_t)1 << 31;
    if (B < 0 || S < 0 || (doc_dtype != PSQ_I32 && doc_dtype != PSQ_I64)) return PSQ_ERR_ARG;
    if (S > 0 && B > (kI32Limit - 1) / S) return PSQ_ERR_OVERFLOW;
    if (cu_seqlens == nullptr || num_segments == nullptr || max_seqlen == nullptr)
        return PSQ_ERR_ARG;
    if (B * S > 0 && doc_ids == nullptr) return PSQ_ERR_ARG;
    // every map the call accepts needs at most 1024 records; the check keeps
    // the array's bound explicit should that ever change
    if (psq::doc_segments_workspace(B, S) > kScratchBytes) return PSQ_ERR_OVERFLOW;
    void *ws = nullptr;
    const int rc = scratch_address((hipStream_t)stream, &ws);
    if (rc != PSQ_OK) return rc;
    const hipError_t e = psq::launch_doc_segments(doc_ids, doc_dtype, B, S, cu_seqlens, nullptr,
                                                  num_segments, max_seqlen, padding_mask,
                                                  status, nullptr, ws, nullptr, 0,
                                                  (hipStream_t)stream);
    return e == hipSuccess ? PSQ_OK : PSQ_ERR_HIP;
}
