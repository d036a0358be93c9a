// k_padids.hip -- the metadata-free padding mask.
//
// NeMo AutoModel 0.5 API, nemo_automodel.components.distributed.thd_utils:
// thd_padding_mask_from_token_ids.  A slot is padding when its id equals the
// pad id; that is only a correct mask when the pad slots form a right-padded
// tail, so the call also checks exactly that: the first pad slot must come
// after the last non-pad slot, otherwise the pad id is also content and the
// status bit PSQ_DATA_PAD_IS_CONTENT is set.
//
// One streaming pass: each workgroup reads tiles of ids with 16-byte loads
// (all issued before any is used when the tile lies wholly in the stream;
// 4 per thread: on MI355X a 131072-id stream took 4.6-4.9 us per call back
// to back, against 5.1-5.7 us with 8 loads used one at a time), writes the
// mask bytes, and reduces two indices over its tiles (the first pad slot,
// the last non-pad slot) with wave64 DPP max scans.  A workgroup takes one
// tile, or several a grid stride apart when the stream needs more than
// kMaxGroups tiles.
//
// Every workgroup but the last publishes its two indices as one tagged
// 64-bit word (bit 63 valid, the first pad slot as T minus it in bits
// 0..30, one past the last non-pad slot in bits 31..61) and is done.  The
// last workgroup waits for those words, reads them all, compares the
// indices, writes status and the content length, and zeroes the words for
// the next call: no completion count and no release, so one device round
// trip (publish, then read) follows the loads.  Only the last workgroup
// waits, so every other one runs to the end whatever the dispatch order,
// and its wait is bounded all the same (a status bit, never a hang).
#include "psq_device.hpp"
#include "psq_internal.hpp"

namespace psq {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kIters = 4;   // 16-byte loads per thread: 2048 int64 ids per workgroup
constexpr uint32_t kMaxGroups = 2048;   // records the last workgroup reads
constexpr uint64_t kRecValid = 1ull << 63;

template <typename TI>
__global__ __launch_bounds__(kThreads) void k_pad_ids(const TI *__restrict__ ids, uint32_t T,
                                                      int64_t pad, uint8_t *__restrict__ mask,
                                                      int32_t *__restrict__ num_content,
                                                      int32_t *__restrict__ status,
                                                      uint64_t *__restrict__ recs,
                                                      uint32_t n_tiles, int vec_in,
                                                      int vec_mask) {
    constexpr int kV = 16 / (int)sizeof(TI);          // ids per 16-byte load
    constexpr uint32_t kTile = (uint32_t)kThreads * kV * kIters;
    __shared__ int32_t s_red[2][kWaves];
    __shared__ uint32_t s_err;

    // fp: T - (first pad slot), 0 when none; ln: 1 + (last non-pad slot), 0 when none
    int32_t fp = 0, ln = 0;
    for (uint32_t tile = blockIdx.x; tile < n_tiles; tile += gridDim.x) {
        const uint64_t base = (uint64_t)tile * kTile;
        // A tile wholly inside the stream loads all its ids before using any
        // (a uniform branch: straight-line loads, no wait between them).
        const bool whole_tile = vec_in && base + kTile <= T;
        u32x4 pre[kIters];
        if (whole_tile) {
#pragma unroll
            for (int it = 0; it < kIters; ++it)
                pre[it] = __builtin_nontemporal_load(
                    (const u32x4 *)(ids + base + ((uint64_t)it * kThreads + threadIdx.x) * kV));
        }
#pragma unroll
        for (int it = 0; it < kIters; ++it) {
            const uint64_t t0 = base + ((uint64_t)it * kThreads + threadIdx.x) * kV;
            if (t0 >= T) break;
            TI v[kV];
            const bool whole = t0 + kV <= T;
            if (whole_tile) {
                __builtin_memcpy(v, &pre[it], 16);
            } else if (vec_in && whole) {
                const u32x4 w = __builtin_nontemporal_load((const u32x4 *)(ids + t0));
                __builtin_memcpy(v, &w, 16);
            } else {
#pragma unroll
                for (int e = 0; e < kV; ++e) v[e] = (t0 + e < T) ? ids[t0 + e] : (TI)0;
            }
            uint32_t bits = 0;
#pragma unroll
            for (int e = 0; e < kV; ++e) {
                const uint32_t t = (uint32_t)t0 + (uint32_t)e;
                if (t0 + e < T) {
                    const bool is_pad = (int64_t)v[e] == pad;
                    bits |= (is_pad ? 1u : 0u) << (8 * e);
                    if (is_pad)
                        fp = max(fp, (int32_t)(T - t));
                    else
                        ln = max(ln, (int32_t)(t + 1u));
                }
            }
            if (vec_mask && whole) {
                if constexpr (kV == 4)
                    *(uint32_t *)(mask + t0) = bits;
                else
                    *(uint16_t *)(mask + t0) = (uint16_t)bits;
            } else {
#pragma unroll
                for (int e = 0; e < kV; ++e)
                    if (t0 + e < T) mask[t0 + e] = (uint8_t)(bits >> (8 * e));
            }
        }
    }

    const int w = wave_id(), lane = lane_id();
    const bool last = blockIdx.x == gridDim.x - 1;
    fp = wave_incl_max(fp);
    ln = wave_incl_max(ln);
    if (lane == kWave - 1) {
        s_red[0][w] = fp;
        s_red[1][w] = ln;
    }
    if (threadIdx.x == 0) s_err = 0;
    __syncthreads();
    if (!last) {
        if (threadIdx.x == 0) {
            uint32_t a = 0, b = 0;
#pragma unroll
            for (int q = 0; q < kWaves; ++q) {
                a = max(a, (uint32_t)s_red[0][q]);
                b = max(b, (uint32_t)s_red[1][q]);
            }
            jitter(5);
            st_relaxed(recs + blockIdx.x, kRecValid | (uint64_t)a | ((uint64_t)b << 31));
        }
        return;
    }

    // ---- the last workgroup: every other workgroup's word, one per thread
    // and pass; each is zeroed once read
    jitter(4);
    uint32_t a = 0, b = 0;
    bool expired = false;
    for (uint32_t g = threadIdx.x; g + 1u < gridDim.x; g += kThreads) {
        uint64_t d = ld_relaxed(recs + g);
        uint32_t spins = 0;
        while (!(d & kRecValid)) {
            if (++spins > kSpinLimit) {
                expired = true;
                break;
            }
            __builtin_amdgcn_s_sleep(1);
            d = ld_relaxed(recs + g);
        }
        if (expired) break;
        a = max(a, (uint32_t)d & 0x7fffffffu);
        b = max(b, (uint32_t)(d >> 31) & 0x7fffffffu);
        st_relaxed(recs + g, 0ull);
    }
    a = (uint32_t)wave_incl_max((int)a);
    b = (uint32_t)wave_incl_max((int)b);
    if (__ballot(expired) != 0 && lane == 0) atomicOr(&s_err, (uint32_t)PSQ_DATA_WORKSPACE);
    __syncthreads();          // every wave has read its own lanes' s_red values
    if (lane == kWave - 1) {
        s_red[0][w] = max((int32_t)a, s_red[0][w]);
        s_red[1][w] = max((int32_t)b, s_red[1][w]);
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t fa = 0, lb = 0;
#pragma unroll
        for (int q = 0; q < kWaves; ++q) {
            fa = max(fa, (uint32_t)s_red[0][q]);
            lb = max(lb, (uint32_t)s_red[1][q]);
        }
        const uint32_t first_pad = T - fa;
        *status = (int32_t)((lb > first_pad ? PSQ_DATA_PAD_IS_CONTENT : 0u) | s_err);
        if (num_content) *num_content = (int32_t)first_pad;
    }
}

// Tiles of the stream and workgroups of the launch.
void pad_grid(int ids_dtype, int64_t T, uint32_t *n_tiles, uint32_t *n_groups) {
    const int per = ids_dtype == PSQ_I64 ? 2 : 4;
    const uint64_t tile = (uint64_t)kThreads * per * kIters;
    const uint64_t nt = T > 0 ? ((uint64_t)T + tile - 1) / tile : 0;
    *n_tiles = (uint32_t)nt;
    *n_groups = nt == 0 ? 1u : (uint32_t)(nt < kMaxGroups ? nt : kMaxGroups);
}

}  // namespace

// The records follow the document-map region, where the multi-workgroup
// table kernel keeps its look-back descriptors: both leave them zero.
size_t pad_ids_workspace() { return round_up(kWsDescOffset + 8 * (size_t)kMaxGroups, 256); }

hipError_t launch_pad_ids(const void *ids, int ids_dtype, int64_t T, int64_t pad,
                          uint8_t *mask, int32_t *num_content, int32_t *status,
                          void *workspace, hipStream_t stream) {
    uint32_t n_tiles, n_groups;
    pad_grid(ids_dtype, T, &n_tiles, &n_groups);
    const int per = ids_dtype == PSQ_I64 ? 2 : 4;
    const int vec_in = ((uintptr_t)ids % 16) == 0;
    const int vec_mask = ((uintptr_t)mask % (uintptr_t)per) == 0;
    uint64_t *recs = (uint64_t *)((char *)workspace + kWsDescOffset);
    if (ids_dtype == PSQ_I64)
        hipLaunchKernelGGL(k_pad_ids<int64_t>, dim3(n_groups), dim3(kThreads), 0, stream,
                           (const int64_t *)ids, (uint32_t)T, pad, mask, num_content, status,
                           recs, n_tiles, vec_in, vec_mask);
    else
        hipLaunchKernelGGL(k_pad_ids<int32_t>, dim3(n_groups), dim3(kThreads), 0, stream,
                           (const int32_t *)ids, (uint32_t)T, pad, mask, num_content, status,
                           recs, n_tiles, vec_in, vec_mask);
    return hipGetLastError();
}

}  // namespace psq
