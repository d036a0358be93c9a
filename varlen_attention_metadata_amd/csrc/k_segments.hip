// k_segments.hip -- document map -> segment boundaries, in one pass.
//
// NeMo AutoModel API, nemo_automodel.components.datasets.packed_seq:
// packed_seq_params_from_doc_ids.  A segment is a maximal run of one
// document index inside a row, and every row start begins a segment, so
// over the flattened B*S axis position t starts a segment iff
//     t % S == 0  or  doc[t] != doc[t-1].
// cu_seqlens lists the segment starts followed by B*S (PackedSeqParams.
// cu_seqlens); max_seqlen is the longest segment, padding runs included
// (PackedSeqParams.max_seqlen).  The padding mask marks doc == 0.
//
// Layout of the work: a tile of 4096 positions per 256-thread workgroup;
// each wave owns 1024 consecutive positions, visited as 4 chunks of 256 with
// 4 consecutive positions per lane (one 16-byte load for int32 maps).  Each
// lane folds its 4 boundary flags into a bit mask; DPP wave scans turn the
// popcounts into output slots, and a max scan of "last boundary + 1" gives
// every boundary the start of the segment before it.  Tiles are chained by
// a decoupled look-back whose descriptors carry (boundary count, last
// boundary + 1), so the compaction and the longest-segment reduction finish
// in the same pass.
#include "psq_device.hpp"
#include "psq_internal.hpp"

namespace psq {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kIters = 4;
constexpr int kPerLane = 4;
constexpr uint32_t kChunk = kWave * kPerLane;          // 256 positions
constexpr uint32_t kWaveSpan = kChunk * kIters;        // 1024 positions
constexpr uint32_t kTile = kWaveSpan * kWaves;         // 4096 positions

template <typename T>
__device__ __forceinline__ int load4(const T *__restrict__ doc, uint32_t pos0, uint32_t total,
                                     bool vec, T (&d)[kPerLane]) {
    if (pos0 + kPerLane <= total) {
        if (vec) {
            if constexpr (sizeof(T) == 4) {
                const i32x4 v = *(const i32x4 *)(doc + pos0);
                d[0] = v.x; d[1] = v.y; d[2] = v.z; d[3] = v.w;
            } else {
                const i64x2 v0 = *(const i64x2 *)(doc + pos0);
                const i64x2 v1 = *(const i64x2 *)(doc + pos0 + 2);
                d[0] = v0.x; d[1] = v0.y; d[2] = v1.x; d[3] = v1.y;
            }
        } else {
#pragma unroll
            for (int k = 0; k < kPerLane; ++k) d[k] = doc[pos0 + k];
        }
        return kPerLane;
    }
    const int present = pos0 < total ? (int)(total - pos0) : 0;
#pragma unroll
    for (int k = 0; k < kPerLane; ++k) d[k] = (k < present) ? doc[pos0 + k] : (T)0;
    return present;
}

// lane l gets lane l-1's value, lane 0 gets `first` (64-bit values move as
// two 32-bit halves)
template <typename T>
__device__ __forceinline__ T shr1(T x, T first) {
    if constexpr (sizeof(T) == 4) {
        return (T)wave_shr1((int)x, (int)first);
    } else {
        const uint64_t ux = (uint64_t)x, uf = (uint64_t)first;
        const uint32_t lo = (uint32_t)wave_shr1((int)(uint32_t)ux, (int)(uint32_t)uf);
        const uint32_t hi = (uint32_t)wave_shr1((int)(uint32_t)(ux >> 32), (int)(uint32_t)(uf >> 32));
        return (T)(((uint64_t)hi << 32) | lo);
    }
}

template <typename T>
__device__ __forceinline__ T bcast_lane(T x, int lane) {
    if constexpr (sizeof(T) == 4) {
        return (T)read_lane((int)x, lane);
    } else {
        const uint64_t ux = (uint64_t)x;
        const uint32_t lo = (uint32_t)read_lane((int)(uint32_t)ux, lane);
        const uint32_t hi = (uint32_t)read_lane((int)(uint32_t)(ux >> 32), lane);
        return (T)(((uint64_t)hi << 32) | lo);
    }
}

template <typename T>
struct DocSegArgs {
    const T *doc;
    uint32_t S, total, n_tiles;
    int vec_in, vec_mask;
    int32_t *cu, *cu2, *num_segments, *max_seqlen;
    uint8_t *mask;
    int32_t *status, *pad_between;
    WsHeader *ws;
};

// One tile per workgroup; `n_groups` is the number of workgroups running
// this body (the launch may append copy workgroups after them).
template <typename T>
__device__ __forceinline__ void doc_segments_body(
    const T *__restrict__ doc, uint32_t S, uint32_t total, uint32_t n_tiles, int vec_in,
    int vec_mask, int32_t *__restrict__ cu, int32_t *__restrict__ cu2,
    int32_t *__restrict__ num_segments, int32_t *__restrict__ max_seqlen,
    uint8_t *__restrict__ mask, int32_t *__restrict__ status,
    int32_t *__restrict__ pad_between, WsHeader *__restrict__ ws, uint32_t n_groups) {
    __shared__ uint32_t s_slot;
    __shared__ uint32_t s_wcnt[kWaves], s_wlast[kWaves];
    __shared__ uint32_t s_ex_a, s_ex_b;
    __shared__ int32_t s_max;
    __shared__ uint32_t s_err;

    uint64_t *desc = (uint64_t *)((char *)ws + kWsDescOffset);
    if (threadIdx.x == 0) {
        s_max = 0;
        s_err = 0;
        s_ex_a = 0;
        s_ex_b = 0;
    }
    // A map of one tile is one workgroup: it needs no ticket, no look-back and
    // no completion counter, and leaves the workspace untouched.
    const bool solo = n_groups == 1 && n_tiles <= 1;
    uint32_t tile = 0;
    if (solo)
        __syncthreads();
    else
        tile = claim_tile(ws, &s_slot);
    const int w = threadIdx.x / kWave;
    const int lane = lane_id();

    if (total == 0) {
        // empty map: cu_seqlens = [0], no segments
        if (threadIdx.x == 0) {
            cu[0] = 0;
            if (cu2) cu2[0] = 0;
            *num_segments = 0;
        }
    } else if (tile >= n_tiles) {
        if (threadIdx.x == 0) s_err = PSQ_DATA_WORKSPACE;
    } else {
        // ---------------- phase 1: flags, masks and local scans ----------
        const uint32_t wave_base = tile * kTile + (uint32_t)w * kWaveSpan;
        T carry = (T)0;
        if (wave_base > 0 && wave_base < total) carry = doc[wave_base - 1];

        // All of the wave's loads are issued before any is used.  A wave whose
        // whole span is in range takes straight-line vector loads (a uniform
        // branch); per-chunk branches would make the compiler wait for each
        // load before issuing the next.
        T dall[kIters][kPerLane];
        int pres[kIters];
        if (vec_in && wave_base + kWaveSpan <= total) {
#pragma unroll
            for (int j = 0; j < kIters; ++j) {
                const uint32_t pos0 = wave_base + (uint32_t)j * kChunk + (uint32_t)lane * kPerLane;
                if constexpr (sizeof(T) == 4) {
                    const i32x4 v = *(const i32x4 *)(doc + pos0);
                    dall[j][0] = v.x; dall[j][1] = v.y; dall[j][2] = v.z; dall[j][3] = v.w;
                } else {
                    const i64x2 v0 = *(const i64x2 *)(doc + pos0);
                    const i64x2 v1 = *(const i64x2 *)(doc + pos0 + 2);
                    dall[j][0] = v0.x; dall[j][1] = v0.y; dall[j][2] = v1.x; dall[j][3] = v1.y;
                }
                pres[j] = kPerLane;
            }
        } else {
#pragma unroll
            for (int j = 0; j < kIters; ++j) {
                const uint32_t pos0 = wave_base + (uint32_t)j * kChunk + (uint32_t)lane * kPerLane;
                pres[j] = load4(doc, pos0, total, vec_in != 0, dall[j]);
            }
        }

        uint32_t fm[kIters], off[kIters], prv[kIters];
        uint32_t run_c = 0, run_l = 0;
        const bool small_s = S < (uint32_t)kPerLane;
#pragma unroll
        for (int j = 0; j < kIters; ++j) {
            const uint32_t pos0 = wave_base + (uint32_t)j * kChunk + (uint32_t)lane * kPerLane;
            const T *d = dall[j];
            const int present = pres[j];

            if (mask != nullptr && present > 0) {
                if (present == kPerLane && vec_mask) {
                    const uint32_t m = (uint32_t)(d[0] == 0) | ((uint32_t)(d[1] == 0) << 8) |
                                       ((uint32_t)(d[2] == 0) << 16) | ((uint32_t)(d[3] == 0) << 24);
                    *(uint32_t *)(mask + pos0) = m;
                } else {
                    for (int k = 0; k < present; ++k) mask[pos0 + k] = (uint8_t)(d[k] == 0);
                }
            }

            const T left = shr1(d[kPerLane - 1], carry);
            uint32_t f = 0;
            if (present > 0) {
                const uint32_t r = pos0 % S;
#pragma unroll
                for (int k = 0; k < kPerLane; ++k) {
                    if (k < present) {
                        bool row_start;
                        if (small_s)
                            row_start = ((pos0 + (uint32_t)k) % S) == 0;
                        else
                            row_start = (r + (uint32_t)k == 0) || (r + (uint32_t)k == S);
                        const T prev = (k == 0) ? left : d[k == 0 ? 0 : k - 1];
                        const bool new_doc = d[k] != prev;
                        if (row_start || new_doc) f |= 1u << k;
                    }
                }
            }
            const uint32_t c = (uint32_t)__builtin_popcount(f);
            const uint32_t last1 = f ? pos0 + (31u - (uint32_t)__builtin_clz(f)) + 1u : 0u;
            const uint32_t incl_c = (uint32_t)wave_incl_sum((int)c);
            const uint32_t incl_l = (uint32_t)wave_incl_max((int)last1);
            const uint32_t excl_l = (uint32_t)wave_shr1((int)incl_l, 0);
            fm[j] = f;
            off[j] = run_c + incl_c - c;
            prv[j] = excl_l ? excl_l : run_l;
            run_c += (uint32_t)read_lane((int)incl_c, kWave - 1);
            const uint32_t tl = (uint32_t)read_lane((int)incl_l, kWave - 1);
            if (tl) run_l = tl;
            carry = bcast_lane(d[kPerLane - 1], kWave - 1);
        }
        if (lane == 0) {
            s_wcnt[w] = run_c;
            s_wlast[w] = run_l;
        }
        __syncthreads();

        // tile aggregate and this wave's prefix inside the tile
        uint32_t agg_c = 0, agg_l = 0, pc = 0, pl = 0;
#pragma unroll
        for (int v = 0; v < kWaves; ++v) {
            if (v == w) {
                pc = agg_c;
                pl = agg_l;
            }
            agg_c += s_wcnt[v];
            if (s_wlast[v]) agg_l = s_wlast[v];
        }

        // ---------------- decoupled look-back (wave 0) --------------------
        if (w == 0) {
            if (tile == 0) {
                if (lane == 0 && !solo) st_relaxed(desc, desc_pack(kDescIncl, agg_c, agg_l));
            } else {
                jitter(5);
                if (lane == 0) st_relaxed(desc + tile, desc_pack(kDescAgg, agg_c, agg_l));
                uint32_t ex_a, ex_b;
                bool timed_out;
                lookback<false>(desc, tile, &ex_a, &ex_b, &timed_out);
                if (lane == 0) {
                    st_relaxed(desc + tile, desc_pack(kDescIncl, ex_a + agg_c, agg_l ? agg_l : ex_b));
                    s_ex_a = ex_a;
                    s_ex_b = ex_b;
                    if (timed_out) s_err = PSQ_DATA_WORKSPACE;
                }
            }
        }
        __syncthreads();

        // ---------------- phase 2: write boundaries ----------------------
        const uint32_t base_c = s_ex_a + pc;
        const uint32_t base_l = pl ? pl : s_ex_b;
        int32_t lmax = 0;
        bool oob = false;
#pragma unroll
        for (int j = 0; j < kIters; ++j) {
            uint32_t f = fm[j];
            if (f) {
                const uint32_t pos0 = wave_base + (uint32_t)j * kChunk + (uint32_t)lane * kPerLane;
                uint32_t o = base_c + off[j];
                uint32_t p = prv[j] ? prv[j] : base_l;
#pragma unroll
                for (int k = 0; k < kPerLane; ++k) {
                    if ((f >> k) & 1u) {
                        const uint32_t pos = pos0 + (uint32_t)k;
                        if (o < total) {
                            cu[o] = (int32_t)pos;
                            if (cu2) cu2[o] = (int32_t)pos;
                        } else {
                            oob = true;
                        }
                        if (p) lmax = max(lmax, (int32_t)(pos + 1u - p));
                        p = pos + 1u;
                        ++o;
                    }
                }
            }
        }
        if (tile == n_tiles - 1 && threadIdx.x == 0) {
            // the last tile closes the flattened axis
            const uint32_t n = s_ex_a + agg_c;
            const uint32_t last1 = agg_l ? agg_l : s_ex_b;
            if (n <= total) {
                cu[n] = (int32_t)total;
                if (cu2) cu2[n] = (int32_t)total;
                *num_segments = (int32_t)n;
            } else {
                oob = true;
            }
            if (last1) lmax = max(lmax, (int32_t)(total + 1u - last1));
        }
        if (oob) atomicOr(&s_err, (uint32_t)PSQ_DATA_WORKSPACE);
        // wave max, then one LDS atomic per wave
        lmax = wave_incl_max(lmax);
        if (lane == kWave - 1) atomicMax(&s_max, lmax);
    }
    __syncthreads();
    if (solo) {
        if (threadIdx.x == 0) {
            *max_seqlen = s_max;
            if (status) *status = (int32_t)s_err;
            if (pad_between) *pad_between = 0;
        }
        return;
    }
    if (threadIdx.x == 0) {
        if (s_max > 0) max_relaxed(&ws->max, s_max);
        if (s_err) or_relaxed(&ws->status, s_err);
    }

    if (finish_is_last(ws, n_groups, &s_slot)) {
        if (threadIdx.x == 0) {
            *max_seqlen = (int32_t)ld_relaxed((const uint32_t *)&ws->max);
            const uint32_t st = ld_relaxed(&ws->status);
            if (status) *status = (int32_t)st;
            if (pad_between) *pad_between = 0;
            st_relaxed((uint32_t *)&ws->max, 0u);
            st_relaxed(&ws->status, 0u);
            st_relaxed(&ws->ticket, 0u);
        }
        for (uint32_t i = threadIdx.x; i < n_tiles; i += kThreads) st_relaxed(desc + i, 0ull);
        __syncthreads();
        if (threadIdx.x == 0) st_relaxed(&ws->done, 0u);
    }
}

#define PSQ_DOC_ARGS(a)                                                                       \
    a.doc, a.S, a.total, a.n_tiles, a.vec_in, a.vec_mask, a.cu, a.cu2, a.num_segments,       \
        a.max_seqlen, a.mask, a.status, a.pad_between, a.ws

template <typename T>
__global__ __launch_bounds__(kThreads) void k_doc_segments(DocSegArgs<T> a) {
    doc_segments_body<T>(PSQ_DOC_ARGS(a), gridDim.x);
}

#undef PSQ_DOC_ARGS

// The metadata launch, then the collapse copies in one-wave workgroups.  The
// copies are not fused into the metadata grid: on MI355X the 8 GiB collapse
// of the stage-embedding workload streamed 3 % faster in its own launch of
// one-wave workgroups (1 KiB each) than as 256-thread workgroups appended to
// the metadata grid, and a fused grid of one-wave workgroups was slower
// again (the look-back chain over 4x as many tiles).
template <typename T>
hipError_t launch_typed(DocSegArgs<T> a, const psq_copy *copies, int n_copies,
                        hipStream_t stream) {
    const uint32_t n_meta = a.n_tiles > 0 ? a.n_tiles : 1u;
    hipLaunchKernelGGL(k_doc_segments<T>, dim3(n_meta), dim3(kThreads), 0, stream, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess || n_copies == 0) return e;
    return launch_copies(copies, n_copies, stream);
}

}  // namespace

size_t doc_segments_workspace(int64_t B, int64_t S) {
    const int64_t total = B * S;
    const int64_t tiles = (total + kTile - 1) / kTile;
    return round_up(kWsDescOffset + 8 * (size_t)(tiles > 0 ? tiles : 1), 256);
}

hipError_t launch_doc_segments(const void *doc, int doc_dtype, int64_t B, int64_t S,
                               int32_t *cu, int32_t *cu2, int32_t *num_segments,
                               int32_t *max_seqlen, uint8_t *mask, int32_t *status,
                               int32_t *pad_between, void *workspace, const psq_copy *copies,
                               int n_copies, hipStream_t stream) {
    const uint32_t total = (uint32_t)(B * S);
    const uint32_t n_tiles = (total + kTile - 1) / kTile;
    const int vec_in = ((uintptr_t)doc % 16) == 0;
    const int vec_mask = ((uintptr_t)mask % 4) == 0;
    WsHeader *ws = (WsHeader *)workspace;
    if (doc_dtype == PSQ_I32) {
        DocSegArgs<int32_t> a{(const int32_t *)doc, (uint32_t)S, total, n_tiles, vec_in,
                              vec_mask, cu, cu2, num_segments, max_seqlen, mask, status,
                              pad_between, ws};
        return launch_typed(a, copies, n_copies, stream);
    }
    DocSegArgs<int64_t> a{(const int64_t *)doc, (uint32_t)S, total, n_tiles, vec_in, vec_mask,
                          cu, cu2, num_segments, max_seqlen, mask, status, pad_between, ws};
    return launch_typed(a, copies, n_copies, stream);
}

}  // namespace psq
