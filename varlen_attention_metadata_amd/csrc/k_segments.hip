// k_segments.hip -- document map -> segment boundaries, max_seqlen and mask.
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
// Layout of the work: a chunk of 1024 k positions (k = 1 ... 16) per pass
// of a 256-thread workgroup; each wave owns 256 k consecutive positions of
// the chunk, visited as k sub-chunks of 256 with 4 consecutive positions per
// lane (one 16-byte load for int32 maps).  Each lane folds its 4 boundary
// flags into a bit mask; DPP wave scans turn the popcounts into output
// slots, and a max scan of "last boundary + 1" gives every boundary the
// start of the segment before it.  A chunk's boundaries are staged in LDS in
// output order and then written as consecutive 4-byte stores, a wave's 64
// slots per store: stored straight from the flags, most lanes would idle in
// each of up to 16 scattered stores per lane.
//
// Three paths, by the map's size (doc_plan):
//  - at most 4096 positions: one workgroup does everything (k_doc_scatter
//    with kSolo), over the smallest chunk that holds the map;
//  - up to 256 chunks of 16384 positions: one launch of one workgroup per
//    chunk that exchange records through memory (k_doc_small, below), over
//    the smallest chunk of 1024 k positions (k = 1, 2, 4, 8 or 16) that
//    needs at most 256 of them;
//  - larger maps: two launches over chunks of 4096 positions, with no
//    cross-workgroup protocol.  Workgroup g owns `cpw` consecutive chunks
//    (one each, unless the map holds more than 1024 chunks).
//     1. k_doc_reduce: each workgroup reduces its range to a 16-byte record
//        -- boundary count, first boundary, last boundary + 1, and the
//        longest segment between two of its own boundaries -- and writes
//        the mask.
//     2. k_doc_scatter: each workgroup sums the counts of the records
//        before its own (its first output slot) and takes the latest
//        boundary among them, then reads its range again (just read by
//        launch 1, so mostly cached) and writes its boundaries.  The last
//        workgroup closes the axis and derives max_seqlen from all records:
//        their interior maxima, the segments that run from one record's
//        last boundary to the next record's first, and the closing segment.
//     No workgroup waits for another and nothing is counted: the kernel
//     boundary orders launch 1's record stores before launch 2's loads, and
//     the records need no clearing (every call writes before it reads).
#include "psq_device.hpp"
#include "psq_internal.hpp"

namespace psq {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kPerLane = 4;
constexpr uint32_t kSub = kWave * kPerLane;            // 256 positions
// A wave visits kIt sub-chunks of 256 positions, so a chunk holds
// 1024 kIt positions.  The two-launch path takes kIt = 4 (4096 positions);
// one-launch maps take the smallest kIt of 1, 2, 4, 8, 16 that needs at most
// 256 chunks, and one-chunk maps the smallest of 1, 2, 4 that holds the map:
// less work per wave before its record is out, and more workgroups.
constexpr int kIters = 4;
template <int kIt> constexpr uint32_t wave_span() { return kSub * (uint32_t)kIt; }
template <int kIt> constexpr uint32_t chunk_of() { return wave_span<kIt>() * kWaves; }
constexpr uint32_t kChunk = chunk_of<kIters>();        // 4096 positions

// One workgroup's range: boundary count, first boundary, one past the last
// boundary (0 = none), and the longest segment between two boundaries of the
// range.  first / last1 / imax are 0 when cnt is 0.
struct DocRec {
    uint32_t cnt, first, last1, imax;
};
static_assert(sizeof(DocRec) == 16, "records are read as 16-byte vectors");

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
struct DocArgs {
    const T *doc;
    uint32_t S, total;
    uint32_t n_chunks, cpw, n_groups;   // chunks (of the launch's size), chunks per group, groups
    int vec_in, vec_mask;
    int32_t *cu, *cu2, *num_segments, *max_seqlen;
    uint8_t *mask;
    int32_t *status, *pad_between;
    DocRec *recs;                       // n_groups records (multi-group maps)
};

// The map values of the 256 kIt positions a wave owns from wave_base
// (positions at or past `total` are absent), and the value before them.
template <typename T, int kIt>
struct WaveData {
    T d[kIt][kPerLane];
    int pres[kIt];
    T left;          // the value before the span, valid when has_left
    bool has_left;
    bool full;       // every position of the span is present (uniform)
};

// Issue the wave's loads (all of them before any is used).  A wave whose
// whole span is in range takes straight-line vector loads (a uniform
// branch); per-chunk branches would make the compiler wait for each load
// before issuing the next.  The value before the span is loaded without a
// branch too (from position 0 when there is none, then dropped): a load
// under a branch is waited for at the join, before the loads after it.
// Requires total > 0.
template <int kIt, typename T>
__device__ __forceinline__ void wave_load(const T *__restrict__ doc, uint32_t total, int vec_in,
                                          uint32_t wave_base, WaveData<T, kIt> &wd) {
    const int lane = lane_id();
    wd.has_left = wave_base > 0 && wave_base < total;
    wd.full = wave_base + wave_span<kIt>() <= total;
    // expected: laid out first, so no wait for the loads of the other path
    // is placed before these loads
    if (__builtin_expect(vec_in && wd.full, 1)) {
#pragma unroll
        for (int j = 0; j < kIt; ++j) {
            const uint32_t pos0 = wave_base + (uint32_t)j * kSub + (uint32_t)lane * kPerLane;
            if constexpr (sizeof(T) == 4) {
                const i32x4 v = *(const i32x4 *)(doc + pos0);
                wd.d[j][0] = v.x; wd.d[j][1] = v.y; wd.d[j][2] = v.z; wd.d[j][3] = v.w;
            } else {
                const i64x2 v0 = *(const i64x2 *)(doc + pos0);
                const i64x2 v1 = *(const i64x2 *)(doc + pos0 + 2);
                wd.d[j][0] = v0.x; wd.d[j][1] = v0.y; wd.d[j][2] = v1.x; wd.d[j][3] = v1.y;
            }
            wd.pres[j] = kPerLane;
        }
    } else {
#pragma unroll
        for (int j = 0; j < kIt; ++j) {
            const uint32_t pos0 = wave_base + (uint32_t)j * kSub + (uint32_t)lane * kPerLane;
            wd.pres[j] = load4(doc, pos0, total, vec_in != 0, wd.d[j]);
        }
    }
    // after the span's loads, as a vector load like them (the index is the
    // same in every lane; as a scalar load it would be waited for before the
    // loads issued after it)
    uint32_t li = wd.has_left ? wave_base - 1 : 0u;
    asm volatile("" : "+v"(li));
    wd.left = doc[li];
}

// Boundary flags of a wave's loaded positions.  For sub-chunk j: fm[j] holds
// the lane's 4 flags (bit k: position pos0 + k), off[j] counts the wave's
// boundaries before the lane's first position, and prv[j] is one past the
// wave's last boundary before the lane's positions (0: none yet in this
// wave).  *cnt and *last1 return the wave's count and one past its last
// boundary (0: none).  With `mask`, also writes mask[t] = (doc[t] == 0).
template <int kIt, typename T>
__device__ __forceinline__ void wave_flags(const WaveData<T, kIt> &wd, uint32_t S,
                                           uint8_t *__restrict__ mask, int vec_mask,
                                           uint32_t wave_base, uint32_t (&fm)[kIt],
                                           uint32_t (&off)[kIt], uint32_t (&prv)[kIt],
                                           uint32_t *cnt, uint32_t *last1) {
    const int lane = lane_id();
    T carry = wd.has_left ? wd.left : (T)0;   // first use of the loads
    uint32_t run_c = 0, run_l = 0;
    const bool small_s = S < (uint32_t)kPerLane;
    // A whole span with rows of at least 4 positions (uniform) takes
    // straight-line code: each lane's row offset r = pos0 % S is advanced by
    // kSub per sub-chunk, and a row starts inside the lane's 4 positions at
    // k = 0 when r == 0, or at k = S - r when that is below 4.
    const bool fast = wd.full && !small_s;
    uint32_t r = 0, step = 0;
    if (fast) {
        r = (wave_base + (uint32_t)lane * kPerLane) % S;
        step = kSub % S;
    }
#pragma unroll
    for (int j = 0; j < kIt; ++j) {
        const uint32_t pos0 = wave_base + (uint32_t)j * kSub + (uint32_t)lane * kPerLane;
        const T *d = wd.d[j];
        const T left = shr1(d[kPerLane - 1], carry);
        uint32_t f = 0;
        if (fast) {
            if (mask != nullptr) {
                const uint32_t m = (uint32_t)(d[0] == 0) | ((uint32_t)(d[1] == 0) << 8) |
                                   ((uint32_t)(d[2] == 0) << 16) | ((uint32_t)(d[3] == 0) << 24);
                if (vec_mask) {
                    *(uint32_t *)(mask + pos0) = m;
                } else {
#pragma unroll
                    for (int k = 0; k < kPerLane; ++k) mask[pos0 + k] = (uint8_t)(m >> (8 * k));
                }
            }
            const uint32_t to_end = S - r;    // 1 .. S
            f = (uint32_t)(d[0] != left) | ((uint32_t)(d[1] != d[0]) << 1) |
                ((uint32_t)(d[2] != d[1]) << 2) | ((uint32_t)(d[3] != d[2]) << 3) |
                (r == 0 ? 1u : 0u) | (to_end < (uint32_t)kPerLane ? 1u << to_end : 0u);
            r += step;
            r = r >= S ? r - S : r;
        } else {
            const int present = wd.pres[j];
            if (mask != nullptr && present > 0) {
                if (present == kPerLane && vec_mask) {
                    const uint32_t m = (uint32_t)(d[0] == 0) | ((uint32_t)(d[1] == 0) << 8) |
                                       ((uint32_t)(d[2] == 0) << 16) | ((uint32_t)(d[3] == 0) << 24);
                    *(uint32_t *)(mask + pos0) = m;
                } else {
                    // unrolled with a predicate: a runtime index into d would put
                    // the loaded values in scratch memory
#pragma unroll
                    for (int k = 0; k < kPerLane; ++k)
                        if (k < present) mask[pos0 + k] = (uint8_t)(d[k] == 0);
                }
            }
            if (present > 0) {
                const uint32_t rr = pos0 % S;
#pragma unroll
                for (int k = 0; k < kPerLane; ++k) {
                    if (k < present) {
                        bool row_start;
                        if (small_s)
                            row_start = ((pos0 + (uint32_t)k) % S) == 0;
                        else
                            row_start = (rr + (uint32_t)k == 0) || (rr + (uint32_t)k == S);
                        const T prev = (k == 0) ? left : d[k == 0 ? 0 : k - 1];
                        if (row_start || d[k] != prev) f |= 1u << k;
                    }
                }
            }
        }
        const uint32_t c = (uint32_t)__builtin_popcount(f);
        const uint32_t l1 = f ? pos0 + (31u - (uint32_t)__builtin_clz(f)) + 1u : 0u;
        const uint32_t incl_c = (uint32_t)wave_incl_sum((int)c);
        const uint32_t incl_l = (uint32_t)wave_incl_max((int)l1);
        const uint32_t excl_l = (uint32_t)wave_shr1((int)incl_l, 0);
        fm[j] = f;
        off[j] = run_c + incl_c - c;
        prv[j] = excl_l ? excl_l : run_l;
        run_c += (uint32_t)read_lane((int)incl_c, kWave - 1);
        const uint32_t tl = (uint32_t)read_lane((int)incl_l, kWave - 1);
        if (tl) run_l = tl;
        carry = bcast_lane(d[kPerLane - 1], kWave - 1);
    }
    *cnt = run_c;
    *last1 = run_l;
}

// The wave's first boundary (0 when it has none) and its longest segment
// that starts at one of its own boundaries and ends at the next, before the
// wave maximum.  Selects, not branches: a branch per position costs more
// than the arithmetic it skips.
template <int kIt>
__device__ __forceinline__ void wave_first_inner(const uint32_t (&fm)[kIt],
                                                 const uint32_t (&prv)[kIt],
                                                 uint32_t wave_base, uint32_t *first,
                                                 int32_t *inner) {
    const int lane = lane_id();
    uint32_t fst = 0;
    bool seen = false;
    int32_t m = 0;
#pragma unroll
    for (int j = 0; j < kIt; ++j) {
        const uint32_t f = fm[j];
        const uint32_t pos0 = wave_base + (uint32_t)j * kSub + (uint32_t)lane * kPerLane;
        const uint64_t any = __ballot(f != 0u);
        if (!seen && any) {
            const int l = __builtin_ctzll(any);
            const uint32_t mine = f ? pos0 + (uint32_t)__builtin_ctz(f) : 0u;
            fst = (uint32_t)read_lane((int)mine, l);
            seen = true;
        }
        uint32_t p = prv[j];
#pragma unroll
        for (int k = 0; k < kPerLane; ++k) {
            const bool b = (f >> k) & 1u;
            const uint32_t pos1 = pos0 + (uint32_t)k + 1u;
            m = max(m, (b && p) ? (int32_t)(pos1 - p) : 0);
            p = b ? pos1 : p;
        }
    }
    *first = fst;
    *inner = m;
}

// Stage a wave's boundary positions in LDS: the chunk's boundaries in order,
// s_pos[i] the i-th, the wave's first at index `base` (the count of the
// chunk's earlier waves).  Every index is below the chunk's boundary count,
// at most the chunk's size.
template <int kIt>
__device__ __forceinline__ void stage_positions(uint32_t *s_pos, uint32_t base,
                                                uint32_t wave_base,
                                                const uint32_t (&fm)[kIt],
                                                const uint32_t (&off)[kIt]) {
    const int lane = lane_id();
#pragma unroll
    for (int j = 0; j < kIt; ++j) {
        const uint32_t f = fm[j];
        if (f) {
            const uint32_t pos0 = wave_base + (uint32_t)j * kSub + (uint32_t)lane * kPerLane;
            uint32_t o = base + off[j];
#pragma unroll
            for (int k = 0; k < kPerLane; ++k)
                if ((f >> k) & 1u) s_pos[o++] = pos0 + (uint32_t)k;
        }
    }
}

// Write a chunk's `cnt` staged boundaries to cu[base_c ..] (and cu2), one
// slot per thread and pass, so each wave stores 256 consecutive bytes.  With
// `lengths`, returns the longest segment starting at one of them (the last
// one runs to the end of the axis); otherwise 0.  *oob is set when a slot
// falls outside the output.
template <typename T>
__device__ __forceinline__ int32_t flush_positions(const DocArgs<T> &a, const uint32_t *s_pos,
                                                   uint32_t cnt, uint32_t base_c, bool lengths,
                                                   bool *oob) {
    int32_t lmax = 0;
    for (uint32_t i = threadIdx.x; i < cnt; i += kThreads) {
        const uint32_t pos = s_pos[i];
        const uint32_t o = base_c + i;
        if (o < a.total) {
            a.cu[o] = (int32_t)pos;
            if (a.cu2) a.cu2[o] = (int32_t)pos;
        } else {
            *oob = true;
        }
        if (lengths) {
            const uint32_t nxt = i + 1u < cnt ? s_pos[i + 1u] : a.total;
            lmax = max(lmax, (int32_t)(nxt - pos));
        }
    }
    return lmax;
}

// ---------------------------------------------------------------------------
// Launch 1: one record per workgroup, and the padding mask.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(kThreads) void k_doc_reduce(DocArgs<T> a) {
    __shared__ uint32_t s_cnt[kWaves], s_first[kWaves], s_last[kWaves], s_imax[kWaves];
    const int w = wave_id();
    const int lane = lane_id();
    const uint32_t c0 = blockIdx.x * a.cpw;
    const uint32_t c1 = min(c0 + a.cpw, a.n_chunks);
    DocRec rec{0u, 0u, 0u, 0u};                 // accumulated by thread 0
    for (uint32_t c = c0; c < c1; ++c) {
        const uint32_t wave_base = c * kChunk + (uint32_t)w * wave_span<kIters>();
        WaveData<T, kIters> wd;
        wave_load(a.doc, a.total, a.vec_in, wave_base, wd);
        uint32_t fm[kIters], off[kIters], prv[kIters], cnt, last1;
        wave_flags(wd, a.S, a.mask, a.vec_mask, wave_base, fm, off, prv, &cnt, &last1);
        uint32_t first;
        int32_t lmax;
        wave_first_inner(fm, prv, wave_base, &first, &lmax);
        lmax = wave_incl_max(lmax);
        if (lane == kWave - 1) s_imax[w] = (uint32_t)lmax;
        if (lane == 0) {
            s_cnt[w] = cnt;
            s_first[w] = first;
            s_last[w] = last1;
        }
        __syncthreads();
        if (threadIdx.x == 0) {
#pragma unroll
            for (int v = 0; v < kWaves; ++v) {
                if (s_cnt[v]) {
                    if (rec.cnt)
                        rec.imax = max(rec.imax, s_first[v] + 1u - rec.last1);
                    else
                        rec.first = s_first[v];
                    rec.cnt += s_cnt[v];
                    rec.last1 = s_last[v];
                }
                rec.imax = max(rec.imax, s_imax[v]);
            }
        }
        __syncthreads();
    }
    if (threadIdx.x == 0)
        *(u32x4 *)(a.recs + blockIdx.x) = u32x4{rec.cnt, rec.first, rec.last1, rec.imax};
}

// What a workgroup of launch 2 needs from the records, reduced by each wave
// on its own (no barrier): the boundary count before the group (its first
// output slot) and one past the last boundary before it (0: none).  In the
// last group (`all`) the wave also reads its own and every other record and
// returns the longest segment they describe, closing segment excepted: the
// records' inner maxima and each segment that runs from the last boundary
// of the records before a record to that record's first boundary.  Records
// are read 64 at a time, lane l taking record 64 i + l of round i; the first
// four rounds (256 groups) are issued together.
__device__ __forceinline__ void wave_records(const DocRec *__restrict__ recs, uint32_t g,
                                             uint32_t n_groups, bool all, uint32_t *base_c,
                                             uint32_t *base_l, uint32_t *seg_max) {
    constexpr int kBatch = 4;
    const uint32_t lane = (uint32_t)lane_id();
    const uint32_t nread = all ? n_groups : g;
    uint32_t c_sum = 0, l_pre = 0, run = 0, m = 0;
    for (uint32_t r0 = 0; r0 < nread; r0 += kBatch * kWave) {
        u32x4 v[kBatch];
#pragma unroll
        for (int i = 0; i < kBatch; ++i) {
            const uint32_t idx = r0 + (uint32_t)i * kWave + lane;
            v[i] = idx < nread ? *(const u32x4 *)(recs + idx) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int i = 0; i < kBatch; ++i) {
            const uint32_t idx = r0 + (uint32_t)i * kWave + lane;
            if (idx < g) {
                c_sum += v[i].x;
                l_pre = max(l_pre, v[i].z);
            }
            if (all) {
                // one past the last boundary of every record before this one
                const uint32_t incl = (uint32_t)wave_incl_max((int)v[i].z);
                const uint32_t p = max(run, (uint32_t)wave_shr1((int)incl, 0));
                if (v[i].x) {
                    if (p) m = max(m, v[i].y + 1u - p);
                    m = max(m, v[i].w);
                }
                run = max(run, (uint32_t)read_lane((int)incl, kWave - 1));
            }
        }
    }
    *base_c = (uint32_t)read_lane(wave_incl_sum((int)c_sum), kWave - 1);
    *base_l = (uint32_t)read_lane(wave_incl_max((int)l_pre), kWave - 1);
    *seg_max = all ? (uint32_t)read_lane(wave_incl_max((int)m), kWave - 1) : 0u;
}

// ---------------------------------------------------------------------------
// Launch 2 (or the only launch of a one-chunk map, kSolo): the boundaries.
// ---------------------------------------------------------------------------
template <typename T, bool kSolo, int kIt>
__global__ __launch_bounds__(kThreads) void k_doc_scatter(DocArgs<T> a) {
    static_assert(kSolo || kIt == kIters, "launch 2 takes the chunks of launch 1");
    constexpr uint32_t kCh = chunk_of<kIt>();
    __shared__ uint32_t s_wcnt[kWaves], s_wlast[kWaves];
    __shared__ uint32_t s_pos[kCh];             // the chunk's boundaries, in order
    __shared__ int32_t s_max;
    const int w = wave_id();
    const int lane = lane_id();
    const uint32_t g = blockIdx.x;
    const bool last = g == a.n_groups - 1;
    const uint32_t c0 = g * a.cpw;
    const uint32_t c1 = min(c0 + a.cpw, a.n_chunks);
    if (threadIdx.x == 0) s_max = 0;

    // the first chunk's map loads go out before the records are read, so the
    // two round trips overlap
    WaveData<T, kIt> wd;
    if (c0 < c1) wave_load(a.doc, a.total, a.vec_in, c0 * kCh + (uint32_t)w * wave_span<kIt>(), wd);
    uint32_t base_c = 0, base_l = 0, rec_max = 0;
    if constexpr (!kSolo) wave_records(a.recs, g, a.n_groups, last, &base_c, &base_l, &rec_max);

    int32_t lmax = 0;
    bool oob = false;
    for (uint32_t c = c0; c < c1; ++c) {
        const uint32_t wave_base = c * kCh + (uint32_t)w * wave_span<kIt>();
        if (c != c0) wave_load(a.doc, a.total, a.vec_in, wave_base, wd);
        uint32_t fm[kIt], off[kIt], prv[kIt], cnt, last1;
        wave_flags(wd, a.S, kSolo ? a.mask : nullptr, a.vec_mask, wave_base, fm, off, prv, &cnt,
                   &last1);
        if (lane == 0) {
            s_wcnt[w] = cnt;
            s_wlast[w] = last1;
        }
        __syncthreads();
        // the chunk's totals and this wave's prefix inside the chunk
        uint32_t agg_c = 0, agg_l = 0, pc = 0;
#pragma unroll
        for (int v = 0; v < kWaves; ++v) {
            if (v == w) pc = agg_c;
            agg_c += s_wcnt[v];
            if (s_wlast[v]) agg_l = s_wlast[v];
        }
        stage_positions(s_pos, pc, wave_base, fm, off);
        __syncthreads();
        // a one-chunk map's segments all start at one of its boundaries
        lmax = max(lmax, flush_positions(a, s_pos, agg_c, base_c, kSolo, &oob));
        base_c += agg_c;
        if (agg_l) base_l = agg_l;
        __syncthreads();
    }
    if constexpr (kSolo) {
        lmax = wave_incl_max(lmax);
        if (lane == kWave - 1) atomicMax(&s_max, lmax);
        __syncthreads();
    }
    // a failed bound check (the map changed between the launches) is the
    // only data error this path can meet; it only reaches the status when it
    // happens in the last group
    if (last && threadIdx.x == 0) {
        const uint32_t n = base_c;
        int32_t mx = kSolo ? s_max : (int32_t)rec_max;
        uint32_t st = oob ? (uint32_t)PSQ_DATA_WORKSPACE : 0u;
        if (n <= a.total) {
            a.cu[n] = (int32_t)a.total;
            if (a.cu2) a.cu2[n] = (int32_t)a.total;
            *a.num_segments = (int32_t)n;
        } else {
            st = PSQ_DATA_WORKSPACE;
        }
        if (base_l) mx = max(mx, (int32_t)(a.total + 1u - base_l));
        *a.max_seqlen = mx;
        if (a.status) *a.status = (int32_t)st;
        if (a.pad_between) *a.pad_between = 0;
    }
}

// ---------------------------------------------------------------------------
// One launch for maps of 2..kDocSmallTiles chunks (k_doc_small).  Workgroup
// t reduces tile t to the record of launch 1 and publishes the record as one
// tagged 64-bit word.  It stages its boundaries in LDS, in order, while its
// waves wait until every earlier tile has published and reduce those records
// themselves, one per lane (wave v takes tiles 64 v .. 64 v + 63: no chained
// look-back); then it writes them out as consecutive stores.  The last tile
// also takes max_seqlen from the records, as the last group of launch 2
// does.  The tile is read once and no workgroup counts itself finished.
//
// Tiles are workgroup ids, not tickets: a workgroup waits only on lower ids,
// and at most 256 workgroups of 256 threads fit the chip's slots at once
// (a CU holds several), so every tile waited on gets a slot whatever the
// dispatch order.  The wait is bounded all the same (a status bit, never a
// hang).
//
// A record is one 64-bit word: bit 63 valid, bit 62 the call's parity, then
// the tile's boundary count (bits 0..14), first boundary (15..28) and one
// past its last boundary (29..43), both relative to the tile, and its inner
// maximum (44..58): tiles of up to 16384 positions.  The 32-bit state word,
// on the line before the records, holds the parity (bit 0) and the previous
// call's tile count (bits 1..10); every workgroup reads it while its map
// loads are in flight (a 32-bit word: with a 64-bit one whose low half goes
// unused, the compiler reused that half's register and so waited for this
// uncached load before the flags).  Once the last tile has seen every other
// tile's record, every workgroup has read the state: it
// clears the words of the tiles the previous call used beyond this call's
// count and stores the next call's state (the other parity, this call's
// count).  At the start of a call the word of every tile below its count is
// therefore zero or tagged with the other parity, and none reads as
// published before its tile publishes it.
// ---------------------------------------------------------------------------
constexpr uint64_t kTagValid = 1ull << 63;

__device__ __forceinline__ uint64_t small_tag(uint32_t parity) {
    return kTagValid | ((uint64_t)parity << 62);
}
__device__ __forceinline__ bool small_published(uint64_t word, uint32_t parity) {
    return (word >> 62) == (2ull | parity);
}

template <typename T, int kIt>
__global__ __launch_bounds__(kThreads) void k_doc_small(DocArgs<T> a, uint32_t *state,
                                                       uint64_t *desc) {
    constexpr uint32_t kCh = chunk_of<kIt>();
    static_assert(kCh <= 16384, "record fields hold tiles of up to 16384 positions");
    __shared__ uint32_t s_cnt[kWaves], s_first[kWaves], s_last[kWaves], s_imax[kWaves];
    __shared__ uint32_t s_lb_c[kWaves], s_lb_l[kWaves], s_err;
    __shared__ int32_t s_max;                   // the last tile's longest segment
    __shared__ uint32_t s_pos[kCh];             // the tile's boundaries, in order
    constexpr uint32_t kStride = kDocSmallLine / 8;     // words per record line
    const int w = wave_id();
    const int lane = lane_id();
    const uint32_t n = a.n_chunks;
    const uint32_t tile = blockIdx.x;
    const uint32_t tile_base = tile * kCh;
    const uint32_t wave_base = tile_base + (uint32_t)w * wave_span<kIt>();
    jitter(1);
    if (threadIdx.x == 0) {
        s_err = 0;
        s_max = 0;
    }

    // ---- the tile's flags, mask and record (as launch 1); every wave reads
    // the state word while its map loads are in flight
    WaveData<T, kIt> wd;
    wave_load(a.doc, a.total, a.vec_in, wave_base, wd);
    const uint32_t sw = ld_relaxed(state);
    const uint32_t parity = sw & 1u;
    const uint32_t prev_n = min((sw >> 1) & 1023u, kDocSmallTiles);
    uint32_t fm[kIt], off[kIt], prv[kIt], cnt, last1;
    wave_flags(wd, a.S, a.mask, a.vec_mask, wave_base, fm, off, prv, &cnt, &last1);
    uint32_t first;
    int32_t imax;
    wave_first_inner(fm, prv, wave_base, &first, &imax);
    imax = wave_incl_max(imax);
    if (lane == kWave - 1) s_imax[w] = (uint32_t)imax;
    if (lane == 0) {
        s_cnt[w] = cnt;
        s_first[w] = first;
        s_last[w] = last1;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        DocRec rec{0u, 0u, 0u, 0u};
#pragma unroll
        for (int v = 0; v < kWaves; ++v) {
            if (s_cnt[v]) {
                if (rec.cnt)
                    rec.imax = max(rec.imax, s_first[v] + 1u - rec.last1);
                else
                    rec.first = s_first[v];
                rec.cnt += s_cnt[v];
                rec.last1 = s_last[v];
            }
            rec.imax = max(rec.imax, s_imax[v]);
        }
        // relative to the tile: count and last1 <= 16384 (15 bits), first
        // < 16384 (14 bits), the inner maximum < 16384 (15 bits)
        const uint64_t f_rel = rec.cnt ? rec.first - tile_base : 0u;
        const uint64_t l_rel = rec.cnt ? rec.last1 - tile_base : 0u;
        jitter(5);
        st_relaxed(desc + tile * kStride, small_tag(parity) | (uint64_t)rec.cnt | (f_rel << 15) |
                                              (l_rel << 29) | ((uint64_t)rec.imax << 44));
    }
    // the tile's totals, and its boundaries staged in LDS while the earlier
    // tiles' records are awaited
    uint32_t agg_c = 0, agg_l = 0, pc = 0;
#pragma unroll
    for (int v = 0; v < kWaves; ++v) {
        if (v == w) pc = agg_c;
        agg_c += s_cnt[v];
        if (s_last[v]) agg_l = s_last[v];
    }
    stage_positions(s_pos, pc, wave_base, fm, off);

    // ---- the records of the earlier tiles: wave v waits for tiles
    // 64 v .. 64 v + 63, one per lane
    {
        jitter(4);
        const uint32_t rt = (uint32_t)w * kWave + (uint32_t)lane;     // record's tile
        uint64_t d = 0;
        bool expired = false;
        if (rt < tile) {
            uint32_t spins = 0;
            d = ld_relaxed(desc + rt * kStride);
            while (!small_published(d, parity)) {
                if (++spins > kSpinLimit) {
                    expired = true;
                    d = 0;
                    break;
                }
                __builtin_amdgcn_s_sleep(1);
                d = ld_relaxed(desc + rt * kStride);
            }
        }
        const uint32_t c = (uint32_t)d & 0x7fffu;
        const uint32_t f_abs = rt * kCh + ((uint32_t)(d >> 15) & 0x3fffu);
        const uint32_t l_rel = (uint32_t)(d >> 29) & 0x7fffu;
        const uint32_t l_abs = l_rel ? rt * kCh + l_rel : 0u;
        const uint32_t im = (uint32_t)(d >> 44) & 0x7fffu;
        const uint32_t incl = (uint32_t)wave_incl_max((int)l_abs);
        const uint32_t csum = (uint32_t)read_lane(wave_incl_sum((int)c), kWave - 1);
        const bool bad = __ballot(expired) != 0;
        if (lane == kWave - 1) {
            s_lb_c[w] = csum;
            s_lb_l[w] = incl;
        }
        if (bad && lane == 0) atomicOr(&s_err, (uint32_t)PSQ_DATA_WORKSPACE);
        __syncthreads();
        if (tile == n - 1) {
            // segments that end at an earlier tile's first boundary, and the
            // earlier tiles' inner maxima
            uint32_t p = (uint32_t)wave_shr1((int)incl, 0);
#pragma unroll
            for (int v = 0; v < kWaves; ++v)
                if (v < w) p = max(p, s_lb_l[v]);
            uint32_t m = im;
            if (c && p) m = max(m, f_abs + 1u - p);
            m = (uint32_t)read_lane(wave_incl_max((int)m), kWave - 1);
            if (lane == 0) atomicMax(&s_max, (int32_t)m);
        }
    }
    uint32_t base_c = 0, base_l = 0;
#pragma unroll
    for (int v = 0; v < kWaves; ++v) {
        base_c += s_lb_c[v];
        base_l = max(base_l, s_lb_l[v]);
    }

    // ---- the boundaries, staged before the wait; in the last tile also the
    // segments that start at them (the last one closes the axis)
    const bool last = tile == n - 1;
    bool oob = false;
    int32_t lmax = flush_positions(a, s_pos, agg_c, base_c, last, &oob);
    if (!last) return;

    // ---- the last tile: scalars, then the state of the next call
    lmax = wave_incl_max(lmax);
    if (lane == kWave - 1) atomicMax(&s_max, lmax);
    if (oob) atomicOr(&s_err, (uint32_t)PSQ_DATA_WORKSPACE);
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint32_t nseg = base_c + agg_c;
        const uint32_t last_l = agg_l ? agg_l : base_l;
        int32_t mx = s_max;
        // the segment that runs into the tile and ends at its first boundary
        if (agg_c && base_l) mx = max(mx, (int32_t)(s_pos[0] + 1u - base_l));
        uint32_t st = s_err;
        if (nseg <= a.total) {
            a.cu[nseg] = (int32_t)a.total;
            if (a.cu2) a.cu2[nseg] = (int32_t)a.total;
            *a.num_segments = (int32_t)nseg;
        } else {
            st |= PSQ_DATA_WORKSPACE;
        }
        if (last_l) mx = max(mx, (int32_t)(a.total + 1u - last_l));
        *a.max_seqlen = mx;
        if (a.status) *a.status = (int32_t)st;
        if (a.pad_between) *a.pad_between = 0;
    }
    if (w == 0) {
        for (uint32_t t = n + (uint32_t)lane; t < prev_n; t += kWave)
            st_relaxed(desc + t * kStride, 0ull);
        if (lane == 0) {
            jitter(2);
            st_relaxed(state, (n << 1) | (parity ^ 1u));
        }
    }
}

// One workgroup for a one-chunk map, or the one-launch kernel, over chunks
// of 1024 kIt positions.
template <typename T, int kIt>
void launch_solo_or_small(const DocArgs<T> &a, bool solo, uint32_t *small_state,
                          uint64_t *small_desc, hipStream_t stream) {
    if constexpr (kIt <= kIters) {
        if (solo) {
            hipLaunchKernelGGL((k_doc_scatter<T, true, kIt>), dim3(1), dim3(kThreads), 0, stream,
                               a);
            return;
        }
    }
    hipLaunchKernelGGL((k_doc_small<T, kIt>), dim3(a.n_chunks), dim3(kThreads), 0, stream, a,
                       small_state, small_desc);
}

// How a map is cut.  A map of at most 4096 positions is one workgroup over
// the smallest chunk of 1024, 2048 or 4096 positions that holds it.  Maps of
// up to 256 chunks of 16384 positions take one launch of k_doc_small over
// the smallest chunk of 1024 kit positions (kit 1, 2, 4, 8 or 16) that needs
// at most 256 of them.  Larger maps take the two launches over chunks of
// 4096 positions.
constexpr int kSmallMaxIt = 16;
struct DocPlan {
    bool solo, small;
    int kit;
    uint32_t n_chunks, cpw, n_groups;
};

// Chunks, chunks per group and groups of the two-launch path.
void doc_grid(uint32_t total, uint32_t *n_chunks, uint32_t *cpw, uint32_t *n_groups) {
    const uint32_t nc = (uint32_t)(((uint64_t)total + kChunk - 1) / kChunk);
    const uint32_t per = nc > kDocMaxGroups ? (nc + kDocMaxGroups - 1) / kDocMaxGroups : 1u;
    *n_chunks = nc;
    *cpw = per;
    *n_groups = nc <= 1 ? 1u : (nc + per - 1) / per;
}

DocPlan doc_plan(uint32_t total) {
    DocPlan p{};
    doc_grid(total, &p.n_chunks, &p.cpw, &p.n_groups);
    p.kit = kIters;
    p.solo = total <= kChunk;
    p.small = !p.solo && (uint64_t)total <= (uint64_t)kDocSmallTiles * chunk_of<kSmallMaxIt>();
    if (!p.solo && !p.small) return p;
    const uint32_t limit = p.solo ? 1u : kDocSmallTiles;
    for (int k = 1; k <= kSmallMaxIt; k *= 2) {
        const uint64_t ch = (uint64_t)kSub * kWaves * (uint64_t)k;
        const uint64_t tiles = ((uint64_t)total + ch - 1) / ch;
        if (tiles <= limit) {
            p.kit = k;
            p.n_chunks = (uint32_t)tiles;
            break;
        }
    }
    p.cpw = 1;
    p.n_groups = 1;
    return p;
}

// The metadata launches, then the collapse copies in one-wave workgroups.
// The copies are not fused into the metadata grid: on MI355X the 8 GiB
// collapse of the stage-embedding workload streamed 3 % faster in its own
// launch of one-wave workgroups (1 KiB each) than as 256-thread workgroups
// appended to the metadata grid.
template <typename T>
hipError_t launch_typed(DocArgs<T> a, const DocPlan &p, uint32_t *small_state,
                        uint64_t *small_desc, const psq_copy *copies, int n_copies,
                        hipStream_t stream) {
    if (p.solo || p.small) {
        switch (p.kit) {
        case 1: launch_solo_or_small<T, 1>(a, p.solo, small_state, small_desc, stream); break;
        case 2: launch_solo_or_small<T, 2>(a, p.solo, small_state, small_desc, stream); break;
        case 4: launch_solo_or_small<T, 4>(a, p.solo, small_state, small_desc, stream); break;
        case 8: launch_solo_or_small<T, 8>(a, p.solo, small_state, small_desc, stream); break;
        default: launch_solo_or_small<T, 16>(a, p.solo, small_state, small_desc, stream); break;
        }
    } else {
        hipLaunchKernelGGL(k_doc_reduce<T>, dim3(a.n_groups), dim3(kThreads), 0, stream, a);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL((k_doc_scatter<T, false, kIters>), dim3(a.n_groups), dim3(kThreads),
                           0, stream, a);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess || n_copies == 0) return e;
    return launch_copies(copies, n_copies, stream);
}

}  // namespace

size_t doc_segments_workspace(int64_t B, int64_t S) {
    const DocPlan p = doc_plan((uint32_t)(B * S));
    if (p.small) return kWsDocEnd;
    return round_up(kWsDocOffset + sizeof(DocRec) * (size_t)p.n_groups, 256);
}

hipError_t launch_doc_segments(const void *doc, int doc_dtype, int64_t B, int64_t S,
                               int32_t *cu, int32_t *cu2, int32_t *num_segments,
                               int32_t *max_seqlen, uint8_t *mask, int32_t *status,
                               int32_t *pad_between, void *workspace, const psq_copy *copies,
                               int n_copies, hipStream_t stream) {
    const uint32_t total = (uint32_t)(B * S);
    const DocPlan p = doc_plan(total);
    const int vec_in = ((uintptr_t)doc % 16) == 0;
    const int vec_mask = ((uintptr_t)mask % 4) == 0;
    DocRec *recs = (DocRec *)((char *)workspace + kWsDocOffset);
    uint32_t *small_state = (uint32_t *)((char *)workspace + kWsDocSmallOffset);
    uint64_t *small_desc = (uint64_t *)((char *)workspace + kWsDocSmallOffset + kDocSmallLine);
    if (doc_dtype == PSQ_I32) {
        DocArgs<int32_t> a{(const int32_t *)doc, (uint32_t)S, total, p.n_chunks, p.cpw,
                           p.n_groups, vec_in, vec_mask, cu, cu2, num_segments, max_seqlen,
                           mask, status, pad_between, recs};
        return launch_typed(a, p, small_state, small_desc, copies, n_copies, stream);
    }
    DocArgs<int64_t> a{(const int64_t *)doc, (uint32_t)S, total, p.n_chunks, p.cpw, p.n_groups,
                       vec_in, vec_mask, cu, cu2, num_segments, max_seqlen, mask, status,
                       pad_between, recs};
    return launch_typed(a, p, small_state, small_desc, copies, n_copies, stream);
}

}  // namespace psq
