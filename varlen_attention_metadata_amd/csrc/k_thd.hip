// k_thd.hip -- THD metadata and layout padding mask from per-row length
// tables, in one pass.
//
// NeMo AutoModel 0.5 API, nemo_automodel.components.distributed.thd_utils:
// process_input_for_thd (sentinel filter of seq_lens / seq_lens_padded,
// cumulative real and physical boundaries, trailing-pad absorption,
// pad_between_seqs, max_seqlen) and _thd_padding_mask (sequence i owns
// [start_i, start_i + padded_i) and holds tokens in its first real_i slots).
//
// Readings where the page leaves a step open:
//   * each row's trailing pad is folded into the row's last sequence, so the
//     physical boundaries of row r end at (r+1)*S and every physical start
//     is r*S + (padded sum of the earlier sequences of row r);
//   * absorption fires when every interior real boundary equals its physical
//     one and the real array ends before B*S; since padded' >= real for every
//     sequence, that is exactly "every sequence but the last is tight"
//     (real == padded', fold included);
//   * max_seqlen is the widest step of cu_seqlens after absorption, i.e. the
//     largest real length, or B*S - cu_seqlens[n-1] when absorption fired.
//
// Work layout: one 256-thread workgroup per (row, chunk of 4096 slots).
// Every workgroup re-derives its row's layout from the row's table (a few
// hundred bytes, read through L2) into LDS and writes its chunk of the mask
// from there: no workgroup waits on another for the mask.  Each slot finds
// its sequence through a per-chunk owner map (one LDS read) built by one
// block-wide max scan over the sequences' start slots.  The chunk-0
// workgroup of each row also takes part in a decoupled look-back over rows
// carrying (sequence count, real-token sum) and writes the row's entries of
// cu_seqlens / cu_seqlens_padded.  The last workgroup to finish applies the
// absorption and writes the scalars.
//
// The same kernel serves split_batch_into_thd_chunks (same page): the rows
// fall into G equal groups and each group is an independent
// process_input_for_thd call.  The look-back restarts at every group's first
// row (that row publishes an inclusive prefix at once), every group keeps its
// own record (count, sums, flags, max) in the workspace, and the last
// workgroup finishes each group.  With G > 1 the boundaries are staged per
// group at a fixed stride and the last workgroup writes them out as one
// [G, L] array, L the longest group's length, shorter groups filled with the
// sentinel.
#include "psq_copy.hpp"
#include "psq_device.hpp"
#include "psq_internal.hpp"

namespace psq {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kPerThread = 4;
constexpr int kBatch = kThreads * kPerThread;     // table entries per LDS batch
constexpr uint32_t kSlots = 4096;                 // mask slots per workgroup

// Per-batch results of one row, kept in LDS.
struct RowLds {
    int32_t start[kBatch];    // physical start inside the row
    int32_t real[kBatch];     // real length (clamped to [0, S+1])
    int32_t rpre[kBatch];     // real tokens of the row before this sequence
    uint32_t wsum[3][kWaves]; // block-scan scratch
    unsigned long long pad64; // exact padded sum of the row (overflow check)
    uint32_t untight;         // sequences with real != padded (unfolded)
    int32_t max_real;
    uint32_t err;
    int32_t last_real, last_pad;
};

// Exclusive block scan of three uint32 values (wrapping arithmetic).
__device__ __forceinline__ void block_scan3(RowLds &s, uint32_t v0, uint32_t v1, uint32_t v2,
                                            uint32_t (&ex)[3], uint32_t (&tot)[3]) {
    const int w = threadIdx.x / kWave, lane = lane_id();
    const uint32_t in[3] = {v0, v1, v2};
    uint32_t inc[3];
#pragma unroll
    for (int q = 0; q < 3; ++q) {
        inc[q] = (uint32_t)wave_incl_sum((int)in[q]);
        if (lane == kWave - 1) s.wsum[q][w] = inc[q];
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 3; ++q) {
        uint32_t before = 0, all = 0;
#pragma unroll
        for (int v = 0; v < kWaves; ++v) {
            if (v == w) before = all;
            all += s.wsum[q][v];
        }
        ex[q] = before + inc[q] - in[q];
        tot[q] = all;
    }
    __syncthreads();
}

// Load one batch of row r's table (entries j0 .. j0+kBatch-1), validate it,
// and store its valid sequences compactly in LDS.  `carry` holds (count,
// padded sum, real sum) of the row's earlier batches and is advanced.
template <typename TL>
__device__ __forceinline__ uint32_t row_batch(RowLds &s, const TL *__restrict__ L,
                                              const TL *__restrict__ Lp, uint64_t row_off,
                                              uint32_t P, uint32_t S, int64_t pad_value,
                                              uint32_t j0, uint32_t (&carry)[3]) {
    int64_t l[kPerThread], lp[kPerThread];
    bool valid[kPerThread];
    uint32_t cnt = 0, pad = 0, real = 0, untight = 0, err = 0;
    unsigned long long pad64 = 0;
    int32_t mreal = 0;
    const uint32_t jt = j0 + (uint32_t)threadIdx.x * kPerThread;
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) {
        const uint32_t j = jt + (uint32_t)e;
        valid[e] = false;
        l[e] = 0;
        lp[e] = 0;
        if (j < P) {
            l[e] = (int64_t)L[row_off + j];
            lp[e] = Lp ? (int64_t)Lp[row_off + j] : l[e];
            valid[e] = l[e] != pad_value;
            if (Lp && ((lp[e] != pad_value) != valid[e])) err |= PSQ_DATA_TABLE_MISMATCH;
            if (valid[e]) {
                if (l[e] < 0 || lp[e] < l[e]) err |= PSQ_DATA_BAD_LENGTH;
                const int64_t lim = (int64_t)S + 1;
                const int64_t pc = lp[e] < 0 ? 0 : (lp[e] > lim ? lim : lp[e]);
                const int64_t rc = l[e] < 0 ? 0 : (l[e] > lim ? lim : l[e]);
                lp[e] = pc;
                l[e] = rc;
                cnt += 1;
                pad += (uint32_t)pc;
                real += (uint32_t)rc;
                pad64 += (unsigned long long)pc;
                untight += (rc != pc);
                mreal = max(mreal, (int32_t)rc);
            }
        }
    }
    uint32_t ex[3], tot[3];
    block_scan3(s, cnt, pad, real, ex, tot);
    uint32_t ci = ex[0], st = carry[1] + ex[1], rp = carry[2] + ex[2];
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) {
        if (valid[e]) {
            s.start[ci] = (int32_t)st;
            s.real[ci] = (int32_t)l[e];
            s.rpre[ci] = (int32_t)rp;
            if (ci == tot[0] - 1u) {
                s.last_real = (int32_t)l[e];
                s.last_pad = (int32_t)lp[e];
            }
            ++ci;
            st += (uint32_t)lp[e];
            rp += (uint32_t)l[e];
        }
    }
    if (pad64) atomicAdd(&s.pad64, pad64);
    if (untight) atomicAdd(&s.untight, untight);
    if (mreal) atomicMax(&s.max_real, mreal);
    if (err) atomicOr(&s.err, err);
    carry[0] += tot[0];
    carry[1] += tot[1];
    carry[2] += tot[2];
    __syncthreads();
    return tot[0];
}

// Per-group record in the workspace (zero between calls).
struct GroupRec {
    uint32_t flags;     // 1: some interior real boundary departs from the physical one
    int32_t max;        // largest real length
    uint32_t n;         // sequences of the group (published by its last row)
    uint32_t total;     // real tokens of the group
    uint32_t cu_last;   // cu_seqlens[n-1] of the group
    uint32_t pad_[3];
};
static_assert(sizeof(GroupRec) == 32, "group record size");

// Workspace layout: header | row descriptors [B] | group records [G] |
// (G > 1) staged cu [G*ld] | staged cp [G*ld].
struct ThdWsLayout {
    size_t recs, stage_cu, stage_cp, bytes;
};
inline ThdWsLayout thd_ws_layout(int64_t B, int64_t G, int64_t ld) {
    ThdWsLayout w;
    w.recs = round_up(kWsDescOffset + 8 * (size_t)(B > 0 ? B : 1), 256);
    const size_t after = round_up(w.recs + sizeof(GroupRec) * (size_t)(G > 0 ? G : 1), 256);
    const size_t stage = G > 1 ? round_up(4 * (size_t)G * (size_t)ld, 256) : 0;
    w.stage_cu = after;
    w.stage_cp = after + stage;
    w.bytes = after + 2 * stage;
    return w;
}

// Owner map of one chunk [lo, hi) for one LDS batch of nb sequences:
// s_own[u - lo] = 1 + the last sequence of the batch starting at or before
// slot u (0 before the batch's first start).  Starts are non-decreasing, so
// each sequence marks its start slot (the last of equal starts wins: the
// others own no slot) and one block-wide max scan fills the gaps; every slot
// then finds its sequence with one LDS read instead of a binary search.
constexpr int kOwnWords = kSlots / kThreads / 2;   // owner-map words per thread
static_assert(kSlots % (kThreads * 8) == 0, "owner map is zeroed 16 bytes per thread");

__device__ __forceinline__ void fill_owner_map(RowLds &s, uint16_t *s_own, uint32_t &s_before,
                                               uint32_t nb, uint32_t lo, uint32_t hi) {
    const int w = threadIdx.x / kWave, lane = lane_id();
    for (uint32_t e = threadIdx.x * 8u; e < kSlots; e += kThreads * 8u)
        *(u32x4 *)(s_own + e) = u32x4{0u, 0u, 0u, 0u};
    if (threadIdx.x == 0) s_before = 0;
    __syncthreads();
    uint32_t before = 0;     // 1 + the last sequence starting at or before lo
    for (uint32_t k = threadIdx.x; k < nb; k += kThreads) {
        const uint32_t st = (uint32_t)s.start[k];
        if (st <= lo)
            before = k + 1u;
        else if (st < hi && (k + 1u == nb || (uint32_t)s.start[k + 1u] != st))
            s_own[st - lo] = (uint16_t)(k + 1u);
    }
    if (before) atomicMax(&s_before, before);
    __syncthreads();
    // thread t owns kOwnWords consecutive words (2 entries each)
    uint32_t v[kOwnWords];
    const uint32_t *own_w = (const uint32_t *)s_own + threadIdx.x * kOwnWords;
#pragma unroll
    for (int e = 0; e < kOwnWords; ++e) v[e] = own_w[e];
    uint32_t run = 0;
#pragma unroll
    for (int e = 0; e < kOwnWords; ++e) {
        const uint32_t a0 = max(run, v[e] & 0xffffu);
        const uint32_t a1 = max(a0, v[e] >> 16);
        run = a1;
        v[e] = a0 | (a1 << 16);
    }
    const uint32_t incl = (uint32_t)wave_incl_max((int)run);
    if (lane == kWave - 1) s.wsum[0][w] = incl;
    __syncthreads();
    uint32_t pre = s_before;
#pragma unroll
    for (int q = 0; q < kWaves; ++q)
        if (q < w) pre = max(pre, s.wsum[0][q]);
    pre = max(pre, (uint32_t)wave_shr1((int)incl, 0));
    uint32_t *own_o = (uint32_t *)s_own + threadIdx.x * kOwnWords;
#pragma unroll
    for (int e = 0; e < kOwnWords; ++e)
        own_o[e] = max(v[e] & 0xffffu, pre) | (max(v[e] >> 16, pre) << 16);
    __syncthreads();
}

template <typename TL>
struct ThdArgs {
    const TL *L, *Lp;
    uint32_t B, P, S;
    int64_t pad_value;
    uint32_t n_chunks;
    int vec_mask;
    uint32_t G, Bc, ld;          // groups, rows per group, staged stride
    int32_t *cu, *cp, *num_seqs, *max_seqlen, *pad_between, *cu_width;
    int32_t *cu_st, *cp_st;      // where leaders write (the outputs when G == 1)
    GroupRec *recs;
    uint8_t *mask;
    int32_t *status;
    WsHeader *ws;
};

// One (row, chunk) per workgroup; `n_groups` is the number of workgroups
// running this body (the launch may append copy workgroups after them).
template <typename TL>
__device__ __forceinline__ void thd_tables_body(const ThdArgs<TL> &args, uint32_t n_groups) {
    const TL *__restrict__ L = args.L;
    const TL *__restrict__ Lp = args.Lp;
    const uint32_t B = args.B, P = args.P, S = args.S;
    const int64_t pad_value = args.pad_value;
    const uint32_t n_chunks = args.n_chunks;
    const int vec_mask = args.vec_mask;
    const uint32_t G = args.G, Bc = args.Bc, ld = args.ld;
    int32_t *__restrict__ cu = args.cu;
    int32_t *__restrict__ cp = args.cp;
    int32_t *__restrict__ cu_st = args.cu_st;
    int32_t *__restrict__ cp_st = args.cp_st;
    GroupRec *__restrict__ recs = args.recs;
    uint8_t *__restrict__ mask = args.mask;
    WsHeader *__restrict__ ws = args.ws;
    __shared__ RowLds s;
    __shared__ __attribute__((aligned(16))) uint8_t s_mask[kSlots];
    __shared__ __attribute__((aligned(16))) uint16_t s_own[kSlots];
    __shared__ uint32_t s_before;
    __shared__ uint32_t s_slot;
    __shared__ uint32_t s_ex_a, s_ex_b, s_wserr;

    uint64_t *desc = (uint64_t *)((char *)ws + kWsDescOffset);
    if (threadIdx.x == 0) {
        s.pad64 = 0;
        s.untight = 0;
        s.max_real = 0;
        s.err = 0;
        s.last_real = 0;
        s.last_pad = 0;
        s_wserr = 0;
    }
    const uint32_t ticket = claim_tile(ws, &s_slot);
    const uint32_t Tc = Bc * S;     // tokens of one group (< 2^31)
    const int lane = lane_id();

    if ((uint64_t)ticket < (uint64_t)B * n_chunks) {
        const uint32_t r = ticket / n_chunks;
        const uint32_t c = ticket % n_chunks;
        const bool leader = (c == 0);
        const uint32_t g = r / Bc;           // group of the row
        const uint32_t rg = r - g * Bc;      // row inside its group
        const uint32_t lo = c * kSlots;
        const uint32_t hi = min(S, lo + kSlots);
        const uint64_t row_off = (uint64_t)r * P;

        // chunk mask starts as all padding; token slots are cleared below
        for (uint32_t u = threadIdx.x * 16u; u < kSlots; u += kThreads * 16u)
            *(u32x4 *)(s_mask + u) = u32x4{0x01010101u, 0x01010101u, 0x01010101u, 0x01010101u};

        uint32_t carry[3] = {0, 0, 0};
        bool one_batch = P <= (uint32_t)kBatch;
        for (uint32_t j0 = 0; j0 < P || j0 == 0; j0 += kBatch) {
            const uint32_t first = carry[1];
            const uint32_t nb = row_batch(s, L, Lp, row_off, P, S, pad_value, j0, carry);
            if (nb == 0 || hi <= lo) {
                if (j0 + kBatch >= P) break;
                continue;
            }
            // slots whose owner is in this batch: [first, end of its last one)
            const uint32_t b_lo = max(lo, first);
            const uint32_t b_hi = min(hi, carry[1]);
            if (b_lo < b_hi) {   // uniform
                fill_owner_map(s, s_own, s_before, nb, lo, hi);
                for (uint32_t u = b_lo + threadIdx.x; u < b_hi; u += kThreads) {
                    const uint32_t a = (uint32_t)s_own[u - lo] - 1u;   // >= 0 here
                    const bool tok = (u - (uint32_t)s.start[a]) < (uint32_t)s.real[a];
                    s_mask[u - lo] = tok ? 0 : 1;
                }
            }
            __syncthreads();
            if (j0 + kBatch >= P) break;
        }

        if (mask != nullptr && hi > lo) {
            const uint64_t g = (uint64_t)r * S + lo;
            const uint32_t len = hi - lo;
            if (vec_mask && (g % 16) == 0 && (len % 16) == 0) {
                for (uint32_t u = threadIdx.x * 16u; u < len; u += kThreads * 16u)
                    *(u32x4 *)(mask + g + u) = *(const u32x4 *)(s_mask + u);
            } else {
                for (uint32_t u = threadIdx.x; u < len; u += kThreads) mask[g + u] = s_mask[u];
            }
        }

        if (leader) {
            const uint32_t count = carry[0];
            const uint32_t realsum = carry[2];
            uint32_t err = s.err;
            if (count == 0) err |= PSQ_DATA_EMPTY_ROW;
            if (s.pad64 > (unsigned long long)S) err |= PSQ_DATA_ROW_OVERFLOW;
            // tightness: every sequence but the global last must have real ==
            // padded'; the row's last sequence carries the fold
            const bool last_untight_unfolded = s.last_real != s.last_pad;
            const uint32_t untight_nonlast = s.untight - (count && last_untight_unfolded ? 1u : 0u);
            const bool last_untight_folded =
                (uint32_t)s.last_real != (uint32_t)s.last_pad + (S - carry[1]);
            bool disagree = untight_nonlast > 0;
            if (rg + 1 < Bc && count) disagree = disagree || last_untight_folded;

            // look-back over the rows of the group: (sequence count, real-token
            // sum); a group's first row publishes an inclusive prefix at once,
            // so no look-back crosses into the previous group
            if (threadIdx.x < kWave) {
                uint32_t ex_a = 0, ex_b = 0;
                if (rg == 0) {
                    if (lane == 0) st_relaxed(desc + r, desc_pack(kDescIncl, count, realsum));
                } else {
                    if (lane == 0) st_relaxed(desc + r, desc_pack(kDescAgg, count, realsum));
                    bool timed_out;
                    lookback<true>(desc, r, &ex_a, &ex_b, &timed_out);
                    if (lane == 0) {
                        st_relaxed(desc + r, desc_pack(kDescIncl, ex_a + count, ex_b + realsum));
                        if (timed_out) s_wserr = PSQ_DATA_WORKSPACE;
                    }
                }
                if (lane == 0) {
                    s_ex_a = ex_a;
                    s_ex_b = ex_b;
                }
            }
            __syncthreads();
            const uint32_t ex_a = s_ex_a, ex_b = s_ex_b;
            const uint64_t cap = (uint64_t)Bc * P;    // a group holds at most Bc*P+1 entries
            bool oob = (uint64_t)ex_a + count > cap;
            int32_t *__restrict__ cu_g = cu_st + (uint64_t)g * ld;
            int32_t *__restrict__ cp_g = cp_st ? cp_st + (uint64_t)g * ld : nullptr;

            // write the row's boundaries (a second pass over the table when
            // the row did not fit one LDS batch)
            uint32_t wcarry[3] = {0, 0, 0};
            for (uint32_t j0 = 0; (j0 < P || j0 == 0) && !oob; j0 += kBatch) {
                uint32_t nb, base;
                if (one_batch) {
                    nb = count;
                    base = 0;
                } else {
                    base = wcarry[0];
                    nb = row_batch(s, L, Lp, row_off, P, S, pad_value, j0, wcarry);
                }
                for (uint32_t k = threadIdx.x; k < nb; k += kThreads) {
                    const uint32_t idx = ex_a + base + k;
                    cu_g[idx] = (int32_t)(ex_b + (uint32_t)s.rpre[k]);
                    if (cp_g) cp_g[idx] = (int32_t)(rg * S + (uint32_t)s.start[k]);
                }
                __syncthreads();
                if (one_batch || j0 + kBatch >= P) break;
            }

            if (threadIdx.x == 0) {
                if (oob) err |= PSQ_DATA_WORKSPACE;
                err |= s_wserr;
                if (err) or_relaxed(&ws->status, err);
                if (disagree) or_relaxed(&recs[g].flags, 1u);
                if (s.max_real > 0) max_relaxed(&recs[g].max, s.max_real);
                if (rg == Bc - 1 && !oob) {
                    const uint32_t n = ex_a + count;
                    const uint32_t total = ex_b + realsum;
                    st_relaxed(&recs[g].n, n);
                    st_relaxed(&recs[g].total, total);
                    st_relaxed(&recs[g].cu_last, total - (uint32_t)s.last_real);
                }
            }
        }
    } else if (B > 0 && threadIdx.x == 0) {
        or_relaxed(&ws->status, PSQ_DATA_WORKSPACE);
    }

    if (finish_is_last(ws, n_groups, &s_slot)) {
        __shared__ uint32_t s_width;
        const uint32_t st = ld_relaxed(&ws->status);
        if (threadIdx.x == 0) s_width = 0;
        __syncthreads();
        // finish every group: absorption, scalars, the closing boundaries
        uint32_t width = 0;
        for (uint32_t g = threadIdx.x; g < G; g += kThreads) {
            const uint32_t n = ld_relaxed(&recs[g].n);
            const uint32_t total = ld_relaxed(&recs[g].total);
            const uint32_t cu_last = ld_relaxed(&recs[g].cu_last);
            const bool disagree = ld_relaxed(&recs[g].flags) != 0;
            int32_t mx = (int32_t)ld_relaxed((const uint32_t *)&recs[g].max);
            if (st == 0 && (uint64_t)n <= (uint64_t)Bc * P) {
                const bool absorbed = !disagree && total < Tc;
                if (G == 1) {
                    cu[n] = (int32_t)(absorbed ? Tc : total);
                    if (cp) cp[n] = (int32_t)Tc;
                }
                if (absorbed) mx = max(mx, (int32_t)(Tc - cu_last));
                args.num_seqs[g] = (int32_t)n;
                args.max_seqlen[g] = mx;
                args.pad_between[g] = disagree ? 1 : 0;
                width = max(width, n + 1u);
            } else {
                args.num_seqs[g] = 0;
                args.max_seqlen[g] = 0;
                args.pad_between[g] = 0;
            }
        }
        if (width) atomicMax(&s_width, width);
        __syncthreads();
        width = st == 0 ? s_width : 0u;
        if (threadIdx.x == 0) {
            *args.status = (int32_t)st;
            if (args.cu_width) *args.cu_width = (int32_t)width;
        }
        // G > 1: staged groups -> one [G, width] array, short rows filled
        // with the sentinel.  Each staged entry is cleared once read (the
        // workspace is zero again after every call); after a data error the
        // whole staging area is cleared instead.
        if (G > 1 && width > 0) {
            const uint64_t total_out = (uint64_t)G * width;
            const int32_t fill = (int32_t)pad_value;
            for (uint64_t e = threadIdx.x; e < total_out; e += kThreads) {
                const uint32_t g = (uint32_t)(e / width);
                const uint32_t j = (uint32_t)(e - (uint64_t)g * width);
                const uint32_t n = ld_relaxed(&recs[g].n);
                int32_t vu = fill, vp = fill;
                if (j < n) {
                    const uint64_t at = (uint64_t)g * ld + j;
                    vu = cu_st[at];
                    cu_st[at] = 0;
                    if (cp) {
                        vp = cp_st[at];
                        cp_st[at] = 0;
                    }
                } else if (j == n) {
                    const uint32_t total = ld_relaxed(&recs[g].total);
                    const bool disagree = ld_relaxed(&recs[g].flags) != 0;
                    vu = (int32_t)((!disagree && total < Tc) ? Tc : total);
                    vp = (int32_t)Tc;
                }
                cu[e] = vu;
                if (cp) cp[e] = vp;
            }
        } else if (G > 1) {
            const uint64_t staged = (uint64_t)G * ld;
            for (uint64_t e = threadIdx.x; e < staged; e += kThreads) {
                cu_st[e] = 0;
                if (cp_st) cp_st[e] = 0;
            }
        }
        __syncthreads();
        for (uint32_t g = threadIdx.x; g < G; g += kThreads) {
            st_relaxed(&recs[g].flags, 0u);
            st_relaxed((uint32_t *)&recs[g].max, 0u);
            st_relaxed(&recs[g].n, 0u);
            st_relaxed(&recs[g].total, 0u);
            st_relaxed(&recs[g].cu_last, 0u);
        }
        for (uint32_t i = threadIdx.x; i < B; i += kThreads) st_relaxed(desc + i, 0ull);
        if (threadIdx.x == 0) {
            st_relaxed(&ws->status, 0u);
            st_relaxed(&ws->ticket, 0u);
        }
        __syncthreads();
        if (threadIdx.x == 0) st_relaxed(&ws->done, 0u);
    }
}

template <typename TL>
__global__ __launch_bounds__(kThreads) void k_thd_tables(ThdArgs<TL> a) {
    thd_tables_body<TL>(a, gridDim.x);
}

// The same workgroups followed, in one grid, by the 16-byte dense copies of
// the THD collapse: one launch per call instead of two.
template <typename TL>
__global__ __launch_bounds__(kThreads) void k_thd_tables_copy(ThdArgs<TL> a, uint32_t n_meta,
                                                              CopyBatch batch) {
    if (blockIdx.x < n_meta)
        thd_tables_body<TL>(a, n_meta);
    else
        copy_group<kThreads, u32x4, true>(batch, (int64_t)blockIdx.x - n_meta);
}

template <typename TL>
hipError_t launch_typed(ThdArgs<TL> a, uint32_t n_meta, const psq_copy *copies, int n_copies,
                        hipStream_t stream) {
    CopyPlan plan;
    plan_copies(copies, n_copies, &plan, kThreads);
    if (plan.groups[0] > 0) {
        const uint64_t grid = (uint64_t)n_meta + (uint64_t)plan.groups[0];
        hipLaunchKernelGGL(k_thd_tables_copy<TL>, dim3((uint32_t)grid), dim3(kThreads), 0,
                           stream, a, n_meta, plan.batch[0]);
    } else {
        hipLaunchKernelGGL(k_thd_tables<TL>, dim3(n_meta), dim3(kThreads), 0, stream, a);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_copy_plan(plan, 1, stream);
}

}  // namespace

size_t thd_tables_workspace(int64_t B, int64_t P, int64_t G) {
    const int64_t Bc = G > 0 ? B / G : 0;
    return thd_ws_layout(B, G, Bc * P + 1).bytes;
}

hipError_t launch_thd_tables(const void *L, const void *Lp, int lens_dtype, int64_t B,
                             int64_t P, int64_t S, int64_t G, int64_t pad_value, int32_t *cu,
                             int32_t *cp, int32_t *num_seqs, int32_t *max_seqlen,
                             int32_t *pad_between, int32_t *cu_width, uint8_t *mask,
                             int32_t *status, void *workspace, const psq_copy *copies,
                             int n_copies, hipStream_t stream) {
    const uint32_t n_chunks = S > 0 ? (uint32_t)((S + kSlots - 1) / kSlots) : 1u;
    const uint64_t groups = (uint64_t)B * n_chunks;
    const uint32_t n_meta = (uint32_t)(groups > 0 ? groups : 1);
    const int vec_mask = ((uintptr_t)mask % 16) == 0;
    const int64_t Bc = B / G;
    const int64_t ld = Bc * P + 1;
    const ThdWsLayout lay = thd_ws_layout(B, G, ld);
    char *wsb = (char *)workspace;
    int32_t *cu_st = G > 1 ? (int32_t *)(wsb + lay.stage_cu) : cu;
    int32_t *cp_st = G > 1 ? (cp ? (int32_t *)(wsb + lay.stage_cp) : nullptr) : cp;
    GroupRec *recs = (GroupRec *)(wsb + lay.recs);
    WsHeader *ws = (WsHeader *)workspace;
    if (lens_dtype == PSQ_I64) {
        ThdArgs<int64_t> a{(const int64_t *)L, (const int64_t *)Lp, (uint32_t)B, (uint32_t)P,
                           (uint32_t)S, pad_value, n_chunks, vec_mask, (uint32_t)G,
                           (uint32_t)Bc, (uint32_t)ld, cu, cp, num_seqs, max_seqlen,
                           pad_between, cu_width, cu_st, cp_st, recs, mask, status, ws};
        return launch_typed(a, n_meta, copies, n_copies, stream);
    }
    ThdArgs<int32_t> a{(const int32_t *)L, (const int32_t *)Lp, (uint32_t)B, (uint32_t)P,
                       (uint32_t)S, pad_value, n_chunks, vec_mask, (uint32_t)G, (uint32_t)Bc,
                       (uint32_t)ld, cu, cp, num_seqs, max_seqlen, pad_between, cu_width,
                       cu_st, cp_st, recs, mask, status, ws};
    return launch_typed(a, n_meta, copies, n_copies, stream);
}

}  // namespace psq
