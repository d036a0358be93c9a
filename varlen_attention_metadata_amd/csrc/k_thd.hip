// k_thd.hip -- THD metadata and layout padding mask from per-row length
// tables, in one pass.
//
// NeMo AutoModel 0.5 API, nemo_automodel.components.distributed.thd_utils:
// process_input_for_thd (sentinel filter of seq_lens / seq_lens_padded,
// cumulative real and physical boundaries, trailing-pad absorption,
// pad_between_seqs, max_seqlen) and _thd_padding_mask (the padded_i slots
// from start_i belong to sequence i, and only the first real_i of them are
// tokens).
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
// Two kernels.  Tables of at most 4096 entries (and at most 64 row groups)
// take k_thd_small, further down: one 1024-thread workgroup derives every
// boundary from the whole table while the others write the mask, with no
// workgroup waiting on another.  Larger tables take k_thd_tables:
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

// Exclusive block scan of three uint32 values (wrapping arithmetic) over a
// workgroup of kW waves.
template <int kW = kWaves>
__device__ __forceinline__ void block_scan3(uint32_t (&wsum)[3][kW], uint32_t v0, uint32_t v1,
                                            uint32_t v2, uint32_t (&ex)[3], uint32_t (&tot)[3]) {
    const int w = wave_id(), lane = lane_id();
    const uint32_t in[3] = {v0, v1, v2};
    uint32_t inc[3];
#pragma unroll
    for (int q = 0; q < 3; ++q) {
        inc[q] = (uint32_t)wave_incl_sum((int)in[q]);
        if (lane == kWave - 1) wsum[q][w] = inc[q];
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 3; ++q) {
        uint32_t before = 0, all = 0;
#pragma unroll
        for (int v = 0; v < kW; ++v) {
            if (v == w) before = all;
            all += wsum[q][v];
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
    block_scan3(s.wsum, cnt, pad, real, ex, tot);
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
    const int w = wave_id(), lane = lane_id();
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

// Row r's layout from its table (batch by batch into LDS) and chunk c of the
// mask.  `s` must hold zeroed accumulators, published by a barrier.  On
// return carry = (sequences, padded sum, real sum) of the row and `s` holds
// the row's last batch and its per-row flags.
template <typename TL>
__device__ __forceinline__ void row_layout_and_mask(const ThdArgs<TL> &args, RowLds &s,
                                                    uint8_t *s_mask, uint16_t *s_own,
                                                    uint32_t &s_before, uint32_t r, uint32_t c,
                                                    uint32_t (&carry)[3]) {
    const TL *__restrict__ L = args.L;
    const TL *__restrict__ Lp = args.Lp;
    const uint32_t P = args.P, S = args.S;
    const int64_t pad_value = args.pad_value;
    uint8_t *__restrict__ mask = args.mask;
    const int vec_mask = args.vec_mask;
    const uint32_t lo = c * kSlots;
    const uint32_t hi = min(S, lo + kSlots);
    const uint64_t row_off = (uint64_t)r * P;

    // chunk mask starts as all padding; token slots are cleared below
    for (uint32_t u = threadIdx.x * 16u; u < kSlots; u += kThreads * 16u)
        *(u32x4 *)(s_mask + u) = u32x4{0x01010101u, 0x01010101u, 0x01010101u, 0x01010101u};

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
}

// One (row, chunk) per workgroup; `n_groups` is the number of workgroups
// running this body (the launch may append copy workgroups after them).
template <typename TL>
__device__ __forceinline__ void thd_tables_body(const ThdArgs<TL> &args, uint32_t n_groups) {
    const TL *__restrict__ L = args.L;
    const TL *__restrict__ Lp = args.Lp;
    const uint32_t B = args.B, P = args.P, S = args.S;
    const int64_t pad_value = args.pad_value;
    const uint32_t n_chunks = args.n_chunks;
    const uint32_t G = args.G, Bc = args.Bc, ld = args.ld;
    int32_t *__restrict__ cu = args.cu;
    int32_t *__restrict__ cp = args.cp;
    int32_t *__restrict__ cu_st = args.cu_st;
    int32_t *__restrict__ cp_st = args.cp_st;
    GroupRec *__restrict__ recs = args.recs;
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
        const uint64_t row_off = (uint64_t)r * P;

        uint32_t carry[3] = {0, 0, 0};
        const bool one_batch = P <= (uint32_t)kBatch;
        row_layout_and_mask(args, s, s_mask, s_own, s_before, r, c, carry);

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
                    jitter(6);
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

// ---------------------------------------------------------------------------
// Small tables (B*P <= kSmallEntries, G <= kSmallGroups).
// Workgroup 0 holds the whole table in registers and LDS and derives every
// group's boundaries and scalars from it with block-wide scans (tables of at
// most 64 rows of at most 64 entries: one wave per row, thd_rows_meta); each of the
// next workgroups writes one (row, chunk) of the mask from its own row's
// table.  No workgroup waits on another, so there is no ticket, look-back or
// completion count, and the workspace is left untouched.  The status bits
// are the same predicates as above, evaluated over the whole table at once.
// ---------------------------------------------------------------------------
constexpr uint32_t kSmallEntries = 4096;
constexpr uint32_t kSmallGroups = 64;
constexpr int kSmallThreads = 1024;      // workgroup size of the small-table launch
constexpr int kSmallWaves = kSmallThreads / kWave;
// table entries per thread: 4 for tables above 2048 entries, else 2 (with
// 4, workload-3 tables of 1024 entries took 6.1 instead of 5.1 us per call)
constexpr int kSmallPerMax = (int)(kSmallEntries / kSmallThreads);
constexpr uint32_t kSmallSlots = 16384;   // mask slots per workgroup (1024 per wave)
constexpr uint32_t kNoSeq = 0xffffffffu;   // real[] of an entry holding no sequence

template <int kPer>
struct SmallMeta {
    uint32_t real[kPer * kSmallThreads];      // clamped real length, or kNoSeq
    uint32_t phys[kPer * kSmallThreads];      // clamped padded length; a row's last folded
    uint32_t g_last[kSmallGroups];            // 1 + the group's last valid entry
    uint32_t g_flag[kSmallGroups];            // an interior boundary departs from its physical one
    int32_t g_max[kSmallGroups];              // largest real length of the group
    uint32_t g_base[3][kSmallGroups + 1];     // (count, real, physical) before each group
    uint32_t wsum[3][kSmallWaves];
    uint32_t err;
};

template <typename TL, int kSmallPer>
__device__ __forceinline__ void thd_small_meta(const ThdArgs<TL> &args, SmallMeta<kSmallPer> &m) {
    const uint32_t B = args.B, P = args.P, S = args.S, G = args.G, Bc = args.Bc;
    const uint32_t E = B * P;       // table entries, 1 .. kSmallPer * kSmallThreads
    const uint32_t Eg = Bc * P;     // entries of one group
    const uint32_t Tc = Bc * S;     // tokens of one group (< 2^31)
    const uint32_t sat = S + 1u;    // clamp of a length, and of a row's padded sum
    const int64_t pv = args.pad_value;
    const TL *__restrict__ L = args.L;
    const TL *__restrict__ Lq = args.Lp ? args.Lp : args.L;
    int32_t *__restrict__ cu = args.cu;
    int32_t *__restrict__ cp = args.cp;
    const int w = wave_id(), lane = lane_id();

    for (uint32_t g = threadIdx.x; g < G; g += kSmallThreads) {
        m.g_last[g] = 0;
        m.g_flag[g] = 0;
        m.g_max[g] = 0;
    }
    if (threadIdx.x == 0) m.err = 0;

    // thread t owns the kSmallPer consecutive entries from e0; every load is
    // issued before any is used (indices clamped into the table)
    const uint32_t e0 = threadIdx.x * (uint32_t)kSmallPer;
    int64_t l[kSmallPer], lp[kSmallPer];
#pragma unroll
    for (int k = 0; k < kSmallPer; ++k) {
        const uint32_t e = min(e0 + (uint32_t)k, E - 1u);
        l[k] = (int64_t)L[e];
        lp[k] = (int64_t)Lq[e];
    }

    // validity, the length checks, clamped lengths (kept in registers, and
    // in LDS for the row pass)
    uint32_t rc[kSmallPer], pc[kSmallPer];
    uint32_t err = 0;
#pragma unroll
    for (int k = 0; k < kSmallPer; ++k) {
        const uint32_t e = e0 + (uint32_t)k;
        rc[k] = kNoSeq;
        pc[k] = 0;
        if (e < E) {
            const bool valid = l[k] != pv;
            if (args.Lp && ((lp[k] != pv) != valid)) err |= PSQ_DATA_TABLE_MISMATCH;
            if (valid) {
                if (l[k] < 0 || lp[k] < l[k]) err |= PSQ_DATA_BAD_LENGTH;
                const int64_t lim = (int64_t)sat;
                pc[k] = (uint32_t)(lp[k] < 0 ? 0 : (lp[k] > lim ? lim : lp[k]));
                rc[k] = (uint32_t)(l[k] < 0 ? 0 : (l[k] > lim ? lim : l[k]));
            }
        }
        m.real[e] = rc[k];
        m.phys[e] = pc[k];
    }
    if (err) atomicOr(&m.err, err);
    __syncthreads();

    // rows: a row needs a sequence and must fit S (its padded sum, saturated
    // at S+1, says so exactly); its tail pad is folded into its last
    // sequence.  Short rows take one thread each, longer rows one wave each
    // (kRowsAtOnce rows side by side per wave, so that their LDS reads and DPP
    // chains would overlap; one is fastest with 16 waves).
    if (P <= 32u) {
        for (uint32_t r = threadIdx.x; r < B; r += kSmallThreads) {
            uint32_t sum = 0, last = 0, last_pd = 0;
            int32_t mx = 0;
            for (uint32_t e = r * P; e < r * P + P; ++e) {
                const uint32_t rl = m.real[e];
                if (rl != kNoSeq) {
                    last_pd = m.phys[e];
                    sum = sat_add(sum, last_pd, sat);
                    last = e + 1u;
                    mx = max(mx, (int32_t)rl);
                }
            }
            uint32_t e2 = 0;
            if (last == 0) e2 |= PSQ_DATA_EMPTY_ROW;
            if (sum > S) e2 |= PSQ_DATA_ROW_OVERFLOW;
            if (e2) atomicOr(&m.err, e2);
            if (last) {
                m.phys[last - 1u] = last_pd + (S - sum);
                atomicMax(&m.g_last[r / Bc], last);
            }
            if (mx) atomicMax(&m.g_max[r / Bc], mx);
        }
    } else {
        constexpr int kRowsAtOnce = 1;
        uint32_t e2 = 0;
        for (uint32_t r0 = (uint32_t)w * kRowsAtOnce; r0 < B; r0 += kSmallWaves * kRowsAtOnce) {
            uint32_t sum[kRowsAtOnce], last[kRowsAtOnce], my_e[kRowsAtOnce], my_pd[kRowsAtOnce];
            int32_t mx[kRowsAtOnce];
#pragma unroll
            for (int q = 0; q < kRowsAtOnce; ++q) {
                const uint32_t r = r0 + (uint32_t)q;
                sum[q] = 0;
                last[q] = 0;
                my_e[q] = kNoSeq;   // + 1 wraps to 0: never a row's last
                my_pd[q] = 0;
                mx[q] = 0;
                if (r < B) {
                    for (uint32_t j = (uint32_t)lane; j < P; j += kWave) {
                        const uint32_t e = r * P + j;
                        const uint32_t rl = m.real[e];
                        if (rl != kNoSeq) {
                            const uint32_t pd = m.phys[e];
                            sum[q] = sat_add(sum[q], pd, sat);
                            last[q] = e + 1u;
                            my_e[q] = e;
                            my_pd[q] = pd;
                            mx[q] = max(mx[q], (int32_t)rl);
                        }
                    }
                }
            }
            // saturating wave sums and wave maxima over DPP (lane 63 holds them)
#pragma unroll
            for (int q = 0; q < kRowsAtOnce; ++q) {
                uint32_t x = sum[q];
                x = sat_add(x, (uint32_t)dpp0<0x111>((int)x), sat);
                x = sat_add(x, (uint32_t)dpp0<0x112>((int)x), sat);
                x = sat_add(x, (uint32_t)dpp0<0x114>((int)x), sat);
                x = sat_add(x, (uint32_t)dpp0<0x118>((int)x), sat);
                x = sat_add(x, (uint32_t)dpp0<0x142, 0xa>((int)x), sat);
                x = sat_add(x, (uint32_t)dpp0<0x143, 0xc>((int)x), sat);
                sum[q] = (uint32_t)read_lane((int)x, kWave - 1);
                last[q] = (uint32_t)read_lane(wave_incl_max((int)last[q]), kWave - 1);
                mx[q] = read_lane(wave_incl_max(mx[q]), kWave - 1);
            }
#pragma unroll
            for (int q = 0; q < kRowsAtOnce; ++q) {
                const uint32_t r = r0 + (uint32_t)q;
                if (r < B) {   // uniform
                    if (last[q] == 0) e2 |= PSQ_DATA_EMPTY_ROW;
                    if (sum[q] > S) e2 |= PSQ_DATA_ROW_OVERFLOW;
                    // the lane holding the row's last sequence folds it
                    if (last[q] && my_e[q] + 1u == last[q])
                        m.phys[my_e[q]] = my_pd[q] + (S - sum[q]);
                    if (lane == 0) {
                        if (last[q]) atomicMax(&m.g_last[r / Bc], last[q]);
                        if (mx[q]) atomicMax(&m.g_max[r / Bc], mx[q]);
                    }
                }
            }
        }
        if (lane == 0 && e2) atomicOr(&m.err, e2);
    }
    __syncthreads();

    // the fold changed some physical lengths: take them back from LDS
#pragma unroll
    for (int k = 0; k < kSmallPer; ++k) pc[k] = m.phys[e0 + (uint32_t)k];

    // one block-wide exclusive scan of (count, real, physical) over the
    // flattened table (wrapping sums: exact whenever no status bit is set)
    uint32_t cnt = 0, rsum = 0, psum = 0;
#pragma unroll
    for (int k = 0; k < kSmallPer; ++k) {
        if (rc[k] != kNoSeq) {
            cnt += 1;
            rsum += rc[k];
            psum += pc[k];
        }
    }
    uint32_t ex[3], tot[3];
    block_scan3<kSmallWaves>(m.wsum, cnt, rsum, psum, ex, tot);
    // group of entry e0, and the first entry of the next group
    const uint32_t g0 = min(e0, E - 1u) / Eg;
    {
        uint32_t c = ex[0], rr = ex[1], pp = ex[2];
        uint32_t g = g0, g_end = (g0 + 1u) * Eg;
#pragma unroll
        for (int k = 0; k < kSmallPer; ++k) {
            const uint32_t e = e0 + (uint32_t)k;
            if (e < E) {
                while (e >= g_end) {
                    ++g;
                    g_end += Eg;
                }
                if (e == g_end - Eg) {
                    m.g_base[0][g] = c;
                    m.g_base[1][g] = rr;
                    m.g_base[2][g] = pp;
                }
                if (rc[k] != kNoSeq) {
                    // every sequence but its group's last must be tight
                    if (e + 1u != m.g_last[g] && rc[k] != pc[k]) m.g_flag[g] = 1u;
                    c += 1;
                    rr += rc[k];
                    pp += pc[k];
                }
            }
        }
        if (threadIdx.x == 0) {
            m.g_base[0][G] = tot[0];
            m.g_base[1][G] = tot[1];
            m.g_base[2][G] = tot[2];
        }
    }
    __syncthreads();

    const uint32_t st = m.err;
    uint32_t width = 0;   // longest group's boundary count, n + 1
    if (st == 0)
        for (uint32_t g = 0; g < G; ++g) width = max(width, m.g_base[0][g + 1] - m.g_base[0][g] + 1u);
    const uint32_t stride = G > 1 ? width : 0u;   // output row of group g starts at g * stride

    // boundaries of every sequence (group-relative), then each group's close
    if (st == 0) {
        uint32_t c = ex[0], rr = ex[1], pp = ex[2];
        uint32_t g = g0, g_end = (g0 + 1u) * Eg;
#pragma unroll
        for (int k = 0; k < kSmallPer; ++k) {
            const uint32_t e = e0 + (uint32_t)k;
            if (rc[k] != kNoSeq) {
                while (e >= g_end) {
                    ++g;
                    g_end += Eg;
                }
                const uint32_t at = g * stride + (c - m.g_base[0][g]);
                cu[at] = (int32_t)(rr - m.g_base[1][g]);
                if (cp) cp[at] = (int32_t)(pp - m.g_base[2][g]);
                c += 1;
                rr += rc[k];
                pp += pc[k];
            }
        }
    }
    for (uint32_t g = threadIdx.x; g < G; g += kSmallThreads) {
        if (st == 0) {
            const uint32_t n = m.g_base[0][g + 1] - m.g_base[0][g];
            const uint32_t total = m.g_base[1][g + 1] - m.g_base[1][g];
            const bool disagree = m.g_flag[g] != 0;
            const bool absorbed = !disagree && total < Tc;
            int32_t mx = m.g_max[g];
            // without a status bit every row, hence every group, holds a sequence
            const uint32_t last = m.g_last[g];
            if (absorbed && last) mx = max(mx, (int32_t)(Tc - (total - m.real[last - 1u])));
            const uint32_t base = g * stride;
            cu[base + n] = (int32_t)(absorbed ? Tc : total);
            if (cp) cp[base + n] = (int32_t)Tc;
            for (uint32_t j = n + 1u; j < stride; ++j) {
                cu[base + j] = (int32_t)pv;
                if (cp) cp[base + j] = (int32_t)pv;
            }
            args.num_seqs[g] = (int32_t)n;
            args.max_seqlen[g] = mx;
            args.pad_between[g] = disagree ? 1 : 0;
        } else {
            args.num_seqs[g] = 0;
            args.max_seqlen[g] = 0;
            args.pad_between[g] = 0;
        }
    }
    if (threadIdx.x == 0) {
        *args.status = (int32_t)st;
        if (args.cu_width) *args.cu_width = (int32_t)(st == 0 ? width : 0u);
    }
}

// ---------------------------------------------------------------------------
// Tables of at most kRowsMax rows of at most one wave of entries (B <= 64,
// P <= 64): each wave owns whole rows, lane j holding entry j of rows w,
// w + 16, w + 32 and w + 48.  Validation, the row's saturating padded sum,
// its fold, its longest sequence, the in-row scans and the tightness test
// all run in registers (ballots and DPP scans), and one LDS exchange of the
// per-row totals, behind one barrier, places every row.  The predicates and
// outputs are those of thd_small_meta; on MI355X the 16 x 64 tables of the
// length-table workload finish workgroup 0 in about half the time, because
// the general path's five barrier-separated phases each wait about 1 us on
// chains of dependent LDS accesses.
// ---------------------------------------------------------------------------
constexpr uint32_t kRowsPerWave = 4;
constexpr uint32_t kRowsMax = kRowsPerWave * (uint32_t)kSmallWaves;   // 64 rows

struct RowsMeta {
    uint32_t rt[3][kRowsMax];               // per row: sequences, real sum, folded padded sum
    uint32_t g_flag[kSmallGroups];          // an interior boundary departs from its physical one
    int32_t g_max[kSmallGroups];            // largest real length of the group
    uint32_t g_last_real[kSmallGroups];     // real length of the group's last sequence
    uint32_t err;
};

// wrapping inclusive sum over the wave
__device__ __forceinline__ uint32_t wave_incl_add(uint32_t x) {
    x += (uint32_t)dpp0<0x111>((int)x);
    x += (uint32_t)dpp0<0x112>((int)x);
    x += (uint32_t)dpp0<0x114>((int)x);
    x += (uint32_t)dpp0<0x118>((int)x);
    x += (uint32_t)dpp0<0x142, 0xa>((int)x);
    x += (uint32_t)dpp0<0x143, 0xc>((int)x);
    return x;
}

bool rows_tables(uint32_t B, uint32_t P) { return B <= kRowsMax && P <= (uint32_t)kWave; }

template <typename TL>
__device__ __forceinline__ void thd_rows_meta(const ThdArgs<TL> &args, RowsMeta &m) {
    const uint32_t B = args.B, P = args.P, S = args.S, G = args.G, Bc = args.Bc;
    const uint32_t Tc = Bc * S;     // tokens of one group (< 2^31)
    const uint32_t sat = S + 1u;    // clamp of a length, and of a row's padded sum
    const bool small_s = S < (1u << 25);
    const int64_t pv = args.pad_value;
    const TL *__restrict__ L = args.L;
    const TL *__restrict__ Lq = args.Lp ? args.Lp : args.L;
    const bool has_lp = args.Lp != nullptr;
    int32_t *__restrict__ cu = args.cu;
    int32_t *__restrict__ cp = args.cp;
    const uint32_t w = (uint32_t)wave_id();
    const uint32_t j = (uint32_t)lane_id();
    // a row's group (uniform; no division when there is one group)
    auto group_of = [G, Bc](uint32_t r) -> uint32_t { return G == 1 ? 0u : r / Bc; };

    if (threadIdx.x < kSmallGroups) {
        m.g_flag[threadIdx.x] = 0;
        m.g_max[threadIdx.x] = 0;
    }
    if (threadIdx.x == 0) m.err = 0;

    // every load is issued before any is used; lanes outside the table read
    // as unused slots
    int64_t l[kRowsPerWave], lp[kRowsPerWave];
#pragma unroll
    for (uint32_t i = 0; i < kRowsPerWave; ++i) {
        const uint32_t r = w + i * (uint32_t)kSmallWaves;
        l[i] = pv;
        lp[i] = pv;
        if (r < B && j < P) {
            l[i] = (int64_t)L[r * P + j];
            lp[i] = (int64_t)Lq[r * P + j];
        }
    }
    __syncthreads();   // the zeroed accumulators before any update

    // each row: validity, the length checks, clamped lengths, the padded sum
    // (saturated at S+1, so ROW_OVERFLOW is exact), the fold of the tail pad
    // into the row's last sequence, and exclusive in-row scans
    uint32_t exc[kRowsPerWave], exr[kRowsPerWave], exq[kRowsPerWave];
    bool val[kRowsPerWave];
    uint32_t err = 0;
#pragma unroll
    for (uint32_t i = 0; i < kRowsPerWave; ++i) {
        const uint32_t r = w + i * (uint32_t)kSmallWaves;
        const bool valid = l[i] != pv;
        if (has_lp && ((lp[i] != pv) != valid)) err |= PSQ_DATA_TABLE_MISMATCH;
        uint32_t r_c = 0, p_c = 0;
        if (valid) {
            if (l[i] < 0 || lp[i] < l[i]) err |= PSQ_DATA_BAD_LENGTH;
            const int64_t lim = (int64_t)sat;
            p_c = (uint32_t)(lp[i] < 0 ? 0 : (lp[i] > lim ? lim : lp[i]));
            r_c = (uint32_t)(l[i] < 0 ? 0 : (l[i] > lim ? lim : l[i]));
        }
        val[i] = valid;
        exc[i] = exr[i] = exq[i] = 0;
        if (r < B) {   // uniform
            const uint64_t vm = __ballot(valid);
            const uint32_t last_j = vm ? 63u - (uint32_t)__clzll(vm) : 0u;
            const bool is_last = vm != 0 && j == last_j;
            uint32_t sum, ir, ip;
            const int32_t mx = read_lane(wave_incl_max((int)r_c), kWave - 1);
            if (small_s) {   // uniform
                // 64 clamped lengths of at most S + 1 < 2^25 + 1 sum without
                // wrapping: plain scans, and the folded padded scan is the
                // unfolded one plus the fold from the row's last entry on
                const uint32_t ipre = wave_incl_add(p_c);
                sum = (uint32_t)read_lane((int)ipre, kWave - 1);
                const uint32_t fold = S - sum;   // matters only if sum <= S
                if (is_last) p_c += fold;
                ir = wave_incl_add(r_c);
                ip = ipre + ((vm != 0 && j >= last_j) ? fold : 0u);
            } else {
                sum = (uint32_t)read_lane((int)wave_incl_sat(p_c, sat), kWave - 1);
                if (is_last) p_c += S - sum;   // the fold (its value matters only if sum <= S)
                ir = wave_incl_add(r_c);
                ip = wave_incl_add(p_c);
            }
            exc[i] = (uint32_t)__popcll(vm & ((1ull << j) - 1ull));
            exr[i] = ir - r_c;
            exq[i] = ip - p_c;
            const uint32_t g = group_of(r);
            const bool group_last_row = r + 1u == (g + 1u) * Bc;
            // every sequence but its group's last must be tight
            const bool loose = valid && r_c != p_c && !(group_last_row && is_last);
            const bool any_loose = __ballot(loose) != 0;
            const uint32_t tot_r = (uint32_t)read_lane((int)ir, kWave - 1);
            const uint32_t tot_p = (uint32_t)read_lane((int)ip, kWave - 1);
            if (j == 0) {
                uint32_t e2 = 0;
                if (vm == 0) e2 |= PSQ_DATA_EMPTY_ROW;
                if (sum > S) e2 |= PSQ_DATA_ROW_OVERFLOW;
                if (e2) atomicOr(&m.err, e2);
                m.rt[0][r] = (uint32_t)__popcll(vm);
                m.rt[1][r] = tot_r;
                m.rt[2][r] = tot_p;
                if (any_loose) atomicOr(&m.g_flag[g], 1u);
                if (mx > 0) atomicMax(&m.g_max[g], mx);
            }
            if (group_last_row && is_last) m.g_last_real[g] = r_c;
        }
    }
    if (err) atomicOr(&m.err, err);
    __syncthreads();

    const uint32_t st = m.err;
    // inclusive scans of the row totals: lane x holds rows 0 .. x
    const uint32_t ic = wave_incl_add(j < B ? m.rt[0][j] : 0u);
    const uint32_t ir = wave_incl_add(j < B ? m.rt[1][j] : 0u);
    const uint32_t ip = wave_incl_add(j < B ? m.rt[2][j] : 0u);
    // sum over rows 0 .. x-1 (x uniform, <= B)
    auto pre = [](uint32_t v, uint32_t x) -> uint32_t {
        return x ? (uint32_t)read_lane((int)v, (int)x - 1) : 0u;
    };
    // longest group's boundary count, n + 1: lane g holds group g's.  The
    // shuffles run on every lane (a source lane outside the exec mask would
    // read as 0); lanes past the groups read lane 0 and are discarded.
    uint32_t width;
    if (G == 1) {   // uniform: one group, the whole table
        width = (uint32_t)read_lane((int)ic, (int)B - 1) + 1u;
    } else {
        const uint32_t g_hi = j < G ? (j + 1u) * Bc - 1u : 0u;
        const uint32_t g_lo = (j < G && j) ? j * Bc - 1u : 0u;
        const uint32_t c_hi = (uint32_t)__shfl((int)ic, (int)g_hi);
        const uint32_t c_lo = (uint32_t)__shfl((int)ic, (int)g_lo);
        const uint32_t n_lane = j < G ? c_hi - (j ? c_lo : 0u) + 1u : 0u;
        width = (uint32_t)read_lane(wave_incl_max((int)n_lane), kWave - 1);
    }
    const uint32_t stride = G > 1 ? width : 0u;   // output row of group g starts at g * stride

    // boundaries of every sequence (group-relative)
    if (st == 0) {
#pragma unroll
        for (uint32_t i = 0; i < kRowsPerWave; ++i) {
            const uint32_t r = w + i * (uint32_t)kSmallWaves;
            if (r < B) {   // uniform
                const uint32_t g = group_of(r), r0 = g * Bc;
                const uint32_t bc = pre(ic, r) - pre(ic, r0);
                const uint32_t br = pre(ir, r) - pre(ir, r0);
                const uint32_t bp = pre(ip, r) - pre(ip, r0);
                if (val[i]) {
                    const uint32_t at = g * stride + bc + exc[i];
                    cu[at] = (int32_t)(br + exr[i]);
                    if (cp) cp[at] = (int32_t)(bp + exq[i]);
                }
            }
        }
    }
    // each group's close, the sentinel fill of its stacked row, its scalars
    for (uint32_t g = w; g < G; g += (uint32_t)kSmallWaves) {   // uniform
        const uint32_t r0 = g * Bc, r1 = r0 + Bc;
        if (st == 0) {
            const uint32_t n = pre(ic, r1) - pre(ic, r0);
            const uint32_t total = pre(ir, r1) - pre(ir, r0);
            const bool disagree = m.g_flag[g] != 0;
            const bool absorbed = !disagree && total < Tc;
            int32_t mx = m.g_max[g];
            // without a status bit every row, hence every group, holds a sequence
            if (absorbed && n) mx = max(mx, (int32_t)(Tc - (total - m.g_last_real[g])));
            const uint32_t base = g * stride;
            if (j == 0) {
                cu[base + n] = (int32_t)(absorbed ? Tc : total);
                if (cp) cp[base + n] = (int32_t)Tc;
                args.num_seqs[g] = (int32_t)n;
                args.max_seqlen[g] = mx;
                args.pad_between[g] = disagree ? 1 : 0;
            }
            for (uint32_t x = n + 1u + j; x < stride; x += (uint32_t)kWave) {
                cu[base + x] = (int32_t)pv;
                if (cp) cp[base + x] = (int32_t)pv;
            }
        } else if (j == 0) {
            args.num_seqs[g] = 0;
            args.max_seqlen[g] = 0;
            args.pad_between[g] = 0;
        }
    }
    if (threadIdx.x == 0) {
        *args.status = (int32_t)st;
        if (args.cu_width) *args.cu_width = (int32_t)(st == 0 ? width : 0u);
    }
}

// 4 mask bits (1 = padding) -> 4 bytes of 0/1
__device__ __forceinline__ uint32_t spread4(uint32_t x) {
    return (x & 1u) | ((x & 2u) << 7) | ((x & 4u) << 14) | ((x & 8u) << 21);
}

// One (row, chunk of kSmallSlots) of the mask.  Each wave owns 1024 slots of
// the chunk and each lane 16 consecutive slots of it.  The wave reads its row's table 64
// entries at a time (one per lane), turns the padded lengths into physical
// starts with a saturating DPP scan, and visits, through a ballot, only the
// sequences whose tokens meet the wave's slots; a lane marks its slots that
// fall in [start, start + real) and stores its 16 mask bytes at once.  No
// LDS and no barrier.
template <typename TL>
__device__ __forceinline__ void thd_small_mask(const ThdArgs<TL> &args, uint32_t wg,
                                               uint32_t n_mchunks) {
    const uint32_t P = args.P, S = args.S;
    const uint32_t r = wg / n_mchunks, c = wg % n_mchunks;
    const int w = wave_id(), lane = lane_id();
    constexpr uint32_t kWaveSlots = kSmallSlots / kSmallWaves;
    const uint32_t lo = c * kSmallSlots + (uint32_t)w * kWaveSlots;
    const uint32_t hi = min(S, lo + kWaveSlots);
    if (lo >= hi) return;   // wave-uniform
    const uint32_t sat = S + 1u;
    const int64_t pv = args.pad_value;
    const TL *__restrict__ L = args.L + (uint64_t)r * P;
    const TL *__restrict__ Lq = (args.Lp ? args.Lp : args.L) + (uint64_t)r * P;
    const uint32_t a = lo + 16u * (uint32_t)lane;   // this lane's first slot
    uint32_t tok = 0;                               // bit i: slot a + i holds a token
    uint32_t run = 0;                               // padded sum of earlier batches (saturated)
    for (uint32_t j0 = 0; j0 < P && run < hi; j0 += kWave) {   // uniform
        const uint32_t j = j0 + (uint32_t)lane;
        uint32_t rl = 0, pd = 0;
        if (j < P) {
            const int64_t x = (int64_t)L[j];
            const int64_t y = (int64_t)Lq[j];
            if (x != pv) {
                const int64_t lim = (int64_t)sat;
                pd = (uint32_t)(y < 0 ? 0 : (y > lim ? lim : y));
                rl = (uint32_t)(x < 0 ? 0 : (x > lim ? lim : x));
            }
        }
        uint32_t incl = pd;
        incl = sat_add(incl, (uint32_t)dpp0<0x111>((int)incl), sat);
        incl = sat_add(incl, (uint32_t)dpp0<0x112>((int)incl), sat);
        incl = sat_add(incl, (uint32_t)dpp0<0x114>((int)incl), sat);
        incl = sat_add(incl, (uint32_t)dpp0<0x118>((int)incl), sat);
        incl = sat_add(incl, (uint32_t)dpp0<0x142, 0xa>((int)incl), sat);
        incl = sat_add(incl, (uint32_t)dpp0<0x143, 0xc>((int)incl), sat);
        const uint32_t st = sat_add(run, (uint32_t)wave_shr1((int)incl, 0), sat);
        const uint32_t en = sat_add(st, rl, sat);   // tokens of entry j: [st, en)
        run = sat_add(run, (uint32_t)read_lane((int)incl, kWave - 1), sat);
        uint64_t meet = __ballot(en > st && st < hi && en > lo);
        while (meet) {   // uniform
            const int q = __builtin_ctzll(meet);
            meet &= meet - 1ull;
            const uint32_t s0 = (uint32_t)read_lane((int)st, q);
            const uint32_t s1 = (uint32_t)read_lane((int)en, q);
            const uint32_t b0 = max(s0, a), b1 = min(s1, a + 16u);
            if (b0 < b1) tok |= ((1u << (b1 - a)) - 1u) & ~((1u << (b0 - a)) - 1u);
        }
    }
    uint8_t *__restrict__ out = args.mask + (uint64_t)r * S;
    const uint32_t pad = ~tok & 0xffffu;   // 1 = padding
    if (args.vec_mask && ((uint64_t)r * S) % 16 == 0 && a + 16u <= hi) {
        *(u32x4 *)(out + a) = u32x4{spread4(pad), spread4(pad >> 4), spread4(pad >> 8),
                                    spread4(pad >> 12)};
    } else {
        for (uint32_t i = 0; i < 16u && a + i < hi; ++i) out[a + i] = (uint8_t)((pad >> i) & 1u);
    }
}

template <typename TL, int kPer>
__global__ __launch_bounds__(kSmallThreads) void k_thd_small(ThdArgs<TL> a, uint32_t n_mask,
                                                             uint32_t n_mchunks,
                                                             CopyBatch batch) {
    if (blockIdx.x == 0) {
        if constexpr (kPer == 0) {
            __shared__ RowsMeta meta;
            thd_rows_meta<TL>(a, meta);
        } else {
            __shared__ SmallMeta<kPer> meta;
            thd_small_meta<TL, kPer>(a, meta);
        }
    } else if (blockIdx.x <= n_mask)
        thd_small_mask<TL>(a, blockIdx.x - 1u, n_mchunks);
    else
        copy_group<kSmallThreads, u32x4, true>(batch, (int64_t)blockIdx.x - 1 - n_mask);
}

bool small_tables(int64_t B, int64_t P, int64_t S, int64_t G) {
    return B >= 1 && P >= 1 && S >= 1 && (uint64_t)B * (uint64_t)P <= kSmallEntries &&
           G <= (int64_t)kSmallGroups;
}

template <typename TL>
bool small_tables(const ThdArgs<TL> &a) {
    return small_tables(a.B, a.P, a.S, a.G);
}

// Threads of the launch carrying the metadata (and the fused 16-byte copies):
// the single-workgroup kernel for small tables, else one workgroup per row
// chunk.  The copies launched alone are bounded by their unit count.
uint64_t thd_meta_threads(int64_t B, int64_t P, int64_t S, int64_t G, const CopyPlan &plan) {
    if (small_tables(B, P, S, G)) {
        const uint64_t n_mask = (uint64_t)B * (((uint64_t)S + kSmallSlots - 1) / kSmallSlots);
        return (1ull + n_mask + (uint64_t)plan.groups[0]) * (uint64_t)kSmallThreads;
    }
    const uint64_t n_chunks = S > 0 ? ((uint64_t)S + kSlots - 1) / kSlots : 1ull;
    const uint64_t n_meta = B > 0 ? (uint64_t)B * n_chunks : 1ull;
    return (n_meta + (uint64_t)plan.groups[0]) * (uint64_t)kThreads;
}

template <typename TL>
hipError_t launch_typed(ThdArgs<TL> a, uint32_t n_meta, const psq_copy *copies, int n_copies,
                        hipStream_t stream) {
    CopyPlan plan;
    const bool small = small_tables(a);
    plan_copies(copies, n_copies, &plan, small ? kSmallThreads : kThreads);
    if (thd_meta_threads(a.B, a.P, a.S, a.G, plan) > kMaxGridThreads)
        return hipErrorInvalidConfiguration;
    if (small) {
        const uint32_t n_mchunks = (a.S + kSmallSlots - 1u) / kSmallSlots;
        const uint32_t n_mask = a.mask ? a.B * n_mchunks : 0u;
        const uint64_t grid = 1ull + n_mask + (uint64_t)plan.groups[0];
        const bool two = (uint64_t)a.B * a.P <= (uint64_t)2 * kSmallThreads;
        hipLaunchKernelGGL((rows_tables(a.B, a.P) ? k_thd_small<TL, 0>
                            : two               ? k_thd_small<TL, 2>
                                                : k_thd_small<TL, kSmallPerMax>),
                           dim3((uint32_t)grid), dim3(kSmallThreads), 0, stream, a, n_mask,
                           n_mchunks, plan.batch[0]);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        return launch_copy_plan(plan, 1, stream);
    }
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

bool thd_tables_grid_fits(int64_t B, int64_t P, int64_t S, int64_t G, const psq_copy *copies,
                          int n_copies) {
    CopyPlan plan;
    plan_copies(copies, n_copies, &plan, small_tables(B, P, S, G) ? kSmallThreads : kThreads);
    return thd_meta_threads(B, P, S, G, plan) <= kMaxGridThreads;
}

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
    // with no rows the row length changes no output; any S is accepted there
    // (B * S = 0), so it is not carried into the kernels' 32-bit arithmetic
    if (B == 0) S = 0;
    const uint32_t n_chunks = S > 0 ? (uint32_t)(((uint64_t)S + kSlots - 1) / kSlots) : 1u;
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
