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
// from there: no workgroup waits on another for the mask.  The chunk-0
// workgroup of each row also takes part in a decoupled look-back over rows
// carrying (sequence count, real-token sum) and writes the row's entries of
// cu_seqlens / cu_seqlens_padded.  The last workgroup to finish applies the
// absorption and writes the scalars.
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

template <typename TL>
struct ThdArgs {
    const TL *L, *Lp;
    uint32_t B, P, S;
    int64_t pad_value;
    uint32_t n_chunks;
    int vec_mask;
    int32_t *cu, *cp, *num_seqs, *max_seqlen, *pad_between;
    uint8_t *mask;
    int32_t *status;
    WsHeader *ws;
};

// One (row, chunk) per workgroup; `n_groups` is the number of workgroups
// running this body (the launch may append copy workgroups after them).
template <typename TL>
__device__ __forceinline__ void thd_tables_body(
    const TL *__restrict__ L, const TL *__restrict__ Lp, uint32_t B, uint32_t P, uint32_t S,
    int64_t pad_value, uint32_t n_chunks, int vec_mask, int32_t *__restrict__ cu,
    int32_t *__restrict__ cp, int32_t *__restrict__ num_seqs, int32_t *__restrict__ max_seqlen,
    int32_t *__restrict__ pad_between, uint8_t *__restrict__ mask, int32_t *__restrict__ status,
    WsHeader *__restrict__ ws, uint32_t n_groups) {
    __shared__ RowLds s;
    __shared__ __attribute__((aligned(16))) uint8_t s_mask[kSlots];
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
    const uint64_t T = (uint64_t)B * S;
    const int lane = lane_id();

    if ((uint64_t)ticket < (uint64_t)B * n_chunks) {
        const uint32_t r = ticket / n_chunks;
        const uint32_t c = ticket % n_chunks;
        const bool leader = (c == 0);
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
            for (uint32_t u = b_lo + threadIdx.x; u < b_hi; u += kThreads) {
                // last sequence of the batch starting at or before u
                uint32_t a = 0, b = nb;
                while (b - a > 1) {
                    const uint32_t m = (a + b) >> 1;
                    if ((uint32_t)s.start[m] <= u) a = m; else b = m;
                }
                const bool tok = (u - (uint32_t)s.start[a]) < (uint32_t)s.real[a];
                s_mask[u - lo] = tok ? 0 : 1;
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
            if (r + 1 < B && count) disagree = disagree || last_untight_folded;

            // look-back over rows: (sequence count, real-token sum)
            if (threadIdx.x < kWave) {
                uint32_t ex_a = 0, ex_b = 0;
                if (r == 0) {
                    if (lane == 0) st_relaxed(desc, desc_pack(kDescIncl, count, realsum));
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
            const uint64_t cap = (uint64_t)B * P;     // caller capacity is B*P+1
            bool oob = (uint64_t)ex_a + count > cap;

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
                    cu[idx] = (int32_t)(ex_b + (uint32_t)s.rpre[k]);
                    if (cp) cp[idx] = (int32_t)(r * S + (uint32_t)s.start[k]);
                }
                __syncthreads();
                if (one_batch || j0 + kBatch >= P) break;
            }

            if (threadIdx.x == 0) {
                if (oob) err |= PSQ_DATA_WORKSPACE;
                err |= s_wserr;
                if (err) or_relaxed(&ws->status, err);
                if (disagree) or_relaxed(&ws->flags, 1u);
                if (s.max_real > 0) max_relaxed(&ws->max, s.max_real);
                if (r == B - 1 && !oob) {
                    const uint32_t n = ex_a + count;
                    const uint32_t total = ex_b + realsum;
                    st_relaxed((uint32_t *)&ws->n, n);
                    st_relaxed((uint32_t *)&ws->total, total);
                    st_relaxed((uint32_t *)&ws->cu_last, total - (uint32_t)s.last_real);
                }
            }
        }
    } else if (B > 0 && threadIdx.x == 0) {
        or_relaxed(&ws->status, PSQ_DATA_WORKSPACE);
    }

    if (finish_is_last(ws, n_groups, &s_slot)) {
        if (threadIdx.x == 0) {
            const uint32_t st = ld_relaxed(&ws->status);
            const uint32_t n = ld_relaxed((const uint32_t *)&ws->n);
            const uint32_t total = ld_relaxed((const uint32_t *)&ws->total);
            const uint32_t cu_last = ld_relaxed((const uint32_t *)&ws->cu_last);
            const bool disagree = ld_relaxed(&ws->flags) != 0;
            int32_t mx = (int32_t)ld_relaxed((const uint32_t *)&ws->max);
            if (st == 0 && (uint64_t)n <= (uint64_t)B * P) {
                const bool absorbed = !disagree && (uint64_t)total < T;
                cu[n] = (int32_t)(absorbed ? (uint32_t)T : total);
                if (cp) cp[n] = (int32_t)T;
                if (absorbed) mx = max(mx, (int32_t)((uint32_t)T - cu_last));
                *num_seqs = (int32_t)n;
                *max_seqlen = mx;
                *pad_between = disagree ? 1 : 0;
            } else {
                *num_seqs = 0;
                *max_seqlen = 0;
                *pad_between = 0;
            }
            *status = (int32_t)st;
            st_relaxed(&ws->status, 0u);
            st_relaxed(&ws->flags, 0u);
            st_relaxed((uint32_t *)&ws->max, 0u);
            st_relaxed((uint32_t *)&ws->n, 0u);
            st_relaxed((uint32_t *)&ws->total, 0u);
            st_relaxed((uint32_t *)&ws->cu_last, 0u);
            st_relaxed(&ws->ticket, 0u);
        }
        for (uint32_t i = threadIdx.x; i < B; i += kThreads) st_relaxed(desc + i, 0ull);
        __syncthreads();
        if (threadIdx.x == 0) st_relaxed(&ws->done, 0u);
    }
}

#define PSQ_THD_ARGS(a)                                                                       \
    a.L, a.Lp, a.B, a.P, a.S, a.pad_value, a.n_chunks, a.vec_mask, a.cu, a.cp, a.num_seqs,    \
        a.max_seqlen, a.pad_between, a.mask, a.status, a.ws

template <typename TL>
__global__ __launch_bounds__(kThreads) void k_thd_tables(ThdArgs<TL> a) {
    thd_tables_body<TL>(PSQ_THD_ARGS(a), gridDim.x);
}

// The same workgroups followed, in one grid, by the 16-byte dense copies of
// the THD collapse: one launch per call instead of two.
template <typename TL>
__global__ __launch_bounds__(kThreads) void k_thd_tables_copy(ThdArgs<TL> a, uint32_t n_meta,
                                                              CopyBatch batch) {
    if (blockIdx.x < n_meta)
        thd_tables_body<TL>(PSQ_THD_ARGS(a), n_meta);
    else
        copy_group<u32x4, true>(batch, (int64_t)blockIdx.x - n_meta);
}
#undef PSQ_THD_ARGS

template <typename TL>
hipError_t launch_typed(ThdArgs<TL> a, uint32_t n_meta, const psq_copy *copies, int n_copies,
                        hipStream_t stream) {
    CopyPlan plan;
    plan_copies(copies, n_copies, &plan);
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

size_t thd_tables_workspace(int64_t B, int64_t /*S*/) {
    return round_up(kWsDescOffset + 8 * (size_t)(B > 0 ? B : 1), 256);
}

hipError_t launch_thd_tables(const void *L, const void *Lp, int lens_dtype, int64_t B,
                             int64_t P, int64_t S, int64_t pad_value, int32_t *cu,
                             int32_t *cp, int32_t *num_seqs, int32_t *max_seqlen,
                             int32_t *pad_between, uint8_t *mask, int32_t *status,
                             void *workspace, const psq_copy *copies, int n_copies,
                             hipStream_t stream) {
    const uint32_t n_chunks = S > 0 ? (uint32_t)((S + kSlots - 1) / kSlots) : 1u;
    const uint64_t groups = (uint64_t)B * n_chunks;
    const uint32_t n_meta = (uint32_t)(groups > 0 ? groups : 1);
    const int vec_mask = ((uintptr_t)mask % 16) == 0;
    WsHeader *ws = (WsHeader *)workspace;
    if (lens_dtype == PSQ_I64) {
        ThdArgs<int64_t> a{(const int64_t *)L, (const int64_t *)Lp, (uint32_t)B, (uint32_t)P,
                           (uint32_t)S, pad_value, n_chunks, vec_mask, cu, cp, num_seqs,
                           max_seqlen, pad_between, mask, status, ws};
        return launch_typed(a, n_meta, copies, n_copies, stream);
    }
    ThdArgs<int32_t> a{(const int32_t *)L, (const int32_t *)Lp, (uint32_t)B, (uint32_t)P,
                       (uint32_t)S, pad_value, n_chunks, vec_mask, cu, cp, num_seqs,
                       max_seqlen, pad_between, mask, status, ws};
    return launch_typed(a, n_meta, copies, n_copies, stream);
}

}  // namespace psq
