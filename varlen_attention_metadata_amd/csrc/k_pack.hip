// k_pack.hip -- the squeeze of padded sources into fixed-capacity packs.
//
// "Who packs the sequences: the loader, or the trainer?", What the data
// looks like at each hop.  Trainer packs: each source is padded to a
// multiple of q and the sources of a bin are laid end to end
// (cu_seqlens [0,5,15], cu_seqlens_padded [0,8,20]).  Loader packs: the row
// is always `capacity` wide, the tail is pad, token_mask is 1 where a token
// counts, and the last padded boundary becomes the capacity
// (cu_seqlens_padded [0,8,36]).
//
// Work layout: one single-wave workgroup (64 threads) per (pack, chunk of
// 896 slots; 256 when 896-slot chunks would give fewer than 1024
// workgroups: a trainer batch of 15 bins then takes 9.5 instead of 11.6 us).
// The wave scans its pack's member lengths into LDS (64 members per batch;
// a saturating scan so an overfull pack is detected exactly).  Each lane
// then finds its slots' owners among the few members that meet the chunk,
// comparing their starts in registers (on MI355X 0.4 % faster on the
// 65536-source workload than a per-chunk owner map filled in LDS by a max
// scan, 3 % on the trainer batch), and every slot takes either its member's
// token or the pad token.  Lane l owns slots l, l+64, l+128, ... of the
// chunk, so every load and store instruction of the wave covers 64
// consecutive slots.  Every slot issues
// its load (a pad slot re-reads a token of its own member, which is already
// in flight), so the loads are straight-line code and the stores wait only
// for the loads they need.  On MI355X this shape beat 256-thread workgroups
// over 4096 slots by 4 %: a one-wave workgroup synchronizes cheaply, and more
// of them stay resident.  Token-mask bytes are staged in LDS and leave as
// 16-byte stores.  Every global load and store of the data is non-temporal
// (each byte is touched once): on MI355X that took the 65536-source workload
// from 194 to 173 us; non-temporal stores alone were slower (212 us), the
// loads alone 181 us.  The stores are the compiler's non-temporal stores:
// the collapse copy's agent-scope streaming stores (inline assembly) gained
// only 0.4 % here (161.7 against 162.3 us), against 2 % on the copy.
// The chunk-0 workgroup of each pack also writes the pack's boundary arrays
// and reports data errors through one relaxed 64-bit word (finished count |
// status bits); the last of those to finish publishes *status.
// Every access is bounds-checked against the caller's sizes, so bad data
// can only produce wrong values and status bits, never a stray access.
//
// Trainer path from the padded rectangle (src_off == NULL): source i is row
// i of an [N, src_stride] array, so its offset is i * src_stride and a length
// beyond the row is a BAD_LENGTH.
#include "psq_device.hpp"
#include "psq_internal.hpp"

namespace psq {
namespace {

constexpr int kThreads = 64;
constexpr int kWaves = kThreads / kWave;
constexpr int kMembers = kThreads;       // members per LDS batch
// Slots per workgroup: 896, or 256 when 896-slot chunks would leave most of
// the chip idle (fewer than kFillGroups workgroups).  896 slots (14 per lane)
// hold 85 VGPRs (88 allocated), so 5 waves per SIMD stay resident, as at 1024
// slots; on MI355X the 65536-source workload took 160 us this way, against
// 168.5 us at 1024 (16 loads per lane), 162-164 us at 640 or 768 and 168 us at
// 512.  Built for 6, 7 or 8 waves per SIMD the compiler spills, and the
// workload took 166, 225 and 278 us.
constexpr uint32_t kBigSlots = 896;
constexpr uint32_t kSmallSlots = 256;
constexpr uint64_t kFillGroups = 1024;

// 4 to 5 waves per SIMD: 5 measured best for this shape (6 were slower).
template <uint32_t kSlots>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4, 5))) void k_pack_rows(
    const int64_t *__restrict__ src, int64_t src_len, const int64_t *__restrict__ src_off,
    int64_t src_stride, const int32_t *__restrict__ real_len, int64_t N, int32_t q,
    const int32_t *__restrict__ order, const int64_t *__restrict__ pack_start, int64_t P,
    int32_t C, int fold, int64_t pad_token, int64_t *__restrict__ packed,
    uint8_t *__restrict__ tmask, int32_t *__restrict__ cu, int32_t *__restrict__ cp,
    int32_t *__restrict__ status, WsHeader *__restrict__ ws, uint32_t n_chunks, int vec_mask) {
    constexpr int kPerThread = (int)(kSlots / kThreads);   // slots per thread: one round
    static_assert(kSlots % 16 == 0 && kSlots % kThreads == 0, "whole 16-byte LDS stores");
    __shared__ uint32_t m_start[kMembers];
    __shared__ uint32_t m_real[kMembers];
    __shared__ int64_t m_so[kMembers];
    __shared__ __attribute__((aligned(16))) uint8_t s_mask[kSlots];
    __shared__ uint32_t s_wsum[2][kWaves];
    __shared__ uint32_t s_err;

    if (P == 0) {
        if (blockIdx.x == 0 && threadIdx.x == 0) *status = 0;
        return;
    }
    const int64_t p = blockIdx.x / n_chunks;
    const uint32_t c = blockIdx.x % n_chunks;
    const bool leader = (c == 0);
    const int w = wave_id(), lane = lane_id();
    const uint32_t sat = (uint32_t)C + 1u;
    const uint32_t lo = c * kSlots;
    const uint32_t hi = min((uint32_t)C, lo + kSlots);

    const int64_t a = pack_start[p];
    const int64_t b = pack_start[p + 1];
    // every slot loads from here; without any source tokens the loads go to
    // pack_start (never empty) and are discarded
    const int64_t *__restrict__ srcp = src_len > 0 ? src : pack_start;
    const bool range_ok = a >= 0 && b <= N && a <= b;
    const int64_t k = range_ok ? b - a : 0;
    if (threadIdx.x == 0) s_err = range_ok ? (k == 0 ? PSQ_DATA_EMPTY_PACK : 0u) : PSQ_DATA_BAD_INDEX;
    for (uint32_t u = threadIdx.x * 16u; u < kSlots; u += kThreads * 16u)
        *(u32x4 *)(s_mask + u) = u32x4{0u, 0u, 0u, 0u};

    int64_t *__restrict__ row = packed + p * (int64_t)C;
    const int64_t csr = a + p;            // this pack's first boundary entry
    if (leader && range_ok && threadIdx.x == 0) {
        cu[csr] = 0;
        cp[csr] = 0;
    }

    uint32_t carry_pos = 0, carry_real = 0;
    for (int64_t m0 = 0; m0 < k; m0 += kMembers) {
        // ---- member lengths of this batch -> starts (saturating scan) ----
        const int64_t j = m0 + threadIdx.x;
        uint32_t real = 0, padded = 0;
        int64_t so = 0;
        bool readable = false;
        uint32_t err = 0;
        if (j < k) {
            const int64_t i = order ? (int64_t)order[a + j] : a + j;
            if (i < 0 || i >= N) {
                err |= PSQ_DATA_BAD_INDEX;
            } else {
                int64_t r = real_len[i];
                so = src_off ? src_off[i] : i * src_stride;
                // a member with a bad length is not checked further: its
                // offset is not looked at and it counts as empty
                if (r < 0 || (!src_off && r > src_stride)) {
                    err |= PSQ_DATA_BAD_LENGTH;
                    r = 0;
                } else if (so < 0 || so > src_len - r) {
                    err |= PSQ_DATA_BAD_INDEX;
                } else {
                    readable = true;
                }
                const int64_t pd = (r + q - 1) / q * q;
                padded = pd > (int64_t)sat ? sat : (uint32_t)pd;
                real = r > (int64_t)sat ? sat : (uint32_t)r;
            }
        }
        if (err) atomicOr(&s_err, err);
        const uint32_t ip = wave_incl_sat(padded, sat);
        const uint32_t ir = wave_incl_sat(real, sat);
        if (lane == kWave - 1) {
            s_wsum[0][w] = ip;
            s_wsum[1][w] = ir;
        }
        __syncthreads();
        uint32_t bp = 0, br = 0, tp = 0, tr = 0;
#pragma unroll
        for (int v = 0; v < kWaves; ++v) {
            if (v == w) {
                bp = tp;
                br = tr;
            }
            tp = sat_add(tp, s_wsum[0][v], sat);
            tr = sat_add(tr, s_wsum[1][v], sat);
        }
        const uint32_t incl_pos = sat_add(carry_pos, sat_add(bp, ip, sat), sat);
        const uint32_t incl_real = sat_add(carry_real, sat_add(br, ir, sat), sat);
        const uint32_t start = incl_pos >= padded ? incl_pos - padded : 0u;
        m_start[threadIdx.x] = j < k ? start : 0xffffffffu;
        m_real[threadIdx.x] = readable ? real : 0u;
        m_so[threadIdx.x] = so;
        if (leader && j < k) {
            cu[csr + j + 1] = (int32_t)incl_real;
            cp[csr + j + 1] = (fold && j == k - 1) ? C : (int32_t)incl_pos;
        }
        const uint32_t first = carry_pos;
        carry_pos = sat_add(carry_pos, tp, sat);
        carry_real = sat_add(carry_real, tr, sat);
        __syncthreads();

        // ---- slots owned by this batch's members --------------------------
        const int64_t nb = min((int64_t)kMembers, k - m0);
        const bool last_batch = m0 + kMembers >= k;
        const uint32_t r_lo = max(lo, first);
        const uint32_t r_hi = last_batch ? hi : min(hi, carry_pos);
        if (r_lo < r_hi) {   // uniform: r_lo, r_hi come from block-wide values
            // Owners: slot s belongs to the last member starting at or before
            // it (starts are non-decreasing; of equal starts, the later one).
            // Only members j0 .. upto-1 can own a slot of [r_lo, r_hi): the
            // last one starting at or before lo (or the batch's first), up to
            // the last one starting before r_hi -- about 3 for this chunk
            // size -- so each lane takes its slots' owners from their starts
            // in registers, with no per-chunk map in LDS.
            const uint32_t my_start = m_start[threadIdx.x];
            const bool mine = (int64_t)threadIdx.x < nb;
            const int before = __syncthreads_count(mine && my_start <= lo);
            const int upto = __syncthreads_count(mine && my_start < r_hi);
            const int j0 = before > 0 ? before - 1 : 0;
            for (uint32_t ub = r_lo; ub < r_hi; ub += kSlots) {
                int64_t val[kPerThread];
                bool in[kPerThread];
                uint32_t own[kPerThread];
#pragma unroll
                for (int t = 0; t < kPerThread; ++t) own[t] = (uint32_t)j0;
                for (int mj = j0 + 1; mj < upto; ++mj) {
                    const uint32_t st = (uint32_t)read_lane((int)my_start, mj);
#pragma unroll
                    for (int t = 0; t < kPerThread; ++t) {
                        const uint32_t s = ub + threadIdx.x + (uint32_t)kThreads * (uint32_t)t;
                        own[t] = s >= st ? (uint32_t)mj : own[t];
                    }
                }
#pragma unroll
                for (int t = 0; t < kPerThread; ++t) {
                    const uint32_t s = ub + threadIdx.x + (uint32_t)kThreads * (uint32_t)t;
                    in[t] = s < r_hi;
                    const uint32_t o1 = in[t] ? own[t] + 1u : 0u;
                    bool tok = false;
                    int64_t idx = 0;
                    if (o1 != 0u) {
                        const uint32_t x = o1 - 1u;
                        const uint32_t off = s - m_start[x];
                        const uint32_t rl = m_real[x];
                        tok = off < rl;
                        // a pad slot re-reads its member's last token (none:
                        // the first element), always inside the buffer
                        idx = m_so[x] + (tok ? off : (rl ? rl - 1u : 0u));
                        if (!tok && !rl) idx = 0;
                    }
                    const int64_t v = __builtin_nontemporal_load(srcp + idx);
                    val[t] = tok ? v : pad_token;
                    if (in[t]) s_mask[s - lo] = tok ? 1 : 0;
                }
#pragma unroll
                for (int t = 0; t < kPerThread; ++t) {
                    const uint32_t s = ub + threadIdx.x + (uint32_t)kThreads * (uint32_t)t;
                    if (in[t]) __builtin_nontemporal_store(val[t], row + s);
                }
            }
        }
        __syncthreads();
    }

    // ---- token mask of the chunk --------------------------------------
    if (k > 0 && hi > lo) {
        uint8_t *__restrict__ mrow = tmask + p * (int64_t)C;
        const uint32_t len = hi - lo;
        if (vec_mask && ((p * (int64_t)C + lo) % 16) == 0 && (len % 16) == 0) {
            for (uint32_t u = threadIdx.x * 16u; u < len; u += kThreads * 16u)
                __builtin_nontemporal_store(*(const u32x4 *)(s_mask + u),
                                            (u32x4 *)(mrow + lo + u));
        } else {
            for (uint32_t u = threadIdx.x; u < len; u += kThreads) mrow[lo + u] = s_mask[u];
        }
    }

    if (leader && threadIdx.x == 0) {
        uint32_t err = s_err;
        if (carry_pos > (uint32_t)C) err |= PSQ_DATA_PACK_OVERFLOW;
        uint32_t all;
        if (finish_status(ws, err, (uint32_t)P, &all)) *status = (int32_t)all;
    }
}

}  // namespace

size_t pack_rows_workspace() { return 256; }

namespace {
uint64_t pack_groups(int64_t P, int32_t C, uint32_t *slots_out) {
    const bool small = (uint64_t)P * (uint64_t)(((int64_t)C + kBigSlots - 1) / kBigSlots) <
                       kFillGroups;
    const uint32_t slots = small ? kSmallSlots : kBigSlots;
    *slots_out = slots;
    const uint64_t n_chunks = ((uint64_t)C + slots - 1) / slots;
    return P > 0 ? (uint64_t)P * n_chunks : 1ull;
}
}  // namespace

bool pack_rows_grid_fits(int64_t P, int32_t C) {
    uint32_t slots;
    return pack_groups(P, C, &slots) * (uint64_t)kThreads <= kMaxGridThreads;
}

hipError_t launch_pack_rows(const int64_t *src, int64_t src_len, const int64_t *src_off,
                            int64_t src_stride, const int32_t *real_len, int64_t N, int32_t q,
                            const int32_t *order, const int64_t *pack_start, int64_t P,
                            int32_t C, int fold, int64_t pad_token, int64_t *packed,
                            uint8_t *tmask, int32_t *cu, int32_t *cp, int32_t *status,
                            void *workspace, hipStream_t stream) {
    uint32_t slots;
    const uint64_t groups = pack_groups(P, C, &slots);
    if (groups * (uint64_t)kThreads > kMaxGridThreads) return hipErrorInvalidConfiguration;
    const uint32_t n_chunks = (uint32_t)(((int64_t)C + slots - 1) / slots);
    const int vec_mask = ((uintptr_t)tmask % 16) == 0;
    hipLaunchKernelGGL(slots == kSmallSlots ? k_pack_rows<kSmallSlots> : k_pack_rows<kBigSlots>,
                       dim3((uint32_t)groups), dim3(kThreads), 0, stream, src,
                       src_len, src_off, src_stride, real_len, N, q, order, pack_start, P, C, fold,
                       pad_token, packed, tmask, cu, cp, status, (WsHeader *)workspace,
                       n_chunks, vec_mask);
    return hipGetLastError();
}

}  // namespace psq
