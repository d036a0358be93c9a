// psq_device.hpp -- device-side building blocks shared by the psq kernels:
// wave64 DPP scans, the workspace header, and the decoupled look-back over
// per-tile descriptors.  gfx950 (CDNA4) only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace psq {

constexpr int kWave = 64;

// ---------------------------------------------------------------------------
// Vector types (native clang vectors, so nontemporal builtins accept them).
// ---------------------------------------------------------------------------
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef int64_t i64x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------
// Streaming stores: non-temporal, at agent scope (sc1 nt), for the 16-byte
// units of the collapse copy (data written once and not read again).  On
// MI355X the stage-embedding step (an 8 GiB copy of one-wave 1 KiB
// workgroups) took 2.550 ms with these stores against 2.601 ms with the
// compiler's non-temporal stores (nt only), 2 % apart in two alternating
// runs each; the squeeze gained only 0.4 % from them and uses the builtin.
// The compiler's hazard tracking does not see inside inline assembly: on
// gfx940 and later a store of more than 8 bytes needs two wait states before
// a VALU instruction may write its data registers, so the store carries its
// own s_nop 1 (two wait states).  With one wait state a squeeze build whose
// scheduler placed a register move right after the mask store wrote wrong
// mask bytes.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void store_stream(u32x4 *p, u32x4 v) {
    asm volatile("global_store_dwordx4 %0, %1, off sc1 nt\n\ts_nop 1" : : "v"(p), "v"(v) : "memory");
}

// ---------------------------------------------------------------------------
// Progress jitter for the race tests.  In the PSQ_JITTER build of the library
// (libpsq_jitter.so) a wave sleeps a pseudo-random time, up to about 15 us, at
// each marked step of a cross-workgroup protocol: claiming a tile, publishing
// a look-back descriptor, looking back, counting itself finished.  The orders
// in which workgroups take those steps then change from call to call, and
// the tests check that the results do not.  In the normal build it is empty.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void jitter(uint32_t site) {
#ifdef PSQ_JITTER
    uint32_t h = (uint32_t)wall_clock64() ^ (blockIdx.x * 0x9e3779b1u) ^ (site * 0x85ebca77u);
    h ^= h >> 16;
    h *= 0x7feb352du;
    h ^= h >> 15;
    h *= 0x846ca68bu;
    h ^= h >> 16;
    for (uint32_t i = 0, n = h & 63u; i < n; ++i) __builtin_amdgcn_s_sleep(8);
#else
    (void)site;
#endif
}

// ---------------------------------------------------------------------------
// Workspace.  The first 256 bytes hold the header; the document-map records
// and then the table kernel's per-row descriptors follow.  Every kernel that
// relies on zeros leaves its part zero-filled on completion (the last
// workgroup to finish clears what the call used), so a workspace needs one
// zero fill per allocation.
// ---------------------------------------------------------------------------
struct WsHeader {
    uint32_t ticket;     // dynamic tile ids (dispatch order is not guaranteed)
    uint32_t done;       // workgroups finished
    uint32_t status;     // OR of data status bits
    int32_t max;         // running maximum (segment / sequence length)
    uint32_t flags;      // kernel-specific OR flags
    int32_t n;           // kernel-specific scalars published by one tile
    int32_t cu_last;
    int32_t total;
    uint64_t fin;        // finished count (high half) | status bits (low half)
};
// The document-map region follows the header; no other kernel touches it,
// so the zero-filled parts of a shared workspace stay zero-filled.
//  - Records of the two-launch path: one 16 bytes per workgroup, at most
//    kDocMaxGroups.  Written before they are read; never cleared.
//  - State of the one-launch path for maps of 2..kDocSmallTiles chunks: a
//    64-bit word (call parity, previous tile count) on a 128-byte line of its
//    own, then one tagged 64-bit record word per tile, each on its own line
//    (every workgroup reads the lines of all tiles before it: spread over
//    many lines, those reads do not queue on a few).  Zero-filled once with
//    the workspace; every call leaves it consistent for the next.
constexpr size_t kWsDocOffset = 256;
constexpr uint32_t kDocMaxGroups = 1024;
constexpr uint32_t kDocSmallTiles = 256;
constexpr size_t kDocSmallLine = 128;
constexpr size_t kWsDocSmallOffset = kWsDocOffset + 16 * (size_t)kDocMaxGroups;
constexpr size_t kWsDocSmallBytes = kDocSmallLine * (1 + (size_t)kDocSmallTiles);
constexpr size_t kWsDocEnd = (kWsDocSmallOffset + kWsDocSmallBytes + 255) / 256 * 256;
// per-row look-back descriptors of the multi-workgroup table kernel
constexpr size_t kWsDescOffset = kWsDocEnd;

__device__ __forceinline__ uint32_t ld_relaxed(const uint32_t *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_relaxed(const uint64_t *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_relaxed(uint32_t *p, uint32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_relaxed(uint64_t *p, uint64_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t fetch_add_relaxed(uint32_t *p, uint32_t v) {
    return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void or_relaxed(uint32_t *p, uint32_t v) {
    __hip_atomic_fetch_or(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void max_relaxed(int32_t *p, int32_t v) {
    __hip_atomic_fetch_max(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Claim a tile id: workgroups that got a smaller ticket were dispatched
// earlier, so waiting on them always makes progress.
__device__ __forceinline__ uint32_t claim_tile(WsHeader *ws, uint32_t *lds_slot) {
    if (threadIdx.x == 0) {
        jitter(1);
        *lds_slot = fetch_add_relaxed(&ws->ticket, 1u);
    }
    __syncthreads();
    return *lds_slot;
}

// Count this workgroup as finished.  Returns true in exactly one workgroup:
// the last to finish, which then sees every earlier workgroup's writes to
// the header (release on every increment, acquire on the last one).
__device__ __forceinline__ bool finish_is_last(WsHeader *ws, uint32_t n_groups,
                                               uint32_t *lds_slot) {
    __syncthreads();
    if (threadIdx.x == 0) {
        jitter(2);
        uint32_t prev = __hip_atomic_fetch_add(&ws->done, 1u, __ATOMIC_RELEASE,
                                               __HIP_MEMORY_SCOPE_AGENT);
        uint32_t last = (prev == n_groups - 1u);
        if (last)
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");   // pairs with the releases
        *lds_slot = last;
    }
    __syncthreads();
    return *lds_slot != 0u;
}

// Count this workgroup as finished and fold `bits` into the shared status in
// one 64-bit word (count in the high half, status bits in the low half).
// Both updates hit the same location, so relaxed atomics keep them ordered:
// the workgroup whose count reaches n_groups holds every other workgroup's
// bits, with no cache write-back (a release would flush L2 once per
// workgroup, which costs more than the work itself).  Returns the final
// status in *final_bits and true in that last workgroup, which also clears
// the word.  Called by one thread.
__device__ __forceinline__ bool finish_status(WsHeader *ws, uint32_t bits, uint32_t n_groups,
                                              uint32_t *final_bits) {
    jitter(3);
    if (bits)
        __hip_atomic_fetch_or(&ws->fin, (uint64_t)bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint64_t old = __hip_atomic_fetch_add(&ws->fin, 1ull << 32, __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT);
    if ((uint32_t)(old >> 32) != n_groups - 1u)
        return false;
    *final_bits = (uint32_t)old;
    st_relaxed(&ws->fin, 0ull);
    return true;
}

// ---------------------------------------------------------------------------
// Wave64 scans with DPP.  Rows of 16 lanes are scanned with row_shr 1/2/4/8
// (source lanes outside the row read the `old` operand, 0 here); rows are
// then joined with row_bcast:15 (rows 1, 3) and row_bcast:31 (rows 2, 3).
// Values must be >= 0 for the max scan (0 is its identity).
// ---------------------------------------------------------------------------
template <int kCtrl, int kRowMask = 0xf>
__device__ __forceinline__ int dpp0(int v) {
    return __builtin_amdgcn_update_dpp(0, v, kCtrl, kRowMask, 0xf, false);
}

__device__ __forceinline__ int wave_incl_sum(int x) {
    x += dpp0<0x111>(x);
    x += dpp0<0x112>(x);
    x += dpp0<0x114>(x);
    x += dpp0<0x118>(x);
    x += dpp0<0x142, 0xa>(x);
    x += dpp0<0x143, 0xc>(x);
    return x;
}

__device__ __forceinline__ int wave_incl_max(int x) {
    x = max(x, dpp0<0x111>(x));
    x = max(x, dpp0<0x112>(x));
    x = max(x, dpp0<0x114>(x));
    x = max(x, dpp0<0x118>(x));
    x = max(x, dpp0<0x142, 0xa>(x));
    x = max(x, dpp0<0x143, 0xc>(x));
    return x;
}

// a + b saturated at `sat` (sat <= 2^31; a, b <= sat, so a wrap is caught)
__device__ __forceinline__ uint32_t sat_add(uint32_t a, uint32_t b, uint32_t sat) {
    const uint32_t s = a + b;
    return (s < a || s > sat) ? sat : s;
}

// Inclusive wave sum, saturated at `sat` (sat <= 2^31).
__device__ __forceinline__ uint32_t wave_incl_sat(uint32_t x, uint32_t sat) {
    x = sat_add(x, (uint32_t)dpp0<0x111>((int)x), sat);
    x = sat_add(x, (uint32_t)dpp0<0x112>((int)x), sat);
    x = sat_add(x, (uint32_t)dpp0<0x114>((int)x), sat);
    x = sat_add(x, (uint32_t)dpp0<0x118>((int)x), sat);
    x = sat_add(x, (uint32_t)dpp0<0x142, 0xa>((int)x), sat);
    x = sat_add(x, (uint32_t)dpp0<0x143, 0xc>((int)x), sat);
    return x;
}

// Lane l receives lane l-1's value; lane 0 receives `first`.
__device__ __forceinline__ int wave_shr1(int x, int first) {
    return __builtin_amdgcn_update_dpp(first, x, 0x138, 0xf, 0xf, false);
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// The wave's index in its workgroup, as a scalar: the compiler cannot tell
// that threadIdx.x / 64 is the same in every lane, and a branch on a value it
// takes for per-lane is laid out as both sides run in turn under the exec
// mask, with waits for the loads of one side placed before the other.
__device__ __forceinline__ int wave_id() {
    return __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
}

__device__ __forceinline__ int read_lane(int v, int lane) {
    return __builtin_amdgcn_readlane(v, lane);
}

// ---------------------------------------------------------------------------
// Decoupled look-back.  A descriptor is one 64-bit word, so relaxed agent-
// scope atomics suffice (one word carries state and payload together):
//   bits 63..62  state: 0 = not yet published, 1 = aggregate, 2 = inclusive
//   bits 61..31  a: 31-bit sum
//   bits 30..0   b: 31-bit second value (summed, or latest non-zero wins)
// The combine of (a, b) pairs adds the a's; the b's either add too or the
// later non-zero b wins.  Both are associative with identity (0, 0).
// ---------------------------------------------------------------------------
constexpr uint64_t kDescAgg = 1ull << 62;
constexpr uint64_t kDescIncl = 2ull << 62;
constexpr uint32_t kSpinLimit = 1u << 22;

__device__ __forceinline__ uint64_t desc_pack(uint64_t state, uint32_t a, uint32_t b) {
    return state | ((uint64_t)(a & 0x7fffffffu) << 31) | (uint64_t)(b & 0x7fffffffu);
}
__device__ __forceinline__ uint32_t desc_a(uint64_t d) { return (uint32_t)(d >> 31) & 0x7fffffffu; }
__device__ __forceinline__ uint32_t desc_b(uint64_t d) { return (uint32_t)d & 0x7fffffffu; }

// Run by one full wave.  Returns the exclusive prefix (a, b) of tile `tile`
// over tiles 0..tile-1 and sets *timed_out when a predecessor never
// published within the spin bound (only possible with a dirty workspace).
// kSumB selects the combine of b: summed (true) or latest non-zero (false).
template <bool kSumB>
__device__ inline void lookback(const uint64_t *desc, uint32_t tile, uint32_t *out_a,
                                uint32_t *out_b, bool *timed_out) {
    jitter(4);
    const int lane = lane_id();
    uint32_t acc_a = 0, acc_b = 0;
    int64_t base = (int64_t)tile - 1;
    uint32_t spins = 0;
    bool expired = false;
    while (base >= 0) {
        const int64_t idx = base - lane;
        uint64_t d = kDescIncl;                 // before tile 0: inclusive identity
        if (idx >= 0) {
            d = ld_relaxed(desc + idx);
            while ((d >> 62) == 0) {
                if (++spins > kSpinLimit) {
                    expired = true;
                    d = kDescIncl;
                    break;
                }
                __builtin_amdgcn_s_sleep(1);
                d = ld_relaxed(desc + idx);
            }
        }
        // nearest lane holding an inclusive prefix
        const uint64_t incl = __ballot((d >> 62) == 2);
        const int stop = incl ? __builtin_ctzll(incl) : kWave - 1;
        // combine lanes 0..stop (nearest first): sums add; b from the
        // nearest lane with a non-zero b
        const bool use = lane <= stop;
        const uint32_t a = use ? desc_a(d) : 0u;
        const uint32_t b = use ? desc_b(d) : 0u;
        const uint32_t sum = (uint32_t)wave_incl_sum((int)a);
        acc_a += (uint32_t)read_lane((int)sum, kWave - 1);
        if constexpr (kSumB) {
            const uint32_t bsum = (uint32_t)wave_incl_sum((int)b);
            acc_b += (uint32_t)read_lane((int)bsum, kWave - 1);
        } else {
            const uint64_t has_b = __ballot(b != 0u);
            uint32_t win_b = 0;
            if (has_b)
                win_b = (uint32_t)read_lane((int)b, __builtin_ctzll(has_b));
            if (acc_b == 0u)
                acc_b = win_b;
        }
        if (incl)
            break;
        base -= kWave;
    }
    *out_a = acc_a;
    *out_b = acc_b;
    *timed_out = __ballot(expired) != 0;
}

}  // namespace psq
