// ccb_kernels.hip -- gfx950 kernels of the soft epoch barrier library.
//
// Persistent grids built on the device barrier of ccb_device.h:
//   barrier-only rounds, witness (slot) rounds, grouped witness rounds and a
//   barrier-separated 3-point stencil;
// plus the batched CntNotify engine, the stream-ordered CntNotify record /
// wait / reset kernels and the floor microbenchmarks.
//
// Sources: "PTO-ISA 跨核同步屏障 SYNCALL 实战指南" (PTO-ISA SYNCALL guide) §2,
// §4-§7 for the barrier, and "CANN Runtime CntNotify（计数型通知）管理接口详解"
// (CANN Runtime CntNotify interfaces) §3.1-§3.3, §4.2-§4.4 for the counter
// operations.  Each kernel cites the passage it implements.

#include <hip/hip_cooperative_groups.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "ccb.h"
#include "ccb_device.h"
#include "ccb_internal.h"

namespace {

constexpr int kWave = 64;
constexpr int kRing = CCB_SLOT_ROWS;  // witness slot rows reused round-robin
constexpr int kSlot = CCB_SLOT_WORDS;  // words from one slot to the next

__device__ __forceinline__ bool leader() { return threadIdx.x == 0; }

// Witness value of member w in round r: SplitMix64 (Steele, Lea & Flood,
// OOPSLA 2014) output number r*2^32 + w + 1 for the given seed -- the state
// advanced that many times by the golden gamma, then the variant-13
// finaliser -- keeping the high 32 bits.
__device__ __forceinline__ uint32_t witness(uint64_t seed, uint32_t r, uint32_t w)
{
    const uint64_t key = ((uint64_t)r << 32) | (uint64_t)w;
    uint64_t z = seed + 0x9E3779B97F4A7C15ull * (key + 1ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    z ^= z >> 31;
    return (uint32_t)(z >> 32);
}

// Sum of v over the workgroup (mod 2^32); the result is valid in thread 0.
// partial: LDS scratch of one word per wave.
__device__ __forceinline__ uint32_t block_sum(uint32_t v, uint32_t* partial)
{
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
    const int wave = threadIdx.x / kWave;
    if ((threadIdx.x % kWave) == 0) partial[wave] = v;
    __syncthreads();
    uint32_t s = 0;
    if (threadIdx.x == 0) {
        const int nw = blockDim.x / kWave;
        for (int i = 0; i < nw; ++i) s += partial[i];
    }
    return s;
}

// Register query of a persistent kernel: a launch with maxPoll == 0 (a real
// launch never has it: the API turns 0 into the default bound) stores the
// HW_REG_GPR_ALLOC value of the kernel's waves in *out (thread 0 of
// workgroup 0) and returns at once in every thread.  The launcher reads the
// SGPR allocation from it to check co-residency.
__device__ __forceinline__ bool register_query(uint32_t maxPoll, int32_t* out)
{
    if (maxPoll != 0) return false;
    if (blockIdx.x == 0 && threadIdx.x == 0)
        *out = (int32_t)__builtin_amdgcn_s_getreg((31 << 11) | 5);  // HW_REG_GPR_ALLOC
    return true;
}

__device__ __forceinline__ void record_placement(uint32_t* placement)
{
    if (placement != nullptr && leader()) {
        placement[2 * blockIdx.x] = __builtin_amdgcn_s_getreg((31 << 11) | 4);       // HW_ID
        placement[2 * blockIdx.x + 1] = __builtin_amdgcn_s_getreg((31 << 11) | 20);  // XCC_ID
    }
}

}  // namespace

// ---------------------------------------------------------------------------
// Barrier variants.  K = stripes (1: the pages' single counter), V = the
// visibility strength.  Shared witness data follows V: device-coherent
// accesses across a CCB_VIS_ORDER barrier, plain accesses across a
// CCB_VIS_FULL one (whose fences make them visible).
// ---------------------------------------------------------------------------
namespace {

template <ccbVisibility V>
__device__ __forceinline__ void shared_store(uint32_t* p, uint32_t v)
{
    if constexpr (V == CCB_VIS_ORDER) ccb_store_coherent(p, v);
    else *p = v;
}
template <ccbVisibility V>
__device__ __forceinline__ uint32_t shared_load(const uint32_t* p)
{
    if constexpr (V == CCB_VIS_ORDER) return ccb_load_coherent(p);
    else return *p;
}

}  // namespace

// ---------------------------------------------------------------------------
// Barrier-only rounds: the latency benchmark of the soft barrier.
// Members (w < nMembers) run `rounds` barriers; the rest take the partial-
// participation exit of the SYNCALL guide §7.2 and mark themselves idle (§8).
//
// kStamps: lane 0 of each member also reads the wall clock when it issues
// its arrival, when the arrival's reply is back and when its poll sees the
// round complete.  The stamps stay in LDS during the loop (a global store
// per round would add its acknowledgement to the next arrival's wait) and
// go to stamps[(r * nGrid + w) * 3 + {0, 1, 2}] at the end.
// ---------------------------------------------------------------------------
namespace {

// Wall-clock stamps of one round's reply and release (lane 0 of wave 0).
struct StampHook {
    uint64_t* atReply;
    uint64_t* atRelease;
    __device__ __forceinline__ void reply() const
    {
        if (__lane_id() == 0) *atReply = wall_clock64();
    }
    __device__ __forceinline__ void released() const
    {
        if (__lane_id() == 0) *atRelease = wall_clock64();
    }
};

}  // namespace

template <int K, ccbVisibility V, bool kStamps>
__global__ __launch_bounds__(1024) void ccb_k_barrier_only(int32_t* ws, uint32_t* placement,
                                                            int32_t* wgStatus, uint64_t* stamps,
                                                            int32_t rounds, int32_t nMembers,
                                                            uint32_t maxPoll)
{
    __shared__ int32_t result[2];
    __shared__ uint64_t lds[kStamps ? 3 * CCB_BREAKDOWN_MAX_ROUNDS : 1];
    if (register_query(maxPoll, ws)) return;
    record_placement(placement);
    const int32_t w = blockIdx.x;
    if (w >= nMembers) {
        if (wgStatus != nullptr && leader()) wgStatus[w] = 2;
        return;
    }
    int32_t* err = ws + CCB_STRIPES * CCB_LINE_WORDS;
    int32_t rc = CCB_OK;
    int32_t done = 0;
    ccb_xcd_team team = {};
    // Rounds follow each other with nothing in between, so the workgroup
    // barrier that releases round r also orders round r + 1's arrival: one
    // per round.  The result word alternates so that wave 0 can publish
    // round r + 1's result while a slow wave still reads round r's.
    for (int32_t r = 0; r < rounds; ++r) {
        if (threadIdx.x < kWave) {
            int32_t before = 0;
            int32_t e;
            if constexpr (kStamps) {
                if (leader()) lds[3 * r] = wall_clock64();
                if (leader()) before = ccb_arrive<K, V>(ws, w, team);
                e = ccb_await<K, V>(ws, nMembers, w, before, maxPoll, err,
                                    StampHook{&lds[3 * r + 1], &lds[3 * r + 2]}, team);
            } else {
                if (leader()) before = ccb_arrive<K, V>(ws, w, team);
                e = ccb_await<K, V>(ws, nMembers, w, before, maxPoll, err, ccb_no_hook(), team);
            }
            if (leader()) result[r & 1] = e;
        }
        __syncthreads();
        rc = result[r & 1];
        done = r + 1;
        if (rc != CCB_OK) break;
    }
    if constexpr (kStamps) {
        // wave 0 wrote the stamps and writes them out
        if (threadIdx.x < kWave)
            for (int32_t i = threadIdx.x; i < 3 * done; i += kWave)
                stamps[((size_t)(i / 3) * gridDim.x + w) * 3 + i % 3] = lds[i];
    }
    if (wgStatus != nullptr && leader()) wgStatus[w] = rc == CCB_OK ? 1 : 3;
}

// ---------------------------------------------------------------------------
// Witness rounds on one barrier (the flag-slot test pattern of the SYNCALL
// guide §6.1, run for many rounds): write own slot, barrier, sum all slots.
//
// With CCB_VIS_FULL each round is written in that order with plain accesses.
// With CCB_VIS_ORDER the rounds are pipelined two deep without changing what
// is computed, and each round costs one workgroup barrier.  In its round i a
// member
//   * arrives at barrier i (its witness for round i was stored and waited
//     for during round i - 1, and so were its loads of row i - 2),
//   * while the arrival is in flight, loads row i - 1 (barrier i - 1 has been
//     passed) without waiting, stores its witness for round i + 1, sums row
//     i - 2 (loaded during round i - 1) into LDS partials and stores out for
//     round i - 3 from the partials of the round before,
//   * waits for barrier i, then for its own loads and stores, and releases
//     the workgroup.
// So the loads and stores of a round overlap a barrier's wait instead of
// adding memory round trips to every round.  Counted in the member's own
// rounds, a witness is written after passing the barrier two rounds before
// its own and a row may be read until the member arrives two rounds after
// it; the brute-force enumerator shows that this needs D >= 4 slot rows
// for the whole grid and D >= 6 for the grouped pattern below, and
// D = CCB_SLOT_ROWS = 6 is used for both.  Slots sit CCB_SLOT_WORDS = 4
// words apart: with packed slots all members' stores of a round land on a
// few lines, whose partial-line writes are merged one after another, and a
// slot store then outlasts the barrier; four words apart (eight writers per
// line) it does not.  The member's last wave does the
// witness and output stores, so wave 0's poll does not wait for them.
// ---------------------------------------------------------------------------
namespace {

// Wave-level sum (mod 2^32) of v; the result is valid in lane 0.
__device__ __forceinline__ uint32_t wave_sum(uint32_t v)
{
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
    return v;
}

// One witness row read by the workgroup, kept in flight across a barrier:
// up to kRowRegs slots per thread are loaded without waiting and summed
// later; members beyond kRowRegs * blockDim.x are read synchronously.
constexpr int kRowRegs = 4;

struct RowRead {
    uint32_t v[kRowRegs];
    uint32_t tail;
    int32_t n;

    __device__ __forceinline__ void issue(const uint32_t* row, int32_t count)
    {
        n = count;
#pragma unroll
        for (int j = 0; j < kRowRegs; ++j) {
            const int32_t i = (int32_t)threadIdx.x + j * (int32_t)blockDim.x;
            // wave-uniform test; lanes past the end reload slot 0 and are
            // left out of the sum
            if (j * (int32_t)blockDim.x < count)
                v[j] = ccb_load_coherent(row + (size_t)(i < count ? i : 0) * kSlot);
        }
        tail = 0;
        for (int32_t i = threadIdx.x + kRowRegs * blockDim.x; i < count; i += blockDim.x)
            tail += ccb_load_coherent(row + (size_t)i * kSlot);
    }

    // This thread's share of the row sum (mod 2^32).
    __device__ __forceinline__ uint32_t sum() const
    {
        uint32_t s = tail;
#pragma unroll
        for (int j = 0; j < kRowRegs; ++j)
            if ((int32_t)threadIdx.x + j * (int32_t)blockDim.x < n) s += v[j];
        return s;
    }
};

// Stores this wave's share of a row sum into the LDS partials.
__device__ __forceinline__ void wave_partial(uint32_t* partial, uint32_t s)
{
    s = wave_sum(s);
    if ((threadIdx.x % kWave) == 0) partial[threadIdx.x / kWave] = s;
}

// Finishes round r's sum from the per-wave partials and stores it.
struct FinishRound {
    const uint32_t* partial;
    int nWave;
    uint32_t* dst;  // nullptr: nothing to store
    __device__ __forceinline__ void operator()() const
    {
        if (dst == nullptr) return;
        uint32_t s = 0;
        for (int i = 0; i < nWave; ++i) s += partial[i];
        *dst = s;
    }
};

// The pipelined witness rounds of one member (CCB_VIS_ORDER).  Sched names
// the member's rounds and where each one's counter, row and slot are:
//   first(), next(q)        the member's first round and the one after q
//                           (`rounds` once there are no more)
//   counter(q), n(q), member(q)   barrier of round q
//   row(q), len(q)          the slots summed in round q
//   slot(q)                 this member's slot in round q
// No round stamps.
struct NoStamps {
    __device__ __forceinline__ void operator()(int32_t) const {}
};

// The wall clock at which the member passed the barrier of its own round i,
// for the first `cap` rounds, into LDS (written out by the caller).
struct RoundStamps {
    uint64_t* lds;
    int32_t cap;
    __device__ __forceinline__ void operator()(int32_t i) const
    {
        if (i < cap) lds[i] = wall_clock64();
    }
};

template <int K, ccbVisibility V, class Sched, class Stamp = NoStamps>
__device__ __forceinline__ int32_t witness_pipeline(const Sched& sc, int32_t rounds,
                                                    uint32_t* out, int32_t nGrid, int32_t w,
                                                    uint64_t seed, uint32_t maxPoll, int32_t* err,
                                                    Stamp stamp = Stamp())
{
    __shared__ uint32_t partials[2][1024 / kWave];
    __shared__ int32_t result[2];
    const int nWave = blockDim.x / kWave;
    const bool scribe = threadIdx.x == (uint32_t)((nWave - 1) * kWave);
    // the member's rounds: cur (this one), nxt, and the three before it
    int32_t cur = sc.first();
    int32_t nxt = cur < rounds ? sc.next(cur) : rounds;
    int32_t p1 = -1, p2 = -1, p3 = -1;
    if (scribe && cur < rounds) ccb_store_coherent(sc.slot(cur), witness(seed, (uint32_t)cur, (uint32_t)w));
    ccb_wait_memory();
    __syncthreads();
    RowRead rowA, rowB;
    auto work = [&](int32_t i, RowRead& into, RowRead& from) {
        if (p1 >= 0) into.issue(sc.row(p1), sc.len(p1));
        if (scribe && nxt < rounds)
            ccb_store_coherent(sc.slot(nxt), witness(seed, (uint32_t)nxt, (uint32_t)w));
        if (p2 >= 0) wave_partial(partials[i & 1], from.sum());
        if (scribe && p3 >= 0)
            FinishRound{partials[(i - 1) & 1], nWave, out + (size_t)p3 * nGrid + w}();
    };
    auto shift = [&]() {
        p3 = p2;
        p2 = p1;
        p1 = cur;
        cur = nxt;
        nxt = nxt < rounds ? sc.next(nxt) : rounds;
    };
    auto round = [&](int32_t i, RowRead& into, RowRead& from) {
        const int32_t q = cur;
        int32_t before = 0;
        if (leader()) before = ccb_arrive<K, V>(sc.counter(q), sc.member(q));
        work(i, into, from);
        if (threadIdx.x < kWave) {
            const int32_t e = ccb_await<K, V>(sc.counter(q), sc.n(q), sc.member(q), before, maxPoll, err);
            if (leader()) {
                result[i & 1] = e;
                stamp(i);
            }
        }
        ccb_wait_memory();  // this round's loads and stores, before the next arrival
        __syncthreads();
        shift();
        return result[i & 1];
    };
    int32_t rc = CCB_OK;
    int32_t i = 0;
    while (cur < rounds) {
        if ((rc = round(i++, rowA, rowB)) != CCB_OK || cur >= rounds) break;
        if ((rc = round(i++, rowB, rowA)) != CCB_OK) break;
    }
    if (rc == CCB_OK) {
        // the last three rounds' reads, sums and stores, with no barrier left
        for (int d = 0; d < 3; ++d, ++i) {
            if ((i & 1) == 0) work(i, rowA, rowB);
            else work(i, rowB, rowA);
            ccb_wait_memory();
            __syncthreads();
            shift();
        }
    }
    return rc;
}

}  // namespace

template <int K, ccbVisibility V>
__global__ __launch_bounds__(1024) void ccb_k_slot_rounds(int32_t* ws, uint32_t* slots,
                                                           uint32_t* out, int32_t* wgStatus,
                                                           uint64_t seed, int32_t rounds,
                                                           int32_t nMembers, uint32_t maxPoll)
{
    __shared__ uint32_t partial[1024 / kWave];
    if (register_query(maxPoll, ws)) return;
    const int32_t w = blockIdx.x;
    const int32_t nGrid = gridDim.x;
    if (w >= nMembers) {
        if (wgStatus != nullptr && leader()) wgStatus[w] = 2;
        return;
    }
    int32_t* err = ws + CCB_STRIPES * CCB_LINE_WORDS;
    int32_t rc = CCB_OK;
    if constexpr (V != CCB_VIS_ORDER) {
        ccb_xcd_team team = {};
        for (int32_t r = 0; r < rounds; ++r) {
            uint32_t* row = slots + (size_t)(r % kRing) * nGrid * kSlot;
            if (leader()) shared_store<V>(row + (size_t)w * kSlot, witness(seed, (uint32_t)r, (uint32_t)w));
            rc = ccb_barrier<K, V>(ws, nMembers, w, maxPoll, err, team);
            if (rc != CCB_OK) break;
            uint32_t s = 0;
            for (int32_t i = threadIdx.x; i < nMembers; i += blockDim.x)
                s += shared_load<V>(row + (size_t)i * kSlot);
            s = block_sum(s, partial);
            if (leader()) out[(size_t)r * nGrid + w] = s;
        }
    } else {
        struct Whole {
            int32_t* ws;
            uint32_t* slots;
            int32_t nGrid, nMembers, w;
            __device__ int32_t first() const { return 0; }
            __device__ int32_t next(int32_t q) const { return q + 1; }
            __device__ int32_t* counter(int32_t) const { return ws; }
            __device__ int32_t n(int32_t) const { return nMembers; }
            __device__ int32_t member(int32_t) const { return w; }
            __device__ const uint32_t* row(int32_t q) const { return slots + (size_t)(q % kRing) * nGrid * kSlot; }
            __device__ int32_t len(int32_t) const { return nMembers; }
            __device__ uint32_t* slot(int32_t q) const
            {
                return slots + ((size_t)(q % kRing) * nGrid + w) * kSlot;
            }
        };
        rc = witness_pipeline<K, V>(Whole{ws, slots, nGrid, nMembers, w}, rounds, out, nGrid, w,
                                    seed, maxPoll, err);
    }
    if (wgStatus != nullptr && leader()) wgStatus[w] = rc == CCB_OK ? 1 : 3;
}

// ---------------------------------------------------------------------------
// Grouped witness rounds: group A (even ids) on barrier 0, group B (odd ids)
// on barrier 1, everyone on barrier 2; round kind r mod 3.  Each barrier's
// members enter it in the same order the same number of times (SYNCALL
// guide §6.2).  Slots are stored group-major (even ids first) so a group's
// slots are contiguous; the sum does not depend on the layout.  With
// CCB_VIS_ORDER the rounds are pipelined two deep as in the witness rounds
// above, counted in the member's own rounds: after passing the barrier of
// its round m_i a member reads row m_i, stores the witness of m_{i+2} and
// sums row m_{i-1} before arriving at m_{i+1}.
// ---------------------------------------------------------------------------
// kStamps: member w also records, for each of its own first
// CCB_BREAKDOWN_MAX_ROUNDS rounds i, the wall clock when it passed that
// round's barrier; they stay in LDS and go to stamps[i * nGrid + w] at the
// end (0 past the member's last round).
template <int K, ccbVisibility V, bool kStamps>
__global__ __launch_bounds__(1024) void ccb_k_grouped_rounds(int32_t* ws, uint32_t* slots,
                                                              uint32_t* out, int32_t* wgStatus,
                                                              uint64_t* stamps, uint64_t seed,
                                                              int32_t rounds, uint32_t maxPoll)
{
    __shared__ uint32_t partial[1024 / kWave];
    __shared__ uint64_t stampLds[kStamps ? CCB_BREAKDOWN_MAX_ROUNDS : 1];
    if (register_query(maxPoll, ws)) return;
    if constexpr (kStamps) {
        for (int32_t i = threadIdx.x; i < CCB_BREAKDOWN_MAX_ROUNDS; i += blockDim.x) stampLds[i] = 0;
        __syncthreads();
    }
    const int32_t w = blockIdx.x;
    const int32_t nGrid = gridDim.x;
    const int32_t half = nGrid / 2;
    const int32_t parity = w & 1;
    const int32_t pos = parity * half + (w >> 1);
    int32_t* err = ws + 3 * CCB_STRIPES * CCB_LINE_WORDS;
    int32_t rc = CCB_OK;
    auto member_of = [&](int32_t r) { return (r % 3) == 2 || (r % 3) == parity; };
    if constexpr (V != CCB_VIS_ORDER) {
        // a member takes part in its own group's barrier and the mixed one;
        // the two states stay in registers (an indexed array would not)
        ccb_xcd_team tGroup = {}, tMix = {};
        int32_t own = 0;  // this member's rounds so far
        for (int32_t r = 0; r < rounds; ++r) {
            const int32_t kind = r % 3;
            if (!member_of(r)) continue;
            uint32_t* row = slots + (size_t)(r % kRing) * nGrid * kSlot;
            if (leader()) shared_store<V>(row + (size_t)pos * kSlot, witness(seed, (uint32_t)r, (uint32_t)w));
            const int32_t n = kind == 2 ? nGrid : half;
            const int32_t member = kind == 2 ? w : (w >> 1);
            auto bar = [&](ccb_xcd_team& team) {
                return ccb_barrier<K, V>(ws + kind * CCB_STRIPES * CCB_LINE_WORDS, n, member,
                                         maxPoll, err, team);
            };
            if constexpr (V == CCB_VIS_XCD) rc = kind == 2 ? bar(tMix) : bar(tGroup);
            else rc = bar(tGroup);  // stateless: one copy of the barrier
            if (rc != CCB_OK) break;
            if constexpr (kStamps) {
                if (leader()) RoundStamps{stampLds, CCB_BREAKDOWN_MAX_ROUNDS}(own);
                ++own;
            }
            const int32_t first = kind == 2 ? 0 : kind * half;
            uint32_t s = 0;
            for (int32_t i = threadIdx.x; i < n; i += blockDim.x)
                s += shared_load<V>(row + (size_t)(first + i) * kSlot);
            s = block_sum(s, partial);
            if (leader()) out[(size_t)r * nGrid + w] = s;
        }
    } else {
        struct Grouped {
            int32_t* ws;
            uint32_t* slots;
            int32_t nGrid, half, w, parity, pos, rounds;
            __device__ bool member_of(int32_t q) const { return (q % 3) == 2 || (q % 3) == parity; }
            __device__ int32_t next(int32_t q) const
            {
                ++q;
                while (q < rounds && !member_of(q)) ++q;
                return q;
            }
            __device__ int32_t first() const { return member_of(0) ? 0 : next(0); }
            __device__ int32_t* counter(int32_t q) const { return ws + (q % 3) * CCB_STRIPES * CCB_LINE_WORDS; }
            __device__ int32_t n(int32_t q) const { return (q % 3) == 2 ? nGrid : half; }
            __device__ int32_t member(int32_t q) const { return (q % 3) == 2 ? w : (w >> 1); }
            __device__ const uint32_t* row(int32_t q) const
            {
                return slots + ((size_t)(q % kRing) * nGrid + ((q % 3) == 2 ? 0 : (q % 3) * half)) * kSlot;
            }
            __device__ int32_t len(int32_t q) const { return n(q); }
            __device__ uint32_t* slot(int32_t q) const
            {
                return slots + ((size_t)(q % kRing) * nGrid + pos) * kSlot;
            }
        };
        const Grouped sched{ws, slots, nGrid, half, w, parity, pos, rounds};
        if constexpr (kStamps)
            rc = witness_pipeline<K, V>(sched, rounds, out, nGrid, w, seed, maxPoll, err,
                                        RoundStamps{stampLds, CCB_BREAKDOWN_MAX_ROUNDS});
        else
            rc = witness_pipeline<K, V>(sched, rounds, out, nGrid, w, seed, maxPoll, err);
    }
    if constexpr (kStamps) {
        __syncthreads();
        const int32_t nStamp = rounds < CCB_BREAKDOWN_MAX_ROUNDS ? rounds : CCB_BREAKDOWN_MAX_ROUNDS;
        for (int32_t i = threadIdx.x; i < nStamp; i += blockDim.x)
            stamps[(size_t)i * nGrid + w] = stampLds[i];
    }
    if (wgStatus != nullptr && leader()) wgStatus[w] = rc == CCB_OK ? 1 : 3;
}

// ---------------------------------------------------------------------------
// Barrier-separated 3-point stencil (persistent).
//
// Layout: the array is cut into chunks of 4 * blockDim.x elements (4 KiB for
// 256 threads).  Workgroup w owns chunks w, w + G, w + 2G, ... (G = grid
// size) in every iteration, so at any moment the whole grid streams one
// compact window of memory -- on MI355X that sweep order reaches about 5.7
// TB/s where per-wave contiguous spans stay near 4.2 TB/s.  Inside a chunk,
// lane l of wave v holds elements 4l..4l+3 of the wave's 256-element piece
// as one 16-byte load.  The left neighbour of a lane's first element is lane
// l-1's last element (DPP wave shift right by one lane), the right
// neighbour of its last element is lane l+1's first (DPP wave shift left);
// lanes 0 and 63 take the element just outside the piece, which belongs to
// the neighbouring wave of the same workgroup or, at a chunk boundary, to
// the neighbouring chunk of another workgroup.  The array ends are clamped.
//
// Chunks never move between workgroups, so the only data that crosses
// workgroups are the two boundary elements of each chunk.  Across a
// CCB_VIS_ORDER barrier they travel through a small exchange buffer written
// and read with device-coherent accesses (halo[t & 1][chunk][0] = first
// output element of the chunk in iteration t, [1] = last); the bulk data
// needs no cache maintenance at all.  Across a CCB_VIS_FULL barrier they
// are read straight from the source buffer.  A partial last chunk is
// processed one element per thread.
// ---------------------------------------------------------------------------
namespace {

__device__ __forceinline__ int32_t lane_from_left(int32_t v)  // lane l gets lane l-1
{
    return __builtin_amdgcn_update_dpp(0, v, 0x138 /* wave_shr:1 */, 0xf, 0xf, false);
}
__device__ __forceinline__ int32_t lane_from_right(int32_t v)  // lane l gets lane l+1
{
    return __builtin_amdgcn_update_dpp(0, v, 0x130 /* wave_shl:1 */, 0xf, 0xf, false);
}

__device__ __forceinline__ int32_t st3(int32_t a, int32_t b, int32_t c)
{
    return (a + 2 * b + c) >> 2;
}

template <bool kNT>
__device__ __forceinline__ void store4(int32_t* p, int4 v)
{
    if constexpr (kNT) {
        typedef int v4i __attribute__((ext_vector_type(4)));
        const v4i nv = {v.x, v.y, v.z, v.w};
        __builtin_nontemporal_store(nv, reinterpret_cast<v4i*>(p));
    } else {
        *reinterpret_cast<int4*>(p) = v;
    }
}

template <bool kNT>
__device__ __forceinline__ int4 load4(const int32_t* p)
{
    if constexpr (kNT) {
        typedef int v4i __attribute__((ext_vector_type(4)));
        const v4i v = __builtin_nontemporal_load(reinterpret_cast<const v4i*>(p));
        return make_int4(v.x, v.y, v.z, v.w);
    } else {
        return *reinterpret_cast<const int4*>(p);
    }
}

__device__ __forceinline__ void set_prio(int p)
{
    switch (p & 3) {
    case 0: __builtin_amdgcn_s_setprio(0); break;
    case 1: __builtin_amdgcn_s_setprio(1); break;
    case 2: __builtin_amdgcn_s_setprio(2); break;
    default: __builtin_amdgcn_s_setprio(3); break;
    }
}

// Largest number of chunks per workgroup whose halos are staged in LDS; a
// launch with more chunks per workgroup reads them one by one instead.
constexpr int kHaloLds = 1024;

// Where a chunk's two outside neighbours come from in one iteration.
enum class HaloSrc { Direct, Staged, Coherent };

struct StencilGeom {
    int64_t n, chunk, nFullChunks, nChunks, G, w, kMax, myChunks;
};

// Exchange-buffer entry (workgroup v, chunk index k, end e) of parity p.
__device__ __forceinline__ int32_t* halo_entry(int32_t* base, const StencilGeom& g, int p,
                                               int64_t v, int64_t k, int e)
{
    return base + (((size_t)p * g.G + v) * g.kMax + k) * 2 + e;
}

// Outside neighbours of chunk k of this workgroup (c = w + k * G):
// x[c0 - 1] and x[c1], clamped at the array ends.
template <HaloSrc S>
__device__ __forceinline__ int32_t chunk_left(const StencilGeom& g, const int32_t* x, int64_t k,
                                              const int32_t* inLeft, int32_t* halo, int p)
{
    const int64_t c = g.w + k * g.G;
    if constexpr (S == HaloSrc::Direct) {
        const int64_t c0 = c * g.chunk;
        return x[c0 > 0 ? c0 - 1 : 0];
    } else if constexpr (S == HaloSrc::Staged) {
        return inLeft[k];
    } else {
        if (c == 0) return x[0];
        return ccb_load_coherent(g.w > 0 ? halo_entry(halo, g, p, g.w - 1, k, 1)
                                         : halo_entry(halo, g, p, g.G - 1, k - 1, 1));
    }
}
template <HaloSrc S>
__device__ __forceinline__ int32_t chunk_right(const StencilGeom& g, const int32_t* x, int64_t k,
                                               const int32_t* inRight, int32_t* halo, int p)
{
    const int64_t c = g.w + k * g.G;
    if constexpr (S == HaloSrc::Direct) {
        const int64_t c1 = c * g.chunk + g.chunk;
        return x[c1 < g.n ? c1 : g.n - 1];
    } else if constexpr (S == HaloSrc::Staged) {
        return inRight[k];
    } else {
        if (c + 1 >= g.nChunks) return x[g.n - 1];
        return ccb_load_coherent(g.w + 1 < g.G ? halo_entry(halo, g, p, g.w + 1, k, 0)
                                               : halo_entry(halo, g, p, 0, k + 1, 0));
    }
}

// One iteration over this workgroup's chunks.  pubFirst/pubLast (LDS, may be
// null) receive each chunk's first and last output; pubHalo (may be null)
// receives them directly with device-coherent stores.
template <HaloSrc S>
__device__ __forceinline__ void stencil_sweep(const StencilGeom& g, const int32_t* __restrict__ x,
                                              int32_t* __restrict__ y, const int32_t* inLeft,
                                              const int32_t* inRight, int32_t* halo, int pIn,
                                              int32_t* pubFirst, int32_t* pubLast,
                                              int32_t* pubHalo, int pOut)
{
    const int lane = threadIdx.x % kWave;
    // wave index as a scalar: branches on it are uniform
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
    const int nWave = blockDim.x / kWave;
    const int64_t fullMine = g.w < g.nFullChunks ? (g.nFullChunks - 1 - g.w) / g.G + 1 : 0;
    // One full chunk in two halves: its loads, then the rest (so that a
    // second chunk's loads can go out before this one's stores).
    struct ChunkIn {
        int4 v;
        int32_t lh, rh;
    };
    auto load = [&](int64_t k) {
        const int64_t c = g.w + k * g.G;
        const int64_t w0 = c * g.chunk + (int64_t)wave * 256;  // this wave's piece
        ChunkIn in;
        in.v = load4<ccb::kStencilNTLoad>(x + w0 + 4 * lane);
        if (wave == 0) in.lh = chunk_left<S>(g, x, k, inLeft, halo, pIn);
        else in.lh = x[w0 - 1];
        if (wave == nWave - 1) in.rh = chunk_right<S>(g, x, k, inRight, halo, pIn);
        else in.rh = x[w0 + 256];
        return in;
    };
    auto finish = [&](int64_t k, const ChunkIn& in) {
        const int64_t w0 = (g.w + k * g.G) * g.chunk + (int64_t)wave * 256;
        int32_t left = lane_from_left(in.v.w);
        int32_t right = lane_from_right(in.v.x);
        if (lane == 0) left = in.lh;
        if (lane == kWave - 1) right = in.rh;
        int4 o;
        o.x = st3(left, in.v.x, in.v.y);
        o.y = st3(in.v.x, in.v.y, in.v.z);
        o.z = st3(in.v.y, in.v.z, in.v.w);
        o.w = st3(in.v.z, in.v.w, right);
        store4<ccb::kStencilNT>(y + w0 + 4 * lane, o);
        if (wave == 0 && lane == 0) {
            if (pubFirst != nullptr) pubFirst[k] = o.x;
            if (pubHalo != nullptr) ccb_store_coherent(halo_entry(pubHalo, g, pOut, g.w, k, 0), o.x);
        }
        if (wave == nWave - 1 && lane == kWave - 1) {
            if (pubLast != nullptr) pubLast[k] = o.w;
            if (pubHalo != nullptr) ccb_store_coherent(halo_entry(pubHalo, g, pOut, g.w, k, 1), o.w);
        }
    };
    // Rotate the wave priority chunk by chunk.  With equal priorities the
    // oldest wave wins every issue arbitration, so of the workgroups sharing
    // a CU the last-dispatched one finishes each iteration ~9 us behind the
    // first, and the barrier waits for it.  Rotating makes the workgroups
    // take turns (w * 4 / G is the dispatch round).
    const int prio0 = (int)(g.w * 4 / g.G);
    int64_t k = 0;
    constexpr int kG = ccb::kStencilGroup;
    if constexpr (kG > 1) {
        for (; k + kG <= fullMine; k += kG) {
            set_prio(prio0 + (int)(k / kG));
            ChunkIn in[kG];
#pragma unroll
            for (int i = 0; i < kG; ++i) in[i] = load(k + i);
#pragma unroll
            for (int i = 0; i < kG; ++i) finish(k + i, in[i]);
        }
    }
    for (; k < fullMine; ++k) {
        set_prio(prio0 + (int)k);
        finish(k, load(k));
    }
    set_prio(0);
    if (fullMine < g.myChunks) {
        // the partial last chunk, one element per thread
        const int64_t k = fullMine;
        const int64_t c0 = (g.w + k * g.G) * g.chunk;
        const int32_t cl = chunk_left<S>(g, x, k, inLeft, halo, pIn);
        for (int64_t e = c0 + threadIdx.x; e < g.n; e += blockDim.x) {
            const int32_t a = e == c0 ? cl : x[e - 1];
            const int32_t b = e + 1 < g.n ? x[e + 1] : x[g.n - 1];
            const int32_t o = st3(a, x[e], b);
            y[e] = o;
            if (e == c0) {
                if (pubFirst != nullptr) pubFirst[k] = o;
                if (pubHalo != nullptr) ccb_store_coherent(halo_entry(pubHalo, g, pOut, g.w, k, 0), o);
            }
            if (e == g.n - 1) {
                if (pubLast != nullptr) pubLast[k] = o;
                if (pubHalo != nullptr) ccb_store_coherent(halo_entry(pubHalo, g, pOut, g.w, k, 1), o);
            }
        }
    }
}

}  // namespace

// The exchange buffer is workgroup-major: halo[parity][w][k][2] holds the
// first and last output element of workgroup w's k-th chunk (chunk
// w + k * G).  Only wave 0 (which needs the left neighbours of the chunks)
// and the last wave (right neighbours) touch it: at the start of an
// iteration each copies the entries it needs into its own LDS array with
// device-coherent loads issued next to its first data load, and at the end
// each publishes its own entries from LDS.  No workgroup barrier is needed
// for that, and the other waves never wait on a coherent access.
template <int K, ccbVisibility V>
__global__ __launch_bounds__(1024) void ccb_k_stencil(int32_t* bufA, int32_t* bufB, int64_t n,
                                                       int32_t iters, int32_t* ws, int32_t* halo,
                                                       uint64_t* timeline, uint32_t maxPoll)
{
    __shared__ int32_t inLeft[kHaloLds], inRight[kHaloLds];   // neighbours of my chunks
    __shared__ int32_t outFirst[kHaloLds], outLast[kHaloLds]; // my chunks' end outputs
    if (register_query(maxPoll, ws)) return;
    StencilGeom g;
    g.n = n;
    g.chunk = 4 * (int64_t)blockDim.x;
    g.nFullChunks = n / g.chunk;
    g.nChunks = (n + g.chunk - 1) / g.chunk;
    g.G = gridDim.x;
    g.w = blockIdx.x;
    g.kMax = (g.nChunks + g.G - 1) / g.G;  // chunks of the busiest workgroup
    g.myChunks = g.w < g.nChunks ? (g.nChunks - 1 - g.w) / g.G + 1 : 0;
    const bool staged = g.kMax <= kHaloLds;
    const int lane = threadIdx.x % kWave;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
    const int nWave = blockDim.x / kWave;
    int32_t* err = ws + CCB_STRIPES * CCB_LINE_WORDS;
    ccb_xcd_team team = {};
    // timeline (optional): per workgroup, the start, then for every iteration
    // the end of its data phase and the moment it left the following barrier
    uint64_t* stamps = timeline != nullptr ? timeline + (size_t)g.w * (2 * (size_t)iters + 1) : nullptr;
    if (stamps != nullptr && threadIdx.x == 0) stamps[0] = wall_clock64();
    for (int32_t t = 0; t < iters; ++t) {
        const int32_t* x = (t & 1) ? bufB : bufA;
        int32_t* y = (t & 1) ? bufA : bufB;
        const bool publish = V == CCB_VIS_ORDER && t + 1 < iters;
        const int pIn = (t - 1) & 1, pOut = t & 1;
        if (V != CCB_VIS_ORDER || t == 0) {
            stencil_sweep<HaloSrc::Direct>(g, x, y, nullptr, nullptr, halo, pIn,
                                           publish && staged ? outFirst : nullptr,
                                           publish && staged ? outLast : nullptr,
                                           publish && !staged ? halo : nullptr, pOut);
        } else if (staged) {
            if (wave == 0)
                for (int64_t k = lane; k < g.myChunks; k += kWave)
                    inLeft[k] = chunk_left<HaloSrc::Coherent>(g, x, k, nullptr, halo, pIn);
            if (wave == nWave - 1)
                for (int64_t k = lane; k < g.myChunks; k += kWave)
                    inRight[k] = chunk_right<HaloSrc::Coherent>(g, x, k, nullptr, halo, pIn);
            if (g.myChunks > 0 && (g.w + (g.myChunks - 1) * g.G) >= g.nFullChunks) {
                // a partial chunk reads its left neighbour from every thread
                __syncthreads();
            }
            stencil_sweep<HaloSrc::Staged>(g, x, y, inLeft, inRight, halo, pIn,
                                           publish ? outFirst : nullptr,
                                           publish ? outLast : nullptr, nullptr, pOut);
        } else {
            stencil_sweep<HaloSrc::Coherent>(g, x, y, nullptr, nullptr, halo, pIn, nullptr,
                                             nullptr, publish ? halo : nullptr, pOut);
        }
        if (publish && staged) {
            const bool partial = g.myChunks > 0 && (g.w + (g.myChunks - 1) * g.G) >= g.nFullChunks;
            if (partial) __syncthreads();  // partial-chunk ends come from any thread
            if (wave == 0 || partial)
                for (int64_t k = (partial ? threadIdx.x : lane); k < g.myChunks;
                     k += (partial ? blockDim.x : kWave))
                    ccb_store_coherent(halo_entry(halo, g, pOut, g.w, k, 0), outFirst[k]);
            if (wave == nWave - 1 || partial)
                for (int64_t k = (partial ? threadIdx.x : lane); k < g.myChunks;
                     k += (partial ? blockDim.x : kWave))
                    ccb_store_coherent(halo_entry(halo, g, pOut, g.w, k, 1), outLast[k]);
        }
        if (stamps != nullptr) {
            __syncthreads();
            if (threadIdx.x == 0) stamps[1 + 2 * t] = wall_clock64();
        }
        if (t + 1 < iters) {
            // Only the coherent halo stores are shared with other workgroups
            // across the barrier, so only the waves that issued them wait for
            // their memory operations; the data stores are read back by this
            // workgroup alone (ordered by the workgroup barrier).
            if (V == CCB_VIS_ORDER) {
                const bool partial =
                    g.myChunks > 0 && (g.w + (g.myChunks - 1) * g.G) >= g.nFullChunks;
                if (wave == 0 || wave == nWave - 1 || partial || !staged) ccb_wait_memory();
            }
            if (ccb_barrier<K, V, false>(ws, (int32_t)g.G, (int32_t)g.w, maxPoll, err, team) != CCB_OK)
                break;
        }
        if (stamps != nullptr && threadIdx.x == 0) stamps[2 + 2 * t] = wall_clock64();
    }
}

// ---------------------------------------------------------------------------
// CntNotify operations (CntNotify interfaces §3.1 record modes, §3.2 wait
// predicates; unsigned 32-bit arithmetic per §3.3).
// ---------------------------------------------------------------------------
namespace {

// Wait predicate; *bad set for a code above 4.
__device__ __forceinline__ bool cnt_holds(uint32_t c, uint32_t mode, uint32_t v, bool& bad)
{
    bad = mode > CCB_CNT_WAIT_EQUAL_WITH_BITMASK;
    bool h = false;
    h = mode == CCB_CNT_WAIT_LESS ? (c < v) : h;
    h = mode == CCB_CNT_WAIT_EQUAL ? (c == v) : h;
    h = mode == CCB_CNT_WAIT_BIGGER ? (c > v) : h;
    h = mode == CCB_CNT_WAIT_BIGGER_OR_EQUAL ? (c >= v) : h;
    h = mode == CCB_CNT_WAIT_EQUAL_WITH_BITMASK ? ((c & v) == v) : h;
    return h;
}

// One op of the batched engine on one counter (meta byte m: bits 0-2 mode,
// bit 3 isClear, bits 4-6 reserved, bit 7 wait).  Returns true when the op
// is a wait (its release flag in flag).  rowOk: the wait has an output row;
// a wait without one is malformed and leaves the count alone.  Written for
// the vector ALU, which bounds this engine about as much as HBM does: a
// record compares its low seven bits with the four record codes directly
// (a set clear or reserved bit, or the missing code 3, matches none of them
// and keeps the count), so the same comparisons give the result and the
// validity.
__device__ __forceinline__ bool cnt_step(uint32_t& c, uint32_t m, uint32_t v, bool rowOk,
                                         bool& bad, uint8_t& flag)
{
    if ((m & 0x80u) != 0) {
        const uint32_t mode = m & 0x77u;  // mode and reserved bits
        bool h = false;
        h = mode == CCB_CNT_WAIT_LESS ? (c < v) : h;
        h = mode == CCB_CNT_WAIT_EQUAL ? (c == v) : h;
        h = mode == CCB_CNT_WAIT_BIGGER ? (c > v) : h;
        h = mode == CCB_CNT_WAIT_BIGGER_OR_EQUAL ? (c >= v) : h;
        h = mode == CCB_CNT_WAIT_EQUAL_WITH_BITMASK ? ((c & v) == v) : h;
        const bool ok = mode <= CCB_CNT_WAIT_EQUAL_WITH_BITMASK && rowOk;
        const bool rel = h && ok;
        // the clear follows the release (CntNotify interfaces §3.3, §7)
        c = (rel && (m & 8u) != 0) ? 0u : c;
        flag = rel ? 1 : 0;
        bad = bad || !ok;
        return true;
    }
    const uint32_t op = m & 0x7Fu;
    const bool set = op == CCB_CNT_RECORD_SET_VALUE, add = op == CCB_CNT_RECORD_ADD;
    const bool bor = op == CCB_CNT_RECORD_BIT_OR, band = op == CCB_CNT_RECORD_BIT_AND;
    uint32_t r = c;
    r = set ? v : r;
    r = add ? c + v : r;
    r = bor ? (c | v) : r;
    r = band ? (c & v) : r;
    c = r;
    bad = bad || !(set || add || bor || band);
    return false;
}

// A record op in the form the fast path below uses: the new count is
// (c & X) + (v & Y), X = (v & A) ^ B, with masks A, B, Y of 0 or ~0 chosen
// by the code:
//   SET (0): A = 0,  B = 0,  Y = ~0  ->  v
//   ADD (1): A = 0,  B = ~0, Y = ~0  ->  c + v
//   OR  (2): A = ~0, B = ~0, Y = ~0  ->  (c & ~v) + v = c | v
//   AND (4): A = ~0, B = 0,  Y = 0   ->  c & v
// and the codes 3, 5, 6, 7: A = 0, B = ~0, Y = 0, the count is kept (they
// are reported once at the end instead of being tested on every op).
//
// For rows whose op bytes are all below 8 (a record code and no clear or
// reserved bit), the four counters of a lane look their masks up together:
// v_perm_b32 with the op word as selector picks byte `code` of an 8-byte
// table (0x00 or 0xFF) for each counter, and each byte is then used sign-
// extended (an SDWA operand) as that counter's 32-bit mask.  A fourth table
// flags the codes that are not records (3, 5, 6, 7).  Table bytes for codes
// 0..7, low dword first (the perm selector's order):
//   A: 00 00 FF 00 | FF 00 00 00     B: 00 FF FF FF | 00 FF FF FF
//   Y: FF FF FF 00 | 00 00 00 00     invalid: 00 00 00 FF | 00 FF FF FF
constexpr uint32_t kPermA[2] = {0x00FF0000u, 0x000000FFu};
constexpr uint32_t kPermB[2] = {0xFFFFFF00u, 0xFFFFFF00u};
constexpr uint32_t kPermY[2] = {0x00FFFFFFu, 0x00000000u};
constexpr uint32_t kPermBad[2] = {0xFF000000u, 0xFFFFFF00u};

__device__ __forceinline__ uint32_t perm_table(const uint32_t (&t)[2], uint32_t sel)
{
    return __builtin_amdgcn_perm(t[1], t[0], sel);
}

// byte i of p, sign-extended: 0x00 -> 0, 0xFF -> ~0
__device__ __forceinline__ uint32_t byte_mask(uint32_t p, int i)
{
    return (uint32_t)(int32_t)(int8_t)(uint8_t)(p >> (8 * i));
}

// A wait op in the form the fast path below uses.  With
// r = (c < v) | (c == v) << 1 | ((c & v) == v) << 2, the predicate of wait
// code m is bit m * 8 + r of kWaitTable (LESS 0: r & 1; EQUAL 1: r & 2;
// BIGGER 2: r & 3 == 0; GE 3: r & 1 == 0; BITMASK 4: r & 4).  A code above 4
// or a reserved bit (clamped to 5) indexes zero bits: never released.
// seen collects 1 << code for the validity check at the end; rowOk (the same
// in every lane) says whether the wait has an output row.
constexpr uint64_t kWaitTable =
    0xAAull | (0xCCull << 8) | (0x11ull << 16) | (0x55ull << 24) | (0xF0ull << 32);
constexpr uint32_t kWaitValid = 0x1Fu;

__device__ __forceinline__ uint32_t cnt_wait_fast(uint32_t& c, uint32_t b, uint32_t v,
                                                  bool rowOk, uint32_t& seen)
{
    const uint32_t mode = b & 0x77u;  // wait code and reserved bits
    const uint32_t mc = mode < 5u ? mode : 5u;
    const uint32_t r = (c < v ? 1u : 0u) | (c == v ? 2u : 0u) | ((c & v) == v ? 4u : 0u);
    const uint32_t rel = rowOk ? (uint32_t)(kWaitTable >> (mc * 8u + r)) & 1u : 0u;
    seen |= 1u << (mode < 31u ? mode : 31u);
    // the clear follows the release (CntNotify interfaces §3.3, §7)
    c = (rel & (b >> 3)) != 0 ? 0u : c;
    return rel;
}

}  // namespace

// C adjacent counters per thread (C = 1, 2 or 4): C-byte meta loads and
// 4C-byte operand loads per op; nCounters must be a multiple of C.
template <int C> struct CntVec;
template <> struct CntVec<4> {
    typedef unsigned int val __attribute__((ext_vector_type(4)));
    typedef uint32_t meta;
};
template <> struct CntVec<2> {
    typedef unsigned int val __attribute__((ext_vector_type(2)));
    typedef uint16_t meta;
};
template <> struct CntVec<1> {
    typedef unsigned int val __attribute__((ext_vector_type(1)));
    typedef uint8_t meta;
};

template <int C, int U>
__global__ __launch_bounds__(256) void ccb_k_cnt_batch(const uint32_t* __restrict__ val,
                                                       const uint8_t* __restrict__ meta,
                                                       int64_t nCounters, int32_t nOps,
                                                       uint32_t* __restrict__ finalOut,
                                                       uint8_t* __restrict__ rel,
                                                       int32_t nRelRows, int32_t* err)
{
    typedef typename CntVec<C>::val VT;
    typedef typename CntVec<C>::meta MT;
    const int64_t c0 = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * C;
    if (c0 >= nCounters) return;
    uint32_t c[C];
    int32_t j[C];
#pragma unroll
    for (int i = 0; i < C; ++i) c[i] = 0u, j[i] = 0;
    bool bad = false;
    uint32_t recBad = 0;  // invalid record codes seen by the fast path
    uint32_t seenW[C];
#pragma unroll
    for (int i = 0; i < C; ++i) seenW[i] = 1u;
    constexpr uint32_t kWaitBits = C == 4 ? 0x80808080u : (C == 2 ? 0x8080u : 0x80u);
    constexpr uint32_t kHighBits = C == 4 ? 0xF8F8F8F8u : (C == 2 ? 0xF8F8u : 0xF8u);
    auto apply = [&](uint32_t m, VT v) {
        if (!__any((m & kHighBits) != 0)) {
            // every op of the wave is a record with a code below 8
            const uint32_t pA = perm_table(kPermA, m), pB = perm_table(kPermB, m);
            const uint32_t pY = perm_table(kPermY, m);
            recBad |= perm_table(kPermBad, m);
#pragma unroll
            for (int i = 0; i < C; ++i)
                c[i] = (c[i] & ((v[i] & byte_mask(pA, i)) ^ byte_mask(pB, i))) +
                       (v[i] & byte_mask(pY, i));
            return;
        }
        const uint32_t waits = m & kWaitBits;
        bool oneRow = true;
#pragma unroll
        for (int i = 1; i < C; ++i) oneRow = oneRow && j[i] == j[0];
        const int32_t jr = __builtin_amdgcn_readfirstlane(j[0]);
        if (__all(waits == kWaitBits && oneRow && j[0] == jr)) {
            // every counter of the wave waits, all on output row jr
            const bool rowOk = jr < nRelRows;
            uint32_t packed = 0;
#pragma unroll
            for (int i = 0; i < C; ++i)
                packed |= cnt_wait_fast(c[i], (m >> (8 * i)) & 0xffu, v[i], rowOk, seenW[i]) << (8 * i);
            if (rowOk) *reinterpret_cast<MT*>(rel + (int64_t)jr * nCounters + c0) = (MT)packed;
            else bad = true;
#pragma unroll
            for (int i = 0; i < C; ++i) j[i]++;
            return;
        }
        uint8_t f[C];
        bool w[C];
        bool allWait = true, sameRow = true;
#pragma unroll
        for (int i = 0; i < C; ++i) {
            f[i] = 0;
            w[i] = cnt_step(c[i], (m >> (8 * i)) & 0xffu, v[i], j[i] < nRelRows, bad, f[i]);
            allWait = allWait && w[i];
            sameRow = sameRow && j[i] == j[0];
        }
        if (allWait && sameRow && j[0] < nRelRows) {
            uint32_t packed = 0;
#pragma unroll
            for (int i = 0; i < C; ++i) packed |= (uint32_t)f[i] << (8 * i);
            *reinterpret_cast<MT*>(rel + (int64_t)j[0] * nCounters + c0) = (MT)packed;
#pragma unroll
            for (int i = 0; i < C; ++i) j[i]++;
        } else {
#pragma unroll
            for (int i = 0; i < C; ++i) {
                if (!w[i]) continue;
                if (j[i] < nRelRows) rel[(int64_t)j[i] * nCounters + c0 + i] = f[i];
                j[i]++;
            }
        }
    };
    auto load = [&](int32_t k, uint32_t& m, VT& v) {
        const MT* mp = reinterpret_cast<const MT*>(meta + (int64_t)k * nCounters + c0);
        const VT* vp = reinterpret_cast<const VT*>(val + (int64_t)k * nCounters + c0);
        if constexpr (ccb::kCntNTLoad) {
            m = __builtin_nontemporal_load(mp);
            v = __builtin_nontemporal_load(vp);
        } else {
            m = *mp;
            v = *vp;
        }
    };
    // Two register sets of U ops, A and B: one set's loads are in flight
    // while the other set is applied, so the vector ALU work of an op
    // overlaps the memory latency of the next.
    int32_t k = 0;
    uint32_t mA[U], mB[U];
    VT vA[U], vB[U];
    if (k + U <= nOps) {
#pragma unroll
        for (int u = 0; u < U; ++u) load(k + u, mA[u], vA[u]);
    }
    for (; k + 2 * U <= nOps; k += 2 * U) {
#pragma unroll
        for (int u = 0; u < U; ++u) load(k + U + u, mB[u], vB[u]);
#pragma unroll
        for (int u = 0; u < U; ++u) apply(mA[u], vA[u]);
        if (k + 3 * U <= nOps) {
#pragma unroll
            for (int u = 0; u < U; ++u) load(k + 2 * U + u, mA[u], vA[u]);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) apply(mB[u], vB[u]);
    }
    if (k + U <= nOps) {  // set A holds ops k .. k + U - 1
#pragma unroll
        for (int u = 0; u < U; ++u) apply(mA[u], vA[u]);
        k += U;
    }
    for (; k < nOps; ++k) {
        uint32_t m;
        VT v;
        load(k, m, v);
        apply(m, v);
    }
    VT out;
    // the perm of a C < 4 op word also reads its zero high bytes (code 0, valid)
    bad = bad || recBad != 0;
#pragma unroll
    for (int i = 0; i < C; ++i) {
        out[i] = c[i];
        bad = bad || (seenW[i] & ~kWaitValid) != 0;
    }
    *reinterpret_cast<VT*>(finalOut + c0) = out;
    if (bad && err != nullptr)
        __hip_atomic_store(err, (int32_t)CCB_ERR_INVALID_VALUE, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}

// Stream-ordered record (CntNotify interfaces §4.2): one device-scope atomic
// update of the count, after a release fence so that the producer stream's
// earlier stores are visible to whoever is released by this record.
__global__ void ccb_k_cnt_record(uint32_t* line, int32_t mode, uint32_t value)
{
    if (!leader()) return;
    ccb_fence_release_agent();
    switch (mode) {
    case CCB_CNT_RECORD_SET_VALUE:
        __hip_atomic_exchange(line, value, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
    case CCB_CNT_RECORD_ADD:
        __hip_atomic_fetch_add(line, value, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
    case CCB_CNT_RECORD_BIT_OR:
        __hip_atomic_fetch_or(line, value, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
    case CCB_CNT_RECORD_BIT_AND:
        __hip_atomic_fetch_and(line, value, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
    default:
        break;
    }
}

// Stream-ordered wait (CntNotify interfaces §4.3): poll the count until the
// predicate holds or the timeout passes.  A release with isClear swaps the
// count it saw for 0 in one compare-and-swap, so a record landing between
// the check and the clear makes the swap fail and the wait looks again.
// The outcome goes to the word after the count.
//
// cancel: a word in host memory (coherent, pinned) that the host changes to
// call off the waits enqueued before it; every 64 polls the wait reads it
// at system scope and, if it no longer holds `token`, ends with
// CCB_ERR_CANCELLED (no clear).  This is how a wait without a time limit
// can still be ended.
__global__ void ccb_k_cnt_wait(uint32_t* line, int32_t mode, uint32_t value, int32_t isClear,
                               uint64_t timeoutTicks, const uint32_t* cancel, uint32_t token)
{
    if (!leader()) return;
    int32_t* outcome = reinterpret_cast<int32_t*>(line + 1);
    const uint64_t t0 = wall_clock64();
    int32_t result = CCB_ERR_TIMEOUT;
    for (uint32_t polls = 1;; ++polls) {
        uint32_t c = __hip_atomic_load(line, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        bool bad;
        if (cnt_holds(c, (uint32_t)mode, value, bad)) {
            if (!isClear) { result = CCB_OK; break; }
            if (__hip_atomic_compare_exchange_strong(line, &c, 0u, __ATOMIC_RELAXED,
                                                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) {
                result = CCB_OK;
                break;
            }
            continue;  // the count moved under us: evaluate the new value
        }
        if (timeoutTicks != 0 && wall_clock64() - t0 >= timeoutTicks) break;
        if ((polls % 64) == 0 &&
            __hip_atomic_load(const_cast<uint32_t*>(cancel), __ATOMIC_RELAXED,
                              __HIP_MEMORY_SCOPE_SYSTEM) != token) {
            result = CCB_ERR_CANCELLED;
            break;
        }
        __builtin_amdgcn_s_sleep(2);
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    __hip_atomic_store(outcome, result, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Stream-ordered reset (CntNotify interfaces §4.4).
__global__ void ccb_k_cnt_reset(uint32_t* line)
{
    if (!leader()) return;
    ccb_fence_release_agent();
    __hip_atomic_store(line, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// One word copied device-to-device with a device-coherent read (the error
// word of a workspace into a caller's status word).
__global__ void ccb_k_copy_word(const int32_t* src, int32_t* dst)
{
    if (threadIdx.x == 0 && blockIdx.x == 0)
        *dst = __hip_atomic_load(const_cast<int32_t*>(src), __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
}

// Zero fill (used instead of a memset so that captured graphs hold no
// memset nodes).
__global__ void ccb_k_fill_zero(int32_t* p, int64_t nWords)
{
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nWords;
         i += (int64_t)gridDim.x * blockDim.x)
        p[i] = 0;
}

// ---------------------------------------------------------------------------
// Floor microbenchmarks.
// ---------------------------------------------------------------------------
// kind 0: dependent fetch-adds; kind 1: dependent atomic loads.  The address
// of each op depends on the previous result through `zero` (always 0), so
// the ops cannot overlap.
__global__ void ccb_k_atomic_chain(int32_t* line, uint64_t* ticks, int32_t iters, int32_t fenced,
                                   int32_t kind, int32_t zero)
{
    if (!leader()) return;
    int32_t v = 0;
    const uint64_t t0 = wall_clock64();
    if (kind == 0) {
        for (int32_t i = 0; i < iters; ++i) {
            if (fenced) ccb_fence_release_agent();
            v = __hip_atomic_fetch_add(line + (v & zero), 1, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
            if (fenced) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        }
    } else {
        for (int32_t i = 0; i < iters; ++i) {
            if (fenced) ccb_fence_release_agent();
            v = __hip_atomic_load(line + (v & zero), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (fenced) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        }
    }
    const uint64_t t1 = wall_clock64();
    ticks[0] = t0;
    ticks[1] = t1;
    if (v == 0x7fffffff) ticks[0] = 0;  // keep v live
}

__global__ void ccb_k_atomic_contended(int32_t* line, uint64_t* ticks, int32_t iters, int32_t zero)
{
    if (!leader()) return;
    int32_t v = 0;
    const uint64_t t0 = wall_clock64();
    for (int32_t i = 0; i < iters; ++i)
        v = __hip_atomic_fetch_add(line + (v & zero), 1, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
    const uint64_t t1 = wall_clock64();
    ticks[2 * blockIdx.x] = t0;
    ticks[2 * blockIdx.x + 1] = t1;
    if (v == 0x7fffffff) ticks[2 * blockIdx.x] = 0;
}

// Notification ping-pong: workgroup 0 and workgroup `peer` (one wave each)
// take turns.  Round i: workgroup 0 adds one to line A and polls line B until
// it holds i; the partner polls A until it holds i, then adds one to B.  The
// update is the barrier's arrival (an agent-scope fetch-add) and the wait is
// its poll (agent-scope loads with the same back-off), so each round trip is
// two notifications: one CU's update reaching another CU's poll.  Every wait
// is bounded by maxPoll (then the error word gets CCB_ERR_DEADLOCK and both
// sides stop).  ticks: start and end on workgroup 0's clock, then the XCC id
// of workgroup 0 and of the partner.
__global__ void ccb_k_notify_pingpong(int32_t* lines, uint64_t* ticks, int32_t iters,
                                      int32_t peer, uint32_t maxPoll, int32_t* err)
{
    const int32_t w = (int32_t)blockIdx.x;
    if (!leader() || (w != 0 && w != peer)) return;
    int32_t* const a = lines;
    int32_t* const b = lines + CCB_LINE_WORDS;
    int32_t* const watched = w == 0 ? b : a;
    bool bad = false;
    const uint64_t t0 = wall_clock64();
    for (int32_t i = 1; i <= iters && !bad; ++i) {
        if (w == 0) __hip_atomic_fetch_add(a, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        uint32_t polls = 0;
        while (__hip_atomic_load(watched, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < i) {
            if (++polls >= maxPoll) {
                bad = true;
                break;
            }
            if (CCB_POLL_SLEEP > 0) __builtin_amdgcn_s_sleep(CCB_POLL_SLEEP);
        }
        if (w != 0 && !bad) __hip_atomic_fetch_add(b, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    const uint64_t t1 = wall_clock64();
    if (w == 0) {
        ticks[0] = t0;
        ticks[1] = t1;
    }
    ticks[w == 0 ? 2 : 3] = __builtin_amdgcn_s_getreg((31 << 11) | 20);  // XCC_ID
    if (bad)
        __hip_atomic_store(err, (int32_t)CCB_ERR_DEADLOCK, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}

// Where the full-visibility barrier's cache maintenance can go: barrier-only
// rounds on the striped counter with one plain store before each barrier and
// one plain load after it, and the release (L2 write-back) and acquire
// (invalidate) placed per variant:
//   0  none (the ordering-only barrier)
//   1  every workgroup: release before its arrival, acquire after its poll
//      (CCB_VIS_FULL)
//   2  every workgroup: release only
//   3  every workgroup: acquire only
//   4  one release per XCD: once all members have arrived, one leader per
//      XCD writes its L2 back (and invalidates it) and raises that XCD's
//      flag; every workgroup waits for the flags of all XCDs with members,
//      then acquires
//   5  as 4, but the workgroups' acquire is the workgroup-scope invalidate
//      (`buffer_inv sc0`) instead of the agent-scope one
// Leaders are found at the start: each member adds one to its XCD's count
// (XCC_ID) and the first one in is the leader; one ordering-only barrier
// later every member reads the counts (which XCDs have members).  In round
// r member w stores r + 1 to its data line and afterwards loads member
// (w + 1) mod N's; stale[w] counts the loads that returned less than r + 1.
// scratch (int32 words, zeroed by the caller): stripes [0, 64 lines), the
// error word at line 64, XCD flags at lines 65..72, XCD counts at lines
// 73..80, then one data line per member.
namespace {
constexpr int kFpErrLine = CCB_STRIPES, kFpFlagLine = CCB_STRIPES + 1;
constexpr int kFpRegLine = CCB_STRIPES + 9, kFpDataLine = CCB_STRIPES + 17;
}  // namespace

template <int kVariant>
__global__ __launch_bounds__(1024) void ccb_k_fence_placement(int32_t* scratch, int32_t* stale,
                                                               int32_t rounds, uint32_t maxPoll)
{
    constexpr int W = CCB_LINE_WORDS;
    __shared__ int32_t result;
    __shared__ int32_t shRank, shMask;
    const int32_t n = gridDim.x, w = blockIdx.x;
    const int lane = (int)__lane_id();
    int32_t* const ws = scratch;
    int32_t* const err = scratch + kFpErrLine * W;
    const uint32_t xcc = __builtin_amdgcn_s_getreg((31 << 11) | 20) & 7u;  // XCC_ID
    constexpr bool kLeaders = kVariant >= 4;
    if constexpr (kLeaders) {
        if (threadIdx.x == 0)
            shRank = __hip_atomic_fetch_add(scratch + (kFpRegLine + xcc) * W, 1, __ATOMIC_RELAXED,
                                            __HIP_MEMORY_SCOPE_AGENT);
        if (ccb_barrier<CCB_STRIPES, CCB_VIS_ORDER>(ws, n, w, maxPoll, err) != CCB_OK) return;
        if (threadIdx.x < kWave) {
            const int32_t c = lane < 8 ? __hip_atomic_load(scratch + (kFpRegLine + lane) * W,
                                                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                                       : 0;
            const uint64_t m = __ballot(c > 0);
            if (threadIdx.x == 0) shMask = (int32_t)m;
        }
        __syncthreads();
    }
    const bool lead = kLeaders && shRank == 0;
    const uint32_t mask = kLeaders ? (uint32_t)shMask : 0u;
    int32_t* const mine = scratch + (kFpDataLine + w) * W;
    const int32_t* const next = scratch + (kFpDataLine + (w + 1) % n) * W;
    int32_t bad = 0;
    for (int32_t r = 0; r < rounds; ++r) {
        if (threadIdx.x == 0) *mine = r + 1;  // plain store
        ccb_wait_memory();
        __syncthreads();
        if (threadIdx.x < kWave) {
            int32_t before = 0, rc;
            if constexpr (kVariant == 1 || kVariant == 2) {
                if (threadIdx.x == 0) before = ccb_arrive<CCB_STRIPES, CCB_VIS_FULL>(ws, w);
            } else {
                if (threadIdx.x == 0) before = ccb_arrive<CCB_STRIPES, CCB_VIS_ORDER>(ws, w);
            }
            if constexpr (kVariant == 1 || kVariant == 3)
                rc = ccb_await<CCB_STRIPES, CCB_VIS_FULL>(ws, n, w, before, maxPoll, err);
            else
                rc = ccb_await<CCB_STRIPES, CCB_VIS_ORDER>(ws, n, w, before, maxPoll, err);
            if constexpr (kLeaders) {
                // the second phase: every member's stores are in its XCD's L2
                const int32_t epoch = r + 2;  // the registration used round 1
                if (rc == CCB_OK && lead) {
                    ccb_fence_release_agent();
                    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
                    if (threadIdx.x == 0)
                        __hip_atomic_store(scratch + (kFpFlagLine + xcc) * W, epoch, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
                }
                bool done = rc != CCB_OK || lane >= 8 || ((mask >> lane) & 1u) == 0;
                uint32_t polls = 0;
                const int32_t* flag = scratch + (kFpFlagLine + (lane < 8 ? lane : 0)) * W;
                while (!__all(done)) {
                    const int32_t v = __hip_atomic_load(const_cast<int32_t*>(flag), __ATOMIC_RELAXED,
                                                        __HIP_MEMORY_SCOPE_AGENT);
                    done = done || v >= epoch;
                    if (__all(done)) break;
                    if (++polls >= maxPoll) {
                        rc = CCB_ERR_DEADLOCK;
                        if (lane == 0)
                            __hip_atomic_store(err, rc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        break;
                    }
                    if ((polls % CCB_ERR_CHECK_EVERY) == 0) {
                        const int32_t e =
                            __hip_atomic_load(err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        if (e != CCB_OK) {
                            rc = e;
                            break;
                        }
                    }
                    __builtin_amdgcn_s_sleep(1);
                }
                if constexpr (kVariant == 4) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
                if constexpr (kVariant == 5) asm volatile("buffer_inv sc0" ::: "memory");
            }
            if (threadIdx.x == 0) result = rc;
        }
        __syncthreads();
        if (result != CCB_OK) break;
        if (threadIdx.x == 0 && *next < r + 1) ++bad;  // plain load
    }
    if (threadIdx.x == 0) stale[w] = bad;
}

// HIP's own grid barrier (cooperative groups' grid sync), `rounds` times in a
// row: the platform's stock answer to the same problem, timed beside ours.
// Workgroup 0 writes `rounds` to *done once it has passed the last one.
__global__ void ccb_k_hip_grid_sync(int32_t rounds, int32_t* done)
{
    cooperative_groups::grid_group g = cooperative_groups::this_grid();
    for (int32_t r = 0; r < rounds; ++r) g.sync();
    if (blockIdx.x == 0 && threadIdx.x == 0)
        __hip_atomic_store(done, rounds, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Streaming copy: every thread moves one 16-byte vector per step and the
// whole grid advances through memory together (the access order that gets
// the most out of HBM on this GPU), loads and stores non-temporal.
__global__ __launch_bounds__(256) void ccb_k_copy(int4* __restrict__ dst,
                                                  const int4* __restrict__ src, int64_t n16)
{
    typedef int v4i __attribute__((ext_vector_type(4)));
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride) {
        const v4i v = __builtin_nontemporal_load(reinterpret_cast<const v4i*>(src + i));
        __builtin_nontemporal_store(v, reinterpret_cast<v4i*>(dst + i));
    }
}

// ---------------------------------------------------------------------------
// Launch helpers (called by the validated C entry points in ccb_api.hip).
// ---------------------------------------------------------------------------
namespace ccb {

static hipError_t coop(const void* fn, int nGrid, int threads, size_t lds, hipStream_t s,
                       void** args)
{
    return hipLaunchCooperativeKernel(fn, dim3(nGrid), dim3(threads), args, (unsigned)lds, s);
}

// Each mode's kernel instance (an invalid mode falls through to the last;
// the entry points reject invalid modes first).
#define CCB_PICK_X(kernel, mode, x)                                                            \
    ((mode) == (CCB_BARRIER_STRIPED | CCB_VISIBILITY_ORDER)                                    \
         ? reinterpret_cast<const void*>(&kernel<CCB_STRIPES, CCB_VIS_ORDER, x>)               \
     : (mode) == (CCB_BARRIER_STRIPED | CCB_VISIBILITY_FULL)                                   \
         ? reinterpret_cast<const void*>(&kernel<CCB_STRIPES, CCB_VIS_FULL, x>)                \
     : (mode) == (CCB_BARRIER_STRIPED | CCB_VISIBILITY_XCD)                                    \
         ? reinterpret_cast<const void*>(&kernel<CCB_STRIPES, CCB_VIS_XCD, x>)                 \
     : (mode) == (CCB_BARRIER_FLAT | CCB_VISIBILITY_ORDER)                                     \
         ? reinterpret_cast<const void*>(&kernel<1, CCB_VIS_ORDER, x>)                         \
     : (mode) == (CCB_BARRIER_FLAT | CCB_VISIBILITY_FULL)                                      \
         ? reinterpret_cast<const void*>(&kernel<1, CCB_VIS_FULL, x>)                          \
     : (mode) == (CCB_BARRIER_FLAT | CCB_VISIBILITY_XCD)                                       \
         ? reinterpret_cast<const void*>(&kernel<1, CCB_VIS_XCD, x>)                           \
     : (mode) == (CCB_BARRIER_TREE | CCB_VISIBILITY_ORDER)                                     \
         ? reinterpret_cast<const void*>(&kernel<ccb_tree(CCB_TREE_GROUPS), CCB_VIS_ORDER, x>) \
     : (mode) == (CCB_BARRIER_TREE | CCB_VISIBILITY_FULL)                                      \
         ? reinterpret_cast<const void*>(&kernel<ccb_tree(CCB_TREE_GROUPS), CCB_VIS_FULL, x>)  \
         : reinterpret_cast<const void*>(&kernel<ccb_tree(CCB_TREE_GROUPS), CCB_VIS_XCD, x>))

#define CCB_PICK(kernel, mode)                                                              \
    ((mode) == (CCB_BARRIER_STRIPED | CCB_VISIBILITY_ORDER)                                 \
         ? reinterpret_cast<const void*>(&kernel<CCB_STRIPES, CCB_VIS_ORDER>)               \
     : (mode) == (CCB_BARRIER_STRIPED | CCB_VISIBILITY_FULL)                                \
         ? reinterpret_cast<const void*>(&kernel<CCB_STRIPES, CCB_VIS_FULL>)                \
     : (mode) == (CCB_BARRIER_STRIPED | CCB_VISIBILITY_XCD)                                 \
         ? reinterpret_cast<const void*>(&kernel<CCB_STRIPES, CCB_VIS_XCD>)                 \
     : (mode) == (CCB_BARRIER_FLAT | CCB_VISIBILITY_ORDER)                                  \
         ? reinterpret_cast<const void*>(&kernel<1, CCB_VIS_ORDER>)                         \
     : (mode) == (CCB_BARRIER_FLAT | CCB_VISIBILITY_FULL)                                   \
         ? reinterpret_cast<const void*>(&kernel<1, CCB_VIS_FULL>)                          \
     : (mode) == (CCB_BARRIER_FLAT | CCB_VISIBILITY_XCD)                                    \
         ? reinterpret_cast<const void*>(&kernel<1, CCB_VIS_XCD>)                           \
     : (mode) == (CCB_BARRIER_TREE | CCB_VISIBILITY_ORDER)                                  \
         ? reinterpret_cast<const void*>(&kernel<ccb_tree(CCB_TREE_GROUPS), CCB_VIS_ORDER>) \
     : (mode) == (CCB_BARRIER_TREE | CCB_VISIBILITY_FULL)                                   \
         ? reinterpret_cast<const void*>(&kernel<ccb_tree(CCB_TREE_GROUPS), CCB_VIS_FULL>)  \
         : reinterpret_cast<const void*>(&kernel<ccb_tree(CCB_TREE_GROUPS), CCB_VIS_XCD>))

const void* kernel_ptr(KernelId id, int32_t mode)
{
    switch (id) {
    case KernelId::BarrierOnly: return CCB_PICK_X(ccb_k_barrier_only, mode, false);
    case KernelId::BarrierStamps: return CCB_PICK_X(ccb_k_barrier_only, mode, true);
    case KernelId::SlotRounds: return CCB_PICK(ccb_k_slot_rounds, mode);
    case KernelId::GroupedRounds: return CCB_PICK_X(ccb_k_grouped_rounds, mode, false);
    case KernelId::GroupedStamps: return CCB_PICK_X(ccb_k_grouped_rounds, mode, true);
    case KernelId::Stencil: return CCB_PICK(ccb_k_stencil, mode);
    }
    return nullptr;
}

hipError_t launch_barrier_only(const LaunchShape& ls, int32_t* ws, uint32_t* placement,
                               int32_t* wgStatus, uint64_t* stamps, int32_t rounds,
                               int32_t nMembers, uint32_t maxPoll)
{
    void* args[] = {&ws, &placement, &wgStatus, &stamps, &rounds, &nMembers, &maxPoll};
    return coop(ls.fn, ls.nGrid, ls.threads, ls.lds, ls.stream, args);
}

hipError_t launch_slot_rounds(const LaunchShape& ls, int32_t* ws, uint32_t* slots, uint32_t* out,
                              int32_t* wgStatus, uint64_t seed, int32_t rounds, int32_t nMembers,
                              uint32_t maxPoll)
{
    void* args[] = {&ws, &slots, &out, &wgStatus, &seed, &rounds, &nMembers, &maxPoll};
    return coop(ls.fn, ls.nGrid, ls.threads, ls.lds, ls.stream, args);
}

hipError_t launch_grouped_rounds(const LaunchShape& ls, int32_t* ws, uint32_t* slots,
                                 uint32_t* out, int32_t* wgStatus, uint64_t* stamps, uint64_t seed,
                                 int32_t rounds, uint32_t maxPoll)
{
    void* args[] = {&ws, &slots, &out, &wgStatus, &stamps, &seed, &rounds, &maxPoll};
    return coop(ls.fn, ls.nGrid, ls.threads, ls.lds, ls.stream, args);
}

hipError_t launch_stencil(const LaunchShape& ls, int32_t* bufA, int32_t* bufB, int64_t n,
                          int32_t iters, int32_t* ws, int32_t* halo, uint64_t* timeline,
                          uint32_t maxPoll)
{
    void* args[] = {&bufA, &bufB, &n, &iters, &ws, &halo, &timeline, &maxPoll};
    return coop(ls.fn, ls.nGrid, ls.threads, ls.lds, ls.stream, args);
}

// Where the register query stores its answer: one word per device, so that
// the query needs no allocation.
__device__ __align__(128) int32_t g_register_query[32];

hipError_t register_query_word(int32_t** out)
{
    return hipGetSymbolAddress(reinterpret_cast<void**>(out), HIP_SYMBOL(g_register_query));
}

hipError_t launch_register_query(KernelId id, int32_t mode, int32_t* out, hipStream_t s)
{
    const void* fn = kernel_ptr(id, mode);
    void* none = nullptr;
    int64_t zero64 = 0;
    int32_t zero = 0;
    uint64_t seed = 0;
    uint32_t query = 0;  // maxPoll == 0: the register query
    switch (id) {
    case KernelId::BarrierOnly:
    case KernelId::BarrierStamps: {
        void* args[] = {&out, &none, &none, &none, &zero, &zero, &query};
        return hipLaunchKernel(fn, dim3(1), dim3(kWave), args, 0, s);
    }
    case KernelId::SlotRounds: {
        void* args[] = {&out, &none, &none, &none, &seed, &zero, &zero, &query};
        return hipLaunchKernel(fn, dim3(1), dim3(kWave), args, 0, s);
    }
    case KernelId::GroupedRounds:
    case KernelId::GroupedStamps: {
        void* args[] = {&out, &none, &none, &none, &none, &seed, &zero, &query};
        return hipLaunchKernel(fn, dim3(1), dim3(kWave), args, 0, s);
    }
    case KernelId::Stencil: {
        void* args[] = {&none, &none, &zero64, &zero, &out, &none, &none, &query};
        return hipLaunchKernel(fn, dim3(1), dim3(kWave), args, 0, s);
    }
    }
    return hipErrorInvalidValue;
}

// ---------------------------------------------------------------------------
// Scratch of the allocation-free stencil entry point: the barrier workspace
// (CCB_STRIPES stripe lines and the error line, padded to 256 bytes) and then
// the halo exchange buffer, in one file-scope device array of
// CCB_NOALLOC_SCRATCH_BYTES.  Every GPU the library runs on holds its own
// copy until the process ends.  In host code the array's name is only a
// host-side stand-in: its device address on the current device comes from
// hipGetSymbolAddress, looked up once per device with that device current
// and kept per device.
// ---------------------------------------------------------------------------
static __device__ __align__(256) int32_t scratch[CCB_NOALLOC_SCRATCH_BYTES / 4];

namespace {
constexpr int kScratchDevices = 64;
std::mutex g_scratch_mu;
int32_t* g_scratch_ptr[kScratchDevices] = {};
}  // namespace

hipError_t noalloc_scratch(int dev, int32_t** out)
{
    if (dev < 0 || dev >= kScratchDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_scratch_ptr[dev] = static_cast<int32_t*>(p);
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

hipError_t launch_copy_word(const int32_t* src, int32_t* dst, hipStream_t s)
{
    hipLaunchKernelGGL(ccb_k_copy_word, dim3(1), dim3(kWave), 0, s, src, dst);
    return hipGetLastError();
}

hipError_t launch_cnt_batch(const uint32_t* val, const uint8_t* meta, int64_t nCounters,
                            int32_t nOps, uint32_t* finalOut, uint8_t* rel, int32_t nRelRows,
                            int32_t* err, int perThread, hipStream_t s)
{
    constexpr int kThreads = 256;
    const int64_t nThreads = nCounters / perThread;
    const dim3 grid((unsigned)((nThreads + kThreads - 1) / kThreads));
    if (perThread == 4)
        hipLaunchKernelGGL((ccb_k_cnt_batch<4, kCntUnroll>), grid, dim3(kThreads), 0, s, val, meta,
                           nCounters, nOps, finalOut, rel, nRelRows, err);
    else if (perThread == 2)
        hipLaunchKernelGGL((ccb_k_cnt_batch<2, kCntUnroll>), grid, dim3(kThreads), 0, s, val, meta,
                           nCounters, nOps, finalOut, rel, nRelRows, err);
    else
        hipLaunchKernelGGL((ccb_k_cnt_batch<1, kCntUnroll>), grid, dim3(kThreads), 0, s, val, meta,
                           nCounters, nOps, finalOut, rel, nRelRows, err);
    return hipGetLastError();
}

hipError_t launch_cnt_record(uint32_t* line, int32_t mode, uint32_t value, hipStream_t s)
{
    hipLaunchKernelGGL(ccb_k_cnt_record, dim3(1), dim3(kWave), 0, s, line, mode, value);
    return hipGetLastError();
}

hipError_t launch_cnt_wait(uint32_t* line, int32_t mode, uint32_t value, int32_t isClear,
                           uint64_t timeoutTicks, const uint32_t* cancel, uint32_t token,
                           hipStream_t s)
{
    hipLaunchKernelGGL(ccb_k_cnt_wait, dim3(1), dim3(kWave), 0, s, line, mode, value, isClear,
                       timeoutTicks, cancel, token);
    return hipGetLastError();
}

hipError_t launch_cnt_reset(uint32_t* line, hipStream_t s)
{
    hipLaunchKernelGGL(ccb_k_cnt_reset, dim3(1), dim3(kWave), 0, s, line);
    return hipGetLastError();
}

hipError_t launch_fill_zero(int32_t* p, int64_t nWords, hipStream_t s)
{
    const int64_t blocks = nWords / 256 + 1 < 1024 ? nWords / 256 + 1 : 1024;
    hipLaunchKernelGGL(ccb_k_fill_zero, dim3((unsigned)blocks), dim3(256), 0, s, p, nWords);
    return hipGetLastError();
}

hipError_t launch_atomic_chain(int32_t* line, uint64_t* ticks, int32_t iters, int32_t fenced,
                               int32_t kind, hipStream_t s)
{
    hipLaunchKernelGGL(ccb_k_atomic_chain, dim3(1), dim3(kWave), 0, s, line, ticks, iters, fenced,
                       kind, 0);
    return hipGetLastError();
}

hipError_t launch_atomic_contended(int32_t* line, uint64_t* ticks, int32_t iters, int32_t nGrid,
                                   hipStream_t s)
{
    int32_t zero = 0;
    void* args[] = {&line, &ticks, &iters, &zero};
    return hipLaunchCooperativeKernel(reinterpret_cast<const void*>(&ccb_k_atomic_contended),
                                      dim3(nGrid), dim3(kWave), args, 0, s);
}

hipError_t launch_notify_pingpong(int32_t* lines, uint64_t* ticks, int32_t iters, int32_t peer,
                                  uint32_t maxPoll, int32_t* err, hipStream_t s)
{
    // the two sides wait on each other: a cooperative launch guarantees that
    // all peer + 1 one-wave workgroups are resident together
    void* args[] = {&lines, &ticks, &iters, &peer, &maxPoll, &err};
    return hipLaunchCooperativeKernel(reinterpret_cast<const void*>(&ccb_k_notify_pingpong),
                                      dim3(peer + 1), dim3(kWave), args, 0, s);
}

hipError_t launch_hip_grid_sync(int32_t rounds, int32_t nGrid, int32_t threads, int32_t* done,
                                int numCUs, hipStream_t s)
{
    // grid sync waits without a bound, so the grid must be shown resident
    // here, not only by the runtime's own check.  The kernel uses few SGPRs
    // (21), where the occupancy API's count is exact.
    const void* fn = reinterpret_cast<const void*>(&ccb_k_hip_grid_sync);
    int perCU = 0;
    const hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&perCU, fn, threads, 0);
    if (e != hipSuccess) return e;
    if ((int64_t)perCU * numCUs < nGrid) return hipErrorCooperativeLaunchTooLarge;
    void* args[] = {&rounds, &done};
    return hipLaunchCooperativeKernel(fn, dim3(nGrid), dim3(threads), args, 0, s);
}

hipError_t launch_fence_placement(int32_t* scratch, int32_t* stale, int32_t rounds, int32_t nGrid,
                                  int32_t threads, int32_t variant, uint32_t maxPoll, hipStream_t s)
{
    const void* fns[] = {
        reinterpret_cast<const void*>(&ccb_k_fence_placement<0>),
        reinterpret_cast<const void*>(&ccb_k_fence_placement<1>),
        reinterpret_cast<const void*>(&ccb_k_fence_placement<2>),
        reinterpret_cast<const void*>(&ccb_k_fence_placement<3>),
        reinterpret_cast<const void*>(&ccb_k_fence_placement<4>),
        reinterpret_cast<const void*>(&ccb_k_fence_placement<5>)};
    void* args[] = {&scratch, &stale, &rounds, &maxPoll};
    return hipLaunchCooperativeKernel(fns[variant], dim3(nGrid), dim3(threads), args, 0, s);
}

hipError_t launch_copy(int4* dst, const int4* src, int64_t n16, int nBlocks, hipStream_t s)
{
    hipLaunchKernelGGL(ccb_k_copy, dim3(nBlocks), dim3(256), 0, s, dst, src, n16);
    return hipGetLastError();
}

}  // namespace ccb
