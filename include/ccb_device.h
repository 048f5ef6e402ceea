/*
 * ccb_device.h -- device-side soft epoch barrier for HIP kernels on gfx950.
 *
 * The in-kernel counterpart of the Soft SYNCALL of "PTO-ISA 跨核同步屏障
 * SYNCALL 实战指南" (PTO-ISA SYNCALL guide), §5.2: every participant adds one
 * to a counter in global memory, takes back the old value, derives from it
 * the count at which its round is complete, and polls until the counter gets
 * there.  The round number is implicit in the count (§5.2), so no per-core
 * state is kept between barriers.
 *
 * Participants are workgroups whose thread count is a multiple of 64.  Every
 * thread of a participating workgroup calls the barrier (uniform control
 * flow); wave 0 does the arrival and the poll, and the workgroup's own
 * barrier spreads the result.
 *
 * Striped counters.  On gfx950 a device-scope atomic on one address costs
 * about 11 ns of that address's time, so N arrivals on a single counter take
 * N * 11 ns one after another (2.9 us at 256 workgroups).  The counter is
 * therefore split into K stripes, each an int32 alone on its own 128-byte
 * line: member m arrives on stripe m mod K, whose participant count is
 * n_s = ceil((N - s) / K).  Each stripe is an epoch counter of its own:
 * from the old value its member derives the round e = before / n_s + 1 (the
 * pages' target rule, target = e * n_s, applied per stripe), and the round is
 * complete once every stripe l has reached e * n_l.  Wave 0 checks that with
 * one gather load -- lane l reads stripe l.  With K = 1 this is exactly the
 * pages' single-counter algorithm.  Because no member can arrive for round
 * e + 1 before every member has arrived for round e, a stripe at or above
 * e * n_l means all its members arrived for round e, and ">=" (not "==") is
 * the correct poll condition (fast members may already be in round e + 1).
 *
 * Rules inherited from the pages:
 *   - Every stripe must be zero (or a multiple of its n_s) before first use
 *     ([SYNCALL] §4.1); each sits alone on its line.
 *   - usedCores == 0 means every launched workgroup; an explicit count means
 *     workgroups that are not members must never call ([SYNCALL] §4.2, §7.2).
 *   - Every member enters the same barriers in the same order the same
 *     number of times ([SYNCALL] §6.2).
 *   - Every member must be resident at once; launch persistent grids
 *     cooperatively ([SYNCALL] §6.3).  On MI355X the occupancy API (and
 *     with it the cooperative launch check) counts a kernel's own SGPRs
 *     only, while each wave also holds 16 trap-handler SGPRs out of 800 per
 *     SIMD: a kernel whose SGPR allocation (16-register granules) is 96
 *     fits 7 waves per SIMD, not the 8 the API reports, and a grid sized by
 *     the API then waits for workgroups that never start until the poll
 *     bound reports DEADLOCK.  Size grids by min(API, 800 / (SGPRs + 16))
 *     waves per SIMD, or keep the kernel at 80 SGPRs or fewer.  A workgroup
 *     of 5-7, 9-11 or 13-15 waves does not spread its waves evenly over the
 *     4 SIMDs: count ceil(waves / 4) of them on one SIMD.
 *
 * Visibility -- two strengths; the full one in two placements (CCB_VIS_FULL,
 * CCB_VIS_XCD):
 *   CCB_VIS_FULL   agent-scope release fence before the arrival and acquire
 *                  fence after the poll: plain global stores made before the
 *                  barrier are visible to plain loads after it on every XCD.
 *                  On gfx950 each fence is an L2 write-back / invalidate that
 *                  the device serialises (about 7 ns each), so this costs
 *                  about N * 14 ns per barrier.
 *   CCB_VIS_ORDER  the pages' own contract ([SYNCALL] §6.1: the barrier
 *                  counts arrivals, cache maintenance is the caller's): every
 *                  thread's earlier memory operations have completed before
 *                  the arrival, and later ones start after the release, but
 *                  no cache is written back or invalidated.  Data that one
 *                  workgroup writes before the barrier and another reads
 *                  after it must go through ccb_store_coherent /
 *                  ccb_load_coherent (device-coherent accesses).
 *   CCB_VIS_XCD    the guarantee of CCB_VIS_FULL with one L2 write-back per
 *                  XCD instead of one per workgroup.  Every thread's stores
 *                  complete before the arrival (so they sit in the L2 of the
 *                  workgroup's XCD: the vector L1 is write-through), the
 *                  round completes as under CCB_VIS_ORDER, then one leader
 *                  workgroup per XCD writes that L2 back and raises the
 *                  XCD's flag, and every member waits for the flags of all
 *                  XCDs with members before its agent-scope acquire (the
 *                  acquire is the only invalidate that reaches a CU's L1,
 *                  so it stays per workgroup).  Saves N - 8 write-backs per
 *                  barrier for the price of a second notification.  Needs
 *                  a ccb_xcd_team per workspace, kept by the caller between
 *                  barriers, and a workspace zeroed before the launch.
 *
 * Failure.  The poll is bounded ([SYNCALL] §5.2 bounds it at 10^6 polls and
 * asserts).  A GPU trap would kill the context, so instead the member that
 * runs out of polls stores CCB_ERR_DEADLOCK into an error word and the call
 * returns CCB_ERR_DEADLOCK; members still polling see the error word and
 * return the same.  The caller must then leave its barrier loop.
 */
#ifndef CCB_DEVICE_H
#define CCB_DEVICE_H

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ccb.h"

/* s_sleep argument between polls (units of 64 clocks); 0 = no sleep. */
#ifndef CCB_POLL_SLEEP
#define CCB_POLL_SLEEP 1
#endif

/* How often (in polls) a waiting wave also looks at the error word. */
#ifndef CCB_ERR_CHECK_EVERY
#define CCB_ERR_CHECK_EVERY 64u
#endif

#define CCB_LINE_WORDS (CCB_LINE_BYTES / 4)

enum ccbVisibility { CCB_VIS_FULL = 0, CCB_VIS_ORDER = 1, CCB_VIS_XCD = 2 };

/* Words of a barrier's workspace used by CCB_VIS_XCD (reserved bytes of
 * stripe lines 1 and 2): the members registered on XCD x, and the last
 * round whose stores XCD x's leader has written back. */
#define CCB_XCD_COUNT_WORD (1 * CCB_LINE_WORDS + 8)
#define CCB_XCD_FLAG_WORD (2 * CCB_LINE_WORDS + 8)
#define CCB_XCDS 8

/* What a member of a CCB_VIS_XCD barrier knows about its XCD.  Zero it
 * (ccb_xcd_team t = {}) before the first barrier on a workspace and pass the
 * same object to every later barrier on that workspace: the first barrier
 * registers the workgroup on its XCD (the first to register is the XCD's
 * leader) and learns which XCDs have members.  Wave 0 keeps the live copy;
 * the other waves' copies are not used. */
struct ccb_xcd_team {
    int32_t joined;  /* 0 until the first barrier has completed */
    int32_t leader;  /* this workgroup writes its XCD's L2 back */
    uint32_t xcc;    /* this workgroup's XCD (the XCC_ID register) */
    uint32_t xcds;   /* bit x: XCD x has members */
};

/* Device-coherent accesses for data shared across a CCB_VIS_ORDER barrier. */
__device__ __forceinline__ void ccb_store_coherent(int32_t* p, int32_t v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void ccb_store_coherent(uint32_t* p, uint32_t v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int32_t ccb_load_coherent(const int32_t* p)
{
    return __hip_atomic_load(const_cast<int32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ccb_load_coherent(const uint32_t* p)
{
    return __hip_atomic_load(const_cast<uint32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

/* Wait until every memory operation this thread issued has completed. */
__device__ __forceinline__ void ccb_wait_memory() { __builtin_amdgcn_s_waitcnt(0); }

/* Agent-scope release fence whose L2 write-back has completed before the
 * next memory access is issued.  LLVM's AMDGPU memory model implements the
 * fence as `buffer_wbl2 sc1` then `s_waitcnt vmcnt(0)`, but the compiler
 * drops that wait wherever it tracks no other vector memory access in
 * flight (it does not count the write-back); the explicit wait keeps it. */
__device__ __forceinline__ void ccb_fence_release_agent()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    ccb_wait_memory();
}

/* No work between the arrival and the poll. */
struct ccb_no_overlap {
    __device__ __forceinline__ void operator()() const {}
};

/* Instrumentation points of ccb_await (all lanes of wave 0 call them):
 * reply() once the arrival's reply is back, before the first poll load;
 * released() once the poll has seen the round complete (or given up),
 * before the acquire fence.  The default does nothing and costs nothing. */
struct ccb_no_hook {
    __device__ __forceinline__ void reply() const {}
    __device__ __forceinline__ void released() const {}
};

/* Split-phase form of the barrier, for callers that order their own
 * workgroup around it (one workgroup barrier per round where back-to-back
 * rounds leave nothing to do between them).
 *
 * ccb_arrive: called by ONE lane of wave 0 (linear thread 0) once every
 * access of the workgroup that the round must publish is complete and
 * ordered before it (for CCB_VIS_ORDER: each thread waited for its own
 * accesses, then a workgroup barrier).  Issues the arrival -- the pages'
 * atomic add of one that returns the old value -- on stripe member mod K
 * and returns that old value; nothing waits for it here, so the caller may
 * issue more memory operations while the arrival is in flight.
 *
 * ccb_await: called by every lane of wave 0 with lane 0's `before`.  Derives
 * the round from it, epoch = before / n_s + 1 with n_s the stripe's member
 * count, and polls until every stripe l in use holds at least epoch * n_l
 * arrivals (for K = 1: the counter reaches (before / n + 1) * n, the
 * pages' target); the first poll goes out only once `before` is back (a
 * poll issued behind the wave's own arrival doubles the barrier's cost),
 * and the arrival's own stripe also counts as complete once before + 1
 * reaches its target.  At most maxPoll polls; past that it stores
 * CCB_ERR_DEADLOCK in the error word and returns it.  Every 64th poll it
 * also reads the error word and returns its value when another member has
 * failed.  For CCB_VIS_FULL it ends with an agent-scope acquire fence.  The
 * caller then releases the rest of its workgroup (a workgroup barrier).
 *
 * The counters are int32 ([SYNCALL] §4.1).  A round whose release count
 * epoch * n_l would pass INT32_MAX on some stripe can never complete, and
 * an old value below zero means a stripe has already wrapped: either way
 * the member stores CCB_ERR_INVALID_VALUE in the error word and returns it
 * without polling, and the others leave when they next read the error
 * word.  Re-zero the workspace before a stripe gets near 2^31 arrivals. */
/* Counter layouts, the template argument K of the functions below:
 *   K = 1 .. 64      K stripes (K = 1: the pages' single counter);
 *   K = ccb_tree(G)  a two-level arrival tree of G group counters (G = 1 .. 32)
 *                    under one top counter: member m arrives on group
 *                    m mod G with the pages' epoch rule for the group's
 *                    n_g = ceil((N - g) / G) members; the arrival whose reply
 *                    completes its group's round adds one to the top counter,
 *                    whose participants are the min(N, G) groups, and every
 *                    member polls the top counter for epoch * min(N, G).
 *                    Group g sits at byte 0 of line g, the top counter at
 *                    byte 64 of line CCB_STRIPES - 1 (so the sum of the lines'
 *                    first words is still the number of member arrivals).
 *                    The same shape as a core -> cluster barrier bus, with
 *                    counters in memory instead of wires. */
__host__ __device__ constexpr int ccb_tree(int groups) { return -groups; }

#define CCB_TREE_TOP_WORD ((CCB_STRIPES - 1) * CCB_LINE_WORDS + CCB_LINE_WORDS / 2)

template <int K, ccbVisibility kVis>
__device__ __forceinline__ int32_t ccb_arrive(int32_t* ctr, int32_t member)
{
    static_assert((K >= 1 && K <= 64) || (K <= -1 && K >= -32),
                  "stripes are polled by one wave; tree groups sit below the top line");
    static_assert(kVis != CCB_VIS_XCD, "CCB_VIS_XCD takes a ccb_xcd_team");
    constexpr int kLines = K > 0 ? K : -K;
    // release: the workgroup's earlier global stores become visible at agent
    // scope before the arrival can be observed
    if (kVis == CCB_VIS_FULL) ccb_fence_release_agent();
    return __hip_atomic_fetch_add(ctr + (member % kLines) * CCB_LINE_WORDS, 1, __ATOMIC_RELAXED,
                                  __HIP_MEMORY_SCOPE_AGENT);
}

/* ccb_arrive for any visibility, with the XCD state of CCB_VIS_XCD (ignored
 * otherwise).  Before its first arrival on the workspace the member
 * registers on its XCD and waits for that to land, so that a round seen
 * complete also has every member registered. */
template <int K, ccbVisibility kVis>
__device__ __forceinline__ int32_t ccb_arrive(int32_t* ctr, int32_t member, ccb_xcd_team& team)
{
    if constexpr (kVis == CCB_VIS_XCD) {
        if (!team.joined) {
            team.xcc = __builtin_amdgcn_s_getreg((31 << 11) | 20) & (CCB_XCDS - 1);  // XCC_ID
            team.leader = __hip_atomic_fetch_add(ctr + CCB_XCD_COUNT_WORD + team.xcc, 1,
                                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0;
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
            ccb_wait_memory();
        }
    }
    return ccb_arrive<K, kVis == CCB_VIS_FULL ? CCB_VIS_FULL : CCB_VIS_ORDER>(ctr, member);
}

/* The poll of a two-level tree (K = ccb_tree(G)); see ccb_await. */
template <int G, ccbVisibility kVis, class Hook>
__device__ __forceinline__ int32_t ccb_await_tree(const int32_t* ctr, int32_t n, int32_t member,
                                                  int32_t before, uint32_t maxPoll, int32_t* err,
                                                  Hook hook)
{
    const int lane = (int)__lane_id();
    int32_t* const top = const_cast<int32_t*>(ctr) + CCB_TREE_TOP_WORD;
    const int32_t b = __shfl(before, 0, 64);
    __builtin_amdgcn_sched_barrier(0x44F);
    hook.reply();
    const int32_t g = member % G;
    const int32_t ng = (n - g + G - 1) / G;  // members of this group
    const int32_t gu = n < G ? n : G;        // groups in use: the top counter's members
    const int32_t q = b / ng;
    // group 0 is the largest; both its count and the top's must stay in int32
    if (b < 0 || q >= INT32_MAX / ((n + G - 1) / G) || q >= INT32_MAX / gu) {
        if (lane == 0)
            __hip_atomic_store(err, (int32_t)CCB_ERR_INVALID_VALUE, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        hook.released();
        return CCB_ERR_INVALID_VALUE;
    }
    const int32_t epoch = q + 1;
    if (b + 1 == epoch * ng) {
        // this arrival completed its group's round: the group arrives on top.
        // With full visibility the group's released stores must reach the
        // pollers of the top counter through this member: acquire from the
        // group counter, release to the top.
        if (kVis == CCB_VIS_FULL) {
            ccb_fence_release_agent();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        }
        if (lane == 0)
            __hip_atomic_fetch_add(top, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    const int32_t need = epoch * gu;
    int32_t rc = CCB_OK;
    uint32_t polls = 0;
    for (;;) {
        const int32_t v = __hip_atomic_load(top, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (v >= need) break;
        if (++polls >= maxPoll) {
            if (lane == 0)
                __hip_atomic_store(err, (int32_t)CCB_ERR_DEADLOCK, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
            rc = CCB_ERR_DEADLOCK;
            break;
        }
        if ((polls % CCB_ERR_CHECK_EVERY) == 0) {
            const int32_t e = __hip_atomic_load(err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (e != CCB_OK) {
                rc = e;
                break;
            }
        }
        if (CCB_POLL_SLEEP > 0) __builtin_amdgcn_s_sleep(CCB_POLL_SLEEP);
    }
    hook.released();
    if (kVis == CCB_VIS_FULL) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    return rc;
}

template <int K, ccbVisibility kVis, class Hook = ccb_no_hook>
__device__ __forceinline__ int32_t ccb_await(const int32_t* ctr, int32_t n, int32_t member,
                                             int32_t before, uint32_t maxPoll, int32_t* err,
                                             Hook hook = Hook())
{
    static_assert(kVis != CCB_VIS_XCD, "CCB_VIS_XCD takes a ccb_xcd_team");
    if constexpr (K < 0) {
        return ccb_await_tree<-K, kVis>(ctr, n, member, before, maxPoll, err, hook);
    } else {
        const int lane = (int)__lane_id();
        const int32_t ks = n < K ? n : K;  // stripes in use
        const int32_t s = member % K;
        int32_t* mine = const_cast<int32_t*>(ctr) + (lane < ks ? lane : 0) * CCB_LINE_WORDS;
        // The first poll goes out only after the arrival's reply is back: a poll
        // load issued while the wave's own arrival is still in flight makes the
        // barrier about twice as slow on gfx950, whichever stripe it reads
        // (measured at 256 workgroups: 1.75-1.85 us against 0.94 us).  The shuffle
        // waits for the reply; the scheduling barrier keeps vector memory reads
        // and the shuffle on their sides of it (mask 0x44F: ALU work and vector
        // memory writes may still move across).
        // The reply itself says whether this arrival completed its own stripe,
        // and counters only grow, so any value read that meets the target proves
        // that stripe complete.
        const int32_t b = __shfl(before, 0, 64);
        __builtin_amdgcn_sched_barrier(0x44F);
        hook.reply();
        const int32_t v0 = __hip_atomic_load(mine, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        // The release count of stripe l is epoch * n_l; stripe 0 has the most
        // members, so the round fits in int32 exactly when
        // (before / n_s + 1) * n_0 <= INT32_MAX, i.e. before / n_s < INT32_MAX / n_0.
        const int32_t q = b / ((n - s + K - 1) / K);
        const int32_t epoch = q + 1;
        if (b < 0 || q >= INT32_MAX / ((n + K - 1) / K)) {
            if (lane == 0)
                __hip_atomic_store(err, (int32_t)CCB_ERR_INVALID_VALUE, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
            hook.released();
            return CCB_ERR_INVALID_VALUE;
        }
        // stripe `lane` is complete for this round at epoch * n_lane arrivals;
        // lanes past the stripes in use re-read stripe 0 and always agree
        const int32_t need = lane < ks ? epoch * ((n - lane + K - 1) / K) : INT32_MIN;
        int32_t rc = CCB_OK;
        uint32_t polls = 0;
        // A stripe seen complete stays complete, so later polls read only the
        // unfinished ones: lanes that are done re-read the first unfinished
        // stripe, which adds no line to the gather.
        int32_t* const base = const_cast<int32_t*>(ctr);
        bool done = v0 >= need || (lane == s && b + 1 >= need);
        if (!__all(done)) {
            for (;;) {
                const uint64_t pending = __ballot(!done);
                int32_t* const addr = done ? base + __builtin_ctzll(pending) * CCB_LINE_WORDS : mine;
                const int32_t v = __hip_atomic_load(addr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                done = done || v >= need;
                if (__all(done)) break;
                if (++polls >= maxPoll) {
                    if (lane == 0)
                        __hip_atomic_store(err, (int32_t)CCB_ERR_DEADLOCK, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
                    rc = CCB_ERR_DEADLOCK;
                    break;
                }
                if ((polls % CCB_ERR_CHECK_EVERY) == 0) {
                    const int32_t e = __hip_atomic_load(err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    if (e != CCB_OK) {
                        rc = e;
                        break;
                    }
                }
                if (CCB_POLL_SLEEP > 0) __builtin_amdgcn_s_sleep(CCB_POLL_SLEEP);
            }
        }
        hook.released();
        // acquire: loads after the barrier see every member's released stores
        if (kVis == CCB_VIS_FULL) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        return rc;
    }
}

/* ccb_await for any visibility, with the XCD state of CCB_VIS_XCD (ignored
 * otherwise).  Under CCB_VIS_XCD, once the round is complete (as under
 * CCB_VIS_ORDER; hook.released() marks that point): on the first barrier
 * the XCDs with members are read from the registrations; the XCD's leader
 * writes its L2 back (agent-scope release fence: every member of the XCD
 * has arrived, so all their stores are in that L2) and stores the round in
 * its XCD's flag; every member then polls the flags of the XCDs with
 * members until each holds the round (bounded by maxPoll like the first
 * poll, and watching the error word) and ends with the agent-scope acquire
 * fence. */
template <int K, ccbVisibility kVis, class Hook = ccb_no_hook>
__device__ __forceinline__ int32_t ccb_await(const int32_t* ctr, int32_t n, int32_t member,
                                             int32_t before, uint32_t maxPoll, int32_t* err,
                                             Hook hook, ccb_xcd_team& team)
{
    if constexpr (kVis != CCB_VIS_XCD) {
        return ccb_await<K, kVis>(ctr, n, member, before, maxPoll, err, hook);
    } else {
        int32_t rc = ccb_await<K, CCB_VIS_ORDER>(ctr, n, member, before, maxPoll, err, hook);
        if (rc != CCB_OK) return rc;
        const int lane = (int)__lane_id();
        constexpr int kLines = K > 0 ? K : -K;
        const int32_t b = __shfl(before, 0, 64);
        const int32_t s = member % kLines;
        const int32_t epoch = b / ((n - s + kLines - 1) / kLines) + 1;  // checked by the poll above
        int32_t* const base = const_cast<int32_t*>(ctr);
        if (!team.joined) {
            // every member registered before it arrived and the round is
            // complete, so every registration is in
            team.xcc = __shfl(team.xcc, 0, 64);
            team.leader = __shfl(team.leader, 0, 64);
            const int32_t c =
                lane < CCB_XCDS ? __hip_atomic_load(base + CCB_XCD_COUNT_WORD + lane, __ATOMIC_RELAXED,
                                                    __HIP_MEMORY_SCOPE_AGENT)
                                : 0;
            team.xcds = (uint32_t)__ballot(c > 0) & ((1u << CCB_XCDS) - 1);
            team.joined = 1;
        }
        int32_t* const flags = base + CCB_XCD_FLAG_WORD;
        if (team.leader) {
            ccb_fence_release_agent();
            if (lane == 0)
                __hip_atomic_store(flags + team.xcc, epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        const bool watch = lane < CCB_XCDS && ((team.xcds >> lane) & 1u) != 0;
        int32_t* const addr = flags + (watch ? lane : (int)team.xcc);
        uint32_t polls = 0;
        for (;;) {
            const int32_t v = __hip_atomic_load(addr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (__all(!watch || v >= epoch)) break;
            if (++polls >= maxPoll) {
                if (lane == 0)
                    __hip_atomic_store(err, (int32_t)CCB_ERR_DEADLOCK, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
                rc = CCB_ERR_DEADLOCK;
                break;
            }
            if ((polls % CCB_ERR_CHECK_EVERY) == 0) {
                const int32_t e = __hip_atomic_load(err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                if (e != CCB_OK) {
                    rc = e;
                    break;
                }
            }
            if (CCB_POLL_SLEEP > 0) __builtin_amdgcn_s_sleep(CCB_POLL_SLEEP);
        }
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        return rc;
    }
}

/* The barrier proper (both phases with the workgroup barriers around them).
 *   ctr      K stripe lines (stripe s: int32 at ctr[s * CCB_LINE_WORDS])
 *   n        participant count (> 0)
 *   member   this workgroup's index among the participants, 0..n-1
 *   maxPoll  poll bound (> 0)
 *   err      error word (on a line of its own)
 *   overlap  run by the arriving lane right after it has issued its arrival,
 *            while the arrival is in flight (work that is not shared across
 *            this barrier, e.g. a private output store)
 * kPreWait (CCB_VIS_ORDER only): every thread first waits for all of its own
 * memory operations.  A caller that has already waited for the stores it
 * shares across the barrier may turn it off.
 * Every thread of the workgroup calls it.  Returns CCB_OK,
 * CCB_ERR_DEADLOCK or CCB_ERR_INVALID_VALUE (the same value in every
 * thread). */
template <int K, ccbVisibility kVis, bool kPreWait = true, class Overlap = ccb_no_overlap>
__device__ __forceinline__ int32_t ccb_barrier(int32_t* ctr, int32_t n, int32_t member,
                                               uint32_t maxPoll, int32_t* err, ccb_xcd_team& team,
                                               Overlap overlap = Overlap())
{
    __shared__ int32_t ccb_result;
    // this thread's accesses are done (CCB_VIS_XCD: its stores are in the L2)
    if ((kVis == CCB_VIS_ORDER && kPreWait) || kVis == CCB_VIS_XCD) ccb_wait_memory();
    __syncthreads();
    const uint32_t tid = threadIdx.x + blockDim.x * (threadIdx.y + blockDim.y * threadIdx.z);
    if (tid < 64) {  // wave 0
        int32_t before = 0;
        if (tid == 0) {
            before = ccb_arrive<K, kVis>(ctr, member, team);
            overlap();
        }
        const int32_t rc = ccb_await<K, kVis>(ctr, n, member, before, maxPoll, err, ccb_no_hook(), team);
        if (tid == 0) ccb_result = rc;
    }
    __syncthreads();
    return ccb_result;
}

/* The same for CCB_VIS_FULL and CCB_VIS_ORDER, which keep no state. */
template <int K, ccbVisibility kVis, bool kPreWait = true, class Overlap = ccb_no_overlap>
__device__ __forceinline__ int32_t ccb_barrier(int32_t* ctr, int32_t n, int32_t member,
                                               uint32_t maxPoll, int32_t* err,
                                               Overlap overlap = Overlap())
{
    static_assert(kVis != CCB_VIS_XCD, "CCB_VIS_XCD takes a ccb_xcd_team");
    ccb_xcd_team unused = {};
    return ccb_barrier<K, kVis, kPreWait, Overlap>(ctr, n, member, maxPoll, err, unused, overlap);
}

/* Linear index of this workgroup in the grid. */
__device__ __forceinline__ int32_t ccb_block_linear()
{
    return (int32_t)(blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z));
}

/* [SYNCALL] §3's Soft overload: ws is a workspace of one barrier
 * (CCB_STRIPES stripe lines, then the error line), usedCores as in §4.2
 * (members are the workgroups with linear index < usedCores).  Full
 * visibility. */
__device__ __forceinline__ int32_t ccb_syncall_soft(int32_t* ws, int32_t usedCores)
{
    const int32_t n = usedCores != 0 ? usedCores : (int32_t)(gridDim.x * gridDim.y * gridDim.z);
    return ccb_barrier<CCB_STRIPES, CCB_VIS_FULL>(ws, n, ccb_block_linear(), CCB_SOFT_MAX_POLL,
                                                  ws + CCB_STRIPES * CCB_LINE_WORDS);
}

/* ccb_syncall_soft with a caller-chosen poll bound instead of
 * CCB_SOFT_MAX_POLL (a test hook: a small bound turns a deliberately
 * broken round into a prompt CCB_ERR_DEADLOCK). */
__device__ __forceinline__ int32_t ccb_syncall_soft_bounded(int32_t* ws, int32_t usedCores,
                                                            uint32_t maxPoll)
{
    const int32_t n = usedCores != 0 ? usedCores : (int32_t)(gridDim.x * gridDim.y * gridDim.z);
    return ccb_barrier<CCB_STRIPES, CCB_VIS_FULL>(ws, n, ccb_block_linear(), maxPoll,
                                                  ws + CCB_STRIPES * CCB_LINE_WORDS);
}

/* The same barrier with the pages' arrival-only contract (CCB_VIS_ORDER). */
__device__ __forceinline__ int32_t ccb_syncall_soft_ordered(int32_t* ws, int32_t usedCores)
{
    const int32_t n = usedCores != 0 ? usedCores : (int32_t)(gridDim.x * gridDim.y * gridDim.z);
    return ccb_barrier<CCB_STRIPES, CCB_VIS_ORDER>(ws, n, ccb_block_linear(), CCB_SOFT_MAX_POLL,
                                                   ws + CCB_STRIPES * CCB_LINE_WORDS);
}

/* [SYNCALL] §4.2's mixed-role participant count, for workgroups in role
 * groups: one leading workgroup with `ratio` companions (the analog of one
 * cube core with its `ratio` vector cores).  The participants are the first
 * groups * (1 + ratio) workgroups in linear order (group g is workgroups
 * g * (1 + ratio) .. g * (1 + ratio) + ratio, the leader first); groups == 0
 * means the whole grid.  ratio >= 0 (the pages default it to 1). */
__host__ __device__ __forceinline__ int32_t ccb_mix_participants(int32_t groups, int32_t ratio,
                                                                 int32_t gridSize)
{
    return groups != 0 ? groups * (1 + ratio) : gridSize;
}

/* ccb_syncall_soft over a mixed-role group set (see ccb_mix_participants):
 * every participant calls it, non-participants never do. */
__device__ __forceinline__ int32_t ccb_syncall_soft_mix(int32_t* ws, int32_t groups, int32_t ratio)
{
    const int32_t n =
        ccb_mix_participants(groups, ratio, (int32_t)(gridDim.x * gridDim.y * gridDim.z));
    return ccb_barrier<CCB_STRIPES, CCB_VIS_FULL>(ws, n, ccb_block_linear(), CCB_SOFT_MAX_POLL,
                                                  ws + CCB_STRIPES * CCB_LINE_WORDS);
}

/* The two-level arrival tree (CCB_TREE_GROUPS group counters under one top
 * counter, see ccb_tree), full visibility; same workspace layout. */
__device__ __forceinline__ int32_t ccb_syncall_soft_tree(int32_t* ws, int32_t usedCores)
{
    const int32_t n = usedCores != 0 ? usedCores : (int32_t)(gridDim.x * gridDim.y * gridDim.z);
    return ccb_barrier<ccb_tree(CCB_TREE_GROUPS), CCB_VIS_FULL>(
        ws, n, ccb_block_linear(), CCB_SOFT_MAX_POLL, ws + CCB_STRIPES * CCB_LINE_WORDS);
}

/* ccb_syncall_soft with one L2 write-back per XCD (CCB_VIS_XCD): the same
 * visibility as ccb_syncall_soft.  `team` is this workgroup's ccb_xcd_team
 * for `ws`, zeroed before the first call and passed to every call on `ws`;
 * the workspace must be zeroed before the launch. */
__device__ __forceinline__ int32_t ccb_syncall_soft_xcd(int32_t* ws, int32_t usedCores,
                                                        ccb_xcd_team& team)
{
    const int32_t n = usedCores != 0 ? usedCores : (int32_t)(gridDim.x * gridDim.y * gridDim.z);
    return ccb_barrier<CCB_STRIPES, CCB_VIS_XCD>(ws, n, ccb_block_linear(), CCB_SOFT_MAX_POLL,
                                                 ws + CCB_STRIPES * CCB_LINE_WORDS, team);
}

/* The pages' single-counter barrier exactly (one counter line, full
 * visibility); same workspace layout, only stripe 0 is used. */
__device__ __forceinline__ int32_t ccb_syncall_soft_flat(int32_t* ws, int32_t usedCores)
{
    const int32_t n = usedCores != 0 ? usedCores : (int32_t)(gridDim.x * gridDim.y * gridDim.z);
    return ccb_barrier<1, CCB_VIS_FULL>(ws, n, ccb_block_linear(), CCB_SOFT_MAX_POLL,
                                        ws + CCB_STRIPES * CCB_LINE_WORDS);
}

#endif /* CCB_DEVICE_H */
