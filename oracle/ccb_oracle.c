/*
 * ccb_oracle.c -- plain, sequential CPU oracle for the soft epoch barrier and
 * the CntNotify counter semantics.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the reference the GPU path is
 * checked against.  Only the tests, the smoke check and the benchmark's CPU
 * baseline leg may load it.  It shares no code, header, table or constant
 * with the HIP library: every definition below is restated from the pages.
 *
 * Sources (web pages; cited by title and section):
 *   [SYNCALL]   "PTO-ISA 跨核同步屏障 SYNCALL 实战指南" (PTO-ISA cross-core barrier
 *               SYNCALL guide): §2 semantics, §4.1 workspace, §4.2 usedCores,
 *               §5.2 Soft mode epoch barrier, §6.1-§6.3 usage rules,
 *               §7.2 partial-participation example, §8 tests.
 *   [CNTNOTIFY] "CANN Runtime CntNotify（计数型通知）管理接口详解" (CANN Runtime
 *               CntNotify interfaces): §3.1 record modes, §3.2 wait modes,
 *               §3.3 info structs, §5 usage example, §7 advice.
 *
 * Everything is integer arithmetic, so the oracle is exact; no tolerance is
 * involved anywhere.  All loops run in the order the pages describe; nothing
 * is blocked, fused or reordered.
 *
 * Parity status of each function (what pins it) is recorded in the header of
 * oracle/__init__.py.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Status codes the oracle reports (mirrors the meaning of the boundary's
 * codes; the values are re-declared here on purpose, the oracle includes no
 * header of the GPU library). */
enum {
    ORC_OK = 0,
    ORC_INVALID_VALUE = 1,
    ORC_DEADLOCK = 6,
};

/* ------------------------------------------------------------------------ */
/* Witness hash.                                                             */
/*                                                                           */
/* The pages fix no witness function; the workload only needs a value that  */
/* depends on (seed, round, workgroup).  We use SplitMix64 as published by   */
/* Steele, Lea and Flood ("Fast splittable pseudorandom number generators",  */
/* OOPSLA 2014): the generator's state advances by the golden gamma          */
/* 0x9E3779B97F4A7C15 and each output is the state passed through the        */
/* variant-13 finaliser (xor-shift 30, multiply 0xBF58476D1CE4E5B9,          */
/* xor-shift 27, multiply 0x94D049BB133111EB, xor-shift 31).                 */
/* hash(seed, r, w) is output number key+1 of a generator seeded with `seed`,*/
/* where key = r * 2^32 + w; the high 32 bits are kept.                      */
/* ------------------------------------------------------------------------ */
static uint64_t splitmix64_output(uint64_t state_after_advance)
{
    uint64_t z = state_after_advance;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

uint64_t ccbo_splitmix64_nth(uint64_t seed, uint64_t n)
{
    /* n-th output (n >= 1) of SplitMix64 seeded with `seed`: the state has
     * advanced n times by the gamma. */
    uint64_t state = seed;
    state += 0x9E3779B97F4A7C15ULL * n;
    return splitmix64_output(state);
}

uint32_t ccbo_witness_hash(uint64_t seed, uint32_t round, uint32_t wg)
{
    uint64_t key = ((uint64_t)round << 32) | (uint64_t)wg;
    return (uint32_t)(ccbo_splitmix64_nth(seed, key + 1) >> 32);
}

/* ------------------------------------------------------------------------ */
/* Epoch target.  [SYNCALL] §5.2: each arriving participant adds one to the  */
/* shared counter and gets the old value back; the release point of its     */
/* round is the count reached once the last participant of that round has   */
/* arrived, i.e. the next multiple of the participant count above `before`. */
/* (The extracted formula lost its '=' and '+'; the prose fixes the reading */
/* target = (before / N + 1) * N with C's truncating division, before >= 0.)*/
/* ------------------------------------------------------------------------ */
int32_t ccbo_epoch_target(int32_t before, int32_t n)
{
    return (before / n + 1) * n;
}

/* The same target with the counter's range checked.  [SYNCALL] §4.1 types  */
/* the counter int32: a round whose target lies above INT32_MAX can never   */
/* be reached, and an old value below zero means the counter has wrapped.   */
/* Either is reported as ORC_INVALID_VALUE (pages silent on the limit).     */
int ccbo_epoch_target_checked(int32_t before, int32_t n, int32_t* target)
{
    if (n <= 0 || before < 0) return ORC_INVALID_VALUE;
    int64_t t = ((int64_t)before / n + 1) * (int64_t)n;
    if (t > INT32_MAX) return ORC_INVALID_VALUE;
    *target = (int32_t)t;
    return ORC_OK;
}

/* Participant count.  [SYNCALL] §4.2: usedCores == 0 means every core of   */
/* the launch; an explicit count may be smaller than the launch.  Negative  */
/* values and counts above the launch are rejected (pages silent).          */
int32_t ccbo_participants(int32_t usedCores, int32_t nLaunched)
{
    if (usedCores < 0 || usedCores > nLaunched || nLaunched <= 0) return -1;
    return usedCores != 0 ? usedCores : nLaunched;
}

/* Mixed-role participant count.  [SYNCALL] §4.2: in Mix mode the count is  */
/* the number of cube blocks times (1 + the vector-core ratio).  Here a      */
/* "block" is a group of one leading workgroup and `ratio` companions;       */
/* groups == 0 takes the whole launch.  Rejected (pages silent): negative    */
/* groups or ratio, and a count above the launch.                            */
int32_t ccbo_mix_participants(int32_t groups, int32_t ratio, int32_t nLaunched)
{
    if (groups < 0 || ratio < 0 || nLaunched <= 0) return -1;
    if (groups == 0) return nLaunched;
    if ((int64_t)groups * (1 + ratio) > nLaunched) return -1;
    return groups * (1 + ratio);
}

/* ------------------------------------------------------------------------ */
/* One barrier round, simulated sequentially.                                */
/*                                                                           */
/* [SYNCALL] §2: a barrier is an arrival relation -- nobody in the current   */
/* participant set continues until every member has executed the barrier.   */
/* [SYNCALL] §5.2 gives the per-participant steps: arrive (atomic +1,        */
/* returning the old value), derive the target, poll until the counter has  */
/* reached it.  The simulation runs the members' steps one phase at a time  */
/* (all writes, all arrivals, all polls, all reads), which is one legal      */
/* schedule; the brute-force enumerator in oracle/enumerate.py covers every  */
/* other schedule on small inputs.                                          */
/*                                                                           */
/* members[0..m-1]: ids of the participants of this round (ascending).       */
/* slot: per-wg witness slot; out_row: per-wg output of this round.          */
/* Returns ORC_OK, ORC_INVALID_VALUE when a round's target leaves the int32 */
/* range, or ORC_DEADLOCK when some member's poll could never               */
/* succeed (the counter sits below its target with every member arrived).   */
/* ------------------------------------------------------------------------ */
static int simulate_round(uint64_t seed, uint32_t round,
                          const int32_t* members, int32_t m,
                          int32_t* counter, uint32_t* slot, uint32_t* out_row,
                          int32_t* target_scratch)
{
    /* data phase before the barrier: each member publishes its witness */
    for (int32_t i = 0; i < m; ++i) {
        int32_t w = members[i];
        slot[w] = ccbo_witness_hash(seed, round, (uint32_t)w);
    }
    /* arrive: atomic fetch-add of one, target from the old value */
    for (int32_t i = 0; i < m; ++i) {
        int32_t before = *counter;
        if (ccbo_epoch_target_checked(before, m, &target_scratch[i]) != ORC_OK)
            return ORC_INVALID_VALUE;
        *counter = before + 1;
    }
    /* poll: released once the counter has reached the target (>=, see the
     * reading of the poll condition in the design notes) */
    for (int32_t i = 0; i < m; ++i) {
        if (!(*counter >= target_scratch[i])) return ORC_DEADLOCK;
    }
    /* data phase after the barrier: each member sums every member's slot */
    for (int32_t i = 0; i < m; ++i) {
        uint32_t sum = 0;
        for (int32_t j = 0; j < m; ++j) sum += slot[members[j]];
        out_row[members[i]] = sum;
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Slot rounds (whole grid or a leading subset).                             */
/*                                                                           */
/* nGrid workgroups are launched; the participants are workgroups            */
/* 0..N-1 with N from ccbo_participants ([SYNCALL] §4.2, and §7.2's partial */
/* example where cores at or beyond the sync count return without calling).*/
/* For each round r every member writes hash(seed, r, w), passes the        */
/* barrier, then writes the sum of all members' slots into out[r][w].       */
/* Non-members write nothing to `out` and mark status 2 (the idle mark of   */
/* [SYNCALL] §8); members mark status 1; 0 means never ran.                 */
/*                                                                           */
/* counter: in/out, the workspace counter (must start at a multiple of N,   */
/* zero per [SYNCALL] §4.1).  out: rounds*nGrid, caller zero-fills it.      */
/* ------------------------------------------------------------------------ */
int ccbo_slot_rounds(uint64_t seed, int32_t rounds, int32_t nGrid, int32_t usedCores,
                     uint32_t* out, int32_t* status, int32_t* counter)
{
    int32_t n = ccbo_participants(usedCores, nGrid);
    if (n < 0 || rounds < 0) return ORC_INVALID_VALUE;
    int32_t* members = (int32_t*)malloc(sizeof(int32_t) * (size_t)n);
    int32_t* targets = (int32_t*)malloc(sizeof(int32_t) * (size_t)n);
    uint32_t* slot = (uint32_t*)calloc((size_t)nGrid, sizeof(uint32_t));
    for (int32_t i = 0; i < n; ++i) members[i] = i;
    int rc = ORC_OK;
    for (int32_t r = 0; r < rounds && rc == ORC_OK; ++r)
        rc = simulate_round(seed, (uint32_t)r, members, n, counter, slot,
                            out + (size_t)r * (size_t)nGrid, targets);
    for (int32_t w = 0; w < nGrid; ++w) status[w] = (w < n) ? 1 : 2;
    free(members); free(targets); free(slot);
    return rc;
}

/* ------------------------------------------------------------------------ */
/* Grouped rounds: two disjoint groups and their union, each with its own    */
/* counter.  Group A = even workgroup ids, group B = odd ids, "mix" = all.   */
/* Round r is an A round when r mod 3 == 0, a B round when r mod 3 == 1 and */
/* a mix round when r mod 3 == 2.  Each barrier uses the counter of its     */
/* group and that group's size as N.  [SYNCALL] §6.2 requires that every    */
/* member of a counter enters that counter's barriers in the same order the */
/* same number of times; this pattern does so per counter.                  */
/* counters: in/out, three counters (A, B, mix).                             */
/* ------------------------------------------------------------------------ */
int ccbo_grouped_rounds(uint64_t seed, int32_t rounds, int32_t nGrid,
                        uint32_t* out, int32_t* status, int32_t* counters)
{
    if (nGrid < 2 || (nGrid % 2) != 0 || rounds < 0) return ORC_INVALID_VALUE;
    int32_t half = nGrid / 2;
    int32_t* even = (int32_t*)malloc(sizeof(int32_t) * (size_t)half);
    int32_t* odd = (int32_t*)malloc(sizeof(int32_t) * (size_t)half);
    int32_t* all = (int32_t*)malloc(sizeof(int32_t) * (size_t)nGrid);
    int32_t* targets = (int32_t*)malloc(sizeof(int32_t) * (size_t)nGrid);
    uint32_t* slot = (uint32_t*)calloc((size_t)nGrid, sizeof(uint32_t));
    for (int32_t i = 0; i < half; ++i) { even[i] = 2 * i; odd[i] = 2 * i + 1; }
    for (int32_t i = 0; i < nGrid; ++i) all[i] = i;
    int rc = ORC_OK;
    for (int32_t r = 0; r < rounds && rc == ORC_OK; ++r) {
        int kind = r % 3;
        const int32_t* members = kind == 0 ? even : (kind == 1 ? odd : all);
        int32_t m = kind == 2 ? nGrid : half;
        rc = simulate_round(seed, (uint32_t)r, members, m, &counters[kind], slot,
                            out + (size_t)r * (size_t)nGrid, targets);
    }
    for (int32_t w = 0; w < nGrid; ++w) status[w] = 1;
    free(even); free(odd); free(all); free(targets); free(slot);
    return rc;
}

/* ------------------------------------------------------------------------ */
/* Barrier-separated 3-point stencil (the data phase of the persistent      */
/* stencil workload).  Iteration t reads buffer t&1 and writes buffer       */
/* (t+1)&1:  x'[i] = (x[i-1] + 2*x[i] + x[i+1]) >> 2, with the ends clamped */
/* (x[-1] := x[0], x[n] := x[n-1]).  The sum is formed in 64 bits and the   */
/* shift is an arithmetic shift, i.e. floor division by 4.                  */
/* bufA holds the input; after `iters` iterations the result is in bufA    */
/* when iters is even and in bufB when it is odd (both are overwritten).    */
/* ------------------------------------------------------------------------ */
void ccbo_stencil(int32_t* bufA, int32_t* bufB, int64_t n, int32_t iters)
{
    int32_t* buf[2] = {bufA, bufB};
    for (int32_t t = 0; t < iters; ++t) {
        const int32_t* x = buf[t & 1];
        int32_t* y = buf[(t + 1) & 1];
        for (int64_t i = 0; i < n; ++i) {
            int64_t left = x[i > 0 ? i - 1 : 0];
            int64_t mid = x[i];
            int64_t right = x[i + 1 < n ? i + 1 : n - 1];
            y[i] = (int32_t)((left + 2 * mid + right) >> 2);
        }
    }
}

/* ------------------------------------------------------------------------ */
/* CntNotify record.  [CNTNOTIFY] §3.1: mode 0 overwrites the count with    */
/* value, mode 1 adds value, mode 2 ORs value in, mode 4 ANDs value in.     */
/* There is no mode 3; any code other than 0, 1, 2, 4 is rejected (pages    */
/* silent).  The count and value are uint32 ([CNTNOTIFY] §3.3), so ADD      */
/* wraps modulo 2^32.                                                        */
/* ------------------------------------------------------------------------ */
int ccbo_cnt_record(uint32_t* count, int32_t mode, uint32_t value)
{
    switch (mode) {
    case 0: *count = value; return ORC_OK;
    case 1: *count = *count + value; return ORC_OK;
    case 2: *count = *count | value; return ORC_OK;
    case 4: *count = *count & value; return ORC_OK;
    default: return ORC_INVALID_VALUE;
    }
}

/* ------------------------------------------------------------------------ */
/* CntNotify wait predicate.  [CNTNOTIFY] §3.2: the wait is released when   */
/*   mode 0: count <  value        mode 1: count == value                   */
/*   mode 2: count >  value        mode 3: count >= value                   */
/*   mode 4: (count & value) == value                                        */
/* Comparisons are unsigned 32-bit.  Other codes are rejected.              */
/* ------------------------------------------------------------------------ */
int ccbo_cnt_wait_holds(uint32_t count, int32_t mode, uint32_t value, int32_t* holds)
{
    switch (mode) {
    case 0: *holds = count < value; return ORC_OK;
    case 1: *holds = count == value; return ORC_OK;
    case 2: *holds = count > value; return ORC_OK;
    case 3: *holds = count >= value; return ORC_OK;
    case 4: *holds = (count & value) == value; return ORC_OK;
    default: *holds = 0; return ORC_INVALID_VALUE;
    }
}

/* ------------------------------------------------------------------------ */
/* One wait applied to a counter with no concurrent writer.                  */
/* [CNTNOTIFY] §3.3 and §7: isClear == 1 zeroes the count after the wait   */
/* has been released.  With no other writer a false predicate can never    */
/* become true, so the wait is not released, the count is left alone and no */
/* clear happens.                                                            */
/* ------------------------------------------------------------------------ */
int ccbo_cnt_wait_apply(uint32_t* count, int32_t mode, uint32_t value, int32_t isClear,
                        int32_t* released)
{
    int32_t holds = 0;
    int rc = ccbo_cnt_wait_holds(*count, mode, value, &holds);
    *released = holds;
    if (rc == ORC_OK && holds && isClear) *count = 0;
    return rc;
}

/* ------------------------------------------------------------------------ */
/* Batched CntNotify interpreter: nCounters independent counters, each      */
/* starting at 0, each receiving nOps operations in order k = 0..nOps-1.    */
/* Inputs are op-major: val[k*nCounters + c], meta[k*nCounters + c].         */
/* meta byte: bits 0-2 mode code, bit 3 isClear (waits only), bits 4-6 zero, */
/* bit 7 set for a wait, clear for a record.                                  */
/* Outputs: final[c]; rel[j*nCounters + c] = 1 if the j-th wait of counter c */
/* was released, else 0 (j counts waits of that counter from 0; at most     */
/* nRelRows waits are recorded).                                              */
/* A malformed op (bad mode code, reserved bit set, isClear on a record, or */
/* more waits than nRelRows) leaves the counter unchanged, writes rel 0 for */
/* a wait that has a row, and makes the call return ORC_INVALID_VALUE.      */
/* ------------------------------------------------------------------------ */
int ccbo_cnt_batch(const uint32_t* val, const uint8_t* meta, int64_t nCounters, int32_t nOps,
                   uint32_t* final_out, uint8_t* rel, int32_t nRelRows)
{
    int rc = ORC_OK;
    for (int64_t c = 0; c < nCounters; ++c) {
        uint32_t count = 0;
        int32_t j = 0;
        for (int32_t k = 0; k < nOps; ++k) {
            uint8_t m = meta[(int64_t)k * nCounters + c];
            uint32_t v = val[(int64_t)k * nCounters + c];
            int32_t mode = m & 7;
            int32_t isClear = (m >> 3) & 1;
            int is_wait = (m >> 7) & 1;
            int reserved = (m >> 4) & 7;
            if (is_wait) {
                if (j >= nRelRows) { rc = ORC_INVALID_VALUE; ++j; continue; }
                int32_t released = 0;
                if (reserved != 0) {
                    rc = ORC_INVALID_VALUE;
                } else if (ccbo_cnt_wait_apply(&count, mode, v, isClear, &released) != ORC_OK) {
                    rc = ORC_INVALID_VALUE;
                    released = 0;
                }
                rel[(int64_t)j * nCounters + c] = (uint8_t)released;
                ++j;
            } else {
                if (reserved != 0 || isClear) { rc = ORC_INVALID_VALUE; continue; }
                if (ccbo_cnt_record(&count, mode, v) != ORC_OK) rc = ORC_INVALID_VALUE;
            }
        }
        final_out[c] = count;
    }
    return rc;
}
