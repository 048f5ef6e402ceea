/*
 * ccb.h -- C ABI of the MI355X (gfx950) soft epoch barrier and CntNotify
 * library (libccb.so).
 *
 * Two pages define what this library computes:
 *   [SYNCALL]   "PTO-ISA 跨核同步屏障 SYNCALL 实战指南" (PTO-ISA cross-core
 *               barrier SYNCALL guide) -- the Soft (global-memory atomic
 *               counter) barrier: §2 semantics, §4.1 workspace, §4.2
 *               usedCores, §5.2 the epoch algorithm, §6.1-§6.3 usage rules,
 *               §7.2 partial participation, §8 tests and idle marks.
 *   [CNTNOTIFY] "CANN Runtime CntNotify（计数型通知）管理接口详解" (CANN Runtime
 *               CntNotify interfaces) -- §3.1 record modes, §3.2 wait modes,
 *               §3.3 info structs, §4.1-§4.6 the six calls, §5 usage, §7 advice.
 *
 * Conventions for every call below.
 *   - Every call returns a ccbStatus; 0 is success ([CNTNOTIFY] §4).
 *   - Pointers documented as "device" point to GPU memory that the CALLER
 *     allocated and owns (for example a torch tensor's data_ptr()); the
 *     library never frees them.  Pointers documented as "host" point to host
 *     memory.
 *   - ccbStream is a hipStream_t passed as an opaque pointer; NULL is the
 *     default (null) stream ([CNTNOTIFY] §5).  Calls that take a stream only
 *     enqueue work on it and return without waiting, unless stated otherwise.
 *   - Every call may be made from several host threads at once (the
 *     library's own state -- device table, register query, launch planning,
 *     CntNotify handle table -- is guarded by mutexes).
 *   - Calls act on the HIP device that is current on the calling thread.
 *     That device must be a gfx950 GPU, else CCB_ERR_UNSUPPORTED_DEVICE.
 *   - Arguments are validated before anything is enqueued; on an error
 *     return nothing has been enqueued and no output has been written.
 *   - A runtime error (CCB_ERR_HIP, or a cooperative launch the runtime
 *     refuses: CCB_ERR_NOT_CORESIDENT) is reported through the returned
 *     status alone: the calling thread's HIP last-error state is left clear,
 *     so it does not resurface as the error of a later, unrelated launch.
 */
#ifndef CCB_H
#define CCB_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CCB_API __attribute__((visibility("default")))

typedef int32_t ccbStatus;
typedef void* ccbStream; /* hipStream_t; NULL = default stream */

enum {
    CCB_OK = 0,
    CCB_ERR_INVALID_VALUE = 1,      /* bad size, count, mode code, flag, alignment */
    CCB_ERR_NULL_POINTER = 2,       /* a required pointer is NULL */
    CCB_ERR_INVALID_HANDLE = 3,     /* unknown or destroyed CntNotify handle */
    CCB_ERR_RESOURCE_EXHAUSTED = 4, /* CntNotify pool full ([CNTNOTIFY] §4.1) */
    CCB_ERR_TIMEOUT = 5,            /* a CntNotify wait expired ([CNTNOTIFY] §3.3) */
    CCB_ERR_DEADLOCK = 6,           /* a barrier poll hit its bound ([SYNCALL] §5.2) */
    CCB_ERR_NOT_CORESIDENT = 7,     /* the grid cannot be resident at once ([SYNCALL] §6.3) */
    CCB_ERR_UNSUPPORTED_DEVICE = 8, /* current device is not gfx950 */
    CCB_ERR_HIP = 9,                /* the HIP runtime reported an error */
    CCB_ERR_NOT_READY = 10,         /* no CntNotify wait has completed yet */
    CCB_ERR_CANCELLED = 11          /* a CntNotify wait ended by abort or destroy */
};

/* Default poll bound of the soft barrier: [SYNCALL] §5.2 bounds the poll at
 * one million iterations before reporting a possible deadlock. */
#define CCB_SOFT_MAX_POLL 1000000u

/* Bytes of one workspace line.  [SYNCALL] §4.1 gives each counter a cache
 * line of its own (64 B on the pages' hardware); gfx950's L2 line is 128 B. */
#define CCB_LINE_BYTES 128

/* Counter stripes reserved per barrier in a workspace (see ccb_device.h). */
#define CCB_STRIPES 64

/* Barrier variant used by a workload launcher: one counter layout ORed with
 * one visibility strength.
 *   CCB_BARRIER_STRIPED   the counter split over CCB_STRIPES lines; member m
 *                         arrives on stripe m mod CCB_STRIPES and one wave
 *                         polls every stripe with a single gather load
 *   CCB_BARRIER_FLAT      the pages' single counter ([SYNCALL] §5.2)
 *   CCB_BARRIER_TREE      a two-level arrival tree: CCB_TREE_GROUPS group
 *                         counters (member m arrives on group m mod 8) under
 *                         one top counter that each group's completing
 *                         arrival adds to; every member polls the top
 *                         counter (see ccb_device.h)
 *   CCB_VISIBILITY_ORDER  arrival plus ordering of each thread's memory
 *                         operations, no cache maintenance ([SYNCALL] §6.1);
 *                         the workloads then share data through
 *                         device-coherent accesses
 *   CCB_VISIBILITY_FULL   agent-scope release and acquire fences around the
 *                         arrival and poll; the workloads share data through
 *                         plain accesses
 *   CCB_VISIBILITY_XCD    what CCB_VISIBILITY_FULL guarantees, with one L2
 *                         write-back per XCD per barrier (by a leader
 *                         workgroup, after every member has arrived) instead
 *                         of one per workgroup; each workgroup still runs
 *                         its own acquire (see ccb_device.h) */
enum {
    CCB_BARRIER_STRIPED = 0,
    CCB_BARRIER_FLAT = 1,
    CCB_BARRIER_TREE = 4,
    CCB_VISIBILITY_ORDER = 0,
    CCB_VISIBILITY_FULL = 2,
    CCB_VISIBILITY_XCD = 8
};

/* Group counters of CCB_BARRIER_TREE: the MI355X's XCD count, so that with
 * the usual round-robin dispatch of workgroups over the XCDs each group's
 * members share one XCD. */
#define CCB_TREE_GROUPS 8

/* CntNotify mode codes, as enumerated in [CNTNOTIFY] §3.1 and §3.2. */
enum {
    CCB_CNT_RECORD_SET_VALUE = 0, /* count = value */
    CCB_CNT_RECORD_ADD = 1,       /* count = count + value (mod 2^32) */
    CCB_CNT_RECORD_BIT_OR = 2,    /* count = count | value */
    CCB_CNT_RECORD_BIT_AND = 4    /* count = count & value (there is no code 3) */
};
enum {
    CCB_CNT_WAIT_LESS = 0,              /* release when count <  value */
    CCB_CNT_WAIT_EQUAL = 1,             /* release when count == value */
    CCB_CNT_WAIT_BIGGER = 2,            /* release when count >  value */
    CCB_CNT_WAIT_BIGGER_OR_EQUAL = 3,   /* release when count >= value */
    CCB_CNT_WAIT_EQUAL_WITH_BITMASK = 4 /* release when (count & value) == value */
};

/* ========================================================================
 * Miscellaneous
 * ======================================================================== */

/* Human-readable name of a status code (static string, never NULL). */
CCB_API const char* ccb_status_string(ccbStatus s);

/* Library version as major*10000 + minor*100 + patch. */
CCB_API int32_t ccb_version(void);

/* Checks that the current device is gfx950 and fills (each may be NULL):
 * number of compute units, LDS bytes per CU, wall-clock rate in kHz.
 * Errors: CCB_ERR_UNSUPPORTED_DEVICE, CCB_ERR_HIP. */
CCB_API ccbStatus ccb_device_info(int32_t* numCUs, int32_t* ldsPerCU, int32_t* wallClockKHz);

/* ========================================================================
 * Soft epoch barrier ([SYNCALL] §4.1, §4.2, §5.2)
 *
 * Workspace layout.  A workspace for k barriers is (k * CCB_STRIPES + 1)
 * lines of CCB_LINE_BYTES bytes, 128-byte aligned, device memory owned by
 * the caller:
 *   lines b*CCB_STRIPES .. (b+1)*CCB_STRIPES-1: the counter stripes of
 *        barrier b, an int32 at byte 0 of each line; the other 124 bytes are
 *        reserved and never shared with data ([SYNCALL] §4.1).  A FLAT
 *        barrier uses only its first stripe;
 *   line k*CCB_STRIPES: int32 error word at byte 0 (CCB_OK, or
 *        CCB_ERR_DEADLOCK once any member's poll hit its bound).
 * With CCB_VISIBILITY_XCD a barrier also uses bytes 32..63 of its stripe
 * lines 1 and 2: the members registered per XCD and each XCD's last
 * written-back round (8 int32 each).
 * Every stripe must be zero (or a multiple of its participant count) when a
 * launch starts ([SYNCALL] §4.1); ccb_syncall_workspace_reset zeroes the
 * workspace.  A stripe stays valid while the number of arrivals on it since
 * the last reset plus the participant count stays below 2^31; the launchers
 * below return CCB_ERR_INVALID_VALUE for a launch that would break this when
 * started from a zeroed workspace (striped: ceil(N / CCB_STRIPES) arrivals
 * per stripe and barrier; FLAT: N; TREE: ceil(N / CCB_TREE_GROUPS) per group
 * counter and min(N, CCB_TREE_GROUPS) on the top counter).  A TREE barrier
 * uses stripe lines 0 .. CCB_TREE_GROUPS - 1 for its group counters and the
 * int32 at byte 64 of line CCB_STRIPES - 1 for its top counter.
 *
 * Every workload launcher below runs one persistent grid in which each
 * workgroup is resident for the whole launch ([SYNCALL] §6.3: the
 * participant set is fixed by the launch).  The launcher checks the
 * occupancy first and returns CCB_ERR_NOT_CORESIDENT when nGrid workgroups of
 * `threads` threads cannot all be resident at once: the smaller of the
 * occupancy API's count and the count the kernel's SGPRs allow, at 800 SGPRs
 * per SIMD and 16 trap-handler SGPRs per wave beyond the kernel's own
 * allocation (which the API leaves out).  Workgroups of 5-7, 9-11 or 13-15
 * waves are counted as if ceil(waves / 4) of their waves shared one SIMD
 * (their waves do not spread evenly; 1-4 waves and multiples of 4 do).  The
 * first persistent launch on a
 * device reads every kernel variant's allocation with one-workgroup query
 * launches on the default stream and waits for them (no allocation, no new
 * stream); make that first call outside stream capture.  After it, every
 * launcher, the workspace reset and the CntNotify record / wait / reset /
 * batch calls can be captured into a HIP graph (kernel nodes only).  `wgsPerCu` > 0 also
 * sizes each workgroup's LDS so that at most that many share a compute unit
 * (0 = no shaping).  `maxPoll` bounds each barrier's poll loop (0 = the
 * default CCB_SOFT_MAX_POLL); a member that exhausts it sets the error word
 * and leaves its round loop, and so does every member that then sees the
 * error word -- no launch traps or hangs.  `mode` picks the barrier variant
 * (CCB_BARRIER_* | CCB_VISIBILITY_*: 0, 1, 2, 3, 4, 6, 8, 9 or 12); any
 * other value is INVALID_VALUE.  Read
 * the outcome with ccb_syncall_status after the stream has run the launch.
 * ======================================================================== */

/* Size in bytes of a workspace for nBarriers barriers:
 * (nBarriers * CCB_STRIPES + 1) * CCB_LINE_BYTES. */
CCB_API size_t ccb_syncall_workspace_bytes(uint32_t nBarriers);

/* Enqueue a zero fill of a workspace of nBarriers barriers (device, 128-B
 * aligned, ccb_syncall_workspace_bytes(nBarriers) bytes).
 * Errors: NULL_POINTER, INVALID_VALUE (nBarriers == 0 or misaligned). */
CCB_API ccbStatus ccb_syncall_workspace_reset(int32_t* ws, uint32_t nBarriers, ccbStream stream);

/* Wait for `stream`, then read the error word of a workspace of nBarriers
 * barriers and (optionally, arrivals may be NULL) store in arrivals[b] the
 * total number of arrivals on barrier b (the sum of its stripes; int64, as
 * the total of 64 int32 stripes can pass 2^31).  Reads the stripe lines a
 * few barriers at a time through a 64-KiB host buffer.  Returns CCB_OK,
 * CCB_ERR_DEADLOCK (a poll hit its bound), or CCB_ERR_INVALID_VALUE (a
 * member found its stripe past the int32 range of [SYNCALL] §4.1: the
 * workspace was not re-zeroed in time); CCB_ERR_HIP, or
 * CCB_ERR_RESOURCE_EXHAUSTED when the host buffer cannot be allocated
 * (arrivals may then be partly written).  Blocks the host thread. */
CCB_API ccbStatus ccb_syncall_status(const int32_t* ws, uint32_t nBarriers, int64_t* arrivals,
                                     ccbStream stream);

/* Barrier-only persistent grid: `rounds` consecutive soft barriers on
 * counter 0 of `ws` (1 counter), with participants chosen as in [SYNCALL]
 * §4.2 and §7.2: usedCores == 0 means all nGrid workgroups; otherwise
 * workgroups 0..usedCores-1 take part and the others return at once without
 * calling the barrier.
 *   ws         device, workspace of 1 barrier
 *   placement  device, 2 * nGrid uint32, may be NULL: per workgroup w the
 *              hardware location it ran on: [2w] = the HW_ID register
 *              (CU id bits 8-11, SH id bit 12, SE id bits 13-15), [2w+1] = the
 *              XCC (XCD) id
 *   wgStatus   device, nGrid int32, may be NULL: 1 member finished, 2 idle
 *              (ran, skipped the barrier: the idle mark of [SYNCALL] §8),
 *              3 member stopped on the error word
 * Errors: NULL_POINTER, INVALID_VALUE (rounds < 0, nGrid < 1, threads not a
 * multiple of 64 in [64, 1024], usedCores < 0 or > nGrid), NOT_CORESIDENT. */
CCB_API ccbStatus ccb_run_barrier_only(int32_t* ws, uint32_t* placement, int32_t* wgStatus,
                                       int32_t rounds, int32_t nGrid, int32_t threads,
                                       int32_t usedCores, int32_t wgsPerCu, uint32_t maxPoll,
                                       int32_t mode, ccbStream stream);

/* Most rounds one ccb_bench_barrier_breakdown launch can stamp. */
#define CCB_BREAKDOWN_MAX_ROUNDS 1024

/* Latency breakdown of the soft barrier (instrumentation, not on the pages):
 * ccb_run_barrier_only's rounds over all nGrid workgroups (usedCores = 0),
 * with lane 0 of every member reading the device wall clock at three points
 * of each round r:
 *   stamps[(r * nGrid + w) * 3 + 0]  just before it issues its arrival
 *   stamps[(r * nGrid + w) * 3 + 1]  when the arrival's reply is back
 *   stamps[(r * nGrid + w) * 3 + 2]  when its poll has seen the round
 *                                    complete (before the acquire fence)
 * (uint64 ticks at the rate ccb_device_info reports).  The stamps are kept
 * in LDS until the last round and written out at the end.
 *   ws      device, workspace of 1 barrier (zeroed)
 *   stamps  device, rounds * nGrid * 3 uint64, 8-B aligned
 * rounds: 1 .. CCB_BREAKDOWN_MAX_ROUNDS.  wgsPerCu and mode as in
 * ccb_run_barrier_only; the poll bound is CCB_SOFT_MAX_POLL.  Read the
 * outcome with ccb_syncall_status.
 * Errors: NULL_POINTER, INVALID_VALUE, NOT_CORESIDENT. */
CCB_API ccbStatus ccb_bench_barrier_breakdown(int32_t* ws, uint64_t* stamps, int32_t rounds,
                                              int32_t nGrid, int32_t threads, int32_t wgsPerCu,
                                              int32_t mode, ccbStream stream);

/* The witness slots of the two witness workloads: a ring of CCB_SLOT_ROWS
 * rows of nGrid slots, one slot every CCB_SLOT_WORDS uint32.  Slot p of
 * ring row q is word ((q mod CCB_SLOT_ROWS) * nGrid + p) * CCB_SLOT_WORDS;
 * a slots buffer holds CCB_SLOT_ROWS * nGrid * CCB_SLOT_WORDS uint32. */
#define CCB_SLOT_ROWS 6
#define CCB_SLOT_WORDS 4

/* Witness rounds on one counter ([SYNCALL] §6.1's pattern of slots written
 * before a barrier and read after it).  For r = 0..rounds-1 every member w
 * stores hash(seed, r, w) into its slot of ring row r mod CCB_SLOT_ROWS,
 * passes the barrier, then stores the sum (mod 2^32) of every member's slot
 * in that row into out[r * nGrid + w].  hash is SplitMix64 output number
 * r * 2^32 + w + 1 for seed `seed`, high 32 bits.  Members are chosen by
 * usedCores as in ccb_run_barrier_only; non-members write no slot and no
 * output.
 *   ws        device, workspace of 1 barrier (zeroed)
 *   slots     device, CCB_SLOT_ROWS * nGrid * CCB_SLOT_WORDS uint32
 *             scratch (contents on entry ignored)
 *   out       device, rounds * nGrid uint32; entries of non-members untouched
 *   wgStatus  device, nGrid int32 (see ccb_run_barrier_only), may be NULL
 * Errors: as ccb_run_barrier_only, plus NULL_POINTER for slots/out (which
 * may be NULL only when rounds == 0). */
CCB_API ccbStatus ccb_run_slot_rounds(int32_t* ws, uint32_t* slots, uint32_t* out,
                                      int32_t* wgStatus, uint64_t seed, int32_t rounds,
                                      int32_t nGrid, int32_t threads, int32_t usedCores,
                                      int32_t wgsPerCu, uint32_t maxPoll, int32_t mode,
                                      ccbStream stream);

/* Grouped witness rounds on three barriers: group A = even workgroup ids on
 * barrier 0, group B = odd ids on barrier 1, "mix" = every workgroup on
 * barrier 2.  Round r is an A round when r mod 3 == 0, B when 1, mix when 2;
 * its members store hash(seed, r, w), pass that group's barrier (N = nGrid/2
 * for A and B, nGrid for mix) and store the sum of the round's members'
 * slots into out[r * nGrid + w].  Non-members of a round do nothing in it.
 * Every member enters each counter's barriers in the same order the same
 * number of times ([SYNCALL] §6.2).
 *   ws     device, workspace of 3 barriers (zeroed)
 *   slots  device, CCB_SLOT_ROWS * nGrid * CCB_SLOT_WORDS uint32 scratch
 *   out    device, rounds * nGrid uint32
 * Errors: as ccb_run_slot_rounds; nGrid must be even. */
CCB_API ccbStatus ccb_run_grouped_rounds(int32_t* ws, uint32_t* slots, uint32_t* out,
                                         int32_t* wgStatus, uint64_t seed, int32_t rounds,
                                         int32_t nGrid, int32_t threads, int32_t wgsPerCu,
                                         uint32_t maxPoll, int32_t mode, ccbStream stream);

/* ccb_run_grouped_rounds (usedCores, wgStatus and maxPoll at their
 * defaults) with a timeline, for per-round-kind timing (instrumentation, not
 * on the pages): member w records, for each of its first
 * CCB_BREAKDOWN_MAX_ROUNDS own rounds i (an even w's rounds are the A and mix
 * rounds, an odd w's the B and mix rounds, in order), the device wall clock
 * when it passed that round's barrier:
 *   stamps  device, min(rounds, CCB_BREAKDOWN_MAX_ROUNDS) * nGrid uint64,
 *           8-B aligned; stamps[i * nGrid + w], 0 past w's last round
 * The stamps are kept in LDS and written out at the end.  Other arguments
 * and errors as ccb_run_grouped_rounds (NULL_POINTER also for stamps). */
CCB_API ccbStatus ccb_bench_grouped_timeline(int32_t* ws, uint32_t* slots, uint32_t* out,
                                             uint64_t* stamps, uint64_t seed, int32_t rounds,
                                             int32_t nGrid, int32_t threads, int32_t wgsPerCu,
                                             int32_t mode, ccbStream stream);

/* Persistent barrier-separated stencil.  Iteration t reads buffer t & 1 and
 * writes buffer (t + 1) & 1 (buffer 0 = bufA, 1 = bufB):
 *   y[i] = (x[i-1] + 2 x[i] + x[i+1]) >> 2,  x[-1] = x[0], x[n] = x[n-1],
 * with one soft barrier over all nGrid workgroups between consecutive
 * iterations (iters - 1 barriers).  The result is in bufA when iters is even,
 * in bufB when odd.  The caller guarantees |x| < 2^29 so that the int32 sum
 * cannot overflow.  The array is cut into chunks of 4 * threads elements;
 * workgroup w owns chunks w, w + nGrid, ... in every iteration, so only the
 * two boundary elements of each chunk cross workgroups; with
 * CCB_VISIBILITY_ORDER they go through `halo`.
 *   bufA, bufB  device, n int32 each, 16-B aligned, not overlapping
 *   ws          device, workspace of 1 barrier (zeroed)
 *   halo        device, haloBytes bytes of scratch (contents ignored), at
 *               least ccb_stencil_halo_bytes(n, threads, nGrid); may be NULL (and
 *               haloBytes 0) with CCB_VISIBILITY_FULL or CCB_VISIBILITY_XCD
 *   timeline    device, nGrid * (2 * iters + 1) uint64 wall-clock stamps, or
 *               NULL: for workgroup w, [w*(2*iters+1)] = its start, then for
 *               each iteration t, [.. + 1 + 2t] = the end of its data phase and
 *               [.. + 2 + 2t] = when it left the following barrier (the end of
 *               the launch for the last iteration); 8-B aligned
 * Errors: NULL_POINTER, INVALID_VALUE (n < 1, iters < 0, misaligned or
 * overlapping buffers, halo scratch too small, bad nGrid/threads/mode),
 * NOT_CORESIDENT. */
CCB_API ccbStatus ccb_run_stencil(int32_t* bufA, int32_t* bufB, int64_t n, int32_t iters,
                                  int32_t* ws, int32_t* halo, size_t haloBytes,
                                  uint64_t* timeline, int32_t nGrid, int32_t threads,
                                  int32_t wgsPerCu, uint32_t maxPoll, int32_t mode,
                                  ccbStream stream);

/* Bytes of the halo exchange scratch ccb_run_stencil needs with
 * CCB_VISIBILITY_ORDER: two parities x nGrid workgroups x the chunks of the
 * busiest workgroup x 2 int32 (0 for invalid arguments). */
CCB_API size_t ccb_stencil_halo_bytes(int64_t n, int32_t threads, int32_t nGrid);

/* Bytes of the device scratch that ccb_run_stencil_noalloc uses on each GPU:
 * a file-scope device array (held by every GPU the library runs on until the
 * process ends) with the workspace of one barrier (8,448 bytes) and then the
 * halo exchange buffer. */
#define CCB_NOALLOC_SCRATCH_BYTES (4u << 20)

/* ccb_run_stencil for callers that cannot allocate device memory: code being
 * captured into a HIP graph, tight serving loops, harnesses that forbid
 * hipMalloc.  It takes no workspace and no halo scratch; both live in the
 * library's own device scratch of CCB_NOALLOC_SCRATCH_BYTES, and the call
 * allocates nothing (no hipMalloc / hipFree, no allocating library call).
 * It enqueues on `stream`: a fill kernel that zeroes the workspace part, the
 * stencil launch, and (statusOut != NULL) a one-lane kernel that copies the
 * outcome word -- CCB_OK, CCB_ERR_DEADLOCK or CCB_ERR_INVALID_VALUE, as
 * ccb_syncall_status reports it -- to *statusOut (device int32, 4-B
 * aligned).  Arguments and results are those of ccb_run_stencil otherwise.
 * Limit: with CCB_VISIBILITY_ORDER, 8,448 + ccb_stencil_halo_bytes(n,
 * threads, nGrid) must fit in CCB_NOALLOC_SCRATCH_BYTES (n up to about
 * 2.6e8 elements at 256 threads per workgroup); CCB_VISIBILITY_FULL and
 * CCB_VISIBILITY_XCD need only the workspace part.  Larger launches return CCB_ERR_INVALID_VALUE.
 * Every call on one GPU shares that GPU's scratch: calls that overlap in
 * time on one GPU (on different streams, or from different host threads
 * without ordering) race on it and give wrong results; order them on one
 * stream.  The first persistent launch of the process on a device also runs
 * the launchers' one-time register query (see above): make one call outside
 * stream capture first.
 * Errors: as ccb_run_stencil (NULL_POINTER for bufA / bufB; INVALID_VALUE
 * also for a launch beyond the scratch or a misaligned statusOut). */
CCB_API ccbStatus ccb_run_stencil_noalloc(int32_t* bufA, int32_t* bufB, int64_t n, int32_t iters,
                                          int32_t* statusOut, int32_t nGrid, int32_t threads,
                                          int32_t wgsPerCu, uint32_t maxPoll, int32_t mode,
                                          ccbStream stream);

/* ========================================================================
 * Floor microbenchmarks (the barrier's latency and bandwidth roofline)
 * ======================================================================== */

/* One lane runs `iters` dependent agent-scope fetch-adds of 1 on the int32 at
 * byte 0 of `line` (device, 128-B aligned, exclusive).  fenced != 0 wraps
 * each one in an agent-scope release fence before and acquire fence after.
 * kind 1 runs dependent agent-scope atomic loads instead of fetch-adds.
 * ticksOut (device, 2 uint64): wall-clock ticks at start and end (rate from
 * ccb_device_info).  Errors: NULL_POINTER, INVALID_VALUE (iters < 1, kind). */
CCB_API ccbStatus ccb_bench_atomic_chain(int32_t* line, uint64_t* ticksOut, int32_t iters,
                                         int32_t fenced, int32_t kind, ccbStream stream);

/* nGrid workgroups, lane 0 of each runs `iters` dependent agent-scope
 * fetch-adds of 1 on the same int32 (device, 128-B line).  Final value grows
 * by nGrid * iters.  ticksOut (device, 2 * nGrid uint64): per workgroup
 * start/end ticks.  Errors: NULL_POINTER, INVALID_VALUE, NOT_CORESIDENT. */
CCB_API ccbStatus ccb_bench_atomic_contended(int32_t* line, uint64_t* ticksOut, int32_t iters,
                                             int32_t nGrid, ccbStream stream);

/* Notification ping-pong between two workgroups: the time one CU's update
 * takes to reach another CU's poll, the step a barrier cannot avoid.
 * Workgroups 0 and `peer` (1..255) of a cooperative launch of peer + 1
 * one-wave workgroups take `iters` turns: workgroup 0 adds one to the int32
 * at byte 0 of lines (line A) and polls line B (byte 128) until it holds the
 * turn; the partner polls A, then adds one to B.  Both use the barrier's
 * arrival (agent-scope fetch-add) and poll (agent-scope loads, same back-off).
 *   lines     device, 2 x 128 B, 128-B aligned, zeroed by the caller; both
 *             words equal iters afterwards
 *   ticksOut  device, 4 uint64: start and end on workgroup 0's wall clock
 *             (rate from ccb_device_info), then the XCC (XCD) id of workgroup
 *             0 and of workgroup `peer`.  One-way latency = (end - start) /
 *             (2 * iters) ticks.
 *   maxPoll   bound on each wait (0: CCB_SOFT_MAX_POLL); past it *err (device
 *             int32, zeroed by the caller) gets CCB_ERR_DEADLOCK and both
 *             sides stop.
 * Errors: NULL_POINTER, INVALID_VALUE (iters < 1, peer outside 1..255,
 * misaligned lines, ticksOut or err), NOT_CORESIDENT. */
CCB_API ccbStatus ccb_bench_notify_pingpong(int32_t* lines, uint64_t* ticksOut, int32_t iters,
                                           int32_t peer, uint32_t maxPoll, int32_t* err,
                                           ccbStream stream);

/* Where a full-visibility barrier's cache maintenance can go (measurement,
 * not on the pages).  nGrid workgroups (at most one per compute unit) run
 * `rounds` barriers on the striped counter; before each, thread 0 of member w
 * stores r + 1 to its data line with a plain store, and after it loads member
 * (w + 1) mod nGrid's with a plain load.  `variant` places the agent-scope
 * release (L2 write-back) and acquire (invalidate):
 *   0  none (the ordering-only barrier)
 *   1  every workgroup: release before its arrival, acquire after its poll
 *      (what CCB_VISIBILITY_FULL does)
 *   2  every workgroup: release only
 *   3  every workgroup: acquire only
 *   4  one release per XCD: once all members have arrived, one leader
 *      workgroup per XCD (the first to register its XCC id at the start)
 *      writes back its L2 and raises a flag; every workgroup waits for the
 *      flags of the XCDs that hold members, then acquires
 *   5  as 4, with a workgroup-scope invalidate (buffer_inv sc0) as each
 *      workgroup's acquire
 *   scratch       device, scratchBytes >= ccb_bench_fence_placement_bytes(nGrid),
 *                 128-B aligned (zeroed here by a fill kernel)
 *   stale         device, nGrid int32: per member, the loads that returned an
 *                 older value than the round's
 * The caller times launches (e.g. two round counts).  Every wait is bounded
 * by CCB_SOFT_MAX_POLL.  Errors: NULL_POINTER, INVALID_VALUE,
 * NOT_CORESIDENT (nGrid above the CU count). */
CCB_API size_t ccb_bench_fence_placement_bytes(int32_t nGrid);
CCB_API ccbStatus ccb_bench_fence_placement(int32_t* scratch, size_t scratchBytes, int32_t* stale,
                                            int32_t rounds, int32_t nGrid, int32_t threads,
                                            int32_t variant, ccbStream stream);

/* HIP's cooperative-groups grid barrier (grid_group::sync) `rounds` times in
 * one cooperative launch of nGrid workgroups of `threads` threads (a
 * multiple of 64, at most 1024): the platform's stock grid barrier, for
 * timing beside the soft barrier (not on the pages).  When the launch ends,
 * *doneOut (device int32) holds `rounds`.  The caller times it (e.g. two
 * launches with different `rounds`).  Errors: NULL_POINTER, INVALID_VALUE,
 * NOT_CORESIDENT (more workgroups than can be resident at once: checked
 * before the launch, since grid sync waits without a bound). */
CCB_API ccbStatus ccb_bench_hip_grid_sync(int32_t rounds, int32_t nGrid, int32_t threads,
                                          int32_t* doneOut, ccbStream stream);

/* Streaming copy of nBytes (multiple of 16) from src to dst (device, 16-B
 * aligned, not overlapping): the achievable HBM ceiling for the data phases.
 * Errors: NULL_POINTER, INVALID_VALUE. */
CCB_API ccbStatus ccb_bench_copy(void* dst, const void* src, int64_t nBytes, ccbStream stream);

/* ========================================================================
 * CntNotify ([CNTNOTIFY] §3, §4)
 *
 * A CntNotify is an opaque handle ([CNTNOTIFY] §1) owned by the library.
 * Its uint32 count lives alone on a 128-byte line of a fixed pool of
 * CCB_CNT_NOTIFY_POOL lines in the device memory of the device that was
 * current at create time; every call on a handle must run with that device
 * current.  Record, wait and reset only enqueue work on their stream
 * ([CNTNOTIFY] §4.2-§4.4, §7): the host thread never waits for them.
 * Handle calls are thread-safe (one mutex guards the handle table).
 * ======================================================================== */

#define CCB_CNT_NOTIFY_POOL 1024

typedef struct ccbCntNotify_st* ccbCntNotify;

/* [CNTNOTIFY] §3.3: record descriptor. mode: CCB_CNT_RECORD_*. 8 bytes. */
typedef struct {
    int32_t mode;
    uint32_t value;
} ccbCntRecordInfo;

/* [CNTNOTIFY] §3.3: wait descriptor. mode: CCB_CNT_WAIT_*; timeout in
 * seconds, 0 = wait forever; isClear = 1 zeroes the count after the wait has
 * been released, 0 leaves it; rev must be zero.  16 bytes. */
typedef struct {
    int32_t mode;
    uint32_t value;
    uint32_t timeout;
    uint8_t isClear;
    uint8_t rev[3];
} ccbCntWaitInfo;

/* [CNTNOTIFY] §4.1.  *out receives a new handle whose count is 0.  flag is
 * reserved and must be 0.  Blocks the host (it initialises the line).
 * Errors: NULL_POINTER (out), INVALID_VALUE (flag != 0), RESOURCE_EXHAUSTED
 * (all CCB_CNT_NOTIFY_POOL lines in use), UNSUPPORTED_DEVICE, HIP. */
CCB_API ccbStatus ccb_cnt_notify_create(ccbCntNotify* out, uint64_t flag);

/* [CNTNOTIFY] §4.2.  Enqueue on `stream` one update of the count by
 * info->mode / info->value (stream is where the counted event happens).
 * The update is atomic at device scope and is ordered after everything
 * enqueued earlier on `stream`.
 * Errors: INVALID_HANDLE, NULL_POINTER (info), INVALID_VALUE (mode). */
CCB_API ccbStatus ccb_cnt_notify_record(ccbCntNotify h, ccbStream stream,
                                        const ccbCntRecordInfo* info);

/* [CNTNOTIFY] §4.3.  Enqueue on `stream` a wait that blocks the stream's
 * later work until the predicate info->mode / info->value holds for the
 * count, or until info->timeout seconds have passed (0 = no limit).  When it
 * is released and isClear is 1 the count is set to 0 atomically with the
 * check that released it (a concurrent record is never lost).  The outcome
 * (CCB_OK, CCB_ERR_TIMEOUT or CCB_ERR_CANCELLED) is stored with the
 * handle; read it with ccb_cnt_notify_query.  A timed-out or cancelled wait
 * does not clear.  The wait is a one-lane polling kernel: streams share a
 * few hardware queues, and a queue runs its kernels in order, so enqueue the
 * records a wait depends on before the wait (or give the wait a timeout); a
 * record queued behind a wait with no limit on the same hardware queue can
 * never run.  Such a wait can still be ended from the host with
 * ccb_cnt_notify_abort or ccb_cnt_notify_destroy.
 * Errors: INVALID_HANDLE, NULL_POINTER (info), INVALID_VALUE (mode,
 * isClear > 1, rev not zero). */
CCB_API ccbStatus ccb_cnt_notify_wait(ccbCntNotify h, ccbStream stream,
                                      const ccbCntWaitInfo* info);

/* [CNTNOTIFY] §4.4.  Enqueue on `stream` a reset of the count to 0.
 * Errors: INVALID_HANDLE. */
CCB_API ccbStatus ccb_cnt_notify_reset(ccbCntNotify h, ccbStream stream);

/* [CNTNOTIFY] §4.5.  *id receives the handle's id (its pool line index,
 * stable for the handle's life; reused after destroy).
 * Errors: INVALID_HANDLE, NULL_POINTER (id). */
CCB_API ccbStatus ccb_cnt_notify_get_id(ccbCntNotify h, uint32_t* id);

/* [CNTNOTIFY] §4.6.  Return the handle's line to the pool; the handle is
 * invalid afterwards (later calls on it return CCB_ERR_INVALID_HANDLE).
 * Waits on the handle that are still queued or polling end as by
 * ccb_cnt_notify_abort, so no stream stays blocked on a destroyed handle.
 * Records and resets still queued for it act on the line's word pair of
 * this handle's generation only: each of the 16 generations of a line uses
 * its own (count, outcome) pair, and freed lines are reused least recently
 * freed first, so they never reach the count of the line's next owner
 * unless that line has since been reused 16 times.
 * Errors: INVALID_HANDLE. */
CCB_API ccbStatus ccb_cnt_notify_destroy(ccbCntNotify h);

/* Calls off every wait on h enqueued before this call (not on the pages,
 * whose waits end only by release or time-out; for a stream whose wait can
 * no longer be satisfied, such as a wait with no time limit).  Each such
 * wait that has not been released ends with CCB_ERR_CANCELLED, does not
 * clear, and unblocks its stream; waits enqueued after the call are not
 * affected.  The host stores a new token for the handle in pinned host
 * memory and returns at once; a polling wait reads the token every 64 polls
 * (tens of microseconds).
 * Errors: INVALID_HANDLE. */
CCB_API ccbStatus ccb_cnt_notify_abort(ccbCntNotify h);

/* Test and diagnostics hook (not on the pages): wait for `stream`, then copy
 * the current count to *value and the outcome of the last completed wait to
 * *lastWait (CCB_OK, CCB_ERR_TIMEOUT, CCB_ERR_CANCELLED, or
 * CCB_ERR_NOT_READY if none has completed since create).  Either pointer may be NULL.  Blocks the host.
 * Errors: INVALID_HANDLE, HIP. */
CCB_API ccbStatus ccb_cnt_notify_query(ccbCntNotify h, uint32_t* value, ccbStatus* lastWait,
                                       ccbStream stream);

/* Batched CntNotify engine: nCounters independent counts, each starting at
 * 0, each applying nOps operations in order k = 0..nOps-1.  Inputs are
 * op-major device arrays:
 *   val[k * nCounters + c]   uint32 operand
 *   meta[k * nCounters + c]  uint8: bits 0-2 mode code, bit 3 isClear (waits
 *                            only), bits 4-6 zero, bit 7 = 1 for a wait,
 *                            0 for a record
 * Records follow [CNTNOTIFY] §3.1; a wait evaluates the §3.2 predicate on
 * the current count, releases if it holds and then clears if isClear; with no
 * concurrent writer a false predicate never becomes true, so it is not
 * released and the count is unchanged.
 * Outputs (device): final[c] uint32; rel[j * nCounters + c] uint8 = 1 if the
 * j-th wait of counter c released, else 0 (j = 0.. per counter, at most
 * nRelRows rows).
 * A malformed op (bad mode, reserved bit, isClear on a record, a wait beyond
 * nRelRows) leaves the count unchanged, writes rel 0 for a wait that has a
 * row, and sets *err (device int32, may be NULL) to CCB_ERR_INVALID_VALUE;
 * *err is not written otherwise, so the caller zeroes it first.
 * val, final and err must be 4-B aligned; nCounters * nOps may be 0.  Performance: a
 * count that is a multiple of 32 (128-B operand rows) with 16-B aligned val
 * and final runs 4 counters per lane at full speed; other counts run 2 or 1
 * per lane, and rows that do not start on a 128-B line cost more lines per
 * load (2^20 + 1 counters x 64 ops: about 93 us, against 55 us for 2^20).
 * Errors: NULL_POINTER, INVALID_VALUE (negative sizes, a misaligned val,
 * final or err, or nCounters above CCB_CNT_BATCH_MAX_COUNTERS). */
#define CCB_CNT_BATCH_MAX_COUNTERS (((int64_t)1 << 31) * 256 - 256)
CCB_API ccbStatus ccb_cnt_notify_batch(const uint32_t* val, const uint8_t* meta,
                                       int64_t nCounters, int32_t nOps, uint32_t* final_,
                                       uint8_t* rel, int32_t nRelRows, int32_t* err,
                                       ccbStream stream);

#ifdef __cplusplus
}
#endif

#endif /* CCB_H */
