// ccb_api.hip -- the C entry points of libccb.so: argument validation,
// device checks, co-residency checks, the CntNotify handle table, and the
// launches (kernels live in ccb_kernels.hip).
//
// Sources: "PTO-ISA 跨核同步屏障 SYNCALL 实战指南" (PTO-ISA SYNCALL guide) §4.1
// workspace, §4.2 usedCores, §6.3 co-residency; "CANN Runtime CntNotify（计数型
// 通知）管理接口详解" (CANN Runtime CntNotify interfaces) §4.1-§4.6 for the handle
// calls and their error cases, §6.1 for handle validation.

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <memory>
#include <mutex>
#include <new>

#include "ccb.h"
#include "ccb_internal.h"

namespace {

constexpr int kMaxDevices = 64;

struct DeviceInfo {
    bool probed = false;
    bool gfx950 = false;
    int numCUs = 0;
    int ldsPerCU = 0;
    int ldsPerBlockMax = 0;
    int wallClockKHz = 0;
};

std::mutex g_dev_mu;
DeviceInfo g_dev[kMaxDevices];

// A runtime error is reported through the returned status only: the
// thread's HIP last-error slot is cleared, so a refused launch here does not
// surface later as the error of the caller's next, unrelated launch.
inline ccbStatus hip_failed()
{
    (void)hipGetLastError();
    return CCB_ERR_HIP;
}

inline ccbStatus from_hip(hipError_t e)
{
    if (e == hipSuccess) return CCB_OK;
    (void)hipGetLastError();
    if (e == hipErrorCooperativeLaunchTooLarge) return CCB_ERR_NOT_CORESIDENT;
    return CCB_ERR_HIP;
}

ccbStatus current_device(int* devOut, DeviceInfo* infoOut)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return hip_failed();
    if (dev < 0 || dev >= kMaxDevices) return CCB_ERR_UNSUPPORTED_DEVICE;
    std::lock_guard<std::mutex> lk(g_dev_mu);
    DeviceInfo& d = g_dev[dev];
    if (!d.probed) {
        hipDeviceProp_t p;
        if (hipGetDeviceProperties(&p, dev) != hipSuccess) return hip_failed();
        d.gfx950 = strncmp(p.gcnArchName, "gfx950", 6) == 0;
        d.numCUs = p.multiProcessorCount;
        int v = 0;
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) !=
            hipSuccess)
            return hip_failed();
        d.ldsPerCU = v;
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess)
            return hip_failed();
        d.ldsPerBlockMax = v;
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeWallClockRate, dev) != hipSuccess)
            return hip_failed();
        d.wallClockKHz = v;
        d.probed = true;
    }
    if (!d.gfx950) return CCB_ERR_UNSUPPORTED_DEVICE;
    if (devOut) *devOut = dev;
    if (infoOut) *infoOut = d;
    return CCB_OK;
}

inline bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }


inline bool valid_threads(int32_t threads)
{
    return threads >= 64 && threads <= 1024 && (threads % 64) == 0;
}

// A mode is one counter layout (striped, flat or tree) ORed with one
// visibility (order, full or per-XCD write-back).
inline bool valid_mode(int32_t mode)
{
    const int32_t layout = mode & (CCB_BARRIER_FLAT | CCB_BARRIER_TREE);
    const int32_t vis = mode & ~(CCB_BARRIER_FLAT | CCB_BARRIER_TREE);
    return mode >= 0 && layout != (CCB_BARRIER_FLAT | CCB_BARRIER_TREE) &&
           (vis == CCB_VISIBILITY_ORDER || vis == CCB_VISIBILITY_FULL || vis == CCB_VISIBILITY_XCD);
}

// The barrier shares data through device-coherent accesses (no fences).
inline bool order_only(int32_t mode)
{
    return (mode & (CCB_VISIBILITY_FULL | CCB_VISIBILITY_XCD)) == 0;
}

// Every valid mode, for the register query.
constexpr int32_t kModes[] = {0, 1, 2, 3, CCB_BARRIER_TREE, CCB_BARRIER_TREE | CCB_VISIBILITY_FULL,
                              CCB_VISIBILITY_XCD, CCB_BARRIER_FLAT | CCB_VISIBILITY_XCD,
                              CCB_BARRIER_TREE | CCB_VISIBILITY_XCD};
constexpr int kModeSlots = 16;  // mode values 0..15 index the query table

// Waves per SIMD that a persistent kernel's SGPR allocation allows.  The
// occupancy API counts only the kernel's own SGPRs.  On MI355X each wave also
// holds 16 trap-handler SGPRs, out of 800 per SIMD.  Measured with a spin
// kernel: allocations of 80 / 96 / 112 SGPRs fit 8 / 7 / 6 waves per SIMD,
// where the API reports 8 / 8 / 7.  The allocations are read from
// HW_REG_GPR_ALLOC (SGPR_SIZE, bits 27:24, in 16-register granules minus
// one) by one-workgroup query launches of every persistent kernel variant,
// all at the first persistent launch on a device.  They run on the default
// stream, so the library never creates a stream (a new stream would take one
// of the process's few hardware queues and could change how the caller's
// streams share them); the host waits for them once.
constexpr int kSgprPerSimd = 800;
constexpr int kTrapSgprs = 16;
constexpr int kKernelIds = 6;

struct RegQuery {
    bool done = false;
    int8_t waves[kKernelIds][kModeSlots] = {};
};
std::mutex g_query_mu;
RegQuery g_query[kMaxDevices];

ccbStatus sgpr_waves(int dev, ccb::KernelId id, int32_t mode, int* waves)
{
    std::lock_guard<std::mutex> lk(g_query_mu);
    RegQuery& q = g_query[dev];
    if (!q.done) {
        int32_t* word = nullptr;
        if (ccb::register_query_word(&word) != hipSuccess) return hip_failed();
        for (int k = 0; k < kKernelIds; ++k)
            for (int32_t m : kModes) {
                int32_t alloc = 0;
                if (ccb::launch_register_query((ccb::KernelId)k, m, word, nullptr) != hipSuccess ||
                    hipMemcpy(&alloc, word, sizeof(alloc), hipMemcpyDeviceToHost) != hipSuccess)
                    return hip_failed();
                const int sgprs = ((((uint32_t)alloc >> 24) & 0xF) + 1) * 16;
                const int w = kSgprPerSimd / (sgprs + kTrapSgprs);
                q.waves[k][m] = (int8_t)(w < 1 ? 1 : (w > 8 ? 8 : w));
            }
        q.done = true;
    }
    *waves = q.waves[(int)id][mode];
    return CCB_OK;
}

// Dynamic LDS that keeps at most wgsPerCu workgroups on one CU, and the check
// that nGrid workgroups fit on the device at once (SYNCALL guide §6.3).
ccbStatus plan_persistent(ccb::KernelId id, int32_t mode, int32_t nGrid, int32_t threads,
                          int32_t wgsPerCu, hipStream_t stream, ccb::LaunchShape* ls)
{
    DeviceInfo info;
    int dev = 0;
    ccbStatus st = current_device(&dev, &info);
    if (st != CCB_OK) return st;
    const void* fn = ccb::kernel_ptr(id, mode);
    hipFuncAttributes attr;
    if (hipFuncGetAttributes(&attr, fn) != hipSuccess) return hip_failed();
    size_t lds = 0;
    if (wgsPerCu > 0) {
        long want = (long)info.ldsPerCU / wgsPerCu - (long)attr.sharedSizeBytes;
        long cap = (long)info.ldsPerBlockMax - (long)attr.sharedSizeBytes;
        if (want > cap) want = cap;
        want = want / 1024 * 1024;
        if (want < 0) want = 0;
        lds = (size_t)want;
        if (lds > 0 && hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                                           (int)lds) != hipSuccess)
            return hip_failed();
    }
    int perCU = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&perCU, fn, threads, lds) != hipSuccess)
        return hip_failed();
    // the SGPR limit the occupancy API misses: `waves` per SIMD, 4 SIMDs per
    // CU.  Workgroups of up to 4 waves, or a multiple of 4, spread evenly over
    // the SIMDs.  Other shapes above 4 waves are counted as if each workgroup
    // put ceil(waves / 4) of its waves on one SIMD: measured at their balanced
    // counts, 5-wave workgroups at 6 per CU (8 waves per SIMD) and 6-wave
    // workgroups at 4 per CU (6 per SIMD) did not all become resident.
    int waves = 0;
    if ((st = sgpr_waves(dev, id, mode, &waves)) != CCB_OK) return st;
    const int wpg = (threads + 63) / 64;
    const int bySgpr = (wpg <= 4 || wpg % 4 == 0) ? 4 * waves / wpg : waves / ((wpg + 3) / 4);
    if (bySgpr < perCU) perCU = bySgpr;
    if ((long)perCU * info.numCUs < nGrid) return CCB_ERR_NOT_CORESIDENT;
    ls->fn = fn;
    ls->nGrid = nGrid;
    ls->threads = threads;
    ls->lds = lds;
    ls->stream = stream;
    return CCB_OK;
}

// Held from plan_persistent's setting of a kernel's dynamic-LDS limit (a
// process-wide attribute) until that kernel is enqueued, so that concurrent
// launches of one kernel with different wgsPerCu cannot each launch under the
// other's limit.  Launches only enqueue, so the hold is short.
std::mutex g_launch_mu;

inline uint32_t poll_bound(uint32_t maxPoll) { return maxPoll == 0 ? CCB_SOFT_MAX_POLL : maxPoll; }

// The counters are int32 (SYNCALL guide §4.1): a stripe stays valid while
// its arrivals since the reset plus its participant count stay below 2^31.
// Member m arrives on stripe m mod CCB_STRIPES, so the fullest stripe takes
// ceil(N / 64) arrivals per barrier; the single-counter variant takes N; the
// tree takes ceil(N / 8) on its fullest group counter and min(N, 8) on top.
// Checked for a launch that starts from a zeroed workspace.
inline bool counts_fit(int64_t barriers, int64_t members, int32_t mode)
{
    int64_t perStripe = (members + CCB_STRIPES - 1) / CCB_STRIPES;
    if (mode & CCB_BARRIER_FLAT) perStripe = members;
    if (mode & CCB_BARRIER_TREE) {
        // the fullest group counter, and the top counter (one per group)
        const int64_t group = (members + CCB_TREE_GROUPS - 1) / CCB_TREE_GROUPS;
        const int64_t top = members < CCB_TREE_GROUPS ? members : CCB_TREE_GROUPS;
        perStripe = group > top ? group : top;
    }
    return barriers <= 0 || perStripe <= INT32_MAX / (barriers + 1);
}

// ---------------------------------------------------------------------------
// CntNotify handle table (CntNotify interfaces §4.1, §4.5, §4.6, §6.1).
// A handle value encodes (generation << 20) | (index + 1); it is never
// dereferenced, so a stale or made-up handle is detected, not followed.
//
// Each handle owns one 128-B line of the device pool.  Within the line,
// generation g uses the word pair (count, outcome) at words 2 (g mod 16) and
// 2 (g mod 16) + 1, so kernels still queued for a destroyed handle act on
// their own generation's pair, never on the count of the line's next owner.
// Freed lines go to the back of a FIFO and are reused least recently freed
// first, so a line comes back to a pair it used before only after 16
// generations of reuse.
//
// Cancel tokens: one uint32 per line in coherent pinned host memory.  A wait
// kernel carries the token its line had when it was enqueued and ends with
// CCB_ERR_CANCELLED once the token changes; abort and destroy change it.
// ---------------------------------------------------------------------------
constexpr uint32_t kGenPairs = CCB_LINE_BYTES / 8;

struct CntSlot {
    bool alive = false;
    uint32_t gen = 0;
    int device = -1;
};

struct CntFreeList {
    uint32_t q[CCB_CNT_NOTIFY_POOL];
    uint32_t head = 0, size = 0;
    CntFreeList()
    {
        for (uint32_t i = 0; i < CCB_CNT_NOTIFY_POOL; ++i) q[i] = i;
        size = CCB_CNT_NOTIFY_POOL;
    }
    bool pop(uint32_t* idx)
    {
        if (size == 0) return false;
        *idx = q[head];
        head = (head + 1) % CCB_CNT_NOTIFY_POOL;
        --size;
        return true;
    }
    void push(uint32_t idx)
    {
        q[(head + size) % CCB_CNT_NOTIFY_POOL] = idx;
        ++size;
    }
};

std::mutex g_cnt_mu;
CntSlot g_cnt[CCB_CNT_NOTIFY_POOL];
CntFreeList g_cnt_free;
uint32_t* g_cnt_pool[kMaxDevices] = {nullptr};
uint32_t* g_cnt_cancel[kMaxDevices] = {nullptr};     // host view of the tokens
uint32_t* g_cnt_cancel_dev[kMaxDevices] = {nullptr}; // the same words, device view
constexpr uint32_t kLineWords = CCB_LINE_BYTES / 4;

ccbCntNotify encode_handle(uint32_t idx, uint32_t gen)
{
    const uintptr_t v = ((uintptr_t)gen << 20) | (uintptr_t)(idx + 1);
    return reinterpret_cast<ccbCntNotify>(v);
}

// What a call on a live handle needs.
struct CntRef {
    uint32_t idx;
    uint32_t* pair;         // device: count, then outcome
    const uint32_t* cancelDev;  // device view of the line's cancel token
    uint32_t token;             // its value at the lookup
};

// Looks a handle up.  `kill` also marks the slot free, under the same lock
// as the check, so that of two concurrent destroys of one handle only one
// succeeds.  `cancel` ends the waits enqueued so far on the line (they see
// a new token); it too happens under the lock, before a destroyed line can
// go back to the free list, so that a wait of the line's next owner never
// carries the old token.
ccbStatus resolve(ccbCntNotify h, CntRef* ref, bool kill = false, bool cancel = false)
{
    const uintptr_t v = reinterpret_cast<uintptr_t>(h);
    if (v == 0) return CCB_ERR_INVALID_HANDLE;
    const uintptr_t idx1 = v & ((1u << 20) - 1);
    const uintptr_t gen = v >> 20;
    if (idx1 == 0 || idx1 > CCB_CNT_NOTIFY_POOL) return CCB_ERR_INVALID_HANDLE;
    const uint32_t idx = (uint32_t)(idx1 - 1);
    std::lock_guard<std::mutex> lk(g_cnt_mu);
    CntSlot& s = g_cnt[idx];
    if (!s.alive || s.gen != gen) return CCB_ERR_INVALID_HANDLE;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return hip_failed();
    if (dev != s.device) return CCB_ERR_INVALID_HANDLE;
    if (cancel) __atomic_fetch_add(g_cnt_cancel[s.device] + idx, 1u, __ATOMIC_RELEASE);
    if (kill) {
        s.alive = false;
        g_cnt_free.push(idx);
    }
    if (ref != nullptr) {
        ref->idx = idx;
        ref->pair = g_cnt_pool[s.device] + (size_t)idx * kLineWords + 2 * (s.gen % kGenPairs);
        ref->cancelDev = g_cnt_cancel_dev[s.device] + idx;
        ref->token = __atomic_load_n(g_cnt_cancel[s.device] + idx, __ATOMIC_ACQUIRE);
    }
    return CCB_OK;
}

}  // namespace

// ===========================================================================
// Miscellaneous
// ===========================================================================
extern "C" {

CCB_API const char* ccb_status_string(ccbStatus s)
{
    switch (s) {
    case CCB_OK: return "CCB_OK";
    case CCB_ERR_INVALID_VALUE: return "CCB_ERR_INVALID_VALUE";
    case CCB_ERR_NULL_POINTER: return "CCB_ERR_NULL_POINTER";
    case CCB_ERR_INVALID_HANDLE: return "CCB_ERR_INVALID_HANDLE";
    case CCB_ERR_RESOURCE_EXHAUSTED: return "CCB_ERR_RESOURCE_EXHAUSTED";
    case CCB_ERR_TIMEOUT: return "CCB_ERR_TIMEOUT";
    case CCB_ERR_DEADLOCK: return "CCB_ERR_DEADLOCK";
    case CCB_ERR_NOT_CORESIDENT: return "CCB_ERR_NOT_CORESIDENT";
    case CCB_ERR_UNSUPPORTED_DEVICE: return "CCB_ERR_UNSUPPORTED_DEVICE";
    case CCB_ERR_HIP: return "CCB_ERR_HIP";
    case CCB_ERR_NOT_READY: return "CCB_ERR_NOT_READY";
    case CCB_ERR_CANCELLED: return "CCB_ERR_CANCELLED";
    default: return "CCB_ERR_UNKNOWN";
    }
}

CCB_API int32_t ccb_version(void) { return 100; }

CCB_API ccbStatus ccb_device_info(int32_t* numCUs, int32_t* ldsPerCU, int32_t* wallClockKHz)
{
    DeviceInfo info;
    ccbStatus st = current_device(nullptr, &info);
    if (st != CCB_OK) return st;
    if (numCUs) *numCUs = info.numCUs;
    if (ldsPerCU) *ldsPerCU = info.ldsPerCU;
    if (wallClockKHz) *wallClockKHz = info.wallClockKHz;
    return CCB_OK;
}

// ===========================================================================
// Soft barrier workspace
// ===========================================================================
CCB_API size_t ccb_syncall_workspace_bytes(uint32_t nBarriers)
{
    return ((size_t)nBarriers * CCB_STRIPES + 1) * CCB_LINE_BYTES;
}

CCB_API ccbStatus ccb_syncall_workspace_reset(int32_t* ws, uint32_t nBarriers, ccbStream stream)
{
    if (ws == nullptr) return CCB_ERR_NULL_POINTER;
    if (nBarriers == 0 || nBarriers > (1u << 20) || !aligned(ws, CCB_LINE_BYTES))
        return CCB_ERR_INVALID_VALUE;
    ccbStatus st = current_device(nullptr, nullptr);
    if (st != CCB_OK) return st;
    const int64_t words = ((int64_t)nBarriers * CCB_STRIPES + 1) * kLineWords;
    return from_hip(ccb::launch_fill_zero(ws, words, (hipStream_t)stream));
}

CCB_API ccbStatus ccb_syncall_status(const int32_t* ws, uint32_t nBarriers, int64_t* arrivals,
                                     ccbStream stream)
{
    if (ws == nullptr) return CCB_ERR_NULL_POINTER;
    if (nBarriers == 0 || nBarriers > (1u << 20) || !aligned(ws, CCB_LINE_BYTES))
        return CCB_ERR_INVALID_VALUE;
    ccbStatus st = current_device(nullptr, nullptr);
    if (st != CCB_OK) return st;
    if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess) return hip_failed();
    int32_t errWord = 0;
    if (hipMemcpy(&errWord, ws + (size_t)nBarriers * CCB_STRIPES * kLineWords, sizeof(errWord),
                  hipMemcpyDeviceToHost) != hipSuccess)
        return hip_failed();
    if (arrivals != nullptr) {
        // whole stripe lines, kChunk barriers (64 KiB) per plain copy
        constexpr uint32_t kChunk = 8;
        constexpr size_t kWords = (size_t)kChunk * CCB_STRIPES * kLineWords;
        std::unique_ptr<int32_t[]> buf(new (std::nothrow) int32_t[kWords]);
        if (!buf) return CCB_ERR_RESOURCE_EXHAUSTED;
        for (uint32_t b0 = 0; b0 < nBarriers; b0 += kChunk) {
            const uint32_t nb = nBarriers - b0 < kChunk ? nBarriers - b0 : kChunk;
            if (hipMemcpy(buf.get(), ws + (size_t)b0 * CCB_STRIPES * kLineWords,
                          (size_t)nb * CCB_STRIPES * CCB_LINE_BYTES,
                          hipMemcpyDeviceToHost) != hipSuccess)
                return hip_failed();
            for (uint32_t b = 0; b < nb; ++b) {
                int64_t sum = 0;
                for (uint32_t k = 0; k < CCB_STRIPES; ++k)
                    sum += buf[((size_t)b * CCB_STRIPES + k) * kLineWords];
                arrivals[b0 + b] = sum;
            }
        }
    }
    // the kernels store CCB_ERR_DEADLOCK or CCB_ERR_INVALID_VALUE (a stripe
    // past the int32 range); anything else is reported as a deadlock
    if (errWord == CCB_OK || errWord == CCB_ERR_INVALID_VALUE) return errWord;
    return CCB_ERR_DEADLOCK;
}

// ===========================================================================
// Persistent workloads
// ===========================================================================
CCB_API ccbStatus ccb_run_barrier_only(int32_t* ws, uint32_t* placement, int32_t* wgStatus,
                                       int32_t rounds, int32_t nGrid, int32_t threads,
                                       int32_t usedCores, int32_t wgsPerCu, uint32_t maxPoll,
                                       int32_t mode, ccbStream stream)
{
    if (ws == nullptr) return CCB_ERR_NULL_POINTER;
    if (!aligned(ws, CCB_LINE_BYTES) || rounds < 0 || nGrid < 1 || !valid_threads(threads) ||
        usedCores < 0 || usedCores > nGrid || wgsPerCu < 0 || !valid_mode(mode) ||
        !counts_fit(rounds, usedCores != 0 ? usedCores : nGrid, mode))
        return CCB_ERR_INVALID_VALUE;
    std::lock_guard<std::mutex> lk(g_launch_mu);
    ccb::LaunchShape ls;
    ccbStatus st = plan_persistent(ccb::KernelId::BarrierOnly, mode, nGrid, threads, wgsPerCu,
                                   (hipStream_t)stream, &ls);
    if (st != CCB_OK) return st;
    const int32_t members = usedCores != 0 ? usedCores : nGrid;
    return from_hip(ccb::launch_barrier_only(ls, ws, placement, wgStatus, nullptr, rounds,
                                             members, poll_bound(maxPoll)));
}

CCB_API ccbStatus ccb_bench_barrier_breakdown(int32_t* ws, uint64_t* stamps, int32_t rounds,
                                              int32_t nGrid, int32_t threads, int32_t wgsPerCu,
                                              int32_t mode, ccbStream stream)
{
    if (ws == nullptr || stamps == nullptr) return CCB_ERR_NULL_POINTER;
    if (!aligned(ws, CCB_LINE_BYTES) || !aligned(stamps, 8) || rounds < 1 ||
        rounds > CCB_BREAKDOWN_MAX_ROUNDS || nGrid < 1 || !valid_threads(threads) ||
        wgsPerCu < 0 || !valid_mode(mode) || !counts_fit(rounds, nGrid, mode))
        return CCB_ERR_INVALID_VALUE;
    std::lock_guard<std::mutex> lk(g_launch_mu);
    ccb::LaunchShape ls;
    ccbStatus st = plan_persistent(ccb::KernelId::BarrierStamps, mode, nGrid, threads, wgsPerCu,
                                   (hipStream_t)stream, &ls);
    if (st != CCB_OK) return st;
    return from_hip(ccb::launch_barrier_only(ls, ws, nullptr, nullptr, stamps, rounds, nGrid,
                                             CCB_SOFT_MAX_POLL));
}

CCB_API ccbStatus ccb_run_slot_rounds(int32_t* ws, uint32_t* slots, uint32_t* out,
                                      int32_t* wgStatus, uint64_t seed, int32_t rounds,
                                      int32_t nGrid, int32_t threads, int32_t usedCores,
                                      int32_t wgsPerCu, uint32_t maxPoll, int32_t mode,
                                      ccbStream stream)
{
    if (ws == nullptr || (rounds > 0 && (slots == nullptr || out == nullptr)))
        return CCB_ERR_NULL_POINTER;
    if (!aligned(ws, CCB_LINE_BYTES) || rounds < 0 || nGrid < 1 || !valid_threads(threads) ||
        usedCores < 0 || usedCores > nGrid || wgsPerCu < 0 || !valid_mode(mode) ||
        !counts_fit(rounds, usedCores != 0 ? usedCores : nGrid, mode))
        return CCB_ERR_INVALID_VALUE;
    std::lock_guard<std::mutex> lk(g_launch_mu);
    ccb::LaunchShape ls;
    ccbStatus st = plan_persistent(ccb::KernelId::SlotRounds, mode, nGrid, threads, wgsPerCu,
                                   (hipStream_t)stream, &ls);
    if (st != CCB_OK) return st;
    const int32_t members = usedCores != 0 ? usedCores : nGrid;
    return from_hip(ccb::launch_slot_rounds(ls, ws, slots, out, wgStatus, seed, rounds, members,
                                            poll_bound(maxPoll)));
}

CCB_API ccbStatus ccb_run_grouped_rounds(int32_t* ws, uint32_t* slots, uint32_t* out,
                                         int32_t* wgStatus, uint64_t seed, int32_t rounds,
                                         int32_t nGrid, int32_t threads, int32_t wgsPerCu,
                                         uint32_t maxPoll, int32_t mode, ccbStream stream)
{
    if (ws == nullptr || (rounds > 0 && (slots == nullptr || out == nullptr)))
        return CCB_ERR_NULL_POINTER;
    if (!aligned(ws, CCB_LINE_BYTES) || rounds < 0 || nGrid < 2 || (nGrid % 2) != 0 ||
        !valid_threads(threads) || wgsPerCu < 0 || !valid_mode(mode) ||
        !counts_fit(((int64_t)rounds + 2) / 3, nGrid, mode))  // the mix counter fills first
        return CCB_ERR_INVALID_VALUE;
    std::lock_guard<std::mutex> lk(g_launch_mu);
    ccb::LaunchShape ls;
    ccbStatus st = plan_persistent(ccb::KernelId::GroupedRounds, mode, nGrid, threads, wgsPerCu,
                                   (hipStream_t)stream, &ls);
    if (st != CCB_OK) return st;
    return from_hip(ccb::launch_grouped_rounds(ls, ws, slots, out, wgStatus, nullptr, seed, rounds,
                                               poll_bound(maxPoll)));
}

CCB_API ccbStatus ccb_bench_grouped_timeline(int32_t* ws, uint32_t* slots, uint32_t* out,
                                             uint64_t* stamps, uint64_t seed, int32_t rounds,
                                             int32_t nGrid, int32_t threads, int32_t wgsPerCu,
                                             int32_t mode, ccbStream stream)
{
    if (ws == nullptr || stamps == nullptr || (rounds > 0 && (slots == nullptr || out == nullptr)))
        return CCB_ERR_NULL_POINTER;
    if (!aligned(ws, CCB_LINE_BYTES) || !aligned(stamps, 8) || rounds < 0 || nGrid < 2 ||
        (nGrid % 2) != 0 || !valid_threads(threads) || wgsPerCu < 0 || !valid_mode(mode) ||
        !counts_fit(((int64_t)rounds + 2) / 3, nGrid, mode))
        return CCB_ERR_INVALID_VALUE;
    std::lock_guard<std::mutex> lk(g_launch_mu);
    ccb::LaunchShape ls;
    ccbStatus st = plan_persistent(ccb::KernelId::GroupedStamps, mode, nGrid, threads, wgsPerCu,
                                   (hipStream_t)stream, &ls);
    if (st != CCB_OK) return st;
    return from_hip(ccb::launch_grouped_rounds(ls, ws, slots, out, nullptr, stamps, seed, rounds,
                                               CCB_SOFT_MAX_POLL));
}

CCB_API size_t ccb_stencil_halo_bytes(int64_t n, int32_t threads, int32_t nGrid)
{
    if (n < 1 || !valid_threads(threads) || nGrid < 1) return 0;
    const int64_t chunk = 4 * (int64_t)threads;
    const int64_t nChunks = (n + chunk - 1) / chunk;
    const int64_t kMax = (nChunks + nGrid - 1) / nGrid;
    return (size_t)2 * (size_t)nGrid * (size_t)kMax * 2 * sizeof(int32_t);
}

}  // extern "C"

namespace {

// Argument checks shared by both stencil entry points (everything but the
// scratch arguments).  NULL buffers are checked by the callers first.
bool stencil_args_ok(const int32_t* bufA, const int32_t* bufB, int64_t n, int32_t iters,
                     int32_t nGrid, int32_t threads, int32_t wgsPerCu, int32_t mode)
{
    if (n < 1 || iters < 0 || !aligned(bufA, 16) || !aligned(bufB, 16) || nGrid < 1 ||
        !valid_threads(threads) || wgsPerCu < 0 || !valid_mode(mode) ||
        !counts_fit((int64_t)iters - 1, nGrid, mode))
        return false;
    const uintptr_t a0 = (uintptr_t)bufA, a1 = a0 + (uintptr_t)n * 4;
    const uintptr_t b0 = (uintptr_t)bufB, b1 = b0 + (uintptr_t)n * 4;
    return !(a0 < b1 && b0 < a1);  // the buffers must not overlap
}

}  // namespace

extern "C" {

CCB_API ccbStatus ccb_run_stencil(int32_t* bufA, int32_t* bufB, int64_t n, int32_t iters,
                                  int32_t* ws, int32_t* halo, size_t haloBytes,
                                  uint64_t* timeline, int32_t nGrid, int32_t threads,
                                  int32_t wgsPerCu, uint32_t maxPoll, int32_t mode,
                                  ccbStream stream)
{
    if (bufA == nullptr || bufB == nullptr || ws == nullptr) return CCB_ERR_NULL_POINTER;
    const bool needHalo = valid_mode(mode) && order_only(mode);
    if (needHalo && halo == nullptr) return CCB_ERR_NULL_POINTER;
    if (!stencil_args_ok(bufA, bufB, n, iters, nGrid, threads, wgsPerCu, mode) ||
        !aligned(ws, CCB_LINE_BYTES) || (halo != nullptr && !aligned(halo, 4)) ||
        (timeline != nullptr && !aligned(timeline, 8)))
        return CCB_ERR_INVALID_VALUE;
    if (needHalo && haloBytes < ccb_stencil_halo_bytes(n, threads, nGrid)) return CCB_ERR_INVALID_VALUE;
    std::lock_guard<std::mutex> lk(g_launch_mu);
    ccb::LaunchShape ls;
    ccbStatus st = plan_persistent(ccb::KernelId::Stencil, mode, nGrid, threads, wgsPerCu,
                                   (hipStream_t)stream, &ls);
    if (st != CCB_OK) return st;
    return from_hip(ccb::launch_stencil(ls, bufA, bufB, n, iters, ws, halo, timeline,
                                        poll_bound(maxPoll)));
}

CCB_API ccbStatus ccb_run_stencil_noalloc(int32_t* bufA, int32_t* bufB, int64_t n, int32_t iters,
                                          int32_t* statusOut, int32_t nGrid, int32_t threads,
                                          int32_t wgsPerCu, uint32_t maxPoll, int32_t mode,
                                          ccbStream stream)
{
    if (bufA == nullptr || bufB == nullptr) return CCB_ERR_NULL_POINTER;
    if (!stencil_args_ok(bufA, bufB, n, iters, nGrid, threads, wgsPerCu, mode) ||
        (statusOut != nullptr && !aligned(statusOut, 4)))
        return CCB_ERR_INVALID_VALUE;
    // the scratch: the workspace of one barrier (padded to 256 B), then the
    // halo buffer, which only the ordering-only barrier uses
    const size_t wsBytes = (ccb_syncall_workspace_bytes(1) + 255) / 256 * 256;
    const bool needHalo = order_only(mode);
    const size_t haloBytes = needHalo ? ccb_stencil_halo_bytes(n, threads, nGrid) : 0;
    if (wsBytes + haloBytes > CCB_NOALLOC_SCRATCH_BYTES) return CCB_ERR_INVALID_VALUE;
    int dev = 0;
    ccbStatus st = current_device(&dev, nullptr);
    if (st != CCB_OK) return st;
    int32_t* scratch = nullptr;
    if (ccb::noalloc_scratch(dev, &scratch) != hipSuccess) return hip_failed();
    int32_t* ws = scratch;
    int32_t* halo = needHalo ? scratch + wsBytes / 4 : nullptr;
    std::lock_guard<std::mutex> lk(g_launch_mu);
    ccb::LaunchShape ls;
    st = plan_persistent(ccb::KernelId::Stencil, mode, nGrid, threads, wgsPerCu,
                         (hipStream_t)stream, &ls);
    if (st != CCB_OK) return st;
    // the scratch keeps the previous call's contents: the stripes and the
    // error word must start at zero (the halo is written before it is read)
    const int64_t wsWords = (int64_t)ccb_syncall_workspace_bytes(1) / 4;
    if ((st = from_hip(ccb::launch_fill_zero(ws, wsWords, (hipStream_t)stream))) != CCB_OK)
        return st;
    if ((st = from_hip(ccb::launch_stencil(ls, bufA, bufB, n, iters, ws, halo, nullptr,
                                           poll_bound(maxPoll)))) != CCB_OK)
        return st;
    if (statusOut == nullptr) return CCB_OK;
    return from_hip(ccb::launch_copy_word(ws + (size_t)CCB_STRIPES * kLineWords, statusOut,
                                          (hipStream_t)stream));
}

// ===========================================================================
// Floor microbenchmarks
// ===========================================================================
CCB_API ccbStatus ccb_bench_atomic_chain(int32_t* line, uint64_t* ticksOut, int32_t iters,
                                         int32_t fenced, int32_t kind, ccbStream stream)
{
    if (line == nullptr || ticksOut == nullptr) return CCB_ERR_NULL_POINTER;
    if (iters < 1 || (kind != 0 && kind != 1) || !aligned(line, CCB_LINE_BYTES))
        return CCB_ERR_INVALID_VALUE;
    ccbStatus st = current_device(nullptr, nullptr);
    if (st != CCB_OK) return st;
    return from_hip(ccb::launch_atomic_chain(line, ticksOut, iters, fenced, kind,
                                             (hipStream_t)stream));
}

CCB_API ccbStatus ccb_bench_atomic_contended(int32_t* line, uint64_t* ticksOut, int32_t iters,
                                             int32_t nGrid, ccbStream stream)
{
    if (line == nullptr || ticksOut == nullptr) return CCB_ERR_NULL_POINTER;
    if (iters < 1 || nGrid < 1 || !aligned(line, CCB_LINE_BYTES)) return CCB_ERR_INVALID_VALUE;
    DeviceInfo info;
    ccbStatus st = current_device(nullptr, &info);
    if (st != CCB_OK) return st;
    return from_hip(ccb::launch_atomic_contended(line, ticksOut, iters, nGrid,
                                                 (hipStream_t)stream));
}

CCB_API ccbStatus ccb_bench_notify_pingpong(int32_t* lines, uint64_t* ticksOut, int32_t iters,
                                           int32_t peer, uint32_t maxPoll, int32_t* err,
                                           ccbStream stream)
{
    if (lines == nullptr || ticksOut == nullptr || err == nullptr) return CCB_ERR_NULL_POINTER;
    if (iters < 1 || peer < 1 || peer > 255 || !aligned(lines, CCB_LINE_BYTES) ||
        !aligned(ticksOut, 8) || !aligned(err, 4))
        return CCB_ERR_INVALID_VALUE;
    ccbStatus st = current_device(nullptr, nullptr);
    if (st != CCB_OK) return st;
    return from_hip(ccb::launch_notify_pingpong(lines, ticksOut, iters, peer, poll_bound(maxPoll),
                                                err, (hipStream_t)stream));
}

CCB_API size_t ccb_bench_fence_placement_bytes(int32_t nGrid)
{
    if (nGrid < 1) return 0;
    return (size_t)(CCB_STRIPES + 17 + nGrid) * CCB_LINE_BYTES;
}

CCB_API ccbStatus ccb_bench_fence_placement(int32_t* scratch, size_t scratchBytes, int32_t* stale,
                                            int32_t rounds, int32_t nGrid, int32_t threads,
                                            int32_t variant, ccbStream stream)
{
    if (scratch == nullptr || stale == nullptr) return CCB_ERR_NULL_POINTER;
    DeviceInfo info;
    if (rounds < 1 || nGrid < 1 || !valid_threads(threads) || variant < 0 || variant > 5 ||
        !aligned(scratch, CCB_LINE_BYTES) || !aligned(stale, 4) ||
        scratchBytes < ccb_bench_fence_placement_bytes(nGrid) ||
        !counts_fit((int64_t)rounds + 1, nGrid, 0))
        return CCB_ERR_INVALID_VALUE;
    ccbStatus st = current_device(nullptr, &info);
    if (st != CCB_OK) return st;
    if (nGrid > info.numCUs) return CCB_ERR_NOT_CORESIDENT;  // one workgroup per CU at most
    const int64_t words = (int64_t)ccb_bench_fence_placement_bytes(nGrid) / 4;
    if ((st = from_hip(ccb::launch_fill_zero(scratch, words, (hipStream_t)stream))) != CCB_OK)
        return st;
    return from_hip(ccb::launch_fence_placement(scratch, stale, rounds, nGrid, threads, variant,
                                                CCB_SOFT_MAX_POLL, (hipStream_t)stream));
}

CCB_API ccbStatus ccb_bench_hip_grid_sync(int32_t rounds, int32_t nGrid, int32_t threads,
                                          int32_t* doneOut, ccbStream stream)
{
    if (doneOut == nullptr) return CCB_ERR_NULL_POINTER;
    if (rounds < 1 || nGrid < 1 || !valid_threads(threads)) return CCB_ERR_INVALID_VALUE;
    DeviceInfo info;
    ccbStatus st = current_device(nullptr, &info);
    if (st != CCB_OK) return st;
    return from_hip(ccb::launch_hip_grid_sync(rounds, nGrid, threads, doneOut, info.numCUs,
                                              (hipStream_t)stream));
}

CCB_API ccbStatus ccb_bench_copy(void* dst, const void* src, int64_t nBytes, ccbStream stream)
{
    if (dst == nullptr || src == nullptr) return CCB_ERR_NULL_POINTER;
    if (nBytes < 0 || (nBytes % 16) != 0 || !aligned(dst, 16) || !aligned(src, 16))
        return CCB_ERR_INVALID_VALUE;
    DeviceInfo info;
    ccbStatus st = current_device(nullptr, &info);
    if (st != CCB_OK) return st;
    if (nBytes == 0) return CCB_OK;
    return from_hip(ccb::launch_copy(static_cast<int4*>(dst), static_cast<const int4*>(src),
                                     nBytes / 16, info.numCUs * 4, (hipStream_t)stream));
}

// ===========================================================================
// CntNotify
// ===========================================================================
CCB_API ccbStatus ccb_cnt_notify_create(ccbCntNotify* out, uint64_t flag)
{
    if (out == nullptr) return CCB_ERR_NULL_POINTER;
    if (flag != 0) return CCB_ERR_INVALID_VALUE;  // the flag is reserved (§4.1)
    int dev = 0;
    ccbStatus st = current_device(&dev, nullptr);
    if (st != CCB_OK) return st;
    std::lock_guard<std::mutex> lk(g_cnt_mu);
    if (g_cnt_pool[dev] == nullptr) {
        void* p = nullptr;
        if (hipMalloc(&p, (size_t)CCB_CNT_NOTIFY_POOL * CCB_LINE_BYTES) != hipSuccess)
            return hip_failed();
        g_cnt_pool[dev] = static_cast<uint32_t*>(p);
    }
    if (g_cnt_cancel[dev] == nullptr) {
        // coherent: the device's system-scope reads see the host's stores
        void* hp = nullptr;
        void* dp = nullptr;
        if (hipHostMalloc(&hp, (size_t)CCB_CNT_NOTIFY_POOL * sizeof(uint32_t),
                          hipHostMallocCoherent | hipHostMallocMapped) != hipSuccess)
            return hip_failed();
        memset(hp, 0, (size_t)CCB_CNT_NOTIFY_POOL * sizeof(uint32_t));
        if (hipHostGetDevicePointer(&dp, hp, 0) != hipSuccess) {
            (void)hipHostFree(hp);
            return hip_failed();
        }
        g_cnt_cancel[dev] = static_cast<uint32_t*>(hp);
        g_cnt_cancel_dev[dev] = static_cast<uint32_t*>(dp);
    }
    uint32_t idx = 0;
    if (!g_cnt_free.pop(&idx)) return CCB_ERR_RESOURCE_EXHAUSTED;
    CntSlot& s = g_cnt[idx];
    uint32_t gen = (s.gen + 1) & 0xFFFFFu;
    if (gen == 0) gen = 1;
    // count 0, no wait completed yet, in this generation's pair
    const uint32_t init[2] = {0u, (uint32_t)CCB_ERR_NOT_READY};
    if (hipMemcpy(g_cnt_pool[dev] + (size_t)idx * kLineWords + 2 * (gen % kGenPairs), init,
                  sizeof(init), hipMemcpyHostToDevice) != hipSuccess) {
        g_cnt_free.push(idx);
        return hip_failed();
    }
    s.alive = true;
    s.gen = gen;
    s.device = dev;
    *out = encode_handle(idx, gen);
    return CCB_OK;
}

CCB_API ccbStatus ccb_cnt_notify_record(ccbCntNotify h, ccbStream stream,
                                        const ccbCntRecordInfo* info)
{
    CntRef ref;
    ccbStatus st = resolve(h, &ref);
    if (st != CCB_OK) return st;
    if (info == nullptr) return CCB_ERR_NULL_POINTER;
    const int32_t m = info->mode;
    if (!(m == CCB_CNT_RECORD_SET_VALUE || m == CCB_CNT_RECORD_ADD || m == CCB_CNT_RECORD_BIT_OR ||
          m == CCB_CNT_RECORD_BIT_AND))
        return CCB_ERR_INVALID_VALUE;
    return from_hip(ccb::launch_cnt_record(ref.pair, m, info->value, (hipStream_t)stream));
}

CCB_API ccbStatus ccb_cnt_notify_wait(ccbCntNotify h, ccbStream stream, const ccbCntWaitInfo* info)
{
    CntRef ref;
    ccbStatus st = resolve(h, &ref);
    if (st != CCB_OK) return st;
    if (info == nullptr) return CCB_ERR_NULL_POINTER;
    if (info->mode < CCB_CNT_WAIT_LESS || info->mode > CCB_CNT_WAIT_EQUAL_WITH_BITMASK ||
        info->isClear > 1 || info->rev[0] != 0 || info->rev[1] != 0 || info->rev[2] != 0)
        return CCB_ERR_INVALID_VALUE;
    DeviceInfo dinfo;
    st = current_device(nullptr, &dinfo);
    if (st != CCB_OK) return st;
    const uint64_t ticks = (uint64_t)info->timeout * (uint64_t)dinfo.wallClockKHz * 1000ull;
    return from_hip(ccb::launch_cnt_wait(ref.pair, info->mode, info->value, info->isClear, ticks,
                                         ref.cancelDev, ref.token, (hipStream_t)stream));
}

CCB_API ccbStatus ccb_cnt_notify_reset(ccbCntNotify h, ccbStream stream)
{
    CntRef ref;
    ccbStatus st = resolve(h, &ref);
    if (st != CCB_OK) return st;
    return from_hip(ccb::launch_cnt_reset(ref.pair, (hipStream_t)stream));
}

CCB_API ccbStatus ccb_cnt_notify_get_id(ccbCntNotify h, uint32_t* id)
{
    CntRef ref;
    ccbStatus st = resolve(h, &ref);
    if (st != CCB_OK) return st;
    if (id == nullptr) return CCB_ERR_NULL_POINTER;
    *id = ref.idx;
    return CCB_OK;
}

CCB_API ccbStatus ccb_cnt_notify_abort(ccbCntNotify h)
{
    return resolve(h, nullptr, false, true);
}

CCB_API ccbStatus ccb_cnt_notify_destroy(ccbCntNotify h)
{
    // a wait still queued for the handle ends instead of spinning
    return resolve(h, nullptr, true, true);
}

CCB_API ccbStatus ccb_cnt_notify_query(ccbCntNotify h, uint32_t* value, ccbStatus* lastWait,
                                       ccbStream stream)
{
    CntRef ref;
    ccbStatus st = resolve(h, &ref);
    if (st != CCB_OK) return st;
    if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess) return hip_failed();
    uint32_t words[2] = {0, 0};
    if (hipMemcpy(words, ref.pair, sizeof(words), hipMemcpyDeviceToHost) != hipSuccess)
        return hip_failed();
    if (value) *value = words[0];
    if (lastWait) *lastWait = (ccbStatus)words[1];
    return CCB_OK;
}

CCB_API ccbStatus ccb_cnt_notify_batch(const uint32_t* val, const uint8_t* meta,
                                       int64_t nCounters, int32_t nOps, uint32_t* final_,
                                       uint8_t* rel, int32_t nRelRows, int32_t* err,
                                       ccbStream stream)
{
    // one counter per thread at most 256 per workgroup: the grid holds < 2^31 workgroups
    if (nCounters < 0 || nOps < 0 || nRelRows < 0 || nCounters > CCB_CNT_BATCH_MAX_COUNTERS)
        return CCB_ERR_INVALID_VALUE;
    if (nCounters == 0) return CCB_OK;
    if (final_ == nullptr) return CCB_ERR_NULL_POINTER;
    if (nOps > 0 && (val == nullptr || meta == nullptr)) return CCB_ERR_NULL_POINTER;
    if (nRelRows > 0 && rel == nullptr) return CCB_ERR_NULL_POINTER;
    if (!aligned(final_, 4) || (val != nullptr && !aligned(val, 4)) ||
        (err != nullptr && !aligned(err, 4)))
        return CCB_ERR_INVALID_VALUE;
    ccbStatus st = current_device(nullptr, nullptr);
    if (st != CCB_OK) return st;
    // C adjacent counters per thread: 4 when the count and the arrays allow
    // 16-B operand and 4-B op-code accesses, else 2, else 1
    auto fits = [&](int C) {
        return (nCounters % C) == 0 && (val == nullptr || aligned(val, 4 * C)) &&
               (meta == nullptr || aligned(meta, C)) && aligned(final_, 4 * C) &&
               (rel == nullptr || aligned(rel, C));
    };
    const int perThread = fits(4) ? 4 : (fits(2) ? 2 : 1);
    return from_hip(ccb::launch_cnt_batch(val, meta, nCounters, nOps, final_, rel, nRelRows, err,
                                          perThread, (hipStream_t)stream));
}

}  // extern "C"
