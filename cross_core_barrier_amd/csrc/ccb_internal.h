// ccb_internal.h -- private interface between the C entry points
// (ccb_api.hip) and the kernels (ccb_kernels.hip).  Not installed.
#ifndef CCB_INTERNAL_H
#define CCB_INTERNAL_H

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ccb {

// Tuning constants of the kernels.
// Stencil: non-temporal loads of the input (+7%); plain stores of the output
// (non-temporal stores measured 4% slower, in both barrier variants).
constexpr bool kStencilNT = false;
constexpr bool kStencilNTLoad = true;
// Stencil: full chunks are taken kStencilGroup at a time, all of the
// group's loads issued before its first stores.
constexpr int kStencilGroup = 2;
constexpr int kCntUnroll = 1;      // ops per register set in the batch engine's two-set pipeline
constexpr bool kCntNTLoad = true;   // non-temporal loads of the op stream (read once)

enum class KernelId { BarrierOnly, SlotRounds, GroupedRounds, Stencil, BarrierStamps, GroupedStamps };

struct LaunchShape {
    const void* fn;  // the kernel instance
    int nGrid;
    int threads;
    size_t lds;  // dynamic LDS bytes per workgroup
    hipStream_t stream;
};

const void* kernel_ptr(KernelId id, int32_t mode);

// One workgroup of the kernel stores its waves' HW_REG_GPR_ALLOC in *out.
hipError_t launch_register_query(KernelId id, int32_t mode, int32_t* out, hipStream_t s);
// Device address (on the current device) of the word the query writes.
hipError_t register_query_word(int32_t** out);

hipError_t launch_barrier_only(const LaunchShape& ls, int32_t* ws, uint32_t* placement,
                               int32_t* wgStatus, uint64_t* stamps, int32_t rounds,
                               int32_t nMembers, uint32_t maxPoll);
hipError_t launch_slot_rounds(const LaunchShape& ls, int32_t* ws, uint32_t* slots, uint32_t* out,
                              int32_t* wgStatus, uint64_t seed, int32_t rounds, int32_t nMembers,
                              uint32_t maxPoll);
hipError_t launch_grouped_rounds(const LaunchShape& ls, int32_t* ws, uint32_t* slots,
                                 uint32_t* out, int32_t* wgStatus, uint64_t* stamps, uint64_t seed,
                                 int32_t rounds, uint32_t maxPoll);
hipError_t launch_stencil(const LaunchShape& ls, int32_t* bufA, int32_t* bufB, int64_t n,
                          int32_t iters, int32_t* ws, int32_t* halo, uint64_t* timeline,
                          uint32_t maxPoll);
hipError_t launch_cnt_batch(const uint32_t* val, const uint8_t* meta, int64_t nCounters,
                            int32_t nOps, uint32_t* finalOut, uint8_t* rel, int32_t nRelRows,
                            int32_t* err, int perThread, hipStream_t s);
hipError_t launch_cnt_record(uint32_t* line, int32_t mode, uint32_t value, hipStream_t s);
hipError_t launch_cnt_wait(uint32_t* line, int32_t mode, uint32_t value, int32_t isClear,
                           uint64_t timeoutTicks, const uint32_t* cancel, uint32_t token,
                           hipStream_t s);
hipError_t launch_cnt_reset(uint32_t* line, hipStream_t s);
hipError_t launch_fill_zero(int32_t* p, int64_t nWords, hipStream_t s);
hipError_t launch_copy_word(const int32_t* src, int32_t* dst, hipStream_t s);
// Device address of the allocation-free entry point's scratch on device
// `dev` (which must be current), looked up on the first call per device.
hipError_t noalloc_scratch(int dev, int32_t** out);
hipError_t launch_atomic_chain(int32_t* line, uint64_t* ticks, int32_t iters, int32_t fenced,
                               int32_t kind, hipStream_t s);
hipError_t launch_atomic_contended(int32_t* line, uint64_t* ticks, int32_t iters, int32_t nGrid,
                                   hipStream_t s);
hipError_t launch_notify_pingpong(int32_t* lines, uint64_t* ticks, int32_t iters, int32_t peer,
                                  uint32_t maxPoll, int32_t* err, hipStream_t s);
hipError_t launch_hip_grid_sync(int32_t rounds, int32_t nGrid, int32_t threads, int32_t* done,
                                int numCUs, hipStream_t s);
hipError_t launch_copy(int4* dst, const int4* src, int64_t n16, int nBlocks, hipStream_t s);
hipError_t launch_fence_placement(int32_t* scratch, int32_t* stale, int32_t rounds, int32_t nGrid,
                                  int32_t threads, int32_t variant, uint32_t maxPoll, hipStream_t s);

}  // namespace ccb

#endif  // CCB_INTERNAL_H
