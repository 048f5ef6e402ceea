// Test kernels for the in-kernel barrier API of include/ccb_device.h, used
// the way a caller's own kernel would use it: the flag-slot pattern of the
// SYNCALL guide §6.1 (write own slot, barrier, read every member's slot)
// over a 2-D grid, with ccb_syncall_soft, ccb_syncall_soft_ordered,
// ccb_syncall_soft_flat, ccb_syncall_soft_tree, ccb_syncall_soft_xcd,
// ccb_syncall_soft_bounded or ccb_syncall_soft_mix
// (role groups of one leader and 1 or 2 companions; usedCores then counts
// groups), or the split-phase pair ccb_arrive / ccb_await with the kernel's
// own workgroup barriers and work between the two halves.  Test code only: the
// GPU tests compare its output with the oracle's witness rounds.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ccb_device.h"

namespace {

// SplitMix64 output number r * 2^32 + w + 1 for the seed, high 32 bits
// (Steele, Lea & Flood, OOPSLA 2014), the witness of member w in round r.
__device__ uint32_t devapi_witness(uint64_t seed, uint32_t r, uint32_t w)
{
    uint64_t z = seed + 0x9E3779B97F4A7C15ull * ((((uint64_t)r << 32) | w) + 1ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return (uint32_t)((z ^ (z >> 31)) >> 32);
}

template <int kVariant>
__global__ __launch_bounds__(1024) void devapi_rounds(int32_t* ws, uint32_t* slots, uint32_t* out,
                                                      int32_t* status, uint64_t seed,
                                                      int32_t rounds, int32_t usedCores,
                                                      uint32_t maxPoll)
{
    __shared__ uint32_t partial[16];
    const int32_t nGrid = (int32_t)(gridDim.x * gridDim.y * gridDim.z);
    const int32_t w = ccb_block_linear();
    const bool mix = kVariant == 4 || kVariant == 5;  // role groups
    const int32_t ratio = kVariant == 4 ? 1 : 2;
    const int32_t n = mix ? ccb_mix_participants(usedCores, ratio, nGrid)
                          : (usedCores != 0 ? usedCores : nGrid);
    const uint32_t tid = threadIdx.x;
    if (w >= n) {  // non-members never call the barrier
        if (tid == 0) status[w] = 2;
        return;
    }
    int32_t rc = CCB_OK;
    ccb_xcd_team team = {};  // variant 8: this workgroup's XCD state for ws
    for (int32_t r = 0; r < rounds; ++r) {
        uint32_t* row = slots + (size_t)(r & 1) * nGrid;  // two rows suffice for this order
        if (tid == 0) {
            const uint32_t h = devapi_witness(seed, (uint32_t)r, (uint32_t)w);
            if (kVariant == 1 || kVariant == 6) ccb_store_coherent(row + w, h);
            else row[w] = h;
        }
        if (kVariant == 0) rc = ccb_syncall_soft(ws, usedCores);
        else if (kVariant == 1) rc = ccb_syncall_soft_ordered(ws, usedCores);
        else if (kVariant == 2) rc = ccb_syncall_soft_flat(ws, usedCores);
        else if (kVariant == 3) rc = ccb_syncall_soft_bounded(ws, usedCores, maxPoll);
        else if (kVariant == 6) {
            // split phase, ordering-only: every thread's stores are complete,
            // one lane arrives, wave 0 waits, the kernel's own barriers
            // order the rest; the next round's witness is computed while the
            // arrival is in flight
            __shared__ int32_t result;
            __shared__ uint32_t nextWitness;
            ccb_wait_memory();
            __syncthreads();
            if (tid < 64) {
                int32_t before = 0;
                if (tid == 0) {
                    before = ccb_arrive<CCB_STRIPES, CCB_VIS_ORDER>(ws, w);
                    nextWitness = devapi_witness(seed, (uint32_t)(r + 1), (uint32_t)w);
                }
                const int32_t e = ccb_await<CCB_STRIPES, CCB_VIS_ORDER>(
                    ws, n, w, before, maxPoll, ws + CCB_STRIPES * CCB_LINE_WORDS);
                if (tid == 0) result = e;
            }
            __syncthreads();
            rc = result;
            if (rc == CCB_OK && tid == 0 && r + 1 < rounds &&
                nextWitness != devapi_witness(seed, (uint32_t)(r + 1), (uint32_t)w))
                rc = CCB_ERR_INVALID_VALUE;  // the overlapped work went wrong
        } else if (kVariant == 7) rc = ccb_syncall_soft_tree(ws, usedCores);
        else if (kVariant == 8) rc = ccb_syncall_soft_xcd(ws, usedCores, team);
        else rc = ccb_syncall_soft_mix(ws, usedCores, ratio);
        if (rc != CCB_OK) break;
        uint32_t s = 0;
        for (int32_t i = (int32_t)tid; i < n; i += (int32_t)blockDim.x)
            s += (kVariant == 1 || kVariant == 6) ? ccb_load_coherent(row + i) : row[i];
        for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off, 64);
        if ((tid % 64) == 0) partial[tid / 64] = s;
        __syncthreads();
        if (tid == 0) {
            uint32_t t = 0;
            for (uint32_t i = 0; i < blockDim.x / 64; ++i) t += partial[i];
            out[(size_t)r * nGrid + w] = t;
        }
        __syncthreads();
    }
    if (tid == 0) status[w] = rc == CCB_OK ? 1 : 3;
}

}  // namespace

// Launches variant 0..8 cooperatively on a gx x gy grid of `threads`
// threads (a multiple of 64, at most 1024).  slots: 2 * gx * gy uint32;
// out: rounds * gx * gy uint32; status: gx * gy int32.  Returns a hipError_t.
extern "C" int devapi_run(int variant, int32_t* ws, uint32_t* slots, uint32_t* out, int32_t* status,
                          uint64_t seed, int32_t rounds, int32_t gx, int32_t gy, int32_t threads,
                          int32_t usedCores, uint32_t maxPoll, hipStream_t stream)
{
    const bool mix = variant == 4 || variant == 5;
    const int32_t members = mix ? ccb_mix_participants(usedCores, variant == 4 ? 1 : 2, gx * gy)
                                : usedCores;
    if (variant < 0 || variant > 8 || threads < 64 || threads > 1024 || threads % 64 != 0 ||
        gx < 1 || gy < 1 || usedCores < 0 || members > gx * gy)
        return (int)hipErrorInvalidValue;
    // every buffer is written by the kernel: never launch with a missing one
    if (ws == nullptr || slots == nullptr || out == nullptr || status == nullptr)
        return (int)hipErrorInvalidValue;
    void* args[] = {&ws, &slots, &out, &status, &seed, &rounds, &usedCores, &maxPoll};
    const void* const fns[9] = {
        reinterpret_cast<const void*>(&devapi_rounds<0>), reinterpret_cast<const void*>(&devapi_rounds<1>),
        reinterpret_cast<const void*>(&devapi_rounds<2>), reinterpret_cast<const void*>(&devapi_rounds<3>),
        reinterpret_cast<const void*>(&devapi_rounds<4>), reinterpret_cast<const void*>(&devapi_rounds<5>),
        reinterpret_cast<const void*>(&devapi_rounds<6>), reinterpret_cast<const void*>(&devapi_rounds<7>),
        reinterpret_cast<const void*>(&devapi_rounds<8>)};
    const void* fn = fns[variant];
    return (int)hipLaunchCooperativeKernel(fn, dim3(gx, gy), dim3(threads), args, 0, stream);
}
