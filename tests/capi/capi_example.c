/*
 * A C11 consumer of libccb.so that uses only include/ccb.h and the HIP
 * runtime's C API (no C++, no Python): the producer/consumer pattern of
 * "CANN Runtime CntNotify（计数型通知）管理接口详解" §5 (one stream records
 * ADD 1, another waits for a count of at least 1 and clears it on release),
 * then one launch of the soft barrier (8 workgroups, 100 rounds) whose
 * arrivals are read back.  It is built as a small shared object so that a
 * test can call it in-process; the one entry point returns 0 on success and
 * writes a one-line report into msg.
 */
#include <stdint.h>
#include <stdio.h>

#include <hip/hip_runtime_api.h>

#include "ccb.h"

#define CCB_TRY(call)                                                                 \
    do {                                                                              \
        ccbStatus st_ = (call);                                                       \
        if (st_ != CCB_OK) {                                                          \
            snprintf(msg, (size_t)msgLen, "%s: %s", #call, ccb_status_string(st_));  \
            return 1;                                                                 \
        }                                                                             \
    } while (0)

#define HIP_TRY(call)                                                                 \
    do {                                                                              \
        hipError_t e_ = (call);                                                       \
        if (e_ != hipSuccess) {                                                       \
            snprintf(msg, (size_t)msgLen, "%s: %s", #call, hipGetErrorString(e_));   \
            return 1;                                                                 \
        }                                                                             \
    } while (0)

__attribute__((visibility("default"))) int ccb_capi_example(char* msg, int msgLen)
{
    hipStream_t producer, consumer;
    HIP_TRY(hipStreamCreate(&producer));
    HIP_TRY(hipStreamCreate(&consumer));

    /* CntNotify: record on the producer stream, wait on the consumer stream */
    ccbCntNotify h;
    CCB_TRY(ccb_cnt_notify_create(&h, 0));
    const ccbCntRecordInfo rec = {CCB_CNT_RECORD_ADD, 1u};
    const ccbCntWaitInfo wait = {CCB_CNT_WAIT_BIGGER_OR_EQUAL, 1u, 10u, 1u, {0, 0, 0}};
    CCB_TRY(ccb_cnt_notify_record(h, producer, &rec));
    CCB_TRY(ccb_cnt_notify_wait(h, consumer, &wait));
    uint32_t value = 12345u;
    ccbStatus last = -1;
    CCB_TRY(ccb_cnt_notify_query(h, &value, &last, consumer));
    uint32_t id = 0;
    CCB_TRY(ccb_cnt_notify_get_id(h, &id));
    CCB_TRY(ccb_cnt_notify_destroy(h));
    if (value != 0u || last != CCB_OK) {
        snprintf(msg, (size_t)msgLen, "cntnotify: count %u, last wait %d", value, (int)last);
        return 1;
    }

    /* soft barrier: 8 workgroups x 64 threads, 100 rounds, every workgroup a member */
    int32_t* ws = NULL;
    HIP_TRY(hipMalloc((void**)&ws, ccb_syncall_workspace_bytes(1)));
    CCB_TRY(ccb_syncall_workspace_reset(ws, 1, consumer));
    CCB_TRY(ccb_run_barrier_only(ws, NULL, NULL, 100, 8, 64, 0, 0, 0,
                                 CCB_BARRIER_STRIPED | CCB_VISIBILITY_ORDER, consumer));
    int64_t arrivals = 0;
    CCB_TRY(ccb_syncall_status(ws, 1, &arrivals, consumer));
    HIP_TRY(hipFree(ws));
    HIP_TRY(hipStreamDestroy(producer));
    HIP_TRY(hipStreamDestroy(consumer));
    if (arrivals != 800) {
        snprintf(msg, (size_t)msgLen, "barrier: %lld arrivals, expected 800", (long long)arrivals);
        return 1;
    }
    snprintf(msg, (size_t)msgLen, "released and cleared (id %u); 800 arrivals", id);
    return 0;
}
