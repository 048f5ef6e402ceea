/*
 * A C11 consumer of libccb.so that uses only include/ccb.h and the HIP
 * runtime's C API (no C++, no Python): the producer/consumer pattern of
 * "CANN Runtime CntNotify（计数型通知）管理接口详解" §5 (one stream records
 * ADD 1, another waits for a count of at least 1 and clears it on release),
 * then one launch of the soft barrier (8 workgroups, 100 rounds) whose
 * arrivals are read back, one batched-engine launch and one stencil launch,
 * each with a result fixed by construction.  It is built as a small shared object so that a
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
    /* the same rounds on the two-level arrival tree */
    int64_t treeArrivals = 0;
    CCB_TRY(ccb_syncall_workspace_reset(ws, 1, consumer));
    CCB_TRY(ccb_run_barrier_only(ws, NULL, NULL, 100, 8, 64, 0, 0, 0,
                                 CCB_BARRIER_TREE | CCB_VISIBILITY_ORDER, consumer));
    CCB_TRY(ccb_syncall_status(ws, 1, &treeArrivals, consumer));
    /* and with full visibility through one L2 write-back per XCD */
    int64_t xcdArrivals = 0;
    CCB_TRY(ccb_syncall_workspace_reset(ws, 1, consumer));
    CCB_TRY(ccb_run_barrier_only(ws, NULL, NULL, 100, 8, 64, 0, 0, 0,
                                 CCB_BARRIER_STRIPED | CCB_VISIBILITY_XCD, consumer));
    CCB_TRY(ccb_syncall_status(ws, 1, &xcdArrivals, consumer));
    HIP_TRY(hipFree(ws));
    if (treeArrivals != 800 || xcdArrivals != 800) {
        snprintf(msg, (size_t)msgLen, "tree / per-XCD barrier: %lld / %lld arrivals, expected 800",
                 (long long)treeArrivals, (long long)xcdArrivals);
        return 1;
    }

    /* a wait nothing will satisfy, ended from the host */
    ccbCntNotify h2;
    CCB_TRY(ccb_cnt_notify_create(&h2, 0));
    ccbCntWaitInfo never = {CCB_CNT_WAIT_BIGGER_OR_EQUAL, 1, 5 /* s */, 0, {0, 0, 0}};
    CCB_TRY(ccb_cnt_notify_wait(h2, consumer, &never));
    CCB_TRY(ccb_cnt_notify_abort(h2));
    ccbStatus aborted = CCB_OK;
    CCB_TRY(ccb_cnt_notify_query(h2, NULL, &aborted, consumer));
    CCB_TRY(ccb_cnt_notify_destroy(h2));
    if (aborted != CCB_ERR_CANCELLED) {
        snprintf(msg, (size_t)msgLen, "abort: last wait %d, expected CANCELLED", (int)aborted);
        return 1;
    }
    HIP_TRY(hipStreamDestroy(producer));
    HIP_TRY(hipStreamDestroy(consumer));
    if (arrivals != 800) {
        snprintf(msg, (size_t)msgLen, "barrier: %lld arrivals, expected 800", (long long)arrivals);
        return 1;
    }

    /* batched engine: 1024 counters, ops 0-6 record ADD 1, op 7 waits for
     * GE 7 with clear -> every counter is released and ends at 0 */
    enum { NC = 1024, NOPS = 8 };
    static uint32_t hval[NOPS * NC];
    static uint8_t hmeta[NOPS * NC];
    for (int k = 0; k < NOPS; ++k)
        for (int c = 0; c < NC; ++c) {
            hval[k * NC + c] = k < 7 ? 1u : 7u;
            hmeta[k * NC + c] = (uint8_t)(k < 7 ? CCB_CNT_RECORD_ADD
                                                : (0x80 | 0x08 | CCB_CNT_WAIT_BIGGER_OR_EQUAL));
        }
    uint32_t *dval = NULL, *dfinal = NULL;
    uint8_t *dmeta = NULL, *drel = NULL;
    int32_t* derr = NULL;
    HIP_TRY(hipMalloc((void**)&dval, sizeof(hval)));
    HIP_TRY(hipMalloc((void**)&dmeta, sizeof(hmeta)));
    HIP_TRY(hipMalloc((void**)&dfinal, NC * sizeof(uint32_t)));
    HIP_TRY(hipMalloc((void**)&drel, NC));
    HIP_TRY(hipMalloc((void**)&derr, sizeof(int32_t)));
    HIP_TRY(hipMemcpy(dval, hval, sizeof(hval), hipMemcpyHostToDevice));
    HIP_TRY(hipMemcpy(dmeta, hmeta, sizeof(hmeta), hipMemcpyHostToDevice));
    HIP_TRY(hipMemset(derr, 0, sizeof(int32_t)));
    CCB_TRY(ccb_cnt_notify_batch(dval, dmeta, NC, NOPS, dfinal, drel, 1, derr, NULL));
    static uint32_t hfinal[NC];
    static uint8_t hrel[NC];
    int32_t herr = -1;
    HIP_TRY(hipMemcpy(hfinal, dfinal, sizeof(hfinal), hipMemcpyDeviceToHost));
    HIP_TRY(hipMemcpy(hrel, drel, sizeof(hrel), hipMemcpyDeviceToHost));
    HIP_TRY(hipMemcpy(&herr, derr, sizeof(herr), hipMemcpyDeviceToHost));
    for (int c = 0; c < NC; ++c)
        if (hfinal[c] != 0u || hrel[c] != 1u || herr != 0) {
            snprintf(msg, (size_t)msgLen, "batch: counter %d final %u released %u err %d", c,
                     hfinal[c], (unsigned)hrel[c], (int)herr);
            return 1;
        }
    HIP_TRY(hipFree(dval));
    HIP_TRY(hipFree(dmeta));
    HIP_TRY(hipFree(dfinal));
    HIP_TRY(hipFree(drel));
    HIP_TRY(hipFree(derr));

    /* stencil: a constant array is a fixed point of the clamped 3-point average */
    enum { N = 5000, ITERS = 3, GRID = 4, THREADS = 64 };
    static int32_t hx[N];
    for (int i = 0; i < N; ++i) hx[i] = 777;
    int32_t *da = NULL, *db = NULL, *dws = NULL, *dhalo = NULL;
    const size_t haloBytes = ccb_stencil_halo_bytes(N, THREADS, GRID);
    HIP_TRY(hipMalloc((void**)&da, sizeof(hx)));
    HIP_TRY(hipMalloc((void**)&db, sizeof(hx)));
    HIP_TRY(hipMalloc((void**)&dws, ccb_syncall_workspace_bytes(1)));
    HIP_TRY(hipMalloc((void**)&dhalo, haloBytes));
    HIP_TRY(hipMemcpy(da, hx, sizeof(hx), hipMemcpyHostToDevice));
    CCB_TRY(ccb_syncall_workspace_reset(dws, 1, NULL));
    CCB_TRY(ccb_run_stencil(da, db, N, ITERS, dws, dhalo, haloBytes, NULL, GRID, THREADS, 0, 0,
                            CCB_BARRIER_STRIPED | CCB_VISIBILITY_ORDER, NULL));
    CCB_TRY(ccb_syncall_status(dws, 1, NULL, NULL));
    static int32_t hy[N];
    /* an odd iteration count leaves the result in the second buffer */
    HIP_TRY(hipMemcpy(hy, db, sizeof(hy), hipMemcpyDeviceToHost));
    for (int i = 0; i < N; ++i)
        if (hy[i] != 777) {
            snprintf(msg, (size_t)msgLen, "stencil: element %d is %d", i, (int)hy[i]);
            return 1;
        }
    /* the same stencil through the entry point that allocates nothing: no
     * workspace, no halo; its outcome lands in a device word */
    int32_t* dstatus = NULL;
    HIP_TRY(hipMalloc((void**)&dstatus, sizeof(int32_t)));
    HIP_TRY(hipMemcpy(da, hx, sizeof(hx), hipMemcpyHostToDevice));
    CCB_TRY(ccb_run_stencil_noalloc(da, db, N, ITERS, dstatus, GRID, THREADS, 0, 0,
                                    CCB_BARRIER_STRIPED | CCB_VISIBILITY_ORDER, NULL));
    int32_t hstatus = -1;
    HIP_TRY(hipMemcpy(&hstatus, dstatus, sizeof(hstatus),
                      hipMemcpyDeviceToHost));
    HIP_TRY(hipMemcpy(hy, db, sizeof(hy), hipMemcpyDeviceToHost));
    for (int i = 0; i < N; ++i)
        if (hy[i] != 777 || hstatus != CCB_OK) {
            snprintf(msg, (size_t)msgLen, "stencil without allocation: element %d is %d, status %d",
                     i, (int)hy[i], (int)hstatus);
            return 1;
        }
    HIP_TRY(hipFree(dstatus));
    HIP_TRY(hipFree(da));
    HIP_TRY(hipFree(db));
    HIP_TRY(hipFree(dws));
    HIP_TRY(hipFree(dhalo));

    snprintf(msg, (size_t)msgLen,
             "released and cleared (id %u); 800 arrivals (stripes and tree); a wait aborted; "
             "batch of %d released; stencil fixed point, also without allocation",
             id, NC);
    return 0;
}
