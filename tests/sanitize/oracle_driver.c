/* Drives the C oracle (oracle/ccb_oracle.c, oracle/host_barrier.c) on small
 * inputs so that it can run under AddressSanitizer, UndefinedBehaviorSanitizer
 * and ThreadSanitizer.  Each step checks a property that holds by
 * construction (the final counter, equal sums across members, the stencil's
 * range, the host-thread barrier's sums against the hashes).  Exit status 0
 * means every check held; the sanitizers abort on their own findings.
 * Usage: oracle_driver [all|threads]   ("threads": the host barrier only). */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

uint32_t ccbo_witness_hash(uint64_t seed, uint32_t round, uint32_t wg);
int32_t ccbo_epoch_target(int32_t before, int32_t n);
int32_t ccbo_participants(int32_t usedCores, int32_t nLaunched);
int32_t ccbo_mix_participants(int32_t groups, int32_t ratio, int32_t nLaunched);
int ccbo_slot_rounds(uint64_t seed, int32_t rounds, int32_t nGrid, int32_t usedCores,
                     uint32_t* out, int32_t* status, int32_t* counter);
int ccbo_grouped_rounds(uint64_t seed, int32_t rounds, int32_t nGrid, uint32_t* out,
                        int32_t* status, int32_t* counters);
void ccbo_stencil(int32_t* bufA, int32_t* bufB, int64_t n, int32_t iters);
int ccbo_cnt_record(uint32_t* count, int32_t mode, uint32_t value);
int ccbo_cnt_wait_holds(uint32_t count, int32_t mode, uint32_t value, int32_t* holds);
int ccbo_cnt_wait_apply(uint32_t* count, int32_t mode, uint32_t value, int32_t isClear,
                        int32_t* released);
int ccbo_cnt_batch(const uint32_t* val, const uint8_t* meta, int64_t nCounters, int32_t nOps,
                   uint32_t* final_out, uint8_t* rel, int32_t nRelRows);
int ccbo_host_barrier(int32_t threads, int32_t rounds, uint64_t seed, uint64_t maxPoll,
                      uint32_t* out, double* nsPerBarrier);

static int failures = 0;
#define CHECK(c)                                                         \
    do {                                                                 \
        if (!(c)) {                                                      \
            fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); \
            ++failures;                                                  \
        }                                                                \
    } while (0)

static uint64_t rng = 0x243F6A8885A308D3ull;
static uint32_t next_u32(void)
{
    rng ^= rng << 13; rng ^= rng >> 7; rng ^= rng << 17;  /* xorshift64 */
    return (uint32_t)(rng >> 32);
}

/* Witness rounds: every member's sum of a round is the same, and the counter
 * ends at rounds x members. */
static void slot_rounds(int32_t rounds, int32_t nGrid, int32_t used)
{
    uint32_t* out = calloc((size_t)rounds * (size_t)nGrid, sizeof(uint32_t));
    int32_t* status = calloc((size_t)nGrid, sizeof(int32_t));
    int32_t counter = 0;
    CHECK(ccbo_slot_rounds(7, rounds, nGrid, used, out, status, &counter) == 0);
    const int32_t n = ccbo_participants(used, nGrid);
    CHECK(counter == rounds * n);
    for (int32_t r = 0; r < rounds; ++r) {
        uint32_t want = 0;
        for (int32_t q = 0; q < n; ++q) want += ccbo_witness_hash(7, (uint32_t)r, (uint32_t)q);
        for (int32_t w = 0; w < n; ++w) CHECK(out[(size_t)r * nGrid + w] == want);
    }
    for (int32_t w = 0; w < nGrid; ++w) CHECK(status[w] == (w < n ? 1 : 2));
    free(out), free(status);
}

static void grouped(int32_t rounds, int32_t nGrid)
{
    uint32_t* out = calloc((size_t)rounds * (size_t)nGrid, sizeof(uint32_t));
    int32_t* status = calloc((size_t)nGrid, sizeof(int32_t));
    int32_t ctr[3] = {0, 0, 0};
    CHECK(ccbo_grouped_rounds(4, rounds, nGrid, out, status, ctr) == 0);
    const int32_t kinds[3] = {(rounds + 2) / 3, (rounds + 1) / 3, rounds / 3};
    CHECK(ctr[0] == kinds[0] * (nGrid / 2));
    CHECK(ctr[1] == kinds[1] * (nGrid / 2));
    CHECK(ctr[2] == kinds[2] * nGrid);
    free(out), free(status);
}

/* The stencil stays within the input's range (a weighted mean, floored). */
static void stencil(int64_t n, int32_t iters)
{
    int32_t* a = malloc(sizeof(int32_t) * (size_t)n);
    int32_t* b = malloc(sizeof(int32_t) * (size_t)n);
    int32_t lo = 1 << 20, hi = -1;
    for (int64_t i = 0; i < n; ++i) {
        a[i] = (int32_t)(next_u32() & ((1u << 20) - 1));
        if (a[i] < lo) lo = a[i];
        if (a[i] > hi) hi = a[i];
    }
    ccbo_stencil(a, b, n, iters);
    const int32_t* y = (iters % 2 == 0) ? a : b;
    for (int64_t i = 0; i < n; ++i) CHECK(y[i] >= lo && y[i] <= hi);
    free(a), free(b);
}

static void cnt_ops(void)
{
    const int32_t rec[4] = {0, 1, 2, 4};
    for (int t = 0; t < 2000; ++t) {
        uint32_t c = next_u32(), v = next_u32();
        CHECK(ccbo_cnt_record(&c, rec[t & 3], v) == 0);
        int32_t h = -1, r = -1;
        CHECK(ccbo_cnt_wait_holds(c, t % 5, v, &h) == 0 && (h == 0 || h == 1));
        uint32_t c2 = c;
        CHECK(ccbo_cnt_wait_apply(&c2, t % 5, v, t & 1, &r) == 0);
        CHECK(r == h && (r && (t & 1) ? c2 == 0 : c2 == c));
    }
    /* a batch with malformed ops sprinkled in, and too few output rows */
    const int64_t nc = 37;
    const int32_t no = 24;
    uint32_t* val = malloc(sizeof(uint32_t) * (size_t)(nc * no));
    uint8_t* meta = malloc((size_t)(nc * no));
    for (int64_t i = 0; i < nc * no; ++i) {
        val[i] = next_u32();
        meta[i] = (uint8_t)next_u32();
    }
    uint32_t* fin = calloc((size_t)nc, sizeof(uint32_t));
    uint8_t* rel = calloc((size_t)(nc * 3), 1);
    const int rc = ccbo_cnt_batch(val, meta, nc, no, fin, rel, 3);
    CHECK(rc == 0 || rc == 1);
    for (int64_t i = 0; i < nc * 3; ++i) CHECK(rel[i] <= 1);
    free(val), free(meta), free(fin), free(rel);
}

/* Host threads running the same arrival rule: each thread's round sum is the
 * sum of all threads' witnesses. */
static void host_barrier(int32_t threads, int32_t rounds)
{
    uint32_t* out = calloc((size_t)threads * (size_t)rounds, sizeof(uint32_t));
    double ns = 0;
    CHECK(ccbo_host_barrier(threads, rounds, 9, (uint64_t)1 << 40, out, &ns) == 0);
    for (int32_t r = 0; r < rounds; ++r) {
        uint32_t want = 0;
        for (int32_t q = 0; q < threads; ++q) want += ccbo_witness_hash(9, (uint32_t)r, (uint32_t)q);
        for (int32_t t = 0; t < threads; ++t) CHECK(out[(size_t)r * threads + t] == want);
    }
    free(out);
}

int main(int argc, char** argv)
{
    const int threadsOnly = argc > 1 && strcmp(argv[1], "threads") == 0;
    if (!threadsOnly) {
        for (int32_t b = 0; b < 200; ++b)
            for (int32_t n = 1; n < 9; ++n) {
                const int32_t t = ccbo_epoch_target(b, n);
                CHECK(t > b && t % n == 0 && t - b <= n);
            }
        CHECK(ccbo_mix_participants(0, 1, 12) == 12 && ccbo_mix_participants(3, 2, 12) == 9);
        slot_rounds(50, 8, 0);
        slot_rounds(30, 37, 19);
        slot_rounds(0, 5, 0);
        grouped(31, 16);
        stencil(1000, 5);
        stencil(3, 4);
        cnt_ops();
    }
    host_barrier(4, 100);
    host_barrier(1, 10);
    if (failures) fprintf(stderr, "%d checks failed\n", failures);
    return failures ? 1 : 0;
}
