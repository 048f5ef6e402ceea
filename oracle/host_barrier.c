/*
 * host_barrier.c -- the soft epoch barrier on host threads.
 *
 * TEST INFRASTRUCTURE ONLY (part of the oracle; same rules as ccb_oracle.c:
 * shares nothing with the HIP library).  Two uses: a concurrency check of
 * the method itself -- T real threads run the flag-slot rounds of [SYNCALL]
 * §6.1 through the arrival rule of [SYNCALL] §5.2 and must produce exactly
 * the sums the sequential simulator gives -- and the CPU context figure of
 * the benchmark (ns per barrier at T host threads).
 *
 * Rule ([SYNCALL] §5.2): each participant adds one to the shared counter and
 * gets the old value back; its round ends once the counter reaches the next
 * multiple of T above that value.  C11 atomics: the add is acq_rel and the
 * poll acquire, so the slot a thread stores before its add is visible to
 * every thread that has seen the round end.  Two slot rows suffice: a row
 * is written again two rounds later, after everyone has passed the barrier
 * that follows their reads of it.
 */
#include <pthread.h>
#include <stdatomic.h>
#include <stdint.h>
#include <stdlib.h>
#include <time.h>

uint32_t ccbo_witness_hash(uint64_t seed, uint32_t round, uint32_t wg);

typedef struct {
    int32_t threads, rounds, id;
    uint64_t seed, maxPoll;
    _Atomic int32_t* ctr;
    _Atomic uint32_t* slots;
    _Atomic int32_t* go;
    _Atomic int32_t* failed;
    uint32_t* out;
} hb_arg;

static inline void cpu_relax(void)
{
#if defined(__x86_64__) || defined(__i386__)
    __builtin_ia32_pause();
#endif
}

static void* hb_thread(void* p)
{
    hb_arg* a = (hb_arg*)p;
    const int32_t T = a->threads;
    while (!atomic_load_explicit(a->go, memory_order_acquire)) cpu_relax();
    for (int32_t r = 0; r < a->rounds; ++r) {
        _Atomic uint32_t* row = a->slots + (size_t)(r & 1) * (size_t)T;
        atomic_store_explicit(&row[a->id], ccbo_witness_hash(a->seed, (uint32_t)r, (uint32_t)a->id),
                              memory_order_relaxed);
        const int32_t before = atomic_fetch_add_explicit(a->ctr, 1, memory_order_acq_rel);
        const int32_t target = (before / T + 1) * T;
        uint64_t polls = 0;
        while (atomic_load_explicit(a->ctr, memory_order_acquire) < target) {
            if (++polls > a->maxPoll || atomic_load_explicit(a->failed, memory_order_relaxed)) {
                atomic_store_explicit(a->failed, 1, memory_order_relaxed);
                return NULL;
            }
            cpu_relax();
        }
        uint32_t s = 0;
        for (int32_t q = 0; q < T; ++q) s += atomic_load_explicit(&row[q], memory_order_relaxed);
        a->out[(size_t)r * (size_t)T + (size_t)a->id] = s;
    }
    return NULL;
}

/* Runs `rounds` rounds on `threads` threads; out[r * threads + t] receives
 * thread t's slot sum of round r.  Returns 0, 1 for bad arguments, 6 when
 * some thread's poll ran past maxPoll.  *nsPerBarrier: wall time per round. */
int ccbo_host_barrier(int32_t threads, int32_t rounds, uint64_t seed, uint64_t maxPoll,
                      uint32_t* out, double* nsPerBarrier)
{
    if (threads < 1 || threads > 1024 || rounds < 0 || out == NULL) return 1;
    _Atomic int32_t ctr = 0, go = 0, failed = 0;
    _Atomic uint32_t* slots = calloc((size_t)2 * (size_t)threads, sizeof(*slots));
    hb_arg* args = calloc((size_t)threads, sizeof(*args));
    pthread_t* tids = calloc((size_t)threads, sizeof(*tids));
    if (!slots || !args || !tids) {
        free(slots), free(args), free(tids);
        return 1;
    }
    int started = 0;
    for (int32_t t = 0; t < threads; ++t) {
        args[t] = (hb_arg){threads, rounds, t, seed, maxPoll, &ctr, slots, &go, &failed, out};
        if (pthread_create(&tids[t], NULL, hb_thread, &args[t]) != 0) {
            atomic_store(&failed, 1);
            break;
        }
        ++started;
    }
    struct timespec t0, t1;
    clock_gettime(CLOCK_MONOTONIC, &t0);
    atomic_store_explicit(&go, 1, memory_order_release);
    for (int t = 0; t < started; ++t) pthread_join(tids[t], NULL);
    clock_gettime(CLOCK_MONOTONIC, &t1);
    if (nsPerBarrier != NULL)
        *nsPerBarrier = rounds > 0 ? ((double)(t1.tv_sec - t0.tv_sec) * 1e9 +
                                      (double)(t1.tv_nsec - t0.tv_nsec)) / rounds
                                   : 0.0;
    free(slots), free(args), free(tids);
    if (started < threads) return 1;
    return atomic_load(&failed) ? 6 : 0;
}
