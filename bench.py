#!/usr/bin/env python3
"""Benchmark of the soft epoch barrier on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--mode striped-order]

A step is one pass of the headline workload: 256 workgroups x 256 threads
(one per CU), 10,000 witness rounds on one barrier with usedCores = 0 (every
round: each workgroup stores its witness, all pass the barrier, each sums all
256 witnesses).  `value` is barriers per second over the K timed steps.

The same run also measures, each on its own stream with HIP events:
  - the floor: dependent agent-scope atomic round trips by one lane
    (fetch-add and load, with and without fences), 256-way contention, and
    the one-way notification latency between two CUs (ping-pong);
  - barrier-only latency for every barrier variant (slope over rounds), the
    chosen variant from 2 to 1024 workgroups, and HIP's cooperative-groups
    grid sync on the same grids for comparison;
  - the 128-member pass and the grouped A/B/mix rounds (512 workgroups);
  - the persistent stencil (2^26 int32, 64 iterations, 1024 workgroups):
    the HBM roofline of the data phases;
  - the batched CntNotify engine (2^20 counters x 64 ops);
  - CntNotify record -> wait latency between streams, and the cost of a
    record + wait pair enqueued eagerly or replayed from a HIP graph;
  - a 512 MiB streaming copy (achievable HBM ceiling);
  - the CPU oracle on the host cores (cpu_baseline).
It prints ONE JSON line.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, 8 TB/s
STENCIL_N = 1 << 26
STENCIL_ITERS = 64
STENCIL_BYTES_PER_ITER = 2 * 4 * STENCIL_N  # read x, write x' (int32)
CNT_COUNTERS, CNT_OPS = 1 << 20, 64


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def sha256_of(a) -> str:
    return hashlib.sha256(memoryview(a).cast("B")).hexdigest()


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--mode", default="striped-order",
                    choices=["striped-order", "flat-order", "striped-full", "flat-full",
                             "tree-order", "tree-full", "striped-xcd", "flat-xcd", "tree-xcd"])
    ap.add_argument("--quick", action="store_true", help="headline only (for profiling runs)")
    ap.add_argument("--only", choices=["counters", "barrier", "cnt"], default=None,
                    help="counters: only the copy ceiling, the stencil and the batched "
                         "CntNotify engine (counter collection); barrier: only the floor, "
                         "the barrier-only latencies and their breakdown; cnt: only the "
                         "CntNotify stream legs")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    return ap.parse_args()


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for rel in ("cross_core_barrier_amd/csrc/ccb_kernels.hip", "include/ccb_device.h",
                "cross_core_barrier_amd/csrc/ccb_internal.h"):
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def profiled_traffic(summary: str):
    """HBM bytes per launch of one kernel from its committed rocprofv3 PMC
    summary (profiles/<summary>), or None when absent or taken on different
    kernel sources."""
    path = os.path.join(ROOT, "profiles", summary)
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"kernel_source_hash:\s*([0-9a-f]+)", text)
    t = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m or not t or m.group(1) != kernel_source_hash():
        return None
    return float(t.group(1))


class Timer:
    """HIP events on the given torch stream."""

    def __init__(self, torch, stream):
        self.torch, self.stream = torch, stream

    def __call__(self, fn, reps=1):
        torch = self.torch
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(self.stream)
        for _ in range(reps):
            fn()
        e1.record(self.stream)
        e1.synchronize()
        return e0.elapsed_time(e1) / reps  # ms per call


class Bench:
    def __init__(self, args):
        import numpy as np
        import torch

        from cross_core_barrier_amd import ccb, inputs, workloads
        self.np, self.torch, self.ccb, self.inputs, self.wl = np, torch, ccb, inputs, workloads
        self.args = args
        self.mode = ccb.MODES[args.mode]
        torch.cuda.set_device(0)
        st, self.n_cu, _, clk_khz = ccb.ccb_device_info()
        ccb.check(st, "ccb_device_info")
        self.tick_ns = 1e6 / clk_khz
        self.stream = torch.cuda.Stream()
        self.timer = Timer(torch, self.stream)
        self.dev = torch.device("cuda")
        self.ws = workloads.workspace(3)
        self.extra = {}
        self.gpu_sha = {}  # SHA-256 of each configuration's GPU outputs

    # ------------------------------------------------------------ headline
    def headline(self):
        torch, ccb, args = self.torch, self.ccb, self.args
        cfg = self.inputs.WITNESS_GRID
        n_grid, threads, rounds = cfg["n_wg"], cfg["threads"], cfg["rounds"]
        ws, stream, mode = self.ws, self.stream, self.mode
        slots = torch.zeros(ccb.CCB_SLOT_ROWS * ccb.CCB_SLOT_WORDS * n_grid, dtype=torch.int32, device=self.dev)
        out = torch.zeros((rounds, n_grid), dtype=torch.int32, device=self.dev)

        def step():
            ccb.check(ccb.ccb_syncall_workspace_reset(ws, 1, stream), "reset")
            ccb.check(ccb.ccb_run_slot_rounds(ws, slots, out, None, cfg["seed"], rounds, n_grid,
                                              threads, 0, 1, 0, mode, stream), "slot_rounds")

        log(f"headline: witness rounds {n_grid}x{threads}, {rounds} rounds, mode {args.mode}")
        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        ms_events = self.timer(step, reps=args.steps)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        st, arrivals = ccb.ccb_syncall_status(ws, 1, stream)
        ccb.check(st, "headline status")
        assert arrivals == [rounds * n_grid], arrivals
        ms_per_step = max(ms_events, wall * 1e3 / args.steps)
        self.extra["ns_per_round_with_witness"] = round(ms_per_step * 1e6 / rounds, 1)
        self.gpu_sha["cfg1"] = sha256_of(out.cpu().numpy())

        def pass2():
            ccb.check(ccb.ccb_syncall_workspace_reset(ws, 1, stream), "reset")
            ccb.check(ccb.ccb_run_slot_rounds(ws, slots, out, None, cfg["seed"], rounds, n_grid,
                                              threads, cfg["used_cores_pass2"], 1, 0, mode, stream),
                      "slot_rounds pass 2")
        pass2()
        ms = min(self.timer(pass2) for _ in range(3))
        st, arr = ccb.ccb_syncall_status(ws, 1, stream)
        ccb.check(st, "pass 2 status")
        assert arr == [rounds * cfg["used_cores_pass2"]], arr
        self.extra["ns_per_round_128_members"] = round(ms * 1e6 / rounds, 1)
        return ms_per_step, rounds

    # ------------------------------------------------------------ full visibility with data
    def full_visibility_witness(self):
        """The headline's witness rounds (256 x 256, 10,000 rounds, plain slot
        accesses) with full visibility two ways: fences in every workgroup,
        or one L2 write-back per XCD; ns per round, outputs checked."""
        torch, ccb = self.torch, self.ccb
        cfg = self.inputs.WITNESS_GRID
        n_grid, threads, rounds = cfg["n_wg"], cfg["threads"], cfg["rounds"]
        ws, stream = self.ws, self.stream
        slots = torch.zeros(ccb.CCB_SLOT_ROWS * ccb.CCB_SLOT_WORDS * n_grid, dtype=torch.int32,
                            device=self.dev)
        out = torch.zeros((rounds, n_grid), dtype=torch.int32, device=self.dev)
        res = {}
        for name in ("striped-full", "striped-xcd"):
            m = ccb.MODES[name]

            def step(m=m):
                ccb.check(ccb.ccb_syncall_workspace_reset(ws, 1, stream), "reset")
                ccb.check(ccb.ccb_run_slot_rounds(ws, slots, out, None, cfg["seed"], rounds, n_grid,
                                                  threads, 0, 1, 0, m, stream), "slot_rounds")
            step()
            ms = min(self.timer(step) for _ in range(3))
            st, arr = ccb.ccb_syncall_status(ws, 1, stream)
            ccb.check(st, "full visibility status")
            assert arr == [rounds * n_grid], arr
            if "cfg1" in self.gpu_sha:  # the same outputs as the ordering-only headline
                assert sha256_of(out.cpu().numpy()) == self.gpu_sha["cfg1"], name
            res[name] = round(ms * 1e6 / rounds, 1)
        self.extra["full_visibility_ns_per_round_with_witness"] = res
        log(f"full visibility, witness rounds at 256: {res}")

    # ------------------------------------------------------------ floor
    def floor(self):
        torch, ccb, stream = self.torch, self.ccb, self.stream
        lines = torch.zeros(64 * 32, dtype=torch.int32, device=self.dev)
        ticks = torch.zeros(2, dtype=torch.int64, device=self.dev)

        def chain(kind, fenced, line_idx, iters=20000):
            line = lines[line_idx * 32:]
            ccb.check(ccb.ccb_bench_atomic_chain(line, ticks, iters, fenced, kind, stream), "chain")
            stream.synchronize()
            t = ticks.cpu().numpy()
            return (t[1] - t[0]) * self.tick_ns / iters

        floor = {}
        for name, kind, fenced in (("fetch_add_ns", 0, 0), ("load_ns", 1, 0),
                                   ("fetch_add_fenced_ns", 0, 1), ("load_fenced_ns", 1, 1)):
            chain(kind, fenced, 0, 1000)
            vals = [chain(kind, fenced, i) for i in range(0, 64, 8)]
            floor[name] = round(statistics.median(vals), 1)
        tk = torch.zeros(2 * 256, dtype=torch.int64, device=self.dev)
        ccb.check(ccb.ccb_bench_atomic_contended(lines, tk, 2000, 256, stream), "contended")
        stream.synchronize()
        t = tk.cpu().numpy().reshape(-1, 2)
        floor["same_address_fetch_add_ns_at_256"] = round(
            float(t[:, 1].max() - t[:, 0].min()) * self.tick_ns / (2000 * 256), 2)
        # one CU's update reaching another CU's poll: a ping-pong between
        # workgroup 0 and workgroup 1 (dealt to another XCD) or 8 (the same XCD)
        pl = torch.empty(2 * 32, dtype=torch.int32, device=self.dev)
        pt = torch.zeros(4, dtype=torch.int64, device=self.dev)
        perr = torch.empty(1, dtype=torch.int32, device=self.dev)
        iters, same, other = 10000, [], []
        for peer in range(1, 9):  # workgroups are dealt to the XCDs in turn
            vals = []
            for _ in range(3):
                with torch.cuda.stream(stream):
                    pl.zero_()
                    perr.zero_()
                ccb.check(ccb.ccb_bench_notify_pingpong(pl, pt, iters, peer, 0, perr, stream),
                          "ping-pong")
                stream.synchronize()
                assert int(perr.item()) == 0
                assert int(pl[0].item()) == int(pl[32].item()) == iters
                t = pt.cpu().numpy()
                vals.append(float(t[1] - t[0]) * self.tick_ns / (2 * iters))
            (same if int(t[2]) == int(t[3]) else other).append(min(vals))
        notify = {}
        if other:  # the median over the partner XCDs, and their range
            notify["other_xcd"] = round(statistics.median(other), 1)
            notify["other_xcd_range"] = [round(min(other), 1), round(max(other), 1)]
        if same:
            notify["same_xcd"] = round(statistics.median(same), 1)
        floor["notify_one_way_ns"] = notify
        self.extra["floor"] = floor
        log(f"floor: {floor}")
        return floor

    # ------------------------------------------------------------ barrier-only latency
    def latency(self, floor):
        ccb, ws, stream = self.ccb, self.ws, self.stream
        lat = {}
        for name, m in ccb.MODES.items():
            res = {}
            for r in (1000, 5000):
                def f(r=r, m=m):
                    ccb.check(ccb.ccb_syncall_workspace_reset(ws, 1, stream), "reset")
                    ccb.check(ccb.ccb_run_barrier_only(ws, None, None, r, 256, 256, 0, 1, 0, m,
                                                       stream), "barrier_only")
                f()
                res[r] = min(self.timer(f) for _ in range(3))
            st, _ = ccb.ccb_syncall_status(ws, 1, stream)
            ccb.check(st, "barrier_only status")
            lat[name] = round((res[5000] - res[1000]) / 4000 * 1e6, 1)
        self.extra["barrier_only_ns_at_256"] = lat
        # the chosen variant against the number of workgroups (256 threads
        # each), and beside it the two-level tree (the striped counter's
        # alternative for cutting same-address serialisation)
        def by_workgroups(m):
            by_n = {}
            for n in (2, 8, 64, 256, 512, 1024):
                res = {}
                for r in (1000, 5000):
                    def f(r=r, n=n):
                        ccb.check(ccb.ccb_syncall_workspace_reset(ws, 1, stream), "reset")
                        ccb.check(ccb.ccb_run_barrier_only(ws, None, None, r, n, 256, 0, 0, 0, m,
                                                           stream), "barrier_only")
                    f()
                    res[r] = min(self.timer(f) for _ in range(3))
                st, arr = ccb.ccb_syncall_status(ws, 1, stream)
                ccb.check(st, "barrier_only status")
                assert arr == [5000 * n], arr
                by_n[str(n)] = round((res[5000] - res[1000]) / 4000 * 1e6, 1)
            return by_n
        self.extra["barrier_only_ns_by_workgroups"] = by_workgroups(ccb.MODES[self.args.mode])
        if self.args.mode != "tree-order":
            self.extra["tree_order_ns_by_workgroups"] = by_workgroups(ccb.MODES["tree-order"])
        # full visibility two ways: fences in every workgroup, or one L2
        # write-back per XCD (a second notification instead of N write-backs)
        self.extra["full_visibility_ns_by_workgroups"] = {
            name: by_workgroups(ccb.MODES[name]) for name in ("striped-full", "striped-xcd")}
        best = lat[self.args.mode]
        roof = {"bound": "atomic_round_trip", "achieved_ns_per_barrier": best,
                "floor_ns": floor["fetch_add_ns"], "ratio": round(best / floor["fetch_add_ns"], 2),
                "target_ratio": 2.0}
        # a poll-based barrier pays at least the arrival's round trip and one
        # notification (another CU's update reaching this CU's poll)
        other = floor["notify_one_way_ns"].get("other_xcd")
        if other is not None:
            composed = floor["fetch_add_ns"] + other
            roof.update({"notify_one_way_ns": other, "composed_floor_ns": round(composed, 1),
                         "ratio_to_composed_floor": round(best / composed, 2)})
        # full visibility (the public device API's default) beside it: the
        # per-workgroup fences and the per-XCD write-back
        full, xcd = lat["striped-full"], lat["striped-xcd"]
        roof["full_visibility"] = {"per_workgroup_fences_ns": full, "per_xcd_writeback_ns": xcd,
                                   "achieved_ns_per_barrier": min(full, xcd),
                                   "ratio": round(min(full, xcd) / floor["fetch_add_ns"], 2),
                                   "ratio_to_ordering_only": round(min(full, xcd) / best, 2)}
        self.extra["latency_roofline"] = roof
        log(f"barrier-only ns/barrier at 256 WGs: {lat}")

    # ------------------------------------------------------------ fence placement
    def fence_placement(self, n_grid=256):
        """ccb_bench_fence_placement: the full-visibility barrier's release and
        acquire placed six ways at n_grid workgroups x 256 threads; ns per
        barrier (slope over 500 -> 2500 rounds) and the fraction of plain
        reads after the barrier that returned a stale value (2000 rounds)."""
        np, torch, ccb, stream = self.np, self.torch, self.ccb, self.stream
        nbytes = ccb.ccb_bench_fence_placement_bytes(n_grid)
        scratch = torch.zeros(nbytes // 4, dtype=torch.int32, device=self.dev)
        stale = torch.zeros(n_grid, dtype=torch.int32, device=self.dev)
        names = ["none", "per_workgroup_release_acquire", "per_workgroup_release_only",
                 "per_workgroup_acquire_only", "per_xcd_release_per_workgroup_acquire",
                 "per_xcd_release_workgroup_scope_invalidate"]
        err_word = ccb.CCB_STRIPES * 32
        out = {}
        for v, name in enumerate(names):
            res = {}
            for r in (500, 2500):
                def f(r=r, v=v):
                    ccb.check(ccb.ccb_bench_fence_placement(scratch, nbytes, stale, r, n_grid, 256, v,
                                                            stream), "fence placement")
                f()
                res[r] = min(self.timer(f) for _ in range(3))
                assert int(scratch[err_word].item()) == 0
            ccb.check(ccb.ccb_bench_fence_placement(scratch, nbytes, stale, 2000, n_grid, 256, v,
                                                    stream), "fence placement")
            torch.cuda.synchronize()
            assert int(scratch[err_word].item()) == 0
            out[name] = {"ns_per_barrier": round((res[2500] - res[500]) / 2000 * 1e6, 1),
                         "stale_read_fraction": round(float(stale.sum().item()) / (2000 * n_grid), 4)}
        self.extra["fence_placement_at_256"] = out
        log(f"fence placement: {out}")

    # ------------------------------------------------------------ where a barrier's time goes
    def barrier_breakdown(self, floor, mode_name=None, n_grid=256, rounds=1024, skip=64):
        """Per-member, per-round wall-clock stamps of barrier-only rounds at
        n_grid workgroups x 256 threads (ccb_bench_barrier_breakdown): issue
        of the arrival, its reply, and the poll seeing the round complete.
        Medians over rounds (after `skip` warm-up rounds) of
          arrival_round_trip     reply - issue, per member
          last_arrival_to_first_observer   first release of a round - the
                                 last issue of that round
          first_to_last_observer last release - first release of a round
          release_to_next_arrival  next issue - release, per member
          round                  last release - the previous round's last
                                 release
        each beside the floor it is compared with."""
        np, torch, ccb, ws, stream = self.np, self.torch, self.ccb, self.ws, self.stream
        mode_name = mode_name or self.args.mode
        mode = ccb.MODES[mode_name]
        stamps = torch.zeros(rounds * n_grid * 3, dtype=torch.int64, device=self.dev)
        ccb.check(ccb.ccb_syncall_workspace_reset(ws, 1, stream), "reset")
        ccb.check(ccb.ccb_bench_barrier_breakdown(ws, stamps, rounds, n_grid, 256, 0, mode, stream),
                  "breakdown")
        st, arr = ccb.ccb_syncall_status(ws, 1, stream)
        ccb.check(st, "breakdown status")
        assert arr == [rounds * n_grid], arr
        t = stamps.cpu().numpy().reshape(rounds, n_grid, 3).astype(np.float64) * self.tick_ns
        issue, reply, rel = t[skip:, :, 0], t[skip:, :, 1], t[skip:, :, 2]
        med = lambda a: round(float(np.median(a)), 1)
        terms = {
            "arrival_round_trip": med(reply - issue),
            "last_arrival_to_first_observer": med(rel.min(axis=1) - issue.max(axis=1)),
            "first_to_last_observer": med(rel.max(axis=1) - rel.min(axis=1)),
            "release_to_next_arrival": med(issue[1:] - rel[:-1]),
        }
        last = rel.max(axis=1)
        out = {"mode": mode_name, "workgroups": n_grid, "rounds_stamped": rounds - skip,
               "median_ns": terms, "round_ns": med(np.diff(last)),
               "mean_round_ns": round(float(np.diff(last).mean()), 1),
               # who sees the release first: the member whose arrival was last
               "first_observer_is_last_arriver": round(float(np.mean(
                   rel.argmin(axis=1) == issue.argmax(axis=1))), 3),
               "floors_ns": {"arrival_round_trip": floor["fetch_add_ns"],
                             "last_arrival_to_first_observer": floor["fetch_add_ns"],
                             "first_to_last_observer": floor["load_ns"],
                             "notify_one_way": floor["notify_one_way_ns"].get("other_xcd")},
               "clock_resolution_ns": round(self.tick_ns, 1)}
        self.extra.setdefault("barrier_breakdown", {})[mode_name] = out
        log(f"barrier breakdown ({mode_name}): {out}")
        return out

    # ------------------------------------------------------------ HIP's own grid barrier
    def hip_grid_sync(self):
        """cooperative_groups grid_group::sync() on the same grids (slope over rounds)."""
        torch, ccb, stream = self.torch, self.ccb, self.stream
        done = torch.zeros(1, dtype=torch.int32, device=self.dev)
        out = {}
        for n_wg, threads in ((256, 256), (1024, 256)):
            res = {}
            for r in (200, 1000):
                def f(r=r):
                    ccb.check(ccb.ccb_bench_hip_grid_sync(r, n_wg, threads, done, stream),
                              "hip grid sync")
                f()
                res[r] = min(self.timer(f) for _ in range(3))
                torch.cuda.synchronize()
                assert int(done.item()) == r
            out[f"{n_wg}x{threads}"] = round((res[1000] - res[200]) / 800 * 1e6, 1)
        self.extra["hip_grid_sync_ns"] = out
        log(f"HIP cooperative-groups grid sync, ns per sync: {out}")

    # ------------------------------------------------------------ grouped rounds
    def grouped(self):
        torch, ccb, ws, stream = self.torch, self.ccb, self.ws, self.stream
        g = self.inputs.GROUPED
        gout = torch.zeros((g["rounds"], g["n_wg"]), dtype=torch.int32, device=self.dev)
        gslots = torch.zeros(ccb.CCB_SLOT_ROWS * ccb.CCB_SLOT_WORDS * g["n_wg"], dtype=torch.int32, device=self.dev)

        def run():
            ccb.check(ccb.ccb_syncall_workspace_reset(ws, 3, stream), "reset")
            ccb.check(ccb.ccb_run_grouped_rounds(ws, gslots, gout, None, g["seed"], g["rounds"],
                                                 g["n_wg"], g["threads"], 2, 0, self.mode, stream),
                      "grouped")
        run()
        ms = min(self.timer(run) for _ in range(2))
        st, _ = ccb.ccb_syncall_status(ws, 3, stream)
        ccb.check(st, "grouped status")
        self.extra["grouped_ns_per_round"] = round(ms * 1e6 / g["rounds"], 1)
        out_sha = sha256_of(gout.cpu().numpy())
        self.grouped_kinds(gslots, gout, out_sha)
        return out_sha

    def grouped_kinds(self, gslots, gout, out_sha, skip=64):
        """Time per round kind from a timeline launch (ccb_bench_grouped_timeline):
        each member's wall clock at every barrier it passes, for its first
        1024 own rounds.  An even member's own rounds alternate A, mix; an odd
        member's B, mix; a round's time is the member's stamp minus its
        previous one.  The timeline launch must compute the same outputs."""
        np, torch, ccb, ws, stream = self.np, self.torch, self.ccb, self.ws, self.stream
        g = self.inputs.GROUPED
        n_wg, cap = g["n_wg"], ccb.CCB_BREAKDOWN_MAX_ROUNDS
        stamps = torch.zeros(cap * n_wg, dtype=torch.int64, device=self.dev)
        ccb.check(ccb.ccb_syncall_workspace_reset(ws, 3, stream), "reset")
        ccb.check(ccb.ccb_bench_grouped_timeline(ws, gslots, gout, stamps, g["seed"], g["rounds"],
                                                 n_wg, g["threads"], 2, self.mode, stream),
                  "grouped timeline")
        st, _ = ccb.ccb_syncall_status(ws, 3, stream)
        ccb.check(st, "grouped timeline status")
        assert sha256_of(gout.cpu().numpy()) == out_sha
        t = stamps.cpu().numpy().reshape(cap, n_wg).astype(np.float64) * self.tick_ns
        d = np.diff(t, axis=0)[skip:]   # row i - 1 - skip: own round i
        first = skip + 1                # own round index of d's first row
        own = np.arange(first, first + d.shape[0])
        even, odd = d[:, 0::2], d[:, 1::2]
        med = lambda a: round(float(np.median(a)), 1)
        self.extra["grouped_ns_per_round_kind"] = {
            "A": med(even[own % 2 == 0]), "B": med(odd[own % 2 == 0]),
            "mix": med(np.concatenate([even[own % 2 == 1], odd[own % 2 == 1]])),
            "own_rounds_stamped": int(d.shape[0]),
            "note": "per member: wall clock at passing a barrier minus at passing its previous "
                    "one; A and B rounds run at the same time on disjoint halves"}
        log(f"grouped per kind: {self.extra['grouped_ns_per_round_kind']}")

    # ------------------------------------------------------------ streaming copy ceiling
    def copy_ceiling(self):
        torch, ccb, stream = self.torch, self.ccb, self.stream
        src = torch.empty(1 << 27, dtype=torch.int32, device=self.dev).fill_(1)
        dst = torch.empty_like(src)
        copy_bytes = 2 * src.numel() * 4

        def copy():
            ccb.check(ccb.ccb_bench_copy(dst, src, src.numel() * 4, stream), "copy")
        copy()
        ms = min(self.timer(copy, reps=10) for _ in range(3))
        gbs = copy_bytes / (ms / 1e3) / 1e9
        self.extra["copy_512MiB_GBs"] = round(gbs, 1)
        return gbs

    # ------------------------------------------------------------ stencil roofline
    def stencil(self, copy_gbs):
        torch, ccb, ws, stream = self.torch, self.ccb, self.ws, self.stream
        s = self.inputs.STENCIL
        x0 = torch.from_numpy(self.inputs.stencil_input(s["seed"], STENCIL_N)).to(self.dev)
        a = torch.empty_like(x0)
        b = torch.empty_like(x0)
        halo = self.wl.halo_scratch(STENCIL_N, s["threads"], s["n_wg"])

        def run():
            ccb.check(ccb.ccb_syncall_workspace_reset(ws, 1, stream), "reset")
            ccb.check(ccb.ccb_run_stencil(a, b, STENCIL_N, STENCIL_ITERS, ws, halo, None, s["n_wg"],
                                          s["threads"], 4, 0, self.mode, stream), "stencil")
        a.copy_(x0)
        run()
        times = []
        for _ in range(5):
            a.copy_(x0)
            torch.cuda.synchronize()
            times.append(self.timer(run))
        st, arr = ccb.ccb_syncall_status(ws, 1, stream)
        ccb.check(st, "stencil status")
        assert arr == [(STENCIL_ITERS - 1) * s["n_wg"]], arr
        st_ms = statistics.median(times)
        self.gpu_sha["cfg2"] = sha256_of(a.cpu().numpy())  # 64 iterations end in bufA
        self.stencil_phases(run_args=(a, b, x0, halo, s))
        alg_bytes = STENCIL_BYTES_PER_ITER * STENCIL_ITERS
        achieved = alg_bytes / (st_ms / 1e3) / 1e9
        self.extra["stencil_barriers_per_launch"] = STENCIL_ITERS - 1
        return {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": profiled_traffic("ccb_k_stencil_counters.md"), "kernel": "ccb_k_stencil",
                "launch_ms": round(st_ms, 4), "algorithmic_bytes": alg_bytes,
                "frac_of_copy_ceiling": round(achieved / copy_gbs, 4) if copy_gbs else None}

    def stencil_phases(self, run_args):
        """One more launch with per-workgroup wall-clock stamps: the data
        phases alone (first release to last data end of each iteration), the
        barriers (last data end to last release) and the finish skew."""
        np, torch, ccb, ws, stream = self.np, self.torch, self.ccb, self.ws, self.stream
        a, b, x0, halo, s = run_args
        G, iters = s["n_wg"], STENCIL_ITERS
        tl = torch.zeros(G * (2 * iters + 1), dtype=torch.int64, device=self.dev)
        a.copy_(x0)
        torch.cuda.synchronize()
        ccb.check(ccb.ccb_syncall_workspace_reset(ws, 1, stream), "reset")
        ccb.check(ccb.ccb_run_stencil(a, b, STENCIL_N, iters, ws, halo, None, G, s["threads"], 4, 0,
                                      self.mode, stream, timeline=tl), "stencil timeline")
        stream.synchronize()
        st, _ = ccb.ccb_syncall_status(ws, 1, stream)
        ccb.check(st, "stencil timeline status")
        t = tl.cpu().numpy().reshape(G, 2 * iters + 1).astype(np.float64) * self.tick_ns
        start, dend, rel = t[:, 0], t[:, 1::2], t[:, 2::2]
        first = np.concatenate([[start.min()], rel[:, :-1].min(axis=0)])
        data = dend.max(axis=0) - first
        barrier = (rel.max(axis=0) - dend.max(axis=0))[:-1]
        skew = dend.max(axis=0) - dend.min(axis=0)
        # Per-workgroup data phases (its release -> its data end): how much of
        # the finish skew is systematic per workgroup (a static assignment
        # could remove that part) and how much is per-iteration noise.
        begin = np.concatenate([start[:, None], rel[:, :-1]], axis=1)
        d = (dend - begin)[:, 2:]  # from the third iteration on
        mu = d.mean(axis=1)
        half = d.shape[1] // 2
        dispatch_round = np.arange(G) * 4 // G  # four workgroups per CU, dealt in order
        equalised = d * (mu.mean() / mu)[:, None]
        skew_model = {
            "per_workgroup_mean_us": {"min": round(float(mu.min()) / 1e3, 2),
                                      "median": round(float(np.median(mu)) / 1e3, 2),
                                      "max": round(float(mu.max()) / 1e3, 2)},
            "split_half_correlation": round(float(np.corrcoef(d[:, :half].mean(1),
                                                              d[:, half:].mean(1))[0, 1]), 3),
            "within_workgroup_std_us": round(float(np.median(d.std(axis=1))) / 1e3, 2),
            "by_dispatch_round_mean_us": [round(float(mu[dispatch_round == r].mean()) / 1e3, 2)
                                          for r in range(4)],
            "mean_of_iteration_max_us": round(float(d.max(axis=0).mean()) / 1e3, 2),
            # every workgroup's work scaled by its own measured speed
            "ideal_static_rebalance_max_us": round(float(equalised.max(axis=0).mean()) / 1e3, 2)}
        self.extra["stencil_phases"] = {
            "skew_model": skew_model,
            "data_phase_us_mean": round(float(data.mean()) / 1e3, 2),
            "data_phase_GBs": round(STENCIL_BYTES_PER_ITER / float(data.mean()), 1),
            "data_phase_frac_of_peak": round(STENCIL_BYTES_PER_ITER / float(data.mean()) / HBM_PEAK_GBS, 4),
            "barrier_us_mean": round(float(barrier.mean()) / 1e3, 3),
            "barrier_us_median": round(float(np.median(barrier)) / 1e3, 3),
            "barrier_us_max": round(float(barrier.max()) / 1e3, 3),
            "finish_skew_us_mean": round(float(skew.mean()) / 1e3, 2),
            "in_kernel_total_ms": round(float(t[:, -1].max() - start.min()) / 1e6, 4)}
        log(f"stencil phases: {self.extra['stencil_phases']}")

    # ------------------------------------------------------------ batched CntNotify
    def cnt_batch(self):
        np, torch, ccb, stream = self.np, self.torch, self.ccb, self.stream
        c = self.inputs.CNT_BATCH
        val, meta, rows = self.inputs.cnt_batch_input(c["seed"], CNT_COUNTERS, CNT_OPS)
        v = torch.from_numpy(val.view(np.int32)).to(self.dev)
        m = torch.from_numpy(meta).to(self.dev)
        fin = torch.empty(CNT_COUNTERS, dtype=torch.int32, device=self.dev)
        rel = torch.empty((rows, CNT_COUNTERS), dtype=torch.uint8, device=self.dev)
        err = torch.zeros(1, dtype=torch.int32, device=self.dev)

        def batch():
            ccb.check(ccb.ccb_cnt_notify_batch(v, m, CNT_COUNTERS, CNT_OPS, fin, rel, rows, err,
                                               stream), "batch")
        batch()
        bms = min(self.timer(batch, reps=20) for _ in range(3))
        assert int(err.item()) == 0
        self.gpu_sha["cfg3"] = (sha256_of(fin.cpu().numpy()), sha256_of(rel.cpu().numpy()))
        cnt_bytes = val.nbytes + meta.nbytes + CNT_COUNTERS * 4 + rows * CNT_COUNTERS
        gbs = cnt_bytes / (bms / 1e3) / 1e9
        self.extra["cntnotify_batch"] = {"us_per_launch": round(bms * 1e3, 2), "GBs": round(gbs, 1),
                                         "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4),
                                         "ops_per_s": round(CNT_COUNTERS * CNT_OPS / (bms / 1e3), 0),
                                         "algorithmic_bytes": cnt_bytes,
                                         "traffic": profiled_traffic("ccb_k_cnt_batch_counters.md")}

    # ------------------------------------------------------------ record + wait in a graph
    def cnt_graph(self):
        """100 (record ADD 1, wait GE 1 with clear) pairs on one stream, enqueued
        eagerly and replayed from a captured HIP graph: the cost of one pair
        each way.  Every pair leaves the count at 0."""
        ccb, torch, s = self.ccb, self.torch, self.stream
        st, h = ccb.ccb_cnt_notify_create(0)
        ccb.check(st, "create")
        rec = ccb.record_info(ccb.CCB_CNT_RECORD_ADD, 1)
        wait = ccb.wait_info(ccb.CCB_CNT_WAIT_BIGGER_OR_EQUAL, 1, 2, 1)

        def pairs():
            for _ in range(100):
                ccb.check(ccb.ccb_cnt_notify_record(h, s, rec), "record")
                ccb.check(ccb.ccb_cnt_notify_wait(h, s, wait), "wait")

        pairs()
        torch.cuda.synchronize()
        eager = min(self.timer(pairs) for _ in range(5))
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            pairs()
        g.replay()
        torch.cuda.synchronize()
        graph = min(self.timer(g.replay) for _ in range(5))
        st, v, last = ccb.ccb_cnt_notify_query(h, s)
        assert (st, v, last) == (0, 0, ccb.CCB_OK), (st, v, last)
        ccb.check(ccb.ccb_cnt_notify_destroy(h), "destroy")
        out = {"eager_us_per_pair": round(eager * 1e3 / 100, 2),
               "graph_us_per_pair": round(graph * 1e3 / 100, 2)}
        self.extra["cntnotify_record_wait_pair"] = out
        log(f"cntnotify record + wait pair: {out}")

    # ------------------------------------------------------------ stream-to-stream notify
    def cnt_stream_latency(self, producers=(1, 2, 4, 8, 16), rounds=210, skip=10):
        """CntNotify §5's pattern on streams at scale: N producer streams each
        spin briefly (so the wait is usually polling already), record an
        event, then record ADD 1; the consumer stream waits GE N with isClear
        and records an event.  Latency = the consumer's event minus the
        latest producer event, so it covers the record kernel's own launch,
        the wait's detection and the wait kernel's completion.  (An event
        recorded after a record kernel is not a usable start: with more
        streams than the process's 4 hardware queues its timestamp can trail
        the consumer's.)  The records are enqueued before the wait, so that a
        wait never sits in a hardware queue in front of a record it needs.
        Beside it, the same shape through HIP's own cross-stream dependency
        (producers run an empty one-lane kernel, the consumer waits for
        their events and runs one), and an empty one-lane kernel between two
        events on one stream: the launch-and-complete cost any kernel on the
        path pays."""
        ccb, torch = self.ccb, self.torch
        out = {}

        def stats(xs):
            xs = sorted(xs)
            return {"median_us": round(xs[len(xs) // 2], 2),
                    "p90_us": round(xs[int(len(xs) * 0.9)], 2)}

        def ev(stream):
            e = torch.cuda.Event(enable_timing=True)
            e.record(stream)
            return e

        for n in producers:
            prods = [torch.cuda.Stream() for _ in range(n)]
            cons = torch.cuda.Stream()
            st, h = ccb.ccb_cnt_notify_create(0)
            ccb.check(st, "create")
            lat, dep = [], []
            for r in range(rounds):
                pre = []
                for s in prods:  # producers first: see the docstring
                    with torch.cuda.stream(s):
                        torch.cuda._sleep(20000)
                    pre.append(ev(s))
                    ccb.check(ccb.ccb_cnt_notify_record(
                        h, s, ccb.record_info(ccb.CCB_CNT_RECORD_ADD, 1)), "record")
                ccb.check(ccb.ccb_cnt_notify_wait(
                    h, cons, ccb.wait_info(ccb.CCB_CNT_WAIT_BIGGER_OR_EQUAL, n, 2, 1)), "wait")
                ev_c = ev(cons)
                torch.cuda.synchronize()
                st, v, last = ccb.ccb_cnt_notify_query(h, cons)
                assert (st, v, last) == (0, 0, ccb.CCB_OK), (n, r, st, v, last)
                # the same dependency through HIP events
                pre2, post2 = [], []
                for s in prods:
                    with torch.cuda.stream(s):
                        torch.cuda._sleep(20000)
                    pre2.append(ev(s))
                    with torch.cuda.stream(s):
                        torch.cuda._sleep(1)  # empty one-lane kernel
                    post2.append(ev(s))
                for e in post2:
                    cons.wait_event(e)
                with torch.cuda.stream(cons):
                    torch.cuda._sleep(1)
                ev_f = ev(cons)
                torch.cuda.synchronize()
                if r >= skip:
                    lat.append(min(e.elapsed_time(ev_c) for e in pre) * 1e3)
                    dep.append(min(e.elapsed_time(ev_f) for e in pre2) * 1e3)
            ccb.check(ccb.ccb_cnt_notify_destroy(h), "destroy")
            out[f"producers_{n}"] = {**stats(lat), "hip_event_dependency": stats(dep)}
        s = torch.cuda.Stream()
        kern = []
        for r in range(rounds):
            # the spin keeps the stream busy while the host enqueues, so that
            # e1 -> e2 is the kernel's launch and completion, not host time
            with torch.cuda.stream(s):
                torch.cuda._sleep(20000)
            e1 = ev(s)
            with torch.cuda.stream(s):
                torch.cuda._sleep(1)
            e2 = ev(s)
            e2.synchronize()
            if r >= skip:
                kern.append(e1.elapsed_time(e2) * 1e3)
        out["empty_kernel_between_events"] = stats(kern)
        self.extra["cntnotify_stream_notify_latency"] = out
        log(f"cntnotify stream notify latency: {out}")

    # ------------------------------------------------------------ parity record
    def parity_record(self):
        """Every configuration at full size: SHA-256 of its input arrays, of
        the GPU's outputs and of the oracle's (one host thread, timed).  The
        witness configurations have no input arrays: their values come from
        the seed inside the kernels."""
        import oracle
        np = self.np
        rec = {}

        def timed(fn):
            t1 = time.perf_counter()
            r = fn()
            return r, time.perf_counter() - t1

        # cfg 0: 8 workgroups x 64 threads, 100 rounds, seed 0 (run here)
        res = self.wl.slot_rounds(0, 100, 8, 64)
        (o0, _, c0, rc), t0 = timed(lambda: oracle.slot_rounds(0, 100, 8, 0))
        assert rc == 0 and res.counters == [c0] == [800]
        rec["cfg0"] = {"inputs": "seed 0 (no input arrays)",
                       "gpu_out_sha256": sha256_of(res.out.cpu().numpy()),
                       "oracle_out_sha256": sha256_of(o0), "oracle_one_thread_s": round(t0, 4)}
        w = self.inputs.WITNESS_GRID
        (o1, _, c1, rc), t1 = timed(lambda: oracle.slot_rounds(w["seed"], w["rounds"], w["n_wg"], 0))
        assert rc == 0
        rec["cfg1"] = {"inputs": "seed 1 (no input arrays)", "gpu_out_sha256": self.gpu_sha["cfg1"],
                       "oracle_out_sha256": sha256_of(o1), "oracle_one_thread_s": round(t1, 3)}
        st = self.inputs.STENCIL
        x = self.inputs.stencil_input(st["seed"], STENCIL_N)
        y, t2 = timed(lambda: oracle.stencil(x, STENCIL_ITERS))
        rec["cfg2"] = {"x_sha256": sha256_of(x), "gpu_out_sha256": self.gpu_sha["cfg2"],
                       "oracle_out_sha256": sha256_of(y), "oracle_one_thread_s": round(t2, 2)}
        c = self.inputs.CNT_BATCH
        val, meta, rows = self.inputs.cnt_batch_input(c["seed"], CNT_COUNTERS, CNT_OPS)
        (fin, rel, rc), t3 = timed(lambda: oracle.cnt_batch(val, meta, rows))
        assert rc == 0
        rec["cfg3"] = {"val_sha256": sha256_of(val), "meta_sha256": sha256_of(meta),
                       "gpu_final_sha256": self.gpu_sha["cfg3"][0],
                       "gpu_rel_sha256": self.gpu_sha["cfg3"][1],
                       "oracle_final_sha256": sha256_of(fin), "oracle_rel_sha256": sha256_of(rel),
                       "oracle_one_thread_s": round(t3, 3)}
        g = self.inputs.GROUPED
        (o4, _, c4, rc), t4 = timed(lambda: oracle.grouped_rounds(g["seed"], g["rounds"], g["n_wg"]))
        assert rc == 0
        rec["cfg4"] = {"inputs": "seed 4 (no input arrays)", "gpu_out_sha256": self.gpu_sha["cfg4"],
                       "oracle_out_sha256": sha256_of(o4), "oracle_one_thread_s": round(t4, 2)}
        for k, r in rec.items():
            gpu = [v for n, v in r.items() if n.startswith("gpu_")]
            ora = [v for n, v in r.items() if n.startswith("oracle_") and n.endswith("sha256")]
            r["match"] = gpu == ora
        self.extra["parity_record"] = rec
        self.oracle_times = {"cfg0_ns_per_barrier": round(t0 / 100 * 1e9, 1),
                             "cfg4_ns_per_round": round(t4 / g["rounds"] * 1e9, 1),
                             "stencil_64_iterations_s": round(t2, 2),
                             "stencil_64_iterations_GBs": round(
                                 STENCIL_BYTES_PER_ITER * STENCIL_ITERS / t2 / 1e9, 3)}
        log(f"parity record: { {k: r['match'] for k, r in rec.items()} }")
        assert all(r["match"] for r in rec.values()), rec

    # ------------------------------------------------------------ CPU baseline
    def cpu_baseline(self):
        import oracle
        cfg = self.inputs.WITNESS_GRID
        reps, t_cpu = 0, 0.0
        while t_cpu < 10.0 and reps < 1000:  # about 10 s of oracle work
            t1 = time.perf_counter()
            _, _, ctr, rc = oracle.slot_rounds(cfg["seed"], cfg["rounds"], cfg["n_wg"], 0)
            t_cpu += time.perf_counter() - t1
            reps += 1
            assert rc == 0 and ctr == cfg["rounds"] * cfg["n_wg"]
        return {"value": round(cfg["rounds"] * reps / t_cpu, 1), "unit": "barriers/s", "cores": 1,
                "kind": "oracle",
                "sample": f"{reps} full runs of the 256-workgroup, 10000-round witness simulation "
                          f"({t_cpu:.1f} s on one thread; the host has {os.cpu_count()} cores)"}


    def cpu_context(self):
        """Context beside the GPU figures (not baselines): the epoch barrier on
        host threads, and the oracle's stencil and batch engine on one core and
        on the host threads this GPU's share allows."""
        import oracle
        nproc = os.cpu_count() or 1
        model = ""
        try:
            with open("/proc/cpuinfo") as f:
                model = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), "")
        except OSError:
            pass
        threads = min(16, nproc)  # this GPU's share of the host
        _, ns, rc = oracle.host_barrier(threads, 20_000, 1)
        assert rc == 0
        x = self.inputs.stencil_input(self.inputs.STENCIL["seed"], STENCIL_N)
        t1 = time.perf_counter()
        y1 = oracle.stencil(x, 1)
        st_s = time.perf_counter() - t1
        c = self.inputs.CNT_BATCH
        val, meta, rows = self.inputs.cnt_batch_input(c["seed"], CNT_COUNTERS, CNT_OPS)
        t1 = time.perf_counter()
        fin1, _, rc = oracle.cnt_batch(val, meta, rows)
        cb_s = time.perf_counter() - t1
        assert rc == 0
        cnt_bytes = val.nbytes + meta.nbytes + CNT_COUNTERS * 4 + rows * CNT_COUNTERS
        # the same oracle calls on `threads` host threads (the C oracle runs
        # without the GIL): the stencil on slices with one element of halo on
        # each side (the slice ends are discarded, the array's own ends keep
        # their clamp), the batch engine on column ranges of its independent
        # counters.  The pieces must reproduce the one-thread results.
        from concurrent.futures import ThreadPoolExecutor
        np = self.np
        sb = np.linspace(0, STENCIL_N, threads + 1).astype(np.int64)

        def st_part(i):
            a, b = int(sb[i]), int(sb[i + 1])
            lo, hi = max(a - 1, 0), min(b + 1, STENCIL_N)
            return oracle.stencil(x[lo:hi], 1)[a - lo:a - lo + (b - a)]
        cb = np.linspace(0, CNT_COUNTERS, threads + 1).astype(np.int64)
        vparts = [np.ascontiguousarray(val[:, cb[i]:cb[i + 1]]) for i in range(threads)]
        mparts = [np.ascontiguousarray(meta[:, cb[i]:cb[i + 1]]) for i in range(threads)]
        with ThreadPoolExecutor(threads) as pool:
            t1 = time.perf_counter()
            yp = list(pool.map(st_part, range(threads)))
            st_par = time.perf_counter() - t1
            t1 = time.perf_counter()
            bp = list(pool.map(lambda i: oracle.cnt_batch(vparts[i], mparts[i], rows), range(threads)))
            cb_par = time.perf_counter() - t1
        assert np.array_equal(np.concatenate(yp), y1)
        assert all(r[2] == 0 for r in bp) and np.array_equal(np.concatenate([r[0] for r in bp]), fin1)
        self.extra["cpu_context"] = {
            "host": {"nproc": nproc, "cpu_model": model},
            "oracle_one_thread": getattr(self, "oracle_times", None),
            "host_thread_barrier": {"threads": threads, "ns_per_barrier": round(ns, 1),
                                    "rounds": 20_000},
            "oracle_stencil_one_iteration_GBs": round(STENCIL_BYTES_PER_ITER / st_s / 1e9, 3),
            "oracle_cnt_batch_GBs": round(cnt_bytes / cb_s / 1e9, 3),
            "oracle_on_threads": {
                "threads": threads,
                "stencil_one_iteration_GBs": round(STENCIL_BYTES_PER_ITER / st_par / 1e9, 3),
                "cnt_batch_GBs": round(cnt_bytes / cb_par / 1e9, 3)}}
        log(f"cpu context: {self.extra['cpu_context']}")


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the library runs each grid on a single MI355X)", file=sys.stderr)
        sys.exit(2)
    b = Bench(args)
    if args.only == "counters":
        gbs = b.copy_ceiling()
        roof = b.stencil(gbs)
        b.cnt_batch()
        print(json.dumps({"copy_512MiB_GBs": round(gbs, 1), "roofline": roof,
                          "cntnotify_batch": b.extra["cntnotify_batch"]}), flush=True)
        return

    if args.only == "barrier":
        floor = b.floor()
        b.latency(floor)
        b.barrier_breakdown(floor)
        b.barrier_breakdown(floor, "striped-full")
        b.barrier_breakdown(floor, "striped-xcd")
        b.fence_placement()
        b.full_visibility_witness()
        print(json.dumps({k: b.extra[k] for k in ("floor", "barrier_only_ns_at_256",
                                                   "barrier_only_ns_by_workgroups",
                                                   "tree_order_ns_by_workgroups",
                                                   "full_visibility_ns_by_workgroups",
                                                   "full_visibility_ns_per_round_with_witness",
                                                   "latency_roofline", "barrier_breakdown",
                                                   "fence_placement_at_256")}),
              flush=True)
        return

    if args.only == "cnt":
        b.cnt_stream_latency()
        b.cnt_graph()
        print(json.dumps({k: b.extra[k] for k in ("cntnotify_stream_notify_latency",
                                                   "cntnotify_record_wait_pair")}), flush=True)
        return

    ms_per_step, rounds = b.headline()
    value = rounds / (ms_per_step / 1e3)
    roofline = None
    cpu = None
    if not args.quick:
        floor = b.floor()
        b.latency(floor)
        b.barrier_breakdown(floor)
        b.barrier_breakdown(floor, "striped-full")
        b.barrier_breakdown(floor, "striped-xcd")
        b.fence_placement()
        b.full_visibility_witness()
        b.hip_grid_sync()
        b.gpu_sha["cfg4"] = b.grouped()
        gbs = b.copy_ceiling()
        roofline = b.stencil(gbs)
        b.cnt_batch()
        b.cnt_stream_latency()
        b.cnt_graph()
        if not args.no_cpu:
            cpu = b.cpu_baseline()
            b.parity_record()
            b.cpu_context()

    line = {
        "metric": "grid barriers/s (ns/barrier) at 256 WGs; data-phase HBM GB/s vs peak",
        "value": round(value, 1),
        "unit": "barriers/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u32",
        "data": "synthetic",
        "config": {"workload": "witness rounds: 256 workgroups x 256 threads (one per CU), "
                               "10000 rounds, usedCores=0, seed 1",
                   "barrier": args.mode, "ns_per_barrier": round(1e9 / value, 1)},
        "roofline": roofline,
        "cpu_baseline": cpu,
        **b.extra,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
