"""Fence review of the library's own gfx950 code (CPU only, no GPU).

The kernels are compiled to assembly with exactly the library's flags and
checked against the code sequences of LLVM's AMDGPU memory model for the
GFX942 family, which gfx950 follows:
  - a release fence at agent scope is `buffer_wbl2 sc1` (write back L2)
    followed by `s_waitcnt vmcnt(0)`;
  - an acquire fence at agent scope is `buffer_inv sc1` (invalidate L2);
  - a relaxed atomic load or store at agent scope carries `sc1`.

What is checked, for every persistent kernel (barrier-only, witness rounds,
grouped rounds, stencil; 64 stripes, one counter, and the two-level tree of
8 group counters):
  - full visibility: the arrival (the returning fetch-add) comes right after
    a release sequence with no memory access in between, and an acquire
    follows the poll;
  - ordering-only visibility: no L2 write-back or invalidate at all (the
    workgroup's own accesses are waited for instead), the poll loads are
    agent-scope, and the data the kernel shares across the barrier (witness
    slots, halo words) is stored with agent-scope stores;
  - the first poll load goes out only after a wait for the arrival's reply
    (a poll issued behind the wave's own arrival doubles the barrier's cost);
  - tree, full visibility: the group completer's arrival on the top counter
    (a non-returning atomic) comes right after an acquire-release sequence
    (`buffer_wbl2 sc1` then `buffer_inv sc1`), so the group's released
    stores reach the top counter's pollers through it;
  - per-XCD write-back: the registration on the XCD (a returning fetch-add
    on the count words) is waited for before the first arrival; the XCD
    flag is stored with an agent-scope store right after a release sequence
    (the leader's L2 write-back), with no memory access in between; an
    acquire follows the flag poll; and there is no write-back right before
    an arrival (that is the per-workgroup placement this mode replaces);
and for every kernel in the file: every L2 write-back is followed by an
`s_waitcnt vmcnt(0)` before the next memory access (the compiler drops the
memory model's wait where it tracks nothing else in flight, so the library
waits explicitly; HIP's own grid sync, timed beside the barrier, is left as
HIP compiles it), no write through the scalar data cache and no packed-FP32
arithmetic.
"""

import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

KINDS = ("barrier_only", "slot_rounds", "grouped_rounds", "stencil")
MEM_PREFIXES = ("global_", "buffer_", "flat_", "scratch_")


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    from cross_core_barrier_amd import build
    out = str(tmp_path_factory.mktemp("isa") / "ccb_kernels.s")
    build.device_assembly(out)
    with open(out) as f:
        return f.read()


def _device_header():
    with open(os.path.join(ROOT, "include", "ccb_device.h")) as f:
        return f.read()


@pytest.fixture(scope="module")
def vis_codes():
    """CCB_VIS_FULL / CCB_VIS_ORDER / CCB_VIS_XCD as the device header defines them."""
    text = _device_header()
    full = int(re.search(r"CCB_VIS_FULL\s*=\s*(\d+)", text).group(1))
    order = int(re.search(r"CCB_VIS_ORDER\s*=\s*(\d+)", text).group(1))
    xcd = int(re.search(r"CCB_VIS_XCD\s*=\s*(\d+)", text).group(1))
    return {full: "full", order: "order", xcd: "xcd"}


def _registration_offset():
    """Byte offset of the per-XCD count words from the workspace base: the
    immediate offset of the registration fetch-add."""
    text = _device_header()
    line_words = 128 // 4
    expr = re.search(r"#define CCB_XCD_COUNT_WORD \((.*)\)", text).group(1)
    return 4 * eval(expr.replace("CCB_LINE_WORDS", str(line_words)), {})


def _functions(asm_text):
    """{mangled name: [instruction lines]} for every function in the file."""
    parts = re.split(r"\n(_Z\w+):[^\n]*\n", asm_text)
    out = {}
    for i in range(1, len(parts) - 1, 2):
        body = parts[i + 1].split(".Lfunc_end")[0]
        out[parts[i]] = [l.strip() for l in body.split("\n")
                         if l.startswith("\t") and l.strip() and not l.strip().startswith((".", ";"))]
    return out


def _persistent(asm_text, vis_codes):
    """{(kind, counter layout K, visibility): instructions} of the persistent
    kernels; K < 0 is the tree of -K groups (mangled as Lin8E)."""
    found = {}
    for name, ins in _functions(asm_text).items():
        m = re.match(r"_Z\d+ccb_k_(\w+?)ILi(n?\d+)EL\d+ccbVisibility(\d+)E", name)
        if m and m.group(1) in KINDS:
            k = m.group(2)
            k = -int(k[1:]) if k.startswith("n") else int(k)
            found[(m.group(1), k, vis_codes[int(m.group(3))])] = ins
    return found


def _op(line):
    return line.split()[0]


def _is_mem(line):
    return _op(line).startswith(MEM_PREFIXES)


def _registrations(ins):
    """Per-XCD write-back: the returning fetch-adds on the XCD count words."""
    off = f"offset:{_registration_offset()} "
    return [i for i, l in enumerate(ins)
            if _op(l) == "global_atomic_add" and " sc0" in l and off in l + " "]


def _arrivals(ins):
    reg = set(_registrations(ins))
    return [i for i, l in enumerate(ins)
            if _op(l) == "global_atomic_add" and " sc0" in l and i not in reg]


def _top_arrivals(ins):
    """The tree's arrivals on the top counter: fetch-adds whose reply is unused."""
    return [i for i, l in enumerate(ins) if _op(l) == "global_atomic_add" and " sc0" not in l]


def test_every_persistent_kernel_present(asm, vis_codes):
    found = _persistent(asm, vis_codes)
    want = {(k, s, v) for k in KINDS for s in (1, 64, -8) for v in ("full", "order", "xcd")}
    assert set(found) == want
    for key, ins in found.items():
        assert _arrivals(ins), f"{key}: no returning fetch-add (the arrival)"


# --- the checks: each returns the problems it finds (empty = passes) ------------

def _check_release(found):
    bad = []
    for key, ins in found.items():
        if key[2] != "full":
            continue
        for a in _arrivals(ins):
            waited = False
            j = a - 1
            while j >= 0 and not _is_mem(ins[j]):
                if _op(ins[j]) == "s_waitcnt" and "vmcnt(0)" in ins[j]:
                    waited = True
                j -= 1
            if not (j >= 0 and ins[j] == "buffer_wbl2 sc1"):
                bad.append(f"{key}: the access before the arrival is {ins[j] if j >= 0 else None!r}")
            elif not waited:
                bad.append(f"{key}: no s_waitcnt vmcnt(0) between the write-back and the arrival")
    return bad


def _check_acquire(found):
    """Full visibility: an acquire (buffer_inv sc1) after the last agent-scope
    load, i.e. after the poll loop."""
    bad = []
    for key, ins in found.items():
        if key[2] != "full":
            continue
        polls = [i for i, l in enumerate(ins) if _op(l).startswith("global_load") and " sc1" in l]
        inv = [i for i, l in enumerate(ins) if l == "buffer_inv sc1"]
        if not polls or not inv or max(inv) < max(polls):
            bad.append(f"{key}: no agent-scope acquire after the poll")
    return bad


def _prev_mem(ins, i):
    """Index of the last memory access before i (-1: none), and whether an
    s_waitcnt vmcnt(0) lies between it and i."""
    waited = False
    j = i - 1
    while j >= 0 and not _is_mem(ins[j]):
        if _op(ins[j]) == "s_waitcnt" and "vmcnt(0)" in ins[j]:
            waited = True
        j -= 1
    return j, waited


def _check_xcd(found):
    """Per-XCD write-back: registration waited for before the arrival; the
    flag store right after the leader's release; an acquire after the flag
    poll; no write-back right before an arrival."""
    bad = []
    for key, ins in found.items():
        if key[2] != "xcd":
            continue
        regs = _registrations(ins)
        if not regs:
            bad.append(f"{key}: no registration on the XCD")
        for a in _arrivals(ins):
            j, waited = _prev_mem(ins, a)
            if j >= 0 and ins[j] == "buffer_wbl2 sc1":
                bad.append(f"{key}: a write-back right before the arrival")
            if j in regs and not waited:
                bad.append(f"{key}: the arrival does not wait for the registration")
        flag_stores = []
        for i, l in enumerate(ins):
            if _op(l) == "buffer_wbl2":
                k = i + 1
                waited = False
                while k < len(ins) and not _is_mem(ins[k]):
                    if _op(ins[k]) == "s_waitcnt" and "vmcnt(0)" in ins[k]:
                        waited = True
                    k += 1
                if k < len(ins) and _op(ins[k]).startswith("global_store") and " sc1" in ins[k] \
                        and waited and l == "buffer_wbl2 sc1":
                    flag_stores.append(k)
        if not flag_stores:
            bad.append(f"{key}: no agent-scope flag store right after a release")
        polls = [i for i, l in enumerate(ins) if _op(l).startswith("global_load") and " sc1" in l]
        inv = [i for i, l in enumerate(ins) if l == "buffer_inv sc1"]
        if not polls or not inv or max(inv) < max(polls):
            bad.append(f"{key}: no agent-scope acquire after the flag poll")
    return bad


def _check_writeback_waits(funcs):
    """Every buffer_wbl2 is followed by s_waitcnt vmcnt(0) before the next
    memory access."""
    bad = []
    for name, ins in funcs.items():
        if "hip_grid_sync" in name:
            continue  # HIP's cooperative-groups grid sync, not library code
        for k, l in enumerate(ins):
            if _op(l) != "buffer_wbl2":
                continue
            j = k + 1
            waited = False
            while j < len(ins) and not _is_mem(ins[j]):
                if _op(ins[j]) == "s_waitcnt" and "vmcnt(0)" in ins[j]:
                    waited = True
                j += 1
            if not waited:
                bad.append(f"{name}: {ins[j] if j < len(ins) else None!r} right after a write-back")
    return bad


def _check_tree_top(found):
    bad = []
    for key, ins in found.items():
        if key[1] >= 0:
            continue
        tops = _top_arrivals(ins)
        if not tops:
            bad.append(f"{key}: no arrival on the top counter")
        if key[2] != "full":
            continue
        for t in tops:
            j = t - 1
            while j >= 0 and not _is_mem(ins[j]):
                j -= 1
            if not (j >= 1 and ins[j] == "buffer_inv sc1"):
                bad.append(f"{key}: the access before the top arrival is "
                           f"{ins[j] if j >= 0 else None!r}")
                continue
            j -= 1
            while j >= 0 and not _is_mem(ins[j]):
                j -= 1
            if not (j >= 0 and ins[j] == "buffer_wbl2 sc1"):
                bad.append(f"{key}: no write-back ahead of the top arrival's acquire")
    return bad


def _check_first_poll(found):
    bad = []
    for key, ins in found.items():
        if key[0] != "barrier_only":
            continue  # the rounds kernels overlap their own data loads with the arrival
        for a in _arrivals(ins):
            j = a + 1
            waited = False
            while j < len(ins) and not _is_mem(ins[j]):
                if _op(ins[j]) == "s_waitcnt" and "vmcnt(0)" in ins[j]:
                    waited = True
                j += 1
            if key[1] < 0:
                # full visibility: the completer's acquire-release comes
                # first (its own check)
                while j < len(ins) and (_op(ins[j]) in ("buffer_wbl2", "buffer_inv")
                                        or not _is_mem(ins[j])):
                    j += 1
            if key[1] < 0 and j < len(ins) and j in _top_arrivals(ins):
                # a tree: a group's completer first arrives on the top counter
                # (whose reply nothing waits for), then polls
                if not waited:
                    bad.append(f"{key}: the top arrival does not wait for the group's reply")
                j += 1
                while j < len(ins) and not _is_mem(ins[j]):
                    j += 1
            if not (j < len(ins) and _op(ins[j]).startswith("global_load") and " sc1" in ins[j]):
                bad.append(f"{key}: the access after the arrival is "
                           f"{ins[j] if j < len(ins) else None!r}")
            elif not waited:
                bad.append(f"{key}: the first poll does not wait for the arrival's reply")
    return bad


def test_full_visibility_release_before_arrival_acquire_after_poll(asm, vis_codes):
    found = _persistent(asm, vis_codes)
    assert _check_release(found) == []
    assert _check_acquire(found) == []


def test_every_writeback_is_waited_for(asm):
    assert _check_writeback_waits(_functions(asm)) == []


def test_xcd_registration_release_flag_acquire(asm, vis_codes):
    assert _check_xcd(_persistent(asm, vis_codes)) == []


def test_tree_full_top_arrival_after_acquire_release(asm, vis_codes):
    assert _check_tree_top(_persistent(asm, vis_codes)) == []


def test_order_visibility_has_no_cache_maintenance(asm, vis_codes):
    for key, ins in _persistent(asm, vis_codes).items():
        if key[2] != "order":
            continue
        maint = [l for l in ins if _op(l) in ("buffer_wbl2", "buffer_inv")]
        assert maint == [], f"{key}: {maint}"


def test_order_visibility_shares_data_through_agent_scope_accesses(asm, vis_codes):
    for key, ins in _persistent(asm, vis_codes).items():
        if key[2] != "order":
            continue
        first = min(_arrivals(ins))
        polls = [l for l in ins[first:] if _op(l).startswith("global_load") and " sc1" in l]
        assert polls, f"{key}: no agent-scope load after the arrival"
        if key[0] == "barrier_only":
            continue  # shares no data
        # witness slots (rounds kernels), halo words (stencil)
        stores = [l for l in ins if _op(l).startswith("global_store") and " sc1" in l]
        assert stores, f"{key}: no agent-scope store for the data shared across the barrier"


def test_first_poll_waits_for_the_arrivals_reply(asm, vis_codes):
    assert _check_first_poll(_persistent(asm, vis_codes)) == []


# --- negative controls: a copy of the device header with one fence taken out
# (or the first poll moved ahead of the reply), compiled the same way; the
# check that guards that step must find it.

NEGATIVE = {
    "no_release": (
        [("if (kVis == CCB_VIS_FULL) ccb_fence_release_agent();", "")],
        _check_release),
    "no_acquire": (
        [('if (kVis == CCB_VIS_FULL) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");', "")],
        _check_acquire),
    "no_tree_acquire_release": (
        [("if (kVis == CCB_VIS_FULL) {\n            ccb_fence_release_agent();\n"
          "            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, \"agent\");\n        }", "")],
        _check_tree_top),
    "writeback_wait_left_to_the_compiler": (
        [('    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");\n    ccb_wait_memory();\n}',
          '    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");\n}')],
        None),
    "no_xcd_leader_release": (
        [("if (team.leader) {\n            ccb_fence_release_agent();", "if (team.leader) {")],
        _check_xcd),
    "no_xcd_acquire": (
        [("            if (CCB_POLL_SLEEP > 0) __builtin_amdgcn_s_sleep(CCB_POLL_SLEEP);\n"
          "        }\n"
          "        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, \"agent\");",
          "            if (CCB_POLL_SLEEP > 0) __builtin_amdgcn_s_sleep(CCB_POLL_SLEEP);\n"
          "        }")],
        _check_xcd),
    "poll_before_reply": (
        [("const int32_t b = __shfl(before, 0, 64);\n"
          "        __builtin_amdgcn_sched_barrier(0x44F);\n"
          "        hook.reply();\n"
          "        const int32_t v0 = __hip_atomic_load(mine, __ATOMIC_RELAXED, "
          "__HIP_MEMORY_SCOPE_AGENT);",
          "const int32_t v0 = __hip_atomic_load(mine, __ATOMIC_RELAXED, "
          "__HIP_MEMORY_SCOPE_AGENT);\n"
          "        __builtin_amdgcn_sched_barrier(0);\n"
          "        const int32_t b = __shfl(before, 0, 64);\n"
          "        hook.reply();")],
        _check_first_poll),
}


@pytest.mark.slow
@pytest.mark.parametrize("name", sorted(NEGATIVE))
def test_negative_control_is_caught(name, tmp_path, vis_codes):
    import shutil
    import subprocess
    from cross_core_barrier_amd import build
    inc = tmp_path / "include"
    shutil.copytree(os.path.join(ROOT, "include"), inc)
    hdr = inc / "ccb_device.h"
    text = hdr.read_text()
    edits, check = NEGATIVE[name]
    for old, new in edits:
        assert text.count(old) >= 1, f"{name}: the header no longer has {old!r}"
        text = text.replace(old, new)
    hdr.write_text(text)
    flags = list(build.CODE_FLAGS)
    flags[flags.index(os.path.join(ROOT, "include"))] = str(inc)
    out = str(tmp_path / "k.s")
    cmd = ["hipcc", *flags, "-S", "--cuda-device-only", "-o", out,
           os.path.join(build.CSRC, "ccb_kernels.hip")]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    with open(out) as f:
        text = f.read()
    if check is None:  # a check over every function
        assert _check_writeback_waits(_functions(text)) != [], f"{name}: not noticed"
        return
    found = _persistent(text, vis_codes)
    assert check(found) != [], f"{name}: {check.__name__} does not notice"


def test_no_scalar_cache_writes_and_no_packed_fp32(asm):
    banned_prefix = ("s_store", "s_buffer_store", "s_scratch_store", "s_atomic", "s_buffer_atomic",
                     "s_dcache_wb", "s_dcache_discard")
    banned = {"v_pk_add_f32", "v_pk_mul_f32", "v_pk_fma_f32"}
    funcs = _functions(asm)
    assert len(funcs) >= 20
    for name, ins in funcs.items():
        bad = [l for l in ins if _op(l).startswith(banned_prefix) or _op(l) in banned]
        assert bad == [], f"{name}: {bad[:3]}"
