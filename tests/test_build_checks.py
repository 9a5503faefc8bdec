"""Checks on the compiled gfx950 code that need no GPU.

Several kernels order memory by hand, with s_waitcnt counts and M0 set in inline asm.
These tests read the assembly hipcc emits and check that:
  * the small-batch W4A16 kernel waits for its staged activations with a count that
    is no larger than the number of vector-memory instructions the compiler actually
    issued after the staging loads (it may merge adjacent loads);
  * every direct-to-LDS buffer load is directly preceded by the M0 write of its own asm
    block, and nothing else reads or writes M0;
  * every barrier wait of the persistent W4A4 / W8A8 pipeline (both its schedules),
    s_waitcnt vmcnt(N) + s_barrier, still covers the step it waits for on every path
    through the kernel (below);
  * no kernel spills to scratch memory (the hand-counted waits assume that no spill
    load or store is issued in between; spills would also cost bandwidth).
"""
import os
import re
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

from bit_floating_point_amd import build as B

SOURCES = ["gemm_w4a4.hip", "gemm_w4a16.hip", "gemm_f8f6.hip", "gemm_lut.hip", "quant.hip", "search.hip"]

pytestmark = pytest.mark.skipif(not os.path.exists(B.HIPCC), reason="hipcc not installed")


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    d = tmp_path_factory.mktemp("asm")

    def one(src):
        out = d / (src + ".s")
        cmd = [B.HIPCC] + B.CFLAGS + ["--cuda-device-only", "-S", os.path.join(B.CSRC, src), "-o", str(out)]
        subprocess.run(cmd, check=True, capture_output=True)
        return src, out.read_text()

    with ThreadPoolExecutor(4) as ex:
        return dict(ex.map(one, SOURCES))


def kernels(s, prefix):
    """(name, body) of every kernel whose mangled name starts with prefix."""
    for name in re.findall(r"^(" + prefix + r"\w*):", s, re.M):
        i = s.index(name + ":")
        yield name, s[i:s.index(".Lfunc_end", i)]


def instructions(body):
    """Instructions and block labels of a kernel body, comments and directives dropped."""
    out = []
    for line in body.split("\n")[1:]:
        t = line.split(";")[0].strip()
        if t and not (t.startswith(".") and not re.match(r"^\.LBB\w+:$", t)):
            out.append(t)
    return out


# ------------------------------------------------------------------ waits ---------
# Both schedules of the W4A4 kernel wait at a workgroup barrier (s_waitcnt vmcnt(N) ...;
# s_barrier) for the step whose direct-to-LDS loads were issued two load groups earlier:
# after those loads the wavefront has issued the loads of the next two steps (and, at a
# tile's start, the previous tile's output stores).  A load group is the direct-to-LDS
# loads between two consecutive barriers.  A thread's vector-memory operations complete
# in issue order, so the wait is sufficient exactly when at least N operations were issued
# after the last load of the third most recent group.  The check runs a forward data-flow
# pass over the kernel's control-flow graph that keeps, per path, the operations issued
# after each of the three most recent load groups, takes the minimum over all paths, and
# requires N <= that count for the third group at every barrier wait.  A full wait
# (vmcnt(0)) retires everything issued before it (SAFE).
# Paths the hardware cannot take are left out:
#   * exec-mask skips (s_cbranch_execz / execnz) are followed as by a wavefront with
#     active lanes: the tile loop runs with every lane active;
#   * branches on vcc computed from a constant flag register (s_mov_b64 s[a:b], -1 / 0,
#     then s_and_b64 / s_andn2_b64 vcc, exec, s[a:b]) follow the flag's value: the
#     compiler joins the two epilogue variants through such a flag.
SAFE = 10 ** 8
VMEM = re.compile(r"^(buffer_|global_|flat_|scratch_)")
LDS_LOAD = re.compile(r"^buffer_load_dword\S*\s.*\blds$")
M0_WRITE = re.compile(r"^s_(mov_b32|add_u32) m0, ")
NO_DST = ("s_waitcnt", "s_barrier", "s_branch", "s_cbranch", "s_endpgm", "buffer_store", "global_store",
          "flat_store", "scratch_store", "ds_write", "s_nop", "s_setprio", "s_sleep", "buffer_load", "s_cmp",
          "v_cmpx", "s_bitcmp", "s_setreg", "s_sendmsg")


def _blocks(ins):
    bl, cur, lab = [], [], None
    for t in ins:
        if re.match(r"^\.LBB\w+:$", t):
            if cur or lab is not None:
                bl.append((lab, cur))
            lab, cur = t[:-1], []
            continue
        cur.append(t)
        if t.startswith(("s_branch", "s_cbranch", "s_endpgm")):
            bl.append((lab, cur))
            lab, cur = None, []
    if cur or lab is not None:
        bl.append((lab, cur))
    return bl, {lab: i for i, (lab, _) in enumerate(bl) if lab}


def _regs(op):
    m = re.match(r"^s\[(\d+):(\d+)\]$", op)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"^s(\d+)$", op)
    if m:
        return {int(m.group(1))}
    return {"vcc"} if op in ("vcc", "vcc_lo", "vcc_hi") else set()


def _sat(x):
    return min(x, SAFE)


def _step(c, k, st, flags):
    """State after instruction c[k], and the (N, bound) of a barrier wait there.
    st = (a0, a1, a2, fresh): operations issued after the last load of the most recent,
    second and third most recent load group; fresh: a barrier came after the last load
    (the next load starts a new group)."""
    t = c[k]
    a0, a1, a2, fresh = st
    chk = None
    if LDS_LOAD.match(t):
        a0, a1, a2 = (0, _sat(a0 + 1), _sat(a1 + 1)) if fresh else (0, _sat(a1 + 1), _sat(a2 + 1))
        fresh = False
    elif VMEM.match(t):
        a0, a1, a2 = _sat(a0 + 1), _sat(a1 + 1), _sat(a2 + 1)
    m = re.match(r"^s_waitcnt vmcnt\((\d+)\)", t)
    if m:
        n = int(m.group(1))
        if n == 0:
            a0 = a1 = a2 = SAFE
        elif k + 1 < len(c) and c[k + 1] == "s_barrier":
            chk = (n, a2)
    if t == "s_barrier":
        fresh = True
    parts = t.split(None, 1)
    mn, ops = parts[0], ([o.strip() for o in parts[1].split(",")] if len(parts) > 1 else [])
    d = dict(flags)
    if mn in ("s_and_b64", "s_andn2_b64") and len(ops) == 3 and ops[0] == "vcc" and ops[1] == "exec" and ops[2] in d:
        nz = (d[ops[2]] == -1) if mn == "s_and_b64" else (d[ops[2]] == 0)
        d["vcc"] = "nz" if nz else "z"
    else:
        dst = _regs(ops[0]) if ops and not t.startswith(NO_DST) else set()
        if mn.startswith("v_cmp") and not mn.endswith("_e64"):
            dst |= {"vcc"}
        for key in [x for x in d if _regs(x) & dst]:
            del d[key]
        if mn == "s_mov_b64" and len(ops) == 2 and ops[1] in ("-1", "0") and ops[0].startswith("s["):
            d[ops[0]] = int(ops[1])
    return (a0, a1, a2, fresh), frozenset(d.items()), chk


def _successors(bl, idx, i, flags):
    c = bl[i][1]
    last = c[-1] if c else ""
    nxt = [i + 1] if i + 1 < len(bl) else []
    target = lambda: [idx[last.split()[1]]]  # noqa: E731
    if last.startswith("s_branch"):
        return target()
    if last.startswith("s_endpgm"):
        return []
    if last.startswith("s_cbranch_execz"):
        return nxt
    if last.startswith("s_cbranch_execnz"):
        return target()
    if last.startswith(("s_cbranch_vccz", "s_cbranch_vccnz")):
        d = dict(flags)
        if "vcc" in d:
            return target() if (d["vcc"] == "z") == last.startswith("s_cbranch_vccz") else nxt
        return target() + nxt
    if last.startswith("s_cbranch"):
        return target() + nxt
    return nxt


def barrier_waits(ins):
    """{(block, index): (N, fewest operations issued after the awaited load group)}."""
    bl, idx = _blocks(ins)
    state = [dict() for _ in bl]
    state[0][(frozenset(), True)] = (SAFE, SAFE, SAFE)
    work, res = [0], {}
    while work:
        i = work.pop()
        for (flags, fresh), cnt in list(state[i].items()):
            c, fl, st = bl[i][1], flags, cnt + (fresh,)
            for k in range(len(c)):
                st, fl, chk = _step(c, k, st, fl)
                if chk:
                    old = res.get((i, k))
                    res[(i, k)] = (chk[0], chk[1] if old is None else min(old[1], chk[1]))
            key, cnt2 = (fl, st[3]), st[:3]
            for j in _successors(bl, idx, i, fl):
                cur = state[j].get(key)
                new = cnt2 if cur is None else tuple(min(x, y) for x, y in zip(cur, cnt2))
                if new != cur:
                    state[j][key] = new
                    if j not in work:
                        work.append(j)
    return res


def m0_problems(ins):
    """Direct-to-LDS loads not directly after an M0 write, M0 writes not directly
    before such a load, and any other instruction that names M0."""
    bad = []
    for k, t in enumerate(ins):
        if LDS_LOAD.match(t):
            if k == 0 or not M0_WRITE.match(ins[k - 1]):
                bad.append(t)
        elif M0_WRITE.match(t):
            if k + 1 >= len(ins) or not LDS_LOAD.match(ins[k + 1]):
                bad.append(t)
        elif re.search(r"\bm0\b", t):
            bad.append(t)
    return bad


W4A4 = r"_ZN3fp415w4a4_fp4_kernel"  # E2M1 x E2M1, SwiGLU and FP8 E4M3 x E4M3 instances


def test_pipeline_barrier_waits_cover_their_step(asm):
    checked = 0
    for name, body in kernels(asm["gemm_w4a4.hip"], W4A4):
        res = barrier_waits(instructions(body))
        assert len(res) >= 8, (name, len(res))
        bad = {k: v for k, v in res.items() if v[0] > v[1]}
        assert not bad, (name, bad)
        checked += 1
    assert checked >= 8


def test_barrier_wait_check_catches_a_short_count(asm):
    """A wait raised above what its step allows, planted in the assembly text, fails."""
    name, body = next(kernels(asm["gemm_w4a4.hip"], W4A4))
    ins = instructions(body)
    waits = [(int(re.search(r"vmcnt\((\d+)\)", t).group(1)), i) for i, t in enumerate(ins)
             if re.match(r"^s_waitcnt vmcnt\([1-9]\d*\) lgkmcnt\(0\)$", t) and ins[i + 1] == "s_barrier"]
    n, k = min(waits)  # a steady-state wait of the main loop
    planted = ins[:k] + [f"s_waitcnt vmcnt({n + 20}) lgkmcnt(0)"] + ins[k + 1:]
    assert any(v[0] > v[1] for v in barrier_waits(planted).values())
    # an extra load between two barriers only makes the waits longer: still covered
    j = next(i for i, t in enumerate(ins) if LDS_LOAD.match(t))
    extra = ins[:j + 1] + ["global_load_dword v0, v[0:1], off"] + ins[j + 1:]
    assert not any(v[0] > v[1] for v in barrier_waits(extra).values())


def test_direct_to_lds_loads_own_m0(asm):
    seen = 0
    for src in ("gemm_w4a4.hip", "gemm_w4a16.hip", "gemm_f8f6.hip", "gemm_lut.hip"):
        for name, body in kernels(asm[src], r"_ZN3fp4"):
            ins = instructions(body)
            if any(LDS_LOAD.match(t) for t in ins):
                seen += 1
                assert not m0_problems(ins), (name, m0_problems(ins)[:4])
    assert seen >= 8
    # planted: an M0 write separated from its load
    name, body = next(kernels(asm["gemm_w4a4.hip"], W4A4))
    ins = instructions(body)
    j = next(i for i, t in enumerate(ins) if LDS_LOAD.match(t))
    assert m0_problems(ins[:j] + ["v_mov_b32_e32 v0, v1"] + ins[j:])


def test_no_kernel_spills(asm):
    for src, s in asm.items():
        for m in re.finditer(r"\.amdhsa_kernel (\S+)\n(.*?)\.end_amdhsa_kernel", s, re.S):
            size = int(re.search(r"\.amdhsa_private_segment_fixed_size (\d+)", m.group(2)).group(1))
            assert size == 0, (src, m.group(1), size)


def test_small_kernel_waits_are_lower_bounds(asm):
    s = asm["gemm_w4a16.hip"]
    names = re.findall(r"^(_ZN3fp418w4a16_small_kernel\w+):", s, re.M)
    assert len(names) > 40
    for name in names:
        body = s[s.index(name + ":"):s.index(".Lfunc_end", s.index(name + ":"))]
        loads, first = 0, None
        for line in body.split("\n"):
            t = line.strip()
            if t.startswith("buffer_load") and " lds" not in t:
                loads += 1
            m = re.match(r"s_waitcnt vmcnt\((\d+)\)", t)
            if m:
                first = int(m.group(1))
                break
        assert first is not None and first <= loads, (name, loads, first)
