"""Static check of the prefill kernels' device code: the destination registers of
a global load issued as inline asm (not counted by the compiler) must not be read
or written by any instruction before the next vector-memory wait.  A violation
means the compiler moved or reused registers of a load still in flight (silent
corruption, or an address overwritten by late data).

The scan follows fall-through order from each load up to the next `s_waitcnt
vmcnt`, and the target of an unconditional branch.  A conditional branch is passed
by falling through, except where it certainly goes the other way: the load's block
is the fall-through of a branch on `vcc = exec & sX` with sX a uniform boolean
(`s_cselect_b64 sX, -1, 0`), so sX is known on entry, and a later branch on a vcc
formed from the same, unwritten sX is then taken for certain -- the scan follows
its target instead of a fall-through path that cannot run.

A second check: the tile kernels hold no LDS atomic and no loop over the lanes of a
wave on the scalar unit (what the compiler makes of an atomic with a divergent
operand: find the first active lane, read its value, fold it in, clear the lane,
repeat).  The CU's waves share the scalar unit, so a few such loops per wave
stall every workgroup for microseconds."""
import os
import re
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "..", "paged_kv_attention_table_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["-O3", "-std=c++17", "--offload-arch=gfx950", "-fno-fast-math", "-Xclang", "-target-feature", "-Xclang",
         "-packed-fp32-ops", "--cuda-device-only", "-S"]


SOURCES = ("pa_prefill_bf16.hip", "pa_prefill_f16.hip", "pa_prefill_fp8_bf16.hip", "pa_prefill_fp8_f16.hip",
           "pa_fused_bf16.hip", "pa_fused_f16.hip", "pa_fused_fp8_bf16.hip", "pa_fused_fp8_f16.hip")


@pytest.fixture(scope="module")
def device_asm(tmp_path_factory):
    """The device assembly of every source above, compiled in parallel."""
    if shutil.which(HIPCC) is None and not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    d = tmp_path_factory.mktemp("asm")

    def build(src):
        out = d / (src + ".s")
        subprocess.run([HIPCC, *FLAGS, os.path.join(CSRC, src), "-o", str(out)], check=True, capture_output=True)
        return src, out.read_text()

    with ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as ex:
        return dict(ex.map(build, SOURCES))


def vgprs(tok):
    m = re.match(r"v\[(\d+):(\d+)\]", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"v(\d+)$", tok)
    return {int(m.group(1))} if m else set()


def sgprs(tok):
    m = re.match(r"s\[(\d+):(\d+)\]", tok)
    if m:
        return frozenset(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"s(\d+)$", tok)
    return frozenset({int(m.group(1))}) if m else frozenset()


# scalar instructions whose first operand is not a destination
_NO_SDST = ("s_cmp", "s_bitcmp", "s_cbranch", "s_branch", "s_waitcnt", "s_barrier", "s_nop", "s_setprio", "s_sleep",
            "s_sched", "s_endpgm", "s_store", "s_dcache", "s_wait", "s_setreg", "s_trap", "s_ttrace", "s_icache")


def _label(t):
    """The label a line defines (".LBB3_7:", possibly followed by a comment), or None."""
    m = re.match(r"(\.L[\w.]+):", t)
    return m.group(1) if m else None


def _parse(t):
    parts = t.split(None, 1)
    ops = [o.strip().split()[0] for o in parts[1].split(",") if o.strip()] if len(parts) > 1 else []
    return parts[0], ops


def _sgpr_dst(op, ops):
    """The SGPRs an instruction writes (its first operand, where that is one)."""
    if not ops:
        return frozenset()
    if (op.startswith("s_") and not op.startswith(_NO_SDST)) or op.startswith(("v_readlane", "v_readfirstlane")) \
            or (op.startswith("v_cmp") and op.endswith("_e64")):
        return sgprs(ops[0])
    return frozenset()


def _writes_vcc(op, ops):
    return (ops[:1] == ["vcc"] and not op.startswith("s_cbranch")) or (op.startswith("v_cmp") and op.endswith("_e32")) \
        or op.startswith(("v_add_co", "v_sub_co", "v_subrev_co", "v_addc", "v_subb"))


def _vcc_from(op, ops):
    """(kind, sX) for vcc = exec & sX ("and") or exec & ~sX ("andn2"), else None."""
    if op in ("s_and_b64", "s_andn2_b64") and len(ops) == 3 and ops[0] == "vcc" and ops[1] == "exec" and sgprs(ops[2]):
        return ("and" if op == "s_and_b64" else "andn2", sgprs(ops[2]))
    return None


def _entry_knowledge(lines, n):
    """What the path into the block holding line n fixes: {sX: True (all ones) | False
    (zero)} when that block is entered only by falling through a vcc branch whose vcc
    came from a uniform boolean sX that nothing writes before line n."""
    j = n - 1
    while j >= 0:
        t = lines[j]
        if _label(t):
            return {}  # a label: other predecessors
        if t and not t.startswith(";"):
            op, ops = _parse(t)
            if op.startswith("s_branch") or op == "s_endpgm":
                return {}
            if op.startswith("s_cbranch"):
                break
        j -= 1
    else:
        return {}
    op, _ = _parse(lines[j])
    if op not in ("s_cbranch_vccz", "s_cbranch_vccnz"):
        return {}
    between = [_parse(t) for t in lines[j + 1:n] if t and not t.startswith((";", "."))]
    k = j - 1
    while k >= 0 and (not lines[k] or lines[k].startswith(";")):
        k -= 1
    if k < 0:
        return {}
    src = _vcc_from(*_parse(lines[k]))
    if src is None:
        return {}
    kind, sx = src
    if any(_sgpr_dst(o, a) & sx for o, a in between):
        return {}
    d = k - 1  # sX must be a uniform boolean: its last definition an s_cselect_b64 sX, -1, 0
    while d >= 0:
        t = lines[d]
        if _label(t):
            return {}
        if t and not t.startswith(";"):
            o, a = _parse(t)
            if _sgpr_dst(o, a) & sx:
                if o == "s_cselect_b64" and a[1:3] == ["-1", "0"] and sgprs(a[0]) == sx:
                    break
                return {}
        d -= 1
    else:
        return {}
    # falling through vccz: vcc != 0; "and": sX != 0, so all ones; "andn2": ~sX != 0, so zero.
    # Falling through vccnz (vcc == 0) fixes nothing (exec may be zero).
    if op == "s_cbranch_vccz":
        return {sx: kind == "and"}
    return {}


def untracked_load_hazards(asm, kernel):
    i = asm.index(kernel + ":")
    lines = [ln.strip() for ln in asm[i:asm.index(".Lfunc_end", i)].split("\n")]
    labels = {_label(t): n for n, t in enumerate(lines) if _label(t)}
    loads, bad = 0, []
    for n, ln in enumerate(lines):
        # the asm loads use a scalar base (saddr form); the compiler's own use a VGPR pair
        if not ln.startswith("global_load_dwordx4") or ", s[" not in ln:
            continue
        loads += 1
        dst = vgprs(ln.split()[1].rstrip(","))
        known = _entry_knowledge(lines, n)
        vsrc = None
        hit = None
        j, steps = n + 1, 0
        while j < len(lines) and steps < 100000:
            steps += 1
            t = lines[j]
            if not t or t.startswith((";", ".")):
                j += 1
                continue
            op, ops = _parse(t)
            if (op.startswith("s_waitcnt") and "vmcnt" in t) or op == "s_endpgm":
                break
            if any(vgprs(o) & dst for o in ops):
                hit = (ln, t)
                break
            w = _sgpr_dst(op, ops)
            if w:
                known = {k: v for k, v in known.items() if not (k & w)}
                if vsrc is not None and vsrc[1] & w:
                    vsrc = None
            src = _vcc_from(op, ops)
            if src is not None:
                vsrc = src
            elif _writes_vcc(op, ops):
                vsrc = None
            if op == "s_branch":
                j = labels[ops[0]]
                continue
            if op == "s_cbranch_vccz" and vsrc is not None and vsrc[1] in known and \
                    ((vsrc[0] == "and" and not known[vsrc[1]]) or (vsrc[0] == "andn2" and known[vsrc[1]])):
                j = labels[ops[0]]  # vcc is certainly zero: the branch is taken
                continue
            j += 1
        if hit is not None:
            bad.append(hit)
    return loads, bad


# Hand-written fragments that pin the scan itself: a read of a load's registers on a
# feasible path is found, on a path the load's own guard rules out is not, and one
# reached only through a branch target is found.
_FRAGMENTS = {
    "straight": ("""k:
\ts_cselect_b64 s[10:11], -1, 0
\ts_and_b64 vcc, exec, s[10:11]
\ts_cbranch_vccz .LB1
\tglobal_load_dwordx4 v[8:11], v2, s[0:1]
.LB1:
\tv_mov_b32_e32 v3, v9
\ts_waitcnt vmcnt(0)
\ts_endpgm
.Lfunc_end0:
""", 1),
    "guarded": ("""k:
\ts_cselect_b64 s[10:11], -1, 0
\ts_and_b64 vcc, exec, s[10:11]
\ts_cbranch_vccz .LB1
\tglobal_load_dwordx4 v[8:11], v2, s[0:1]
.LB1:
\ts_andn2_b64 vcc, exec, s[10:11]
\ts_cbranch_vccz .LB2
\tds_read_b128 v[8:11], v4
.LB2:
\ts_waitcnt vmcnt(0)
\ts_endpgm
.Lfunc_end0:
""", 0),
    "guard rewritten": ("""k:
\ts_cselect_b64 s[10:11], -1, 0
\ts_and_b64 vcc, exec, s[10:11]
\ts_cbranch_vccz .LB1
\tglobal_load_dwordx4 v[8:11], v2, s[0:1]
.LB1:
\ts_cselect_b64 s[10:11], -1, 0
\ts_andn2_b64 vcc, exec, s[10:11]
\ts_cbranch_vccz .LB2
\tds_read_b128 v[8:11], v4
.LB2:
\ts_waitcnt vmcnt(0)
\ts_endpgm
.Lfunc_end0:
""", 1),
    "through a branch": ("""k:
\tglobal_load_dwordx4 v[8:11], v2, s[0:1]
\ts_branch .LB3
\tv_mov_b32_e32 v3, v1
\ts_waitcnt vmcnt(0)
.LB3:
\tv_add_u32_e32 v10, v1, v1
\ts_waitcnt vmcnt(0)
\ts_endpgm
.Lfunc_end0:
""", 1),
}


@pytest.mark.parametrize("name", sorted(_FRAGMENTS))
def test_scan_on_fragments(name):
    asm, want = _FRAGMENTS[name]
    loads, bad = untracked_load_hazards(asm, "k")
    assert loads == 1 and len(bad) == want, bad


@pytest.mark.parametrize("src,tname,kv8", [("pa_prefill_bf16.hip", "4BF16", "0"), ("pa_prefill_f16.hip", "3F16", "0"),
                                           ("pa_prefill_fp8_bf16.hip", "4BF16", "1"),
                                           ("pa_prefill_fp8_f16.hip", "3F16", "1")])
def test_no_register_reuse_under_inflight_loads(device_asm, src, tname, kv8):
    """16-bit caches (K straight to LDS, V through registers) and fp8 caches (K and V
    through registers)."""
    asm = device_asm[src]
    # ALiBi; merged into a prior state; two key segments (without ALiBi)
    flags = [(a, m, "0") for a in "01" for m in "01"] + [("0", m, "1") for m in "01"]
    for dims in ("128ELi128", "192ELi128") + (("64ELi64",) if kv8 == "0" else ()):
        for alibi, merge, seg2 in flags:
            kernel = (f"_ZN2pa14prefill_kernelINS_{tname}ELi{dims}ELb{alibi}ELb{merge}ELb{seg2}ELb{kv8}"
                      "EEEvNS_11PrefillArgsE")
            loads, bad = untracked_load_hazards(asm, kernel)
            assert loads > 0, kernel
            assert not bad, f"{kernel}: {bad[:3]}"


@pytest.mark.parametrize("src,tname,f8", [("pa_fused_bf16.hip", "4BF16", "0"), ("pa_fused_f16.hip", "3F16", "0"),
                                          ("pa_fused_fp8_bf16.hip", "4BF16", "1"),
                                          ("pa_fused_fp8_f16.hip", "3F16", "1")])
def test_fused_varlen_kernel_no_register_reuse(device_asm, src, tname, f8):
    """The fused varlen kernel carries the prefill tile loop (head dim 128) beside
    the decode rows: the same check on it."""
    asm = device_asm[src]
    for alibi, merge in (("0", "0"), ("1", "0"), ("0", "1"), ("1", "1")):
        kernel = (f"_ZN2pa19varlen_fused_kernelINS_{tname}ELb{alibi}ELb{merge}ELb{f8}"
                  "EEEvNS_11PrefillArgsENS_8RowsArgsEij")
        loads, bad = untracked_load_hazards(asm, kernel)
        assert loads > 0, kernel
        assert not bad, f"{kernel}: {bad[:3]}"


_LDS_ATOMIC = re.compile(r"ds_(min|max|add|sub|rsub|inc|dec|and|or|xor|wrxchg|cmpst|cmpswap)_")


def lane_serial_loops(asm, kernel):
    """(LDS atomics, lane-serial loops) of a kernel.  A loop runs from a label the
    compiler marks as a loop header to the first branch back to it; it is
    lane-serial when it finds the first set bit of a lane mask (s_ff1_i32_b64)."""
    i = asm.index(kernel + ":")
    lines = [ln.strip() for ln in asm[i:asm.index(".Lfunc_end", i)].split("\n")]
    atomics = [ln for ln in lines if _LDS_ATOMIC.match(ln)]
    loops = []
    for n, ln in enumerate(lines):
        lab = _label(ln)
        if lab is None or "Loop Header" not in ln:
            continue
        for m in range(n + 1, len(lines)):
            op, ops = _parse(lines[m]) if lines[m] else ("", [])
            if op.startswith(("s_cbranch", "s_branch")) and ops and ops[-1] == lab:
                if any(t.startswith("s_ff1_i32_b64") for t in lines[n + 1:m]):
                    loops.append(lab)
                break
    return atomics, loops


_LOOP_FRAGMENTS = {
    # an LDS min over divergent lanes, as the compiler expands it
    "lane loop": ("""k:
\ts_mov_b64 s[12:13], exec
\ts_brev_b32 s20, -2
.LBB3_40:                               ; =>This Inner Loop Header: Depth=1
\ts_ff1_i32_b64 s21, s[12:13]
\tv_readlane_b32 s24, v212, s21
\ts_lshl_b64 s[22:23], 1, s21
\ts_min_i32 s20, s20, s24
\ts_andn2_b64 s[12:13], s[12:13], s[22:23]
\ts_cmp_lg_u64 s[12:13], 0
\ts_cbranch_scc1 .LBB3_40
\tv_mov_b32_e32 v37, s20
\tds_min_i32 v36, v37 offset:52224
\ts_endpgm
.Lfunc_end0:
""", 1, 1),
    # a find-first-lane outside any loop, and a loop without one
    "single ff1, plain loop": ("""k:
\ts_ff1_i32_b64 s4, vcc
.LBB0_2:                                ; =>This Inner Loop Header: Depth=1
\tv_add_u32_e32 v1, 1, v1
\ts_add_i32 s5, s5, -1
\ts_cmp_lg_u32 s5, 0
\ts_cbranch_scc1 .LBB0_2
\ts_endpgm
.Lfunc_end0:
""", 0, 0),
}


@pytest.mark.parametrize("name", sorted(_LOOP_FRAGMENTS))
def test_lane_loop_scan_on_fragments(name):
    asm, n_atomics, n_loops = _LOOP_FRAGMENTS[name]
    atomics, loops = lane_serial_loops(asm, "k")
    assert (len(atomics), len(loops)) == (n_atomics, n_loops), (atomics, loops)


@pytest.mark.parametrize("src", SOURCES)
def test_tile_kernels_no_lane_serial_loops(device_asm, src):
    asm = device_asm[src]
    kernels = re.findall(r"^(_ZN2pa(?:14prefill_kernel|19varlen_fused_kernel)\w+):", asm, re.M)
    assert kernels, src
    for kernel in kernels:
        atomics, loops = lane_serial_loops(asm, kernel)
        assert not atomics and not loops, f"{kernel}: {atomics[:2]} {loops[:2]}"
