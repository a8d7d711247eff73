"""Static check of the prefill kernels' device code: the destination registers of
a global load issued as inline asm (not counted by the compiler) must not be read
or written by any instruction before the next vector-memory wait.  A violation
means the compiler moved or reused registers of a load still in flight (silent
corruption, or an address overwritten by late data).  The scan follows
fall-through order from each load up to the next `s_waitcnt vmcnt`."""
import os
import re
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "..", "paged_kv_attention_table_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["-O3", "-std=c++17", "--offload-arch=gfx950", "-fno-fast-math", "-Xclang", "-target-feature", "-Xclang",
         "-packed-fp32-ops", "--cuda-device-only", "-S"]


def vgprs(tok):
    m = re.match(r"v\[(\d+):(\d+)\]", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"v(\d+)$", tok)
    return {int(m.group(1))} if m else set()


def untracked_load_hazards(asm, kernel):
    i = asm.index(kernel + ":")
    lines = [ln.strip() for ln in asm[i:asm.index(".Lfunc_end", i)].split("\n")]
    loads, bad = 0, []
    for n, ln in enumerate(lines):
        # the asm loads use a scalar base (saddr form); the compiler's own use a VGPR pair
        if not ln.startswith("global_load_dwordx4") or ", s[" not in ln:
            continue
        loads += 1
        dst = vgprs(ln.split()[1].rstrip(","))
        for t in lines[n + 1:]:
            if not t or t.startswith((";", ".")):
                continue
            if (t.startswith("s_waitcnt") and "vmcnt" in t) or t.startswith("s_endpgm"):
                break
            parts = t.split(None, 1)
            ops = [o.strip().split()[0] for o in parts[1].split(",") if o.strip()] if len(parts) > 1 else []
            if any(vgprs(o) & dst for o in ops):
                bad.append((ln, t))
                break
    return loads, bad


@pytest.mark.skipif(shutil.which(HIPCC) is None and not os.path.exists(HIPCC), reason="hipcc not available")
@pytest.mark.parametrize("src,tname", [("pa_prefill_bf16.hip", "4BF16"), ("pa_prefill_f16.hip", "3F16")])
def test_no_register_reuse_under_inflight_loads(tmp_path, src, tname):
    out = tmp_path / (src + ".s")
    subprocess.run([HIPCC, *FLAGS, os.path.join(CSRC, src), "-o", str(out)], check=True, capture_output=True)
    asm = out.read_text()
    # ALiBi; merged into a prior state; two key segments (without ALiBi)
    flags = [(a, m, "0") for a in "01" for m in "01"] + [("0", m, "1") for m in "01"]
    for dims in ("128ELi128", "192ELi128", "64ELi64"):
        for alibi, merge, seg2 in flags:
            kernel = f"_ZN2pa14prefill_kernelINS_{tname}ELi{dims}ELb{alibi}ELb{merge}ELb{seg2}EEEvNS_11PrefillArgsE"
            loads, bad = untracked_load_hazards(asm, kernel)
            assert loads > 0, kernel
            assert not bad, f"{kernel}: {bad[:3]}"


@pytest.mark.skipif(shutil.which(HIPCC) is None and not os.path.exists(HIPCC), reason="hipcc not available")
@pytest.mark.parametrize("src,tname", [("pa_fused_bf16.hip", "4BF16"), ("pa_fused_f16.hip", "3F16")])
def test_fused_varlen_kernel_no_register_reuse(tmp_path, src, tname):
    """The fused varlen kernel carries the prefill tile loop (head dim 128) beside
    the decode rows: the same check on it."""
    out = tmp_path / (src + ".s")
    subprocess.run([HIPCC, *FLAGS, os.path.join(CSRC, src), "-o", str(out)], check=True, capture_output=True)
    asm = out.read_text()
    for alibi, merge in (("0", "0"), ("1", "0"), ("0", "1"), ("1", "1")):
        kernel = f"_ZN2pa19varlen_fused_kernelINS_{tname}ELb{alibi}ELb{merge}EEEvNS_11PrefillArgsENS_8RowsArgsEij"
        loads, bad = untracked_load_hazards(asm, kernel)
        assert loads > 0, kernel
        assert not bad, f"{kernel}: {bad[:3]}"
