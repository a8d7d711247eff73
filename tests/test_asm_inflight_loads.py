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
