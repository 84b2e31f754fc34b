"""The decode down + combine kernel waits for its h loads with a partial
vector-memory count: it lets the loads issued after the h loads (the
experts' weight rows, scales and side data) stay in flight.  That count is
only right if the compiler issues exactly those loads after the h loads and
before the wait, so this test compiles the kernel to gfx950 assembly and
checks, for every instance, that the wait before the first barrier equals
the number of vector loads issued after the last direct-to-LDS (h) load.
CPU only: it needs hipcc, not a GPU.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "quantized_expert_ffn_histogram_amd", "csrc", "decode.hip")


def _hipcc():
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        pytest.skip("hipcc not available")
    return exe


def test_down_kernel_waits_exactly_for_the_h_loads(tmp_path):
    out = tmp_path / "decode.s"
    cmd = [_hipcc(), "--offload-arch=gfx950", "-O3", "-std=c++17", "-I", os.path.join(ROOT, "include"),
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "--cuda-device-only", "-S", SRC,
           "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    asm = out.read_text()
    names = sorted(set(re.findall(r"^(_Z\S*decode_down_combine_kernel\S*):", asm, re.M)))
    assert len(names) >= 18, names
    for name in names:
        body = asm[asm.index("\n" + name + ":"):]
        body = body[:body.index(".Lfunc_end")]
        ops = [ln.strip() for ln in body.split("\n")
               if re.match(r"\s*(global_load|buffer_load|s_waitcnt\s+vmcnt|s_barrier)", ln)]
        first_barrier = next(i for i, ln in enumerate(ops) if ln.startswith("s_barrier"))
        before = ops[:first_barrier]
        last_h = max(i for i, ln in enumerate(before) if ln.endswith(" lds") or " lds " in ln)
        younger = [ln for ln in before[last_h + 1:] if ln.startswith(("global_load", "buffer_load"))]
        waits = [int(re.search(r"vmcnt\((\d+)\)", ln).group(1)) for ln in before[last_h + 1:]
                 if ln.startswith("s_waitcnt")]
        assert waits, f"{name}: no vmcnt wait between the h loads and the barrier"
        # (An earlier wait there, vmcnt(8), is the one for the expert ids,
        # which the weight addresses need.)  The last wait before the barrier
        # comes after every younger load: it must leave no more than those
        # outstanding, so that every h load has landed, and exactly those,
        # so that the weight stream stays in flight.
        assert waits[-1] == len(younger), (name, len(younger), waits)
