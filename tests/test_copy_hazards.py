"""The direct global -> LDS tile copies are inline assembly, which the
compiler's hazard checks do not see.  A vector instruction that writes an SGPR
needs 5 wait states before a vector memory instruction reads that SGPR as an
address (gfx9), so every copy must carry its own s_nop 4.  This compiles the
library's device code to assembly (no GPU needed) and checks each copy in
every kernel, and that no copy reads a base SGPR written by a vector
instruction within the 5 wait states."""
import os
import re
import subprocess

import pytest

from scaled_dot_product_qk_amd import build as b


def _device_asm(tmp_path):
    out = tmp_path / "attn.s"
    cmd = [b.hipcc(), "--offload-arch=gfx950", "-O3", "-std=c++17", "--cuda-device-only", "-S",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-mllvm", "-amdgpu-mfma-vgpr-form", "-I", b.INCLUDE, "-I", b.CSRC,
           os.path.join(b.CSRC, "attn_api.hip"), "-o", str(out)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        pytest.skip("hipcc unavailable: " + res.stderr[-400:])
    return out.read_text().splitlines()


def _sgprs(tok):
    m = re.match(r"s\[(\d+):(\d+)\]$", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"s(\d+)$", tok)
    return {int(m.group(1))} if m else set()


def test_every_lds_copy_is_guarded(tmp_path):
    lines = _device_asm(tmp_path)
    hist, copies, unguarded, hazards = [], 0, [], []
    for raw in lines:
        line = raw.strip()
        if re.match(r"^_ZN[^:\s]+:", line):
            hist = []
            continue
        if not line or line.startswith((";", ".")) or line.endswith(":"):
            continue
        if line.startswith("global_load_lds"):
            copies += 1
            if not (hist and hist[-1].startswith("s_nop 4")):
                unguarded.append(line)
            base = _sgprs(line.split(None, 1)[1].split(",")[1].strip())
            waits = 0
            for prev in reversed(hist[-12:]):
                op = prev.split()[0]
                if op == "s_nop":
                    waits += int(prev.split()[1]) + 1
                    continue
                if waits >= 5:
                    break
                dst = prev.split(None, 1)[1].split(",")[0].strip() if " " in prev else ""
                if op.startswith("v_") and _sgprs(dst) & base:
                    hazards.append((prev, line, waits))
                waits += 1
        hist.append(line)
    assert copies > 0
    assert not unguarded, unguarded[:3]
    assert not hazards, hazards[:3]
