"""The library's compile flags do what they say on gfx950.

Every HIP source is compiled to gfx950 assembly with the flags the build uses,
and the device code must contain no packed fp32 arithmetic (v_pk_fma_f32,
v_pk_mul_f32, v_pk_add_f32): the build disables that target feature, and the
compiler would otherwise form such instructions from plain float code. A
small float2 kernel built without the flag shows that the check can fail.
"""

import concurrent.futures
import os
import re
import shutil
import subprocess

import pytest

from linear_hybrid_attention_zebra_amd import build as zbuild

PACKED_F32 = re.compile(r"\bv_pk_(fma|mul|add)_f32\b")

pytestmark = pytest.mark.skipif(shutil.which("hipcc") is None and
                                not os.path.exists("/opt/rocm/bin/hipcc"),
                                reason="hipcc not available")


def test_no_packed_fp32_in_device_code(tmp_path):
    srcs = [s for s in zbuild.sources() if s.endswith(".hip")]
    assert srcs

    def one(src):
        out = str(tmp_path / (os.path.basename(src) + ".s"))
        zbuild.device_asm(src, out)
        text = open(out).read()
        assert "gfx950" in text
        return os.path.basename(src), len(PACKED_F32.findall(text))

    with concurrent.futures.ThreadPoolExecutor(max_workers=8) as ex:
        found = dict(ex.map(one, srcs))
    assert all(n == 0 for n in found.values()), f"packed fp32 instructions: {found}"


def test_check_detects_packed_fp32_without_the_flag(tmp_path):
    src = tmp_path / "pk.hip"
    src.write_text(
        "#include <hip/hip_runtime.h>\n"
        "__global__ void k(float2* a, const float2* b, const float2* c, int n) {\n"
        "  int i = blockIdx.x * blockDim.x + threadIdx.x;\n"
        "  if (i < n) { float2 x = a[i], y = b[i], z = c[i];\n"
        "    x.x = x.x * y.x + z.x; x.y = x.y * y.y + z.y; a[i] = x; }\n}\n")
    flags = [f for f in zbuild.COMMON_FLAGS]
    i = flags.index("-packed-fp32-ops")
    without = flags[:i - 3] + flags[i + 1:]
    outs = {}
    for name, fl in (("with", flags), ("without", without)):
        out = tmp_path / f"{name}.s"
        subprocess.run([zbuild.hipcc()] + fl + ["--cuda-device-only", "-S", "-o", str(out),
                                                str(src)], check=True, capture_output=True)
        outs[name] = len(PACKED_F32.findall(out.read_text()))
    assert outs["without"] > 0 and outs["with"] == 0, outs
