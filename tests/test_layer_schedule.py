"""The one-launch block kernel's work schedule, checked on the host (no GPU):
the library's planner and the kernel's own schedule view (LayerSched) cover
every row tile exactly once, split every tile's K blocks exactly over the
waves of its sub-group, and give every wave the slot count its cursors run
(a wave that ran a different number of iterations would miss a barrier)."""
import os
import subprocess

import pytest

from conftest import ROOT

PKG = os.path.join(ROOT, "ternary_weight_quantized_bt_amd")
LIB = os.path.join(PKG, "libternary.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.mark.skipif(not os.path.exists(LIB) or not os.path.exists(HIPCC),
                    reason="needs the built library and hipcc")
def test_layer_schedule_host_check(tmp_path):
    exe = str(tmp_path / "layer_schedule_check")
    r = subprocess.run([HIPCC, "-O2", "-std=c++17", f"-I{ROOT}/include", f"-I{PKG}/csrc",
                        os.path.join(ROOT, "tests", "layer_schedule_check.cpp"),
                        "-o", exe, f"-L{PKG}", "-lternary", f"-Wl,-rpath,{PKG}"],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    r = subprocess.run([exe, "3000"], capture_output=True, text=True, timeout=600)
    print(r.stdout)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-2000:]
    assert "70B-class block, 256 workgroups: sched 1" in r.stdout  # two classes
