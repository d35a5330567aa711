"""The per-work-group timeline build on the GPU: one decode1 call through
libmoe_q2_timeline.so (a separate process: the library it loads is the timeline
variant, not the one this test process holds), every launch recorded with
consistent roles and times."""
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TL = os.path.join(ROOT, "bit_quantized_routed_amd", "libmoe_q2_timeline.so")


@pytest.mark.gpu
def test_timeline_decode1():
    if not os.path.exists(TL):       # a diagnostic build, not the library the other tests load
        pytest.skip("libmoe_q2_timeline.so is not built (bit_quantized_routed_amd.build.build(timeline=True))")
    print("timeline: decode1, one call, 2 layers", flush=True)
    p = subprocess.run([sys.executable, "-m", "bit_quantized_routed_amd.timeline", "decode1", "--calls", "1",
                        "--rotate", "2"], cwd=ROOT, capture_output=True, text=True, timeout=240)
    assert p.returncode == 0, p.stderr[-2000:]
    out = p.stdout
    launches = re.findall(r"(gate/up|down) launch: (\d+) work-groups, last end ([\d.]+) us", out)
    assert [l[0] for l in launches] == ["gate/up", "down"], out
    for name, n, end in launches:
        assert int(n) > 0 and 0.0 < float(end) < 1000.0, out
    # one token: 8 routed units, every routed work-group has a prologue before its columns
    routed = re.findall(r"routed +n= *(\d+) +start p50/p90/max ([\d.]+)/([\d.]+)/([\d.]+) +duration "
                        r"([\d.]+)/([\d.]+)/([\d.]+) +end ([\d.]+)/([\d.]+)/([\d.]+) +prologue ([\d.]+)", out)
    assert len(routed) == 2, out
    for r in routed:
        n, st_max, dur_max, end_max, pro = int(r[0]), float(r[3]), float(r[6]), float(r[9]), float(r[10])
        assert n > 0 and 0.0 < pro < dur_max and end_max >= dur_max and st_max < end_max, out
    assert "shared" in out                      # the shared expert's rows ride in both launches
