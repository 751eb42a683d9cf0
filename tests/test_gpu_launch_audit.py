"""Launch audit: under `rocprofv3 --kernel-trace`, one call of each entry point
(tests/launch_audit.py, a child process) dispatches exactly the library's own
kernels, in the documented order, and nothing else: no copy, transpose or fill
kernels around the HIP path."""
import csv
import glob
import os
import shutil
import subprocess
import sys

import pytest

from tests.launch_audit import EXPECTED

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))


def _short(name: str) -> str:
    name = name.replace("sage::(anonymous namespace)::", "").replace("sage::", "").replace("void ", "")
    return name.split("(")[0]


def test_each_call_launches_only_its_kernels(tmp_path):
    prof = shutil.which("rocprofv3")
    if prof is None:
        pytest.skip("rocprofv3 not installed")
    env = dict(os.environ, TMPDIR="/tmp")
    cmd = [prof, "--kernel-trace", "-d", str(tmp_path), "-o", "run", "--output-format", "csv", "--",
           sys.executable, os.path.join(HERE, "launch_audit.py")]
    print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=240, env=env, cwd=str(tmp_path))
    assert "launch audit: %d calls done" % len(EXPECTED) in r.stdout, r.stdout[-2000:] + r.stderr[-2000:]
    traces = glob.glob(str(tmp_path / "**" / "run_kernel_trace.csv"), recursive=True)
    assert traces, "no kernel trace written (rocprofv3 exit %d)" % r.returncode
    rows = sorted(csv.DictReader(open(traces[0])), key=lambda row: int(row["Start_Timestamp"]))
    names = [_short(row["Kernel_Name"]) for row in rows]
    first = next(i for i, n in enumerate(names) if "kmean_partial_kernel" in n)
    want = [k for _, ks in EXPECTED for k in ks]
    print("dispatches after setup:", names[first:], flush=True)
    assert names[first:] == want
