"""Host-side checks of the benchmark's contract: a request for more than one
GPU ends with a message and exit status 2 before anything touches a device,
and every committed profile summary names the rocprofv3 command it came
from."""
import glob
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line["n_gpus"] == 2 and "one GPU" in line["error"]
    assert "one GPU" in r.stderr


def test_profile_summaries_name_their_commands():
    files = sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md")))
    assert files
    for f in files:
        text = open(f).read()
        assert "rocprofv3" in text and "bench.py" in text, os.path.basename(f)
