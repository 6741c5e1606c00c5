"""bench.py's command line on a host without a GPU: more than one GPU is
refused with a message before anything touches a device."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("argv,env", [(["--gpus", "2"], {}), (["--gpus", "8"], {}),
                                      ([], {"WORLD_SIZE": "4"})])
def test_multi_gpu_request_is_refused(argv, env):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + argv,
                       env={**os.environ, **env}, capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "single GPU" in r.stderr and r.stdout == ""
