"""Loading the binding leaves exactly one HIP runtime in the process (torch's).

With /opt/rocm/lib on LD_LIBRARY_PATH, a library loaded before torch would pull
in a second HIP/HSA runtime, which then sees no device.
"""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_one_hip_runtime_after_loading_the_binding():
    code = ("from zero_sharded_mixed_flat_amd import abi\n"
            "import torch\n"
            "libs = {l.split()[-1] for l in open('/proc/self/maps') if 'libamdhip64' in l}\n"
            "print(len(libs), sorted(libs))\n")
    env = dict(os.environ)
    env["LD_LIBRARY_PATH"] = "/opt/rocm/lib:" + env.get("LD_LIBRARY_PATH", "")
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, check=True,
                         cwd=ROOT, env=env)
    assert int(out.stdout.split()[0]) == 1, out.stdout
