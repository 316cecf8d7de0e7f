"""The library's host code under the compiler's sanitizers (CPU only).

``tests/host_sanitize_driver.cpp`` drives the partitioner, the host AdamW with
its worker threads (concurrent callers included) and the sharded checkpoints
through the C ABI, on host memory only.  It is built with g++ from the
library's host sources twice, with AddressSanitizer plus
UndefinedBehaviorSanitizer and with ThreadSanitizer, and each build must run
clean.  A planted use after free, signed overflow and data race show that
each build reports what it should in this environment, so a clean run means
something.
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "zero_sharded_mixed_flat_amd", "csrc")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
DRIVER = os.path.join(ROOT, "tests", "host_sanitize_driver.cpp")
LIBRARY_HOST_SOURCES = [os.path.join(CSRC, f) for f in ("plan.cpp", "offload.cpp", "ckpt.cpp")]
FLAGS = {
    "address": ["-fsanitize=address,undefined", "-fno-sanitize-recover=all"],
    "thread": ["-fsanitize=thread"],
}
PLANTED = [
    ("address", "int main() { int* p = new int[4]; delete[] p; volatile int x = p[1]; return x; }\n",
     "heap-use-after-free"),
    ("address", "#include <climits>\nint main() { volatile int a = INT_MAX; int b = a + 1; return b == 0; }\n",
     "signed integer overflow"),
    ("thread", "#include <thread>\nint counter = 0;\n"
               "int main() { std::thread a([] { for (int i = 0; i < 100000; ++i) ++counter; });\n"
               "  for (int i = 0; i < 100000; ++i) ++counter; a.join(); return counter == 0; }\n",
     "data race"),
]


def _gxx():
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not found")
    return gxx


def _build(sources, kind, exe, link_runtime):
    cmd = [_gxx(), "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", *FLAGS[kind], "-ffp-contract=off",
           f"-I{os.path.join(ROOT, 'include')}", f"-I{ROCM}/include", "-D__HIP_PLATFORM_AMD__",
           *sources, "-pthread", "-o", exe]
    if link_runtime:
        # offload.cpp and ckpt.cpp name HIP calls that only their device paths make
        cmd += [f"-L{ROCM}/lib", "-lamdhip64", f"-Wl,-rpath,{ROCM}/lib"]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-4000:]


def _run(exe, *args):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", TSAN_OPTIONS="halt_on_error=1")
    return subprocess.run([exe, *args], capture_output=True, text=True, timeout=600, env=env)


@pytest.mark.parametrize("kind, src, marker", PLANTED, ids=["use-after-free", "signed-overflow", "race"])
def test_planted_error_is_reported(kind, src, marker, tmp_path):
    path = tmp_path / "planted.cpp"
    path.write_text(src)
    exe = str(tmp_path / "planted")
    _build([str(path)], kind, exe, link_runtime=False)
    r = _run(exe)
    assert r.returncode != 0 and marker in r.stderr, r.stderr[-2000:]


@pytest.mark.parametrize("kind", ["address", "thread"])
def test_host_code_runs_clean(kind, tmp_path):
    exe = str(tmp_path / f"driver_{kind}")
    _build([DRIVER, *LIBRARY_HOST_SOURCES], kind, exe, link_runtime=True)
    work = tmp_path / "ckpt"
    work.mkdir()
    r = _run(exe, str(work))
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert r.stdout.startswith("ok:"), r.stdout
    assert "Sanitizer" not in r.stderr and "runtime error" not in r.stderr, r.stderr[-4000:]
