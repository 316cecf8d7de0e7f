"""The boundary is usable from plain C: the header compiles as C99 with every
warning enabled, and a C program linked against the library calls its host
functions (version, partition, accounting, workspace size, error channel).

Runs on the CPU: none of these functions touches the HIP runtime.  The
expected values are the oracle's.
"""

import os
import shutil
import subprocess

import pytest

from oracle import accounting, partition

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
INCLUDE = os.path.join(ROOT, "include")
LIBDIR = os.path.join(ROOT, "zero_sharded_mixed_flat_amd", "lib")

PROGRAM = r"""
#include <stdio.h>
#include <stdint.h>
#include "zero_flat.h"

int main(void) {
    const int64_t units[3] = {1000, 37, 2050};
    zero_plan* plan = NULL;
    int64_t shard = 0, real = 0, full = 0;
    double bytes = 0.0;
    if (zero_plan_create(units, 3, 4, 3, 8, &plan) != ZERO_OK) return 1;
    if (zero_plan_rank(plan, 3, &shard, &real) != ZERO_OK) return 2;
    if (zero_plan_full_numel(plan, &full) != ZERO_OK) return 3;
    zero_plan_destroy(plan);
    if (zero_model_state_bytes(7.5e9, 64, 2, 12, &bytes) != ZERO_OK) return 4;
    printf("version %d\n", zero_version());
    printf("shard %lld real %lld full %lld\n", (long long)shard, (long long)real, (long long)full);
    printf("bytes %.17g\n", bytes);
    printf("workspace %lld\n", (long long)zero_workspace_bytes(4096, 2));
    /* an invalid call: rejected with a negative code and a message */
    int rc = zero_plan_create(units, 3, 0, 3, 8, &plan);
    printf("reject %d %s\n", rc < 0, zero_last_error()[0] != '\0' ? "message" : "empty");
    return 0;
}
"""


def _gcc():
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    return gcc


def test_header_compiles_as_c99():
    subprocess.run([_gcc(), "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror", "-fsyntax-only", "-x", "c",
                    os.path.join(INCLUDE, "zero_flat.h")], check=True)


def test_c_program_calls_the_library(tmp_path):
    src, exe = tmp_path / "prog.c", tmp_path / "prog"
    src.write_text(PROGRAM)
    subprocess.run([_gcc(), "-std=c99", "-Wall", "-Wextra", "-Werror", f"-I{INCLUDE}", str(src), "-o", str(exe),
                    f"-L{LIBDIR}", "-lzero_flat", f"-Wl,-rpath,{LIBDIR}"], check=True)
    p = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert p.returncode == 0, p.stderr
    out = dict(line.split(" ", 1) for line in p.stdout.splitlines())
    ref = partition.make_plan([1000, 37, 2050], 4, 3, 8)
    assert out["version"] == "10301"
    assert out["shard"] == f"{ref.shard_numel} real {ref.real_numel(3)} full {ref.full_numel}"
    assert float(out["bytes"]) == accounting.model_state_bytes(7.5e9, 64, 2)
    assert out["reject"] == "1 message"
