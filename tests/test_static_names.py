"""Every name a function of a shipped Python module reads as a global is
defined in that module or is a builtin.

Runs on the CPU from the sources alone (nothing is imported or executed), so
a helper deleted while its callers stay, on a path no other CPU test runs
(the GPU tests and the GPU-only branches of bench.py), fails here rather than
at run time on the GPU.
"""

import builtins
import os
import symtable

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
MODULES = ["bench.py", "__graft_entry__.py"] + [
    os.path.join(d, f) for d in ("zero_sharded_mixed_flat_amd", "oracle", "tests", os.path.join("tests", "golden"))
    if os.path.isdir(os.path.join(ROOT, d))
    for f in sorted(os.listdir(os.path.join(ROOT, d))) if f.endswith(".py")]


def _module_names(table):
    return {s.get_name() for s in table.get_symbols() if s.is_assigned() or s.is_imported()
            or s.is_namespace()}


def _global_reads(table, out):
    for child in table.get_children():
        for sym in child.get_symbols():
            if sym.is_referenced() and sym.is_global() and not sym.is_declared_global():
                out.add((child.get_name(), sym.get_name()))
        _global_reads(child, out)
    return out


@pytest.mark.parametrize("path", MODULES)
def test_global_names_are_defined(path):
    with open(os.path.join(ROOT, path)) as f:
        table = symtable.symtable(f.read(), path, "exec")
    defined = _module_names(table) | set(dir(builtins)) | {"__file__", "__name__"}
    missing = sorted((fn, name) for fn, name in _global_reads(table, set()) if name not in defined)
    assert not missing, f"{path}: names read but never defined: {missing}"


def test_checker_finds_a_missing_helper():
    src = "def used():\n    return helper() + len([])\n"
    table = symtable.symtable(src, "<planted>", "exec")
    defined = _module_names(table) | set(dir(builtins))
    assert [n for _, n in _global_reads(table, set()) if n not in defined] == ["helper"]
