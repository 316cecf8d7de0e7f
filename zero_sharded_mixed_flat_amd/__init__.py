"""One data-parallel rank's share of a ZeRO mixed-precision Adam step, on MI355X.

The step runs in hand-written HIP kernels for gfx950 behind a C ABI
(``include/zero_flat.h``, built into ``lib/libzero_flat.so``).  ``abi`` is the
thin ctypes binding with the same function names; ``workloads`` holds the
workload definitions and ``synth`` the seeded input generators.
"""

import importlib

__all__ = ["abi", "synth", "workloads"]


def __getattr__(name):
    # The binding loads the shared library, so submodules load only when asked for.
    if name in __all__:
        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
