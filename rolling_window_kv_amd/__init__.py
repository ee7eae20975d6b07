"""Rolling-window KV streaming decode on AMD MI355X (gfx950).

The compute lives in ``librkv.so`` (hand-written HIP kernels behind a C ABI,
declared in ``include/rkv.h``); :mod:`rolling_window_kv_amd.rkv` is the thin
ctypes binding with the same entry-point names.  Submodules are imported on
first use so that :mod:`rolling_window_kv_amd.synth` can be used on its own.
"""
import importlib

__all__ = ["rkv", "synth", "build"]


def __getattr__(name):
    if name in __all__:
        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
