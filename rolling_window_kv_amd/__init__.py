"""Rolling-window KV streaming decode on AMD MI355X (gfx950).

The compute lives in ``librkv.so`` (hand-written HIP kernels behind a C ABI,
declared in ``include/rkv.h``); :mod:`rolling_window_kv_amd.rkv` is the thin
ctypes binding with the same entry-point names.  The binding is imported
lazily so that :mod:`rolling_window_kv_amd.synth` can be used on its own.
"""

__all__ = ["rkv", "synth"]


def __getattr__(name):
    if name == "rkv":
        from . import rkv
        return rkv
    if name == "synth":
        from . import synth
        return synth
    raise AttributeError(name)
