"""quantized_kv_top_amd: top-k sparse attention over a paged, quantized KV
cache, as hand-written HIP kernels for MI355X (gfx950) behind a C ABI.

``quantized_kv_top_amd.qsakv`` is the thin ctypes binding of the C ABI
(``include/qsakv.h``); ``quantized_kv_top_amd.workloads`` draws the seeded
synthetic inputs.  The binding is imported lazily so that the input
generators can be used without loading the native library.
"""

__all__ = ["qsakv", "workloads"]


def __getattr__(name):
    if name in __all__:
        import importlib
        return importlib.import_module("." + name, __name__)
    raise AttributeError(name)
