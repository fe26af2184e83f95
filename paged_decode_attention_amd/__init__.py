"""Block-scaled 8-bit paged KV cache for AMD Instinct MI355X (gfx950).

The HIP kernels and C-ABI entry points live in ``libkvq.so`` (sources under
``csrc/``, declarations in ``include/kvq.h``); ``kvq`` is its Python binding
and ``workloads`` the seeded synthetic input generators.  Attribute access on
this package (``paged_decode_attention_amd.store`` etc.) loads the binding,
which raises if the library is not built.
"""
import importlib


def __getattr__(name):
    if name.startswith("__") or name in ("kvq", "workloads", "build"):
        raise AttributeError(name)
    kvq = importlib.import_module(__name__ + ".kvq")
    try:
        return getattr(kvq, name)
    except AttributeError:
        raise AttributeError("module %r has no attribute %r" % (__name__, name)) from None
