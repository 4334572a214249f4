"""Routed MoE layer with a shared expert-slot cache, for MI355X (gfx950).

The compute path is the HIP library ``libmoe_gfx950.so`` (C ABI in
``include/moe.h``); ``routed_expert_cache_amd.binding`` is its ctypes binding
and raises ImportError when the library is not built.  Build it with
``python -m routed_expert_cache_amd.build``.
"""


def __getattr__(name):
    if name == "binding":
        import importlib
        return importlib.import_module(".binding", __name__)
    raise AttributeError(name)
