"""2-bit MLA latent cache for MI355X: quantize-append and decode over a paged cache.

The compute path is the HIP library ``librlq.so`` (C ABI, ``include/rlq.h``);
``decode_attention_rlq_amd.rlq`` marshals torch tensors into its calls.
Importing this package does not load the library; the binding loads it on
first use and raises if it is missing.
"""

__all__ = ["rlq", "workloads"]


def __getattr__(name):
    if name in ("rlq", "workloads"):
        import importlib
        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
