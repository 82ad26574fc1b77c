"""MI355X-native decode context parallelism (DCP) for MLA/DSA decode.

The compute lives in ``libdcpmla.so`` (hand-written HIP for gfx950 behind a
C ABI declared in ``include/dcp_mla.h``).  ``sharded_kv_sparse_amd.binding``
marshals torch tensors into that ABI; ``workloads`` draws seeded synthetic
inputs.  Importing the package loads nothing; the library is opened on first
use of the binding and its absence is an error, never a fallback.
"""

__all__ = ["binding", "workloads"]


def __getattr__(name):
    if name in __all__:
        import importlib
        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
