"""MI355X-native CONF-KV decode-step library (HIP kernels behind a C ABI).

Importing the package loads nothing native; `adaptive_kv_cache_amd.binding`
loads the built shared library on first use and fails loudly when it is absent.
"""
from . import workloads  # noqa: F401

__all__ = ["workloads"]
