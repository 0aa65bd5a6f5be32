"""CPU oracle for the CONF-KV decode step: TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
anything under this package.  The product path (the HIP library and its Python
binding) never imports, links or calls it, and it imports nothing from the
product path.
"""
from .confkv import *  # noqa: F401,F403
