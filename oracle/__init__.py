"""CPU float64 oracle for NVFP4 quantization and the W4A4 product.

Test infrastructure: only tests/, the smoke check of __graft_entry__ and the CPU-baseline leg of
bench.py use it.  The library never imports it.
"""
from .nvfp4_oracle import *  # noqa: F401,F403
from . import nvfp4_oracle  # noqa: F401
