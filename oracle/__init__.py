"""Plain CPU oracle for exact attention (fp64 numpy + a pure-Python brute force).

TEST INFRASTRUCTURE ONLY: imported by tests/, __graft_entry__.smoke() and the cpu_baseline
leg of bench.py, never by the product library, which must fail loudly if its HIP extension is
missing rather than fall back to anything here.
"""

from . import attention, brute, dropout, fp8, rounding  # noqa: F401
