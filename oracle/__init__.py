"""fp64 CPU oracle and pure-Python brute force.

TEST INFRASTRUCTURE: imported only by tests/, by __graft_entry__.smoke() and by
the CPU-baseline leg of bench.py. The HIP library and its Python binding never
import, link or call anything here, and nothing here imports them.
"""
