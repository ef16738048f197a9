"""MLA decode attention for MI355X (gfx950): HIP kernels behind a C ABI.

``inputs`` holds the seeded synthetic workloads; ``binding`` the thin ctypes
layer over ``libmla_decode.so`` (loaded on first use).
"""
