"""TurboQuant KV-cache encode and decode attention on AMD MI355X (gfx950).

The compute lives in the HIP library libtq.so (C ABI declared in
include/tq.h); this package only marshals arguments to it (binding.py) and
draws seeded synthetic inputs (workloads.py).
"""
