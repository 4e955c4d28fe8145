"""Stratified sparse decode attention for MI355X (gfx950).

The compute path is the HIP library ``libssa.so`` built from ``csrc/`` (C ABI
declared in ``include/ssa.h``); ``ssa`` is its thin ctypes binding and
``synth`` builds seeded synthetic workloads.
"""
