"""Reference oracle for paged-KV speculative verification — TEST INFRASTRUCTURE ONLY.

This package is a plain, slow, obviously-correct CPU statement of what the GPU
path computes.  It exists so that tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` can check the HIP library against it.
Nothing in the product package may import it, and it imports nothing from the
product package: the two share no kernels, headers, helpers, tables or
pre/post-processing.  Only the seeded input generators (which hold none of the
method's arithmetic) feed both sides, and they are passed in as plain arrays.

Floating point is fp64 unless a step is defined in a narrower precision (the
FP8 quantiser, which follows the OCP 8-bit floating point specification in
fp32 so that its integer codes are reproducible).

Modules
-------
philox     Philox4x32-10 counter-based generator (Salmon, Moraes, Dror, Shaw,
           "Parallel random numbers: as easy as 1, 2, 3", SC'11).
fp8        OCP E4M3 ("e4m3fn") decode/encode, written from the OCP spec.
attention  O-A: masked softmax attention over contiguous K/V gathered from pages.
pool       O-B: page pool + block tables (refcounts, shared prefix, CoW,
           append, rollback, release), with gather back to contiguous K/V.
accept     O-C: per-token acceptance rule, accepted length, residual/bonus
           sampling.

Parity status: every function here is pinned by a CPU test against facts
fixed outside this code (worked numbers, closed forms, brute force, library
routines, invariants); see tests/test_oracle_*.py.
"""
