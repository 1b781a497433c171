"""HSQ decode path and TurboQuant codec for MI355X (gfx950).

The compute runs in ``libhsq.so`` (hand-written HIP kernels behind a C ABI);
``hsq`` is its thin Python binding and ``workloads`` draws seeded synthetic
inputs.  Importing the package does not load the library; the first call into
``hsq`` does, and raises if the library is missing.
"""
