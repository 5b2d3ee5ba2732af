"""libkvq2: OSCAR-style INT2 KV-cache quantize-append and split-K decode attention
for AMD Instinct MI355X (gfx950).

The compute path is the in-tree shared library libkvq2.so (HIP kernels +
C ABI, include/kvq2.h); ``kvq2`` is its thin ctypes binding and
``workloads`` holds the seeded synthetic inputs.  Importing the package does
not load the library; the first call into ``kvq2`` does.
"""
