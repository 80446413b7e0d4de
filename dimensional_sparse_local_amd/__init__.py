"""MI355X-native N-dimensional local attention (forward).

The compute lives in the C-ABI library ``libna.so`` (host planner + HIP
kernels for gfx950); ``dimensional_sparse_local_amd.na`` is its thin ctypes
binding.  ``workloads`` holds plain workload descriptions and seeded inputs.
"""
