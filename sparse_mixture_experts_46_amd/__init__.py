"""MI355X-native forward pass of a token-choice Mixture-of-Experts FFN layer.

The compute path is libmoe.so (hand-written HIP kernels for gfx950 behind a
C ABI, include/moe.h); `api` is its Python binding.  Importing the package
does not load the library, so the shape and input modules can be used
without a GPU; calling any `api` function loads it and raises if it is
missing.
"""
from .workloads import ALL as WORKLOADS, Workload  # noqa: F401
