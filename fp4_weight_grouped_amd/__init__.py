"""libv4moe: the DeepSeek-V4-style MoE layer forward on one MI355X.

The compute lives in the HIP library ``libv4moe.so`` (C ABI, ``include/v4moe.h``);
:mod:`fp4_weight_grouped_amd.v4moe` is a thin ctypes binding with the same
names.  :mod:`fp4_weight_grouped_amd.inputs` generates seeded synthetic
workloads.  Importing the package does not load the library.
"""

__all__ = ["v4moe", "inputs"]
