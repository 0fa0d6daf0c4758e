"""sparse_mla_amd: absorbed-weight sparse MLA decode for MI355X (gfx950).

The compute path is the C-ABI library ``libmla_decode.so`` (hand-written HIP
kernels, built from ``csrc/``); :mod:`sparse_mla_amd.binding` marshals torch
tensors into its calls.  :mod:`sparse_mla_amd.workload` draws seeded inputs.
Importing this package loads nothing; the binding loads the library on first
use and raises if it is missing.
"""
__all__ = ["binding", "workload"]
