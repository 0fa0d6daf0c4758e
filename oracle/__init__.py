"""Plain CPU oracle for the absorbed sparse MLA decode step.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import, call, link or execute anything
under ``oracle/``.  The product path (``sparse_mla_amd``) never does, and the
two share no code: the only common module is the seeded input generator
``sparse_mla_amd.workload``, which holds none of the method's arithmetic.

Contents
--------
``mla_oracle.c``      fp64 gather formulation (the timed oracle), built with gcc
                      into ``libmla_oracle.so`` by :func:`build`.
``formulations.py``   numpy fp64 dense masked formulations, absorbed and
                      non-absorbed, used to pin the C oracle on small inputs.

Parity status of each function is listed in ``formulations.py`` and in the
design notes; every function here is pinned by a ``-m "not gpu"`` test.
"""
from .core import (  # noqa: F401
    build,
    load,
    decode,
    absorb,
    value_up,
    output_proj,
    prefill,
    dequant_fp8,
    e4m3_to_double,
    bf16_bits_to_double,
    double_to_bf16_bits,
    ORACLE_ERR_INDEX_RANGE,
    ORACLE_ERR_EMPTY,
)
