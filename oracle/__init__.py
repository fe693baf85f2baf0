"""KDA oracle (test infrastructure only).

A plain fp64 CPU implementation of what the KDA forward computes, written from
the pages and independent of the HIP library: the two share no code, header,
helper or constant. Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU
baseline leg of ``bench.py`` may import this package; the product path never
does.

Parity pins: every function here is pinned by ``tests/test_oracle_*.py``
against closed forms, invariants and brute force (see the docstrings there).
"""
from .oracle import (  # noqa: F401
    build_oracle,
    oracle_cumsum,
    oracle_gate,
    oracle_recurrence,
    oracle_forward,
    oracle_backward,
    oracle_gate_backward,
    oracle_forward_softplus,
    oracle_gate_softplus,
    library_path,
    host_threads,
)
from .epilogue import oracle_gated_rmsnorm  # noqa: F401
