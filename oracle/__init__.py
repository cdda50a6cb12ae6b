"""CPU fp64 oracle for paged decode attention and the paged K/V append.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import or run anything in this package.
It shares no code with the HIP library in ``paged_kv_attention_decode_amd``:
``pkv_oracle.c`` (plain C loops, pthreads) and ``paged.py`` (numpy) each write
the layout offsets, format decoders and attention arithmetic out from their
definitions, and are cross-checked against each other and pinned by the
``-m "not gpu"`` tests (library routines, closed forms, brute force and
invariants).  Parity status: every function here is pinned; none is unpinned.
"""
from . import paged, c_oracle  # noqa: F401
