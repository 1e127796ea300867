"""CPU oracle for the SketchSSM decode path (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package; the HIP library never does.
"""
from .sketchssm_oracle import (  # noqa: F401
    KINDS,
    BatchOracle,
    ItemOracle,
    gather_items,
    items_oracle,
    plan,
    transition,
    write_weight,
)
