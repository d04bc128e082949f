"""CPU oracle for the per-decode-step sparse KV assembly path (test infrastructure).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never calls it; it shares no code with it.
"""
from .kvs_oracle import (  # noqa: F401
    PAD,
    SLOT_PAD,
    KvsError,
    OracleUnit,
    StepRecord,
    attention_fp64,
    bf16_bits_to_f64,
    run_unit,
)
