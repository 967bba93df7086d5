"""fp64 CPU oracle for the Muon matrix step (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path never does.
"""
from .muon_oracle import (  # noqa: F401
    DEFAULT_EPS,
    decayed_weight_update,
    frobenius_normalize,
    muon_step,
    muon_step_ex,
    nesterov_momentum,
    newton_schulz,
    normuon_scale,
    orthogonalize,
    relative_frobenius_error,
    weight_update,
)
