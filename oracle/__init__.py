"""CPU oracle for the Muon optimizer step (test infrastructure only).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg
may import this package.  The GPU library never imports, links or runs it.
"""
from .muon_oracle import (  # noqa: F401
    NS_COEFFS,
    momentum,
    frobenius_normalize,
    newton_schulz,
    apply_update,
    muon_step,
    qk_clip,
)
