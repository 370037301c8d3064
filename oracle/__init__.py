"""CPU oracle for the IPA forward (test infrastructure only).

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may
import anything from this package; the library path never does.
"""
from .ipa_oracle import (softplus, point_weight, to_global, ipa_dense, ipa_factored,
                         ipa_loops, pair_from_factors)

__all__ = ["softplus", "point_weight", "to_global", "ipa_dense", "ipa_factored",
           "ipa_loops", "pair_from_factors"]
