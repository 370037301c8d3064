"""CPU oracles for the IPA forward, the kNN distogram and attention with a
low-rank bias (test infrastructure only).

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may
import anything from this package; the library path never does.
"""
from .ipa_oracle import (softplus, point_weight, to_global, ipa_dense, ipa_factored,
                         ipa_loops, pair_from_factors)
from .knn_oracle import (bin_width, sqdist_f32, distance_bins, one_hot, knn_distogram,
                         knn_loops)

__all__ = ["softplus", "point_weight", "to_global", "ipa_dense", "ipa_factored",
           "ipa_loops", "pair_from_factors", "bin_width", "sqdist_f32", "distance_bins",
           "one_hot", "knn_distogram", "knn_loops"]
from .flashbias_oracle import (alibi_slopes, alibi_bias, alibi_factors, sqdist_factors,
                               attention_with_bias, flashbias_attention, flashbias_rows,
                               attention_loops)

__all__ += ["alibi_slopes", "alibi_bias", "alibi_factors", "sqdist_factors",
            "attention_with_bias", "flashbias_attention", "flashbias_rows", "attention_loops"]
