"""fp64 CPU oracle of the In-Place TTT fast-weight MLP layer (test infrastructure).

Imported only by tests, the smoke check and the benchmark's CPU-baseline leg.
"""
from .oracle import (ALIGNS, TARGETS, build, final_weight_grid, forward, gated_activations, lm_target,
                     num_threads, set_num_threads, set_progress)

__all__ = ["ALIGNS", "TARGETS", "build", "final_weight_grid", "forward", "gated_activations", "lm_target",
           "num_threads", "set_num_threads", "set_progress"]
