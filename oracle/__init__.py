"""CPU oracle of the Domino draft-block rollout (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  It shares no code with the HIP path.
"""
from .domino_oracle import (base_logits, candidate_pool, first_max_index, gru_cell,
                            rollout, silu, step_offsets, top1_and_margin)

__all__ = ["base_logits", "candidate_pool", "first_max_index", "gru_cell", "rollout",
           "silu", "step_offsets", "top1_and_margin"]
