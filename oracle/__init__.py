"""CPU oracle for layer-streamed training -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline``
leg may import this package.  The HIP product path never imports, links or
calls it, and it imports nothing from the product path (only the seeded input
module ``synth``).  See ``oracle/model.py`` for what is computed and which
passages of the pages each part follows.

Parity status: every function here is pinned by ``tests/test_oracle_pins.py``
(finite differences in fp64, closed forms, library special cases, invariants).
"""
from .model import (bf16_round, to_float, rmsnorm_fwd, rmsnorm_bwd, rope_tables, rope_fwd, rope_bwd,
                    attention_fwd, attention_bwd, attention_suffix, silu, swiglu_fwd, swiglu_bwd, layer_fwd, layer_bwd, layer_rows,
                    head_fwd_bwd, adam_update, adam_consts, accumulate_micro, accumulated_mean, embed_fwd, embed_bwd, forward_backward,
                    HostState, train_step, labels_of)
