"""CPU oracle of the looped weight-shared decoder forward pass.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The GPU library
never calls it, and it shares no code with the GPU library: the two meet only
in ``synth`` (seeded input draws, no model arithmetic).

It is the plain definition, written for a reader to check by eye against the
pages, in float64 (NumPy), with no blocking, fusion or reordering beyond what
the definition states.  For bf16 configurations the values are rounded to bf16
exactly where the storage format of the GPU path stores bf16 (see
``model.STORAGE_ROUNDING``); the arithmetic between those points stays float64.

Pages cited (by title; the section follows the title):
  P1 "SenseTime's Loop-9B runs its own layers twice, and gets a deeper model for free"
  P2 "SenseTime Open-Sources Loop-9B: Same Layers, Run Twice"
  P3 "SenseTime's SenseNova-Loop-9B Runs Its Own Layers Twice, and It's Open Source"
  P4 "SenseTime open-sourced its experimental SenseNova-Loop-9B-Preview" (frontword.com)
  P5 "How Does SenseNova-Loop Get More Depth Without More Parameters?"

Parity status: every function here is pinned by a ``-m "not gpu"`` test except
the parameter-count arithmetic (parity unpinned against the pages' ~9B/~14.6B,
which the assumed shapes do not reproduce) and trained-model behaviour (no
weights exist to compare with).
"""
from .model import (  # noqa: F401
    Config, Weights, LayerWeights, State, schedule, forward, rmsnorm,
    mhc_maps, sinkhorn, full_attention, linear_attention, swiglu_ffn,
    round_bf16, make_weights, tiny_config, nine_b_config, group_config,
    max_row_rel_err,
)
