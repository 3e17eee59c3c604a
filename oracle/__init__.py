"""fp64 CPU oracle for ReplaySSM decode / speculative verify of GDN and KDA layers.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import, call or run anything under
``oracle/``.  The library (``linear_attention_recurrent_rs_amd``) never does, and the
oracle imports nothing from it: the two share no code.  Inputs come from
``workloads`` (random numbers only) and are passed in as arrays.

Contents
  delta_rule  -- the token-by-token gated delta rule (the definition), folds, readout.
  replay      -- the ReplaySSM state machine (verify with history replay and the fused
                 fold, cursor advance with fold policies, commit fold, materialize) and
                 the token-stream model it is checked against.
  exact       -- exact rational evaluation of the literal dense update, used as a pin.
  conv        -- the short causal convolution before the recurrence, its per-slot window
                 state and the rollback of that window at commit, with the token-stream
                 definition it is checked against.

Parity status: every function here is pinned by a ``-m "not gpu"`` test in
``tests/test_oracle_pins.py`` (exact rational brute force, closed forms, special cases,
replay == sequential, fold invariance, exhaustive cursor sequences; the convolution against
numpy's correlate and scipy's logistic function, exact taps, exhaustive accept sequences).
"""
from . import conv, delta_rule, replay, exact  # noqa: F401
