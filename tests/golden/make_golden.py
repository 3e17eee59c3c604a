"""Writes the stored expected values under tests/golden/.  Calls only oracle/ (and the
seeded input generator in workloads/); nothing here touches the HIP library.

  exact_tiny.json -- a 4-token GDN and KDA sequence on dk=3, dv=2 in exact rational
                     arithmetic (oracle.exact, the dense literal form), as "p/q" strings.
  c0_oracle.json  -- the tiny decode workload (1 request, dk=dv=16, ring 4, 12 steps)
                     through the fp64 replay oracle: outputs, write_pos and cursor per
                     step, the steps at which the fused fold fires, the final state.

Run:  python tests/golden/make_golden.py
"""
import json
import os
import sys
from fractions import Fraction

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import workloads as W                      # noqa: E402
from oracle import exact                  # noqa: E402
from oracle import replay as rp           # noqa: E402


def _s(x):
    return f"{x.numerator}/{x.denominator}"


def exact_fixture():
    rng = np.random.default_rng(2024)
    cases = []
    for kda in (False, True):
        dk, dv, T = 3, 2, 4
        S0 = [[Fraction(int(rng.integers(-8, 9)), 8) for _ in range(dk)] for _ in range(dv)]
        toks = []
        for _ in range(T):
            q = [Fraction(int(rng.integers(-8, 9)), 8) for _ in range(dk)]
            k = [Fraction(int(rng.integers(-8, 9)), 8) for _ in range(dk)]
            v = [Fraction(int(rng.integers(-8, 9)), 8) for _ in range(dv)]
            beta = Fraction(int(rng.integers(1, 5)), 4)
            alpha = ([Fraction(int(rng.integers(4, 8)), 8) for _ in range(dk)] if kda
                     else Fraction(int(rng.integers(4, 8)), 8))
            toks.append((q, k, v, beta, alpha))
        S, outs = exact.run(S0, toks, kda)
        cases.append({
            'kda': kda,
            'S0_kv': [[_s(x) for x in row] for row in S0],
            'tokens': [{'q': [_s(x) for x in q], 'k': [_s(x) for x in k], 'v': [_s(x) for x in v],
                        'beta': _s(beta),
                        'alpha': [_s(x) for x in alpha] if kda else _s(alpha)}
                       for (q, k, v, beta, alpha) in toks],
            'outputs': [[_s(x) for x in o] for o in outs],
            'S_final_kv': [[_s(x) for x in row] for row in S],
        })
    return {'source': 'oracle.exact (dense literal form, exact rationals)', 'cases': cases}


def c0_fixture():
    cfg = W.CONFIGS['c0']
    slots = W.slot_map(cfg)
    S0 = W.initial_state(cfg)
    cur = W.initial_cursor(cfg, slots)
    rk, rd, rg = W.initial_ring(cfg, cur)
    layer = rp.ReplayLayer(S0, rk, rd, rg, cfg.kda, cfg.G, cfg.L)
    fold_len = np.zeros(cfg.num_slots, np.int32)
    steps = []
    for j in range(cfg.steps):
        inp = W.step_inputs(cfg, j)
        acc = W.accept_lengths(cfg, j)
        before = layer.fused_folds
        out, wp = rp.verify(layer, cur, slots, inp)
        pol, next_T = W.step_policy(cfg, j)
        rp.cursor_advance(cur, fold_len, slots, acc, cfg.T, cfg.L, pol, next_T)
        rp.commit_fold(layer, fold_len, slots)
        steps.append({'out': out[0].tolist(), 'write_pos': int(wp[0]),
                      'cursor': int(cur[slots[0]]), 'fused_fold': layer.fused_folds != before})
    s = int(slots[0])
    return {'source': 'oracle.replay on workloads c0', 'slot': s, 'steps': steps,
            'S_final': layer.S[s].tolist(),
            'materialized': layer.committed_state(s, int(cur[s])).tolist()}


if __name__ == '__main__':
    with open(os.path.join(HERE, 'exact_tiny.json'), 'w') as f:
        json.dump(exact_fixture(), f, indent=1)
    with open(os.path.join(HERE, 'c0_oracle.json'), 'w') as f:
        json.dump(c0_fixture(), f)
    print('wrote exact_tiny.json, c0_oracle.json')
