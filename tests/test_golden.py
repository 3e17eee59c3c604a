"""CPU tests: the oracle reproduces the stored fixtures under tests/golden/.

exact_tiny.json holds exact rational results of the dense literal rule (written by
tests/golden/make_golden.py through oracle.exact); c0_oracle.json holds the tiny decode
workload through the replay oracle, with the two fused folds its 12 steps force.
"""
import json
import os
from fractions import Fraction

import numpy as np

import workloads as W
from oracle import delta_rule as dr
from oracle import replay as rp

HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), 'golden')


def _fr(s):
    return float(Fraction(s))


def test_exact_fixture_fp64():
    d = json.load(open(os.path.join(HERE, 'exact_tiny.json')))
    for case in d['cases']:
        kda = case['kda']
        S = np.array([[_fr(x) for x in row] for row in case['S0_kv']]).T
        for tok, want in zip(case['tokens'], case['outputs']):
            alpha = np.array([_fr(x) for x in tok['alpha']]) if kda else _fr(tok['alpha'])
            S, _ = dr.token_update(S, np.array([_fr(x) for x in tok['k']]),
                                   np.array([_fr(x) for x in tok['v']]), _fr(tok['beta']),
                                   alpha, kda)
            o = dr.readout(S, np.array([_fr(x) for x in tok['q']]))
            want = np.array([_fr(x) for x in want])
            assert np.max(np.abs(o - want)) <= 1e-13 * np.max(np.abs(want))
        Sf = np.array([[_fr(x) for x in row] for row in case['S_final_kv']]).T
        assert np.max(np.abs(S - Sf)) <= 1e-13 * np.max(np.abs(Sf))


def test_c0_fixture():
    g = json.load(open(os.path.join(HERE, 'c0_oracle.json')))
    cfg = W.CONFIGS['c0']
    slots = W.slot_map(cfg)
    assert int(slots[0]) == g['slot']
    S0 = W.initial_state(cfg)
    cur = W.initial_cursor(cfg, slots)
    rk, rd, rg = W.initial_ring(cfg, cur)
    layer = rp.ReplayLayer(S0, rk, rd, rg, cfg.kda, cfg.G, cfg.L)
    fl = np.zeros(cfg.num_slots, np.int32)
    for j, st in enumerate(g['steps']):
        before = layer.fused_folds
        out, wp = rp.verify(layer, cur, slots, W.step_inputs(cfg, j))
        rp.cursor_advance(cur, fl, slots, W.accept_lengths(cfg, j), cfg.T, cfg.L,
                          *W.step_policy(cfg, j))
        rp.commit_fold(layer, fl, slots)
        assert wp[0] == st['write_pos'] and cur[slots[0]] == st['cursor']
        assert (layer.fused_folds != before) == st['fused_fold']
        assert np.allclose(out[0], np.array(st['out']), rtol=0, atol=1e-13)
    assert sum(s['fused_fold'] for s in g['steps']) == 2
    assert np.allclose(layer.S[g['slot']], np.array(g['S_final']), rtol=0, atol=1e-13)
