"""Pins for the fp64 oracle: checks against facts fixed by mathematics, not by the oracle.

Each ``pin_*`` raises AssertionError on failure.  ``tests/test_oracle_pins.py`` runs them
against the oracle as it is, and again against planted mistakes (a dropped term, a
wrong sign, a transposed operand, a wrong head map, an off-by-one in the fold rule) to
show that each plausible mistake fails at least one pin.
"""
from __future__ import annotations

import itertools
from fractions import Fraction
from types import SimpleNamespace

import numpy as np

import oracle.conv as cv
import oracle.delta_rule as dr
import oracle.replay as rp
from oracle import exact

# ----------------------------------------------------------------------------- helpers


def _frac_vec(rng, n, denom=8):
    return [Fraction(int(x), denom) for x in rng.integers(-denom, denom + 1, size=n)]


def _tiny_tokens(rng, T, dk, dv, kda):
    toks = []
    for _ in range(T):
        q = _frac_vec(rng, dk)
        k = _frac_vec(rng, dk)
        v = _frac_vec(rng, dv)
        beta = Fraction(int(rng.integers(1, 5)), 4)
        if kda:
            alpha = [Fraction(int(rng.integers(4, 8)), 8) for _ in range(dk)]
        else:
            alpha = Fraction(int(rng.integers(4, 8)), 8)
        toks.append((q, k, v, beta, alpha))
    return toks


def _f(x):
    return np.array([float(e) for e in x]) if isinstance(x, list) else float(x)


def _rel(a, b):
    a, b = np.asarray(a, float), np.asarray(b, float)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


def _inputs(B, T, hk, hv, dk, dv, kda, rng, beta=None, alpha=None, unit=True):
    def unit_vec(shape):
        x = rng.standard_normal(shape)
        return x / np.linalg.norm(x, axis=-1, keepdims=True) if unit else x
    q = unit_vec((B, T, hk, dk))
    k = unit_vec((B, T, hk, dk))
    v = rng.standard_normal((B, T, hv, dv))
    b = rng.uniform(0, 1, (B, T, hv)) if beta is None else np.full((B, T, hv), beta)
    gshape = (B, T, hv, dk) if kda else (B, T, hv)
    g = rng.uniform(0.3, 0.99, gshape) if alpha is None else np.full(gshape, alpha)
    return SimpleNamespace(q=q, k=k, v=v, beta=b, gate=g)


def _layer(S0, L, hk, hv, dk, dv, kda, cursor=None, rng=None):
    nslots = S0.shape[0]
    rk = np.full((nslots, L, hk, dk), np.nan)
    rd = np.full((nslots, L, hv, dv), np.nan)
    rg = np.full((nslots, L, hv, dk) if kda else (nslots, L, hv), np.nan)
    if cursor is not None:
        for s in range(nslots):
            c = int(cursor[s])
            rk[s, :c] = rng.standard_normal((c, hk, dk)) / np.sqrt(dk)
            rd[s, :c] = rng.standard_normal((c, hv, dv))
            rg[s, :c] = rng.uniform(0.3, 0.99, rg[s, :c].shape)
    return rp.ReplayLayer(S0, rk, rd, rg, kda, hv // hk, L)


def run_both(S0, steps_inputs, accepts, slots, L, T, hk, hv, kda, policies,
             cursor0=None, ring_rng=None, force_masks=None, lens=None):
    """Run the replay state machine and the token-stream definition side by side
    (``lens``: per-step ragged window widths, or None).  Returns (max relative output
    gap, max relative committed-state gap, fused folds, cursor trace)."""
    nslots = S0.shape[0]
    dk, dv = S0.shape[2], S0.shape[3]
    cursor = np.zeros(nslots, np.int32) if cursor0 is None else cursor0.copy()
    fold_len = np.zeros(nslots, np.int32)
    layer = _layer(S0, L, hk, hv, dk, dv, kda, cursor if cursor0 is not None else None,
                   ring_rng)
    ts = rp.TokenStream.from_replay(layer, cursor)
    gap_o = gap_s = 0.0
    trace = []
    for j, (inp, acc) in enumerate(zip(steps_inputs, accepts)):
        ln = None if lens is None else lens[j]
        o_rep, wp = rp.verify(layer, cursor, slots, inp, lens=ln)
        o_def, _ = ts.verify(slots, inp, lens=ln)
        live = slots >= 0
        fin = np.isfinite(o_def[live])
        assert np.array_equal(fin, np.isfinite(o_rep[live])), 'processed positions differ'
        if fin.any():
            gap_o = max(gap_o, _rel(o_rep[live][fin], o_def[live][fin]))
        pol, next_T = policies[j]
        fm = None if force_masks is None else force_masks[j]
        rp.cursor_advance(cursor, fold_len, slots, acc, T, L, pol, next_T, fm, lens=ln)
        rp.commit_fold(layer, fold_len, slots)
        ts.accept(slots, acc)
        trace.append(cursor.copy())
        for r, s in enumerate(slots):
            if s < 0:
                continue
            assert 0 <= cursor[s] <= L
            gap_s = max(gap_s, _rel(layer.committed_state(s, int(cursor[s])), ts.H[s]))
    return gap_o, gap_s, layer.fused_folds, trace


# ----------------------------------------------------------------------------- pins


def pin_exact_rational():
    """fp64 oracle vs exact rational dense literal form, GDN and KDA, several tokens."""
    rng = np.random.default_rng(11)
    for kda in (False, True):
        dk, dv, T = 3, 2, 5
        S0 = [_frac_vec(rng, dk) for _ in range(dv)]          # [dv][dk], key-to-value
        toks = _tiny_tokens(rng, T, dk, dv, kda)
        S_ex, outs_ex = exact.run(S0, toks, kda)
        S = np.array([[float(x) for x in row] for row in S0]).T    # stored [dk, dv]
        for t, (q, k, v, beta, alpha) in enumerate(toks):
            S, _ = dr.token_update(S, _f(k), _f(v), _f(beta), _f(alpha), kda)
            o = dr.readout(S, _f(q))
            assert _rel(o, _f(outs_ex[t])) < 1e-13, ('output', kda, t)
        S_ex_stored = np.array([[float(x) for x in row] for row in S_ex]).T
        assert _rel(S, S_ex_stored) < 1e-13, ('state', kda)


def pin_exact_grouped_heads():
    """Grouped heads against the exact rule run per value head with key head h // G."""
    rng = np.random.default_rng(12)
    hk, G, dk, dv, T = 2, 2, 2, 3, 3
    hv = hk * G
    S0 = [[_frac_vec(rng, dk) for _ in range(dv)] for _ in range(hv)]
    toks = [[_tiny_tokens(rng, 1, dk, dv, False)[0] for _ in range(hv)] for _ in range(T)]
    # key-head inputs: token t, key head j takes q, k of value head j*G
    q = np.array([[_f(toks[t][j * G][0]) for j in range(hk)] for t in range(T)])
    k = np.array([[_f(toks[t][j * G][1]) for j in range(hk)] for t in range(T)])
    v = np.array([[_f(toks[t][h][2]) for h in range(hv)] for t in range(T)])
    beta = np.array([[_f(toks[t][h][3]) for h in range(hv)] for t in range(T)])
    alpha = np.array([[_f(toks[t][h][4]) for h in range(hv)] for t in range(T)])
    S = np.array([[[float(x) for x in row] for row in S0[h]] for h in range(hv)]).transpose(0, 2, 1)
    for h in range(hv):
        j = h // G
        seq = [(toks[t][j * G][0], toks[t][j * G][1], toks[t][h][2], toks[t][h][3],
                toks[t][h][4]) for t in range(T)]
        _, outs = exact.run(S0[h], seq, False)
        Sh = S.copy()
        for t in range(T):
            Sh, _ = dr.token_update(Sh, dr.expand_heads(k[t], G), v[t], beta[t], alpha[t], False)
            o = dr.readout(Sh, dr.expand_heads(q[t], G))
            assert _rel(o[h], _f(outs[t])) < 1e-13, ('grouped head', h, t)


def pin_pure_decay():
    """beta = 0: no writes, so o_t = (prod alpha) S0^T q_t (GDN) or S0^T (Gamma (.) q_t)
    (KDA), through history replay, fused folds and commit folds."""
    for kda in (False, True):
        rng = np.random.default_rng(13)
        hk, hv, dk, dv, L, T, steps = 1, 2, 4, 3, 5, 2, 7
        S0 = rng.standard_normal((2, hv, dk, dv))
        slots = np.array([1], np.int32)
        layer = _layer(S0, L, hk, hv, dk, dv, kda)
        cursor = np.zeros(2, np.int32)
        fold_len = np.zeros(2, np.int32)
        Gam = np.ones((hv, dk) if kda else (hv,))
        for j in range(steps):
            inp = _inputs(1, T, hk, hv, dk, dv, kda, rng, beta=0.0, alpha=None)
            out, _ = rp.verify(layer, cursor, slots, inp)
            a = np.array([int(rng.integers(1, T + 1))])
            g = Gam.copy()
            for t in range(T):
                g = g * inp.gate[0, t]
                qx = dr.expand_heads(inp.q[0, t], hv // hk)
                want = np.einsum('hij,hi->hj', S0[1], g * qx) if kda else \
                    g[:, None] * np.einsum('hij,hi->hj', S0[1], qx)
                assert _rel(out[0, t], want) < 1e-12, ('pure decay', kda, j, t)
            for t in range(int(a[0])):
                Gam = Gam * inp.gate[0, t]
            pol = rp.FOLD_FORCE if j == 5 else rp.FOLD_NONE
            rp.cursor_advance(cursor, fold_len, slots, a, T, L, pol)
            rp.commit_fold(layer, fold_len, slots)
        assert layer.fused_folds >= 1


def pin_identity_readout():
    """alpha = 1, beta = 0, q = e_i  ->  o = row i of the stored state of each value head."""
    rng = np.random.default_rng(14)
    hk, hv, dk, dv = 2, 4, 5, 3
    S0 = rng.standard_normal((hv, dk, dv))
    for i in range(dk):
        q = np.zeros((hk, dk))
        q[:, i] = 1.0
        k = rng.standard_normal((hk, dk))
        S, _ = dr.token_update(S0, dr.expand_heads(k, 2), rng.standard_normal((hv, dv)),
                               np.zeros(hv), np.ones(hv), False)
        o = dr.readout(S, dr.expand_heads(q, 2))
        assert np.array_equal(o, S0[:, i, :]), ('identity readout', i)


def pin_write_then_read():
    """beta = 1 and a unit key: afterwards S^T k = v whatever the old state and decay, so
    q = k reads back v (GDN and KDA)."""
    rng = np.random.default_rng(15)
    for kda in (False, True):
        hv, dk, dv = 3, 6, 4
        S = rng.standard_normal((hv, dk, dv))
        k = rng.standard_normal((hv, dk))
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
        v = rng.standard_normal((hv, dv))
        alpha = rng.uniform(0.2, 0.9, (hv, dk) if kda else (hv,))
        S2, d = dr.token_update(S, k, v, np.ones(hv), alpha, kda)
        assert _rel(dr.readout(S2, k), v) < 1e-13, ('write then read', kda)


def pin_grouped_write():
    """alpha = 1, beta = 1, k = e_i on key head j only: value heads h with h // G == j get
    row i replaced by v exactly; every other head is unchanged."""
    rng = np.random.default_rng(16)
    hk, G, dk, dv = 3, 2, 4, 5
    hv = hk * G
    for j in range(hk):
        for i in range(dk):
            S0 = rng.standard_normal((hv, dk, dv))
            k = np.zeros((hk, dk))
            k[j, i] = 1.0
            v = rng.standard_normal((hv, dv))
            S, _ = dr.token_update(S0, dr.expand_heads(k, G), v, np.ones(hv), np.ones(hv), False)
            for h in range(hv):
                if h // G == j:
                    assert np.allclose(S[h, i], v[h], rtol=0, atol=1e-14)
                    others = [x for x in range(dk) if x != i]
                    assert np.array_equal(S[h, others], S0[h, others])
                else:
                    assert np.array_equal(S[h], S0[h]), ('grouped write', j, h)


def pin_replay_equals_sequential():
    """Replay state machine == token-stream definition, every step, with history, fused
    folds, commit folds, null rows and staggered cursors (fp64, 1e-12)."""
    rng = np.random.default_rng(17)
    for kda, T, L, pol in ((False, 1, 4, rp.FOLD_NONE), (False, 3, 8, rp.FOLD_LAZY),
                           (True, 3, 7, rp.FOLD_NONE), (False, 4, 6, rp.FOLD_EVERY_COMMIT),
                           (True, 2, 5, rp.FOLD_FORCE)):
        hk, hv, dk, dv, B, steps = 2, 4, 6, 5, 4, 9
        nslots = B + 2
        S0 = rng.standard_normal((nslots, hv, dk, dv)) * 0.3
        slots = np.array([3, -1, 0, 5], np.int32)
        cursor0 = np.zeros(nslots, np.int32)
        for s in (3, 0, 5):
            cursor0[s] = int(rng.integers(0, L - T + 1))
        ins = [_inputs(B, T, hk, hv, dk, dv, kda, rng) for _ in range(steps)]
        accs = [rng.integers(0, T + 1, size=B).astype(np.int32) for _ in range(steps)]
        fms = [rng.integers(0, 2, size=B).astype(np.uint8) for _ in range(steps)]
        go, gs, nf, _ = run_both(S0, ins, accs, slots, L, T, hk, hv, kda,
                                 [(pol, T)] * steps, cursor0, rng, fms)
        assert go < 1e-12 and gs < 1e-12, ('replay vs sequential', kda, T, L, pol, go, gs)


def pin_fold_invariance():
    """Folding at any point changes nothing: a ring too large to ever fold, forced folds at
    random steps, every-commit and lazy folds all give the same outputs (1e-12)."""
    rng = np.random.default_rng(18)
    for kda in (False, True):
        hk, hv, dk, dv, B, T, steps = 1, 2, 4, 4, 3, 3, 10
        S0 = rng.standard_normal((B, hv, dk, dv))
        slots = np.arange(B, dtype=np.int32)
        ins = [_inputs(B, T, hk, hv, dk, dv, kda, rng) for _ in range(steps)]
        accs = [rng.integers(0, T + 1, size=B).astype(np.int32) for _ in range(steps)]
        outs = []
        for L, pols in ((T * steps, [(rp.FOLD_NONE, T)] * steps),
                        (T * steps, [((rp.FOLD_FORCE if rng.random() < 0.4 else rp.FOLD_NONE), T)
                                     for _ in range(steps)]),
                        (T, [(rp.FOLD_EVERY_COMMIT, T)] * steps),
                        (2 * T, [(rp.FOLD_LAZY, T)] * steps),
                        (T + 1, [(rp.FOLD_NONE, T)] * steps)):
            layer = _layer(S0, L, hk, hv, dk, dv, kda)
            cursor = np.zeros(B, np.int32)
            fl = np.zeros(B, np.int32)
            o_all = []
            for j in range(steps):
                o, _ = rp.verify(layer, cursor, slots, ins[j])
                o_all.append(o)
                rp.cursor_advance(cursor, fl, slots, accs[j], T, L, *pols[j])
                rp.commit_fold(layer, fl, slots)
            outs.append((np.array(o_all), rp.materialize(layer, cursor, slots)))
        for o, m in outs[1:]:
            assert _rel(o, outs[0][0]) < 1e-12, ('fold invariance outputs', kda)
            assert _rel(m, outs[0][1]) < 1e-12, ('fold invariance state', kda)


def pin_cursor_bruteforce():
    """Every accept sequence over 6 steps with T = 2, L = 4 (3^6 = 729), three policies:
    cursor stays in [0, L], committed records sit at ring rows [0, cursor) in accept
    order, and the replay outputs equal the definition's."""
    T, L, steps = 2, 4, 6
    hk = hv = 1
    dk = dv = 2
    rng = np.random.default_rng(19)
    S0 = rng.standard_normal((1, hv, dk, dv))
    ins = [_inputs(1, T, hk, hv, dk, dv, False, rng) for _ in range(steps)]
    slots = np.array([0], np.int32)
    for pol in (rp.FOLD_NONE, rp.FOLD_LAZY, rp.FOLD_EVERY_COMMIT):
        for seq in itertools.product(range(T + 1), repeat=steps):
            layer = _layer(S0, L, hk, hv, dk, dv, False)
            ts = rp.TokenStream.from_replay(layer, np.zeros(1, np.int32))
            cursor = np.zeros(1, np.int32)
            fl = np.zeros(1, np.int32)
            pending = []            # keys committed since the last fold, in order
            for j, a in enumerate(seq):
                n = int(cursor[0])
                o, wp = rp.verify(layer, cursor, slots, ins[j])
                o2, _ = ts.verify(slots, ins[j])
                assert _rel(o, o2) < 1e-12
                exp_base = 0 if n + T > L else n
                assert wp[0] == exp_base
                if exp_base == 0:
                    pending = []
                acc = np.array([a], np.int32)
                folds_before = layer.fused_folds
                rp.cursor_advance(cursor, fl, slots, acc, T, L, pol, T)
                if pol == rp.FOLD_LAZY:
                    # lazy: fold exactly when the next verify of width T would overflow
                    assert (fl[0] > 0) == (exp_base + a + T > L)
                    assert layer.fused_folds == 0
                rp.commit_fold(layer, fl, slots)
                ts.accept(slots, acc)
                pending = pending + [ins[j].k[0, t] for t in range(a)]
                if fl[0]:
                    pending = []
                assert 0 <= cursor[0] <= L and cursor[0] == len(pending)
                for i, key in enumerate(pending):
                    assert np.array_equal(layer.rk[0][i], key)
            assert _rel(rp.materialize(layer, cursor, slots)[0], ts.H[0]) < 1e-12


def pin_c0_fold_count():
    """Tiny decode: capacity 4, one token per step, 12 steps -> the fused fold fires
    exactly twice, at steps 4 and 8 (cursor after each step 1,2,3,4 | 1,2,3,4 | 1,2,3,4)."""
    rng = np.random.default_rng(20)
    L, T, steps = 4, 1, 12
    S0 = rng.standard_normal((2, 1, 16, 16))
    layer = _layer(S0, L, 1, 1, 16, 16, False)
    cursor = np.zeros(2, np.int32)
    fl = np.zeros(2, np.int32)
    slots = np.array([1], np.int32)
    fired = []
    for j in range(steps):
        before = layer.fused_folds
        rp.verify(layer, cursor, slots, _inputs(1, T, 1, 1, 16, 16, False, rng))
        if layer.fused_folds != before:
            fired.append(j)
        rp.cursor_advance(cursor, fl, slots, np.array([1], np.int32), T, L, rp.FOLD_NONE)
    assert fired == [4, 8], fired
    assert cursor[1] == 4


def pin_nan_isolation():
    """Non-finite v at rejected positions never reaches accepted outputs, committed
    records or the folded state."""
    rng = np.random.default_rng(21)
    hk, hv, dk, dv, B, T, L, steps = 1, 2, 4, 4, 3, 4, 8, 6
    S0 = rng.standard_normal((B, hv, dk, dv))
    slots = np.arange(B, dtype=np.int32)
    layer = _layer(S0, L, hk, hv, dk, dv, False)
    cursor = np.zeros(B, np.int32)
    fl = np.zeros(B, np.int32)
    for j in range(steps):
        inp = _inputs(B, T, hk, hv, dk, dv, False, rng)
        acc = rng.integers(0, T, size=B).astype(np.int32)
        for r in range(B):
            for t in range(acc[r], T):
                inp.v[r, t, int(rng.integers(hv)), int(rng.integers(dv))] = \
                    (np.nan, np.inf, -np.inf)[int(rng.integers(3))]
        with np.errstate(invalid='ignore'):
            o, _ = rp.verify(layer, cursor, slots, inp)
        for r in range(B):
            assert np.all(np.isfinite(o[r, :acc[r]]))
        pol = rp.FOLD_EVERY_COMMIT if j % 2 else rp.FOLD_LAZY
        rp.cursor_advance(cursor, fl, slots, acc, T, L, pol, T)
        rp.commit_fold(layer, fl, slots)
        for s in range(B):
            assert np.all(np.isfinite(layer.S[s]))
            assert np.all(np.isfinite(layer.rd[s][:cursor[s]]))


def pin_ragged_replay_equals_sequential():
    """Ragged windows (row r verifies T_r <= T tokens, T_r = 0 included): the replay state
    machine equals the token-stream definition every step, with staggered cursors,
    history, fused and commit folds and null rows (fp64, 1e-12)."""
    rng = np.random.default_rng(22)
    for kda, T, L, pol in ((False, 4, 6, rp.FOLD_NONE), (False, 3, 5, rp.FOLD_LAZY),
                           (True, 4, 7, rp.FOLD_NONE), (False, 4, 8, rp.FOLD_EVERY_COMMIT),
                           (True, 3, 4, rp.FOLD_FORCE)):
        hk, hv, dk, dv, B, steps = 2, 4, 5, 6, 5, 10
        nslots = B + 2
        S0 = rng.standard_normal((nslots, hv, dk, dv)) * 0.3
        slots = np.array([3, -1, 0, 6, 2], np.int32)
        cursor0 = np.zeros(nslots, np.int32)
        for s in (3, 0, 6, 2):
            cursor0[s] = int(rng.integers(0, L + 1))
        ins = [_inputs(B, T, hk, hv, dk, dv, kda, rng) for _ in range(steps)]
        lens = [rng.integers(0, T + 1, size=B).astype(np.int32) for _ in range(steps)]
        accs = [np.array([rng.integers(0, l + 1) for l in ln], np.int32) for ln in lens]
        fms = [rng.integers(0, 2, size=B).astype(np.uint8) for _ in range(steps)]
        go, gs, nf, _ = run_both(S0, ins, accs, slots, L, T, hk, hv, kda,
                                 [(pol, T)] * steps, cursor0, rng, fms, lens)
        assert go < 1e-12 and gs < 1e-12, ('ragged replay vs sequential', kda, T, L, pol, go, gs)


def pin_ragged_cursor_bruteforce():
    """Every sequence of (window width, accept length) pairs over 4 steps with T = 2,
    L = 3 (6^4 = 1296), fused-only and lazy policies: each row's own width decides its
    overflow (write_pos = 0 exactly when cursor + T_r > L), the window always fits the
    ring, a width-0 window changes nothing, committed keys sit at ring rows [0, cursor)
    in accept order, and outputs and the final state equal the definition's."""
    T, L, steps = 2, 3, 4
    hk = hv = 1
    dk = dv = 2
    rng = np.random.default_rng(23)
    S0 = rng.standard_normal((1, hv, dk, dv))
    ins = [_inputs(1, T, hk, hv, dk, dv, False, rng) for _ in range(steps)]
    slots = np.array([0], np.int32)
    pairs = [(w, a) for w in range(T + 1) for a in range(w + 1)]
    for pol in (rp.FOLD_NONE, rp.FOLD_LAZY):
        for seq in itertools.product(pairs, repeat=steps):
            layer = _layer(S0, L, hk, hv, dk, dv, False)
            ts = rp.TokenStream.from_replay(layer, np.zeros(1, np.int32))
            cursor = np.zeros(1, np.int32)
            fl = np.zeros(1, np.int32)
            pending = []
            for j, (w, a) in enumerate(seq):
                n = int(cursor[0])
                ln = np.array([w], np.int32)
                S_before = layer.S[0].copy()
                o, wp = rp.verify(layer, cursor, slots, ins[j], lens=ln)
                o2, _ = ts.verify(slots, ins[j], lens=ln)
                assert np.all(np.isfinite(o[0, :w])) and np.all(np.isnan(o[0, w:]))
                if w:
                    assert _rel(o[0, :w], o2[0, :w]) < 1e-12
                exp_base = 0 if n + w > L else n
                assert wp[0] == exp_base and exp_base + w <= L
                if w == 0:
                    assert np.array_equal(layer.S[0], S_before)
                if exp_base == 0:
                    pending = []
                acc = np.array([a], np.int32)
                rp.cursor_advance(cursor, fl, slots, acc, T, L, pol, T, lens=ln)
                if pol == rp.FOLD_LAZY:
                    assert (fl[0] > 0) == (exp_base + a + T > L)
                rp.commit_fold(layer, fl, slots)
                ts.accept(slots, acc)
                pending = pending + [ins[j].k[0, t] for t in range(a)]
                if fl[0]:
                    pending = []
                assert 0 <= cursor[0] <= L and cursor[0] == len(pending)
                for i, key in enumerate(pending):
                    assert np.array_equal(layer.rk[0][i], key)
            assert _rel(rp.materialize(layer, cursor, slots)[0], ts.H[0]) < 1e-12


def pin_query_scale():
    """The query scale multiplies the outputs and nothing else: against the exact rational
    dense rule with scale 3/8 (outputs and the final state), and through the replay state
    machine, where a layer read out at scale 3/8 gives 3/8 of the scale-1 outputs with
    bit-identical states, rings and cursors."""
    rng = np.random.default_rng(24)
    sc = Fraction(3, 8)
    for kda in (False, True):
        dk, dv, T = 3, 2, 4
        S0 = [_frac_vec(rng, dk) for _ in range(dv)]
        toks = _tiny_tokens(rng, T, dk, dv, kda)
        S_ex, outs_ex = exact.run(S0, toks, kda, sc)
        S = np.array([[float(x) for x in row] for row in S0]).T
        for t, (q, k, v, beta, alpha) in enumerate(toks):
            S, _ = dr.token_update(S, _f(k), _f(v), _f(beta), _f(alpha), kda)
            assert _rel(dr.readout(S, _f(q), float(sc)), _f(outs_ex[t])) < 1e-13, ('scaled', kda, t)
        S_ex_stored = np.array([[float(x) for x in row] for row in S_ex]).T
        assert _rel(S, S_ex_stored) < 1e-13, ('scale reached the state', kda)
    hk, hv, dk, dv, B, T, L, steps = 1, 2, 4, 3, 3, 2, 5, 6
    S0 = rng.standard_normal((B, hv, dk, dv))
    slots = np.arange(B, dtype=np.int32)
    ins = [_inputs(B, T, hk, hv, dk, dv, False, rng) for _ in range(steps)]
    accs = [rng.integers(0, T + 1, size=B).astype(np.int32) for _ in range(steps)]
    runs = []
    for scale in (1.0, float(sc)):
        layer = _layer(S0, L, hk, hv, dk, dv, False)
        layer.scale = scale
        cursor = np.zeros(B, np.int32)
        fl = np.zeros(B, np.int32)
        outs = []
        for j in range(steps):
            o, _ = rp.verify(layer, cursor, slots, ins[j])
            outs.append(o)
            rp.cursor_advance(cursor, fl, slots, accs[j], T, L, rp.FOLD_NONE)
        runs.append((np.array(outs), layer, cursor.copy()))
    (o1, l1, c1), (o2, l2, c2) = runs
    assert _rel(o2, float(sc) * o1) < 1e-15, 'scaled outputs'
    assert np.array_equal(c1, c2)
    for s in range(B):
        assert np.array_equal(l1.S[s], l2.S[s]) and np.array_equal(l1.rd[s], l2.rd[s],
                                                                   equal_nan=True)


def pin_fold_policies():
    """The commit's fold policies, derived from what a fold means rather than read back
    from the oracle.  A row's committed records are either in S or in the ring, so after
    a commit that folds, the canonical S itself equals the definition's committed state
    and the cursor is 0; after one that does not, S keeps its bits and the cursor counts
    the records committed since the last fold.  Per policy:
      EVERY_COMMIT -- every live row ends every step folded;
      FORCE (seeded per-row masks) -- exactly the masked-in rows fold, the others keep
        cursor = write_pos + accept and an unchanged S;
      LAZY (next window widths 1..T+1, not only T) -- a row folds exactly when its m
        committed records plus the next window would overflow the ring.
    The pending-record count is kept here by the pin itself: a verify whose window would
    overflow first folds the whole prefix (then writes at 0), and the accept adds to it."""
    rng = np.random.default_rng(25)
    hk, hv, dk, dv, B, T, L, steps = 1, 2, 3, 3, 5, 3, 6, 14
    nslots = B + 2
    slots = np.array([4, 0, -1, 6, 2], np.int32)
    ins = [_inputs(B, T, hk, hv, dk, dv, False, rng) for _ in range(steps)]
    accs = [rng.integers(0, T + 1, size=B).astype(np.int32) for _ in range(steps)]
    masks = [rng.integers(0, 2, size=B).astype(np.uint8) for _ in range(steps)]
    next_Ts = [int(rng.integers(1, T + 2)) for _ in range(steps)]
    S0 = rng.standard_normal((nslots, hv, dk, dv)) * 0.5
    for pol in (rp.FOLD_EVERY_COMMIT, rp.FOLD_FORCE, rp.FOLD_LAZY):
        layer = _layer(S0, L, hk, hv, dk, dv, False)
        ts = rp.TokenStream.from_replay(layer, np.zeros(nslots, np.int32))
        cursor = np.zeros(nslots, np.int32)
        fl = np.zeros(nslots, np.int32)
        pend = {int(s): 0 for s in slots if s >= 0}
        folds = stays = 0
        for j in range(steps):
            rp.verify(layer, cursor, slots, ins[j])
            ts.verify(slots, ins[j])
            base = {}
            for s in pend:
                base[s] = 0 if pend[s] + T > L else pend[s]
            S_before = {s: layer.S[s].copy() for s in pend}
            rp.cursor_advance(cursor, fl, slots, accs[j], T, L, pol, next_Ts[j], masks[j])
            rp.commit_fold(layer, fl, slots)
            ts.accept(slots, accs[j])
            for r in range(B):
                s = int(slots[r])
                if s < 0:
                    continue
                m = base[s] + int(accs[j][r])
                if pol == rp.FOLD_EVERY_COMMIT:
                    want = True
                elif pol == rp.FOLD_FORCE:
                    want = bool(masks[j][r])
                else:
                    want = m + next_Ts[j] > L
                if want:
                    assert cursor[s] == 0, ('policy must fold', pol, j, r)
                    assert _rel(layer.S[s], ts.H[s]) < 1e-12, ('folded S is not committed', pol, j)
                    assert fl[s] == m
                    pend[s] = 0
                    folds += m > 0
                else:
                    assert cursor[s] == m, ('policy must not fold', pol, j, r, cursor[s], m)
                    assert np.array_equal(layer.S[s], S_before[s]), ('S changed', pol, j, r)
                    assert fl[s] == 0
                    pend[s] = m
                    stays += 1
        assert folds > 0 and (pol == rp.FOLD_EVERY_COMMIT or stays > 0), (pol, folds, stays)


# ----------------------------------------------------------------------------- conv window


def pin_conv_correlate():
    """The conv output against numpy's correlate, channel by channel (tap K-1 on the
    current input), plus the bias; with SiLU against scipy's logistic function."""
    from scipy.special import expit
    rng = np.random.default_rng(26)
    for K, T, C in ((4, 3, 5), (2, 1, 3), (3, 6, 4)):
        state = rng.standard_normal((K - 1, C))
        xw = rng.standard_normal((T, C))
        w = rng.standard_normal((C, K))
        b = rng.standard_normal(C)
        seq = np.concatenate([state, xw])
        want = np.stack([np.correlate(seq[:, c], w[c], 'valid') for c in range(C)], axis=1) + b
        got = cv.conv_verify(state, xw, w, b, cv.ACT_NONE)
        assert _rel(got, want) < 1e-14, ('conv vs correlate', K, T)
        got = cv.conv_verify(state, xw, w, b, cv.ACT_SILU)
        assert _rel(got, want * expit(want)) < 1e-14, ('conv silu', K, T)
        assert np.array_equal(cv.conv_verify(state, xw, w, None, cv.ACT_NONE),
                              cv.conv_verify(state, xw, w, np.zeros(C), cv.ACT_NONE))


def pin_conv_taps():
    """Tap K-1 alone (no bias, no activation) returns the window inputs exactly; tap 0
    alone returns the input K-1 positions back, so the first outputs are the state rows,
    oldest first."""
    rng = np.random.default_rng(27)
    K, T, C = 4, 5, 3
    state = rng.standard_normal((K - 1, C))
    xw = rng.standard_normal((T, C))
    w = np.zeros((C, K))
    w[:, K - 1] = 1.0
    assert np.array_equal(cv.conv_verify(state, xw, w, None, cv.ACT_NONE), xw)
    w = np.zeros((C, K))
    w[:, 0] = 1.0
    got = cv.conv_verify(state, xw, w, None, cv.ACT_NONE)
    assert np.array_equal(got, np.concatenate([state, xw])[:T])


def pin_conv_rollback_bruteforce():
    """Every accept sequence over 5 steps with T = 3, K = 4 (4^5 = 1024), and every
    (window width, accept) sequence over 4 steps with T = 2, K = 3 (6^4 = 1296): after each
    commit the window state equals, bit for bit, the last K-1 accepted inputs of the
    token-stream definition, and the window outputs equal the definition's convolution
    over the whole accepted history; a null row's state never changes."""
    rng = np.random.default_rng(28)
    for K, T, steps, ragged in ((4, 3, 5, False), (3, 2, 4, True)):
        C = 2
        init = rng.standard_normal((K - 1, C))
        other = rng.standard_normal((K - 1, C))
        xs = [rng.standard_normal((2, T, C)) for _ in range(steps)]
        w = rng.standard_normal((C, K))
        b = rng.standard_normal(C)
        slots = np.array([0, -1], np.int32)
        if ragged:
            pairs = [(wd, a) for wd in range(T + 1) for a in range(wd + 1)]
        else:
            pairs = [(T, a) for a in range(T + 1)]
        for seq in itertools.product(pairs, repeat=steps):
            states = {0: init.copy(), 1: other.copy()}
            stream = cv.ConvStream({0: init.copy()})
            for j, (wd, a) in enumerate(seq):
                lens = np.array([wd, 0], np.int32) if ragged else None
                y = np.full((2, T, C), np.nan)
                y[0, :wd] = cv.conv_verify(states[0], xs[j][0, :wd], w, b, cv.ACT_SILU)
                y_def = stream.verify(slots, xs[j], w, b, cv.ACT_SILU, lens=lens)
                assert np.array_equal(y[0, :wd], y_def[0, :wd])
                acc = np.array([a, T], np.int32)
                cv.conv_commit(states, slots, xs[j], acc, lens=lens)
                stream.accept(slots, xs[j], acc, lens=lens)
                assert np.array_equal(states[0], stream.state(0, K)), ('rolled state', seq, j)
                assert np.array_equal(states[1], other)


def pin_prefill_then_replay():
    """Prefill hands over to the replay state machine: prompts of ragged lengths (0
    included) through prefill, then verify steps with history, fused and commit folds,
    equal the token-stream definition that takes each prompt as accepted tokens, at every
    output and committed state (1e-12); prefill leaves every live cursor at 0 and a null
    row's slot untouched; a prompt split in two prefill calls equals one call."""
    rng = np.random.default_rng(29)
    for kda in (False, True):
        hk, hv, dk, dv, B, P, T, L, steps = 2, 4, 5, 4, 4, 9, 3, 7, 8
        nslots = B + 2
        S0 = rng.standard_normal((nslots, hv, dk, dv)) * 0.3
        slots = np.array([2, -1, 5, 0], np.int32)
        lens = np.array([9, 4, 0, 6], np.int32)
        prompt = _inputs(B, P, hk, hv, dk, dv, kda, rng)
        layer = _layer(S0, L, hk, hv, dk, dv, kda)
        ts = rp.TokenStream({s: S0[s].copy() for s in range(nslots)}, kda, hv // hk)
        cursor = np.full(nslots, 3, np.int32)          # stale counts: prefill clears them
        out = rp.prefill(layer, cursor, slots, prompt, lens)
        o_def, _ = ts.verify(slots, prompt, lens=lens)
        ts.accept(slots, lens)
        live = slots >= 0
        assert np.array_equal(np.isfinite(out), np.isfinite(o_def))
        fin = np.isfinite(o_def)
        assert _rel(out[fin], o_def[fin]) < 1e-12, ('prefill outputs', kda)
        assert np.all(cursor[slots[live]] == 0) and cursor[1] == 3 and cursor[4] == 3
        assert np.array_equal(layer.S[4], S0[4]) and np.array_equal(layer.S[5], S0[5])
        # split prompts: the first a tokens, then the rest, through two prefill calls
        l2 = _layer(S0, L, hk, hv, dk, dv, kda)
        c2 = np.zeros(nslots, np.int32)
        first = np.minimum(lens, 3)
        rp.prefill(l2, c2, slots, prompt, first)
        rest = SimpleNamespace(**{f: np.concatenate([getattr(prompt, f)[:, 3:],
                                                     getattr(prompt, f)[:, :3]], axis=1)
                                  for f in ('q', 'k', 'v', 'beta', 'gate')})
        rp.prefill(l2, c2, slots, rest, lens - first)
        for s in (2, 5, 0):
            assert _rel(l2.S[s], layer.S[s]) < 1e-12, ('split prefill', kda)
        fl = np.zeros(nslots, np.int32)
        for j in range(steps):
            inp = _inputs(B, T, hk, hv, dk, dv, kda, rng)
            acc = rng.integers(0, T + 1, size=B).astype(np.int32)
            o_rep, _ = rp.verify(layer, cursor, slots, inp)
            o2, _ = ts.verify(slots, inp)
            f = np.isfinite(o2)
            assert _rel(o_rep[f], o2[f]) < 1e-12, ('replay after prefill', kda, j)
            pol = rp.FOLD_FORCE if j % 3 == 2 else rp.FOLD_NONE
            rp.cursor_advance(cursor, fl, slots, acc, T, L, pol)
            rp.commit_fold(layer, fl, slots)
            ts.accept(slots, acc)
            for r in range(B):
                s_ = int(slots[r])
                if s_ >= 0:
                    assert _rel(layer.committed_state(s_, int(cursor[s_])), ts.H[s_]) < 1e-12


ALL_PINS = [pin_exact_rational, pin_exact_grouped_heads, pin_pure_decay, pin_identity_readout,
            pin_write_then_read, pin_grouped_write, pin_replay_equals_sequential,
            pin_fold_invariance, pin_cursor_bruteforce, pin_c0_fold_count, pin_nan_isolation,
            pin_ragged_replay_equals_sequential, pin_ragged_cursor_bruteforce, pin_query_scale,
            pin_fold_policies, pin_conv_correlate, pin_conv_taps, pin_conv_rollback_bruteforce,
            pin_prefill_then_replay]
