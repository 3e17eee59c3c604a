"""CPU tests: the fp64 oracle against its pins, and planted mistakes against the pins."""
import numpy as np
import pytest

import oracle.conv as cv
import oracle.delta_rule as dr
import oracle.replay as rp
from tests import oracle_pins as pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    with np.errstate(invalid='ignore', over='ignore'):
        pin()


# ---------------------------------------------------------------- planted mistakes
# Each mutant replaces one oracle function with a plausible wrong version.  The pins
# must reject every one of them (at least one pin fails).

def _tu_sign(S, k, v, beta, alpha, kda):
    Sd = dr.decay(S, alpha, kda)
    d = np.asarray(beta)[..., None] * (v + np.einsum('...ij,...i->...j', Sd, k))
    return Sd + np.einsum('...i,...j->...ij', k, d), d


def _tu_nobeta(S, k, v, beta, alpha, kda):
    Sd = dr.decay(S, alpha, kda)
    d = v - np.einsum('...ij,...i->...j', Sd, k)
    return Sd + np.einsum('...i,...j->...ij', k, d), d


def _tu_pred_undecayed(S, k, v, beta, alpha, kda):
    Sd = dr.decay(S, alpha, kda)
    d = np.asarray(beta)[..., None] * (v - np.einsum('...ij,...i->...j', S, k))
    return Sd + np.einsum('...i,...j->...ij', k, d), d


def _tu_decay_after(S, k, v, beta, alpha, kda):
    d = np.asarray(beta)[..., None] * (v - np.einsum('...ij,...i->...j', S, k))
    return dr.decay(S + np.einsum('...i,...j->...ij', k, d), alpha, kda), d


def _tu_kda_columns(S, k, v, beta, alpha, kda):
    alpha = np.asarray(alpha)
    Sd = S * alpha[..., None, :] if kda else dr.decay(S, alpha, kda)
    d = np.asarray(beta)[..., None] * (v - np.einsum('...ij,...i->...j', Sd, k))
    return Sd + np.einsum('...i,...j->...ij', k, d), d


def _readout_transposed(S, q, scale=1.0):
    return float(scale) * np.einsum('...ij,...j->...i', S, q)


def _expand_tile(x, G):
    return np.concatenate([x] * G, axis=-2)


def _apply_record_nodecay(S, k, d, alpha, kda):
    return S + np.einsum('...i,...j->...ij', k, d)


def _fold_now_early(n, T, L):
    return n + T >= L


def _lazy_late(m, next_T, L):
    return m + next_T > L + 1


def _window_ignored(T, lens, r):
    return T


def _readout_unscaled(S, q, scale=1.0):
    return np.einsum('...ij,...i->...j', S, q)


def _readout_scaled_twice(S, q, scale=1.0):
    return float(scale) ** 2 * np.einsum('...ij,...i->...j', S, q)


_policy_folds = rp.policy_folds


def _every_commit_never(policy, m, next_T, L, masked_in):
    return False if policy == rp.FOLD_EVERY_COMMIT else _policy_folds(policy, m, next_T, L, masked_in)


def _force_ignores_mask(policy, m, next_T, L, masked_in):
    return True if policy == rp.FOLD_FORCE else _policy_folds(policy, m, next_T, L, masked_in)


def _force_mask_inverted(policy, m, next_T, L, masked_in):
    return (not masked_in) if policy == rp.FOLD_FORCE else _policy_folds(policy, m, next_T, L,
                                                                          masked_in)


def _lazy_ignores_next_width(policy, m, next_T, L, masked_in):
    return rp.lazy_fold(m, 1, L) if policy == rp.FOLD_LAZY else _policy_folds(policy, m, next_T,
                                                                                L, masked_in)


def _rolled_one_late(state, xw, a):
    seq = np.concatenate([state, xw[:a + 1]], axis=0)
    return seq[len(seq) - state.shape[0]:].copy()


def _rolled_newest_first(state, xw, a):
    seq = np.concatenate([state, xw[:a]], axis=0)
    return seq[len(seq) - state.shape[0]:][::-1].copy()


def _conv_taps_reversed(seq, t, w, b, act):
    K = w.shape[1]
    y = np.zeros(seq.shape[1])
    for j in range(K):
        y = y + w[:, K - 1 - j] * seq[t - K + 1 + j]
    return cv.activate(y + (0 if b is None else b), act)


def _conv_bias_after_act(seq, t, w, b, act):
    K = w.shape[1]
    y = np.zeros(seq.shape[1])
    for j in range(K):
        y = y + w[:, j] * seq[t - K + 1 + j]
    return cv.activate(y, act) + (0 if b is None else b)


_prefill = rp.prefill


def _prefill_keeps_cursor(layer, cursor, slots, inp, lens, rows=None):
    saved = cursor.copy()
    out = _prefill(layer, cursor, slots, inp, lens, rows)
    cursor[:] = saved
    return out


def _prefill_from_zero(layer, cursor, slots, inp, lens, rows=None):
    for s in slots:
        if s >= 0 and int(s) in layer.S:
            layer.S[int(s)] = np.zeros_like(layer.S[int(s)])
    return _prefill(layer, cursor, slots, inp, lens, rows)


def _prefill_drops_last(layer, cursor, slots, inp, lens, rows=None):
    return _prefill(layer, cursor, slots, inp, np.maximum(np.asarray(lens) - 1, 0), rows)


MUTANTS = {
    'ragged window width ignored': [('window', _window_ignored)],
    'd sign flipped': [('token_update', _tu_sign)],
    'beta dropped from d': [('token_update', _tu_nobeta)],
    'prediction from undecayed state': [('token_update', _tu_pred_undecayed)],
    'decay applied after the write': [('token_update', _tu_decay_after)],
    'KDA decay on value axis': [('token_update', _tu_kda_columns)],
    'readout transposed': [('readout', _readout_transposed)],
    'key heads tiled, not grouped': [('expand_heads', _expand_tile)],
    'record replay drops decay': [('apply_record', _apply_record_nodecay)],
    'fused fold one record early': [('fold_now', _fold_now_early)],
    'lazy fold one record late': [('lazy_fold', _lazy_late)],
    'query scale dropped': [('readout', _readout_unscaled)],
    'query scale applied twice': [('readout', _readout_scaled_twice)],
    'every-commit policy never folds': [('policy_folds', _every_commit_never)],
    'force policy ignores its mask': [('policy_folds', _force_ignores_mask)],
    'force policy mask inverted': [('policy_folds', _force_mask_inverted)],
    'lazy policy ignores the next window width': [('policy_folds', _lazy_ignores_next_width)],
    'conv state rolled one input late': [('rolled_state', _rolled_one_late)],
    'conv state kept newest first': [('rolled_state', _rolled_newest_first)],
    'conv taps reversed': [('conv_at', _conv_taps_reversed)],
    'conv bias added after the activation': [('conv_at', _conv_bias_after_act)],
    'prefill keeps the stale cursor': [('prefill', _prefill_keeps_cursor)],
    'prefill starts from a zero state': [('prefill', _prefill_from_zero)],
    'prefill drops the last prompt token': [('prefill', _prefill_drops_last)],
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_reject_mutant(name, monkeypatch):
    for attr, fn in MUTANTS[name]:
        for mod in (dr, rp, cv):
            if hasattr(mod, attr):
                monkeypatch.setattr(mod, attr, fn)
    caught = []
    for pin in pins.ALL_PINS:
        try:
            with np.errstate(all='ignore'):
                pin()
        except (AssertionError, ValueError, IndexError):
            caught.append(pin.__name__)
    assert caught, f"no pin rejects the mutant '{name}'"
