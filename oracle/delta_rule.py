"""The gated delta rule in fp64 (oracle; test infrastructure only).

Definition (Gated DeltaNet; KDA when the decay is a vector over the key channels).  In
the key-to-value orientation the rule reads

    S_t = S_{t-1} . diag-or-scalar(alpha_t) . (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
    o_t = S_t q_t,

with S_t of shape [dv, dk].  The state is stored transposed, one [dk, dv] matrix per
value head, which is the layout the LightLLM page "feat: add ReplaySSM state modes for
GDN and KDA" keeps as the canonical SSM (commit messages on accepted-state
materialization and on folding with real strides).  Written for the stored matrix
S = S_math^T the same rule is

    S'  = alpha (.) S          GDN: scalar alpha; KDA: row i (key channel i) times alpha[i]
    d   = beta (v - S'^T k)    the fp32 "delta" / update the history ring stores
    S   = S' + k d^T
    o   = scale S^T q          (read from the post-update state; scale is the caller's
                                query scale, applied to the output and nothing else)

Expanding (I - beta k k^T) shows the two forms are equal; ``oracle.exact`` evaluates the
dense left-hand form in rational arithmetic and the pin tests hold this one to it.

Grouped heads: value head h reads key head h // G with G = hv / hk, so neighbouring value
heads share a key head (LightLLM page, commit on program order: adjacent value heads
share the key-head fold barrier).
"""
from __future__ import annotations

import numpy as np


def expand_heads(x: np.ndarray, G: int) -> np.ndarray:
    """[..., hk, dk] -> [..., hk*G, dk]; value head h takes key head h // G."""
    return np.repeat(x, G, axis=-2)


def decay(S: np.ndarray, alpha, kda: bool) -> np.ndarray:
    """alpha (.) S on S[..., dk, dv]: a scalar per head (GDN) or a dk-vector per head (KDA)."""
    alpha = np.asarray(alpha, dtype=np.float64)
    if kda:
        return S * alpha[..., :, None]
    return S * alpha[..., None, None]


def token_update(S, k, v, beta, alpha, kda: bool):
    """One token of the rule.  S [..., dk, dv], k [..., dk], v [..., dv], beta [...],
    alpha [...] (GDN) or [..., dk] (KDA).  Returns (S_new, d) with d [..., dv]."""
    Sd = decay(S, alpha, kda)
    pred = np.einsum('...ij,...i->...j', Sd, k)
    d = np.asarray(beta, dtype=np.float64)[..., None] * (v - pred)
    return Sd + np.einsum('...i,...j->...ij', k, d), d


def readout(S, q, scale=1.0):
    """o = scale * S^T q over the key axis: S [..., dk, dv], q [..., dk] -> [..., dv]."""
    return float(scale) * np.einsum('...ij,...i->...j', S, q)


def apply_record(S, k, d, alpha, kda: bool):
    """Replay one stored record (k, d, alpha): S <- alpha (.) S + k d^T.  With d taken from
    token_update this reproduces that token's update exactly (same d)."""
    return decay(S, alpha, kda) + np.einsum('...i,...j->...ij', k, d)


def fold(S, ks, ds, gs, kda: bool):
    """Apply records i = 0..n-1 in order.  ks [n, ..., dk], ds [n, ..., dv], gs [n, ...]
    (GDN) or [n, ..., dk] (KDA).  n = 0 returns S unchanged (a copy)."""
    S = np.array(S, dtype=np.float64, copy=True)
    for i in range(len(ks)):
        S = apply_record(S, ks[i], ds[i], gs[i], kda)
    return S


def run_tokens(S, ks, vs, betas, alphas, qs, kda: bool, scale=1.0):
    """Sequential recurrence over tokens t = 0..T-1 (leading axis).  Returns
    (final state, outputs [T, ..., dv], deltas [T, ..., dv], states after each token)."""
    outs, dels, states = [], [], []
    for t in range(len(ks)):
        S, d = token_update(S, ks[t], vs[t], betas[t], alphas[t], kda)
        outs.append(readout(S, qs[t], scale))
        dels.append(d)
        states.append(S)
    return S, np.array(outs), np.array(dels), states
