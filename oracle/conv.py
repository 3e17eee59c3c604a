"""Short causal convolution with a per-slot window state, and its rollback at commit, in
fp64 (oracle; test infrastructure only).

What the pages give.  The LightLLM page ("feat: add ReplaySSM state modes for GDN and
KDA") lists Conv/SSM state management and MTP accept/rollback among what the state modes
cover (PR description), copies "the accepted conv window" together with the canonical SSM
when a page is saved or moved between processes, and gives a restored slot only the
canonical conv and SSM state (commit messages).  The sglang page (GDN ReplaySSM spec
verify for DFLASH/DSPARK) has the GDN ring commit do three things: cursor advance, fold of
the accepted window into the checkpoint, and conv rollback (commit 4); its verify views
the window "from the conv on" (commit 2).  The pages print none of the convolution.

Readings (the plainest ones the rest supports; each listed in the design notes):
  * The convolution is the short causal depthwise convolution a GDN layer applies to its
    mixed q/k/v channels before the recurrence: channel c of token t is
        y_t[c] = act( sum_{j<K} w[c][j] * x_{t-K+1+j}[c] + b[c] ),
    tap K-1 on the current token, act = identity or SiLU (x * sigmoid(x)), bias optional.
  * The conv state of a slot is its last K-1 committed pre-conv inputs, oldest first:
    state [K-1, C].  A verify of T draft tokens reads the state and the window and writes
    T outputs; it leaves the state alone.
  * The commit rolls the state to the window ending at the last accepted draft: over the
    sequence state ++ window (K-1+T inputs), the new state is inputs [a, a+K-1) for an
    accept length a; a = 0 keeps it.  (A rejected draft's input never enters the state.)

Two models, checked against each other by the pins:
  ConvStream -- the definition: the full list of a slot's accepted inputs, the conv taken
                directly over it.
  conv_verify / conv_commit -- the window-state machine above.
"""
from __future__ import annotations

from typing import Dict, List, Optional

import numpy as np

ACT_NONE, ACT_SILU = 0, 1


def silu(x):
    """x * sigmoid(x) = x / (1 + exp(-x)), in fp64."""
    x = np.asarray(x, dtype=np.float64)
    return x / (1.0 + np.exp(-x))


def activate(y, act: int):
    if act == ACT_NONE:
        return y
    if act == ACT_SILU:
        return silu(y)
    raise ValueError(act)


def conv_at(seq: np.ndarray, t: int, w: np.ndarray, b: Optional[np.ndarray], act: int):
    """Output at position t of a sequence seq [n, C] (t >= K-1): the K inputs ending at t,
    tap j on seq[t-K+1+j]."""
    K = w.shape[1]
    y = np.zeros(seq.shape[1])
    for j in range(K):
        y = y + w[:, j] * seq[t - K + 1 + j]
    if b is not None:
        y = y + b
    return activate(y, act)


def conv_verify(state: np.ndarray, xw: np.ndarray, w, b, act: int):
    """Window outputs of one row: state [K-1, C] (oldest first), window inputs xw [T, C].
    Returns y [T, C]; the state is not changed."""
    seq = np.concatenate([state, xw], axis=0)
    K = w.shape[1]
    y = np.zeros(xw.shape)
    for t in range(xw.shape[0]):
        y[t] = conv_at(seq, K - 1 + t, w, b, act)
    return y


def rolled_state(state: np.ndarray, xw: np.ndarray, a: int) -> np.ndarray:
    """The state after accepting the first a drafts of the window: inputs [a, a+K-1) of
    state ++ window."""
    seq = np.concatenate([state, xw[:a]], axis=0)
    return seq[len(seq) - state.shape[0]:].copy()


def conv_commit(states: Dict[int, np.ndarray], slots, x, accept, lens=None):
    """Roll every live row's state (in place).  x [B, T, C] window inputs; accept [B];
    lens: ragged window widths [B] or None.  Null rows (slot < 0) are skipped."""
    for r, s in enumerate(slots):
        s = int(s)
        if s < 0:
            continue
        T = x.shape[1] if lens is None else int(lens[r])
        a = min(max(int(accept[r]), 0), T)
        states[s] = rolled_state(states[s], x[r, :T], a)


class ConvStream:
    """The definition: each slot's accepted pre-conv inputs in order, starting with the K-1
    inputs its state was initialised with; outputs are the convolution taken over that
    list extended by the window."""

    def __init__(self, init_states: Dict[int, np.ndarray]):
        self.seq: Dict[int, List[np.ndarray]] = {s: [row for row in st]
                                                 for s, st in init_states.items()}

    def verify(self, slots, x, w, b, act, lens=None):
        B, Tb, C = x.shape
        y = np.full(x.shape, np.nan)
        for r, s in enumerate(slots):
            s = int(s)
            if s < 0 or s not in self.seq:
                continue
            T = Tb if lens is None else int(lens[r])
            full = np.array(self.seq[s] + [x[r, t] for t in range(T)])
            n0 = len(self.seq[s])
            for t in range(T):
                y[r, t] = conv_at(full, n0 + t, w, b, act)
        return y

    def accept(self, slots, x, accept, lens=None):
        for r, s in enumerate(slots):
            s = int(s)
            if s < 0 or s not in self.seq:
                continue
            T = x.shape[1] if lens is None else int(lens[r])
            a = min(max(int(accept[r]), 0), T)
            self.seq[s].extend(x[r, t] for t in range(a))

    def state(self, s: int, K: int) -> np.ndarray:
        """The last K-1 accepted inputs of slot s, oldest first."""
        return np.array(self.seq[s][len(self.seq[s]) - (K - 1):])
