"""ReplaySSM state machine and token-stream model in fp64 (oracle; test infrastructure only).

Method (the three pages, read together):
  * The canonical per-slot state S[hv, dk, dv] stays in place.  Accepted tokens become
    history records (key, fp32 delta, gate) in a per-slot ring, and a per-slot cursor
    counts the committed records (LightLLM "feat: add ReplaySSM state modes for GDN and
    KDA": history buffers and cursors live on the state; delta history is fp32).
  * Verify writes the T draft records at ring positions [write_pos, write_pos + T)
    (sglang GDN ReplaySSM spec-verify PR, commit 1) after replaying the committed
    history over S (commit 5: history terms, skipped when write_pos is 0).
  * When the next verify would exceed the ring, the whole prefix is folded into S first,
    inside the verify (LightLLM commit messages: compaction is lazy and triggered by a
    verify that would not fit, a decision taken on the device; PR description: the fold
    runs inside the decode kernel).
    Then write_pos = 0.
  * After every layer of a step, the shared cursor advances by the accept length (the
    rejected tail is trimmed; LightLLM commits on the shared cursor being advanced only
    after the last layer).  A fold policy may fold the committed window into S at commit
    time (sglang commit 4: fold every commit; lazy fold with an early flush that reads
    the draft length; LightLLM force_compress).
  * Rows whose state slot is negative are skipped by every kernel (sglang commit 1).

Ragged windows (LightLLM commit: decode reads every request's window from cumulative
sequence lengths, q, k, v laid out [tokens, heads, dim]; sglang Modifications: per-request
verify lengths packed into one token list).  Row r may verify T_r <= T draft tokens; every
per-row rule below then reads the row's own T_r, and T_r = 0 leaves the row as it is.

Readings where the pages are silent (each listed in the design notes):
  * cursor n, window T, capacity L:  fold_now = n + T > L;  write_pos = 0 if fold_now else n.
  * advance: m = write_pos + accept; fold_len = policy(m); cursor = 0 if fold_len else m.
  * the commit fold reads fold_len only, never the cursor, so layers sharing one cursor
    all fold the same prefix.

Two models are kept and tested against each other:
  TokenStream  -- the definition: per slot the committed state is the recurrence over
                  accepted tokens; a verify continues it over the window.
  ReplayLayer  -- the state machine above, with an explicit ring and cursor.
Integer results of the state machine (cursor, write_pos, fold_len, record positions)
are the exact reference for the GPU.
"""
from __future__ import annotations

from typing import Dict, Iterable, Optional

import numpy as np

from .delta_rule import expand_heads, fold, readout, token_update

FOLD_NONE, FOLD_EVERY_COMMIT, FOLD_LAZY, FOLD_FORCE = 0, 1, 2, 3


def fold_now(n: int, T: int, L: int) -> bool:
    """A verify of width T on a cursor of n records overflows a ring of L: fold first."""
    return n + T > L


def lazy_fold(m: int, next_T: int, L: int) -> bool:
    """Lazy policy: fold at commit only when the next verify (width next_T) would overflow."""
    return m + next_T > L


def policy_folds(policy: int, m: int, next_T: int, L: int, masked_in: bool) -> bool:
    """Whether the commit folds a row that ends its step with m committed records.

    EVERY_COMMIT folds every accepted window into S (sglang commit 4: the DFLASH/DSPARK
    commit folds the accepted window into the checkpoint).  LAZY folds only when the next
    verify, of width next_T, would not fit in the ring (LightLLM lazy compaction; sglang
    commit 4: the lazy fold's early flush reads the draft length).  FORCE folds the rows
    the caller selects (LightLLM force_compress).  NONE leaves every fold to the verify."""
    if policy == FOLD_NONE:
        return False
    if policy == FOLD_EVERY_COMMIT:
        return True
    if policy == FOLD_LAZY:
        return lazy_fold(m, next_T, L)
    if policy == FOLD_FORCE:
        return bool(masked_in)
    raise ValueError(policy)


def window(T: int, lens, r: int) -> int:
    """Window width of row r: the batch's T, or lens[r] when windows are ragged."""
    return T if lens is None else int(lens[r])


def _rows(slots, rows: Optional[Iterable[int]]):
    rr = range(len(slots)) if rows is None else rows
    return [r for r in rr if slots[r] >= 0]


class ReplayLayer:
    """One layer: canonical state and history ring per tracked slot (fp64 copies).

    S0 [num_slots, hv, dk, dv]; ring_k [num_slots, L, hk, dk]; ring_d [num_slots, L, hv,
    dv]; ring_g [num_slots, L, hv] (GDN) or [num_slots, L, hv, dk] (KDA).  Only ``slots``
    (default: all) are tracked, so a few rows of a large batch can be followed alone.
    """

    def __init__(self, S0, ring_k, ring_d, ring_g, kda: bool, G: int, L: int,
                 slots: Optional[Iterable[int]] = None, scale: float = 1.0):
        self.kda, self.G, self.L, self.scale = kda, G, L, float(scale)
        idx = range(S0.shape[0]) if slots is None else sorted(set(int(s) for s in slots if s >= 0))
        self.S: Dict[int, np.ndarray] = {s: np.array(S0[s], dtype=np.float64) for s in idx}
        self.rk = {s: np.array(ring_k[s], dtype=np.float64) for s in idx}
        self.rd = {s: np.array(ring_d[s], dtype=np.float64) for s in idx}
        self.rg = {s: np.array(ring_g[s], dtype=np.float64) for s in idx}
        self.fused_folds = 0

    def _fold_prefix(self, S, s, n):
        """fold(S, ring[s, 0:n]) -- the records' keys expanded to value heads."""
        ks = expand_heads(self.rk[s][:n], self.G)
        return fold(S, ks, self.rd[s][:n], self.rg[s][:n], self.kda)

    def committed_state(self, s, n):
        return self._fold_prefix(self.S[s], s, n)


def verify(layer: ReplayLayer, cursor, slots, inp, rows=None, lens=None):
    """Verify of one layer.  ``inp`` has q, k [B,T,hk,dk], v [B,T,hv,dv], beta [B,T,hv],
    gate [B,T,hv] or [B,T,hv,dk].  With ``lens`` (ragged windows) row r verifies its
    first lens[r] <= T tokens.  Returns (out [B,T,hv,dv] with NaN for rows and positions
    not processed, write_pos [B] with -1 for rows not processed).  The cursor is read
    only."""
    B, Tb = inp.v.shape[:2]
    L, G, kda = layer.L, layer.G, layer.kda
    out = np.full(inp.v.shape, np.nan)
    write_pos = np.full(B, -1, dtype=np.int32)
    for r in _rows(slots, rows):
        s = int(slots[r])
        if s not in layer.S:
            continue
        n = int(cursor[s])
        T = window(Tb, lens, r)
        if fold_now(n, T, L):               # the window would overflow: fold first
            layer.S[s] = layer._fold_prefix(layer.S[s], s, n)
            layer.fused_folds += 1
            base = 0
        else:
            base = n
        H = layer._fold_prefix(layer.S[s], s, base)
        ks = expand_heads(inp.k[r], G)
        qs = expand_heads(inp.q[r], G)
        for t in range(T):
            H, d = token_update(H, ks[t], inp.v[r, t], inp.beta[r, t], inp.gate[r, t], kda)
            out[r, t] = readout(H, qs[t], layer.scale)
            layer.rk[s][base + t] = inp.k[r, t]
            layer.rd[s][base + t] = d
            layer.rg[s][base + t] = inp.gate[r, t]
        write_pos[r] = base
    return out, write_pos


def cursor_advance(cursor, fold_len, slots, accept, T: int, L: int, policy: int,
                   next_T: int = 0, force_mask=None, lens=None):
    """Advance the shared cursor once per step, after every layer's verify (in place).

    write_pos is recomputed from the unchanged cursor exactly as verify derived it (with
    the row's own window width when ``lens`` gives ragged windows).
    fold_len[s] = m under EVERY_COMMIT, under LAZY when m + next_T > L, under FORCE for
    rows in force_mask (all rows when None), else 0.  Null rows touch nothing."""
    for r in range(len(slots)):
        s = int(slots[r])
        if s < 0:
            continue
        n = int(cursor[s])
        base = 0 if fold_now(n, window(T, lens, r), L) else n
        m = base + int(accept[r])
        masked_in = force_mask is None or bool(force_mask[r])
        fl = m if policy_folds(policy, m, next_T, L, masked_in) else 0
        fold_len[s] = fl
        cursor[s] = 0 if fl else m


def commit_fold(layer: ReplayLayer, fold_len, slots, rows=None):
    """S[s] = fold(S[s], ring[s, 0:fold_len[s]]) for live rows; reads fold_len only."""
    for r in _rows(slots, rows):
        s = int(slots[r])
        if s not in layer.S:
            continue
        n = int(fold_len[s])
        if n:
            layer.S[s] = layer._fold_prefix(layer.S[s], s, n)


def materialize(layer: ReplayLayer, cursor, slots, rows=None):
    """Accepted state fold(S[s], ring[s, 0:cursor[s]]) per live row, read-only.
    Returns [B, hv, dk, dv] with NaN for rows not processed."""
    B = len(slots)
    some = next(iter(layer.S.values()))
    out = np.full((B,) + some.shape, np.nan)
    for r in _rows(slots, rows):
        s = int(slots[r])
        if s in layer.S:
            out[r] = layer.committed_state(s, int(cursor[s]))
    return out


def prefill(layer: ReplayLayer, cursor, slots, inp, lens, rows=None):
    """Prefill of each row's prompt (LightLLM commit messages: prefill writes the canonical
    SSM directly and leaves the cursor at zero).  ``inp`` holds q, k [B, P, hk, dk], v
    [B, P, hv, dv], beta, gate [B, P, hv] with row r's prompt in its first lens[r] tokens.
    The state runs token by token from the slot's canonical S, which then holds the
    state after the last prompt token; the cursor becomes 0.  A slot's ring records are
    not read: the caller folds any pending ones first (a forced commit), so S is the
    committed state.  Returns out [B, P, hv, dv], NaN where no token was processed."""
    B, P = inp.v.shape[:2]
    out = np.full(inp.v.shape, np.nan)
    for r in _rows(slots, rows):
        s = int(slots[r])
        if s not in layer.S:
            continue
        H = layer.S[s]
        ks = expand_heads(inp.k[r], layer.G)
        qs = expand_heads(inp.q[r], layer.G)
        for t in range(int(lens[r])):
            H, _ = token_update(H, ks[t], inp.v[r, t], inp.beta[r, t], inp.gate[r, t], layer.kda)
            out[r, t] = readout(H, qs[t], layer.scale)
        layer.S[s] = H
        cursor[s] = 0
    return out


class TokenStream:
    """The definition: per slot, the committed state is the gated delta rule run over the
    accepted tokens in order; a verify runs the T draft tokens on from it."""

    def __init__(self, committed: Dict[int, np.ndarray], kda: bool, G: int, scale: float = 1.0):
        self.H = {s: np.array(v, dtype=np.float64) for s, v in committed.items()}
        self.kda, self.G, self.scale = kda, G, float(scale)
        self._window = {}

    @classmethod
    def from_replay(cls, layer: ReplayLayer, cursor):
        return cls({s: layer.committed_state(s, int(cursor[s])) for s in layer.S},
                   layer.kda, layer.G, layer.scale)

    def verify(self, slots, inp, rows=None, lens=None):
        B, Tb = inp.v.shape[:2]
        out = np.full(inp.v.shape, np.nan)
        dels = np.full(inp.v.shape, np.nan)
        self._window = {}
        for r in _rows(slots, rows):
            s = int(slots[r])
            if s not in self.H:
                continue
            H = self.H[s]
            ks = expand_heads(inp.k[r], self.G)
            qs = expand_heads(inp.q[r], self.G)
            states = []
            for t in range(window(Tb, lens, r)):
                H, d = token_update(H, ks[t], inp.v[r, t], inp.beta[r, t], inp.gate[r, t],
                                    self.kda)
                out[r, t] = readout(H, qs[t], self.scale)
                dels[r, t] = d
                states.append(H)
            self._window[s] = states
        return out, dels

    def window_state(self, s: int, t: int) -> np.ndarray:
        """The state after draft token t of slot s's last verify: what the snapshot-verify
        baseline keeps per draft token (sglang PR, the snapshot verify it replaces)."""
        return self._window[s][t]

    def accept(self, slots, accept, rows=None):
        for r in _rows(slots, rows):
            s = int(slots[r])
            if s in self._window and accept[r] > 0:
                self.H[s] = self._window[s][int(accept[r]) - 1]
        self._window = {}
