"""Seeded synthetic workloads for the ReplaySSM decode / speculative-verify path.

This module only draws random numbers: token inputs (q, k, v, beta, gate), accept
lengths, row-to-slot maps, NaN/Inf injection sites, an initial recurrent state and a
prefilled history ring.  It evaluates none of the gated delta rule.  Both the fp64
oracle (``oracle/``) and the HIP library take its arrays as given, so it is the only
code the two sides share.

Every array is returned as float64 holding values that are exactly representable in
the dtype they will be stored in (fp32 or bf16): casts go fp64 -> fp32 -> bf16 with
round-to-nearest-even, so handing the same numbers to the GPU in that dtype is exact.

Distributions follow the workload descriptions: q, k ~ N(0,1) then L2-normalised over
the key dimension; v ~ N(0,1); beta ~ U(0,1); the gate is a linear decay
alpha = exp(-softplus(x)), x ~ N(0,1), a scalar per value head (GDN) or a vector over
dk per head (KDA).  The pages print no initial state; ``initial_state`` draws a
plausible one (a decayed sum of random outer products) with no recurrence in it.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Optional

import numpy as np

# fold policies, numbered as in include/rs.h
FOLD_NONE, FOLD_EVERY_COMMIT, FOLD_LAZY, FOLD_FORCE = 0, 1, 2, 3


@dataclass(frozen=True)
class Config:
    name: str
    kda: bool
    B: int               # request rows in the batch
    null_rows: int       # rows whose state slot is -1
    hk: int              # key heads
    hv: int              # value heads (GQA group G = hv // hk)
    dk: int
    dv: int
    state_dtype: str     # 'f32' | 'bf16'
    act_dtype: str       # 'f32' | 'bf16'
    L: int               # history ring capacity (records)
    T: int               # verify window
    accept: tuple        # ('const', a) | ('uniform', lo, hi) | ('binomial', n, p)
    steps: int
    layers: int = 1
    seed: int = 0
    nan_frac: float = 0.0        # probability a rejected position gets a non-finite v entry
    cursor_init: str = 'zero'    # 'zero' | 'stagger' (cursor = row mod L, ring prefilled)
    policy: str = 'none'         # 'none' | 'every_commit' | 'lazy' | 'force_mask' | 'c4_schedule'
    extra_slots: int = 16
    ragged: tuple = ()           # () = every row verifies T tokens; ('uniform', lo, hi) =
                                 # per-row window widths U{lo..hi} (packed token list)
    scale: float = 1.0           # query scale of the outputs, o = scale S^T q
    force_p: float = 0.0         # 'force_mask' policy: probability a row is masked in

    @property
    def G(self) -> int:
        return self.hv // self.hk

    @property
    def scale32(self) -> float:
        """The query scale as the fp32 value the library receives."""
        return float(np.float32(self.scale))

    @property
    def num_slots(self) -> int:
        return self.B + self.extra_slots

    @property
    def live_rows(self) -> int:
        return self.B - self.null_rows

    def with_(self, **kw) -> "Config":
        return replace(self, **kw)


# The five workload configurations (tiny GDN, GDN decode, GDN spec verify, KDA verify,
# large ring with compact commit).  Unstated choices (step counts of the spec-verify and
# large-ring cases, the slot pool, the stagger) are documented readings.
CONFIGS = {
    'c0': Config('c0', False, B=1, null_rows=0, hk=1, hv=1, dk=16, dv=16,
                 state_dtype='f32', act_dtype='f32', L=4, T=1, accept=('const', 1),
                 steps=12, seed=0, extra_slots=1),
    'c1': Config('c1', False, B=64, null_rows=4, hk=16, hv=32, dk=128, dv=128,
                 state_dtype='f32', act_dtype='bf16', L=16, T=1, accept=('const', 1),
                 steps=32, seed=1, cursor_init='stagger'),
    'c2': Config('c2', False, B=128, null_rows=0, hk=16, hv=32, dk=128, dv=128,
                 state_dtype='bf16', act_dtype='bf16', L=16, T=4, accept=('uniform', 0, 4),
                 steps=12, seed=2, nan_frac=0.05, policy='every_commit'),
    'c3': Config('c3', True, B=64, null_rows=0, hk=32, hv=32, dk=128, dv=128,
                 state_dtype='f32', act_dtype='bf16', L=16, T=3, accept=('uniform', 1, 3),
                 steps=24, seed=3),
    'c4': Config('c4', False, B=256, null_rows=0, hk=16, hv=32, dk=128, dv=128,
                 state_dtype='f32', act_dtype='bf16', L=64, T=8, accept=('binomial', 8, 0.7),
                 steps=32, layers=4, seed=4, policy='c4_schedule'),
}


# Ragged verify windows (packed per-request verify lengths), beside the five workloads:
# GDN and KDA layers of the same shapes, widths U{0..4} per row and step, staggered cursors.
CONFIGS['ragged_gdn'] = Config('ragged_gdn', False, B=64, null_rows=4, hk=16, hv=32, dk=128,
                               dv=128, state_dtype='f32', act_dtype='bf16', L=16, T=4,
                               accept=('uniform', 0, 4), steps=16, seed=5,
                               cursor_init='stagger', ragged=('uniform', 0, 4))
CONFIGS['ragged_kda'] = Config('ragged_kda', True, B=64, null_rows=0, hk=32, hv=32, dk=128,
                               dv=128, state_dtype='f32', act_dtype='bf16', L=16, T=4,
                               accept=('uniform', 0, 4), steps=16, seed=6,
                               cursor_init='stagger', ragged=('uniform', 0, 4))


def step_policy(cfg: Config, step: int):
    """(policy, next_T) used by the cursor advance after ``step``'s verifies.

    c4_schedule: steps 0-15 rely on the fused in-verify fold only; from step 16 on, every
    third step forces a commit fold of every live row (the force_compress switch).
    lazy: fold at commit when the next verify would overflow; the next window width
    alternates between T and T + 1 (capped at 16), so the policy must read next_T, not T.
    force_mask: FORCE with a seeded per-row mask every step (``force_mask``).
    """
    if cfg.policy == 'none':
        return FOLD_NONE, cfg.T
    if cfg.policy == 'every_commit':
        return FOLD_EVERY_COMMIT, cfg.T
    if cfg.policy == 'lazy':
        return FOLD_LAZY, min(cfg.T + (step % 2), 16)
    if cfg.policy == 'force_mask':
        return FOLD_FORCE, cfg.T
    if cfg.policy == 'c4_schedule':
        if step >= 16 and (step - 16) % 3 == 0:
            return FOLD_FORCE, cfg.T
        return FOLD_NONE, cfg.T
    raise ValueError(cfg.policy)


# ----------------------------------------------------------------------------- rounding

def to_f32(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def to_bf16(x) -> np.ndarray:
    """fp64 -> fp32 -> bf16, round-to-nearest-even; returned as float64.  Finite inputs only."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float64).astype(np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def to_dtype(x, dtype: str) -> np.ndarray:
    if dtype == 'f32':
        return to_f32(x)
    if dtype == 'bf16':
        return to_bf16(x)
    raise ValueError(dtype)


# ----------------------------------------------------------------------------- RNG

def _rng(cfg: Config, *purpose: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([cfg.seed, *purpose]))


_P_SLOTS, _P_STATE, _P_RING, _P_TOKENS, _P_ACCEPT, _P_NAN, _P_WINDOW, _P_FORCE = 1, 2, 3, 4, 5, 6, 7, 8


def _unit(rng, shape):
    x = rng.standard_normal(shape)
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _gate(rng, shape):
    x = rng.standard_normal(shape)
    return np.exp(-np.logaddexp(0.0, x))      # exp(-softplus(x)) in (0, 1)


# ----------------------------------------------------------------------------- pieces

def slot_map(cfg: Config) -> np.ndarray:
    """int32 [B]: a seeded injective row -> slot map; ``null_rows`` seeded rows get -1."""
    rng = _rng(cfg, _P_SLOTS)
    slots = rng.permutation(cfg.num_slots)[:cfg.B].astype(np.int32)
    if cfg.null_rows:
        null = rng.choice(cfg.B, size=cfg.null_rows, replace=False)
        slots[null] = -1
    return slots


def initial_state(cfg: Config, layer: int = 0) -> np.ndarray:
    """[num_slots, hv, dk, dv] in the state dtype: sum_i w_i k_i u_i^T, W=16 random unit
    keys, u_i ~ N(0, 0.5^2), w_i = 0.6^(W-1-i).  Every slot gets one (unused slots too)."""
    rng = _rng(cfg, _P_STATE, layer)
    W = 16
    ks = _unit(rng, (cfg.num_slots, cfg.hv, W, cfg.dk))
    us = 0.5 * rng.standard_normal((cfg.num_slots, cfg.hv, W, cfg.dv))
    w = 0.6 ** np.arange(W - 1, -1, -1, dtype=np.float64)
    S = np.einsum('shwi,w,shwj->shij', ks, w, us, optimize=True)
    return to_dtype(S, cfg.state_dtype)


def initial_cursor(cfg: Config, slots: np.ndarray) -> np.ndarray:
    """int32 [num_slots]; 0 everywhere, or row mod L for live rows under 'stagger'."""
    cur = np.zeros(cfg.num_slots, dtype=np.int32)
    if cfg.cursor_init == 'stagger':
        for r, s in enumerate(slots):
            if s >= 0:
                cur[s] = r % cfg.L
    return cur


def initial_ring(cfg: Config, cursor: np.ndarray, layer: int = 0, fill=np.nan):
    """History ring (ring_k [S,L,hk,dk], ring_d [S,L,hv,dv], ring_g [S,L,hv] or [S,L,hv,dk]).

    Records [0, cursor[s]) hold random committed history: unit keys in the activation
    dtype, deltas ~ N(0, 0.5^2) in fp32, gates from the gate distribution.  Every other
    entry holds ``fill`` (NaN by default), so a read outside the committed prefix shows.
    """
    rng = _rng(cfg, _P_RING, layer)
    S, L = cfg.num_slots, cfg.L
    rk = np.full((S, L, cfg.hk, cfg.dk), fill)
    rd = np.full((S, L, cfg.hv, cfg.dv), fill)
    gshape = (S, L, cfg.hv, cfg.dk) if cfg.kda else (S, L, cfg.hv)
    rg = np.full(gshape, fill)
    for s in range(S):
        c = int(cursor[s])
        if c == 0:
            continue
        rk[s, :c] = to_dtype(_unit(rng, (c, cfg.hk, cfg.dk)), cfg.act_dtype)
        rd[s, :c] = to_f32(0.5 * rng.standard_normal((c, cfg.hv, cfg.dv)))
        rg[s, :c] = to_dtype(_gate(rng, (c,) + gshape[2:]), cfg.act_dtype)
    return rk, rd, rg


def force_mask(cfg: Config, step: int) -> Optional[np.ndarray]:
    """uint8 [B]: the rows a FORCE commit folds at ``step`` under the 'force_mask' policy
    (each row masked in with probability force_p), else None (every live row)."""
    if cfg.policy != 'force_mask':
        return None
    rng = _rng(cfg, _P_FORCE, step)
    return (rng.random(cfg.B) < cfg.force_p).astype(np.uint8)


def window_lengths(cfg: Config, step: int) -> Optional[np.ndarray]:
    """int32 [B]: each row's verify window width at ``step`` (ragged configs), else None."""
    if not cfg.ragged:
        return None
    kind, lo, hi = cfg.ragged
    if kind != 'uniform':
        raise ValueError(kind)
    rng = _rng(cfg, _P_WINDOW, step)
    return np.clip(rng.integers(lo, hi + 1, size=cfg.B), 0, cfg.T).astype(np.int32)


def accept_lengths(cfg: Config, step: int) -> np.ndarray:
    """int32 [B] in [0, T] (ragged: in [0, T_r]), drawn before the step's verify."""
    rng = _rng(cfg, _P_ACCEPT, step)
    kind = cfg.accept[0]
    if kind == 'const':
        a = np.full(cfg.B, cfg.accept[1])
    elif kind == 'uniform':
        a = rng.integers(cfg.accept[1], cfg.accept[2] + 1, size=cfg.B)
    elif kind == 'binomial':
        a = rng.binomial(cfg.accept[1], cfg.accept[2], size=cfg.B)
    else:
        raise ValueError(kind)
    a = np.clip(a, 0, cfg.T)
    lens = window_lengths(cfg, step)
    if lens is not None:
        a = np.minimum(a, lens)
    return a.astype(np.int32)


@dataclass
class StepInputs:
    q: np.ndarray        # [B, T, hk, dk]
    k: np.ndarray        # [B, T, hk, dk]
    v: np.ndarray        # [B, T, hv, dv]   (may hold injected NaN/Inf at rejected positions)
    beta: np.ndarray     # [B, T, hv]
    gate: np.ndarray     # [B, T, hv] (GDN) or [B, T, hv, dk] (KDA)
    v_clean: np.ndarray  # v before injection
    injected: list = field(default_factory=list)   # (row, t, head, col) of each injected entry


def step_inputs(cfg: Config, step: int, layer: int = 0,
                accept: Optional[np.ndarray] = None) -> StepInputs:
    rng = _rng(cfg, _P_TOKENS, layer, step)
    B, T = cfg.B, cfg.T
    q = to_dtype(_unit(rng, (B, T, cfg.hk, cfg.dk)), cfg.act_dtype)
    k = to_dtype(_unit(rng, (B, T, cfg.hk, cfg.dk)), cfg.act_dtype)
    v = to_dtype(rng.standard_normal((B, T, cfg.hv, cfg.dv)), cfg.act_dtype)
    beta = to_dtype(rng.uniform(0.0, 1.0, (B, T, cfg.hv)), cfg.act_dtype)
    gshape = (B, T, cfg.hv, cfg.dk) if cfg.kda else (B, T, cfg.hv)
    gate = to_dtype(_gate(rng, gshape), cfg.act_dtype)
    v_clean = v.copy()
    injected = []
    if cfg.nan_frac > 0.0:
        if accept is None:
            accept = accept_lengths(cfg, step)
        nrng = _rng(cfg, _P_NAN, layer, step)
        specials = (np.nan, np.inf, -np.inf)
        for r in range(B):
            for t in range(int(accept[r]), T):
                if nrng.random() < cfg.nan_frac:
                    h = int(nrng.integers(cfg.hv))
                    c = int(nrng.integers(cfg.dv))
                    v[r, t, h, c] = specials[int(nrng.integers(3))]
                    injected.append((r, t, h, c))
    return StepInputs(q, k, v, beta, gate, v_clean, injected)


def reduced(cfg: Config, **kw) -> Config:
    """A smaller copy of a config for exhaustive (all-row) parity at oracle-friendly sizes."""
    return cfg.with_(**kw)


# ----------------------------------------------------------------------------- conv window
# The short causal convolution before the recurrence: window inputs, taps, bias and the
# initial per-slot window state, all drawn at random (nothing of the convolution itself).

@dataclass(frozen=True)
class ConvConfig:
    name: str
    B: int
    null_rows: int
    C: int               # channels (the mixed q/k/v channels of a GDN layer)
    K: int               # convolution width
    T: int               # verify window
    accept: tuple
    steps: int
    act_dtype: str = 'bf16'
    out_dtype: str = 'f32'
    silu: bool = True
    bias: bool = True
    seed: int = 7
    extra_slots: int = 16
    ragged: tuple = ()

    @property
    def num_slots(self) -> int:
        return self.B + self.extra_slots

    def with_(self, **kw) -> "ConvConfig":
        return replace(self, **kw)

    def as_config(self) -> Config:
        """The matching recurrent-layer config, for the slot map, accepts and windows."""
        return Config(self.name, False, B=self.B, null_rows=self.null_rows, hk=1, hv=1, dk=16,
                      dv=16, state_dtype='f32', act_dtype=self.act_dtype, L=max(self.T, 16),
                      T=self.T, accept=self.accept, steps=self.steps, seed=self.seed,
                      extra_slots=self.extra_slots, ragged=self.ragged)


# Qwen3.5-shaped GDN layer: 16 key heads x 128 for q and for k, 32 value heads x 128 for v
CONV_CONFIGS = {
    'conv_decode': ConvConfig('conv_decode', B=64, null_rows=4, C=2 * 16 * 128 + 32 * 128, K=4,
                              T=1, accept=('const', 1), steps=8),
    'conv_spec': ConvConfig('conv_spec', B=128, null_rows=0, C=2 * 16 * 128 + 32 * 128, K=4,
                            T=4, accept=('uniform', 0, 4), steps=8, seed=8),
}


def conv_params(cfg: ConvConfig):
    """(weight [C, K], bias [C] or None, initial state [num_slots, K-1, C]) in the
    activation dtype, as float64."""
    rng = _rng(cfg.as_config(), 9)
    w = to_dtype(rng.standard_normal((cfg.C, cfg.K)) / np.sqrt(cfg.K), cfg.act_dtype)
    b = to_dtype(0.1 * rng.standard_normal(cfg.C), cfg.act_dtype) if cfg.bias else None
    st = to_dtype(rng.standard_normal((cfg.num_slots, cfg.K - 1, cfg.C)), cfg.act_dtype)
    return w, b, st


def conv_inputs(cfg: ConvConfig, step: int) -> np.ndarray:
    """Window inputs x [B, T, C] of a step, N(0, 1) in the activation dtype."""
    rng = _rng(cfg.as_config(), 10, step)
    return to_dtype(rng.standard_normal((cfg.B, cfg.T, cfg.C)), cfg.act_dtype)
