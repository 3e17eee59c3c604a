"""Drives a workload step by step on the GPU (through the C ABI binding) and on the fp64
oracle, and compares them.  Used by the gpu tests and by __graft_entry__.smoke().

A step of a workload: for every layer, verify; then one cursor advance for the shared
cursor; then, when the step's policy folds, one commit fold per layer.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Dict, List, Optional

import numpy as np
import torch

import workloads as W
from oracle import replay as rp

SENTINEL_OUT = 12345.0       # what null rows' outputs hold before and after a verify
SENTINEL_WP = -7


def tol_for(cfg: W.Config) -> float:
    return 5e-3 if cfg.state_dtype == 'bf16' else 1e-4


def torch_dtype(s: str):
    return torch.bfloat16 if s == 'bf16' else torch.float32


def to_dev(x: np.ndarray, dtype: str, dev) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(dev).to(torch_dtype(dtype)).contiguous()


def rel_err(gpu, ref) -> float:
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    if ref.size == 0:
        return 0.0
    denom = np.max(np.abs(ref))
    return float(np.max(np.abs(gpu - ref)) / (denom if denom > 0 else 1.0))


# ----------------------------------------------------------------------------- initial data

@dataclass
class Initial:
    slots: np.ndarray
    cursor: np.ndarray
    S: List[np.ndarray]          # per layer [num_slots, hv, dk, dv]
    rk: List[np.ndarray]
    rd: List[np.ndarray]
    rg: List[np.ndarray]


def initial(cfg: W.Config) -> Initial:
    slots = W.slot_map(cfg)
    cur = W.initial_cursor(cfg, slots)
    S, rk, rd, rg = [], [], [], []
    for layer in range(cfg.layers):
        S.append(W.initial_state(cfg, layer))
        k_, d_, g_ = W.initial_ring(cfg, cur, layer)
        rk.append(k_); rd.append(d_); rg.append(g_)
    return Initial(slots, cur, S, rk, rd, rg)


def step_windows(cfg: W.Config, j: int):
    """Per-row verify window widths of step j (ragged configs), else None."""
    return W.window_lengths(cfg, j)


def pack_windows(lens: np.ndarray, T: int):
    """Packed-token layout of ragged windows: cumulative lengths [B + 1] and, for each
    packed token, its index in the dense [B * T] layout (row r's first lens[r] tokens).
    The packed buffers get one spare token row when every window is empty, so that
    they are never empty."""
    cu = np.zeros(len(lens) + 1, np.int32)
    cu[1:] = np.cumsum(lens)
    idx = np.array([r * T + t for r in range(len(lens)) for t in range(int(lens[r]))], np.int64)
    ntok = max(int(cu[-1]), 1)
    return cu, idx, ntok


def step_data(cfg: W.Config, j: int):
    acc = W.accept_lengths(cfg, j)
    ins = [W.step_inputs(cfg, j, layer, acc) for layer in range(cfg.layers)]
    pol, next_T = W.step_policy(cfg, j)
    return acc, ins, pol, next_T


def step_force_mask(cfg: W.Config, j: int):
    """The FORCE commit's per-row mask of step j (None: every live row)."""
    return W.force_mask(cfg, j)


# ----------------------------------------------------------------------------- GPU side

class DeviceRun:
    def __init__(self, cfg: W.Config, init: Initial, dev='cuda', tile_v: int = 0):
        import linear_attention_recurrent_rs_amd as rs
        self.rs, self.cfg, self.dev = rs, cfg, dev
        self.d = rs.Dims(cfg.B, cfg.T, cfg.hk, cfg.hv, cfg.dk, cfg.dv, cfg.L, cfg.num_slots,
                         rs.BF16 if cfg.act_dtype == 'bf16' else rs.F32,
                         rs.BF16 if cfg.state_dtype == 'bf16' else rs.F32, tile_v,
                         scale=cfg.scale32)
        self.slots = torch.from_numpy(init.slots.astype(np.int32)).to(dev)
        self.cursor = torch.from_numpy(init.cursor.astype(np.int32)).to(dev)
        self.fold_len = torch.zeros(cfg.num_slots, dtype=torch.int32, device=dev)
        self.counter = torch.zeros(cfg.B * cfg.hk, dtype=torch.int32, device=dev)
        self.S = [to_dev(x, cfg.state_dtype, dev) for x in init.S]
        self.rk = [to_dev(x, cfg.act_dtype, dev) for x in init.rk]
        self.rd = [to_dev(x, 'f32', dev) for x in init.rd]
        self.rg = [to_dev(x, 'f32', dev) for x in init.rg]
        self.out = torch.full((cfg.B * cfg.T, cfg.hv, cfg.dv), SENTINEL_OUT, dtype=torch.float32, device=dev)
        self.wp = torch.full((cfg.B,), SENTINEL_WP, dtype=torch.int32, device=dev)

    def set_windows(self, lens):
        """Ragged windows for the next verifies and advance (None: every row T tokens)."""
        self.lens = lens
        if lens is None:
            return
        cu, self.pack_idx, self.ntok = pack_windows(lens, self.cfg.T)
        self.cu = torch.from_numpy(cu).to(self.dev)

    lens = None

    def inputs_dev(self, inp: W.StepInputs, clean: bool = False):
        c, dev = self.cfg, self.dev
        v = inp.v_clean if clean else inp.v
        BT = c.B * c.T
        arrays = (inp.q.reshape(BT, c.hk, c.dk), inp.k.reshape(BT, c.hk, c.dk),
                  v.reshape(BT, c.hv, c.dv), inp.beta.reshape(BT, c.hv),
                  inp.gate.reshape((BT, c.hv, c.dk) if c.kda else (BT, c.hv)))
        if self.lens is not None:
            # packed token list: the rows' windows back to back, then spare rows of zeros
            def pack(x):
                p = np.zeros((self.ntok,) + x.shape[1:])
                p[:len(self.pack_idx)] = x[self.pack_idx]
                return p
            arrays = tuple(pack(x) for x in arrays)
        return tuple(to_dev(x, c.act_dtype, dev) for x in arrays)

    def verify(self, layer: int, dev_inputs):
        q, k, v, beta, gate = dev_inputs
        self.wp.fill_(SENTINEL_WP)
        if self.lens is None:
            fn = self.rs.kda_verify if self.cfg.kda else self.rs.gdn_verify
            self.out.fill_(SENTINEL_OUT)
            fn(self.d, q, k, v, beta, gate, self.S[layer], self.rk[layer], self.rd[layer],
               self.rg[layer], self.cursor, self.slots, self.out, self.wp, self.counter)
            return self.out.clone(), self.wp.clone()
        c = self.cfg
        fn = self.rs.kda_verify_varlen if c.kda else self.rs.gdn_verify_varlen
        packed = torch.full((self.ntok, c.hv, c.dv), SENTINEL_OUT, dtype=torch.float32,
                            device=self.dev)
        fn(self.d, self.cu, q, k, v, beta, gate, self.S[layer], self.rk[layer], self.rd[layer],
           self.rg[layer], self.cursor, self.slots, packed, self.wp, self.counter)
        # back to the dense [B * T] layout; positions past a row's window hold the sentinel
        out = torch.full((c.B * c.T, c.hv, c.dv), SENTINEL_OUT, dtype=torch.float32,
                         device=self.dev)
        if len(self.pack_idx):
            out[torch.from_numpy(self.pack_idx).to(self.dev)] = packed[:len(self.pack_idx)]
        if self.ntok > len(self.pack_idx):
            assert torch.all(packed[len(self.pack_idx):] == SENTINEL_OUT), 'spare rows written'
        return out, self.wp.clone()

    def advance(self, acc: np.ndarray, pol: int, next_T: int, force_mask=None):
        a = torch.from_numpy(acc.astype(np.int32)).to(self.dev)
        fm = None if force_mask is None else torch.from_numpy(force_mask.astype(np.uint8)).to(self.dev)
        if self.lens is None:
            self.rs.cursor_advance(self.d, self.cursor, self.fold_len, self.slots, a, pol,
                                   next_T, fm)
        else:
            self.rs.cursor_advance_varlen(self.d, self.cu, self.ntok, self.cursor, self.fold_len,
                                          self.slots, a, pol, next_T, fm)

    def commit(self, layer: int):
        self.rs.commit_fold(self.d, self.cfg.kda, self.S[layer], self.rk[layer], self.rd[layer],
                            self.rg[layer], self.fold_len, self.slots)

    def materialize(self, layer: int):
        c = self.cfg
        out = torch.full((c.B, c.hv, c.dk, c.dv), SENTINEL_OUT, dtype=torch.float32, device=self.dev)
        self.rs.materialize(self.d, c.kda, self.S[layer], self.rk[layer], self.rd[layer],
                            self.rg[layer], self.cursor, self.slots, out)
        return out

    def step(self, acc, ins, pol, next_T, clean=False, lens=None, force_mask=None):
        self.set_windows(lens)
        outs, wps = [], []
        for layer in range(self.cfg.layers):
            o, w = self.verify(layer, self.inputs_dev(ins[layer], clean))
            outs.append(o); wps.append(w)
        self.advance(acc, pol, next_T, force_mask)
        if pol != W.FOLD_NONE:
            for layer in range(self.cfg.layers):
                self.commit(layer)
        return outs, wps


# ----------------------------------------------------------------------------- oracle side

class OracleRun:
    def __init__(self, cfg: W.Config, init: Initial, rows: Optional[List[int]] = None):
        self.cfg = cfg
        self.slots = init.slots.copy()
        self.rows = rows
        tracked = None if rows is None else [int(init.slots[r]) for r in rows if init.slots[r] >= 0]
        self.cursor = init.cursor.copy()
        self.fold_len = np.zeros(cfg.num_slots, np.int32)
        self.layers = [rp.ReplayLayer(init.S[l], init.rk[l], init.rd[l], init.rg[l], cfg.kda,
                                      cfg.G, cfg.L, slots=tracked, scale=cfg.scale32)
                       for l in range(cfg.layers)]
        self.streams = [rp.TokenStream.from_replay(ly, self.cursor) for ly in self.layers]

    def step(self, acc, ins, pol, next_T, with_stream=True, lens=None, force_mask=None):
        outs, wps = [], []
        for l, ly in enumerate(self.layers):
            o, w = rp.verify(ly, self.cursor, self.slots, ins[l], rows=self.rows, lens=lens)
            outs.append(o); wps.append(w)
            if with_stream:
                o2, _ = self.streams[l].verify(self.slots, ins[l], rows=self.rows, lens=lens)
                live = [r for r in (self.rows or range(self.cfg.B)) if self.slots[r] >= 0]
                for r in live:
                    fin = np.isfinite(o[r])
                    assert rel_err(o[r][fin], o2[r][fin]) < 1e-9, 'oracle models disagree'
        rp.cursor_advance(self.cursor, self.fold_len, self.slots, acc, self.cfg.T, self.cfg.L,
                          pol, next_T, force_mask, lens=lens)
        for ly in self.layers:
            rp.commit_fold(ly, self.fold_len, self.slots, rows=self.rows)
        if with_stream:
            for st in self.streams:
                st.accept(self.slots, acc, rows=self.rows)
        return outs, wps


# ----------------------------------------------------------------------------- comparison

@dataclass
class StepReport:
    out_err: float = 0.0
    state_err: float = 0.0
    ring_d_err: float = 0.0
    ints_exact: bool = True
    commit_folds: int = 0        # (row, step) pairs a folding policy folded at commit
    commit_stays: int = 0        # (row, step) pairs a folding policy left unfolded


def compare_step(cfg: W.Config, g: DeviceRun, o: OracleRun, g_outs, g_wps, o_outs, o_wps, acc,
                 rows: List[int], init: Initial, check_state: bool = True) -> StepReport:
    rep = StepReport()
    tol = tol_for(cfg)
    cursor_g = g.cursor.cpu().numpy()
    fold_g = g.fold_len.cpu().numpy()
    for l in range(cfg.layers):
        out_g = g_outs[l].cpu().numpy().reshape(cfg.B, cfg.T, cfg.hv, cfg.dv)
        wp_g = g_wps[l].cpu().numpy()
        live = [r for r in rows if o.slots[r] >= 0]
        null = [r for r in rows if o.slots[r] < 0]
        for r in null:
            assert np.all(out_g[r] == SENTINEL_OUT), f'null row {r} output written'
            assert wp_g[r] == SENTINEL_WP, f'null row {r} write_pos written'
        if live:
            ref = o_outs[l][live]
            got = out_g[live]
            fin = np.isfinite(ref)
            for i, r in enumerate(live):   # accepted positions of a row are always finite
                assert np.all(fin[i, :acc[r]]), f'oracle output not finite at accepted row {r}'
                assert np.all(np.isfinite(got[i, :acc[r]])), f'GPU output not finite at accepted row {r}'
            rep.out_err = max(rep.out_err, rel_err(got[fin], ref[fin]))
            wp_ok = all(wp_g[r] == o_wps[l][r] for r in live)
            rep.ints_exact &= wp_ok
            assert wp_ok, f'write_pos mismatch layer {l}: {[(r, wp_g[r], o_wps[l][r]) for r in live]}'
        if check_state and live:
            sl = [int(o.slots[r]) for r in live]
            idx = torch.tensor(sl, dtype=torch.long, device=g.S[l].device)
            S_g = g.S[l].index_select(0, idx).float().cpu().numpy()
            rk_g = g.rk[l].index_select(0, idx).float().cpu().numpy()
            rd_g = g.rd[l].index_select(0, idx).cpu().numpy()
            rg_g = g.rg[l].index_select(0, idx).cpu().numpy()
            ly = o.layers[l]
            for i, s in enumerate(sl):
                rep.state_err = max(rep.state_err, rel_err(S_g[i], ly.S[s]))
                c = int(o.cursor[s])
                if c:
                    assert np.array_equal(rk_g[i, :c], ly.rk[s][:c]), f'ring keys differ slot {s}'
                    assert np.array_equal(rg_g[i, :c], ly.rg[s][:c]), f'ring gates differ slot {s}'
                    rep.ring_d_err = max(rep.ring_d_err, rel_err(rd_g[i, :c], ly.rd[s][:c]))
    for r in rows:
        s = int(o.slots[r])
        if s >= 0:
            assert cursor_g[s] == o.cursor[s], f'cursor slot {s}: {cursor_g[s]} vs {o.cursor[s]}'
            assert fold_g[s] == o.fold_len[s], f'fold_len slot {s}: {fold_g[s]} vs {o.fold_len[s]}'
    assert rep.out_err <= tol, f'output error {rep.out_err:.3e} > {tol}'
    assert rep.state_err <= tol, f'state error {rep.state_err:.3e} > {tol}'
    assert rep.ring_d_err <= tol, f'ring delta error {rep.ring_d_err:.3e} > {tol}'
    return rep


def unused_slots(cfg: W.Config, init: Initial) -> List[int]:
    used = set(int(s) for s in init.slots if s >= 0)
    return [s for s in range(cfg.num_slots) if s not in used]


def check_untouched(cfg: W.Config, g: DeviceRun, init: Initial):
    """Slots no row maps to keep their state, ring and cursor bit for bit."""
    un = unused_slots(cfg, init)
    if not un:
        return
    cur = g.cursor.cpu().numpy()
    assert np.array_equal(cur[un], init.cursor[un])
    for l in range(cfg.layers):
        S0 = to_dev(init.S[l][un], cfg.state_dtype, 'cpu')
        assert torch.equal(g.S[l][un].cpu(), S0), 'unused slot state modified'
        rd = g.rd[l][un].cpu().numpy()
        assert np.array_equal(np.isnan(rd), np.isnan(init.rd[l][un])), 'unused slot ring modified'
