"""GPU parity of the conv window (rs_conv_verify, rs_conv_commit) against the fp64 oracle
(oracle.conv), through the C ABI.

Each step: the window's outputs against the token-stream definition (fp32 outputs within
1e-5 of the largest magnitude; bf16 outputs within one bf16 rounding, 2^-8, plus 1e-5),
then the rollback: every live slot's state bit for bit equal to the oracle's (a copy of
the K-1 inputs ending at the last accepted draft); null rows' outputs keep their sentinel
and slots no row maps to keep their bits.
"""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import conv as cv
from tests import harness as H

pytestmark = pytest.mark.gpu

SENT = 4352.0                  # exact in bf16 and fp32


def _run(cfg, rows=None):
    import linear_attention_recurrent_rs_amd as rs
    rc = cfg.as_config()
    slots = W.slot_map(rc)
    w, b, st0 = W.conv_params(cfg)
    act = rs.BF16 if cfg.act_dtype == 'bf16' else rs.F32
    out = rs.BF16 if cfg.out_dtype == 'bf16' else rs.F32
    d = rs.ConvDims(cfg.B, cfg.T, cfg.C, cfg.K, cfg.num_slots, act, out,
                    rs.ACT_SILU if cfg.silu else rs.ACT_NONE)
    state = H.to_dev(st0, cfg.act_dtype, 'cuda')
    w_d = H.to_dev(w, cfg.act_dtype, 'cuda')
    b_d = None if b is None else H.to_dev(b, cfg.act_dtype, 'cuda')
    slot_d = torch.from_numpy(slots.astype(np.int32)).cuda()
    live = [r for r in range(cfg.B) if slots[r] >= 0]
    rows = live if rows is None else [r for r in rows if slots[r] >= 0]
    states = {int(slots[r]): st0[slots[r]].copy() for r in rows}
    stream = cv.ConvStream({int(slots[r]): st0[slots[r]].copy() for r in rows})
    sub = np.full(cfg.B, -1, np.int32)
    sub[rows] = slots[rows]
    tol = (2.0 ** -8 + 1e-5) if cfg.out_dtype == 'bf16' else 1e-5
    worst = 0.0
    for j in range(cfg.steps):
        x = W.conv_inputs(cfg, j)
        acc = W.accept_lengths(rc, j)
        lens = W.window_lengths(rc, j)
        print(f'[{cfg.name}] step {j} accept {acc.tolist()[:8]}', flush=True)
        if lens is None:
            x_d = H.to_dev(x.reshape(cfg.B * cfg.T, cfg.C), cfg.act_dtype, 'cuda')
            cu_d, idx = None, np.arange(cfg.B * cfg.T)
        else:
            cu, idx, ntok = H.pack_windows(lens, cfg.T)
            packed = np.zeros((ntok, cfg.C))
            packed[:len(idx)] = x.reshape(cfg.B * cfg.T, cfg.C)[idx]
            x_d = H.to_dev(packed, cfg.act_dtype, 'cuda')
            cu_d = torch.from_numpy(cu).cuda()
        y = torch.full((x_d.shape[0], cfg.C), SENT, dtype=H.torch_dtype(cfg.out_dtype),
                       device='cuda')
        rs.conv_verify(d, x_d, w_d, b_d, state, slot_d, y, cu_seqlens=cu_d)
        yd = np.full((cfg.B * cfg.T, cfg.C), np.nan)
        yd[idx] = y.float().cpu().numpy()[:len(idx)]
        yd = yd.reshape(cfg.B, cfg.T, cfg.C)
        ref = stream.verify(sub, x, w, b, cv.ACT_SILU if cfg.silu else cv.ACT_NONE, lens=lens)
        for r in range(cfg.B):
            T_r = cfg.T if lens is None else int(lens[r])
            if slots[r] < 0:
                assert np.all(yd[r, :T_r] == SENT), f'null row {r} written'
            elif r in rows and T_r:
                err = H.rel_err(yd[r, :T_r], ref[r, :T_r])
                worst = max(worst, err)
                assert err <= tol, f'step {j} row {r}: output error {err:.3e} > {tol}'
        before = state.clone()
        rs.conv_commit(d, state, x_d, slot_d, torch.from_numpy(acc).cuda(), cu_seqlens=cu_d)
        stream.accept(sub, x, acc, lens=lens)
        cv.conv_commit(states, sub, x, acc, lens=lens)
        got = state.float().cpu().numpy()
        for r in rows:
            s = int(slots[r])
            assert np.array_equal(got[s], states[s]), f'step {j} slot {s}: rolled state differs'
            assert np.array_equal(states[s], stream.state(s, cfg.K))
        used = set(int(s) for s in slots if s >= 0)
        un = [s for s in range(cfg.num_slots) if s not in used]
        assert torch.equal(state[un], before[un]), 'a slot no row maps to changed'
    print(f'[{cfg.name}] worst output error {worst:.2e}', flush=True)


SMALL = W.ConvConfig('conv_small', B=17, null_rows=2, C=64, K=4, T=1, accept=('const', 1), steps=6)
CASES = {
    'decode_bf16_silu': SMALL,
    'spec_window4_bf16_out': SMALL.with_(B=7, C=48, T=4, accept=('uniform', 0, 4), out_dtype='bf16',
                                         steps=8, seed=12),
    'fp32_width3_plain': SMALL.with_(B=5, null_rows=1, C=32, K=3, T=3, accept=('uniform', 0, 3),
                                     act_dtype='f32', silu=False, bias=False, seed=13),
    'width2_window16': SMALL.with_(B=4, null_rows=0, C=16, K=2, T=16, accept=('uniform', 0, 16),
                                   steps=4, seed=14),
    'ragged_windows': SMALL.with_(B=9, null_rows=2, C=40, T=4, accept=('uniform', 0, 4),
                                  ragged=('uniform', 0, 4), steps=8, seed=15),
}


@pytest.mark.parametrize('name', sorted(CASES))
def test_conv_window(name):
    _run(CASES[name])


def test_conv_full_size_sampled():
    """Qwen3.5-shaped channels (2 x 16 x 128 q/k + 32 x 128 v = 8192), batch 128, window
    4, accept U{0..4}: every row on the GPU, 6 rows checked against the oracle."""
    cfg = W.CONV_CONFIGS['conv_spec'].with_(steps=4)
    _run(cfg, rows=[0, 1, 37, 64, 100, 127])


def test_conv_commit_layers():
    """One rs_conv_commit launch rolls back three layers stacked layer-major (each with its
    own states and window inputs); every layer's states equal the oracle's bit for bit."""
    import linear_attention_recurrent_rs_amd as rs
    cfg = SMALL.with_(B=6, null_rows=1, C=24, T=3, accept=('uniform', 0, 3), seed=16)
    rc = cfg.as_config()
    slots = W.slot_map(rc)
    layers = 3
    d = rs.ConvDims(cfg.B, cfg.T, cfg.C, cfg.K, cfg.num_slots, rs.BF16, rs.F32, rs.ACT_SILU)
    sts = [W.conv_params(cfg.with_(seed=20 + l))[2] for l in range(layers)]
    xs = [W.conv_inputs(cfg.with_(seed=30 + l), 0) for l in range(layers)]
    acc = W.accept_lengths(rc, 0)
    state = H.to_dev(np.stack(sts), cfg.act_dtype, 'cuda')
    x_d = H.to_dev(np.stack(xs).reshape(layers, cfg.B * cfg.T, cfg.C), cfg.act_dtype, 'cuda')
    rs.conv_commit(d, state, x_d, torch.from_numpy(slots.astype(np.int32)).cuda(),
                   torch.from_numpy(acc).cuda(), layers=layers)
    got = state.float().cpu().numpy()
    assert any(acc[r] > 0 for r in range(cfg.B) if slots[r] >= 0)
    for l in range(layers):
        want = {s: sts[l][s].copy() for s in range(cfg.num_slots)}
        cv.conv_commit(want, slots, xs[l], acc)
        for s in range(cfg.num_slots):
            assert np.array_equal(got[l, s], want[s]), f'layer {l} slot {s}'
