"""GPU parity: the HIP library against the fp64 oracle, through the C ABI.

Reduced-size copies of the five workloads compare every row, every step: outputs (finite
oracle positions; accepted positions must be finite on both sides), states and committed
ring deltas within the tolerance (1e-4 of the largest magnitude for fp32 states, 5e-3 for
bf16), ring keys/gates, write_pos, cursors and fold_len bit-exact, null rows untouched,
unused slots untouched.
"""
import json
import os

import numpy as np
import pytest
import torch

import workloads as W
from tests import harness as H

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))

REDUCED = {
    # decode: 17 rows with staggered cursors 0..15,0 (two null), 2 key / 4 value heads
    'c1': W.CONFIGS['c1'].with_(B=17, null_rows=2, hk=2, hv=4, steps=20),
    # spec verify, bf16 state, every-commit fold, NaN/Inf in rejected drafts
    'c2': W.CONFIGS['c2'].with_(B=7, hk=2, hv=4),
    # KDA, per-channel decay, fused folds
    'c3': W.CONFIGS['c3'].with_(B=5, hk=3, hv=3),
    # large ring, 4 layers sharing one cursor, forced commit folds
    'c4': W.CONFIGS['c4'].with_(B=5, hk=2, hv=4),
}


def _run(cfg, rows=None, steps=None, tile_v=0):
    init = H.initial(cfg)
    g = H.DeviceRun(cfg, init, tile_v=tile_v)
    o = H.OracleRun(cfg, init, rows=rows)
    rows = list(range(cfg.B)) if rows is None else rows
    worst = H.StepReport()
    for j in range(cfg.steps if steps is None else steps):
        acc, ins, pol, next_T = H.step_data(cfg, j)
        lens = H.step_windows(cfg, j)
        fm = H.step_force_mask(cfg, j)
        print(f'[{cfg.name}] step {j} policy {pol} next_T {next_T}' +
              ('' if lens is None else f' windows {lens.tolist()}') +
              ('' if fm is None else f' force_mask {fm.tolist()}'), flush=True)
        g_outs, g_wps = g.step(acc, ins, pol, next_T, lens=lens, force_mask=fm)
        o_outs, o_wps = o.step(acc, ins, pol, next_T, lens=lens, force_mask=fm)
        rep = H.compare_step(cfg, g, o, g_outs, g_wps, o_outs, o_wps, acc, rows, init)
        worst.out_err = max(worst.out_err, rep.out_err)
        worst.state_err = max(worst.state_err, rep.state_err)
        worst.ring_d_err = max(worst.ring_d_err, rep.ring_d_err)
        if pol != W.FOLD_NONE:
            live_s = [int(init.slots[r]) for r in rows if init.slots[r] >= 0]
            worst.commit_folds += sum(int(o.fold_len[s] > 0) for s in live_s)
            worst.commit_stays += sum(int(o.fold_len[s] == 0) for s in live_s)
    H.check_untouched(cfg, g, init)
    # the accepted state, read-only
    for l in range(cfg.layers):
        m = g.materialize(l).cpu().numpy()
        live = [r for r in rows if init.slots[r] >= 0]
        for r in rows:
            if init.slots[r] < 0:
                assert np.all(m[r] == H.SENTINEL_OUT)
        ref = np.array([o.streams[l].H[int(init.slots[r])] for r in live])
        err = H.rel_err(m[live], ref)
        assert err <= H.tol_for(cfg), f'materialize error {err:.3e}'
    print(f'[{cfg.name}] worst out {worst.out_err:.2e} state {worst.state_err:.2e} '
          f'ring_d {worst.ring_d_err:.2e}', flush=True)
    return g, o, init, worst


def test_c0_against_golden():
    cfg = W.CONFIGS['c0']
    g, o, init, _ = _run(cfg)
    gold = json.load(open(os.path.join(HERE, 'golden', 'c0_oracle.json')))
    # replay the GPU run again, checking each step against the stored fixture
    init = H.initial(cfg)
    g = H.DeviceRun(cfg, init)
    for j, st in enumerate(gold['steps']):
        acc, ins, pol, next_T = H.step_data(cfg, j)
        outs, wps = g.step(acc, ins, pol, next_T)
        assert int(wps[0][0]) == st['write_pos']
        assert int(g.cursor[gold['slot']]) == st['cursor']
        ref = np.array(st['out'])
        assert H.rel_err(outs[0].cpu().numpy().reshape(ref.shape), ref) <= 1e-4
    assert sum(s['fused_fold'] for s in gold['steps']) == 2
    S = g.S[0][gold['slot']].cpu().numpy()
    assert H.rel_err(S, np.array(gold['S_final'])) <= 1e-4


@pytest.mark.parametrize('name', sorted(REDUCED))
def test_reduced_all_rows(name):
    _run(REDUCED[name])


# ----------------------------------------------------------------------------- fold policies
# The lazy policy (fold at commit when the next verify, of width next_T, would overflow;
# next_T alternates between T and T + 1) and FORCE with a seeded per-row mask, on the
# large-ring shapes (ring 64, window 8, 4 layers sharing one cursor) and on an fp32-state
# decode with staggered cursors.

POLICIES = {
    'large_ring_lazy': REDUCED['c4'].with_(policy='lazy', steps=24),
    'large_ring_force_mask': REDUCED['c4'].with_(policy='force_mask', force_p=0.4, steps=16),
    'decode_lazy': REDUCED['c1'].with_(policy='lazy', steps=24),
    'decode_force_mask': REDUCED['c1'].with_(policy='force_mask', force_p=0.3, steps=20),
    'decode_T3_lazy': REDUCED['c1'].with_(T=3, accept=('uniform', 0, 3), policy='lazy',
                                          steps=16),
}


@pytest.mark.parametrize('name', sorted(POLICIES))
def test_fold_policies(name):
    """LAZY and per-row FORCE through rs_cursor_advance and rs_commit_fold: cursors and
    fold_len bit-exact against the oracle every step, outputs, states and ring deltas at
    tolerance.  Some rows must fold at commit and some must not."""
    cfg = POLICIES[name]
    _, _, _, worst = _run(cfg)
    print(f'[{name}] commit folds {worst.commit_folds}, rows left unfolded {worst.commit_stays}')
    assert worst.commit_folds > 0 and worst.commit_stays > 0


# ----------------------------------------------------------------------------- decode, T = 3
# The benchmark's second window width: fp32 state, 64-column tiles, window 3 (the readout
# on bf16 MFMAs over the state split into high and low parts, the fused fold on bf16 MFMAs,
# six workgroups per CU), staggered cursors so that every launch mixes history lengths
# 0..13 with rows folding in-verify.

def test_decode_T3_all_rows():
    cfg = REDUCED['c1'].with_(T=3, accept=('uniform', 1, 3), steps=24)
    _run(cfg)


@pytest.mark.parametrize('scale_name', ['rsqrt_dk', 'two'])
def test_query_scale(scale_name):
    """A query scale other than 1 (dk^-1/2 as the usual attention scale, and 2): outputs
    scaled, states and rings as at scale 1, on the fp32 decode at T = 3, the bf16 spec
    verify and KDA."""
    sc = 128 ** -0.5 if scale_name == 'rsqrt_dk' else 2.0
    _run(REDUCED['c1'].with_(T=3, accept=('uniform', 1, 3), steps=10, scale=sc))
    _run(REDUCED['c2'].with_(steps=6, scale=sc))
    _run(REDUCED['c3'].with_(steps=6, scale=sc))
    _run(W.CONFIGS['c0'].with_(steps=8, scale=sc))        # the general kernels


@pytest.mark.parametrize('tile_v', [16, 32, 128])
def test_tile_widths(tile_v):
    """Every value-tile width gives the same results (C1 shape, few steps)."""
    _run(REDUCED['c1'].with_(steps=18), tile_v=tile_v)


@pytest.mark.parametrize('name,cfg', [
    ('c1', REDUCED['c1'].with_(B=16, steps=18)),
    ('c3', REDUCED['c3'].with_(B=8, steps=10)),
])
def test_key_group_xcd_order(name, cfg):
    """Batch * key heads a multiple of 8: the verify hands whole key groups to the XCDs in
    turn (the other tests take the contiguous order)."""
    assert (cfg.B * cfg.hk) % 8 == 0
    _run(cfg)


@pytest.mark.parametrize('T,L', [(4, 16), (6, 24), (8, 40), (16, 16)])
def test_wide_windows(T, L):
    """fp32 state, 64-column tiles, windows of 4 and more (from 5 on, the readout over the
    tile runs as an MFMA contraction; T = 16: two blocks of 16 window vectors).  Windows of
    5..8 over rings of 17..64 records hold the history keys in registers, and a folding
    workgroup copies them over the scores (rings of 24 and 40 records here)."""
    cfg = W.CONFIGS['c1'].with_(B=6, null_rows=1, hk=2, hv=4, T=T, L=L,
                                accept=('uniform', 0, T), steps=8, cursor_init='zero')
    _run(cfg)


@pytest.mark.parametrize('T,L', [(3, 24), (3, 40), (4, 20)])
def test_kda_rings(T, L):
    """KDA, fp32 state, windows 3 and 4 (the split MFMA readout and the fp32-MFMA fold)
    over rings that are not multiples of 16 records: at window 3 the LDS plan places the
    history scores and the history readout over the window gates, raw keys and decayed
    vectors, and the window's gates reach the ring during the scores (or, on a fold, from
    the inputs)."""
    cfg = W.CONFIGS['c3'].with_(B=5, hk=3, hv=3, T=T, L=L, accept=('uniform', 0, T),
                                cursor_init='stagger', steps=24)
    _run(cfg)


@pytest.mark.parametrize('T', [2, 3, 4, 8])
def test_bf16_state_history_and_fused_folds(T):
    """bf16 state, 128-column tiles (the readout on bf16 MFMAs), no commit folds: rows
    replay up to L - T history records and fold in-verify when the ring would overflow,
    with staggered cursors."""
    cfg = W.CONFIGS['c2'].with_(B=6, hk=2, hv=4, T=T, accept=('uniform', 1, T), policy='none',
                                nan_frac=0.0, cursor_init='stagger', steps=14)
    _run(cfg)


@pytest.mark.parametrize('policy', ['every_commit', 'none'])
def test_kda_bf16_state(policy):
    """KDA with a bf16 state: commit folds of every accepted window, or history replay
    and in-verify folds, and the materialized state at the end."""
    cfg = W.CONFIGS['c3'].with_(B=5, hk=3, hv=3, state_dtype='bf16', policy=policy,
                                accept=('uniform', 0, 3), steps=10)
    _run(cfg)


def test_odd_shapes():
    """dk=dv=16 (one 16-wide tile), dv=48 (three 16-wide tiles), dk=64, ring == window."""
    _run(W.CONFIGS['c0'].with_(B=3, hk=1, hv=2, dk=16, dv=48, L=3, T=3, accept=('uniform', 0, 3),
                               steps=10, act_dtype='bf16'))
    _run(W.CONFIGS['c3'].with_(B=3, hk=2, hv=2, dk=64, dv=32, L=5, T=2, steps=9))


def test_error_codes():
    """Argument errors surface as exceptions before any kernel runs: the binding refuses
    host tensors and wrong sizes; the library reports RS_E_RING_TOO_SMALL and RS_E_SHAPE."""
    import linear_attention_recurrent_rs_amd as rs
    cfg = REDUCED['c1']
    init = H.initial(cfg)
    g = H.DeviceRun(cfg, init)
    acc, ins, pol, next_T = H.step_data(cfg, 0)
    q, k, v, beta, gate = g.inputs_dev(ins[0])
    args = [q, k, v, beta, gate, g.S[0], g.rk[0], g.rd[0], g.rg[0], g.cursor, g.slots, g.out,
            g.wp, g.counter]
    with pytest.raises(ValueError):                      # a host tensor
        rs.gdn_verify(g.d, q.cpu(), *args[1:])
    with pytest.raises(ValueError):                      # wrong element count
        rs.gdn_verify(g.d, q[:-1], *args[1:])
    small = rs.Dims(cfg.B, 4, cfg.hk, cfg.hv, cfg.dk, cfg.dv, 3, cfg.num_slots, rs.BF16, rs.F32, 0)
    with pytest.raises(rs.RSError) as e:
        rs.verify_launch_info(small)
    assert e.value.status == 4                           # RS_E_RING_TOO_SMALL
    kda = rs.Dims(cfg.B, 1, cfg.hk, cfg.hv, cfg.dk, cfg.dv, cfg.L, cfg.num_slots, rs.BF16, rs.F32, 0)
    with pytest.raises(rs.RSError) as e:
        rs.verify_launch_info(kda, kda=True)             # KDA needs hv == hk
    assert e.value.status == 2
    assert rs.verify_launch_info(g.d)[1] == cfg.B * cfg.hv * (cfg.dv // 64)
    rs.gdn_verify(g.d, *args)                            # the same arguments, valid
    torch.cuda.synchronize()


def test_empty_batch_and_all_null():
    import linear_attention_recurrent_rs_amd as rs
    cfg = REDUCED['c1'].with_(B=4, null_rows=4, steps=2)
    init = H.initial(cfg)
    g = H.DeviceRun(cfg, init)
    for j in range(2):
        acc, ins, pol, next_T = H.step_data(cfg, j)
        outs, wps = g.step(acc, ins, pol, next_T)
        assert torch.all(outs[0] == H.SENTINEL_OUT) and torch.all(wps[0] == H.SENTINEL_WP)
    H.check_untouched(cfg, g, init)
    d0 = rs.Dims(0, 1, 1, 1, 16, 16, 4, 1, rs.F32, rs.F32, 0)   # empty batch: a no-op
    assert rs._lib().rs_gdn_verify(rs.ctypes.byref(d0), *([None] * 14), None) == 0


# ----------------------------------------------------------------------------- ragged windows
# Each row verifies its own number of draft tokens from one packed token list (cumulative
# lengths), widths U{0..T} per row and step, so empty windows occur in every step.

RAGGED = {
    # GDN, fp32 state, staggered cursors, fused folds decided by each row's own width
    'gdn': W.CONFIGS['ragged_gdn'].with_(B=13, null_rows=2, hk=2, hv=4),
    # KDA, per-channel decays
    'kda': W.CONFIGS['ragged_kda'].with_(B=7, hk=3, hv=3),
    # spec verify flavour: bf16 state, every-commit fold, NaN/Inf in rejected drafts
    'gdn_bf16_every_commit': W.CONFIGS['c2'].with_(B=7, hk=2, hv=4, ragged=('uniform', 0, 4)),
    # large ring, windows up to 8 (the MFMA readout), 4 layers sharing one cursor
    'large_ring': W.CONFIGS['c4'].with_(B=5, hk=2, hv=4, steps=20, ragged=('uniform', 0, 8)),
    # the general kernels (dk 32, dv 48, fp32 activations)
    'general_kernel': W.CONFIGS['ragged_gdn'].with_(B=9, null_rows=1, hk=1, hv=2, dk=32, dv=48,
                                                    act_dtype='f32', steps=12),
}


@pytest.mark.parametrize('name', sorted(RAGGED))
def test_ragged_windows(name):
    _run(RAGGED[name])


def test_ragged_empty_and_full_windows():
    """Edge widths: a step where every window is empty (cursors, states and rings keep
    their bits; write_pos = cursor), then steps where every window is full width (the
    ragged call then gives exactly the uniform call's bits)."""
    import linear_attention_recurrent_rs_amd as rs
    cfg = RAGGED['gdn'].with_(steps=3)
    init = H.initial(cfg)
    g = H.DeviceRun(cfg, init)
    o = H.OracleRun(cfg, init)
    u = H.DeviceRun(cfg, init)                      # the same workload through the uniform call
    zeros = np.zeros(cfg.B, np.int32)
    acc, ins, pol, next_T = H.step_data(cfg, 0)
    S0 = [x.clone() for x in g.S]
    cur0 = g.cursor.clone()
    g_outs, g_wps = g.step(zeros, ins, pol, next_T, lens=zeros)
    o_outs, o_wps = o.step(zeros, ins, pol, next_T, lens=zeros)
    H.compare_step(cfg, g, o, g_outs, g_wps, o_outs, o_wps, zeros, list(range(cfg.B)), init)
    live = init.slots >= 0
    assert torch.equal(g.cursor, cur0)
    assert all(torch.equal(a, b) for a, b in zip(g.S, S0))
    assert torch.all(g_outs[0] == H.SENTINEL_OUT)
    assert np.array_equal(g_wps[0].cpu().numpy()[live], init.cursor[init.slots[live]])
    u.step(zeros, ins, pol, next_T, lens=zeros)
    full = np.full(cfg.B, cfg.T, np.int32)
    for j in range(1, 3):
        acc, ins, pol, next_T = H.step_data(cfg, j)
        g_outs, g_wps = g.step(acc, ins, pol, next_T, lens=full)
        u_outs, u_wps = u.step(acc, ins, pol, next_T)
        assert torch.equal(g_outs[0], u_outs[0]) and torch.equal(g_wps[0], u_wps[0])
        assert torch.equal(g.cursor, u.cursor) and torch.equal(g.S[0], u.S[0])
        assert torch.equal(torch.nan_to_num(g.rd[0], nan=7.0), torch.nan_to_num(u.rd[0], nan=7.0))
    d = g.d
    with pytest.raises(ValueError):               # cu_seqlens of the wrong length
        rs.gdn_verify_varlen(d, g.cu[:-1], *g.inputs_dev(ins[0]), g.S[0], g.rk[0], g.rd[0],
                             g.rg[0], g.cursor, g.slots,
                             torch.empty(g.ntok, cfg.hv, cfg.dv, device=g.dev), g.wp, g.counter)
    torch.cuda.synchronize()
