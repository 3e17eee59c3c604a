"""GPU parity of the snapshot-verify baseline (rs_snapshot_verify / rs_snapshot_commit)
against the fp64 token-stream definition, through the C ABI.

The snapshot verify runs the recurrence token by token from the slot's state and writes
the state after every draft token; the commit copies the accepted one back.  Checked per
step of a chained run (the definition is never restarted from the GPU's state): outputs
and every snapshot against the definition's states after each draft token (at positions
where the definition is finite), the committed state bit for bit equal to the accepted
snapshot, null rows and unused slots untouched, and the ReplaySSM verify of the same
workload giving the same outputs within tolerance.  fp32 states are held to 1e-4; bf16
states to a bound derived from the roundings this baseline performs (``_run_snapshot``).
"""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import replay as rp
from tests import harness as H

pytestmark = pytest.mark.gpu


def _dev_inputs(cfg, inp):
    BT = cfg.B * cfg.T
    gsh = (BT, cfg.hv, cfg.dk) if cfg.kda else (BT, cfg.hv)
    return (H.to_dev(inp.q.reshape(BT, cfg.hk, cfg.dk), cfg.act_dtype, 'cuda'),
            H.to_dev(inp.k.reshape(BT, cfg.hk, cfg.dk), cfg.act_dtype, 'cuda'),
            H.to_dev(inp.v.reshape(BT, cfg.hv, cfg.dv), cfg.act_dtype, 'cuda'),
            H.to_dev(inp.beta.reshape(BT, cfg.hv), cfg.act_dtype, 'cuda'),
            H.to_dev(inp.gate.reshape(gsh), cfg.act_dtype, 'cuda'))


U_BF16 = 2.0 ** -8      # bf16 round-to-nearest-even: |x - rne(x)| <= 2^-8 |x|


def _colnorm(x):
    """2-norms of the state columns (over dk) of [..., dk, dv] arrays."""
    return np.sqrt(np.sum(np.asarray(x, np.float64) ** 2, axis=-2))


def _run_snapshot(cfg, steps):
    """Chained run against the fp64 definition (never restarted from the GPU's state).

    fp32 states: every output, snapshot and committed state within 1e-4 of the largest
    magnitude.  bf16 states: the baseline keeps each workgroup's tile in fp32 through a
    verify and rounds twice: every snapshot it writes, and (by copying a rounded snapshot)
    the state at every commit.  The error a rounding adds to one state column (a dk-vector)
    is at most 2^-8 times that column's 2-norm, and the token map column by column,
    s <- alpha (I - beta k k^T) s + beta k v (GDN; KDA: with diag(alpha)), never lengthens an
    error vector: alpha <= 1, and (I - beta k k^T) has eigenvalues 1 and 1 - beta |k|^2, in
    [-1, 1] for beta in [0, 1] and |k| ~ 1.  So after j commits a column's error is at most
    j 2^-8 smax (smax the largest column 2-norm the definition reaches), a snapshot's at most
    (j + 1) 2^-8 smax, and an output's at most scale |q| j 2^-8 smax, plus fp32 arithmetic
    (slack 1e-5 smax).  The bound is checked column by column; the one-step error of a
    teacher-forced definition (restarted from the committed bf16 state each step) is
    printed beside it as a diagnostic."""
    import linear_attention_recurrent_rs_amd as rs
    init = H.initial(cfg)
    slots = init.slots
    live = [r for r in range(cfg.B) if slots[r] >= 0]
    tol = H.tol_for(cfg)
    bf16 = cfg.state_dtype == 'bf16'
    d = rs.Dims(cfg.B, cfg.T, cfg.hk, cfg.hv, cfg.dk, cfg.dv, cfg.L, cfg.num_slots,
                rs.BF16 if cfg.act_dtype == 'bf16' else rs.F32,
                rs.BF16 if cfg.state_dtype == 'bf16' else rs.F32, 0, scale=cfg.scale32)
    sdt = H.torch_dtype(cfg.state_dtype)
    S = H.to_dev(init.S[0], cfg.state_dtype, 'cuda')
    S_init = S.clone()
    snaps = torch.full((cfg.B, cfg.T, cfg.hv, cfg.dk, cfg.dv), 7.0, dtype=sdt, device='cuda')
    out = torch.full((cfg.B * cfg.T, cfg.hv, cfg.dv), H.SENTINEL_OUT, device='cuda')
    slot_d = torch.from_numpy(slots.astype(np.int32)).cuda()
    committed0 = {int(slots[r]): init.S[0][slots[r]] for r in live}
    ts = rp.TokenStream(committed0, cfg.kda, cfg.G, cfg.scale32)
    forced = rp.TokenStream(committed0, cfg.kda, cfg.G, cfg.scale32)   # diagnostic only
    smax = max(float(_colnorm(x).max()) for x in committed0.values())
    worst = worst_ratio = forced_err = 0.0
    for j in range(steps):
        acc, ins, _, _ = H.step_data(cfg, j)
        print(f'[{cfg.name} snapshot] step {j}', flush=True)
        rs.snapshot_verify(d, cfg.kda, *_dev_inputs(cfg, ins[0]), S, snaps, slot_d, out)
        o_ref, _ = ts.verify(slots, ins[0])
        o_frc, _ = forced.verify(slots, ins[0])
        o_gpu = out.cpu().numpy().reshape(cfg.B, cfg.T, cfg.hv, cfg.dv)
        sn = snaps.float().cpu().numpy()
        for r in live:
            s = int(slots[r])
            for t in range(cfg.T):
                ref = ts.window_state(s, t)
                if np.all(np.isfinite(ref)):
                    smax = max(smax, float(_colnorm(ref).max()))
        qn = float(np.max(np.linalg.norm(ins[0].q, axis=-1)))
        for r in range(cfg.B):
            if slots[r] < 0:
                assert np.all(o_gpu[r] == H.SENTINEL_OUT) and np.all(sn[r] == 7.0), 'null row written'
                continue
            s = int(slots[r])
            fin = np.isfinite(o_ref[r])
            assert np.all(fin[:acc[r]]) and np.all(np.isfinite(o_gpu[r, :acc[r]]))
            if bf16:
                bound = abs(cfg.scale32) * qn * (j * U_BF16 + 1e-5) * smax
                err = float(np.max(np.abs(o_gpu[r][fin] - o_ref[r][fin]), initial=0.0))
                worst_ratio = max(worst_ratio, err / bound)
                assert err <= bound, f'step {j} row {r}: output error {err:.3e} > {bound:.3e}'
                forced_err = max(forced_err, H.rel_err(o_gpu[r][o_frc[r] == o_frc[r]],
                                                       o_frc[r][o_frc[r] == o_frc[r]]))
            else:
                worst = max(worst, H.rel_err(o_gpu[r][fin], o_ref[r][fin]))
            for t in range(cfg.T):
                ref = ts.window_state(s, t)
                if not np.all(np.isfinite(ref)):
                    continue
                if bf16:
                    bound = ((j + 1) * U_BF16 + 1e-5) * smax
                    err = float(_colnorm(sn[r, t] - ref).max())
                    worst_ratio = max(worst_ratio, err / bound)
                    assert err <= bound, f'step {j} row {r} draft {t}: snapshot {err:.3e} > {bound:.3e}'
                else:
                    worst = max(worst, H.rel_err(sn[r, t], ref))
        before = S.clone()
        rs.snapshot_commit(d, S, snaps, slot_d, torch.from_numpy(acc.astype(np.int32)).cuda())
        ts.accept(slots, acc)
        forced.accept(slots, acc)
        for r in live:
            s = int(slots[r])
            if acc[r] > 0:
                assert torch.equal(S[s], snaps[r, acc[r] - 1]), 'commit is not the accepted snapshot'
            else:
                assert torch.equal(S[s], before[s]), 'a zero accept changed the state'
            got = S[s].float().cpu().numpy()
            if bf16:
                bound = ((j + 1) * U_BF16 + 1e-5) * smax
                err = float(_colnorm(got - ts.H[s]).max())
                worst_ratio = max(worst_ratio, err / bound)
                assert err <= bound, f'step {j} slot {s}: state {err:.3e} > {bound:.3e}'
                forced.H[s] = got.astype(np.float64)
            else:
                worst = max(worst, H.rel_err(got, ts.H[s]))
        assert worst <= tol, f'snapshot baseline error {worst:.3e} > {tol}'
    un = H.unused_slots(cfg, init)
    assert torch.equal(S[un], S_init[un]), 'unused slot state modified'
    if bf16:
        print(f'[{cfg.name} snapshot] chained: worst error / derived bound {worst_ratio:.3f}; '
              f'teacher-forced one-step output error {forced_err:.2e}', flush=True)
    else:
        print(f'[{cfg.name} snapshot] worst {worst:.2e}', flush=True)
    return worst


@pytest.mark.parametrize('name,cfg', [
    ('decode_T3', W.CONFIGS['c1'].with_(B=9, null_rows=2, hk=2, hv=4, T=3, accept=('uniform', 0, 3),
                                        cursor_init='zero')),
    ('spec_bf16_nan', W.CONFIGS['c2'].with_(B=7, hk=2, hv=4)),
    ('kda', W.CONFIGS['c3'].with_(B=5, hk=3, hv=3)),
    ('odd_shapes', W.CONFIGS['c0'].with_(B=3, hk=1, hv=2, dk=48, dv=32, T=2, L=2,
                                         accept=('uniform', 0, 2))),
])
def test_snapshot_baseline(name, cfg):
    _run_snapshot(cfg, steps=5)


def test_snapshot_baseline_bf16_chain():
    """The spec-verify shapes with a bf16 state, NaN/Inf drafts, 12 chained steps (the
    sglang PR's chain length), against the derived rounding bound."""
    _run_snapshot(W.CONFIGS['c2'].with_(B=9, hk=2, hv=4, steps=12), steps=12)


def test_snapshot_query_scale():
    _run_snapshot(W.CONFIGS['c1'].with_(B=5, null_rows=1, hk=2, hv=4, T=3,
                                        accept=('uniform', 0, 3), cursor_init='zero',
                                        scale=128 ** -0.5), steps=3)


def test_snapshot_matches_ring_verify():
    """The baseline and the ReplaySSM verify of the same workload (full decode shapes at
    T = 3, one step from cursor 0) give the same outputs within tolerance."""
    import linear_attention_recurrent_rs_amd as rs
    cfg = W.CONFIGS['c1'].with_(T=3, accept=('uniform', 1, 3), cursor_init='zero', steps=1)
    init = H.initial(cfg)
    g = H.DeviceRun(cfg, init)
    acc, ins, pol, next_T = H.step_data(cfg, 0)
    ring_out, _ = g.verify(0, g.inputs_dev(ins[0]))
    snaps = torch.empty((cfg.B, cfg.T, cfg.hv, cfg.dk, cfg.dv), device='cuda')
    out = torch.full((cfg.B * cfg.T, cfg.hv, cfg.dv), H.SENTINEL_OUT, device='cuda')
    S = H.to_dev(init.S[0], cfg.state_dtype, 'cuda')
    slot_d = torch.from_numpy(init.slots.astype(np.int32)).cuda()
    rs.snapshot_verify(g.d, False, *_dev_inputs(cfg, ins[0]), S, snaps, slot_d, out)
    live = torch.from_numpy(np.repeat(init.slots >= 0, cfg.T))
    a, b = out[live.cuda()].cpu().numpy(), ring_out[live.cuda()].cpu().numpy()
    assert H.rel_err(a, b) <= 1e-4
