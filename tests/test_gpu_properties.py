"""GPU properties beyond element-wise parity, all through the C ABI:

* determinism: two runs of the same workload are bitwise identical;
* NaN isolation, bitwise: a run whose rejected drafts hold NaN/Inf in v equals, bit for
  bit, a run with finite values there, at every accepted output, committed ring record,
  state and cursor (causal terms are selected, never multiplied by zero);
* fold invariance on the GPU: committing (folding) after every step and never folding
  give the same accepted outputs and the same materialized state, within tolerance;
* HIP graph replay: a captured decode step, replayed with fresh inputs copied in between,
  matches the eager launches bit for bit, replay after replay (uniform and ragged windows);
* full-size workloads: every row and head on the GPU, sampled rows checked against the
  oracle, at the sizes and in the launch configuration the benchmark uses.
"""
import numpy as np
import pytest
import torch

import workloads as W
from tests import harness as H

pytestmark = pytest.mark.gpu


def _bits(t: torch.Tensor) -> torch.Tensor:
    t = t.contiguous()
    return t.view(torch.int16) if t.element_size() == 2 else t.view(torch.int32)


def _same(a: torch.Tensor, b: torch.Tensor) -> bool:
    return torch.equal(_bits(a), _bits(b))


SPEC = W.CONFIGS['c2'].with_(B=7, hk=2, hv=4, steps=12)          # bf16 state, NaN drafts
KDA = W.CONFIGS['c3'].with_(B=5, hk=3, hv=3, steps=12)
LARGE = W.CONFIGS['c4'].with_(B=5, hk=2, hv=4, steps=20)


@pytest.mark.parametrize('cfg', [SPEC, KDA, LARGE], ids=['spec_bf16', 'kda', 'large_ring'])
def test_deterministic(cfg):
    init = H.initial(cfg)
    a, b = H.DeviceRun(cfg, init), H.DeviceRun(cfg, init)
    for j in range(cfg.steps):
        acc, ins, pol, next_T = H.step_data(cfg, j)
        oa, wa = a.step(acc, ins, pol, next_T)
        ob, wb = b.step(acc, ins, pol, next_T)
        for l in range(cfg.layers):
            assert _same(oa[l], ob[l]) and torch.equal(wa[l], wb[l]), f'step {j} outputs differ'
            assert _same(a.S[l], b.S[l]), f'step {j} state differs'
            assert _same(a.rd[l], b.rd[l]) and _same(a.rk[l], b.rk[l]) and _same(a.rg[l], b.rg[l])
        assert torch.equal(a.cursor, b.cursor) and torch.equal(a.fold_len, b.fold_len)


def test_nan_isolation_bitwise():
    cfg = SPEC.with_(nan_frac=0.5)           # many poisoned rejected positions
    init = H.initial(cfg)
    poisoned, clean = H.DeviceRun(cfg, init), H.DeviceRun(cfg, init)
    n_injected = 0
    for j in range(cfg.steps):
        acc, ins, pol, next_T = H.step_data(cfg, j)
        n_injected += sum(len(x.injected) for x in ins)
        op, _ = poisoned.step(acc, ins, pol, next_T)
        oc, _ = clean.step(acc, ins, pol, next_T, clean=True)
        cur = poisoned.cursor.cpu().numpy()
        assert torch.equal(poisoned.cursor, clean.cursor)
        for l in range(cfg.layers):
            p = op[l].view(cfg.B, cfg.T, cfg.hv, cfg.dv)
            c = oc[l].view(cfg.B, cfg.T, cfg.hv, cfg.dv)
            for r in range(cfg.B):
                if init.slots[r] < 0:
                    continue
                a = int(acc[r])
                assert _same(p[r, :a], c[r, :a]), f'step {j} row {r}: accepted outputs differ'
                assert torch.isfinite(p[r, :a]).all()
                s = int(init.slots[r])
                n = int(cur[s])
                assert _same(poisoned.rd[l][s, :n], clean.rd[l][s, :n]), f'step {j} slot {s} ring'
            assert _same(poisoned.S[l], clean.S[l]), f'step {j}: state differs'
            assert torch.isfinite(poisoned.S[l].float()).all()
    assert n_injected > 20


def test_commit_fold_equals_history_replay():
    """Verify with history replay (no commit fold) vs fold at every commit: the same
    accepted outputs within the fp32 tolerance, the same materialized state."""
    base = W.CONFIGS['c1'].with_(B=9, null_rows=1, hk=2, hv=4, T=3, accept=('uniform', 0, 3),
                                 steps=14, cursor_init='zero')
    init = H.initial(base)
    keep = H.DeviceRun(base, init)
    fold = H.DeviceRun(base.with_(policy='every_commit'), init)
    worst = 0.0
    for j in range(base.steps):
        acc, ins, _, _ = H.step_data(base, j)
        ok, _ = keep.step(acc, ins, W.FOLD_NONE, base.T)
        of, _ = fold.step(acc, ins, W.FOLD_EVERY_COMMIT, base.T)
        a_ = ok[0].view(base.B, base.T, base.hv, base.dv).cpu().numpy()
        b_ = of[0].view(base.B, base.T, base.hv, base.dv).cpu().numpy()
        for r in range(base.B):
            if init.slots[r] >= 0 and acc[r] > 0:
                worst = max(worst, H.rel_err(a_[r, :acc[r]], b_[r, :acc[r]]))
    assert worst <= 1e-4, worst
    assert int(fold.cursor.max()) == 0                 # every commit folded
    mk = keep.materialize(0).cpu().numpy()
    mf = fold.materialize(0).cpu().numpy()
    live = [r for r in range(base.B) if init.slots[r] >= 0]
    assert H.rel_err(mk[live], mf[live]) <= 1e-4


def test_graph_replay_matches_eager():
    """One decode step (a verify per layer, then the cursor advance) captured in a HIP
    graph through the C ABI; inputs are copied into the captured buffers between replays
    (outside the graph), and every replay matches eager launches bit for bit."""
    import linear_attention_recurrent_rs_amd as rs
    cfg = W.CONFIGS['c1'].with_(B=12, null_rows=2, hk=2, hv=4, T=3, accept=('uniform', 1, 3),
                                layers=2, steps=6)
    init = H.initial(cfg)
    eager, graphed = H.DeviceRun(cfg, init), H.DeviceRun(cfg, init)
    BT = cfg.B * cfg.T
    dev = 'cuda'
    static = [tuple(torch.zeros_like(x) for x in graphed.inputs_dev(H.step_data(cfg, 0)[1][l]))
              for l in range(cfg.layers)]
    acc_buf = torch.zeros(cfg.B, dtype=torch.int32, device=dev)
    calls = [rs.prepare_verify(False, graphed.d, *static[l], graphed.S[l], graphed.rk[l],
                               graphed.rd[l], graphed.rg[l], graphed.cursor, graphed.slots,
                               graphed.out if l == 0 else torch.full_like(graphed.out, H.SENTINEL_OUT),
                               graphed.wp, graphed.counter) for l in range(cfg.layers)]
    outs = [calls[l].tensors[11] for l in range(cfg.layers)]
    adv = rs.prepare_cursor_advance(graphed.d, graphed.cursor, graphed.fold_len, graphed.slots,
                                    acc_buf, rs.FOLD_NONE, cfg.T)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    stream = torch.cuda.Stream()
    # capture on a side stream; capture enqueues nothing, so the buffers stay untouched
    with torch.cuda.stream(stream):
        with torch.cuda.graph(g, stream=stream):
            s = torch.cuda.current_stream()
            for l in range(cfg.layers):
                calls[l](s)
            adv(s)
    torch.cuda.synchronize()
    for j in range(cfg.steps):
        acc, ins, pol, next_T = H.step_data(cfg, j)
        for l in range(cfg.layers):
            for dst, src in zip(static[l], graphed.inputs_dev(ins[l])):
                dst.copy_(src)
        acc_buf.copy_(torch.from_numpy(acc.astype(np.int32)))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        eo, _ = eager.step(acc, ins, pol, next_T)
        torch.cuda.synchronize()
        for l in range(cfg.layers):
            assert _same(outs[l], eo[l]), f'replay {j} layer {l}: outputs differ'
            assert _same(graphed.S[l], eager.S[l]) and _same(graphed.rd[l], eager.rd[l])
            assert _same(graphed.rk[l], eager.rk[l]) and _same(graphed.rg[l], eager.rg[l])
        assert torch.equal(graphed.cursor, eager.cursor), f'replay {j}: cursors differ'


# ----------------------------------------------------------------------------- full size

def _sampled(cfg, rows, steps):
    init = H.initial(cfg)
    g = H.DeviceRun(cfg, init)
    o = H.OracleRun(cfg, init, rows=rows)
    worst = H.StepReport()
    for j in range(steps):
        acc, ins, pol, next_T = H.step_data(cfg, j)
        lens = H.step_windows(cfg, j)
        fm = H.step_force_mask(cfg, j)
        print(f'[{cfg.name} full] step {j} policy {pol}', flush=True)
        g_outs, g_wps = g.step(acc, ins, pol, next_T, lens=lens, force_mask=fm)
        o_outs, o_wps = o.step(acc, ins, pol, next_T, with_stream=False, lens=lens,
                               force_mask=fm)
        rep = H.compare_step(cfg, g, o, g_outs, g_wps, o_outs, o_wps, acc, rows, init)
        worst.out_err = max(worst.out_err, rep.out_err)
        worst.state_err = max(worst.state_err, rep.state_err)
    print(f'[{cfg.name} full] worst out {worst.out_err:.2e} state {worst.state_err:.2e}', flush=True)
    return g, init


def _rows(cfg, k):
    """k sampled rows: the first null row (if any), rows with the smallest and largest
    starting cursors, and a spread of others."""
    slots = W.slot_map(cfg)
    null = [r for r in range(cfg.B) if slots[r] < 0][:1]
    live = [r for r in range(cfg.B) if slots[r] >= 0]
    pick = sorted(set([live[0], live[-1]] + live[::max(1, len(live) // (k - 1))][:k - 1]))
    return null + pick[:k]


def test_full_size_decode_sampled():
    """The benchmark's workload, full size (64 rows, 16/32 heads, dk = dv = 128, ring 16,
    staggered cursors): 18 steps so that every row folds in-verify at least once."""
    cfg = W.CONFIGS['c1'].with_(steps=18)
    _sampled(cfg, _rows(cfg, 5), cfg.steps)


def test_full_size_decode_T3_sampled():
    """The benchmark's T = 3 workload at full size (64 rows, fp32 state, ring 16, accept
    U{1..3}, staggered cursors): 32 steps, so rows replay 0..13 history records and fold
    in-verify repeatedly, in the launch configuration the benchmark times (the key-group
    XCD order, six workgroups per CU)."""
    cfg = W.CONFIGS['c1'].with_(T=3, accept=('uniform', 1, 3), steps=32)
    _sampled(cfg, _rows(cfg, 5), cfg.steps)


@pytest.mark.timeout(900)
def test_full_size_large_ring_sampled():
    """The large-ring workload at full size: 256 rows, 16/32 heads, ring 64, window 8,
    4 layers sharing one cursor array, Binomial(8, 0.7) accepts; fused folds only for 16
    steps, then a forced commit fold of every row every third step (steps 16 and 19 here;
    batch x key heads a multiple of 8, so the verify takes the key-group XCD order).  The
    fp64 oracle replays up to 64 history records per sampled row, layer and step, so the
    sample is three rows over 20 steps."""
    cfg = W.CONFIGS['c4'].with_(steps=20)
    assert (cfg.B * cfg.hk) % 8 == 0
    _sampled(cfg, _rows(cfg, 3), cfg.steps)


def test_full_size_spec_verify_sampled():
    cfg = W.CONFIGS['c2'].with_(steps=6)
    _sampled(cfg, _rows(cfg, 3), cfg.steps)


def test_full_size_kda_sampled():
    cfg = W.CONFIGS['c3'].with_(steps=8)
    _sampled(cfg, _rows(cfg, 3), cfg.steps)


def test_full_size_ragged_sampled():
    """Ragged windows at full size (64 rows, 16/32 heads, dk = dv = 128, ring 16, widths
    U{0..4}, staggered cursors)."""
    cfg = W.CONFIGS['ragged_gdn'].with_(steps=8)
    _sampled(cfg, _rows(cfg, 4), cfg.steps)


def test_graph_replay_ragged_matches_eager():
    """Ragged windows under graph capture: the cumulative lengths and the packed tokens sit
    in fixed-capacity device buffers captured once (capacity B * T tokens); between
    replays only their contents change, so each step may pack a different set of widths.
    Every replay matches eager ragged launches bit for bit."""
    import linear_attention_recurrent_rs_amd as rs
    cfg = W.CONFIGS['ragged_gdn'].with_(B=10, null_rows=2, hk=2, hv=4, layers=2, steps=6)
    init = H.initial(cfg)
    eager, graphed = H.DeviceRun(cfg, init), H.DeviceRun(cfg, init)
    cap = cfg.B * cfg.T
    dev = 'cuda'
    gsh = (cfg.hv, cfg.dk) if cfg.kda else (cfg.hv,)
    at = H.torch_dtype(cfg.act_dtype)
    static = [(torch.zeros(cap, cfg.hk, cfg.dk, dtype=at, device=dev),
               torch.zeros(cap, cfg.hk, cfg.dk, dtype=at, device=dev),
               torch.zeros(cap, cfg.hv, cfg.dv, dtype=at, device=dev),
               torch.zeros(cap, cfg.hv, dtype=at, device=dev),
               torch.zeros((cap,) + gsh, dtype=at, device=dev)) for _ in range(cfg.layers)]
    cu_buf = torch.zeros(cfg.B + 1, dtype=torch.int32, device=dev)
    acc_buf = torch.zeros(cfg.B, dtype=torch.int32, device=dev)
    outs = [torch.full((cap, cfg.hv, cfg.dv), H.SENTINEL_OUT, device=dev) for _ in range(cfg.layers)]
    calls = [rs.prepare_verify_varlen(False, graphed.d, cu_buf, *static[l], graphed.S[l],
                                      graphed.rk[l], graphed.rd[l], graphed.rg[l],
                                      graphed.cursor, graphed.slots, outs[l], graphed.wp,
                                      graphed.counter) for l in range(cfg.layers)]
    adv = rs.prepare_cursor_advance_varlen(graphed.d, cu_buf, cap, graphed.cursor,
                                           graphed.fold_len, graphed.slots, acc_buf,
                                           rs.FOLD_NONE, cfg.T)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(g, stream=stream):
            s = torch.cuda.current_stream()
            for l in range(cfg.layers):
                calls[l](s)
            adv(s)
    torch.cuda.synchronize()
    for j in range(cfg.steps):
        acc, ins, pol, next_T = H.step_data(cfg, j)
        lens = H.step_windows(cfg, j)
        cu, idx, _ = H.pack_windows(lens, cfg.T)
        graphed.set_windows(lens)
        for l in range(cfg.layers):
            for dst, src in zip(static[l], graphed.inputs_dev(ins[l])):
                dst.zero_()
                dst[:src.shape[0]].copy_(src)
            outs[l].fill_(H.SENTINEL_OUT)
        cu_buf.copy_(torch.from_numpy(cu))
        acc_buf.copy_(torch.from_numpy(acc.astype(np.int32)))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        eo, _ = eager.step(acc, ins, pol, next_T, lens=lens)
        torch.cuda.synchronize()
        sel = torch.from_numpy(idx).to(dev)
        for l in range(cfg.layers):
            assert _same(outs[l][:len(idx)], eo[l][sel]), f'replay {j} layer {l}: outputs differ'
            assert _same(graphed.S[l], eager.S[l]) and _same(graphed.rd[l], eager.rd[l])
        assert torch.equal(graphed.cursor, eager.cursor), f'replay {j}: cursors differ'
