"""GPU parity of the chunked prefill (rs_gdn_prefill) against the fp64 oracle, through the
C ABI: ragged prompts (up to 512 tokens, a length that is not a multiple of the chunk,
an empty prompt, a null row) from a nonzero canonical state; every prompt token's output
and the final state within the tolerance (1e-4 of the largest magnitude for fp32 states,
5e-3 for bf16), live cursors 0, null rows and unused slots untouched.  Then the replay
verify continues from the prefilled state, against the oracle continuing likewise."""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import replay as rp
from tests import harness as H

pytestmark = pytest.mark.gpu

SENT = 2048.0


def _prefill(cfg, lens, rows=None, verify_steps=0):
    import linear_attention_recurrent_rs_amd as rs
    P = int(max(lens))
    init = H.initial(cfg)
    slots = init.slots
    stale = np.where(init.cursor >= 0, 5, 0).astype(np.int32)      # cleared by prefill
    g = H.DeviceRun(cfg, init)
    g.cursor.copy_(torch.from_numpy(stale))
    o = H.OracleRun(cfg, init, rows=rows)
    o.cursor[:] = stale
    inp = W.step_inputs(cfg.with_(T=P, nan_frac=0.0), 10 ** 6, 0)
    cu, idx, ntok = H.pack_windows(lens, P)
    BT = cfg.B * P

    def pack(x, shape):
        p = np.zeros((ntok,) + shape)
        p[:len(idx)] = x.reshape((BT,) + shape)[idx]
        return H.to_dev(p, cfg.act_dtype, 'cuda')
    q = pack(inp.q, (cfg.hk, cfg.dk))
    k = pack(inp.k, (cfg.hk, cfg.dk))
    v = pack(inp.v, (cfg.hv, cfg.dv))
    beta = pack(inp.beta, (cfg.hv,))
    gate = pack(inp.gate, (cfg.hv,))
    out = torch.full((ntok, cfg.hv, cfg.dv), SENT, device='cuda')
    S_before = g.S[0].clone()
    print(f'[prefill {cfg.name}] lens {lens.tolist()} tokens {ntok}', flush=True)
    rs.gdn_prefill(g.d, torch.from_numpy(cu).cuda(), q, k, v, beta, gate, g.S[0], g.cursor,
                   g.slots, out)
    ref = rp.prefill(o.layers[0], o.cursor, slots, inp, lens, rows=rows)
    o.streams = [rp.TokenStream.from_replay(o.layers[0], o.cursor)]
    got = np.full((BT, cfg.hv, cfg.dv), np.nan)
    got[idx] = out.cpu().numpy()[:len(idx)]
    got = got.reshape(cfg.B, P, cfg.hv, cfg.dv)
    tol = H.tol_for(cfg)
    rows_ = [r for r in (range(cfg.B) if rows is None else rows)]
    worst_o = worst_s = 0.0
    cur = g.cursor.cpu().numpy()
    for r in rows_:
        s = int(slots[r])
        L_r = int(lens[r])
        if s < 0:
            assert np.all(got[r, :L_r] == SENT), f'null row {r} written'
            continue
        assert cur[s] == 0, f'row {r}: cursor {cur[s]} after prefill'
        if L_r:
            worst_o = max(worst_o, H.rel_err(got[r, :L_r], ref[r, :L_r]))
        worst_s = max(worst_s, H.rel_err(g.S[0][s].float().cpu().numpy(), o.layers[0].S[s]))
    un = H.unused_slots(cfg, init)
    assert torch.equal(g.S[0][un], S_before[un]), 'unused slot state changed'
    nulls = [int(x) for x in slots if x < 0]
    assert np.array_equal(cur[[s for s in range(cfg.num_slots) if s in un]], stale[un])
    print(f'[prefill {cfg.name}] worst out {worst_o:.2e} state {worst_s:.2e}', flush=True)
    assert worst_o <= tol and worst_s <= tol, (worst_o, worst_s)
    # the replay verify continues from the prefilled state
    for j in range(verify_steps):
        acc, ins, pol, next_T = H.step_data(cfg, j)
        g_outs, g_wps = g.step(acc, ins, pol, next_T)
        o_outs, o_wps = o.step(acc, ins, pol, next_T, with_stream=False)
        H.compare_step(cfg, g, o, g_outs, g_wps, o_outs, o_wps, acc, rows_, init)
    return worst_o, worst_s


BASE = W.CONFIGS['c1'].with_(B=6, null_rows=1, hk=2, hv=4, T=3, accept=('uniform', 1, 3),
                             cursor_init='zero', steps=6, seed=21)


@pytest.mark.parametrize('name', ['fp32', 'bf16_state', 'scaled', 'grouped_heads'])
def test_prefill_ragged_prompts(name):
    cfg = {'fp32': BASE, 'bf16_state': BASE.with_(state_dtype='bf16'),
           'scaled': BASE.with_(scale=128 ** -0.5, seed=22),
           'grouped_heads': BASE.with_(hk=1, hv=4, seed=23)}[name]
    slots = W.slot_map(cfg)
    lens = np.array([512, 37, 0, 200, 16, 1][:cfg.B], np.int32)
    _prefill(cfg, lens, verify_steps=4)


def test_prefill_full_size_sampled():
    """Qwen3.5-shaped layer (16 key / 32 value heads, dk = dv = 128, fp32 state), 8 rows
    with prompts up to 512 tokens, every row and head on the GPU; two rows against the
    oracle, then three replay verify steps on them."""
    cfg = W.CONFIGS['c1'].with_(B=8, null_rows=1, T=1, cursor_init='zero', steps=3, seed=24)
    lens = np.array([512, 300, 511, 64, 129, 7, 256, 480], np.int32)
    slots = W.slot_map(cfg)
    live = [r for r in range(cfg.B) if slots[r] >= 0]
    _prefill(cfg, lens, rows=[live[0], live[-1]], verify_steps=3)
