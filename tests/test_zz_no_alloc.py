"""GPU test of the allocation-free verify entry point (rs_gdn_verify_noalloc), through the
C ABI: two calls in a row, the second with a smaller batch, each against rs_gdn_verify
(same kernels, a caller workspace for the fold counters) on copies of the same state,
ring and cursors.  Rows fold in-verify in both calls, so the static counters are used,
and both calls must leave outputs, write_pos, states and rings bit for bit equal to the
workspace call's (cursors are read only)."""
import ctypes

import numpy as np
import pytest
import torch

import workloads as W
from tests import harness as H

pytestmark = pytest.mark.gpu


def _pair(cfg, step):
    import linear_attention_recurrent_rs_amd as rs
    init = H.initial(cfg)
    a, b = H.DeviceRun(cfg, init), H.DeviceRun(cfg, init)
    acc, ins, pol, next_T = H.step_data(cfg, step)
    live = init.slots >= 0
    folding = int(np.sum(init.cursor[init.slots[live]] + cfg.T > cfg.L))
    print(f'[no-alloc] B={cfg.B} hk={cfg.hk} T={cfg.T} folding rows {folding}', flush=True)
    assert folding > 0
    dev_in = a.inputs_dev(ins[0])
    out_a, wp_a = a.verify(0, dev_in)                # rs_gdn_verify, caller workspace
    assert int(a.counter.abs().sum()) == 0           # the workspace call leaves it zeroed
    b.out.fill_(H.SENTINEL_OUT)
    b.wp.fill_(H.SENTINEL_WP)
    rs.gdn_verify_noalloc(b.d, *dev_in, b.S[0], b.rk[0], b.rd[0], b.rg[0], b.cursor, b.slots,
                          b.out, b.wp)
    torch.cuda.synchronize()

    def bits(t):                                     # NaN-filled ring rows compare by bits
        t = t.contiguous()
        return t.view(torch.int16) if t.element_size() == 2 else t.view(torch.int32)
    assert torch.equal(bits(out_a), bits(b.out)), 'outputs differ'
    assert torch.equal(wp_a, b.wp), 'write_pos differs'
    assert torch.equal(bits(a.S[0]), bits(b.S[0])), 'state differs'
    assert torch.equal(bits(a.rd[0]), bits(b.rd[0])) and torch.equal(bits(a.rk[0]), bits(b.rk[0]))
    assert torch.equal(bits(a.rg[0]), bits(b.rg[0])) and torch.equal(a.cursor, b.cursor)


def test_noalloc_matches_workspace_verify():
    big = W.CONFIGS['c1'].with_(B=32, null_rows=3, T=2, accept=('uniform', 1, 2), steps=1)
    small = W.CONFIGS['c1'].with_(B=7, null_rows=1, hk=2, hv=4, T=3, L=4, accept=('uniform', 1, 3),
                                  steps=1, seed=11)
    _pair(big, 0)
    _pair(small, 0)


def test_noalloc_rejects_oversized_batch():
    import linear_attention_recurrent_rs_amd as rs
    d = rs.Dims(4097, 1, 16, 32, 128, 128, 16, 4097, rs.BF16, rs.F32, 0)   # 65552 counters
    fake = ctypes.c_void_p(256)                      # never dereferenced: refused first
    assert rs._lib().rs_gdn_verify_noalloc(ctypes.byref(d), *([fake] * 13), None) == 7
