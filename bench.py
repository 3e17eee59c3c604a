#!/usr/bin/env python3
"""Benchmark: ReplaySSM GDN decode verify on one MI355X.

Workload (GDN standard decode, Qwen3.5-shaped layers): batch 64 request rows of which 4
are null (state slot -1), 16 key heads shared by 32 value heads, dk = dv = 128, fp32
state, bf16 q/k/v/beta/gate, fp32 delta history, ring capacity 16, T = 1 (the metric's
T = 3 case is reported alongside).  Cursors start staggered (row r at r mod 16, ring
prefilled), so every launch mixes rows replaying 0..15 history records with rows that
overflow and fold in-kernel, as a steady decode does.

One step = one decode step of an 8-layer stack: a verify on each of 8 layer pools (each
pool has its own state, ring and inputs; together > 1 GiB, so the 256 MB Infinity Cache
cannot serve the state from one use to the next) and one advance of the shared cursor.
Inputs are synthetic (seeded, from ``workloads``) and resident in HBM before timing.

value = verified tokens per second per layer = live rows * T * layers / step time.
roofline: the verify kernel; achieved = algorithmic bytes per launch (from the integer
cursor model: state read, inputs, history records read, outputs and ring writes, the
state write of rows that fold) / mean launch time from HIP events on the launch stream
around each timed step's back-to-back verifies (divided by the layer count).
cpu_baseline: the fp64 oracle on a bounded sample of the same workload, one process per
host core (and a single-thread run beside it), with the CPU model.

extra: the T = 3 case; the T = 1 verify at three history states (none, steady, every row
folding); and full step loops (verify per layer, cursor advance, commit folds by policy)
of the spec-verify (batch 128, bf16 state, T = 4, fold every commit), KDA (batch 64, T = 3)
and large-ring (batch 256, ring 64, T = 8, 4 layers, forced commit folds) workloads and of
ragged GDN and KDA verifies (batch 64, widths U{0..4} per row from one packed token list),
each with verify and commit-fold kernel times and verified / committed tokens per second;
and the snapshot-verify baseline on the spec-verify shapes (time and per-layer memory).
"""
from __future__ import annotations

import argparse
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, vendor figure


def verify_bytes(cfg, n_list, fold_list):
    """Algorithmic bytes of one verify launch: per live row, the state tile read once,
    the window inputs, n history records, outputs and ring writes, and one state write
    when the row folds in-kernel; plus its slot index and cursor."""
    a = 2 if cfg.act_dtype == 'bf16' else 4
    s = 2 if cfg.state_dtype == 'bf16' else 4
    g_in = cfg.hv * cfg.dk * a if cfg.kda else cfg.hv * a
    g_ring = cfg.hv * cfg.dk * 4 if cfg.kda else cfg.hv * 4
    S_bytes = cfg.hv * cfg.dk * cfg.dv * s
    inputs = cfg.T * (2 * cfg.hk * cfg.dk * a + cfg.hv * cfg.dv * a + cfg.hv * a + g_in)
    record = cfg.hk * cfg.dk * a + cfg.hv * cfg.dv * 4 + g_ring
    writes = cfg.T * (cfg.hv * cfg.dv * 4 + cfg.hk * cfg.dk * a + cfg.hv * cfg.dv * 4 + g_ring)
    total = 0
    for n, f in zip(n_list, fold_list):
        total += S_bytes + inputs + n * record + writes + (S_bytes if f else 0) + 8
    return total


def advance_model(cursor, slots, acc, T, L):
    """The cursor advance of the fused-fold policy on the host, for byte accounting."""
    for r, s in enumerate(slots):
        if s < 0:
            continue
        n = int(cursor[s])
        base = 0 if n + T > L else n
        cursor[s] = base + int(acc[r])


def run_gpu(T: int, steps: int, warmup: int, layers: int, tile_v: int, n_inputs: int = 4):
    import torch
    import linear_attention_recurrent_rs_amd as rs
    import workloads as W

    cfg = W.CONFIGS['c1'].with_(T=T, layers=layers,
                                accept=('const', 1) if T == 1 else ('uniform', 1, T))
    dev = torch.device('cuda:0')
    slots_np = W.slot_map(cfg)
    cursor_np = W.initial_cursor(cfg, slots_np)

    def to_dev(x, dt):
        return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(dev).to(dt).contiguous()

    bf, f32 = torch.bfloat16, torch.float32
    S, RK, RD, RG = [], [], [], []
    for l in range(layers):
        S.append(to_dev(W.initial_state(cfg, l), f32))
        rk, rd, rg = W.initial_ring(cfg, cursor_np, l, fill=0.0)
        RK.append(to_dev(rk, bf)); RD.append(to_dev(rd, f32)); RG.append(to_dev(rg, f32))
    slots = torch.from_numpy(slots_np.astype(np.int32)).to(dev)
    cursor = torch.from_numpy(cursor_np.astype(np.int32)).to(dev)
    fold_len = torch.zeros(cfg.num_slots, dtype=torch.int32, device=dev)
    counter = torch.zeros(cfg.B * cfg.hk, dtype=torch.int32, device=dev)
    out = torch.empty(cfg.B * T, cfg.hv, cfg.dv, dtype=f32, device=dev)
    d = rs.Dims(cfg.B, T, cfg.hk, cfg.hv, cfg.dk, cfg.dv, cfg.L, cfg.num_slots, rs.BF16, rs.F32,
                tile_v)
    BT = cfg.B * T
    inputs, accepts, verify_calls, advance_calls = [], [], [], []
    for j in range(n_inputs):
        acc = W.accept_lengths(cfg, j)
        accepts.append(acc)
        acc_d = torch.from_numpy(acc.astype(np.int32)).to(dev)
        per_layer = []
        for l in range(layers):
            inp = W.step_inputs(cfg, j, l)
            t = (to_dev(inp.q.reshape(BT, cfg.hk, cfg.dk), bf), to_dev(inp.k.reshape(BT, cfg.hk, cfg.dk), bf),
                 to_dev(inp.v.reshape(BT, cfg.hv, cfg.dv), bf), to_dev(inp.beta.reshape(BT, cfg.hv), bf),
                 to_dev(inp.gate.reshape(BT, cfg.hv), bf))
            inputs.append(t)
            per_layer.append(rs.prepare_verify(False, d, *t, S[l], RK[l], RD[l], RG[l], cursor,
                                               slots, out, None, counter))
        verify_calls.append(per_layer)
        advance_calls.append(rs.prepare_cursor_advance(d, cursor, fold_len, slots, acc_d,
                                                       rs.FOLD_NONE, T))
    tile, workgroups, lds = rs.verify_launch_info(d)
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    host_cursor = cursor_np.copy()
    live = [r for r in range(cfg.B) if slots_np[r] >= 0]

    def step(s, events=None):
        # the layers' verifies run back to back between one pair of events: a pair around
        # every launch would add the events' own stream synchronisation to each launch
        j = s % n_inputs
        if events is not None:
            events[0].record(stream)
        for l in range(layers):
            verify_calls[j][l](stream)
        if events is not None:
            events[1].record(stream)
        advance_calls[j](stream)

    for s in range(warmup):
        step(s)
        advance_model(host_cursor, slots_np, accepts[s % n_inputs], T, cfg.L)
    torch.cuda.synchronize()

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    bytes_per_launch = []
    t0 = time.perf_counter()
    for s in range(steps):
        step(warmup + s, ev[s])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for s in range(steps):
        n = [int(host_cursor[slots_np[r]]) for r in live]
        folds = [x + T > cfg.L for x in n]
        bytes_per_launch.append(verify_bytes(cfg, n, folds))
        advance_model(host_cursor, slots_np, accepts[(warmup + s) % n_inputs], T, cfg.L)
    # the device cursors must follow the host model exactly
    assert np.array_equal(cursor.cpu().numpy(), host_cursor), 'cursor model diverged'
    durs = np.array([ev[s][0].elapsed_time(ev[s][1]) / layers for s in range(steps)])  # ms
    ms_step = (t1 - t0) * 1e3 / steps
    mean_launch_ms = float(durs.mean())
    mean_bytes = float(np.mean(bytes_per_launch))
    achieved = mean_bytes / (mean_launch_ms * 1e-3) / 1e9
    live_rows = len(live)
    return {
        'cfg': cfg, 'ms_per_step': ms_step,
        'value': live_rows * T * layers / (ms_step * 1e-3),
        'kernel_us': mean_launch_ms * 1e3, 'kernel_us_median': float(np.median(durs)) * 1e3,
        'bytes_per_launch': mean_bytes, 'achieved_gbs': achieved,
        'tokens_per_s_kernel': live_rows * T / (mean_launch_ms * 1e-3),
        'tile_v': tile, 'workgroups': workgroups, 'lds_bytes': lds, 'live_rows': live_rows,
    }


KERNEL_SOURCES = ('rs_verify_fast.hip', 'rs_device.h', 'rs_internal.h')


def kernel_source_hash():
    """sha256 over the sources of the fast verify kernel, so that counter readings taken
    on an older kernel are not reported against a changed one."""
    import hashlib
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, 'linear_attention_recurrent_rs_amd', 'csrc', name), 'rb') as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_from_profiles(T):
    """HBM bytes per verify launch from the committed counter summary, if one exists for
    this workload and was taken on the current kernel sources (FETCH_SIZE + WRITE_SIZE per
    dispatch, each calibrated on a plain copy); else None."""
    path = os.path.join(ROOT, 'profiles', 'gdn_verify_decode_b64_counters.md')
    if not os.path.exists(path):
        return None
    text = open(path).read()
    src = re.search(r'^kernel_source_sha256: ([0-9a-f]+)', text, re.M)
    if not src or src.group(1) != kernel_source_hash():
        return None
    m = re.search(rf'^traffic_bytes_per_launch T={T}: ([0-9.eE+]+)', text, re.M)
    return float(m.group(1)) if m else None


def copy_calibration(mib: int = 256, reps: int = 4):
    """Plain device-to-device copies of a known size (mib MiB read + mib MiB written per
    launch), run before the benchmark so that one hardware-counter pass sees both them and
    the verify launches: the ratio of a counter's reading on the copy to the copy's true
    bytes calibrates that counter."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device='cuda:0')
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(f'# copy calibration: {reps} copies of {mib} MiB', file=sys.stderr, flush=True)


def _oracle_decode(T: int, rows_pick, budget_s: float, start=None):
    """The fp64 oracle, as it stands, running consecutive decode steps of one layer of the
    decode workload for the given live-row indices until budget_s of timed work is spent
    (input generation is not timed).  BLAS limited to one thread.  Returns (verified
    tokens, seconds, steps)."""
    from threadpoolctl import threadpool_limits
    import workloads as W
    from oracle import replay as rp

    cfg = W.CONFIGS['c1'].with_(T=T, accept=('const', 1) if T == 1 else ('uniform', 1, T))
    slots = W.slot_map(cfg)
    cursor = W.initial_cursor(cfg, slots)
    live = [r for r in range(cfg.B) if slots[r] >= 0]
    rows = [live[i % len(live)] for i in rows_pick]
    rows = sorted(set(rows))
    rk, rd, rg = W.initial_ring(cfg, cursor, 0)
    layer = rp.ReplayLayer(W.initial_state(cfg, 0), rk, rd, rg, False, cfg.G, cfg.L,
                           slots=[slots[r] for r in rows])
    fl = np.zeros(cfg.num_slots, np.int32)
    sub = np.full(cfg.B, -1, np.int32)
    sub[rows] = slots[rows]
    steps, tokens, elapsed = 0, 0, 0.0
    if start is not None:
        start.wait()                                   # every worker starts its clock together
    with threadpool_limits(limits=1):
        while elapsed < budget_s:
            inp = W.step_inputs(cfg, steps, 0)
            acc = W.accept_lengths(cfg, steps)
            ts = time.perf_counter()
            rp.verify(layer, cursor, slots, inp, rows=rows)
            rp.cursor_advance(cursor, fl, sub, acc, T, cfg.L, rp.FOLD_NONE)
            elapsed += time.perf_counter() - ts
            tokens += len(rows) * T
            steps += 1
    return tokens, elapsed, steps


def _cpu_model():
    try:
        for line in open('/proc/cpuinfo'):
            if line.startswith('model name'):
                return line.split(':', 1)[1].strip()
    except OSError:
        pass
    return 'unknown'


def cpu_baseline(T: int, budget_s: float = 10.0):
    """The fp64 oracle on a bounded sample of the decode workload, on the host's cores:
    one process per core of this process's CPU affinity (at most 16, the host share of one
    GPU), each running the oracle single-threaded on 4 live rows of its own (all 32 value
    heads, dk = dv = 128, one layer) for budget_s of timed work, started together; the rate
    is the sum of the processes' rates.  A single-thread run on 8 live rows is reported
    beside it.  Runs before anything initialises the GPU (the workers are forked)."""
    import multiprocessing as mp
    n = max(1, min(len(os.sched_getaffinity(0)), 16))
    single = _oracle_decode(T, range(8), budget_s)
    ctx = mp.get_context('fork')
    start = ctx.Barrier(n)
    q = ctx.Queue()

    def work(i):
        q.put(_oracle_decode(T, range(4 * i, 4 * i + 4), budget_s, start))

    procs = [ctx.Process(target=work, args=(i,)) for i in range(n)]
    for p in procs:
        p.start()
    res = [q.get() for _ in procs]
    for p in procs:
        p.join()
    rate = sum(t / e for t, e, _ in res)
    return {'value': rate, 'unit': 'verified tokens/s per layer', 'cores': n, 'kind': 'oracle',
            'cpu_model': _cpu_model(), 'host_cpus': os.cpu_count(),
            'sample': f'{n} processes x 4 live rows x 32 value heads (dk=dv=128, ring 16, '
                      f'T={T}), {sum(x[2] for x in res)} decode steps of one layer in all, '
                      f'{budget_s:.0f} s each, fp64 numpy, one thread per process',
            'single_thread': {'value': round(single[0] / single[1], 2), 'cores': 1,
                              'sample': f'8 live rows x 32 value heads, {single[2]} decode '
                                        f'steps of one layer, {single[1]:.1f} s'}}


# ----------------------------------------------------------------------------- more workloads
# Timing only: the other workloads and the history states run on random device-side data of
# the same shapes and distributions (unit q/k rows, v ~ N(0,1), beta ~ U(0,1), gates
# exp(-softplus(N(0,1)))), so that the benchmark does not spend minutes building fp64 data.

def _rand_setup(cfg, layers, seed=1234, tile_v=0):
    import torch
    import linear_attention_recurrent_rs_amd as rs
    import workloads as W
    dev = torch.device('cuda:0')
    g = torch.Generator(device=dev).manual_seed(seed)
    bf, f32 = torch.bfloat16, torch.float32
    sd = bf if cfg.state_dtype == 'bf16' else f32
    ns, L = cfg.num_slots, cfg.L

    def unit(*shape):
        x = torch.randn(*shape, generator=g, device=dev)
        return x / x.norm(dim=-1, keepdim=True)

    def gates(*shape):
        return torch.exp(-torch.nn.functional.softplus(torch.randn(*shape, generator=g, device=dev)))

    gsh = (cfg.hv, cfg.dk) if cfg.kda else (cfg.hv,)
    st = dict(
        S=[(torch.randn(ns, cfg.hv, cfg.dk, cfg.dv, generator=g, device=dev) * 0.05).to(sd)
           for _ in range(layers)],
        rk=[unit(ns, L, cfg.hk, cfg.dk).to(bf) for _ in range(layers)],
        rd=[torch.randn(ns, L, cfg.hv, cfg.dv, generator=g, device=dev) * 0.5 for _ in range(layers)],
        rg=[gates(ns, L, *gsh) for _ in range(layers)])
    BT = cfg.B * cfg.T

    def inputs():
        return (unit(BT, cfg.hk, cfg.dk).to(bf), unit(BT, cfg.hk, cfg.dk).to(bf),
                torch.randn(BT, cfg.hv, cfg.dv, generator=g, device=dev).to(bf),
                torch.rand(BT, cfg.hv, generator=g, device=dev).to(bf),
                gates(BT, *gsh).to(bf))
    slots_np = W.slot_map(cfg)
    d = rs.Dims(cfg.B, cfg.T, cfg.hk, cfg.hv, cfg.dk, cfg.dv, L, ns, rs.BF16,
                rs.BF16 if cfg.state_dtype == 'bf16' else rs.F32, tile_v)
    st.update(slots_np=slots_np, slots=torch.from_numpy(slots_np.astype(np.int32)).to(dev),
              inputs=inputs, d=d, dev=dev)
    return st


def history_states(T=1, iters=60, layers=8):
    """The decode verify at three history states, cursors held fixed: no history (every
    write_pos 0), steady (cursors staggered over [0, L - T]: row mod (L - T + 1)), and
    every row folding in the verify (cursor = L).  Kernel time from HIP events on the
    stream."""
    import torch
    import linear_attention_recurrent_rs_amd as rs
    import workloads as W
    cfg = W.CONFIGS['c1'].with_(T=T)
    st = _rand_setup(cfg, layers)
    dev, slots_np = st['dev'], st['slots_np']
    live = [r for r in range(cfg.B) if slots_np[r] >= 0]
    out = torch.empty(cfg.B * T, cfg.hv, cfg.dv, device=dev)
    counter = torch.zeros(cfg.B * cfg.hk, dtype=torch.int32, device=dev)
    ins = st['inputs']()
    res = {}
    for name in ('no_history', 'steady', 'all_fold'):
        cur = np.zeros(cfg.num_slots, np.int32)
        for r in live:
            cur[slots_np[r]] = (0 if name == 'no_history' else
                                r % (cfg.L - T + 1) if name == 'steady' else cfg.L)
        cursor = torch.from_numpy(cur).to(dev)
        calls = [rs.prepare_verify(False, st['d'], *ins, st['S'][l], st['rk'][l], st['rd'][l],
                                   st['rg'][l], cursor, st['slots'], out, None, counter)
                 for l in range(layers)]
        stream = torch.cuda.current_stream()
        for i in range(16):
            calls[i % layers](stream)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(iters):
            calls[i % layers](stream)
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) / iters * 1e3
        n = [int(cur[slots_np[r]]) for r in live]
        byts = verify_bytes(cfg, n, [x + T > cfg.L for x in n])
        res[name] = {'kernel_us': round(us, 3), 'achieved_gbs': round(byts / us / 1e3, 1),
                     'frac': round(byts / us / 1e3 / HBM_PEAK_GBS, 4), 'bytes_per_launch': byts}
    return res


def stream_reference(nbytes, pools=8, iters=48):
    """Read rate of the library's plain streaming-read kernel (the verify's load
    instructions and workgroup size, nothing else) over buffers of the verify's size,
    rotating over `pools` buffers like the layer pools.  GB/s from HIP events."""
    import torch
    import linear_attention_recurrent_rs_amd as rs
    n = (int(nbytes) + 15) // 16 * 4                  # float32 elements, whole 16-byte words
    bufs = [torch.zeros(n, dtype=torch.float32, device='cuda:0') for _ in range(pools)]
    sink = torch.zeros(256, dtype=torch.float32, device='cuda:0')
    stream = torch.cuda.current_stream()
    for i in range(2 * pools):
        rs.stream_read(bufs[i % pools], sink, stream)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(iters):
        rs.stream_read(bufs[i % pools], sink, stream)
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / iters * 1e3
    del bufs
    return {'bytes': n * 4, 'us': round(us, 3), 'gbs': round(n * 4 / us / 1e3, 1)}


def _bytes_of(cfg):
    """Per-row byte terms of one layer: state, window inputs per token, history record,
    writes per token (outputs, ring keys, deltas, gates)."""
    a = 2 if cfg.act_dtype == 'bf16' else 4
    s = 2 if cfg.state_dtype == 'bf16' else 4
    g_in = cfg.hv * cfg.dk * a if cfg.kda else cfg.hv * a
    g_ring = cfg.hv * cfg.dk * 4 if cfg.kda else cfg.hv * 4
    return dict(S=cfg.hv * cfg.dk * cfg.dv * s,
                tok_in=2 * cfg.hk * cfg.dk * a + cfg.hv * cfg.dv * a + cfg.hv * a + g_in,
                record=cfg.hk * cfg.dk * a + cfg.hv * cfg.dv * 4 + g_ring,
                tok_out=cfg.hv * cfg.dv * 4 + cfg.hk * cfg.dk * a + cfg.hv * cfg.dv * 4 + g_ring)


class CursorModel:
    """The cursor advance on the host (every policy, uniform or ragged windows), for the
    algorithmic bytes of each verify and commit-fold launch; the device cursors must end
    equal to it."""

    def __init__(self, cfg, slots, cursor):
        self.cfg, self.slots, self.cursor = cfg, slots, cursor.copy()
        self.b = _bytes_of(cfg)

    def step(self, acc, policy, next_T, lens=None, force_mask=None):
        """Returns (verify bytes of one layer, commit-fold bytes of one layer) and advances."""
        c, b = self.cfg, self.b
        vb = cb = 0
        for r, s in enumerate(self.slots):
            if s < 0:
                continue
            T = c.T if lens is None else int(lens[r])
            n = int(self.cursor[s])
            if T == 0:                      # an empty ragged window reads only its indices
                vb += 8
                continue
            fold = n + T > c.L
            base = 0 if fold else n
            vb += b['S'] + T * b['tok_in'] + n * b['record'] + T * b['tok_out'] + \
                (b['S'] if fold else 0) + 8
            m = base + min(int(acc[r]), T)
            if policy == 1:
                fl = m
            elif policy == 2:
                fl = m if m + next_T > c.L else 0
            elif policy == 3:
                fl = m if (force_mask is None or force_mask[r]) else 0
            else:
                fl = 0
            if fl:
                cb += 2 * b['S'] + fl * b['record'] + 8
            self.cursor[s] = 0 if fl else m
        return vb, cb


def _frac(byts, us):
    return round(byts / us / 1e3 / HBM_PEAK_GBS, 4) if us > 0 else None


def run_workload(name, steps=30, warmup=10, tile_v=0, min_pool_bytes=1 << 30):
    """A full step loop of another workload: a verify per layer, the cursor advance, and the
    commit folds its policy asks for.  Layer pools rotate so that their state and rings
    together exceed the 256 MB Infinity Cache (at least 8 pools and 1 GiB, or the config's
    own layers when those are already larger).  Kernel times from one pair of HIP events
    around each step's verifies and one around its commit folds, divided by the layers;
    algorithmic bytes per launch from the host cursor model; verified tokens/s per layer =
    verified tokens * layers / step time; committed tokens/s per layer = accepted tokens *
    layers / step time (as the headline: the rate of a one-layer stack)."""
    import torch
    import linear_attention_recurrent_rs_amd as rs
    import workloads as W
    cfg = W.CONFIGS[name]
    b = _bytes_of(cfg)
    ring_bytes = cfg.num_slots * cfg.L * (b['record'])
    pool = cfg.num_slots * b['S'] + ring_bytes
    layers = cfg.layers if cfg.layers * pool >= min_pool_bytes else \
        max(cfg.layers, 8, -(-min_pool_bytes // pool))
    st = _rand_setup(cfg, layers, tile_v=tile_v)
    dev, slots_np, d = st['dev'], st['slots_np'], st['d']
    cursor = torch.zeros(cfg.num_slots, dtype=torch.int32, device=dev)
    fold_len = torch.zeros_like(cursor)
    counter = torch.zeros(cfg.B * cfg.hk, dtype=torch.int32, device=dev)
    out = torch.empty(cfg.B * cfg.T, cfg.hv, cfg.dv, device=dev)
    n_sets = 4
    sets = [st['inputs']() for _ in range(n_sets)]
    total = warmup + steps
    live = [r for r in range(cfg.B) if slots_np[r] >= 0]
    accs = [W.accept_lengths(cfg, j) for j in range(total)]
    acc_d = [torch.from_numpy(a.astype(np.int32)).to(dev) for a in accs]
    pols = [W.step_policy(cfg, j) for j in range(total)]
    lens = [W.window_lengths(cfg, j) for j in range(total)]
    if cfg.ragged:
        # ragged windows: each step packs its rows' windows (widths drawn per row and step)
        # into the leading rows of the input buffers, with cumulative lengths on the device
        cus = [np.concatenate([[0], np.cumsum(x)]).astype(np.int32) for x in lens]
        cu_d = [torch.from_numpy(c).to(dev) for c in cus]
        ntok = [max(int(c[-1]), 1) for c in cus]
        verify = [[rs.prepare_verify_varlen(cfg.kda, d, cu_d[j],
                                            *[x[:ntok[j]] for x in sets[j % n_sets]],
                                            st['S'][l], st['rk'][l], st['rd'][l], st['rg'][l],
                                            cursor, st['slots'], out[:ntok[j]], None, counter)
                   for l in range(layers)] for j in range(total)]
        adv = [rs.prepare_cursor_advance_varlen(d, cu_d[j], ntok[j], cursor, fold_len,
                                                st['slots'], acc_d[j], pols[j][0], pols[j][1])
               for j in range(total)]
        verified = [sum(int(lens[j][r]) for r in live) for j in range(total)]
    else:
        verify = [[rs.prepare_verify(cfg.kda, d, *sets[j % n_sets], st['S'][l], st['rk'][l],
                                     st['rd'][l], st['rg'][l], cursor, st['slots'], out, None,
                                     counter)
                   for l in range(layers)] for j in range(n_sets)]
        adv = [rs.prepare_cursor_advance(d, cursor, fold_len, st['slots'], acc_d[j], pols[j][0],
                                         pols[j][1]) for j in range(total)]
        verified = [len(live) * cfg.T] * total
    commit = [rs.prepare_commit_fold(d, cfg.kda, st['S'][l], st['rk'][l], st['rd'][l],
                                     st['rg'][l], fold_len, st['slots']) for l in range(layers)]
    model = CursorModel(cfg, slots_np, np.zeros(cfg.num_slots, np.int32))
    vbytes, cbytes = [], []
    for j in range(total):
        v_, c_ = model.step(accs[j], *pols[j], lens=lens[j])
        vbytes.append(v_)
        cbytes.append(c_)
    stream = torch.cuda.current_stream()
    ev_v, ev_c = [], []

    def step(j, timed):
        if timed:
            e = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            e[0].record(stream)
        for l in range(layers):
            verify[j % len(verify)][l](stream)
        if timed:
            e[1].record(stream)
            ev_v.append(e)
        adv[j](stream)
        if pols[j][0] != rs.FOLD_NONE:
            if timed:
                e = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                e[0].record(stream)
            for l in range(layers):
                commit[l](stream)
            if timed:
                e[1].record(stream)
                ev_c.append((j, e))

    for j in range(warmup):
        step(j, False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for j in range(warmup, total):
        step(j, True)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    assert np.array_equal(cursor.cpu().numpy(), model.cursor), 'cursor model diverged'
    step_s = (t1 - t0) / steps
    acc_per_step = float(np.mean([sum(int(accs[j][r]) for r in live) for j in range(warmup, total)]))
    v_us = float(np.mean([a.elapsed_time(b_) for a, b_ in ev_v])) * 1e3 / layers
    v_b = float(np.mean(vbytes[warmup:]))
    res = {'workload': name, 'batch': cfg.B, 'T': cfg.T, 'ring': cfg.L, 'layers': layers,
           'layer_pool_bytes': pool,
           'windows': f'ragged U{{{cfg.ragged[1]}..{cfg.ragged[2]}}}' if cfg.ragged else 'T',
           'kda': cfg.kda, 'state': cfg.state_dtype, 'ms_per_step': round(step_s * 1e3, 5),
           'verified_tokens_per_s_per_layer':
               round(float(np.mean(verified[warmup:])) * layers / step_s, 1),
           'committed_tokens_per_s_per_layer': round(acc_per_step * layers / step_s, 1),
           'verify_us': round(v_us, 3), 'verify_bytes_per_launch': int(v_b),
           'verify_gbs': round(v_b / v_us / 1e3, 1), 'verify_frac': _frac(v_b, v_us),
           'verify_bytes_all_steps': int(np.mean(vbytes))}
    if ev_c:
        c_us = float(np.mean([e[0].elapsed_time(e[1]) for _, e in ev_c])) * 1e3 / layers
        c_b = float(np.mean([cbytes[j] for j, _ in ev_c]))
        res.update({'commit_fold_us': round(c_us, 3), 'commit_bytes_per_launch': int(c_b),
                    'commit_gbs': round(c_b / c_us / 1e3, 1), 'commit_frac': _frac(c_b, c_us),
                    'commit_steps': len(ev_c),
                    'commit_bytes_all_steps': int(np.mean([cbytes[j] for j in range(total)
                                                            if pols[j][0] != rs.FOLD_NONE]))})
    return res


def snapshot_baseline(name='c2', steps=30, warmup=10, layers=8):
    """The snapshot-verify baseline on a workload's shapes: per layer a verify that writes
    the state after every draft token, then, after every layer's verify, a commit per
    layer that copies the accepted snapshot into the state; against ReplaySSM's ring of
    records.  8 layer pools (state and snapshots, about 5 GB) rotate, so the Infinity Cache
    serves none of them.  Kernel times from one pair of HIP events around each step's
    verifies and one around its commits, divided by the layers; algorithmic bytes: the
    state read, window inputs, outputs and T snapshot writes per live row (verify); the
    accepted snapshot read and the state write per row with accept > 0 (commit).  Memory =
    the per-layer buffers each design keeps for the batch."""
    import torch
    import linear_attention_recurrent_rs_amd as rs
    import workloads as W
    cfg = W.CONFIGS[name]
    st = _rand_setup(cfg, layers)
    dev, slots_np, d = st['dev'], st['slots_np'], st['d']
    sd = torch.bfloat16 if cfg.state_dtype == 'bf16' else torch.float32
    snaps = [torch.empty(cfg.B, cfg.T, cfg.hv, cfg.dk, cfg.dv, dtype=sd, device=dev)
             for _ in range(layers)]
    out = torch.empty(cfg.B * cfg.T, cfg.hv, cfg.dv, device=dev)
    sets = [st['inputs']() for _ in range(4)]
    total = warmup + steps
    accs_np = [W.accept_lengths(cfg, j) for j in range(total)]
    accs = [torch.from_numpy(a.astype(np.int32)).to(dev) for a in accs_np]
    live = [r for r in range(cfg.B) if slots_np[r] >= 0]
    b = _bytes_of(cfg)
    v_b = len(live) * (b['S'] + cfg.T * b['tok_in'] + cfg.T * cfg.hv * cfg.dv * 4 +
                       cfg.T * b['S'] + 8)
    c_b = [sum(2 * b['S'] + 8 for r in live if accs_np[j][r] > 0) for j in range(total)]
    stream = torch.cuda.current_stream()
    ev_v, ev_c = [], []

    def step(j, timed):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(3)] if timed else None
        if timed:
            e[0].record(stream)
        for l in range(layers):
            rs.snapshot_verify(d, cfg.kda, *sets[j % 4], st['S'][l], snaps[l], st['slots'], out,
                               stream=stream)
        if timed:
            e[1].record(stream)
        for l in range(layers):
            rs.snapshot_commit(d, st['S'][l], snaps[l], st['slots'], accs[j], stream=stream)
        if timed:
            e[2].record(stream)
            ev_v.append((e[0], e[1]))
            ev_c.append((e[1], e[2]))

    for j in range(warmup):
        step(j, False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for j in range(warmup, total):
        step(j, True)
    torch.cuda.synchronize()
    step_s = (time.perf_counter() - t0) / steps
    acc_sum = float(np.mean([int(accs_np[j][live].sum()) for j in range(warmup, total)]))
    v_us = float(np.mean([a.elapsed_time(b_) for a, b_ in ev_v])) * 1e3 / layers
    c_us = float(np.mean([a.elapsed_time(b_) for a, b_ in ev_c])) * 1e3 / layers
    cb = float(np.mean(c_b[warmup:]))
    return {'workload': name, 'batch': cfg.B, 'T': cfg.T, 'state': cfg.state_dtype,
            'layers': layers, 'ms_per_step': round(step_s * 1e3, 5),
            'verify_us': round(v_us, 3), 'verify_bytes_per_launch': int(v_b),
            'verify_gbs': round(v_b / v_us / 1e3, 1), 'verify_frac': _frac(v_b, v_us),
            'commit_us': round(c_us, 3), 'commit_bytes_per_launch': int(cb),
            'commit_gbs': round(cb / c_us / 1e3, 1), 'commit_frac': _frac(cb, c_us),
            'verified_tokens_per_s_per_layer': round(len(live) * cfg.T * layers / step_s, 1),
            'committed_tokens_per_s_per_layer': round(acc_sum * layers / step_s, 1),
            'snapshot_bytes_per_layer': cfg.B * cfg.T * cfg.hv * cfg.dk * cfg.dv * b['S'] //
                                        (cfg.hv * cfg.dk * cfg.dv),
            'ring_bytes_per_layer': cfg.B * cfg.L * b['record']}


def conv_workload(name='conv_spec', steps=30, warmup=10, min_pool_bytes=1 << 30):
    """The conv window of a GDN layer (rs_conv_verify, then rs_conv_commit with the step's
    accept lengths) on Qwen3.5-shaped channels (2 x 16 x 128 q/k + 32 x 128 v), bf16
    inputs, taps and state, fp32 outputs, width 4, SiLU.  Layer pools (state, inputs,
    outputs) rotate past 1 GiB; one rollback launch covers every layer (layer-major
    stacks).  Kernel times from one pair of HIP events around each step's verifies and one
    around its rollback, divided by the layers.  Algorithmic bytes: verify
    = per live row the K-1 state rows, the window inputs and outputs, plus the taps and
    bias once; commit = per live row with accept > 0 its K-1 new state rows read and
    written."""
    import torch
    import linear_attention_recurrent_rs_amd as rs
    import workloads as W
    cfg = W.CONV_CONFIGS[name]
    rc = cfg.as_config()
    dev = torch.device('cuda:0')
    g = torch.Generator(device=dev).manual_seed(77)
    a, o = 2, 4
    per_layer = (cfg.num_slots * (cfg.K - 1) * cfg.C * a + cfg.B * cfg.T * cfg.C * (a + o))
    layers = max(8, -(-min_pool_bytes // per_layer))
    bf = torch.bfloat16
    # layer-major stacks: one rollback launch covers every layer, as after the last layer
    state = torch.randn(layers, cfg.num_slots, cfg.K - 1, cfg.C, generator=g, device=dev).to(bf)
    xs = torch.randn(layers, cfg.B * cfg.T, cfg.C, generator=g, device=dev).to(bf)
    ys = [torch.empty(cfg.B * cfg.T, cfg.C, device=dev) for _ in range(layers)]
    w = (torch.randn(cfg.C, cfg.K, generator=g, device=dev) / 2).to(bf)
    b = (0.1 * torch.randn(cfg.C, generator=g, device=dev)).to(bf)
    slots_np = W.slot_map(rc)
    slots = torch.from_numpy(slots_np.astype(np.int32)).to(dev)
    live = [r for r in range(cfg.B) if slots_np[r] >= 0]
    total = warmup + steps
    accs_np = [W.accept_lengths(rc, j) for j in range(total)]
    accs = [torch.from_numpy(x.astype(np.int32)).to(dev) for x in accs_np]
    d = rs.ConvDims(cfg.B, cfg.T, cfg.C, cfg.K, cfg.num_slots, rs.BF16, rs.F32, rs.ACT_SILU)
    verify = [rs.prepare_conv_verify(d, xs[l], w, b, state[l], slots, ys[l]) for l in range(layers)]
    commit = [rs.prepare_conv_commit(d, state, xs, slots, accs[j], layers=layers)
              for j in range(total)]
    v_b = len(live) * ((cfg.K - 1) * cfg.C * a + cfg.T * cfg.C * (a + o) + 8) + cfg.C * (cfg.K + 1) * a
    c_b = [sum(2 * (cfg.K - 1) * cfg.C * a + 8 for r in live if accs_np[j][r] > 0) for j in range(total)]
    stream = torch.cuda.current_stream()
    ev_v, ev_c = [], []

    def step(j, timed):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(3)] if timed else None
        if timed:
            e[0].record(stream)
        for l in range(layers):
            verify[l](stream)
        if timed:
            e[1].record(stream)
        commit[j](stream)
        if timed:
            e[2].record(stream)
            ev_v.append((e[0], e[1]))
            ev_c.append((e[1], e[2]))

    for j in range(warmup):
        step(j, False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for j in range(warmup, total):
        step(j, True)
    torch.cuda.synchronize()
    step_s = (time.perf_counter() - t0) / steps
    v_us = float(np.mean([x.elapsed_time(y) for x, y in ev_v])) * 1e3 / layers
    c_us = float(np.mean([x.elapsed_time(y) for x, y in ev_c])) * 1e3 / layers
    cb = float(np.mean(c_b[warmup:]))
    return {'workload': name, 'batch': cfg.B, 'T': cfg.T, 'channels': cfg.C, 'width': cfg.K,
            'layers': layers, 'ms_per_step': round(step_s * 1e3, 5),
            'verify_us': round(v_us, 3), 'verify_bytes_per_launch': int(v_b),
            'verify_gbs': round(v_b / v_us / 1e3, 1), 'verify_frac': _frac(v_b, v_us),
            'commit_us': round(c_us, 3), 'commit_bytes_per_launch': int(cb),
            'commit_gbs': round(cb / c_us / 1e3, 1), 'commit_frac': _frac(cb, c_us),
            'tokens_per_s_per_layer': round(len(live) * cfg.T * layers / step_s, 1)}


def prefill_workload(B=16, P=512, steps=10, warmup=3):
    """Chunked prefill (rs_gdn_prefill) of a Qwen3.5-shaped GDN layer: B requests with
    P-token prompts each, 16 key / 32 value heads, dk = dv = 128, fp32 state, bf16 inputs.
    Layer pools rotate (8, each with its own state and inputs, past 1 GiB).  Time from one
    pair of HIP events around each step's launches, divided by the layers.  Algorithmic
    bytes per launch: per row the state read and written once, and per token its q, k, v,
    beta, gate (bf16) and output (fp32); flops: per token and value head 4 dk dv for the
    readout of q and k, 2 dk dv for the state update, and the chunk's scores and solve."""
    import torch
    import linear_attention_recurrent_rs_amd as rs
    import workloads as W
    cfg = W.CONFIGS['c1'].with_(B=B, null_rows=0, cursor_init='zero')
    dev = torch.device('cuda:0')
    g = torch.Generator(device=dev).manual_seed(99)
    layers = 8
    bf = torch.bfloat16
    ntok = B * P

    def unit(*shape):
        x = torch.randn(*shape, generator=g, device=dev)
        return x / x.norm(dim=-1, keepdim=True)
    S = [(torch.randn(cfg.num_slots, cfg.hv, cfg.dk, cfg.dv, generator=g, device=dev) * 0.05)
         for _ in range(layers)]
    ins = [(unit(ntok, cfg.hk, cfg.dk).to(bf), unit(ntok, cfg.hk, cfg.dk).to(bf),
            torch.randn(ntok, cfg.hv, cfg.dv, generator=g, device=dev).to(bf),
            torch.rand(ntok, cfg.hv, generator=g, device=dev).to(bf),
            torch.exp(-torch.nn.functional.softplus(
                torch.randn(ntok, cfg.hv, generator=g, device=dev))).to(bf))
           for _ in range(layers)]
    out = torch.empty(ntok, cfg.hv, cfg.dv, device=dev)
    cursor = torch.zeros(cfg.num_slots, dtype=torch.int32, device=dev)
    slots_np = W.slot_map(cfg)
    slots = torch.from_numpy(slots_np.astype(np.int32)).to(dev)
    cu = torch.arange(0, ntok + 1, P, dtype=torch.int32, device=dev)
    d = rs.Dims(cfg.B, 1, cfg.hk, cfg.hv, cfg.dk, cfg.dv, cfg.L, cfg.num_slots, rs.BF16, rs.F32)
    calls = [rs.prepare_gdn_prefill(d, cu, *ins[l], S[l], cursor, slots, out) for l in range(layers)]
    stream = torch.cuda.current_stream()
    for j in range(warmup):
        for l in range(layers):
            calls[l](stream)
    torch.cuda.synchronize()
    ev = []
    t0 = time.perf_counter()
    for j in range(steps):
        e = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
        e[0].record(stream)
        for l in range(layers):
            calls[l](stream)
        e[1].record(stream)
        ev.append(e)
    torch.cuda.synchronize()
    step_s = (time.perf_counter() - t0) / steps
    us = float(np.mean([a.elapsed_time(b_) for a, b_ in ev])) * 1e3 / layers
    sbytes = cfg.hv * cfg.dk * cfg.dv * 4
    tok_bytes = (2 * cfg.hk * cfg.dk + cfg.hv * cfg.dv + 2 * cfg.hv) * 2 + cfg.hv * cfg.dv * 4
    byts = B * (2 * sbytes + 8) + ntok * tok_bytes
    flops = ntok * cfg.hv * (6 * cfg.dk * cfg.dv + 4 * 16 * (cfg.dk + cfg.dv))
    return {'workload': 'gdn_prefill', 'batch': B, 'prompt': P, 'chunk': 16, 'layers': layers,
            'ms_per_step': round(step_s * 1e3, 4), 'kernel_us': round(us, 3),
            'bytes_per_launch': int(byts), 'achieved_gbs': round(byts / us / 1e3, 1),
            'frac_hbm': _frac(byts, us), 'tflops': round(flops / us / 1e6, 2),
            'prefill_tokens_per_s_per_layer': round(ntok / (us * 1e-6), 1)}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split('\n')[0])
    ap.add_argument('--gpus', type=int, default=1)
    ap.add_argument('--steps', type=int, default=50)
    ap.add_argument('--warmup', type=int, default=10)
    ap.add_argument('--layers', type=int, default=8, help='layer pools per step (rotating)')
    ap.add_argument('--tile-v', type=int, default=0)
    ap.add_argument('--only-T', type=int, default=0, help='run one window width only')
    ap.add_argument('--no-cpu-baseline', action='store_true')
    ap.add_argument('--source-hash', action='store_true',
                    help='print the hash of the verify kernel sources and exit')
    ap.add_argument('--copy-calibration', action='store_true',
                    help='first run plain copies of 256 MiB (for counter calibration)')
    ap.add_argument('--no-extra', action='store_true',
                    help='skip the history states and the other workloads')
    ap.add_argument('--only-workload', default='',
                    help='run one of the other workloads (c2, c3, c4, ragged_gdn, '
                         'ragged_kda, snapshot_c2, conv_decode, conv_spec, prefill) alone and exit')
    args = ap.parse_args()
    if args.source_hash:
        print(kernel_source_hash())
        return
    world = int(os.environ.get('WORLD_SIZE', '1'))
    if args.gpus != 1 or world != 1:
        print(f'bench.py runs on one GPU only; --gpus {args.gpus} (WORLD_SIZE {world}) is not '
              'supported: the decode/verify path shards by request or by key-head group with '
              'no exchange inside it, so one GPU shows the per-GPU kernel.', file=sys.stderr)
        sys.exit(2)

    if args.only_workload:
        if args.copy_calibration:
            copy_calibration()
        if args.only_workload.startswith('snapshot_'):
            print(json.dumps(snapshot_baseline(args.only_workload[len('snapshot_'):])), flush=True)
        elif args.only_workload.startswith('conv_'):
            print(json.dumps(conv_workload(args.only_workload)), flush=True)
        elif args.only_workload == 'prefill':
            print(json.dumps(prefill_workload()), flush=True)
        else:
            print(json.dumps(run_workload(args.only_workload, tile_v=args.tile_v)), flush=True)
        return
    Ts = [args.only_T] if args.only_T else [1, 3]
    cpu = None
    if not args.no_cpu_baseline:
        # first: its worker processes are forked before anything initialises the GPU
        cpu = cpu_baseline(Ts[0])
        print(f'# cpu baseline: {cpu}', file=sys.stderr, flush=True)
    if args.copy_calibration:
        copy_calibration()
    res = {}
    for T in Ts:
        res[T] = run_gpu(T, args.steps, args.warmup, args.layers, args.tile_v)
        r = res[T]
        print(f'# T={T}: {r["ms_per_step"]:.4f} ms/step, verify {r["kernel_us"]:.2f} us '
              f'(median {r["kernel_us_median"]:.2f}), {r["achieved_gbs"]:.0f} GB/s, '
              f'{r["value"] / 1e6:.3f} M tok/s/layer', file=sys.stderr, flush=True)
    p = res[Ts[0]]
    cfg = p['cfg']
    traffic = traffic_from_profiles(Ts[0])
    line = {
        'metric': 'verified tokens/s per layer (GDN decode verify, batch 64, T=%d)' % Ts[0],
        'value': round(p['value'], 1),
        'unit': 'tokens/s',
        'n_gpus': 1,
        'steps': args.steps,
        'warmup': args.warmup,
        'ms_per_step': round(p['ms_per_step'], 5),
        'higher_is_better': True,
        'scaling': 'weak',
        'vs_baseline': None,
        'dtype': 'f32',
        'data': 'synthetic',
        'config': {'workload': 'gdn_decode_qwen35_shaped_b64', 'batch': cfg.B,
                   'live_rows': p['live_rows'], 'hk': cfg.hk, 'hv': cfg.hv, 'dk': cfg.dk,
                   'dv': cfg.dv, 'ring': cfg.L, 'T': cfg.T, 'state': 'f32', 'inputs': 'bf16',
                   'layers_per_step': args.layers, 'tile_v': p['tile_v']},
        'roofline': {'bound': 'hbm', 'achieved': round(p['achieved_gbs'], 1),
                     'peak': HBM_PEAK_GBS, 'unit': 'GB/s',
                     'frac': round(p['achieved_gbs'] / HBM_PEAK_GBS, 4),
                     'traffic': traffic, 'kernel': 'rs::verify_fast_kernel',
                     'kernel_us': round(p['kernel_us'], 3),
                     'bytes_per_launch': int(p['bytes_per_launch'])},
    }
    extra = {}
    for T in Ts[1:]:
        r = res[T]
        extra[f'T{T}'] = {'value': round(r['value'], 1), 'ms_per_step': round(r['ms_per_step'], 5),
                          'kernel_us': round(r['kernel_us'], 3),
                          'achieved_gbs': round(r['achieved_gbs'], 1),
                          'frac': round(r['achieved_gbs'] / HBM_PEAK_GBS, 4),
                          'bytes_per_launch': int(r['bytes_per_launch'])}
    if not args.no_extra:
        ref = stream_reference(p['bytes_per_launch'])
        line['roofline']['stream_read_gbs'] = ref['gbs']
        line['roofline']['frac_of_stream_read'] = round(p['achieved_gbs'] / ref['gbs'], 4)
        print(f'# plain streaming read of {ref["bytes"]} B: {ref["us"]} us, {ref["gbs"]} GB/s',
              file=sys.stderr, flush=True)
        for T in (1, 3):
            extra[f'history_states_T{T}'] = history_states(T)
            print(f'# history states T={T}: {extra[f"history_states_T{T}"]}', file=sys.stderr,
                  flush=True)
        for name in ('c2', 'c3', 'c4', 'ragged_gdn', 'ragged_kda'):
            extra[name] = run_workload(name)
            print(f'# {name}: {extra[name]}', file=sys.stderr, flush=True)
        extra['snapshot_baseline_c2'] = snapshot_baseline('c2')
        print(f'# snapshot baseline: {extra["snapshot_baseline_c2"]}', file=sys.stderr, flush=True)
        for name in ('conv_decode', 'conv_spec'):
            extra[name] = conv_workload(name)
            print(f'# {name}: {extra[name]}', file=sys.stderr, flush=True)
        extra['prefill_b16_p512'] = prefill_workload()
        print(f'# prefill: {extra["prefill_b16_p512"]}', file=sys.stderr, flush=True)
    if extra:
        line['extra'] = extra
    if cpu is not None:
        cpu['value'] = round(cpu['value'], 2)
        line['cpu_baseline'] = cpu
    print(json.dumps(line), flush=True)


if __name__ == '__main__':
    main()
