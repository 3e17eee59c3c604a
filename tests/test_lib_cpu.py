"""CPU tests of the C ABI library: it loads, exports every entry point include/rs.h
declares, and validates arguments on the host (no GPU needed: validation precedes any
device work)."""
import ctypes
import os
import re

import pytest

import linear_attention_recurrent_rs_amd as rs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    text = open(os.path.join(ROOT, 'include', 'rs.h')).read()
    return sorted(set(re.findall(r'^\s*(?:rs_status|const char\*)\s+(rs_\w+)\s*\(', text, re.M)))


def test_library_built():
    assert os.path.exists(rs.library_path), 'run python -m linear_attention_recurrent_rs_amd.build'


def test_exports_every_declared_symbol():
    names = _declared()
    assert {'rs_gdn_verify', 'rs_kda_verify', 'rs_cursor_advance', 'rs_commit_fold',
            'rs_materialize', 'rs_status_str'} <= set(names)
    lib = ctypes.CDLL(rs.library_path)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings():
    lib = rs._lib()
    for code in range(8):
        assert lib.rs_status_str(code).decode().startswith('RS_')


def _dims(**kw):
    d = dict(batch=4, T=1, hk=2, hv=4, dk=128, dv=128, ring_cap=16, num_slots=8,
             act_dtype=rs.BF16, state_dtype=rs.F32, tile_v=0, scale=1.0)
    d.update(kw)
    return rs.Dims(**d)


def test_dims_layout():
    """The Python struct matches rs_dims: the query scale sits between the dtypes and the
    tile width, and defaults to 1."""
    assert [f for f, _ in rs.Dims._fields_][-2:] == ['scale', 'tile_v']
    assert ctypes.sizeof(rs.Dims) == 12 * 4
    d = rs.Dims(1, 2, 3, 4, 16, 32, 8, 9, rs.BF16, rs.F32, 64)
    assert (d.tile_v, d.scale, d.dv) == (64, 1.0, 32)
    assert rs.Dims(1, 1, 1, 1, 16, 16, 4, 1, scale=0.125).scale == 0.125


@pytest.mark.parametrize('scale', [0.0, float('nan'), float('inf'), -float('inf')])
def test_scale_validation(scale):
    """The verifies refuse a query scale that is zero or not finite (RS_E_VALUE = 6), on
    the host before any launch; the commit fold and materialize do not read it."""
    lib = rs._lib()
    d = _dims(scale=scale)
    fake = ctypes.c_void_p(256)
    assert lib.rs_gdn_verify(ctypes.byref(d), *([fake] * 14), None) == 6
    assert lib.rs_kda_verify(ctypes.byref(_dims(scale=scale, hk=4)), *([fake] * 14), None) == 6
    assert lib.rs_snapshot_verify(ctypes.byref(d), 0, *([fake] * 9), None) == 6
    assert lib.rs_verify_launch_info(ctypes.byref(d), 0, None, None, None) == 6
    assert lib.rs_commit_fold(ctypes.byref(d), 0, *([None] * 6), None) == 1   # NULLPTR, not VALUE


@pytest.mark.parametrize('kw,code', [
    (dict(T=0), 2), (dict(T=17), 2), (dict(hv=3), 2), (dict(dk=24), 2), (dict(dk=272), 2),
    (dict(dv=40), 2), (dict(act_dtype=7), 3), (dict(ring_cap=0), 2), (dict(T=4, ring_cap=3), 4),
    (dict(tile_v=48), 2), (dict(tile_v=128, dv=64), 2), (dict(num_slots=0), 2),
])
def test_verify_validation(kw, code):
    lib = rs._lib()
    d = _dims(**kw)
    assert lib.rs_gdn_verify(ctypes.byref(d), *([None] * 14), None) == code


def test_verify_nullptr_and_kda_shape():
    lib = rs._lib()
    d = _dims()
    assert lib.rs_gdn_verify(ctypes.byref(d), *([None] * 14), None) == 1
    assert lib.rs_kda_verify(ctypes.byref(d), *([None] * 14), None) == 2   # hv != hk
    assert lib.rs_gdn_verify(None, *([None] * 14), None) == 1


def test_launch_info():
    tv, wg, lds = rs.verify_launch_info(_dims(batch=64, hk=16, hv=32))
    assert tv == 64 and wg == 64 * 32 * 2 and 0 < lds <= 160 * 1024
    tv, wg, lds = rs.verify_launch_info(_dims(batch=64, hk=16, hv=32, tile_v=128))
    assert tv == 128 and wg == 64 * 32


@pytest.mark.parametrize('kw,kda,per_cu', [
    (dict(T=1), False, 5),                                  # the decode, held at five
    (dict(T=3), False, 7),                                  # (its register cap sets six)
    (dict(T=3, hk=32), True, 6),                            # KDA's compact split-readout plan
    (dict(T=8, ring_cap=64, batch=256, num_slots=256), False, 4),   # history keys in registers
])
def test_launch_plan_residency(kw, kda, per_cu):
    """Workgroups per CU that the verify's LDS plan allows (160 KiB of LDS a CU) for the
    benchmark's shapes: the plans are laid out for these residencies."""
    d = dict(batch=64, hk=16, hv=32, num_slots=96)
    d.update(kw)
    _, _, lds = rs.verify_launch_info(_dims(**d), kda=kda)
    assert (160 * 1024) // lds == per_cu, lds


def test_advance_and_fold_validation():
    lib = rs._lib()
    d = _dims()
    assert lib.rs_cursor_advance(ctypes.byref(d), None, None, None, None, 0, 0, None, None) == 1
    assert lib.rs_cursor_advance(ctypes.byref(d), None, None, None, None, 9, 0, None, None) == 2
    assert lib.rs_cursor_advance(ctypes.byref(d), None, None, None, None, 2, 0, None, None) == 2
    assert lib.rs_commit_fold(ctypes.byref(d), 0, *([None] * 6), None) == 1
    assert lib.rs_commit_fold(ctypes.byref(d), 1, *([None] * 6), None) == 2
    assert lib.rs_materialize(ctypes.byref(d), 0, *([None] * 7), None) == 1


def test_stream_read_validation():
    """The bandwidth reference rejects bad arguments on the host, before any launch."""
    lib = rs._lib()
    fake = ctypes.c_void_p(0x10000)                  # never dereferenced: rejected first
    assert lib.rs_stream_read(None, 1024, fake, None) == 1
    assert lib.rs_stream_read(fake, 1024, None, None) == 1
    assert lib.rs_stream_read(fake, 0, fake, None) == 2
    assert lib.rs_stream_read(fake, 1000, fake, None) == 2             # not a multiple of 16
    assert lib.rs_stream_read(ctypes.c_void_p(0x10008), 1024, fake, None) == 2   # misaligned


def test_varlen_validation():
    """The ragged-window entry points: a missing cu_seqlens is RS_E_NULLPTR, a negative
    token count RS_E_SHAPE, and dimension errors are reported as for the uniform calls."""
    lib = rs._lib()
    fake = ctypes.c_void_p(256)            # never dereferenced: validation fails first
    d = _dims(T=4)
    dk = _dims(T=4, hk=4)
    assert lib.rs_gdn_verify_varlen(ctypes.byref(d), None, 8, *([None] * 14), None) == 1
    assert lib.rs_kda_verify_varlen(ctypes.byref(dk), None, 8, *([None] * 14), None) == 1
    assert lib.rs_gdn_verify_varlen(ctypes.byref(d), fake, -1, *([None] * 14), None) == 2
    assert lib.rs_kda_verify_varlen(ctypes.byref(dk), fake, -1, *([None] * 14), None) == 2
    bad = _dims(T=0)
    assert lib.rs_gdn_verify_varlen(ctypes.byref(bad), fake, 8, *([None] * 14), None) == 2
    adv = lib.rs_cursor_advance_varlen
    assert adv(ctypes.byref(d), None, 8, *([None] * 4), 0, 0, None, None) == 1
    assert adv(ctypes.byref(d), fake, -1, *([None] * 4), 0, 0, None, None) == 2
    assert adv(ctypes.byref(_dims(T=4, ring_cap=3)), fake, 8, *([None] * 4), 0, 0, None,
               None) == 4
    empty = _dims(batch=0)
    assert lib.rs_gdn_verify_varlen(ctypes.byref(empty), None, 0, *([None] * 14), None) == 0


def test_snapshot_validation():
    """The snapshot-verify baseline validates like the ring calls: RS_E_SHAPE for bad dims
    or KDA with hv != hk, RS_E_RING_TOO_SMALL when the ring cannot hold T, RS_E_NULLPTR for
    missing buffers, and an empty batch is a no-op."""
    lib = rs._lib()
    d = _dims(T=4)
    assert lib.rs_snapshot_verify(ctypes.byref(d), 0, *([None] * 9), None) == 1
    assert lib.rs_snapshot_verify(ctypes.byref(d), 1, *([None] * 9), None) == 2   # hv != hk
    assert lib.rs_snapshot_verify(ctypes.byref(_dims(T=0)), 0, *([None] * 9), None) == 2
    assert lib.rs_snapshot_verify(ctypes.byref(_dims(T=4, ring_cap=3)), 0, *([None] * 9),
                                  None) == 4
    assert lib.rs_snapshot_commit(ctypes.byref(d), *([None] * 4), None) == 1
    assert lib.rs_snapshot_commit(ctypes.byref(_dims(T=17)), *([None] * 4), None) == 2
    empty = _dims(batch=0, T=4)
    assert lib.rs_snapshot_verify(ctypes.byref(empty), 0, *([None] * 9), None) == 0
    assert lib.rs_snapshot_commit(ctypes.byref(empty), *([None] * 4), None) == 0


def _cdims(**kw):
    d = dict(batch=4, T=2, channels=64, width=4, num_slots=8, act_dtype=rs.BF16,
             out_dtype=rs.F32, activation=rs.ACT_SILU)
    d.update(kw)
    return rs.ConvDims(*[d[f] for f, _ in rs.ConvDims._fields_])


@pytest.mark.parametrize('kw,code', [
    (dict(T=0), 2), (dict(T=17), 2), (dict(channels=12), 2), (dict(channels=0), 2),
    (dict(width=1), 2), (dict(width=5), 2), (dict(num_slots=0), 2), (dict(batch=-1), 2),
    (dict(act_dtype=5), 3), (dict(out_dtype=9), 3), (dict(activation=2), 6),
])
def test_conv_validation(kw, code):
    """The conv window's entry points validate on the host before any launch."""
    lib = rs._lib()
    fake = ctypes.c_void_p(256)
    d = _cdims(**kw)
    assert lib.rs_conv_verify(ctypes.byref(d), None, 0, *([fake] * 6), None) == code
    assert lib.rs_conv_commit(ctypes.byref(d), None, 0, 1, *([fake] * 4), None) == code


def test_conv_nullptr_and_empty():
    lib = rs._lib()
    fake = ctypes.c_void_p(256)
    d = _cdims()
    assert lib.rs_conv_verify(ctypes.byref(d), None, 0, None, *([fake] * 5), None) == 1
    assert lib.rs_conv_commit(ctypes.byref(d), None, 0, 1, fake, fake, fake, None, None) == 1
    assert lib.rs_conv_commit(ctypes.byref(d), None, 0, 0, *([fake] * 4), None) == 2   # layers
    assert lib.rs_conv_commit(ctypes.byref(d), None, 0, 65536, *([fake] * 4), None) == 2
    assert lib.rs_conv_verify(ctypes.byref(d), fake, -1, *([fake] * 6), None) == 2
    empty = _cdims(batch=0)
    assert lib.rs_conv_verify(ctypes.byref(empty), None, 0, *([None] * 6), None) == 0
    assert lib.rs_conv_commit(ctypes.byref(empty), None, 0, 1, *([None] * 4), None) == 0
    assert lib.rs_conv_verify(None, None, 0, *([None] * 6), None) == 1


def test_prefill_validation():
    """The prefill entry point validates on the host before any launch: it covers dk = 128
    with bf16 inputs and dv a multiple of 64; it needs cu_seqlens and a valid scale."""
    lib = rs._lib()
    fake = ctypes.c_void_p(256)
    f = lib.rs_gdn_prefill
    ok = _dims(T=1)
    assert f(ctypes.byref(ok), None, 8, *([fake] * 9), None) == 1          # cu_seqlens
    assert f(ctypes.byref(ok), fake, 8, fake, None, *([fake] * 7), None) == 1
    assert f(ctypes.byref(ok), fake, -1, *([fake] * 9), None) == 2
    assert f(ctypes.byref(_dims(dk=64)), fake, 8, *([fake] * 9), None) == 2
    assert f(ctypes.byref(_dims(dv=96)), fake, 8, *([fake] * 9), None) == 2
    assert f(ctypes.byref(_dims(hv=3)), fake, 8, *([fake] * 9), None) == 2
    assert f(ctypes.byref(_dims(act_dtype=rs.F32)), fake, 8, *([fake] * 9), None) == 3
    assert f(ctypes.byref(_dims(scale=0.0)), fake, 8, *([fake] * 9), None) == 6
    assert f(ctypes.byref(_dims(batch=0)), None, 0, *([None] * 9), None) == 0
    assert f(None, fake, 8, *([fake] * 9), None) == 1
