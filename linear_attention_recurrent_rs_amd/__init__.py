"""ReplaySSM decode / speculative verify for GDN and KDA layers on MI355X (gfx950).

Thin Python binding over the C ABI in include/rs.h (librs.so, built in-tree by
``linear_attention_recurrent_rs_amd.build``).  Every function here marshals torch
tensors into pointers and sizes and calls the library; all computation runs in the HIP
kernels.  Before a call it checks that each tensor lives on the GPU, is contiguous and
has the element count and dtype the dimensions imply, so a wrong tensor becomes an
exception instead of an out-of-bounds device access.  There is no fallback: without the
built library every call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

__all__ = ['Dims', 'RSError', 'gdn_verify', 'kda_verify', 'cursor_advance', 'commit_fold',
           'gdn_verify_varlen', 'kda_verify_varlen', 'cursor_advance_varlen',
           'snapshot_verify', 'snapshot_commit',
           'prepare_verify_varlen', 'prepare_cursor_advance_varlen',
           'materialize', 'verify_launch_info', 'stream_read', 'library_path', 'F32', 'BF16',
           'prepare_verify', 'prepare_cursor_advance', 'prepare_commit_fold',
           'FOLD_NONE', 'FOLD_EVERY_COMMIT', 'FOLD_LAZY', 'FOLD_FORCE', 'gdn_verify_noalloc',
           'ConvDims', 'conv_verify', 'conv_commit', 'prepare_conv_verify',
           'prepare_conv_commit', 'ACT_NONE', 'ACT_SILU', 'gdn_prefill', 'prepare_gdn_prefill']

F32, BF16 = 0, 1
ACT_NONE, ACT_SILU = 0, 1
FOLD_NONE, FOLD_EVERY_COMMIT, FOLD_LAZY, FOLD_FORCE = 0, 1, 2, 3
_TORCH_DTYPE = {F32: torch.float32, BF16: torch.bfloat16}

library_path = os.path.join(os.path.dirname(os.path.abspath(__file__)), 'librs.so')


class RSError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {_lib().rs_status_str(status).decode()}")
        self.status = status


class Dims(ctypes.Structure):
    """rs_dims: batch, T, hk, hv, dk, dv, ring_cap, num_slots, act_dtype, state_dtype,
    scale, tile_v (the C field order).  Built as Dims(batch, T, hk, hv, dk, dv, ring_cap,
    num_slots, act_dtype, state_dtype, tile_v=0, scale=1.0): the query scale is a keyword,
    1.0 unless given."""
    _fields_ = [('batch', ctypes.c_int32), ('T', ctypes.c_int32), ('hk', ctypes.c_int32),
                ('hv', ctypes.c_int32), ('dk', ctypes.c_int32), ('dv', ctypes.c_int32),
                ('ring_cap', ctypes.c_int32), ('num_slots', ctypes.c_int32),
                ('act_dtype', ctypes.c_int), ('state_dtype', ctypes.c_int),
                ('scale', ctypes.c_float), ('tile_v', ctypes.c_int32)]

    def __init__(self, batch=0, T=1, hk=1, hv=1, dk=16, dv=16, ring_cap=1, num_slots=1,
                 act_dtype=0, state_dtype=0, tile_v=0, scale=1.0):
        super().__init__(batch, T, hk, hv, dk, dv, ring_cap, num_slots, act_dtype,
                         state_dtype, scale, tile_v)

    def __repr__(self):
        return 'Dims(' + ', '.join(f'{f}={getattr(self, f)}' for f, _ in self._fields_) + ')'


class ConvDims(ctypes.Structure):
    """rs_conv_dims: batch, T, channels, width, num_slots, act_dtype, out_dtype, activation."""
    _fields_ = [('batch', ctypes.c_int32), ('T', ctypes.c_int32), ('channels', ctypes.c_int32),
                ('width', ctypes.c_int32), ('num_slots', ctypes.c_int32),
                ('act_dtype', ctypes.c_int), ('out_dtype', ctypes.c_int),
                ('activation', ctypes.c_int)]

    def __repr__(self):
        return 'ConvDims(' + ', '.join(f'{f}={getattr(self, f)}' for f, _ in self._fields_) + ')'


_LIB = None
_P = ctypes.c_void_p


def _lib():
    global _LIB
    if _LIB is None:
        if not os.path.exists(library_path):
            raise RuntimeError(f"{library_path} is not built; run "
                               "`python -m linear_attention_recurrent_rs_amd.build`")
        lib = ctypes.CDLL(library_path)
        dp = ctypes.POINTER(Dims)
        verify_args = [dp] + [_P] * 14 + [_P]
        for name in ('rs_gdn_verify', 'rs_kda_verify'):
            getattr(lib, name).argtypes = verify_args
            getattr(lib, name).restype = ctypes.c_int
        varlen_args = [dp, _P, ctypes.c_int32] + [_P] * 14 + [_P]
        for name in ('rs_gdn_verify_varlen', 'rs_kda_verify_varlen'):
            getattr(lib, name).argtypes = varlen_args
            getattr(lib, name).restype = ctypes.c_int
        lib.rs_gdn_verify_noalloc.argtypes = [dp] + [_P] * 13 + [_P]
        lib.rs_gdn_verify_noalloc.restype = ctypes.c_int
        lib.rs_cursor_advance.argtypes = [dp, _P, _P, _P, _P, ctypes.c_int, ctypes.c_int32, _P, _P]
        lib.rs_cursor_advance.restype = ctypes.c_int
        lib.rs_cursor_advance_varlen.argtypes = [dp, _P, ctypes.c_int32, _P, _P, _P, _P,
                                                 ctypes.c_int, ctypes.c_int32, _P, _P]
        lib.rs_cursor_advance_varlen.restype = ctypes.c_int
        lib.rs_commit_fold.argtypes = [dp, ctypes.c_int, _P, _P, _P, _P, _P, _P, _P]
        lib.rs_commit_fold.restype = ctypes.c_int
        lib.rs_materialize.argtypes = [dp, ctypes.c_int, _P, _P, _P, _P, _P, _P, _P, _P]
        lib.rs_materialize.restype = ctypes.c_int
        lib.rs_snapshot_verify.argtypes = [dp, ctypes.c_int] + [_P] * 10
        lib.rs_snapshot_verify.restype = ctypes.c_int
        lib.rs_snapshot_commit.argtypes = [dp] + [_P] * 5
        lib.rs_snapshot_commit.restype = ctypes.c_int
        lib.rs_status_str.argtypes = [ctypes.c_int]
        lib.rs_status_str.restype = ctypes.c_char_p
        lib.rs_verify_launch_info.argtypes = [dp, ctypes.c_int, _P, _P, _P]
        lib.rs_verify_launch_info.restype = ctypes.c_int
        lib.rs_gdn_prefill.argtypes = [dp, _P, ctypes.c_int32] + [_P] * 9 + [_P]
        lib.rs_gdn_prefill.restype = ctypes.c_int
        cdp = ctypes.POINTER(ConvDims)
        lib.rs_conv_verify.argtypes = [cdp, _P, ctypes.c_int32] + [_P] * 6 + [_P]
        lib.rs_conv_verify.restype = ctypes.c_int
        lib.rs_conv_commit.argtypes = [cdp, _P, ctypes.c_int32, ctypes.c_int32] + [_P] * 4 + [_P]
        lib.rs_conv_commit.restype = ctypes.c_int
        lib.rs_stream_read.argtypes = [_P, ctypes.c_uint64, _P, _P]
        lib.rs_stream_read.restype = ctypes.c_int
        _LIB = lib
    return _LIB


def _ptr(t: Optional[torch.Tensor], name: str, numel: int, dtype: torch.dtype,
         optional: bool = False):
    if t is None:
        if optional:
            return None
        raise ValueError(f"{name} is required")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if t.numel() != numel:
        raise ValueError(f"{name}: {t.numel()} elements, expected {numel}")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _check(status: int, where: str):
    if status != 0:
        raise RSError(status, where)


def _verify_ptrs(kda: bool, d: Dims, q, k, v, beta, gate, state, ring_k, ring_d, ring_g, cursor,
                 slot_idx, out, write_pos_out, group_counter, ntok=None,
                 counter_optional=False):
    at, st = _TORCH_DTYPE[d.act_dtype], _TORCH_DTYPE[d.state_dtype]
    BT = d.batch * d.T if ntok is None else ntok
    S, L = d.num_slots, d.ring_cap
    g_per = d.hv * d.dk if kda else d.hv
    args = [
        _ptr(q, 'q', BT * d.hk * d.dk, at), _ptr(k, 'k', BT * d.hk * d.dk, at),
        _ptr(v, 'v', BT * d.hv * d.dv, at), _ptr(beta, 'beta', BT * d.hv, at),
        _ptr(gate, 'gate', BT * g_per, at),
        _ptr(state, 'state', S * d.hv * d.dk * d.dv, st),
        _ptr(ring_k, 'ring_k', S * L * d.hk * d.dk, at),
        _ptr(ring_d, 'ring_d', S * L * d.hv * d.dv, torch.float32),
        _ptr(ring_g, 'ring_g', S * L * g_per, torch.float32),
        _ptr(cursor, 'cursor', S, torch.int32), _ptr(slot_idx, 'slot_idx', d.batch, torch.int32),
        _ptr(out, 'out', BT * d.hv * d.dv, torch.float32),
        _ptr(write_pos_out, 'write_pos_out', d.batch, torch.int32, optional=True),
        _ptr(group_counter, 'group_counter', d.batch * d.hk, torch.int32,
             optional=counter_optional),
    ]
    return args


def _verify(kda: bool, d: Dims, q, k, v, beta, gate, state, ring_k, ring_d, ring_g, cursor,
            slot_idx, out, write_pos_out, group_counter, stream):
    args = _verify_ptrs(kda, d, q, k, v, beta, gate, state, ring_k, ring_d, ring_g, cursor,
                        slot_idx, out, write_pos_out, group_counter)
    fn = _lib().rs_kda_verify if kda else _lib().rs_gdn_verify
    _check(fn(ctypes.byref(d), *args, _stream(stream)), 'rs_kda_verify' if kda else 'rs_gdn_verify')


def gdn_verify(d: Dims, q, k, v, beta, gate, state, ring_k, ring_d, ring_g, cursor, slot_idx,
               out, write_pos_out=None, group_counter=None, stream=None):
    """rs_gdn_verify: one GDN layer's verify (decode when T == 1)."""
    _verify(False, d, q, k, v, beta, gate, state, ring_k, ring_d, ring_g, cursor, slot_idx, out,
            write_pos_out, group_counter, stream)


def gdn_verify_noalloc(d: Dims, q, k, v, beta, gate, state, ring_k, ring_d, ring_g, cursor,
                       slot_idx, out, write_pos_out=None, stream=None):
    """rs_gdn_verify_noalloc: rs_gdn_verify with the fold counters in the library's static
    device workspace (no group_counter argument; nothing is allocated)."""
    args = _verify_ptrs(False, d, q, k, v, beta, gate, state, ring_k, ring_d, ring_g, cursor,
                        slot_idx, out, write_pos_out, None, counter_optional=True)
    _check(_lib().rs_gdn_verify_noalloc(ctypes.byref(d), *args[:-1], _stream(stream)),
           'rs_gdn_verify_noalloc')


def kda_verify(d: Dims, q, k, v, beta, gate, state, ring_k, ring_d, ring_g, cursor, slot_idx,
               out, write_pos_out=None, group_counter=None, stream=None):
    """rs_kda_verify: one KDA layer's verify (per-channel decay)."""
    _verify(True, d, q, k, v, beta, gate, state, ring_k, ring_d, ring_g, cursor, slot_idx, out,
            write_pos_out, group_counter, stream)


def _ntok(q) -> int:
    if q is None or q.dim() < 1:
        raise ValueError('q must be a [total_tokens, hk, dk] tensor')
    return int(q.shape[0])


def _verify_varlen(kda: bool, d: Dims, cu_seqlens, q, k, v, beta, gate, state, ring_k, ring_d,
                   ring_g, cursor, slot_idx, out, write_pos_out, group_counter, stream):
    ntok = _ntok(q)
    args = _verify_ptrs(kda, d, q, k, v, beta, gate, state, ring_k, ring_d, ring_g, cursor,
                        slot_idx, out, write_pos_out, group_counter, ntok)
    cu = _ptr(cu_seqlens, 'cu_seqlens', d.batch + 1, torch.int32)
    name = 'rs_kda_verify_varlen' if kda else 'rs_gdn_verify_varlen'
    _check(getattr(_lib(), name)(ctypes.byref(d), cu, ctypes.c_int32(ntok), *args,
                                 _stream(stream)), name)


def gdn_verify_varlen(d: Dims, cu_seqlens, q, k, v, beta, gate, state, ring_k, ring_d, ring_g,
                      cursor, slot_idx, out, write_pos_out=None, group_counter=None,
                      stream=None):
    """rs_gdn_verify_varlen: GDN verify with ragged windows.  Row r owns packed tokens
    [cu_seqlens[r], cu_seqlens[r+1]) (at most d.T of them); the token count is q.shape[0]."""
    _verify_varlen(False, d, cu_seqlens, q, k, v, beta, gate, state, ring_k, ring_d, ring_g,
                   cursor, slot_idx, out, write_pos_out, group_counter, stream)


def kda_verify_varlen(d: Dims, cu_seqlens, q, k, v, beta, gate, state, ring_k, ring_d, ring_g,
                      cursor, slot_idx, out, write_pos_out=None, group_counter=None,
                      stream=None):
    """rs_kda_verify_varlen: KDA verify with ragged windows (as gdn_verify_varlen)."""
    _verify_varlen(True, d, cu_seqlens, q, k, v, beta, gate, state, ring_k, ring_d, ring_g,
                   cursor, slot_idx, out, write_pos_out, group_counter, stream)


def cursor_advance(d: Dims, cursor, fold_len, slot_idx, accept_len, policy: int = FOLD_NONE,
                   next_T: int = 0, force_mask=None, stream=None):
    """rs_cursor_advance: once per step, after every layer's verify."""
    args = [_ptr(cursor, 'cursor', d.num_slots, torch.int32),
            _ptr(fold_len, 'fold_len', d.num_slots, torch.int32),
            _ptr(slot_idx, 'slot_idx', d.batch, torch.int32),
            _ptr(accept_len, 'accept_len', d.batch, torch.int32)]
    fm = _ptr(force_mask, 'force_mask', d.batch, torch.uint8, optional=True)
    _check(_lib().rs_cursor_advance(ctypes.byref(d), *args, int(policy), int(next_T), fm,
                                    _stream(stream)), 'rs_cursor_advance')


def cursor_advance_varlen(d: Dims, cu_seqlens, total_tokens: int, cursor, fold_len, slot_idx,
                          accept_len, policy: int = FOLD_NONE, next_T: int = 0,
                          force_mask=None, stream=None):
    """rs_cursor_advance_varlen: the advance after ragged verifies (same cu_seqlens and
    total token count as the step's verifies)."""
    args = [_ptr(cu_seqlens, 'cu_seqlens', d.batch + 1, torch.int32),
            ctypes.c_int32(int(total_tokens)),
            _ptr(cursor, 'cursor', d.num_slots, torch.int32),
            _ptr(fold_len, 'fold_len', d.num_slots, torch.int32),
            _ptr(slot_idx, 'slot_idx', d.batch, torch.int32),
            _ptr(accept_len, 'accept_len', d.batch, torch.int32)]
    fm = _ptr(force_mask, 'force_mask', d.batch, torch.uint8, optional=True)
    _check(_lib().rs_cursor_advance_varlen(ctypes.byref(d), *args, int(policy), int(next_T), fm,
                                           _stream(stream)), 'rs_cursor_advance_varlen')


def _fold_ptrs(d: Dims, kda: bool, state, ring_k, ring_d, ring_g):
    at, st = _TORCH_DTYPE[d.act_dtype], _TORCH_DTYPE[d.state_dtype]
    S, L = d.num_slots, d.ring_cap
    g_per = d.hv * d.dk if kda else d.hv
    return [_ptr(state, 'state', S * d.hv * d.dk * d.dv, st),
            _ptr(ring_k, 'ring_k', S * L * d.hk * d.dk, at),
            _ptr(ring_d, 'ring_d', S * L * d.hv * d.dv, torch.float32),
            _ptr(ring_g, 'ring_g', S * L * g_per, torch.float32)]


def commit_fold(d: Dims, kda: bool, state, ring_k, ring_d, ring_g, fold_len, slot_idx,
                stream=None):
    """rs_commit_fold: fold ring[0:fold_len[s]] into S[s] for live rows."""
    p = _fold_ptrs(d, kda, state, ring_k, ring_d, ring_g)
    _check(_lib().rs_commit_fold(ctypes.byref(d), int(kda), *p,
                                 _ptr(fold_len, 'fold_len', d.num_slots, torch.int32),
                                 _ptr(slot_idx, 'slot_idx', d.batch, torch.int32),
                                 _stream(stream)), 'rs_commit_fold')


def materialize(d: Dims, kda: bool, state, ring_k, ring_d, ring_g, cursor, slot_idx, out_state,
                stream=None):
    """rs_materialize: fold(S[s], ring[s, 0:cursor[s]]) into out_state [B, hv, dk, dv] fp32."""
    p = _fold_ptrs(d, kda, state, ring_k, ring_d, ring_g)
    _check(_lib().rs_materialize(ctypes.byref(d), int(kda), *p,
                                 _ptr(cursor, 'cursor', d.num_slots, torch.int32),
                                 _ptr(slot_idx, 'slot_idx', d.batch, torch.int32),
                                 _ptr(out_state, 'out_state', d.batch * d.hv * d.dk * d.dv,
                                      torch.float32),
                                 _stream(stream)), 'rs_materialize')


def snapshot_verify(d: Dims, kda: bool, q, k, v, beta, gate, state, snapshots, slot_idx, out,
                    stream=None):
    """rs_snapshot_verify: the snapshot-verify baseline; snapshots [B, T, hv, dk, dv] in the
    state dtype receive S after every draft token."""
    at, st = _TORCH_DTYPE[d.act_dtype], _TORCH_DTYPE[d.state_dtype]
    BT = d.batch * d.T
    g_per = d.hv * d.dk if kda else d.hv
    args = [_ptr(q, 'q', BT * d.hk * d.dk, at), _ptr(k, 'k', BT * d.hk * d.dk, at),
            _ptr(v, 'v', BT * d.hv * d.dv, at), _ptr(beta, 'beta', BT * d.hv, at),
            _ptr(gate, 'gate', BT * g_per, at),
            _ptr(state, 'state', d.num_slots * d.hv * d.dk * d.dv, st),
            _ptr(snapshots, 'snapshots', BT * d.hv * d.dk * d.dv, st),
            _ptr(slot_idx, 'slot_idx', d.batch, torch.int32),
            _ptr(out, 'out', BT * d.hv * d.dv, torch.float32)]
    _check(_lib().rs_snapshot_verify(ctypes.byref(d), int(kda), *args, _stream(stream)),
           'rs_snapshot_verify')


def snapshot_commit(d: Dims, state, snapshots, slot_idx, accept_len, stream=None):
    """rs_snapshot_commit: state[slot] <- snapshots[row, accept - 1] for accept > 0."""
    st = _TORCH_DTYPE[d.state_dtype]
    args = [_ptr(state, 'state', d.num_slots * d.hv * d.dk * d.dv, st),
            _ptr(snapshots, 'snapshots', d.batch * d.T * d.hv * d.dk * d.dv, st),
            _ptr(slot_idx, 'slot_idx', d.batch, torch.int32),
            _ptr(accept_len, 'accept_len', d.batch, torch.int32)]
    _check(_lib().rs_snapshot_commit(ctypes.byref(d), *args, _stream(stream)),
           'rs_snapshot_commit')


def _prefill_ptrs(d: Dims, cu_seqlens, q, k, v, beta, gate, state, cursor, slot_idx, out):
    at, st = _TORCH_DTYPE[d.act_dtype], _TORCH_DTYPE[d.state_dtype]
    ntok = _ntok(q)
    return ntok, [_ptr(cu_seqlens, 'cu_seqlens', d.batch + 1, torch.int32),
                  ctypes.c_int32(ntok),
                  _ptr(q, 'q', ntok * d.hk * d.dk, at), _ptr(k, 'k', ntok * d.hk * d.dk, at),
                  _ptr(v, 'v', ntok * d.hv * d.dv, at), _ptr(beta, 'beta', ntok * d.hv, at),
                  _ptr(gate, 'gate', ntok * d.hv, at),
                  _ptr(state, 'state', d.num_slots * d.hv * d.dk * d.dv, st),
                  _ptr(cursor, 'cursor', d.num_slots, torch.int32),
                  _ptr(slot_idx, 'slot_idx', d.batch, torch.int32),
                  _ptr(out, 'out', ntok * d.hv * d.dv, torch.float32)]


def gdn_prefill(d: Dims, cu_seqlens, q, k, v, beta, gate, state, cursor, slot_idx, out,
                stream=None):
    """rs_gdn_prefill: row r's prompt is packed tokens [cu_seqlens[r], cu_seqlens[r+1]) of
    q [tokens, hk, 128] (tokens = q.shape[0]); S of each live slot becomes the state after
    its prompt, its cursor 0; out [tokens, hv, dv] fp32."""
    _, args = _prefill_ptrs(d, cu_seqlens, q, k, v, beta, gate, state, cursor, slot_idx, out)
    _check(_lib().rs_gdn_prefill(ctypes.byref(d), *args, _stream(stream)), 'rs_gdn_prefill')


def prepare_gdn_prefill(d: Dims, cu_seqlens, q, k, v, beta, gate, state, cursor, slot_idx, out):
    """gdn_prefill with the tensors checked and marshalled once (for launch loops)."""
    _, args = _prefill_ptrs(d, cu_seqlens, q, k, v, beta, gate, state, cursor, slot_idx, out)
    fn, dref = _lib().rs_gdn_prefill, ctypes.byref(d)

    def call(stream=None):
        st = fn(dref, *args, _stream(stream))
        if st:
            raise RSError(st, 'rs_gdn_prefill')
    call.tensors = (cu_seqlens, q, k, v, beta, gate, state, cursor, slot_idx, out)
    return call


def _conv_common(d: ConvDims, cu_seqlens, x):
    at = _TORCH_DTYPE[d.act_dtype]
    if cu_seqlens is None:
        ntok = d.batch * d.T
        cu = None
    else:
        if x is None or x.dim() < 1:
            raise ValueError('x must be a [total_tokens, channels] tensor')
        ntok = int(x.shape[0])
        cu = _ptr(cu_seqlens, 'cu_seqlens', d.batch + 1, torch.int32)
    return at, ntok, cu


def conv_verify(d: ConvDims, x, weight, bias, conv_state, slot_idx, y, cu_seqlens=None,
                stream=None):
    """rs_conv_verify: the window's conv outputs y [tokens, C] (out dtype) from the window
    inputs x [tokens, C], weight [C, K], bias [C] or None and the conv state
    [num_slots, K-1, C]; cu_seqlens [B + 1] for ragged windows (tokens = x.shape[0])."""
    at, ntok, cu = _conv_common(d, cu_seqlens, x)
    C, K = d.channels, d.width
    args = [_ptr(x, 'x', ntok * C, at), _ptr(weight, 'weight', C * K, at),
            _ptr(bias, 'bias', C, at, optional=True),
            _ptr(conv_state, 'conv_state', d.num_slots * (K - 1) * C, at),
            _ptr(slot_idx, 'slot_idx', d.batch, torch.int32),
            _ptr(y, 'y', ntok * C, _TORCH_DTYPE[d.out_dtype])]
    _check(_lib().rs_conv_verify(ctypes.byref(d), cu, ctypes.c_int32(ntok), *args,
                                 _stream(stream)), 'rs_conv_verify')


def conv_commit(d: ConvDims, conv_state, x, slot_idx, accept_len, cu_seqlens=None, layers=1,
                stream=None):
    """rs_conv_commit: roll each live row's conv state to the K-1 inputs ending at its
    last accepted draft (x, cu_seqlens as the step's conv_verify calls received them).
    layers > 1: conv_state [layers, num_slots, K-1, C] and x [layers, tokens, C], one
    launch for all of them."""
    at, ntok, cu = _conv_common(d, cu_seqlens, None if x is None or cu_seqlens is None
                                else x.reshape(layers, -1, d.channels)[0])
    C, K = d.channels, d.width
    args = [_ptr(conv_state, 'conv_state', layers * d.num_slots * (K - 1) * C, at),
            _ptr(x, 'x', layers * ntok * C, at), _ptr(slot_idx, 'slot_idx', d.batch, torch.int32),
            _ptr(accept_len, 'accept_len', d.batch, torch.int32)]
    _check(_lib().rs_conv_commit(ctypes.byref(d), cu, ctypes.c_int32(ntok), ctypes.c_int32(layers),
                                 *args, _stream(stream)), 'rs_conv_commit')


def prepare_conv_verify(d: ConvDims, x, weight, bias, conv_state, slot_idx, y, cu_seqlens=None):
    """conv_verify with the tensors checked and marshalled once (for launch loops)."""
    at, ntok, cu = _conv_common(d, cu_seqlens, x)
    C, K = d.channels, d.width
    args = [_ptr(x, 'x', ntok * C, at), _ptr(weight, 'weight', C * K, at),
            _ptr(bias, 'bias', C, at, optional=True),
            _ptr(conv_state, 'conv_state', d.num_slots * (K - 1) * C, at),
            _ptr(slot_idx, 'slot_idx', d.batch, torch.int32),
            _ptr(y, 'y', ntok * C, _TORCH_DTYPE[d.out_dtype])]
    fn, dref, nt = _lib().rs_conv_verify, ctypes.byref(d), ctypes.c_int32(ntok)

    def call(stream=None):
        st = fn(dref, cu, nt, *args, _stream(stream))
        if st:
            raise RSError(st, 'rs_conv_verify')
    call.tensors = (x, weight, bias, conv_state, slot_idx, y, cu_seqlens)
    return call


def prepare_conv_commit(d: ConvDims, conv_state, x, slot_idx, accept_len, layers=1):
    """conv_commit (uniform windows) with the tensors checked and marshalled once."""
    at = _TORCH_DTYPE[d.act_dtype]
    C, K, ntok = d.channels, d.width, d.batch * d.T
    args = [_ptr(conv_state, 'conv_state', layers * d.num_slots * (K - 1) * C, at),
            _ptr(x, 'x', layers * ntok * C, at), _ptr(slot_idx, 'slot_idx', d.batch, torch.int32),
            _ptr(accept_len, 'accept_len', d.batch, torch.int32)]
    fn, dref = _lib().rs_conv_commit, ctypes.byref(d)

    def call(stream=None):
        st = fn(dref, None, ctypes.c_int32(ntok), ctypes.c_int32(layers), *args, _stream(stream))
        if st:
            raise RSError(st, 'rs_conv_commit')
    call.tensors = (conv_state, x, slot_idx, accept_len)
    return call


def verify_launch_info(d: Dims, kda: bool = False):
    """(tile_v, workgroups, lds_bytes) the verify launches with for these dims."""
    tv, wg, lds = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    _check(_lib().rs_verify_launch_info(ctypes.byref(d), int(kda), ctypes.byref(tv),
                                        ctypes.byref(wg), ctypes.byref(lds)),
           'rs_verify_launch_info')
    return tv.value, wg.value, lds.value


def stream_read(src: torch.Tensor, sink: torch.Tensor, stream=None):
    """Measurement aid: stream all of src (a contiguous GPU tensor) with the verify's load
    instructions; sink is a float32 GPU tensor of 256 elements the kernel may write."""
    if not src.is_cuda or not src.is_contiguous():
        raise ValueError('src must be a contiguous GPU tensor')
    nbytes = src.numel() * src.element_size()
    _check(_lib().rs_stream_read(ctypes.c_void_p(src.data_ptr()), ctypes.c_uint64(nbytes),
                                 _ptr(sink, 'sink', 256, torch.float32), _stream(stream)),
           'rs_stream_read')


# ----------------------------------------------------------------------------- prepared calls
# For launch loops: the tensors are checked and their pointers marshalled once; each call
# of the returned function is then a single C call on the given stream.  The returned
# function holds references to its tensors, so their memory stays allocated while it lives.

def prepare_verify(kda: bool, d: Dims, q, k, v, beta, gate, state, ring_k, ring_d, ring_g,
                   cursor, slot_idx, out, write_pos_out=None, group_counter=None):
    args = _verify_ptrs(kda, d, q, k, v, beta, gate, state, ring_k, ring_d, ring_g, cursor,
                        slot_idx, out, write_pos_out, group_counter)
    fn = _lib().rs_kda_verify if kda else _lib().rs_gdn_verify
    dref = ctypes.byref(d)
    name = 'rs_kda_verify' if kda else 'rs_gdn_verify'

    def call(stream=None):
        st = fn(dref, *args, _stream(stream))
        if st:
            raise RSError(st, name)
    call.dims = d
    call.tensors = (q, k, v, beta, gate, state, ring_k, ring_d, ring_g, cursor, slot_idx, out,
                    write_pos_out, group_counter)
    return call


def prepare_cursor_advance(d: Dims, cursor, fold_len, slot_idx, accept_len,
                           policy: int = FOLD_NONE, next_T: int = 0, force_mask=None):
    args = [_ptr(cursor, 'cursor', d.num_slots, torch.int32),
            _ptr(fold_len, 'fold_len', d.num_slots, torch.int32),
            _ptr(slot_idx, 'slot_idx', d.batch, torch.int32),
            _ptr(accept_len, 'accept_len', d.batch, torch.int32)]
    fm = _ptr(force_mask, 'force_mask', d.batch, torch.uint8, optional=True)
    fn, dref = _lib().rs_cursor_advance, ctypes.byref(d)

    def call(stream=None):
        st = fn(dref, *args, int(policy), int(next_T), fm, _stream(stream))
        if st:
            raise RSError(st, 'rs_cursor_advance')
    call.tensors = (cursor, fold_len, slot_idx, accept_len, force_mask)
    return call


def prepare_commit_fold(d: Dims, kda: bool, state, ring_k, ring_d, ring_g, fold_len, slot_idx):
    p = _fold_ptrs(d, kda, state, ring_k, ring_d, ring_g)
    rest = [_ptr(fold_len, 'fold_len', d.num_slots, torch.int32),
            _ptr(slot_idx, 'slot_idx', d.batch, torch.int32)]
    fn, dref = _lib().rs_commit_fold, ctypes.byref(d)

    def call(stream=None):
        st = fn(dref, int(kda), *p, *rest, _stream(stream))
        if st:
            raise RSError(st, 'rs_commit_fold')
    call.tensors = (state, ring_k, ring_d, ring_g, fold_len, slot_idx)
    return call


def prepare_verify_varlen(kda: bool, d: Dims, cu_seqlens, q, k, v, beta, gate, state, ring_k,
                          ring_d, ring_g, cursor, slot_idx, out, write_pos_out=None,
                          group_counter=None):
    ntok = _ntok(q)
    args = _verify_ptrs(kda, d, q, k, v, beta, gate, state, ring_k, ring_d, ring_g, cursor,
                        slot_idx, out, write_pos_out, group_counter, ntok)
    cu = _ptr(cu_seqlens, 'cu_seqlens', d.batch + 1, torch.int32)
    name = 'rs_kda_verify_varlen' if kda else 'rs_gdn_verify_varlen'
    fn, dref, nt = getattr(_lib(), name), ctypes.byref(d), ctypes.c_int32(ntok)

    def call(stream=None):
        st = fn(dref, cu, nt, *args, _stream(stream))
        if st:
            raise RSError(st, name)
    call.dims = d
    call.tensors = (cu_seqlens, q, k, v, beta, gate, state, ring_k, ring_d, ring_g, cursor,
                    slot_idx, out, write_pos_out, group_counter)
    return call


def prepare_cursor_advance_varlen(d: Dims, cu_seqlens, total_tokens: int, cursor, fold_len,
                                  slot_idx, accept_len, policy: int = FOLD_NONE,
                                  next_T: int = 0, force_mask=None):
    args = [_ptr(cu_seqlens, 'cu_seqlens', d.batch + 1, torch.int32),
            ctypes.c_int32(int(total_tokens)),
            _ptr(cursor, 'cursor', d.num_slots, torch.int32),
            _ptr(fold_len, 'fold_len', d.num_slots, torch.int32),
            _ptr(slot_idx, 'slot_idx', d.batch, torch.int32),
            _ptr(accept_len, 'accept_len', d.batch, torch.int32)]
    fm = _ptr(force_mask, 'force_mask', d.batch, torch.uint8, optional=True)
    fn, dref = _lib().rs_cursor_advance_varlen, ctypes.byref(d)

    def call(stream=None):
        st = fn(dref, *args, int(policy), int(next_T), fm, _stream(stream))
        if st:
            raise RSError(st, 'rs_cursor_advance_varlen')
    call.tensors = (cu_seqlens, cursor, fold_len, slot_idx, accept_len, force_mask)
    return call
