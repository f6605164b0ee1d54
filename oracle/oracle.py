"""ctypes wrapper over liboracle.so (float64 CPU reference; test infrastructure).

Inputs are widened to float64 here (bfloat16 and float32 widen exactly), so the
oracle sees exactly the values the GPU sees.
"""
import ctypes
import os

import numpy as np

from .build import LIB, build_oracle

_I32P = ctypes.POINTER(ctypes.c_int32)
_F64P = ctypes.POINTER(ctypes.c_double)
_cache = {}


def load(path=LIB):
    """Load (building if absent) the oracle library at `path`."""
    if path in _cache:
        return _cache[path]
    if not os.path.exists(path):
        if path != LIB:
            raise FileNotFoundError(path)
        build_oracle()
    lib = ctypes.CDLL(path)
    lib.oracle_ssd_varlen.restype = ctypes.c_int
    lib.oracle_ssd_varlen.argtypes = [
        ctypes.c_int32, _I32P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
        _F64P, _F64P, _F64P, _F64P, _F64P, _F64P, _F64P, _F64P, _I32P, ctypes.c_int32, _F64P,
        _F64P, _F64P, ctypes.c_int32]
    lib.oracle_varlen_metadata.restype = ctypes.c_int
    lib.oracle_varlen_metadata.argtypes = [ctypes.c_int32, _I32P, ctypes.c_int32, ctypes.c_int32,
                                           _I32P, _I32P, _I32P, _I32P, _I32P]
    lib.oracle_checkpoint_plan.restype = ctypes.c_int
    lib.oracle_checkpoint_plan.argtypes = [ctypes.c_int32, _I32P, _I32P, ctypes.c_int32, _I32P,
                                           _I32P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                           _I32P, _I32P]
    lib.oracle_ssd_decode.restype = ctypes.c_int
    lib.oracle_ssd_decode.argtypes = [
        ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
        _F64P, _F64P, _F64P, _F64P, _F64P, _F64P, _F64P, _F64P, ctypes.c_int32, _I32P, _I32P, _F64P]
    lib.oracle_causal_conv1d.argtypes = [
        ctypes.c_int32, _I32P, ctypes.c_int32, ctypes.c_int32, _F64P, _F64P, _F64P, ctypes.c_int32,
        _F64P, ctypes.c_int32, _I32P, _I32P, _F64P]
    lib.oracle_gated_delta.restype = ctypes.c_int
    lib.oracle_gated_delta.argtypes = [
        ctypes.c_int32, _I32P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
        _F64P, _F64P, _F64P, _F64P, _F64P, ctypes.c_double, _F64P, _I32P, ctypes.c_int32, _F64P, _F64P, _F64P]
    lib.oracle_prefill_bites.restype = ctypes.c_int
    lib.oracle_prefill_bites.argtypes = [ctypes.c_int32, _I32P, _I32P, _I32P, ctypes.c_int32, _I32P]
    lib.oracle_num_threads.restype = ctypes.c_int
    _cache[path] = lib
    return lib


def _np(a, dtype):
    if a is None:
        return None
    if hasattr(a, "detach"):          # torch tensor (any float dtype) -> numpy
        a = a.detach().cpu()
        a = a.double().numpy() if dtype == np.float64 else a.numpy()
    return np.ascontiguousarray(np.asarray(a, dtype=dtype))


def _p(a, ptype):
    return None if a is None else a.ctypes.data_as(ptype)


def num_threads(lib=None):
    return (lib or load()).oracle_num_threads()


def ssd_varlen(x, dt, dt_bias, A, B, C, D, cu_seqlens, initial_states=None, has_initial_state=None,
               chunk_size=0, nthreads=0, lib=None):
    """Token-by-token float64 recurrence. Returns (y, final_states, chunk_states|None)."""
    lib = lib or load()
    x, dt, B, C = (_np(v, np.float64) for v in (x, dt, B, C))
    dt_bias, A, D, init = (_np(v, np.float64) for v in (dt_bias, A, D, initial_states))
    cu = _np(cu_seqlens, np.int32)
    has = _np(has_initial_state, np.int32)
    T, H, P = x.shape
    G, N = B.shape[1], B.shape[2]
    S = cu.shape[0] - 1
    y = np.empty((T, H, P), np.float64)
    final = np.empty((S, H, P, N), np.float64)
    chunk_states = None
    if chunk_size:
        lens = np.diff(cu.astype(np.int64))
        nch = int(((lens + chunk_size - 1) // chunk_size).sum())
        chunk_states = np.full((nch, H, P, N), np.nan, np.float64)
    rc = lib.oracle_ssd_varlen(S, _p(cu, _I32P), H, P, N, G, _p(x, _F64P), _p(dt, _F64P),
                               _p(dt_bias, _F64P), _p(A, _F64P), _p(B, _F64P), _p(C, _F64P),
                               _p(D, _F64P), _p(init, _F64P), _p(has, _I32P), int(chunk_size),
                               _p(chunk_states, _F64P), _p(y, _F64P), _p(final, _F64P),
                               int(nthreads))
    if rc != 0:
        raise ValueError(f"oracle_ssd_varlen failed ({rc})")
    return y, final, chunk_states


def varlen_metadata(cu_seqlens, chunk_size, max_chunks, lib=None):
    """Chunk grid by enumeration: dict of int32 arrays + nchunks."""
    lib = lib or load()
    cu = _np(cu_seqlens, np.int32)
    S = cu.shape[0] - 1
    off = np.empty(max_chunks + 1, np.int32)
    sidx = np.empty(max_chunks, np.int32)
    start = np.empty(S + 1, np.int32)
    order = np.empty(max(S, 1), np.int32)
    n = np.zeros(1, np.int32)
    rc = lib.oracle_varlen_metadata(S, _p(cu, _I32P), int(chunk_size), int(max_chunks),
                                    _p(off, _I32P), _p(sidx, _I32P), _p(start, _I32P),
                                    _p(n, _I32P), _p(order, _I32P))
    if rc != 0:
        raise ValueError(f"oracle_varlen_metadata failed ({rc})")
    return dict(chunk_offsets=off, chunk_seq_idx=sidx, seq_chunk_start=start,
                nchunks=int(n[0]), seq_order=order[:S])


def checkpoint_plan(cu_seqlens, seq_chunk_start, max_chunks, block_table, block_size, chunk_size,
                    num_computed_tokens=None, lib=None):
    """Block-checkpoint plan: (ckpt_src [S,max_blocks], chunk_state_dst [max_chunks])."""
    lib = lib or load()
    cu = _np(cu_seqlens, np.int32)
    start = _np(seq_chunk_start, np.int32)
    bt = _np(block_table, np.int32)
    ncomp = _np(num_computed_tokens, np.int32)
    S, maxb = bt.shape
    src = np.empty((S, maxb), np.int32)
    dst = np.empty(max_chunks, np.int32)
    rc = lib.oracle_checkpoint_plan(S, _p(cu, _I32P), _p(start, _I32P), int(max_chunks),
                                    _p(ncomp, _I32P), _p(bt, _I32P), maxb, int(block_size),
                                    int(chunk_size), _p(src, _I32P), _p(dst, _I32P))
    if rc != 0:
        raise ValueError(f"oracle_checkpoint_plan failed ({rc})")
    return src, dst


def gated_delta(q, k, v, gate, beta, cu_seqlens, scale, initial_states=None, has_initial_state=None,
                chunk_size=0, lib=None):
    """Token-by-token float64 gated delta rule. q, k (T,G,dk); v (T,H,dv); gate, beta (T,H);
    states value-major (S,H,dv,dk). Returns (o, final_states, chunk_states|None)."""
    lib = lib or load()
    q, k, v = _np(q, np.float64), _np(k, np.float64), _np(v, np.float64)
    gate, beta = _np(gate, np.float64), _np(beta, np.float64)
    cu = _np(cu_seqlens, np.int32)
    T, G, dk = q.shape
    H, dv = v.shape[1], v.shape[2]
    S = cu.size - 1
    init = _np(initial_states, np.float64)
    has = _np(has_initial_state, np.int32)
    o = np.zeros((T, H, dv))
    fin = np.zeros((S, H, dv, dk))
    nch = sum((int(cu[i + 1] - cu[i]) + chunk_size - 1) // chunk_size for i in range(S)) if chunk_size else 0
    cst = np.zeros((nch, H, dv, dk)) if chunk_size else None
    rc = lib.oracle_gated_delta(S, _p(cu, _I32P), H, G, dk, dv, _p(q, _F64P), _p(k, _F64P), _p(v, _F64P),
                                _p(gate, _F64P), _p(beta, _F64P), float(scale), _p(init, _F64P), _p(has, _I32P),
                                int(chunk_size), _p(o, _F64P), _p(fin, _F64P), _p(cst, _F64P))
    if rc != 0:
        raise ValueError(f"oracle_gated_delta failed ({rc})")
    return o, fin, cst


def prefill_bites(num_computed_tokens, prompt_len, budget, align, lib=None):
    """Tokens the scheduler gives each sequence this step (the re-alignment rule)."""
    lib = lib or load()
    nc = _np(num_computed_tokens, np.int32)
    pl = _np(prompt_len, np.int32)
    bu = _np(np.broadcast_to(np.asarray(budget, np.int32), nc.shape), np.int32)
    out = np.empty(nc.shape, np.int32)
    rc = lib.oracle_prefill_bites(nc.size, _p(nc, _I32P), _p(pl, _I32P), _p(bu, _I32P), int(align),
                                  _p(out, _I32P))
    if rc != 0:
        raise ValueError(f"oracle_prefill_bites failed ({rc})")
    return out


def prefill_schedule(start, prompt_len, budget, align, lib=None):
    """The whole bite sequence of one prompt from `start`: [(first, last + 1), ...]."""
    bites = []
    while start < prompt_len:
        n = int(prefill_bites([start], [prompt_len], budget, align, lib=lib)[0])
        if n <= 0:
            raise ValueError("no progress")
        bites.append((start, start + n))
        start += n
    return bites


def ssd_decode(x, dt, dt_bias, A, B, C, D, state_cache, read_slot, write_slot, lib=None):
    """One decode token per sequence with dual state anchors (float64).
    x (S,H,P), dt (S,H), B, C (S,G,N), state_cache (slots,H,P,N); read_slot /
    write_slot (S,) int, < 0 meaning zero state / no write.
    Returns (y (S,H,P), updated copy of the cache, status: 0, or -2 if a slot
    was out of range and its sequence skipped)."""
    lib = lib or load()
    x, dt, B, C = (_np(v, np.float64) for v in (x, dt, B, C))
    dt_bias, A, D = (_np(v, np.float64) for v in (dt_bias, A, D))
    cache = _np(state_cache, np.float64).copy()
    rs, ws = _np(read_slot, np.int32), _np(write_slot, np.int32)
    S, H, P = x.shape
    G, N = B.shape[1], B.shape[2]
    y = np.zeros((S, H, P), np.float64)
    rc = lib.oracle_ssd_decode(S, H, P, N, G, _p(x, _F64P), _p(dt, _F64P), _p(dt_bias, _F64P),
                               _p(A, _F64P), _p(B, _F64P), _p(C, _F64P), _p(D, _F64P),
                               _p(cache, _F64P), cache.shape[0], _p(rs, _I32P), _p(ws, _I32P),
                               _p(y, _F64P))
    if rc == -1:
        raise ValueError("oracle_ssd_decode: bad shapes")
    return y, cache, rc


def causal_conv1d(x, cu_seqlens, weight, bias, silu, conv_states, read_slot, write_slot, lib=None):
    """Varlen causal conv1d with a conv-state cache (float64).
    x (T, C); weight (C, W); bias (C,) or None; conv_states (slots, W-1, C);
    read_slot / write_slot (S,) int, < 0 meaning zero leading inputs / no write.
    Returns (out (T, C), updated copy of conv_states, status: 0, or -2 if a slot
    was out of range and its sequence skipped)."""
    lib = lib or load()
    x, weight = _np(x, np.float64), _np(weight, np.float64)
    bias = None if bias is None else _np(bias, np.float64)
    states = _np(conv_states, np.float64).copy()
    cu = _np(cu_seqlens, np.int32)
    rs, ws = _np(read_slot, np.int32), _np(write_slot, np.int32)
    T, C = x.shape
    W = weight.shape[1]
    out = np.zeros((T, C), np.float64)
    rc = lib.oracle_causal_conv1d(len(cu) - 1, _p(cu, _I32P), C, W, _p(x, _F64P), _p(weight, _F64P),
                                  _p(bias, _F64P), int(bool(silu)), _p(states, _F64P), states.shape[0],
                                  _p(rs, _I32P), _p(ws, _I32P), _p(out, _F64P))
    if rc == -1:
        raise ValueError("oracle_causal_conv1d: bad shapes")
    return out, states, rc
