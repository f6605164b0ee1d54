"""Thin ctypes binding of libssd.so (declared in include/ssd.h).

Argument marshalling only: torch tensors provide device memory and the current
HIP stream; every step of the scan runs in the library's HIP kernels. There is
no fallback: if libssd.so is missing or fails to load, every call raises.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libssd.so")

SSD_F32, SSD_BF16 = 0, 1
DATA_BAD_CU_SEQLENS, DATA_TOO_MANY_CHUNKS, DATA_BAD_SLOT, DATA_BAD_BLOCK = 1, 2, 4, 8

# names exported by libssd.so (checked by the CPU tests against include/ssd.h)
EXPORTS = ("ssd_varlen_metadata", "ssd_chunk_scan_varlen", "ssd_export_chunk_states",
           "ssd_decode_step", "ssd_causal_conv1d_varlen", "ssd_gated_delta_chunk_varlen", "ssd_gated_delta_workspace_size",
           "ssd_gated_delta_chunk_varlen_noalloc",
           "ssd_prefill_bites",
           "ssd_status_string")


class SSDError(RuntimeError):
    """A libssd call returned a non-zero ssd_status."""

    def __init__(self, fn, status, text):
        super().__init__(f"{fn} failed: status {status} ({text})")
        self.status = status


class _Meta(ctypes.Structure):
    _fields_ = [("nseqs", ctypes.c_int32), ("total_tokens", ctypes.c_int32),
                ("chunk_size", ctypes.c_int32), ("max_chunks", ctypes.c_int32),
                ("cu_seqlens", ctypes.c_void_p), ("chunk_offsets", ctypes.c_void_p),
                ("chunk_seq_idx", ctypes.c_void_p), ("seq_chunk_start", ctypes.c_void_p),
                ("nchunks", ctypes.c_void_p), ("seq_order", ctypes.c_void_p),
                ("error_flag", ctypes.c_void_p)]


_lib = None


def load_library(path: str = LIB_PATH):
    """Load libssd.so (once). Raises if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"libssd.so not found at {path}: build it with "
                           "`python -c 'import __graft_entry__ as g; g.build()'`")
    lib = ctypes.CDLL(path)
    vp, i32, st = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int
    lib.ssd_status_string.restype = ctypes.c_char_p
    lib.ssd_status_string.argtypes = [st]
    lib.ssd_varlen_metadata.restype = st
    lib.ssd_varlen_metadata.argtypes = [ctypes.POINTER(_Meta), vp]
    lib.ssd_chunk_scan_varlen.restype = st
    lib.ssd_chunk_scan_varlen.argtypes = [vp, vp, vp, vp, vp, vp, vp, st, ctypes.POINTER(_Meta),
                                          i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, i32, vp]
    lib.ssd_export_chunk_states.restype = st
    lib.ssd_export_chunk_states.argtypes = [ctypes.POINTER(_Meta), vp, vp, i32, i32, vp, vp, vp,
                                            i32, vp, i32, vp]
    lib.ssd_decode_step.restype = st
    lib.ssd_decode_step.argtypes = [vp, vp, vp, vp, vp, vp, vp, st, i32, i32, i32, i32, i32, vp, i32,
                                    vp, vp, vp, vp, vp]
    lib.ssd_causal_conv1d_varlen.restype = st
    lib.ssd_causal_conv1d_varlen.argtypes = [vp, vp, vp, st, ctypes.POINTER(_Meta), i32, i32, i32, vp, i32,
                                             vp, vp, vp, vp]
    lib.ssd_gated_delta_chunk_varlen.restype = st
    lib.ssd_gated_delta_chunk_varlen.argtypes = [vp, vp, vp, vp, vp, ctypes.c_float, st, ctypes.POINTER(_Meta),
                                                 i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, i32, vp,
                                                 ctypes.c_size_t, vp]
    lib.ssd_gated_delta_chunk_varlen_noalloc.restype = st
    lib.ssd_gated_delta_chunk_varlen_noalloc.argtypes = [vp, vp, vp, vp, vp, ctypes.c_float, st,
                                                         ctypes.POINTER(_Meta), i32, i32, i32, i32, vp, vp, vp, vp,
                                                         vp, vp, i32, vp]
    lib.ssd_gated_delta_workspace_size.restype = ctypes.c_size_t
    lib.ssd_gated_delta_workspace_size.argtypes = [i32, i32]
    lib.ssd_prefill_bites.restype = st
    lib.ssd_prefill_bites.argtypes = [i32, vp, vp, vp, i32, vp]
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load_library().ssd_status_string(status).decode()


def _check(fn, status):
    if status != 0:
        raise SSDError(fn, status, status_string(status))


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _data(t: torch.Tensor, name: str, device, dtype=None):
    """Data tensors must already be contiguous and on the device (no hidden copies)."""
    if t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    return t


def _shape(t: Optional[torch.Tensor], name: str, *shape):
    """The kernels index every buffer from the sizes passed beside it: a tensor of
    another shape would be read or written out of its bounds, so refuse it here."""
    if t is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _dst_len(dst: Optional[torch.Tensor], meta):
    """The kernels read one checkpoint slot per chunk of the batch's chunk grid."""
    if dst is not None and dst.numel() < meta.max_chunks:
        raise ValueError(f"chunk_state_dst needs {meta.max_chunks} entries (one per chunk), got {dst.numel()}")


def _index(t: torch.Tensor, device):
    """Index arrays are normalised to contiguous int32 on the device."""
    t = t.to(device=device, dtype=torch.int32)
    return t if t.stride(-1) == 1 and t.is_contiguous() else t.contiguous()


@dataclasses.dataclass
class VarlenMeta:
    """Device-resident chunk metadata of one packed batch (see ssd_varlen_meta)."""
    nseqs: int
    total_tokens: int
    chunk_size: int
    max_chunks: int
    cu_seqlens: torch.Tensor
    chunk_offsets: torch.Tensor
    chunk_seq_idx: torch.Tensor
    seq_chunk_start: torch.Tensor
    nchunks: torch.Tensor
    seq_order: torch.Tensor
    error_flag: torch.Tensor

    def c_struct(self) -> _Meta:
        return _Meta(self.nseqs, self.total_tokens, self.chunk_size, self.max_chunks,
                     *(t.data_ptr() for t in (self.cu_seqlens, self.chunk_offsets,
                                              self.chunk_seq_idx, self.seq_chunk_start,
                                              self.nchunks, self.seq_order, self.error_flag)))


def varlen_metadata(cu_seqlens: torch.Tensor, chunk_size: int, total_tokens: Optional[int] = None,
                    max_chunks: Optional[int] = None, device=None) -> VarlenMeta:
    """ssd_varlen_metadata: build the chunk grid on the device (no host sync).

    `total_tokens` defaults to cu_seqlens[-1] (read on the host if cu_seqlens is a
    CPU tensor; pass it explicitly for device-resident cu_seqlens)."""
    lib = load_library()
    device = torch.device(device) if device is not None else (
        cu_seqlens.device if cu_seqlens.is_cuda else torch.device("cuda", torch.cuda.current_device()))
    S = cu_seqlens.numel() - 1
    if total_tokens is None:
        if cu_seqlens.is_cuda:
            raise ValueError("pass total_tokens when cu_seqlens lives on the device")
        total_tokens = int(cu_seqlens[-1])
    if max_chunks is None:
        max_chunks = total_tokens // chunk_size + S
    cu = _index(cu_seqlens, device)
    i32 = dict(dtype=torch.int32, device=device)
    meta = VarlenMeta(S, int(total_tokens), int(chunk_size), int(max_chunks), cu,
                      torch.empty(max_chunks + 1, **i32), torch.empty(max(max_chunks, 1), **i32),
                      torch.empty(S + 1, **i32), torch.empty(1, **i32),
                      torch.empty(max(S, 1), **i32), torch.zeros(1, **i32))
    c = meta.c_struct()
    _check("ssd_varlen_metadata", lib.ssd_varlen_metadata(ctypes.byref(c), _stream(device)))
    return meta


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return SSD_BF16
    if t.dtype == torch.float32:
        return SSD_F32
    raise ValueError(f"x/B/C must be float32 or bfloat16, got {t.dtype}")


def chunk_scan_varlen(x: torch.Tensor, dt: torch.Tensor, A: torch.Tensor, B: torch.Tensor,
                      C: torch.Tensor, meta: VarlenMeta, dt_bias: Optional[torch.Tensor] = None,
                      D: Optional[torch.Tensor] = None,
                      initial_states: Optional[torch.Tensor] = None,
                      has_initial_state: Optional[torch.Tensor] = None,
                      y: Optional[torch.Tensor] = None,
                      final_states: Optional[torch.Tensor] = None,
                      chunk_states: Optional[torch.Tensor] = None,
                      chunk_state_dst: Optional[torch.Tensor] = None):
    """ssd_chunk_scan_varlen. x (T,H,P), dt (T,H), A (H,), B/C (T,G,N).

    Returns (y, final_states). `chunk_states` (float32 [slots,H,P,N]) receives the
    state after each chunk, at index c or at chunk_state_dst[c] when given."""
    lib = load_library()
    device = x.device
    T, H, P = x.shape
    G, N = B.shape[1], B.shape[2]
    S = meta.nseqs
    _data(x, "x", device)
    if T != meta.total_tokens:
        raise ValueError(f"x has {T} tokens, the metadata {meta.total_tokens}")
    for name, t, shp in (("B", B, (T, G, N)), ("C", C, (T, G, N)), ("dt", dt, (T, H)), ("A", A, (H,)),
                         ("dt_bias", dt_bias, (H,)), ("D", D, (H,)),
                         ("initial_states", initial_states, (S, H, P, N)), ("y", y, (T, H, P)),
                         ("final_states", final_states, (S, H, P, N))):
        _shape(t, name, *shp)
    if has_initial_state is not None:
        _shape(has_initial_state, "has_initial_state", S)
    if chunk_states is not None:
        _shape(chunk_states, "chunk_states", chunk_states.shape[0], H, P, N)
    _dst_len(chunk_state_dst, meta)
    dtype = x.dtype
    for name, t in (("B", B), ("C", C)):
        _data(t, name, device, dtype)
    _data(dt, "dt", device, torch.float32)
    _data(A, "A", device, torch.float32)
    for name, t in (("dt_bias", dt_bias), ("D", D), ("initial_states", initial_states)):
        if t is not None:
            _data(t, name, device, torch.float32)
    if y is None:
        y = torch.empty_like(x)
    _data(y, "y", device, dtype)
    if final_states is None:
        final_states = torch.empty((S, H, P, N), dtype=torch.float32, device=device)
    _data(final_states, "final_states", device, torch.float32)
    has = _index(has_initial_state, device) if has_initial_state is not None else None
    dst = _index(chunk_state_dst, device) if chunk_state_dst is not None else None
    cap = 0
    if chunk_states is not None:
        _data(chunk_states, "chunk_states", device, torch.float32)
        cap = chunk_states.shape[0]
    m = meta.c_struct()
    _check("ssd_chunk_scan_varlen", lib.ssd_chunk_scan_varlen(
        _ptr(x), _ptr(dt), _ptr(dt_bias), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _dtype_code(x),
        ctypes.byref(m), H, P, N, G, _ptr(initial_states), _ptr(has), _ptr(y),
        _ptr(final_states), _ptr(chunk_states), _ptr(dst), cap, _stream(device)))
    return y, final_states


def export_chunk_states(meta: VarlenMeta, block_table: torch.Tensor, block_size: int,
                        num_computed_tokens: Optional[torch.Tensor] = None,
                        chunk_states: Optional[torch.Tensor] = None,
                        state_cache: Optional[torch.Tensor] = None,
                        num_slots: Optional[int] = None):
    """ssd_export_chunk_states: block-checkpoint plan (and scatter when chunk_states
    is given). Returns (ckpt_src [S, max_blocks], chunk_state_dst [max_chunks])."""
    lib = load_library()
    device = meta.cu_seqlens.device
    bt = _index(block_table, device)
    S, maxb = bt.shape if bt.dim() == 2 else (meta.nseqs, 0)
    ncomp = _index(num_computed_tokens, device) if num_computed_tokens is not None else None
    ckpt_src = torch.empty((S, maxb), dtype=torch.int32, device=device)
    dst = torch.empty(max(meta.max_chunks, 1), dtype=torch.int32, device=device)
    state_elems = 0
    if state_cache is not None:
        _data(state_cache, "state_cache", device, torch.float32)
        state_elems = state_cache[0].numel() if state_cache.shape[0] else 0
        if num_slots is None:
            num_slots = state_cache.shape[0]
    if chunk_states is not None:
        _data(chunk_states, "chunk_states", device, torch.float32)
    m = meta.c_struct()
    _check("ssd_export_chunk_states", lib.ssd_export_chunk_states(
        ctypes.byref(m), _ptr(ncomp), _ptr(bt), maxb, int(block_size), _ptr(ckpt_src), _ptr(dst),
        _ptr(chunk_states), state_elems, _ptr(state_cache), int(num_slots or 0), _stream(device)))
    return ckpt_src, dst[: meta.max_chunks]


def gated_delta_chunk_varlen(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, gate: torch.Tensor,
                             beta: torch.Tensor, meta: VarlenMeta, scale: Optional[float] = None,
                             initial_states: Optional[torch.Tensor] = None,
                             has_initial_state: Optional[torch.Tensor] = None,
                             o: Optional[torch.Tensor] = None, final_states: Optional[torch.Tensor] = None,
                             chunk_states: Optional[torch.Tensor] = None,
                             chunk_state_dst: Optional[torch.Tensor] = None,
                             workspace: Optional[torch.Tensor] = None, no_alloc: bool = False):
    """ssd_gated_delta_chunk_varlen: q, k (T,G,dk), v (T,H,dv) bf16; gate, beta (T,H) float32;
    states (S,H,dv,dk) float32. `workspace` (uint8 on the device, at least
    gated_delta_workspace_size(meta, H) bytes) is allocated per call when not
    given. no_alloc=True calls ssd_gated_delta_chunk_varlen_noalloc instead (the
    library's static workspace; pass o and final_states too for a call that
    allocates nothing).
    Returns (o, final_states)."""
    lib = load_library()
    device = v.device
    T, H, DV = v.shape
    G, DK = k.shape[1], k.shape[2]
    S = meta.nseqs
    for name, t, shp in (("q", q, (T, G, DK)), ("k", k, (T, G, DK)), ("gate", gate, (T, H)), ("beta", beta, (T, H)),
                         ("o", o, (T, H, DV)), ("initial_states", initial_states, (S, H, DV, DK)),
                         ("final_states", final_states, (S, H, DV, DK)), ("has_initial_state", has_initial_state, (S,))):
        _shape(t, name, *shp)
    if chunk_states is not None:
        _shape(chunk_states, "chunk_states", chunk_states.shape[0], H, DV, DK)
    _dst_len(chunk_state_dst, meta)
    if T != meta.total_tokens:
        raise ValueError(f"v has {T} tokens, the metadata {meta.total_tokens}")
    dtype = v.dtype
    _data(v, "v", device)
    for name, t in (("q", q), ("k", k)):
        _data(t, name, device, dtype)
    for name, t in (("gate", gate), ("beta", beta)):
        _data(t, name, device, torch.float32)
    if o is None:
        o = torch.empty_like(v)
    _data(o, "o", device, dtype)
    if final_states is None:
        final_states = torch.empty((S, H, DV, DK), dtype=torch.float32, device=device)
    _data(final_states, "final_states", device, torch.float32)
    if initial_states is not None:
        _data(initial_states, "initial_states", device, torch.float32)
    has = _index(has_initial_state, device) if has_initial_state is not None else None
    cap = 0
    if chunk_states is not None:
        _data(chunk_states, "chunk_states", device, torch.float32)
        cap = chunk_states.shape[0]
    dst = _index(chunk_state_dst, device) if chunk_state_dst is not None else None
    if no_alloc:
        m = meta.c_struct()
        _check("ssd_gated_delta_chunk_varlen_noalloc", lib.ssd_gated_delta_chunk_varlen_noalloc(
            _ptr(q), _ptr(k), _ptr(v), _ptr(gate), _ptr(beta), float(scale if scale is not None else DK ** -0.5),
            _dtype_code(v), ctypes.byref(m), H, G, DK, DV, _ptr(initial_states), _ptr(has), _ptr(o),
            _ptr(final_states), _ptr(chunk_states), _ptr(dst), cap, _stream(device)))
        return o, final_states
    ws_bytes = gated_delta_workspace_size(meta, H)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=device)
    _data(workspace, "workspace", device, torch.uint8)
    m = meta.c_struct()
    _check("ssd_gated_delta_chunk_varlen", lib.ssd_gated_delta_chunk_varlen(
        _ptr(q), _ptr(k), _ptr(v), _ptr(gate), _ptr(beta), float(scale if scale is not None else DK ** -0.5),
        _dtype_code(v), ctypes.byref(m), H, G, DK, DV, _ptr(initial_states), _ptr(has), _ptr(o), _ptr(final_states),
        _ptr(chunk_states), _ptr(dst), cap, _ptr(workspace), workspace.numel(), _stream(device)))
    return o, final_states


def gated_delta_workspace_size(meta: VarlenMeta, nheads: int) -> int:
    """Bytes of device workspace ssd_gated_delta_chunk_varlen needs for this batch."""
    return int(load_library().ssd_gated_delta_workspace_size(meta.max_chunks, int(nheads)))


def prefill_bites(num_computed_tokens, prompt_len, budget, align: int):
    """ssd_prefill_bites (host): tokens each prefilling sequence gets this step.
    Arguments are host sequences, arrays or CPU tensors of nseqs entries (budget may
    be a single int); returns a host int32 tensor of nseqs entries."""
    lib = load_library()
    nc = torch.as_tensor(num_computed_tokens, dtype=torch.int32).reshape(-1).contiguous()
    pl = torch.as_tensor(prompt_len, dtype=torch.int32).reshape(-1).contiguous()
    bu = torch.as_tensor(budget, dtype=torch.int32).reshape(-1).expand(nc.numel()).contiguous()
    if pl.numel() != nc.numel():
        raise ValueError("prompt_len and num_computed_tokens differ in length")
    out = torch.empty_like(nc)
    _check("ssd_prefill_bites", lib.ssd_prefill_bites(nc.numel(), nc.data_ptr(), pl.data_ptr(), bu.data_ptr(),
                                                     int(align), out.data_ptr()))
    return out


def decode_step(x: torch.Tensor, dt: torch.Tensor, A: torch.Tensor, B: torch.Tensor,
                C: torch.Tensor, state_cache: torch.Tensor, read_slot: torch.Tensor,
                write_slot: torch.Tensor, dt_bias: Optional[torch.Tensor] = None,
                D: Optional[torch.Tensor] = None, y: Optional[torch.Tensor] = None,
                error_flag: Optional[torch.Tensor] = None):
    """ssd_decode_step: one token per sequence, state read from
    state_cache[read_slot[s]] (zero if < 0) and written to
    state_cache[write_slot[s]] (skipped if < 0). x (S,H,P), dt (S,H), A (H,),
    B/C (S,G,N), state_cache float32 (slots,H,P,N). Returns y (S,H,P)."""
    lib = load_library()
    device = x.device
    S, H, P = x.shape
    G, N = B.shape[1], B.shape[2]
    _data(x, "x", device)
    for name, t, shp in (("B", B, (S, G, N)), ("C", C, (S, G, N)), ("dt", dt, (S, H)), ("A", A, (H,)),
                         ("dt_bias", dt_bias, (H,)), ("D", D, (H,)), ("y", y, (S, H, P)),
                         ("state_cache", state_cache, (state_cache.shape[0], H, P, N)),
                         ("read_slot", read_slot, (S,)), ("write_slot", write_slot, (S,))):
        _shape(t, name, *shp)
    dtype = x.dtype
    for name, t in (("B", B), ("C", C)):
        _data(t, name, device, dtype)
    _data(dt, "dt", device, torch.float32)
    _data(A, "A", device, torch.float32)
    _data(state_cache, "state_cache", device, torch.float32)
    for name, t in (("dt_bias", dt_bias), ("D", D)):
        if t is not None:
            _data(t, name, device, torch.float32)
    if y is None:
        y = torch.empty_like(x)
    _data(y, "y", device, dtype)
    rs, ws = _index(read_slot, device), _index(write_slot, device)
    if error_flag is not None:
        _data(error_flag, "error_flag", device, torch.int32)
    _check("ssd_decode_step", lib.ssd_decode_step(
        _ptr(x), _ptr(dt), _ptr(dt_bias), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _dtype_code(x),
        S, H, P, N, G, _ptr(state_cache), state_cache.shape[0], _ptr(rs), _ptr(ws), _ptr(y),
        _ptr(error_flag), _stream(device)))
    return y


def causal_conv1d_varlen(x: torch.Tensor, weight: torch.Tensor, meta: VarlenMeta,
                         bias: Optional[torch.Tensor] = None, silu: bool = True,
                         conv_states: Optional[torch.Tensor] = None,
                         read_slot: Optional[torch.Tensor] = None,
                         write_slot: Optional[torch.Tensor] = None,
                         out: Optional[torch.Tensor] = None):
    """ssd_causal_conv1d_varlen: depthwise causal conv1d of x (T, C) with
    weight (C, W) float32 over the chunk grid of `meta`; the W-1 inputs before
    each sequence come from conv_states[read_slot[s]] (zero if < 0) and its last
    W-1 inputs go to conv_states[write_slot[s]] (skipped if < 0); conv_states
    (slots, W-1, C) has x's dtype. Returns out (T, C)."""
    lib = load_library()
    device = x.device
    _data(x, "x", device)
    T, C = x.shape
    W = weight.shape[1]
    if T != meta.total_tokens:
        raise ValueError(f"x has {T} tokens, the metadata {meta.total_tokens}")
    S = meta.nseqs
    for name, t, shp in (("weight", weight, (C, W)), ("bias", bias, (C,)), ("out", out, (T, C)),
                         ("read_slot", read_slot, (S,)), ("write_slot", write_slot, (S,))):
        _shape(t, name, *shp)
    if conv_states is not None:
        _shape(conv_states, "conv_states", conv_states.shape[0], W - 1, C)
    _data(weight, "weight", device, torch.float32)
    if bias is not None:
        _data(bias, "bias", device, torch.float32)
    if conv_states is not None:
        _data(conv_states, "conv_states", device, x.dtype)
    if out is None:
        out = torch.empty_like(x)
    _data(out, "out", device, x.dtype)
    rs = _index(read_slot, device) if read_slot is not None else None
    ws = _index(write_slot, device) if write_slot is not None else None
    m = meta.c_struct()
    _check("ssd_causal_conv1d_varlen", lib.ssd_causal_conv1d_varlen(
        _ptr(x), _ptr(weight), _ptr(bias), _dtype_code(x), ctypes.byref(m), C, W, int(bool(silu)),
        _ptr(conv_states), 0 if conv_states is None else conv_states.shape[0], _ptr(rs), _ptr(ws),
        _ptr(out), _stream(device)))
    return out
