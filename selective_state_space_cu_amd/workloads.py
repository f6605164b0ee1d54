"""Seeded synthetic inputs for the varlen SSD scan.

This module only draws random numbers and casts them to storage dtypes; it holds
none of the scan's arithmetic. It is the one module that both the CPU oracle
(through the tests and the bench's CPU baseline) and the HIP library's callers
use, so both sides always see bit-identical inputs.

Distributions (per the workload statements of the Mamba2 SSD varlen problem):
  x ~ N(0,1) (T,H,P); raw dt ~ N(0,1) (T,H); dt_bias ~ U(-4,-2) per head;
  A = -exp(U(log 1, log 16)) per head; B, C ~ N(0,1)/sqrt(N) (T,G,N);
  D ~ N(0,1) per head; initial states ~ N(0, 0.5^2) (S,H,P,N).
Draw order from numpy.default_rng(seed): lengths (only for the drawn-length
workloads) -> x -> dt -> dt_bias -> A -> B -> C -> D -> init -> block table.
Everything is drawn in float64, then rounded to float32 (RNE) and, for the bf16
workloads, x/B/C are further rounded float32 -> bfloat16 (RNE).
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np
import torch

# Sequence lengths of the drawn-length workloads. They are what
# default_rng(seed).integers(lo, hi+1, n), redrawn until |sum - 16384| <= 1024,
# yields for the stated seeds; the constants win if numpy's stream ever changes.
_LEN_MAMBA2_PREFILL = [3514, 1449, 903, 1582, 1995, 3430, 2129, 841]
_LEN_CONT_BATCH = [312, 339, 267, 477, 476, 107, 312, 323, 127, 153, 250, 380, 150, 370, 335, 112,
                   199, 425, 432, 337, 3, 350, 116, 420, 468, 220, 490, 389, 167, 450, 197, 53,
                   304, 436, 337, 202, 462, 246, 198, 75, 109, 358, 410, 150, 322, 447, 76, 141,
                   269, 288, 204, 205, 67, 314, 477, 101, 409, 93, 23, 383, 93, 386, 170, 291]

# The five workloads. `len_draw` = (n, lo, hi) marks drawn lengths.
CONFIGS = {
    0: dict(name="tiny_fp32", lengths=[17, 64, 47], nheads=4, headdim=16, dstate=16, ngroups=1,
            chunk_size=16, dtype="f32", init_seqs=[0, 2]),
    1: dict(name="single_prompt_768_fp32", lengths=[768], nheads=8, headdim=64, dstate=64, ngroups=1,
            chunk_size=128, dtype="f32", init_seqs=[0], alt_chunk_sizes=[32, 256]),
    2: dict(name="mamba2_2p7b_prefill_layer", lengths=_LEN_MAMBA2_PREFILL, len_draw=(8, 512, 4096),
            nheads=80, headdim=64, dstate=128, ngroups=1, chunk_size=256, dtype="bf16",
            init_seqs=[0, 2, 4, 6]),
    3: dict(name="continuous_batching_mix", lengths=_LEN_CONT_BATCH, len_draw=(64, 1, 512),
            nheads=128, headdim=64, dstate=128, ngroups=8, chunk_size=256, dtype="bf16",
            init_seqs=list(range(64))),
    4: dict(name="prefix_cache_checkpoint_4x8894", lengths=[8894] * 4, nheads=32, headdim=128,
            dstate=128, ngroups=4, chunk_size=64, dtype="bf16", init_seqs=[],
            block_size=256, num_slots=140, resume_token=6912),
}


@dataclasses.dataclass
class Workload:
    """One batch of packed varlen inputs (torch CPU tensors in storage dtypes)."""
    lengths: list
    cu_seqlens: torch.Tensor      # int32 [S+1]
    x: torch.Tensor               # (T,H,P) float32 or bfloat16
    dt: torch.Tensor              # (T,H) float32
    dt_bias: torch.Tensor         # (H,) float32
    A: torch.Tensor               # (H,) float32
    B: torch.Tensor               # (T,G,N) like x
    C: torch.Tensor               # (T,G,N) like x
    D: torch.Tensor               # (H,) float32
    initial_states: torch.Tensor  # (S,H,P,N) float32
    has_initial_state: torch.Tensor  # int32 [S]
    chunk_size: int
    dtype: str
    block_table: Optional[torch.Tensor] = None   # int32 [S, max_blocks]
    block_size: Optional[int] = None
    num_slots: Optional[int] = None
    name: str = ""

    @property
    def nseqs(self):
        return len(self.lengths)

    @property
    def total_tokens(self):
        return int(sum(self.lengths))

    @property
    def nheads(self):
        return self.x.shape[1]

    @property
    def headdim(self):
        return self.x.shape[2]

    @property
    def ngroups(self):
        return self.B.shape[1]

    @property
    def dstate(self):
        return self.B.shape[2]


def draw_lengths(seed: int, n: int, lo: int, hi: int, target: int = 16384, slack: int = 1024):
    """The length rule of the drawn-length workloads (kept for documentation and a test)."""
    rng = np.random.default_rng(seed)
    while True:
        L = rng.integers(lo, hi + 1, size=n)
        if abs(int(L.sum()) - target) <= slack:
            return [int(v) for v in L], rng


def _cast(a64: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a64.astype(np.float32)))
    return t.to(torch.bfloat16) if dtype == "bf16" else t


def make_inputs(lengths, nheads, headdim, dstate, ngroups, chunk_size, dtype="f32", init_seqs=(),
                seed=0, rng=None, dt_bias_range=(-4.0, -2.0), a_log_range=(0.0, float(np.log(16.0))),
                x_scale=1.0, block_size=None, num_slots=None, name=""):
    """Draw one workload. `rng` continues a stream (used after a length draw)."""
    if rng is None:
        rng = np.random.default_rng(seed)
    lengths = [int(v) for v in lengths]
    S, T, H, P, N, G = len(lengths), int(sum(lengths)), nheads, headdim, dstate, ngroups
    cu = np.zeros(S + 1, dtype=np.int64)
    cu[1:] = np.cumsum(lengths)
    x = rng.standard_normal((T, H, P)) * x_scale
    dt = rng.standard_normal((T, H))
    dt_bias = rng.uniform(dt_bias_range[0], dt_bias_range[1], size=H)
    A = -np.exp(rng.uniform(a_log_range[0], a_log_range[1], size=H))
    B = rng.standard_normal((T, G, N)) / np.sqrt(N)
    C = rng.standard_normal((T, G, N)) / np.sqrt(N)
    D = rng.standard_normal(H)
    init = rng.standard_normal((S, H, P, N)) * 0.5
    has = np.zeros(S, dtype=np.int32)
    has[list(init_seqs)] = 1
    block_table = None
    if block_size is not None:
        nblk = -(-max(lengths) // block_size) if lengths else 0
        slots = num_slots if num_slots is not None else S * nblk
        block_table = torch.from_numpy(
            rng.permutation(slots)[: S * nblk].reshape(S, nblk).astype(np.int32))
    return Workload(
        lengths=lengths,
        cu_seqlens=torch.from_numpy(cu.astype(np.int32)),
        x=_cast(x, dtype), dt=_cast(dt, "f32"), dt_bias=_cast(dt_bias, "f32"), A=_cast(A, "f32"),
        B=_cast(B, dtype), C=_cast(C, dtype), D=_cast(D, "f32"),
        initial_states=_cast(init, "f32"), has_initial_state=torch.from_numpy(has),
        chunk_size=int(chunk_size), dtype=dtype, block_table=block_table, block_size=block_size,
        num_slots=num_slots, name=name)


def make_config(index: int, chunk_size: Optional[int] = None) -> Workload:
    """The seeded workload of configuration `index` (seed = index)."""
    cfg = CONFIGS[index]
    rng = np.random.default_rng(index)
    lengths = cfg["lengths"]
    if "len_draw" in cfg:
        n, lo, hi = cfg["len_draw"]
        drawn, rng = draw_lengths(index, n, lo, hi)
        if drawn != lengths:   # numpy stream changed: keep the constants, restart the stream
            rng = np.random.default_rng(index)
    return make_inputs(lengths, cfg["nheads"], cfg["headdim"], cfg["dstate"], cfg["ngroups"],
                       chunk_size or cfg["chunk_size"], dtype=cfg["dtype"],
                       init_seqs=cfg["init_seqs"], rng=rng, block_size=cfg.get("block_size"),
                       num_slots=cfg.get("num_slots"), name=cfg["name"])


@dataclasses.dataclass
class DecodeBatch:
    """One decode token for each of `nseqs` sequences, with a state cache and
    the read / write cache slot of every sequence (dual anchors)."""
    x: torch.Tensor            # (S, H, P)
    dt: torch.Tensor           # (S, H) float32, raw (before bias and softplus)
    dt_bias: torch.Tensor      # (H,)
    A: torch.Tensor            # (H,)
    B: torch.Tensor            # (S, G, N)
    C: torch.Tensor            # (S, G, N)
    D: torch.Tensor            # (H,)
    state_cache: torch.Tensor  # (num_slots, H, P, N) float32
    read_slot: torch.Tensor    # (S,) int32, < 0: start from zero
    write_slot: torch.Tensor   # (S,) int32, < 0: no write
    dtype: str
    name: str = ""

    @property
    def nseqs(self):
        return self.x.shape[0]


# Decode workload timed next to the prefill scan: the prefix-cache layer shape,
# 256 sequences each reading one slot of a 512-slot cache and writing another.
DECODE_CONFIG = dict(name="decode_dual_anchor_256x_h32p128n128g4", nseqs=256, nheads=32,
                     headdim=128, dstate=128, ngroups=4, num_slots=512, dtype="bf16", seed=5)


def make_decode_inputs(nseqs, nheads, headdim, dstate, ngroups, num_slots, dtype="f32", seed=0,
                       anchors="dual", name=""):
    """Draw one decode batch (same distributions as the prefill inputs; cache
    states ~ N(0, 0.5^2)). Draw order: x -> dt -> dt_bias -> A -> B -> C -> D ->
    cache -> slot permutation. anchors: "dual" (read and write slots all
    distinct; needs num_slots >= 2 S), "inplace" (write slot = read slot), or
    "mixed" (dual, with every fourth sequence in place, every seventh reading
    no slot and every fifth writing none)."""
    rng = np.random.default_rng(seed)
    S, H, P, N, G = nseqs, nheads, headdim, dstate, ngroups
    x = rng.standard_normal((S, H, P))
    dt = rng.standard_normal((S, H))
    dt_bias = rng.uniform(-4.0, -2.0, size=H)
    A = -np.exp(rng.uniform(0.0, float(np.log(16.0)), size=H))
    B = rng.standard_normal((S, G, N)) / np.sqrt(N)
    C = rng.standard_normal((S, G, N)) / np.sqrt(N)
    D = rng.standard_normal(H)
    cache = rng.standard_normal((num_slots, H, P, N)).astype(np.float32) * np.float32(0.5)
    perm = rng.permutation(num_slots).astype(np.int32)
    if anchors == "inplace":
        rs = perm[:S].copy()
        ws = rs.copy()
    else:
        assert num_slots >= 2 * S, "dual anchors need two distinct slots per sequence"
        rs, ws = perm[:S].copy(), perm[S:2 * S].copy()
        if anchors == "mixed":
            ws[::4] = rs[::4]
            rs[3::7] = -1
            ws[2::5] = -1
    return DecodeBatch(x=_cast(x, dtype), dt=_cast(dt, "f32"), dt_bias=_cast(dt_bias, "f32"),
                       A=_cast(A, "f32"), B=_cast(B, dtype), C=_cast(C, dtype), D=_cast(D, "f32"),
                       state_cache=torch.from_numpy(cache), read_slot=torch.from_numpy(rs),
                       write_slot=torch.from_numpy(ws), dtype=dtype, name=name)


def make_decode_config() -> DecodeBatch:
    c = DECODE_CONFIG
    return make_decode_inputs(c["nseqs"], c["nheads"], c["headdim"], c["dstate"], c["ngroups"],
                              c["num_slots"], dtype=c["dtype"], seed=c["seed"], name=c["name"])


@dataclasses.dataclass
class ConvBatch:
    """Inputs of one varlen causal conv1d call (the step before the scan)."""
    x: torch.Tensor             # (T, C) in dtype
    weight: torch.Tensor        # (C, W) float32
    bias: torch.Tensor          # (C,) float32
    cu_seqlens: torch.Tensor    # (S+1,) int32
    conv_states: torch.Tensor   # (num_slots, W-1, C) in dtype
    read_slot: torch.Tensor     # (S,) int32, < 0: zero leading inputs
    write_slot: torch.Tensor    # (S,) int32, < 0: no state written
    silu: bool
    dtype: str
    name: str = ""


# The channels of the prefix-cache workload's layer: x (H P = 4096) then B and C
# (2 G N = 1024), convolved with width 4 before the scan.
CONV_CONFIG = dict(name="conv1d_prefix_cache_4x8894_c5120_w4", lengths=[8894] * 4, channels=5120,
                   width=4, silu=True, chunk_size=64, num_slots=8, dtype="bf16", seed=6)


def make_conv_inputs(lengths, channels, width, num_slots, dtype="f32", seed=0, anchors="dual",
                     silu=True, name=""):
    """Draw one conv1d batch. Draw order: x ~ N(0,1) -> weight, bias ~ U(-1/sqrt(W),
    1/sqrt(W)) (the usual fan-in init) -> cached states ~ N(0,1) -> slot
    permutation. anchors: "dual" (read and write slots all distinct; needs
    num_slots >= 2 S) or "mixed" (dual, with every third sequence reading no
    slot and every fourth writing none)."""
    rng = np.random.default_rng(seed)
    S, C, W = len(lengths), channels, width
    cu = np.zeros(S + 1, np.int32)
    cu[1:] = np.cumsum(lengths)
    T = int(cu[-1])
    k = 1.0 / np.sqrt(W)
    x = rng.standard_normal((T, C))
    weight = rng.uniform(-k, k, size=(C, W))
    bias = rng.uniform(-k, k, size=C)
    states = rng.standard_normal((num_slots, max(W - 1, 0), C))
    assert num_slots >= 2 * S, "dual anchors need two distinct slots per sequence"
    perm = rng.permutation(num_slots).astype(np.int32)
    rs, ws = perm[:S].copy(), perm[S:2 * S].copy()
    if anchors == "mixed":
        rs[1::3] = -1
        ws[2::4] = -1
    return ConvBatch(x=_cast(x, dtype), weight=_cast(weight, "f32"), bias=_cast(bias, "f32"),
                     cu_seqlens=torch.from_numpy(cu), conv_states=_cast(states, dtype),
                     read_slot=torch.from_numpy(rs), write_slot=torch.from_numpy(ws), silu=silu,
                     dtype=dtype, name=name)


def make_conv_config() -> ConvBatch:
    c = CONV_CONFIG
    return make_conv_inputs(c["lengths"], c["channels"], c["width"], c["num_slots"], dtype=c["dtype"],
                            seed=c["seed"], silu=c["silu"], name=c["name"])


@dataclasses.dataclass
class GdnBatch:
    """Packed varlen inputs of one gated-delta-rule (GDN) chunk call."""
    lengths: list
    cu_seqlens: torch.Tensor       # (S+1,) int32
    q: torch.Tensor                # (T, G, dk) in dtype, unit rows
    k: torch.Tensor                # (T, G, dk) in dtype, unit rows
    v: torch.Tensor                # (T, H, dv) in dtype
    gate: torch.Tensor             # (T, H) float32 log-decay (<= 0)
    beta: torch.Tensor             # (T, H) float32 in (0, 1)
    scale: float
    initial_states: torch.Tensor   # (S, H, dv, dk) float32
    has_initial_state: torch.Tensor  # (S,) int32
    chunk_size: int
    dtype: str
    block_table: Optional[torch.Tensor] = None
    block_size: Optional[int] = None
    num_slots: Optional[int] = None
    name: str = ""

    @property
    def nseqs(self):
        return len(self.lengths)

    @property
    def total_tokens(self):
        return int(sum(self.lengths))


# GDN workload timed next to the scan: the prefix-caching page's ~8.9k-token
# prompt, four sequences, 32 value heads on 16 key heads, key and value head
# dimensions 128, chunk 64, 256-token cache blocks.
GDN_CONFIG = dict(name="gdn_prefix_cache_4x8894_h32g16", lengths=[8894] * 4, nheads=32, nkheads=16,
                  dk=128, dv=128, chunk_size=64, block_size=256, num_slots=140, dtype="bf16", seed=7)


def make_gdn_inputs(lengths, nheads, nkheads, dk, dv, chunk_size=64, dtype="bf16", init_seqs=(), seed=0,
                    block_size=None, num_slots=None, name=""):
    """Draw one GDN batch. Draw order: q, k ~ N(0,1) rows scaled to unit length
    (the layer normalises them before the kernel) -> v ~ N(0,1) -> gate =
    -e^U(ln 1e-3, ln 0.2) (log-decay per token and value head: per-token decay
    factors between 0.82 and 0.999, about 0.09 over a chunk) -> beta ~ U(0.05, 0.95)
    -> initial states ~ N(0, 0.5^2) -> block table (a slot permutation).
    scale = 1/sqrt(dk)."""
    rng = np.random.default_rng(seed)
    lengths = [int(v) for v in lengths]
    S, T = len(lengths), int(sum(lengths))
    cu = np.zeros(S + 1, np.int32)
    cu[1:] = np.cumsum(lengths)
    q = rng.standard_normal((T, nkheads, dk))
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k = rng.standard_normal((T, nkheads, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((T, nheads, dv))
    gate = -np.exp(rng.uniform(np.log(1e-3), np.log(0.2), size=(T, nheads)))
    beta = rng.uniform(0.05, 0.95, size=(T, nheads))
    init = rng.standard_normal((S, nheads, dv, dk)) * 0.5
    has = np.zeros(S, np.int32)
    has[list(init_seqs)] = 1
    block_table = None
    if block_size is not None:
        nblk = -(-max(lengths) // block_size) if lengths else 0
        slots = num_slots if num_slots is not None else S * nblk
        block_table = torch.from_numpy(rng.permutation(slots)[: S * nblk].reshape(S, nblk).astype(np.int32))
    return GdnBatch(lengths=lengths, cu_seqlens=torch.from_numpy(cu), q=_cast(q, dtype), k=_cast(k, dtype),
                    v=_cast(v, dtype), gate=_cast(gate, "f32"), beta=_cast(beta, "f32"),
                    scale=float(1.0 / np.sqrt(dk)), initial_states=_cast(init, "f32"),
                    has_initial_state=torch.from_numpy(has), chunk_size=chunk_size, dtype=dtype,
                    block_table=block_table, block_size=block_size, num_slots=num_slots, name=name)


def make_gdn_config() -> GdnBatch:
    c = GDN_CONFIG
    return make_gdn_inputs(c["lengths"], c["nheads"], c["nkheads"], c["dk"], c["dv"], c["chunk_size"],
                           dtype=c["dtype"], seed=c["seed"], block_size=c["block_size"], num_slots=c["num_slots"],
                           name=c["name"])
