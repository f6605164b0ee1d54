"""Helpers of the GPU parity tests: run the HIP path through the C ABI and the
CPU oracle on the same seeded inputs, and compare at the stated tolerances."""
import sys

import numpy as np
import torch

import oracle
from selective_state_space_cu_amd import ssd

# |gpu - ref| <= atol + rtol * |ref|  (float32 inputs: 5e-3; bf16 inputs with float32 state: 2e-2)
TOL = {"f32": 5e-3, "bf16": 2e-2}


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(w, dev="cuda"):
    out = {}
    for k in ("x", "dt", "dt_bias", "A", "B", "C", "D", "initial_states", "has_initial_state",
              "cu_seqlens"):
        out[k] = getattr(w, k).to(dev).contiguous()
    return out


def gpu_run(w, chunk_size=None, export=None, state_cache=None, chunk_state_dst=None,
            init=True, d=None):
    """metadata + scan on the GPU. export='dense' also returns per-chunk states."""
    d = d or to_dev(w)
    cs = chunk_size or w.chunk_size
    meta = ssd.varlen_metadata(d["cu_seqlens"], cs, total_tokens=w.total_tokens)
    cst = None
    if export == "dense":
        cst = torch.full((meta.max_chunks, w.nheads, w.headdim, w.dstate), float("nan"),
                         device="cuda")
    elif export == "cache":
        cst = state_cache
    y, fin = ssd.chunk_scan_varlen(d["x"], d["dt"], d["A"], d["B"], d["C"], meta,
                                   dt_bias=d["dt_bias"], D=d["D"],
                                   initial_states=d["initial_states"] if init else None,
                                   has_initial_state=d["has_initial_state"] if init else None,
                                   chunk_states=cst, chunk_state_dst=chunk_state_dst)
    torch.cuda.synchronize()
    return meta, y, fin, cst


def oracle_run(w, chunk_size=0, init=True):
    return oracle.ssd_varlen(w.x, w.dt, w.dt_bias, w.A, w.B, w.C, w.D, w.cu_seqlens,
                             w.initial_states if init else None,
                             w.has_initial_state if init else None, chunk_size=chunk_size)


def oracle_pair(w, s, h, chunk_size=0):
    """Oracle for one (sequence, head): sliced inputs, 1 head, 1 group."""
    cu = w.cu_seqlens
    t0, t1 = int(cu[s]), int(cu[s + 1])
    g = h // (w.nheads // w.ngroups)
    hs, gs = slice(h, h + 1), slice(g, g + 1)
    return oracle.ssd_varlen(w.x[t0:t1, hs], w.dt[t0:t1, hs], w.dt_bias[hs], w.A[hs],
                             w.B[t0:t1, gs], w.C[t0:t1, gs], w.D[hs],
                             np.array([0, t1 - t0], np.int32), w.initial_states[s:s + 1, hs],
                             w.has_initial_state[s:s + 1], chunk_size=chunk_size)


def check_close(got, ref, tol, what):
    got = np.asarray(got.float().cpu().numpy() if hasattr(got, "cpu") else got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, f"{what}: shape {got.shape} vs {ref.shape}"
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - ref)
    bound = tol + tol * np.abs(ref)
    bad = err > bound
    worst = float(np.max(err / bound)) if err.size else 0.0
    assert not bad.any(), (f"{what}: {int(bad.sum())}/{bad.size} outside atol=rtol={tol}; "
                           f"max err {float(err.max()):.3e}, worst err/bound {worst:.3f}")
    return worst
