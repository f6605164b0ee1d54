"""GPU continuation from num_computed_tokens > 0: prompts computed in scheduler
bites through the HIP path (C ABI) against one pass of the float64 oracle.

Workload: the prefix-cache layer shape (4 x 8894 tokens, 32 heads, headdim 128,
dstate 128, 4 groups, chunk 64, blocks of 256 tokens, bf16 inputs). Each
sequence starts from its own computed prefix -- none, a cached aligned prefix
(6912 = 27 blocks, the resume point of the prefix-caching page's Correctness
section), a misaligned one (6900, as from externally loaded state) and one in
the final partial block (8800) -- with its state taken from the oracle. Every
scheduler step packs the bites the library's rule gives (budget 2048, align 256)
into one varlen batch: metadata, the checkpoint plan at num_computed_tokens =
the bite starts, and the scan with the running states as initial states and the
checkpoints written at the source. Checked: the bites equal the oracle rule's,
the plan integers equal the oracle plan bit for bit, y of every computed token
and the final states are within 2e-2 of the one-pass oracle, and every block
that ends in a sequence's computed range holds the one-pass state at that block
end (within 2e-2) while every other slot is untouched.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import TOL, check_close, log
from selective_state_space_cu_amd import ssd
from selective_state_space_cu_amd.workloads import make_config

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

STARTS = [0, 6912, 6900, 8800]
BUDGET, ALIGN = 2048, 256


def _prefix_state(w, s, n):
    """One-pass oracle state of sequence s after its first n tokens (zero for n = 0)."""
    H, P, N = w.nheads, w.headdim, w.dstate
    if n == 0:
        return np.zeros((H, P, N))
    t0 = int(w.cu_seqlens[s])
    _, fin, _ = oracle.ssd_varlen(w.x[t0:t0 + n], w.dt[t0:t0 + n], w.dt_bias, w.A, w.B[t0:t0 + n],
                                  w.C[t0:t0 + n], w.D, np.array([0, n], np.int32))
    return fin[0]


def test_continuation_in_scheduler_bites():
    w = make_config(4)
    S, H, P, N, G = w.nseqs, w.nheads, w.headdim, w.dstate, w.ngroups
    cs, bs = w.chunk_size, w.block_size
    cu = w.cu_seqlens.numpy()
    L = int(cu[1] - cu[0])
    nblocks = (L + bs - 1) // bs
    log("continuation: one-pass oracle")
    y_ref, fin_ref, cst_ref = oracle.ssd_varlen(w.x, w.dt, w.dt_bias, w.A, w.B, w.C, w.D, w.cu_seqlens,
                                                chunk_size=cs)
    # one-pass state at the end of block k of sequence s
    def block_state(s, k):
        end = min((k + 1) * bs, L)
        return cst_ref[s * (L // cs + 1) + (end + cs - 1) // cs - 1]

    dev = torch.device("cuda")
    x, dt, B, C = (getattr(w, k).to(dev) for k in ("x", "dt", "B", "C"))
    A, dt_bias, D = (getattr(w, k).to(dev) for k in ("A", "dt_bias", "D"))
    bt = w.block_table.numpy()
    cache = torch.full((w.num_slots, H, P, N), float("nan"), device=dev)
    state = torch.from_numpy(np.stack([_prefix_state(w, s, STARTS[s]) for s in range(S)]).astype(np.float32)).to(dev)
    has = torch.tensor([1 if n > 0 else 0 for n in STARTS], dtype=torch.int32, device=dev)
    y = torch.full_like(x, float("nan"))
    pos = list(STARTS)
    step = 0
    while any(p < L for p in pos):
        live = [s for s in range(S) if pos[s] < L]
        n = ssd.prefill_bites([pos[s] for s in live], [L] * len(live), BUDGET, ALIGN).numpy()
        ref_n = oracle.prefill_bites([pos[s] for s in live], [L] * len(live), BUDGET, ALIGN)
        assert np.array_equal(n, ref_n), step
        log(f"step {step}: bites " + ", ".join(f"s{s}[{pos[s]},{pos[s] + int(k)})" for s, k in zip(live, n)))
        rows = torch.cat([torch.arange(int(cu[s]) + pos[s], int(cu[s]) + pos[s] + int(k)) for s, k in zip(live, n)])
        rows = rows.to(dev)
        cu_b = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
        T = int(cu_b[-1])
        meta = ssd.varlen_metadata(torch.from_numpy(cu_b).to(dev), cs, total_tokens=T)
        ncomp = np.array([pos[s] for s in live], np.int32)
        bt_b = np.ascontiguousarray(bt[live])
        src, dst = ssd.export_chunk_states(meta, torch.from_numpy(bt_b), bs,
                                           num_computed_tokens=torch.from_numpy(ncomp), num_slots=w.num_slots)
        rsrc, rdst = oracle.checkpoint_plan(cu_b, meta.seq_chunk_start.cpu().numpy(), meta.max_chunks, bt_b,
                                            bs, cs, num_computed_tokens=ncomp)
        assert np.array_equal(src.cpu().numpy(), rsrc), step
        assert np.array_equal(dst.cpu().numpy(), rdst), step
        idx = torch.tensor(live, device=dev)
        yb, fb = ssd.chunk_scan_varlen(x[rows].contiguous(), dt[rows].contiguous(), A, B[rows].contiguous(),
                                       C[rows].contiguous(), meta, dt_bias=dt_bias, D=D,
                                       initial_states=state[idx].contiguous(),
                                       has_initial_state=has[idx].contiguous(),
                                       chunk_states=cache, chunk_state_dst=dst)
        torch.cuda.synchronize()
        assert int(meta.error_flag.item()) == 0, step
        y[rows] = yb
        state[idx] = fb
        has[idx] = 1
        for s, k in zip(live, n):
            pos[s] += int(k)
        step += 1
    # outputs of every computed token and the final states
    for s in range(S):
        a, b = int(cu[s]) + STARTS[s], int(cu[s + 1])
        check_close(y[a:b], y_ref[a:b], TOL["bf16"], f"y of sequence {s} from {STARTS[s]}")
    check_close(state, fin_ref, TOL["bf16"], "final states")
    # checkpoints: exact states for every block ending in the computed range, nothing else touched
    for s in range(S):
        for k in range(nblocks):
            slot = int(bt[s, k])
            if min((k + 1) * bs, L) > STARTS[s]:
                check_close(cache[slot], block_state(s, k), TOL["bf16"], f"block {k} of sequence {s}")
            else:
                assert torch.isnan(cache[slot]).all(), f"block {k} of sequence {s} was written"
    log(f"continuation: {step} steps, all checks passed")
