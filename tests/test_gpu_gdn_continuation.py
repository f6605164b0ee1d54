"""GPU continuation of the gated delta rule from num_computed_tokens > 0: GDN
prompts computed in the scheduler's bites through the HIP path (C ABI) against
one pass of the float64 oracle.

Workload: 4 x 8894 tokens, 8 value heads on 4 key heads, dk = dv = 128, chunk
64, blocks of 256 tokens, bf16 q/k/v. Each sequence starts from its own
computed prefix -- none, a cached aligned prefix (6912 tokens = 27 blocks), a
misaligned one (6900) and one in the final partial block (8800) -- with its
state from the oracle. Every scheduler step packs the bites the library's rule
gives (budget 2048, align 256) into one varlen batch: metadata, the checkpoint
plan at num_computed_tokens = the bite starts, and the GDN call with the running
states as initial states and the checkpoints written at the source. Checked:
the bites equal the oracle rule's, o of every computed token and the final
states are within 2e-2 of the one-pass oracle, every block that ends in a
sequence's computed range holds the one-pass state at that block end (within
2e-2), and every other slot is untouched.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import TOL, check_close, log
from selective_state_space_cu_amd import ssd
from selective_state_space_cu_amd.workloads import make_gdn_inputs

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

STARTS = [0, 6912, 6900, 8800]
BUDGET, ALIGN, CS = 2048, 256, 64


def _f64(t):
    return t.float().numpy().astype(np.float64)


def test_gdn_continuation_in_scheduler_bites():
    L, S, H, G = 8894, 4, 8, 4
    w = make_gdn_inputs([L] * S, H, G, 128, 128, seed=17, block_size=ALIGN, num_slots=140)
    cu = w.cu_seqlens.numpy()
    q, k, v, gate, beta = (_f64(getattr(w, n)) for n in ("q", "k", "v", "gate", "beta"))
    log("gdn continuation: one-pass oracle")
    zero = np.zeros((S, H, 128, 128))
    o_ref, fin_ref, cst_ref = oracle.gated_delta(q, k, v, gate, beta, cu, w.scale, zero, np.zeros(S, np.int32),
                                                 chunk_size=CS)
    nch = (L + CS - 1) // CS

    def prefix_state(s, n):
        if n == 0:
            return np.zeros((H, 128, 128))
        if n % CS == 0:
            return cst_ref[s * nch + n // CS - 1]
        t0 = int(cu[s])
        _, f, _ = oracle.gated_delta(q[t0:t0 + n], k[t0:t0 + n], v[t0:t0 + n], gate[t0:t0 + n], beta[t0:t0 + n],
                                     np.array([0, n], np.int32), w.scale, None, None)
        return f[0]

    dev = torch.device("cuda")
    dq, dk_, dv_, dg, db = (getattr(w, n).to(dev) for n in ("q", "k", "v", "gate", "beta"))
    bt = w.block_table.numpy()
    nblocks = bt.shape[1]
    cache = torch.full((w.num_slots, H, 128, 128), float("nan"), device=dev)
    state = torch.from_numpy(np.stack([prefix_state(s, STARTS[s]) for s in range(S)]).astype(np.float32)).to(dev)
    has = torch.tensor([1 if n > 0 else 0 for n in STARTS], dtype=torch.int32, device=dev)
    o = torch.full_like(dv_, float("nan"))
    pos = list(STARTS)
    step = 0
    while any(p < L for p in pos):
        live = [s for s in range(S) if pos[s] < L]
        n = ssd.prefill_bites([pos[s] for s in live], [L] * len(live), BUDGET, ALIGN).numpy()
        assert np.array_equal(n, oracle.prefill_bites([pos[s] for s in live], [L] * len(live), BUDGET, ALIGN)), step
        rows = torch.cat([torch.arange(int(cu[s]) + pos[s], int(cu[s]) + pos[s] + int(c)) for s, c in zip(live, n)])
        rows = rows.to(dev)
        cu_b = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
        meta = ssd.varlen_metadata(torch.from_numpy(cu_b).to(dev), CS, total_tokens=int(cu_b[-1]))
        ncomp = np.array([pos[s] for s in live], np.int32)
        _, dst = ssd.export_chunk_states(meta, torch.from_numpy(np.ascontiguousarray(bt[live])), ALIGN,
                                         num_computed_tokens=torch.from_numpy(ncomp), num_slots=w.num_slots)
        idx = torch.tensor(live, device=dev)
        ob, fb = ssd.gated_delta_chunk_varlen(dq[rows].contiguous(), dk_[rows].contiguous(), dv_[rows].contiguous(),
                                              dg[rows].contiguous(), db[rows].contiguous(), meta, scale=w.scale,
                                              initial_states=state[idx].contiguous(),
                                              has_initial_state=has[idx].contiguous(),
                                              chunk_states=cache, chunk_state_dst=dst)
        torch.cuda.synchronize()
        assert int(meta.error_flag.item()) == 0, step
        o[rows] = ob
        state[idx] = fb
        has[idx] = 1
        for s, c in zip(live, n):
            pos[s] += int(c)
        step += 1
    log(f"gdn continuation: {step} scheduler steps")
    for s in range(S):
        a, b = int(cu[s]) + STARTS[s], int(cu[s + 1])
        check_close(o[a:b], o_ref[a:b], TOL["bf16"], f"o of sequence {s} from {STARTS[s]}")
    check_close(state, fin_ref, TOL["bf16"], "final states")
    for s in range(S):
        for kb in range(nblocks):
            slot = int(bt[s, kb])
            end = min((kb + 1) * ALIGN, L)
            if end > STARTS[s]:
                check_close(cache[slot], cst_ref[s * nch + (end + CS - 1) // CS - 1], TOL["bf16"],
                            f"block {kb} of sequence {s}")
            else:
                assert torch.isnan(cache[slot]).all(), f"block {kb} of sequence {s} was written"
