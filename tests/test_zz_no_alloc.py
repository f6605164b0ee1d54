"""The allocation-free GDN entry point (ssd_gated_delta_chunk_varlen_noalloc,
the library's static device workspace) against the entry point that takes a
workspace: identical outputs, final states and checkpoints on two calls in a
row, the second smaller, and a clear refusal above the static workspace's size.
"""
import numpy as np
import pytest
import torch

from gpu_util import log
from selective_state_space_cu_amd import ssd
from selective_state_space_cu_amd.workloads import make_gdn_inputs

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def _call(w, no_alloc):
    dev = torch.device("cuda")
    d = {k: getattr(w, k).to(dev).contiguous() for k in ("q", "k", "v", "gate", "beta", "initial_states",
                                                         "has_initial_state", "cu_seqlens")}
    meta = ssd.varlen_metadata(d["cu_seqlens"], 64, total_tokens=w.total_tokens)
    S, H, DV, DK = w.nseqs, w.v.shape[1], w.v.shape[2], w.q.shape[2]
    o = torch.full_like(d["v"], float("nan"))
    fin = torch.full((S, H, DV, DK), float("nan"), device=dev)
    cst = torch.full((meta.max_chunks, H, DV, DK), float("nan"), device=dev)
    ssd.gated_delta_chunk_varlen(d["q"], d["k"], d["v"], d["gate"], d["beta"], meta, scale=w.scale,
                                 initial_states=d["initial_states"], has_initial_state=d["has_initial_state"],
                                 o=o, final_states=fin, chunk_states=cst, no_alloc=no_alloc)
    torch.cuda.synchronize()
    assert int(meta.error_flag.item()) == 0
    return o, fin, cst


def _same(a, b):
    return torch.equal(a.nan_to_num(7.0), b.nan_to_num(7.0))


def test_no_alloc_matches_workspace_entry_point_twice():
    for step, (lengths, H, G, dv, seed) in enumerate([([300, 17, 129, 64], 4, 2, 128, 21), ([70, 5], 2, 1, 64, 22)]):
        log(f"no-alloc call {step}: lengths={lengths} H={H} G={G} dv={dv}")
        w = make_gdn_inputs(lengths, H, G, 128, dv, init_seqs=(0,), seed=seed)
        o_na, f_na, c_na = _call(w, True)
        o_ws, f_ws, c_ws = _call(w, False)
        assert [_same(o_na, o_ws), _same(f_na, f_ws), _same(c_na, c_ws)] == [True, True, True], step
        assert torch.isfinite(o_na).all() and torch.isfinite(f_na).all()


def test_no_alloc_refuses_above_its_workspace():
    # 8894 tokens x 32 heads: 139 chunks x 32 heads x 8 KiB > 32 MiB
    w = make_gdn_inputs([8894], 32, 16, 128, 128, seed=23)
    need = 139 * 32 * 64 * 64 * 2
    assert need > 32 << 20
    with pytest.raises(ssd.SSDError, match="capacity"):
        _call(w, True)
