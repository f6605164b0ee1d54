"""The seeded input generator: the drawn lengths reproduce, and inputs are deterministic."""
import torch

from selective_state_space_cu_amd.workloads import CONFIGS, draw_lengths, make_inputs


def test_drawn_lengths_reproduce():
    for idx in (2, 3):
        n, lo, hi = CONFIGS[idx]["len_draw"]
        got, _ = draw_lengths(idx, n, lo, hi)
        assert got == CONFIGS[idx]["lengths"]
        assert abs(sum(got) - 16384) <= 1024


def test_inputs_are_deterministic_and_typed():
    a = make_inputs([5, 7], 4, 16, 32, 2, 16, dtype="bf16", init_seqs=[1], seed=3)
    b = make_inputs([5, 7], 4, 16, 32, 2, 16, dtype="bf16", init_seqs=[1], seed=3)
    assert a.x.dtype == torch.bfloat16 and a.B.dtype == torch.bfloat16 and a.dt.dtype == torch.float32
    for k in ("x", "dt", "dt_bias", "A", "B", "C", "D", "initial_states"):
        assert torch.equal(getattr(a, k), getattr(b, k))
    assert a.cu_seqlens.tolist() == [0, 5, 12] and a.has_initial_state.tolist() == [0, 1]
    assert bool((a.A < 0).all()) and bool((a.dt_bias <= -2).all()) and bool((a.dt_bias >= -4).all())
