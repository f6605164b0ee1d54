"""The library's host-side scheduler rule (ssd_prefill_bites) against the oracle's,
bit for bit, and its argument errors (CPU only: nothing is launched)."""
import numpy as np
import pytest

import oracle
from selective_state_space_cu_amd import ssd


def test_prefill_bites_match_the_oracle():
    rng = np.random.default_rng(5)
    for trial in range(200):
        S = int(rng.integers(1, 40))
        align = int(2 ** rng.integers(4, 10))
        plen = rng.integers(0, 30 * align, size=S).astype(np.int32)
        start = np.array([int(rng.integers(0, p + 1)) for p in plen], np.int32)
        budget = (align * rng.integers(1, 9, size=S) + rng.integers(0, align, size=S)).astype(np.int32)
        got = ssd.prefill_bites(start, plen, budget, align).numpy()
        want = oracle.prefill_bites(start, plen, budget, align)
        assert np.array_equal(got, want), trial


def test_prefill_bites_whole_prompts_match_the_oracle():
    """Bite sequences of whole prompts (each step's start = the previous end)."""
    for start, plen, budget, align in [(6900, 8894, 1000, 256), (0, 8894, 2048, 256), (8100, 8894, 2000, 256),
                                       (37, 530, 160, 64), (0, 0, 64, 64)]:
        pos, bites = start, []
        while pos < plen:
            n = int(ssd.prefill_bites([pos], [plen], budget, align)[0])
            assert n > 0
            bites.append((pos, pos + n))
            pos += n
        assert bites == oracle.prefill_schedule(start, plen, budget, align)


@pytest.mark.parametrize("args", [
    dict(start=[5], plen=[10], budget=[64], align=0),       # align <= 0
    dict(start=[5], plen=[10], budget=[32], align=64),      # budget below align
    dict(start=[11], plen=[10], budget=[64], align=64),     # start past the prompt
    dict(start=[-1], plen=[10], budget=[64], align=64),     # negative start
])
def test_prefill_bites_argument_errors(args):
    with pytest.raises(ssd.SSDError) as e:
        ssd.prefill_bites(args["start"], args["plen"], args["budget"], args["align"])
    assert e.value.status == 3   # SSD_ERR_SHAPE
    with pytest.raises(ValueError):
        oracle.prefill_bites(args["start"], args["plen"], args["budget"], args["align"])


def test_prefill_bites_null_arrays():
    lib = ssd.load_library()
    assert lib.ssd_prefill_bites(1, None, None, None, 64, None) == 1   # SSD_ERR_NULL_ARG
    assert lib.ssd_prefill_bites(0, None, None, None, 64, None) == 0
