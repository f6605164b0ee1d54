"""GPU parity of the varlen causal conv1d (through the C ABI) against the
float64 oracle.

Tolerance, from the arithmetic: the kernel sums bias + taps with fmaf in fp32,
so before the output rounding it is within about (W + 1) 2^-24 mag of the exact
value, mag = |bias| + sum_k |w_k u_k| (the oracle on absolute values, identity
activation); SiLU's slope is below 1.1 and expf adds a few fp32 ulps. bf16
outputs then round to nearest even (half a bf16 ulp, 2^-8 relative at most),
so |gpu - ref| <= 2^-8 |ref| + 2^-20 mag; fp32 outputs |gpu - ref| <=
2^-21 |ref| + 2^-20 mag. The written states are copies of inputs: bit-exact.
"""
import numpy as np
import pytest
import torch

import oracle
from selective_state_space_cu_amd import ssd
from selective_state_space_cu_amd.workloads import make_conv_config, make_conv_inputs

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _run(b, chunk_size, rs=None, ws=None, states=None, bias="keep", out=None):
    cu = b.cu_seqlens.to(DEV)
    T = int(b.cu_seqlens[-1])
    meta = ssd.varlen_metadata(cu, chunk_size, total_tokens=T)
    st = (b.conv_states if states is None else states).to(DEV).contiguous()
    o = ssd.causal_conv1d_varlen(b.x.to(DEV).contiguous(), b.weight.to(DEV).contiguous(), meta,
                                 bias=b.bias.to(DEV) if bias == "keep" else bias, silu=b.silu,
                                 conv_states=st,
                                 read_slot=(b.read_slot if rs is None else torch.as_tensor(rs)).to(DEV),
                                 write_slot=(b.write_slot if ws is None else torch.as_tensor(ws)).to(DEV),
                                 out=None if out is None else out.to(DEV))
    torch.cuda.synchronize()
    return o.cpu(), st.cpu(), int(meta.error_flag.item())


def _ref(b, rs=None, ws=None, states=None, bias="keep"):
    rs = b.read_slot if rs is None else rs
    ws = b.write_slot if ws is None else ws
    states = b.conv_states if states is None else states
    bias = b.bias if bias == "keep" else bias
    out, st, rc = oracle.causal_conv1d(b.x, b.cu_seqlens, b.weight, bias, b.silu, states, rs, ws)
    mag, _, _ = oracle.causal_conv1d(b.x.double().abs(), b.cu_seqlens, b.weight.double().abs(),
                                     None if bias is None else bias.double().abs(), False,
                                     states.double().abs(), rs, ws)
    return out, st, rc, mag


def _compare(b, got, st, ref, st_ref, mag, what):
    g = got.double().numpy()
    rel = 2.0 ** -8 if b.dtype == "bf16" else 2.0 ** -21
    tol = rel * np.abs(ref) + 2.0 ** -20 * mag
    err = np.abs(g - ref)
    bad = err > tol
    assert not bad.any(), (f"{what}: {int(bad.sum())} outputs out of tolerance; worst at "
                           f"{np.unravel_index(np.argmax(err - tol), err.shape)}: got "
                           f"{g.flat[np.argmax(err - tol)]:.6g} want {ref.flat[np.argmax(err - tol)]:.6g}")
    want_st = torch.from_numpy(st_ref).to(st.dtype)
    assert torch.equal(st, want_st), f"{what}: written conv states differ"


CASES = [
    # (lengths, channels, width, chunk_size, dtype, silu, anchors, seed)
    ([0, 1, 2, 3, 63, 64, 65, 130, 0, 200], 64, 4, 64, "bf16", True, "mixed", 71),
    ([5, 17, 16, 15, 33, 1], 24, 3, 16, "bf16", False, "dual", 72),
    ([300, 2, 257, 0, 256], 1040, 4, 256, "bf16", True, "dual", 73),
    ([40, 9, 1, 77], 16, 2, 32, "f32", True, "mixed", 74),
    ([12, 0, 31], 8, 1, 16, "f32", False, "dual", 75),
    ([129, 64, 3, 190, 7, 2, 66, 128], 2048 + 8, 4, 64, "f32", True, "mixed", 76),
]


@pytest.mark.parametrize("lengths,C,W,cs,dtype,silu,anchors,seed", CASES,
                         ids=[f"W{c[2]}-cs{c[3]}-{c[4]}-{'silu' if c[5] else 'id'}-C{c[1]}" for c in CASES])
def test_conv1d_matches_oracle(lengths, C, W, cs, dtype, silu, anchors, seed):
    print(f"conv1d parity: lengths={lengths} C={C} W={W} cs={cs} {dtype} silu={silu} seed={seed}", flush=True)
    b = make_conv_inputs(lengths, C, W, 2 * len(lengths) + 3, dtype=dtype, seed=seed, anchors=anchors,
                         silu=silu)
    got, st, flag = _run(b, cs)
    ref, st_ref, rc, mag = _ref(b)
    assert rc == 0 and flag == 0
    _compare(b, got, st, ref, st_ref, mag, f"conv1d {lengths}")


def test_conv1d_without_bias_and_in_place_single_chunk():
    """bias NULL; sequences of at most one chunk that read and write the same slot."""
    b = make_conv_inputs([10, 64, 3, 0], 32, 4, 10, dtype="bf16", seed=77)
    rs = b.read_slot.numpy().copy()
    got, st, flag = _run(b, 64, ws=rs, bias=None)
    ref, st_ref, rc, mag = _ref(b, ws=rs, bias=None)
    assert rc == 0 and flag == 0
    _compare(b, got, st, ref, st_ref, mag, "in place, no bias")


def test_conv1d_refuses_slot_past_the_cache():
    """A slot >= num_slots: SSD_DATA_BAD_SLOT, that sequence skipped (its rows
    and slots untouched), the others computed."""
    b = make_conv_inputs([70, 5, 140], 16, 4, 8, dtype="bf16", seed=78)
    rs = b.read_slot.numpy().copy()
    rs[1] = 8
    sentinel = torch.full_like(b.x, 7.0)
    got, st, flag = _run(b, 64, rs=rs, out=sentinel)
    ref, st_ref, rc, mag = _ref(b, rs=rs)
    assert rc == -2 and flag & ssd.DATA_BAD_SLOT
    cu = b.cu_seqlens.numpy()
    assert torch.all(got[cu[1]:cu[2]] == 7.0), "refused sequence's rows were written"
    ref[cu[1]:cu[2]] = 7.0
    mag[cu[1]:cu[2]] = 0.0
    _compare(b, got, st, ref, st_ref, mag, "with a refused sequence")


def test_conv1d_refuses_in_place_multi_chunk_sequence():
    """read_slot == write_slot for a sequence of more than one chunk (its last
    chunk could overwrite the slot before its first chunk reads it):
    SSD_DATA_BAD_SLOT, that sequence skipped (rows and slot untouched), the
    others computed, a single-chunk in-place sequence included."""
    b = make_conv_inputs([70, 10, 140], 16, 4, 8, dtype="bf16", seed=80)
    rs = b.read_slot.numpy().copy()
    ws = b.write_slot.numpy().copy()
    ws[0] = rs[0]   # 70 tokens = 2 chunks of 64: refused
    ws[1] = rs[1]   # 10 tokens = 1 chunk: allowed
    sentinel = torch.full_like(b.x, 7.0)
    got, st, flag = _run(b, 64, rs=rs, ws=ws, out=sentinel)
    assert flag & ssd.DATA_BAD_SLOT
    rs_ref, ws_ref = rs.copy(), ws.copy()
    rs_ref[0] = ws_ref[0] = -1   # the oracle leaves the refused sequence's slot alone
    ref, st_ref, rc, mag = _ref(b, rs=rs_ref, ws=ws_ref)
    cu = b.cu_seqlens.numpy()
    assert torch.all(got[cu[0]:cu[1]] == 7.0), "refused sequence's rows were written"
    ref[cu[0]:cu[1]] = 7.0
    mag[cu[0]:cu[1]] = 0.0
    _compare(b, got, st, ref, st_ref, mag, "with a refused in-place sequence")


def test_conv1d_continues_through_the_cache():
    """Two calls: the second part of every sequence reads the slot the first
    part wrote; the outputs equal one call over the whole sequences."""
    lengths = [150, 7, 64]
    whole = make_conv_inputs(lengths, 48, 4, 9, dtype="f32", seed=79)
    cuts = [70, 3, 64]
    cu = whole.cu_seqlens.numpy()
    i1 = np.concatenate([np.arange(cu[s], cu[s] + cuts[s]) for s in range(3)])
    i2 = np.concatenate([np.arange(cu[s] + cuts[s], cu[s + 1]) for s in range(3)])
    first = make_conv_inputs(cuts, 48, 4, 9, dtype="f32", seed=79)
    first.x, first.weight, first.bias, first.conv_states = whole.x[i1], whole.weight, whole.bias, whole.conv_states
    second = make_conv_inputs([l - c for l, c in zip(lengths, cuts)], 48, 4, 9, dtype="f32", seed=79)
    second.x, second.weight, second.bias = whole.x[i2], whole.weight, whole.bias
    used = np.concatenate([whole.read_slot.numpy(), whole.write_slot.numpy()])
    mid = np.setdiff1d(np.arange(9), used).astype(np.int32)   # the three free slots
    o1, s1, f1 = _run(first, 64, rs=whole.read_slot, ws=mid)
    o2, s2, f2 = _run(second, 64, rs=mid, ws=whole.write_slot, states=s1)
    ow, sw, fw = _run(whole, 64)
    assert f1 == f2 == fw == 0
    joined = torch.empty_like(ow)
    joined[i1], joined[i2] = o1, o2
    assert torch.allclose(joined, ow, rtol=2.0 ** -20, atol=2.0 ** -20)
    assert torch.equal(s2[whole.write_slot], sw[whole.write_slot])


def test_conv1d_full_size_prefix_cache_channels():
    """The benchmarked workload (4 x 8894 tokens, 5120 channels, width 4, SiLU,
    bf16, chunk grid of 64), every output against the oracle."""
    b = make_conv_config()
    print(f"conv1d full size: {b.name}", flush=True)
    got, st, flag = _run(b, 64)
    ref, st_ref, rc, mag = _ref(b)
    assert rc == 0 and flag == 0
    _compare(b, got, st, ref, st_ref, mag, b.name)


def test_conv1d_decode_shaped_batch():
    """One token per sequence (the conv state advanced by one step, as in decode
    with dual anchors): 128 sequences, width 4, SiLU, mixed anchors."""
    b = make_conv_inputs([1] * 128, 5120, 4, 300, dtype="bf16", seed=80, anchors="mixed")
    got, st, flag = _run(b, 16)
    ref, st_ref, rc, mag = _ref(b)
    assert rc == 0 and flag == 0
    _compare(b, got, st, ref, st_ref, mag, "decode-shaped conv1d")
