"""Pins of the CPU oracle against facts fixed by the pages and by mathematics.

Each pin takes an oracle library handle, so the same checks run against the
real oracle (tests/test_oracle_pins.py) and against deliberately broken copies
of it (tests/test_oracle_mutations.py), which must each fail at least one pin.
"""
import json
import math
import os

import numpy as np

import oracle
from ssd_brute import chunked, gdn_chunked, semiseparable
from selective_state_space_cu_amd.workloads import (make_config, make_conv_inputs, make_decode_inputs,
                                                     make_inputs)

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _run(lib, w, chunk_size=0, init=True):
    return oracle.ssd_varlen(w.x, w.dt, w.dt_bias, w.A, w.B, w.C, w.D, w.cu_seqlens,
                             w.initial_states if init else None,
                             w.has_initial_state if init else None, chunk_size=chunk_size, lib=lib)


def _close(a, b, tol, what):
    a, b = np.asarray(a), np.asarray(b)
    err = np.max(np.abs(a - b)) if a.size else 0.0
    scale = max(1.0, float(np.max(np.abs(b)))) if b.size else 1.0
    assert np.all(np.isfinite(a)), f"{what}: non-finite values"
    assert err <= tol * scale, f"{what}: max abs err {err:.3e} > {tol:.1e}*{scale:.2f}"


def _tiny_cases():
    # (lengths, H, P, N, G, init_seqs, seed): varlen, zero-length, groups, P != N
    return [([5, 0, 11, 3], 4, 3, 2, 2, [0, 2], 11),
            ([17, 9], 2, 2, 4, 1, [1], 12),
            ([1, 30, 2], 6, 4, 3, 3, [0, 1, 2], 13),
            ([40], 1, 1, 1, 1, [0], 14)]


def pin_brute_force_semiseparable(lib):
    """Oracle == materialised semiseparable matrix on tiny inputs (1e-12)."""
    for L, H, P, N, G, ini, seed in _tiny_cases():
        w = make_inputs(L, H, P, N, G, 4, dtype="f32", init_seqs=ini, seed=seed)
        y, fin, _ = _run(lib, w)
        yb, fb = semiseparable(w.x, w.dt, w.dt_bias, w.A, w.B, w.C, w.D, w.cu_seqlens,
                               w.initial_states, w.has_initial_state)
        _close(y, yb, 1e-12, f"y vs semiseparable {L}")
        _close(fin, fb, 1e-12, f"final vs semiseparable {L}")


def pin_scalar_closed_form(lib):
    """P=N=1, B=C=x=1, constant delta: h_t = a^(t+1) h0 + delta (1-a^(t+1))/(1-a), y = h + D."""
    delta, Ah, h0, D, T = 0.5, -0.7, 0.3, 0.25, 37
    u = math.log(math.expm1(delta))          # the argument whose softplus is exactly `delta`
    ones = np.ones((T, 1, 1))
    y, fin, _ = oracle.ssd_varlen(ones, np.full((T, 1), u), np.zeros(1), np.array([Ah]), ones,
                                  ones, np.array([D]), np.array([0, T], np.int32),
                                  np.full((1, 1, 1, 1), h0), np.array([1], np.int32), lib=lib)
    a = math.exp(delta * Ah)
    t = np.arange(T)
    h = a ** (t + 1) * h0 + delta * (1 - a ** (t + 1)) / (1 - a)
    _close(y[:, 0, 0], h + D, 1e-12, "scalar closed form y")
    _close(fin[0, 0, 0, 0], h[-1], 1e-12, "scalar closed form final")


def pin_linear_attention(lib):
    """A = 0: h_t = h0 + sum_{k<=t} delta_k x_k B_k^T (prefix sums), y_t = C_t h_t + D x_t."""
    w = make_inputs([9, 14, 1], 4, 3, 5, 2, 4, init_seqs=[1], seed=21)
    A0 = np.zeros(4)
    y, fin, _ = oracle.ssd_varlen(w.x, w.dt, w.dt_bias, A0, w.B, w.C, w.D, w.cu_seqlens,
                                  w.initial_states, w.has_initial_state, lib=lib)
    x, B, C = (v.double().numpy() for v in (w.x, w.B, w.C))
    delta = np.logaddexp(0.0, w.dt.double().numpy() + w.dt_bias.double().numpy()[None])
    D = w.D.double().numpy()
    cu = w.cu_seqlens.numpy()
    for s in range(3):
        t0, t1 = cu[s], cu[s + 1]
        for h in range(4):
            g = h // 2
            h0 = w.initial_states[s, h].double().numpy() if w.has_initial_state[s] else 0.0
            upd = np.einsum("t,tp,tn->tpn", delta[t0:t1, h], x[t0:t1, h], B[t0:t1, g])
            hs = h0 + np.cumsum(upd, axis=0)
            yr = np.einsum("tpn,tn->tp", hs, C[t0:t1, g]) + D[h] * x[t0:t1, h]
            _close(y[t0:t1, h], yr, 1e-12, "A=0 y")
            _close(fin[s, h], hs[-1], 1e-12, "A=0 final")


def pin_diagonal_limit(lib):
    """A = -1e4 with delta ~ 1.3: only the current token survives:
    y_t = delta_t (C_t.B_t) x_t + D x_t, final = delta_last x_last B_last^T."""
    w = make_inputs([6, 3], 2, 3, 4, 1, 4, init_seqs=[0, 1], seed=31)
    delta = 1.25
    u = math.log(math.expm1(delta))
    T = w.total_tokens
    y, fin, _ = oracle.ssd_varlen(w.x, np.full((T, 2), u), np.zeros(2), np.full(2, -1e4), w.B,
                                  w.C, w.D, w.cu_seqlens, w.initial_states, w.has_initial_state,
                                  lib=lib)
    x, B, C, D = (v.double().numpy() for v in (w.x, w.B, w.C, w.D))
    cb = np.einsum("tn,tn->t", C[:, 0], B[:, 0])
    yr = delta * cb[:, None, None] * x + D[None, :, None] * x
    _close(y, yr, 1e-12, "diagonal limit y")
    cu = w.cu_seqlens.numpy()
    for s in range(2):
        t = cu[s + 1] - 1
        _close(fin[s], delta * np.einsum("hp,n->hpn", x[t], B[t, 0]), 1e-12, "diagonal final")


def pin_zero_dt(lib):
    """dt_bias = -1e4 makes softplus exactly 0: state unchanged, y = C.h0 + D x."""
    w = make_inputs([7, 12], 2, 3, 4, 2, 4, init_seqs=[0, 1], seed=41)
    y, fin, _ = oracle.ssd_varlen(w.x, w.dt, np.full(2, -1e4), w.A, w.B, w.C, w.D, w.cu_seqlens,
                                  w.initial_states, w.has_initial_state, lib=lib)
    h0 = w.initial_states.double().numpy()
    _close(fin, h0, 0.0, "dt=0 final == init")
    x, C, D = (v.double().numpy() for v in (w.x, w.C, w.D))
    cu = w.cu_seqlens.numpy()
    for s in range(2):
        for h in range(2):
            t0, t1 = cu[s], cu[s + 1]
            yr = C[t0:t1, h] @ h0[s, h].T + D[h] * x[t0:t1, h]
            _close(y[t0:t1, h], yr, 1e-12, "dt=0 y")


def pin_superposition(lib):
    """Linear in (x, h0): y(x,h0) = y(x,0) + y(0,h0); y(2x,0) = 2 y(x,0)."""
    w = make_inputs([13, 20], 2, 4, 3, 1, 4, init_seqs=[0, 1], seed=51)
    args = (w.dt, w.dt_bias, w.A, w.B, w.C)
    xz = np.zeros(w.x.shape)
    y_full, f_full, _ = oracle.ssd_varlen(w.x, *args, w.D, w.cu_seqlens, w.initial_states,
                                          w.has_initial_state, lib=lib)
    y_x, f_x, _ = oracle.ssd_varlen(w.x, *args, w.D, w.cu_seqlens, lib=lib)
    y_h, f_h, _ = oracle.ssd_varlen(xz, *args, w.D, w.cu_seqlens, w.initial_states,
                                    w.has_initial_state, lib=lib)
    _close(y_full, y_x + y_h, 1e-12, "superposition y")
    _close(f_full, f_x + f_h, 1e-12, "superposition final")
    y2, _, _ = oracle.ssd_varlen(2 * w.x.double().numpy(), *args, w.D, w.cu_seqlens, lib=lib)
    _close(y2, 2 * y_x, 1e-12, "homogeneity")


def pin_no_leakage(lib):
    """A packed batch equals each sequence run alone, bit for bit."""
    w = make_inputs([11, 4, 0, 23], 2, 3, 4, 2, 4, init_seqs=[0, 3], seed=61)
    y, fin, _ = _run(lib, w)
    cu = w.cu_seqlens.numpy()
    for s in range(4):
        t0, t1 = cu[s], cu[s + 1]
        ys, fs, _ = oracle.ssd_varlen(w.x[t0:t1], w.dt[t0:t1], w.dt_bias, w.A, w.B[t0:t1],
                                      w.C[t0:t1], w.D, np.array([0, t1 - t0], np.int32),
                                      w.initial_states[s:s + 1], w.has_initial_state[s:s + 1],
                                      lib=lib)
        assert np.array_equal(ys, y[t0:t1]) and np.array_equal(fs[0], fin[s]), f"leak seq {s}"


def pin_chunked_decomposition(lib):
    """The chunked decomposition equals the recurrence at every chunk size
    (y, final states, and the state after each chunk)."""
    w = make_inputs([37, 1, 64, 50], 4, 3, 5, 2, 16, init_seqs=[0, 2], seed=71)
    for cs in (1, 4, 16, 32, 64):
        y, fin, cst = _run(lib, w, chunk_size=cs)
        yc, fc, sc = chunked(w.x, w.dt, w.dt_bias, w.A, w.B, w.C, w.D, w.cu_seqlens, cs,
                             w.initial_states, w.has_initial_state)
        _close(y, yc, 1e-10, f"chunked y cs={cs}")
        _close(fin, fc, 1e-10, f"chunked final cs={cs}")
        assert cst.shape == sc.shape, f"chunk count cs={cs}"
        _close(cst, sc, 1e-10, f"chunk states cs={cs}")


def pin_initial_state_decay(lib):
    """x = 0: y_t = exp(sum_{k<=t} a_k) C_t.h0 -- the entering state carries the decay of
    every token up to and including t (the quantity the initial-state bug under-decayed)."""
    w = make_inputs([10, 25], 2, 2, 3, 1, 4, init_seqs=[0, 1], seed=81)
    xz = np.zeros(w.x.shape)
    y, _, _ = oracle.ssd_varlen(xz, w.dt, w.dt_bias, w.A, w.B, w.C, None, w.cu_seqlens,
                                w.initial_states, w.has_initial_state, lib=lib)
    delta = np.logaddexp(0.0, w.dt.double().numpy() + w.dt_bias.double().numpy()[None])
    A = w.A.double().numpy()
    C = w.C.double().numpy()
    h0 = w.initial_states.double().numpy()
    cu = w.cu_seqlens.numpy()
    for s in range(2):
        t0, t1 = cu[s], cu[s + 1]
        for h in range(2):
            decay = np.exp(np.cumsum(delta[t0:t1, h] * A[h]))
            yr = decay[:, None] * (C[t0:t1, 0] @ h0[s, h].T)
            _close(y[t0:t1, h], yr, 1e-12, "init decay")


def pin_768_token_chunk128(lib):
    """The bug-fix page's larger case: 768 tokens, chunk_size 128 (8 heads, P=N=64, fp32,
    random initial state): the oracle equals the chunked decomposition at chunk sizes
    32/128/256, and the semiseparable form on two heads."""
    w = make_config(1)
    y, fin, _ = _run(lib, w)
    for cs in (32, 128, 256):
        yc, fc, _ = chunked(w.x, w.dt, w.dt_bias, w.A, w.B, w.C, w.D, w.cu_seqlens, cs,
                            w.initial_states, w.has_initial_state)
        _close(y, yc, 1e-10, f"768 y cs={cs}")
        _close(fin, fc, 1e-10, f"768 final cs={cs}")
    sl = slice(0, 2)
    yb, fb = semiseparable(w.x[:, sl], w.dt[:, sl], w.dt_bias[sl], w.A[sl], w.B, w.C, w.D[sl],
                           w.cu_seqlens, w.initial_states[:, sl], w.has_initial_state)
    _close(y[:, sl], yb, 1e-10, "768 y semiseparable")
    _close(fin[:, sl], fb, 1e-10, "768 final semiseparable")


# ----- integer outputs: chunk metadata and checkpoint plan -----

def brute_metadata(lengths, cs, max_chunks):
    """Enumerate the chunk grid the slow way (token by token)."""
    T = int(sum(lengths))
    offsets, seq_idx, start = [], [], []
    t = 0
    for s, L in enumerate(lengths):
        start.append(len(offsets))
        for i in range(L):
            if i % cs == 0:
                offsets.append(t + i)
                seq_idx.append(s)
        t += L
    n = len(offsets)
    start.append(n)
    offsets += [T] * (max_chunks + 1 - n)
    seq_idx += [-1] * (max_chunks - n)
    order = sorted(range(len(lengths)), key=lambda s: (-lengths[s], s))
    return dict(chunk_offsets=offsets, chunk_seq_idx=seq_idx, seq_chunk_start=start, nchunks=n,
                seq_order=order)


def _check_meta(got, ref, what):
    for k in ("chunk_offsets", "chunk_seq_idx", "seq_chunk_start", "seq_order"):
        assert list(np.asarray(got[k])) == list(ref[k]), f"{what}: {k}"
    assert got["nchunks"] == ref["nchunks"], f"{what}: nchunks"


def pin_metadata_enumeration(lib):
    """Oracle metadata == token-by-token enumeration; nchunks == sum ceil(L/cs)."""
    rng = np.random.default_rng(5)
    for trial in range(40):
        S = int(rng.integers(1, 12))
        lengths = [int(v) for v in rng.integers(0, 300, size=S)]
        if trial % 5 == 0:
            lengths[0] = lengths[-1] = 64     # ties
        cs = int(2 ** rng.integers(4, 9))
        mc = sum(lengths) // cs + S + 2
        cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
        got = oracle.varlen_metadata(cu, cs, mc, lib=lib)
        _check_meta(got, brute_metadata(lengths, cs, mc), f"trial {trial}")
        assert got["nchunks"] == sum(-(-L // cs) for L in lengths)


def pin_metadata_golden_tiny(lib):
    """The tiny workload's chunk grid, worked out by hand (tests/golden/tiny_metadata.json)."""
    with open(os.path.join(GOLDEN, "tiny_metadata.json")) as f:
        g = json.load(f)
    got = oracle.varlen_metadata(np.array(g["cu_seqlens"], np.int32), g["chunk_size"],
                                 g["max_chunks"], lib=lib)
    _check_meta(got, g["expected"], "tiny golden")


def pin_plan_prefix_cache_closed_form(lib):
    """4 x 8894 tokens, chunk 64, block 256: 139 chunks per sequence; interior blocks
    k = 0..33 take chunk 139 s + 4 k + 3; block 34 (190 tokens) takes the final state,
    chunk 139 s + 138. The resume block for token 6912 is k = 26 -> chunk 139 s + 107."""
    cu = np.array([0, 8894, 17788, 26682, 35576], np.int32)
    mc = 35576 // 64 + 4
    meta = oracle.varlen_metadata(cu, 64, mc, lib=lib)
    assert meta["nchunks"] == 556 and list(meta["seq_chunk_start"]) == [0, 139, 278, 417, 556]
    bt = np.arange(140, dtype=np.int32)[::-1].reshape(4, 35).copy()
    src, dst = oracle.checkpoint_plan(cu, meta["seq_chunk_start"], mc, bt, 256, 64, lib=lib)
    for s in range(4):
        for k in range(34):
            assert src[s, k] == 139 * s + 4 * k + 3, (s, k, src[s, k])
            assert dst[139 * s + 4 * k + 3] == bt[s, k]
        assert src[s, 34] == 139 * s + 138 and dst[139 * s + 138] == bt[s, 34]
        assert src[s, 26] == 139 * s + 107
    assert (dst >= 0).sum() == 140


def pin_plan_misaligned_and_resume(lib):
    """A computed prefix that is not chunk-aligned gets no interior checkpoints (only the
    final-state block); an aligned one (6912 = 27 blocks) maps blocks to exact chunk ends."""
    L = 1982
    cu = np.array([0, L, 2 * L], np.int32)
    mc = 2 * L // 64 + 2
    meta = oracle.varlen_metadata(cu, 64, mc, lib=lib)
    bt = np.arange(70, dtype=np.int32).reshape(2, 35)
    ncomp = np.array([6912, 6912 + 32], np.int32)
    src, dst = oracle.checkpoint_plan(cu, meta["seq_chunk_start"], mc, bt, 256, 64,
                                      num_computed_tokens=ncomp, lib=lib)
    c0, c1 = meta["seq_chunk_start"][0], meta["seq_chunk_start"][1]
    # sequence 0: blocks 27..33 interior (ends at 7168 + 256 i), block 34 gets the final state
    for k in range(27, 34):
        assert src[0, k] == c0 + ((k + 1) * 256 - 6912) // 64 - 1
    assert src[0, 34] == c1 - 1
    assert all(src[0, k] == -1 for k in range(27))
    # sequence 1: misaligned -> only its last block (6944+1981)//256 = 34 is written
    last = (6944 + L - 1) // 256
    assert [k for k in range(35) if src[1, k] >= 0] == [last]
    assert src[1, last] == meta["nchunks"] - 1


def gather_plan(cu, seq_chunk_start, max_chunks, block_table, bs, cs, ncomp=None):
    """Per-chunk formulation of the plan (each chunk asks which block ends with it)."""
    S, maxb = block_table.shape
    dst = np.full(max_chunks, -1, np.int64)
    for s in range(S):
        L = int(cu[s + 1] - cu[s])
        if L <= 0:
            continue
        nc = 0 if ncomp is None else int(ncomp[s])
        last = (nc + L - 1) // bs
        for c in range(int(seq_chunk_start[s]), int(seq_chunk_start[s + 1])):
            lc = c - int(seq_chunk_start[s])
            end = nc + min((lc + 1) * cs, L)
            if c == int(seq_chunk_start[s + 1]) - 1:
                dst[c] = block_table[s, last]
            elif nc % cs == 0 and end % bs == 0:
                dst[c] = block_table[s, end // bs - 1]
    return np.where(dst < 0, -1, dst)


def pin_plan_scatter_equals_gather(lib):
    """The oracle's block-loop plan equals the per-chunk formulation on random batches."""
    rng = np.random.default_rng(9)
    for trial in range(30):
        S = int(rng.integers(1, 7))
        cs = int(2 ** rng.integers(4, 7))
        bs = cs * int(rng.integers(1, 5))
        lengths = [int(v) for v in rng.integers(0, 700, size=S)]
        ncomp = (rng.integers(0, 6, size=S) * (cs if trial % 3 else 7)).astype(np.int32)
        maxb = max(((n + max(L, 1) - 1) // bs) + 1 for n, L in zip(ncomp, lengths))
        bt = rng.permutation(S * maxb).reshape(S, maxb).astype(np.int32)
        bt[rng.random(bt.shape) < 0.1] = -1
        cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
        mc = sum(lengths) // cs + S
        meta = oracle.varlen_metadata(cu, cs, mc, lib=lib)
        _, dst = oracle.checkpoint_plan(cu, meta["seq_chunk_start"], mc, bt, bs, cs,
                                        num_computed_tokens=ncomp, lib=lib)
        ref = gather_plan(cu, meta["seq_chunk_start"], mc, bt, bs, cs, ncomp)
        assert list(dst) == list(ref), f"trial {trial}"


# ---- continuation: the scheduler's prefill bites ------------------------------

def pin_bites_golden(lib):
    """Bites worked out by hand from the scheduler rule (tests/golden/prefill_bites.json)."""
    with open(os.path.join(GOLDEN, "prefill_bites.json")) as f:
        g = json.load(f)
    for c in g["cases"]:
        got = oracle.prefill_bites([c["start"]], [c["prompt_len"]], [c["budget"]], g["align"], lib=lib)
        assert int(got[0]) == c["num_scheduled"], (c, int(got[0]))


def pin_bites_invariants(lib):
    """On random prompts the bites tile [start, prompt_len) with at most `budget`
    tokens each; a bite that ends at or before the last boundary ends on the
    grid; only the first bite, or one past the last boundary, starts off it, and
    then it ends at the next boundary when that is <= the last boundary; a bite
    from the grid ends at the last boundary it can reach."""
    rng = np.random.default_rng(31)
    for trial in range(300):
        align = int(2 ** rng.integers(4, 10))
        budget = align * int(rng.integers(1, 9)) + int(rng.integers(0, align))
        plen = int(rng.integers(0, 20 * align))
        start = int(rng.integers(0, plen + 1)) if trial % 2 else int(rng.integers(0, plen // align + 1)) * align
        start = min(start, plen)
        bites = oracle.prefill_schedule(start, plen, budget, align, lib=lib)
        last_aligned = plen // align * align
        pos = start
        for i, (a, b) in enumerate(bites):
            assert a == pos and 0 < b - a <= budget, (trial, bites)
            if b <= last_aligned:
                assert b % align == 0, (trial, bites)
            if i > 0 and a < last_aligned:
                assert a % align == 0, (trial, bites)
            if a % align != 0 and (a // align + 1) * align <= last_aligned:
                assert b == (a // align + 1) * align, (trial, a, b)
            elif a % align == 0 and a + budget < last_aligned:
                assert b == (a + budget) // align * align, (trial, a, b)
            pos = b
        assert pos == plen


def pin_bites_checkpoints_exact(lib):
    """A prompt computed in scheduler bites (each bite's initial state = the previous
    bite's final state, the plan at num_computed_tokens = the bite's start) gives
    the same outputs as one pass, and every block whose end lies in the computed
    range gets a checkpoint equal to the one-pass state at that block end --
    also when the computation resumes from a start off the grid."""
    cs, bs, budget = 16, 64, 160
    L = 530
    w = make_inputs([L], 2, 3, 2, 1, cs, dtype="f32", init_seqs=[0], seed=41)
    y_full, _, cst_full = _run(lib, w, chunk_size=cs)
    nblocks = (L + bs - 1) // bs
    for start in (0, 64, 37, 515):
        # state after `start` tokens, from a one-pass run of the prefix
        if start > 0:
            wp = make_inputs([start], 2, 3, 2, 1, cs, dtype="f32", init_seqs=[0], seed=41)
            for k in ("x", "dt", "B", "C"):
                setattr(wp, k, getattr(w, k)[:start])
            for k in ("dt_bias", "A", "D", "initial_states"):
                setattr(wp, k, getattr(w, k))
            _, h, _ = _run(lib, wp)
        else:
            h = w.initial_states.double().numpy()
        got = {}
        for a, b in oracle.prefill_schedule(start, L, budget, bs, lib=lib):
            n = b - a
            wb = make_inputs([n], 2, 3, 2, 1, cs, dtype="f32", init_seqs=[0], seed=41)
            for k in ("x", "dt", "B", "C"):
                setattr(wb, k, getattr(w, k)[a:b])
            for k in ("dt_bias", "A", "D"):
                setattr(wb, k, getattr(w, k))
            wb.initial_states = torch_from(h)
            yb, h, cstb = _run(lib, wb, chunk_size=cs)
            _close(yb, y_full[a:b], 1e-12, f"bite [{a},{b}) y")
            cu = np.array([0, n], np.int32)
            meta = oracle.varlen_metadata(cu, cs, n // cs + 1, lib=lib)
            bt = np.arange(nblocks, dtype=np.int32)[None, :]
            src, _ = oracle.checkpoint_plan(cu, meta["seq_chunk_start"], n // cs + 1, bt, bs, cs,
                                            num_computed_tokens=np.array([a], np.int32), lib=lib)
            for k in range(nblocks):
                if src[0, k] >= 0:
                    got[k] = (cstb[src[0, k]], min((k + 1) * bs, b))
        # every block ending inside [start, L) (or ending the prompt) is covered, exactly
        want = [k for k in range(nblocks) if min((k + 1) * bs, L) > start]
        assert sorted(got) == want, (start, sorted(got), want)
        for k, (state, end) in got.items():
            assert end == min((k + 1) * bs, L), (start, k, end)
            _close(state, cst_full[(end + cs - 1) // cs - 1], 1e-12, f"start {start} block {k}")


def torch_from(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(np.asarray(a, np.float64)))


# ---- gated delta rule (GDN) ------------------------------------------------------

def gdn_inputs(lengths, H, G, dk, dv, seed, unit_keys=True, gate_scale=1.0, init=True):
    """Small float64 inputs: unit-norm keys, gates in (-gate_scale, 0], beta in (0, 1)."""
    rng = np.random.default_rng(seed)
    T = int(sum(lengths))
    q = rng.normal(size=(T, G, dk)) / math.sqrt(dk)
    k = rng.normal(size=(T, G, dk))
    if unit_keys:
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.normal(size=(T, H, dv))
    gate = -gate_scale * rng.uniform(0.0, 1.0, size=(T, H))
    beta = rng.uniform(0.05, 1.0, size=(T, H))
    h0 = rng.normal(0.0, 0.5, size=(len(lengths), H, dv, dk)) if init else None
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    return q, k, v, gate, beta, cu, h0


def _gdn(lib, q, k, v, gate, beta, cu, scale, h0, cs=0, has=None):
    return oracle.gated_delta(q, k, v, gate, beta, cu, scale, initial_states=h0, has_initial_state=has,
                              chunk_size=cs, lib=lib)


def pin_gdn_chunked_wy_form(lib):
    """The token loop equals an independent chunked (WY) evaluation -- a triangular
    solve per chunk -- at several chunk sizes, with partial chunks and states."""
    for lengths, H, G, dk, dv, seed in [([13, 0, 40, 7], 4, 2, 6, 5, 1), ([64, 33], 2, 1, 8, 8, 2),
                                        ([100], 3, 3, 4, 7, 3)]:
        q, k, v, gate, beta, cu, h0 = gdn_inputs(lengths, H, G, dk, dv, seed)
        for cs in (1, 3, 8, 16, 64):
            o, fin, cst = _gdn(lib, q, k, v, gate, beta, cu, 0.7, h0, cs)
            ob, fb, cb = gdn_chunked(q, k, v, gate, beta, cu, 0.7, h0, cs)
            _close(o, ob, 1e-10, f"gdn o cs={cs}")
            _close(fin, fb, 1e-10, f"gdn final cs={cs}")
            _close(cst, cb, 1e-10, f"gdn chunk states cs={cs}")


def pin_gdn_delta_write(lib):
    """With no decay and beta = 1, a write stores v_t under the unit key k_t exactly:
    the output read with q_t = k_t (scale 1) is v_t, whatever came before."""
    q, k, v, gate, beta, cu, h0 = gdn_inputs([30], 2, 1, 8, 3, 4)
    gate[:] = 0.0
    beta[:] = 1.0
    o, _, _ = _gdn(lib, k, k, v, gate, beta, cu, 1.0, h0)
    _close(o, v, 1e-12, "gdn delta write")


def pin_gdn_orthogonal_keys(lib):
    """Mutually orthogonal unit keys, no decay, zero initial state: the delta term
    vanishes and the layer is beta-weighted causal linear attention,
    o_t = scale sum_{j <= t} beta_j (q_t . k_j) v_j, h_T = sum_j beta_j k_j v_j^T."""
    T, dk, dv, H = 6, 8, 3, 2
    q, _, v, gate, beta, cu, _ = gdn_inputs([T], H, 1, dk, dv, 5, init=False)
    k = np.eye(dk)[:T][:, None, :]   # k_t = e_t
    gate[:] = 0.0
    o, fin, _ = _gdn(lib, q, k, v, gate, beta, cu, 0.5, None)
    for h in range(H):
        qk = q[:, 0] @ k[:, 0].T
        want = 0.5 * np.tril(qk) @ (beta[:, h, None] * v[:, h])
        _close(o[:, h], want, 1e-12, "gdn linear attention o")
        _close(fin[0, h], (k[:, 0].T @ (beta[:, h, None] * v[:, h])).T, 1e-12, "gdn linear attention S")


def pin_gdn_no_write(lib):
    """beta = 0: the state only decays, h_t = e^(sum of gates) h0, and
    o_t = scale e^(G_t) h0^T q_t."""
    q, k, v, gate, beta, cu, h0 = gdn_inputs([25, 9], 2, 2, 5, 4, 6)
    beta[:] = 0.0
    o, fin, _ = _gdn(lib, q, k, v, gate, beta, cu, 0.3, h0)
    for s in range(2):
        a, b = cu[s], cu[s + 1]
        for h in range(2):
            G = np.cumsum(gate[a:b, h])
            want = 0.3 * np.exp(G)[:, None] * (q[a:b, h] @ h0[s, h].T)
            _close(o[a:b, h], want, 1e-12, "gdn beta=0 o")
            _close(fin[s, h], np.exp(G[-1]) * h0[s, h], 1e-12, "gdn beta=0 h")


def pin_gdn_linear_in_values_and_state(lib):
    """For fixed q, k, gates and beta the layer is linear in (v, S0):
    o(v, h0) = o(v, 0) + o(0, h0), and likewise the final state."""
    q, k, v, gate, beta, cu, h0 = gdn_inputs([20, 31], 3, 1, 6, 4, 7)
    o, fin, _ = _gdn(lib, q, k, v, gate, beta, cu, 1.0, h0)
    o1, f1, _ = _gdn(lib, q, k, v, gate, beta, cu, 1.0, np.zeros_like(h0))
    o2, f2, _ = _gdn(lib, q, k, np.zeros_like(v), gate, beta, cu, 1.0, h0)
    _close(o, o1 + o2, 1e-12, "gdn superposition o")
    _close(fin, f1 + f2, 1e-12, "gdn superposition h")


def pin_gdn_no_leakage_and_init_flag(lib):
    """Packed sequences equal separate runs; a sequence without its flag starts from zero."""
    q, k, v, gate, beta, cu, h0 = gdn_inputs([11, 23, 5], 2, 1, 4, 3, 8)
    has = np.array([1, 0, 1], np.int32)
    o, fin, _ = _gdn(lib, q, k, v, gate, beta, cu, 1.0, h0, has=has)
    for s in range(3):
        a, b = cu[s], cu[s + 1]
        hs = h0[s:s + 1] if has[s] else np.zeros_like(h0[s:s + 1])
        os_, fs, _ = _gdn(lib, q[a:b], k[a:b], v[a:b], gate[a:b], beta[a:b], np.array([0, b - a], np.int32),
                          1.0, hs)
        _close(o[a:b], os_, 1e-14, f"gdn sequence {s} o")
        _close(fin[s:s + 1], fs, 1e-14, f"gdn sequence {s} h")


# ---- decode step with dual state anchors -------------------------------------

def _decode(lib, b, cache=None, rs=None, ws=None, dt_bias=None, A=None):
    return oracle.ssd_decode(b.x, b.dt, b.dt_bias if dt_bias is None else dt_bias,
                             b.A if A is None else A, b.B, b.C, b.D,
                             b.state_cache if cache is None else cache,
                             b.read_slot if rs is None else rs, b.write_slot if ws is None else ws,
                             lib=lib)


def _decode_cases():
    # (S, H, P, N, G, slots, anchors, seed)
    return [(7, 4, 3, 2, 2, 16, "mixed", 21), (3, 2, 4, 5, 1, 6, "dual", 22),
            (4, 6, 2, 3, 3, 4, "inplace", 23)]


def pin_decode_is_one_recurrence_token(lib):
    """A decode step equals the recurrence oracle over one-token sequences whose
    initial states are the read slots (zero for none); the write slots then hold
    its final states and every other slot is untouched."""
    for S, H, P, N, G, slots, anchors, seed in _decode_cases():
        b = make_decode_inputs(S, H, P, N, G, slots, anchors=anchors, seed=seed)
        y, cache, rc = _decode(lib, b)
        assert rc == 0, "decode refused valid slots"
        rs, ws = b.read_slot.numpy(), b.write_slot.numpy()
        c0 = b.state_cache.double().numpy()
        init = np.where((rs >= 0)[:, None, None, None], c0[np.maximum(rs, 0)], 0.0)
        yr, fr, _ = oracle.ssd_varlen(b.x, b.dt, b.dt_bias, b.A, b.B, b.C, b.D,
                                      np.arange(S + 1, dtype=np.int32), init,
                                      np.ones(S, np.int32), lib=lib)
        _close(y, yr, 1e-12, f"decode y vs recurrence ({anchors})")
        want = c0.copy()
        for i in range(S):
            if ws[i] >= 0:
                want[ws[i]] = fr[i]
        _close(cache, want, 1e-12, f"decode cache vs recurrence ({anchors})")
        untouched = np.setdiff1d(np.arange(slots), ws[ws >= 0])
        assert np.array_equal(cache[untouched], c0[untouched]), "decode wrote an unlisted slot"


def pin_decode_limits(lib):
    """dt_bias = -1e4 (delta = 0): the read state reaches the write slot bit for bit
    and y = C.h + D x; A = -1e6 (decay underflows to 0): the new state is
    delta x B^T alone and y = delta (C.B) x + D x."""
    b = make_decode_inputs(4, 3, 4, 5, 1, 8, anchors="dual", seed=31)
    rs, ws = b.read_slot.numpy(), b.write_slot.numpy()
    x, B, C, D = (v.double().numpy() for v in (b.x, b.B, b.C, b.D))
    c0 = b.state_cache.double().numpy()
    y, cache, _ = _decode(lib, b, dt_bias=np.full(3, -1e4))
    assert np.array_equal(cache[ws], c0[rs]), "delta = 0 changed the state"
    for i in range(4):
        yr = np.einsum("hpn,n->hp", c0[rs[i]], C[i, 0]) + D[:, None] * x[i]
        _close(y[i], yr, 1e-12, "delta = 0 y")
    delta = 0.75
    u = math.log(math.expm1(delta))
    y, cache, _ = oracle.ssd_decode(b.x, np.full((4, 3), u), np.zeros(3), np.full(3, -1e6), b.B,
                                    b.C, b.D, b.state_cache, b.read_slot, b.write_slot, lib=lib)
    for i in range(4):
        _close(cache[ws[i]], delta * np.einsum("hp,n->hpn", x[i], B[i, 0]), 1e-12, "no-decay state")
        yr = delta * float(C[i, 0] @ B[i, 0]) * x[i] + D[:, None] * x[i]
        _close(y[i], yr, 1e-12, "no-decay y")


def pin_decode_anchor_rules(lib):
    """Read slot < 0 equals reading an all-zero slot; write slot < 0 leaves the
    cache alone; in place (read == write) equals reading one slot and writing
    another; a slot past the cache is refused (-2) and its sequence skipped."""
    b = make_decode_inputs(5, 2, 3, 4, 2, 12, anchors="dual", seed=41)
    rs, ws = b.read_slot.numpy().copy(), b.write_slot.numpy().copy()
    c0 = b.state_cache.double().numpy()
    y_ref, cache_ref, _ = _decode(lib, b)
    zc = c0.copy()
    zc[rs[1]] = 0.0
    rs_none = rs.copy()
    rs_none[1] = -1
    y1, c1, _ = _decode(lib, b, rs=rs_none)
    y2, c2, _ = _decode(lib, b, cache=zc)
    assert np.array_equal(y1, y2) and np.array_equal(c1[ws], c2[ws]), "read < 0 is not a zero state"
    ws_none = np.full_like(ws, -1)
    y3, c3, _ = _decode(lib, b, ws=ws_none)
    assert np.array_equal(c3, c0) and np.array_equal(y3, y_ref), "write < 0 wrote or changed y"
    y4, c4, _ = _decode(lib, b, ws=rs)
    assert np.array_equal(y4, y_ref) and np.array_equal(c4[rs], cache_ref[ws]), "in place differs"
    bad = rs.copy()
    bad[2] = 12
    y5, c5, rc = _decode(lib, b, rs=bad)
    assert rc == -2, "out-of-range slot accepted"
    assert np.all(y5[2] == 0.0) and np.array_equal(c5[ws[2]], c0[ws[2]]), "bad sequence not skipped"
    others = [0, 1, 3, 4]
    assert np.array_equal(y5[others], y_ref[others]), "a bad slot disturbed other sequences"


def pin_decode_continues_prefill(lib):
    """Prefill of L tokens == prefill of L - 1 tokens whose final state sits in a
    cache slot, then one decode step reading it (last y and final state, 1e-12);
    and two decode steps chained through the cache (read a, write b; read b,
    write c) == the recurrence over two tokens."""
    L, H, P, N, G = 9, 4, 3, 5, 2
    w = make_inputs([L, L + 3], H, P, N, G, 4, init_seqs=[0], seed=51)
    y, fin, _ = _run(lib, w)
    cu = w.cu_seqlens.numpy()
    part = make_inputs([L - 1, L + 2], H, P, N, G, 4, init_seqs=[0], seed=51)
    keep = np.concatenate([np.arange(cu[0], cu[1] - 1), np.arange(cu[1], cu[2] - 1)])
    yp, fp, _ = oracle.ssd_varlen(w.x[keep], w.dt[keep], w.dt_bias, w.A, w.B[keep], w.C[keep], w.D,
                                  part.cu_seqlens, w.initial_states, w.has_initial_state, lib=lib)
    last = cu[1:] - 1
    cache = np.zeros((6, H, P, N))
    cache[[4, 1]] = fp
    yd, cd, rc = oracle.ssd_decode(w.x[last], w.dt[last], w.dt_bias, w.A, w.B[last], w.C[last], w.D,
                                   cache, np.array([4, 1], np.int32), np.array([0, 5], np.int32),
                                   lib=lib)
    assert rc == 0
    _close(yd, y[last], 1e-12, "decode after prefill y")
    _close(cd[[0, 5]], fin, 1e-12, "decode after prefill state")
    _close(yp, y[keep], 1e-12, "prefill prefix y")
    b = make_decode_inputs(6, 2, 3, 4, 1, 18, anchors="dual", seed=52)
    b2 = make_decode_inputs(6, 2, 3, 4, 1, 18, anchors="dual", seed=53)
    rs, ws = b.read_slot.numpy(), b.write_slot.numpy()
    free = np.setdiff1d(np.arange(18), np.concatenate([rs, ws]))
    ya, ca, _ = _decode(lib, b)
    yb, cb, _ = oracle.ssd_decode(b2.x, b2.dt, b.dt_bias, b.A, b2.B, b2.C, b.D, ca, ws, free,
                                  lib=lib)
    xs = np.stack([b.x.double().numpy(), b2.x.double().numpy()], 1).reshape(12, 2, 3)
    dts = np.stack([b.dt.double().numpy(), b2.dt.double().numpy()], 1).reshape(12, 2)
    Bs = np.stack([b.B.double().numpy(), b2.B.double().numpy()], 1).reshape(12, 1, 4)
    Cs = np.stack([b.C.double().numpy(), b2.C.double().numpy()], 1).reshape(12, 1, 4)
    c0 = b.state_cache.double().numpy()
    yr, fr, _ = oracle.ssd_varlen(xs, dts, b.dt_bias, b.A, Bs, Cs, b.D,
                                  np.arange(0, 13, 2, dtype=np.int32), c0[rs], np.ones(6, np.int32),
                                  lib=lib)
    _close(np.stack([ya, yb], 1).reshape(12, 2, 3), yr, 1e-12, "two chained decode steps y")
    _close(cb[free], fr, 1e-12, "two chained decode steps state")


# ---- varlen causal conv1d with a conv-state cache ------------------------------

def _conv(lib, b, states=None, rs=None, ws=None, silu=None, bias="keep"):
    return oracle.causal_conv1d(b.x, b.cu_seqlens, b.weight, b.bias if bias == "keep" else bias,
                                b.silu if silu is None else silu,
                                b.conv_states if states is None else states,
                                b.read_slot if rs is None else rs, b.write_slot if ws is None else ws,
                                lib=lib)


def pin_conv_is_numpy_convolve(lib):
    """No cached state, identity activation: each sequence's channel c is
    numpy.convolve(x_s[:, c], weight[c] reversed) truncated to the sequence,
    plus bias[c] (widths 1-4, empty and shorter-than-window sequences). Then
    with a cached state: the convolution of the cached rows followed by the
    sequence, keeping the sequence's outputs."""
    for W, lengths, seed in ((4, [7, 0, 2, 11], 61), (3, [1, 5], 62), (2, [6, 3, 4], 63), (1, [3, 4], 64)):
        b = make_conv_inputs(lengths, 5, W, 2 * len(lengths), seed=seed, silu=False)
        none = -np.ones(len(lengths), np.int32)
        out, _, rc = _conv(lib, b, rs=none)
        assert rc == 0
        x, w, bias = b.x.double().numpy(), b.weight.double().numpy(), b.bias.double().numpy()
        cu = b.cu_seqlens.numpy()
        states = b.conv_states.double().numpy()
        out2, _, _ = _conv(lib, b)
        for s in range(len(lengths)):
            xs = x[cu[s]:cu[s + 1]]
            if len(xs) == 0:   # no outputs (its state is pinned below)
                continue
            pre = np.concatenate([states[b.read_slot[s]], xs], 0)
            for c in range(5):
                want = np.convolve(xs[:, c], w[c, ::-1])[:len(xs)] + bias[c]
                _close(out[cu[s]:cu[s + 1], c], want, 1e-13, f"conv vs numpy.convolve W={W} s={s}")
                want2 = np.convolve(pre[:, c], w[c, ::-1])[W - 1:W - 1 + len(xs)] + bias[c]
                _close(out2[cu[s]:cu[s + 1], c], want2, 1e-13, f"conv after cached rows W={W} s={s}")


def pin_conv_silu(lib):
    """Width 1, weight 1, bias 0: the output is SiLU(x) = x * logistic(x), with
    the logistic from scipy; with silu off it is x itself."""
    from scipy.special import expit
    b = make_conv_inputs([9, 4], 6, 1, 4, seed=65)
    b.weight = torch_ones(6, 1)
    b.x = b.x * 4.0
    x = b.x.double().numpy()
    out, _, _ = _conv(lib, b, silu=True, bias=None)
    _close(out, x * expit(x), 1e-14, "SiLU")
    out, _, _ = _conv(lib, b, silu=False, bias=None)
    _close(out, x, 0.0, "identity activation")


def torch_ones(*shape):
    import torch
    return torch.ones(*shape)


def pin_conv_state_rows(lib):
    """The written state is the last W-1 rows of (cached rows, then the
    sequence): for long sequences the sequence's last W-1 inputs in order; for
    short and empty ones the tail of the cached rows followed by the inputs.
    Slots not written keep their contents; a write slot of -1 writes nothing;
    a read slot of -1 means zero leading inputs; a slot past the cache is
    refused (status -2, that sequence skipped)."""
    W = 4
    b = make_conv_inputs([10, 2, 0, 1, 5], 3, W, 12, seed=66, anchors="dual")
    _, st, rc = _conv(lib, b)
    assert rc == 0
    x, s0 = b.x.double().numpy(), b.conv_states.double().numpy()
    cu = b.cu_seqlens.numpy()
    for s in range(5):
        rows = np.concatenate([s0[b.read_slot[s]], x[cu[s]:cu[s + 1]]], 0)[-(W - 1):]
        assert np.array_equal(st[b.write_slot[s]], rows), f"state rows of sequence {s}"
    untouched = np.setdiff1d(np.arange(12), b.write_slot.numpy())
    assert np.array_equal(st[untouched], s0[untouched]), "conv wrote an unlisted slot"
    ws = b.write_slot.numpy().copy()
    ws[1] = -1
    _, st2, _ = _conv(lib, b, ws=ws)
    assert np.array_equal(st2[b.write_slot[1]], s0[b.write_slot[1]]), "write slot -1 wrote"
    zero = s0.copy()
    zero[b.read_slot[3]] = 0.0
    rs = b.read_slot.numpy().copy()
    rs[3] = -1
    o1, _, _ = _conv(lib, b, rs=rs)
    o2, _, _ = _conv(lib, b, states=zero)
    assert np.array_equal(o1, o2), "read slot -1 differs from a zero state"
    bad = b.read_slot.numpy().copy()
    bad[2] = 12
    o3, st3, rc = _conv(lib, b, rs=bad)
    o4, st4, _ = _conv(lib, b)
    assert rc == -2, "slot past the cache not refused"
    keep = np.setdiff1d(np.arange(5), [2])
    assert np.array_equal(st3[b.write_slot[keep]], st4[b.write_slot[keep]])
    assert np.array_equal(st3[b.write_slot[2]], s0[b.write_slot[2]]), "refused sequence wrote"


def pin_conv_split_invariance(lib):
    """A sequence convolved in two parts, the first part's state written to a
    slot that the second part reads, gives the same outputs and final state as
    the whole sequence (split points inside and at the window's reach)."""
    W, L = 4, 13
    whole = make_conv_inputs([L], 4, W, 2, seed=67)
    x = whole.x.double().numpy()
    out, st, _ = _conv(lib, whole)
    for cut in (1, 2, 3, 7, 12):
        b1 = make_conv_inputs([cut], 4, W, 2, seed=67)
        b1.x = whole.x[:cut]
        b1.weight, b1.bias, b1.conv_states = whole.weight, whole.bias, whole.conv_states
        o1, s1, _ = _conv(lib, b1, rs=whole.read_slot, ws=np.array([1 - whole.read_slot[0]], np.int32))
        b2 = make_conv_inputs([L - cut], 4, W, 2, seed=67)
        b2.x = whole.x[cut:]
        b2.weight, b2.bias = whole.weight, whole.bias
        o2, s2, _ = _conv(lib, b2, states=s1, rs=np.array([1 - whole.read_slot[0]], np.int32),
                          ws=whole.write_slot)
        _close(np.concatenate([o1, o2], 0), out, 1e-14, f"split at {cut}: outputs")
        assert np.array_equal(s2[whole.write_slot[0]], st[whole.write_slot[0]]), f"split at {cut}: state"
    del x


ALL_PINS = [pin_brute_force_semiseparable, pin_scalar_closed_form, pin_linear_attention,
            pin_diagonal_limit, pin_zero_dt, pin_superposition, pin_no_leakage,
            pin_chunked_decomposition, pin_initial_state_decay, pin_768_token_chunk128,
            pin_metadata_enumeration, pin_metadata_golden_tiny,
            pin_plan_prefix_cache_closed_form, pin_plan_misaligned_and_resume,
            pin_plan_scatter_equals_gather, pin_bites_golden, pin_bites_invariants,
            pin_bites_checkpoints_exact, pin_gdn_chunked_wy_form, pin_gdn_delta_write,
            pin_gdn_orthogonal_keys, pin_gdn_no_write, pin_gdn_linear_in_values_and_state,
            pin_gdn_no_leakage_and_init_flag, pin_decode_is_one_recurrence_token,
            pin_decode_limits, pin_decode_anchor_rules, pin_decode_continues_prefill,
            pin_conv_is_numpy_convolve, pin_conv_silu, pin_conv_state_rows, pin_conv_split_invariance]
