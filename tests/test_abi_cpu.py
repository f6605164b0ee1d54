"""The C ABI on the CPU: the library loads, exports every declared symbol, and
rejects bad arguments synchronously (no GPU needed: nothing is launched)."""
import ctypes
import os
import re

import pytest

from selective_state_space_cu_amd import ssd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ssd.h")

pytestmark = pytest.mark.skipif(not os.path.exists(ssd.LIB_PATH), reason="libssd.so not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(ssd_\w+)\s*\(", text, flags=re.M)))


def test_exports_every_declared_symbol():
    lib = ssd.load_library()
    names = declared_functions()
    assert set(names) == set(ssd.EXPORTS), names
    for n in names:
        assert getattr(lib, n) is not None


def test_status_strings():
    assert ssd.status_string(0) == "ok"
    for code in range(1, 9):
        assert ssd.status_string(code) not in ("ok", "unknown status")
    assert ssd.status_string(99) == "unknown status"


FAKE = 0x1000  # a non-NULL, 16-byte aligned address that is never dereferenced


def _meta(S=2, T=100, cs=64, max_chunks=None, null_field=None):
    mc = T // cs + S if max_chunks is None else max_chunks
    m = ssd._Meta(S, T, cs, mc, *([FAKE] * 7))
    if null_field:
        setattr(m, null_field, None)
    return m


def _scan(m, **kw):
    args = dict(x=FAKE, dt=FAKE, dt_bias=None, A=FAKE, B=FAKE, C=FAKE, D=None, dtype=1, H=4, P=64,
                N=128, G=2, init=None, has=None, y=FAKE, final=FAKE, cst=None, dst=None, cap=0)
    args.update(kw)
    lib = ssd.load_library()
    return lib.ssd_chunk_scan_varlen(args["x"], args["dt"], args["dt_bias"], args["A"], args["B"],
                                     args["C"], args["D"], args["dtype"], ctypes.byref(m), args["H"],
                                     args["P"], args["N"], args["G"], args["init"], args["has"],
                                     args["y"], args["final"], args["cst"], args["dst"], args["cap"],
                                     None)


@pytest.mark.parametrize("cs", [0, 8, 17, 48, 100, 512, -64])
def test_metadata_rejects_bad_chunk_size(cs):
    lib = ssd.load_library()
    m = _meta(cs=cs, max_chunks=1000)
    assert lib.ssd_varlen_metadata(ctypes.byref(m), None) == 2


def test_metadata_rejects_small_capacity_and_nulls():
    lib = ssd.load_library()
    assert lib.ssd_varlen_metadata(ctypes.byref(_meta(S=3, T=128, cs=16, max_chunks=10)), None) == 5
    assert lib.ssd_varlen_metadata(None, None) == 1
    for f in ("cu_seqlens", "chunk_offsets", "chunk_seq_idx", "seq_chunk_start", "nchunks",
              "seq_order", "error_flag"):
        assert lib.ssd_varlen_metadata(ctypes.byref(_meta(null_field=f)), None) == 1
    assert lib.ssd_varlen_metadata(ctypes.byref(_meta(S=-1)), None) == 3


def test_scan_argument_errors():
    m = _meta()
    assert _scan(m, H=6, G=4) == 3                 # nheads % ngroups
    assert _scan(m, H=0) == 3
    assert _scan(m, P=40) == 8                     # headdim % 16
    assert _scan(m, N=48) == 8                     # dstate
    assert _scan(m, N=256, dtype=0) == 8           # f32 dstate 256
    assert _scan(m, dtype=5) == 6
    assert _scan(m, x=None) == 1
    assert _scan(m, A=None) == 1
    assert _scan(m, final=None) == 1
    assert _scan(m, y=FAKE + 4) == 3               # misaligned
    assert _scan(m, cst=FAKE, cap=0) == 5
    assert _scan(m, cst=FAKE, cap=2) == 5          # dense export needs max_chunks slots
    assert _scan(_meta(cs=24, max_chunks=100)) == 2


def test_export_argument_errors():
    lib = ssd.load_library()
    m = _meta()

    def call(bs=128, bt=FAKE, maxb=4, src=FAKE, dst=FAKE, cst=None, elems=0, cache=None, slots=8):
        return lib.ssd_export_chunk_states(ctypes.byref(m), None, bt, maxb, bs, src, dst, cst, elems,
                                           cache, slots, None)
    assert call(bs=96) == 4          # not a multiple of chunk_size
    assert call(bs=0) == 4
    assert call(bt=None) == 1
    assert call(dst=None) == 1
    assert call(cst=FAKE, cache=None) == 1
    assert call(cst=FAKE, cache=FAKE, elems=6) == 3
    assert call(maxb=-1) == 3


def _decode(**kw):
    args = dict(x=FAKE, dt=FAKE, dt_bias=None, A=FAKE, B=FAKE, C=FAKE, D=None, dtype=1, S=4, H=4,
                P=64, N=128, G=2, cache=FAKE, slots=8, rs=FAKE, ws=FAKE, y=FAKE, flag=None)
    args.update(kw)
    lib = ssd.load_library()
    return lib.ssd_decode_step(args["x"], args["dt"], args["dt_bias"], args["A"], args["B"],
                               args["C"], args["D"], args["dtype"], args["S"], args["H"],
                               args["P"], args["N"], args["G"], args["cache"], args["slots"],
                               args["rs"], args["ws"], args["y"], args["flag"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=7), 6), (dict(G=3), 3), (dict(H=0), 3), (dict(S=-1), 3), (dict(slots=-1), 3),
    (dict(N=48), 8), (dict(N=512), 8), (dict(x=None), 1), (dict(rs=None), 1), (dict(ws=None), 1),
    (dict(cache=None), 1), (dict(A=None), 1), (dict(cache=FAKE + 4), 3),
])
def test_decode_rejects_bad_arguments(kw, code):
    assert _decode(**kw) == code


def test_decode_empty_batch_launches_nothing():
    assert _decode(S=0, x=None, dt=None, B=None, C=None, y=None, cache=None, rs=None, ws=None) == 0


def _conv(m=None, **kw):
    args = dict(x=FAKE, w=FAKE, bias=None, dtype=1, C=64, W=4, act=1, states=FAKE, slots=8, rs=FAKE,
                ws=FAKE, out=FAKE)
    args.update(kw)
    lib = ssd.load_library()
    m = _meta() if m is None else m
    return lib.ssd_causal_conv1d_varlen(args["x"], args["w"], args["bias"], args["dtype"], ctypes.byref(m),
                                        args["C"], args["W"], args["act"], args["states"], args["slots"],
                                        args["rs"], args["ws"], args["out"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=7), 6), (dict(C=0), 3), (dict(C=-8), 3), (dict(slots=-1), 3), (dict(C=12), 8),
    (dict(W=0), 8), (dict(W=5), 8), (dict(act=2), 8), (dict(x=None), 1), (dict(out=None), 1),
    (dict(w=None), 1), (dict(states=None), 1), (dict(states=FAKE + 4), 3), (dict(x=FAKE + 8), 3),
    (dict(out=FAKE + 2), 3),
])
def test_conv1d_rejects_bad_arguments(kw, code):
    assert _conv(**kw) == code


def test_conv1d_rejects_bad_meta():
    assert _conv(m=_meta(null_field="chunk_seq_idx")) == 1
    assert _conv(m=_meta(cs=48)) == 2
    assert _conv(m=_meta(max_chunks=1)) == 5


def test_conv1d_empty_batch_launches_nothing():
    assert _conv(m=_meta(S=0, T=0, max_chunks=0), x=None, out=None, states=None, rs=None, ws=None) == 0


def test_bindings_refuse_mismatched_shapes():
    """The Python bindings check every tensor's shape against x, B and the
    metadata before anything reaches the device."""
    import torch
    z = lambda *s, dt=torch.float32: torch.zeros(*s, dtype=dt)
    meta = ssd.VarlenMeta(2, 10, 16, 3, *([z(1, dt=torch.int32)] * 7))
    x = z(10, 16)
    with pytest.raises(ValueError, match="weight"):
        ssd.causal_conv1d_varlen(x, z(8, 4), meta)
    with pytest.raises(ValueError, match="conv_states"):
        ssd.causal_conv1d_varlen(x, z(16, 4), meta, conv_states=z(4, 4, 16))
    with pytest.raises(ValueError, match="read_slot"):
        ssd.causal_conv1d_varlen(x, z(16, 4), meta, read_slot=z(3, dt=torch.int32))
    with pytest.raises(ValueError, match="tokens"):
        ssd.causal_conv1d_varlen(z(11, 16), z(16, 4), meta)
    xs = z(10, 4, 8)
    with pytest.raises(ValueError, match="B must"):
        ssd.chunk_scan_varlen(xs, z(10, 4), z(4), z(9, 2, 16), z(9, 2, 16), meta)
    with pytest.raises(ValueError, match="C must"):
        ssd.chunk_scan_varlen(xs, z(10, 4), z(4), z(10, 2, 16), z(10, 2, 8), meta)
    with pytest.raises(ValueError, match="initial_states"):
        ssd.chunk_scan_varlen(xs, z(10, 4), z(4), z(10, 2, 16), z(10, 2, 16), meta,
                              initial_states=z(3, 4, 8, 16))
    xd = z(3, 4, 8)
    with pytest.raises(ValueError, match="write_slot"):
        ssd.decode_step(xd, z(3, 4), z(4), z(3, 2, 16), z(3, 2, 16), z(6, 4, 8, 16),
                        z(3, dt=torch.int32), z(2, dt=torch.int32))
    with pytest.raises(ValueError, match="state_cache"):
        ssd.decode_step(xd, z(3, 4), z(4), z(3, 2, 16), z(3, 2, 16), z(6, 4, 8, 32),
                        z(3, dt=torch.int32), z(3, dt=torch.int32))
