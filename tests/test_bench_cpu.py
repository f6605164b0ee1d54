"""bench.py's host side on the CPU: the one-GPU contract and the algorithmic
work behind the roofline fractions (hand-computed byte counts)."""
import os
import subprocess
import sys

import numpy as np

import bench
from selective_state_space_cu_amd.workloads import make_config, make_decode_config, make_decode_inputs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_prefix_cache_algorithmic_bytes():
    # per token: x and y (32 heads x 128 x 2 bytes each), dt (32 x 4), B and C (4 groups x 128 x 2
    # each); 4 final states and 140 block checkpoints of 32 x 128 x 128 x 4 bytes
    w = make_config(4)
    per_token = 2 * 32 * 128 * 2 + 32 * 4 + 2 * 4 * 128 * 2
    state = 32 * 128 * 128 * 4
    want = 35576 * per_token + 4 * state + 140 * state
    got, flops = bench.algorithmic_work(w, 140)
    assert got == want == 962_280_448
    assert flops > 0


def test_decode_algorithmic_bytes():
    b = make_decode_config()
    state = 32 * 128 * 128 * 4
    want = 256 * 2 * state + 256 * (2 * 32 * 128 * 2 + 32 * 4 + 2 * 4 * 128 * 2)
    assert bench.decode_work(b) == want == 1_078_493_184


def test_decode_batches_respect_the_slot_precondition():
    """Write slots are unique and never another sequence's read slot."""
    for anchors in ("dual", "mixed", "inplace"):
        b = make_decode_inputs(40, 2, 4, 4, 1, 100, anchors=anchors, seed=11)
        rs, ws = b.read_slot.numpy(), b.write_slot.numpy()
        w = ws[ws >= 0]
        assert len(np.unique(w)) == len(w)
        for i, slot in enumerate(ws):
            if slot >= 0:
                others = np.delete(rs, i)
                assert slot not in others


def test_counter_ingest_counts_only_the_steps_before_the_calibration_copy(tmp_path):
    """rocprofv3 --pmc rows: two scan steps (800 KiB), small torch kernels, the
    calibration copy (512 MiB read and written: FETCH_SIZE reads half, as in the
    real counter), then export-overhead launches that write less. Only the two
    steps before the copy count."""
    import csv as _csv
    import json as _json
    hdr = ["Dispatch_Id", "Kernel_Name", "Counter_Value"]

    def write(path, calib, late):
        rows = [(1, "void at::native::vectorized_elementwise_kernel<fill>", 0.03),
                (2, "void ssd::ssd_scan_split_kernel<128, false>(ssd::ScanArgs)", 800.0),
                (3, "void at::native::vectorized_elementwise_kernel<fill>", 0.03),
                (4, "void ssd::ssd_scan_split_kernel<128, false>(ssd::ScanArgs)", 800.0),
                (5, "void at::native::vectorized_elementwise_kernel<add>", calib),
                (6, "void at::native::vectorized_elementwise_kernel<fill>", 0.5)]
        rows += [(7 + i, "void ssd::ssd_scan_split_kernel<128, false>(ssd::ScanArgs)", late) for i in range(10)]
        with open(path, "w", newline="") as f:
            wr = _csv.writer(f)
            wr.writerow(hdr)
            wr.writerows(rows)

    fc, wc, out = tmp_path / "f.csv", tmp_path / "w.csv", tmp_path / "rec.json"
    write(fc, 512 * 1024 / 2, 100.0)
    write(wc, 512 * 1024, 100.0)
    rec = bench.ingest_counters(str(fc), str(wc), 4, 512, out=str(out))
    assert rec["dispatches"] == 2
    assert rec["fetch_scale"] == 2.0 and rec["write_scale"] == 1.0
    assert rec["hbm_bytes_per_launch"] == (800.0 * 2.0 + 800.0 * 1.0) * 1024.0
    assert _json.load(open(out)) == rec


def test_conv1d_algorithmic_bytes():
    """4 x 8894 tokens x 5120 bf16 channels read and written, 4 read and 4
    written slots of 3 x 5120 bf16, 5120 x 4 + 5120 float32 weights and bias."""
    from selective_state_space_cu_amd.workloads import make_conv_config
    b = make_conv_config()
    want = 2 * 35576 * 5120 * 2 + 8 * 3 * 5120 * 2 + 5120 * 4 * 4 + 5120 * 4
    assert want == 728_944_640
    assert bench.conv1d_work(b) == want


def test_gdn_algorithmic_bytes():
    """4 x 8894 tokens; q and k (16 key heads x 128 bf16) read once, v read and o
    written (32 value heads x 128 bf16), gate and beta (32 float32 each); no
    initial states, 4 final states and 140 block checkpoints (35 blocks of 256
    tokens per sequence) of 32 x 128 x 128 float32. Shapes only: the tensors live
    on the meta device, so nothing is drawn."""
    from types import SimpleNamespace

    import torch

    from selective_state_space_cu_amd.workloads import GDN_CONFIG as c
    assert (c["lengths"], c["nheads"], c["nkheads"], c["dk"], c["dv"], c["chunk_size"], c["block_size"]) == \
        ([8894] * 4, 32, 16, 128, 128, 64, 256)
    T = sum(c["lengths"])
    w = SimpleNamespace(q=torch.empty(T, 16, 128, device="meta"), v=torch.empty(T, 32, 128, device="meta"),
                        has_initial_state=torch.zeros(4, dtype=torch.bool), nseqs=4, lengths=c["lengths"],
                        chunk_size=64)
    per_token = 2 * 16 * 128 * 2 + 2 * 32 * 128 * 2 + 2 * 32 * 4
    state = 32 * 128 * 128 * 4
    want = 35576 * per_token + 4 * state + 140 * state
    got, flops = bench.gdn_work(w, 140)
    assert got == want == 1_185_413_120
    # flops: 138 full chunks and one of 62 tokens per sequence; the full chunk's count
    # by hand (lower triangles of 2080 entries)
    full = 2 * 32 * (2 * 2080 * 128 + 2 * 64 * 128 * 128 + 2 * 2080 * 128 + 64 * 128 * 128)
    assert full == 269_484_032
    tail = 2 * 32 * (2 * 1953 * 128 + 2 * 62 * 128 * 128 + 2 * 1953 * 128 + 62 * 128 * 128)
    assert flops == 4 * (138 * full + tail)


def test_other_prefill_workloads_algorithmic_bytes():
    """The 8-sequence layer: 15843 tokens, per token x and y (80 heads x 64 bf16
    each), dt (80 float32), B and C (1 group x 128 bf16 each); 4 initial and 8
    final states of 80 x 64 x 128 float32. The 64-sequence batch: 17252 tokens,
    per token x and y (128 x 64 bf16), dt (128 float32), B and C (8 x 128 bf16);
    64 initial and 64 final states of 128 x 64 x 128 float32. Shapes only, from
    the workload table, so nothing is drawn."""
    from types import SimpleNamespace

    from selective_state_space_cu_amd.workloads import CONFIGS

    def shapes(i):
        c = CONFIGS[i]
        has = np.zeros(len(c["lengths"]), dtype=bool)
        has[c["init_seqs"]] = True
        return SimpleNamespace(total_tokens=sum(c["lengths"]), nheads=c["nheads"], headdim=c["headdim"],
                               dstate=c["dstate"], ngroups=c["ngroups"], dtype=c["dtype"], has_initial_state=has,
                               nseqs=len(c["lengths"]), lengths=c["lengths"], chunk_size=c["chunk_size"])

    want2 = 15843 * (2 * 80 * 64 * 2 + 80 * 4 + 2 * 128 * 2) + (4 + 8) * 80 * 64 * 128 * 4
    assert bench.algorithmic_work(shapes(2), 0)[0] == want2 == 369_103_296
    want3 = 17252 * (2 * 128 * 64 * 2 + 128 * 4 + 2 * 8 * 128 * 2) + (64 + 64) * 128 * 64 * 128 * 4
    assert bench.algorithmic_work(shapes(3), 0)[0] == want3 == 1_181_681_664
