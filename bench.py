"""Benchmark of the varlen SSD scan hot path on one MI355X.

One step = the whole hot path over one batch already resident in HBM:
  ssd_varlen_metadata  (chunk grid)
  ssd_export_chunk_states  (block-checkpoint plan)
  ssd_chunk_scan_varlen  (scan, writing the block checkpoints at the source)
on the prefix-cache checkpoint workload (4 sequences x 8894 tokens, 32 heads,
headdim 128, dstate 128, 4 groups, chunk 64, 256-token blocks, bf16 inputs,
float32 state). Prints one JSON line.

  python bench.py [--steps K] [--warmup W] [--config I] [--no-cpu-baseline]
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 matrix, TFLOP/s
# Untimed steps before the warm-up, for at least this long: after idle the GPU
# clock takes some tens of milliseconds of sustained work to reach its
# steady-state level (the first ~80 back-to-back prefix-cache scans run up to
# 25 % slower), so the timed steps see the clock a serving loop runs at.
CLOCK_SETTLE_S = 0.2
DECODE_COUNTERS = os.path.join(ROOT, "profiles", "decode_dual_anchor_256_counters.json")
KERNEL_SOURCES = ["ssd_scan.hpp", "ssd_scan_bf16.hip", "ssd_scan_f32.hip", "ssd_internal.h",
                  "ssd_scan_split.hpp", "ssd_scan_split_bf16.hip", "ssd_scan_ws.hpp", "ssd_scan_ws_bf16.hip"]
DECODE_SOURCES = ["ssd_decode.hip", "ssd_scan.hpp", "ssd_internal.h"]
CONV_COUNTERS = os.path.join(ROOT, "profiles", "conv1d_prefix_cache_4x8894_counters.json")
CONV_SOURCES = ["ssd_conv1d.hip", "ssd_scan.hpp", "ssd_internal.h"]


def kernel_hash(sources=KERNEL_SOURCES):
    h = hashlib.sha256()
    for f in sources:
        with open(os.path.join(ROOT, "selective_state_space_cu_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def ingest_counters(fetch_csv, write_csv, config, calib_mib, workload="prefill", out=None):
    """Turn two rocprofv3 --pmc runs of `bench.py --copy-calib-mib M` (FETCH_SIZE,
    then WRITE_SIZE; KiB per dispatch) into the HBM traffic of one launch of the
    workload's kernel, each counter scaled by what it reads for the calibration
    kernel (one elementwise pass that reads and writes M MiB)."""
    other = {"decode": (DECODE_COUNTERS, "ssd_decode_kernel", DECODE_SOURCES),
             "conv1d": (CONV_COUNTERS, "ssd_conv1d_kernel", CONV_SOURCES),
             "gdn": (GDN_COUNTERS, "ssd_gdn_kernel", GDN_SOURCES)}.get(workload)
    out = out or (other[0] if other else counter_path(config))
    kname = other[1] if other else scan_kernel_name(config)
    tag = kname[: -len("_kernel")] if other else "ssd_scan"
    import csv

    def read(path):
        """(readings per kernel name, calibration reading) of one pass: the
        calibration dispatch is the elementwise kernel with the largest reading
        (the add); only the workload's dispatches issued before it count, which
        are the warm-up and timed steps (the export-overhead runs after it
        include launches that write no checkpoints)."""
        rows = [(int(r["Dispatch_Id"]), r["Kernel_Name"], float(r["Counter_Value"]))
                for r in csv.DictReader(open(path))]
        cal_id, cal = max(((i, v) for i, k, v in rows if "elementwise" in k), key=lambda t: t[1])
        per = {}
        for i, k, v in rows:
            if tag in k and i < cal_id:
                per.setdefault(k, []).append(v)
        if not per:
            raise ValueError(f"{path}: no {tag} dispatch before the calibration copy")
        return per, cal

    (per_f, cal_f), (per_w, cal_w) = read(fetch_csv), read(write_csv)
    calib_kib = calib_mib * 1024.0
    ff, fw = calib_kib / cal_f, calib_kib / cal_w
    # one launch of each matching kernel per call: sum of the per-kernel averages
    fk = sum(sum(v) / len(v) for v in per_f.values())
    wk = sum(sum(v) / len(v) for v in per_w.values())
    rec = {"kernel": kname if len(per_f) == 1 else " + ".join(sorted(per_f)),
           "kernel_hash": kernel_hash(other[2] if other else KERNEL_SOURCES),
           "config": workload if other else config,
           "fetch_kib_per_dispatch": fk, "write_kib_per_dispatch": wk,
           "dispatches": min(len(v) for v in per_f.values()),
           "per_kernel_kib": {k: {"fetch": sum(per_f[k]) / len(per_f[k]),
                                  "write": sum(per_w.get(k, [0.0])) / max(len(per_w.get(k, [])), 1)}
                              for k in per_f},
           "calibration_mib": calib_mib, "calibration_fetch_kib": cal_f, "calibration_write_kib": cal_w,
           "fetch_scale": ff, "write_scale": fw,
           "hbm_bytes_per_launch": (fk * ff + wk * fw) * 1024.0}
    with open(out, "w") as f:
        json.dump(rec, f, indent=1)
    return rec


def settle_clock(step):
    """Runs `step()` untimed in batches of 20 until CLOCK_SETTLE_S seconds have
    passed (synchronising after each batch); returns the number of steps run."""
    import torch
    n = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < CLOCK_SETTLE_S:
        for _ in range(20):
            step()
        torch.cuda.synchronize()
        n += 20
    return n


def scan_kernel_name(config):
    """The scan kernel the library launches for a workload (the choice of
    ssd_chunk_scan_varlen in ssd_api.hip): bf16 with dstate 128 and headdim a
    multiple of 64 takes the warp-specialised kernel when chunks are at least
    one 64-token tile (one head or several heads per workgroup), else the
    split-state kernel; every other shape the general kernel."""
    from selective_state_space_cu_amd.workloads import CONFIGS
    c = CONFIGS[config]
    if not (c["dtype"] == "bf16" and c["dstate"] == 128 and c["headdim"] % 64 == 0):
        return "ssd_scan_kernel"
    return "ssd_scan_ws_kernel" if c["chunk_size"] >= 64 else "ssd_scan_split_kernel"


def algorithmic_work(w, n_ckpt):
    """Bytes the method must move and flops it must do for one pass. Bytes: x and
    y once per token and head, dt once per token and head (float32), B and C once
    per token and group, each flagged initial state read, each final state and
    block checkpoint written, once. Flops: per chunk of Lc tokens, the C B^T lower
    triangle per group and its application to x per head, and the two Lc x P x N
    products per head (chunk state and the inter-chunk output term)."""
    T, H, P, N, G = w.total_tokens, w.nheads, w.headdim, w.dstate, w.ngroups
    sx = 2 if w.dtype == "bf16" else 4
    n_init = int(w.has_initial_state.sum())
    state = H * P * N * 4
    bytes_ = T * (2 * H * P * sx + 4 * H + 2 * G * N * sx) + (n_init + w.nseqs) * state + n_ckpt * state
    flops = 0
    for L in w.lengths:
        for c0 in range(0, L, w.chunk_size):
            Lc = min(w.chunk_size, L - c0)
            flops += 2 * (Lc * (Lc + 1) // 2 * (N * G + P * H) + 2 * Lc * P * N * H)
    return bytes_, flops


def cpu_baseline(w, heads):
    """The float64 oracle on the host cores over a bounded sample: every sequence,
    the first `heads` heads, per-chunk state recording on."""
    import oracle
    per = w.nheads // w.ngroups          # heads per group
    t = time.perf_counter()
    for h0 in range(0, heads, per):      # one call per group, so the oracle sees one group
        h1, g = min(h0 + per, heads), h0 // per
        hs, gs = slice(h0, h1), slice(g, g + 1)
        oracle.ssd_varlen(w.x[:, hs], w.dt[:, hs], w.dt_bias[hs], w.A[hs], w.B[:, gs], w.C[:, gs],
                          w.D[hs], w.cu_seqlens, w.initial_states[:, hs], w.has_initial_state,
                          chunk_size=w.chunk_size)
    dt_s = time.perf_counter() - t
    frac = heads / w.nheads
    return dict(value=w.total_tokens * frac / dt_s, unit="tokens/s", cores=oracle.num_threads(),
                kind="oracle",
                sample=f"all {w.nseqs} sequences ({w.total_tokens} tokens), heads 0-{heads - 1} of "
                       f"{w.nheads} ({frac:.3f} of the work), float64, chunk-state recording on; "
                       f"{dt_s:.2f} s wall; value scaled to whole-workload tokens/s")


def calib_copy(mib, dev):
    """One plain elementwise kernel that reads and writes `mib` MiB each (the
    scale for the FETCH_SIZE / WRITE_SIZE counters)."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dstb = torch.empty_like(src)
    torch.cuda.synchronize()
    torch.add(src, 1.0, out=dstb)
    torch.cuda.synchronize()


def decode_work(b):
    """Algorithmic bytes of one decode step: every read slot read once, every
    write slot written once (float32 states), x, dt, B, C read and y written once."""
    S, H, P = b.x.shape
    G, N = b.B.shape[1], b.B.shape[2]
    sx = 2 if b.dtype == "bf16" else 4
    state = H * P * N * 4
    n_read = int((b.read_slot >= 0).sum())
    n_write = int((b.write_slot >= 0).sum())
    return (n_read + n_write) * state + S * (2 * H * P * sx + 4 * H + 2 * G * N * sx)


def bench_decode(args):
    """One JSON line for the decode step (dual anchors) on the decode batch."""
    import torch
    from selective_state_space_cu_amd import ssd
    from selective_state_space_cu_amd.workloads import DECODE_CONFIG, make_decode_config

    b = make_decode_config()
    dev = torch.device("cuda:0")
    d = {k: getattr(b, k).to(dev).contiguous() for k in
         ("x", "dt", "dt_bias", "A", "B", "C", "D", "state_cache", "read_slot", "write_slot")}
    y = torch.empty_like(d["x"])
    flag = torch.zeros(1, dtype=torch.int32, device=dev)
    ev = []

    def step(timed):
        if timed:
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
        ssd.decode_step(d["x"], d["dt"], d["A"], d["B"], d["C"], d["state_cache"], d["read_slot"],
                        d["write_slot"], dt_bias=d["dt_bias"], D=d["D"], y=y, error_flag=flag)
        if timed:
            e1.record()
            ev.append((e0, e1))

    n_settle = settle_clock(lambda: step(False))
    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    if int(flag.item()) != 0:
        raise RuntimeError("device error flag set")
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    k_ms = sum(a.elapsed_time(e) for a, e in ev) / len(ev)
    if args.copy_calib_mib:
        calib_copy(args.copy_calib_mib, dev)
    alg = decode_work(b)
    traffic = None
    if os.path.exists(DECODE_COUNTERS):
        with open(DECODE_COUNTERS) as f:
            c = json.load(f)
        if c.get("kernel_hash") == kernel_hash(DECODE_SOURCES):
            traffic = c["hbm_bytes_per_launch"]
    ms_per_step = wall * 1e3 / args.steps
    out = {
        "metric": "SSD decode step (dual state anchors) tokens/s on 1 MI355X; % of HBM roofline",
        "value": b.nseqs / (ms_per_step * 1e-3), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "clock_settle_steps": n_settle, "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": b.dtype,
        "data": "synthetic (seeded; inputs and state cache resident in HBM)",
        "config": {"workload": DECODE_CONFIG["name"], "nseqs": b.nseqs,
                   "nheads": DECODE_CONFIG["nheads"], "headdim": DECODE_CONFIG["headdim"],
                   "dstate": DECODE_CONFIG["dstate"], "ngroups": DECODE_CONFIG["ngroups"],
                   "num_slots": DECODE_CONFIG["num_slots"],
                   "step": "one token per sequence: read slot -> state update -> write slot"},
        "roofline": {"bound": "hbm", "kernel": "ssd_decode_kernel",
                     "achieved": alg / (k_ms * 1e-3) / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": alg / (k_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, "traffic": traffic,
                     "algorithmic_bytes": alg, "kernel_ms": k_ms},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_decode(b)
    print(json.dumps(out), flush=True)


def cpu_baseline_decode(b, nseqs=64):
    """The float64 decode oracle on the host cores over the first `nseqs`
    sequences, their read slots gathered into a small cache."""
    import numpy as np
    import oracle
    rs = b.read_slot.numpy()[:nseqs]
    small = b.state_cache.numpy()[np.maximum(rs, 0)]
    t = time.perf_counter()
    oracle.ssd_decode(b.x[:nseqs], b.dt[:nseqs], b.dt_bias, b.A, b.B[:nseqs], b.C[:nseqs], b.D,
                      small, np.where(rs >= 0, np.arange(nseqs), -1).astype(np.int32),
                      np.arange(nseqs, dtype=np.int32))
    dt_s = time.perf_counter() - t
    return dict(value=nseqs / dt_s, unit="tokens/s", cores=1, kind="oracle",
                sample=f"first {nseqs} of {b.nseqs} sequences (all heads), float64, single thread "
                       f"(the decode oracle is not threaded); {dt_s:.2f} s wall including the "
                       f"float64 widening of their {nseqs} state slots")


def conv1d_work(b):
    """Algorithmic bytes of one conv1d call: x read and out written once, each
    read slot's and write slot's W-1 rows once, weights and bias once."""
    T, C = b.x.shape
    W = b.weight.shape[1]
    sx = 2 if b.dtype == "bf16" else 4
    n_read = int((b.read_slot >= 0).sum())
    n_write = int((b.write_slot >= 0).sum())
    return 2 * T * C * sx + (n_read + n_write) * (W - 1) * C * sx + C * W * 4 + C * 4


def bench_conv1d(args):
    """One JSON line for the varlen causal conv1d on the prefix-cache batch's
    channels; a step is the chunk metadata plus the convolution."""
    import torch
    from selective_state_space_cu_amd import ssd
    from selective_state_space_cu_amd.workloads import CONV_CONFIG, make_conv_config

    b = make_conv_config()
    dev = torch.device("cuda:0")
    d = {k: getattr(b, k).to(dev).contiguous() for k in
         ("x", "weight", "bias", "cu_seqlens", "conv_states", "read_slot", "write_slot")}
    T = int(b.cu_seqlens[-1])
    out = torch.empty_like(d["x"])
    ev = []

    def step(timed):
        meta = ssd.varlen_metadata(d["cu_seqlens"], CONV_CONFIG["chunk_size"], total_tokens=T)
        if timed:
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
        ssd.causal_conv1d_varlen(d["x"], d["weight"], meta, bias=d["bias"], silu=b.silu,
                                 conv_states=d["conv_states"], read_slot=d["read_slot"],
                                 write_slot=d["write_slot"], out=out)
        if timed:
            e1.record()
            ev.append((e0, e1))
        return meta

    n_settle = settle_clock(lambda: step(False))
    for _ in range(args.warmup):
        meta = step(False)
    torch.cuda.synchronize()
    if int(meta.error_flag.item()) != 0:
        raise RuntimeError("device error flag set")
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    k_ms = sum(a.elapsed_time(e) for a, e in ev) / len(ev)
    if args.copy_calib_mib:
        calib_copy(args.copy_calib_mib, dev)
    alg = conv1d_work(b)
    traffic = None
    if os.path.exists(CONV_COUNTERS):
        with open(CONV_COUNTERS) as f:
            c = json.load(f)
        if c.get("kernel_hash") == kernel_hash(CONV_SOURCES):
            traffic = c["hbm_bytes_per_launch"]
    ms_per_step = wall * 1e3 / args.steps
    res = {
        "metric": "Varlen causal conv1d tokens/s on 1 MI355X; % of HBM roofline",
        "value": T / (ms_per_step * 1e-3), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "clock_settle_steps": n_settle, "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": b.dtype,
        "data": "synthetic (seeded; inputs and conv-state cache resident in HBM)",
        "config": {"workload": CONV_CONFIG["name"], "nseqs": len(CONV_CONFIG["lengths"]),
                   "total_tokens": T, "channels": CONV_CONFIG["channels"], "width": CONV_CONFIG["width"],
                   "activation": "silu" if b.silu else "identity", "chunk_size": CONV_CONFIG["chunk_size"],
                   "num_slots": CONV_CONFIG["num_slots"],
                   "step": "chunk metadata + conv1d (read slot -> window -> write slot)"},
        "roofline": {"bound": "hbm", "kernel": "ssd_conv1d_kernel",
                     "achieved": alg / (k_ms * 1e-3) / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": alg / (k_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, "traffic": traffic,
                     "algorithmic_bytes": alg, "kernel_ms": k_ms},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_conv1d(b)
    print(json.dumps(res), flush=True)


def cpu_baseline_conv1d(b):
    """The float64 conv1d oracle (single thread) over the whole workload."""
    import oracle
    t = time.perf_counter()
    oracle.causal_conv1d(b.x, b.cu_seqlens, b.weight, b.bias, b.silu, b.conv_states, b.read_slot,
                         b.write_slot)
    dt_s = time.perf_counter() - t
    T = int(b.cu_seqlens[-1])
    return dict(value=T / dt_s, unit="tokens/s", cores=1, kind="oracle",
                sample=f"the whole workload ({T} tokens, all {b.x.shape[1]} channels), float64, "
                       f"single thread (the conv oracle is not threaded); {dt_s:.2f} s wall "
                       f"including the float64 widening of x")


GDN_COUNTERS = os.path.join(ROOT, "profiles", "gdn_prefix_cache_4x8894_h32g16_counters.json")
GDN_SOURCES = ["ssd_gdn.hip", "ssd_scan.hpp", "ssd_internal.h"]


def gdn_work(w, n_ckpt):
    """Algorithmic bytes and flops of one GDN chunk call. Bytes: q, k read once
    per key head, v read and o written once, gate and beta read once, each
    flagged initial state read, each final state and checkpoint written once.
    Flops: per chunk of Lc tokens and value head, the products of the form the
    kernels compute (K K^T and Q K^T lower triangles, K H0, Q H0, the triangular
    T (beta V - beta gamma K H0), the causal Mq U and the state update K^T U),
    counted once per value head."""
    T, G, dk = w.q.shape
    H, dv = w.v.shape[1], w.v.shape[2]
    state = H * dv * dk * 4
    n_init = int(w.has_initial_state.sum())
    bytes_ = T * (2 * G * dk * 2 + 2 * H * dv * 2 + 2 * H * 4) + (n_init + w.nseqs) * state + n_ckpt * state
    flops = 0
    for L in w.lengths:
        for c0 in range(0, L, w.chunk_size):
            Lc = min(w.chunk_size, L - c0)
            tri = Lc * (Lc + 1) // 2
            flops += 2 * H * (2 * tri * dk + 2 * Lc * dk * dv + tri * dv + tri * dv + Lc * dk * dv)
    return bytes_, flops


class GdnRun:
    """Device inputs and outputs of the GDN workload, and its step."""

    def __init__(self, dev):
        import torch
        from selective_state_space_cu_amd import ssd
        from selective_state_space_cu_amd.workloads import make_gdn_config
        self.ssd = ssd
        w = self.w = make_gdn_config()
        self.d = {k: getattr(w, k).to(dev).contiguous() for k in
                  ("q", "k", "v", "gate", "beta", "initial_states", "has_initial_state", "cu_seqlens")}
        S, H, dv, dk = w.nseqs, w.v.shape[1], w.v.shape[2], w.q.shape[2]
        self.bt = w.block_table.to(dev)
        self.o = torch.empty_like(self.d["v"])
        self.fin = torch.empty((S, H, dv, dk), dtype=torch.float32, device=dev)
        self.cache = torch.zeros((w.num_slots, H, dv, dk), dtype=torch.float32, device=dev)
        self.init = self.d["initial_states"] if int(w.has_initial_state.sum()) else None
        self.has = self.d["has_initial_state"] if self.init is not None else None
        self.ev, self.ev_meta = [], []
        self.prepare()
        self.n_ckpt = int((self.dst >= 0).sum().item())
        self.ws = torch.empty(ssd.gated_delta_workspace_size(self.meta, H), dtype=torch.uint8, device=dev)

    def prepare(self):
        self.meta = self.ssd.varlen_metadata(self.d["cu_seqlens"], self.w.chunk_size,
                                             total_tokens=self.w.total_tokens)
        _, self.dst = self.ssd.export_chunk_states(self.meta, self.bt, self.w.block_size, num_slots=self.w.num_slots)

    def scan(self, export=True):
        d = self.d
        self.ssd.gated_delta_chunk_varlen(d["q"], d["k"], d["v"], d["gate"], d["beta"], self.meta,
                                          scale=self.w.scale, initial_states=self.init,
                                          has_initial_state=self.has, o=self.o, final_states=self.fin,
                                          chunk_states=self.cache if export else None,
                                          chunk_state_dst=self.dst if export else None, workspace=self.ws)



def bench_gdn(args):
    """One JSON line for the chunked gated delta rule with per-chunk state export
    on the prefix-cache batch (4 x 8894 tokens, 32 value heads on 16 key heads,
    dk = dv = 128, chunk 64, 256-token blocks); a step is the chunk metadata, the
    checkpoint plan and the GDN chunk kernel writing the block checkpoints."""
    import numpy as np
    import torch
    from selective_state_space_cu_amd.workloads import GDN_CONFIG

    dev = torch.device("cuda:0")
    run = GdnRun(dev)
    w = run.w
    n_settle = settle_clock(lambda: run.step(False))
    for _ in range(args.warmup):
        run.step(False)
    torch.cuda.synchronize()
    if int(run.meta.error_flag.item()) != 0:
        raise RuntimeError("device error flag set")
    run.ev.clear()
    run.ev_meta.clear()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        run.step(True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    k_ms = sum(a.elapsed_time(b) for a, b in run.ev) / len(run.ev)
    meta_ms = sum(a.elapsed_time(b) for a, b in run.ev_meta) / len(run.ev_meta)
    if args.copy_calib_mib:
        calib_copy(args.copy_calib_mib, dev)
    flush = torch.empty(FLUSH_MIB << 20, dtype=torch.uint8, device=dev)
    cold = []
    for i in range(args.cold_calls):
        flush.fill_(i & 0xff)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        run.scan()
        e1.record()
        cold.append((e0, e1))
    torch.cuda.synchronize()
    cold_ms = np.array([a.elapsed_time(b) for a, b in cold]) if cold else np.array([k_ms])
    alg, flops = gdn_work(w, run.n_ckpt)
    traffic = None
    if os.path.exists(GDN_COUNTERS):
        with open(GDN_COUNTERS) as f:
            c = json.load(f)
        if c.get("kernel_hash") == kernel_hash(GDN_SOURCES):
            traffic = c["hbm_bytes_per_launch"]
    ms_per_step = wall * 1e3 / args.steps
    T = w.total_tokens
    H, G, dk, dv = w.v.shape[1], w.q.shape[1], w.q.shape[2], w.v.shape[2]
    med = float(np.median(cold_ms))
    res = {
        "metric": "Gated delta rule (GDN) chunked prefill tokens/s on 1 MI355X; % of HBM roofline",
        "value": T / (ms_per_step * 1e-3), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "clock_settle_steps": n_settle, "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic (seeded; inputs and checkpoint cache resident in HBM)",
        "config": {"workload": GDN_CONFIG["name"], "nseqs": w.nseqs, "total_tokens": T, "nheads": H,
                   "nkheads": G, "dk": dk, "dv": dv, "chunk_size": w.chunk_size, "block_size": w.block_size,
                   "checkpoints_per_step": run.n_ckpt,
                   "step": "metadata + checkpoint plan + GDN chunk kernel with at-source checkpoint export"},
        "roofline": {"bound": "hbm", "kernel": "ssd_gdn_prep_kernel + ssd_gdn_scan_kernel (one call)",
                     "achieved": alg / (k_ms * 1e-3) / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": alg / (k_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, "traffic": traffic,
                     "algorithmic_bytes": alg, "kernel_ms": k_ms, "metadata_and_plan_ms": meta_ms,
                     "mfma_tflops": flops / (k_ms * 1e-3) / 1e12,
                     "mfma_frac": flops / (k_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS},
        "cold": {"calls": len(cold), "kernel_ms_median": med, "kernel_ms_p10": float(np.percentile(cold_ms, 10)),
                 "kernel_ms_p90": float(np.percentile(cold_ms, 90)),
                 "hbm_frac_median": alg / (med * 1e-3) / 1e9 / HBM_PEAK_GBS},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_gdn(w)
    print(json.dumps(res), flush=True)


def cpu_baseline_gdn(w):
    """The float64 GDN oracle over the whole workload, one key head (its value
    heads) per call so that the float64 copies stay small."""
    import numpy as np
    import oracle
    H, G = w.v.shape[1], w.q.shape[1]
    per = H // G
    f = lambda t: t.float().numpy().astype(np.float64)   # noqa: E731
    t = time.perf_counter()
    for g in range(G):
        hs = slice(g * per, (g + 1) * per)
        oracle.gated_delta(f(w.q[:, g:g + 1]), f(w.k[:, g:g + 1]), f(w.v[:, hs]), f(w.gate[:, hs]),
                           f(w.beta[:, hs]), w.cu_seqlens.numpy(), w.scale, f(w.initial_states[:, hs]),
                           w.has_initial_state.numpy(), chunk_size=w.chunk_size)
    dt_s = time.perf_counter() - t
    return dict(value=w.total_tokens / dt_s, unit="tokens/s", cores=oracle.num_threads(), kind="oracle",
                sample=f"the whole workload ({w.total_tokens} tokens, all {H} value heads), float64, "
                       f"chunk-state recording on, one key head per call; {dt_s:.2f} s wall including "
                       f"the float64 widening of the inputs")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=4)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-heads", type=int, default=32)
    ap.add_argument("--cold-calls", type=int, default=50,
                    help="HBM-cold timed scans per graded workload (flush write before each)")
    ap.add_argument("--single-config", dest="all_configs", action="store_false",
                    help="cold protocol on --config only (default: every graded prefill workload)")
    ap.add_argument("--copy-calib-mib", type=int, default=0,
                    help="also run one plain device copy of this size (counter calibration)")
    ap.add_argument("--workload", choices=("prefill", "decode", "conv1d", "gdn"), default="prefill",
                    help="prefill (default): the scan step; decode: one dual-anchor decode step "
                         "per sequence on the 256-sequence decode batch; conv1d: the causal conv1d "
                         "before the scan on the prefix-cache batch's 5120 channels; gdn: the chunked "
                         "gated delta rule with per-chunk state export on the same batch")
    ap.add_argument("--ingest-counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write the traffic record from two rocprofv3 counter CSVs and exit "
                         "(with --copy-calib-mib giving the calibration size)")
    args = ap.parse_args()
    if args.ingest_counters:
        print(json.dumps(ingest_counters(*args.ingest_counters, config=args.config,
                                         calib_mib=args.copy_calib_mib or 512,
                                         workload=args.workload)))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (sequences and "
              "head groups are independent in the scan, so a batch would shard by either "
              "across GPUs with no collective inside the step)", file=sys.stderr)
        sys.exit(2)

    if args.workload == "decode":
        bench_decode(args)
        return
    if args.workload == "conv1d":
        bench_conv1d(args)
        return
    if args.workload == "gdn":
        bench_gdn(args)
        return
    import torch
    from selective_state_space_cu_amd import ssd
    from selective_state_space_cu_amd.workloads import CONFIGS

    dev = torch.device("cuda:0")
    flush = torch.empty(FLUSH_MIB << 20, dtype=torch.uint8, device=dev)
    cfgd = CONFIGS[args.config]
    run = PrefillRun(args.config, dev)
    w = run.w
    S, T, H, P, N = w.nseqs, w.total_tokens, w.nheads, w.headdim, w.dstate

    # (1) the step loop: K steps back to back (metadata + plan + scan), wall
    # clock for `value`, HIP events on the launch stream around each scan for
    # the kernel's average duration (what a rocprofv3 trace of this command shows)
    n_settle = settle_clock(lambda: run.step(False))
    for _ in range(args.warmup):
        run.step(False)
    torch.cuda.synchronize()
    if int(run.meta.error_flag.item()) != 0:
        raise RuntimeError("device error flag set")
    run.ev.clear()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        run.step(True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    scan_ms = sum(a.elapsed_time(b) for a, b in run.ev) / len(run.ev)
    meta_ms = sum(a.elapsed_time(b) for a, b in run.ev_meta) / len(run.ev_meta)

    if args.copy_calib_mib:
        calib_copy(args.copy_calib_mib, dev)

    alg_bytes, alg_flops = algorithmic_work(w, run.n_ckpt)
    achieved = alg_bytes / (scan_ms * 1e-3) / 1e9
    ms_per_step = wall * 1e3 / args.steps
    out = {
        "metric": "SSD varlen prefill tokens/s on 1 MI355X; % of HBM/MFMA roofline",
        "value": T / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup, "clock_settle_steps": n_settle,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded; inputs resident in HBM)",
        "config": {"workload": cfgd["name"], "nseqs": S, "total_tokens": T, "nheads": H,
                   "headdim": P, "dstate": N, "ngroups": w.ngroups, "chunk_size": w.chunk_size,
                   "block_size": w.block_size, "checkpoints_per_step": run.n_ckpt,
                   "step": "metadata + checkpoint plan + scan with at-source checkpoint export"},
        "roofline": {"bound": "hbm", "kernel": scan_kernel_name(args.config), "achieved": achieved,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": counter_traffic(args.config), "algorithmic_bytes": alg_bytes,
                     "kernel_ms": scan_ms, "metadata_and_plan_ms": meta_ms,
                     "mfma_tflops": alg_flops / (scan_ms * 1e-3) / 1e12,
                     "mfma_frac": alg_flops / (scan_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS},
        "cpu_baseline": None,
    }
    # (2) the cold protocol on this workload and on the other graded prefill
    # workloads: each timed scan preceded by a write of FLUSH_MIB outside the
    # events (evicts L2 and the Infinity Cache), median / p10 / p90
    graded = {}
    for ci in (([args.config] + [c for c in GRADED if c != args.config] if args.all_configs else [args.config])
               if args.cold_calls > 0 else []):
        r = run if ci == args.config else PrefillRun(ci, dev)
        graded[CONFIGS[ci]["name"]] = cold_stats(r, flush, args.cold_calls)
        if r is not run:
            del r
            torch.cuda.empty_cache()
    out["cold"] = graded
    # (3) yardstick: a plain device copy of the same byte count, cold
    if graded:
        ref = copy_reference(alg_bytes, flush)
        for g in graded.values():
            g["frac_of_copy_rate"] = (g["algorithmic_bytes"] / (g["kernel_ms_median"] * 1e-3) / 1e9) / ref["gbs"]
        out["copy_reference"] = ref
    if run.has_blocks:
        out["checkpoint_export"] = export_overhead(ssd, run)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, min(args.cpu_heads, H))
    print(json.dumps(out), flush=True)


GRADED = (4, 2, 3)   # the prefill workloads whose roofline fractions are reported
FLUSH_MIB = 512


class PrefillRun:
    """Device inputs and outputs of one prefill workload, and its step."""

    def __init__(self, config, dev):
        import torch
        from selective_state_space_cu_amd import ssd
        from selective_state_space_cu_amd.workloads import make_config
        self.ssd, self.config = ssd, config
        w = self.w = make_config(config)
        d = self.d = {k: getattr(w, k).to(dev).contiguous() for k in
                      ("x", "dt", "dt_bias", "A", "B", "C", "D", "initial_states", "has_initial_state",
                       "cu_seqlens")}
        S, H, P, N = w.nseqs, w.nheads, w.headdim, w.dstate
        self.has_blocks = w.block_table is not None
        self.bt = w.block_table.to(dev) if self.has_blocks else None
        self.y = torch.empty_like(d["x"])
        self.fin = torch.empty((S, H, P, N), dtype=torch.float32, device=dev)
        self.cache = (torch.zeros((w.num_slots, H, P, N), dtype=torch.float32, device=dev)
                      if self.has_blocks else None)
        self.init = d["initial_states"] if int(w.has_initial_state.sum()) else None
        self.has = d["has_initial_state"] if self.init is not None else None
        self.ev, self.ev_meta = [], []
        self.meta, self.dst = None, None
        self.prepare()
        self.n_ckpt = int((self.dst >= 0).sum().item()) if self.has_blocks else 0

    def prepare(self):
        """Metadata and checkpoint plan (built once per batch)."""
        self.meta = self.ssd.varlen_metadata(self.d["cu_seqlens"], self.w.chunk_size,
                                             total_tokens=self.w.total_tokens)
        self.dst = None
        if self.has_blocks:
            _, self.dst = self.ssd.export_chunk_states(self.meta, self.bt, self.w.block_size,
                                                       num_slots=self.w.num_slots)

    def scan(self, export=True):
        d = self.d
        self.ssd.chunk_scan_varlen(d["x"], d["dt"], d["A"], d["B"], d["C"], self.meta,
                                   dt_bias=d["dt_bias"], D=d["D"], initial_states=self.init,
                                   has_initial_state=self.has, y=self.y, final_states=self.fin,
                                   chunk_states=self.cache if export else None,
                                   chunk_state_dst=self.dst if export else None)

    def step(self, timed):
        import torch
        if timed:
            m0 = torch.cuda.Event(enable_timing=True)
            m0.record()
        self.prepare()
        if timed:
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
        self.scan()
        if timed:
            e1.record()
            self.ev.append((e0, e1))
            self.ev_meta.append((m0, e0))


def cold_stats(run, flush, calls, warmup=5):
    """The scan timed alone, HBM-cold: `warmup` untimed calls, then `calls`
    calls each preceded by a write of the flush buffer outside the events."""
    import numpy as np
    import torch
    for _ in range(warmup):
        run.scan()
    ev = []
    for i in range(calls):
        flush.fill_(i & 0xff)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        run.scan()
        e1.record()
        ev.append((e0, e1))
    torch.cuda.synchronize()
    if int(run.meta.error_flag.item()) != 0:
        raise RuntimeError("device error flag set")
    ms = np.array([a.elapsed_time(b) for a, b in ev])
    alg, flops = algorithmic_work(run.w, run.n_ckpt)
    med = float(np.median(ms))
    return {"kernel": scan_kernel_name(run.config), "calls": calls,
            "kernel_ms_median": med, "kernel_ms_p10": float(np.percentile(ms, 10)),
            "kernel_ms_p90": float(np.percentile(ms, 90)), "kernel_ms_mean": float(ms.mean()),
            "algorithmic_bytes": alg, "hbm_frac_median": alg / (med * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "mfma_frac_median": flops / (med * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
            "tokens_per_s_median": run.w.total_tokens / (med * 1e-3),
            "traffic": counter_traffic(run.config)}


def counter_path(config):
    from selective_state_space_cu_amd.workloads import CONFIGS
    return os.path.join(ROOT, "profiles", f"scan_{CONFIGS[config]['name']}_counters.json")


def counter_traffic(config):
    """HBM bytes per launch from the committed counter record of this workload,
    or None when the kernel sources changed since it was taken."""
    path = counter_path(config)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        c = json.load(f)
    if c.get("kernel_hash") == kernel_hash() and c.get("config") == config:
        return c["hbm_bytes_per_launch"]
    return None


def copy_reference(nbytes, flush, calls=20):
    """A plain device copy (torch) that moves `nbytes` in total (half read, half
    written), timed like the cold protocol: each timed copy after a write of the
    flush buffer outside the events, median. The rate a library streaming kernel
    reaches on this GPU for a comparable byte count, beside the peak."""
    import numpy as np
    import torch
    half = nbytes // 2 // 16 * 16
    src = torch.full((half,), 1, dtype=torch.uint8, device=flush.device)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    ev = []
    for i in range(calls):
        flush.fill_(i & 0xff)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        dst.copy_(src)
        e1.record()
        ev.append((e0, e1))
    torch.cuda.synchronize()
    med = float(np.median([a.elapsed_time(b) for a, b in ev]))
    gbs = 2 * half / (med * 1e-3) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    return {"bytes": 2 * half, "ms_median": med, "gbs": gbs, "frac_of_peak": gbs / HBM_PEAK_GBS}


def export_overhead(ssd, run, rounds=6, per=10):
    """Scan time with the at-source block-checkpoint export against the same scan
    without it (interleaved rounds of HIP-event-timed launches, medians): the
    kernel-level cost of writing the checkpoints."""
    import statistics
    import torch
    t = {True: [], False: []}
    for _ in range(rounds):
        for exp in (True, False):
            for _ in range(per):
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record()
                run.scan(export=exp)
                e1.record()
                t[exp].append((e0, e1))
    torch.cuda.synchronize()
    med = {k: statistics.median(a.elapsed_time(b) for a, b in v) for k, v in t.items()}
    return {"scan_ms_with": med[True], "scan_ms_without": med[False],
            "overhead_frac": med[True] / med[False] - 1.0,
            "note": "kernel-level: the same scan with and without writing the block checkpoints"}


GdnRun.step = PrefillRun.step   # same step shape: metadata + plan, then the timed kernel


if __name__ == "__main__":
    main()
