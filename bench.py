"""Benchmark of the SSD forward pass on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--config IDX] [--no-cpu-baseline]

One step = one whole forward pass (all steps of the chunked path: cumsum,
chunk states, state passing, chunk scan with the chunk output) over one batch
of seeded synthetic inputs already resident in HBM. Prints ONE JSON line.

Besides the headline tokens/s, it times every kernel on its own with HIP
events recorded on the stream the kernels run on, and reports the dominant
kernel against its roofline (algorithmic bytes or flops per launch divided
by its average duration), next to the fp64 CPU oracle timed on a bounded
sample of the same workload. It also times the one-pass path
(ssd_forward_fused) next to the split path on the headline workload and on a
larger-batch workload, where ssd_forward takes the one-pass path.

Before the W warm-up steps the GPU runs forward passes for --device-warm-ms
(untimed): from idle, its clocks take a few hundred milliseconds of load to
reach their steady state, and a timed region that starts earlier measures
the ramp (about 10% slower on the headline workload).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "SSD fwd tokens/s + % of bf16 MFMA / HBM roofline, B=8 L=2048 H=64 P=64 N=128"
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, published
MFMA_BF16_PEAK_TFS = 2500.0  # MI355X dense bf16 matrix, published
FP32_VECTOR_PEAK_TFS = 157.3


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=1, help="workload index (1 = the headline workload)")
    ap.add_argument("--chunk", type=int, default=0)
    ap.add_argument("--kernel-reps", type=int, default=None)
    ap.add_argument("--device-warm-ms", type=float, default=500.0,
                    help="untimed forward passes before the warm-up steps, to reach steady clocks")
    ap.add_argument("--no-one-pass", action="store_true", help="skip the one-pass path measurement")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true", help="skip the decode-step, packed-sequence and convolution measurements")
    ap.add_argument("--cpu-sample-seqs", type=int, default=8)
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="also run a plain fp32 elementwise copy (negation) of MIB MiB, "
                         "the reference kernel for scaling rocprofv3 byte counters")
    return ap.parse_args()


def algorithmic_model(cfg, Q, io_bytes):
    """Algorithmic bytes and flops per launch of each kernel (whole batch).

    Bytes count each operand and result once per launch, at its storage
    dtype: states in the io dtype, dA_cumsum/dt_chunked fp32. Flops count
    2 per multiply-add of the useful (causal) work, C.B^T once per group.
    """
    b, L, H, P, N, G = cfg.batch, cfg.seqlen, cfg.nheads, cfg.headdim, cfg.dstate, cfg.ngroups
    T = b * L
    nc = -(-L // Q)
    s = io_bytes
    st = b * H * nc * P * N * s          # all chunk states, one pass
    cs = b * H * nc * Q * 4              # dA_cumsum or dt_chunked
    out = {
        "chunk_cumsum": dict(bytes=T * H * 4 + 2 * cs, flops=2 * T * H),
        "chunk_state": dict(bytes=T * H * P * s + T * G * N * s + 2 * cs + st,
                            flops=2 * T * H * P * N + 2 * T * H * P),
        # steps 1 and 2 in one kernel: dt in, dA_cumsum / dt_chunked / states out
        "cumsum_chunk_state": dict(bytes=T * H * P * s + T * G * N * s + T * H * 4 + 2 * cs + st,
                                   flops=2 * T * H * P * N + 2 * T * H * P + 2 * T * H),
        "state_passing": dict(bytes=2 * st + 4 * b * H * P * N * (2 if cfg.init_state else 1) + b * H * nc * 4,
                              flops=2 * b * H * nc * P * N),
        "chunk_scan": dict(bytes=2 * T * H * P * s + 2 * T * G * N * s + 2 * cs + st,
                           flops=T * H * (Q + 1) * P + T * G * (Q + 1) * N + 2 * T * H * P * N + 3 * T * H * P),
    }
    return out


def kernel_source_digest(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "mamba_ssd_scan_fwd_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_from_profile(kernel, cfg_name, per_launch_algo):
    """HBM traffic of `kernel` from the committed rocprofv3 counter summary,
    or None when absent or taken on another version of the kernel source."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    if not os.path.exists(path):
        return None
    try:
        with open(path) as fh:
            rec = json.load(fh)
        ent = rec["kernels"][kernel]
        if ent["workload"] != cfg_name:
            return None
        if ent["source_digest"] != kernel_source_digest(ent["source_files"]):
            return None
        return float(ent["hbm_bytes_per_launch"])
    except Exception:
        return None


def cpu_baseline(cfg, inp, nseq, min_seconds=10.0, max_reps=4):
    """The fp64 oracle as it stands, on `nseq` whole sequences (all heads),
    repeated until about `min_seconds` of CPU work have been timed."""
    import numpy as np
    try:
        from threadpoolctl import threadpool_limits
    except Exception:  # pragma: no cover
        threadpool_limits = None
    from oracle import ssd_recurrent

    def f64(t):
        return None if t is None else t.detach().cpu().float().numpy().astype(np.float64)

    sl = slice(0, nseq)
    args = [f64(inp["x"][sl]), f64(inp["dt"][sl]), f64(inp["A"]), f64(inp["B"][sl]), f64(inp["C"][sl]),
            f64(inp["D"]), f64(inp["init_state"][sl]) if inp["init_state"] is not None else None]
    ctx = threadpool_limits(limits=1) if threadpool_limits else None
    if ctx:
        ctx.__enter__()
    reps, total = 0, 0.0
    try:
        while reps < max_reps and (reps == 0 or total < min_seconds):
            t0 = time.perf_counter()
            ssd_recurrent(*args)
            total += time.perf_counter() - t0
            reps += 1
    finally:
        if ctx:
            ctx.__exit__(None, None, None)
    tokens = nseq * cfg.seqlen
    return {
        "value": tokens * reps / total,
        "unit": "tokens/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"{nseq} of {cfg.batch} sequences x {cfg.seqlen} tokens, all {cfg.nheads} heads, "
                  f"{reps} pass(es) ({tokens * reps} tokens in {total:.1f} s; fp64 NumPy sequential "
                  f"recurrence, one thread, {platform.processor() or platform.machine()})",
    }


def decode_measure(cfg, batch, steps, dev):
    """The recurrent (decode) step on the layer shape of `cfg` for `batch`
    sequences: average time per step (HIP events on the launch stream) and
    algorithmic bytes (fp32 state read and written once, plus x, y, dt, B, C)."""
    import torch

    import mamba_ssd_scan_fwd_amd as ssd
    from ssd_inputs import make_inputs

    inp = make_inputs(cfg.with_(batch=batch, seqlen=1, init_state=True), seed=101)
    d = {k: (v.to(dev) if v is not None else None) for k, v in inp.items()}
    x, dt, Bm, Cm = d["x"][:, 0], d["dt"][:, 0], d["B"][:, 0], d["C"][:, 0]
    state = d["init_state"]
    y = torch.empty_like(x)
    stream = torch.cuda.current_stream(dev)
    for _ in range(3):
        ssd.decode_step(x, dt, d["A"], Bm, Cm, d["D"], state, y=y)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(steps):
        ssd.decode_step(x, dt, d["A"], Bm, Cm, d["D"], state, y=y)
    b.record(stream)
    torch.cuda.synchronize()
    us = a.elapsed_time(b) / steps * 1e3
    s = 2 if cfg.io_dtype == "bf16" else 4
    H, P, N, G = cfg.nheads, cfg.headdim, cfg.dstate, cfg.ngroups
    nbytes = batch * (2 * 4 * H * P * N + 2 * H * P * s + 2 * G * N * s + 4 * H)
    gbs = nbytes / (us * 1e-6) / 1e9
    return {"workload": f"decode step, {batch} sequences x {cfg.name} layer (H {H}, P {P}, N {N}, G {G})",
            "batch": batch, "avg_us": round(us, 2), "tokens_per_s": round(batch / (us * 1e-6), 1),
            "algo_bytes": nbytes, "GB_per_s": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}


def varlen_measure(cfg, steps, dev):
    """The workload's tokens as packed sequences of mixed lengths (seeded;
    same total as batch x seqlen): time per forward pass and tokens/s."""
    import numpy as np
    import torch

    import mamba_ssd_scan_fwd_amd as ssd
    from ssd_inputs import make_inputs

    T = cfg.batch * cfg.seqlen
    rng = np.random.default_rng(7)
    w = rng.uniform(0.1, 1.0, size=4 * cfg.batch)
    lengths = np.floor(w / w.sum() * T).astype(np.int64)
    lengths[-1] += T - lengths.sum()
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lengths)]), dtype=torch.int32, device=dev)
    inp = make_inputs(cfg.with_(batch=1, seqlen=T), seed=102)
    d = {k: (v.to(dev) if v is not None else None) for k, v in inp.items()}
    S = len(lengths)
    y = torch.empty_like(d["x"])
    hT = torch.empty((S, cfg.nheads, cfg.headdim, cfg.dstate), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def run():
        ssd.forward_varlen(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], cu_seqlens=cu, y=y, final_states=hT)

    for _ in range(3):
        run()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(steps):
        run()
    b.record(stream)
    torch.cuda.synchronize()
    us = a.elapsed_time(b) / steps * 1e3
    return {"workload": f"{S} packed sequences, {T} tokens in all (lengths {int(lengths.min())}..{int(lengths.max())}), "
                        f"{cfg.name} layer", "num_seqs": S, "avg_us": round(us, 2),
            "tokens_per_s": round(T / (us * 1e-6), 1)}


def conv_measure(cfg, steps, dev):
    """The short causal convolution (width 4, SiLU) on the workload's packed
    [x | B | C] channels, split into x, B, C: time per call and algorithmic
    GB/s (every input and output once)."""
    import torch

    import mamba_ssd_scan_fwd_amd as ssd

    CH = cfg.nheads * cfg.headdim + 2 * cfg.ngroups * cfg.dstate
    g = torch.Generator().manual_seed(103)
    dt_ = torch.bfloat16 if cfg.io_dtype == "bf16" else torch.float32
    u = torch.randn((cfg.batch, cfg.seqlen, CH), generator=g).to(dt_).to(dev)
    w = (torch.randn((CH, 4), generator=g) / 4).to(dev)
    bias = torch.randn(CH, generator=g).to(dev)
    kw = dict(nheads=cfg.nheads, headdim=cfg.headdim, ngroups=cfg.ngroups, dstate=cfg.dstate, silu=True)
    stream = torch.cuda.current_stream(dev)
    for _ in range(3):
        ssd.conv1d_split(u, w, bias, **kw)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(steps):
        ssd.conv1d_split(u, w, bias, **kw)
    b.record(stream)
    torch.cuda.synchronize()
    us = a.elapsed_time(b) / steps * 1e3
    nbytes = 2 * cfg.batch * cfg.seqlen * CH * (2 if cfg.io_dtype == "bf16" else 4)
    gbs = nbytes / (us * 1e-6) / 1e9
    return {"workload": f"causal conv width 4 + SiLU, [{cfg.batch}, {cfg.seqlen}, {CH}] channels split into x, B, C",
            "avg_us": round(us, 2), "algo_bytes": nbytes, "GB_per_s": round(gbs, 1),
            "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}


def one_pass_measure(cfg, steps, dev, bufs=None):
    """The one-pass path (ssd_forward_fused: the dt cumsum, then one kernel
    for chunk states, state hand-over and chunk output) next to the split
    path, on the same buffers: time per forward pass each, which one
    ssd_forward takes, and the one-pass kernel's algorithmic bytes (x and y,
    B and C, dA_cumsum and dt_chunked once, each hand-over state written and
    read once in fp32, the final state). `bufs` = (inputs, y, final state,
    workspace) already allocated for `cfg`, else fresh ones (the two paths are
    always compared on the same buffers: where in HBM the buffers lie changes
    both paths' times)."""
    import torch

    import mamba_ssd_scan_fwd_amd as ssd
    from ssd_inputs import make_inputs

    desc = ssd.make_desc(cfg.batch, cfg.seqlen, cfg.nheads, cfg.headdim, cfg.dstate, cfg.ngroups, cfg.io_dtype)
    if bufs is None:
        inp = make_inputs(cfg, seed=104)
        d = {k: (v.to(dev) if v is not None else None) for k, v in inp.items()}
        y = torch.empty_like(d["x"])
        hT = torch.empty((cfg.batch, cfg.nheads, cfg.headdim, cfg.dstate), dtype=torch.float32, device=dev)
        ws = torch.empty(ssd.workspace_bytes(desc), dtype=torch.uint8, device=dev)
    else:
        d, y, hT, ws = bufs
    stream = torch.cuda.current_stream(dev)

    def run(**kw):
        ssd.forward(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["init_state"], y=y, final_state=hT,
                    workspace=ws, **kw)

    def timed(**kw):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(steps):
            run(**kw)
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / steps * 1e3

    paths = {"split": dict(split=True), "fused": dict(fused=True), "auto": {}}
    try:
        for kw in paths.values():
            for _ in range(5):
                run(**kw)
    except ssd.SSDError:
        return {"workload": cfg.name, "supported": False}
    torch.cuda.synchronize()
    # the three paths in turn, three times: the medians (a path timed only
    # first or only last would carry any drift of the clocks)
    times = {k: [] for k in paths}
    for _ in range(3):
        for k, kw in paths.items():
            times[k].append(timed(**kw))
    split_us, fused_us, auto_us = (statistics.median(times[k]) for k in ("split", "fused", "auto"))
    T = cfg.tokens
    Q = ssd.effective_chunk_size(desc)
    nc = -(-cfg.seqlen // Q)
    s = 2
    H, P, N, G = cfg.nheads, cfg.headdim, cfg.dstate, cfg.ngroups
    nbytes = (2 * T * H * P * s + 2 * T * G * N * s + 2 * cfg.batch * H * nc * Q * 4
              + 2 * cfg.batch * H * (nc - 1) * P * N * 4 + cfg.batch * H * P * N * 4 * (2 if cfg.init_state else 1))
    out = {"workload": f"{cfg.name}: B {cfg.batch}, L {cfg.seqlen}, H {H}, P {P}, N {N}, G {G}",
           "supported": True, "one_pass_us": round(fused_us, 2), "one_pass_tokens_per_s": round(T / (fused_us * 1e-6), 1),
           "one_pass_algo_bytes": nbytes}
    # which path ssd_forward takes here: the one its own time matches
    out.update({"split_us": round(split_us, 2), "split_tokens_per_s": round(T / (split_us * 1e-6), 1),
                "ssd_forward_takes": "one-pass" if abs(auto_us - fused_us) < abs(auto_us - split_us) else "split"})
    return out


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(how it would shard is described in DESIGN.md). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    import mamba_ssd_scan_fwd_amd as ssd
    from ssd_inputs import CONFIGS, make_inputs

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    ssd.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cfg = CONFIGS[args.config]
    inp = make_inputs(cfg, seed=args.config)
    d = {k: (v.to(dev) if v is not None else None) for k, v in inp.items()}
    io_bytes = 2 if cfg.io_dtype == "bf16" else 4
    desc = ssd.make_desc(cfg.batch, cfg.seqlen, cfg.nheads, cfg.headdim, cfg.dstate, cfg.ngroups,
                         cfg.io_dtype, args.chunk)
    Q = ssd.effective_chunk_size(desc)
    ws = torch.empty(ssd.workspace_bytes(desc), dtype=torch.uint8, device=dev)
    y = torch.empty_like(d["x"])
    hT = torch.empty((cfg.batch, cfg.nheads, cfg.headdim, cfg.dstate), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step():
        ssd.forward(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["init_state"], chunk_size=args.chunk,
                    y=y, final_state=hT, workspace=ws)

    if args.copy_calibration:
        # known traffic: reads and writes exactly MIB MiB each
        src = torch.ones(args.copy_calibration * (1 << 18), dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    t_warm = time.perf_counter()
    while time.perf_counter() - t_warm < args.device_warm_ms / 1e3:
        for _ in range(10):
            step()
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = ev0.elapsed_time(ev1)
    ms_per_step = gpu_ms / args.steps
    tokens_per_s = cfg.tokens * args.steps / (gpu_ms / 1e3)

    # ---- every kernel on its own: HIP events on the launch stream ----------
    reps = args.kernel_reps or max(10, min(args.steps, 50))
    nc = -(-cfg.seqlen // Q)
    cs = torch.empty((cfg.batch, cfg.nheads, nc, Q), dtype=torch.float32, device=dev)
    dtc = torch.empty_like(cs)
    st = torch.empty((cfg.batch, cfg.nheads, nc, cfg.headdim, cfg.dstate), dtype=d["x"].dtype, device=dev)
    kw = dict(chunk_size=args.chunk)
    common = dict(headdim=cfg.headdim, dstate=cfg.dstate, ngroups=cfg.ngroups, io_dtype=cfg.io_dtype)

    def k_cumsum():
        lib = ssd.load_library()
        import ctypes
        r = lib.ssd_chunk_cumsum(ctypes.byref(desc), ctypes.c_void_p(d["dt"].data_ptr()),
                                 ctypes.c_void_p(d["A"].data_ptr()), ctypes.c_void_p(cs.data_ptr()),
                                 ctypes.c_void_p(dtc.data_ptr()), ctypes.c_void_p(stream.cuda_stream))
        assert r == 0

    def k_state():
        lib = ssd.load_library()
        import ctypes
        r = lib.ssd_chunk_state(ctypes.byref(desc), ctypes.c_void_p(d["x"].data_ptr()),
                                ctypes.c_void_p(d["B"].data_ptr()), ctypes.c_void_p(cs.data_ptr()),
                                ctypes.c_void_p(dtc.data_ptr()), ctypes.c_void_p(st.data_ptr()),
                                ctypes.c_void_p(stream.cuda_stream))
        assert r == 0

    def k_cumsum_state():
        lib = ssd.load_library()
        import ctypes
        r = lib.ssd_cumsum_chunk_state(ctypes.byref(desc), ctypes.c_void_p(d["x"].data_ptr()),
                                       ctypes.c_void_p(d["B"].data_ptr()), ctypes.c_void_p(d["dt"].data_ptr()),
                                       ctypes.c_void_p(d["A"].data_ptr()), ctypes.c_void_p(cs.data_ptr()),
                                       ctypes.c_void_p(dtc.data_ptr()), ctypes.c_void_p(st.data_ptr()),
                                       ctypes.c_void_p(stream.cuda_stream))
        assert r == 0

    def k_pass():
        lib = ssd.load_library()
        import ctypes
        h0 = d["init_state"]
        r = lib.ssd_state_passing(ctypes.byref(desc), ctypes.c_void_p(st.data_ptr()),
                                  ctypes.c_void_p(cs.data_ptr()),
                                  None if h0 is None else ctypes.c_void_p(h0.data_ptr()),
                                  ctypes.c_void_p(hT.data_ptr()), ctypes.c_void_p(stream.cuda_stream))
        assert r == 0

    def k_scan():
        lib = ssd.load_library()
        import ctypes
        Dp = None if d["D"] is None else ctypes.c_void_p(d["D"].data_ptr())
        r = lib.ssd_chunk_scan(ctypes.byref(desc), ctypes.c_void_p(d["x"].data_ptr()),
                               ctypes.c_void_p(d["B"].data_ptr()), ctypes.c_void_p(d["C"].data_ptr()), Dp,
                               ctypes.c_void_p(cs.data_ptr()), ctypes.c_void_p(dtc.data_ptr()),
                               ctypes.c_void_p(st.data_ptr()), ctypes.c_void_p(y.data_ptr()),
                               ctypes.c_void_p(stream.cuda_stream))
        assert r == 0

    del kw, common
    # The same four launches as one forward step, issued through the step
    # entry points with an event between consecutive kernels: each kernel's
    # duration in the context of the whole pass (caches as the pass leaves them).
    names = ["cumsum_chunk_state", "state_passing", "chunk_scan"]
    fns = [k_cumsum_state, k_pass, k_scan]
    if cfg.io_dtype != "bf16":  # ssd_forward runs the two steps as two kernels there
        names = ["chunk_cumsum", "chunk_state", "state_passing", "chunk_scan"]
        fns = [k_cumsum, k_state, k_pass, k_scan]
    for _ in range(2):
        for fn in fns:
            fn()
    torch.cuda.synchronize()
    rec = []
    for _ in range(reps):
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(len(fns) + 1)]
        evs[0].record(stream)
        for i, fn in enumerate(fns):
            fn()
            evs[i + 1].record(stream)
        rec.append(evs)
    torch.cuda.synchronize()
    rec = rec[2:] if len(rec) > 4 else rec  # the first passes may wait for the host to queue launches
    durations = {n: sum(ev[i].elapsed_time(ev[i + 1]) for ev in rec) / len(rec) * 1e3 for i, n in enumerate(names)}
    model = algorithmic_model(cfg, Q, io_bytes)
    per_kernel = {}
    for name, us in durations.items():
        m = model[name]
        per_kernel[name] = {
            "avg_us": round(us, 2),
            "algo_bytes": m["bytes"],
            "algo_flops": m["flops"],
            "GB_per_s": round(m["bytes"] / (us * 1e-6) / 1e9, 1),
            "TFLOP_per_s": round(m["flops"] / (us * 1e-6) / 1e12, 2),
        }
    dom = max(durations, key=durations.get)
    m = model[dom]
    ach_gbs = m["bytes"] / (durations[dom] * 1e-6) / 1e9
    traffic = traffic_from_profile(dom, cfg.name, m["bytes"])
    roofline = {
        "kernel": dom,
        "bound": "hbm",
        "achieved": round(ach_gbs, 1),
        "peak": HBM_PEAK_GBS,
        "unit": "GB/s",
        "frac": round(ach_gbs / HBM_PEAK_GBS, 4),
        "traffic": traffic,
        "algo_bytes_per_launch": m["bytes"],
        "avg_launch_us": round(durations[dom], 2),
        "mfma_frac_useful": round(m["flops"] / (durations[dom] * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFS, 4),
    }

    one_pass = None
    if not args.no_one_pass and cfg.io_dtype == "bf16":
        one_pass = [one_pass_measure(cfg, 30, dev, (d, y, hT, ws)),
                    one_pass_measure(cfg.with_(name=f"{cfg.name} x4 batch", batch=4 * cfg.batch), 30, dev)]

    decode = None
    if not args.no_decode:
        decode = [decode_measure(cfg, bsz, 50, dev) for bsz in (cfg.batch, 256)]
    varlen = None if args.no_decode else varlen_measure(cfg, 20, dev)
    conv = None if args.no_decode else conv_measure(cfg, 20, dev)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(cfg, inp, min(args.cpu_sample_seqs, cfg.batch))

    total_flops = sum(v["flops"] for v in model.values())
    line = {
        "metric": METRIC,
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.io_dtype,
        "data": "synthetic",
        "config": {"workload": cfg.name, "batch": cfg.batch, "seqlen": cfg.seqlen, "nheads": cfg.nheads,
                   "headdim": cfg.headdim, "dstate": cfg.dstate, "ngroups": cfg.ngroups,
                   "chunk": Q, "init_state": cfg.init_state},
        "tflops_per_s": round(total_flops * args.steps / (gpu_ms / 1e3) / 1e12, 2),
        "wall_s_timed": round(wall, 3),
        "roofline": roofline,
        "kernels": per_kernel,
        "cpu_baseline": cpu,
        "decode_step": decode,
        "varlen": varlen,
        "conv1d_split": conv,
        "one_pass": one_pass,
        "device_warm_ms": args.device_warm_ms,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
