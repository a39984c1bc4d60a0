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

Timing protocol. Inputs are resident in HBM and the workspace is allocated
before the timed region. Each of the K timed steps is preceded, outside its
own pair of HIP events, by a read of --flush-mib MiB of scratch memory
(default 1024), which evicts the 256 MB last-level cache (MALL) and the L2s,
so every step reads its inputs from HBM. The headline is the median of those
flushed per-step times; the back-to-back (warm) rate over the same K steps
is reported beside it. The per-kernel times behind `roofline` are taken the
same way (a flush before each pass, events between the kernels of the pass).
The other workloads are measured with the same protocol in `workloads`.
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
    ap.add_argument("--one-pass-steps", type=int, default=10, help="flushed steps per path and round in one_pass")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true", help="skip the decode-step, packed-sequence and convolution measurements")
    ap.add_argument("--cpu-sample-seqs", type=int, default=8)
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="also run a plain fp32 elementwise copy (negation) of MIB MiB, "
                         "the reference kernel for scaling rocprofv3 byte counters")
    ap.add_argument("--flush-mib", type=int, default=1024,
                    help="scratch read before every timed step (0: no flush, back-to-back steps only)")
    ap.add_argument("--no-workloads", action="store_true", help="skip the other workloads' entries")
    ap.add_argument("--workload-steps", type=int, default=20)
    ap.add_argument("--cpu-workers", type=int, default=0,
                    help="oracle worker processes for the CPU baseline (0: one per host core, at most 16)")
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
    # one-pass kernel (steps 2-5 after the cumsum): x in, y out, B and C,
    # dA_cumsum and dt_chunked once, every hand-over state written and read
    # once in fp32, the initial and final states
    # segmented state passing: the plain chain's bytes plus each segment's
    # fp32 aggregate written once and read by every later segment
    nseg = -(-nc // 32)
    agg = b * H * P * N * 4
    out["state_passing_seg"] = dict(bytes=out["state_passing"]["bytes"] + agg * (nseg - 1) * (1 + nseg / 2),
                                    flops=out["state_passing"]["flops"])
    hand = 2 * b * H * (nc - 1) * P * N * 4
    out["one_pass"] = dict(bytes=2 * T * H * P * s + 2 * T * G * N * s + 2 * cs + hand
                           + b * H * P * N * 4 * (2 if cfg.init_state else 1),
                           flops=out["chunk_state"]["flops"] + out["state_passing"]["flops"]
                           + out["chunk_scan"]["flops"])
    return out


def forward_kernels(cfg, path):
    """The kernels one ssd_forward launches on `path`, by name in the model."""
    if path == "one-pass":
        return ["chunk_cumsum", "one_pass"]
    if path == "split-segmented":
        return ["cumsum_chunk_state", "state_passing_seg", "chunk_scan"]
    if cfg.io_dtype != "bf16":
        return ["chunk_cumsum", "chunk_state", "state_passing", "chunk_scan"]
    return ["cumsum_chunk_state", "state_passing", "chunk_scan"]


class Flusher:
    """Reads `mib` MiB of scratch memory on the current stream (a sum over
    it): more than the 256 MB last-level cache and the L2s hold, so the next
    kernel finds none of its data in them and reads HBM. A read, not a write:
    a write would leave the caches full of dirty lines, and their write-back
    would be charged to the next kernel."""

    def __init__(self, dev, mib):
        import torch
        self.buf = torch.ones(mib << 18, dtype=torch.float32, device=dev) if mib > 0 else None
        self.out = torch.empty((), dtype=torch.float32, device=dev) if mib > 0 else None

    def __call__(self):
        if self.buf is not None:
            import torch
            torch.sum(self.buf, 0, out=self.out)


def timed_steps(fn, steps, stream, flush=None):
    """Per-step times (us) of `steps` calls of fn, each between its own pair of
    HIP events on `stream`, each preceded by flush() outside the pair.
    Returns (sorted times, wall seconds between the two synchronisations)."""
    import torch
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    evs = []
    for _ in range(steps):
        if flush is not None:
            flush()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        fn()
        b.record(stream)
        evs.append((a, b))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return sorted(a.elapsed_time(b) * 1e3 for a, b in evs), wall


def quantile(xs, q):
    i = min(len(xs) - 1, max(0, int(round(q * (len(xs) - 1)))))
    return xs[i]


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


def cpu_model():
    """The host CPU's model name from /proc/cpuinfo."""
    try:
        with open("/proc/cpuinfo") as fh:
            for ln in fh:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def _oracle_task(args):
    """Worker task of the CPU baseline: the fp64 oracle recurrence on one
    block of chains, one thread; returns its CPU seconds."""
    import numpy as np  # noqa: F401
    import contextlib
    try:
        from threadpoolctl import threadpool_limits
        limit = threadpool_limits(limits=1)
    except Exception:  # pragma: no cover
        limit = contextlib.nullcontext()
    from oracle import ssd_recurrent
    with limit:
        t0 = time.perf_counter()
        ssd_recurrent(*args)
        return time.perf_counter() - t0


def cpu_baseline(cfg, inp, nseq, workers):
    """The fp64 oracle as it stands on `nseq` whole sequences (all heads) of
    the workload: once in `workers` processes (one per core, tasks of one
    sequence and a block of heads), and once on one sequence in this process
    with one thread."""
    import concurrent.futures as cf
    import multiprocessing as mp

    import numpy as np

    def f64(t):
        return None if t is None else t.detach().cpu().float().numpy().astype(np.float64)

    H, G = cfg.nheads, cfg.ngroups
    hpg = H // G
    hb = 8 if hpg % 8 == 0 else hpg
    tasks = []
    for b in range(nseq):
        for h0 in range(0, H, hb):
            h1 = min(h0 + hb, H)
            g0, g1 = h0 // hpg, (h1 - 1) // hpg + 1
            sl = (slice(b, b + 1), slice(None), slice(h0, h1))
            tasks.append((f64(inp["x"][sl]), f64(inp["dt"][sl]), f64(inp["A"][h0:h1]),
                          f64(inp["B"][b:b + 1, :, g0:g1]), f64(inp["C"][b:b + 1, :, g0:g1]),
                          f64(inp["D"][h0:h1]),
                          None if inp["init_state"] is None else f64(inp["init_state"][b:b + 1, h0:h1])))
    with cf.ProcessPoolExecutor(max_workers=workers, mp_context=mp.get_context("spawn")) as ex:
        list(ex.map(_oracle_task, tasks[:workers]))  # start the workers and import numpy first
        t0 = time.perf_counter()
        cpu_s = sum(ex.map(_oracle_task, tasks))
        wall = time.perf_counter() - t0
    # one thread, this process: the first sequence
    single_s = sum(_oracle_task(t) for t in tasks[:H // hb + (H % hb > 0)])
    tokens = nseq * cfg.seqlen
    return {
        "value": round(tokens / wall, 1),
        "unit": "tokens/s",
        "cores": workers,
        "kind": "oracle",
        "sample": f"{nseq} of {cfg.batch} sequences x {cfg.seqlen} tokens, all {H} heads ({len(tasks)} tasks "
                  f"of one sequence and {hb} heads), fp64 NumPy sequential recurrence in {workers} worker "
                  f"processes of one thread: {tokens} tokens in {wall:.1f} s wall, {cpu_s:.1f} s of CPU time",
        "host_cpu_count": os.cpu_count(),
        "cpu_model": cpu_model(),
        "single_thread_tokens_per_s": round(cfg.seqlen / single_s, 1),
    }


def decode_measure(cfg, batch, steps, dev, flush):
    """The recurrent (decode) step on the layer shape of `cfg` for `batch`
    sequences: median time per step (flushed; HIP events on the launch stream)
    and algorithmic bytes (fp32 state read and written once, plus x, y, dt,
    B, C)."""
    import torch

    import mamba_ssd_scan_fwd_amd as ssd
    from ssd_inputs import make_inputs

    inp = make_inputs(cfg.with_(batch=batch, seqlen=1, init_state=True), seed=101)
    d = {k: (v.to(dev) if v is not None else None) for k, v in inp.items()}
    x, dt, Bm, Cm = d["x"][:, 0], d["dt"][:, 0], d["B"][:, 0], d["C"][:, 0]
    state = d["init_state"]
    y = torch.empty_like(x)
    stream = torch.cuda.current_stream(dev)

    def run():
        ssd.decode_step(x, dt, d["A"], Bm, Cm, d["D"], state, y=y)

    for _ in range(3):
        run()
    ts, _ = timed_steps(run, steps, stream, flush)
    us = statistics.median(ts)
    s = 2 if cfg.io_dtype == "bf16" else 4
    H, P, N, G = cfg.nheads, cfg.headdim, cfg.dstate, cfg.ngroups
    nbytes = batch * (2 * 4 * H * P * N + 2 * H * P * s + 2 * G * N * s + 4 * H)
    gbs = nbytes / (us * 1e-6) / 1e9
    return {"workload": f"decode step, {batch} sequences x {cfg.name} layer (H {H}, P {P}, N {N}, G {G})",
            "batch": batch, "median_us": round(us, 2), "tokens_per_s": round(batch / (us * 1e-6), 1),
            "algo_bytes": nbytes, "GB_per_s": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}


def varlen_measure(cfg, steps, dev, flush):
    """The workload's tokens as packed sequences of mixed lengths (seeded;
    same total as batch x seqlen): median time per forward pass (flushed) and
    tokens/s."""
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
    h0 = torch.zeros_like(hT)
    stream = torch.cuda.current_stream(dev)

    def timed(init, finals=True):
        # without initial states: fixed chunks of the packed stream; with
        # them: chunks per sequence
        def run():
            ssd.forward_varlen(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], cu_seqlens=cu, y=y,
                               final_states=hT if finals else None, return_final_states=finals,
                               init_states=h0 if init else None)

        for _ in range(3):
            run()
        ts, _ = timed_steps(run, steps, stream, flush)
        return statistics.median(ts)

    us = timed(False)
    us_init = timed(True)
    # y only: the end windows and the fp32 final states (S of them, four
    # times the batched pass's here) are skipped
    us_y = timed(False, finals=False)
    return {"workload": f"{S} packed sequences, {T} tokens in all (lengths {int(lengths.min())}..{int(lengths.max())}), "
                        f"{cfg.name} layer", "num_seqs": S, "median_us": round(us, 2),
            "tokens_per_s": round(T / (us * 1e-6), 1),
            "with_initial_states_median_us": round(us_init, 2),
            "without_final_states_median_us": round(us_y, 2)}


def conv_measure(cfg, steps, dev, flush):
    """The short causal convolution (width 4, SiLU) on the workload's packed
    [x | B | C] channels, split into x, B, C: median time per call (flushed)
    and algorithmic GB/s (every input and output once)."""
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

    def run():
        ssd.conv1d_split(u, w, bias, **kw)

    for _ in range(3):
        run()
    ts, _ = timed_steps(run, steps, stream, flush)
    us = statistics.median(ts)
    nbytes = 2 * cfg.batch * cfg.seqlen * CH * (2 if cfg.io_dtype == "bf16" else 4)
    gbs = nbytes / (us * 1e-6) / 1e9
    return {"workload": f"causal conv width 4 + SiLU, [{cfg.batch}, {cfg.seqlen}, {CH}] channels split into x, B, C",
            "median_us": round(us, 2), "algo_bytes": nbytes, "GB_per_s": round(gbs, 1),
            "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}


class Workload:
    """One workload's device buffers, ready for timed forward passes."""

    def __init__(self, cfg, seed, dev, chunk=0):
        import torch

        import mamba_ssd_scan_fwd_amd as ssd
        from ssd_inputs import make_inputs

        self.cfg, self.dev, self.chunk = cfg, dev, chunk
        self.inp = make_inputs(cfg, seed=seed)
        self.d = {k: (v.to(dev) if v is not None else None) for k, v in self.inp.items()}
        self.desc = ssd.make_desc(cfg.batch, cfg.seqlen, cfg.nheads, cfg.headdim, cfg.dstate, cfg.ngroups,
                                  cfg.io_dtype, chunk)
        self.Q = ssd.effective_chunk_size(self.desc)
        self.nc = -(-cfg.seqlen // self.Q)
        self.ws = torch.empty(ssd.workspace_bytes(self.desc), dtype=torch.uint8, device=dev)
        self.y = torch.empty_like(self.d["x"])
        self.hT = torch.empty((cfg.batch, cfg.nheads, cfg.headdim, cfg.dstate), dtype=torch.float32, device=dev)
        self.stream = torch.cuda.current_stream(dev)
        self.io_bytes = 2 if cfg.io_dtype == "bf16" else 4
        self._args = None

    def forward(self, fused=False, split=False):
        """One whole forward pass: a direct call of the C entry point with the
        arguments marshalled once (the checked binding costs tens of
        microseconds of Python per call, enough to starve back-to-back
        steps of the smaller workloads)."""
        import ctypes

        import mamba_ssd_scan_fwd_amd as ssd
        if self._args is None:
            P = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())  # noqa: E731
            d = self.d
            self._args = (ctypes.byref(self.desc), P(d["x"]), P(d["dt"]), P(d["A"]), P(d["B"]), P(d["C"]), P(d["D"]),
                          P(d["init_state"]), P(self.y), P(self.hT), P(self.ws),
                          ctypes.c_size_t(self.ws.numel()), ctypes.c_void_p(self.stream.cuda_stream))
            lib = ssd.load_library()
            self._fns = {(False, False): lib.ssd_forward, (True, False): lib.ssd_forward_fused,
                         (False, True): lib.ssd_forward_split}
        st = self._fns[(fused, split)](*self._args)
        if st != 0:
            raise ssd.SSDError(st, "forward")

    def path(self):
        """The path ssd_forward takes here (its workspace record), after one call."""
        import mamba_ssd_scan_fwd_amd as ssd
        self.forward()
        path, status = ssd.workspace_status(self.desc, self.ws)
        if status != 0:
            raise RuntimeError(f"{self.cfg.name}: status record {status:#x} after a forward call")
        return path

    def step_fns(self):
        """The launches of one split-path pass through the step entry points,
        by kernel name (the same kernels ssd_forward launches there), on
        intermediates of their own."""
        import ctypes

        import mamba_ssd_scan_fwd_amd as ssd
        lib = ssd.load_library()
        d, desc, st = self.d, self.desc, self.stream
        vp = ctypes.c_void_p
        cfg = self.cfg
        import torch
        cs = torch.empty((cfg.batch, cfg.nheads, self.nc, self.Q), dtype=torch.float32, device=self.dev)
        dtc = torch.empty_like(cs)
        states = torch.empty((cfg.batch, cfg.nheads, self.nc, cfg.headdim, cfg.dstate), dtype=d["x"].dtype,
                             device=self.dev)
        self._keep = (cs, dtc, states)
        S = vp(st.cuda_stream)
        P = lambda t: None if t is None else vp(t.data_ptr())  # noqa: E731

        def k_cumsum():
            assert lib.ssd_chunk_cumsum(ctypes.byref(desc), P(d["dt"]), P(d["A"]), P(cs), P(dtc), S) == 0

        def k_state():
            assert lib.ssd_chunk_state(ctypes.byref(desc), P(d["x"]), P(d["B"]), P(cs), P(dtc), P(states), S) == 0

        def k_cumsum_state():
            assert lib.ssd_cumsum_chunk_state(ctypes.byref(desc), P(d["x"]), P(d["B"]), P(d["dt"]), P(d["A"]),
                                              P(cs), P(dtc), P(states), S) == 0

        def k_pass():
            assert lib.ssd_state_passing(ctypes.byref(desc), P(states), P(cs), P(d["init_state"]), P(self.hT),
                                         S) == 0

        def k_scan():
            assert lib.ssd_chunk_scan(ctypes.byref(desc), P(d["x"]), P(d["B"]), P(d["C"]), P(d["D"]), P(cs),
                                      P(dtc), P(states), P(self.y), S) == 0

        return {"chunk_cumsum": k_cumsum, "chunk_state": k_state, "cumsum_chunk_state": k_cumsum_state,
                "state_passing": k_pass, "chunk_scan": k_scan}


def kernel_times(wl, path, reps, flush):
    """Average duration (us) of every kernel of one forward pass on `path`,
    each pass preceded by a flush, with a HIP event between consecutive
    kernels on the launch stream (the pass runs through the step entry
    points). On the one-pass path, whose fused kernel has no entry point of
    its own, the one-pass kernel's time is the whole path's minus the
    cumsum's (both flushed), marked derived."""
    import torch
    names = forward_kernels(wl.cfg, path)
    fns = wl.step_fns()
    if path == "one-pass":
        ts_all, _ = timed_steps(lambda: wl.forward(fused=True), reps, wl.stream, flush)
        ts_cs, _ = timed_steps(fns["chunk_cumsum"], reps, wl.stream, flush)
        t_all, t_cs = statistics.median(ts_all), statistics.median(ts_cs)
        return {"chunk_cumsum": t_cs, "one_pass": t_all - t_cs}, True
    if path == "split-segmented":
        # the segmented state passing has no step entry point of its own
        # (the step entry runs the plain chain): whole pass minus the others
        times, _ = kernel_times(wl, "split", reps, flush)
        ts_all, _ = timed_steps(wl.forward, reps, wl.stream, flush)
        times["state_passing_seg"] = statistics.median(ts_all) - times["cumsum_chunk_state"] - times["chunk_scan"]
        del times["state_passing"]
        return times, True
    calls = [fns[n] for n in names]
    for _ in range(2):
        for fn in calls:
            fn()
    torch.cuda.synchronize()
    rec = []
    for _ in range(reps):
        if flush is not None:
            flush()
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 1)]
        evs[0].record(wl.stream)
        for i, fn in enumerate(calls):
            fn()
            evs[i + 1].record(wl.stream)
        rec.append(evs)
    torch.cuda.synchronize()
    rec = rec[2:] if len(rec) > 4 else rec
    return {n: sum(ev[i].elapsed_time(ev[i + 1]) for ev in rec) / len(rec) * 1e3 for i, n in enumerate(names)}, False


def kernel_table(wl, times):
    model = algorithmic_model(wl.cfg, wl.Q, wl.io_bytes)
    out = {}
    for name, us in times.items():
        m = model[name]
        out[name] = {"avg_us": round(us, 2), "algo_bytes": m["bytes"], "algo_flops": m["flops"],
                     "GB_per_s": round(m["bytes"] / (us * 1e-6) / 1e9, 1),
                     "TFLOP_per_s": round(m["flops"] / (us * 1e-6) / 1e12, 2)}
    return out


def workload_entry(cfg, seed, dev, steps, flush, chunk=0):
    """Flushed and warm time per forward pass of one workload, the path
    ssd_forward takes, its useful TFLOP/s and its dominant kernel against the
    HBM roofline."""
    import torch
    wl = Workload(cfg, seed, dev, chunk)
    path = wl.path()
    for _ in range(3):
        wl.forward()
    ts, _ = timed_steps(wl.forward, steps, wl.stream, flush)
    warm, _ = timed_steps(wl.forward, steps, wl.stream, None)
    times, derived = kernel_times(wl, path, max(6, steps), flush)
    ktab = kernel_table(wl, times)
    model = algorithmic_model(cfg, wl.Q, wl.io_bytes)
    flops = sum(model[k]["flops"] for k in forward_kernels(cfg, path))
    med = statistics.median(ts)
    dom = max(times, key=times.get)
    out = {
        "workload": f"{cfg.name}: B {cfg.batch}, L {cfg.seqlen}, H {cfg.nheads}, P {cfg.headdim}, N {cfg.dstate}, "
                    f"G {cfg.ngroups}, {cfg.io_dtype}",
        "path": path, "chunk": wl.Q,
        "ms_per_step": round(med / 1e3, 4), "p10_ms": round(quantile(ts, 0.1) / 1e3, 4),
        "p90_ms": round(quantile(ts, 0.9) / 1e3, 4), "warm_ms_per_step": round(statistics.median(warm) / 1e3, 4),
        "tokens_per_s": round(cfg.tokens / (med * 1e-6), 1),
        "useful_TFLOP_per_s": round(flops / (med * 1e-6) / 1e12, 2),
        "kernels": ktab, "kernel_times_derived": derived,
        "dominant": {"kernel": dom, "avg_us": round(times[dom], 2),
                     "hbm_frac": round(ktab[dom]["GB_per_s"] / HBM_PEAK_GBS, 4),
                     "mfma_frac_useful": round(ktab[dom]["TFLOP_per_s"] / MFMA_BF16_PEAK_TFS, 4)},
    }
    del wl
    torch.cuda.empty_cache()
    return out


def one_pass_measure(wl, steps, flush):
    """The one-pass path (ssd_forward_fused) next to the split path
    (ssd_forward_split) and ssd_forward itself, on the same buffers `wl`
    (where in HBM buffers lie changes both paths' times): the three in turn,
    three times, flushed medians."""
    import mamba_ssd_scan_fwd_amd as ssd
    cfg = wl.cfg
    paths = {"split": dict(split=True), "fused": dict(fused=True), "auto": {}}
    try:
        for kw in paths.values():
            for _ in range(3):
                wl.forward(**kw)
    except ssd.SSDError:
        return {"workload": cfg.name, "supported": False}
    times = {k: [] for k in paths}
    for _ in range(3):
        for k, kw in paths.items():
            ts, _ = timed_steps(lambda: wl.forward(**kw), steps, wl.stream, flush)
            times[k].extend(ts)
    split_us, fused_us, auto_us = (statistics.median(times[k]) for k in ("split", "fused", "auto"))
    T = cfg.tokens
    model = algorithmic_model(cfg, wl.Q, wl.io_bytes)
    return {"workload": f"{cfg.name}: B {cfg.batch}, L {cfg.seqlen}, H {cfg.nheads}, P {cfg.headdim}, "
                        f"N {cfg.dstate}, G {cfg.ngroups}",
            "supported": True, "one_pass_us": round(fused_us, 2),
            "one_pass_tokens_per_s": round(T / (fused_us * 1e-6), 1),
            "one_pass_algo_bytes": model["one_pass"]["bytes"],
            "split_us": round(split_us, 2), "split_tokens_per_s": round(T / (split_us * 1e-6), 1),
            "ssd_forward_us": round(auto_us, 2), "ssd_forward_takes": wl.path()}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(how it would shard is described in DESIGN.md). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    import mamba_ssd_scan_fwd_amd as ssd
    from ssd_inputs import CONFIGS

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    ssd.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cfg = CONFIGS[args.config]
    # the headline's buffers are the first the process allocates (as in a
    # fresh program; where later allocations land changes the times)
    wl = Workload(cfg, args.config, dev, args.chunk)
    flush = Flusher(dev, args.flush_mib) if args.flush_mib > 0 else None
    path = wl.path()

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
            wl.forward()
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        wl.forward()
    # the K timed steps: each flushed, between its own events
    ts, wall = timed_steps(wl.forward, args.steps, wl.stream, flush)
    med_us = statistics.median(ts)
    # the same K steps back to back (warm caches), one event pair
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(wl.stream)
    for _ in range(args.steps):
        wl.forward()
    ev1.record(wl.stream)
    torch.cuda.synchronize()
    warm_us = ev0.elapsed_time(ev1) / args.steps * 1e3
    tokens_per_s = cfg.tokens / (med_us * 1e-6)

    # ---- every kernel of the pass, flushed passes, events between kernels ----
    reps = args.kernel_reps or max(10, min(args.steps, 50))
    times, derived = kernel_times(wl, path, reps, flush)
    per_kernel = kernel_table(wl, times)
    model = algorithmic_model(cfg, wl.Q, wl.io_bytes)
    dom = max(times, key=times.get)
    m = model[dom]
    ach_gbs = m["bytes"] / (times[dom] * 1e-6) / 1e9
    traffic = None if derived else traffic_from_profile(dom, cfg.name, m["bytes"])
    roofline = {
        "kernel": dom,
        "bound": "hbm",
        "achieved": round(ach_gbs, 1),
        "peak": HBM_PEAK_GBS,
        "unit": "GB/s",
        "frac": round(ach_gbs / HBM_PEAK_GBS, 4),
        "traffic": traffic,
        "algo_bytes_per_launch": m["bytes"],
        "avg_launch_us": round(times[dom], 2),
        "mfma_frac_useful": round(m["flops"] / (times[dom] * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFS, 4),
    }
    fwd_flops = sum(model[k]["flops"] for k in forward_kernels(cfg, path))

    one_pass = None
    if not args.no_one_pass and cfg.io_dtype == "bf16":
        one_pass = [one_pass_measure(wl, args.one_pass_steps, flush)]
        big = Workload(cfg.with_(name=f"{cfg.name} x4 batch", batch=4 * cfg.batch), 104, dev, args.chunk)
        one_pass.append(one_pass_measure(big, args.one_pass_steps, flush))
        del big
        torch.cuda.empty_cache()

    decode = varlen = conv = None
    if not args.no_decode:
        decode = [decode_measure(cfg, bsz, 30, dev, flush) for bsz in (cfg.batch, 256)]
        varlen = varlen_measure(cfg, 20, dev, flush)
        conv = conv_measure(cfg, 20, dev, flush)

    workloads = None
    if not args.no_workloads:
        workloads = []
        for i, c in enumerate(CONFIGS):
            if i != args.config:
                workloads.append(workload_entry(c, i, dev, args.workload_steps, flush))

    cpu = None
    if not args.no_cpu_baseline:
        workers = args.cpu_workers or max(1, min(16, os.cpu_count() or 1))
        cpu = cpu_baseline(cfg, wl.inp, min(args.cpu_sample_seqs, cfg.batch), workers)

    line = {
        "metric": METRIC,
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(med_us / 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.io_dtype,
        "data": "synthetic",
        "config": {"workload": cfg.name, "batch": cfg.batch, "seqlen": cfg.seqlen, "nheads": cfg.nheads,
                   "headdim": cfg.headdim, "dstate": cfg.dstate, "ngroups": cfg.ngroups,
                   "chunk": wl.Q, "init_state": cfg.init_state, "path": path},
        "timing": {"protocol": f"median of {args.steps} steps, each after a {args.flush_mib} MiB scratch read "
                               "outside its HIP event pair" if flush else "back-to-back steps",
                   "p10_ms": round(quantile(ts, 0.1) / 1e3, 4), "p90_ms": round(quantile(ts, 0.9) / 1e3, 4),
                   "warm_ms_per_step": round(warm_us / 1e3, 4),
                   "warm_tokens_per_s": round(cfg.tokens / (warm_us * 1e-6), 1),
                   "wall_s_timed": round(wall, 3)},
        "tflops_per_s": round(fwd_flops / (med_us * 1e-6) / 1e12, 2),
        "roofline": roofline,
        "kernels": per_kernel,
        "cpu_baseline": cpu,
        "workloads": workloads,
        "decode_step": decode,
        "varlen": varlen,
        "conv1d_split": conv,
        "one_pass": one_pass,
        "device_warm_ms": args.device_warm_ms,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
