"""Benchmark of the Mamba-2 SSD layer hot path on one MI355X.

One step = one pass of the prefill hot path over one batch of the
Nemotron-H 8B layer shape (batch 4 x 4096 tokens, 128 heads x 64, d_state
128, 8 groups): the depthwise conv1d(4)+SiLU on x|B|C, then the chunked SSD
scan (chunk 128) writing y and the final states.  Inputs are synthetic and
already resident in HBM.  The headline value is layer tokens/s.

The decode step at batch 256 through 29 Mamba-2 layers (1 GiB fp32 state per
layer) is timed in the same run and reported as HBM GB/s, and so are the
other synthetic configs (tiny fp32, Nemotron 3 Nano, packed 3B stream).

Order of the run: decode first, then the other configs, then the headline
step.  The scan is bound by the shader clock, which ramps up over the first
~100 ms of load; by the time the headline step is timed the GPU has been
busy for well over that, so its W warm-up steps and K timed steps run at the
clock a loaded GPU holds.

Per-kernel times come from HIP events recorded on the stream the kernels
run on (torch's current stream, which the C ABI launches on).

The fp64 oracle (test infrastructure) is timed beside every config on the
host's cores, on all OpenMP threads and on one, over a bounded sample of
each workload; its all-core outputs also give each config's parity error.

    python bench.py [--gpus 1] [--steps 20] [--warmup 20]
    python bench.py --only nemotron_h_8b     # one part only (profiler runs)
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16
PROFILES = os.path.join(ROOT, "profiles")
SCAN_SOURCES = ["chunk_scan.hip", "chunk_scan_bf16.hip", "quad_scan_f32.hip", "scan_items.h", "common.h", "kernels.h"]
CONV_SOURCES = ["conv1d_silu.hip", "common.h", "kernels.h"]
DECODE_SOURCES = ["decode_step.hip", "common.h", "kernels.h"]
NORM_SOURCES = ["gated_rmsnorm.hip", "common.h", "kernels.h"]
LINEAR_SOURCES = ["linear_bf16.hip", "common.h", "kernels.h"]
BWD_SOURCES = ["chunk_scan_bwd.hip", "common.h", "kernels.h"]
FP32_MFMA_PEAK_TFLOPS = 157.3  # MI355X dense fp32 matrix


def source_hash(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "state_space_sequence_ssd_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def read_traffic(kernel_tag, files):
    """HBM bytes per launch from a committed rocprofv3 --pmc summary, or None
    when the kernel source changed since the counters were taken."""
    path = os.path.join(PROFILES, f"traffic_{kernel_tag}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha256") != source_hash(files):
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def read_traffic_all(workload):
    """Per-kernel HBM bytes per launch of one workload (profiles/traffic_<workload>.txt),
    keeping only kernels whose source is unchanged since the counters were taken."""
    path = os.path.join(PROFILES, f"traffic_{workload}.txt")
    if not os.path.exists(path):
        return None
    out, cur = {}, {}
    sources = {"chunk_scan": SCAN_SOURCES, "plan": SCAN_SOURCES, "combine": SCAN_SOURCES, "quad_scan": SCAN_SOURCES,
               "conv1d_silu": CONV_SOURCES, "conv_state_out": CONV_SOURCES, "decode_step": DECODE_SOURCES,
               "gated_rmsnorm": NORM_SOURCES, "decode_mimo": ["decode_mimo.hip", "common.h", "kernels.h"],
               "linear": LINEAR_SOURCES, "bwd": BWD_SOURCES}

    def flush():
        t = cur.get("tag")
        if not t or "hbm_bytes_per_launch" not in cur:
            return
        key = next((k for k in sources if t.startswith(k)), None)
        if key and cur.get("kernel_source_sha256") == source_hash(sources[key]):
            out[t] = float(cur["hbm_bytes_per_launch"])

    for line in open(path):
        if line.startswith("kernel:"):
            flush()
            cur = {}
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            cur[k.strip()] = v.strip()
    flush()
    return out or None


def scan_algorithmic_bytes(w, with_final=True):
    """Each input / output tensor of the scan moved once (chunk states excluded):
    x, y, B, C, dt per token in the I/O dtype, seq_idx (int32) when packed, the
    fp32 initial states when given and the final states, the per-head params."""
    T = w.batch * w.seqlen
    H, G, P, N = w.nheads, w.ngroups, w.headdim, w.dstate
    es = 2 if w.bf16 else 4
    per_tok = (2 * (H * P) + 2 * (G * N) + H) * es + (4 if w.packed_lengths is not None else 0)
    state = w.num_seqs * H * P * N * 4
    states = (state if with_final else 0) + (state if w.init_std > 0 else 0)
    return T * per_tok + states + 3 * H * 4


def scan_flops(w):
    """Useful flops: causal triangles counted once, C B^T once per (chunk, group)."""
    T = w.batch * w.seqlen
    H, G, P, N, Q = w.nheads, w.ngroups, w.headdim, w.dstate, w.chunk
    return T * (G * (Q + 1) * N + H * (Q + 1) * P + 4 * H * P * N)


def conv_algorithmic_bytes(w, channels=None):
    """The conv over `channels` (all by default): input read and output written
    once, the fp32 taps, seq_idx when packed."""
    es = 2 if w.bf16 else 4
    ch = w.conv_dim if channels is None else channels
    return (w.batch * w.seqlen * ch * 2 * es + ch * 4 * 4
            + (w.batch * w.seqlen * 4 if w.packed_lengths is not None else 0))


def fused_scan_algorithmic_bytes(w):
    """The scan kernel with the x channels' conv inside: the scan's bytes (raw x
    has post-conv x's size) plus those channels' taps and bias."""
    return scan_algorithmic_bytes(w) + w.nheads * w.headdim * (4 + 1) * 4


def step_algorithmic_bytes(w):
    """The whole conv + scan step at its minimum: xBC read once, y written
    once, dt, states and parameters; no intermediate."""
    T = w.batch * w.seqlen
    H, P = w.nheads, w.headdim
    es = 2 if w.bf16 else 4
    state = w.num_seqs * H * P * w.dstate * 4
    return (T * (w.conv_dim + H * P + H) * es + state + (state if w.init_std > 0 else 0)
            + w.conv_dim * 5 * 4 + 3 * H * 4 + (T * 4 if w.packed_lengths is not None else 0))


def decode_algorithmic_bytes(dw):
    H, G, P, N = dw.nheads, dw.ngroups, dw.headdim, dw.dstate
    CD = dw.conv_dim
    b = dw.batch
    return (2 * b * H * P * N * 4            # state read + write
            + b * CD * 2                     # token
            + 2 * b * (dw.conv_width - 1) * CD * 2   # conv state read + write
            + b * H * P * 2 + b * H * 2      # y, dt
            + CD * dw.conv_width * 4 + 3 * H * 4)


class ScanRun:
    """Device tensors of one prefill config and its step, launched through the
    C ABI: the fused conv + scan (ssd_conv_scan_fwd) when the workload has a
    conv, else the scan; both with final states.  The unfused pair (conv then
    scan) and the fused call's first kernel alone (the B|C conv) are timed
    beside it."""

    def __init__(self, w, seed):
        import torch
        from state_space_sequence_ssd_amd import inputs, ssd
        self.w, self.ssd = w, ssd
        dev = torch.device("cuda:0")
        dtp = torch.bfloat16 if w.bf16 else torch.float32
        self.d = d = inputs.make_scan_inputs(w, seed=seed)
        H, G, P, N = w.nheads, w.ngroups, w.headdim, w.dstate
        Bt, L = w.batch, w.seqlen
        self.seq = torch.from_numpy(d["seq_idx"]).to(dev) if "seq_idx" in d else None
        self.nseq = w.num_seqs if self.seq is not None else None
        if w.conv:
            self.xbc = torch.from_numpy(d["xBC"]).to(dev, dtp)
            self.conv_w = torch.from_numpy(d["conv_w"]).to(dev)
            self.conv_out = torch.empty_like(self.xbc)
            co = self.conv_out
            self.x = co[..., :H * P].view(Bt, L, H, P)
            self.B = co[..., H * P:H * P + G * N].view(Bt, L, G, N)
            self.C = co[..., H * P + G * N:].view(Bt, L, G, N)
        else:
            self.x = torch.from_numpy(d["x"]).to(dev, dtp)
            self.B = torch.from_numpy(d["B"]).to(dev, dtp)
            self.C = torch.from_numpy(d["C"]).to(dev, dtp)
        self.dt = torch.from_numpy(d["dt"]).to(dev, dtp)
        self.A, self.D = torch.from_numpy(d["A"]).to(dev), torch.from_numpy(d["D"]).to(dev)
        self.dt_bias = torch.from_numpy(d["dt_bias"]).to(dev)
        self.init = torch.from_numpy(d["initial_state"]).to(dev) if "initial_state" in d else None
        self.y = torch.empty((Bt, L, H, P), dtype=dtp, device=dev)
        self.fs = torch.empty((w.num_seqs, H, P, N), dtype=torch.float32, device=dev)
        wsb = ssd.ssd_chunk_scan_workspace_size(self.x, self.dt, self.A, self.B, self.C, seq_idx=self.seq,
                                                num_seqs=self.nseq)
        self.ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev)
        if w.conv:
            fwb = ssd.ssd_conv_scan_workspace_size(self.xbc, self.conv_w, self.dt, self.A, H, G,
                                                   seq_idx=self.seq, num_seqs=self.nseq)
            self.fws = torch.empty(max(fwb, 1), dtype=torch.uint8, device=dev)
            # the fused call's B|C conv on its own (same kernel, same launch)
            self.bc_in = self.xbc[..., H * P:]
            self.bc_w = self.conv_w[H * P:]
            self.bc_out = torch.empty((Bt, L, 2 * G * N), dtype=dtp, device=dev)
        self.stream = torch.cuda.current_stream()

    def scan_call(self):
        self.ssd.ssd_chunk_scan_fwd(self.x, self.dt, self.A, self.B, self.C, dt_bias=self.dt_bias, D=self.D,
                                    seq_idx=self.seq, num_seqs=self.nseq, initial_state=self.init,
                                    final_state=self.fs, y=self.y, workspace=self.ws)

    def step(self, ev=None):
        """The timed step: fused conv + scan (conv workloads) or the scan."""
        if ev is not None:
            ev[0].record(self.stream)
        if self.w.conv:
            H, G = self.w.nheads, self.w.ngroups
            self.ssd.ssd_conv_scan_fwd(self.xbc, self.conv_w, self.dt, self.A, H, G, dt_bias=self.dt_bias,
                                       D=self.D, seq_idx=self.seq, num_seqs=self.nseq, initial_state=self.init,
                                       final_state=self.fs, y=self.y, workspace=self.fws)
        else:
            self.scan_call()
        if ev is not None:
            ev[1].record(self.stream)

    def step_unfused(self, ev):
        """Reference: the conv kernel over every channel, then the scan."""
        ev[0].record(self.stream)
        self.ssd.ssd_conv1d_silu(self.xbc, self.conv_w, seq_idx=self.seq, num_seqs=self.nseq, out=self.conv_out)
        ev[1].record(self.stream)
        self.scan_call()
        ev[2].record(self.stream)

    def step_conv_bc(self, ev):
        """The fused call's first kernel alone: the conv of the B|C channels."""
        ev[0].record(self.stream)
        self.ssd.ssd_conv1d_silu(self.bc_in, self.bc_w, seq_idx=self.seq, num_seqs=self.nseq, out=self.bc_out)
        ev[1].record(self.stream)

    def timed(self, steps, warmup):
        """W untimed steps, then K steps, each bracketed by events, and events
        around the whole region.  Returns (total_ms, step_ms list, wall_s)."""
        import torch
        for _ in range(warmup):
            self.step()
        torch.cuda.synchronize()
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        wall0 = time.perf_counter()
        t0.record(self.stream)
        for i in range(steps):
            self.step(evs[i])
        t1.record(self.stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - wall0
        return t0.elapsed_time(t1), [e[0].elapsed_time(e[1]) for e in evs], wall

    def timed_parts(self, steps, warmup):
        """Conv workloads: per-kernel event times of the unfused pair (conv,
        scan) and of the fused call's B|C conv alone, each over K steps after
        W warm-ups.  Returns {"conv": [...], "scan": [...], "conv_bc": [...]}."""
        import torch
        out = {"conv": [], "scan": [], "conv_bc": []}
        for k in range(warmup + steps):
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
            self.step_unfused(ev)
            if k >= warmup:
                out["conv"].append(ev)
        for k in range(warmup + steps):
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            self.step_conv_bc(ev)
            if k >= warmup:
                out["conv_bc"].append(ev)
        torch.cuda.synchronize()
        evs = out["conv"]
        out["conv"] = [e[0].elapsed_time(e[1]) for e in evs]
        out["scan"] = [e[1].elapsed_time(e[2]) for e in evs]
        out["conv_bc"] = [e[0].elapsed_time(e[1]) for e in out["conv_bc"]]
        return out

    def graph_ms(self, steps, replays=3):
        """GPU time per step with `steps` steps captured in one HIP graph and
        replayed, so no host work sits between the kernels.  Every replay's y
        and final states must equal the eager step's bit for bit (the kernels
        sum in a fixed order); the outputs are cleared by eager work between
        replays.  Returns the median over `replays` replays."""
        import numpy as np
        import torch
        self.step()
        torch.cuda.synchronize()
        y0, fs0 = self.y.clone(), self.fs.clone()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            self.step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(steps):
                self.step()
        times = []
        for _ in range(replays):
            self.y.zero_()
            self.fs.zero_()
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            g.replay()
            b.record()
            torch.cuda.synchronize()
            times.append(a.elapsed_time(b) / steps)
            if not (torch.equal(self.y, y0) and torch.equal(self.fs, fs0)):
                raise RuntimeError(f"{self.w.name}: graph replay differs from the eager step")
        del g
        return float(np.median(times))

    def launch_inclusive_ms(self, steps):
        """Host wall clock per back-to-back call of the whole step."""
        import torch
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            self.step()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / steps


def rate(nbytes, ms):
    gbs = nbytes / (ms * 1e-3) / 1e9
    return round(gbs, 1), round(gbs / HBM_PEAK_GBS, 4)


def config_result(run, steps, warmup):
    """One synthetic config, event-timed on the launch stream; rates against
    the HBM roofline.  Conv workloads time the fused step; its scan kernel is
    the step minus the fused call's B|C conv (that launch timed alone), and
    the unfused pair is reported beside it."""
    import numpy as np
    w = run.w
    _, step_list, _ = run.timed(steps, warmup)
    step_ms = float(np.mean(step_list))
    tokens = w.batch * w.seqlen
    out = {"tokens": tokens, "io_dtype": "bf16" if w.bf16 else "f32", "step_avg_ms": round(step_ms, 5),
           "layer_tokens_per_s": round(tokens / (step_ms * 1e-3), 1)}
    if w.conv:
        parts = run.timed_parts(steps, warmup)
        bc_ms = float(np.mean(parts["conv_bc"]))
        scan_ms = step_ms - bc_ms
        sb = fused_scan_algorithmic_bytes(w)
        cbb = conv_algorithmic_bytes(w, 2 * w.ngroups * w.dstate)
        stb = step_algorithmic_bytes(w)
        u_conv, u_scan = float(np.mean(parts["conv"])), float(np.mean(parts["scan"]))
        out.update({
            "step": "fused conv + scan (ssd_conv_scan_fwd): B|C conv kernel, then the scan with the x conv inside",
            "step_algorithmic_bytes": stb, "step_gbs": rate(stb, step_ms)[0], "step_hbm_frac": rate(stb, step_ms)[1],
            "conv_bc_avg_ms": round(bc_ms, 5), "conv_bc_algorithmic_bytes": cbb,
            "conv_bc_hbm_frac": rate(cbb, bc_ms)[1],
            "scan_timing": "fused step minus the B|C conv launched alone (HIP events)",
            "unfused": {"conv_avg_ms": round(u_conv, 5), "scan_avg_ms": round(u_scan, 5),
                        "step_ms": round(u_conv + u_scan, 5),
                        "layer_tokens_per_s": round(tokens / ((u_conv + u_scan) * 1e-3), 1),
                        "conv_hbm_frac": rate(conv_algorithmic_bytes(w), u_conv)[1],
                        "scan_hbm_frac": rate(scan_algorithmic_bytes(w), u_scan)[1]}})
    else:
        scan_ms = step_ms
        sb = scan_algorithmic_bytes(w)
    out.update({"scan_avg_ms": round(scan_ms, 5), "scan_algorithmic_bytes": sb,
                "scan_gbs": rate(sb, scan_ms)[0], "scan_hbm_frac": rate(sb, scan_ms)[1],
                "scan_tokens_per_s": round(tokens / (scan_ms * 1e-3), 1)})
    out["step_launch_inclusive_ms"] = round(run.launch_inclusive_ms(steps), 5)
    gms = run.graph_ms(steps)
    out["step_graph_ms"] = round(gms, 5)
    out["layer_tokens_per_s_graph"] = round(tokens / (gms * 1e-3), 1)
    out["traffic_per_kernel"] = read_traffic_all(w.name)
    return out


# ---------------------------------------------------------------------------
# the fp64 oracle beside the GPU: all OpenMP threads and one, bounded samples
# ---------------------------------------------------------------------------
_GOMP = None


def omp_threads(n=None):
    """Get (n None) or set the OpenMP thread count of the oracle's runtime."""
    global _GOMP
    import ctypes
    if _GOMP is None:
        _GOMP = ctypes.CDLL("libgomp.so.1")
    if n is None:
        return _GOMP.omp_get_max_threads()
    _GOMP.omp_set_num_threads(int(n))
    return n


def host_info():
    import torch
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    rocm = None
    try:
        rocm = open("/opt/rocm/.info/version").read().strip()
    except OSError:
        pass
    drv = None
    try:
        drv = open("/sys/module/amdgpu/version").read().strip()
    except OSError:
        pass
    return {"cpu_model": model, "host_cpus_usable": len(os.sched_getaffinity(0)),
            "omp_threads": omp_threads(), "rocm": rocm, "amdgpu_driver": drv,
            "torch": torch.__version__, "torch_hip": getattr(torch.version, "hip", None),
            "gpu": torch.cuda.get_device_name(0)}


def oracle_scan_sample(w, d, rows=None, seqs=None, tokens=None):
    """The oracle's conv (if any) + scan with final states over a sample of one
    workload: the first `rows` batch rows, or the first `seqs` packed
    sequences, or the first `tokens` tokens of a one-row stream.  Returns
    (y, final_state, seconds, tokens, description)."""
    import numpy as np
    import oracle
    H, G, P, N = w.nheads, w.ngroups, w.headdim, w.dstate
    seq_idx = d.get("seq_idx")
    init = d.get("initial_state")
    if seqs is None and rows is None and tokens is None and seq_idx is not None:
        seqs = w.num_seqs            # a packed stream: the sample is whole sequences
    if seqs is not None:
        T = int(np.sum(w.packed_lengths[:seqs]))
        bsel, tsel = slice(0, 1), slice(0, T)
        seq_idx, nseq = seq_idx[:T], seqs
        init = None if init is None else init[:seqs]
        desc = f"first {seqs} of {w.num_seqs} packed sequences ({T} tokens), all {H} heads"
    else:
        r = rows if rows is not None else w.batch
        T = tokens if tokens is not None else w.seqlen
        bsel, tsel = slice(0, r), slice(0, T)
        nseq = None
        init = None if init is None else init[:r]
        desc = (f"batch rows 0..{r - 1} of {w.batch}, tokens 0..{T - 1} of {w.seqlen}, all {H} heads")
    t0 = time.perf_counter()
    if w.conv:
        v = oracle.conv1d_silu(d["xBC"][bsel, tsel], d["conv_w"], seq_idx=seq_idx, num_seqs=nseq)
        b_ = v.shape[0]
        x = v[..., :H * P].reshape(b_, -1, H, P)
        B = v[..., H * P:H * P + G * N].reshape(b_, -1, G, N)
        C = v[..., H * P + G * N:].reshape(b_, -1, G, N)
    else:
        x, B, C = d["x"][bsel, tsel], d["B"][bsel, tsel], d["C"][bsel, tsel]
    y, fs = oracle.ssd_scan(x, d["dt"][bsel, tsel], d["dt_bias"], d["A"], B, C, d["D"], seq_idx=seq_idx,
                            num_seqs=nseq, initial_state=init, want_final_state=True)
    el = time.perf_counter() - t0
    ntok = (bsel.stop - bsel.start) * (tsel.stop - tsel.start)
    step = "fp64 conv then fp64 sequential recurrence" if w.conv else "fp64 sequential recurrence"
    return y, fs, el, ntok, f"{desc}: {step} with final states"


def rel_err(a, ref):
    import numpy as np
    den = float(np.max(np.abs(ref))) if ref.size else 0.0
    err = float(np.max(np.abs(np.asarray(a, np.float64) - ref))) if ref.size else 0.0
    return err / den if den > 0 else err


def oracle_beside(run, all_sample, one_sample, parity=True):
    """Oracle tokens/s on all threads (all_sample) and on one (one_sample), and
    the parity error of the GPU outputs against the all-thread outputs, which
    are the oracle's result on the same inputs (the sample's rows/tokens)."""
    import numpy as np
    w, d = run.w, run.d
    n = omp_threads()
    y, fs, el, ntok, desc = oracle_scan_sample(w, d, **all_sample)
    res = {"value": round(ntok / el, 1), "unit": "tokens/s/layer", "cores": n, "kind": "oracle",
           "sample": f"{desc}, {el:.2f} s wall"}
    if parity:
        bs = dict(all_sample)
        if d.get("seq_idx") is not None and not bs:
            bs["seqs"] = w.num_seqs       # a packed stream: the whole-sequence sample
        if "seqs" in bs:
            T = y.shape[1]
            yg = run.y[:, :T]
            fg = run.fs[:bs["seqs"]]
        else:
            r = bs.get("rows") or w.batch
            T = bs.get("tokens") or w.seqlen
            yg = run.y[:r, :T]
            fg = run.fs[:r] if T == w.seqlen else None
        ey = rel_err(yg.float().cpu().numpy(), y)
        res["parity"] = {"y_rel_err": float(f"{ey:.3e}"), "bar": 2e-2 if w.bf16 else 1e-4}
        if fg is not None:
            res["parity"]["final_state_rel_err"] = float(f"{rel_err(fg.cpu().numpy(), fs):.3e}")
    del y, fs
    omp_threads(1)
    try:
        _, _, el1, ntok1, desc1 = oracle_scan_sample(w, d, **one_sample)
    finally:
        omp_threads(n)
    one = {"value": round(ntok1 / el1, 1), "unit": "tokens/s/layer", "cores": 1, "kind": "oracle",
           "sample": f"{desc1}, {el1:.2f} s wall"}
    return res, one


def oracle_decode_beside(dw, rows_all, rows_one):
    """Oracle decode on a sample of batch rows of one layer (fresh inputs of
    the same workload), all threads and one: tokens/s and algorithmic GB/s
    scaled per token."""
    import oracle
    from state_space_sequence_ssd_amd import inputs
    n = omp_threads()
    out = {}
    for tag, rows in (("all", rows_all), ("one", rows_one)):
        w = inputs.DecodeWorkload(dw.name, rows, dw.nheads, dw.ngroups, 1, bf16=dw.bf16)
        dd = inputs.make_decode_small_inputs(w, seed=4, layer=0)
        st = inputs.decode_state_host(w, 4, 0)
        if tag == "one":
            omp_threads(1)
        try:
            t0 = time.perf_counter()
            oracle.decode_step(dd["xBC"], dd["dt"], dd["dt_bias"], dd["A"], dd["D"], st, dw.nheads,
                               dw.headdim, dw.dstate, dw.ngroups, conv_w=dd["conv_w"],
                               conv_state=dd["conv_state"])
            el = time.perf_counter() - t0
        finally:
            omp_threads(n)
        bytes_per_tok = decode_algorithmic_bytes(dw) / dw.batch
        out[tag] = {"value": round(rows / el, 1), "unit": "tokens/s/layer",
                    "gbs": round(rows * bytes_per_tok / el / 1e9, 2),
                    "cores": n if tag == "all" else 1, "kind": "oracle",
                    "sample": f"one layer, {rows} of {dw.batch} batch rows (fresh inputs of the same "
                              f"distributions): fp64 conv window + recurrence step, {el:.2f} s wall"}
    return out["all"], out["one"]


# ---------------------------------------------------------------------------
class DecodeRun:
    """Batch-256 decode through 29 layers, inputs resident on the device:
    HBM GB/s of the whole sweep, one layer's event-timed kernel, and the
    parity of the first application on 16 rows of layer 0 against the oracle."""

    PROW = 16

    def __init__(self):
        import torch
        from state_space_sequence_ssd_amd import inputs
        dev = torch.device("cuda:0")
        bf = torch.bfloat16
        self.dw = dw = inputs.decode_29_layers()
        self.layers = []
        for l in range(dw.layers):
            dd = inputs.make_decode_small_inputs(dw, seed=4, layer=l)
            self.layers.append({
                "xBC": torch.from_numpy(dd["xBC"]).to(dev, bf),
                "dt": torch.from_numpy(dd["dt"]).to(dev, bf),
                "conv_state": torch.from_numpy(dd["conv_state"]).to(dev, bf),
                "conv_w": torch.from_numpy(dd["conv_w"]).to(dev),
                "A": torch.from_numpy(dd["A"]).to(dev), "D": torch.from_numpy(dd["D"]).to(dev),
                "dt_bias": torch.from_numpy(dd["dt_bias"]).to(dev),
                "state": inputs.decode_state_device(dw, 4, l, dev),
                "y": torch.empty((dw.batch, dw.nheads, dw.headdim), dtype=bf, device=dev)})
            if l == 0:
                self.host0 = dd
        self.st0 = self.layers[0]["state"][:self.PROW].cpu().numpy()

    def dstep(self, stream, ev=None):
        from state_space_sequence_ssd_amd import ssd
        dw = self.dw
        for li, L_ in enumerate(self.layers):
            if ev is not None and li == 0:
                ev[0].record(stream)
            ssd.ssd_decode_step(L_["xBC"], L_["dt"], L_["A"], L_["state"], dw.nheads, dw.ngroups,
                                dt_bias=L_["dt_bias"], D=L_["D"], conv_state=L_["conv_state"],
                                conv_weight=L_["conv_w"], y=L_["y"])
            if ev is not None and li == 0:
                ev[1].record(stream)

    def timed(self, args, stream):
        import numpy as np
        import torch
        dw, prow = self.dw, self.PROW
        self.dstep(stream)
        torch.cuda.synchronize()
        self.y_first = self.layers[0]["y"][:prow].float().cpu().numpy()
        self.s_first = self.layers[0]["state"][:prow].cpu().numpy()
        for _ in range(2):
            self.dstep(stream)
        torch.cuda.synchronize()
        devs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.decode_steps)]
        d0, d1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        d0.record(stream)
        for i in range(args.decode_steps):
            self.dstep(stream, devs[i])
        d1.record(stream)
        torch.cuda.synchronize()
        dms = d0.elapsed_time(d1) / args.decode_steps
        one_layer_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in devs]))
        dbytes = decode_algorithmic_bytes(dw)
        gbs = dbytes * dw.layers / (dms * 1e-3) / 1e9
        self.layers = None
        torch.cuda.empty_cache()
        return {"metric": "decode-step HBM GB/s", "value": round(gbs, 1), "unit": "GB/s",
                "frac": round(gbs / HBM_PEAK_GBS, 4), "ms_per_29_layers": round(dms, 4),
                "tokens_per_s": round(dw.batch / (dms * 1e-3), 1),
                "layer_kernel_avg_ms": round(one_layer_ms, 4),
                "layer_kernel_gbs": round(dbytes / (one_layer_ms * 1e-3) / 1e9, 1),
                "algorithmic_bytes_per_layer": dbytes,
                "traffic": read_traffic("decode_step_b256_h128", DECODE_SOURCES),
                "workload": dw.name}

    def parity(self):
        import oracle
        h, dw, prow = self.host0, self.dw, self.PROW
        ry, rs, _ = oracle.decode_step(h["xBC"][:prow], h["dt"][:prow], h["dt_bias"], h["A"], h["D"], self.st0,
                                       dw.nheads, dw.headdim, dw.dstate, dw.ngroups, conv_w=h["conv_w"],
                                       conv_state=h["conv_state"][:prow])
        return {"y_rel_err": float(f"{rel_err(self.y_first, ry):.3e}"),
                "state_rel_err": float(f"{rel_err(self.s_first, rs):.3e}"), "bar": 2e-2,
                "sample": f"layer 0, batch rows 0..{prow - 1}, first application"}


CONFIG_SAMPLES = {
    # name: (all-thread sample, one-thread sample)
    "tiny_fp32_h8_l512": ({}, {}),
    "nemotron3_nano_b1_l16384": ({}, {"tokens": 2048}),
    "packed_3b_h40_32seqs": ({}, {"seqs": 2}),
}


def progress(msg):
    """One line per finished part on stderr (the JSON line alone goes to stdout)."""
    print(f"bench: {msg}", file=sys.stderr, flush=True)


class NormRun:
    """The gated RMSNorm after the scan at the headline shape: y is the scan's
    output tensor, z the gate half of a synthetic in-projection output."""

    def __init__(self, w, y):
        import torch
        from state_space_sequence_ssd_amd import inputs
        dev = torch.device("cuda:0")
        self.w, self.y = w, y
        CH = w.nheads * w.headdim
        self.gs = CH // w.ngroups
        d = inputs.norm_inputs(w.batch, w.seqlen, CH, seed=1)
        self.z = torch.from_numpy(d["z"]).to(dev, y.dtype)
        self.wt = torch.from_numpy(d["w"]).to(dev)
        self.z_host, self.w_host = d["z"], d["w"]
        self.out = torch.empty((w.batch, w.seqlen, CH), dtype=y.dtype, device=dev)

    def step(self):
        from state_space_sequence_ssd_amd import ssd
        ssd.ssd_gated_rmsnorm(self.y, self.wt, self.gs, z=self.z, out=self.out)

    def timed(self, steps, warmup, stream):
        import numpy as np
        import torch
        for _ in range(warmup):
            self.step()
        torch.cuda.synchronize()
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
        for e in evs:
            e[0].record(stream)
            self.step()
            e[1].record(stream)
        torch.cuda.synchronize()
        ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
        w = self.w
        T, CH = w.batch * w.seqlen, w.nheads * w.headdim
        nbytes = 3 * T * CH * 2 + CH * 4          # y, z, out (bf16), weights
        return {"avg_ms": round(ms, 5), "algorithmic_bytes": nbytes,
                "gbs": round(nbytes / (ms * 1e-3) / 1e9, 1),
                "hbm_frac": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                "tokens_per_s": round(T / (ms * 1e-3), 1), "group_size": self.gs,
                "gate": "after (y * SiLU(z), then the norm)",
                "traffic": read_traffic("gated_rmsnorm_nemotron_h_8b", NORM_SOURCES)}

    def parity(self, rows):
        """Oracle on the first `rows` token rows of batch row 0 (all channels)."""
        import oracle
        yh = self.y[0, :rows].float().cpu().numpy().reshape(rows, -1)
        ref = oracle.gated_rmsnorm(yh, self.z_host[0, :rows], self.w_host, self.gs)
        og = self.out[0, :rows].float().cpu().numpy()
        return {"out_rel_err": float(f"{rel_err(og, ref):.3e}"), "bar": 2e-2,
                "sample": f"batch row 0, tokens 0..{rows - 1}, all channels"}


def mimo_algorithmic_bytes(dw, R, trap, es=2):
    """MIMO decode step: state read + written once (fp32), x, B, C, dt, lam, y
    in the I/O dtype, and with the trapezoidal term the previous-input caches
    read and rewritten, per-head params."""
    b, H, G, P, N = dw.batch, dw.nheads, dw.ngroups, dw.headdim, dw.dstate
    n = 2 * b * H * P * N * 4 + (2 * b * H * P * R + 2 * b * G * N * R + b * H) * es + 3 * H * 4
    if trap:
        n += b * H * es + 2 * (b * H * P * R + b * G * N * R) * es
    return n


class MimoRun:
    """MIMO decode step at the decode workload's shape (batch 256, 128 heads,
    8 groups, 1 GiB fp32 state): rank 1 and 4, Euler and trapezoidal."""

    VARIANTS = [(1, False), (4, False), (4, True), (8, True)]

    def __init__(self):
        import torch
        from state_space_sequence_ssd_amd import inputs
        dev = torch.device("cuda:0")
        self.dw = dw = inputs.decode_29_layers()
        self.state = inputs.decode_state_device(dw, 12, 0, dev)
        self.t = {}
        for R, trap in self.VARIANTS:
            d = inputs.mimo_decode_inputs(dw.batch, dw.nheads, dw.ngroups, R, seed=12)
            self.t[(R, trap)] = {k: torch.from_numpy(v).to(dev, torch.bfloat16 if k not in ("dt_bias", "A", "D")
                                                         else None) for k, v in d.items()}

    def timed(self, steps, stream):
        import numpy as np
        import torch
        from state_space_sequence_ssd_amd import ssd
        out = {}
        traffic = read_traffic_all("decode_b256_h128") or {}
        for (R, trap), t in self.t.items():
            def step():
                ssd.ssd_decode_step_mimo(t["x"], t["B"], t["C"], t["dt"], t["A"], self.state, dt_bias=t["dt_bias"],
                                         D=t["D"], trapezoid=trap, lam=t["lam"] if trap else None,
                                         prev_x=t["prev_x"] if trap else None, prev_B=t["prev_B"] if trap else None)
            for _ in range(3):
                step()
            torch.cuda.synchronize()
            evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
            for e in evs:
                e[0].record(stream)
                step()
                e[1].record(stream)
            torch.cuda.synchronize()
            ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
            nb = mimo_algorithmic_bytes(self.dw, R, trap)
            out[f"rank{R}_{'trapezoid' if trap else 'euler'}"] = {
                "avg_ms": round(ms, 4), "algorithmic_bytes": nb, "gbs": round(nb / (ms * 1e-3) / 1e9, 1),
                "hbm_frac": round(nb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                "tokens_per_s": round(self.dw.batch / (ms * 1e-3), 1),
                "traffic": traffic.get(f"decode_mimo_r{R}_{'trapezoid' if trap else 'euler'}")}
        self.state = None
        torch.cuda.empty_cache()
        return out


class MixerRun:
    """The whole Mamba-2 mixer at the headline layer shape (d_model 4096,
    d_inner 8192, 128 heads, 8 groups, batch 4 x 4096 tokens): in_proj, the
    fused conv + scan, the gated RMSNorm and out_proj, each a libssd call on
    the views of the in_proj output, event-timed per call; the projections
    against the bf16 matrix-core roofline, with sampled rows against the oracle."""
    D_MODEL = 4096

    def __init__(self, w):
        import torch
        from state_space_sequence_ssd_amd import inputs
        self.w = w
        d = inputs.mixer_inputs(w.batch, w.seqlen, self.D_MODEL, w.nheads, w.ngroups, seed=9)
        self.d = d
        dev = torch.device("cuda:0")
        self.t = {k: torch.from_numpy(v).to(dev, torch.bfloat16 if k in ("hidden", "in_proj_w", "out_proj_w")
                                               else None) for k, v in d.items()}

    def timed(self, steps, warmup, stream):
        import numpy as np
        import torch
        from state_space_sequence_ssd_amd import ssd
        w, t = self.w, self.t
        H, G, P, N = w.nheads, w.ngroups, w.headdim, w.dstate
        d_inner, conv_dim = H * P, H * P + 2 * G * N
        Bt, L, dm = w.batch, w.seqlen, self.D_MODEL
        d_in_proj = 2 * d_inner + 2 * G * N + H
        zx = torch.empty((Bt, L, d_in_proj), dtype=torch.bfloat16, device="cuda")
        y = torch.empty((Bt, L, H, P), dtype=torch.bfloat16, device="cuda")
        yn = torch.empty((Bt, L, d_inner), dtype=torch.bfloat16, device="cuda")
        out = torch.empty((Bt, L, dm), dtype=torch.bfloat16, device="cuda")
        xbc, dt, z = zx[..., d_inner:d_inner + conv_dim], zx[..., d_inner + conv_dim:], zx[..., :d_inner]
        wsb = ssd.ssd_conv_scan_workspace_size(xbc, t["conv_w"], dt, t["A"], H, G)
        ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device="cuda")

        def step(ev=None):
            rec = (lambda i: ev[i].record(stream)) if ev is not None else (lambda i: None)
            rec(0)
            ssd.ssd_linear(t["hidden"], t["in_proj_w"], y=zx)
            rec(1)
            ssd.ssd_conv_scan_fwd(xbc, t["conv_w"], dt, t["A"], H, G, dt_bias=t["dt_bias"], D=t["D"], y=y,
                                  workspace=ws)
            rec(2)
            ssd.ssd_gated_rmsnorm(y.flatten(2), t["norm_w"], d_inner // G, z=z, out=yn)
            rec(3)
            ssd.ssd_linear(yn, t["out_proj_w"], y=out)
            rec(4)

        for _ in range(warmup):
            step()
        torch.cuda.synchronize()
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(steps)]
        for e in evs:
            step(e)
        torch.cuda.synchronize()
        names = ["in_proj", "conv_scan", "gated_rmsnorm", "out_proj"]
        ms = {n: float(np.mean([e[i].elapsed_time(e[i + 1]) for e in evs])) for i, n in enumerate(names)}
        layer_ms = float(np.mean([e[0].elapsed_time(e[4]) for e in evs]))
        T = Bt * L
        fl_in, fl_out = 2.0 * T * d_in_proj * dm, 2.0 * T * dm * d_inner

        traffic = read_traffic_all(w.name) or {}

        def gemm(name, flops, M, Nn, K):
            tf = flops / (ms[name] * 1e-3) / 1e12
            # operands and result once: x (M x K) and w (N x K) read, y (M x N) written, bf16
            return {"avg_ms": round(ms[name], 5), "M": M, "N": Nn, "K": K, "tflops": round(tf, 1),
                    "roofline": {"bound": "mfma", "achieved": round(tf, 1), "peak": BF16_MFMA_PEAK_TFLOPS,
                                 "unit": "TFLOP/s", "frac": round(tf / BF16_MFMA_PEAK_TFLOPS, 4),
                                 "traffic": traffic.get(f"linear_bf16_{name}")},
                    "algorithmic_bytes": 2 * (M * K + Nn * K + M * Nn)}
        res = {"workload": f"Mamba-2 mixer, d_model {dm}, d_inner {d_inner}, {w.name}",
               "ms_per_layer": round(layer_ms, 5), "tokens_per_s": round(T / (layer_ms * 1e-3), 1),
               "in_proj": gemm("in_proj", fl_in, T, d_in_proj, dm),
               "out_proj": gemm("out_proj", fl_out, T, dm, d_inner),
               "conv_scan_ms": round(ms["conv_scan"], 5), "gated_rmsnorm_ms": round(ms["gated_rmsnorm"], 5)}
        self.zx, self.out = zx, out
        return res

    def parity(self, nrows=8):
        """Sampled token rows of the timed in_proj output against the oracle's
        product of the same hidden rows (out_proj's parity is in the GPU tests)."""
        import numpy as np
        import oracle
        T = self.w.batch * self.w.seqlen
        rows = np.random.default_rng(3).choice(T, nrows, replace=False)
        h = self.d["hidden"].reshape(T, -1)[rows]
        ref = oracle.linear(h, self.d["in_proj_w"])
        got = self.zx.reshape(T, -1)[rows].float().cpu().numpy()
        return {"in_proj_rel_err": float(f"{rel_err(got, ref):.3e}"), "rows": int(nrows), "bar": 2 ** -8}


def bwd_flops(w, Q=32):
    """Matrix-core flops of the backward's chunked form (chunks of Q tokens),
    per (batch row, head, chunk): the forward state walk (x^T B), the token
    products C B^T and dy x^T, the state-sized products G1 B, S0 C, x G1,
    S0^T dy and dy C^T, and the in-chunk products of dx, dB and dC."""
    P, N = w.headdim, w.dstate
    nch = -(-w.seqlen // Q)
    per = 2 * (3 * Q * Q * N + 2 * Q * Q * P + 6 * Q * P * N)
    return per * w.batch * w.nheads * nch


class BwdRun:
    """The scan's backward pass at the headline shape (bf16 inputs; products
    on the bf16 matrix cores with fp32 intermediates split into bf16 hi + lo
    parts, fp32 sums): gradients of x, dt, B, C, the per-head parameters and
    the initial state from dy and a final-state gradient."""

    def __init__(self, w):
        import torch
        from state_space_sequence_ssd_amd import inputs, ssd
        dev = torch.device("cuda:0")
        self.w = w
        d = inputs.make_scan_inputs(inputs.ScanWorkload(w.name, w.batch, w.seqlen, w.nheads, w.ngroups, bf16=True,
                                                        conv=False, final_state=True), seed=1)
        bf = torch.bfloat16
        self.t = {k: torch.from_numpy(d[k]).to(dev, bf) for k in ("x", "dt", "B", "C")}
        self.t.update({k: torch.from_numpy(d[k]).to(dev) for k in ("A", "D", "dt_bias")})
        self.t["dy"] = torch.from_numpy(inputs.normal((w.batch, w.seqlen, w.nheads, w.headdim), 1.0, 1, 61,
                                                      True)).to(dev, bf)
        self.t["df"] = torch.from_numpy(inputs.normal((w.batch, w.nheads, w.headdim, w.dstate), 0.1, 1, 62,
                                                      False)).to(dev)
        t = self.t
        self.ws = None
        g = ssd.ssd_chunk_scan_bwd(t["x"], t["dt"], t["A"], t["B"], t["C"], t["dy"], dt_bias=t["dt_bias"],
                                   D=t["D"], d_final_state=t["df"], want_d_initial_state=True)
        del g

    def timed(self, steps, warmup, stream):
        import numpy as np
        import torch
        from state_space_sequence_ssd_amd import ssd
        t, w = self.t, self.w

        def step():
            return ssd.ssd_chunk_scan_bwd(t["x"], t["dt"], t["A"], t["B"], t["C"], t["dy"], dt_bias=t["dt_bias"],
                                          D=t["D"], d_final_state=t["df"], want_d_initial_state=True)
        for _ in range(warmup):
            step()
        torch.cuda.synchronize()
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
        for e in evs:
            e[0].record(stream)
            step()
            e[1].record(stream)
        torch.cuda.synchronize()
        ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
        T, H, G, P, N = w.batch * w.seqlen, w.nheads, w.ngroups, w.headdim, w.dstate
        nbytes = T * (2 * (2 * H * P) + 2 * (2 * G * N) + 2 * H) * 2 + 2 * w.batch * H * P * N * 4
        flops = bwd_flops(w)
        tf = flops / (ms * 1e-3) / 1e12
        traffic = read_traffic_all(w.name) or {}
        bwd_traffic = {k: v for k, v in traffic.items() if k.startswith("bwd")} or None
        out = {"avg_ms": round(ms, 4), "tokens_per_s": round(T / (ms * 1e-3), 1),
               "algorithmic_bytes": nbytes, "gbs": round(nbytes / (ms * 1e-3) / 1e9, 1),
               "hbm_frac": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
               "roofline": {"bound": "mfma", "dtype": "bf16", "achieved": round(tf, 1), "peak": BF16_MFMA_PEAK_TFLOPS,
                            "unit": "TFLOP/s", "frac": round(tf / BF16_MFMA_PEAK_TFLOPS, 4), "flops": flops,
                            "fp32_matrix_equivalent_frac": round(tf / FP32_MFMA_PEAK_TFLOPS, 4)},
               "traffic_per_kernel": bwd_traffic,
               "note": "launch-inclusive time of the three backward launches (chunk states, reverse chunks, "
                       "fixed-order reductions); flops are those of the chunked form, each counted once, although "
                       "a product with a split fp32 operand runs as two (or three) bf16 matrix-core products"}
        if bwd_traffic:
            moved = sum(bwd_traffic.values())
            out["measured_traffic"] = {"bytes": moved, "gbs": round(moved / (ms * 1e-3) / 1e9, 1),
                                       "hbm_frac": round(moved / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                                       "note": "HBM bytes the three launches move, workspace included"}
        return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--decode-steps", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the oracle timing and parity (profiler runs)")
    ap.add_argument("--no-decode", action="store_true", help="skip the decode measurement")
    ap.add_argument("--no-norm", action="store_true", help="skip the gated RMSNorm measurement")
    ap.add_argument("--no-mimo", action="store_true", help="skip the MIMO decode measurement")
    ap.add_argument("--no-bwd", action="store_true", help="skip the scan backward measurement")
    ap.add_argument("--no-mixer", action="store_true", help="skip the whole-mixer measurement")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the other synthetic configs (profiler runs: same kernel names)")
    ap.add_argument("--only", choices=["nemotron_h_8b", "decode", "tiny_fp32", "nemotron3_nano", "packed_3b"],
                    help="run one part only (profiler runs: one workload per kernel name)")
    ap.add_argument("--cpu-rows", type=int, default=4, help="batch rows in the all-thread oracle sample "
                    "of the headline workload (4 = the whole step)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (for HBM counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: one GPU only (there is no multi-GPU path); use --gpus 1",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from state_space_sequence_ssd_amd import inputs, ssd

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    ssd.load_library()
    stream = torch.cuda.current_stream()
    want = (lambda part: args.only is None or args.only == part)
    cpu_on = not args.no_cpu_baseline

    if args.copy_calibration:
        # a plain 1 GiB device copy, three times: the HBM counters' scale
        src = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        torch.cuda.empty_cache()

    # Every input is drawn and made resident first; then the timed parts run
    # back to back (decode, the other configs, the headline step), so the GPU
    # never idles between them; the oracle runs after all of them.
    drun = DecodeRun() if want("decode") and not args.no_decode else None
    config_runs = []
    if not args.no_configs or args.only in ("tiny_fp32", "nemotron3_nano", "packed_3b"):
        for key, cw, seed in [("tiny_fp32", inputs.tiny_fp32(), 0), ("nemotron3_nano", inputs.nemotron3_nano(), 2),
                              ("packed_3b", inputs.packed_3b(), 3)]:
            if want(key):
                config_runs.append(ScanRun(cw, seed))
    run = ScanRun(inputs.nemotron_h_8b(), seed=1) if want("nemotron_h_8b") else None

    nrun = NormRun(run.w, run.y) if run is not None and not args.no_norm else None
    mimo_run = MimoRun() if want("decode") and not args.no_decode and not args.no_mimo else None
    brun = BwdRun(run.w) if run is not None and not args.no_bwd else None
    mrun = MixerRun(run.w) if run is not None and not args.no_mixer else None
    progress("inputs resident")

    # ---------------- decode: batch 256 through 29 layers ----------------
    decode = drun.timed(args, stream) if drun is not None else None
    if decode is not None:
        progress(f"decode timed: {decode['value']} GB/s")
    if mimo_run is not None and decode is not None:
        decode["mimo"] = mimo_run.timed(args.decode_steps, stream)
        progress("mimo decode timed")

    # ---------------- the other synthetic configs (parity workloads) ----------------
    configs = None if not config_runs else {}
    for crun in config_runs:
        configs[crun.w.name] = config_result(crun, args.steps, args.warmup)
        progress(f"{crun.w.name} timed: scan {configs[crun.w.name]['scan_avg_ms']} ms")

    def oracle_configs():
        for crun in config_runs:
            if cpu_on:
                a, o = CONFIG_SAMPLES[crun.w.name]
                configs[crun.w.name]["cpu_baseline"], configs[crun.w.name]["cpu_baseline_single_core"] = \
                    oracle_beside(crun, a, o)
        if drun is not None and cpu_on:
            decode["parity"] = drun.parity()
            decode["cpu_baseline"], decode["cpu_baseline_single_core"] = oracle_decode_beside(drun.dw, 128, 16)

    if run is None:
        oracle_configs()
        print(json.dumps({"only": args.only, "decode": decode, "configs": configs}))
        return

    # ---------------- headline: prefill step at the Nemotron-H 8B layer shape ----------------
    w = run.w
    H, G, P, N = w.nheads, w.ngroups, w.headdim, w.dstate
    total_ms, step_list, wall = run.timed(args.steps, args.warmup)
    progress(f"headline timed: {total_ms / args.steps:.4f} ms per step")
    graph_step_ms = run.graph_ms(args.steps)
    parts = run.timed_parts(args.steps, args.warmup)
    norm = nrun.timed(args.steps, args.warmup, stream) if nrun is not None else None
    bwd = brun.timed(args.steps, min(args.warmup, 3), stream) if brun is not None else None
    if bwd is not None:
        progress(f"backward timed: {bwd['avg_ms']} ms")
    mixer = mrun.timed(args.steps, min(args.warmup, 5), stream) if mrun is not None else None
    if mixer is not None:
        progress(f"mixer timed: {mixer['ms_per_layer']} ms per layer")
    ms_per_step = total_ms / args.steps
    tokens = w.batch * w.seqlen
    value = tokens / (ms_per_step / 1e3)

    step_avg = float(np.mean(step_list))
    bc_avg = float(np.mean(parts["conv_bc"]))
    scan_avg = step_avg - bc_avg
    scan_bytes = fused_scan_algorithmic_bytes(w)
    bc_bytes = conv_algorithmic_bytes(w, 2 * G * N)
    u_conv, u_scan = float(np.mean(parts["conv"])), float(np.mean(parts["scan"]))

    def kern(avg, nbytes, **extra):
        d = {"avg_ms": avg, "algorithmic_bytes": nbytes, "gbs": nbytes / (avg * 1e-3) / 1e9,
             "hbm_frac": nbytes / (avg * 1e-3) / 1e9 / HBM_PEAK_GBS}
        d.update(extra)
        return d

    kernels = {
        "chunk_scan_bf16 (x conv fused)": kern(
            scan_avg, scan_bytes, useful_tflops=scan_flops(w) / (scan_avg * 1e-3) / 1e12,
            tokens_per_s=tokens / (scan_avg * 1e-3),
            timing="fused step minus the B|C conv launched alone (HIP events)",
            traffic=read_traffic("chunk_scan_fused_nemotron_h_8b", SCAN_SOURCES)),
        "conv1d_silu (B|C channels)": kern(bc_avg, bc_bytes,
                                           traffic=read_traffic("conv1d_silu_bc_nemotron_h_8b", CONV_SOURCES)),
    }
    dom_name = max(kernels, key=lambda k: kernels[k]["avg_ms"])
    dom = kernels[dom_name]
    roofline = {"kernel": dom_name, "bound": "hbm", "achieved": round(dom["gbs"], 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(dom["gbs"] / HBM_PEAK_GBS, 4),
                "traffic": dom["traffic"]}
    stb = step_algorithmic_bytes(w)
    step_summary = {"algorithmic_bytes": stb, "gbs": round(stb / (ms_per_step * 1e-3) / 1e9, 1),
                    "hbm_frac": round(stb / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    unfused = {
        "ssd_conv1d_silu": kern(u_conv, conv_algorithmic_bytes(w),
                                traffic=read_traffic("conv1d_silu_nemotron_h_8b", CONV_SOURCES)),
        "ssd_chunk_scan_fwd": kern(u_scan, scan_algorithmic_bytes(w),
                                   traffic=read_traffic("chunk_scan_nemotron_h_8b", SCAN_SOURCES)),
        "step_ms": u_conv + u_scan, "layer_tokens_per_s": tokens / ((u_conv + u_scan) * 1e-3)}

    cpu = cpu1 = None
    if cpu_on:
        cpu, cpu1 = oracle_beside(run, {"rows": args.cpu_rows}, {"rows": 1})
        if norm is not None:
            norm["parity"] = nrun.parity(512)
        if mixer is not None:
            mixer["parity"] = mrun.parity()
    oracle_configs()
    progress("oracle done")

    line = {
        "metric": "SSD scan tokens/s/layer @Nemotron-H-8B shape; decode-step HBM GB/s",
        "value": round(value, 1),
        "unit": "tokens/s/layer",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "seq_len": w.seqlen, "nheads": H,
                   "headdim": P, "dstate": N, "ngroups": G, "chunk": w.chunk,
                   "step": "conv1d(4)+SiLU and the chunked SSD scan with final states, fused "
                           "(ssd_conv_scan_fwd)",
                   "parallelism": "single GPU"},
        "wall_s_timed": round(wall, 4),
        "ms_per_step_graph": round(graph_step_ms, 5),
        "roofline": roofline,
        "step_bytes": step_summary,
        "unfused_reference": unfused,
        "cpu_baseline": cpu,
        "cpu_baseline_single_core": cpu1,
        "kernels": kernels,
        "decode": decode,
        "gated_rmsnorm": norm,
        "scan_backward": bwd,
        "mixer": mixer,
        "configs": configs,
        "host": host_info(),
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
