"""Benchmark of the Mamba-2 SSD layer hot path on one MI355X.

One step = one pass of the prefill hot path over one batch of the
Nemotron-H 8B layer shape (batch 4 x 4096 tokens, 128 heads x 64, d_state
128, 8 groups): the depthwise conv1d(4)+SiLU on x|B|C, then the chunked SSD
scan (chunk 128) writing y and the final states.  Inputs are synthetic and
already resident in HBM.  The headline value is layer tokens/s.

The decode step at batch 256 through 29 Mamba-2 layers (1 GiB fp32 state per
layer) is timed in the same run and reported as HBM GB/s.

Per-kernel times come from HIP events recorded on the stream the kernels
run on (torch's current stream, which the C ABI launches on).

    python bench.py [--gpus 1] [--steps 20] [--warmup 200]
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
SCAN_SOURCES = ["chunk_scan.hip", "chunk_scan_bf16.hip", "scan_items.h", "common.h", "kernels.h"]
CONV_SOURCES = ["conv1d_silu.hip", "common.h", "kernels.h"]
DECODE_SOURCES = ["decode_step.hip", "common.h", "kernels.h"]


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


def conv_algorithmic_bytes(w):
    es = 2 if w.bf16 else 4
    return (w.batch * w.seqlen * w.conv_dim * 2 * es + w.conv_dim * 4 * 4
            + (w.batch * w.seqlen * 4 if w.packed_lengths is not None else 0))


def decode_algorithmic_bytes(dw):
    H, G, P, N = dw.nheads, dw.ngroups, dw.headdim, dw.dstate
    CD = dw.conv_dim
    b = dw.batch
    return (2 * b * H * P * N * 4            # state read + write
            + b * CD * 2                     # token
            + 2 * b * (dw.conv_width - 1) * CD * 2   # conv state read + write
            + b * H * P * 2 + b * H * 2      # y, dt
            + CD * dw.conv_width * 4 + 3 * H * 4)


def time_config(w, seed, steps, warmup):
    """conv (if the workload has one) + scan of one synthetic config, event-timed
    per kernel on the launch stream; rates against the HBM roofline."""
    import numpy as np
    import torch
    from state_space_sequence_ssd_amd import inputs, ssd
    dev = torch.device("cuda:0")
    dtp = torch.bfloat16 if w.bf16 else torch.float32
    d = inputs.make_scan_inputs(w, seed=seed)
    H, G, P, N = w.nheads, w.ngroups, w.headdim, w.dstate
    Bt, L = w.batch, w.seqlen
    seq = torch.from_numpy(d["seq_idx"]).to(dev) if "seq_idx" in d else None
    nseq = w.num_seqs if seq is not None else None
    if w.conv:
        xbc = torch.from_numpy(d["xBC"]).to(dev, dtp)
        conv_w = torch.from_numpy(d["conv_w"]).to(dev)
        conv_out = torch.empty_like(xbc)
        x = conv_out[..., :H * P].view(Bt, L, H, P)
        Bm = conv_out[..., H * P:H * P + G * N].view(Bt, L, G, N)
        Cm = conv_out[..., H * P + G * N:].view(Bt, L, G, N)
    else:
        x = torch.from_numpy(d["x"]).to(dev, dtp)
        Bm = torch.from_numpy(d["B"]).to(dev, dtp)
        Cm = torch.from_numpy(d["C"]).to(dev, dtp)
    dt = torch.from_numpy(d["dt"]).to(dev, dtp)
    A, D = torch.from_numpy(d["A"]).to(dev), torch.from_numpy(d["D"]).to(dev)
    dt_bias = torch.from_numpy(d["dt_bias"]).to(dev)
    init = torch.from_numpy(d["initial_state"]).to(dev) if "initial_state" in d else None
    y = torch.empty((Bt, L, H, P), dtype=dtp, device=dev)
    fs = torch.empty((w.num_seqs, H, P, N), dtype=torch.float32, device=dev)
    wsb = ssd.ssd_chunk_scan_workspace_size(x, dt, A, Bm, Cm, seq_idx=seq, num_seqs=nseq)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        if w.conv:
            ssd.ssd_conv1d_silu(xbc, conv_w, seq_idx=seq, num_seqs=nseq, out=conv_out)
        if ev is not None:
            ev[1].record(stream)
        ssd.ssd_chunk_scan_fwd(x, dt, A, Bm, Cm, dt_bias=dt_bias, D=D, seq_idx=seq, num_seqs=nseq,
                               initial_state=init, final_state=fs, y=y, workspace=ws)
        if ev is not None:
            ev[2].record(stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for i in range(steps):
        step(evs[i])
    torch.cuda.synchronize()
    scan_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
    # launch-inclusive: host wall clock over back-to-back calls of the whole step
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    host_ms = (time.perf_counter() - t0) * 1e3 / steps
    sb = scan_algorithmic_bytes(w)
    out = {"tokens": Bt * L, "io_dtype": "bf16" if w.bf16 else "f32",
           "scan_avg_ms": round(scan_ms, 5), "scan_algorithmic_bytes": sb,
           "scan_gbs": round(sb / (scan_ms * 1e-3) / 1e9, 1),
           "scan_hbm_frac": round(sb / (scan_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
           "scan_tokens_per_s": round(Bt * L / (scan_ms * 1e-3), 1)}
    step_ms = scan_ms
    if w.conv:
        conv_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
        cb = conv_algorithmic_bytes(w)
        out.update({"conv_avg_ms": round(conv_ms, 5), "conv_algorithmic_bytes": cb,
                    "conv_gbs": round(cb / (conv_ms * 1e-3) / 1e9, 1),
                    "conv_hbm_frac": round(cb / (conv_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)})
        step_ms += conv_ms
    out["layer_tokens_per_s"] = round(Bt * L / (step_ms * 1e-3), 1)
    out["step_launch_inclusive_ms"] = round(host_ms, 5)
    return out


def cpu_baseline(w, d, rows):
    """The fp64 oracle (as it stands) on a bounded sample of the same workload:
    the first `rows` batch rows, all tokens and heads, conv then scan with final
    states.  Reported as tokens/s of that sample."""
    import oracle
    H, G, P, N = w.nheads, w.ngroups, w.headdim, w.dstate
    L = w.seqlen
    t0 = time.perf_counter()
    v = oracle.conv1d_silu(d["xBC"][:rows], d["conv_w"])
    x = v[..., :H * P].reshape(rows, L, H, P)
    B = v[..., H * P:H * P + G * N].reshape(rows, L, G, N)
    C = v[..., H * P + G * N:].reshape(rows, L, G, N)
    oracle.ssd_scan(x, d["dt"][:rows], d["dt_bias"], d["A"], B, C, d["D"], want_final_state=True)
    el = time.perf_counter() - t0
    threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0))
    return {"value": rows * L / el, "unit": "tokens/s/layer", "cores": threads, "kind": "oracle",
            "sample": f"batch rows 0..{rows - 1} of {w.batch}, all {L} tokens and {H} heads: fp64 conv "
                      f"then fp64 sequential recurrence with final states, {el:.1f} s wall",
            "seconds": el}


def cpu_baseline_single_core(w, d):
    """The same oracle on one host thread over one batch row, so that the
    per-core rate sits beside the all-core one.  The oracle's recurrences are
    an OpenMP loop; its thread count is set through the OpenMP runtime the
    oracle library is linked against, and restored afterwards."""
    import ctypes
    gomp = ctypes.CDLL("libgomp.so.1")
    n = gomp.omp_get_max_threads()
    gomp.omp_set_num_threads(1)
    try:
        r = cpu_baseline(w, d, 1)
    finally:
        gomp.omp_set_num_threads(n)
    r["cores"] = 1
    return r


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    # The scan is bound by the shader clock, which ramps up over the first
    # ~100 ms of load: 200 untimed steps (~80 ms) reach the steady state.
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--decode-steps", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the oracle timing (profiler runs)")
    ap.add_argument("--no-decode", action="store_true", help="skip the decode measurement")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the other synthetic configs (profiler runs: same kernel names)")
    ap.add_argument("--cpu-rows", type=int, default=4, help="batch rows in the oracle sample (4 = the whole step)")
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
    bf = torch.bfloat16

    # ---------------- prefill workload (Nemotron-H 8B layer shape) ----------------
    w = inputs.nemotron_h_8b()
    d = inputs.make_scan_inputs(w, seed=1)
    H, G, P, N = w.nheads, w.ngroups, w.headdim, w.dstate
    xbc = torch.from_numpy(d["xBC"]).to(dev, bf)
    conv_w = torch.from_numpy(d["conv_w"]).to(dev)
    dt = torch.from_numpy(d["dt"]).to(dev, bf)
    A = torch.from_numpy(d["A"]).to(dev)
    D = torch.from_numpy(d["D"]).to(dev)
    dt_bias = torch.from_numpy(d["dt_bias"]).to(dev)
    conv_out = torch.empty_like(xbc)
    x = conv_out[..., :H * P].view(w.batch, w.seqlen, H, P)
    Bm = conv_out[..., H * P:H * P + G * N].view(w.batch, w.seqlen, G, N)
    Cm = conv_out[..., H * P + G * N:].view(w.batch, w.seqlen, G, N)
    y = torch.empty((w.batch, w.seqlen, H, P), dtype=bf, device=dev)
    fs = torch.empty((w.batch, H, P, N), dtype=torch.float32, device=dev)
    ws_bytes = ssd.ssd_chunk_scan_workspace_size(x, dt, A, Bm, Cm)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        ssd.ssd_conv1d_silu(xbc, conv_w, out=conv_out)
        if ev is not None:
            ev[1].record(stream)
        ssd.ssd_chunk_scan_fwd(x, dt, A, Bm, Cm, dt_bias=dt_bias, D=D, final_state=fs, y=y,
                               workspace=ws)
        if ev is not None:
            ev[2].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record(stream)
    for i in range(args.steps):
        step(evs[i])
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = t_start.elapsed_time(t_end)
    conv_ms = [e[0].elapsed_time(e[1]) for e in evs]
    scan_ms = [e[1].elapsed_time(e[2]) for e in evs]
    ms_per_step = total_ms / args.steps
    tokens = w.batch * w.seqlen
    value = tokens / (ms_per_step / 1e3)

    conv_avg, scan_avg = float(np.mean(conv_ms)), float(np.mean(scan_ms))
    scan_bytes = scan_algorithmic_bytes(w)
    conv_bytes = conv_algorithmic_bytes(w)
    kernels = {
        "ssd_chunk_scan_fwd": {
            "avg_ms": scan_avg, "median_ms": float(np.median(scan_ms)),
            "algorithmic_bytes": scan_bytes, "gbs": scan_bytes / (scan_avg * 1e-3) / 1e9,
            "hbm_frac": scan_bytes / (scan_avg * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "useful_tflops": scan_flops(w) / (scan_avg * 1e-3) / 1e12,
            "tokens_per_s": tokens / (scan_avg * 1e-3),
            "traffic": read_traffic("chunk_scan_nemotron_h_8b", SCAN_SOURCES)},
        "ssd_conv1d_silu": {
            "avg_ms": conv_avg, "median_ms": float(np.median(conv_ms)),
            "algorithmic_bytes": conv_bytes, "gbs": conv_bytes / (conv_avg * 1e-3) / 1e9,
            "hbm_frac": conv_bytes / (conv_avg * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "traffic": read_traffic("conv1d_silu_nemotron_h_8b", CONV_SOURCES)},
    }
    dom_name = max(kernels, key=lambda k: kernels[k]["avg_ms"])
    dom = kernels[dom_name]
    roofline = {"kernel": dom_name, "bound": "hbm", "achieved": round(dom["gbs"], 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(dom["gbs"] / HBM_PEAK_GBS, 4),
                "traffic": dom["traffic"]}

    if args.copy_calibration:
        src = torch.empty(1 << 28, dtype=torch.float32, device=dev)   # 1 GiB
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()

    # ---------------- decode: batch 256 through 29 layers ----------------
    decode = None
    if not args.no_decode:
        dw = inputs.decode_29_layers()
        layers = []
        for l in range(dw.layers):
            dd = inputs.make_decode_small_inputs(dw, seed=4, layer=l)
            layers.append({
                "xBC": torch.from_numpy(dd["xBC"]).to(dev, bf),
                "dt": torch.from_numpy(dd["dt"]).to(dev, bf),
                "conv_state": torch.from_numpy(dd["conv_state"]).to(dev, bf),
                "conv_w": torch.from_numpy(dd["conv_w"]).to(dev),
                "A": torch.from_numpy(dd["A"]).to(dev), "D": torch.from_numpy(dd["D"]).to(dev),
                "dt_bias": torch.from_numpy(dd["dt_bias"]).to(dev),
                "state": inputs.decode_state_device(dw, 4, l, dev),
                "y": torch.empty((dw.batch, dw.nheads, dw.headdim), dtype=bf, device=dev)})

        def dstep(ev=None):
            for li, L_ in enumerate(layers):
                if ev is not None and li == 0:
                    ev[0].record(stream)
                ssd.ssd_decode_step(L_["xBC"], L_["dt"], L_["A"], L_["state"], dw.nheads, dw.ngroups,
                                    dt_bias=L_["dt_bias"], D=L_["D"], conv_state=L_["conv_state"],
                                    conv_weight=L_["conv_w"], y=L_["y"])
                if ev is not None and li == 0:
                    ev[1].record(stream)

        for _ in range(2):
            dstep()
        torch.cuda.synchronize()
        devs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.decode_steps)]
        d0 = torch.cuda.Event(enable_timing=True)
        d1 = torch.cuda.Event(enable_timing=True)
        d0.record(stream)
        for i in range(args.decode_steps):
            dstep(devs[i])
        d1.record(stream)
        torch.cuda.synchronize()
        dms = d0.elapsed_time(d1) / args.decode_steps
        one_layer_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in devs]))
        dbytes = decode_algorithmic_bytes(dw)
        gbs = dbytes * dw.layers / (dms * 1e-3) / 1e9
        decode = {"metric": "decode-step HBM GB/s", "value": round(gbs, 1), "unit": "GB/s",
                  "frac": round(gbs / HBM_PEAK_GBS, 4), "ms_per_29_layers": round(dms, 4),
                  "tokens_per_s": round(dw.batch / (dms * 1e-3), 1),
                  "layer_kernel_avg_ms": round(one_layer_ms, 4),
                  "algorithmic_bytes_per_layer": dbytes,
                  "traffic": read_traffic("decode_step_b256_h128", DECODE_SOURCES),
                  "workload": dw.name}
        del layers
        torch.cuda.empty_cache()

    # ---------------- the other synthetic configs (parity workloads) ----------------
    configs = None
    if not args.no_configs:
        configs = {}
        for cw, seed in [(inputs.tiny_fp32(), 0), (inputs.nemotron3_nano(), 2), (inputs.packed_3b(), 3)]:
            configs[cw.name] = time_config(cw, seed, steps=10, warmup=2)
            torch.cuda.empty_cache()

    cpu = cpu1 = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, d, args.cpu_rows)
        cpu1 = cpu_baseline_single_core(w, d)

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
                   "step": "conv1d(4)+SiLU then chunked SSD scan with final states",
                   "parallelism": "single GPU"},
        "wall_s_timed": round(wall, 4),
        "roofline": roofline,
        "cpu_baseline": None if cpu is None else {k: v for k, v in cpu.items() if k != "seconds"},
        "cpu_baseline_single_core": None if cpu1 is None else {k: v for k, v in cpu1.items() if k != "seconds"},
        "kernels": kernels,
        "decode": decode,
        "configs": configs,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
