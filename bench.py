"""Benchmark of the quantized-KV decode hot path on one MI355X.

A step is one decode step of the KV8 absorbed-MLA workload (1 sequence,
T = 32768 cached rows, 128 heads, 512-dim fp8 latent + 64-dim bf16 rope key):
  1. fp8-encode the step's new latent row into the cache (row T-1),
  2. decode attention over all T rows: split plan + query preparation, the
     split kernel (the dominant kernel), the merge.
The steps cycle through --kv-copies independent caches (16 x 21 MB > the
256 MB last-level cache) so every step reads its KV from HBM, as consecutive
layers of a model do; one step per cache, in order, is captured as one HIP
graph and replayed, as a serving loop replays a captured forward pass, so the
step time is GPU time rather than launch overhead (leftover steps replay
single-step graphs).  Inputs are seeded synthetic data, resident in HBM before the
timed region.

The split kernel's average duration is timed with HIP events on the launch
stream around graphs of back-to-back split launches (one per cache copy), so
no host gap falls inside the bracket.

Prints one JSON line on stdout; progress goes to stderr.
"""
import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "KV rows/s + achieved HBM GB/s (% roofline), fp8/TQ4 MLA decode, T=32k"
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 matrix-core peak
PEAK_HBM_GBPS = 8000.0     # MI355X HBM3E


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def decode_flops(T, H):
    # score K = 512 + 64 and PV N = 512: 2 * H * (576 + 512) per row
    return 2.0 * H * (576 + 512) * T


def decode_bytes(T, qmode):
    # per row: codes (512 fp8 or 256 nibble bytes) + fp32 scale + 64 bf16 rope
    return T * ((512 if qmode == 1 else 256) + 4 + 128)


COPY_BYTES = 256 << 20
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_fp8_T32768_hbm_traffic.txt")
KERNEL_SOURCE = os.path.join(ROOT, "quantized_kv_cache_row_amd", "csrc", "kvq_attn.hip")


def copy_calibration():
    import torch

    src = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(10):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": COPY_BYTES, "copies": 10}), flush=True)


def measured_traffic():
    """HBM bytes per split-kernel launch from the committed counter summary:
    FETCH_SIZE and WRITE_SIZE (KiB per dispatch) of the kernel, each scaled by
    what the same counter reads for a plain copy of known size.  None when the
    kernel source has changed since the counters were taken."""
    import hashlib

    if not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    for line in open(TRAFFIC_FILE):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    sha = hashlib.sha256(open(KERNEL_SOURCE, "rb").read()).hexdigest()
    if kv.get("source_sha256") != sha:
        return None
    fetch = float(kv["fetch_kib_per_dispatch"]) * COPY_BYTES / float(kv["copy_fetch_kib_per_dispatch"])
    write = float(kv["write_kib_per_dispatch"]) * COPY_BYTES / float(kv["copy_write_kib_per_dispatch"])
    return fetch + write


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--qmode", default="fp8", choices=["fp8", "tq4"])
    ap.add_argument("--kv-copies", type=int, default=16)
    ap.add_argument("--split-rows", type=int, default=0)
    ap.add_argument("--precision", type=int, default=0, choices=[0, 1])
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="target CPU time of the oracle baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 256 MiB device-to-device copy 10 times (HBM counter calibration)")
    args = ap.parse_args()
    if args.copy_calibration:
        copy_calibration()
        return
    if args.gpus != 1:
        print(f"bench.py: measures one GPU only; --gpus {args.gpus} is not supported (decode attention would "
              f"shard the cached rows across GPUs and all-gather the partial softmax states; no multi-GPU "
              f"path is built)", file=sys.stderr)
        sys.exit(2)

    import torch

    from quantized_kv_cache_row_amd import kvq, workloads

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    log(f"device {torch.cuda.get_device_name(0)}")
    qmode = 1 if args.qmode == "fp8" else 2
    w = workloads.kv8_decode() if qmode == 1 else workloads.tq4_decode()
    T, H = w.total_rows, w.n_heads
    log(f"workload {w.name}: T={T} H={H} copies={args.kv_copies}")

    # ---- device-resident inputs
    x = torch.from_numpy(w.latent).to(dev)
    new_rows = torch.from_numpy(workloads.fp8_rows_for_encode(args.kv_copies, seed=77)).to(dev)
    kr0 = torch.from_numpy(w.k_rope.view(np.int16)).to(dev)
    offs = torch.from_numpy(w.offsets).to(dev)
    ql = torch.from_numpy(w.q_lat).to(dev)
    qr = torch.from_numpy(w.q_rope).to(dev)
    mask = torch.from_numpy(w.sign_mask).to(dev)
    cb = 512 if qmode == 1 else 256
    codes0 = torch.empty((T, cb), dtype=torch.uint8, device=dev)
    scales0 = torch.empty(T, dtype=torch.float32, device=dev)
    if qmode == 1:
        kvq.kvq_encode_fp8(x, codes0, scales0)
    else:
        kvq.kvq_encode_tq4(x, mask, codes0, scales0)
    copies = []
    for _ in range(args.kv_copies):
        copies.append((codes0.clone(), scales0.clone(), kr0.clone()))
    out = torch.empty((1, H, 512), dtype=torch.float32, device=dev)
    lse = torch.empty((1, H), dtype=torch.float32, device=dev)
    argsets = [kvq.attn_args(qmode, args.precision, offs, T, c, s, k, ql, qr, w.sm_scale, out, lse,
                             sign_mask=mask if qmode == 2 else None, split_rows=args.split_rows)
               for (c, s, k) in copies]
    ws = kvq.alloc_workspace(argsets[0])
    torch.cuda.synchronize()

    def step(c, stage=None):
        codes_c, scales_c, _ = copies[c]
        a = argsets[c]
        if stage is None:
            row = new_rows[c:c + 1]
            if qmode == 1:
                kvq.kvq_encode_fp8(row, codes_c[T - 1:T], scales_c[T - 1:T])
            else:
                kvq.kvq_encode_tq4(row, mask, codes_c[T - 1:T], scales_c[T - 1:T])
            for st in (kvq.KVQ_STAGE_PREP, kvq.KVQ_STAGE_SPLITS, kvq.KVQ_STAGE_MERGE):
                kvq.kvq_decode_attn_stage(a, st, ws)
        else:
            kvq.kvq_decode_attn_stage(a, stage, ws)

    n_copies = len(copies)
    # eager reference of one step per copy, then capture
    for c in range(n_copies):
        step(c)
    torch.cuda.synchronize()
    eager_out = [None] * n_copies
    for c in range(n_copies):
        step(c)
        torch.cuda.synchronize()
        eager_out[c] = out.clone()
    side = torch.cuda.Stream()
    step_graphs = []
    for c in range(n_copies):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            step(c)
        step_graphs.append(g)
    round_graph = torch.cuda.CUDAGraph()  # one step per copy, in order: consecutive layers of a model
    with torch.cuda.graph(round_graph, stream=side):
        for c in range(n_copies):
            step(c)
    split_graph = torch.cuda.CUDAGraph()  # one split launch per copy, back to back
    with torch.cuda.graph(split_graph, stream=side):
        for c in range(n_copies):
            step(c, kvq.KVQ_STAGE_SPLITS)
    torch.cuda.synchronize()
    for rep in range(2):  # replays reproduce the eager results exactly
        for c in (0, n_copies - 1):
            out.zero_()
            step_graphs[c].replay()
            torch.cuda.synchronize()
            assert torch.equal(out, eager_out[c]), f"graph replay {rep} of copy {c} differs from the eager step"
        out.zero_()
        round_graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager_out[n_copies - 1]), f"round replay {rep} differs from the eager steps"

    def run_steps(k):
        for _ in range(k // n_copies):
            round_graph.replay()
        for c in range(k % n_copies):
            step_graphs[c].replay()

    log(f"warmup {args.warmup}")
    run_steps(args.warmup)
    torch.cuda.synchronize()
    log(f"timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    run_steps(args.steps)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1000.0 / args.steps

    # split kernel: HIP events around back-to-back launches on the replay stream
    reps = max(1, args.steps // n_copies)
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    split_graph.replay()
    e0.record(stream)
    for _ in range(reps):
        split_graph.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    kern_ms = e0.elapsed_time(e1) / (reps * n_copies)
    rows_per_s = T / (ms_per_step / 1000.0)
    flops = decode_flops(T, H)
    nbytes = decode_bytes(T, qmode)
    tflops = flops / (kern_ms / 1000.0) / 1e12
    gbps = nbytes / (kern_ms / 1000.0) / 1e9
    log(f"step {ms_per_step * 1000:.1f} us, split kernel {kern_ms * 1000:.1f} us ({reps * n_copies} launches), "
        f"{tflops:.1f} TFLOP/s, {gbps:.0f} GB/s")

    # ---- CPU baseline: the oracle on the same decode step
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        threads = oracle.set_threads(0)
        log(f"cpu baseline: oracle, {threads} threads, ~{args.cpu_seconds:.0f} s")
        c_host = codes0.cpu().numpy()
        s_host = scales0.cpu().numpy()
        newrow = new_rows[:1].cpu().numpy()
        reps = 0
        t_start = time.perf_counter()
        while True:
            if qmode == 1:
                oracle.encode_fp8(newrow)
            else:
                oracle.encode_tq4(newrow, w.sign_mask)
            oracle.decode_attn(qmode, w.offsets, c_host, s_host, w.k_rope, w.q_lat, w.q_rope, w.sm_scale,
                               sign_mask=w.sign_mask)
            reps += 1
            el = time.perf_counter() - t_start
            if el >= args.cpu_seconds or reps >= 1000:
                break
        cpu = {"value": T * reps / el, "unit": "rows/s", "cores": threads, "kind": "oracle",
               "sample": f"{reps} full decode steps of the same workload (1-row encode + {H}-head fp64 "
                         f"attention over T={T}) in {el:.1f} s"}
        log(f"cpu baseline {cpu['value']:.3g} rows/s")

    line = {
        "metric": METRIC,
        "value": rows_per_s,
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16",
        "data": "synthetic (seeded; N(0,1) latents x lognormal row gain, outlier channels, zero rows)",
        "config": {"workload": w.name, "seqs": 1, "T": T, "heads": H, "qmode": "fp8" if qmode == 1 else "tq4",
                   "precision": "mfma-fp16" if args.precision == 0 else "fp32", "kv_copies": args.kv_copies,
                   "parallelism": "single-gpu"},
        "roofline": {"bound": "mfma", "achieved": tflops, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": tflops / PEAK_BF16_TFLOPS,
                     "traffic": measured_traffic() if (qmode == 1 and args.precision == 0) else None},
        "hbm": {"achieved": gbps, "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": gbps / PEAK_HBM_GBPS,
                "bytes_per_launch": nbytes},
        "kernel_us": kern_ms * 1000.0,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
