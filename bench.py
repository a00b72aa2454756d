"""Benchmark of the quantized-KV decode hot path on one MI355X.

A step is one decode step of the KV8 absorbed-MLA workload (1 sequence,
T = 32768 cached rows, 128 heads, 512-dim fp8 latent + 64-dim bf16 rope key),
one kvq_decode_attn_append call:
  1. fp8-encode the step's new latent row into the cache (row T-1), in the
     same launch as 2's query preparation,
  2. decode attention over all T rows: query preparation, the split kernel
     (the dominant kernel, which plans its own split), the merge.
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
PEAK_F16_TFLOPS = 2500.0  # MI355X dense fp16 (and bf16) matrix-core peak
PEAK_HBM_GBPS = 8000.0     # MI355X HBM3E


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def decode_flops(T, H):
    # score K = 512 + 64 and PV N = 512: 2 * H * (576 + 512) per row
    return 2.0 * H * (576 + 512) * T


def decode_bytes(T, qmode):
    # per row: codes (512 fp8 bytes, or 64 * bits for the rotated codec) + fp32 scale + 64 bf16 rope
    return T * ({1: 512, 2: 256, 3: 192, 4: 384}[qmode] + 4 + 128)


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


def fp8_kernel_sha256():
    """sha256 of the fp8 split kernel's source: kvq_attn.hip up to the end of that
    kernel (the kernel and every helper, constant and struct it uses are defined
    above that point), then kvq_device.h and kvq_internal.h."""
    import hashlib

    src = open(KERNEL_SOURCE, "rb").read()
    end = src.index(b"// Rotated-codec query preparation:")
    h = hashlib.sha256(src[:end])
    for name in ("kvq_device.h", "kvq_internal.h"):
        h.update(open(os.path.join(os.path.dirname(KERNEL_SOURCE), name), "rb").read())
    return h.hexdigest()


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
    if kv.get("source_sha256") != fp8_kernel_sha256():
        return None
    fetch = float(kv["fetch_kib_per_dispatch"]) * COPY_BYTES / float(kv["copy_fetch_kib_per_dispatch"])
    write = float(kv["write_kib_per_dispatch"]) * COPY_BYTES / float(kv["copy_write_kib_per_dispatch"])
    return fetch + write


def gpu_latents(torch, n_rows, seed, lengths=None, dim=512):
    """Seeded synthetic latents generated on the device, with the recipe of
    quantized_kv_cache_row_amd/workloads.py (N(0,1) x lognormal(0, 0.5) row
    gain, channels 7 and 300 x20, rows 0 and 100 of every sequence zero) --
    the same distribution, not the same stream (for sizes where host
    generation would dominate the run)."""
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    x = torch.randn((n_rows, dim), generator=g, device="cuda")
    x *= torch.exp(0.5 * torch.randn((n_rows, 1), generator=g, device="cuda"))
    x[:, 7] *= 20.0
    x[:, 300] *= 20.0
    if lengths is not None:
        starts = np.concatenate([[0], np.cumsum(lengths)[:-1]])
        zero = np.concatenate([starts + z for z in (0, 100)])
        zero = zero[zero < n_rows]
        x[torch.from_numpy(zero).cuda()] = 0.0
    return x


def time_graph(torch, fn, reps, warm_s=0.03, timed=3):
    """Average duration (ms) of fn() over reps back-to-back launches captured
    in one HIP graph, by HIP events on the replay stream: the median of
    `timed` replays after untimed ones for at least warm_s seconds (the first
    few milliseconds of a new load run measurably slower, e.g. about 25% for a
    600 MB streaming pass)."""
    fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    with torch.cuda.graph(g, stream=side):
        for _ in range(reps):
            fn()
    t0, n = time.perf_counter(), 0
    while n < 3 or time.perf_counter() - t0 < warm_s:
        g.replay()
        torch.cuda.synchronize()
        n += 1
    times = []
    for _ in range(timed):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) / reps)
    return sorted(times)[len(times) // 2]


ROWS = ("encode", "tq4", "tq3", "tq6", "ragged", "sparse", "q4", "q4attn")
MALL_BYTES = 256 << 20  # MI355X last-level (Infinity) cache


def measure_other_rows(torch, kvq, workloads, x_kv8, only=None):
    """The other hot-path rows, each on its own workload: encoders, the rotated
    codec's decode at 4, 3 and 6 bits, the ragged long-context decode, the
    sparse decode, q4_0 append and gather, the fused q4_0 decode.  Inputs resident on the device; HIP events
    around graphs of back-to-back launches.  Rates are algorithmic bytes (or
    flops) over kernel time.  only: one of ROWS (the others are skipped)."""
    res = {}
    dev = "cuda"
    PEAK_T = PEAK_F16_TFLOPS
    want = (lambda r: True) if only is None else (lambda r: r == only)

    def hbm(name, nbytes, ms, extra=None):
        gbps = nbytes / (ms / 1000.0) / 1e9
        d = {"us": ms * 1000.0, "GB/s": gbps, "frac_hbm": gbps / PEAK_HBM_GBPS, "bytes": nbytes}
        d.update(extra or {})
        res[name] = d
        log(f"{name}: {ms * 1000:.1f} us, {gbps:.0f} GB/s ({100 * gbps / PEAK_HBM_GBPS:.1f}% of HBM)")

    mask = torch.from_numpy(workloads.tq4_decode(T=256).sign_mask).to(dev)
    if want("encode"):
        # a1: fp8 encode of the 32768-row cache
        N = x_kv8.shape[0]
        c8 = torch.empty((N, 512), dtype=torch.uint8, device=dev)
        s8 = torch.empty(N, dtype=torch.float32, device=dev)
        ms = time_graph(torch, lambda: kvq.kvq_encode_fp8(x_kv8, c8, s8), 20)
        hbm("fp8_encode_32768", N * (2048 + 516), ms, {"rows/s": N / (ms / 1000.0)})
        # a2: TQ4 encode, the 8192-row pass and a 262144-row asymptote
        x8k = torch.from_numpy(workloads.tq4_encode_rows(8192)).to(dev)
        for n, xs in ((8192, x8k), (262144, gpu_latents(torch, 262144, 5))):
            ct = torch.empty((n, 256), dtype=torch.uint8, device=dev)
            rt = torch.empty(n, dtype=torch.float32, device=dev)
            ms = time_graph(torch, lambda: kvq.kvq_encode_tq4(xs, mask, ct, rt), 20)
            hbm(f"tq4_encode_{n}", n * (2048 + 260) + 64, ms, {"rows/s": n / (ms / 1000.0)})
        del x8k

    def decode(name, qmode, x, lengths, n_heads, seed, copies):
        T = x.shape[0]
        offs = torch.from_numpy(np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)).to(dev)
        g = torch.Generator(device=dev)
        g.manual_seed(seed)
        S = len(lengths)
        ql = torch.randn((S, n_heads, 512), generator=g, device=dev) / math.sqrt(576.0)
        qr = torch.randn((S, n_heads, 64), generator=g, device=dev) / math.sqrt(576.0)
        kr = torch.randn((T, 64), generator=g, device=dev).to(torch.bfloat16).view(torch.int16)
        cb = kvq.code_bytes(qmode)
        if copies > 1:  # enough copies that the cycled caches exceed the last-level cache
            copies = max(copies, -(-(MALL_BYTES + (64 << 20)) // decode_bytes(T, qmode)))
        sets = []
        for _ in range(copies):
            codes = torch.empty((T, cb), dtype=torch.uint8, device=dev)
            sc = torch.empty(T, dtype=torch.float32, device=dev)
            if qmode == 1:
                kvq.kvq_encode_fp8(x, codes, sc)
            elif qmode == 2:
                kvq.kvq_encode_tq4(x, mask, codes, sc)
            else:
                kvq.kvq_encode_tq(kvq.TQ_QMODE_BITS[qmode], x, mask, codes, sc)
            sets.append((codes, sc, kr.clone() if copies > 1 else kr))
        out = torch.empty((S, n_heads, 512), dtype=torch.float32, device=dev)
        lse = torch.empty((S, n_heads), dtype=torch.float32, device=dev)
        argsets = [kvq.attn_args(qmode, 0, offs, T, c, s_, k, ql, qr, workloads.SM_SCALE, out, lse,
                                 sign_mask=mask if qmode != 1 else None) for (c, s_, k) in sets]
        ws = kvq.alloc_workspace(argsets[0])
        it = [0]

        def full():
            a = argsets[it[0] % copies]
            it[0] += 1
            kvq.kvq_decode_attn(a, ws)

        def splits():
            a = argsets[it[0] % copies]
            it[0] += 1
            kvq.kvq_decode_attn_stage(a, kvq.KVQ_STAGE_SPLITS, ws)

        kvq.kvq_decode_attn_stage(argsets[0], kvq.KVQ_STAGE_PREP, ws)
        ms_full = time_graph(torch, full, 2 * copies)
        ms_split = time_graph(torch, splits, 2 * copies)
        flops = 2.0 * n_heads * (576 + 512) * T
        nbytes = T * (cb + 4 + 128)
        tf = flops / (ms_split / 1000.0) / 1e12
        res[name] = {"us_per_call": ms_full * 1000.0, "rows/s": T / (ms_full / 1000.0), "split_us": ms_split * 1000.0,
                     "TFLOP/s": tf, "frac_mfma": tf / PEAK_T, "GB/s": nbytes / (ms_split / 1000.0) / 1e9,
                     "rows": T, "seqs": S, "copies": copies}
        log(f"{name}: attention call {ms_full * 1000:.1f} us ({T / (ms_full / 1000.0):.3g} rows/s), split kernel "
            f"{ms_split * 1000:.1f} us, {tf:.0f} TFLOP/s ({100 * tf / PEAK_T:.1f}% of MFMA)")

    def sparse_row():
        # sparse (DSA-style) decode: a 32768-row fp8 cache, 16 queries x 2048 selected rows, 128 heads.
        # The fp8 matrix-core path reads the selected rows in place through the index list; cache
        # copies are cycled past the last-level cache.  The row gather into a compact copy (what the
        # other paths run first) is timed beside it.
        w = workloads.dsa_sparse_decode()
        xs = torch.from_numpy(w.latent).to(dev)
        cs = torch.empty((w.cache_rows, 512), dtype=torch.uint8, device=dev)
        ss = torch.empty(w.cache_rows, dtype=torch.float32, device=dev)
        kvq.kvq_encode_fp8(xs, cs, ss)
        krs = torch.from_numpy(w.k_rope.view(np.int16)).to(dev)
        idx = torch.from_numpy(w.row_index).to(dev)
        outs = torch.empty((w.n_seqs, w.n_heads, 512), dtype=torch.float32, device=dev)
        lses = torch.empty((w.n_seqs, w.n_heads), dtype=torch.float32, device=dev)
        copies = max(16, -(-(MALL_BYTES + (64 << 20)) // decode_bytes(w.cache_rows, 1)))
        sets = [(cs.clone(), ss.clone(), krs.clone()) for _ in range(copies)]
        offs, ql, qr = (torch.from_numpy(v).to(dev) for v in (w.offsets, w.q_lat, w.q_rope))
        sargs = [kvq.attn_args(1, 0, offs, w.total_rows, c, s, k, ql, qr, w.sm_scale, outs, lses) for c, s, k in sets]
        sws = kvq.alloc_workspace_sparse(sargs[0])
        it = [0]

        def call():
            kvq.kvq_decode_attn_sparse(sargs[it[0] % copies], idx, w.cache_rows, sws)
            it[0] += 1

        ms_sp = time_graph(torch, call, 2 * copies)
        gc = torch.empty((w.total_rows, 512), dtype=torch.uint8, device=dev)
        gs = torch.empty(w.total_rows, dtype=torch.float32, device=dev)
        gr = torch.empty((w.total_rows, 64), dtype=torch.int16, device=dev)

        def gather():
            c, s, k = sets[it[0] % copies]
            kvq.kvq_gather_rows(1, c, s, k, idx, gc, gs, gr)
            it[0] += 1

        ms_g = time_graph(torch, gather, 2 * copies)
        n = w.total_rows
        res["dsa_sparse_decode_T32768_q16_k2048"] = {
            "us_per_call": ms_sp * 1000.0, "rows/s": n / (ms_sp / 1000.0), "gather_us": ms_g * 1000.0,
            "gather_GB/s": n * (8 + 2 * 644) / (ms_g / 1000.0) / 1e9, "rows": n, "queries": w.n_seqs,
            "copies": copies}
        log(f"dsa_sparse_decode_T32768_q16_k2048: call {ms_sp * 1000:.1f} us ({n / (ms_sp / 1000.0):.3g} rows/s, "
            f"rows read in place); row gather alone {ms_g * 1000:.1f} us "
            f"({n * (8 + 2 * 644) / (ms_g / 1000.0) / 1e9:.0f} GB/s)")
        del xs, cs, ss, krs, idx, sws, gc, gs, gr, sets, sargs
        torch.cuda.empty_cache()


    def q4_rows(want):
        # a9 / a10: q4_0 bulk append of the 16 prefills, then the gather of everything
        q = workloads.Q4Workload()
        tok = int(q.prefill_off[-1])
        kp = torch.zeros((q.n_cells, 8, 144), dtype=torch.uint8, device=dev)
        vp = torch.zeros_like(kp)
        cache = kvq.q4_cache(kp, vp, torch.from_numpy(q.table).to(dev), 64)
        ks = torch.from_numpy(q.k_prefill).to(dev)
        vs = torch.from_numpy(q.v_prefill).to(dev)
        pos0 = torch.from_numpy(q.pos0_prefill).to(dev)
        off = torch.from_numpy(q.prefill_off).to(dev)
        ms = time_graph(torch, lambda: kvq.kvq_append_q4_0(cache, pos0, off, tok, ks, vs), 5)
        if want("q4"):
            hbm("q4_0_append_bulk", tok * 8 * 2 * (1024 + 144), ms, {"tokens": tok})
        del ks, vs
        if want("q4"):
            kd = torch.empty((tok, 8, 256), dtype=torch.int16, device=dev)
            vd = torch.empty_like(kd)
            ms = time_graph(torch, lambda: kvq.kvq_gather_q4_0(cache, off, tok, kd, vd), 5)
            hbm("q4_0_gather", tok * 8 * 2 * (144 + 512), ms, {"tokens": tok})
            del kd, vd
        if not want("q4attn"):
            return
        # fused decode attention over the same pools: 32 query heads over the 8 KV heads, one
        # query per sequence; three copies of the pools (3 x 131 MB) rotate past the 256 MB MALL
        qq = torch.from_numpy(workloads.q4_queries(1007, q.n_seqs)).to(dev)
        oq = torch.empty_like(qq)
        lq = torch.empty(qq.shape[:2], dtype=torch.float32, device=dev)
        tab = torch.from_numpy(q.table).to(dev)
        caches = [cache] + [kvq.q4_cache(kp.clone(), vp.clone(), tab, 64) for _ in range(2)]
        qa = kvq.q4_attn_args(off, tok, qq, oq, lq, workloads.Q4_SM_SCALE)
        qws = kvq.alloc_workspace_q4(cache, qa)
        it = [0]

        def q4_call():
            kvq.kvq_decode_attn_q4_0(caches[it[0] % 3], qa, qws)
            it[0] += 1

        ms = time_graph(torch, q4_call, 6)
        kv_bytes = tok * 8 * 2 * 144
        hbm("q4_0_decode_attn_g4", kv_bytes, ms, {"tokens": tok, "q_heads": 32, "kv_heads": 8,
                                                   "tokens/s": tok / (ms / 1000.0)})
        # the same pools read by 64 query heads (8 per KV head)
        q8 = torch.from_numpy(workloads.q4_queries(1007, q.n_seqs, n_q_heads=64)).to(dev)
        o8 = torch.empty_like(q8)
        qa = kvq.q4_attn_args(off, tok, q8, o8, None, workloads.Q4_SM_SCALE)
        qws = kvq.alloc_workspace_q4(cache, qa)
        ms = time_graph(torch, q4_call, 6)
        hbm("q4_0_decode_attn_g8", kv_bytes, ms, {"tokens": tok, "q_heads": 64, "kv_heads": 8,
                                                   "tokens/s": tok / (ms / 1000.0)})

    if want("tq4"):
        # a2 + a3-a8 on TQ4 rows: T = 32768, 128 heads, copies past the last-level cache
        decode("tq4_decode_T32768_H128", 2, x_kv8, [x_kv8.shape[0]], 128, 1002, 16)
    for bits, qm in ((3, kvq.KVQ_QMODE_TQ3), (6, kvq.KVQ_QMODE_TQ6)):
        if not want(f"tq{bits}"):
            continue
        # the 3- and 6-bit tiers: the 8192-row encode pass and a 262144-row asymptote, then
        # the T = 32768, 128-head decode
        for n in (8192, 262144):
            xe = (torch.from_numpy(workloads.tq4_encode_rows(n)).to(dev) if n == 8192
                  else gpu_latents(torch, n, 5))
            ct = torch.empty((n, 64 * bits), dtype=torch.uint8, device=dev)
            rt = torch.empty(n, dtype=torch.float32, device=dev)
            ms = time_graph(torch, lambda b=bits, xe=xe, ct=ct, rt=rt: kvq.kvq_encode_tq(b, xe, mask, ct, rt), 20)
            hbm(f"tq{bits}_encode_{n}", n * (2048 + 64 * bits + 4) + 64, ms, {"rows/s": n / (ms / 1000.0)})
            del xe, ct, rt
        decode(f"tq{bits}_decode_T32768_H128", qm, x_kv8, [x_kv8.shape[0]], 128, 1002, 16)
        torch.cuda.empty_cache()
    if want("ragged"):
        # ragged long-context fp8 decode: 32 sequences U[1024, 16384] + one of 131072
        L = workloads.ragged_lengths()
        xr = gpu_latents(torch, int(L.sum()), 1003, lengths=L)
        decode("ragged_kv8_decode_33seq", 1, xr, L, 128, 1003, 1)
        del xr
        torch.cuda.empty_cache()
    if want("sparse"):
        sparse_row()
    if want("q4") or want("q4attn"):
        q4_rows(want)
    return res




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
    ap.add_argument("--no-other-rows", action="store_true",
                    help="skip the encoders, TQ4 decode, ragged decode and q4_0 measurements")
    ap.add_argument("--only", choices=("fp8",) + ROWS,
                    help="measure one row only (for a profiler run): fp8 = the decode step alone, else one of the "
                         "other rows; prints no benchmark line")
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
    if args.only is not None and args.only != "fp8":
        x = torch.from_numpy(workloads.kv8_decode().latent).to("cuda")
        res = measure_other_rows(torch, kvq, workloads, x, only=args.only)
        print(json.dumps({"only": args.only, "rows": res}), flush=True)
        return
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
            # the new token's row is encoded into the cache's last row and the
            # attention runs over the whole cache, in one call (on the fp8
            # matrix-core path the encode shares the query-preparation launch)
            kvq.kvq_decode_attn_append(a, new_rows[c:c + 1], codes_c[T - 1:T], scales_c[T - 1:T], ws)
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

    if args.only == "fp8":
        print(json.dumps({"only": "fp8", "step_us": ms_per_step * 1000.0, "split_us": kern_ms * 1000.0}), flush=True)
        return
    other = None
    if not args.no_other_rows and qmode == 1 and args.precision == 0:
        other = measure_other_rows(torch, kvq, workloads, x)

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
        "roofline": {"bound": "mfma", "achieved": tflops, "peak": PEAK_F16_TFLOPS, "unit": "TFLOP/s",
                     "frac": tflops / PEAK_F16_TFLOPS,
                     "traffic": measured_traffic() if (qmode == 1 and args.precision == 0) else None},
        "hbm": {"achieved": gbps, "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": gbps / PEAK_HBM_GBPS,
                "bytes_per_launch": nbytes},
        "kernel_us": kern_ms * 1000.0,
        "cpu_baseline": cpu,
        "other_rows": other,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
