"""Benchmark of the chunkwise KDA prefill (and the decode step) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one kda_chunk_fwd over the whole workload (default: one sequence of
8192 tokens, H = 96, d_k = d_v = 128, C = 64, bf16 q/k/v, fp32 g/beta), with
every input already resident in HBM.  The decode step (256 requests, H = 96,
fp32 states updated in place) is timed after it and reported under "decode".
Rank 0 prints one JSON line.

Roofline figures (per launch):
  prefill bytes  B_alg = N_tok H [e_in (2 d_k + d_v) + 4 d_k + 4 + e_out d_v]
                         + N_seq H d_k d_v 4 (has_initial + has_final)
  prefill flops  F     = N_tok H [C (3 d_k + 2 d_v) + 6 d_k d_v]
                 (K K^T, Q K^T, T R, P U at C^2 d / 2 each, triangle-aware, and
                  K e^G S, Q e^G S, Kbar^T U at 2 C d_k d_v / C each per token)
  decode bytes   N H [8 d_k d_v + e_in (2 d_k + d_v) + 4 d_k + 4 + e_out d_v]
The prefill at these shapes is bound by HBM (90 flop per byte, below the
bf16 ridge of 2.5e15 / 8e12 = 312), so the roofline object uses HBM bandwidth;
the matrix-core fraction is reported beside it.
"""
from __future__ import annotations

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
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 matrix cores
METRIC = "KDA prefill tokens/s (H=96, d_k=d_v=128) + % bf16 MFMA peak; decode HBM GB/s"
EXEC_CHUNK = 64                # tokens per state step of the kernel, for either chunk_size


def prefill_bytes(n_tok, n_seq, H, dk, dv, e_in, e_out, has_s0, has_sf):
    return (n_tok * H * (e_in * (2 * dk + dv) + 4 * dk + 4 + e_out * dv)
            + n_seq * H * dk * dv * 4 * (int(has_s0) + int(has_sf)))


def prefill_flops(n_tok, H, dk, dv, C):
    return n_tok * H * (C * (3 * dk + 2 * dv) + 6 * dk * dv)


def decode_bytes(N, H, dk, dv, e_in, e_out):
    return N * H * (8 * dk * dv + e_in * (2 * dk + dv) + 4 * dk + 4 + e_out * dv)


def fused_prefill_bytes(n_tok, n_seq, H, dk, dv, e, has_s0, has_sf):
    """kda_chunk_fwd_fused: raw q, k and decay logits z in the input type
    instead of normalised q, k and fp32 g (plus the per-head gate parameters)."""
    return (n_tok * H * (e * (3 * dk + dv) + 4 + e * dv) + H * (4 + 4 * dk)
            + n_seq * H * dk * dv * 4 * (int(has_s0) + int(has_sf)))


def _gbs(nbytes, ms):
    return nbytes / (ms * 1e-3) / 1e9


def bench_configs(args, torch, kda, inputs, dev):
    """The other workloads of the benchmark table, each timed on its own: the
    tiny fp32 case, the 131072-token sequence (chunk_size 128) and the 16
    packed sequences with prefix states."""
    res = {}
    for name, steps in (("tiny_fp32", args.steps), ("k3_prefill_128k", 5), ("k3_varlen_prefix", 5)):
        wc = inputs.WORKLOADS[name]
        xc = inputs.prefill_inputs(wc, seed=2, device=dev)
        nt, ns = int(xc["q"].shape[0]), len(xc["seqlens"])
        oc = torch.empty_like(xc["v"])
        sfc = torch.empty((ns, wc.H, wc.dk, wc.dv), dtype=torch.float32, device=dev)

        def cstep():
            kda.chunk_fwd(xc["q"], xc["k"], xc["v"], xc["g"], xc["beta"], xc["initial_state"],
                          xc["cu_seqlens"], chunk_size=wc.chunk, out=oc, final_state=sfc)

        ms, _ = time_launches(cstep, steps, 2, torch)
        e = xc["q"].element_size()
        b = prefill_bytes(nt, ns, wc.H, wc.dk, wc.dv, e, e, xc["initial_state"] is not None, True)
        f = prefill_flops(nt, wc.H, wc.dk, wc.dv, EXEC_CHUNK)
        res[name] = {"tokens": nt, "sequences": ns, "H": wc.H, "d": wc.dk, "chunk": wc.chunk,
                     "ms_per_step": ms, "tokens/s": nt / (ms * 1e-3),
                     "roofline": {"bound": "hbm", "achieved": _gbs(b, ms), "peak": HBM_PEAK_GBS,
                                  "unit": "GB/s", "frac": _gbs(b, ms) / HBM_PEAK_GBS,
                                  "traffic": None, "kernel": "kda::prefill_kernel",
                                  "bytes_per_launch": b},
                     "mfma_frac": f / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS}
        del xc, oc, sfc
        torch.cuda.empty_cache()
    return res


def bench_layer(args, w, x, torch, kda, inputs, dev):
    """The layer steps around the recurrence, each on the prefill workload's
    shapes, plus the nano-K3 prefill and decode: one JSON object."""
    res = {}
    li = inputs.layer_inputs(w, seed=3, device=dev)
    n_tok, n_seq = int(x["q"].shape[0]), len(x["seqlens"])
    e = x["q"].element_size()
    # fused front end (L2Norm of q, k and the bounded gate in the prefill kernel)
    o = x["v"].clone()                      # stands in for a raw output below

    def fstep():
        kda.chunk_fwd_fused(li["q_raw"], li["k_raw"], x["v"], li["z"], li["A_log"], li["b_alpha"],
                            x["beta"], x["initial_state"], x["cu_seqlens"], chunk_size=w.chunk)

    ms, _ = time_launches(fstep, args.steps, args.warmup, torch)
    fb = fused_prefill_bytes(n_tok, n_seq, w.H, w.dk, w.dv, e, x["initial_state"] is not None, True)
    res["prefill_fused_prologue"] = {
        "workload": w.name, "ms_per_step": ms, "tokens/s": n_tok / (ms * 1e-3),
        "roofline": {"bound": "hbm", "achieved": _gbs(fb, ms), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": _gbs(fb, ms) / HBM_PEAK_GBS,
                     "traffic": _traffic("kda_prefill.hip", "k3_prefill_8k_fused_prologue"),
                     "kernel": "kda::prefill_kernel<..., fused prologue>", "bytes_per_launch": fb}}
    # the prefill with its attention output in fp32 (kda_chunk_fwd_ex)
    o32 = torch.empty(x["v"].shape, dtype=torch.float32, device=dev)
    sf32 = torch.empty((n_seq, w.H, w.dk, w.dv), dtype=torch.float32, device=dev)

    def f32step():
        kda.chunk_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["initial_state"],
                      x["cu_seqlens"], chunk_size=w.chunk, out=o32, final_state=sf32,
                      o_dtype=torch.float32)

    ms, _ = time_launches(f32step, args.steps, args.warmup, torch)
    pb = prefill_bytes(n_tok, n_seq, w.H, w.dk, w.dv, e, 4, x["initial_state"] is not None, True)
    res["prefill_fp32_output"] = {
        "workload": w.name, "ms_per_step": ms, "tokens/s": n_tok / (ms * 1e-3),
        "roofline": {"bound": "hbm", "achieved": _gbs(pb, ms), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": _gbs(pb, ms) / HBM_PEAK_GBS, "traffic": None,
                     "kernel": "kda::prefill_kernel<..., fp32 o>", "bytes_per_launch": pb}}
    del o32, sf32
    # output epilogue on the prefill's output rows
    rows = n_tok * w.H
    og = torch.empty_like(o)
    ms, _ = time_launches(lambda: kda.output_gate(o, li["gate"], li["rms_weight"], out=og),
                          args.steps, args.warmup, torch)
    ob = rows * w.dv * 3 * e + 4 * w.dv
    res["output_gate"] = {"rows": rows, "d_v": w.dv, "ms_per_step": ms, "GB/s": _gbs(ob, ms),
                          "roofline": {"bound": "hbm", "achieved": _gbs(ob, ms),
                                       "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                       "frac": _gbs(ob, ms) / HBM_PEAK_GBS,
                                       "traffic": _traffic("kda_layer.hip", "output_gate_k3_8k"),
                                       "kernel": "kda::output_gate_kernel",
                                       "bytes_per_launch": ob}}
    # ShortConv over one projection (H * d_k channels), with streaming state
    xc = li["k_raw"].view(n_tok, w.H * w.dk)
    st = torch.zeros(n_seq, 3, w.H * w.dk, device=dev)
    ms, _ = time_launches(lambda: kda.short_conv(xc, li["conv_w"], x["cu_seqlens"], st),
                          args.steps, args.warmup, torch)
    cb = n_tok * w.H * w.dk * 2 * e + w.H * w.dk * 16 + n_seq * 3 * w.H * w.dk * 8
    res["short_conv"] = {"tokens": n_tok, "channels": w.H * w.dk, "ms_per_step": ms,
                         "GB/s": _gbs(cb, ms),
                         "roofline": {"bound": "hbm", "achieved": _gbs(cb, ms),
                                      "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                      "frac": _gbs(cb, ms) / HBM_PEAK_GBS,
                                      "traffic": _traffic("kda_layer.hip", "short_conv_k3_8k"),
                                      "kernel": "kda::short_conv_kernel (+ state update)",
                                      "bytes_per_launch": cb}}
    del li, o, og, xc, st
    # segment summaries of the prefill sequence split in 4, and their scan
    cu = x["cu_seqlens"]
    if n_seq == 1:
        T = n_tok
        cuts = torch.tensor([0, T // 4, T // 2, 3 * T // 4, T], dtype=torch.int32, device=dev)
        M, St = kda.kcp_summaries(x["q"], x["k"], x["v"], x["g"], x["beta"], cuts)
        ms_sum, _ = time_launches(lambda: kda.kcp_summaries(x["q"], x["k"], x["v"], x["g"],
                                                            x["beta"], cuts), 3, 1, torch)
        ms_scan, _ = time_launches(lambda: kda.kcp_scan(M, St), args.steps, args.warmup, torch)
        cnt = w.H
        out = torch.empty_like(St[0])
        ms_c, _ = time_launches(lambda: kda.state_compose(M[0], St[0], St[1], out=out),
                                args.steps, args.warmup, torch)
        d = w.dk
        res["kcp"] = {"segments": 4, "summaries_ms": ms_sum, "scan_ms": ms_scan,
                      "compose": {"count": cnt, "ms": ms_c,
                                  "TFLOP/s": 2 * d ** 3 * cnt / (ms_c * 1e-3) / 1e12,
                                  "GB/s": _gbs(4 * d * d * 4 * cnt, ms_c),
                                  "roofline": {"bound": "hbm", "achieved": _gbs(4 * d * d * 4 * cnt, ms_c),
                                               "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                               "frac": _gbs(4 * d * d * 4 * cnt, ms_c) / HBM_PEAK_GBS,
                                               "traffic": None, "kernel": "kda::compose_kernel",
                                               "bytes_per_launch": 4 * d * d * 4 * cnt}}}
        del M, St, out
    # nano-K3 shapes
    wn = inputs.WORKLOADS["nano_k3_prefill"]
    xn = inputs.prefill_inputs(wn, seed=2, device=dev)
    nt, ns = int(xn["q"].shape[0]), len(xn["seqlens"])
    on = torch.empty_like(xn["v"])
    sfn = torch.empty((ns, wn.H, wn.dk, wn.dv), dtype=torch.float32, device=dev)
    ms, _ = time_launches(lambda: kda.chunk_fwd(xn["q"], xn["k"], xn["v"], xn["g"], xn["beta"],
                                                None, xn["cu_seqlens"], out=on, final_state=sfn),
                          args.steps, args.warmup, torch)
    nb = prefill_bytes(nt, ns, wn.H, wn.dk, wn.dv, e, e, False, True)
    res["nano_k3_prefill"] = {"workload": wn.name, "tokens": nt, "ms_per_step": ms,
                              "tokens/s": nt / (ms * 1e-3),
                              "roofline": {"bound": "hbm", "achieved": _gbs(nb, ms),
                                           "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                           "frac": _gbs(nb, ms) / HBM_PEAK_GBS,
                                           "traffic": _traffic("kda_prefill.hip", "nano_k3_prefill"),
                                           "kernel": "kda::prefill_kernel<bf16, 64, 64>",
                                           "bytes_per_launch": nb}}
    del xn, on, sfn
    wd = inputs.WORKLOADS["nano_k3_decode"]
    xd = inputs.decode_inputs(wd, seed=5, device=dev)
    od = torch.empty_like(xd["v"])
    ms, _ = time_launches(lambda: kda.step_decode(xd["q"], xd["k"], xd["v"], xd["g"], xd["beta"],
                                                  xd["state"], out=od), args.steps, args.warmup, torch)
    db = decode_bytes(wd.decode_requests, wd.H, wd.dk, wd.dv, e, e)
    res["nano_k3_decode"] = {"workload": wd.name, "ms_per_step": ms, "GB/s": _gbs(db, ms),
                             "roofline": {"bound": "hbm", "achieved": _gbs(db, ms),
                                          "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                          "frac": _gbs(db, ms) / HBM_PEAK_GBS,
                                          "traffic": _traffic("kda_decode.hip", "nano_k3_decode"),
                                          "kernel": "kda::decode_kernel<bf16, 64>",
                                          "bytes_per_launch": db}}
    return res


def _source_sha(name):
    p = os.path.join(ROOT, "linear_attention_recurrence_chunk_amd", "csrc", name)
    return hashlib.sha256(open(p, "rb").read()).hexdigest()[:16]


def _traffic(kernel_file, workload):
    """HBM bytes per launch measured by rocprofv3 counters, if the committed
    measurement was taken on the current kernel source; else None."""
    p = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(p):
        return None
    try:
        rec = json.load(open(p))
    except (OSError, ValueError):
        return None
    if rec.get("source_sha") != _source_sha(kernel_file):
        return None
    return rec.get("hbm_bytes_per_launch")


def time_launches(fn, steps, warmup, torch):
    """Average duration of `fn` (one launch) with HIP events on the current stream."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record()
    for _ in range(steps):
        fn()
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return start.elapsed_time(end) / steps, wall


def cpu_baseline(x, w, min_seconds=10.0, max_seconds=30.0):
    """The fp64 oracle on a bounded sample of the workload: the first H'
    heads (every token), threaded over (sequence, head) on all host cores,
    repeated until at least `min_seconds` have elapsed."""
    import oracle
    cores = oracle.default_threads()
    h = min(w.H, max(1, 4 * cores))
    heads = list(range(h))
    sub = {n: x[n][:, heads].cpu() for n in ("q", "k", "v", "g", "beta")}
    s0 = None if x["initial_state"] is None else x["initial_state"][:, heads].cpu()
    cu = x["cu_seqlens"].cpu().numpy()
    n_tok = int(cu[-1])
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.forward(sub["q"], sub["k"], sub["v"], sub["g"], sub["beta"], s0, cu,
                       nthreads=cores)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds or dt * (reps + 1) / reps > max_seconds:
            break
    # full-workload tokens per second (a token carries all H heads)
    return {"value": reps * n_tok * h / w.H / dt, "unit": "tokens/s",
            "cores": min(cores, h * (len(cu) - 1)), "kind": "oracle",
            "sample": f"{reps} pass(es) over {h} of {w.H} heads x all {n_tok} tokens of "
                      f"{w.name}, fp64, {dt:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="k3_prefill_8k")
    ap.add_argument("--decode-workload", default="k3_decode_256")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the other workloads (tiny fp32, 128K tokens, varlen with prefixes)")
    ap.add_argument("--no-layer", action="store_true",
                    help="skip the layer steps (fused front end, output gate, ShortConv, "
                         "segment composition) and the nano-K3 shapes")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain 1 GiB device copy (to scale HBM counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "the benchmark runs on one GPU (the kernels shard across GPUs by (sequence, head) with no exchange, which is not implemented here); --gpus must be 1"}))
        sys.exit(2)

    import torch
    from linear_attention_recurrence_chunk_amd import _lib as kda
    from linear_attention_recurrence_chunk_amd import inputs

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    kda.library()                                  # fails loudly if not built

    # ---- prefill
    w = inputs.WORKLOADS[args.workload]
    x = inputs.prefill_inputs(w, seed=2, device=dev)
    n_tok, n_seq = int(x["q"].shape[0]), len(x["seqlens"])
    o = torch.empty_like(x["v"])
    sf = torch.empty((n_seq, w.H, w.dk, w.dv), dtype=torch.float32, device=dev)

    def step():
        kda.chunk_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["initial_state"],
                      x["cu_seqlens"], chunk_size=w.chunk, out=o, final_state=sf)

    ms, wall = time_launches(step, args.steps, args.warmup, torch)
    e = x["q"].element_size()
    bytes_ = prefill_bytes(n_tok, n_seq, w.H, w.dk, w.dv, e, e,
                           x["initial_state"] is not None, True)
    flops = prefill_flops(n_tok, w.H, w.dk, w.dv, EXEC_CHUNK)
    gbs = bytes_ / (ms * 1e-3) / 1e9
    tflops = flops / (ms * 1e-3) / 1e12
    toks = n_tok / (ms * 1e-3)
    out = {
        "metric": METRIC,
        "value": toks,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if x["q"].dtype == torch.bfloat16 else "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "num_seqs": n_seq, "tokens": n_tok, "H": w.H,
                   "d_k": w.dk, "d_v": w.dv, "chunk": w.chunk, "state_step": EXEC_CHUNK,
                   "initial_state": x["initial_state"] is not None,
                   "parallelism": "single_gpu"},
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs / HBM_PEAK_GBS,
                     "traffic": _traffic("kda_prefill.hip", w.name),
                     "kernel": "kda::prefill_kernel", "bytes_per_launch": bytes_},
        "mfma": {"tflops": tflops, "peak": BF16_PEAK_TFLOPS, "frac": tflops / BF16_PEAK_TFLOPS,
                 "flops_per_launch": flops},
        "wall_s_timed": wall,
    }

    # ---- decode
    if not args.no_decode:
        wd = inputs.WORKLOADS[args.decode_workload]
        xd = inputs.decode_inputs(wd, seed=5, device=dev)
        od = torch.empty_like(xd["v"])

        def dstep():
            kda.step_decode(xd["q"], xd["k"], xd["v"], xd["g"], xd["beta"], xd["state"], out=od)

        dms, _ = time_launches(dstep, args.steps, args.warmup, torch)
        ed = xd["q"].element_size()
        dbytes = decode_bytes(wd.decode_requests, wd.H, wd.dk, wd.dv, ed, ed)
        dgbs = dbytes / (dms * 1e-3) / 1e9
        out["decode"] = {"workload": wd.name, "requests": wd.decode_requests, "ms_per_step": dms,
                         "GB/s": dgbs, "roofline": {"bound": "hbm", "achieved": dgbs,
                                                    "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                                    "frac": dgbs / HBM_PEAK_GBS,
                                                    "traffic": _traffic("kda_decode.hip", wd.name),
                                                    "kernel": "kda::decode_kernel",
                                                    "bytes_per_launch": dbytes}}
        del xd

    if not args.no_layer:
        out["layer"] = bench_layer(args, w, x, torch, kda, inputs, dev)
    if not args.no_configs:
        out["other_configs"] = bench_configs(args, torch, kda, inputs, dev)

    if args.calibrate_copy:
        src = torch.empty(1 << 28, dtype=torch.float32, device=dev).uniform_()
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        out["copy_calibration_bytes"] = {"read": src.numel() * 4, "write": src.numel() * 4}
        del src, dst

    # ---- oracle on the host cores (context only)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(x, w)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
