"""Benchmark of the chunkwise KDA prefill (and the decode step) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one kda_chunk_fwd over the whole workload (default: one sequence of
8192 tokens, H = 96, d_k = d_v = 128, C = 64, bf16 q/k/v, fp32 g/beta), with
every input already resident in HBM, on the default algorithm (KDA_ALGO_AUTO:
the fused kernel at C = 64).  The other measurements run before it, so that
the headline prefill is timed on a GPU whose clocks have settled: the other
workloads ("other_configs"), the decode step (256 requests, H = 96, fp32
states updated in place; "decode"), the layer steps ("layer") and the
two-pass algorithm on the same workload ("two_pass").  One JSON line.

Roofline figures (per launch):
  prefill bytes  B_alg = N_tok H [e_in (2 d_k + d_v) + 4 d_k + 4 + e_out d_v]
                         + N_seq H d_k d_v 4 (has_initial + has_final)
  prefill flops  F     = N_tok H [C (2 d_k + 2 d_v) + 6 d_k d_v]
                 (the four triangular products K K^T, Q K^T, T R and P U, each
                  C^2 d / 2 multiply-adds a chunk, i.e. C d flops per token,
                  and the three state products (K o e^G) S, (Q o e^G) S and
                  Kbar^T U, 2 d_k d_v flops per token each; C is the state step)
  decode bytes   N H [8 d_k d_v + e_in (2 d_k + d_v) + 4 d_k + 4 + e_out d_v]
The prefill at these shapes is bound by HBM (86 flop per byte, below the
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


def state_step(algo, chunk):
    """Tokens the state advances by: the fused kernel always steps 64 tokens
    (it takes chunk_size 64 only), the two-pass path steps chunk_size."""
    return 64 if algo in ("auto", "fused") and chunk == 64 else chunk


def prefill_bytes(n_tok, n_seq, H, dk, dv, e_in, e_out, has_s0, has_sf):
    return (n_tok * H * (e_in * (2 * dk + dv) + 4 * dk + 4 + e_out * dv)
            + n_seq * H * dk * dv * 4 * (int(has_s0) + int(has_sf)))


def prefill_flops(n_tok, H, dk, dv, C):
    return n_tok * H * (C * (2 * dk + 2 * dv) + 6 * dk * dv)


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
    tiny fp32 case, the 131072-token sequence at chunk_size 128 (the two-pass
    path, whose state advances 128 tokens a step) and, beside it, the same
    sequence on the fused kernel's 64-token steps, and the 16 packed sequences
    with prefix states."""
    res = {}
    for label, name, steps, algo, chunk in (
            ("tiny_fp32", "tiny_fp32", args.steps, "auto", None),
            ("k3_prefill_128k", "k3_prefill_128k", 5, "auto", None),
            ("k3_prefill_128k_fused_c64", "k3_prefill_128k", 5, "fused", 64),
            ("k3_varlen_prefix", "k3_varlen_prefix", 5, "auto", None)):
        wc = inputs.WORKLOADS[name]
        C = wc.chunk if chunk is None else chunk
        xc = inputs.prefill_inputs(wc, seed=2, device=dev)
        nt, ns = int(xc["q"].shape[0]), len(xc["seqlens"])
        oc = torch.empty_like(xc["v"])
        sfc = torch.empty((ns, wc.H, wc.dk, wc.dv), dtype=torch.float32, device=dev)
        wsb = kda.workspace_size(ns, nt, wc.H, wc.dk, C, xc["q"].dtype, algo)
        ws = torch.empty(wsb, dtype=torch.uint8, device=dev) if wsb else None

        def cstep():
            kda.chunk_fwd(xc["q"], xc["k"], xc["v"], xc["g"], xc["beta"], xc["initial_state"],
                          xc["cu_seqlens"], chunk_size=C, out=oc, final_state=sfc, algo=algo,
                          workspace=ws)

        ms, _ = time_launches(cstep, steps, 2, torch)
        e = xc["q"].element_size()
        b = prefill_bytes(nt, ns, wc.H, wc.dk, wc.dv, e, e, xc["initial_state"] is not None, True)
        two = wsb > 0
        f = prefill_flops(nt, wc.H, wc.dk, wc.dv, state_step(algo, C))
        res[label] = {"workload": name, "tokens": nt, "sequences": ns, "H": wc.H, "d": wc.dk,
                      "chunk": C, "state_step": state_step(algo, C),
                      "algo": "two_pass" if two else "fused", "workspace_bytes": wsb,
                      "ms_per_step": ms, "tokens/s": nt / (ms * 1e-3),
                      "roofline": {"bound": "hbm", "achieved": _gbs(b, ms), "peak": HBM_PEAK_GBS,
                                   "unit": "GB/s", "frac": _gbs(b, ms) / HBM_PEAK_GBS,
                                   "traffic": _traffic("kda_chunked.hip" if two else "kda_prefill.hip",
                                                       label),
                                   "kernel": ("kda::cp::intra_kernel + kda::cp::state_kernel"
                                              if two else "kda::prefill_kernel"),
                                   "bytes_per_launch": b},
                      "mfma_frac": f / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS}
        del xc, oc, sfc, ws
        torch.cuda.empty_cache()
    return res


def bench_two_pass(args, w, x, torch, kda, dev):
    """The two-pass algorithm (chunk-parallel intra pass, then the state pass)
    on the headline workload, at chunk_size 64 and 128.  The algorithmic bytes
    are those of the operation; the packet round trip through the workspace
    (written by the intra pass, read by the state pass) is reported apart."""
    res = {}
    n_tok, n_seq = int(x["q"].shape[0]), len(x["seqlens"])
    e = x["q"].element_size()
    o = torch.empty_like(x["v"])
    sf = torch.empty((n_seq, w.H, w.dk, w.dv), dtype=torch.float32, device=dev)
    b = prefill_bytes(n_tok, n_seq, w.H, w.dk, w.dv, e, e, x["initial_state"] is not None, True)
    for C in (64, 128):
        wsb = kda.workspace_size(n_seq, n_tok, w.H, w.dk, C, x["q"].dtype, "two_pass")
        ws = torch.empty(wsb, dtype=torch.uint8, device=dev)

        def tstep():
            kda.chunk_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["initial_state"],
                          x["cu_seqlens"], chunk_size=C, out=o, final_state=sf, algo="two_pass",
                          workspace=ws)

        ms, _ = time_launches(tstep, args.steps, args.warmup, torch)
        # packets actually used: one per (chunk, head); written once, read by
        # each of the state pass's value slices (shared through L2)
        nch = (n_tok + C - 1) // C
        pk = kda.workspace_size(1, C, 1, w.dk, C, x["q"].dtype, "two_pass") // 2
        res[f"chunk_{C}"] = {
            "workload": w.name, "chunk": C, "state_step": C, "ms_per_step": ms,
            "tokens/s": n_tok / (ms * 1e-3), "workspace_bytes": wsb,
            "packet_bytes": pk, "packet_round_trip_bytes": 2 * nch * w.H * pk,
            "roofline": {"bound": "hbm", "achieved": _gbs(b, ms), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": _gbs(b, ms) / HBM_PEAK_GBS,
                         "traffic": _traffic("kda_chunked.hip", f"{w.name}_two_pass_c{C}"),
                         "kernel": "kda::cp::intra_kernel + kda::cp::state_kernel",
                         "bytes_per_launch": b},
            "mfma_frac": prefill_flops(n_tok, w.H, w.dk, w.dv, C) / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS}
        del ws
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
    # the same prefill from raw inputs by the other routes: the front end as a
    # pass of its own (L2Norm and gate), then the plain prefill ("unfused");
    # a pass for L2Norm only, then the prefill with the gate fused ("split")
    qn, kn = torch.empty_like(li["q_raw"]), torch.empty_like(li["k_raw"])
    gn = torch.empty(li["z"].shape, dtype=torch.float32, device=dev)
    of = torch.empty_like(x["v"])
    sff = torch.empty((n_seq, w.H, w.dk, w.dv), dtype=torch.float32, device=dev)

    def fe_all():
        kda.front_end(li["q_raw"], li["k_raw"], li["z"], li["A_log"], li["b_alpha"], q=qn, k=kn, g=gn)

    def fe_norm():
        kda.front_end(li["q_raw"], li["k_raw"], q=qn, k=kn)

    ms_fe, _ = time_launches(fe_all, args.steps, args.warmup, torch)
    ms_fn, _ = time_launches(fe_norm, args.steps, args.warmup, torch)

    def unfused():
        fe_all()
        kda.chunk_fwd(qn, kn, x["v"], gn, x["beta"], x["initial_state"], x["cu_seqlens"],
                      chunk_size=w.chunk, out=of, final_state=sff)

    def split():
        fe_norm()
        kda.chunk_fwd_fused(qn, kn, x["v"], li["z"], li["A_log"], li["b_alpha"], x["beta"],
                            x["initial_state"], x["cu_seqlens"], l2norm=False, out=of,
                            final_state=sff)

    ms_un, _ = time_launches(unfused, args.steps, args.warmup, torch)
    ms_sp, _ = time_launches(split, args.steps, args.warmup, torch)
    el = n_tok * w.H * w.dk
    feb, fnb = el * (3 * e + 2 * e + 4), el * 4 * e
    res["front_end"] = {
        "workload": w.name,
        "fused_ms": res["prefill_fused_prologue"]["ms_per_step"],
        "unfused_ms": ms_un, "split_ms": ms_sp,
        "pass_l2norm_gate": {"ms": ms_fe, "GB/s": _gbs(feb, ms_fe), "bytes_per_launch": feb,
                             "frac": _gbs(feb, ms_fe) / HBM_PEAK_GBS,
                             "traffic": _traffic("kda_layer.hip", "front_end_k3_8k")},
        "pass_l2norm": {"ms": ms_fn, "GB/s": _gbs(fnb, ms_fn), "bytes_per_launch": fnb,
                        "frac": _gbs(fnb, ms_fn) / HBM_PEAK_GBS,
                        "traffic": _traffic("kda_layer.hip", "front_end_l2norm_k3_8k")},
        "gate_fused_prefill_traffic": _traffic("kda_prefill.hip", "k3_prefill_8k_gate_fused"),
        "kernel": "kda::front_end_kernel"}
    del qn, kn, gn, of, sff
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
                     "frac": _gbs(pb, ms) / HBM_PEAK_GBS,
                     "traffic": _traffic("kda_prefill.hip", "k3_prefill_8k_fp32_output"),
                     "kernel": "kda::prefill_kernel<..., fp32 o>", "bytes_per_launch": pb}}
    del o32, sf32
    # output epilogue on the prefill's output rows.  Each launch takes the next
    # of three input sets and writes the next of three outputs (1.8 GB in all),
    # so that no launch reads what the previous one left in the 256 MB
    # Infinity Cache: the figure is HBM's
    rows = n_tok * w.H
    og_sets = [(o, li["gate"]), (li["q_raw"], li["k_raw"]), (li["z"], x["q"])]
    ogs = [torch.empty_like(o) for _ in range(3)]
    ms, _ = time_launches(cycled([lambda i=i: kda.output_gate(og_sets[i][0], og_sets[i][1],
                                                              li["rms_weight"], out=ogs[i])
                                  for i in range(3)]), args.steps, args.warmup, torch)
    ob = rows * w.dv * 3 * e + 4 * w.dv
    res["output_gate"] = {"rows": rows, "d_v": w.dv, "ms_per_step": ms, "GB/s": _gbs(ob, ms),
                          "roofline": {"bound": "hbm", "achieved": _gbs(ob, ms),
                                       "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                       "frac": _gbs(ob, ms) / HBM_PEAK_GBS,
                                       "traffic": _traffic("kda_layer.hip", "output_gate_k3_8k"),
                                       "kernel": "kda::output_gate_kernel",
                                       "bytes_per_launch": ob}}
    # ShortConv over one projection (H * d_k channels), with streaming state;
    # the launches cycle over three projections and outputs, as above
    C3 = w.H * w.dk
    xcs = [li["q_raw"].view(n_tok, C3), li["k_raw"].view(n_tok, C3), x["v"].view(n_tok, C3)]
    ycs = [torch.empty_like(xcs[0]) for _ in range(3)]
    st = torch.zeros(n_seq, 3, C3, device=dev)
    ms, _ = time_launches(cycled([lambda i=i: kda.short_conv(xcs[i], li["conv_w"], x["cu_seqlens"],
                                                             st, out=ycs[i])
                                  for i in range(3)]), args.steps, args.warmup, torch)
    cb = n_tok * w.H * w.dk * 2 * e + w.H * w.dk * 16 + n_seq * 3 * w.H * w.dk * 8
    res["short_conv"] = {"tokens": n_tok, "channels": w.H * w.dk, "ms_per_step": ms,
                         "GB/s": _gbs(cb, ms),
                         "roofline": {"bound": "hbm", "achieved": _gbs(cb, ms),
                                      "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                      "frac": _gbs(cb, ms) / HBM_PEAK_GBS,
                                      "traffic": _traffic("kda_layer.hip", "short_conv_k3_8k"),
                                      "kernel": "kda::short_conv_kernel (+ state update)",
                                      "bytes_per_launch": cb}}
    # the layer's q, k, v from their projections: ShortConv of each, then a
    # pass for the L2Norm of q and k ("separate"), against ShortConv with the
    # L2Norm in the same pass for q and k ("fused")
    xs = [li["q_raw"].view(n_tok, C3), li["k_raw"].view(n_tok, C3), x["v"].view(n_tok, C3)]
    ys = [torch.empty_like(xs[0]) for _ in range(3)]
    qn, kn = torch.empty_like(ys[0]), torch.empty_like(ys[1])
    sts = [torch.zeros(n_seq, 3, C3, device=dev) for _ in range(3)]

    def conv_sep():
        for i in range(3):
            kda.short_conv(xs[i], li["conv_w"], x["cu_seqlens"], sts[i], out=ys[i])
        kda.front_end(ys[0].view(li["q_raw"].shape), ys[1].view(li["q_raw"].shape),
                      q=qn.view(li["q_raw"].shape), k=kn.view(li["q_raw"].shape))

    def conv_fused():
        for i in range(3):
            kda.short_conv(xs[i], li["conv_w"], x["cu_seqlens"], sts[i], out=ys[i],
                           l2norm_d=w.dk if i < 2 else 0)

    ms_cs, _ = time_launches(conv_sep, args.steps, args.warmup, torch)
    ms_cf, _ = time_launches(conv_fused, args.steps, args.warmup, torch)
    res["short_conv_l2norm"] = {"tokens": n_tok, "streams": 3, "separate_ms": ms_cs,
                                "fused_ms": ms_cf,
                                "fused_GB/s": _gbs(3 * cb, ms_cf),
                                "traffic_per_normalising_launch": _traffic("kda_layer.hip",
                                                                           "short_conv_l2norm_k3_8k"),
                                "kernel": "kda::short_conv_kernel<..., NORMD = d_k>"}
    del xs, ys, qn, kn, sts
    del li, o, ogs, og_sets, xcs, ycs, st
    # context-parallel segments: the sequence split in P = 4 ("Glossaire",
    # entry "KCP").  Each of P devices would compute its segment's summaries,
    # take part in the scan and run its segment's prefill from the state the
    # scan hands it; on one device that critical path is timed piece by piece.
    cu = x["cu_seqlens"]
    if n_seq == 1:
        T, P = n_tok, 4
        cuts = torch.tensor([0, T // 4, T // 2, 3 * T // 4, T], dtype=torch.int32, device=dev)
        M, St = kda.kcp_summaries(x["q"], x["k"], x["v"], x["g"], x["beta"], cuts)
        ms_sum, _ = time_launches(lambda: kda.kcp_summaries(x["q"], x["k"], x["v"], x["g"],
                                                            x["beta"], cuts), 5, 2, torch)
        seg = slice(0, T // 4)
        xs = {n: x[n][seg] for n in ("q", "k", "v", "g", "beta")}
        cu1 = torch.tensor([0, T // 4], dtype=torch.int32, device=dev)
        ms_seg_sum, _ = time_launches(lambda: kda.kcp_summaries(xs["q"], xs["k"], xs["v"], xs["g"],
                                                                xs["beta"], cu1), 5, 2, torch)
        S_in, S_fin = kda.kcp_scan(M, St)
        ms_scan, _ = time_launches(lambda: kda.kcp_scan(M, St, S_in=S_in, S_final=S_fin),
                                   args.steps, args.warmup, torch)
        s_in1 = S_in[1].unsqueeze(0).contiguous()
        os_ = torch.empty_like(xs["v"])
        sfs = torch.empty_like(s_in1)
        ms_seg, _ = time_launches(lambda: kda.chunk_fwd(xs["q"], xs["k"], xs["v"], xs["g"], xs["beta"],
                                                        s_in1, cu1, chunk_size=w.chunk, out=os_,
                                                        final_state=sfs),
                                  args.steps, args.warmup, torch)
        d = w.dk
        sb = P * w.H * d * d * 4 * 3 + w.H * d * d * 4
        res["kcp"] = {"segments": P, "summaries_all_segments_ms": ms_sum,
                      "segment_summaries_ms": ms_seg_sum, "scan_ms": ms_scan,
                      "segment_prefill_ms": ms_seg,
                      "critical_path_ms": ms_seg_sum + ms_scan + ms_seg,
                      "scan": {"roofline": {"bound": "hbm", "achieved": _gbs(sb, ms_scan),
                                            "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                            "frac": _gbs(sb, ms_scan) / HBM_PEAK_GBS,
                                            "traffic": _traffic("kda_layer.hip", "kcp_scan_k3_8k"),
                                            "kernel": "kda::scan_kernel",
                                            "bytes_per_launch": sb}}}
        cnt = w.H
        out = torch.empty_like(St[0])
        ms_c, _ = time_launches(lambda: kda.state_compose(M[0], St[0], St[1], out=out),
                                args.steps, args.warmup, torch)
        res["kcp"]["compose"] = {"count": cnt, "ms": ms_c, "kernel": "kda::scan_kernel (P = 1)",
                                 "TFLOP/s": 2 * d ** 3 * cnt / (ms_c * 1e-3) / 1e12,
                                 "GB/s": _gbs(4 * d * d * 4 * cnt, ms_c)}
        del M, St, out, S_in, S_fin, xs, os_, sfs
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
    ms_g = graph_time(lambda: kda.chunk_fwd(xn["q"], xn["k"], xn["v"], xn["g"], xn["beta"], None,
                                            xn["cu_seqlens"], out=on, final_state=sfn),
                      args.steps, min(args.warmup, 5), torch)
    res["nano_k3_prefill"] = {"workload": wn.name, "tokens": nt, "ms_per_step": ms,
                              "graph_ms_per_step": ms_g,
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
    ms_g = graph_time(lambda: kda.step_decode(xd["q"], xd["k"], xd["v"], xd["g"], xd["beta"],
                                              xd["state"], out=od), args.steps, min(args.warmup, 5),
                      torch)
    res["nano_k3_decode"] = {"workload": wd.name, "ms_per_step": ms, "GB/s": _gbs(db, ms),
                             "graph_ms_per_step": ms_g, "graph_GB/s": _gbs(db, ms_g),
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


def cycled(fns):
    """A callable that runs fns[0], fns[1], ... in turn, one per call."""
    state = {"i": 0}

    def call():
        fns[state["i"] % len(fns)]()
        state["i"] += 1
    return call


def graph_time(fn, steps, warmup, torch, per_graph=10):
    """Average duration of `fn` replayed from a captured HIP graph of `per_graph`
    calls (the binding launches on the current stream, which capture records):
    the device's pace without the Python binding's per-call host work."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(per_graph):
            fn()
    ms, _ = time_launches(g.replay, steps, warmup, torch)
    del g
    return ms / per_graph


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


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
            "cores": min(cores, h * (len(cu) - 1)), "kind": "oracle", "cpu_model": cpu_model(),
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
    ap.add_argument("--algo", default="auto", choices=("auto", "fused", "two_pass"),
                    help="prefill algorithm of the headline measurement")
    ap.add_argument("--chunk", type=int, default=None, help="chunk_size (default: the workload's)")
    ap.add_argument("--no-two-pass", action="store_true",
                    help="skip the two-pass measurements on the headline workload")
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
    C = w.chunk if args.chunk is None else args.chunk
    wsb = kda.workspace_size(n_seq, n_tok, w.H, w.dk, C, x["q"].dtype, args.algo)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev) if wsb else None
    algo_run = "two_pass" if wsb else "fused"

    # The other sections run first and the headline prefill last: the GPU's
    # clocks settle over the first tens of milliseconds of load, and the
    # headline figure is meant to be the kernel's, not the ramp's.  (With the
    # other sections switched off it runs on a cold GPU; W warm-up steps then
    # may not be enough to settle it.)
    sections = {}
    if not args.no_configs:
        sections["other_configs"] = bench_configs(args, torch, kda, inputs, dev)

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
        sections["decode"] = {
            "workload": wd.name, "requests": wd.decode_requests, "ms_per_step": dms, "GB/s": dgbs,
            "roofline": {"bound": "hbm", "achieved": dgbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": dgbs / HBM_PEAK_GBS,
                         "traffic": _traffic("kda_decode.hip", wd.name),
                         "kernel": "kda::decode_kernel", "bytes_per_launch": dbytes}}
        # the step with the output epilogue (RMSNorm, sigmoid gate) in the
        # kernel, against the step followed by the separate epilogue kernel
        gen = torch.Generator(device=dev).manual_seed(9)
        gate = torch.randn(xd["v"].shape, generator=gen, device=dev).to(xd["v"].dtype)
        rw = torch.ones(wd.dv, device=dev)
        yd = torch.empty_like(od)
        gms, _ = time_launches(lambda: kda.step_decode_gated(xd["q"], xd["k"], xd["v"], xd["g"],
                                                             xd["beta"], xd["state"], gate, rw,
                                                             out=yd),
                               args.steps, args.warmup, torch)
        ums, _ = time_launches(lambda: (dstep(), kda.output_gate(od, gate, rw, out=yd)),
                               args.steps, args.warmup, torch)
        gbytes = dbytes + wd.decode_requests * wd.H * wd.dv * ed + 4 * wd.dv
        sections["decode"]["gated"] = {"ms_per_step": gms, "GB/s": gbytes / (gms * 1e-3) / 1e9,
                                       "unfused_ms_per_step": ums, "bytes_per_launch": gbytes,
                                       "kernel": "kda::decode_kernel<..., gated>"}
        del xd, gate, yd

    if not args.no_layer:
        sections["layer"] = bench_layer(args, w, x, torch, kda, inputs, dev)
    # the two-pass prefill last: it is the same kind of sustained load as the
    # headline prefill that follows it
    if not args.no_two_pass:
        sections["two_pass"] = bench_two_pass(args, w, x, torch, kda, dev)

    def step():
        kda.chunk_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["initial_state"],
                      x["cu_seqlens"], chunk_size=C, out=o, final_state=sf, algo=args.algo,
                      workspace=ws)

    ms, wall = time_launches(step, args.steps, args.warmup, torch)
    e = x["q"].element_size()
    bytes_ = prefill_bytes(n_tok, n_seq, w.H, w.dk, w.dv, e, e,
                           x["initial_state"] is not None, True)
    flops = prefill_flops(n_tok, w.H, w.dk, w.dv, state_step(algo_run, C))
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
                   "d_k": w.dk, "d_v": w.dv, "chunk": C, "state_step": state_step(algo_run, C),
                   "algo": algo_run, "initial_state": x["initial_state"] is not None,
                   "parallelism": "single_gpu"},
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs / HBM_PEAK_GBS,
                     "traffic": (_traffic("kda_chunked.hip", f"{w.name}_two_pass_c{C}") if wsb
                                 else _traffic("kda_prefill.hip", w.name)),
                     "kernel": ("kda::cp::intra_kernel + kda::cp::state_kernel" if wsb
                                else "kda::prefill_kernel"),
                     "bytes_per_launch": bytes_},
        "mfma": {"tflops": tflops, "peak": BF16_PEAK_TFLOPS, "frac": tflops / BF16_PEAK_TFLOPS,
                 "flops_per_launch": flops},
        "wall_s_timed": wall,
    }
    del ws
    out.update(sections)
    if "kcp" in out.get("layer", {}):
        out["layer"]["kcp"]["whole_prefill_ms"] = ms

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
