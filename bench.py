#!/usr/bin/env python3
"""Benchmark of the DeepSeek-V4 CSA/HCA decode hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--rotate R] [--no-cpu-baseline]
                    [--no-secondary] [--copy-probe]

A step is one CSA decode step of the 1M-context workload (4 sequences at position
1,048,575, 262,144 compressed entries each, 128 query heads, head dim 512, 64 MXFP4
indexer heads, top-1024, 128-token window, sink), as one v4a_decode_step_csa call on one
stream (five launches):
  1. score every entry with the lightning indexer (the kernel also compresses the indexer key
     of the block each sequence's newest token completes);
  2. select the top-1024 (threshold scan, then the final selection, whose extra workgroups
     compress the new entry records and clear the histograms for the next call);
  3. attend over the selected entries plus the window with the sink, then combine the splits.
Inputs are seeded synthetic data (N(0,1) before quantisation).  Every input set is cloned
R times in HBM and step i uses set i mod R, so the 256 MB Infinity Cache cannot hold the
working set; the inputs are resident in HBM when timing starts.

One JSON line is printed: throughput (tokens/s = sequences decoded per second), the roofline
of the dominant launch (the MXFP4 scoring kernel, timed live with HIP events the library
records around each of its launches on the step's stream in a second loop of the same
steps), the step composed of the separate entry points for comparison, the oracle timed on
the host cores, a parity check of set 0 against the oracle, and secondary figures: the
1M-context HCA decode step, one 4096-token prefill chunk per layer kind, the 131K CSA decode
step, the standalone compressors and the grouped output projection.

--copy-probe first runs a plain device copy (an elementwise negation of 1 GiB) five times, so
that a hardware-counter run of this command can scale FETCH_SIZE / WRITE_SIZE by what the
counters read for a known byte count.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

METRIC = "CSA/HCA decode tokens/s at 1M ctx; achieved HBM GB/s and indexer MFMA util"
HBM_PEAK_GBS = 8000.0
COPY_PROBE_BYTES = 1 << 30
# Counter summary of the indexer + top-k call (FETCH_SIZE / WRITE_SIZE per call, already
# scaled by the copy probe) and the hash of the kernel sources it was taken with.
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "indexer_mxfp4_kernel_traffic_csa_decode_pro_1m.txt")
TRAFFIC_SOURCES = ["indexer.hip", "common.hpp", "compress.hpp", "encoders.hpp"]
MXFP4_PEAK_TFLOPS = 10100.0
BF16_PEAK_TFLOPS = 2500.0


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--rotate", type=int, default=16, help="input copies cycled through (MALL defeat)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-secondary", action="store_true")
    p.add_argument("--copy-probe", action="store_true", help="run the 1 GiB copy used to scale counters")
    return p.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported (the hot path "
              "is measured on one MI355X; see the design notes for how it would shard).", file=sys.stderr)
        sys.exit(2)

    import torch
    import compressed_sparse_attention_02_amd as v4
    from workloads import CSA_FLASH, CSA_PRO_1M, HCA_1M, decode_inputs, normal, to_bf16_bits

    torch.cuda.set_device(0)
    dev = "cuda"
    wl = CSA_PRO_1M
    B, H, D, R, W, k, HI, dI, m = wl.B, wl.H, wl.D, wl.R, wl.W, wl.k, wl.H_I, wl.d_I, wl.m
    T = wl.T
    N = wl.n_csa
    scale = 1.0 / math.sqrt(D)
    q_pos = [T - 1] * B
    print(f"[bench] drawing inputs for {wl.name}", file=sys.stderr, flush=True)
    inp = decode_inputs(wl, threads=16)
    s = wl.seed
    # raw streams of the last two blocks (B-block N-2, A-block N-1) of every sequence
    ntok = 2 * m
    tok0 = T - ntok
    raw = {
        "kv_a": normal(s, "kv_a", (B, ntok, D)), "kv_b": normal(s, "kv_b", (B, ntok, D)),
        "gate_a": normal(s, "gate_a", (B, ntok, 1)), "gate_b": normal(s, "gate_b", (B, ntok, 1)),
        "bias_a": normal(s, "bias_a", (m, 1)), "bias_b": normal(s, "bias_b", (m, 1)),
        "idx_a": normal(s, "idx_a", (B, ntok, dI)), "idx_b": normal(s, "idx_b", (B, ntok, dI)),
        "idx_gate_a": normal(s, "idx_gate_a", (B, ntok, 1)), "idx_gate_b": normal(s, "idx_gate_b", (B, ntok, 1)),
        "idx_bias_a": normal(s, "idx_bias_a", (m, 1)), "idx_bias_b": normal(s, "idx_bias_b", (m, 1)),
    }

    def f32(a):
        return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dev)

    def bf16(a):
        return torch.from_numpy(to_bf16_bits(a).view(np.int16)).view(torch.bfloat16).to(dev)

    print("[bench] quantising set 0 on the GPU", file=sys.stderr, flush=True)
    kv0 = v4.KV.empty(B, N, D, R)
    for b in range(B):  # one sequence at a time keeps the fp32 staging buffer at 537 MB
        v4.v4a_quantize_kv(f32(inp["records"][b]), kv0, b * N)
    keys0 = v4.Idx.empty(B, N, dI)
    v4.v4a_quantize_mxfp4(f32(inp["keys"].reshape(-1, dI)), keys0)
    qi0 = v4.Idx.empty(B, HI, dI)
    v4.v4a_quantize_mxfp4(f32(inp["q_idx"].reshape(-1, dI)), qi0)
    set0 = dict(kv=kv0, keys=keys0, qi=qi0, w=f32(inp["w"]), q=bf16(inp["q"]), win=bf16(inp["window"]),
                sink=f32(inp["sink"]),
                kv_a=bf16(raw["kv_a"]), kv_b=bf16(raw["kv_b"]), gate_a=f32(raw["gate_a"]), gate_b=f32(raw["gate_b"]),
                bias_a=f32(raw["bias_a"]), bias_b=f32(raw["bias_b"]),
                idx_a=bf16(raw["idx_a"]), idx_b=bf16(raw["idx_b"]), idx_gate_a=f32(raw["idx_gate_a"]),
                idx_gate_b=f32(raw["idx_gate_b"]), idx_bias_a=f32(raw["idx_bias_a"]),
                idx_bias_b=f32(raw["idx_bias_b"]))
    recs_host = inp.pop("records")   # the entry records stay on the host for the oracle check

    def clone(st):
        c = {}
        for name, v in st.items():
            if isinstance(v, v4.KV):
                c[name] = v4.KV(v.fmt, v.D, v.R, v.nope.clone(), v.rope.clone(), v.scale.clone(), v.cap)
            elif isinstance(v, v4.Idx):
                c[name] = v4.Idx(v.fmt, v.d, v.codes.clone(), v.scales.clone(), v.cap)
            else:
                c[name] = v.clone()
        return c

    sets = [set0] + [clone(set0) for _ in range(max(1, args.rotate) - 1)]
    ws = v4.workspace(max(v4.v4a_indexer_topk_workspace(B, 1, N, k), v4.v4a_decode_workspace(B, H, D, k, W)))
    sel = torch.empty((B, 1, k), dtype=torch.int32, device=dev)
    outs = [torch.empty((B, H, D), dtype=torch.bfloat16, device=dev) for _ in range(2)]
    win_len = [W] * B

    def stage_compress(st):
        v4.v4a_compress_csa(st["kv_a"], st["kv_b"], st["gate_a"], st["gate_b"], st["bias_a"], st["bias_b"],
                            tok0=tok0, m=m, first_entry=N - 1, n_entries=1, out_kv=st["kv"])
        v4.v4a_compress_csa(st["idx_a"], st["idx_b"], st["idx_gate_a"], st["idx_gate_b"], st["idx_bias_a"],
                            st["idx_bias_b"], tok0=tok0, m=m, first_entry=N - 1, n_entries=1, out_idx=st["keys"])

    def stage_indexer(st):
        v4.v4a_indexer_topk(st["keys"], [N] * B, m, st["qi"], st["w"], B, 1, HI, q_pos, k, sel, ws)

    def stage_attend(st, out):
        v4.v4a_decode_csa(st["q"], st["kv"], sel.view(B, k), k, st["win"], win_len, W, st["sink"], q_pos,
                          softmax_scale=scale, out=out, ws=ws)

    # the step as one call on every input set: the new indexer keys are compressed inside the
    # scoring kernel and the entry records in the final selection's launch; from the second
    # call on, the step's own workspace is known to hold clear histograms (ws_clean), so the
    # call is five launches: scoring, scan, final selection, attention, combine
    step_kwargs = [dict(q_pos=q_pos, n_entries=[N] * B, m=m, kv_a=st["kv_a"], kv_b=st["kv_b"], gate_a=st["gate_a"],
                        gate_b=st["gate_b"], bias_a=st["bias_a"], bias_b=st["bias_b"], idx_a=st["idx_a"],
                        idx_b=st["idx_b"], idx_gate_a=st["idx_gate_a"], idx_gate_b=st["idx_gate_b"],
                        idx_bias_a=st["idx_bias_a"], idx_bias_b=st["idx_bias_b"], kv=st["kv"], keys=st["keys"],
                        q_idx=st["qi"], w=st["w"], k=k, q=st["q"], win=st["win"], win_len=win_len, W=W,
                        sink=st["sink"], softmax_scale=scale) for st in sets]
    step_args = [[v4.DecodeStepArgs(**kw, out=outs[j]) for j in range(2)] for kw in step_kwargs]
    step_args_clean = [[v4.DecodeStepArgs(**kw, out=outs[j], ws_clean=True) for j in range(2)] for kw in step_kwargs]
    step_ws = v4.workspace(v4.v4a_decode_step_workspace(step_args[0][0]))
    step_calls = [0]

    def step(i):
        # step_ws serves only these calls: every call leaves its histograms clear
        a = (step_args_clean if step_calls[0] else step_args)[i % len(sets)][i % 2]
        v4.v4a_decode_step_csa(a, step_ws)
        step_calls[0] += 1

    def step_separate(i):
        # the same step composed of the separate entry points (the record compressor, read
        # only by attention, runs on a second stream meanwhile)
        st = sets[i % len(sets)]
        main = torch.cuda.current_stream()
        ev_start.record(main)
        side_rec.wait_event(ev_start)
        with torch.cuda.stream(side_rec):
            v4.v4a_compress_csa(st["kv_a"], st["kv_b"], st["gate_a"], st["gate_b"], st["bias_a"], st["bias_b"],
                                tok0=tok0, m=m, first_entry=N - 1, n_entries=1, out_kv=st["kv"])
        ev_rec.record(side_rec)
        v4.v4a_compress_csa(st["idx_a"], st["idx_b"], st["idx_gate_a"], st["idx_gate_b"], st["idx_bias_a"],
                            st["idx_bias_b"], tok0=tok0, m=m, first_entry=N - 1, n_entries=1, out_idx=st["keys"])
        stage_indexer(st)
        main.wait_event(ev_rec)
        stage_attend(st, outs[i % 2])

    side_rec = torch.cuda.Stream()
    ev_start, ev_rec = torch.cuda.Event(), torch.cuda.Event()

    if args.copy_probe:
        src = torch.randn((COPY_PROBE_BYTES // 4,), device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    print(f"[bench] warmup {args.warmup} steps", file=sys.stderr, flush=True)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    t_start.record()
    for i in range(args.steps):
        step(args.warmup + i)
    t_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms_step = t_start.elapsed_time(t_end) / args.steps
    tok_s = B / (ms_step / 1e3)
    # the same steps again, each between its own pair of events on the step's stream (the host
    # enqueues faster than the GPU drains, so each interval is that step's GPU time): percentiles
    step_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        step_ev[i][0].record()
        step(args.warmup + i)
        step_ev[i][1].record()
    torch.cuda.synchronize()
    step_pct = percentiles([a.elapsed_time(b) for a, b in step_ev])

    # the fused step again with the library's kernel timing: each kernel launch carries its own
    # start and stop HIP events (on the step's stream), so every kernel's live duration is known;
    # the MXFP4 scoring kernel is the roofline's kernel
    n_tr = max(20, args.steps // 2)
    v4.v4a_trace_begin(6 * n_tr + 8)
    for i in range(n_tr):
        step(args.warmup + i)
    n_timed = v4.v4a_trace_end()
    torch.cuda.synchronize()
    kernel_ms = {}
    for name, ms in v4.trace_kernels(n_timed):
        kernel_ms.setdefault(name, []).append(ms)
    kernel_ms = {name: float(np.mean(v)) for name, v in kernel_ms.items()}
    score_ms = kernel_ms["indexer_mxfp4_kernel"]

    # the step composed of six calls from Python, for comparison with the fused call
    n_sep = max(10, args.steps // 2)
    for i in range(args.warmup):
        step_separate(i)
    s_start, s_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    s_start.record()
    for i in range(n_sep):
        step_separate(args.warmup + i)
    s_end.record()
    torch.cuda.synchronize()
    ms_step_sep = s_start.elapsed_time(s_end) / n_sep

    # the indexer + top-k call alone, back to back on the rotated input sets, with HIP events
    # around every call on the stream its kernels run on; the host enqueues faster than the
    # GPU drains, so each interval is the call's own GPU time
    n_idx = max(20, args.steps)
    for i in range(args.warmup):
        stage_indexer(sets[i % len(sets)])
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_idx)]
    torch.cuda.synchronize()
    for i in range(n_idx):
        evs[i][0].record()
        stage_indexer(sets[(args.warmup + i) % len(sets)])
        evs[i][1].record()
    torch.cuda.synchronize()
    idx_ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))

    # the BF16-score selector, timed the same way, and the overlap of its selection with the
    # fp32 one on every sequence of set 0 (with the secondary figures)
    bf16_variant = None
    if not args.no_secondary:
        sel_b = torch.empty_like(sel)
        for i in range(args.warmup):
            st = sets[i % len(sets)]
            v4.v4a_indexer_topk_bf16(st["keys"], [N] * B, m, st["qi"], st["w"], B, 1, HI, q_pos, k, sel_b, ws)
        torch.cuda.synchronize()
        for i in range(n_idx):
            st = sets[(args.warmup + i) % len(sets)]
            evs[i][0].record()
            v4.v4a_indexer_topk_bf16(st["keys"], [N] * B, m, st["qi"], st["w"], B, 1, HI, q_pos, k, sel_b, ws)
            evs[i][1].record()
        torch.cuda.synchronize()
        idx_bf16_ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))
        stage_indexer(sets[0])
        v4.v4a_indexer_topk_bf16(sets[0]["keys"], [N] * B, m, sets[0]["qi"], sets[0]["w"], B, 1, HI, q_pos, k,
                                 sel_b, ws)
        torch.cuda.synchronize()
        sf, sb = sel.cpu().numpy()[:, 0], sel_b.cpu().numpy()[:, 0]
        bf16_variant = {"entry_point": "v4a_indexer_topk_bf16", "ms_per_call": idx_bf16_ms,
                        "ms_per_call_f32_scores": idx_ms,
                        "recall_vs_f32_scores": float(np.mean([np.intersect1d(sf[b], sb[b]).size / k
                                                               for b in range(B)]))}

    # algorithmic bytes of the indexer + top-k call: keys, indexer queries and weights read,
    # the top-k list written
    idx_bytes = B * N * (dI // 2 + dI // 32) + B * HI * (dI // 2 + dI // 32) + B * HI * 4 + B * k * 4
    idx_flops = 2.0 * B * N * HI * dI
    # the scoring kernel alone: 68 B per key scored (MXFP4 codes + scales), the indexer queries
    # and weights
    score_bytes = B * N * (dI // 2 + dI // 32) + B * HI * (dI // 2 + dI // 32) + B * HI * 4
    achieved = score_bytes / (score_ms / 1e3) / 1e9
    # whole-step algorithmic bytes: keys + gathered records + window + queries + output + raw blocks
    rec_bytes = (D - R) + 2 * R + 4
    step_bytes = idx_bytes + B * k * rec_bytes + B * W * D * 2 + B * H * D * 2 * 2 + \
        B * ntok * (D + dI) * 2 * 2
    step_flops = idx_flops + 4.0 * B * H * D * (k + W)

    # parity of the step on set 0 against the oracle (sequence 0, full indexer scan); the
    # fused call must give bitwise the composed calls' output
    step_separate(0)
    torch.cuda.synchronize()
    gpu_sel = sel.cpu().numpy()[:, 0]
    sep_out = outs[0].clone()
    step(0)
    torch.cuda.synchronize()
    fused_equal = bool(torch.equal(sep_out, outs[0]))
    gpu_out = outs[0].float().cpu().numpy()

    result = {
        "metric": METRIC, "value": tok_s, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "mxfp4+bf16", "data": "synthetic",
        "config": {"workload": wl.name, "batch": B, "context_tokens": T, "csa_entries": N, "heads": H,
                   "head_dim": D, "rope_dims": R, "indexer_heads": HI, "indexer_dim": dI, "topk": k,
                   "window": W, "input_copies": len(sets), "entry_point": "v4a_decode_step_csa"},
        "roofline": {"kernel": "indexer_mxfp4_kernel (the MXFP4 scoring launch of the fused step)",
                     "scope": "the dominant kernel alone; the whole step's HBM fraction is step.hbm_frac",
                     "bound": "hbm",
                     "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": measured_traffic(), "ms_per_launch": score_ms, "algorithmic_bytes": score_bytes,
                     "mfma_util": idx_flops / (score_ms / 1e3) / (MXFP4_PEAK_TFLOPS * 1e12),
                     "units_per_launch": f"{B} x {N} keys scored, 68 B each"},
        "indexer_topk_call": {"entry_point": "v4a_indexer_topk", "ms_per_call": idx_ms, "algorithmic_bytes": idx_bytes,
                              "hbm_gbs": idx_bytes / (idx_ms / 1e3) / 1e9,
                              "frac": idx_bytes / (idx_ms / 1e3) / 1e9 / HBM_PEAK_GBS},
        "step": {"algorithmic_bytes": step_bytes, "hbm_gbs": step_bytes / (ms_step / 1e3) / 1e9,
                 "hbm_frac": step_bytes / (ms_step / 1e3) / 1e9 / HBM_PEAK_GBS, "flops": step_flops,
                 "ms_per_step_pct": step_pct,
                 "ms_separate_calls": ms_step_sep,
                 "kernel_ms": kernel_ms,
                 "wall_s": wall},
    }

    if bf16_variant is not None:
        result["variants"] = {"bf16_scores": bf16_variant}
    if not args.no_secondary:
        # the same fused step with split-free attention (bitwise equal to prefill, no split-K)
        ns_args = [v4.DecodeStepArgs(**{**sa_kw, "out": outs[0]}, no_split=True) for sa_kw in step_kwargs]
        ns_ws = v4.workspace(v4.v4a_decode_step_workspace(ns_args[0]))
        for i in range(args.warmup):
            v4.v4a_decode_step_csa(ns_args[i % len(ns_args)], ns_ws)
        torch.cuda.synchronize()
        t_start.record()
        for i in range(n_sep):
            v4.v4a_decode_step_csa(ns_args[(args.warmup + i) % len(ns_args)], ns_ws)
        t_end.record()
        torch.cuda.synchronize()
        ms_ns = t_start.elapsed_time(t_end) / n_sep
        result.setdefault("variants", {})["split_free_attention"] = {
            "entry_point": "v4a_decode_step_csa (no_split)", "ms_per_step": ms_ns, "tokens_per_s": B / (ms_ns / 1e3),
            "ms_per_step_split_k": ms_step}
        result["variants"]["multi_token_q2"] = mtp_variant(v4, torch, args, sets, step_kwargs, inp, bf16, f32, B, H,
                                                           D, W, HI, dI, N)
    if not args.no_secondary:
        del sets, step_args, step_kwargs, ns_args
        torch.cuda.empty_cache()
        result["secondary"] = {"hca_decode_1m": hca_secondary(v4, torch, HCA_1M, args, f32, bf16)}
        torch.cuda.empty_cache()
        result["secondary"]["prefill_csa_4k_on_64k"] = prefill_secondary(v4, torch, "csa", args)
        torch.cuda.empty_cache()
        result["secondary"]["prefill_hca_4k_on_64k"] = prefill_secondary(v4, torch, "hca", args)
        torch.cuda.empty_cache()
        result["secondary"]["csa_decode_flash_131k"] = csa_step_secondary(v4, torch, CSA_FLASH, args, f32, bf16)
        torch.cuda.empty_cache()
        result["secondary"]["compress_1m"] = compress_secondary(v4, torch, args)
        torch.cuda.empty_cache()
        result["secondary"]["output_projection"] = projection_secondary(v4, torch, args)

    if not args.no_cpu_baseline:
        import oracle
        from workloads import bf16_bits_to_f64
        print("[bench] oracle on the host", file=sys.stderr, flush=True)
        t0 = time.perf_counter()
        chk = {"topk_equal": True, "topk_recall": 1.0, "max_abs": 0.0, "rel_l2": 0.0, "inexact_dots": 0}
        reps = 3  # passes of the whole step (about 10 s of host work); the check uses the first
        for rep, b in [(r, bb) for r in range(reps) for bb in range(B)]:   # every sequence's token
            ent = oracle.compress_csa(raw["kv_a"][b], raw["kv_b"][b], raw["gate_a"][b], raw["gate_b"][b],
                                      raw["bias_a"], raw["bias_b"], tok0=tok0, m=m, first_entry=N - 1,
                                      n_entries=1, apply_rope=True, R=R)
            key = oracle.compress_csa(raw["idx_a"][b], raw["idx_b"][b], raw["idx_gate_a"][b], raw["idx_gate_b"][b],
                                      raw["idx_bias_a"], raw["idx_bias_b"], tok0=tok0, m=m, first_entry=N - 1,
                                      n_entries=1, apply_rope=False, R=0)
            keys_b = inp["keys"][b].copy()
            keys_b[N - 1] = key[0]
            kc, ksc = oracle.quant_mxfp4(keys_b)
            qc, qs = oracle.quant_mxfp4(inp["q_idx"][b])
            scores, bad = oracle.indexer_scores_mxfp4(qc, qs, inp["w"][b], kc, ksc)
            ref_sel = oracle.topk(scores, k)
            chosen = ref_sel[ref_sel >= 0]
            rows = recs_host[b][chosen].copy()
            rows[chosen == N - 1] = ent[0]
            ents = oracle.dequant_kv(*oracle.quant_kv(rows, R))
            qd = bf16_bits_to_f64(to_bf16_bits(inp["q"][b]))
            wd = bf16_bits_to_f64(to_bf16_bits(inp["window"][b]))
            ref = oracle.attend(qd, ents, wd, inp["sink"], scale, rope_inverse=True, R=R, t_q=T - 1)
            if rep > 0:
                continue
            ref_bf16 = torch.from_numpy(ref.astype(np.float32)).to(torch.bfloat16).float().numpy()
            chk["topk_equal"] &= bool(np.array_equal(gpu_sel[b], ref_sel))
            chk["topk_recall"] = min(chk["topk_recall"], len(np.intersect1d(gpu_sel[b], ref_sel)) / k)
            chk["max_abs"] = max(chk["max_abs"], float(np.abs(gpu_out[b] - ref_bf16).max()))
            chk["rel_l2"] = max(chk["rel_l2"],
                                float(np.linalg.norm(gpu_out[b] - ref_bf16) / np.linalg.norm(ref_bf16)))
            chk["inexact_dots"] += bad
        cpu_s = time.perf_counter() - t0
        result["cpu_baseline"] = {"value": reps * B / cpu_s, "unit": "tokens/s", "cores": oracle.threads(),
                                  "kind": "oracle", "seconds": cpu_s,
                                  "sample": f"{reps} passes of the whole step ({B} sequences, one token each): "
                                            f"compress each new block, exact MXFP4 scores of all {N} entries, "
                                            f"full-sort top-{k}, double-precision attention"}
        result["check"] = {"sequences": B, "fused_equals_separate_calls": fused_equal, **chk}
    print(json.dumps(result), flush=True)


def hca_secondary(v4, torch, wl, args, f32, bf16):
    """The 1M-context HCA decode step (16 x 8192 entries, 128 heads): dense MQA + window + sink."""
    from workloads import decode_inputs
    print(f"[bench] secondary: {wl.name}", file=sys.stderr, flush=True)
    inp = decode_inputs(wl, threads=16)
    B, H, D, R, W, N = wl.B, wl.H, wl.D, wl.R, wl.W, inp["N"]
    kv0 = v4.KV.empty(B, N, D, R)
    v4.v4a_quantize_kv(f32(inp["records"].reshape(-1, D)), kv0)
    q, win, sink = bf16(inp["q"]), bf16(inp["window"]), f32(inp["sink"])
    rot = max(1, min(args.rotate, 8))
    kvs = [kv0] + [v4.KV(kv0.fmt, D, R, kv0.nope.clone(), kv0.rope.clone(), kv0.scale.clone(), N)
                   for _ in range(rot - 1)]
    ws = v4.workspace(v4.v4a_decode_workspace(B, H, D, N, W))
    out = torch.empty((B, H, D), dtype=torch.bfloat16, device="cuda")
    q_pos = [wl.T - 1] * B

    def step(i):
        v4.v4a_decode_hca(q, kvs[i % rot], [N] * B, wl.m_hca, win, [W] * B, W, sink, q_pos,
                          softmax_scale=1.0 / math.sqrt(D), out=out, ws=ws)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    steps = args.steps
    a.record()
    for i in range(steps):
        step(i)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / steps
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for i in range(steps):
        ev[i][0].record()
        step(i)
        ev[i][1].record()
    torch.cuda.synchronize()
    pct = percentiles([x.elapsed_time(y) for x, y in ev])

    # the whole per-token step in one call (v4a_decode_step_hca): the newest token completes a
    # 128-token block, which is compressed into entry N-1 first; the window is a ring
    from workloads import normal
    rows = bf16(normal(wl.seed, "kv_h", (B, wl.m_hca, D)))
    gates = f32(normal(wl.seed, "gate_h", (B, wl.m_hca, 1)))
    hbias = f32(normal(wl.seed, "bias_h", (wl.m_hca, 1)))
    step_args = [v4.DecodeStepHcaArgs(q_pos=q_pos, n_entries=[N] * B, m=wl.m_hca, kv_a=rows, gate_a=gates,
                                      bias_a=hbias, kv=kvs[r], q=q, win=win, win_len=[W] * B, W=W, sink=sink,
                                      softmax_scale=1.0 / math.sqrt(D), out=out, ring=True) for r in range(rot)]
    ws_step = v4.workspace(v4.v4a_decode_step_hca_workspace(step_args[0]))
    for i in range(args.warmup):
        v4.v4a_decode_step_hca(step_args[i % rot], ws_step)
    torch.cuda.synchronize()
    a.record()
    for i in range(steps):
        v4.v4a_decode_step_hca(step_args[i % rot], ws_step)
    b.record()
    torch.cuda.synchronize()
    ms_step = a.elapsed_time(b) / steps
    ns_args = [v4.DecodeStepHcaArgs(q_pos=q_pos, n_entries=[N] * B, m=wl.m_hca, kv_a=rows, gate_a=gates,
                                    bias_a=hbias, kv=kvs[r], q=q, win=win, win_len=[W] * B, W=W, sink=sink,
                                    softmax_scale=1.0 / math.sqrt(D), out=out, ring=True, no_split=True)
               for r in range(rot)]
    for i in range(args.warmup):
        v4.v4a_decode_step_hca(ns_args[i % rot], None)
    torch.cuda.synchronize()
    a.record()
    for i in range(steps):
        v4.v4a_decode_step_hca(ns_args[i % rot], None)
    b.record()
    torch.cuda.synchronize()
    ms_ns = a.elapsed_time(b) / steps

    nbytes = B * N * ((D - R) + 2 * R + 4) + B * W * D * 2 + B * H * D * 2 * 2
    flops = 4.0 * B * H * D * (N + W)
    return {"workload": wl.name, "tokens_per_s": B / (ms / 1e3), "ms_per_step": ms, "ms_per_step_pct": pct,
            "bound": "mfma", "mfma_tflops": flops / (ms / 1e3) / 1e12,
            "mfma_frac": flops / (ms / 1e3) / (BF16_PEAK_TFLOPS * 1e12),
            "hbm_gbs": nbytes / (ms / 1e3) / 1e9, "input_copies": rot,
            "fused_step": {"entry_point": "v4a_decode_step_hca", "ms_per_step": ms_step,
                           "tokens_per_s": B / (ms_step / 1e3),
                           "note": "block compression of every sequence's newest 128 tokens + attention, ring window",
                           "ms_per_step_split_free": ms_ns}}


def prefill_secondary(v4, torch, kind, args):
    """One 4096-token prefill chunk at positions 65536..69631 of a sequence whose 65536 earlier
    tokens are cached (16384 CSA entries + keys, or 512 HCA entries); the chunk's own blocks are
    compressed and appended by the call.  Throughput = chunk tokens / call time."""
    from workloads import PREFILL_64K, prefill_inputs, to_bf16_bits
    wl = PREFILL_64K
    print(f"[bench] secondary: prefill {kind} {wl.name}", file=sys.stderr, flush=True)
    x = prefill_inputs(wl, kind=kind, threads=16)
    C, tok0, n_prev, N0 = x["C"], x["tok0"], x["n_prev"], x["N0"]
    D, R, H, W = wl.D, wl.R, wl.H, wl.W

    def f32(a):
        return torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda()

    def bf16(a):
        return torch.from_numpy(to_bf16_bits(a).view(np.int16)).view(torch.bfloat16).cuda()

    q = bf16(x["q"])
    out = torch.empty((C, H, D), dtype=torch.bfloat16, device="cuda")
    m = x["m"]
    n_total = (tok0 + C) // m
    kv = v4.KV.empty(1, n_total, D, R)
    v4.v4a_quantize_kv(f32(x["records"]), kv, 0)
    common = dict(tok0=tok0, n_prev=n_prev, m=m, kv_a=bf16(x["kv_a"]), gate_a=f32(x["gate_a"]),
                  bias_a=f32(x["bias_a"]), kv=kv, q=q, W=W, sink=f32(x["sink"]), softmax_scale=wl.scale, out=out)
    if kind == "csa":
        keys = v4.Idx.empty(1, n_total, wl.d_I)
        v4.v4a_quantize_mxfp4(f32(x["keys"]), keys, 0)
        qi = v4.Idx.empty(1, C * wl.H_I, wl.d_I)
        v4.v4a_quantize_mxfp4(f32(x["q_idx"].reshape(-1, wl.d_I)), qi)
        csa = dict(kv_b=bf16(x["kv_b"]), gate_b=f32(x["gate_b"]), bias_b=f32(x["bias_b"]),
                   idx_a=bf16(x["idx_a"]), idx_b=bf16(x["idx_b"]), idx_gate_a=f32(x["idx_gate_a"]),
                   idx_gate_b=f32(x["idx_gate_b"]), idx_bias_a=f32(x["idx_bias_a"]),
                   idx_bias_b=f32(x["idx_bias_b"]), keys=keys, q_idx=qi, w=f32(x["w"]), k=wl.k)
        a = v4.PrefillArgs(**csa, **common)
        a_bf16 = v4.PrefillArgs(**csa, **common, score_bf16=True)
        layer = v4.V4A_LAYER_CSA
    else:
        a = v4.PrefillArgs(**common)
        layer = v4.V4A_LAYER_HCA
    ws = v4.workspace(v4.v4a_prefill_workspace(layer, a))
    del x

    def time_chunk(a, reps=5):
        for _ in range(2):
            v4.v4a_prefill_chunk(layer, a, ws)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            v4.v4a_prefill_chunk(layer, a, ws)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    ms = time_chunk(a)
    # each kernel of the chunk, timed by the library's per-launch events
    v4.v4a_trace_begin(64)
    for _ in range(3):
        v4.v4a_prefill_chunk(layer, a, ws)
    n_tr = v4.v4a_trace_end()
    torch.cuda.synchronize()
    kms = {}
    for name, kt in v4.trace_kernels(n_tr):
        kms[name] = kms.get(name, 0.0) + kt / 3
    # algorithmic flops: every query's indexer dots over its visible entries (MXFP4) and its
    # attention over its keys (BF16, 4*H*D per key: QK and PV)
    vis = [min(n_total, (tok0 + j + 1) // m) for j in range(C)]
    wins = [min(W, tok0 + j + 1) for j in range(C)]
    attn_keys = sum((wl.k if kind == "csa" else v) + w_ for v, w_ in zip(vis, wins))
    bf16_flops = 4.0 * H * D * attn_keys
    mx_flops = 2.0 * wl.H_I * wl.d_I * sum(vis) if kind == "csa" else 0.0
    t = ms / 1e3
    res = {"tokens_per_s": C / t, "ms_per_chunk": ms, "bound": "mfma", "kernel_ms": kms,
           "bf16_tflops": bf16_flops / t / 1e12, "bf16_mfma_frac": bf16_flops / t / (BF16_PEAK_TFLOPS * 1e12),
           "attention_kernel_bf16_mfma_frac": bf16_flops / (kms["attn_mfma_kernel"] / 1e3) / (BF16_PEAK_TFLOPS * 1e12)}
    if kind == "csa":
        res.update(scoring_kernel_mxfp4_mfma_frac=mx_flops / (kms["indexer_mxfp4_kernel"] / 1e3) /
                   (MXFP4_PEAK_TFLOPS * 1e12),
                   mxfp4_tflops=mx_flops / t / 1e12, mxfp4_mfma_frac=mx_flops / t / (MXFP4_PEAK_TFLOPS * 1e12),
                   mfma_time_frac=(bf16_flops / (BF16_PEAK_TFLOPS * 1e12) + mx_flops / (MXFP4_PEAK_TFLOPS * 1e12)) / t)
        ms_b = time_chunk(a_bf16)
        res.update(ms_per_chunk_bf16_scores=ms_b, tokens_per_s_bf16_scores=C / (ms_b / 1e3))
    else:
        res["mfma_time_frac"] = bf16_flops / (BF16_PEAK_TFLOPS * 1e12) / t
    return res


def percentiles(ms):
    """Median and 10th / 90th percentiles of per-step times (ms)."""
    v = np.asarray(ms, np.float64)
    return {"p10": float(np.percentile(v, 10)), "p50": float(np.percentile(v, 50)), "p90": float(np.percentile(v, 90)),
            "mean": float(v.mean()), "n": int(v.size)}


def timed(torch, fn, steps, warmup):
    """Mean GPU time (ms) of fn(i) over `steps` back-to-back calls, and its per-call percentiles."""
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for i in range(steps):
        fn(warmup + i)
    b.record()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for i in range(steps):
        ev[i][0].record()
        fn(warmup + i)
        ev[i][1].record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / steps, percentiles([x.elapsed_time(y) for x, y in ev])


def mtp_variant(v4, torch, args, sets, step_kwargs, inp, bf16, f32, B, H, D, W, HI, dI, N):
    """The headline step verifying two tokens per sequence (multi-token prediction with depth 1):
    queries at positions T-2 and T-1 of every sequence, evaluated together in one call."""
    from workloads import CSA_PRO_1M, normal
    wl = CSA_PRO_1M
    s = wl.seed
    Q = 2
    q2 = bf16(normal(s, "q", (B, Q, H, D)))
    qi2 = v4.Idx.empty(B, Q * HI, dI)
    v4.v4a_quantize_mxfp4(f32(normal(s, "q_idx", (B * Q * HI, dI))), qi2)
    w2 = f32(normal(s, "w", (B, Q, HI)))
    win2 = bf16(normal(s, "window", (B, W + Q - 1, D)))
    out2 = torch.empty((B, Q, H, D), dtype=torch.bfloat16, device="cuda")
    margs = []
    for kw in step_kwargs:
        kw2 = dict(kw)
        kw2.update(q=q2, q_idx=qi2, w=w2, win=win2, out=out2, Q=Q)
        margs.append(v4.DecodeStepArgs(**kw2))
    mws = v4.workspace(v4.v4a_decode_step_workspace(margs[0]))
    ms, pct = timed(torch, lambda i: v4.v4a_decode_step_csa(margs[i % len(margs)], mws), args.steps, args.warmup)
    return {"entry_point": "v4a_decode_step_csa (Q = 2)", "queries_per_sequence": Q, "ms_per_step": ms,
            "ms_per_step_pct": pct, "tokens_per_s": B * Q / (ms / 1e3)}


def csa_step_secondary(v4, torch, wl, args, f32, bf16):
    """The fused CSA decode step of a second workload (the Flash-like 131K-context batch): tokens/s
    and the step's algorithmic HBM bytes over its time."""
    from workloads import decode_inputs, normal
    print(f"[bench] secondary: {wl.name}", file=sys.stderr, flush=True)
    inp = decode_inputs(wl, threads=16)
    B, H, D, R, W, k, HI, dI, m, N = wl.B, wl.H, wl.D, wl.R, wl.W, wl.k, wl.H_I, wl.d_I, wl.m, inp["N"]
    T = wl.T
    s = wl.seed
    kv0 = v4.KV.empty(B, N, D, R)
    v4.v4a_quantize_kv(f32(inp.pop("records").reshape(-1, D)), kv0)
    keys0 = v4.Idx.empty(B, N, dI)
    v4.v4a_quantize_mxfp4(f32(inp.pop("keys").reshape(-1, dI)), keys0)
    qi = v4.Idx.empty(B, HI, dI)
    v4.v4a_quantize_mxfp4(f32(inp["q_idx"].reshape(-1, dI)), qi)
    raw = {n: (bf16 if n in ("kv_a", "kv_b", "idx_a", "idx_b") else f32)(
        normal(s, n, (B, 2 * m, D if n in ("kv_a", "kv_b") else (dI if n.startswith("idx_") and "gate" not in n else 1))))
        for n in ("kv_a", "kv_b", "gate_a", "gate_b", "idx_a", "idx_b", "idx_gate_a", "idx_gate_b")}
    bias = {n: f32(normal(s, n, (m, 1))) for n in ("bias_a", "bias_b", "idx_bias_a", "idx_bias_b")}
    # input copies rotated so that the keys and records do not stay in the 256 MB Infinity Cache
    rot = max(1, min(args.rotate, 8))
    copies = [(kv0, keys0)] + [(v4.KV(kv0.fmt, D, R, kv0.nope.clone(), kv0.rope.clone(), kv0.scale.clone(), N),
                                v4.Idx(keys0.fmt, dI, keys0.codes.clone(), keys0.scales.clone(), N))
                               for _ in range(rot - 1)]
    out = torch.empty((B, H, D), dtype=torch.bfloat16, device="cuda")
    q_pos = [T - 1] * B
    sargs = [v4.DecodeStepArgs(q_pos=q_pos, n_entries=[N] * B, m=m, kv=kv, keys=keys, q_idx=qi, w=f32(inp["w"]), k=k,
                               q=bf16(inp["q"]), win=bf16(inp["window"]), win_len=[W] * B, W=W,
                               sink=f32(inp["sink"]), softmax_scale=wl.scale, out=out, **raw, **bias)
             for kv, keys in copies]
    sws = v4.workspace(v4.v4a_decode_step_workspace(sargs[0]))
    v4.v4a_decode_step_csa(sargs[0], sws)
    cargs = [v4.DecodeStepArgs(q_pos=q_pos, n_entries=[N] * B, m=m, kv=kv, keys=keys, q_idx=qi, w=f32(inp["w"]),
                               k=k, q=bf16(inp["q"]), win=bf16(inp["window"]), win_len=[W] * B, W=W,
                               sink=f32(inp["sink"]), softmax_scale=wl.scale, out=out, ws_clean=True, **raw, **bias)
             for kv, keys in copies]
    ms, pct = timed(torch, lambda i: v4.v4a_decode_step_csa(cargs[i % rot], sws), args.steps, args.warmup)
    nbytes = B * N * (dI // 2 + dI // 32) + B * HI * (dI // 2 + dI // 32 + 4) + B * k * ((D - R) + 2 * R + 4) + \
        B * W * D * 2 + B * H * D * 2 * 2 + B * 2 * m * (D + dI) * 2 * 2
    return {"workload": wl.name, "tokens_per_s": B / (ms / 1e3), "ms_per_step": ms, "ms_per_step_pct": pct,
            "bound": "hbm", "algorithmic_bytes": nbytes, "hbm_gbs": nbytes / (ms / 1e3) / 1e9,
            "hbm_frac": nbytes / (ms / 1e3) / 1e9 / HBM_PEAK_GBS, "input_copies": rot,
            "entry_point": "v4a_decode_step_csa"}


def compress_secondary(v4, torch, args):
    """The standalone compressors over 1,048,576 raw BF16 tokens of one sequence: HCA (m' = 128,
    8192 records) and CSA (m = 4, overlapped, 262,144 records plus 262,144 MXFP4 indexer keys).
    Inputs are seeded draws on the device (torch's generator); the figure is algorithmic bytes
    (every raw row read once, records and keys written) over the call's time."""
    print("[bench] secondary: compressors over 1M tokens", file=sys.stderr, flush=True)
    T, D, R, dI = 1 << 20, 512, 64, 128
    g = torch.Generator(device="cuda")
    g.manual_seed(20260425 + 5)

    def bf16n(*shape):
        return torch.randn(shape, generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)

    def f32n(*shape):
        return torch.randn(shape, generator=g, device="cuda", dtype=torch.float32)

    res = {}
    kv_h, gate_h, bias_h = bf16n(T, D), f32n(T, 1), f32n(128, 1)
    rec_h = v4.KV.empty(1, T // 128, D, R)
    ms, pct = timed(torch, lambda i: v4.v4a_compress_hca(kv_h, gate_h, bias_h, tok0=0, m=128, first_entry=0,
                                                         n_entries=T // 128, out_kv=rec_h), 10, 2)
    nb = T * D * 2 + T * 4 + (T // 128) * ((D - R) + 2 * R + 4)
    res["hca"] = {"tokens": T, "entries": T // 128, "ms": ms, "ms_pct": pct, "algorithmic_bytes": nb,
                  "hbm_gbs": nb / (ms / 1e3) / 1e9, "hbm_frac": nb / (ms / 1e3) / 1e9 / HBM_PEAK_GBS}
    del kv_h, gate_h
    kv_a, kv_b, ga, gb = bf16n(T, D), bf16n(T, D), f32n(T, 1), f32n(T, 1)
    ba, bb = f32n(4, 1), f32n(4, 1)
    rec = v4.KV.empty(1, T // 4, D, R)
    ms_r, pct_r = timed(torch, lambda i: v4.v4a_compress_csa(kv_a, kv_b, ga, gb, ba, bb, tok0=0, m=4, first_entry=0,
                                                             n_entries=T // 4, out_kv=rec), 10, 2)
    del kv_a, kv_b
    ia, ib = bf16n(T, dI), bf16n(T, dI)
    keys = v4.Idx.empty(1, T // 4, dI)
    ms_k, pct_k = timed(torch, lambda i: v4.v4a_compress_csa(ia, ib, ga, gb, ba, bb, tok0=0, m=4, first_entry=0,
                                                             n_entries=T // 4, out_idx=keys), 10, 2)
    nb_r = 2 * T * D * 2 + 2 * T * 4 + (T // 4) * ((D - R) + 2 * R + 4)
    nb_k = 2 * T * dI * 2 + 2 * T * 4 + (T // 4) * (dI // 2 + dI // 32)
    res["csa_records"] = {"tokens": T, "entries": T // 4, "ms": ms_r, "ms_pct": pct_r, "algorithmic_bytes": nb_r,
                          "hbm_gbs": nb_r / (ms_r / 1e3) / 1e9, "hbm_frac": nb_r / (ms_r / 1e3) / 1e9 / HBM_PEAK_GBS}
    res["csa_keys"] = {"tokens": T, "entries": T // 4, "ms": ms_k, "ms_pct": pct_k, "algorithmic_bytes": nb_k,
                       "hbm_gbs": nb_k / (ms_k / 1e3) / 1e9, "hbm_frac": nb_k / (ms_k / 1e3) / 1e9 / HBM_PEAK_GBS}
    return res


def projection_secondary(v4, torch, args):
    """The grouped output projection (128 heads of 512 in 16 groups, each reduced to 1024, then
    projected to 7168) for the decode batch of the headline workload (4 tokens: weight-streaming,
    HBM-bound) and a 4096-token prefill chunk (MFMA-bound).  Synthetic seeded weights."""
    print("[bench] secondary: grouped output projection", file=sys.stderr, flush=True)
    H, D, G, r, d = 128, 512, 16, 1024, 7168
    g = torch.Generator(device="cuda")
    g.manual_seed(20260425 + 6)
    Kg = H * D // G
    wg = (torch.randn((G, r, Kg), generator=g, device="cuda") / math.sqrt(Kg)).to(torch.bfloat16)
    wf = (torch.randn((d, G * r), generator=g, device="cuda") / math.sqrt(G * r)).to(torch.bfloat16)
    res = {}
    for name, T in (("decode_4_tokens", 4), ("prefill_4096_tokens", 4096)):
        o = (0.3 * torch.randn((T, H, D), generator=g, device="cuda")).to(torch.bfloat16)
        out = torch.empty((T, d), dtype=torch.bfloat16, device="cuda")
        ws = v4.workspace(v4.v4a_output_projection_workspace(T, G, r))
        ms, pct = timed(torch, lambda i: v4.v4a_output_projection(o, G, r, wg, wf, out, ws), 20, 3)
        flops = 2.0 * T * (G * r * Kg + d * G * r)
        nbytes = 2 * (G * r * Kg + d * G * r) + 2 * T * (H * D + 2 * G * r + d)
        res[name] = {"tokens": T, "ms": ms, "ms_pct": pct, "flops": flops, "algorithmic_bytes": nbytes,
                     "mfma_tflops": flops / (ms / 1e3) / 1e12, "mfma_frac": flops / (ms / 1e3) / (BF16_PEAK_TFLOPS * 1e12),
                     "hbm_gbs": nbytes / (ms / 1e3) / 1e9, "hbm_frac": nbytes / (ms / 1e3) / 1e9 / HBM_PEAK_GBS,
                     "bound": "hbm" if T <= 64 else "mfma"}
    return res


def source_hash(names):
    import hashlib
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "compressed_sparse_attention_02_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per launch of the MXFP4 scoring kernel from the committed counter summary, or
    None when it is missing or was taken with other kernel sources."""
    try:
        fields = {}
        with open(TRAFFIC_FILE) as f:
            for line in f:
                if ":" in line and not line.startswith("#"):
                    key, val = line.split(":", 1)
                    fields[key.strip()] = val.strip()
        if fields.get("kernel_sources_sha256") != source_hash(TRAFFIC_SOURCES):
            return None
        return float(fields["hbm_bytes_scoring_kernel"])
    except (OSError, KeyError, ValueError):
        return None


if __name__ == "__main__":
    main()
