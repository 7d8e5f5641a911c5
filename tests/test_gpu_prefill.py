"""GPU parity of the prefill chunk (a8, v4a_prefill_chunk) against the oracle.

A chunk of C tokens is compressed into the caches (with its raw state), then every chunk
query attends causally: CSA over its top-k entries, HCA over all its visible entries, both
with the window of raw tokens ending at the query and the sink.  Checked here:
  - the fp32 workload in two chained chunks, end to end from the raw streams against the
    oracle (entries to 1e-5 relative, outputs to 1e-5 absolute), with the selections exact;
  - BF16/FP8/MXFP4 chunks (CSA and HCA) against the oracle fed the caches the GPU wrote:
    the selections of sampled queries exact, the outputs to the BF16 bar;
  - the appended entries bitwise equal to one compressor call over the whole stream buffer;
  - prefill == decode: a chunk query's output against the decode call at the same position
    on the same caches (bitwise on the unsplit fp32 path, to the BF16 bar where decode splits);
  - the long-context chunk (4096 tokens on a 65536-token cache) on sampled queries.
"""
import math

import numpy as np
import pytest
import torch

import compressed_sparse_attention_02_amd as v4
import oracle
from gpu_util import (MAX_ABS_BF16, MAX_ABS_F32, REL_L2_BF16, announce, bf16_from_bits, bf16_round, check_close,
                      f32, idx_from_f32, out_f64, rel_close)
from workloads import PREFILL_64K, TINY, bf16_bits_to_f64, normal, prefill_inputs, scaled, to_bf16_bits

pytestmark = pytest.mark.gpu
CSA, HCA = v4.V4A_LAYER_CSA, v4.V4A_LAYER_HCA


def sample_queries(C, step=64, tail=8):
    """Every step-th chunk query plus the last `tail` ones."""
    return sorted(set(range(0, C, step)) | set(range(max(0, C - tail), C)))


def bf16_dev(x):
    """BF16 device copy of fp32 x and the float64 values it holds."""
    bits = to_bf16_bits(x)
    return bf16_from_bits(bits), bf16_bits_to_f64(bits)


def slot_view(t, b):
    return t[b:b + 1]


def kv_slot(kv, b):
    return v4.KV(kv.fmt, kv.D, kv.R, slot_view(kv.nope, b), slot_view(kv.rope, b), slot_view(kv.scale, b), kv.cap)


def idx_slot(ix, b):
    return v4.Idx(ix.fmt, ix.d, slot_view(ix.codes, b), slot_view(ix.scales, b), ix.cap)


def dequant_slot(kv, n):
    """float64 entries [n][D] of a one-slot FP8/BF16 cache, decoded by the oracle."""
    nope = kv.nope[0, :n].cpu().numpy()
    rope = kv.rope[0, :n].cpu().numpy().view(np.uint16)
    scale = kv.scale[0, :n].cpu().numpy()
    return oracle.dequant_kv(nope, rope, scale)


# ------------------------------------------------------------ fp32, two chunks ----

def test_tiny_fp32_two_chunks():
    w = TINY
    D, R, H, HI, dI, k, W = w.D, w.R, w.H, w.H_I, w.d_I, w.k, w.W
    T, s = 762, w.seed
    x = dict(kv_a=normal(s, "kv_a", (T, D)), kv_b=normal(s, "kv_b", (T, D)), gate_a=normal(s, "gate_a", (T, 1)),
             gate_b=normal(s, "gate_b", (T, 1)), bias_a=normal(s, "bias_a", (4, 1)), bias_b=normal(s, "bias_b", (4, 1)),
             idx_a=normal(s, "idx_a", (T, dI)), idx_b=normal(s, "idx_b", (T, dI)),
             idx_gate_a=normal(s, "idx_gate_a", (T, 1)), idx_gate_b=normal(s, "idx_gate_b", (T, 1)),
             idx_bias_a=normal(s, "idx_bias_a", (4, 1)), idx_bias_b=normal(s, "idx_bias_b", (4, 1)),
             kv_h=normal(s, "kv_h", (T, D)), gate_h=normal(s, "gate_h", (T, 1)), bias_h=normal(s, "bias_h", (128, 1)))
    q = normal(s, "q_chunk", (T, H, D))
    q_idx = normal(s, "q_idx_chunk", (T, HI, dI))
    wts = normal(s, "w_chunk", (T, HI))
    sink = normal(s, "sink", (H,))
    scale = 1.0 / math.sqrt(D)
    rec_c = v4.KV.empty(1, 256, D, R, fmt=v4.V4A_KV_F32)
    keys = v4.Idx.empty(1, 256, dI, fmt=v4.V4A_IDX_F32)
    rec_h = v4.KV.empty(1, 8, D, R, fmt=v4.V4A_KV_F32)
    chunks = [(0, 0, 512), (512, 128, 250)]
    outs, keep = [], []
    for tok0, n_prev, C in chunks:
        lo, hi = tok0 - n_prev, tok0 + C
        announce(f"prefill fp32 chunk tok0={tok0} C={C} n_prev={n_prev}")
        qi = idx_from_f32(q_idx[tok0:hi].reshape(1, C * HI, dI), v4.V4A_IDX_F32)
        out_c = torch.empty((C, H, D), dtype=torch.float32, device="cuda")
        out_h = torch.empty((C, H, D), dtype=torch.float32, device="cuda")
        a = v4.PrefillArgs(tok0=tok0, n_prev=n_prev, m=4, kv_a=f32(x["kv_a"][lo:hi]), kv_b=f32(x["kv_b"][lo:hi]),
                           gate_a=f32(x["gate_a"][lo:hi]), gate_b=f32(x["gate_b"][lo:hi]), bias_a=f32(x["bias_a"]),
                           bias_b=f32(x["bias_b"]), kv=rec_c, idx_a=f32(x["idx_a"][lo:hi]),
                           idx_b=f32(x["idx_b"][lo:hi]), idx_gate_a=f32(x["idx_gate_a"][lo:hi]),
                           idx_gate_b=f32(x["idx_gate_b"][lo:hi]), idx_bias_a=f32(x["idx_bias_a"]),
                           idx_bias_b=f32(x["idx_bias_b"]), keys=keys, q_idx=qi, w=f32(wts[tok0:hi]), k=k,
                           q=f32(q[tok0:hi]), W=W, sink=f32(sink), softmax_scale=scale, out=out_c)
        ws = v4.workspace(v4.v4a_prefill_workspace(CSA, a))
        v4.v4a_prefill_chunk(CSA, a, ws)
        ah = v4.PrefillArgs(tok0=tok0, n_prev=n_prev, m=128, kv_a=f32(x["kv_h"][lo:hi]),
                            gate_a=f32(x["gate_h"][lo:hi]), bias_a=f32(x["bias_h"]), kv=rec_h, q=f32(q[tok0:hi]),
                            W=W, sink=f32(sink), softmax_scale=scale, out=out_h)
        assert v4.v4a_prefill_workspace(HCA, ah) == 0
        v4.v4a_prefill_chunk(HCA, ah, None)
        torch.cuda.synchronize()
        outs.append((out_c, out_h))
        keep.append((a, ah, ws))
    Nc, Nh = T // 4, T // 128

    # entries: the oracle compresses the whole stream at once
    ent = oracle.compress_csa(x["kv_a"], x["kv_b"], x["gate_a"], x["gate_b"], x["bias_a"], x["bias_b"], tok0=0,
                              m=4, first_entry=0, n_entries=Nc, apply_rope=True, R=R)
    ik = oracle.compress_csa(x["idx_a"], x["idx_b"], x["idx_gate_a"], x["idx_gate_b"], x["idx_bias_a"],
                             x["idx_bias_b"], tok0=0, m=4, first_entry=0, n_entries=Nc, apply_rope=False, R=0)
    he = oracle.compress_hca(x["kv_h"], x["gate_h"], x["bias_h"], tok0=0, m=128, first_entry=0, n_entries=Nh,
                             apply_rope=True, R=R)
    g_ent = rec_c.nope[0, :Nc].cpu().numpy()
    g_keys = keys.codes[0, :Nc].cpu().numpy()
    g_he = rec_h.nope[0, :Nh].cpu().numpy()
    rel_close(g_ent, ent)
    rel_close(g_keys, ik)
    rel_close(g_he, he)

    for (tok0, n_prev, C), (out_c, out_h) in zip(chunks, outs):
        lo, hi = tok0 - n_prev, tok0 + C
        announce(f"prefill fp32 chunk tok0={tok0}: selections through v4a_indexer_topk")
        qi = idx_from_f32(q_idx[tok0:hi].reshape(1, C * HI, dI), v4.V4A_IDX_F32)
        sel = torch.empty((1, C, k), dtype=torch.int32, device="cuda")
        ws = v4.workspace(v4.v4a_indexer_topk_workspace(1, C, Nc, k))
        v4.v4a_indexer_topk(keys, [Nc], 4, qi, f32(wts[tok0:hi]), 1, C, HI, [tok0 + j for j in range(C)], k, sel, ws)
        torch.cuda.synchronize()
        ref_c, ref_sel = oracle.prefill_queries(
            "csa", q[tok0:hi].astype(np.float64), g_ent.astype(np.float64), (tok0 + C) // 4,
            x["kv_a"][lo:hi].astype(np.float64), n_prev=n_prev, tok0=tok0, queries=range(C), W=W, sink=sink,
            scale=scale, m=4, k=k, idx=dict(q=q_idx[tok0:hi], w=wts[tok0:hi], keys=g_keys), R=R)
        gsel = sel[0].cpu().numpy()
        bad = [j for j in range(C) if not np.array_equal(gsel[j], ref_sel[j])]
        assert not bad, f"top-k differs for chunk queries {bad[:10]}"
        check_close(out_f64(out_c), np.stack([ref_c[j] for j in range(C)]), MAX_ABS_F32, what=f"csa chunk {tok0}")
        ref_h, _ = oracle.prefill_queries(
            "hca", q[tok0:hi].astype(np.float64), g_he.astype(np.float64), (tok0 + C) // 128,
            x["kv_h"][lo:hi].astype(np.float64), n_prev=n_prev, tok0=tok0, queries=range(C), W=W, sink=sink,
            scale=scale, m=128, R=R)
        check_close(out_f64(out_h), np.stack([ref_h[j] for j in range(C)]), MAX_ABS_F32, what=f"hca chunk {tok0}")

        # prefill == decode, bitwise (the fp32 kernel never splits)
        for j in (0, 5, C // 2, C - 1):
            t = tok0 + j
            wl = min(W, t + 1)
            win_c = torch.zeros((1, W, D), dtype=torch.float32, device="cuda")
            win_h = torch.zeros((1, W, D), dtype=torch.float32, device="cuda")
            win_c[0, :wl] = f32(x["kv_a"][t - wl + 1:t + 1])
            win_h[0, :wl] = f32(x["kv_h"][t - wl + 1:t + 1])
            dc = torch.empty((1, H, D), dtype=torch.float32, device="cuda")
            dh = torch.empty((1, H, D), dtype=torch.float32, device="cuda")
            v4.v4a_decode_csa(f32(q[t][None]), rec_c, sel[0, j][None].contiguous(), k, win_c, [wl], W, f32(sink),
                              [t], softmax_scale=scale, out=dc)
            v4.v4a_decode_hca(f32(q[t][None]), rec_h, [(tok0 + C) // 128], 128, win_h, [wl], W, f32(sink), [t],
                              softmax_scale=scale, out=dh)
            torch.cuda.synchronize()
            assert torch.equal(dc[0], out_c[j]), f"csa prefill != decode at t={t}"
            assert torch.equal(dh[0], out_h[j]), f"hca prefill != decode at t={t}"


# ----------------------------------------------------- BF16 / FP8 / MXFP4 chunks ----

def run_csa_chunk(w, slot=1, n_slots=2, score_bf16=False, norm=False):
    """Cache the drawn entries in `slot`, run one CSA prefill chunk; returns everything a check needs."""
    x = prefill_inputs(w, kind="csa")
    C, tok0, n_prev, N0 = x["C"], x["tok0"], x["n_prev"], x["N0"]
    D, R, H, HI, dI, k, W = w.D, w.R, w.H, w.H_I, w.d_I, w.k, w.W
    n_total = (tok0 + C) // 4
    cap = n_total + 64
    announce(f"prefill csa: tok0={tok0} C={C} cached={N0} H={H} k={k} score_bf16={score_bf16}")
    kv = v4.KV.empty(n_slots, cap, D, R)
    keys = v4.Idx.empty(n_slots, cap, dI)
    v4.v4a_quantize_kv(f32(x["records"]), kv, slot * cap)
    v4.v4a_quantize_mxfp4(f32(x["keys"]), keys, slot * cap)
    qi = v4.Idx.empty(1, C * HI, dI)
    v4.v4a_quantize_mxfp4(f32(x["q_idx"].reshape(-1, dI)), qi)
    dev, val = {}, {}
    for name in ("kv_a", "kv_b", "idx_a", "idx_b"):
        dev[name], val[name] = bf16_dev(x[name])
    q_dev, _ = bf16_dev(x["q"])
    gnw = np.random.default_rng(70)
    nw = f32(0.5 + gnw.random(D)) if norm else None
    nwi = f32(0.5 + gnw.random(dI)) if norm else None
    out = torch.empty((C, H, D), dtype=torch.bfloat16, device="cuda")
    a = v4.PrefillArgs(tok0=tok0, n_prev=n_prev, m=4, kv_a=dev["kv_a"], kv_b=dev["kv_b"], gate_a=f32(x["gate_a"]),
                       gate_b=f32(x["gate_b"]), bias_a=f32(x["bias_a"]), bias_b=f32(x["bias_b"]), kv=kv, slot=slot,
                       idx_a=dev["idx_a"], idx_b=dev["idx_b"], idx_gate_a=f32(x["idx_gate_a"]),
                       idx_gate_b=f32(x["idx_gate_b"]), idx_bias_a=f32(x["idx_bias_a"]),
                       idx_bias_b=f32(x["idx_bias_b"]), keys=keys, q_idx=qi, w=f32(x["w"]), k=k, q=q_dev, W=W,
                       sink=f32(x["sink"]), softmax_scale=w.scale, out=out, score_bf16=score_bf16, norm_w=nw,
                       idx_norm_w=nwi)
    ws = v4.workspace(v4.v4a_prefill_workspace(CSA, a))
    v4.v4a_prefill_chunk(CSA, a, ws)
    torch.cuda.synchronize()
    return dict(x=x, a=a, ws=ws, kv=kv, keys=keys, qi=qi, dev=dev, val=val, q_dev=q_dev, out=out, n_total=n_total,
                cap=cap, slot=slot, score_bf16=score_bf16, norm_w=nw, idx_norm_w=nwi)


def check_csa_chunk(w, r, queries, decode_queries=()):
    x, kv1, keys1 = r["x"], kv_slot(r["kv"], r["slot"]), idx_slot(r["keys"], r["slot"])
    C, tok0, n_prev, N0, n_total = x["C"], x["tok0"], x["n_prev"], x["N0"], r["n_total"]
    D, R, H, HI, dI, k, W = w.D, w.R, w.H, w.H_I, w.d_I, w.k, w.W
    # appended entries: bitwise one compressor call over the whole stream buffer
    announce("prefill csa: appended entries vs one compressor call")
    ref_kv = v4.KV.empty(1, r["cap"], D, R)
    ref_keys = v4.Idx.empty(1, r["cap"], dI)
    n_new = n_total - N0
    v4.v4a_compress_csa(r["dev"]["kv_a"], r["dev"]["kv_b"], f32(x["gate_a"]), f32(x["gate_b"]), f32(x["bias_a"]),
                        f32(x["bias_b"]), tok0=tok0 - n_prev, m=4, first_entry=N0, n_entries=n_new, out_kv=ref_kv,
                        norm_w=r["norm_w"])
    v4.v4a_compress_csa(r["dev"]["idx_a"], r["dev"]["idx_b"], f32(x["idx_gate_a"]), f32(x["idx_gate_b"]),
                        f32(x["idx_bias_a"]), f32(x["idx_bias_b"]), tok0=tok0 - n_prev, m=4, first_entry=N0,
                        n_entries=n_new, out_idx=ref_keys, norm_w=r["idx_norm_w"])
    torch.cuda.synchronize()
    for got, ref in ((kv1.nope, ref_kv.nope), (kv1.rope, ref_kv.rope), (kv1.scale, ref_kv.scale),
                     (keys1.codes, ref_keys.codes), (keys1.scales, ref_keys.scales)):
        assert torch.equal(got[0, N0:n_total], ref[0, N0:n_total])

    announce("prefill csa: selections through v4a_indexer_topk, oracle on sampled queries")
    sel = torch.empty((1, C, k), dtype=torch.int32, device="cuda")
    ws = v4.workspace(v4.v4a_indexer_topk_workspace(1, C, n_total, k))
    topk_call = v4.v4a_indexer_topk_bf16 if r["score_bf16"] else v4.v4a_indexer_topk
    topk_call(keys1, [n_total], 4, r["qi"], f32(x["w"]), 1, C, HI, [tok0 + j for j in range(C)], k, sel, ws)
    torch.cuda.synchronize()
    recs = dequant_slot(kv1, n_total)
    kc = keys1.codes[0, :n_total].cpu().numpy()
    ks = keys1.scales[0, :n_total].cpu().numpy()
    qc = r["qi"].codes[0].cpu().numpy().reshape(C, HI, dI // 2)
    qs = r["qi"].scales[0].cpu().numpy().reshape(C, HI, dI // 32)
    q64 = bf16_bits_to_f64(to_bf16_bits(x["q"]))
    ref, ref_sel = oracle.prefill_queries(
        "csa", q64, recs, n_total, r["val"]["kv_a"], n_prev=n_prev, tok0=tok0, queries=queries, W=W,
        sink=x["sink"], scale=w.scale, m=4, k=k,
        idx=dict(q_codes=qc, q_scales=qs, w=x["w"], k_codes=kc, k_scales=ks), R=R, score_bf16=r["score_bf16"])
    gsel = sel[0].cpu().numpy()
    bad = [j for j in queries if not np.array_equal(gsel[j], ref_sel[j])]
    assert not bad, f"top-k differs for chunk queries {bad[:10]}"
    got = out_f64(r["out"])
    check_close(got[queries], bf16_round(np.stack([ref[j] for j in queries])), MAX_ABS_BF16, REL_L2_BF16,
                what="csa prefill vs oracle")

    for j in decode_queries:
        t = tok0 + j
        announce(f"prefill csa == decode at t={t}")
        win = r["dev"]["kv_a"][n_prev + j - W + 1:n_prev + j + 1][None].contiguous()
        dc = torch.empty((1, H, D), dtype=torch.bfloat16, device="cuda")
        dws = v4.workspace(v4.v4a_decode_workspace(1, H, D, k, W))
        v4.v4a_decode_csa(r["q_dev"][j][None].contiguous(), kv1, sel[0, j][None].contiguous(), k, win, [W], W,
                          f32(x["sink"]), [t], softmax_scale=w.scale, out=dc, ws=dws)
        torch.cuda.synchronize()
        check_close(out_f64(dc)[0], got[j], MAX_ABS_BF16, REL_L2_BF16, what=f"decode vs prefill t={t}")


def test_csa_mxfp4_chunk():
    w = scaled(PREFILL_64K, T=8192, chunk=700)
    r = run_csa_chunk(w)
    check_csa_chunk(w, r, sample_queries(700), decode_queries=(0, 349, 699))


def test_csa_mxfp4_chunk_rmsnorm():
    """The chunk with RMS-normalised new entries and keys: appended entries bitwise equal to one
    compressor call with the same weights, selections and outputs against the oracle fed the
    caches the GPU wrote."""
    w = scaled(PREFILL_64K, T=8192, chunk=700)
    r = run_csa_chunk(w, norm=True)
    check_csa_chunk(w, r, sample_queries(700), decode_queries=(349,))


def test_csa_mxfp4_chunk_bf16_scores():
    """The chunk with the BF16-score selector: selections equal v4a_indexer_topk_bf16's and the
    oracle's over BF16-rounded scores."""
    w = scaled(PREFILL_64K, T=8192, chunk=700)
    r = run_csa_chunk(w, score_bf16=True)
    check_csa_chunk(w, r, sample_queries(700), decode_queries=(349,))


def run_hca_chunk(w, q_norm_w=None):
    x = prefill_inputs(w, kind="hca")
    C, tok0, n_prev, N0 = x["C"], x["tok0"], x["n_prev"], x["N0"]
    D, R, H, W = w.D, w.R, w.H, w.W
    n_total = (tok0 + C) // 128
    cap = n_total + 8
    announce(f"prefill hca: tok0={tok0} C={C} cached={N0} H={H}")
    kv = v4.KV.empty(1, cap, D, R)
    v4.v4a_quantize_kv(f32(x["records"]), kv, 0)
    kv_dev, kv_val = bf16_dev(x["kv_a"])
    q_dev, _ = bf16_dev(x["q"])
    out = torch.empty((C, H, D), dtype=torch.bfloat16, device="cuda")
    a = v4.PrefillArgs(tok0=tok0, n_prev=n_prev, m=128, kv_a=kv_dev, gate_a=f32(x["gate_a"]), bias_a=f32(x["bias_a"]),
                       kv=kv, q=q_dev, W=W, sink=f32(x["sink"]), softmax_scale=w.scale, out=out,
                       q_norm_w=None if q_norm_w is None else f32(q_norm_w))
    v4.v4a_prefill_chunk(HCA, a, None)
    torch.cuda.synchronize()
    return dict(x=x, a=a, kv=kv, kv_dev=kv_dev, kv_val=kv_val, q_dev=q_dev, out=out, n_total=n_total, cap=cap)


def check_hca_chunk(w, r, queries, decode_queries=()):
    x, kv = r["x"], r["kv"]
    C, tok0, n_prev, N0, n_total = x["C"], x["tok0"], x["n_prev"], x["N0"], r["n_total"]
    D, R, H, W = w.D, w.R, w.H, w.W
    announce("prefill hca: appended entries vs one compressor call")
    ref_kv = v4.KV.empty(1, r["cap"], D, R)
    v4.v4a_compress_hca(r["kv_dev"], f32(x["gate_a"]), f32(x["bias_a"]), tok0=tok0 - n_prev, m=128, first_entry=N0,
                        n_entries=n_total - N0, out_kv=ref_kv)
    torch.cuda.synchronize()
    for got, ref in ((kv.nope, ref_kv.nope), (kv.rope, ref_kv.rope), (kv.scale, ref_kv.scale)):
        assert torch.equal(got[0, N0:n_total], ref[0, N0:n_total])
    announce("prefill hca: oracle on sampled queries")
    recs = dequant_slot(kv, n_total)
    q64 = bf16_bits_to_f64(to_bf16_bits(x["q"]))
    ref, _ = oracle.prefill_queries("hca", q64, recs, n_total, r["kv_val"], n_prev=n_prev, tok0=tok0,
                                    queries=queries, W=W, sink=x["sink"], scale=w.scale, m=128, R=R)
    got = out_f64(r["out"])
    check_close(got[queries], bf16_round(np.stack([ref[j] for j in queries])), MAX_ABS_BF16, REL_L2_BF16,
                what="hca prefill vs oracle")
    for j in decode_queries:
        t = tok0 + j
        announce(f"prefill hca == decode at t={t}")
        win = r["kv_dev"][n_prev + j - W + 1:n_prev + j + 1][None].contiguous()
        dh = torch.empty((1, H, D), dtype=torch.bfloat16, device="cuda")
        dws = v4.workspace(v4.v4a_decode_workspace(1, H, D, n_total, W))
        v4.v4a_decode_hca(r["q_dev"][j][None].contiguous(), kv, [n_total], 128, win, [W], W, f32(x["sink"]), [t],
                          softmax_scale=w.scale, out=dh, ws=dws)
        torch.cuda.synchronize()
        check_close(out_f64(dh)[0], got[j], MAX_ABS_BF16, REL_L2_BF16, what=f"decode vs prefill t={t}")


def test_hca_chunk():
    w = scaled(PREFILL_64K, T=16384, chunk=640)
    r = run_hca_chunk(w)
    check_hca_chunk(w, r, sample_queries(640), decode_queries=(0, 320, 639))


# ------------------------------------------ the long-context chunk, full size ----

def test_csa_chunk_full_size():
    w = PREFILL_64K
    r = run_csa_chunk(w, slot=0, n_slots=1)
    check_csa_chunk(w, r, [0, 1, 2047, 4092, 4093, 4094, 4095], decode_queries=(4095,))


def test_hca_chunk_full_size():
    w = PREFILL_64K
    r = run_hca_chunk(w)
    check_hca_chunk(w, r, [0, 1, 2047, 4093, 4094, 4095], decode_queries=(4095,))


# ------------------------------------------- prefill == split-free decode, bit for bit ---
# "DeepSeek-V4 technical report walkthrough" (cyqw.cn), section 3.3: attention without
# split-KV keeps results bitwise identical; the split-free decode step then equals the prefill
# chunk for the same query and caches.

def decode_positions(tok0, C, m, n=6):
    """Chunk queries spread over the chunk whose token completes no block (the step compresses
    nothing, so it reads the caches the chunk left)."""
    js = [j for j in np.linspace(0, C - 1, 3 * n).astype(int) if (tok0 + j + 1) % m != 0]
    return js[:n]


def test_hca_prefill_equals_split_free_decode():
    w = scaled(PREFILL_64K, T=8192, chunk=700)
    r = run_hca_chunk(w)
    x, kv = r["x"], r["kv"]
    tok0, n_prev, D, H, W = x["tok0"], x["n_prev"], w.D, w.H, w.W
    rows = torch.zeros((1, 128, D), dtype=torch.bfloat16, device="cuda")  # read only when a block completes
    gates = torch.zeros((1, 128, 1), dtype=torch.float32, device="cuda")
    js = decode_positions(tok0, x["C"], 128)
    got = {}
    for j in js:
        t = tok0 + j
        announce(f"hca prefill == split-free decode at t={t}")
        win = r["kv_dev"][n_prev + j - W + 1:n_prev + j + 1][None].contiguous()
        out = torch.empty((1, H, D), dtype=torch.bfloat16, device="cuda")
        args = v4.DecodeStepHcaArgs(q_pos=[t], n_entries=[r["n_total"]], m=128, kv_a=rows, gate_a=gates,
                                    bias_a=f32(x["bias_a"]), kv=kv, q=r["q_dev"][j][None].contiguous(), win=win,
                                    win_len=[W], W=W, sink=f32(x["sink"]), softmax_scale=w.scale, out=out,
                                    no_split=True)
        assert v4.v4a_decode_step_hca_workspace(args) == 0
        v4.v4a_decode_step_hca(args, None)
        torch.cuda.synchronize()
        assert torch.equal(out[0], r["out"][j]), f"hca t={t}"
        got[j] = out_f64(out[0])
    # the split-free decode outputs against the oracle directly
    announce("hca split-free decode vs oracle")
    q64 = bf16_bits_to_f64(to_bf16_bits(x["q"]))
    ref, _ = oracle.prefill_queries("hca", q64, dequant_slot(kv, r["n_total"]), r["n_total"], r["kv_val"],
                                    n_prev=n_prev, tok0=tok0, queries=js, W=W, sink=x["sink"], scale=w.scale, m=128,
                                    R=w.R)
    check_close(np.stack([got[j] for j in js]), bf16_round(np.stack([ref[j] for j in js])), MAX_ABS_BF16, REL_L2_BF16,
                what="hca split-free decode vs oracle")


def test_csa_prefill_equals_split_free_decode():
    w = scaled(PREFILL_64K, T=8192, chunk=700)
    r = run_csa_chunk(w)
    x = r["x"]
    tok0, n_prev, C, D, dI, H, HI, k, W = x["tok0"], x["n_prev"], x["C"], w.D, w.d_I, w.H, w.H_I, w.k, w.W
    kv1, keys1 = kv_slot(r["kv"], r["slot"]), idx_slot(r["keys"], r["slot"])
    z = lambda *shape, dt=torch.bfloat16: torch.zeros(shape, dtype=dt, device="cuda")  # rows read only on completion
    zf = lambda *shape: z(*shape, dt=torch.float32)
    js = decode_positions(tok0, C, 4)
    got, got_sel = {}, {}
    for j in js:
        t = tok0 + j
        announce(f"csa prefill == split-free decode at t={t}")
        qi = v4.Idx(r["qi"].fmt, dI, r["qi"].codes[:, j * HI:(j + 1) * HI], r["qi"].scales[:, j * HI:(j + 1) * HI], HI)
        win = r["dev"]["kv_a"][n_prev + j - W + 1:n_prev + j + 1][None].contiguous()
        out = torch.empty((1, H, D), dtype=torch.bfloat16, device="cuda")
        args = v4.DecodeStepArgs(q_pos=[t], n_entries=[r["n_total"]], m=4, kv_a=z(1, 8, D), kv_b=z(1, 8, D),
                                 gate_a=zf(1, 8, 1), gate_b=zf(1, 8, 1), bias_a=zf(4, 1), bias_b=zf(4, 1),
                                 idx_a=z(1, 8, dI), idx_b=z(1, 8, dI), idx_gate_a=zf(1, 8, 1), idx_gate_b=zf(1, 8, 1),
                                 idx_bias_a=zf(4, 1), idx_bias_b=zf(4, 1), kv=kv1, keys=keys1, q_idx=qi,
                                 w=f32(x["w"][j][None]), k=k, q=r["q_dev"][j][None].contiguous(), win=win,
                                 win_len=[W], W=W, sink=f32(x["sink"]), softmax_scale=w.scale, out=out,
                                 no_split=True)
        ws = v4.workspace(v4.v4a_decode_step_workspace(args))
        v4.v4a_decode_step_csa(args, ws)
        torch.cuda.synchronize()
        assert torch.equal(out[0], r["out"][j]), f"csa t={t}"
        got[j] = out_f64(out[0])
        got_sel[j] = ws[:4 * k].view(torch.int32).cpu().numpy()  # the step's selection heads its workspace
    # the split-free decode outputs and selections against the oracle directly
    announce("csa split-free decode vs oracle")
    n_total = r["n_total"]
    qc = r["qi"].codes[0].cpu().numpy().reshape(C, HI, dI // 2)
    qs = r["qi"].scales[0].cpu().numpy().reshape(C, HI, dI // 32)
    idx = dict(q_codes=qc, q_scales=qs, w=x["w"], k_codes=keys1.codes[0, :n_total].cpu().numpy(),
               k_scales=keys1.scales[0, :n_total].cpu().numpy())
    q64 = bf16_bits_to_f64(to_bf16_bits(x["q"]))
    ref, ref_sel = oracle.prefill_queries("csa", q64, dequant_slot(kv1, n_total), n_total, r["val"]["kv_a"],
                                          n_prev=n_prev, tok0=tok0, queries=js, W=W, sink=x["sink"], scale=w.scale,
                                          m=4, k=k, idx=idx, R=w.R)
    for j in js:
        assert np.array_equal(got_sel[j], ref_sel[j]), j
    check_close(np.stack([got[j] for j in js]), bf16_round(np.stack([ref[j] for j in js])), MAX_ABS_BF16, REL_L2_BF16,
                what="csa split-free decode vs oracle")



# --------------------------------------------------------------- query prologue ---
# "DeepSeek-V4 technical report walkthrough" (cyqw.cn), section 2.3: RMSNorm acts directly on the
# queries; with q_norm_w the queries arrive projected only and are normalised and rotated here.

def test_hca_chunk_query_prologue_and_split_free_decode():
    w = scaled(PREFILL_64K, T=8192, chunk=700)
    D, R, H, W = w.D, w.R, w.H, w.W
    qw = (0.5 + np.random.default_rng(80).random(D)).astype(np.float32)
    r = run_hca_chunk(w, q_norm_w=qw)
    x, kv = r["x"], r["kv"]
    tok0, n_prev, C, n_total = x["tok0"], x["n_prev"], x["C"], r["n_total"]
    queries = sample_queries(C)
    announce("hca prefill with query prologue: oracle on sampled queries")
    q_bits = to_bf16_bits(x["q"])
    q64 = np.zeros((C, H, D))
    for j in queries:
        q64[j] = bf16_bits_to_f64(oracle.query_prologue(q_bits[j], qw, pos=tok0 + j, R=R))
    recs = dequant_slot(kv, n_total)
    ref, _ = oracle.prefill_queries("hca", q64, recs, n_total, r["kv_val"], n_prev=n_prev, tok0=tok0, queries=queries,
                                    W=W, sink=x["sink"], scale=w.scale, m=128, R=R)
    got = out_f64(r["out"])
    check_close(got[queries], bf16_round(np.stack([ref[j] for j in queries])), MAX_ABS_BF16, REL_L2_BF16,
                what="hca prefill with query prologue vs oracle")
    rows = torch.zeros((1, 128, D), dtype=torch.bfloat16, device="cuda")
    gates = torch.zeros((1, 128, 1), dtype=torch.float32, device="cuda")
    for j in decode_positions(tok0, C, 128, n=3):
        t = tok0 + j
        announce(f"hca prefill == split-free decode with query prologue at t={t}")
        win = r["kv_dev"][n_prev + j - W + 1:n_prev + j + 1][None].contiguous()
        out = torch.empty((1, H, D), dtype=torch.bfloat16, device="cuda")
        args = v4.DecodeStepHcaArgs(q_pos=[t], n_entries=[n_total], m=128, kv_a=rows, gate_a=gates,
                                    bias_a=f32(x["bias_a"]), kv=kv, q=r["q_dev"][j][None].contiguous(), win=win,
                                    win_len=[W], W=W, sink=f32(x["sink"]), softmax_scale=w.scale, out=out,
                                    no_split=True, q_norm_w=f32(qw))
        v4.v4a_decode_step_hca(args, None)
        torch.cuda.synchronize()
        assert torch.equal(out[0], r["out"][j]), f"t={t}"
