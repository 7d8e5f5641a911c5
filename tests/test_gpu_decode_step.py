"""GPU check of the fused CSA decode step (v4a_decode_step_csa): one call must give bitwise
the same caches, selections and outputs as the separate calls it replaces (v4a_compress_csa
for the entry record and the indexer key of every sequence whose newest token completes a
block, v4a_indexer_topk, v4a_decode_csa), for a batch mixing sequences that complete a block,
one that does not, and one that completes its first block.  Every sequence of the fused call
(plain rows and ring state) is also checked against the oracle fed the caches the GPU wrote."""
import math

import numpy as np
import pytest
import torch

import compressed_sparse_attention_02_amd as v4
import oracle
from gpu_util import (MAX_ABS_BF16, REL_L2_BF16, announce, bf16_from_bits, bf16_round, check_close, f32, few_key_seqs,
                      out_f64)
from workloads import bf16_bits_to_f64, normal, to_bf16_bits

pytestmark = pytest.mark.gpu

HIST_COPIES = 2  # histogram copies per decode query in the step's workspace (kHistCopies)


def clone_kv(kv):
    return v4.KV(kv.fmt, kv.D, kv.R, kv.nope.clone(), kv.rope.clone(), kv.scale.clone(), kv.cap)


def clone_idx(ix):
    return v4.Idx(ix.fmt, ix.d, ix.codes.clone(), ix.scales.clone(), ix.cap)


@pytest.mark.parametrize("score_bf16,norm,key_gate_dim,unaligned",
                         [(False, False, False, False), (True, False, False, False), (False, True, False, False),
                          (False, False, True, False), (False, False, False, True)],
                         ids=["f32_scores", "bf16_scores", "rmsnorm", "key_gate_per_dim", "unaligned_streams"])
def test_fused_step_equals_separate_calls(score_bf16, norm, key_gate_dim, unaligned):
    """With one gate per token the new indexer keys are compressed inside the scoring kernel
    (the step starts with a histogram clear); with a gate per dim, or streams not aligned for
    vector loads, a first launch compresses them."""
    seed, m, D, R, H, HI, dI, k, W = 4242, 4, 512, 64, 128, 64, 128, 512, 128
    q_pos = [4003, 4001, 3, 8191]            # completes entry 1000 / none / entry 0 / entry 2047
    B, cap = len(q_pos), 2304
    n_ent = [(p + 1) // m for p in q_pos]
    entry = [(p + 1) // m - 1 if (p + 1) % m == 0 else -1 for p in q_pos]
    announce(f"fused decode step: q_pos={q_pos} score_bf16={score_bf16} norm={norm} key_gate_dim={key_gate_dim}")
    gnw = np.random.default_rng(seed + 1)
    nw = f32(0.5 + gnw.random(D)) if norm else None
    nwi = f32(0.5 + gnw.random(dI)) if norm else None
    kv = v4.KV.empty(B, cap, D, R)
    v4.v4a_quantize_kv(f32(normal(seed, "records", (B * cap, D))), kv, 0)
    keys = v4.Idx.empty(B, cap, dI)
    v4.v4a_quantize_mxfp4(f32(normal(seed, "keys", (B * cap, dI))), keys, 0)
    qi = v4.Idx.empty(B, HI, dI)  # slot b holds sequence b's H_I query rows
    v4.v4a_quantize_mxfp4(f32(normal(seed, "q_idx", (B * HI, dI))), qi)
    bits = {n: to_bf16_bits(normal(seed, n, (B, 2 * m, D if n.startswith("kv") else dI)))
            for n in ("kv_a", "kv_b", "idx_a", "idx_b")}
    dev = {n: bf16_from_bits(v) for n, v in bits.items()}
    if unaligned:  # the same values one BF16 element past an aligned address
        for n, t in list(dev.items()):
            buf = torch.empty(t.numel() + 1, dtype=t.dtype, device=t.device)
            dev[n] = buf[1:].view(t.shape)
            dev[n].copy_(t)
    gi = dI if key_gate_dim else 1
    gates = {n: f32(normal(seed, n, (B, 2 * m, gi if n.startswith("idx") else 1)))
             for n in ("gate_a", "gate_b", "idx_gate_a", "idx_gate_b")}
    bias = {n: f32(normal(seed, n, (m, gi if n.startswith("idx") else 1)))
            for n in ("bias_a", "bias_b", "idx_bias_a", "idx_bias_b")}
    w = f32(normal(seed, "w", (B, HI)))
    q = bf16_from_bits(to_bf16_bits(normal(seed, "q", (B, H, D))))
    win = bf16_from_bits(to_bf16_bits(normal(seed, "window", (B, W, D))))
    win_len = [min(W, p + 1) for p in q_pos]
    sink = f32(normal(seed, "sink", (H,)))
    scale = 1.0 / math.sqrt(D)

    # the fused call
    def step_args(kv_, keys_, out_, ws_clean=False):
        return v4.DecodeStepArgs(q_pos=q_pos, n_entries=n_ent, m=m, kv_a=dev["kv_a"], kv_b=dev["kv_b"],
                                 gate_a=gates["gate_a"], gate_b=gates["gate_b"], bias_a=bias["bias_a"],
                                 bias_b=bias["bias_b"], idx_a=dev["idx_a"], idx_b=dev["idx_b"],
                                 idx_gate_a=gates["idx_gate_a"], idx_gate_b=gates["idx_gate_b"],
                                 idx_bias_a=bias["idx_bias_a"], idx_bias_b=bias["idx_bias_b"], kv=kv_, keys=keys_,
                                 q_idx=qi, w=w, k=k, q=q, win=win, win_len=win_len, W=W, sink=sink,
                                 softmax_scale=scale, out=out_, score_bf16=score_bf16, norm_w=nw, idx_norm_w=nwi,
                                 ws_clean=ws_clean)

    kv1, keys1 = clone_kv(kv), clone_idx(keys)
    out1 = torch.empty((B, H, D), dtype=torch.bfloat16, device="cuda")
    args = step_args(kv1, keys1, out1)
    ws1 = v4.workspace(v4.v4a_decode_step_workspace(args))
    ws1.fill_(0x55)  # without ws_clean the call clears what it needs
    # timed: the call's kernels in launch order, each with a positive duration
    v4.v4a_trace_begin(16)
    v4.v4a_decode_step_csa(args, ws1)
    n = v4.v4a_trace_end()
    torch.cuda.synchronize()
    kernels = v4.trace_kernels(n)
    first = "decode_prologue_kernel" if key_gate_dim or unaligned else "zero_kernel"
    assert [name for name, _ in kernels] == [first, "indexer_mxfp4_kernel", "select_scan_kernel",
                                             "select_final_kernel", "attn_mfma_kernel", "attn_combine_kernel"], kernels
    assert all(ms > 0 for _, ms in kernels), kernels

    # the separate calls
    kv2, keys2 = clone_kv(kv), clone_idx(keys)
    for b, i in enumerate(entry):
        if i < 0:
            continue
        v4.v4a_compress_csa(dev["kv_a"][b], dev["kv_b"][b], gates["gate_a"][b], gates["gate_b"][b], bias["bias_a"],
                            bias["bias_b"], tok0=m * (i - 1), m=m, first_entry=i, n_entries=1, out_kv=kv2, b=b,
                            norm_w=nw)
        v4.v4a_compress_csa(dev["idx_a"][b], dev["idx_b"][b], gates["idx_gate_a"][b], gates["idx_gate_b"][b],
                            bias["idx_bias_a"], bias["idx_bias_b"], tok0=m * (i - 1), m=m, first_entry=i,
                            n_entries=1, out_idx=keys2, b=b, norm_w=nwi)
    sel = torch.empty((B, 1, k), dtype=torch.int32, device="cuda")
    ws2 = v4.workspace(max(v4.v4a_indexer_topk_workspace(B, 1, max(n_ent), k),
                           v4.v4a_decode_workspace(B, H, D, k, W)))
    (v4.v4a_indexer_topk_bf16 if score_bf16 else v4.v4a_indexer_topk)(keys2, n_ent, m, qi, w, B, 1, HI, q_pos, k,
                                                                        sel, ws2)
    out2 = torch.empty((B, H, D), dtype=torch.bfloat16, device="cuda")
    v4.v4a_decode_csa(q, kv2, sel.view(B, k), k, win, win_len, W, sink, q_pos, softmax_scale=scale, out=out2, ws=ws2)
    torch.cuda.synchronize()

    for a, c in ((kv1.nope, kv2.nope), (kv1.rope, kv2.rope), (kv1.scale, kv2.scale),
                 (keys1.codes, keys2.codes), (keys1.scales, keys2.scales)):
        assert torch.equal(a, c)
    assert not torch.equal(kv1.nope, kv.nope)   # the completing sequences did write entries
    assert torch.equal(out1, out2)
    # the fused call keeps its selection at the start of its workspace: the same top-k
    assert torch.equal(ws1[:B * k * 4].view(torch.int32).view(B, k), sel.view(B, k))
    # and its histograms right after, which it leaves clear; a second call that relies on that
    # (ws_clean) writes the same caches and output with one launch fewer
    h0 = (B * k * 4 + 255) // 256 * 256
    assert not ws1[h0:h0 + B * HIST_COPIES * 4096 * 4].any()
    kv3, keys3 = clone_kv(kv), clone_idx(keys)
    out3 = torch.empty_like(out1)
    v4.v4a_trace_begin(16)
    v4.v4a_decode_step_csa(step_args(kv3, keys3, out3, ws_clean=True), ws1)
    n3 = v4.v4a_trace_end()
    torch.cuda.synchronize()
    assert [name for name, _ in v4.trace_kernels(n3)] == [name for name, _ in kernels][(0 if first != "zero_kernel" else 1):]
    assert torch.equal(out3, out1) and torch.equal(keys3.codes, keys1.codes) and torch.equal(kv3.nope, kv1.nope)
    assert not ws1[h0:h0 + B * HIST_COPIES * 4096 * 4].any()

    # every sequence against the oracle, fed the caches the GPU wrote
    for b in range(B):
        recs = oracle.dequant_kv(kv1.nope[b, :n_ent[b]].cpu().numpy(),
                                 kv1.rope[b, :n_ent[b]].cpu().numpy().view(np.uint16),
                                 kv1.scale[b, :n_ent[b]].cpu().numpy())
        idx = dict(q_codes=qi.codes[b].cpu().numpy(), q_scales=qi.scales[b].cpu().numpy(),
                   w=w[b].cpu().numpy(), k_codes=keys1.codes[b, :n_ent[b]].cpu().numpy(),
                   k_scales=keys1.scales[b, :n_ent[b]].cpu().numpy())
        wins = bf16_bits_to_f64(win[b, :win_len[b]].contiguous().view(torch.int16).cpu().numpy().view(np.uint16))
        ref, ref_sel = oracle.decode_csa(bf16_bits_to_f64(q[b].view(torch.int16).cpu().numpy().view(np.uint16)), recs,
                                         n_ent[b], k, wins, sink.cpu().numpy(), scale, q_pos=q_pos[b], m=m, idx=idx,
                                         R=R, score_bf16=score_bf16)
        assert np.array_equal(sel[b, 0].cpu().numpy(), ref_sel), b
        few = few_key_seqs([int((ref_sel >= 0).sum()) + win_len[b]])
        check_close(out_f64(out1[b]), bf16_round(ref), MAX_ABS_BF16, REL_L2_BF16,
                    what=f"fused step vs oracle, sequence {b}", ulp_seqs="all" if few else ())


def test_fused_step_ring_state_equals_plain_rows():
    """The same step with the per-token state in rings (stream rows at position mod 2m, window
    at position mod W) gives bitwise the output and caches of the plain row layout."""
    seed, m, D, R, H, HI, dI, k, W = 4343, 4, 512, 64, 128, 64, 128, 512, 128
    q_pos = [4003, 4001, 3, 8191, 130]      # entry 1000 / none / entry 0 / entry 2047 / none
    B, cap = len(q_pos), 2304
    n_ent = [(p + 1) // m for p in q_pos]
    win_len = [min(W, p + 1) for p in q_pos]
    win_len[4] = 77                           # a shorter window than the tokens so far
    announce(f"fused decode step, ring state: q_pos={q_pos}")
    kv = v4.KV.empty(B, cap, D, R)
    v4.v4a_quantize_kv(f32(normal(seed, "records", (B * cap, D))), kv, 0)
    keys = v4.Idx.empty(B, cap, dI)
    v4.v4a_quantize_mxfp4(f32(normal(seed, "keys", (B * cap, dI))), keys, 0)
    qi = v4.Idx.empty(B, HI, dI)
    v4.v4a_quantize_mxfp4(f32(normal(seed, "q_idx", (B * HI, dI))), qi)
    w = f32(normal(seed, "w", (B, HI)))
    q = bf16_from_bits(to_bf16_bits(normal(seed, "q", (B, H, D))))
    sink = f32(normal(seed, "sink", (H,)))
    bias = {n: f32(normal(seed, n, (m, 1))) for n in ("bias_a", "bias_b", "idx_bias_a", "idx_bias_b")}
    # token rows by position: row p of each stream, for the positions any step reads
    T = max(q_pos) + 1
    tok = {n: normal(seed, n, (B, T, D if n in ("kv_a", "kv_b") else dI)) for n in ("kv_a", "kv_b", "idx_a", "idx_b")}
    gt = {n: normal(seed, n, (B, T, 1)) for n in ("gate_a", "gate_b", "idx_gate_a", "idx_gate_b")}
    plain, ring = {}, {}
    for n, src in list(tok.items()) + list(gt.items()):
        width = src.shape[-1]
        pl_rows = np.zeros((B, 2 * m, width), np.float32)
        rg_rows = np.zeros((B, 2 * m, width), np.float32)
        for b, t in enumerate(q_pos):
            for r in range(2 * m):
                p = t + 1 - 2 * m + r
                if p >= 0:
                    pl_rows[b, r] = src[b, p]
                    rg_rows[b, p % (2 * m)] = src[b, p]
        conv = bf16_from_bits if n in tok else f32
        plain[n] = conv(to_bf16_bits(pl_rows)) if n in tok else f32(pl_rows)
        ring[n] = conv(to_bf16_bits(rg_rows)) if n in tok else f32(rg_rows)
    win_plain = np.zeros((B, W, D), np.float32)
    win_ring = np.zeros((B, W, D), np.float32)
    for b, t in enumerate(q_pos):
        for j in range(win_len[b]):
            p = t - win_len[b] + 1 + j
            win_plain[b, j] = tok["kv_a"][b, p]
            win_ring[b, p % W] = tok["kv_a"][b, p]
    scale = 1.0 / math.sqrt(D)
    results = []
    for rows, win, is_ring in ((plain, win_plain, False), (ring, win_ring, True)):
        kv1, keys1 = clone_kv(kv), clone_idx(keys)
        out = torch.empty((B, H, D), dtype=torch.bfloat16, device="cuda")
        args = v4.DecodeStepArgs(q_pos=q_pos, n_entries=n_ent, m=m, kv_a=rows["kv_a"], kv_b=rows["kv_b"],
                                 gate_a=rows["gate_a"], gate_b=rows["gate_b"], bias_a=bias["bias_a"],
                                 bias_b=bias["bias_b"], idx_a=rows["idx_a"], idx_b=rows["idx_b"],
                                 idx_gate_a=rows["idx_gate_a"], idx_gate_b=rows["idx_gate_b"],
                                 idx_bias_a=bias["idx_bias_a"], idx_bias_b=bias["idx_bias_b"], kv=kv1, keys=keys1,
                                 q_idx=qi, w=w, k=k, q=q, win=bf16_from_bits(to_bf16_bits(win)), win_len=win_len,
                                 W=W, sink=sink, softmax_scale=scale, out=out, ring=is_ring)
        ws = v4.workspace(v4.v4a_decode_step_workspace(args))
        v4.v4a_decode_step_csa(args, ws)
        torch.cuda.synchronize()
        results.append((out, kv1, keys1))
    (o1, k1, i1), (o2, k2, i2) = results
    for a, c in ((k1.nope, k2.nope), (k1.rope, k2.rope), (k1.scale, k2.scale), (i1.codes, i2.codes),
                 (i1.scales, i2.scales)):
        assert torch.equal(a, c)
    assert not torch.equal(k1.nope, kv.nope)
    assert torch.equal(o1, o2)
    # every sequence of the ring step against the oracle, fed the caches the step wrote and the
    # window tokens by position
    q_bits = q.view(torch.int16).cpu().numpy().view(np.uint16)
    for b in range(B):
        recs = oracle.dequant_kv(k2.nope[b, :n_ent[b]].cpu().numpy(),
                                 k2.rope[b, :n_ent[b]].cpu().numpy().view(np.uint16), k2.scale[b, :n_ent[b]].cpu().numpy())
        idx = dict(q_codes=qi.codes[b].cpu().numpy(), q_scales=qi.scales[b].cpu().numpy(), w=w[b].cpu().numpy(),
                   k_codes=i2.codes[b, :n_ent[b]].cpu().numpy(), k_scales=i2.scales[b, :n_ent[b]].cpu().numpy())
        t = q_pos[b]
        wins = bf16_bits_to_f64(to_bf16_bits(tok["kv_a"][b, t - win_len[b] + 1:t + 1]))
        ref, ref_sel = oracle.decode_csa(bf16_bits_to_f64(q_bits[b]), recs, n_ent[b], k, wins, sink.cpu().numpy(),
                                         scale, q_pos=t, m=m, idx=idx, R=R)
        few = few_key_seqs([int((ref_sel >= 0).sum()) + win_len[b]])
        check_close(out_f64(o2[b]), bf16_round(ref), MAX_ABS_BF16, REL_L2_BF16, what=f"ring step vs oracle, sequence {b}",
                    ulp_seqs="all" if few else ())


@pytest.mark.parametrize("ring", [False, True], ids=["rows", "ring"])
def test_fused_hca_step_equals_separate_calls(ring):
    """v4a_decode_step_hca against v4a_compress_hca + v4a_decode_hca (bitwise), for sequences that
    complete a 128-token block and one that does not; every sequence also against the oracle."""
    seed, m, D, R, H, W = 4444, 128, 512, 64, 128, 128
    q_pos = [128 * 40 - 1, 128 * 40 + 5, 127, 128 * 64 - 1]   # entry 39 / none / entry 0 / entry 63
    B, cap = len(q_pos), 80
    n_ent = [(p + 1) // m for p in q_pos]
    entry = [(p + 1) // m - 1 if (p + 1) % m == 0 else -1 for p in q_pos]
    win_len = [min(W, p + 1) for p in q_pos]
    announce(f"fused hca decode step: q_pos={q_pos} ring={ring}")
    kv = v4.KV.empty(B, cap, D, R)
    v4.v4a_quantize_kv(f32(normal(seed, "records", (B * cap, D))), kv, 0)
    T = max(q_pos) + 1
    tok = normal(seed, "kv_h", (B, T, D))
    gt = normal(seed, "gate_h", (B, T, 1))
    bias = f32(normal(seed, "bias_h", (m, 1)))
    rows = np.zeros((B, m, D), np.float32)
    grows = np.zeros((B, m, 1), np.float32)
    win = np.zeros((B, W, D), np.float32)
    for b, t in enumerate(q_pos):
        for r in range(m):
            p = t + 1 - m + r
            if p >= 0:
                rr = p % m if ring else r
                rows[b, rr], grows[b, rr] = tok[b, p], gt[b, p]
        for j in range(win_len[b]):
            p = t - win_len[b] + 1 + j
            win[b, p % W if ring else j] = tok[b, p]
    rows_dev, win_dev = bf16_from_bits(to_bf16_bits(rows)), bf16_from_bits(to_bf16_bits(win))
    q = bf16_from_bits(to_bf16_bits(normal(seed, "q", (B, H, D))))
    sink = f32(normal(seed, "sink", (H,)))
    scale = 1.0 / math.sqrt(D)

    kv1 = clone_kv(kv)
    out1 = torch.empty((B, H, D), dtype=torch.bfloat16, device="cuda")
    args = v4.DecodeStepHcaArgs(q_pos=q_pos, n_entries=n_ent, m=m, kv_a=rows_dev, gate_a=f32(grows), bias_a=bias,
                                kv=kv1, q=q, win=win_dev, win_len=win_len, W=W, sink=sink, softmax_scale=scale,
                                out=out1, ring=ring)
    ws1 = v4.workspace(v4.v4a_decode_step_hca_workspace(args))
    v4.v4a_decode_step_hca(args, ws1)

    # the separate calls on the plain layout
    kv2 = clone_kv(kv)
    for b, i in enumerate(entry):
        if i < 0:
            continue
        blk = bf16_from_bits(to_bf16_bits(tok[b, m * i:m * i + m]))
        v4.v4a_compress_hca(blk, f32(gt[b, m * i:m * i + m]), bias, tok0=m * i, m=m, first_entry=i, n_entries=1,
                            out_kv=kv2, b=b)
    win_plain = np.zeros((B, W, D), np.float32)
    for b, t in enumerate(q_pos):
        win_plain[b, :win_len[b]] = tok[b, t - win_len[b] + 1:t + 1]
    wp = bf16_from_bits(to_bf16_bits(win_plain))
    out2 = torch.empty((B, H, D), dtype=torch.bfloat16, device="cuda")
    ws2 = v4.workspace(v4.v4a_decode_workspace(B, H, D, cap, W))
    v4.v4a_decode_hca(q, kv2, n_ent, m, wp, win_len, W, sink, q_pos, softmax_scale=scale, out=out2, ws=ws2)
    torch.cuda.synchronize()
    for a, c in ((kv1.nope, kv2.nope), (kv1.rope, kv2.rope), (kv1.scale, kv2.scale)):
        assert torch.equal(a, c)
    assert not torch.equal(kv1.nope, kv.nope)
    assert torch.equal(out1, out2)

    for b in range(B):
        recs = oracle.dequant_kv(kv1.nope[b, :n_ent[b]].cpu().numpy(),
                                 kv1.rope[b, :n_ent[b]].cpu().numpy().view(np.uint16),
                                 kv1.scale[b, :n_ent[b]].cpu().numpy())
        ref = oracle.decode_hca(bf16_bits_to_f64(q[b].view(torch.int16).cpu().numpy().view(np.uint16)), recs, n_ent[b],
                                bf16_bits_to_f64(wp[b, :win_len[b]].view(torch.int16).cpu().numpy().view(np.uint16)),
                                sink.cpu().numpy(), scale, q_pos=q_pos[b], m=m, R=R)
        few = few_key_seqs([oracle.visible_entries(n_ent[b], m, q_pos[b]) + win_len[b]])
        check_close(out_f64(out1[b]), bf16_round(ref), MAX_ABS_BF16, REL_L2_BF16,
                    what=f"fused hca step vs oracle, sequence {b}", ulp_seqs="all" if few else ())



def test_fused_step_query_prologue():
    """The fused CSA step with the query prologue (RMSNorm + RoPE of projected queries) against
    the oracle fed the oracle's own prologue of the same queries, on every sequence."""
    seed, m, D, R, H, HI, dI, k, W = 4545, 4, 512, 64, 128, 64, 128, 512, 128
    q_pos = [4003, 2001, 8191]
    B, cap = len(q_pos), 2304
    n_ent = [(p + 1) // m for p in q_pos]
    announce(f"fused decode step with query prologue: q_pos={q_pos}")
    kv = v4.KV.empty(B, cap, D, R)
    v4.v4a_quantize_kv(f32(normal(seed, "records", (B * cap, D))), kv, 0)
    keys = v4.Idx.empty(B, cap, dI)
    v4.v4a_quantize_mxfp4(f32(normal(seed, "keys", (B * cap, dI))), keys, 0)
    qi = v4.Idx.empty(B, HI, dI)
    v4.v4a_quantize_mxfp4(f32(normal(seed, "q_idx", (B * HI, dI))), qi)
    rows = {n: bf16_from_bits(to_bf16_bits(normal(seed, n, (B, 2 * m, D if n.startswith("kv") else dI))))
            for n in ("kv_a", "kv_b", "idx_a", "idx_b")}
    gates = {n: f32(normal(seed, n, (B, 2 * m, 1))) for n in ("gate_a", "gate_b", "idx_gate_a", "idx_gate_b")}
    bias = {n: f32(normal(seed, n, (m, 1))) for n in ("bias_a", "bias_b", "idx_bias_a", "idx_bias_b")}
    w = f32(normal(seed, "w", (B, HI)))
    q_bits = to_bf16_bits(2.0 * normal(seed, "q", (B, H, D)))
    win_bits = to_bf16_bits(normal(seed, "window", (B, W, D)))
    win_len = [W] * B
    sink = normal(seed, "sink", (H,))
    qw = (0.5 + np.random.default_rng(seed).random(D)).astype(np.float32)
    scale = 1.0 / math.sqrt(D)
    out = torch.empty((B, H, D), dtype=torch.bfloat16, device="cuda")
    args = v4.DecodeStepArgs(q_pos=q_pos, n_entries=n_ent, m=m, kv_a=rows["kv_a"], kv_b=rows["kv_b"],
                             gate_a=gates["gate_a"], gate_b=gates["gate_b"], bias_a=bias["bias_a"],
                             bias_b=bias["bias_b"], idx_a=rows["idx_a"], idx_b=rows["idx_b"],
                             idx_gate_a=gates["idx_gate_a"], idx_gate_b=gates["idx_gate_b"],
                             idx_bias_a=bias["idx_bias_a"], idx_bias_b=bias["idx_bias_b"], kv=kv, keys=keys,
                             q_idx=qi, w=w, k=k, q=bf16_from_bits(q_bits), win=bf16_from_bits(win_bits),
                             win_len=win_len, W=W, sink=f32(sink), softmax_scale=scale, out=out, q_norm_w=f32(qw))
    ws = v4.workspace(v4.v4a_decode_step_workspace(args))
    v4.v4a_decode_step_csa(args, ws)
    torch.cuda.synchronize()
    for b in range(B):
        recs = oracle.dequant_kv(kv.nope[b, :n_ent[b]].cpu().numpy(),
                                 kv.rope[b, :n_ent[b]].cpu().numpy().view(np.uint16), kv.scale[b, :n_ent[b]].cpu().numpy())
        idx = dict(q_codes=qi.codes[b].cpu().numpy(), q_scales=qi.scales[b].cpu().numpy(), w=w[b].cpu().numpy(),
                   k_codes=keys.codes[b, :n_ent[b]].cpu().numpy(), k_scales=keys.scales[b, :n_ent[b]].cpu().numpy())
        qp = bf16_bits_to_f64(oracle.query_prologue(q_bits[b], qw, pos=q_pos[b], R=R))
        ref, _ = oracle.decode_csa(qp, recs, n_ent[b], k, bf16_bits_to_f64(win_bits[b]), sink, scale, q_pos=q_pos[b],
                                   m=m, idx=idx, R=R)
        check_close(out_f64(out[b]), bf16_round(ref), MAX_ABS_BF16, REL_L2_BF16, what=f"query prologue, sequence {b}")
