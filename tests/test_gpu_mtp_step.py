"""GPU check of the multi-token decode steps (v4a_decode_step_csa / v4a_decode_step_hca with Q = 2
and 3 new tokens per sequence; "DeepSeek-V4 technical report walkthrough" (cyqw.cn), section 2
and section 4.2: multi-token prediction with depth 1).

For a batch whose sequences place the step's tokens differently against a block end (the block
completed by the last token, by an earlier one, by none, and the first block of a sequence), in
both the plain and the ring state layouts:
  - the caches and every query's output are bitwise those of Q one-token steps taken in order
    (each token's step on its own window, with the entry of an earlier token already written);
  - every query's selection and output match the oracle's multi-token step (decode_tokens) fed
    the caches the GPU wrote: selections exact, outputs within the BF16 bar.
"""
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


def clone_kv(kv):
    return v4.KV(kv.fmt, kv.D, kv.R, kv.nope.clone(), kv.rope.clone(), kv.scale.clone(), kv.cap)


def clone_idx(ix):
    return v4.Idx(ix.fmt, ix.d, ix.codes.clone(), ix.scales.clone(), ix.cap)


def stream_rows(src, q_pos, Q, m, rows, ring):
    """Per-sequence stream rows of one step: the plain layout holds the B-block and the block
    completed by a token of the step (block-aligned, rows blocks of m), zeros when none
    completes; a ring holds position p at row p mod rows."""
    B, _, width = src.shape
    out = np.zeros((B, rows, width), np.float32)
    for b, t in enumerate(q_pos):
        if ring:
            for p in range(max(0, t - rows + 1), t + 1):
                out[b, p % rows] = src[b, p]
        else:
            done = [tj for tj in range(t - Q + 1, t + 1) if (tj + 1) % m == 0]
            if done:
                first = done[0] + 1 - rows  # the block's start minus the blocks before it
                for r in range(rows):
                    if first + r >= 0:
                        out[b, r] = src[b, first + r]
    return out


def window_rows(src, q_pos, Q, W, win_len, ring):
    """The window buffer of a step: W + Q - 1 rows per sequence (W when Q = 1)."""
    B, _, D = src.shape
    rows = W + Q - 1
    out = np.zeros((B, rows, D), np.float32)
    for b, t in enumerate(q_pos):
        lo = max(0, t - win_len[b] - Q + 2)
        for p in range(lo, t + 1):
            out[b, p % rows if ring else p - lo] = src[b, p]
    return out


CSA_POS = [4 * 1000 - 1, 4 * 1000, 4 * 1000 + 2, 1, 4]   # last token / first token / none / none / entry 0


@pytest.mark.parametrize("Q,ring", [(2, False), (2, True), (3, False)], ids=["q2_rows", "q2_ring", "q3_rows"])
def test_csa_multi_token_step(Q, ring):
    seed, m, D, R, H, HI, dI, k, W = 5151 + Q, 4, 512, 64, 128, 64, 128, 512, 128
    # Q = 3: the block completed by the last, the first, the middle token, none, entry 0
    q_pos = CSA_POS if Q == 2 else [4 * 1000 - 1, 4 * 1000 + 1, 4 * 1000, 2, 5]
    B, cap = len(q_pos), 1024
    T = max(q_pos) + 1
    announce(f"csa multi-token step Q={Q} ring={ring} q_pos={q_pos}")
    n_after = [(t + 1) // m for t in q_pos]
    kv = v4.KV.empty(B, cap, D, R)
    v4.v4a_quantize_kv(f32(normal(seed, "records", (B * cap, D), threads=16)), kv, 0)
    keys = v4.Idx.empty(B, cap, dI)
    v4.v4a_quantize_mxfp4(f32(normal(seed, "keys", (B * cap, dI), threads=16)), keys, 0)
    qi = v4.Idx.empty(B, Q * HI, dI)
    v4.v4a_quantize_mxfp4(f32(normal(seed, "q_idx", (B * Q * HI, dI))), qi)
    w = f32(normal(seed, "w", (B, Q, HI)))
    q = bf16_from_bits(to_bf16_bits(normal(seed, "q", (B, Q, H, D))))
    sink = f32(normal(seed, "sink", (H,)))
    bias = {n: f32(normal(seed, n, (m, 1))) for n in ("bias_a", "bias_b", "idx_bias_a", "idx_bias_b")}
    tok = {n: normal(seed, n, (B, T, D if n in ("kv_a", "kv_b") else dI)) for n in ("kv_a", "kv_b", "idx_a", "idx_b")}
    gt = {n: normal(seed, n, (B, T, 1)) for n in ("gate_a", "gate_b", "idx_gate_a", "idx_gate_b")}
    # the token rows as the step reads them (BF16 streams, fp32 gates)
    tok = {n: bf16_bits_to_f64(to_bf16_bits(v)).astype(np.float32) for n, v in tok.items()}
    win_len = [W] * B
    scale = 1.0 / math.sqrt(D)

    def step(qp, Qs, j0, kv_, keys_, ring_, out_):
        rows = 2 * m + (Qs - 1 if ring_ else 0)
        dev = {n: (bf16_from_bits(to_bf16_bits(stream_rows(src, qp, Qs, m, rows, ring_))) if n in tok
                   else f32(stream_rows(src, qp, Qs, m, rows, ring_))) for n, src in list(tok.items()) + list(gt.items())}
        wl = win_len if Qs > 1 else [min(W, t + 1) for t in qp]
        win = bf16_from_bits(to_bf16_bits(window_rows(tok["kv_a"], qp, Qs, W, wl, ring_)))
        qq = q[:, j0:j0 + Qs].contiguous() if Qs > 1 else q[:, j0].contiguous()
        qix = v4.Idx(qi.fmt, dI, qi.codes[:, j0 * HI:(j0 + Qs) * HI].contiguous(),
                     qi.scales[:, j0 * HI:(j0 + Qs) * HI].contiguous(), Qs * HI)
        args = v4.DecodeStepArgs(q_pos=qp, n_entries=[(t + 1) // m for t in qp], m=m, kv=kv_, keys=keys_, q_idx=qix,
                                 w=w[:, j0:j0 + Qs].contiguous(), k=k, q=qq, win=win, win_len=wl, W=W, sink=sink,
                                 softmax_scale=scale, out=out_, ring=ring_, Q=Qs, **dev, **bias)
        ws = v4.workspace(v4.v4a_decode_step_workspace(args))
        v4.v4a_decode_step_csa(args, ws)
        torch.cuda.synchronize()
        return ws

    kv1, keys1 = clone_kv(kv), clone_idx(keys)
    out1 = torch.empty((B, Q, H, D), dtype=torch.bfloat16, device="cuda")
    ws1 = step(q_pos, Q, 0, kv1, keys1, ring, out1)
    sel1 = ws1[:B * Q * k * 4].view(torch.int32).view(B, Q, k).cpu().numpy()  # the step's selections head its workspace

    # Q one-token steps in order, on copies of the caches
    kv2, keys2 = clone_kv(kv), clone_idx(keys)
    out2 = torch.empty((B, Q, H, D), dtype=torch.bfloat16, device="cuda")
    for j in range(Q):
        announce(f"csa one-token step {j} of {Q}")
        o = torch.empty((B, H, D), dtype=torch.bfloat16, device="cuda")
        step([t - Q + 1 + j for t in q_pos], 1, j, kv2, keys2, False, o)
        out2[:, j] = o
    for a, c in ((kv1.nope, kv2.nope), (kv1.rope, kv2.rope), (kv1.scale, kv2.scale), (keys1.codes, keys2.codes),
                 (keys1.scales, keys2.scales)):
        assert torch.equal(a, c)
    assert not torch.equal(kv1.nope, kv.nope)
    assert torch.equal(out1, out2)

    # every query against the oracle's multi-token step, fed the caches the GPU wrote
    q_bits = q.view(torch.int16).cpu().numpy().view(np.uint16)
    qc = qi.codes.cpu().numpy().reshape(B, Q, HI, dI // 2)
    qs = qi.scales.cpu().numpy().reshape(B, Q, HI, dI // 32)
    wn = w.cpu().numpy()
    for b in range(B):
        n = n_after[b]
        recs = oracle.dequant_kv(kv1.nope[b, :n].cpu().numpy(), kv1.rope[b, :n].cpu().numpy().view(np.uint16),
                                 kv1.scale[b, :n].cpu().numpy())
        idx = dict(q_codes=qc[b], q_scales=qs[b], w=wn[b], k_codes=keys1.codes[b, :n].cpu().numpy(),
                   k_scales=keys1.scales[b, :n].cpu().numpy())
        ref, ref_sel = oracle.decode_tokens("csa", bf16_bits_to_f64(q_bits[b]), recs, n, tok["kv_a"][b].astype(np.float64),
                                            t_last=q_pos[b], Q=Q, win_len=W, sink=sink.cpu().numpy(), scale=scale, m=m,
                                            k=k, idx=idx, R=R)
        assert np.array_equal(sel1[b], ref_sel), b
        n_keys = [int((ref_sel[j] >= 0).sum()) + min(W, q_pos[b] - Q + 2 + j) for j in range(Q)]
        check_close(out_f64(out1[b]), bf16_round(ref), MAX_ABS_BF16, REL_L2_BF16,
                    what=f"csa multi-token step vs oracle, sequence {b}", ulp_seqs=few_key_seqs(n_keys))


HCA_POS = [128 * 40 - 1, 128 * 40, 128 * 40 + 5, 1, 128]


@pytest.mark.parametrize("Q,ring", [(2, False), (2, True)], ids=["q2_rows", "q2_ring"])
def test_hca_multi_token_step(Q, ring):
    seed, m, D, R, H, W = 5252, 128, 512, 64, 128, 128
    q_pos = HCA_POS
    B, cap = len(q_pos), 48
    T = max(q_pos) + 1
    announce(f"hca multi-token step Q={Q} ring={ring} q_pos={q_pos}")
    kv = v4.KV.empty(B, cap, D, R)
    v4.v4a_quantize_kv(f32(normal(seed, "records", (B * cap, D))), kv, 0)
    tokv = bf16_bits_to_f64(to_bf16_bits(normal(seed, "kv_h", (B, T, D)))).astype(np.float32)
    gt = normal(seed, "gate_h", (B, T, 1))
    bias = f32(normal(seed, "bias_h", (m, 1)))
    q = bf16_from_bits(to_bf16_bits(normal(seed, "q", (B, Q, H, D))))
    sink = f32(normal(seed, "sink", (H,)))
    scale = 1.0 / math.sqrt(D)

    def step(qp, Qs, j0, kv_, ring_, out_):
        rows = m + (Qs - 1 if ring_ else 0)
        wl = [W] * B if Qs > 1 else [min(W, t + 1) for t in qp]
        args = v4.DecodeStepHcaArgs(q_pos=qp, n_entries=[(t + 1) // m for t in qp], m=m,
                                    kv_a=bf16_from_bits(to_bf16_bits(stream_rows(tokv, qp, Qs, m, rows, ring_))),
                                    gate_a=f32(stream_rows(gt, qp, Qs, m, rows, ring_)), bias_a=bias, kv=kv_,
                                    q=q[:, j0:j0 + Qs].contiguous() if Qs > 1 else q[:, j0].contiguous(),
                                    win=bf16_from_bits(to_bf16_bits(window_rows(tokv, qp, Qs, W, wl, ring_))),
                                    win_len=wl, W=W, sink=sink, softmax_scale=scale, out=out_, ring=ring_, Q=Qs)
        ws = v4.workspace(v4.v4a_decode_step_hca_workspace(args))
        v4.v4a_decode_step_hca(args, ws)
        torch.cuda.synchronize()

    kv1 = clone_kv(kv)
    out1 = torch.empty((B, Q, H, D), dtype=torch.bfloat16, device="cuda")
    step(q_pos, Q, 0, kv1, ring, out1)
    kv2 = clone_kv(kv)
    out2 = torch.empty((B, Q, H, D), dtype=torch.bfloat16, device="cuda")
    for j in range(Q):
        o = torch.empty((B, H, D), dtype=torch.bfloat16, device="cuda")
        step([t - Q + 1 + j for t in q_pos], 1, j, kv2, False, o)
        out2[:, j] = o
    for a, c in ((kv1.nope, kv2.nope), (kv1.rope, kv2.rope), (kv1.scale, kv2.scale)):
        assert torch.equal(a, c)
    assert not torch.equal(kv1.nope, kv.nope)
    assert torch.equal(out1, out2)

    q_bits = q.view(torch.int16).cpu().numpy().view(np.uint16)
    for b in range(B):
        n = (q_pos[b] + 1) // m
        recs = oracle.dequant_kv(kv1.nope[b, :n].cpu().numpy(), kv1.rope[b, :n].cpu().numpy().view(np.uint16),
                                 kv1.scale[b, :n].cpu().numpy())
        ref, _ = oracle.decode_tokens("hca", bf16_bits_to_f64(q_bits[b]), recs, n, tokv[b].astype(np.float64),
                                      t_last=q_pos[b], Q=Q, win_len=W, sink=sink.cpu().numpy(), scale=scale, m=m, R=R)
        n_keys = [oracle.visible_entries(n, m, q_pos[b] - Q + 1 + j) + min(W, q_pos[b] - Q + 2 + j) for j in range(Q)]
        check_close(out_f64(out1[b]), bf16_round(ref), MAX_ABS_BF16, REL_L2_BF16,
                    what=f"hca multi-token step vs oracle, sequence {b}", ulp_seqs=few_key_seqs(n_keys))
