"""End-to-end parity of the fp32 tiny workload (4096 tokens): compress CSA records, CSA
indexer keys and HCA records on the GPU, select the top-64 entries with the indexer, run the
CSA and HCA decode steps, and compare with the oracle running every stage itself from the
same raw streams.  Also the CSA decode end to end at the 131072-token and 1M-token sizes
(indexer, top-k and attention on the GPU; scores, top-k and attention in the oracle)."""
import numpy as np
import pytest
import torch

import compressed_sparse_attention_02_amd as v4
import oracle
from gpu_util import (MAX_ABS_BF16, MAX_ABS_F32, REL_L2_BF16, announce, bf16_from_bits, bf16_round, check_close,
                      f32, idx_from_f32, kv_from_f32, out_f64)
from workloads import CSA_FLASH, CSA_PRO_1M, TINY, bf16_bits_to_f64, decode_inputs, tiny_inputs, to_bf16_bits

pytestmark = pytest.mark.gpu


def test_tiny_pipeline():
    w = TINY
    x = tiny_inputs(w)
    T, D, R, dI, H, HI, k, W = w.T, w.D, w.R, w.d_I, w.H, w.H_I, w.k, w.W
    Nc, Nh = w.n_csa, w.n_hca
    announce("tiny pipeline: compress")
    rec_c = v4.KV.empty(1, Nc, D, R, fmt=v4.V4A_KV_F32)
    keys = v4.Idx.empty(1, Nc, dI, fmt=v4.V4A_IDX_F32)
    rec_h = v4.KV.empty(1, Nh, D, R, fmt=v4.V4A_KV_F32)
    v4.v4a_compress_csa(f32(x["kv_a"]), f32(x["kv_b"]), f32(x["gate_a"]), f32(x["gate_b"]), f32(x["bias_a"]),
                        f32(x["bias_b"]), tok0=0, m=4, first_entry=0, n_entries=Nc, out_kv=rec_c)
    v4.v4a_compress_csa(f32(x["idx_a"]), f32(x["idx_b"]), f32(x["idx_gate_a"]), f32(x["idx_gate_b"]),
                        f32(x["idx_bias_a"]), f32(x["idx_bias_b"]), tok0=0, m=4, first_entry=0, n_entries=Nc,
                        out_idx=keys)
    v4.v4a_compress_hca(f32(x["kv_h"]), f32(x["gate_h"]), f32(x["bias_h"]), tok0=0, m=128, first_entry=0,
                        n_entries=Nh, out_kv=rec_h)
    announce("tiny pipeline: indexer + top-k")
    qi = idx_from_f32(x["q_idx"][None], v4.V4A_IDX_F32)
    sel = torch.empty((1, 1, k), dtype=torch.int32, device="cuda")
    ws = v4.workspace(v4.v4a_indexer_topk_workspace(1, 1, Nc, k))
    v4.v4a_indexer_topk(keys, [Nc], 4, qi, f32(x["w"][None]), 1, 1, HI, [T - 1], k, sel, ws)
    announce("tiny pipeline: decode")
    q = f32(x["q"][None])
    win_c = f32(x["kv_a"][T - W:][None])
    win_h = f32(x["kv_h"][T - W:][None])
    out_c = torch.empty((1, H, D), dtype=torch.float32, device="cuda")
    out_h = torch.empty((1, H, D), dtype=torch.float32, device="cuda")
    sink = f32(x["sink"])
    scale = 1.0 / np.sqrt(D)
    v4.v4a_decode_csa(q, rec_c, sel.view(1, k), k, win_c, [W], W, sink, [T - 1], softmax_scale=scale, out=out_c)
    v4.v4a_decode_hca(q, rec_h, [Nh], 128, win_h, [W], W, sink, [T - 1], softmax_scale=scale, out=out_h)
    torch.cuda.synchronize()

    # the oracle, every stage from the raw streams
    ent = oracle.compress_csa(x["kv_a"], x["kv_b"], x["gate_a"], x["gate_b"], x["bias_a"], x["bias_b"], tok0=0,
                              m=4, first_entry=0, n_entries=Nc, apply_rope=True, R=R)
    ikeys = oracle.compress_csa(x["idx_a"], x["idx_b"], x["idx_gate_a"], x["idx_gate_b"], x["idx_bias_a"],
                                x["idx_bias_b"], tok0=0, m=4, first_entry=0, n_entries=Nc, apply_rope=False, R=0)
    hent = oracle.compress_hca(x["kv_h"], x["gate_h"], x["bias_h"], tok0=0, m=128, first_entry=0, n_entries=Nh,
                               apply_rope=True, R=R)
    ref_c, ref_sel = oracle.decode_csa(x["q"], ent.astype(np.float64), Nc, k, x["kv_a"][T - W:].astype(np.float64),
                                       x["sink"], scale, q_pos=T - 1, m=4,
                                       idx={"q": x["q_idx"], "w": x["w"], "keys": ikeys}, R=R)
    ref_h = oracle.decode_hca(x["q"], hent.astype(np.float64), Nh, x["kv_h"][T - W:].astype(np.float64), x["sink"],
                              scale, q_pos=T - 1, m=128, R=R)
    got_sel = sel.cpu().numpy()[0, 0]
    recall = len(np.intersect1d(got_sel, ref_sel)) / k
    print(f"top-k recall {recall:.4f}", flush=True)
    assert recall >= 0.99
    assert np.array_equal(got_sel, ref_sel)   # no near-tie at this seed
    check_close(out_f64(out_c)[0], ref_c, MAX_ABS_F32, what="tiny csa e2e")
    check_close(out_f64(out_h)[0], ref_h, MAX_ABS_F32, what="tiny hca e2e")


@pytest.mark.parametrize("wl", [CSA_FLASH, CSA_PRO_1M], ids=lambda w: w.name)
def test_csa_decode_full_size(wl):
    """Indexer -> top-k -> sparse MQA with window and sink at full size, bf16 outputs."""
    inp = decode_inputs(wl, threads=16)
    N, B, H, D, R, W, k = inp["N"], wl.B, wl.H, wl.D, wl.R, wl.W, wl.k
    announce(f"csa decode full size {wl.name}")
    kv = kv_from_f32(inp["records"], R)
    keys = idx_from_f32(inp["keys"])
    qi = idx_from_f32(inp["q_idx"])
    qb, wb = to_bf16_bits(inp["q"]), to_bf16_bits(inp["window"])
    sel = torch.empty((B, 1, k), dtype=torch.int32, device="cuda")
    ws = v4.workspace(max(v4.v4a_indexer_topk_workspace(B, 1, N, k), v4.v4a_decode_workspace(B, H, D, k, W)))
    q_pos = [wl.T - 1] * B
    v4.v4a_indexer_topk(keys, [N] * B, 4, qi, f32(inp["w"]), B, 1, wl.H_I, q_pos, k, sel, ws)
    out = torch.empty((B, H, D), dtype=torch.bfloat16, device="cuda")
    v4.v4a_decode_csa(bf16_from_bits(qb), kv, sel.view(B, k), k, bf16_from_bits(wb), [W] * B, W, f32(inp["sink"]),
                      q_pos, softmax_scale=1.0 / np.sqrt(D), out=out, ws=ws)
    torch.cuda.synchronize()
    got = out_f64(out)
    gsel = sel.cpu().numpy()[:, 0]
    qd, wd = bf16_bits_to_f64(qb), bf16_bits_to_f64(wb)
    for b in range(B):
        kc, ks = oracle.quant_mxfp4(inp["keys"][b])
        qc, qs = oracle.quant_mxfp4(inp["q_idx"][b])
        s, bad = oracle.indexer_scores_mxfp4(qc, qs, inp["w"][b], kc, ks)
        assert bad == 0
        rsel = oracle.topk(s, k)
        assert np.array_equal(gsel[b], rsel), b
        chosen = rsel[rsel >= 0]
        ents = oracle.dequant_kv(*oracle.quant_kv(inp["records"][b][chosen], R))
        ref = oracle.attend(qd[b], ents, wd[b], inp["sink"], 1.0 / np.sqrt(D), rope_inverse=True, R=R,
                            t_q=wl.T - 1)
        check_close(got[b], bf16_round(ref), MAX_ABS_BF16, REL_L2_BF16, what=f"{wl.name} seq {b}")
