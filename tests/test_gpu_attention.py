"""GPU parity of the shared-KV MQA with window and sink (a6) and the split combine with the
output's inverse RoPE (a7), against the oracle's double-precision attention.

Bars: max-abs 1e-2 and relative L2 5e-3 for FP8/BF16 records with BF16 queries, window and
outputs; max-abs 1e-5 for fp32 records, queries and outputs.  Cases: the fp32 tiny workload
(CSA gather and HCA dense), several head counts, both head dims, ragged entry counts, window
lengths and query positions, -1 padding in the top-k list, sink extremes, empty key sets,
determinism, batch invariance, and the full 1M-context HCA decode (B=16, 8192 entries,
128 heads) in the launch configuration the benchmark times."""
import numpy as np
import pytest
import torch

import compressed_sparse_attention_02_amd as v4
import oracle
from gpu_util import (MAX_ABS_BF16, MAX_ABS_F32, REL_L2_BF16, announce, bf16_from_bits, bf16_round, check_close,
                      f32, few_key_seqs, kv_from_f32, out_f64)
from workloads import HCA_1M, TINY, bf16_bits_to_f64, normal, to_bf16_bits

pytestmark = pytest.mark.gpu


def make_inputs(seed, B, N, H, D, W, bf16=True):
    rec = normal(seed, "records", (B, N, D), threads=16)
    q = normal(seed, "q", (B, H, D))
    win = normal(seed, "window", (B, W, D))
    sink = normal(seed, "sink", (H,))
    if bf16:
        qb, wb = to_bf16_bits(q), to_bf16_bits(win)
        return rec, qb, wb, sink
    return rec, q, win, sink


def oracle_records(rec_f32, R, fmt):
    """float64 values of the records as stored (FP8/BF16 via the oracle's encoder)."""
    if fmt == v4.V4A_KV_F32:
        return rec_f32.astype(np.float64)
    B, N, D = rec_f32.shape
    out = np.empty((B, N, D))
    for b in range(B):
        out[b] = oracle.dequant_kv(*oracle.quant_kv(rec_f32[b], R))
    return out


def run_decode(kind, rec, q, win, sink, *, R, n_entries=None, topk=None, k=0, win_len=None,
               q_pos, m=128, fmt=v4.V4A_KV_FP8_BF16, bf16=True, scale=None, rope_inv=True):
    B, N, D = rec.shape
    H = q.shape[1]
    W = win.shape[1]
    kv = kv_from_f32(rec, R, fmt)
    qt = bf16_from_bits(q) if bf16 else f32(q)
    wt = bf16_from_bits(win) if bf16 else f32(win)
    out = torch.empty((B, H, D), dtype=torch.bfloat16 if bf16 else torch.float32, device="cuda")
    win_len = [W] * B if win_len is None else win_len
    scale = 1.0 / np.sqrt(D) if scale is None else scale
    n_keys_max = (k if kind == "csa" else N) + W
    ws = v4.workspace(v4.v4a_decode_workspace(B, H, D, n_keys_max - W, W))
    if kind == "csa":
        v4.v4a_decode_csa(qt, kv, torch.from_numpy(np.ascontiguousarray(topk, np.int32)).cuda(), k, wt, win_len,
                          W, f32(sink), q_pos, softmax_scale=scale, out_rope_inverse=rope_inv, out=out, ws=ws)
    else:
        v4.v4a_decode_hca(qt, kv, n_entries, m, wt, win_len, W, f32(sink), q_pos, softmax_scale=scale,
                          out_rope_inverse=rope_inv, out=out, ws=ws)
    torch.cuda.synchronize()
    return out_f64(out)


def oracle_decode(kind, rec64, q, win, sink, *, R, n_entries=None, topk=None, win_len=None, q_pos, m=128,
                  bf16=True, scale=None, rope_inv=True):
    B, N, D = rec64.shape
    W = win.shape[1]
    win_len = [W] * B if win_len is None else win_len
    qd = bf16_bits_to_f64(q) if bf16 else q.astype(np.float64)
    wd = bf16_bits_to_f64(win) if bf16 else win.astype(np.float64)
    scale = 1.0 / np.sqrt(D) if scale is None else scale
    outs = []
    for b in range(B):
        if kind == "csa":
            sel = topk[b][topk[b] >= 0]
            ents = rec64[b][sel]
        else:
            ents = rec64[b][:oracle.visible_entries(n_entries[b], m, q_pos[b])]
        outs.append(oracle.attend(qd[b], ents, wd[b, :win_len[b]], sink, scale, rope_inverse=rope_inv, R=R,
                                  t_q=q_pos[b]))
    out = np.stack(outs)
    return bf16_round(out) if bf16 else out


def sorted_topk(g, n, k, n_valid):
    idx = np.sort(g.choice(n, size=n_valid, replace=False)).astype(np.int32)
    return np.concatenate([idx, -np.ones(k - n_valid, np.int32)])


def test_tiny_f32_csa_and_hca():
    w = TINY
    rec_c = normal(w.seed, "misc0", (1, w.n_csa, w.D))
    rec_h = normal(w.seed, "misc1", (1, w.n_hca, w.D))
    q = normal(w.seed, "q", (1, w.H, w.D))
    win = normal(w.seed, "window", (1, w.W, w.D))
    sink = np.zeros(w.H, np.float32)
    g = np.random.default_rng(w.seed)
    topk = sorted_topk(g, w.n_csa, w.k, w.k)[None]
    announce("tiny fp32 csa")
    got = run_decode("csa", rec_c, q, win, sink, R=w.R, topk=topk, k=w.k, q_pos=[w.T - 1],
                     fmt=v4.V4A_KV_F32, bf16=False)
    ref = oracle_decode("csa", rec_c.astype(np.float64), q, win, sink, R=w.R, topk=topk, q_pos=[w.T - 1],
                        bf16=False)
    check_close(got, ref, MAX_ABS_F32, what="tiny csa f32")
    announce("tiny fp32 hca")
    got = run_decode("hca", rec_h, q, win, sink, R=w.R, n_entries=[w.n_hca], q_pos=[w.T - 1],
                     fmt=v4.V4A_KV_F32, bf16=False)
    ref = oracle_decode("hca", rec_h.astype(np.float64), q, win, sink, R=w.R, n_entries=[w.n_hca],
                        q_pos=[w.T - 1], bf16=False)
    check_close(got, ref, MAX_ABS_F32, what="tiny hca f32")


MFMA_CASES = {
    # name: (kind, B, N, H, D, R, W, k, win_len, n_entries or n_valid, q_pos)
    "hca_h128_ragged": ("hca", 3, 1000, 128, 512, 64, 128, 0, [128, 50, 0], [1000, 700, 3], [128 * 1000 - 1, 128 * 650 + 5, 1000]),
    "hca_h64": ("hca", 2, 700, 64, 512, 64, 128, 0, [128, 128], [700, 700], [128 * 700 - 1] * 2),
    "hca_h16": ("hca", 2, 300, 16, 512, 64, 77, 0, [77, 10], [300, 300], [128 * 300 - 1] * 2),
    "hca_h48": ("hca", 1, 513, 48, 512, 64, 128, 0, [128], [513], [128 * 513 - 1]),
    "hca_h80": ("hca", 1, 400, 80, 512, 64, 128, 0, [128], [400], [128 * 400 - 1]),
    "hca_d128": ("hca", 2, 900, 32, 128, 32, 128, 0, [128, 128], [900, 900], [128 * 900 - 1] * 2),
    "csa_h128_pad": ("csa", 3, 5000, 128, 512, 64, 128, 1024, [128, 128, 31], [1024, 600, 0], [4 * 5000 - 1] * 3),
    "csa_h64_k512": ("csa", 2, 3000, 64, 512, 64, 128, 512, [128, 128], [512, 512], [4 * 3000 - 1] * 2),
    "empty_keys": ("hca", 1, 10, 64, 512, 64, 128, 0, [0], [10], [50]),
}


@pytest.mark.parametrize("name", list(MFMA_CASES))
def test_mfma_decode(name):
    kind, B, N, H, D, R, W, k, win_len, ne, q_pos = MFMA_CASES[name]
    seed = 400 + list(MFMA_CASES).index(name)
    rec, q, win, sink = make_inputs(seed, B, N, H, D, W)
    rec64 = oracle_records(rec, R, v4.V4A_KV_FP8_BF16)
    announce(f"mfma decode {name}")
    if kind == "csa":
        g = np.random.default_rng(seed)
        topk = np.stack([sorted_topk(g, N, k, ne[b]) for b in range(B)])
        got = run_decode("csa", rec, q, win, sink, R=R, topk=topk, k=k, win_len=win_len, q_pos=q_pos)
        ref = oracle_decode("csa", rec64, q, win, sink, R=R, topk=topk, win_len=win_len, q_pos=q_pos)
    else:
        got = run_decode("hca", rec, q, win, sink, R=R, n_entries=ne, win_len=win_len, q_pos=q_pos)
        ref = oracle_decode("hca", rec64, q, win, sink, R=R, n_entries=ne, win_len=win_len, q_pos=q_pos)
    # Only sequences attending over a handful of keys (few_key_seqs) may differ by one BF16
    # spacing of the reference; every other sequence keeps the plain bar.
    if kind == "csa":
        n_keys = [ne[b] + win_len[b] for b in range(B)]
    else:
        n_keys = [oracle.visible_entries(ne[b], 128, q_pos[b]) + win_len[b] for b in range(B)]
    check_close(got, ref, MAX_ABS_BF16, REL_L2_BF16, what=name, ulp_seqs=few_key_seqs(n_keys))


def test_sink_extremes():
    B, N, H, D, R, W = 1, 600, 64, 512, 64, 128
    rec, q, win, _ = make_inputs(450, B, N, H, D, W)
    rec64 = oracle_records(rec, R, v4.V4A_KV_FP8_BF16)
    for sv in (-60.0, 0.0, 60.0):
        sink = np.full(H, sv, np.float32)
        announce(f"sink {sv}")
        got = run_decode("hca", rec, q, win, sink, R=R, n_entries=[N], q_pos=[128 * N - 1])
        ref = oracle_decode("hca", rec64, q, win, sink, R=R, n_entries=[N], q_pos=[128 * N - 1])
        check_close(got, ref, MAX_ABS_BF16, REL_L2_BF16 if sv < 60 else None, what=f"sink {sv}")


def test_determinism_and_batch_invariance():
    B, N, H, D, R, W = 4, 2500, 128, 512, 64, 128
    rec, q, win, sink = make_inputs(460, B, N, H, D, W)
    ne = [2500, 1200, 2500, 40]
    q_pos = [128 * 2500 - 1, 128 * 1200 - 1, 128 * 2000 + 7, 128 * 40 - 1]
    announce("determinism / batch invariance")
    a = run_decode("hca", rec, q, win, sink, R=R, n_entries=ne, q_pos=q_pos)
    b = run_decode("hca", rec, q, win, sink, R=R, n_entries=ne, q_pos=q_pos)
    assert np.array_equal(a, b)
    for s in (0, 2, 3):
        one = run_decode("hca", rec[s:s + 1], q[s:s + 1], win[s:s + 1], sink, R=R, n_entries=[ne[s]],
                         q_pos=[q_pos[s]])
        assert np.array_equal(one[0], a[s]), s


def test_hca_1m_full_size():
    """The 1M-context HCA decode workload at full size: 16 sequences x 8192 entries x 128
    heads, every output element checked."""
    w = HCA_1M
    rec, q, win, sink = make_inputs(w.seed, w.B, w.n_hca, w.H, w.D, w.W)
    announce("hca 1M full size")
    q_pos = [w.T - 1] * w.B
    got = run_decode("hca", rec, q, win, sink, R=w.R, n_entries=[w.n_hca] * w.B, q_pos=q_pos)
    rec64 = oracle_records(rec, w.R, v4.V4A_KV_FP8_BF16)
    ref = oracle_decode("hca", rec64, q, win, sink, R=w.R, n_entries=[w.n_hca] * w.B, q_pos=q_pos)
    check_close(got, ref, MAX_ABS_BF16, REL_L2_BF16, what="hca 1M")


# k and window lengths whose key counts k + win_len put the sequences of one batch on both sides
# of the split plan's boundaries: k = 288 gives 10-13 splits of one tile, k = 1024 gives 16-18
# splits of two tiles (one or two combine rounds), k = 1408 gives 22-24.
CSA_SPLIT_MIX = {
    "k288": (288, [32, 128, 0, 77]),
    "k1024": (1024, [0, 31, 128, 64]),
    "k1408": (1408, [0, 64, 128, 100]),
}


@pytest.mark.parametrize("name", list(CSA_SPLIT_MIX))
def test_csa_batch_invariance_across_split_counts(name):
    """CSA decode over a batch whose sequences take different split counts: each sequence is
    bitwise equal to the same sequence decoded alone, and every sequence matches the oracle."""
    k, win_len = CSA_SPLIT_MIX[name]
    B, N, H, D, R, W = len(win_len), 4096, 128, 512, 64, 128
    seed = 470 + list(CSA_SPLIT_MIX).index(name)
    rec, q, win, sink = make_inputs(seed, B, N, H, D, W)
    g = np.random.default_rng(seed)
    n_valid = [k, k - 5, k // 2, k]
    topk = np.stack([sorted_topk(g, N, k, n_valid[b]) for b in range(B)])
    q_pos = [4 * N - 1] * B
    announce(f"csa batch invariance {name}: k={k} win_len={win_len}")
    a = run_decode("csa", rec, q, win, sink, R=R, topk=topk, k=k, win_len=win_len, q_pos=q_pos)
    for s in range(B):
        one = run_decode("csa", rec[s:s + 1], q[s:s + 1], win[s:s + 1], sink, R=R, topk=topk[s:s + 1], k=k,
                         win_len=[win_len[s]], q_pos=[q_pos[s]])
        assert np.array_equal(one[0], a[s]), s
    rec64 = oracle_records(rec, R, v4.V4A_KV_FP8_BF16)
    ref = oracle_decode("csa", rec64, q, win, sink, R=R, topk=topk, win_len=win_len, q_pos=q_pos)
    check_close(a, ref, MAX_ABS_BF16, REL_L2_BF16, what=f"csa split mix {name}")
