"""GPU parity of the lightning indexer (a4) and the top-k selection (a5).

Scores are compared bit for bit with the oracle (same quantised keys and queries: the HIP
quantiser is itself bit-exact against the oracle's); the top-k index lists must be equal.
Cases: the fp32 tiny workload, ragged key counts and causal visibility, padded head counts,
adversarial ties, k above the visible count, nothing visible, and the full CSA decode sizes
of the 131072-token (B=8, top-512) and 1M-token (B=4, top-1024) workloads in the launch
configuration the benchmark times.  The BF16-score selector (v4a_indexer_topk_bf16) is held to
the same bar against the oracle's selection over the scores rounded to BF16."""
import numpy as np
import pytest
import torch

import compressed_sparse_attention_02_amd as v4
import oracle
from gpu_util import announce, f32, idx_from_f32
from workloads import CSA_FLASH, CSA_PRO_1M, TINY, decode_inputs, normal, scaled

pytestmark = pytest.mark.gpu


def run_topk(keys_f, q_f, w, n_entries, q_pos, k, m=4, fmt=v4.V4A_IDX_MXFP4, Q=1, bf16=False):
    """HIP indexer + top-k (bf16: the BF16-score selector); keys_f [B][N][d], q_f [B][Q*H][d],
    w [B][Q][H]."""
    B, N, d = keys_f.shape
    H = w.shape[-1]
    keys = idx_from_f32(keys_f, fmt)
    qi = idx_from_f32(q_f, fmt)
    wt = f32(w)
    out = torch.full((B, Q, k), -7, dtype=torch.int32, device="cuda")
    n_max = max(min(int(n), (int(p) + 1) // m) for n, p in zip(np.repeat(n_entries, Q), q_pos))
    ws = v4.workspace(v4.v4a_indexer_topk_workspace(B, Q, max(n_max, 0), k))
    call = v4.v4a_indexer_topk_bf16 if bf16 else v4.v4a_indexer_topk
    call(keys, n_entries, m, qi, wt, B, Q, H, q_pos, k, out, ws)
    torch.cuda.synchronize()
    return out.cpu().numpy(), keys, qi


def oracle_topk(keys_f, q_f, w, n_entries, q_pos, k, m=4, fmt=v4.V4A_IDX_MXFP4, Q=1, bf16=False):
    B, N, d = keys_f.shape
    H = w.shape[-1]
    res = np.empty((B, Q, k), np.int32)
    for b in range(B):
        if fmt == v4.V4A_IDX_MXFP4:
            kc, ks = oracle.quant_mxfp4(keys_f[b])
        for j in range(Q):
            n_vis = oracle.visible_entries(int(n_entries[b]), m, int(q_pos[b * Q + j]))
            qrows = q_f[b, j * H:(j + 1) * H]
            if fmt == v4.V4A_IDX_MXFP4:
                qc, qs = oracle.quant_mxfp4(qrows)
                s, bad = oracle.indexer_scores_mxfp4(qc, qs, w[b, j], kc, ks, n_vis)
                assert bad == 0
            else:
                s = oracle.indexer_scores_f32(qrows, w[b, j], keys_f[b], n_vis)
            res[b, j] = oracle.topk(s, k, n_vis, score_bf16=bf16)
    return res


def test_scores_mxfp4_bit_exact():
    B, N, H = 2, 3000, 64
    keys = normal(101, "keys", (B, N, 128))
    q = normal(101, "q_idx", (B, H, 128))
    w = normal(101, "w", (B, 1, H))
    n_entries, q_pos = [N, N], [4 * N - 1, 4 * 1000 + 2]
    announce("indexer scores MXFP4 B=2 N=3000")
    ki, qi = idx_from_f32(keys), idx_from_f32(q)
    out = torch.empty((B, N), dtype=torch.float32, device="cuda")
    v4.v4a_indexer_scores(ki, n_entries, 4, qi, f32(w), B, 1, H, q_pos, N, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    for b in range(B):
        kc, ks = oracle.quant_mxfp4(keys[b])
        qc, qs = oracle.quant_mxfp4(q[b])
        n_vis = oracle.visible_entries(N, 4, q_pos[b])
        ref, bad = oracle.indexer_scores_mxfp4(qc, qs, w[b, 0], kc, ks, n_vis)
        assert bad == 0
        assert np.array_equal(got[b, :n_vis].view(np.uint32), ref.view(np.uint32)), b
        assert np.all(got[b, n_vis:] == -np.inf)


def test_scores_mxfp4_streaming_ragged():
    """A long one-query-per-sequence scan (the streaming scoring kernel: B * n_max >= 256K keys)
    with ragged visible counts that are not multiples of a 64-key batch and one sequence too
    short to reach most workgroups' ranges: every visible score bit-exact, -inf past it."""
    B, N, H = 3, 150000, 64
    keys = normal(105, "keys", (B, N, 128))
    q = normal(105, "q_idx", (B, H, 128))
    w = normal(105, "w", (B, 1, H))
    n_entries = [100003, N, 70001]
    q_pos = [4 * 100003 - 1, 4 * 149985 + 2, 4 * 1000 + 1]  # visible 100003, 149985, 1000
    announce("indexer scores MXFP4 streaming, ragged B=3 N=150000")
    ki, qi = idx_from_f32(keys), idx_from_f32(q)
    out = torch.empty((B, N), dtype=torch.float32, device="cuda")
    v4.v4a_indexer_scores(ki, n_entries, 4, qi, f32(w), B, 1, H, q_pos, N, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    for b in range(B):
        kc, ks = oracle.quant_mxfp4(keys[b, :n_entries[b]])
        qc, qs = oracle.quant_mxfp4(q[b])
        n_vis = oracle.visible_entries(n_entries[b], 4, q_pos[b])
        ref, bad = oracle.indexer_scores_mxfp4(qc, qs, w[b, 0], kc, ks, n_vis)
        assert bad == 0
        assert np.array_equal(got[b, :n_vis].view(np.uint32), ref.view(np.uint32)), b
        assert np.all(got[b, n_vis:] == -np.inf)


@pytest.mark.parametrize("bf16", [False, True], ids=["f32_scores", "bf16_scores"])
def test_topk_streaming_ragged(bf16):
    """The top-k call over the same ragged long scan (streaming scoring kernel, then the
    selection), bit-exact against the oracle for every sequence."""
    B, N, H, k = 3, 150000, 64, 1024
    keys = normal(106, "keys", (B, N, 128))
    q = normal(106, "q_idx", (B, H, 128))
    w = normal(106, "w", (B, 1, H))
    n_entries = np.array([100003, N, 70001])
    q_pos = [4 * 100003 - 1, 4 * 149985 + 2, 4 * 1000 + 1]
    announce(f"topk streaming, ragged B=3 N=150000 bf16={bf16}")
    got, _, _ = run_topk(keys, q, w, n_entries, q_pos, k, bf16=bf16)
    ref = oracle_topk(keys, q, w, n_entries, q_pos, k, bf16=bf16)
    for b in range(B):
        assert np.array_equal(got[b, 0], ref[b, 0]), (b, np.setdiff1d(got[b, 0], ref[b, 0])[:10])


def test_scores_f32_bit_exact():
    w_ = TINY
    N = w_.n_csa
    keys = normal(w_.seed, "misc0", (1, N, w_.d_I))
    q = normal(w_.seed, "q_idx", (1, w_.H_I, w_.d_I))
    w = normal(w_.seed, "w", (1, 1, w_.H_I))
    announce("indexer scores fp32 tiny")
    ki, qi = idx_from_f32(keys, v4.V4A_IDX_F32), idx_from_f32(q, v4.V4A_IDX_F32)
    out = torch.empty((1, N), dtype=torch.float32, device="cuda")
    v4.v4a_indexer_scores(ki, [N], 4, qi, f32(w), 1, 1, w_.H_I, [w_.T - 1], N, out)
    torch.cuda.synchronize()
    ref = oracle.indexer_scores_f32(q[0], w[0, 0], keys[0])
    assert np.array_equal(out.cpu().numpy()[0].view(np.uint32), ref.view(np.uint32))


CASES = {
    # name: (B, N list, H, k, q_pos list or None (decode at the end), fmt, d)
    "tiny_f32": (1, [1024], 4, 64, None, v4.V4A_IDX_F32, 32),
    "ragged_causal": (3, [5000, 3000, 100], 64, 512, [4 * 5000 - 1, 4 * 2000 + 1, 399], v4.V4A_IDX_MXFP4, 128),
    "nothing_visible": (2, [100, 100], 64, 16, [2, 399], v4.V4A_IDX_MXFP4, 128),
    "k_equals_visible": (1, [777], 64, 777, None, v4.V4A_IDX_MXFP4, 128),
    "heads_4": (2, [2500, 2500], 4, 100, None, v4.V4A_IDX_MXFP4, 128),
    "heads_36": (2, [2500, 1500], 36, 300, None, v4.V4A_IDX_MXFP4, 128),
    "k_1": (2, [9000, 17000], 64, 1, None, v4.V4A_IDX_MXFP4, 128),
    "k_2048": (1, [20000], 64, 2048, None, v4.V4A_IDX_MXFP4, 128),
}


@pytest.mark.parametrize("name", list(CASES))
def test_topk_bit_exact(name):
    B, Ns, H, k, q_pos, fmt, d = CASES[name]
    N = max(Ns)
    seed = 200 + list(CASES).index(name)
    keys = normal(seed, "keys", (B, N, d))
    q = normal(seed, "q_idx", (B, H, d))
    w = normal(seed, "w", (B, 1, H))
    if q_pos is None:
        q_pos = [4 * n - 1 for n in Ns]
    announce(f"topk {name}")
    got, _, _ = run_topk(keys, q, w, np.array(Ns), q_pos, k, fmt=fmt)
    ref = oracle_topk(keys, q, w, np.array(Ns), q_pos, k, fmt=fmt)
    for b in range(B):
        assert np.array_equal(got[b, 0], ref[b, 0]), (name, b, np.setdiff1d(got[b, 0], ref[b, 0])[:10])


def test_topk_adversarial_ties():
    """Keys from a handful of distinct vectors make many exactly equal scores: the lowest
    indices must win at the threshold; identical keys everywhere give indices 0..k-1."""
    B, N, H, k = 2, 12000, 64, 700
    g = np.random.default_rng(300)
    base = normal(300, "keys", (5, 128))
    choice = g.integers(0, 5, size=(B, N))
    keys = base[choice]
    keys[1] = base[0]                           # sequence 1: every key identical
    q = normal(300, "q_idx", (B, H, 128))
    w = normal(300, "w", (B, 1, H))
    announce("topk adversarial ties")
    got, _, _ = run_topk(keys, q, w, np.array([N, N]), [4 * N - 1] * 2, k)
    ref = oracle_topk(keys, q, w, np.array([N, N]), [4 * N - 1] * 2, k)
    assert np.array_equal(got, ref)
    assert np.array_equal(got[1, 0], np.arange(k))


def test_topk_small_tie_groups():
    """Keys drawn from 3000 vectors (about four copies each): equal scores come in small
    groups, so the few keys sharing the threshold's first 22 bits (ranked by one wavefront
    instead of a second digit pass) hold repeats, and the lowest indices must win."""
    B, N, H, k = 2, 12000, 64, 700
    g = np.random.default_rng(305)
    base = normal(305, "keys", (3000, 128))
    keys = base[g.integers(0, 3000, size=(B, N))]
    q = normal(305, "q_idx", (B, H, 128))
    w = normal(305, "w", (B, 1, H))
    announce("topk small tie groups")
    for bf16 in (False, True):
        got, _, _ = run_topk(keys, q, w, np.array([N, N]), [4 * N - 1] * 2, k, bf16=bf16)
        ref = oracle_topk(keys, q, w, np.array([N, N]), [4 * N - 1] * 2, k, bf16=bf16)
        assert np.array_equal(got, ref), bf16


def test_topk_list_longer_than_lds():
    """Every key identical: the threshold bin lists all 30000 keys, more than the final
    selection keeps in LDS, so it reads them from the list in global memory."""
    B, N, H, k = 1, 30000, 64, 900
    keys = np.repeat(normal(310, "keys", (1, 1, 128)), N, axis=1)
    q = normal(310, "q_idx", (B, H, 128))
    w = normal(310, "w", (B, 1, H))
    announce("topk list longer than LDS")
    got, _, _ = run_topk(keys, q, w, np.array([N]), [4 * N - 1], k)
    ref = oracle_topk(keys, q, w, np.array([N]), [4 * N - 1], k)
    assert np.array_equal(got, ref)
    assert np.array_equal(got[0, 0], np.arange(k))


def test_topk_more_than_32_slices():
    """270000 keys make 33 slices of 8192: the final selection places the listed keys with
    the slice-offset scan instead of 16 threads per slice."""
    B, N, H, k = 1, 270000, 64, 1024
    keys = normal(311, "keys", (B, N, 128))
    q = normal(311, "q_idx", (B, H, 128))
    w = normal(311, "w", (B, 1, H))
    announce("topk 33 slices")
    got, _, _ = run_topk(keys, q, w, np.array([N]), [4 * N - 1], k)
    ref = oracle_topk(keys, q, w, np.array([N]), [4 * N - 1], k)
    assert np.array_equal(got, ref)


def test_topk_prefill_queries():
    """Several queries per sequence at consecutive positions (the prefill form)."""
    B, N, H, k, Q = 1, 6000, 64, 512, 24
    keys = normal(301, "keys", (B, N, 128))
    q = normal(301, "q_idx", (B, Q * H, 128))
    w = normal(301, "w", (B, Q, H))
    pos0 = 4 * 5000
    q_pos = [pos0 + j for j in range(Q)]
    announce("topk prefill-form queries")
    got, _, _ = run_topk(keys, q, w, np.array([N]), q_pos, k, Q=Q)
    ref = oracle_topk(keys, q, w, np.array([N]), q_pos, k, Q=Q)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("wl", [CSA_FLASH, CSA_PRO_1M], ids=lambda w: w.name)
def test_topk_full_size(wl):
    """Full decode sizes (every key of every sequence scored), checked bit for bit."""
    inp = decode_inputs(wl, threads=16)
    N = inp["N"]
    announce(f"topk full size {wl.name} B={wl.B} N={N} k={wl.k}")
    q_pos = [wl.T - 1] * wl.B
    got, _, _ = run_topk(inp["keys"], inp["q_idx"], inp["w"][:, None, :], np.array([N] * wl.B), q_pos, wl.k)
    ref = oracle_topk(inp["keys"], inp["q_idx"], inp["w"][:, None, :], np.array([N] * wl.B), q_pos, wl.k)
    assert np.array_equal(got, ref)
    # deterministic: a second run gives the same bits
    got2, _, _ = run_topk(inp["keys"], inp["q_idx"], inp["w"][:, None, :], np.array([N] * wl.B), q_pos, wl.k)
    assert np.array_equal(got, got2)


@pytest.mark.parametrize("name", list(CASES))
def test_topk_bf16_bit_exact(name):
    B, Ns, H, k, q_pos, fmt, d = CASES[name]
    N = max(Ns)
    seed = 200 + list(CASES).index(name)
    keys = normal(seed, "keys", (B, N, d))
    q = normal(seed, "q_idx", (B, H, d))
    w = normal(seed, "w", (B, 1, H))
    if q_pos is None:
        q_pos = [4 * n - 1 for n in Ns]
    announce(f"topk bf16 {name}")
    got, _, _ = run_topk(keys, q, w, np.array(Ns), q_pos, k, fmt=fmt, bf16=True)
    ref = oracle_topk(keys, q, w, np.array(Ns), q_pos, k, fmt=fmt, bf16=True)
    for b in range(B):
        assert np.array_equal(got[b, 0], ref[b, 0]), (name, b, np.setdiff1d(got[b, 0], ref[b, 0])[:10])


def test_topk_bf16_rounding_ties():
    """Scores packed into a narrow range, so that BF16 rounding merges many of them: the ties
    it creates at the threshold must go to the lowest indices, and the selection must differ
    from the fp32 one (which separates them)."""
    B, N, H, k = 2, 9000, 64, 600
    keys = normal(302, "keys", (B, N, 128))
    keys[:, :, 64:] = 0.0
    keys += 8.0  # every per-head dot large and positive, the spread small relative to it
    q = np.abs(normal(302, "q_idx", (B, H, 128)))
    w = np.abs(normal(302, "w", (B, 1, H)))
    announce("topk bf16 rounding ties")
    got, _, _ = run_topk(keys, q, w, np.array([N, N]), [4 * N - 1] * 2, k, bf16=True)
    ref = oracle_topk(keys, q, w, np.array([N, N]), [4 * N - 1] * 2, k, bf16=True)
    assert np.array_equal(got, ref)
    f32_ref = oracle_topk(keys, q, w, np.array([N, N]), [4 * N - 1] * 2, k)
    assert not np.array_equal(ref, f32_ref)


def test_topk_bf16_adversarial_ties_and_prefill_queries():
    B, N, H, k = 2, 12000, 64, 700
    g = np.random.default_rng(300)
    base = normal(300, "keys", (5, 128))
    keys = base[g.integers(0, 5, size=(B, N))]
    keys[1] = base[0]
    q = normal(300, "q_idx", (B, H, 128))
    w = normal(300, "w", (B, 1, H))
    announce("topk bf16 adversarial ties")
    got, _, _ = run_topk(keys, q, w, np.array([N, N]), [4 * N - 1] * 2, k, bf16=True)
    ref = oracle_topk(keys, q, w, np.array([N, N]), [4 * N - 1] * 2, k, bf16=True)
    assert np.array_equal(got, ref)
    assert np.array_equal(got[1, 0], np.arange(k))
    B, N, H, k, Q = 1, 6000, 64, 512, 24
    keys = normal(301, "keys", (B, N, 128))
    q = normal(301, "q_idx", (B, Q * H, 128))
    w = normal(301, "w", (B, Q, H))
    q_pos = [4 * 5000 + j for j in range(Q)]
    announce("topk bf16 prefill-form queries")
    got, _, _ = run_topk(keys, q, w, np.array([N]), q_pos, k, Q=Q, bf16=True)
    ref = oracle_topk(keys, q, w, np.array([N]), q_pos, k, Q=Q, bf16=True)
    assert np.array_equal(got, ref)


def test_topk_bf16_full_size():
    """1M-token CSA decode sizes, bit for bit; prints the recall against the fp32 selection."""
    wl = CSA_PRO_1M
    inp = decode_inputs(wl, threads=16)
    N = inp["N"]
    announce(f"topk bf16 full size {wl.name} B={wl.B} N={N} k={wl.k}")
    q_pos = [wl.T - 1] * wl.B
    args = (inp["keys"], inp["q_idx"], inp["w"][:, None, :], np.array([N] * wl.B), q_pos, wl.k)
    got, _, _ = run_topk(*args, bf16=True)
    ref = oracle_topk(*args, bf16=True)
    assert np.array_equal(got, ref)
    f32_sel, _, _ = run_topk(*args)
    recall = np.mean([np.intersect1d(got[b, 0], f32_sel[b, 0]).size / wl.k for b in range(wl.B)])
    print(f"recall of the BF16 selection against the fp32 one: {recall:.4f}", flush=True)
