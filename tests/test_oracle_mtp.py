"""CPU pins of the oracle's multi-token decode step (decode_tokens): Q consecutive new tokens of
one sequence evaluated together ("DeepSeek-V4 technical report walkthrough" (cyqw.cn), section 2
and section 4.2: multi-token prediction with depth 1).

- With m = 1, B-stream gates -inf, no RoPE and k covering every entry, query j attends over raw
  tokens 0 .. t_j and its window: brute-force causal softmax with the sink (torch.softmax), one
  query at a time.  An entry or window token leaking from a later token of the step fails it.
- Against Q one-token steps taken in order from scratch-built caches (each query sees only the
  entries that exist once its own token is in, and the window that ends at it): equal for every
  token placement relative to a block end (the block completed by the first token, by the second,
  or by neither), for CSA (MXFP4 and fp32 indexers) and HCA.
"""
import math

import numpy as np
import torch


def rand(g, *shape):
    return g.standard_normal(shape)


def textbook(q, K, sink, scale):
    q = torch.from_numpy(q)
    K = torch.from_numpy(K)
    z = scale * q @ K.T
    sk = torch.as_tensor(np.asarray(sink, np.float64)).reshape(-1, 1).expand(z.shape[0], 1)
    p = torch.softmax(torch.cat([z, sk], 1), 1)[:, :-1]
    return (p @ K).numpy()


def test_mtp_m1_is_causal_attention_per_token(orc):
    g = np.random.default_rng(60)
    T, D, H, Q, W = 30, 16, 3, 3, 4
    kv_a = rand(g, T, D).astype(np.float32)
    kv_b = rand(g, T, D).astype(np.float32)
    ent = orc.compress_csa(kv_a, kv_b, rand(g, T, 1).astype(np.float32), np.full((T, 1), -np.inf, np.float32),
                           np.zeros((1, 1), np.float32), np.zeros((1, 1), np.float32), tok0=0, m=1, first_entry=0,
                           n_entries=T, apply_rope=False, R=0)
    q = rand(g, Q, H, D)
    idx = {"q": rand(g, Q, 2, 8).astype(np.float32), "w": np.ones((Q, 2), np.float32),
           "keys": rand(g, T, 8).astype(np.float32)}
    sink = np.array([0.3, -1.0, 2.0], np.float32)
    toks = kv_a.astype(np.float64)
    out, sel = orc.decode_tokens("csa", q, ent.astype(np.float64), T, toks, t_last=T - 1, Q=Q, win_len=W, sink=sink,
                                 scale=0.25, m=1, k=64, idx=idx, rope_inverse=False, R=0)
    for j in range(Q):
        tj = T - Q + j
        assert np.array_equal(sel[j][:tj + 1], np.arange(tj + 1)) and (sel[j][tj + 1:] == -1).all()
        # entries 0..t_j, then the window tokens t_j-W+1 .. t_j again (no dedup)
        keys = np.concatenate([toks[:tj + 1], toks[tj - W + 1:tj + 1]])
        np.testing.assert_allclose(out[j], textbook(q[j], keys, sink, 0.25), rtol=1e-12, atol=1e-12)


def sequential_csa(orc, q, ents, keys, stream, t_last, Q, win_len, sink, scale, m, k, idx_q, R):
    """Q one-token steps in order: token j's step sees the entries complete once t_j is in."""
    outs, sels = [], []
    for j in range(Q):
        tj = t_last - Q + 1 + j
        n_j = (tj + 1) // m
        wl = min(win_len, tj + 1)
        idx = dict(idx_q[j], **keys(n_j))
        o, s = orc.decode_csa(q[j], ents[:n_j], n_j, k, stream[tj - wl + 1:tj + 1], sink, scale, q_pos=tj, m=m, idx=idx,
                              R=R)
        outs.append(o)
        sels.append(s)
    return np.stack(outs), np.stack(sels)


def test_mtp_csa_equals_sequential_one_token_steps(orc):
    g = np.random.default_rng(61)
    m, D, R, H, HI, dI, k, W = 4, 64, 16, 4, 8, 128, 16, 12
    for t_last, Q in ((99, 2), (100, 2), (101, 2), (102, 3), (7, 2), (4, 2), (3, 3)):
        T = t_last + 1
        s = {n: rand(g, T, D).astype(np.float32) for n in ("kv_a", "kv_b")}
        ia, ib = rand(g, T, dI).astype(np.float32), rand(g, T, dI).astype(np.float32)
        ga, gb = rand(g, T, 1).astype(np.float32), rand(g, T, 1).astype(np.float32)
        ba, bb = rand(g, m, 1).astype(np.float32), rand(g, m, 1).astype(np.float32)
        N = T // m
        ents = orc.compress_csa(s["kv_a"], s["kv_b"], ga, gb, ba, bb, tok0=0, m=m, first_entry=0, n_entries=N,
                                apply_rope=True, R=R).astype(np.float64)
        kf = orc.compress_csa(ia, ib, ga, gb, ba, bb, tok0=0, m=m, first_entry=0, n_entries=N, apply_rope=False, R=0)
        kc, ks = orc.quant_mxfp4(kf)
        qc, qs = orc.quant_mxfp4(rand(g, Q * HI, dI).astype(np.float32))
        qc, qs = qc.reshape(Q, HI, -1), qs.reshape(Q, HI, -1)
        w = rand(g, Q, HI).astype(np.float32)
        q = rand(g, Q, H, D)
        sink = rand(g, H).astype(np.float32)
        stream = s["kv_a"].astype(np.float64)
        scale = 1.0 / math.sqrt(D)
        out, sel = orc.decode_tokens("csa", q, ents, N, stream, t_last=t_last, Q=Q, win_len=W, sink=sink, scale=scale,
                                     m=m, k=k, idx=dict(q_codes=qc, q_scales=qs, w=w, k_codes=kc, k_scales=ks), R=R)
        ref, ref_sel = sequential_csa(orc, q, ents, lambda n: dict(k_codes=kc[:n], k_scales=ks[:n]), stream, t_last,
                                      Q, W, sink, scale, m, k,
                                      [dict(q_codes=qc[j], q_scales=qs[j], w=w[j]) for j in range(Q)], R)
        assert np.array_equal(sel, ref_sel), (t_last, Q)
        assert np.array_equal(out, ref), (t_last, Q)
        # the entry a later token completes is never selected by an earlier query
        for j in range(Q - 1):
            tj = t_last - Q + 1 + j
            assert sel[j].max() < (tj + 1) // m


def test_mtp_hca_equals_sequential_one_token_steps(orc):
    g = np.random.default_rng(62)
    m, D, R, H, W = 8, 32, 8, 4, 6
    for t_last, Q in ((63, 2), (64, 2), (65, 2), (66, 3), (8, 2), (7, 2)):
        T = t_last + 1
        kv = rand(g, T, D).astype(np.float32)
        N = T // m
        ents = orc.compress_hca(kv, rand(g, T, 1).astype(np.float32), rand(g, m, 1).astype(np.float32), tok0=0, m=m,
                                first_entry=0, n_entries=N, apply_rope=True, R=R).astype(np.float64)
        q = rand(g, Q, H, D)
        sink = rand(g, H).astype(np.float32)
        stream = kv.astype(np.float64)
        out, _ = orc.decode_tokens("hca", q, ents, N, stream, t_last=t_last, Q=Q, win_len=W, sink=sink, scale=0.2, m=m,
                                   R=R)
        for j in range(Q):
            tj = t_last - Q + 1 + j
            n_j = (tj + 1) // m
            wl = min(W, tj + 1)
            ref = orc.decode_hca(q[j], ents[:n_j], n_j, stream[tj - wl + 1:tj + 1], sink, 0.2, q_pos=tj, m=m, R=R)
            assert np.array_equal(out[j], ref), (t_last, Q, j)
