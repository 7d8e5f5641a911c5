"""Pins of the oracle's prefill composition (steps per chunk query, causal).

Each case reduces the prefill of a chunk to textbook softmax-with-sink attention over rows
picked by absolute position, written independently here: which raw tokens a query's window
holds (t-W+1 .. t, clipped at 0) and which entries it sees (block end at or before t)."""
import numpy as np

import oracle


def brute(q, X, sink, scale):
    """softmax over [scale * q.x_j ; sink] per head, sink column dropped, times X."""
    z = scale * (q @ X.T)                                  # [H][n]
    sink = np.asarray(sink, np.float64)
    M = np.maximum(z.max(axis=1) if X.shape[0] else -np.inf, sink)
    p = np.exp(z - M[:, None])
    den = p.sum(axis=1) + np.exp(sink - M)
    return (p @ X) / den[:, None]


def setup(seed, rows, H=3, D=16):
    g = np.random.default_rng(seed)
    # the sink is an fp32 parameter on both sides
    return g.standard_normal((rows, D)), g.standard_normal((40, H, D)), g.standard_normal(H).astype(np.float32)


def test_window_only_is_full_causal_attention():
    tok0, n_prev, C, W = 64, 64, 32, 128
    X, q, sink = setup(1, n_prev + C)
    pos = np.arange(tok0 - n_prev, tok0 + C)
    outs, _ = oracle.prefill_queries("hca", q, np.zeros((0, 16)), 0, X, n_prev=n_prev, tok0=tok0,
                                     queries=range(C), W=W, sink=sink, scale=0.25, m=128,
                                     rope_inverse=False, R=0)
    for j in range(C):
        t = tok0 + j
        ref = brute(q[j], X[pos <= t], sink, 0.25)
        assert np.allclose(outs[j], ref, rtol=1e-12, atol=1e-13)


def test_window_is_the_last_W_tokens_by_position():
    tok0, n_prev, C, W = 40, 20, 24, 16
    X, q, sink = setup(2, n_prev + C)
    pos = np.arange(tok0 - n_prev, tok0 + C)
    outs, _ = oracle.prefill_queries("hca", q, np.zeros((0, 16)), 0, X, n_prev=n_prev, tok0=tok0,
                                     queries=range(C), W=W, sink=sink, scale=0.3, m=128,
                                     rope_inverse=False, R=0)
    for j in range(C):
        t = tok0 + j
        ref = brute(q[j], X[(pos <= t) & (pos > t - W)], sink, 0.3)
        assert np.allclose(outs[j], ref, rtol=1e-12, atol=1e-13)


def test_first_chunk_window_starts_at_position_zero():
    tok0, n_prev, C, W = 0, 0, 20, 8
    X, q, sink = setup(3, C)
    outs, _ = oracle.prefill_queries("hca", q, np.zeros((0, 16)), 0, X, n_prev=0, tok0=0,
                                     queries=range(C), W=W, sink=sink, scale=0.3, m=128,
                                     rope_inverse=False, R=0)
    for j in range(C):
        ref = brute(q[j], X[max(0, j - W + 1):j + 1], sink, 0.3)
        assert np.allclose(outs[j], ref, rtol=1e-12, atol=1e-13)


def test_csa_entries_visible_by_block_end():
    """k >= N and no window: query t attends over exactly the entries with 4(i+1)-1 <= t."""
    tok0, n_prev, C, m, H, D, dI = 32, 0, 40, 4, 3, 16, 8
    g = np.random.default_rng(4)
    N = (tok0 + C) // m
    E = g.standard_normal((N, D))
    q = g.standard_normal((C, H, D))
    sink = g.standard_normal(H).astype(np.float32)
    idx = dict(q=g.standard_normal((C, 4, dI)).astype(np.float32), w=g.standard_normal((C, 4)).astype(np.float32),
               keys=g.standard_normal((N, dI)).astype(np.float32))
    outs, sels = oracle.prefill_queries("csa", q, E, N, np.zeros((n_prev + C, D)), n_prev=n_prev, tok0=tok0,
                                        queries=range(C), W=0, sink=sink, scale=0.3, m=m, k=64, idx=idx,
                                        rope_inverse=False, R=0)
    ends = m * (np.arange(N) + 1) - 1
    for j in range(C):
        t = tok0 + j
        vis = ends <= t
        assert np.array_equal(sels[j][sels[j] >= 0], np.nonzero(vis)[0])
        assert np.allclose(outs[j], brute(q[j], E[vis], sink, 0.3), rtol=1e-12, atol=1e-13)


def test_csa_m1_with_masked_b_stream_is_causal_attention_over_tokens():
    """m = 1, B-gates -inf, no RoPE: entry i is token i, so with k >= N and no window the chunk
    query t attends over tokens 0..t (the compressor and the prefill composition together)."""
    tok0, C, D, H = 8, 12, 16, 2
    g = np.random.default_rng(5)
    T = tok0 + C
    A = g.standard_normal((T, D)).astype(np.float32)
    ent = oracle.compress_csa(A, g.standard_normal((T, D)).astype(np.float32),
                              g.standard_normal((T, 1)).astype(np.float32),
                              np.full((T, 1), -np.inf, np.float32), np.zeros((1, 1), np.float32),
                              np.zeros((1, 1), np.float32), tok0=0, m=1, first_entry=0, n_entries=T,
                              apply_rope=False, R=0).astype(np.float64)
    assert np.array_equal(ent, A.astype(np.float64))
    q = g.standard_normal((C, H, D))
    sink = g.standard_normal(H).astype(np.float32)
    idx = dict(q=g.standard_normal((C, 4, 8)).astype(np.float32), w=np.ones((C, 4), np.float32),
               keys=g.standard_normal((T, 8)).astype(np.float32))
    outs, _ = oracle.prefill_queries("csa", q, ent, T, np.zeros((C, D)), n_prev=0, tok0=tok0, queries=range(C),
                                     W=0, sink=sink, scale=0.2, m=1, k=T, idx=idx, rope_inverse=False, R=0)
    for j in range(C):
        assert np.allclose(outs[j], brute(q[j], A[:tok0 + j + 1].astype(np.float64), sink, 0.2),
                           rtol=1e-12, atol=1e-13)
