"""Pins of the oracle's KV compressors (CSA: ratio 4, two streams, overlapped blocks;
HCA: ratio 128, one stream).

References: scipy's softmax for the gate weights (read out with one-hot token rows, which
also pins which tokens each entry covers), constant streams, equal-logit means, RoPE at
the entry position, and chunked versus whole-sequence compression.  Cited: "DeepSeek-V4
technical report walkthrough" (cyqw.cn), section 2.2 (two independent KV sequences,
softmax-normalised gates, adjacent blocks share indices; HCA merges 128 tokens without
overlap); "DeepSeek V4 preview and technical report" (chooseai.net), section 1 (softmax with
positional bias).
"""
import numpy as np
import pytest
from scipy.special import softmax

from workloads import TINY, normal


def onehot_streams(T, D, off):
    x = np.zeros((T, D), np.float32)
    x[np.arange(T), off + np.arange(T)] = 1.0
    return x


@pytest.mark.parametrize("m", [1, 2, 4])
def test_csa_overlap_structure_and_gate_softmax(orc, m):
    """Token t of stream A is one-hot at dim t, of stream B at dim T + t, so entry i's
    dims hold exactly the merge weight of each token it covers."""
    g = np.random.default_rng(30 + m)
    T = 8 * m
    D = 2 * T
    kv_a = onehot_streams(T, D, 0)
    kv_b = onehot_streams(T, D, T)
    gate_a = g.standard_normal((T, 1)).astype(np.float32)
    gate_b = g.standard_normal((T, 1)).astype(np.float32)
    bias_a = g.standard_normal((m, 1)).astype(np.float32)
    bias_b = g.standard_normal((m, 1)).astype(np.float32)
    N = T // m
    ent = orc.compress_csa(kv_a, kv_b, gate_a, gate_b, bias_a, bias_b, tok0=0, m=m, first_entry=0,
                           n_entries=N, apply_rope=False, R=0)
    for i in range(N):
        a_tok = np.arange(m * i, m * i + m)
        logits = list(gate_a[a_tok, 0].astype(np.float64) + bias_a[:, 0])
        dims = list(a_tok)
        if i >= 1:
            b_tok = np.arange(m * (i - 1), m * i)
            logits += list(gate_b[b_tok, 0].astype(np.float64) + bias_b[:, 0])
            dims += list(T + b_tok)
        wts = softmax(np.array(logits))
        expect = np.zeros(D)
        expect[dims] = wts
        np.testing.assert_allclose(ent[i], expect.astype(np.float32), rtol=1e-6, atol=1e-7)
        assert abs(ent[i].astype(np.float64).sum() - 1.0) < 1e-6       # weights sum to 1
        assert (ent[i] >= 0).all() and (ent[i] <= 1).all()


def test_csa_per_channel_gates(orc):
    """G = D: each channel has its own softmax over the same candidates."""
    g = np.random.default_rng(35)
    m, T, D = 4, 16, 6
    kv_a = g.standard_normal((T, D)).astype(np.float32)
    kv_b = g.standard_normal((T, D)).astype(np.float32)
    gate_a = g.standard_normal((T, D)).astype(np.float32)
    gate_b = g.standard_normal((T, D)).astype(np.float32)
    bias_a = g.standard_normal((m, D)).astype(np.float32)
    bias_b = g.standard_normal((m, D)).astype(np.float32)
    ent = orc.compress_csa(kv_a, kv_b, gate_a, gate_b, bias_a, bias_b, tok0=0, m=m, first_entry=0,
                           n_entries=4, apply_rope=False, R=0)
    i = 2
    for d in range(D):
        za = gate_a[m * i:m * i + m, d].astype(np.float64) + bias_a[:, d]
        zb = gate_b[m * (i - 1):m * i, d].astype(np.float64) + bias_b[:, d]
        w = softmax(np.concatenate([za, zb]))
        x = np.concatenate([kv_a[m * i:m * i + m, d], kv_b[m * (i - 1):m * i, d]]).astype(np.float64)
        assert abs(ent[i, d] - np.float32(w @ x)) <= 1e-6 * max(1.0, abs(w @ x))


def test_constant_stream_and_equal_logits(orc):
    T, D, m = 32, 8, 4
    c = np.full((T, D), 2.5, np.float32)
    z = np.zeros((T, 1), np.float32)
    b = np.zeros((m, 1), np.float32)
    g = np.random.default_rng(36)
    gates = g.standard_normal((T, 1)).astype(np.float32)
    ent = orc.compress_csa(c, c, gates, gates, b, b, tok0=0, m=m, first_entry=0, n_entries=8,
                           apply_rope=False, R=0)
    np.testing.assert_allclose(ent, 2.5, rtol=1e-7)
    xa = g.standard_normal((T, D)).astype(np.float32)
    xb = g.standard_normal((T, D)).astype(np.float32)
    ent = orc.compress_csa(xa, xb, z, z, b, b, tok0=0, m=m, first_entry=0, n_entries=8,
                           apply_rope=False, R=0)
    np.testing.assert_allclose(ent[0], xa[0:4].astype(np.float64).mean(0), rtol=1e-6, atol=1e-7)
    for i in range(1, 8):
        mean = np.concatenate([xa[4 * i:4 * i + 4], xb[4 * i - 4:4 * i]]).astype(np.float64).mean(0)
        np.testing.assert_allclose(ent[i], mean, rtol=1e-6, atol=1e-7)
    h = orc.compress_hca(xa, z, np.zeros((16, 1), np.float32), tok0=0, m=16, first_entry=0,
                         n_entries=2, apply_rope=False, R=0)
    np.testing.assert_allclose(h, xa.astype(np.float64).reshape(2, 16, D).mean(1), rtol=1e-6, atol=1e-7)


def test_minus_inf_logit_gets_zero_weight(orc):
    T, D, m = 8, 4, 4
    g = np.random.default_rng(37)
    xa = g.standard_normal((T, D)).astype(np.float32)
    xb = g.standard_normal((T, D)).astype(np.float32)
    ga = np.zeros((T, 1), np.float32)
    gb = np.full((T, 1), -np.inf, np.float32)
    b = np.zeros((m, 1), np.float32)
    ent = orc.compress_csa(xa, xb, ga, gb, b, b, tok0=0, m=m, first_entry=0, n_entries=2,
                           apply_rope=False, R=0)
    np.testing.assert_allclose(ent[1], xa[4:8].astype(np.float64).mean(0), rtol=1e-6)


def test_rope_applied_at_entry_position(orc):
    g = np.random.default_rng(38)
    T, D, R, m = 64, 32, 8, 4
    xa = g.standard_normal((T, D)).astype(np.float32)
    xb = g.standard_normal((T, D)).astype(np.float32)
    ga = g.standard_normal((T, 1)).astype(np.float32)
    gb = g.standard_normal((T, 1)).astype(np.float32)
    b = g.standard_normal((m, 1)).astype(np.float32)
    plain = orc.compress_csa(xa, xb, ga, gb, b, b, tok0=0, m=m, first_entry=0, n_entries=16,
                             apply_rope=False, R=R)
    rot = orc.compress_csa(xa, xb, ga, gb, b, b, tok0=0, m=m, first_entry=0, n_entries=16,
                           apply_rope=True, R=R)
    ref = orc.rope(plain.astype(np.float64), R, m * np.arange(16.0))
    np.testing.assert_allclose(rot, ref, rtol=2e-6, atol=2e-6)
    assert np.array_equal(rot[:, :D - R], plain[:, :D - R])


def test_p14_chunked_compression_equals_whole_sequence(orc):
    """Compressing in chunks, each chunk given the B-stream block before it (the state
    cache), yields exactly the whole-sequence entries."""
    w = TINY
    T, D = 1024, w.D
    s = w.seed
    xa, xb = normal(s, "kv_a", (T, D)), normal(s, "kv_b", (T, D))
    ga, gb = normal(s, "gate_a", (T, 1)), normal(s, "gate_b", (T, 1))
    ba, bb = normal(s, "bias_a", (4, 1)), normal(s, "bias_b", (4, 1))
    whole = orc.compress_csa(xa, xb, ga, gb, ba, bb, tok0=0, m=4, first_entry=0, n_entries=T // 4,
                             apply_rope=True, R=w.R)
    parts = []
    for c0 in range(0, T, 256):
        r0 = max(0, c0 - 4)                  # one block of state before the chunk
        sl = slice(r0, c0 + 256)
        parts.append(orc.compress_csa(xa[sl], xb[sl], ga[sl], gb[sl], ba, bb, tok0=r0, m=4,
                                      first_entry=c0 // 4, n_entries=64, apply_rope=True, R=w.R))
    assert np.array_equal(np.concatenate(parts), whole)
    with pytest.raises(ValueError):          # without the state block the first entry is uncovered
        orc.compress_csa(xa[256:512], xb[256:512], ga[256:512], gb[256:512], ba, bb, tok0=256, m=4,
                         first_entry=64, n_entries=64, apply_rope=True, R=w.R)
    xh, gh, bh = normal(s, "kv_h", (T, D)), normal(s, "gate_h", (T, 1)), normal(s, "bias_h", (128, 1))
    whole_h = orc.compress_hca(xh, gh, bh, tok0=0, m=128, first_entry=0, n_entries=8,
                               apply_rope=True, R=w.R)
    part_h = np.concatenate([orc.compress_hca(xh[c:c + 256], gh[c:c + 256], bh, tok0=c, m=128,
                                              first_entry=c // 128, n_entries=2, apply_rope=True,
                                              R=w.R) for c in range(0, T, 256)])
    assert np.array_equal(part_h, whole_h)


# ------------------------------------------------------------- RMSNorm of entries ---
# "DeepSeek-V4 technical report walkthrough" (cyqw.cn), section 2.3: RMSNorm acts directly on
# the queries and KV entries.  Reading: it normalises each merged entry before RoPE.

def rms_norm_torch(x, w, eps):
    """torch's own RMSNorm (a library implementation) in float64."""
    import torch
    t = torch.from_numpy(np.asarray(x, np.float64))
    return torch.nn.functional.rms_norm(t, (t.shape[-1],), torch.from_numpy(np.asarray(w, np.float64)),
                                        eps).numpy()


def csa_inputs(seed, T=64, D=64, m=4):
    g = np.random.default_rng(seed)
    f = lambda *s: g.standard_normal(s).astype(np.float32)
    return dict(kv_a=f(T, D), kv_b=f(T, D), gate_a=f(T, 1), gate_b=f(T, 1), bias_a=f(m, 1), bias_b=f(m, 1))


def test_entry_rmsnorm_matches_torch_and_precedes_rope(orc):
    D, R, m, eps = 64, 16, 4, 1e-6
    x = csa_inputs(41, D=D)
    g = np.random.default_rng(42)
    w = (0.5 + g.random(D)).astype(np.float32)  # unequal within RoPE pairs: the orders differ
    kw = dict(tok0=0, m=m, first_entry=0, n_entries=16, R=R)
    plain = orc.compress_csa(**x, apply_rope=False, **kw).astype(np.float64)
    normed = orc.compress_csa(**x, apply_rope=False, norm_w=w, eps=eps, **kw)
    np.testing.assert_allclose(normed, rms_norm_torch(plain, w, eps), rtol=2e-6, atol=1e-7)
    # with RoPE: the norm comes first, then the rotation at the entry position
    full = orc.compress_csa(**x, apply_rope=True, norm_w=w, eps=eps, **kw)
    pos = m * np.arange(16)
    expect = orc.rope(rms_norm_torch(plain, w, eps), R, pos)
    np.testing.assert_allclose(full, expect, rtol=2e-6, atol=1e-7)
    rotated_first = rms_norm_torch(orc.compress_csa(**x, apply_rope=True, **kw), w, eps)
    assert np.abs(full - rotated_first).max() > 1e-3


def test_entry_rmsnorm_unit_weights_give_unit_mean_square(orc):
    x = csa_inputs(43, D=128)
    y = orc.compress_csa(**x, tok0=0, m=4, first_entry=0, n_entries=16, apply_rope=True, R=32,
                         norm_w=np.ones(128, np.float32), eps=0.0).astype(np.float64)
    np.testing.assert_allclose((y * y).mean(axis=1), 1.0, rtol=1e-6)


def test_hca_entry_rmsnorm_matches_torch(orc):
    g = np.random.default_rng(44)
    T, D, m = 512, 64, 128
    kv = g.standard_normal((T, D)).astype(np.float32)
    gate = g.standard_normal((T, 1)).astype(np.float32)
    bias = g.standard_normal((m, 1)).astype(np.float32)
    w = (0.5 + g.random(D)).astype(np.float32)
    kw = dict(tok0=0, m=m, first_entry=0, n_entries=4, R=16)
    plain = orc.compress_hca(kv, gate, bias, apply_rope=False, **kw)
    normed = orc.compress_hca(kv, gate, bias, apply_rope=False, norm_w=w, eps=1e-6, **kw)
    np.testing.assert_allclose(normed, rms_norm_torch(plain, w, 1e-6), rtol=2e-6, atol=1e-7)
