"""Pins of the oracle's shared-KV MQA with sliding window and sink, and of its RoPE.

References: torch.softmax over [logits; sink] in float64 (textbook attention with a sink
column that carries no value), the closed form for duplicated keys, the sink limits, and
complex-number rotation for RoPE.  Cited: "DeepSeek V4 technical report explained"
(firecat-web.com), item 2 "Hybrid attention" (MQA over selected entries, 128-token window,
sink logit, head dim 512, partial RoPE on the last 64 dims); "DeepSeek-V4 technical report
walkthrough" (cyqw.cn), section 2.2 (window and sink in the core attention).
"""
import math

import numpy as np
import pytest
import torch


def textbook(q, K, sink, scale):
    """softmax([scale q.K^T, sink]) with the sink column dropped, times K (values = keys)."""
    q = torch.from_numpy(q)
    K = torch.from_numpy(K)
    z = scale * q @ K.T                                   # [H][n]
    sk = torch.as_tensor(np.asarray(sink, np.float64)).reshape(-1, 1).expand(z.shape[0], 1)
    p = torch.softmax(torch.cat([z, sk], 1), 1)[:, :-1]
    return (p @ K).numpy(), p.sum(1).numpy()


def rand(g, *shape):
    return g.standard_normal(shape)


def test_p1_csa_path_is_textbook_attention(orc):
    """m = 1, B-stream gates -inf, no RoPE, k >= N, no window: each entry is one raw
    A token and the whole CSA path is plain softmax attention with a sink."""
    g = np.random.default_rng(20)
    T, D, H = 24, 16, 3
    kv_a = rand(g, T, D).astype(np.float32)
    kv_b = rand(g, T, D).astype(np.float32)
    gate_a = rand(g, T, 1).astype(np.float32)
    gate_b = np.full((T, 1), -np.inf, np.float32)
    ent = orc.compress_csa(kv_a, kv_b, gate_a, gate_b, np.zeros((1, 1), np.float32),
                           np.zeros((1, 1), np.float32), tok0=0, m=1, first_entry=0,
                           n_entries=T, apply_rope=False, R=0)
    assert np.array_equal(ent, kv_a)
    q = rand(g, H, D)
    keys = rand(g, T, 8).astype(np.float32)
    idx = {"q": rand(g, 2, 8).astype(np.float32), "w": np.ones(2, np.float32), "keys": keys}
    sink = np.array([0.3, -1.0, 2.0], np.float32)
    out, sel = orc.decode_csa(q, ent.astype(np.float64), T, 64, None, sink, 0.25, q_pos=T - 1, m=1,
                              idx=idx, rope_inverse=False, R=0)
    assert np.array_equal(sel[:T], np.arange(T)) and (sel[T:] == -1).all()
    ref, _ = textbook(q, kv_a.astype(np.float64), sink, 0.25)
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)


def test_p2_window_alone_is_causal_attention(orc):
    g = np.random.default_rng(21)
    T, D, H = 50, 32, 4
    toks = rand(g, T, D)
    q = rand(g, H, D)
    sink = rand(g, H).astype(np.float32)
    out = orc.decode_hca(q, np.zeros((0, D)), 0, toks, sink, 0.2, q_pos=T - 1, rope_inverse=False)
    ref, _ = textbook(q, toks, sink, 0.2)
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)


def test_p3_no_dedup_duplicates_shift_sink_by_ln2(orc):
    """Keys present both as entries and in the window count twice: the result equals
    attention over one copy with the sink lowered by ln 2."""
    g = np.random.default_rng(22)
    T, D, H = 40, 16, 5
    toks = rand(g, T, D)
    q = rand(g, H, D)
    sink = rand(g, H).astype(np.float32)
    out = orc.attend(q, toks, toks, sink, 0.3)
    ref, _ = textbook(q, toks, sink.astype(np.float64) - math.log(2.0), 0.3)
    np.testing.assert_allclose(out, ref, rtol=1e-11, atol=1e-12)
    # sink = -inf gives exact full attention over the (duplicated) keys
    out2 = orc.attend(q, toks, toks, np.full(H, -np.inf, np.float32), 0.3)
    ref2, _ = textbook(q, toks, np.full(H, -np.inf), 0.3)
    np.testing.assert_allclose(out2, ref2, rtol=1e-12, atol=1e-12)


def test_p4_topk_covering_all_equals_dense(orc):
    g = np.random.default_rng(23)
    N, D, H, dI = 30, 32, 4, 32
    rec = rand(g, N, D)
    q = rand(g, H, D)
    win = rand(g, 8, D)
    sink = rand(g, H).astype(np.float32)
    idx = {"q": rand(g, 4, dI).astype(np.float32), "w": rand(g, 4).astype(np.float32),
           "keys": rand(g, N, dI).astype(np.float32)}
    out, sel = orc.decode_csa(q, rec, N, 64, win, sink, 0.1, q_pos=4 * N - 1, m=4, idx=idx, R=8)
    dense = orc.decode_hca(q, rec, N, win, sink, 0.1, q_pos=4 * N - 1, m=4, R=8)
    np.testing.assert_allclose(out, dense, rtol=1e-13, atol=1e-13)


def test_p5_sink_semantics(orc):
    g = np.random.default_rng(24)
    n, D, H = 20, 16, 3
    K = rand(g, n, D)
    q = rand(g, H, D)
    _, mass = orc.attend(q, K, None, np.full(H, -np.inf, np.float32), 0.5, with_mass=True)
    np.testing.assert_allclose(mass, 1.0, rtol=0, atol=1e-15)
    sink = np.array([0.0, 1.0, -2.0], np.float32)
    out, mass = orc.attend(q, K, None, sink, 0.5, with_mass=True)
    z = 0.5 * q @ K.T
    M = np.maximum(z.max(1), sink)
    den = np.exp(sink - M) + np.exp(z - M[:, None]).sum(1)
    np.testing.assert_allclose(mass, 1.0 - np.exp(sink - M) / den, rtol=1e-13)
    assert (mass < 1).all()
    out_big, _ = orc.attend(q, K, None, np.full(H, 1e4, np.float32), 0.5, with_mass=True)
    assert np.abs(out_big).max() < 1e-300
    # empty key set: output is zero whatever the sink
    out0 = orc.attend(q, None, None, sink, 0.5)
    assert not out0.any()


def test_p12_rope_identities(orc):
    g = np.random.default_rng(25)
    R, D = 64, 128
    x = rand(g, 7, D)
    p = np.array([0, 1, 5, 100, 4096, 65535, 1048575], np.float64)
    y = orc.rope(x, R, p)
    assert np.array_equal(y[:, :D - R], x[:, :D - R])
    np.testing.assert_allclose(np.linalg.norm(y[:, D - R:], axis=1), np.linalg.norm(x[:, D - R:], axis=1),
                               rtol=1e-7)
    back = orc.rope(y, R, p, sign=-1)
    np.testing.assert_allclose(back, x, rtol=0, atol=2e-7 * np.abs(x).max())
    # interleaved pairs rotate as complex numbers by p * theta^(-2j/R)
    j = np.arange(R // 2)
    ang = p[:, None] * 10000.0 ** (-2.0 * j / R)
    c = np.cos(ang).astype(np.float32).astype(np.float64)
    s = np.sin(ang).astype(np.float32).astype(np.float64)
    z = (x[:, D - R::2] + 1j * x[:, D - R + 1::2]) * (c + 1j * s)
    np.testing.assert_allclose(y[:, D - R::2], z.real, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(y[:, D - R + 1::2], z.imag, rtol=1e-13, atol=1e-13)
    # relative position: (R_a q).(R_b k) depends on a - b only (up to the fp32 cos/sin)
    q1, k1 = rand(g, 1, R), rand(g, 1, R)
    d1 = (orc.rope(q1, R, [10.0]) * orc.rope(k1, R, [3.0])).sum()
    d2 = (orc.rope(q1, R, [1010.0]) * orc.rope(k1, R, [1003.0])).sum()
    assert abs(d1 - d2) < 1e-5 * np.abs(q1).sum() * np.abs(k1).sum()


def test_output_rope_inverse_is_applied_at_query_position(orc):
    g = np.random.default_rng(26)
    n, D, H, R = 10, 64, 2, 16
    K = rand(g, n, D)
    q = rand(g, H, D)
    sink = np.zeros(H, np.float32)
    plain = orc.attend(q, K, None, sink, 0.1)
    rot = orc.attend(q, K, None, sink, 0.1, rope_inverse=True, R=R, t_q=777.0)
    np.testing.assert_allclose(rot, orc.rope(plain, R, 777.0, sign=-1), rtol=1e-14, atol=1e-14)


# ------------------------------------------------------------ query prologue ---
# "DeepSeek-V4 technical report walkthrough" (cyqw.cn), section 2.3: RMSNorm acts directly on
# the queries; the rotation of the last R dims follows at the query position.

def _bf16_bits_of(x64):
    import torch
    t = torch.from_numpy(np.asarray(x64, np.float64)).to(torch.float32).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def test_query_prologue_matches_torch_norm_then_rope(orc):
    import torch
    g = np.random.default_rng(91)
    H, D, R, pos = 8, 128, 32, 12345
    q = _bf16_bits_of(g.standard_normal((H, D)))
    w = (0.5 + g.random(D)).astype(np.float32)
    got = orc.query_prologue(q, w, pos=pos, R=R)
    x = torch.from_numpy(orc_bf16_values(q))
    normed = torch.nn.functional.rms_norm(x, (D,), torch.from_numpy(w.astype(np.float64)), 1e-6).numpy()
    expect = _bf16_bits_of(orc.rope(normed, R, np.full(H, pos)))
    assert np.array_equal(got, expect)
    # rotating first and normalising after gives another result (w differs within pairs)
    other = _bf16_bits_of(torch.nn.functional.rms_norm(torch.from_numpy(orc.rope(orc_bf16_values(q), R, np.full(H, pos))),
                                                       (D,), torch.from_numpy(w.astype(np.float64)), 1e-6).numpy())
    assert not np.array_equal(got, other)


def test_query_prologue_unit_weights_unit_rms(orc):
    g = np.random.default_rng(92)
    H, D = 4, 512
    q = _bf16_bits_of(3.0 * g.standard_normal((H, D)))
    got = orc_bf16_values(orc.query_prologue(q, np.ones(D, np.float32), pos=7, R=64, eps=0.0))
    np.testing.assert_allclose(np.sqrt((got * got).mean(axis=1)), 1.0, atol=4e-3)


def orc_bf16_values(bits):
    from workloads import bf16_bits_to_f64
    return bf16_bits_to_f64(np.asarray(bits, np.uint16))
