"""Pins of the oracle's lightning-indexer scores and top-k selection.

Scores: per-head dots (fp32 fma chain for fp32 data; exact MXFP4 dot rounded once for FP4
data) followed by the fixed-order ReLU-weighted head sum.  The references here are exact
rational arithmetic (tests/exact.py), numpy float64 products of dequantised values, and
integer-valued cases in which every ordering gives the same exact sum.  Top-k: brute force
with numpy's lexsort, and the adversarial tie cases.  Cited: "DeepSeek-V4 technical report
walkthrough" (cyqw.cn), section 2.2 (lightning indexer, top-k), section 3.4 (FP4 QK path).
"""
from fractions import Fraction

import numpy as np
import pytest

from exact import addf, f32_round, fmaf


def combine_ref(s, w):
    """Head combine as specified: ReLU, four fma chains by (h >> 2) & 3, fixed final sum."""
    c = [0.0, 0.0, 0.0, 0.0]
    for h in range(len(s)):
        r = float(s[h]) if s[h] > 0 else 0.0
        g = (h >> 2) & 3
        c[g] = fmaf(w[h], r, c[g])
    v = addf(addf(addf(c[0], c[1]), c[2]), c[3])
    return 0.0 if v == 0 else v


def test_f32_round_helper_matches_numpy():
    g = np.random.default_rng(10)
    xs = g.standard_normal(3000) * np.exp2(g.integers(-140, 120, 3000).astype(float))
    for x in xs:
        assert f32_round(Fraction(float(x))) == float(np.float32(x))


def test_f32_indexer_matches_exact_fma_chain(orc):
    g = np.random.default_rng(11)
    H, d, n = 8, 32, 40
    q = g.standard_normal((H, d)).astype(np.float32)
    w = g.standard_normal(H).astype(np.float32)
    keys = g.standard_normal((n, d)).astype(np.float32)
    got = orc.indexer_scores_f32(q, w, keys)
    for i in range(n):
        s = []
        for h in range(H):
            acc = 0.0
            for e in range(d):
                acc = fmaf(q[h, e], keys[i, e], acc)
            s.append(acc)
        assert got[i] == np.float32(combine_ref(s, w)), i


def test_head_combine_integer_cases_are_exact_sums(orc):
    """With small integers every evaluation order gives the exact sum, so a dropped head,
    a wrong ReLU or a wrong weight shows regardless of the chain order."""
    g = np.random.default_rng(12)
    for H in (4, 8, 64):
        q = g.integers(-3, 4, size=(H, 32)).astype(np.float32)
        w = g.integers(-5, 6, size=H).astype(np.float32)
        keys = g.integers(-3, 4, size=(30, 32)).astype(np.float32)
        got = orc.indexer_scores_f32(q, w, keys)
        s = keys.astype(np.int64) @ q.astype(np.int64).T            # [n][H]
        ref = (np.maximum(s, 0) * w.astype(np.int64)).sum(1)
        assert np.array_equal(got, ref.astype(np.float32))


def test_mxfp4_scores_vs_dequantised_float64(orc):
    g = np.random.default_rng(13)
    H, d, n = 64, 128, 300
    qc, qs = orc.quant_mxfp4(g.standard_normal((H, d)).astype(np.float32))
    kc, ks = orc.quant_mxfp4(g.standard_normal((n, d)).astype(np.float32))
    w = g.standard_normal(H).astype(np.float32)
    got, bad = orc.indexer_scores_mxfp4(qc, qs, w, kc, ks)
    assert bad == 0
    qv = orc.dequant_mxfp4(qc, qs)
    kv = orc.dequant_mxfp4(kc, ks)
    dots = kv @ qv.T            # exact in float64 for these exponent ranges
    for i in range(0, n, 7):
        s = [float(np.float32(x)) for x in dots[i]]
        assert got[i] == np.float32(combine_ref(s, w)), i


def test_mxfp4_inexact_dots_are_counted(orc):
    """A dot whose exact value needs more than 24 significant bits is reported."""
    qx = np.zeros((1, 64), np.float32)
    kx = np.zeros((1, 64), np.float32)
    qx[0, 0] = 6.0            # block 0 at scale 2^0
    kx[0, 0] = 6.0
    qx[0, 32] = 6.0 * 2.0 ** -30   # block 1 at scale 2^-30
    kx[0, 32] = 0.5
    qc, qs = orc.quant_mxfp4(qx)
    kc, ks = orc.quant_mxfp4(kx)
    s, bad = orc.indexer_scores_mxfp4(qc, qs, np.ones(1, np.float32), kc, ks)
    assert bad == 1
    assert s[0] == np.float32(36.0 + 3.0 * 2.0 ** -30)


def brute_topk(scores, k):
    n = len(scores)
    order = np.lexsort((np.arange(n), -scores.astype(np.float64)))
    sel = np.sort(order[:min(k, n)])
    return np.concatenate([sel, -np.ones(k - len(sel), np.int64)]).astype(np.int32)


@pytest.mark.parametrize("n,k", [(1000, 64), (64, 64), (10, 64), (5000, 1), (3000, 512)])
def test_topk_vs_lexsort(orc, n, k):
    g = np.random.default_rng(n + k)
    s = g.standard_normal(n).astype(np.float32)
    assert np.array_equal(orc.topk(s, k), brute_topk(s, k))


def test_topk_adversarial_ties(orc):
    # all equal: the lowest indices win
    assert np.array_equal(orc.topk(np.zeros(100, np.float32), 10), np.arange(10, dtype=np.int32))
    # many ties at the threshold
    g = np.random.default_rng(5)
    s = np.round(g.standard_normal(4000)).astype(np.float32)
    for k in (1, 7, 100, 1024):
        assert np.array_equal(orc.topk(s, k), brute_topk(s, k))
    # nothing visible: all -1
    assert np.array_equal(orc.topk(np.zeros(5, np.float32), 4, n_vis=0), -np.ones(4, np.int32))
    # only the visible prefix competes
    s = np.arange(20, dtype=np.float32)
    assert np.array_equal(orc.topk(s, 3, n_vis=10), np.array([7, 8, 9], np.int32))
    # -0 and +0 are the same score
    s = np.array([0.0, -0.0, 0.0, 1.0], np.float32)
    assert np.array_equal(orc.topk(s, 2), np.array([0, 3], np.int32))


def bf16_values_torch(s):
    """Nearest-even BF16 values of fp32 scores by torch's own conversion (an independent
    implementation of the rounding)."""
    import torch
    return torch.from_numpy(np.asarray(s, np.float32)).to(torch.bfloat16).to(torch.float32).numpy()


def test_topk_bf16_rounding_decides_ties(orc):
    # "DeepSeek-V4 technical report walkthrough" (cyqw.cn), section 3.4: the selector works on
    # BF16 scores.  BF16 keeps 8 significant bits, so near 1 its spacing is 2^-7.
    e = 2.0 ** -8
    # 1 + 2^-8 is the midpoint of 1 and 1 + 2^-7 and rounds to the even 1: it then ties with
    # index 0, which wins
    s = np.array([1.0, 1.0 + e, 1.0 + 2 * e], np.float32)
    assert np.array_equal(orc.topk(s, 2), np.array([1, 2], np.int32))
    assert np.array_equal(orc.topk(s, 2, score_bf16=True), np.array([0, 2], np.int32))
    # 1 + 3*2^-8 is the midpoint of 1 + 2^-7 and 1 + 2^-6 and rounds up to the even 1 + 2^-6
    s = np.array([1.0 + 3 * e, 1.0 + 4 * e], np.float32)
    assert np.array_equal(orc.topk(s, 1), np.array([1], np.int32))
    assert np.array_equal(orc.topk(s, 1, score_bf16=True), np.array([0], np.int32))
    # a negative subnormal score rounds to -0, the same score as +0
    s = np.array([-2.0 ** -149, 0.0], np.float32)
    assert np.array_equal(orc.topk(s, 1), np.array([1], np.int32))
    assert np.array_equal(orc.topk(s, 1, score_bf16=True), np.array([0], np.int32))
    # only the visible prefix competes, -1 padding as before
    assert np.array_equal(orc.topk(np.ones(8, np.float32), 4, n_vis=2, score_bf16=True),
                          np.array([0, 1, -1, -1], np.int32))


@pytest.mark.parametrize("n,k", [(4000, 64), (3000, 512), (50, 64)])
def test_topk_bf16_vs_lexsort_of_torch_rounding(orc, n, k):
    g = np.random.default_rng(7 * n + k)
    s = (g.standard_normal(n) * 4.0).astype(np.float32)
    assert np.array_equal(orc.topk(s, k, score_bf16=True), brute_topk(bf16_values_torch(s), k))


def test_topk_bf16_equals_f32_on_bf16_scores(orc):
    # scores that are already BF16 values select identically in both variants
    g = np.random.default_rng(11)
    s = bf16_values_torch(g.standard_normal(5000).astype(np.float32))
    for k in (1, 100, 1024):
        assert np.array_equal(orc.topk(s, k, score_bf16=True), orc.topk(s, k))
