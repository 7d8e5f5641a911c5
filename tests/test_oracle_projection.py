"""CPU pins of the oracle's grouped output projection ("DeepSeek-V4 technical report walkthrough"
(cyqw.cn), section 2.2, Grouped Output Projection: the head outputs are reduced group by group,
then concatenated and projected).

- round_bf16 (double -> BF16, ties to even, no fp32 step): equals torch's fp32 -> BF16 on values
  that fp32 holds exactly, rounds values just off a midpoint to the nearer neighbour, and sends
  exact midpoints to the even neighbour.
- group_reduce equals one dense projection with the block-diagonal matrix of the group weights
  (numpy float64), rounded to BF16: a wrong group offset, a transposed weight or a head order
  mix-up fails it.  One-hot weights copy chosen inputs exactly.
- project equals numpy's float64 matrix product; the whole projection with one head per group
  and identity group weights is a single dense projection of the attention output.
"""
import numpy as np
import torch


def bf16_bits(x):
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(
        np.uint16)


def bf16_vals(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).double().numpy()


def test_round_bf16(orc):
    g = np.random.default_rng(70)
    x = g.standard_normal(2000).astype(np.float32)
    ref = bf16_vals(bf16_bits(x))
    assert all(orc.round_bf16(float(v)) == r for v, r in zip(x, ref))
    for base in (1.0, 1.5, -3.25, 2.0 ** -20, 1000.0):
        ulp = 2.0 ** (np.floor(np.log2(abs(base))) - 7)
        mid_even = base + 0.5 * ulp          # base has an even last bit: ties go back to base
        assert orc.round_bf16(mid_even) == base
        assert orc.round_bf16(base + 1.5 * ulp) == base + 2 * ulp   # odd neighbour: ties go up
        assert orc.round_bf16(mid_even + ulp * 2.0 ** -30) == base + ulp
        assert orc.round_bf16(mid_even - ulp * 2.0 ** -30) == base
    assert orc.round_bf16(0.0) == 0.0


def test_group_reduce_is_block_diagonal_dense_projection(orc):
    g = np.random.default_rng(71)
    T, H, D, G, r = 3, 8, 32, 4, 16
    o = bf16_bits(g.standard_normal((T, H, D)) * 0.3)
    wg = bf16_bits(g.standard_normal((G, r, H * D // G)) / np.sqrt(H * D // G))
    y = orc.group_reduce(o, G, r, wg)
    Kg = H * D // G
    dense = np.zeros((G * r, H * D))
    for k in range(G):
        dense[k * r:(k + 1) * r, k * Kg:(k + 1) * Kg] = bf16_vals(wg[k])
    ref = bf16_vals(o).reshape(T, H * D) @ dense.T
    ref = np.vectorize(orc.round_bf16)(ref)
    assert np.array_equal(y, ref)
    # one-hot group weights copy chosen inputs exactly (BF16 inputs stay BF16)
    pick = g.integers(0, Kg, (G, r))
    one = np.zeros((G, r, Kg), np.float32)
    for k in range(G):
        one[k, np.arange(r), pick[k]] = 1.0
    y1 = orc.group_reduce(o, G, r, bf16_bits(one))
    ov = bf16_vals(o).reshape(T, G, Kg)
    for k in range(G):
        assert np.array_equal(y1[:, k * r:(k + 1) * r], ov[:, k, pick[k]])


def test_project_and_whole_projection(orc):
    g = np.random.default_rng(72)
    T, H, D, d = 4, 4, 16, 24
    x = g.standard_normal((T, 40))
    w = bf16_bits(g.standard_normal((d, 40)))
    np.testing.assert_allclose(orc.project(x, w), x @ bf16_vals(w).T, rtol=1e-13, atol=1e-13)
    # one head per group with identity group weights: y is the attention output itself, and the
    # projection is one dense product with the final weights
    o = bf16_bits(g.standard_normal((T, H, D)))
    eye = bf16_bits(np.broadcast_to(np.eye(D, dtype=np.float32), (H, D, D)))
    wf = bf16_bits(g.standard_normal((d, H * D)))
    out = orc.grouped_projection(o, H, D, eye, wf)
    ref = bf16_vals(o).reshape(T, H * D) @ bf16_vals(wf).T
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)
