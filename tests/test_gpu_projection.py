"""GPU parity of the grouped output projection (v4a_output_projection; "DeepSeek-V4 technical report
walkthrough" (cyqw.cn), section 2.2, Grouped Output Projection) against the oracle.

Stage by stage, since the reduced groups y are a BF16 rounding decided in floating point: the
GPU's y against the oracle's, then the GPU's output against the oracle's final projection of the
GPU's y.  Per element the bar is one BF16 spacing of the reference (the two sums may fall on
either side of a rounding midpoint) plus the fp32 accumulation error, taken as
2^-24 * 4 sqrt(K) * sum_c |x_c w_c| (products of BF16 values are exact in fp32; the sum's
rounding errors add up like a random walk over the K terms).  Near zero the second term is the
larger one.  At most 1% of the y elements may differ at all; BF16 outputs also keep relative
L2 <= 5e-3, fp32 outputs relative L2 <= 1e-4.  Shapes: the decode workload (4 tokens, 128 heads of 512, 16
groups reduced to 1024, projected to 7168), ragged token counts on all three kernels (1 .. 8
tokens on the LDS-staged GEMV, 9 .. 64 on the skinny one, 65 .. 300 with partial tiles on the
tiled one), a final stage whose K (384) is not a multiple of 512 (the GEMV's limit, so the
skinny kernel takes it), and the 4096-token prefill chunk on sampled tokens."""
import numpy as np
import pytest
import torch

import compressed_sparse_attention_02_amd as v4
import oracle
from gpu_util import announce, bf16_from_bits, bf16_round, bf16_ulp
from workloads import bf16_bits_to_f64, normal, to_bf16_bits

pytestmark = pytest.mark.gpu


def make(seed, T, H, D, G, r, d):
    Kg = H * D // G
    o = to_bf16_bits(0.3 * normal(seed, "o_attn", (T, H, D), threads=16))
    wg = to_bf16_bits(normal(seed, "w_group", (G, r, Kg), threads=16) / np.float32(np.sqrt(Kg)))
    wf = to_bf16_bits(normal(seed, "w_final", (d, G * r), threads=16) / np.float32(np.sqrt(G * r)))
    return o, wg, wf


def run(o, wg, wf, G, r, out_dtype=torch.bfloat16):
    T = o.shape[0]
    d = wf.shape[0]
    out = torch.empty((T, d), dtype=out_dtype, device="cuda")
    ws = v4.workspace(v4.v4a_output_projection_workspace(T, G, r))
    v4.v4a_output_projection(bf16_from_bits(o), G, r, bf16_from_bits(wg), bf16_from_bits(wf), out, ws)
    torch.cuda.synchronize()
    y = bf16_bits_to_f64(ws[:T * G * r * 2].view(torch.int16).cpu().numpy().view(np.uint16)).reshape(T, G * r)
    return y, out.float().cpu().numpy().astype(np.float64)


def fp32_sum_error(x_abs, w_abs):
    """2^-24 * 4 sqrt(K) * sum_c |x_c| |w_c| for every (row of x_abs, row of w_abs)."""
    K = x_abs.shape[1]
    return 2.0 ** -24 * 4.0 * np.sqrt(K) * (x_abs @ w_abs.T)


def within(got, ref, slack, what):
    err = np.abs(got - ref)
    bar = bf16_ulp(ref) * 1.0000001 + slack
    worst = np.unravel_index(int(np.argmax(err - bar)), err.shape)
    assert (err <= bar).all(), (f"{what}: element {tuple(int(i) for i in worst)} got {got[worst]:.8g} ref "
                                f"{ref[worst]:.8g} (bar {bar[worst]:.3g})")


def check(o, wg, wf, G, r, y_gpu, out_gpu, rows, bf16_out=True, what=""):
    y_ref = oracle.group_reduce(o[rows], G, r, wg)
    yg = y_gpu[rows]
    T, H, D = o.shape
    Kg = H * D // G
    ov = np.abs(bf16_bits_to_f64(o[rows])).reshape(len(rows), G, Kg)
    wgv = np.abs(bf16_bits_to_f64(wg))
    slack = np.concatenate([fp32_sum_error(ov[:, g], wgv[g]) for g in range(G)], axis=1)
    within(yg, y_ref, slack, f"{what}: y")
    frac = float((yg != y_ref).mean())
    print(f"{what}: y elements one BF16 spacing apart: {frac:.2e}", flush=True)
    assert frac <= 0.01, f"{what}: y differs in {frac:.2%} of the elements"
    z = oracle.project(yg, wf)
    got = out_gpu[rows]
    zslack = fp32_sum_error(np.abs(yg), np.abs(bf16_bits_to_f64(wf)))
    if bf16_out:
        ref = bf16_round(z)
        within(got, ref, zslack, f"{what}: out")
        rl = float(np.linalg.norm(got - ref) / np.linalg.norm(ref))
        print(f"{what}: out rel-L2 {rl:.3e}", flush=True)
        assert rl <= 5e-3, f"{what}: rel-L2 {rl:.3e}"
    else:
        assert (np.abs(got - z) <= zslack + 1e-30).all(), f"{what}: fp32 out beyond the fp32 sum error"
        rl = float(np.linalg.norm(got - z) / np.linalg.norm(z))
        print(f"{what}: out rel-L2 {rl:.3e}", flush=True)
        assert rl <= 1e-4, f"{what}: rel-L2 {rl:.3e}"


def test_decode_shape():
    T, H, D, G, r, d = 4, 128, 512, 16, 1024, 7168
    o, wg, wf = make(810, T, H, D, G, r, d)
    announce("output projection, decode shape (GEMV kernel)")
    y, out = run(o, wg, wf, G, r)
    check(o, wg, wf, G, r, y, out, np.arange(T), what="decode")
    _, out32 = run(o, wg, wf, G, r, torch.float32)
    check(o, wg, wf, G, r, y, out32, np.arange(T), bf16_out=False, what="decode fp32 out")


def kernel_name(T):
    return "gemv" if T <= 8 else "skinny" if T <= 64 else "tiled"


@pytest.mark.parametrize("T", [1, 2, 5, 8, 9, 17, 33, 64, 65, 200, 300])
def test_ragged_tokens(T):
    H, D, G, r, d = 16, 512, 4, 256, 400
    o, wg, wf = make(820 + T, T, H, D, G, r, d)
    announce(f"output projection, T={T} ({kernel_name(T)} kernel)")
    y, out = run(o, wg, wf, G, r)
    check(o, wg, wf, G, r, y, out, np.arange(T), what=f"T={T}")


@pytest.mark.parametrize("T", [3, 8])
def test_final_k_not_multiple_of_512(T):
    # group stage K = 2048 (GEMV), final stage K = G*r = 384 (skinny kernel)
    H, D, G, r, d = 16, 512, 4, 96, 272
    o, wg, wf = make(840 + T, T, H, D, G, r, d)
    announce(f"output projection, T={T}, final K=384")
    y, out = run(o, wg, wf, G, r)
    check(o, wg, wf, G, r, y, out, np.arange(T), what=f"T={T} K=384")


def test_prefill_shape_sampled():
    T, H, D, G, r, d = 4096, 128, 512, 16, 1024, 7168
    o, wg, wf = make(830, T, H, D, G, r, d)
    announce("output projection, 4096-token prefill chunk (tiled kernel)")
    y, out = run(o, wg, wf, G, r)
    rows = np.array(sorted(set(range(0, T, 256)) | {127, 128, 129, 4095}))
    check(o, wg, wf, G, r, y, out, rows, what="prefill")
