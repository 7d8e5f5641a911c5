"""GPU parity of the KV compressors (a1 CSA, a2 HCA) against the oracle.

The HIP compressor merges in fp32 with expf while the oracle merges in double, so fp32
entries are compared to 1e-5 relative; quantised outputs must hold the same codes except
where the two fp32 values straddle a rounding boundary, and there the codes must be
neighbours.  The same holds with the RMSNorm of the merged entries.  Chunked compression
(with the one-block state before each chunk) must give bitwise the whole-sequence entries on
the GPU."""
import numpy as np
import pytest
import torch

import compressed_sparse_attention_02_amd as v4
import oracle
from gpu_util import announce, f32, bf16_from_bits
from workloads import TINY, normal, to_bf16_bits, bf16_bits_to_f64

pytestmark = pytest.mark.gpu


def streams(seed, T, D, G=1, m=4, bf16=False):
    s = dict(kv_a=normal(seed, "kv_a", (T, D)), kv_b=normal(seed, "kv_b", (T, D)),
             gate_a=normal(seed, "gate_a", (T, G)), gate_b=normal(seed, "gate_b", (T, G)),
             bias_a=normal(seed, "bias_a", (m, G)), bias_b=normal(seed, "bias_b", (m, G)))
    if bf16:   # raw KV stored as BF16: both sides read the same BF16 values
        s["kv_a_bits"], s["kv_b_bits"] = to_bf16_bits(s["kv_a"]), to_bf16_bits(s["kv_b"])
        s["kv_a"] = bf16_bits_to_f64(s["kv_a_bits"]).astype(np.float32)
        s["kv_b"] = bf16_bits_to_f64(s["kv_b_bits"]).astype(np.float32)
    return s


def dev_streams(s, bf16=False):
    if bf16:
        a, b = bf16_from_bits(s["kv_a_bits"]), bf16_from_bits(s["kv_b_bits"])
    else:
        a, b = f32(s["kv_a"]), f32(s["kv_b"])
    return a, b, f32(s["gate_a"]), f32(s["gate_b"]), f32(s["bias_a"]), f32(s["bias_b"])


def rel_close(got, ref, tol=1e-5):
    err = np.abs(got.astype(np.float64) - ref.astype(np.float64))
    bound = tol * np.maximum(1.0, np.abs(ref))
    worst = float((err / np.maximum(1.0, np.abs(ref))).max())
    print(f"max relative error {worst:.3e}", flush=True)
    assert (err <= bound).all(), worst


def neighbours_only(got_codes, ref_codes, decode, max_frac=2e-3):
    """Codes equal except isolated neighbours (values one grid step apart)."""
    diff = got_codes != ref_codes
    frac = diff.mean()
    print(f"code mismatches: {int(diff.sum())} of {diff.size}", flush=True)
    assert frac <= max_frac
    for gc, rc in zip(got_codes[diff][:2000], ref_codes[diff][:2000]):
        gv, rv = decode(int(gc)), decode(int(rc))
        lo, hi = min(gv, rv), max(gv, rv)
        between = [c for c in range(256) if lo < decode(c) < hi]
        assert not between, (gc, rc)


@pytest.mark.parametrize("G", [1, 128])
def test_csa_f32_records(G):
    w = TINY
    T, D, R = 2048, w.D, w.R
    s = streams(w.seed, T, D, G)
    announce(f"compress csa f32 G={G}")
    out = v4.KV.empty(1, T // 4, D, R, fmt=v4.V4A_KV_F32)
    v4.v4a_compress_csa(*dev_streams(s), tok0=0, m=4, first_entry=0, n_entries=T // 4, out_kv=out)
    torch.cuda.synchronize()
    ref = oracle.compress_csa(s["kv_a"], s["kv_b"], s["gate_a"], s["gate_b"], s["bias_a"], s["bias_b"],
                              tok0=0, m=4, first_entry=0, n_entries=T // 4, apply_rope=True, R=R)
    rel_close(out.nope[0].cpu().numpy(), ref)


def test_hca_f32_records():
    w = TINY
    T, D, R = 4096, w.D, w.R
    x, gt, bi = normal(w.seed, "kv_h", (T, D)), normal(w.seed, "gate_h", (T, 1)), normal(w.seed, "bias_h", (128, 1))
    announce("compress hca f32")
    out = v4.KV.empty(1, T // 128, D, R, fmt=v4.V4A_KV_F32)
    v4.v4a_compress_hca(f32(x), f32(gt), f32(bi), tok0=0, m=128, first_entry=0, n_entries=T // 128, out_kv=out)
    torch.cuda.synchronize()
    ref = oracle.compress_hca(x, gt, bi, tok0=0, m=128, first_entry=0, n_entries=T // 128, apply_rope=True, R=R)
    rel_close(out.nope[0].cpu().numpy(), ref)


def norm_weights(seed, D):
    """RMSNorm weights in [0.5, 1.5), unequal within RoPE pairs."""
    return (0.5 + np.random.default_rng(seed).random(D)).astype(np.float32)


@pytest.mark.parametrize("G", [1, 128])
def test_csa_f32_records_rmsnorm(G):
    w = TINY
    T, D, R = 2048, w.D, w.R
    s = streams(w.seed + 7, T, D, G)
    nw = norm_weights(60 + G, D)
    announce(f"compress csa f32 rmsnorm G={G}")
    out = v4.KV.empty(1, T // 4, D, R, fmt=v4.V4A_KV_F32)
    v4.v4a_compress_csa(*dev_streams(s), tok0=0, m=4, first_entry=0, n_entries=T // 4, out_kv=out, norm_w=f32(nw))
    torch.cuda.synchronize()
    ref = oracle.compress_csa(s["kv_a"], s["kv_b"], s["gate_a"], s["gate_b"], s["bias_a"], s["bias_b"],
                              tok0=0, m=4, first_entry=0, n_entries=T // 4, apply_rope=True, R=R, norm_w=nw)
    rel_close(out.nope[0].cpu().numpy(), ref)


def test_hca_f32_records_rmsnorm():
    w = TINY
    T, D, R = 4096, w.D, w.R
    x, gt, bi = normal(w.seed, "kv_h", (T, D)), normal(w.seed, "gate_h", (T, 1)), normal(w.seed, "bias_h", (128, 1))
    nw = norm_weights(62, D)
    announce("compress hca f32 rmsnorm")
    out = v4.KV.empty(1, T // 128, D, R, fmt=v4.V4A_KV_F32)
    v4.v4a_compress_hca(f32(x), f32(gt), f32(bi), tok0=0, m=128, first_entry=0, n_entries=T // 128, out_kv=out,
                        norm_w=f32(nw))
    torch.cuda.synchronize()
    ref = oracle.compress_hca(x, gt, bi, tok0=0, m=128, first_entry=0, n_entries=T // 128, apply_rope=True, R=R,
                              norm_w=nw)
    rel_close(out.nope[0].cpu().numpy(), ref)


@pytest.mark.parametrize("norm", [False, True], ids=["plain", "rmsnorm"])
def test_csa_bf16_stream_fp8_records_and_mxfp4_keys(norm):
    T, D, R, dI = 8192, 512, 64, 128
    s = streams(510, T, D, bf16=True)
    nw, nwi = (norm_weights(63, D), norm_weights(64, dI)) if norm else (None, None)
    announce(f"compress csa bf16 -> fp8 records, norm={norm}")
    out = v4.KV.empty(1, T // 4, D, R)
    v4.v4a_compress_csa(*dev_streams(s, bf16=True), tok0=0, m=4, first_entry=0, n_entries=T // 4, out_kv=out,
                        norm_w=f32(nw) if norm else None)
    si = streams(511, T, dI, bf16=True)
    keys = v4.Idx.empty(1, T // 4, dI)
    v4.v4a_compress_csa(*dev_streams(si, bf16=True), tok0=0, m=4, first_entry=0, n_entries=T // 4, out_idx=keys,
                        norm_w=f32(nwi) if norm else None)
    torch.cuda.synchronize()
    ref = oracle.compress_csa(s["kv_a"], s["kv_b"], s["gate_a"], s["gate_b"], s["bias_a"], s["bias_b"], tok0=0,
                              m=4, first_entry=0, n_entries=T // 4, apply_rope=True, R=R, norm_w=nw)
    nope, rope, scale = oracle.quant_kv(ref, R)
    got_scale = out.scale[0].cpu().numpy()
    rel_close(got_scale, scale)
    neighbours_only(out.nope[0].cpu().numpy(), nope, oracle.e4m3_decode)
    # BF16 RoPE dims: equal, or one BF16 spacing apart where the fp32 entries straddle a rounding
    # boundary (values near zero may also flip sign within the fp32 difference)
    gv = bf16_bits_to_f64(out.rope[0].cpu().numpy().view(np.uint16))
    rv = bf16_bits_to_f64(rope)
    spacing = np.exp2(np.floor(np.log2(np.maximum(np.maximum(np.abs(gv), np.abs(rv)), 1e-30))) - 7)
    diff = np.abs(gv - rv)
    print(f"bf16 mismatches: {int((diff > 0).sum())} of {diff.size}", flush=True)
    assert (diff <= spacing + 1e-6).all() and (diff > 0).mean() < 2e-3
    refk = oracle.compress_csa(si["kv_a"], si["kv_b"], si["gate_a"], si["gate_b"], si["bias_a"], si["bias_b"],
                               tok0=0, m=4, first_entry=0, n_entries=T // 4, apply_rope=False, R=0, norm_w=nwi)
    kc, ks = oracle.quant_mxfp4(refk)
    gs = keys.scales[0].cpu().numpy()
    assert (gs != ks).mean() < 1e-3
    gc = keys.codes[0].cpu().numpy()
    same_scale = np.repeat(gs == ks, 16, axis=1)
    lo_g, lo_r = gc & 15, kc & 15
    hi_g, hi_r = gc >> 4, kc >> 4
    for a, b in ((lo_g, lo_r), (hi_g, hi_r)):
        neighbours_only(a[same_scale], b[same_scale], lambda c: oracle.e2m1_decode(c & 15))


def test_chunked_equals_whole_on_gpu():
    T, D, R = 4096, 512, 64
    s = streams(520, T, D)
    announce("compress chunk invariance")
    whole = v4.KV.empty(1, T // 4, D, R)
    v4.v4a_compress_csa(*dev_streams(s), tok0=0, m=4, first_entry=0, n_entries=T // 4, out_kv=whole)
    parts = v4.KV.empty(1, T // 4, D, R)
    for c0 in range(0, T, 1024):
        r0 = max(0, c0 - 4)
        sl = {k: v[r0:c0 + 1024] if k.startswith(("kv", "gate")) else v for k, v in s.items()}
        v4.v4a_compress_csa(*dev_streams(sl), tok0=r0, m=4, first_entry=c0 // 4, n_entries=256, out_kv=parts)
    hw = v4.KV.empty(1, T // 128, D, R)
    hp = v4.KV.empty(1, T // 128, D, R)
    x, gt, bi = normal(521, "kv_h", (T, D)), normal(521, "gate_h", (T, 1)), normal(521, "bias_h", (128, 1))
    v4.v4a_compress_hca(f32(x), f32(gt), f32(bi), tok0=0, m=128, first_entry=0, n_entries=T // 128, out_kv=hw)
    for c0 in range(0, T, 1024):
        v4.v4a_compress_hca(f32(x[c0:c0 + 1024]), f32(gt[c0:c0 + 1024]), f32(bi), tok0=c0, m=128,
                            first_entry=c0 // 128, n_entries=8, out_kv=hp)
    torch.cuda.synchronize()
    for a, b in ((whole, parts), (hw, hp)):
        assert torch.equal(a.nope, b.nope) and torch.equal(a.rope, b.rope) and torch.equal(a.scale, b.scale)


def test_unaligned_bf16_streams_equal_aligned():
    """Streams that start 2 bytes past an aligned address take the element-wise load path;
    the entries (CSA records and keys, HCA records) are bitwise those of aligned streams."""
    T, D, R, dI = 1024, 512, 64, 128
    announce("compress with unaligned bf16 streams")

    def shifted(t):  # the same values, starting one BF16 element past a 256-byte boundary
        buf = torch.empty(t.numel() + 1, dtype=t.dtype, device=t.device)
        out = buf[1:].view(t.shape)
        out.copy_(t)
        return out

    for d, to_idx in ((D, False), (dI, True)):
        s = streams(530 + d, T, d, bf16=True)
        a, b, ga, gb, ba, bb = dev_streams(s, bf16=True)
        res = []
        for xa, xb in ((a, b), (shifted(a), shifted(b))):
            assert (xa.data_ptr() % 16 == 0) == (xa is a)
            out = v4.Idx.empty(1, T // 4, d) if to_idx else v4.KV.empty(1, T // 4, d, R)
            v4.v4a_compress_csa(xa, xb, ga, gb, ba, bb, tok0=0, m=4, first_entry=0, n_entries=T // 4,
                                **({"out_idx": out} if to_idx else {"out_kv": out}))
            res.append(out)
        torch.cuda.synchronize()
        if to_idx:
            assert torch.equal(res[0].codes, res[1].codes) and torch.equal(res[0].scales, res[1].scales)
        else:
            assert torch.equal(res[0].nope, res[1].nope) and torch.equal(res[0].rope, res[1].rope)
            assert torch.equal(res[0].scale, res[1].scale)
    x = bf16_from_bits(to_bf16_bits(normal(532, "kv_h", (T, D))))
    gt, bi = f32(normal(532, "gate_h", (T, 1))), f32(normal(532, "bias_h", (128, 1)))
    res = []
    for xs in (x, shifted(x)):
        out = v4.KV.empty(1, T // 128, D, R)
        v4.v4a_compress_hca(xs, gt, bi, tok0=0, m=128, first_entry=0, n_entries=T // 128, out_kv=out)
        res.append(out)
    torch.cuda.synchronize()
    assert torch.equal(res[0].nope, res[1].nope) and torch.equal(res[0].rope, res[1].rope)
    assert torch.equal(res[0].scale, res[1].scale)
