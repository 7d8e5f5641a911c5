"""GPU check of v4a_decode_step_csa_noalloc, the fused CSA decode step on the library's own
per-device scratch: two calls in a row, the second with a smaller batch, fewer entries and a
smaller k, each bitwise equal (output, record cache, key cache) to v4a_decode_step_csa with the
same arguments on a fresh caller workspace.  The second call finds the first call's contents in
the scratch, so it also checks that the call clears what must start at zero."""
import math

import numpy as np
import pytest
import torch

import compressed_sparse_attention_02_amd as v4
from gpu_util import announce, bf16_from_bits, f32
from workloads import normal, to_bf16_bits

pytestmark = pytest.mark.gpu


def clone_kv(kv):
    return v4.KV(kv.fmt, kv.D, kv.R, kv.nope.clone(), kv.rope.clone(), kv.scale.clone(), kv.cap)


def clone_idx(ix):
    return v4.Idx(ix.fmt, ix.d, ix.codes.clone(), ix.scales.clone(), ix.cap)


def make_step(seed, q_pos, cap, k, H=128, HI=64):
    m, D, R, dI, W = 4, 512, 64, 128, 128
    B = len(q_pos)
    kv = v4.KV.empty(B, cap, D, R)
    v4.v4a_quantize_kv(f32(normal(seed, "records", (B * cap, D), threads=16)), kv, 0)
    keys = v4.Idx.empty(B, cap, dI)
    v4.v4a_quantize_mxfp4(f32(normal(seed, "keys", (B * cap, dI), threads=16)), keys, 0)
    qi = v4.Idx.empty(B, HI, dI)
    v4.v4a_quantize_mxfp4(f32(normal(seed, "q_idx", (B * HI, dI))), qi)
    rows = {n: bf16_from_bits(to_bf16_bits(normal(seed, n, (B, 2 * m, D if n.startswith("kv") else dI))))
            for n in ("kv_a", "kv_b", "idx_a", "idx_b")}
    gates = {n: f32(normal(seed, n, (B, 2 * m, 1))) for n in ("gate_a", "gate_b", "idx_gate_a", "idx_gate_b")}
    bias = {n: f32(normal(seed, n, (m, 1))) for n in ("bias_a", "bias_b", "idx_bias_a", "idx_bias_b")}
    common = dict(q_pos=q_pos, n_entries=[(p + 1) // m for p in q_pos], m=m, q_idx=qi,
                  w=f32(normal(seed, "w", (B, HI))), k=k,
                  q=bf16_from_bits(to_bf16_bits(normal(seed, "q", (B, H, D)))),
                  win=bf16_from_bits(to_bf16_bits(normal(seed, "window", (B, W, D)))),
                  win_len=[min(W, p + 1) for p in q_pos], W=W, sink=f32(normal(seed, "sink", (H,))),
                  softmax_scale=1.0 / math.sqrt(D), **rows, **gates, **bias)
    return kv, keys, common, (B, H, D)


@pytest.mark.parametrize("clean_flag", [False, True], ids=["ws_clean_0", "ws_clean_1"])
def test_noalloc_equals_workspace_call_twice(clean_flag):
    # first call: 4 sequences (1M-context style positions scaled down), k = 1024; second call: a
    # smaller input (2 sequences, fewer entries, k = 512), on the same device's scratch
    cases = [(901, [4 * 30000 - 1, 4 * 29000 + 2, 4 * 25000 - 1, 4 * 30000 - 1], 30016, 1024),
             (902, [4 * 6000 - 1, 4 * 5000 + 1], 6016, 512)]
    for seed, q_pos, cap, k in cases:
        kv, keys, common, shape = make_step(seed, q_pos, cap, k)
        outs = []
        for noalloc in (True, False):
            kv1, keys1 = clone_kv(kv), clone_idx(keys)
            out = torch.empty(shape, dtype=torch.bfloat16, device="cuda")
            # ws_clean is ignored by the scratch variant: it always clears the histograms
            args = v4.DecodeStepArgs(kv=kv1, keys=keys1, out=out, ws_clean=clean_flag and noalloc, **common)
            need = v4.v4a_decode_step_workspace(args)
            assert 0 < need <= v4.V4A_NOALLOC_SCRATCH_BYTES
            announce(f"decode step noalloc={noalloc}: B={len(q_pos)} k={k} needs {need} bytes")
            if noalloc:
                v4.v4a_decode_step_csa_noalloc(args)
            else:
                ws = v4.workspace(need)
                ws.fill_(0x55)  # a dirty workspace: the call clears what it needs itself
                v4.v4a_decode_step_csa(args, ws)
            torch.cuda.synchronize()
            outs.append((out, kv1, keys1))
        (o1, k1, i1), (o2, k2, i2) = outs
        assert not torch.equal(k1.nope, kv.nope)
        for a, c in ((o1, o2), (k1.nope, k2.nope), (k1.rope, k2.rope), (k1.scale, k2.scale), (i1.codes, i2.codes),
                     (i1.scales, i2.scales)):
            assert torch.equal(a, c)
        assert torch.isfinite(o1.float()).all()
