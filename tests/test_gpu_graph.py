"""Graph capture of a CSA decode step (indexer + top-k + attention through the C ABI on the
capture stream): every replay, with eager work and synchronisations between replays, must
reproduce the eager result bit for bit (the kernels are deterministic and the library
records no runtime memset into the graph)."""
import numpy as np
import pytest
import torch

import compressed_sparse_attention_02_amd as v4
from gpu_util import announce, f32, idx_from_f32, kv_from_f32
from workloads import normal, to_bf16_bits

pytestmark = pytest.mark.gpu


def test_graph_replays_match_eager():
    B, N, H, HI, D, R, W, k = 2, 20000, 64, 64, 512, 64, 128, 512
    announce("graph capture of a csa decode step")
    kv = kv_from_f32(normal(600, "records", (B, N, D)), R)
    keys = idx_from_f32(normal(600, "keys", (B, N, 128)))
    qi = idx_from_f32(normal(600, "q_idx", (B, HI, 128)))
    w = f32(normal(600, "w", (B, HI)))
    q = torch.from_numpy(to_bf16_bits(normal(600, "q", (B, H, D))).view(np.int16)).view(torch.bfloat16).cuda()
    win = torch.from_numpy(to_bf16_bits(normal(600, "window", (B, W, D))).view(np.int16)).view(torch.bfloat16).cuda()
    sink = f32(normal(600, "sink", (H,)))
    sel = torch.empty((B, 1, k), dtype=torch.int32, device="cuda")
    out = torch.empty((B, H, D), dtype=torch.bfloat16, device="cuda")
    ws = v4.workspace(max(v4.v4a_indexer_topk_workspace(B, 1, N, k), v4.v4a_decode_workspace(B, H, D, k, W)))
    q_pos = [4 * N - 1] * B

    def step():
        v4.v4a_indexer_topk(keys, [N] * B, 4, qi, w, B, 1, HI, q_pos, k, sel, ws)
        v4.v4a_decode_csa(q, kv, sel.view(B, k), k, win, [W] * B, W, sink, q_pos,
                          softmax_scale=1.0 / np.sqrt(D), out=out, ws=ws)

    step()
    torch.cuda.synchronize()
    ref_sel, ref_out = sel.clone(), out.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(4):
        sel.fill_(-5)
        out.zero_()
        ws.fill_(0xAB)                       # eager work that scribbles over the workspace
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(sel, ref_sel), rep
        assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16)), rep
