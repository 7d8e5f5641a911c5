"""CPU checks of the C ABI: the library loads, exports every entry point include/v4attn.h
declares, sizes workspaces, and rejects bad arguments on the host before any launch (these
calls never reach the GPU, so they run without one)."""
import ctypes
import re

import numpy as np
import pytest

import compressed_sparse_attention_02_amd as v4

FAKE = 0x10000  # an aligned address that host validation never dereferences


def declared_symbols():
    text = open(v4.HEADER).read()
    return sorted(set(re.findall(r"^V4A_API\s+[\w\s\*]*?\b(v4a_\w+)\s*\(", text, re.M)))


def test_library_exports_every_declared_symbol():
    L = v4.lib()
    names = declared_symbols()
    assert len(names) >= 12
    for n in names:
        assert hasattr(L, n), n
    assert v4.v4a_version().startswith("v4attn")


def kv(fmt=v4.V4A_KV_FP8_BF16, D=512, R=64, cap=100, nope=FAKE, rope=FAKE, scale=FAKE):
    return v4.c_kv(fmt, D, R, nope, rope, scale, cap)


def idx(fmt=v4.V4A_IDX_MXFP4, d=128, cap=100, codes=FAKE, scales=FAKE):
    return v4.c_idx(fmt, d, codes, scales, cap)


def i64(*v):
    return (ctypes.c_int64 * len(v))(*v)


def i32(*v):
    return (ctypes.c_int32 * len(v))(*v)


def status(name, *args):
    return getattr(v4.lib(), name)(*args)


def test_workspace_sizes_are_monotone_and_aligned():
    a = v4.v4a_indexer_topk_workspace(4, 1, 262144, 1024)
    b = v4.v4a_indexer_topk_workspace(4, 1, 262145, 1024)
    assert a > 4 * 262144 * 12 and b >= a and a % 256 == 0
    # BF16 partial sums of 16 splits plus their fp32 (m, l)
    assert v4.v4a_decode_workspace(16, 128, 512, 8192, 128) >= 16 * 16 * 128 * (512 * 2 + 8)
    assert v4.v4a_decode_workspace(1, 8, 128, 0, 0) == 0   # a single split needs no partials


def test_quantize_rejects():
    L = v4.lib()
    assert L.v4a_quantize_kv(FAKE, 10, None, 0, None) == 1
    assert L.v4a_quantize_kv(FAKE, -1, ctypes.byref(kv()), 0, None) == 1
    assert L.v4a_quantize_kv(FAKE, 10, ctypes.byref(kv(D=500, R=64)), 0, None) == 2
    assert L.v4a_quantize_kv(FAKE + 4, 10, ctypes.byref(kv()), 0, None) == 1   # misaligned x
    assert L.v4a_quantize_mxfp4(FAKE, 10, ctypes.byref(idx(d=100)), 0, None) == 2
    assert L.v4a_quantize_mxfp4(FAKE, 10, ctypes.byref(idx(scales=0)), 0, None) == 1
    assert "scales" in v4.lib().v4a_last_error().decode()


def test_compress_rejects():
    L = v4.lib()
    out = kv(D=512, R=64, cap=1000)
    args = dict(kv_a=FAKE, kv_b=FAKE, in_t=1, D=512, ga=FAKE, gb=FAKE, G=1, ba=FAKE, bb=FAKE,
                tok0=0, n_tok=4096, m=4, first=0, n=1024, rope=1)

    def call(**kw):
        a = dict(args)
        a.update(kw)
        return L.v4a_compress_csa(a["kv_a"], a["kv_b"], a["in_t"], a["D"], a["ga"], a["gb"], a["G"],
                                  a["ba"], a["bb"], a["tok0"], a["n_tok"], a["m"], a["first"], a["n"],
                                  a["rope"], 10000.0, a.get("norm", None),
                                  ctypes.byref(a.get("out", out)), a.get("oidx", None), 0, 1, None)
    assert call(m=0) == 2
    assert call(m=129) == 2
    assert call(G=7) == 2
    assert call(tok0=2) == 1                      # not a multiple of m
    assert call(n_tok=4095) == 1                  # last block uncovered
    assert call(first=10, tok0=40) == 1           # B-block of entry 10 starts at 36
    assert call(norm=FAKE + 2) == 1               # misaligned RMSNorm weights
    assert call(out=kv(D=512, R=64, cap=1000), n=1001) == 1
    assert call(oidx=ctypes.byref(idx())) == 1     # both outputs given
    assert call(kv_a=0) == 1


def test_indexer_rejects():
    L = v4.lib()
    keys, q = idx(cap=1000), idx(cap=64)
    n, pos, out = i64(1000), i64(3999), FAKE

    def call(keys=keys, q=q, H_I=64, k=512, B=1, Q=1, m=4, ws=FAKE, wsb=1 << 30, n=n, pos=pos):
        return L.v4a_indexer_topk(ctypes.byref(keys), n, m, ctypes.byref(q), FAKE, B, Q, H_I, pos, k,
                                  out, ws, wsb, None)
    assert call(H_I=6) == 2
    assert call(H_I=68) == 2
    assert call(k=0) == 2 and call(k=4096) == 2
    assert call(q=idx(cap=32)) == 1                  # Q*H_I rows do not fit
    assert call(keys=idx(d=64, cap=1000)) == 1       # d differs from q
    assert call(keys=idx(d=64, cap=1000), q=idx(d=64, cap=64)) == 2   # MXFP4 needs d = 128
    assert call(n=i64(2000)) == 1                    # more entries than capacity
    assert call(pos=i64(-1)) == 1
    assert call(wsb=100) == 3
    assert call(ws=FAKE + 8) == 3
    assert call(B=200) == 2


def test_decode_rejects():
    L = v4.lib()
    rec = kv(cap=1000)
    win_len, pos = i32(128), i64(4095)
    sink = FAKE

    def call(H=128, W=128, k=1024, wl=win_len, rec=rec, ws=FAKE, wsb=1 << 30, q=FAKE):
        return L.v4a_decode_csa(q, 1, 1, H, ctypes.byref(rec), FAKE, k, FAKE, 1, wl, W, sink, pos,
                                0.04, 1, 10000.0, FAKE, 1, ws, wsb, None)
    assert call(H=0) == 2 and call(H=256) == 2
    assert call(W=129) == 2
    assert call(wl=i32(129)) == 1
    assert call(k=0) == 2
    assert call(wsb=16) == 3
    assert call(q=FAKE + 2) == 1
    assert call(rec=kv(D=512, R=64, cap=0)) == 1
    assert L.v4a_decode_hca(FAKE, 1, 1, 128, ctypes.byref(rec), i64(2000), 128, FAKE, 1, win_len, 128,
                            sink, pos, 0.04, 1, 10000.0, FAKE, 1, FAKE, 1 << 30, None) == 1


def test_prefill_args_layout_matches_the_header(tmp_path):
    """The binding's v4a_prefill_args has the C struct's size and field offsets (gcc on the header)."""
    import subprocess
    fields = [f for f, _ in v4.c_prefill_args._fields_]
    src = tmp_path / "layout.c"
    src.write_text('#include <stdio.h>\n#include <stddef.h>\n#include "v4attn.h"\nint main(void){\n'
                   '  printf("%zu\\n", sizeof(v4a_prefill_args));\n' +
                   "".join(f'  printf("%zu\\n", offsetof(v4a_prefill_args, {f}));\n' for f in fields) +
                   "  return 0;\n}\n")
    exe = tmp_path / "layout"
    inc = str(v4.HEADER).rsplit("/", 1)[0]
    subprocess.run(["gcc", "-std=c11", "-I", inc, str(src), "-o", str(exe)], check=True)
    got = [int(x) for x in subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split()]
    assert got[0] == ctypes.sizeof(v4.c_prefill_args)
    assert got[1:] == [getattr(v4.c_prefill_args, f).offset for f in fields]


def prefill_struct(**kw):
    """A valid CSA prefill chunk at the long-context prefill shape (fake device pointers)."""
    rec, keys, q_idx = kv(cap=17408), idx(cap=17408), idx(cap=4096 * 64)
    a = dict(tok0=65536, C=4096, n_prev=128, m=4, in_t=1, G=1, kv_a=FAKE, kv_b=FAKE, gate_a=FAKE, gate_b=FAKE,
             bias_a=FAKE, bias_b=FAKE, apply_rope=1, rope_theta=10000.0, kv=ctypes.pointer(rec), slot=0, idx_G=1,
             idx_a=FAKE, idx_b=FAKE, idx_gate_a=FAKE, idx_gate_b=FAKE, idx_bias_a=FAKE, idx_bias_b=FAKE,
             keys=ctypes.pointer(keys), q_idx=ctypes.pointer(q_idx), w=FAKE, H_I=64, k=1024, q=FAKE, q_t=1,
             H=128, W=128, sink=FAKE, softmax_scale=0.044, out_rope_inverse=1, out=FAKE, out_t=1)
    a.update(kw)
    s = v4.c_prefill_args(**a)
    s._keep = (rec, keys, q_idx, a)
    return s


def test_prefill_workspace_and_rejects():
    L = v4.lib()
    csa, hca = v4.V4A_LAYER_CSA, v4.V4A_LAYER_HCA
    s = prefill_struct()
    need = L.v4a_prefill_workspace(csa, ctypes.byref(s))
    # the chunk's top-k lists plus the indexer workspace for 4096 queries over 17408 entries
    assert need >= 4096 * 1024 * 4 + v4.v4a_indexer_topk_workspace(1, 4096, 17408, 1024) - 256
    assert need % 256 == 0

    def call(kind=csa, ws=FAKE, wsb=1 << 40, **kw):
        return L.v4a_prefill_chunk(kind, ctypes.byref(prefill_struct(**kw)), ws, wsb, None)
    assert L.v4a_prefill_chunk(csa, None, FAKE, 1 << 40, None) == 1
    assert call(kind=7) == 1
    assert call(tok0=65537) == 1                 # not a multiple of m
    assert call(n_prev=100) == 1                 # the window needs 127 rows before tok0
    assert call(n_prev=70000) == 1               # more rows than positions before tok0
    assert call(tok0=0, n_prev=0, C=70000) == 2
    assert call(kv=ctypes.pointer(kv(cap=16000))) == 1     # 17408 entries do not fit
    assert call(k=4096) == 2
    assert call(H_I=6) == 2
    assert call(kv_b=0) == 1
    assert call(wsb=need - 1) == 3
    assert call(ws=FAKE + 64) == 3
    assert call(q=FAKE + 2) == 1
    assert call(W=129) == 2
    assert call(G=7) == 2
    # HCA: m' = 128, no indexer, no workspace
    h = prefill_struct(m=128, kv_b=0, gate_b=0, bias_b=0, keys=None, q_idx=None, w=0, k=0)
    assert L.v4a_prefill_workspace(hca, ctypes.byref(h)) == 0
    assert L.v4a_prefill_chunk(hca, ctypes.byref(prefill_struct(m=128, tok0=65600)), None, 0, None) == 1


def test_decode_step_args_layout_matches_the_header(tmp_path):
    import subprocess
    fields = [f for f, _ in v4.c_decode_step_args._fields_]
    src = tmp_path / "layout2.c"
    src.write_text('#include <stdio.h>\n#include <stddef.h>\n#include "v4attn.h"\nint main(void){\n'
                   '  printf("%zu\\n", sizeof(v4a_decode_step_args));\n' +
                   "".join(f'  printf("%zu\\n", offsetof(v4a_decode_step_args, {f}));\n' for f in fields) +
                   "  return 0;\n}\n")
    exe = tmp_path / "layout2"
    inc = str(v4.HEADER).rsplit("/", 1)[0]
    subprocess.run(["gcc", "-std=c11", "-I", inc, str(src), "-o", str(exe)], check=True)
    got = [int(x) for x in subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split()]
    assert got[0] == ctypes.sizeof(v4.c_decode_step_args)
    assert got[1:] == [getattr(v4.c_decode_step_args, f).offset for f in fields]


def step_struct(**kw):
    """A valid fused CSA decode step at the 1M-context shape (fake device pointers)."""
    rec, keys, q_idx = kv(cap=262144), idx(cap=262144), idx(cap=64)
    pos, nent, wl = i64(*[1048575] * 4), i64(*[262144] * 4), i32(*[128] * 4)
    a = dict(B=4, m=4, q_pos=ctypes.cast(pos, ctypes.c_void_p), n_entries=ctypes.cast(nent, ctypes.c_void_p), in_t=1,
             G=1, idx_G=1, kv_a=FAKE, kv_b=FAKE, gate_a=FAKE, gate_b=FAKE, bias_a=FAKE, bias_b=FAKE, idx_a=FAKE,
             idx_b=FAKE, idx_gate_a=FAKE, idx_gate_b=FAKE, idx_bias_a=FAKE, idx_bias_b=FAKE, apply_rope=1,
             rope_theta=10000.0, kv=ctypes.pointer(rec), keys=ctypes.pointer(keys), q_idx=ctypes.pointer(q_idx),
             w=FAKE, H_I=64, k=1024, q=FAKE, q_t=1, H=128, win=FAKE, win_t=1, win_len=ctypes.cast(wl, ctypes.c_void_p),
             W=128, sink=FAKE, softmax_scale=0.044, out_rope_inverse=1, out=FAKE, out_t=1)
    a.update(kw)
    s = v4.c_decode_step_args(**a)
    s._keep = (rec, keys, q_idx, pos, nent, wl, a)
    return s


def test_decode_step_workspace_and_rejects():
    L = v4.lib()
    s = step_struct()
    need = L.v4a_decode_step_workspace(ctypes.byref(s))
    # the top-k lists, the indexer workspace and the BF16 split partials of 1152 keys (18 splits)
    assert need >= 4 * 1024 * 4 + v4.v4a_indexer_topk_workspace(4, 1, 262144, 1024) + 4 * 18 * 128 * (512 * 2 + 8)
    assert need % 256 == 0

    def call(ws=FAKE, wsb=1 << 40, **kw):
        return L.v4a_decode_step_csa(ctypes.byref(step_struct(**kw)), ws, wsb, None)
    assert L.v4a_decode_step_csa(None, FAKE, 1 << 40, None) == 1
    assert call(B=0) == 2 and call(B=200) == 2
    assert call(k=0) == 2
    assert call(H_I=6) == 2
    assert call(H=24) == 2                                   # not a multiple of 16: no MFMA attention
    assert call(keys=ctypes.pointer(idx(d=64, cap=262144))) == 2
    assert call(kv_b=0) == 1
    assert call(wsb=need - 1) == 3
    assert call(ws=FAKE + 64) == 3
    pos = i64(*[1048575] * 4)
    short = i64(262143, 262144, 262144, 262144)   # sequence 0 would not hold the entry it completes
    assert call(n_entries=ctypes.cast(short, ctypes.c_void_p), q_pos=ctypes.cast(pos, ctypes.c_void_p)) == 1


def test_decode_step_noalloc_rejects_before_any_hip_call():
    """The entry point without a workspace validates like v4a_decode_step_csa and refuses
    arguments whose scratch exceeds the library's per-device array, before touching the device."""
    L = v4.lib()
    assert L.v4a_decode_step_csa_noalloc(None, None) == 1
    assert L.v4a_decode_step_csa_noalloc(ctypes.byref(step_struct(k=0)), None) == 2
    assert L.v4a_decode_step_csa_noalloc(ctypes.byref(step_struct(kv_b=0)), None) == 1
    # 128 sequences at the 1M-context shape need far more than 64 MiB of scratch
    B = 128
    pos, nent, wl = i64(*[1048575] * B), i64(*[262144] * B), i32(*[128] * B)
    big = step_struct(B=B, q_pos=ctypes.cast(pos, ctypes.c_void_p), n_entries=ctypes.cast(nent, ctypes.c_void_p),
                      win_len=ctypes.cast(wl, ctypes.c_void_p), q_idx=ctypes.pointer(idx(cap=64)))
    big._keep2 = (pos, nent, wl)
    assert L.v4a_decode_step_workspace(ctypes.byref(big)) > v4.V4A_NOALLOC_SCRATCH_BYTES
    assert L.v4a_decode_step_csa_noalloc(ctypes.byref(big), None) == 3
    assert b"scratch" in L.v4a_last_error()
    # the 1M-context step of 4 sequences fits
    assert L.v4a_decode_step_workspace(ctypes.byref(step_struct())) <= v4.V4A_NOALLOC_SCRATCH_BYTES


def test_trace_without_marks_is_an_error():
    # no trace has recorded anything in this process: asking for a mark fails before any HIP call
    assert v4.v4a_trace_end() == 0
    with pytest.raises(v4.V4AError):
        v4.v4a_trace_kernel(0)


def test_decode_step_hca_args_layout_matches_the_header(tmp_path):
    import subprocess
    fields = [f for f, _ in v4.c_decode_step_hca_args._fields_]
    src = tmp_path / "layout3.c"
    src.write_text('#include <stdio.h>\n#include <stddef.h>\n#include "v4attn.h"\nint main(void){\n'
                   '  printf("%zu\\n", sizeof(v4a_decode_step_hca_args));\n' +
                   "".join(f'  printf("%zu\\n", offsetof(v4a_decode_step_hca_args, {f}));\n' for f in fields) +
                   "  return 0;\n}\n")
    exe = tmp_path / "layout3"
    inc = str(v4.HEADER).rsplit("/", 1)[0]
    subprocess.run(["gcc", "-std=c11", "-I", inc, str(src), "-o", str(exe)], check=True)
    got = [int(x) for x in subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split()]
    assert got[0] == ctypes.sizeof(v4.c_decode_step_hca_args)
    assert got[1:] == [getattr(v4.c_decode_step_hca_args, f).offset for f in fields]


def hca_step_struct(**kw):
    """A valid fused HCA decode step at the 1M-context shape (fake device pointers)."""
    rec = kv(cap=8192)
    pos, nent, wl = i64(*[1048575] * 16), i64(*[8192] * 16), i32(*[128] * 16)
    a = dict(B=16, m=128, q_pos=ctypes.cast(pos, ctypes.c_void_p), n_entries=ctypes.cast(nent, ctypes.c_void_p),
             in_t=1, G=1, kv_a=FAKE, gate_a=FAKE, bias_a=FAKE, apply_rope=1, rope_theta=10000.0,
             kv=ctypes.pointer(rec), q=FAKE, q_t=1, H=128, win=FAKE, win_t=1,
             win_len=ctypes.cast(wl, ctypes.c_void_p), W=128, sink=FAKE, softmax_scale=0.044, out_rope_inverse=1,
             out=FAKE, out_t=1)
    a.update(kw)
    s = v4.c_decode_step_hca_args(**a)
    s._keep = (rec, pos, nent, wl, a)
    return s


def test_decode_workspace_follows_the_split_plan():
    """The decode workspace holds, per sequence and split, H x D BF16 partial sums and H fp32
    (m, l) pairs, where the split count is the most any sequence up to the given key count takes:
    target 16 splits, at most two 32-key tiles per split for lists of at most 48 tiles."""
    per = 128 * (512 * 2 + 2 * 4)
    # top-1024 + 128 window = 36 tiles: 18 splits of 2 tiles (33..36 tiles give 17..18)
    assert v4.v4a_decode_workspace(4, 128, 512, 1024, 128) == 4 * 18 * per
    # top-512 + 128 window = 20 tiles: lists of up to 16 tiles take one tile per split (16)
    assert v4.v4a_decode_workspace(4, 128, 512, 512, 128) == 4 * 16 * per
    # 48 tiles still take two per split (24); longer lists fall back to 16 splits
    assert v4.v4a_decode_workspace(1, 128, 512, 48 * 32 - 128, 128) == 24 * per
    assert v4.v4a_decode_workspace(1, 128, 512, 8192, 128) == 24 * per


def test_decode_step_hca_workspace_and_rejects():
    L = v4.lib()
    need = L.v4a_decode_step_hca_workspace(ctypes.byref(hca_step_struct()))
    # the step sizes for its own sequences (8192 entries + 128 window = 260 tiles: 16 splits of
    # BF16 partial sums plus fp32 (m, l)); the generic query bounds any sequence up to that many
    # keys, shorter lists included (up to 24 splits of two tiles)
    assert need == 16 * 16 * 128 * (512 * 2 + 2 * 4)
    assert need <= v4.v4a_decode_workspace(16, 128, 512, 8192, 128)
    assert v4.v4a_decode_workspace(16, 128, 512, 8192, 128) == 16 * 24 * 128 * (512 * 2 + 2 * 4)
    assert need % 256 == 0

    def call(ws=FAKE, wsb=1 << 40, **kw):
        return L.v4a_decode_step_hca(ctypes.byref(hca_step_struct(**kw)), ws, wsb, None)
    assert L.v4a_decode_step_hca(None, FAKE, 1 << 40, None) == 1
    assert call(B=0) == 2 and call(B=200) == 2
    assert call(m=0) == 2 and call(m=129) == 2
    assert call(H=24) == 2
    assert call(kv_a=0) == 1
    assert call(wsb=need - 1) == 3
    short = i64(8191, *[8192] * 15)      # sequence 0 would not hold the entry it completes
    assert call(n_entries=ctypes.cast(short, ctypes.c_void_p)) == 1
    wl = i32(*[128] * 16)
    early = i64(99, *[1048575] * 15)     # a ring window longer than the tokens so far
    assert call(ring=1, win_len=ctypes.cast(wl, ctypes.c_void_p), q_pos=ctypes.cast(early, ctypes.c_void_p)) == 1
