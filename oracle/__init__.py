"""CPU oracle for the DeepSeek-V4 CSA/HCA attention hot path (test infrastructure).

TEST INFRASTRUCTURE ONLY: imported by tests/, by ``__graft_entry__.smoke()`` and
by the ``cpu_baseline`` leg of ``bench.py``; never by the product package.  The
arithmetic lives in ``oracle.c`` (plain C, double precision, exact MXFP4
integer dots); this module only marshals numpy arrays through ctypes and
composes the per-stage functions into whole steps in the order the pages give
(compress -> indexer scores -> top-k -> shared-KV MQA with window and sink;
"DeepSeek V4 technical report explained" (firecat-web.com), item 2 "Hybrid
attention").  Every function is pinned by the CPU tests; none is
"parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

GCC_CMD = ["gcc", "-O2", "-std=gnu11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
           "-fno-fast-math", "-fvisibility=hidden", _SRC, "-o", _LIB, "-lm"]


def build(force: bool = True) -> str:
    """Compile liboracle.so with gcc (host code only)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        subprocess.run(GCC_CMD, check=True)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        _lib = ctypes.CDLL(_LIB)
        _declare(_lib)
    return _lib


P = ctypes.c_void_p
I32 = ctypes.c_int
I64 = ctypes.c_int64
F64 = ctypes.c_double


def _declare(L):
    L.orc_threads.restype = I32
    L.orc_e4m3_decode.argtypes = [ctypes.c_uint8]
    L.orc_e4m3_decode.restype = F64
    L.orc_e4m3_encode.argtypes = [ctypes.c_float]
    L.orc_e4m3_encode.restype = ctypes.c_uint8
    L.orc_bf16_encode.argtypes = [ctypes.c_float]
    L.orc_bf16_encode.restype = ctypes.c_uint16
    L.orc_bf16_decode.argtypes = [ctypes.c_uint16]
    L.orc_bf16_decode.restype = F64
    L.orc_e2m1_decode.argtypes = [ctypes.c_uint8]
    L.orc_e2m1_decode.restype = F64
    L.orc_e2m1_encode.argtypes = [F64]
    L.orc_e2m1_encode.restype = ctypes.c_uint8
    L.orc_quant_kv.argtypes = [P, I64, I32, I32, P, P, P]
    L.orc_dequant_kv.argtypes = [P, P, P, I64, I32, I32, P]
    L.orc_quant_mxfp4.argtypes = [P, I64, I32, P, P]
    L.orc_dequant_mxfp4.argtypes = [P, P, I64, I32, P]
    L.orc_rope.argtypes = [P, I64, I32, I32, P, F64, I32]
    L.orc_compress_csa.argtypes = [P, P, I32, P, P, I32, P, P, I64, I64, I32, I64, I64, I32, I32,
                                   F64, P, F64, P]
    L.orc_compress_csa.restype = I32
    L.orc_compress_hca.argtypes = [P, I32, P, I32, P, I64, I64, I32, I64, I64, I32, I32, F64, P, F64, P]
    L.orc_compress_hca.restype = I32
    L.orc_indexer_scores_mxfp4.argtypes = [P, P, P, I32, I32, P, P, I64, P, P]
    L.orc_indexer_scores_f32.argtypes = [P, P, I32, I32, P, I64, P]
    L.orc_topk.argtypes = [P, I64, I32, P]
    L.orc_topk_bf16.argtypes = [P, I64, I32, P]
    L.orc_query_prologue.argtypes = [P, I32, I32, P, F64, I32, F64, F64, P]
    L.orc_attend.argtypes = [P, I32, I32, P, I64, P, I64, P, F64, I32, I32, F64, F64, P, P]
    L.orc_round_bf16.argtypes = [F64]
    L.orc_round_bf16.restype = F64
    L.orc_group_reduce.argtypes = [P, I64, I32, I32, I32, I32, P, P]
    L.orc_project.argtypes = [P, I64, I64, P, I64, P]


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a, a.ctypes.data_as(P)


def threads() -> int:
    return int(lib().orc_threads())


# ---------------------------------------------------------------- formats ----

def e4m3_encode(x: float) -> int:
    return int(lib().orc_e4m3_encode(float(np.float32(x))))


def e4m3_decode(c: int) -> float:
    return float(lib().orc_e4m3_decode(int(c)))


def bf16_encode(x: float) -> int:
    return int(lib().orc_bf16_encode(float(np.float32(x))))


def bf16_decode(b: int) -> float:
    return float(lib().orc_bf16_decode(int(b)))


def e2m1_encode(x: float) -> int:
    return int(lib().orc_e2m1_encode(float(x)))


def e2m1_decode(c: int) -> float:
    return float(lib().orc_e2m1_decode(int(c)))


def quant_kv(x: np.ndarray, R: int):
    """Entry records of fp32 rows x [rows][D]: (nope u8 [rows][D-R], rope bf16 bits u16 [rows][R],
    scale f32 [rows])."""
    x, px = _c(x, np.float32)
    rows, D = x.reshape(-1, x.shape[-1]).shape
    nope = np.empty((rows, D - R), np.uint8)
    rope = np.empty((rows, R), np.uint16)
    scale = np.empty((rows,), np.float32)
    lib().orc_quant_kv(px, rows, D, R, nope.ctypes.data_as(P), rope.ctypes.data_as(P),
                       scale.ctypes.data_as(P))
    return nope, rope, scale


def dequant_kv(nope, rope, scale) -> np.ndarray:
    nope, pn = _c(nope, np.uint8)
    rope, pr = _c(rope, np.uint16)
    scale, ps = _c(scale, np.float32)
    rows = scale.size
    R = rope.size // max(rows, 1) if rows else 0
    Dn = nope.size // max(rows, 1) if rows else 0
    out = np.empty((rows, Dn + R), np.float64)
    lib().orc_dequant_kv(pn, pr, ps, rows, Dn + R, R, out.ctypes.data_as(P))
    return out


def quant_mxfp4(x: np.ndarray):
    """MXFP4 of fp32 rows x [rows][d]: (codes u8 [rows][d/2], scales u8 [rows][d/32])."""
    x, px = _c(x, np.float32)
    x2 = x.reshape(-1, x.shape[-1])
    rows, d = x2.shape
    codes = np.empty((rows, d // 2), np.uint8)
    scales = np.empty((rows, d // 32), np.uint8)
    lib().orc_quant_mxfp4(px, rows, d, codes.ctypes.data_as(P), scales.ctypes.data_as(P))
    return codes, scales


def dequant_mxfp4(codes, scales) -> np.ndarray:
    codes, pc = _c(codes, np.uint8)
    scales, ps = _c(scales, np.uint8)
    rows = codes.shape[0]
    d = codes.shape[1] * 2
    out = np.empty((rows, d), np.float64)
    lib().orc_dequant_mxfp4(pc, ps, rows, d, out.ctypes.data_as(P))
    return out


def rope(x: np.ndarray, R: int, pos, theta: float = 10000.0, sign: int = 1) -> np.ndarray:
    """Rotate the last R dims of each row of x (float64 copy) at positions pos."""
    x = np.array(x, dtype=np.float64, order="C")
    rows, D = x.reshape(-1, x.shape[-1]).shape
    pos, pp = _c(np.broadcast_to(np.asarray(pos, np.float64), (rows,)), np.float64)
    lib().orc_rope(x.ctypes.data_as(P), rows, D, R, pp, float(theta), int(sign))
    return x


# ------------------------------------------------------------- compressors ---

def compress_csa(kv_a, kv_b, gate_a, gate_b, bias_a, bias_b, *, tok0, m, first_entry, n_entries,
                 apply_rope, R, theta=10000.0, norm_w=None, eps=1e-6) -> np.ndarray:
    """fp32 CSA entries [n_entries][D] (before quantisation); norm_w [D] RMS-normalises each merged
    entry before RoPE."""
    kv_a, pa = _c(kv_a, np.float32)
    kv_b, pb = _c(kv_b, np.float32)
    gate_a, pga = _c(gate_a, np.float32)
    gate_b, pgb = _c(gate_b, np.float32)
    bias_a, pba = _c(bias_a, np.float32)
    bias_b, pbb = _c(bias_b, np.float32)
    n_tok, D = kv_a.shape
    G = gate_a.shape[1]
    out = np.empty((n_entries, D), np.float32)
    nw, pnw = _c(norm_w, np.float32) if norm_w is not None else (None, None)
    rc = lib().orc_compress_csa(pa, pb, D, pga, pgb, G, pba, pbb, tok0, n_tok, m, first_entry,
                                n_entries, int(apply_rope), R, float(theta), pnw, float(eps),
                                out.ctypes.data_as(P))
    if rc != 0:
        raise ValueError("rows do not cover the blocks these entries need")
    return out


def compress_hca(kv, gate, bias, *, tok0, m, first_entry, n_entries, apply_rope, R,
                 theta=10000.0, norm_w=None, eps=1e-6) -> np.ndarray:
    kv, pk = _c(kv, np.float32)
    gate, pg = _c(gate, np.float32)
    bias, pbi = _c(bias, np.float32)
    n_tok, D = kv.shape
    G = gate.shape[1]
    out = np.empty((n_entries, D), np.float32)
    nw, pnw = _c(norm_w, np.float32) if norm_w is not None else (None, None)
    rc = lib().orc_compress_hca(pk, D, pg, G, pbi, tok0, n_tok, m, first_entry, n_entries,
                                int(apply_rope), R, float(theta), pnw, float(eps), out.ctypes.data_as(P))
    if rc != 0:
        raise ValueError("rows do not cover the blocks these entries need")
    return out


# ----------------------------------------------------------------- indexer ---

def indexer_scores_mxfp4(q_codes, q_scales, w, k_codes, k_scales, n_keys=None):
    """Scores [n_keys] fp32 of one query (H heads) and the count of non-fp32-exact dots."""
    q_codes, pqc = _c(q_codes, np.uint8)
    q_scales, pqs = _c(q_scales, np.uint8)
    w, pw = _c(w, np.float32)
    k_codes, pkc = _c(k_codes, np.uint8)
    k_scales, pks = _c(k_scales, np.uint8)
    H = q_codes.shape[0]
    d = q_codes.shape[1] * 2
    n = k_codes.shape[0] if n_keys is None else int(n_keys)
    scores = np.empty((n,), np.float32)
    bad = np.zeros((1,), np.int64)
    lib().orc_indexer_scores_mxfp4(pqc, pqs, pw, H, d, pkc, pks, n, scores.ctypes.data_as(P),
                                   bad.ctypes.data_as(P))
    return scores, int(bad[0])


def indexer_scores_f32(q, w, keys, n_keys=None) -> np.ndarray:
    q, pq = _c(q, np.float32)
    w, pw = _c(w, np.float32)
    keys, pk = _c(keys, np.float32)
    H, d = q.shape
    n = keys.shape[0] if n_keys is None else int(n_keys)
    scores = np.empty((n,), np.float32)
    lib().orc_indexer_scores_f32(pq, pw, H, d, pk, n, scores.ctypes.data_as(P))
    return scores


def topk(scores, k: int, n_vis=None, score_bf16: bool = False) -> np.ndarray:
    """The k best of scores[:n_vis] (lowest index wins ties), ascending, -1 padded; with
    score_bf16 the scores are first rounded to BF16."""
    scores, ps = _c(scores, np.float32)
    n = scores.size if n_vis is None else int(n_vis)
    out = np.empty((k,), np.int32)
    (lib().orc_topk_bf16 if score_bf16 else lib().orc_topk)(ps, n, int(k), out.ctypes.data_as(P))
    return out


# --------------------------------------------------------------- attention ---

def query_prologue(q_bits, norm_w, *, pos, R, eps=1e-6, theta=10000.0) -> np.ndarray:
    """BF16 bits [H][D] of the queries after RMSNorm (weights norm_w [D]) and RoPE at pos."""
    q_bits, pq = _c(q_bits, np.uint16)
    H, D = q_bits.shape
    w, pw = _c(norm_w, np.float32)
    out = np.empty((H, D), np.uint16)
    lib().orc_query_prologue(pq, H, D, pw, float(eps), int(R), float(pos), float(theta), out.ctypes.data_as(P))
    return out


def attend(q, E, Wn, sink, scale, *, rope_inverse=False, R=0, theta=10000.0, t_q=0.0,
           with_mass=False):
    """Attention of one query position: q [H][D], entries E [n][D], window Wn [w][D] (float64)."""
    q, pq = _c(q, np.float64)
    H, D = q.shape
    E = np.zeros((0, D)) if E is None else E
    Wn = np.zeros((0, D)) if Wn is None else Wn
    E, pe = _c(E.reshape(-1, D), np.float64)
    Wn, pw = _c(Wn.reshape(-1, D), np.float64)
    sink, psk = _c(np.broadcast_to(np.asarray(sink, np.float32), (H,)), np.float32)
    out = np.empty((H, D), np.float64)
    mass = np.empty((H,), np.float64)
    lib().orc_attend(pq, H, D, pe, E.shape[0], pw, Wn.shape[0], psk, float(scale),
                     int(rope_inverse), int(R), float(theta), float(t_q), out.ctypes.data_as(P),
                     mass.ctypes.data_as(P))
    return (out, mass) if with_mass else out


# ------------------------------------------------------- composed steps ------

def visible_entries(n_entries: int, m: int, pos: int) -> int:
    """Entries i with m*(i+1)-1 <= pos (causal visibility by block end)."""
    return int(max(0, min(n_entries, (pos + 1) // m)))


def decode_csa(q, records, n_entries, k, window, sink, scale, *, q_pos, m=4, idx=None,
               rope_inverse=True, R=64, theta=10000.0, scores=None, score_bf16=False):
    """One CSA decode step for one sequence.

    records: float64 [N][D] dequantised entries; idx: dict(q_codes, q_scales, w, k_codes,
    k_scales) for MXFP4, or dict(q, w, keys) for fp32; scores may be given precomputed;
    score_bf16 selects on the scores rounded to BF16.
    Returns (out [H][D] float64, topk indices [k]).
    """
    n_vis = visible_entries(n_entries, m, q_pos)
    if scores is None:
        if "k_codes" in idx:
            scores, bad = indexer_scores_mxfp4(idx["q_codes"], idx["q_scales"], idx["w"],
                                               idx["k_codes"], idx["k_scales"], n_vis)
            if bad:
                raise AssertionError(f"{bad} indexer dots are not fp32-exact")
        else:
            scores = indexer_scores_f32(idx["q"], idx["w"], idx["keys"], n_vis)
    sel = topk(scores, k, n_vis, score_bf16=score_bf16)
    chosen = sel[sel >= 0]
    out = attend(q, records[chosen], window, sink, scale, rope_inverse=rope_inverse, R=R,
                 theta=theta, t_q=q_pos)
    return out, sel


def decode_hca(q, records, n_entries, window, sink, scale, *, q_pos, m=128, rope_inverse=True,
               R=64, theta=10000.0):
    n_vis = visible_entries(n_entries, m, q_pos)
    return attend(q, records[:n_vis], window, sink, scale, rope_inverse=rope_inverse, R=R,
                  theta=theta, t_q=q_pos)


def prefill_queries(kind, q, records, n_entries, stream, *, n_prev, tok0, queries, W, sink, scale,
                    m, k=None, idx=None, rope_inverse=True, R=64, theta=10000.0, score_bf16=False):
    """Attention of chosen queries of a prefill chunk, each exactly as a decode step.

    The chunk's own compression is the compressor run on the chunk with its state (the
    caller does it, so ``records`` / ``idx`` already hold the appended entries).  Query j
    sits at t = tok0 + j: it sees the entries whose block ends at or before t, keeps its
    top-k of them (CSA) or all of them (HCA), and its window is the raw rows t-W+1 .. t of
    ``stream`` (row r of ``stream`` is position tok0 - n_prev + r).  "DeepSeek-V4 technical
    report walkthrough" (cyqw.cn), section 3.5: the state cache keeps the window and the
    incomplete block; the compressed entries are the classical cache.

    q: [C][H][D] float64; idx (CSA): per-query dicts are made from the chunk arrays
    dict(q_codes [C][H_I][..], q_scales, w [C][H_I], k_codes, k_scales) or
    dict(q [C][H_I][d], w, keys).  Returns {j: out [H][D]} and, for CSA, {j: top-k}.
    """
    outs, sels = {}, {}
    row0 = tok0 - n_prev
    for j in queries:
        t = tok0 + int(j)
        lo = max(0, t - W + 1)
        window = stream[lo - row0:t - row0 + 1] if W > 0 else None
        if kind == "csa":
            if "k_codes" in idx:
                qi = dict(q_codes=idx["q_codes"][j], q_scales=idx["q_scales"][j], w=idx["w"][j],
                          k_codes=idx["k_codes"], k_scales=idx["k_scales"])
            else:
                qi = dict(q=idx["q"][j], w=idx["w"][j], keys=idx["keys"])
            outs[j], sels[j] = decode_csa(q[j], records, n_entries, k, window, sink, scale, q_pos=t,
                                          m=m, idx=qi, rope_inverse=rope_inverse, R=R, theta=theta,
                                          score_bf16=score_bf16)
        else:
            outs[j] = decode_hca(q[j], records, n_entries, window, sink, scale, q_pos=t, m=m,
                                 rope_inverse=rope_inverse, R=R, theta=theta)
    return outs, sels


def decode_tokens(kind, q, records, n_entries, stream, *, t_last, Q, win_len, sink, scale, m, k=None, idx=None,
                  rope_inverse=True, R=64, theta=10000.0, score_bf16=False):
    """A multi-token decode step of one sequence: its Q new tokens at positions t_last-Q+1 .. t_last
    evaluated together.  "DeepSeek-V4 technical report walkthrough" (cyqw.cn), section 2 and the
    model table of section 4.2: V4 keeps multi-token prediction with depth 1, so a step can verify a
    drafted token together with the new one.  Each query is the decode step at its own position:
    ``records`` (and, for CSA, the keys in ``idx``) hold every entry cached after the step,
    including one that a token of the step completes, and query j, at t_j = t_last-Q+1+j, sees only
    the entries whose block ends at or before t_j (causal visibility by block end) and the
    min(win_len, t_j+1) raw tokens ending at t_j.  stream: raw rows by position 0 .. t_last.
    q [Q][H][D]; idx per query as in prefill_queries.  Returns (out [Q][H][D], selections [Q][k]
    for CSA or None)."""
    tok0 = t_last - Q + 1
    outs, sels = prefill_queries(kind, q, records, n_entries, stream, n_prev=tok0, tok0=tok0, queries=range(Q),
                                 W=win_len, sink=sink, scale=scale, m=m, k=k, idx=idx, rope_inverse=rope_inverse,
                                 R=R, theta=theta, score_bf16=score_bf16)
    out = np.stack([outs[j] for j in range(Q)])
    return out, (np.stack([sels[j] for j in range(Q)]) if kind == "csa" else None)


# ------------------------------------------------------ grouped output projection ---

def round_bf16(x: float) -> float:
    """x rounded to the nearest BF16 value, ties to even, from double directly."""
    return float(lib().orc_round_bf16(float(x)))


def group_reduce(o_bits, G: int, r: int, wg_bits) -> np.ndarray:
    """The reduced groups y [T][G*r] (BF16 values as float64) of the attention output o_bits
    [T][H][D] (BF16 bits) with the group weights wg_bits [G][r][H*D/G] (BF16 bits).
    "DeepSeek-V4 technical report walkthrough" (cyqw.cn), section 2.2, Grouped Output Projection."""
    o_bits, po = _c(o_bits, np.uint16)
    T, H, D = o_bits.shape
    wg_bits, pw = _c(wg_bits, np.uint16)
    assert wg_bits.shape == (G, r, H * D // G)
    y = np.empty((T, G * r), np.float64)
    lib().orc_group_reduce(po, T, H, D, G, r, pw, y.ctypes.data_as(P))
    return y


def project(x, w_bits) -> np.ndarray:
    """x [T][K] (float64 values) times the rows of w_bits [N][K] (BF16 bits): [T][N] float64."""
    x, px = _c(x, np.float64)
    w_bits, pw = _c(w_bits, np.uint16)
    T, K = x.shape
    N = w_bits.shape[0]
    assert w_bits.shape == (N, K)
    out = np.empty((T, N), np.float64)
    lib().orc_project(px, T, K, pw, N, out.ctypes.data_as(P))
    return out


def grouped_projection(o_bits, G: int, r: int, wg_bits, wf_bits) -> np.ndarray:
    """The grouped output projection [T][d] (float64, before the output cast)."""
    return project(group_reduce(o_bits, G, r, wg_bits), wf_bits)
