"""Seeded synthetic inputs and workload shapes, shared by the tests, the benchmark and the
oracle checks.

This module holds no arithmetic of the attention method: it only draws N(0,1) numbers from
numpy's PCG64 generator (and converts them to BF16 storage where a workload stores BF16),
so that the HIP path and the CPU oracle receive identical bits.  Quantisation, compression,
scoring, selection and attention all happen on either side of the comparison, never here.

Every tensor is drawn from ``numpy.random.default_rng(SeedSequence([seed, tensor_id,
chunk]))`` in fixed-size chunks, so the values do not depend on the number of threads used
to draw them.  The workload seed is ``20260425 + index`` (index 0..4 for the five workloads
below).
"""
from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

BASE_SEED = 20260425
_CHUNK = 1 << 22  # numbers per independently seeded chunk

# Fixed tensor ids: the draw of one tensor never depends on which others were drawn.
TID = {name: i for i, name in enumerate([
    "kv_a", "kv_b", "gate_a", "gate_b", "bias_a", "bias_b",
    "idx_a", "idx_b", "idx_gate_a", "idx_gate_b", "idx_bias_a", "idx_bias_b",
    "kv_h", "gate_h", "bias_h",
    "q", "q_idx", "w", "sink", "window", "window_h", "records", "keys", "records_h",
    "cache_raw", "cache_b_tail", "q_chunk", "q_idx_chunk", "w_chunk",
    "misc0", "misc1", "misc2", "misc3",
    "o_attn", "w_group", "w_final",
])}


def normal(seed: int, name: str, shape, scale: float = 1.0, threads: int = 8) -> np.ndarray:
    """float32 N(0, scale^2) array of the given shape, reproducible from (seed, name)."""
    shape = tuple(int(s) for s in shape)
    n = int(np.prod(shape)) if shape else 1
    out = np.empty((n,), np.float32)
    tid = TID[name]
    nchunk = max(1, math.ceil(n / _CHUNK))

    def fill(c):
        lo, hi = c * _CHUNK, min(n, (c + 1) * _CHUNK)
        g = np.random.default_rng(np.random.SeedSequence([seed, tid, c]))
        g.standard_normal(hi - lo, dtype=np.float32, out=out[lo:hi])

    if nchunk == 1:
        fill(0)
    else:
        with ThreadPoolExecutor(max_workers=threads) as ex:
            list(ex.map(fill, range(nchunk)))
    if scale != 1.0:
        out *= np.float32(scale)
    return out.reshape(shape)


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """BF16 storage (round to nearest even) of an fp32 array, as uint16 bits."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


@dataclass(frozen=True)
class Workload:
    """Shape of one synthetic workload (all tensors N(0,1) before any quantisation)."""
    index: int
    name: str
    kind: str            # "decode_csa", "decode_hca", "tiny", "prefill"
    B: int
    T: int               # context tokens; the decode query sits at T-1
    D: int
    R: int
    H: int
    W: int = 128
    m: int = 4
    m_hca: int = 128
    H_I: int = 0
    d_I: int = 0
    k: int = 0
    fp32: bool = False   # fp32 records / window / queries / outputs
    sink_zero: bool = False
    chunk: int = 0       # prefill: new tokens in the chunk
    notes: str = ""
    extra: dict = field(default_factory=dict)

    @property
    def seed(self) -> int:
        return BASE_SEED + self.index

    @property
    def n_csa(self) -> int:
        return self.T // self.m

    @property
    def n_hca(self) -> int:
        return self.T // self.m_hca

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)


TINY = Workload(0, "tiny_csa_hca_fp32_4k", "tiny", B=1, T=4096, D=128, R=32, H=8, W=128,
                H_I=4, d_I=32, k=64, fp32=True, sink_zero=True,
                notes="compress 4096 tokens (CSA m=4 overlapped, HCA m'=128) then one decode step "
                      "per layer kind, fp32")
CSA_FLASH = Workload(1, "csa_decode_flash_131k", "decode_csa", B=8, T=131072, D=512, R=64, H=64,
                     H_I=64, d_I=128, k=512,
                     notes="CSA decode, 32768 entries drawn directly, MXFP4 indexer, top-512")
HCA_1M = Workload(2, "hca_decode_1m", "decode_hca", B=16, T=1048576, D=512, R=64, H=128,
                  notes="HCA decode, 8192 entries drawn directly, dense + window + sink")
CSA_PRO_1M = Workload(3, "csa_decode_pro_1m", "decode_csa", B=4, T=1048576, D=512, R=64, H=128,
                      H_I=64, d_I=128, k=1024,
                      notes="CSA decode, 262144 entries drawn directly, MXFP4 indexer, top-1024")
PREFILL_64K = Workload(4, "prefill_chunk_4k_on_64k", "prefill", B=1, T=65536, D=512, R=64, H=128,
                       H_I=64, d_I=128, k=1024, chunk=4096,
                       notes="4096-token chunk on a 65536-token cache, CSA and HCA layers")

WORKLOADS = [TINY, CSA_FLASH, HCA_1M, CSA_PRO_1M, PREFILL_64K]
BY_NAME = {w.name: w for w in WORKLOADS}


def scaled(w: Workload, **kw) -> Workload:
    """A smaller copy of a workload (same seed and structure) for quick parity runs."""
    d = dict(w.__dict__)
    d.update(kw)
    return Workload(**d)


# ------------------------------------------------------------------ draws ----

def decode_inputs(w: Workload, threads: int = 8) -> dict:
    """fp32 inputs of a decode workload (entries drawn directly, not compressed).

    records [B][N][D] f32, q [B][H][D] f32, window [B][W][D] f32, sink [H] f32,
    and for CSA: keys [B][N][d_I] f32, q_idx [B][H_I][d_I] f32, w [B][H_I] f32.
    BF16 storage of q and window is derived by the caller with ``to_bf16_bits``.
    """
    s = w.seed
    N = w.n_csa if w.kind == "decode_csa" else w.n_hca
    out = {
        "records": normal(s, "records", (w.B, N, w.D), threads=threads),
        "q": normal(s, "q", (w.B, w.H, w.D)),
        "window": normal(s, "window", (w.B, w.W, w.D)),
        "sink": (np.zeros((w.H,), np.float32) if w.sink_zero else normal(s, "sink", (w.H,))),
        "N": N,
    }
    if w.kind == "decode_csa":
        out["keys"] = normal(s, "keys", (w.B, N, w.d_I), threads=threads)
        out["q_idx"] = normal(s, "q_idx", (w.B, w.H_I, w.d_I))
        out["w"] = normal(s, "w", (w.B, w.H_I))
    return out


def tiny_inputs(w: Workload = TINY) -> dict:
    """Raw streams of the fp32 compress-then-decode workload (G = 1 gates)."""
    s, T, D, dI = w.seed, w.T, w.D, w.d_I
    return {
        "kv_a": normal(s, "kv_a", (T, D)), "kv_b": normal(s, "kv_b", (T, D)),
        "gate_a": normal(s, "gate_a", (T, 1)), "gate_b": normal(s, "gate_b", (T, 1)),
        "bias_a": normal(s, "bias_a", (w.m, 1)), "bias_b": normal(s, "bias_b", (w.m, 1)),
        "idx_a": normal(s, "idx_a", (T, dI)), "idx_b": normal(s, "idx_b", (T, dI)),
        "idx_gate_a": normal(s, "idx_gate_a", (T, 1)), "idx_gate_b": normal(s, "idx_gate_b", (T, 1)),
        "idx_bias_a": normal(s, "idx_bias_a", (w.m, 1)),
        "idx_bias_b": normal(s, "idx_bias_b", (w.m, 1)),
        "kv_h": normal(s, "kv_h", (T, D)), "gate_h": normal(s, "gate_h", (T, 1)),
        "bias_h": normal(s, "bias_h", (w.m_hca, 1)),
        "q": normal(s, "q", (w.H, D)), "q_idx": normal(s, "q_idx", (w.H_I, dI)),
        "w": normal(s, "w", (w.H_I,)),
        "sink": np.zeros((w.H,), np.float32),
    }


def prefill_inputs(w: Workload, C: int | None = None, tok0: int | None = None, n_prev: int = 128,
                   kind: str = "csa", threads: int = 8) -> dict:
    """fp32 inputs of one prefill chunk of C tokens at positions tok0 .. tok0+C-1.

    The entries cached before tok0 are drawn directly (records [tok0/m][D], and for CSA the
    indexer keys [tok0/m][d_I]); the chunk's raw streams hold n_prev + C rows (row r is
    position tok0 - n_prev + r) and are compressed by the call under test.  Queries:
    q [C][H][D], and for CSA q_idx [C][H_I][d_I], w [C][H_I].
    """
    s = w.seed
    C = w.chunk if C is None else C
    tok0 = w.T if tok0 is None else tok0
    rows = n_prev + C
    m = w.m if kind == "csa" else w.m_hca
    out = {"C": C, "tok0": tok0, "n_prev": n_prev, "m": m, "N0": tok0 // m,
           "q": normal(s, "q_chunk", (C, w.H, w.D), threads=threads),
           "sink": (np.zeros((w.H,), np.float32) if w.sink_zero else normal(s, "sink", (w.H,)))}
    if kind == "csa":
        out.update(records=normal(s, "records", (tok0 // m, w.D), threads=threads),
                   keys=normal(s, "keys", (tok0 // m, w.d_I), threads=threads),
                   kv_a=normal(s, "kv_a", (rows, w.D)), kv_b=normal(s, "kv_b", (rows, w.D)),
                   gate_a=normal(s, "gate_a", (rows, 1)), gate_b=normal(s, "gate_b", (rows, 1)),
                   bias_a=normal(s, "bias_a", (m, 1)), bias_b=normal(s, "bias_b", (m, 1)),
                   idx_a=normal(s, "idx_a", (rows, w.d_I)), idx_b=normal(s, "idx_b", (rows, w.d_I)),
                   idx_gate_a=normal(s, "idx_gate_a", (rows, 1)), idx_gate_b=normal(s, "idx_gate_b", (rows, 1)),
                   idx_bias_a=normal(s, "idx_bias_a", (m, 1)), idx_bias_b=normal(s, "idx_bias_b", (m, 1)),
                   q_idx=normal(s, "q_idx_chunk", (C, w.H_I, w.d_I), threads=threads),
                   w=normal(s, "w_chunk", (C, w.H_I)))
    else:
        out.update(records=normal(s, "records_h", (tok0 // m, w.D), threads=threads),
                   kv_a=normal(s, "kv_h", (rows, w.D)), gate_a=normal(s, "gate_h", (rows, 1)),
                   bias_a=normal(s, "bias_h", (m, 1)))
    return out
