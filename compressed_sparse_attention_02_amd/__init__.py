"""Python binding of libv4attn (DeepSeek-V4 CSA/HCA attention hot path on MI355X / gfx950).

Argument marshalling only: each function here forwards torch device tensors (as raw
pointers) and host integers to the C entry point of the same name in ``include/v4attn.h``,
on the current torch stream, and raises ``V4AError`` with the library's message when the
call is rejected.  Every step of the path runs in the HIP kernels of ``libv4attn.so``; there
is no fallback: importing the binding without the built library raises.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "_lib", "libv4attn.so")
HEADER = os.path.join(os.path.dirname(_HERE), "include", "v4attn.h")

# enums (include/v4attn.h)
V4A_F32, V4A_BF16 = 0, 1
V4A_KV_F32, V4A_KV_FP8_BF16 = 0, 1
V4A_IDX_F32, V4A_IDX_MXFP4 = 0, 1
STATUS = {0: "V4A_OK", 1: "V4A_EINVAL", 2: "V4A_EUNSUPPORTED", 3: "V4A_EWORKSPACE", 4: "V4A_EHIP"}


class V4AError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status


class c_kv(ctypes.Structure):
    _fields_ = [("fmt", ctypes.c_int), ("D", ctypes.c_int32), ("R", ctypes.c_int32),
                ("nope", ctypes.c_void_p), ("rope", ctypes.c_void_p), ("scale", ctypes.c_void_p),
                ("cap", ctypes.c_int64)]


class c_idx(ctypes.Structure):
    _fields_ = [("fmt", ctypes.c_int), ("d", ctypes.c_int32), ("codes", ctypes.c_void_p),
                ("scales", ctypes.c_void_p), ("cap", ctypes.c_int64)]


class c_prefill_args(ctypes.Structure):
    P = ctypes.c_void_p
    _fields_ = [("tok0", ctypes.c_int64), ("C", ctypes.c_int32), ("n_prev", ctypes.c_int32),
                ("m", ctypes.c_int32), ("in_t", ctypes.c_int), ("G", ctypes.c_int32),
                ("kv_a", P), ("kv_b", P), ("gate_a", P), ("gate_b", P), ("bias_a", P), ("bias_b", P),
                ("apply_rope", ctypes.c_int32), ("rope_theta", ctypes.c_float),
                ("kv", ctypes.POINTER(c_kv)), ("slot", ctypes.c_int32), ("idx_G", ctypes.c_int32),
                ("idx_a", P), ("idx_b", P), ("idx_gate_a", P), ("idx_gate_b", P), ("idx_bias_a", P),
                ("idx_bias_b", P), ("keys", ctypes.POINTER(c_idx)), ("q_idx", ctypes.POINTER(c_idx)),
                ("w", P), ("H_I", ctypes.c_int32), ("k", ctypes.c_int32), ("q", P), ("q_t", ctypes.c_int),
                ("H", ctypes.c_int32), ("W", ctypes.c_int32), ("sink", P), ("softmax_scale", ctypes.c_float),
                ("out_rope_inverse", ctypes.c_int32), ("out", P), ("out_t", ctypes.c_int),
                ("score_bf16", ctypes.c_int32), ("norm_w", P), ("idx_norm_w", P), ("q_norm_w", P)]


V4A_LAYER_CSA, V4A_LAYER_HCA = 0, 1


class c_decode_step_args(ctypes.Structure):
    P = ctypes.c_void_p
    _fields_ = [("B", ctypes.c_int32), ("m", ctypes.c_int32), ("q_pos", P), ("n_entries", P),
                ("in_t", ctypes.c_int), ("G", ctypes.c_int32), ("idx_G", ctypes.c_int32),
                ("kv_a", P), ("kv_b", P), ("gate_a", P), ("gate_b", P), ("bias_a", P), ("bias_b", P),
                ("idx_a", P), ("idx_b", P), ("idx_gate_a", P), ("idx_gate_b", P), ("idx_bias_a", P),
                ("idx_bias_b", P), ("apply_rope", ctypes.c_int32), ("rope_theta", ctypes.c_float),
                ("kv", ctypes.POINTER(c_kv)), ("keys", ctypes.POINTER(c_idx)), ("q_idx", ctypes.POINTER(c_idx)),
                ("w", P), ("H_I", ctypes.c_int32), ("k", ctypes.c_int32), ("q", P), ("q_t", ctypes.c_int),
                ("H", ctypes.c_int32), ("win", P), ("win_t", ctypes.c_int), ("win_len", P), ("W", ctypes.c_int32),
                ("sink", P), ("softmax_scale", ctypes.c_float), ("out_rope_inverse", ctypes.c_int32),
                ("out", P), ("out_t", ctypes.c_int), ("score_bf16", ctypes.c_int32), ("norm_w", P),
                ("idx_norm_w", P), ("ring", ctypes.c_int32), ("no_split", ctypes.c_int32), ("q_norm_w", P),
                ("ws_clean", ctypes.c_int32), ("Q", ctypes.c_int32)]



class c_decode_step_hca_args(ctypes.Structure):
    P = ctypes.c_void_p
    _fields_ = [("B", ctypes.c_int32), ("m", ctypes.c_int32), ("q_pos", P), ("n_entries", P),
                ("in_t", ctypes.c_int), ("G", ctypes.c_int32), ("kv_a", P), ("gate_a", P), ("bias_a", P),
                ("apply_rope", ctypes.c_int32), ("rope_theta", ctypes.c_float), ("norm_w", P),
                ("kv", ctypes.POINTER(c_kv)), ("q", P), ("q_t", ctypes.c_int), ("H", ctypes.c_int32),
                ("win", P), ("win_t", ctypes.c_int), ("win_len", P), ("W", ctypes.c_int32), ("sink", P),
                ("softmax_scale", ctypes.c_float), ("out_rope_inverse", ctypes.c_int32), ("out", P),
                ("out_t", ctypes.c_int), ("ring", ctypes.c_int32), ("no_split", ctypes.c_int32), ("q_norm_w", P),
                ("Q", ctypes.c_int32)]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libv4attn.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m compressed_sparse_attention_02_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P, I32, I64, F32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
        KVP, IDXP = ctypes.POINTER(c_kv), ctypes.POINTER(c_idx)
        sig = {
            "v4a_quantize_kv": [P, I64, KVP, I64, P],
            "v4a_quantize_mxfp4": [P, I64, IDXP, I64, P],
            "v4a_compress_csa": [P, P, ctypes.c_int, I32, P, P, I32, P, P, I64, I64, I32, I64, I64,
                                 I32, F32, P, KVP, IDXP, I32, I32, P],
            "v4a_compress_hca": [P, ctypes.c_int, I32, P, I32, P, I64, I64, I32, I64, I64, I32, F32,
                                 P, KVP, I32, I32, P],
            "v4a_indexer_topk": [IDXP, P, I32, IDXP, P, I32, I32, I32, P, I32, P, P, SZ, P],
            "v4a_indexer_topk_bf16": [IDXP, P, I32, IDXP, P, I32, I32, I32, P, I32, P, P, SZ, P],
            "v4a_indexer_scores": [IDXP, P, I32, IDXP, P, I32, I32, I32, P, I64, P, P],
            "v4a_decode_csa": [P, ctypes.c_int, I32, I32, KVP, P, I32, P, ctypes.c_int, P, I32, P,
                               P, F32, I32, F32, P, ctypes.c_int, P, SZ, P],
            "v4a_decode_hca": [P, ctypes.c_int, I32, I32, KVP, P, I32, P, ctypes.c_int, P, I32, P,
                               P, F32, I32, F32, P, ctypes.c_int, P, SZ, P],
        }
        for name, args in sig.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = ctypes.c_int
        DSP = ctypes.POINTER(c_decode_step_args)
        L.v4a_decode_step_csa.argtypes = [DSP, P, SZ, P]
        L.v4a_decode_step_csa.restype = ctypes.c_int
        L.v4a_decode_step_workspace.argtypes = [DSP]
        L.v4a_decode_step_workspace.restype = SZ
        L.v4a_output_projection.argtypes = [P, I32, I32, I32, I32, I32, P, P, I32, P, ctypes.c_int, P, SZ, P]
        L.v4a_output_projection.restype = ctypes.c_int
        L.v4a_output_projection_workspace.argtypes = [I32, I32, I32]
        L.v4a_output_projection_workspace.restype = SZ
        L.v4a_decode_step_csa_noalloc.argtypes = [DSP, P]
        L.v4a_decode_step_csa_noalloc.restype = ctypes.c_int
        DHP = ctypes.POINTER(c_decode_step_hca_args)
        L.v4a_decode_step_hca.argtypes = [DHP, P, SZ, P]
        L.v4a_decode_step_hca.restype = ctypes.c_int
        L.v4a_decode_step_hca_workspace.argtypes = [DHP]
        L.v4a_decode_step_hca_workspace.restype = SZ
        PAP = ctypes.POINTER(c_prefill_args)
        L.v4a_prefill_chunk.argtypes = [ctypes.c_int, PAP, P, SZ, P]
        L.v4a_prefill_chunk.restype = ctypes.c_int
        L.v4a_prefill_workspace.argtypes = [ctypes.c_int, PAP]
        L.v4a_prefill_workspace.restype = SZ
        L.v4a_indexer_topk_workspace.argtypes = [I32, I32, I64, I32]
        L.v4a_indexer_topk_workspace.restype = SZ
        L.v4a_decode_workspace.argtypes = [I32, I32, I32, I64, I32]
        L.v4a_decode_workspace.restype = SZ
        L.v4a_last_error.restype = ctypes.c_char_p
        L.v4a_version.restype = ctypes.c_char_p
        L.v4a_trace_begin.argtypes = [I32]
        L.v4a_trace_begin.restype = ctypes.c_int
        L.v4a_trace_end.argtypes = []
        L.v4a_trace_end.restype = I32
        L.v4a_trace_kernel.argtypes = [I32, ctypes.POINTER(ctypes.c_char_p), ctypes.POINTER(F32)]
        L.v4a_trace_kernel.restype = ctypes.c_int
        _lib = L
    return _lib


def _check(status: int):
    if status != 0:
        raise V4AError(status, lib().v4a_last_error().decode())


def _ptr(t) -> int | None:
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch tensor")
    if not t.is_contiguous():
        raise ValueError("tensors passed to libv4attn must be contiguous")
    return t.data_ptr()


def _host_i64(vals):
    arr = (ctypes.c_int64 * len(vals))(*[int(v) for v in vals])
    return arr


def _host_i32(vals):
    return (ctypes.c_int32 * len(vals))(*[int(v) for v in vals])


def _stream(stream=None) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _ftype(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return V4A_BF16
    if t.dtype == torch.float32:
        return V4A_F32
    raise TypeError(f"unsupported element type {t.dtype}")


@dataclass
class KV:
    """A batch of entry records (device tensors); see ``v4a_kv`` in include/v4attn.h."""
    fmt: int
    D: int
    R: int
    nope: torch.Tensor
    rope: torch.Tensor | None
    scale: torch.Tensor | None
    cap: int

    @staticmethod
    def empty(B: int, cap: int, D: int, R: int, fmt: int = V4A_KV_FP8_BF16, device="cuda"):
        if fmt == V4A_KV_FP8_BF16:
            return KV(fmt, D, R, torch.zeros((B, cap, D - R), dtype=torch.uint8, device=device),
                      torch.zeros((B, cap, R), dtype=torch.int16, device=device),
                      torch.zeros((B, cap), dtype=torch.float32, device=device), cap)
        return KV(fmt, D, R, torch.zeros((B, cap, D), dtype=torch.float32, device=device), None, None, cap)

    def c(self) -> c_kv:
        return c_kv(self.fmt, self.D, self.R, _ptr(self.nope), _ptr(self.rope), _ptr(self.scale), self.cap)


@dataclass
class Idx:
    """A batch of indexer vectors (device tensors); see ``v4a_idx`` in include/v4attn.h."""
    fmt: int
    d: int
    codes: torch.Tensor
    scales: torch.Tensor | None
    cap: int

    @staticmethod
    def empty(B: int, cap: int, d: int, fmt: int = V4A_IDX_MXFP4, device="cuda"):
        if fmt == V4A_IDX_MXFP4:
            return Idx(fmt, d, torch.zeros((B, cap, d // 2), dtype=torch.uint8, device=device),
                       torch.zeros((B, cap, d // 32), dtype=torch.uint8, device=device), cap)
        return Idx(fmt, d, torch.zeros((B, cap, d), dtype=torch.float32, device=device), None, cap)

    def c(self) -> c_idx:
        return c_idx(self.fmt, self.d, _ptr(self.codes), _ptr(self.scales), self.cap)


# ------------------------------------------------------------------ entry points ----

def v4a_version() -> str:
    return lib().v4a_version().decode()


def v4a_trace_begin(capacity: int):
    _check(lib().v4a_trace_begin(capacity))


def v4a_trace_end() -> int:
    return int(lib().v4a_trace_end())


def v4a_trace_kernel(i: int) -> tuple[str, float]:
    """(kernel name, milliseconds) of the i-th kernel timed by the last trace."""
    name, ms = ctypes.c_char_p(), ctypes.c_float()
    _check(lib().v4a_trace_kernel(i, ctypes.byref(name), ctypes.byref(ms)))
    return name.value.decode(), float(ms.value)


def trace_kernels(n: int) -> list[tuple[str, float]]:
    """Every kernel of the last trace of n kernels (the caller has synchronised its streams)."""
    return [v4a_trace_kernel(i) for i in range(n)]


def v4a_quantize_kv(x: torch.Tensor, out: KV, row0: int = 0, stream=None):
    rows = x.numel() // out.D if x.numel() else 0
    _check(lib().v4a_quantize_kv(_ptr(x), rows, ctypes.byref(out.c()), row0, _stream(stream)))


def v4a_quantize_mxfp4(x: torch.Tensor, out: Idx, row0: int = 0, stream=None):
    rows = x.numel() // out.d if x.numel() else 0
    _check(lib().v4a_quantize_mxfp4(_ptr(x), rows, ctypes.byref(out.c()), row0, _stream(stream)))


def v4a_compress_csa(kv_a, kv_b, gate_a, gate_b, bias_a, bias_b, *, tok0: int, m: int,
                     first_entry: int, n_entries: int, apply_rope: bool = True,
                     rope_theta: float = 10000.0, out_kv: KV | None = None,
                     out_idx: Idx | None = None, b: int = 0, norm_w=None, stream=None):
    """Streams are [n_tok][D] (one sequence, slot b) or [n_seq][n_tok][D] (slots b..b+n_seq-1);
    norm_w [D] f32 RMS-normalises each merged entry before RoPE."""
    D = kv_a.shape[-1]
    G = gate_a.shape[-1]
    n_tok = kv_a.shape[-2]
    n_seq = kv_a.shape[0] if kv_a.dim() == 3 else 1
    _check(lib().v4a_compress_csa(
        _ptr(kv_a), _ptr(kv_b), _ftype(kv_a), D, _ptr(gate_a), _ptr(gate_b), G, _ptr(bias_a),
        _ptr(bias_b), tok0, n_tok, m, first_entry, n_entries, int(apply_rope), rope_theta, _ptr(norm_w),
        ctypes.byref(out_kv.c()) if out_kv is not None else None,
        ctypes.byref(out_idx.c()) if out_idx is not None else None, b, n_seq, _stream(stream)))


def v4a_compress_hca(kv, gate, bias, *, tok0: int, m: int, first_entry: int, n_entries: int,
                     apply_rope: bool = True, rope_theta: float = 10000.0, out_kv: KV, b: int = 0,
                     norm_w=None, stream=None):
    n_seq = kv.shape[0] if kv.dim() == 3 else 1
    _check(lib().v4a_compress_hca(
        _ptr(kv), _ftype(kv), kv.shape[-1], _ptr(gate), gate.shape[-1], _ptr(bias), tok0,
        kv.shape[-2], m, first_entry, n_entries, int(apply_rope), rope_theta, _ptr(norm_w),
        ctypes.byref(out_kv.c()), b, n_seq, _stream(stream)))


def v4a_indexer_topk_workspace(B: int, Q: int, n_max: int, k: int) -> int:
    return int(lib().v4a_indexer_topk_workspace(B, Q, n_max, k))


def v4a_indexer_topk(keys: Idx, n_entries, m: int, q_idx: Idx, w: torch.Tensor, B: int, Q: int,
                     H_I: int, q_pos, k: int, out: torch.Tensor, ws: torch.Tensor, stream=None):
    _check(lib().v4a_indexer_topk(
        ctypes.byref(keys.c()), _host_i64(n_entries), m, ctypes.byref(q_idx.c()), _ptr(w), B, Q,
        H_I, _host_i64(q_pos), k, _ptr(out), _ptr(ws), ws.numel() * ws.element_size(),
        _stream(stream)))


def v4a_indexer_topk_bf16(keys: Idx, n_entries, m: int, q_idx: Idx, w: torch.Tensor, B: int, Q: int,
                          H_I: int, q_pos, k: int, out: torch.Tensor, ws: torch.Tensor, stream=None):
    _check(lib().v4a_indexer_topk_bf16(
        ctypes.byref(keys.c()), _host_i64(n_entries), m, ctypes.byref(q_idx.c()), _ptr(w), B, Q,
        H_I, _host_i64(q_pos), k, _ptr(out), _ptr(ws), ws.numel() * ws.element_size(),
        _stream(stream)))


def v4a_indexer_scores(keys: Idx, n_entries, m: int, q_idx: Idx, w: torch.Tensor, B: int, Q: int,
                       H_I: int, q_pos, n_max: int, out: torch.Tensor, stream=None):
    _check(lib().v4a_indexer_scores(
        ctypes.byref(keys.c()), _host_i64(n_entries), m, ctypes.byref(q_idx.c()), _ptr(w), B, Q,
        H_I, _host_i64(q_pos), n_max, _ptr(out), _stream(stream)))


def v4a_decode_workspace(B: int, H: int, D: int, n_keys_max: int, W: int) -> int:
    return int(lib().v4a_decode_workspace(B, H, D, n_keys_max, W))


def v4a_decode_csa(q, kv: KV, topk_idx, k: int, win, win_len, W: int, sink, q_pos, *,
                   softmax_scale: float, out_rope_inverse: bool = True, rope_theta: float = 10000.0,
                   out: torch.Tensor, ws: torch.Tensor | None = None, stream=None):
    B, H = q.shape[0], q.shape[1]
    _check(lib().v4a_decode_csa(
        _ptr(q), _ftype(q), B, H, ctypes.byref(kv.c()), _ptr(topk_idx), k, _ptr(win),
        _ftype(win) if win is not None else V4A_BF16, _host_i32(win_len), W, _ptr(sink),
        _host_i64(q_pos), softmax_scale, int(out_rope_inverse), rope_theta, _ptr(out), _ftype(out),
        _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)))


def v4a_decode_hca(q, kv: KV, n_entries, m: int, win, win_len, W: int, sink, q_pos, *,
                   softmax_scale: float, out_rope_inverse: bool = True, rope_theta: float = 10000.0,
                   out: torch.Tensor, ws: torch.Tensor | None = None, stream=None):
    B, H = q.shape[0], q.shape[1]
    _check(lib().v4a_decode_hca(
        _ptr(q), _ftype(q), B, H, ctypes.byref(kv.c()), _host_i64(n_entries), m, _ptr(win),
        _ftype(win) if win is not None else V4A_BF16, _host_i32(win_len), W, _ptr(sink),
        _host_i64(q_pos), softmax_scale, int(out_rope_inverse), rope_theta, _ptr(out), _ftype(out),
        _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)))


class PrefillArgs:
    """The arguments of one prefill chunk (v4a_prefill_args), holding every tensor it points to.

    Streams hold n_prev + C rows (row r = position tok0 - n_prev + r); q is [C][H][D]; for CSA
    the indexer streams, key cache, q_idx ([C*H_I] rows), w ([C][H_I]) and k are required.
    """

    def __init__(self, *, tok0: int, n_prev: int, m: int, kv_a, gate_a, bias_a, kv: KV, q, W: int, sink,
                 softmax_scale: float, out, kv_b=None, gate_b=None, bias_b=None, slot: int = 0,
                 apply_rope: bool = True, rope_theta: float = 10000.0, idx_a=None, idx_b=None,
                 idx_gate_a=None, idx_gate_b=None, idx_bias_a=None, idx_bias_b=None, keys: Idx | None = None,
                 q_idx: Idx | None = None, w=None, k: int = 0, out_rope_inverse: bool = True,
                 score_bf16: bool = False, norm_w=None, idx_norm_w=None, q_norm_w=None):
        self._kv = kv.c()
        self._keys = keys.c() if keys is not None else None
        self._q_idx = q_idx.c() if q_idx is not None else None
        self._refs = (kv_a, kv_b, gate_a, gate_b, bias_a, bias_b, idx_a, idx_b, idx_gate_a, idx_gate_b,
                      idx_bias_a, idx_bias_b, w, q, sink, out, kv, keys, q_idx, norm_w, idx_norm_w, q_norm_w)
        C, H = q.shape[0], q.shape[1]
        H_I = (w.numel() // C) if (w is not None and C > 0) else 0
        self.s = c_prefill_args(
            tok0=tok0, C=C, n_prev=n_prev, m=m, in_t=_ftype(kv_a), G=gate_a.shape[-1],
            kv_a=_ptr(kv_a), kv_b=_ptr(kv_b), gate_a=_ptr(gate_a), gate_b=_ptr(gate_b), bias_a=_ptr(bias_a),
            bias_b=_ptr(bias_b), apply_rope=int(apply_rope), rope_theta=rope_theta,
            kv=ctypes.pointer(self._kv), slot=slot,
            idx_G=idx_gate_a.shape[-1] if idx_gate_a is not None else 0,
            idx_a=_ptr(idx_a), idx_b=_ptr(idx_b), idx_gate_a=_ptr(idx_gate_a), idx_gate_b=_ptr(idx_gate_b),
            idx_bias_a=_ptr(idx_bias_a), idx_bias_b=_ptr(idx_bias_b),
            keys=ctypes.pointer(self._keys) if self._keys is not None else None,
            q_idx=ctypes.pointer(self._q_idx) if self._q_idx is not None else None,
            w=_ptr(w), H_I=H_I, k=k, q=_ptr(q), q_t=_ftype(q), H=H, W=W, sink=_ptr(sink),
            softmax_scale=softmax_scale, out_rope_inverse=int(out_rope_inverse), out=_ptr(out),
            out_t=_ftype(out), score_bf16=int(score_bf16), norm_w=_ptr(norm_w), idx_norm_w=_ptr(idx_norm_w),
            q_norm_w=_ptr(q_norm_w))


def v4a_prefill_workspace(kind: int, args: PrefillArgs) -> int:
    return int(lib().v4a_prefill_workspace(kind, ctypes.byref(args.s)))


def v4a_prefill_chunk(kind: int, args: PrefillArgs, ws: torch.Tensor | None = None, stream=None):
    _check(lib().v4a_prefill_chunk(kind, ctypes.byref(args.s), _ptr(ws),
                                   0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)))


class DecodeStepArgs:
    """The arguments of one fused CSA decode step (v4a_decode_step_args), holding every tensor
    and host array it points to.  Streams hold [B][2m] rows per sequence (a ring [B][2m+Q-1]).
    With Q new tokens per sequence q and out are [B][Q][H][D] and w is [B][Q][H_I]."""

    def __init__(self, *, q_pos, n_entries, m: int, kv_a, kv_b, gate_a, gate_b, bias_a, bias_b, idx_a, idx_b,
                 idx_gate_a, idx_gate_b, idx_bias_a, idx_bias_b, kv: KV, keys: Idx, q_idx: Idx, w, k: int, q,
                 win, win_len, W: int, sink, softmax_scale: float, out, apply_rope: bool = True,
                 rope_theta: float = 10000.0, out_rope_inverse: bool = True, score_bf16: bool = False,
                 norm_w=None, idx_norm_w=None, ring: bool = False, no_split: bool = False, q_norm_w=None,
                 ws_clean: bool = False, Q: int = 1):
        B, H = q.shape[0], q.shape[-2]
        assert q.dim() == (4 if Q > 1 else 3), "q is [B][H][D], or [B][Q][H][D] with Q > 1"
        self._kv, self._keys, self._q_idx = kv.c(), keys.c(), q_idx.c()
        self._pos, self._nent, self._wl = _host_i64(q_pos), _host_i64(n_entries), _host_i32(win_len)
        self._refs = (kv_a, kv_b, gate_a, gate_b, bias_a, bias_b, idx_a, idx_b, idx_gate_a, idx_gate_b, idx_bias_a,
                      idx_bias_b, kv, keys, q_idx, w, q, win, sink, out, norm_w, idx_norm_w, q_norm_w)
        self.s = c_decode_step_args(
            B=B, m=m, q_pos=ctypes.cast(self._pos, ctypes.c_void_p), n_entries=ctypes.cast(self._nent, ctypes.c_void_p),
            in_t=_ftype(kv_a), G=gate_a.shape[-1], idx_G=idx_gate_a.shape[-1], kv_a=_ptr(kv_a), kv_b=_ptr(kv_b),
            gate_a=_ptr(gate_a), gate_b=_ptr(gate_b), bias_a=_ptr(bias_a), bias_b=_ptr(bias_b), idx_a=_ptr(idx_a),
            idx_b=_ptr(idx_b), idx_gate_a=_ptr(idx_gate_a), idx_gate_b=_ptr(idx_gate_b),
            idx_bias_a=_ptr(idx_bias_a), idx_bias_b=_ptr(idx_bias_b), apply_rope=int(apply_rope),
            rope_theta=rope_theta, kv=ctypes.pointer(self._kv), keys=ctypes.pointer(self._keys),
            q_idx=ctypes.pointer(self._q_idx), w=_ptr(w), H_I=w.numel() // (B * Q), k=k, q=_ptr(q), q_t=_ftype(q), H=H,
            win=_ptr(win), win_t=_ftype(win), win_len=ctypes.cast(self._wl, ctypes.c_void_p), W=W, sink=_ptr(sink),
            softmax_scale=softmax_scale, out_rope_inverse=int(out_rope_inverse), out=_ptr(out), out_t=_ftype(out),
            score_bf16=int(score_bf16), norm_w=_ptr(norm_w), idx_norm_w=_ptr(idx_norm_w), ring=int(ring),
            no_split=int(no_split), q_norm_w=_ptr(q_norm_w), ws_clean=int(ws_clean), Q=Q)


def v4a_decode_step_workspace(args: DecodeStepArgs) -> int:
    return int(lib().v4a_decode_step_workspace(ctypes.byref(args.s)))


def v4a_decode_step_csa(args: DecodeStepArgs, ws: torch.Tensor, stream=None):
    _check(lib().v4a_decode_step_csa(ctypes.byref(args.s), _ptr(ws), ws.numel() * ws.element_size(),
                                     _stream(stream)))


def v4a_output_projection_workspace(T: int, G: int, r: int) -> int:
    return int(lib().v4a_output_projection_workspace(T, G, r))


def v4a_output_projection(o: torch.Tensor, G: int, r: int, wg: torch.Tensor, wf: torch.Tensor, out: torch.Tensor,
                          ws: torch.Tensor, stream=None):
    """Grouped output projection of the attention output o [T][H][D] (bf16): group weights wg
    [G][r][H*D/G], final weights wf [d][G*r] (bf16), out [T][d]; ws holds the reduced groups y
    [T][G*r] (bf16)."""
    T, H, D = o.shape
    _check(lib().v4a_output_projection(_ptr(o), T, H, D, G, r, _ptr(wg), _ptr(wf), wf.shape[0], _ptr(out),
                                       _ftype(out), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


V4A_NOALLOC_SCRATCH_BYTES = 64 << 20  # the library's per-device scratch (include/v4attn.h)


def v4a_decode_step_csa_noalloc(args: DecodeStepArgs, stream=None):
    """The fused CSA decode step on the library's own per-device scratch (no workspace)."""
    _check(lib().v4a_decode_step_csa_noalloc(ctypes.byref(args.s), _stream(stream)))


def workspace(nbytes: int, device="cuda") -> torch.Tensor:
    """A caller-owned workspace buffer (torch allocations are 256-byte aligned)."""
    return torch.empty((max(int(nbytes), 1),), dtype=torch.uint8, device=device)


class DecodeStepHcaArgs:
    """The arguments of one fused HCA decode step (v4a_decode_step_hca_args), holding every tensor
    and host array it points to.  The stream holds [B][m] rows per sequence (a ring [B][m+Q-1]).
    With Q new tokens per sequence q and out are [B][Q][H][D]."""

    def __init__(self, *, q_pos, n_entries, m: int, kv_a, gate_a, bias_a, kv: KV, q, win, win_len, W: int, sink,
                 softmax_scale: float, out, apply_rope: bool = True, rope_theta: float = 10000.0,
                 out_rope_inverse: bool = True, norm_w=None, ring: bool = False, no_split: bool = False,
                 q_norm_w=None, Q: int = 1):
        B, H = q.shape[0], q.shape[-2]
        assert q.dim() == (4 if Q > 1 else 3), "q is [B][H][D], or [B][Q][H][D] with Q > 1"
        self._kv = kv.c()
        self._pos, self._nent, self._wl = _host_i64(q_pos), _host_i64(n_entries), _host_i32(win_len)
        self._refs = (kv_a, gate_a, bias_a, kv, q, win, sink, out, norm_w, q_norm_w)
        self.s = c_decode_step_hca_args(
            B=B, m=m, q_pos=ctypes.cast(self._pos, ctypes.c_void_p), n_entries=ctypes.cast(self._nent, ctypes.c_void_p),
            in_t=_ftype(kv_a), G=gate_a.shape[-1], kv_a=_ptr(kv_a), gate_a=_ptr(gate_a), bias_a=_ptr(bias_a),
            apply_rope=int(apply_rope), rope_theta=rope_theta, norm_w=_ptr(norm_w), kv=ctypes.pointer(self._kv),
            q=_ptr(q), q_t=_ftype(q), H=H, win=_ptr(win), win_t=_ftype(win),
            win_len=ctypes.cast(self._wl, ctypes.c_void_p), W=W, sink=_ptr(sink), softmax_scale=softmax_scale,
            out_rope_inverse=int(out_rope_inverse), out=_ptr(out), out_t=_ftype(out), ring=int(ring),
            no_split=int(no_split), q_norm_w=_ptr(q_norm_w), Q=Q)


def v4a_decode_step_hca_workspace(args: DecodeStepHcaArgs) -> int:
    return int(lib().v4a_decode_step_hca_workspace(ctypes.byref(args.s)))


def v4a_decode_step_hca(args: DecodeStepHcaArgs, ws: torch.Tensor | None, stream=None):
    _check(lib().v4a_decode_step_hca(ctypes.byref(args.s), _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(),
                                     _stream(stream)))
