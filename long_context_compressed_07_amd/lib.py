"""ctypes binding of libcsa (include/csa.h). Argument marshalling only: every step of the layer runs
in the library's HIP kernels; torch provides device memory and the current stream.

The names mirror the C entry points. Tensors must already live on the GPU in the layouts the
header documents; bf16 data may be passed as torch.bfloat16 or as int16/uint16 codes, e4m3 data as
torch.float8_e4m3fn or uint8 codes. Raises RuntimeError on any non-OK status and if the shared
library is missing (there is no fallback path).
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

F32, BF16, E4M3 = 0, 1, 2
DTYPES = {"f32": F32, "bf16": BF16, "e4m3": E4M3}

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libcsa.so")
_lib = None

EXPORTS = ("csa_compress", "csa_index", "csa_topk", "csa_topk_workspace_bytes", "csa_attend",
           "csa_attend_workspace_bytes", "hca_attend", "hca_attend_workspace_bytes",
           "csa_status_str", "csa_last_error", "csa_abi_version", "csa_kernel_timing_enable",
           "csa_kernel_timing_read", "csa_peak_mfma_bf16", "csa_peak_sink_floats",
           "csa_cache_append", "csa_attend_tokens", "csa_index_mxfp4", "csa_topk_bf16",
           "csa_topk_noalloc")


class KV(ctypes.Structure):
    _fields_ = [("c", ctypes.c_void_p), ("r", ctypes.c_void_p), ("scale", ctypes.c_void_p),
                ("pos0", ctypes.c_void_p), ("dtype_c", ctypes.c_int32), ("d_c", ctypes.c_int32),
                ("d_r", ctypes.c_int32), ("rows", ctypes.c_int64), ("ld_c", ctypes.c_int64),
                ("ld_r", ctypes.c_int64)]


class KVOut(ctypes.Structure):
    _fields_ = [("c", ctypes.c_void_p), ("r", ctypes.c_void_p), ("scale", ctypes.c_void_p),
                ("dtype_c", ctypes.c_int32), ("d_c", ctypes.c_int32), ("d_r", ctypes.c_int32),
                ("rows", ctypes.c_int64), ("ld_c", ctypes.c_int64), ("ld_r", ctypes.c_int64)]


class Queries(ctypes.Structure):
    _fields_ = [("seq", ctypes.c_void_p), ("pos", ctypes.c_void_p), ("nq", ctypes.c_int32)]


def load(path: str = LIB_PATH):
    """Open libcsa.so (once) and declare the exported signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -m long_context_compressed_07_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i32, i64, f32, sz = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float,
                             ctypes.c_size_t)
    P = ctypes.POINTER
    lib.csa_compress.argtypes = [vp, vp, i32, vp, i32, i32, i64, i32, i32, vp, vp, vp, i32,
                                 P(KVOut), vp, vp]
    lib.csa_index.argtypes = [P(Queries), vp, vp, i32, vp, i32, i32, vp, vp, i32, i32, i64, i32,
                              vp, i64, vp]
    lib.csa_topk.argtypes = [P(Queries), vp, i64, i64, i32, i32, vp, vp, sz, vp]
    lib.csa_topk_workspace_bytes.argtypes = [i32, i64, i32]
    lib.csa_topk_bf16.argtypes = [P(Queries), vp, i64, i64, i32, i32, vp, vp, sz, vp]
    lib.csa_topk_noalloc.argtypes = [P(Queries), vp, i64, i64, i32, i32, vp, vp]
    lib.csa_index_mxfp4.argtypes = [P(Queries), vp, vp, vp, i32, i32, vp, vp, i32, i64, i32, vp,
                                    i64, vp]
    lib.csa_attend.argtypes = [P(Queries), vp, i32, i32, P(KV), i32, vp, i32, P(KV), i32, f32,
                               vp, vp, vp, sz, vp]
    lib.csa_attend_workspace_bytes.argtypes = [i32, i32, i32, i64]
    lib.hca_attend.argtypes = [P(Queries), vp, i32, i32, P(KV), i32, f32, vp, vp, vp, sz, vp]
    lib.csa_attend_tokens.argtypes = [P(Queries), vp, i32, i32, P(KV), i32, vp, i32, i32, f32,
                                      vp, vp, vp, sz, vp]
    lib.hca_attend_workspace_bytes.argtypes = [i32, i32, i32, i64]
    lib.csa_kernel_timing_enable.argtypes = [i32]
    lib.csa_kernel_timing_read.argtypes = [i32, P(ctypes.c_double), P(i32)]
    lib.csa_peak_mfma_bf16.argtypes = [i32, vp, P(ctypes.c_double), vp]
    lib.csa_peak_sink_floats.argtypes = []
    lib.csa_cache_append.argtypes = [vp, vp, i32, vp, i32, i32, vp, i32, i32, vp, vp, P(KVOut),
                                     P(KVOut), vp, vp]
    for fn in ("csa_compress", "csa_index", "csa_topk", "csa_attend", "hca_attend",
               "csa_abi_version", "csa_kernel_timing_enable", "csa_kernel_timing_read",
               "csa_peak_mfma_bf16", "csa_peak_sink_floats", "csa_cache_append",
               "csa_attend_tokens", "csa_index_mxfp4", "csa_topk_bf16", "csa_topk_noalloc"):
        getattr(lib, fn).restype = ctypes.c_int32
    for fn in ("csa_topk_workspace_bytes", "csa_attend_workspace_bytes",
               "hca_attend_workspace_bytes"):
        getattr(lib, fn).restype = ctypes.c_size_t
    lib.csa_status_str.argtypes = [ctypes.c_int32]
    lib.csa_status_str.restype = ctypes.c_char_p
    lib.csa_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensor must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr()


def _stream(stream) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _check(status: int, what: str):
    if status != 0:
        lib = load()
        raise RuntimeError(f"{what}: {lib.csa_status_str(status).decode()} "
                           f"({lib.csa_last_error().decode()})")


class Bound:
    """A library call with its arguments marshalled once (the bind=True form of the call
    functions below): `bound(stream_handle)` enqueues the same call, on the same tensors, on a
    raw stream handle (`torch.cuda.Stream.cuda_stream`). It keeps the tensors it points into
    alive. Marshalling once keeps the host's cost per call at one foreign call, which matters
    where a decode step's kernels are a few tens of microseconds each."""
    __slots__ = ("fn", "args", "what", "keep")

    def __init__(self, fn, args: tuple, what: str, keep: tuple):
        self.fn, self.args, self.what, self.keep = fn, args, what, keep

    def __call__(self, stream_handle: int):
        status = self.fn(*self.args, stream_handle)
        if status != 0:
            _check(status, self.what)


def _call(fn, args: tuple, what: str, stream, bind: bool, keep: tuple):
    if bind:
        return Bound(fn, args, what, keep)
    _check(fn(*args, _stream(stream)), what)
    return None


@dataclass
class Store:
    """A cache-row store (csa_kv_t): c [B, rows, ld_c], r [B, rows, ld_r] (or a view into c's
    buffer via r_offset), scale [B, rows] for e4m3, pos0 [B] int64 for raw stores."""
    c: torch.Tensor
    dtype: int
    d_c: int
    d_r: int
    rows: int
    ld_c: int
    r: Optional[torch.Tensor] = None
    ld_r: int = 0
    scale: Optional[torch.Tensor] = None
    pos0: Optional[torch.Tensor] = None
    r_offset: int = -1   # >= 0: r lives inside c's rows at this element offset

    def _r_ptr(self):
        if self.d_r == 0:
            return None
        if self.r_offset >= 0:
            return _ptr(self.c) + self.r_offset * self.c.element_size()
        return _ptr(self.r)

    def _ld_r(self):
        return self.ld_c if self.r_offset >= 0 else self.ld_r

    def as_c(self) -> KV:
        return KV(_ptr(self.c), self._r_ptr(), _ptr(self.scale), _ptr(self.pos0), self.dtype,
                  self.d_c, self.d_r, self.rows, self.ld_c, self._ld_r())

    def as_out(self) -> KVOut:
        return KVOut(_ptr(self.c), self._r_ptr(), _ptr(self.scale), self.dtype, self.d_c,
                     self.d_r, self.rows, self.ld_c, self._ld_r())


def _queries(seq: torch.Tensor, pos: torch.Tensor) -> Queries:
    if seq.dtype != torch.int32 or pos.dtype != torch.int64:
        raise ValueError("seq must be int32 and pos int64")
    return Queries(_ptr(seq), _ptr(pos), seq.numel())


def csa_cache_append(x_new, g_new, in_dtype: int, bias, m: int, pos, d_c: int, d_r: int,
                     stage_x, stage_g, entries: Store, raw: Optional[Store], raw_pos0=None,
                     stream=None):
    """One new token per sequence: staging ring, raw ring row (raw may be None), and the entry of
    a completed block (csa_cache_append in include/csa.h)."""
    lib = load()
    if pos.dtype != torch.int64 or (raw_pos0 is not None and raw_pos0.dtype != torch.int64):
        raise ValueError("pos and raw_pos0 must be int64")
    e = entries.as_out()
    r = raw.as_out() if raw is not None else None
    _check(lib.csa_cache_append(_ptr(x_new), _ptr(g_new), in_dtype, _ptr(bias), m, pos.numel(),
                                _ptr(pos), d_c, d_r, _ptr(stage_x), _ptr(stage_g),
                                ctypes.byref(e), ctypes.byref(r) if r is not None else None,
                                _ptr(raw_pos0), _stream(stream)), "csa_cache_append")


def csa_compress(x, g, in_dtype: int, bias, m: int, B: int, T: int, d_c: int, d_r: int,
                 out: Store, hidden=None, w_x=None, w_g=None, d_model: int = 0,
                 raw_x_out=None, stream=None, bind: bool = False):
    lib = load()
    o = out.as_out()
    args = (_ptr(x), _ptr(g), in_dtype, _ptr(bias), m, B, T, d_c, d_r, _ptr(hidden), _ptr(w_x),
            _ptr(w_g), d_model, ctypes.byref(o), _ptr(raw_x_out))
    return _call(lib.csa_compress, args, "csa_compress", stream, bind,
                 (x, g, bias, out, hidden, w_x, w_g, raw_x_out, o))


def csa_index(seq, pos, q_i, w, k_i, scores, dtype: int, H_I: int, d_I: int, B: int, N: int,
              m: int, q_i_scale=None, k_i_scale=None, ld_scores: Optional[int] = None,
              stream=None, bind: bool = False):
    lib = load()
    Q = _queries(seq, pos)
    ld = N if ld_scores is None else ld_scores
    args = (ctypes.byref(Q), _ptr(q_i), _ptr(q_i_scale), dtype, _ptr(w), H_I, d_I, _ptr(k_i),
            _ptr(k_i_scale), dtype, B, N, m, _ptr(scores), ld)
    return _call(lib.csa_index, args, "csa_index", stream, bind,
                 (seq, pos, q_i, w, k_i, scores, q_i_scale, k_i_scale, Q))


def csa_topk_workspace_bytes(nq: int, N: int, k: int) -> int:
    return load().csa_topk_workspace_bytes(nq, N, k)


def csa_topk(seq, pos, scores, idx, N: int, m: int, k: int, ld_scores: Optional[int] = None,
             ws: Optional[torch.Tensor] = None, stream=None, bind: bool = False):
    lib = load()
    Q = _queries(seq, pos)
    need = lib.csa_topk_workspace_bytes(Q.nq, N, k)
    if ws is None and need > 0:
        ws = torch.empty(need, dtype=torch.uint8, device=scores.device)
    ld = N if ld_scores is None else ld_scores
    args = (ctypes.byref(Q), _ptr(scores), ld, N, m, k, _ptr(idx), _ptr(ws),
            0 if ws is None else ws.numel())
    return _call(lib.csa_topk, args, "csa_topk", stream, bind, (seq, pos, scores, idx, ws, Q))


def csa_index_mxfp4(seq, pos, q_i, q_i_scale, w, k_i, k_i_scale, scores, H_I: int, d_I: int,
                    B: int, N: int, m: int, ld_scores: Optional[int] = None, stream=None):
    """MXFP4 indexer with bf16 scores (csa_index_mxfp4 in include/csa.h); scores are int16/uint16
    (bf16 codes) or torch.bfloat16."""
    lib = load()
    Q = _queries(seq, pos)
    ld = N if ld_scores is None else ld_scores
    _check(lib.csa_index_mxfp4(ctypes.byref(Q), _ptr(q_i), _ptr(q_i_scale), _ptr(w), H_I, d_I,
                               _ptr(k_i), _ptr(k_i_scale), B, N, m, _ptr(scores), ld,
                               _stream(stream)), "csa_index_mxfp4")


def csa_topk_bf16(seq, pos, scores, idx, N: int, m: int, k: int,
                  ld_scores: Optional[int] = None, ws: Optional[torch.Tensor] = None,
                  stream=None):
    """Top-k on bf16 scores (csa_topk_bf16 in include/csa.h)."""
    lib = load()
    Q = _queries(seq, pos)
    need = lib.csa_topk_workspace_bytes(Q.nq, N, k)
    if ws is None and need > 0:
        ws = torch.empty(need, dtype=torch.uint8, device=scores.device)
    ld = N if ld_scores is None else ld_scores
    _check(lib.csa_topk_bf16(ctypes.byref(Q), _ptr(scores), ld, N, m, k, _ptr(idx), _ptr(ws),
                             0 if ws is None else ws.numel(), _stream(stream)), "csa_topk_bf16")


def csa_topk_noalloc(seq, pos, scores, idx, N: int, m: int, k: int,
                     ld_scores: Optional[int] = None, stream=None):
    """Top-k with the library's own scratch, allocating nothing (csa_topk_noalloc in
    include/csa.h)."""
    lib = load()
    Q = _queries(seq, pos)
    ld = N if ld_scores is None else ld_scores
    _check(lib.csa_topk_noalloc(ctypes.byref(Q), _ptr(scores), ld, N, m, k, _ptr(idx),
                                _stream(stream)), "csa_topk_noalloc")


def csa_attend_workspace_bytes(nq: int, H: int, d_c: int, max_keys: int) -> int:
    return load().csa_attend_workspace_bytes(nq, H, d_c, max_keys)


def hca_attend_workspace_bytes(nq: int, H: int, d_c: int, N: int) -> int:
    return load().hca_attend_workspace_bytes(nq, H, d_c, N)


def csa_attend(seq, pos, q, q_dtype: int, H: int, entries: Store, m: int, idx, k: int,
               raw: Optional[Store], window: int, sm_scale: float, out, lse=None,
               ws: Optional[torch.Tensor] = None, stream=None, bind: bool = False):
    lib = load()
    Q = _queries(seq, pos)
    need = lib.csa_attend_workspace_bytes(Q.nq, H, entries.d_c, k + window)
    if ws is None and need > 0:
        ws = torch.empty(need, dtype=torch.uint8, device=q.device)
    e = entries.as_c()
    r = raw.as_c() if raw is not None else None
    args = (ctypes.byref(Q), _ptr(q), q_dtype, H, ctypes.byref(e), m, _ptr(idx), k,
            ctypes.byref(r) if r is not None else None, window, sm_scale, _ptr(out), _ptr(lse),
            _ptr(ws), 0 if ws is None else ws.numel())
    return _call(lib.csa_attend, args, "csa_attend", stream, bind,
                 (seq, pos, q, entries, idx, raw, out, lse, ws, Q, e, r))


def csa_attend_tokens(seq, pos, q, q_dtype: int, H: int, raw: Store, m: int, idx, k: int,
                      window: int, sm_scale: float, out, lse=None,
                      ws: Optional[torch.Tensor] = None, stream=None):
    """Attention over the m raw tokens of each selected block plus the window
    (csa_attend_tokens in include/csa.h)."""
    lib = load()
    Q = _queries(seq, pos)
    need = lib.csa_attend_workspace_bytes(Q.nq, H, raw.d_c, k * m + window)
    if ws is None and need > 0:
        ws = torch.empty(need, dtype=torch.uint8, device=q.device)
    r = raw.as_c()
    _check(lib.csa_attend_tokens(ctypes.byref(Q), _ptr(q), q_dtype, H, ctypes.byref(r), m,
                                 _ptr(idx), k, window, sm_scale, _ptr(out), _ptr(lse), _ptr(ws),
                                 0 if ws is None else ws.numel(), _stream(stream)),
           "csa_attend_tokens")


def hca_attend(seq, pos, q, q_dtype: int, H: int, entries: Store, m_prime: int,
               sm_scale: float, out, lse=None, ws: Optional[torch.Tensor] = None, stream=None,
               bind: bool = False):
    lib = load()
    Q = _queries(seq, pos)
    need = lib.hca_attend_workspace_bytes(Q.nq, H, entries.d_c, entries.rows)
    if ws is None and need > 0:
        ws = torch.empty(need, dtype=torch.uint8, device=q.device)
    e = entries.as_c()
    args = (ctypes.byref(Q), _ptr(q), q_dtype, H, ctypes.byref(e), m_prime, sm_scale, _ptr(out),
            _ptr(lse), _ptr(ws), 0 if ws is None else ws.numel())
    return _call(lib.hca_attend, args, "hca_attend", stream, bind,
                 (seq, pos, q, entries, out, lse, ws, Q, e))


def kernel_timing_enable(cap: int):
    """Record HIP events around the next `cap` main attention kernels of csa_attend (slot 0) and
    hca_attend (slot 1); cap = 0 stops."""
    _check(load().csa_kernel_timing_enable(cap), "csa_kernel_timing_enable")


def peak_mfma_bf16(iters: int = 50000, stream=None) -> float:
    """Measured dense bf16 MFMA rate of the current device in TFLOP/s (waits for the stream)."""
    L = load()
    sink = torch.empty(L.csa_peak_sink_floats(), dtype=torch.float32, device="cuda")
    tf = ctypes.c_double()
    _check(L.csa_peak_mfma_bf16(iters, _ptr(sink), ctypes.byref(tf), _stream(stream)),
           "csa_peak_mfma_bf16")
    return tf.value


def kernel_timing_read(slot: int) -> tuple[float, int]:
    """(total milliseconds, launches) recorded in a slot since the last read."""
    ms, n = ctypes.c_double(), ctypes.c_int32()
    _check(load().csa_kernel_timing_read(slot, ctypes.byref(ms), ctypes.byref(n)),
           "csa_kernel_timing_read")
    return ms.value, n.value
