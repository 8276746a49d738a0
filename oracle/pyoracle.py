"""ctypes wrapper of the CPU oracle.  TEST INFRASTRUCTURE ONLY.

Used by the test suite, the smoke check and the benchmark's CPU-baseline leg;
nothing in the product package imports it.
"""
from __future__ import annotations

import ctypes as C

import numpy as np

from .build import ensure_built

_lib = None


class OrcCfg(C.Structure):
    _fields_ = [("n_layers", C.c_int), ("hidden", C.c_int), ("n_q_heads", C.c_int), ("n_kv_heads", C.c_int),
                ("head_dim", C.c_int), ("ffn", C.c_int), ("vocab", C.c_int), ("rms_eps", C.c_float),
                ("rope_theta", C.c_double), ("qk_norm", C.c_int), ("max_seq", C.c_int), ("n_threads", C.c_int),
                ("lora_rank", C.c_int)]


def lib():
    global _lib
    if _lib is None:
        L = C.CDLL(ensure_built())
        u16p, f32p, f64p = C.POINTER(C.c_uint16), C.POINTER(C.c_float), C.POINTER(C.c_double)
        L.orc_n_weights.argtypes = [C.POINTER(OrcCfg)]
        L.orc_weight_numel.argtypes = [C.POINTER(OrcCfg), C.c_int]
        L.orc_weight_numel.restype = C.c_int64
        L.orc_create.argtypes = [C.POINTER(OrcCfg), C.POINTER(u16p), C.c_int]
        L.orc_create.restype = C.c_void_p
        L.orc_destroy.argtypes = [C.c_void_p]
        L.orc_seq_create.argtypes = [C.c_void_p]
        L.orc_seq_create.restype = C.c_void_p
        L.orc_seq_destroy.argtypes = [C.c_void_p]
        L.orc_seq_set_kv.argtypes = [C.c_void_p, C.c_int, u16p, u16p]
        L.orc_seq_pos.argtypes = [C.c_void_p]
        L.orc_seq_step.argtypes = [C.c_void_p, C.c_int, f32p]
        L.orc_bf16_to_f32.argtypes = [C.c_uint16]
        L.orc_bf16_to_f32.restype = C.c_float
        L.orc_f32_to_bf16.argtypes = [C.c_float]
        L.orc_f32_to_bf16.restype = C.c_uint16
        L.orc_matvec.argtypes = [u16p, C.c_int, C.c_int, f64p, f64p, C.c_int]
        L.orc_lora_linear.argtypes = [u16p, u16p, u16p, C.c_int, C.c_int, C.c_int, f64p, f64p, C.c_int]
        L.orc_rmsnorm.argtypes = [f32p, u16p, C.c_int, C.c_float, f64p]
        L.orc_rope.argtypes = [f64p, C.c_int, C.c_int, C.c_double]
        L.orc_attend.argtypes = [f64p, u16p, u16p, C.c_int, C.c_int, C.c_int, f32p]
        L.orc_silu.argtypes = [C.c_double]
        L.orc_silu.restype = C.c_double
        L.orc_argmax.argtypes = [f32p, C.c_int]
        _lib = L
    return _lib


def _f32(a):
    a = np.ascontiguousarray(a, dtype=np.float32)
    return a, a.ctypes.data_as(C.POINTER(C.c_float))


def _f64(a):
    a = np.ascontiguousarray(a, dtype=np.float64)
    return a, a.ctypes.data_as(C.POINTER(C.c_double))


def _u16(a):
    a = np.ascontiguousarray(a, dtype=np.uint16)
    return a, a.ctypes.data_as(C.POINTER(C.c_uint16))


# ---- primitives -------------------------------------------------------------
def bf16_to_f32(b: int) -> float:
    return lib().orc_bf16_to_f32(b)


def f32_to_bf16(f: float) -> int:
    return lib().orc_f32_to_bf16(f)


def matvec(W16: np.ndarray, x: np.ndarray, n_threads: int = 1) -> np.ndarray:
    """fp64 W @ x (x is taken as float64)."""
    rows, cols = W16.shape
    W16, wp = _u16(W16)
    x, xp = _f64(x)
    y = np.zeros(rows, np.float64)
    lib().orc_matvec(wp, rows, cols, xp, y.ctypes.data_as(C.POINTER(C.c_double)), n_threads)
    return y


def lora_linear(W16: np.ndarray, A16: np.ndarray | None, B16: np.ndarray | None, x: np.ndarray,
                n_threads: int = 1) -> np.ndarray:
    """fp64 W @ x + B @ fp32(A @ x), one sequential sum per concatenated row."""
    rows, cols = W16.shape
    r = 0 if A16 is None else A16.shape[0]
    W16, wp = _u16(W16)
    ap = bp = None
    if A16 is not None:
        A16, ap = _u16(A16)
        B16, bp = _u16(B16)
    x, xp = _f64(x)
    y = np.zeros(rows, np.float64)
    lib().orc_lora_linear(wp, ap, bp, rows, cols, r, xp, y.ctypes.data_as(C.POINTER(C.c_double)), n_threads)
    return y


def rmsnorm(x: np.ndarray, gamma16: np.ndarray, eps: float) -> np.ndarray:
    """fp64 RMSNorm of an fp32 vector."""
    x, xp = _f32(x)
    gamma16, gp = _u16(gamma16)
    y = np.zeros(x.size, np.float64)
    lib().orc_rmsnorm(xp, gp, x.size, eps, y.ctypes.data_as(C.POINTER(C.c_double)))
    return y


def rope(x: np.ndarray, pos: int, theta: float) -> np.ndarray:
    """fp64 rotate-half RoPE."""
    x = np.array(x, dtype=np.float64, copy=True)
    lib().orc_rope(x.ctypes.data_as(C.POINTER(C.c_double)), x.size, pos, theta)
    return x


def attend(q: np.ndarray, K16: np.ndarray, V16: np.ndarray) -> np.ndarray:
    """fp64 attention of one head; fp32 output."""
    n, d = K16.shape
    q, qp = _f64(q)
    K16, kp = _u16(K16)
    V16, vp = _u16(V16)
    o = np.zeros(d, np.float32)
    lib().orc_attend(qp, kp, vp, n, d, d, o.ctypes.data_as(C.POINTER(C.c_float)))
    return o


def silu(z: float) -> float:
    return lib().orc_silu(z)


def argmax(x: np.ndarray) -> int:
    x, xp = _f32(x)
    return lib().orc_argmax(xp, x.size)


# ---- decoder ----------------------------------------------------------------
class Oracle:
    """A model (weights by reference) plus one KV cache per sequence."""

    def __init__(self, shape, weights16: list[np.ndarray], max_seq: int, n_seq: int = 1, n_threads: int = 1):
        self.cfg = OrcCfg(shape.n_layers, shape.hidden, shape.n_q_heads, shape.n_kv_heads, shape.head_dim,
                          shape.ffn, shape.vocab, shape.rms_eps, shape.rope_theta, int(shape.qk_norm), max_seq,
                          n_threads, int(getattr(shape, "lora_rank", 0)))
        L = lib()
        n = L.orc_n_weights(C.byref(self.cfg))
        if n != len(weights16):
            raise ValueError(f"expected {n} weight tensors, got {len(weights16)}")
        self._keep = [np.ascontiguousarray(w, dtype=np.uint16).reshape(-1) for w in weights16]
        for i, w in enumerate(self._keep):
            if w.size != L.orc_weight_numel(C.byref(self.cfg), i):
                raise ValueError(f"weight {i}: numel {w.size} != {L.orc_weight_numel(C.byref(self.cfg), i)}")
        arr = (C.POINTER(C.c_uint16) * n)(*[w.ctypes.data_as(C.POINTER(C.c_uint16)) for w in self._keep])
        self._arr = arr
        self.m = L.orc_create(C.byref(self.cfg), arr, n)
        if not self.m:
            raise ValueError("orc_create failed")
        self.vocab = shape.vocab
        self.seqs = [L.orc_seq_create(self.m) for _ in range(n_seq)]
        if not all(self.seqs):
            raise MemoryError("orc_seq_create failed")

    def set_kv(self, seq: int, k16: np.ndarray, v16: np.ndarray):
        n_pos = k16.shape[1]
        k16, kp = _u16(k16)
        v16, vp = _u16(v16)
        if lib().orc_seq_set_kv(self.seqs[seq], n_pos, kp, vp) != 0:
            raise ValueError("orc_seq_set_kv failed")

    def pos(self, seq: int = 0) -> int:
        return lib().orc_seq_pos(self.seqs[seq])

    def step(self, seq: int, token: int, want_logits: bool = True):
        out = np.zeros(self.vocab, np.float32) if want_logits else None
        p = out.ctypes.data_as(C.POINTER(C.c_float)) if want_logits else None
        if lib().orc_seq_step(self.seqs[seq], int(token), p) != 0:
            raise ValueError("orc_seq_step failed (cache full or bad token)")
        return out

    def close(self):
        L = lib()
        for s in self.seqs:
            L.orc_seq_destroy(s)
        self.seqs = []
        if self.m:
            L.orc_destroy(self.m)
            self.m = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
