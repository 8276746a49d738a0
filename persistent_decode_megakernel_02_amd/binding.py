"""ctypes binding of libmk.so: the same entry points as include/mk.h.

Argument marshalling only: every step of decode runs in the library's HIP
kernels.  torch tensors are accepted where the C ABI takes device or host
pointers; torch's current stream is handed to the library.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
# MK_LIBRARY selects a variant build (build.py VARIANTS) for measurements; the default is the
# in-tree library.
LIB_PATH = os.environ.get("MK_LIBRARY") or os.path.join(HERE, "libmk.so")

MK_OK = 0
MK_ERR = {-1: "INVALID_ARG", -2: "UNSUPPORTED", -3: "OOM", -4: "HIP", -5: "CAPACITY", -6: "TIMEOUT", -7: "STATE"}
(MK_ERR_INVALID_ARG, MK_ERR_UNSUPPORTED, MK_ERR_OOM, MK_ERR_HIP, MK_ERR_CAPACITY, MK_ERR_TIMEOUT,
 MK_ERR_STATE) = range(-1, -8, -1)
MK_MODE_MEGAKERNEL = 0
MK_MODE_PER_OP = 1
MK_PREFILL_PER_OP = 0
MK_PREFILL_MEGAKERNEL = 1
MK_SCHEDULE_FROZEN = 0
MK_SCHEDULE_GIVEN = 1
SCHEDULE_FIELDS = ("qkv_tiles", "wo_tiles", "gu_tiles", "down_tiles", "lm_tiles", "rotate", "attn_offset",
                   "wo_ksplit", "down_ksplit", "qkv_ksplit")


class MkError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{MK_ERR.get(code, code)}: {msg}")
        self.code = code


class MkModelCfg(C.Structure):
    _fields_ = [("n_layers", C.c_int32), ("hidden", C.c_int32), ("n_q_heads", C.c_int32), ("n_kv_heads", C.c_int32),
                ("head_dim", C.c_int32), ("ffn", C.c_int32), ("vocab", C.c_int32), ("rms_eps", C.c_float),
                ("rope_theta", C.c_double), ("qk_norm", C.c_int32), ("batch", C.c_int32), ("max_seq", C.c_int32),
                ("mode", C.c_int32), ("split", C.c_int32), ("n_workers", C.c_int32), ("watchdog_polls", C.c_uint32),
                ("stream", C.c_void_p), ("schedule", C.c_int32), ("qkv_tiles", C.c_int32), ("wo_tiles", C.c_int32),
                ("gu_tiles", C.c_int32), ("down_tiles", C.c_int32), ("lm_tiles", C.c_int32), ("rotate", C.c_int32),
                ("attn_offset", C.c_int32), ("wo_ksplit", C.c_int32), ("down_ksplit", C.c_int32),
                ("qkv_ksplit", C.c_int32),
                ("lora_rank", C.c_int32), ("prefill", C.c_int32)]


class MkTensor(C.Structure):
    _fields_ = [("name", C.c_char_p), ("data", C.c_void_p), ("numel", C.c_int64), ("on_device", C.c_int32)]


EXPORTS = ["mk_create", "mk_load_weights", "mk_prefill", "mk_prefill_noalloc", "mk_load_kv", "mk_decode", "mk_set_mode",
           "mk_set_prefill", "mk_get_state",
           "mk_get_config",
           "mk_get_graph", "mk_build_graph", "mk_build_prefill_graph", "mk_reset", "mk_last_decode_ms", "mk_set_trace", "mk_get_trace",
           "mk_read_bandwidth", "mk_copy_bandwidth", "mk_debug_poison",
           "mk_last_error", "mk_destroy"]

_lib = None


def lib():
    """Load libmk.so; fails loudly if the HIP library has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with `python -m persistent_decode_megakernel_02_amd.build`"
                              " (or __graft_entry__.build())")
        L = C.CDLL(LIB_PATH)
        vp, i32, sz = C.c_void_p, C.c_int32, C.c_size_t
        L.mk_create.argtypes = [C.POINTER(MkModelCfg), C.POINTER(vp)]
        L.mk_load_weights.argtypes = [vp, C.POINTER(MkTensor), C.c_int]
        L.mk_prefill.argtypes = [vp, C.POINTER(i32), C.c_int]
        L.mk_prefill_noalloc.argtypes = [vp, C.POINTER(i32), C.c_int]
        L.mk_load_kv.argtypes = [vp, C.c_int, C.c_int, vp, vp, i32, C.c_int]
        L.mk_decode.argtypes = [vp, C.c_int, vp, vp]
        L.mk_set_mode.argtypes = [vp, C.c_int]
        L.mk_set_prefill.argtypes = [vp, C.c_int]
        L.mk_debug_poison.argtypes = [vp]
        L.mk_get_state.argtypes = [vp, C.POINTER(i32), C.POINTER(i32)]
        L.mk_get_config.argtypes = [vp, C.POINTER(MkModelCfg)]
        L.mk_get_graph.argtypes = [vp, vp, C.POINTER(sz)]
        L.mk_build_graph.argtypes = [C.POINTER(MkModelCfg), C.c_int, vp, C.POINTER(sz)]
        L.mk_build_prefill_graph.argtypes = [C.POINTER(MkModelCfg), C.c_int, C.c_int, C.c_int, vp, C.POINTER(sz)]
        L.mk_reset.argtypes = [vp]
        L.mk_last_decode_ms.argtypes = [vp, C.POINTER(C.c_float)]
        L.mk_read_bandwidth.argtypes = [sz, C.c_int, C.POINTER(C.c_float)]
        L.mk_copy_bandwidth.argtypes = [sz, C.c_int, C.POINTER(C.c_float)]
        L.mk_set_trace.argtypes = [vp, C.c_int]
        L.mk_get_trace.argtypes = [vp, C.POINTER(C.c_uint64), C.POINTER(sz), C.POINTER(i32), C.POINTER(i32),
                                   C.POINTER(i32)]
        L.mk_last_error.argtypes = [vp]
        L.mk_last_error.restype = C.c_char_p
        L.mk_destroy.argtypes = [vp]
        L.mk_destroy.restype = None
        for name in EXPORTS:
            if name not in ("mk_last_error", "mk_destroy"):
                getattr(L, name).restype = C.c_int
        _lib = L
    return _lib


def _check(rc: int, ctx=None):
    if rc != MK_OK:
        msg = lib().mk_last_error(ctx)
        raise MkError(rc, msg.decode() if msg else "")


def make_cfg(shape, batch: int, max_seq: int, mode: int = MK_MODE_MEGAKERNEL, split: int = 0, n_workers: int = 0,
             watchdog_polls: int = 0, stream=None, schedule: dict | None = None,
             prefill: int = MK_PREFILL_PER_OP) -> MkModelCfg:
    """schedule: None for the frozen schedule, else a dict of SCHEDULE_FIELDS (missing ones 0)."""
    cfg = MkModelCfg(shape.n_layers, shape.hidden, shape.n_q_heads, shape.n_kv_heads, shape.head_dim, shape.ffn,
                     shape.vocab, shape.rms_eps, shape.rope_theta, int(shape.qk_norm), batch, max_seq, mode, split,
                     n_workers, watchdog_polls, stream)
    cfg.lora_rank = int(getattr(shape, "lora_rank", 0))
    cfg.prefill = int(prefill)
    if schedule is not None:
        unknown = set(schedule) - set(SCHEDULE_FIELDS)
        _need(not unknown, f"unknown schedule fields {sorted(unknown)}")
        cfg.schedule = MK_SCHEDULE_GIVEN
        for k, v in schedule.items():
            setattr(cfg, k, int(v))
    return cfg


def _current_stream_handle():
    import torch
    return C.c_void_p(torch.cuda.current_stream().cuda_stream)


# ---- the C ABI, one Python function per entry point -------------------------
def mk_create(cfg: MkModelCfg):
    h = C.c_void_p()
    _check(lib().mk_create(C.byref(cfg), C.byref(h)))
    return h


def mk_load_weights(ctx, named_tensors):
    """named_tensors: iterable of (name, bf16 torch tensor on any device)."""
    import torch
    keep, arr = [], []
    for name, t in named_tensors:
        _need(isinstance(t, torch.Tensor) and t.dtype == torch.bfloat16, f"{name} must be a bf16 torch tensor")
        t = t.contiguous()
        keep.append(t)
        arr.append(MkTensor(name.encode(), C.c_void_p(t.data_ptr()), t.numel(), int(t.is_cuda)))
    a = (MkTensor * len(arr))(*arr)
    _check(lib().mk_load_weights(ctx, a, len(arr)), ctx)


def mk_get_config(ctx) -> MkModelCfg:
    cfg = MkModelCfg()
    _check(lib().mk_get_config(ctx, C.byref(cfg)), ctx)
    return cfg


# Argument checks.  The C calls take plain pointers and trust the sizes they imply; a host tensor, a
# wrong dtype or a buffer too small for what the kernels write would make them access memory out of
# bounds.  These checks compare each buffer with the sizes the context's configuration implies.
def _need(cond: bool, msg: str):
    if not cond:
        raise MkError(MK_ERR_INVALID_ARG, msg)


def _check_device_buffer(t, dtype, numel: int, what: str):
    import torch
    _need(isinstance(t, torch.Tensor), f"{what} must be a torch tensor")
    _need(t.is_cuda, f"{what} must be on the GPU")
    _need(t.dtype == dtype, f"{what} must be {dtype}, got {t.dtype}")
    _need(t.is_contiguous(), f"{what} must be contiguous")
    _need(t.numel() >= numel, f"{what} holds {t.numel()} elements, the call writes {numel}")


def mk_prefill(ctx, prompts):
    """prompts: int [B, len] host array (B = the context's batch)."""
    p = np.ascontiguousarray(np.asarray(prompts, dtype=np.int32))
    cfg = mk_get_config(ctx)
    _need(p.ndim == 2 and p.shape[0] == cfg.batch, f"prompts must be [batch={cfg.batch}, len], got {p.shape}")
    _check(lib().mk_prefill(ctx, p.ctypes.data_as(C.POINTER(C.c_int32)), p.shape[1]), ctx)


def mk_prefill_noalloc(ctx, prompts):
    """As mk_prefill, with the prompt tokens staged in the library's static device array."""
    p = np.ascontiguousarray(np.asarray(prompts, dtype=np.int32))
    cfg = mk_get_config(ctx)
    _need(p.ndim == 2 and p.shape[0] == cfg.batch, f"prompts must be [batch={cfg.batch}, len], got {p.shape}")
    _check(lib().mk_prefill_noalloc(ctx, p.ctypes.data_as(C.POINTER(C.c_int32)), p.shape[1]), ctx)


def mk_load_kv(ctx, seq: int, k, v, pending: int):
    """k, v: bf16 torch tensors [L, n_pos, Hkv*D] on the GPU or the host."""
    import torch
    cfg = mk_get_config(ctx)
    k, v = k.contiguous(), v.contiguous()
    for t, nm in ((k, "k"), (v, "v")):
        _need(t.dtype == torch.bfloat16, f"{nm} must be bf16")
        _need(t.dim() == 3 and t.shape[0] == cfg.n_layers and t.shape[2] == cfg.n_kv_heads * cfg.head_dim,
              f"{nm} must be [n_layers={cfg.n_layers}, n_pos, {cfg.n_kv_heads * cfg.head_dim}], got {tuple(t.shape)}")
    _need(k.shape == v.shape and k.is_cuda == v.is_cuda, "k and v must have the same shape and device")
    _check(lib().mk_load_kv(ctx, seq, k.shape[1], C.c_void_p(k.data_ptr()), C.c_void_p(v.data_ptr()), int(pending),
                            int(k.is_cuda)), ctx)


def mk_decode(ctx, n_steps: int, out_tokens, out_logits=None):
    """out_tokens: int32 cuda tensor [n_steps, B]; out_logits: fp32 cuda tensor [n_steps, B, V] or None."""
    import torch
    cfg = mk_get_config(ctx)
    if n_steps > 0:
        _check_device_buffer(out_tokens, torch.int32, n_steps * cfg.batch, "out_tokens")
        if out_logits is not None:
            _check_device_buffer(out_logits, torch.float32, n_steps * cfg.batch * cfg.vocab, "out_logits")
    tp = C.c_void_p(out_tokens.data_ptr()) if out_tokens is not None else None
    _check(lib().mk_decode(ctx, n_steps, tp, C.c_void_p(out_logits.data_ptr()) if out_logits is not None else None),
           ctx)


def mk_set_mode(ctx, mode: int):
    _check(lib().mk_set_mode(ctx, mode), ctx)


def mk_debug_poison(ctx):
    _check(lib().mk_debug_poison(ctx), ctx)


def mk_set_prefill(ctx, prefill: int):
    _check(lib().mk_set_prefill(ctx, prefill), ctx)


def mk_get_state(ctx, batch: int):
    pos = C.c_int32()
    pend = (C.c_int32 * batch)()
    _check(lib().mk_get_state(ctx, C.byref(pos), pend), ctx)
    return pos.value, list(pend)


def mk_get_graph(ctx) -> bytes:
    n = C.c_size_t(0)
    _check(lib().mk_get_graph(ctx, None, C.byref(n)), ctx)
    buf = C.create_string_buffer(n.value)
    _check(lib().mk_get_graph(ctx, buf, C.byref(n)), ctx)
    return buf.raw[: n.value]


def mk_build_graph(cfg: MkModelCfg, n_workers: int) -> bytes:
    n = C.c_size_t(0)
    _check(lib().mk_build_graph(C.byref(cfg), n_workers, None, C.byref(n)))
    buf = C.create_string_buffer(n.value)
    _check(lib().mk_build_graph(C.byref(cfg), n_workers, buf, C.byref(n)))
    return buf.raw[: n.value]


def mk_build_prefill_graph(cfg: MkModelCfg, n_workers: int, chunk: int, split: int) -> bytes:
    n = C.c_size_t(0)
    _check(lib().mk_build_prefill_graph(C.byref(cfg), n_workers, chunk, split, None, C.byref(n)))
    buf = C.create_string_buffer(n.value)
    _check(lib().mk_build_prefill_graph(C.byref(cfg), n_workers, chunk, split, buf, C.byref(n)))
    return buf.raw[: n.value]


def mk_reset(ctx):
    _check(lib().mk_reset(ctx), ctx)


def mk_last_decode_ms(ctx) -> float:
    ms = C.c_float()
    _check(lib().mk_last_decode_ms(ctx, C.byref(ms)), ctx)
    return ms.value


def mk_read_bandwidth(nbytes: int, iters: int = 5) -> float:
    g = C.c_float()
    _check(lib().mk_read_bandwidth(nbytes, iters, C.byref(g)))
    return g.value


def mk_copy_bandwidth(nbytes: int, iters: int = 5) -> float:
    g = C.c_float()
    _check(lib().mk_copy_bandwidth(nbytes, iters, C.byref(g)))
    return g.value


def mk_set_trace(ctx, step: int):
    _check(lib().mk_set_trace(ctx, step), ctx)


def mk_get_trace(ctx):
    """Returns (uint64 array [n_workers, max_list, 4], clock_khz)."""
    n = C.c_size_t(0)
    nw, ml, khz = C.c_int32(), C.c_int32(), C.c_int32()
    _check(lib().mk_get_trace(ctx, None, C.byref(n), C.byref(nw), C.byref(ml), C.byref(khz)), ctx)
    out = np.zeros(n.value, dtype=np.uint64)
    _check(lib().mk_get_trace(ctx, out.ctypes.data_as(C.POINTER(C.c_uint64)), C.byref(n), None, None, None), ctx)
    return out.reshape(nw.value, ml.value, 4), khz.value


def mk_last_error(ctx=None) -> str:
    m = lib().mk_last_error(ctx)
    return m.decode() if m else ""


def mk_destroy(ctx):
    if ctx:
        lib().mk_destroy(ctx)


class Engine:
    """Owns one context: create -> load weights -> prefill/load_kv -> decode."""

    def __init__(self, shape, batch: int, max_seq: int, mode: int = MK_MODE_MEGAKERNEL, split: int = 0,
                 n_workers: int = 0, watchdog_polls: int = 0, schedule: dict | None = None,
                 prefill: int = MK_PREFILL_PER_OP):
        self.shape, self.batch, self.max_seq = shape, batch, max_seq
        self.cfg = make_cfg(shape, batch, max_seq, mode, split, n_workers, watchdog_polls, _current_stream_handle(),
                            schedule, prefill)
        self.ctx = mk_create(self.cfg)

    def load_weights(self, named_tensors):
        mk_load_weights(self.ctx, named_tensors)

    def prefill(self, prompts):
        mk_prefill(self.ctx, prompts)

    def load_kv(self, seq, k, v, pending):
        mk_load_kv(self.ctx, seq, k, v, pending)

    def decode(self, n_steps: int, want_logits: bool = True):
        import torch
        toks = torch.empty((n_steps, self.batch), dtype=torch.int32, device="cuda")
        logits = torch.empty((n_steps, self.batch, self.shape.vocab), dtype=torch.float32, device="cuda") \
            if want_logits else None
        mk_decode(self.ctx, n_steps, toks, logits)
        return toks, logits

    def set_mode(self, mode: int):
        mk_set_mode(self.ctx, mode)

    def set_prefill(self, prefill: int):
        mk_set_prefill(self.ctx, prefill)

    def state(self):
        return mk_get_state(self.ctx, self.batch)

    def graph(self) -> bytes:
        return mk_get_graph(self.ctx)

    def last_ms(self) -> float:
        return mk_last_decode_ms(self.ctx)

    def reset(self):
        mk_reset(self.ctx)

    def close(self):
        if self.ctx:
            mk_destroy(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
