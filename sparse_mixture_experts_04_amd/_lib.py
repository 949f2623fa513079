"""ctypes binding of libmoe.so (the C ABI declared in include/moe.h).

Argument marshalling only: every step of the layer runs in the library's HIP
kernels.  Tensors are passed as raw device pointers; the stream is torch's
current HIP stream unless one is given.  There is no fallback: if libmoe.so is
missing or cannot be loaded, importing this module raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch  # loads torch's HIP runtime first, so libmoe binds to that same copy

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe.so")

MOE_OK = 0
MOE_ERR_INVALID_ARG = 1
MOE_ERR_UNSUPPORTED = 2
MOE_ERR_WORKSPACE_TOO_SMALL = 3
MOE_ERR_HIP = 4

MOE_F32 = 0
MOE_BF16 = 1

MOE_OP_DISPATCH = 0
MOE_OP_EXPERT_FFN = 1
MOE_OP_FORWARD = 2
MOE_OP_ROUTE = 3
MOE_OP_ROUTE_STATS = 4
MOE_OP_DISPATCH_REROUTE = 5
MOE_OP_FORWARD_REROUTE = 6

NOALLOC_MAX_WORKSPACE_BYTES = 64 << 20  # MOE_NOALLOC_MAX_WORKSPACE_BYTES of include/moe.h

# Every symbol include/moe.h declares.
EXPORTED = ("moe_status_string", "moe_version", "moe_workspace_size", "moe_capacity_from_factor", "moe_route",
            "moe_route_stats", "moe_dispatch",
            "moe_expert_up", "moe_expert_up_gather", "moe_expert_up_gather_supported", "moe_expert_down",
            "moe_expert_ffn", "moe_combine", "moe_forward", "moe_route_ranked", "moe_dispatch_reroute",
            "moe_forward_reroute", "moe_forward_noalloc")


class MoeConfig(ctypes.Structure):
    _fields_ = [("num_tokens", ctypes.c_int32), ("hidden_size", ctypes.c_int32),
                ("intermediate_size", ctypes.c_int32), ("num_experts", ctypes.c_int32),
                ("num_experts_per_tok", ctypes.c_int32), ("expert_capacity", ctypes.c_int32),
                ("dtype", ctypes.c_int32)]

    def __repr__(self):
        return ("MoeConfig(T=%d, d=%d, F=%d, E=%d, k=%d, C=%d, dtype=%s)" %
                (self.num_tokens, self.hidden_size, self.intermediate_size, self.num_experts,
                 self.num_experts_per_tok, self.expert_capacity, "bf16" if self.dtype == MOE_BF16 else "f32"))


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn}: {status_string(status)}")


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python sparse_mixture_experts_04_amd/build.py`")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    CFG = ctypes.POINTER(MoeConfig)
    sig = {
        "moe_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        "moe_version": (ctypes.c_char_p, []),
        "moe_workspace_size": (ctypes.c_int, [CFG, ctypes.c_int32, ctypes.POINTER(ctypes.c_size_t)]),
        "moe_capacity_from_factor": (ctypes.c_int, [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                                    ctypes.c_double, ctypes.POINTER(ctypes.c_int32)]),
        "moe_route": (ctypes.c_int, [CFG, P, P, P, P, P, P, ctypes.c_size_t, P]),
        "moe_route_stats": (ctypes.c_int, [CFG, P, P, P, ctypes.c_float, P, P, P, P, P, P, ctypes.c_size_t, P]),
        "moe_dispatch": (ctypes.c_int, [CFG, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]),
        "moe_expert_up": (ctypes.c_int, [CFG, P, P, P, P, P]),
        "moe_expert_up_gather": (ctypes.c_int, [CFG, P, P, P, P, P, P]),
        "moe_expert_up_gather_supported": (ctypes.c_int, [CFG, ctypes.POINTER(ctypes.c_int32)]),
        "moe_expert_down": (ctypes.c_int, [CFG, P, P, P, P, P]),
        "moe_expert_ffn": (ctypes.c_int, [CFG, P, P, P, P, P, P, ctypes.c_size_t, P]),
        "moe_combine": (ctypes.c_int, [CFG, P, P, P, P, P]),
        "moe_forward": (ctypes.c_int, [CFG, P, P, P, P, P, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]),
        "moe_route_ranked": (ctypes.c_int, [CFG, P, P, P, P, P, P, P, ctypes.c_size_t, P]),
        "moe_dispatch_reroute": (ctypes.c_int, [CFG, P, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]),
        "moe_forward_reroute": (ctypes.c_int, [CFG, P, P, P, P, P, P, P, P, P, P, P, P, P, P, ctypes.c_size_t,
                                               P]),
        "moe_forward_noalloc": (ctypes.c_int, [CFG, P, P, P, P, P, P, P, P, P, P, P, P, P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    hip_copies = set()
    try:
        with open("/proc/self/maps") as f:
            for line in f:
                if "libamdhip64" in line:
                    hip_copies.add(line.split()[-1])
    except OSError:
        pass
    if len(hip_copies) > 1:
        raise ImportError(f"two HIP runtimes are loaded ({sorted(hip_copies)}); libmoe must share torch's")
    return lib


LIB = _load()


def status_string(status: int) -> str:
    return LIB.moe_status_string(int(status)).decode()


def version() -> str:
    return LIB.moe_version().decode()


def _check(fn: str, status: int) -> None:
    if status != MOE_OK:
        raise MoeError(fn, status)


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _layer_dtype(cfg) -> torch.dtype:
    return torch.bfloat16 if cfg.dtype == MOE_BF16 else torch.float32


def _arg(fn: str, name: str, t, dtype, numel: int) -> None:
    """Check one buffer before its pointer goes to the library, which
    cannot see sizes: a tensor must live on the GPU, be contiguous, have the
    element type moe.h documents and hold at least the elements it
    documents.  None (checked by the library) and raw integer pointers (the
    caller's responsibility) pass unchanged, as does any buffer of a call
    that reads or writes nothing (numel 0)."""
    if t is None or isinstance(t, int) or numel <= 0:
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{fn}: {name} must be a torch.Tensor, an int pointer or None, not {type(t).__name__}")
    if t.device.type != "cuda":
        raise ValueError(f"{fn}: {name} must be a GPU tensor, got device {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{fn}: {name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{fn}: {name} must have dtype {dtype}, got {t.dtype}")
    if t.numel() < numel:
        raise ValueError(f"{fn}: {name} holds {t.numel()} elements, needs {numel}")


def _dims(cfg):
    T, k = max(cfg.num_tokens, 0), cfg.num_experts_per_tok
    return T, cfg.hidden_size, cfg.intermediate_size, cfg.num_experts, k, T * k


def _stream(stream) -> Optional[int]:
    if stream is None:
        try:
            return torch.cuda.current_stream().cuda_stream
        except (RuntimeError, AssertionError):  # no GPU: only argument checks can run
            return 0
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _route_args(fn, cfg, X, Wg, gate_bias, topk_ids, topk_w):
    T, d, F, E, k, Tk = _dims(cfg)
    dt = _layer_dtype(cfg)
    for name, t, ty, n in (("X", X, dt, T * d), ("Wg", Wg, dt, d * E * (T > 0)),
                           ("gate_bias", gate_bias, torch.float32, E * (T > 0)),
                           ("topk_ids", topk_ids, torch.int32, Tk), ("topk_w", topk_w, torch.float32, Tk)):
        _arg(fn, name, t, ty, n)


def _dispatch_args(fn, cfg, topk_ids, X, expert_counts, expert_offsets, perm, inv_perm, Xp):
    T, d, F, E, k, Tk = _dims(cfg)
    dt = _layer_dtype(cfg)
    for name, t, ty, n in (("topk_ids", topk_ids, torch.int32, Tk), ("X", X, dt, T * d),
                           ("expert_counts", expert_counts, torch.int32, E),
                           ("expert_offsets", expert_offsets, torch.int32, E + 1),
                           ("perm", perm, torch.int32, Tk), ("inv_perm", inv_perm, torch.int32, Tk),
                           ("Xp", Xp, dt, Tk * d)):
        _arg(fn, name, t, ty, n)


def _forward_args(fn, cfg, X, Wg, gate_bias, W1, W2, out, topk_ids, topk_w, expert_counts, expert_offsets, perm,
                  inv_perm):
    T, d, F, E, k, Tk = _dims(cfg)
    dt = _layer_dtype(cfg)
    _route_args(fn, cfg, X, Wg, gate_bias, topk_ids, topk_w)
    _dispatch_args(fn, cfg, topk_ids, X, expert_counts, expert_offsets, perm, inv_perm, None)
    for name, t, ty, n in (("W1", W1, dt, E * F * d * (T > 0)), ("W2", W2, dt, E * d * F * (T > 0)),
                           ("out", out, dt, T * d)):
        _arg(fn, name, t, ty, n)


def config(T: int, d: int, F: int, E: int, k: int, capacity: int = -1, dtype: str = "bf16") -> MoeConfig:
    """The layer's shape: num_tokens, hidden, intermediate, num_experts,
    num_experts_per_tok, expert_capacity (< 0: dropless), dtype ("bf16"|"f32")."""
    return MoeConfig(int(T), int(d), int(F), int(E), int(k), int(capacity),
                     MOE_BF16 if dtype == "bf16" else MOE_F32)


def moe_workspace_size(cfg: MoeConfig, op: int) -> int:
    n = ctypes.c_size_t(0)
    _check("moe_workspace_size", LIB.moe_workspace_size(ctypes.byref(cfg), int(op), ctypes.byref(n)))
    return n.value


def moe_capacity_from_factor(batch: int, seq_len: int, E: int, k: int, factor: float = 2.0) -> int:
    c = ctypes.c_int32(0)
    _check("moe_capacity_from_factor",
           LIB.moe_capacity_from_factor(int(batch), int(seq_len), int(E), int(k), float(factor), ctypes.byref(c)))
    return c.value


def moe_route(cfg, X, Wg, gate_bias, topk_ids, topk_w, ws=None, ws_bytes=None, stream=None) -> None:
    _route_args("moe_route", cfg, X, Wg, gate_bias, topk_ids, topk_w)
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size() if ws is not None else 0
    _check("moe_route", LIB.moe_route(ctypes.byref(cfg), _ptr(X), _ptr(Wg), _ptr(gate_bias), _ptr(topk_ids),
                                      _ptr(topk_w), _ptr(ws), int(ws_bytes), _stream(stream)))


def moe_route_stats(cfg, X, Wg, gate_bias, temperature, topk_ids, topk_w, prob_mean, sel_freq, aux, ws=None,
                    ws_bytes=None, stream=None) -> None:
    _route_args("moe_route_stats", cfg, X, Wg, gate_bias, topk_ids, topk_w)
    E = cfg.num_experts if cfg.num_tokens > 0 else 0
    for name, t, n in (("prob_mean", prob_mean, E), ("sel_freq", sel_freq, E), ("aux", aux, 1 if E else 0)):
        _arg("moe_route_stats", name, t, torch.float32, n)
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size() if ws is not None else 0
    _check("moe_route_stats", LIB.moe_route_stats(ctypes.byref(cfg), _ptr(X), _ptr(Wg), _ptr(gate_bias),
                                                  float(temperature), _ptr(topk_ids), _ptr(topk_w), _ptr(prob_mean),
                                                  _ptr(sel_freq), _ptr(aux), _ptr(ws), int(ws_bytes),
                                                  _stream(stream)))


def moe_dispatch(cfg, topk_ids, X, expert_counts, expert_offsets, perm, inv_perm, Xp, ws, ws_bytes=None,
                 stream=None) -> None:
    _dispatch_args("moe_dispatch", cfg, topk_ids, X, expert_counts, expert_offsets, perm, inv_perm, Xp)
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size() if ws is not None else 0
    _check("moe_dispatch", LIB.moe_dispatch(ctypes.byref(cfg), _ptr(topk_ids), _ptr(X), _ptr(expert_counts),
                                            _ptr(expert_offsets), _ptr(perm), _ptr(inv_perm), _ptr(Xp), _ptr(ws),
                                            int(ws_bytes), _stream(stream)))


def moe_expert_up(cfg, Xp, expert_offsets, W1, H, stream=None) -> None:
    T, d, F, E, k, Tk = _dims(cfg)
    dt = _layer_dtype(cfg)
    for name, t, ty, n in (("Xp", Xp, dt, Tk * d), ("expert_offsets", expert_offsets, torch.int32, (E + 1) * (T > 0)),
                           ("W1", W1, dt, E * F * d * (T > 0)), ("H", H, dt, Tk * F)):
        _arg("moe_expert_up", name, t, ty, n)
    _check("moe_expert_up", LIB.moe_expert_up(ctypes.byref(cfg), _ptr(Xp), _ptr(expert_offsets), _ptr(W1), _ptr(H),
                                              _stream(stream)))


def moe_expert_up_gather(cfg, X, perm, expert_offsets, W1, H, stream=None) -> None:
    T, d, F, E, k, Tk = _dims(cfg)
    dt = _layer_dtype(cfg)
    for name, t, ty, n in (("X", X, dt, T * d), ("perm", perm, torch.int32, Tk),
                           ("expert_offsets", expert_offsets, torch.int32, (E + 1) * (T > 0)),
                           ("W1", W1, dt, E * F * d * (T > 0)), ("H", H, dt, Tk * F)):
        _arg("moe_expert_up_gather", name, t, ty, n)
    _check("moe_expert_up_gather", LIB.moe_expert_up_gather(ctypes.byref(cfg), _ptr(X), _ptr(perm),
                                                            _ptr(expert_offsets), _ptr(W1), _ptr(H),
                                                            _stream(stream)))


def moe_expert_up_gather_supported(cfg) -> bool:
    v = ctypes.c_int32(0)
    _check("moe_expert_up_gather_supported", LIB.moe_expert_up_gather_supported(ctypes.byref(cfg), ctypes.byref(v)))
    return bool(v.value)


def moe_expert_down(cfg, H, expert_offsets, W2, Yp, stream=None) -> None:
    T, d, F, E, k, Tk = _dims(cfg)
    dt = _layer_dtype(cfg)
    for name, t, ty, n in (("H", H, dt, Tk * F), ("expert_offsets", expert_offsets, torch.int32, (E + 1) * (T > 0)),
                           ("W2", W2, dt, E * d * F * (T > 0)), ("Yp", Yp, dt, Tk * d)):
        _arg("moe_expert_down", name, t, ty, n)
    _check("moe_expert_down", LIB.moe_expert_down(ctypes.byref(cfg), _ptr(H), _ptr(expert_offsets), _ptr(W2),
                                                  _ptr(Yp), _stream(stream)))


def moe_expert_ffn(cfg, Xp, expert_offsets, W1, W2, Yp, ws, ws_bytes=None, stream=None) -> None:
    T, d, F, E, k, Tk = _dims(cfg)
    dt = _layer_dtype(cfg)
    for name, t, ty, n in (("Xp", Xp, dt, Tk * d), ("expert_offsets", expert_offsets, torch.int32, (E + 1) * (T > 0)),
                           ("W1", W1, dt, E * F * d * (T > 0)), ("W2", W2, dt, E * d * F * (T > 0)),
                           ("Yp", Yp, dt, Tk * d)):
        _arg("moe_expert_ffn", name, t, ty, n)
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size() if ws is not None else 0
    _check("moe_expert_ffn", LIB.moe_expert_ffn(ctypes.byref(cfg), _ptr(Xp), _ptr(expert_offsets), _ptr(W1),
                                                _ptr(W2), _ptr(Yp), _ptr(ws), int(ws_bytes), _stream(stream)))


def moe_combine(cfg, Yp, inv_perm, topk_w, out, stream=None) -> None:
    T, d, F, E, k, Tk = _dims(cfg)
    dt = _layer_dtype(cfg)
    for name, t, ty, n in (("Yp", Yp, dt, Tk * d), ("inv_perm", inv_perm, torch.int32, Tk),
                           ("topk_w", topk_w, torch.float32, Tk), ("out", out, dt, T * d)):
        _arg("moe_combine", name, t, ty, n)
    _check("moe_combine", LIB.moe_combine(ctypes.byref(cfg), _ptr(Yp), _ptr(inv_perm), _ptr(topk_w), _ptr(out),
                                          _stream(stream)))


def moe_forward(cfg, X, Wg, gate_bias, W1, W2, out, topk_ids, topk_w, expert_counts, expert_offsets, perm,
                inv_perm, ws, ws_bytes=None, stream=None) -> None:
    _forward_args("moe_forward", cfg, X, Wg, gate_bias, W1, W2, out, topk_ids, topk_w, expert_counts,
                  expert_offsets, perm, inv_perm)
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size() if ws is not None else 0
    _check("moe_forward", LIB.moe_forward(ctypes.byref(cfg), _ptr(X), _ptr(Wg), _ptr(gate_bias), _ptr(W1), _ptr(W2),
                                          _ptr(out), _ptr(topk_ids), _ptr(topk_w), _ptr(expert_counts),
                                          _ptr(expert_offsets), _ptr(perm), _ptr(inv_perm), _ptr(ws), int(ws_bytes),
                                          _stream(stream)))


def moe_route_ranked(cfg, X, Wg, gate_bias, topk_ids, topk_w, expert_order, ws=None, ws_bytes=None,
                     stream=None) -> None:
    _route_args("moe_route_ranked", cfg, X, Wg, gate_bias, topk_ids, topk_w)
    _arg("moe_route_ranked", "expert_order", expert_order, torch.uint8, max(cfg.num_tokens, 0) * cfg.num_experts)
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size() if ws is not None else 0
    _check("moe_route_ranked", LIB.moe_route_ranked(ctypes.byref(cfg), _ptr(X), _ptr(Wg), _ptr(gate_bias),
                                                    _ptr(topk_ids), _ptr(topk_w), _ptr(expert_order), _ptr(ws),
                                                    int(ws_bytes), _stream(stream)))


def moe_dispatch_reroute(cfg, topk_ids, expert_order, X, expert_counts, expert_offsets, perm, inv_perm, Xp, ws,
                         ws_bytes=None, stream=None) -> None:
    _dispatch_args("moe_dispatch_reroute", cfg, topk_ids, X, expert_counts, expert_offsets, perm, inv_perm, Xp)
    _arg("moe_dispatch_reroute", "expert_order", expert_order, torch.uint8, max(cfg.num_tokens, 0) * cfg.num_experts)
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size() if ws is not None else 0
    _check("moe_dispatch_reroute", LIB.moe_dispatch_reroute(ctypes.byref(cfg), _ptr(topk_ids), _ptr(expert_order),
                                                            _ptr(X), _ptr(expert_counts), _ptr(expert_offsets),
                                                            _ptr(perm), _ptr(inv_perm), _ptr(Xp), _ptr(ws),
                                                            int(ws_bytes), _stream(stream)))


def moe_forward_reroute(cfg, X, Wg, gate_bias, W1, W2, out, topk_ids, topk_w, expert_order, expert_counts,
                        expert_offsets, perm, inv_perm, ws, ws_bytes=None, stream=None) -> None:
    _forward_args("moe_forward_reroute", cfg, X, Wg, gate_bias, W1, W2, out, topk_ids, topk_w, expert_counts,
                  expert_offsets, perm, inv_perm)
    _arg("moe_forward_reroute", "expert_order", expert_order, torch.uint8, max(cfg.num_tokens, 0) * cfg.num_experts)
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size() if ws is not None else 0
    _check("moe_forward_reroute", LIB.moe_forward_reroute(ctypes.byref(cfg), _ptr(X), _ptr(Wg), _ptr(gate_bias),
                                                          _ptr(W1), _ptr(W2), _ptr(out), _ptr(topk_ids),
                                                          _ptr(topk_w), _ptr(expert_order), _ptr(expert_counts),
                                                          _ptr(expert_offsets), _ptr(perm), _ptr(inv_perm), _ptr(ws),
                                                          int(ws_bytes), _stream(stream)))


def moe_forward_noalloc(cfg, X, Wg, gate_bias, W1, W2, out, topk_ids, topk_w, expert_counts, expert_offsets, perm,
                        inv_perm, stream=None) -> None:
    """moe_forward with the library's own per-GPU workspace array (no workspace argument)."""
    _forward_args("moe_forward_noalloc", cfg, X, Wg, gate_bias, W1, W2, out, topk_ids, topk_w, expert_counts,
                  expert_offsets, perm, inv_perm)
    _check("moe_forward_noalloc", LIB.moe_forward_noalloc(ctypes.byref(cfg), _ptr(X), _ptr(Wg), _ptr(gate_bias),
                                                          _ptr(W1), _ptr(W2), _ptr(out), _ptr(topk_ids),
                                                          _ptr(topk_w), _ptr(expert_counts), _ptr(expert_offsets),
                                                          _ptr(perm), _ptr(inv_perm), _stream(stream)))
