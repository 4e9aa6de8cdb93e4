"""ctypes binding of libecho_amd.so (include/echo.h), same names as the C ABI.

Argument marshalling only: torch tensors are passed as device pointers and
host descriptor arrays are built for the payload tables.  Every step of the
all-reduce share runs in the library's kernels; there is no fallback: if the
library is not built, loading it raises.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

from .build import library_path

# constants of include/echo.h
ECHO_OK, ECHO_ERR_ARG, ECHO_ERR_SHAPE, ECHO_ERR_ALIGN, ECHO_ERR_HIP = 0, -1, -2, -3, -4
ECHO_IN_BF16, ECHO_IN_F16 = 0, 1
ECHO_OUT_BF16, ECHO_OUT_F32 = 0, 1
ECHO_STATE_F32, ECHO_STATE_BF16 = 0, 1
ECHO_MAX_RANKS = 16
ECHO_GROUP = 128

EXPORTED = ("echo_state_reset", "echo_quantize_feedback", "echo_owner_reduce_requant",
            "echo_dequant_gather", "echo_segment_len", "echo_codes_bytes", "echo_params_bytes",
            "echo_state_bytes", "echo_error_string")


class echo_config(ctypes.Structure):
    _fields_ = [("bits", ctypes.c_int32), ("group", ctypes.c_int32),
                ("in_dtype", ctypes.c_int32), ("out_dtype", ctypes.c_int32),
                ("state_dtype", ctypes.c_int32), ("eta", ctypes.c_float),
                ("beta_short", ctypes.c_float), ("beta_long", ctypes.c_float),
                ("mix_long", ctypes.c_float)]


class echo_seg(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("params", ctypes.c_void_p)]


class EchoError(RuntimeError):
    def __init__(self, code: int, where: str):
        super().__init__(f"{where}: {error_string(code)} (code {code})")
        self.code = code


_LIB = None


def load_library() -> ctypes.CDLL:
    global _LIB
    if _LIB is None:
        path = library_path()
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: build the HIP library first "
                               "(python -c 'import __graft_entry__ as g; g.build()')")
        L = ctypes.CDLL(path)
        vp, i32, i64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
        cfgp, segp = ctypes.POINTER(echo_config), ctypes.POINTER(echo_seg)
        L.echo_state_reset.argtypes = [cfgp, vp, i64, vp]
        L.echo_quantize_feedback.argtypes = [cfgp, i32, i32, i64, vp, vp, segp, vp]
        L.echo_owner_reduce_requant.argtypes = [cfgp, i32, i32, i64, vp, vp, segp, segp, vp]
        L.echo_dequant_gather.argtypes = [cfgp, i32, i64, segp, vp, vp]
        L.echo_codes_bytes.argtypes = [i64, i32]
        L.echo_params_bytes.argtypes = [i64, i32]
        L.echo_state_bytes.argtypes = [i64, i32]
        L.echo_segment_len.argtypes = [i64, i32, i32]
        L.echo_segment_len.restype = ctypes.c_int64
        L.echo_codes_bytes.restype = ctypes.c_size_t
        L.echo_params_bytes.restype = ctypes.c_size_t
        L.echo_state_bytes.restype = ctypes.c_size_t
        L.echo_error_string.argtypes = [i32]
        L.echo_error_string.restype = ctypes.c_char_p
        for name in ("echo_state_reset", "echo_quantize_feedback",
                     "echo_owner_reduce_requant", "echo_dequant_gather"):
            getattr(L, name).restype = ctypes.c_int
        _LIB = L
    return _LIB


def error_string(code: int) -> str:
    return load_library().echo_error_string(code).decode()


def make_config(bits=4, group=ECHO_GROUP, eta=1.0, beta_short=0.5, beta_long=0.9,
                mix_long=1.0 / 80.0, in_dtype=ECHO_IN_BF16, out_dtype=ECHO_OUT_BF16,
                state_dtype=ECHO_STATE_F32) -> echo_config:
    return echo_config(bits, group, in_dtype, out_dtype, state_dtype, eta, beta_short,
                       beta_long, mix_long)


@dataclass
class Payload:
    """One segment's payload: codes (uint8) and params (int32 words, scale | zero << 16)."""
    codes: torch.Tensor
    params: torch.Tensor

    def seg(self) -> echo_seg:
        return echo_seg(_ptr(self.codes), _ptr(self.params))


def echo_codes_bytes(seg_len: int, bits: int) -> int:
    return load_library().echo_codes_bytes(seg_len, bits)


def echo_params_bytes(seg_len: int, group: int = ECHO_GROUP) -> int:
    return load_library().echo_params_bytes(seg_len, group)


def echo_segment_len(n: int, P: int, group: int = ECHO_GROUP) -> int:
    return load_library().echo_segment_len(n, P, group)


def echo_state_bytes(n: int, state_dtype: int) -> int:
    return load_library().echo_state_bytes(n, state_dtype)


def alloc_payload(seg_len: int, bits: int, device, fill: int | None = None,
                  group: int = ECHO_GROUP) -> Payload:
    """Payload buffers for seg_len elements; `fill` sets every byte (sentinels)."""
    cb, pb = echo_codes_bytes(seg_len, bits), echo_params_bytes(seg_len, group)
    if cb == 0 or pb == 0:
        raise ValueError(f"no payload layout for {seg_len} elements at {bits} bits")
    if fill is None:
        return Payload(torch.empty(cb, dtype=torch.uint8, device=device),
                       torch.empty(pb // 4, dtype=torch.int32, device=device))
    return Payload(torch.full((cb,), fill, dtype=torch.uint8, device=device),
                   torch.full((pb,), fill, dtype=torch.uint8, device=device).view(torch.int32))


def _ptr(t: torch.Tensor | None) -> int | None:
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("echo buffers must be contiguous")
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream


def _seg_table(P: int, payloads) -> ctypes.Array:
    tab = (echo_seg * P)()
    for p, pay in enumerate(payloads):
        if pay is not None:
            tab[p] = pay.seg()
    return tab


def _check(rc: int, where: str):
    if rc != ECHO_OK:
        raise EchoError(rc, where)


def echo_state_reset(cfg: echo_config, state: torch.Tensor, n: int, stream=None):
    """state: 2n elements (S_j, L_j pairs) of the config's state type."""
    _check(load_library().echo_state_reset(ctypes.byref(cfg), _ptr(state), n, _stream(stream)),
           "echo_state_reset")


def echo_quantize_feedback(cfg: echo_config, P: int, rank: int, n: int, x: torch.Tensor,
                           state: torch.Tensor, out, stream=None):
    """out: list of P Payloads (entry `rank` may be None)."""
    _check(load_library().echo_quantize_feedback(ctypes.byref(cfg), P, rank, n, _ptr(x),
                                                 _ptr(state), _seg_table(P, out), _stream(stream)),
           "echo_quantize_feedback")


def echo_owner_reduce_requant(cfg: echo_config, P: int, rank: int, n: int, x: torch.Tensor,
                              state: torch.Tensor, inp, out: Payload, stream=None):
    """inp: list of P Payloads received for segment `rank` (entry `rank` may be None)."""
    out_seg = out.seg()
    _check(load_library().echo_owner_reduce_requant(ctypes.byref(cfg), P, rank, n, _ptr(x),
                                                    _ptr(state), _seg_table(P, inp),
                                                    ctypes.byref(out_seg), _stream(stream)),
           "echo_owner_reduce_requant")


def echo_dequant_gather(cfg: echo_config, P: int, n: int, inp, out: torch.Tensor, stream=None):
    """inp: list of the P owners' requantized Payloads, in segment order."""
    _check(load_library().echo_dequant_gather(ctypes.byref(cfg), P, n, _seg_table(P, inp),
                                              _ptr(out), _stream(stream)),
           "echo_dequant_gather")


class Prepared:
    """One entry-point call with every argument marshalled once (config,
    payload tables, pointers and stream): calling it makes only the foreign
    call.  For callers that repeat the same call on the same buffers, where
    marshalling would cost more host time than a small message's kernels.
    It holds references to every tensor it was given, so they stay allocated
    while it exists; it always launches on the stream it was prepared with."""

    def __init__(self, fn, args, keep, where: str):
        self._fn = fn
        self._args = args
        self._keep = keep          # the ctypes objects the byref arguments point at
        self._where = where

    def __call__(self):
        rc = self._fn(*self._args)
        if rc != ECHO_OK:
            raise EchoError(rc, self._where)


def prepare_quantize_feedback(cfg: echo_config, P: int, rank: int, n: int, x: torch.Tensor,
                              state: torch.Tensor, out, stream=None) -> Prepared:
    L = load_library()
    c = echo_config(*(getattr(cfg, f) for f, _ in echo_config._fields_))
    return Prepared(L.echo_quantize_feedback,
                    (ctypes.byref(c), P, rank, n, _ptr(x), _ptr(state), _seg_table(P, out),
                     _stream(stream)), (c, x, state, list(out)), "echo_quantize_feedback")


def prepare_owner_reduce_requant(cfg: echo_config, P: int, rank: int, n: int, x: torch.Tensor,
                                 state: torch.Tensor, inp, out: Payload, stream=None) -> Prepared:
    L = load_library()
    c = echo_config(*(getattr(cfg, f) for f, _ in echo_config._fields_))
    out_seg = out.seg()
    return Prepared(L.echo_owner_reduce_requant,
                    (ctypes.byref(c), P, rank, n, _ptr(x), _ptr(state), _seg_table(P, inp),
                     ctypes.byref(out_seg), _stream(stream)), (c, out_seg, x, state, list(inp), out),
                    "echo_owner_reduce_requant")


def prepare_dequant_gather(cfg: echo_config, P: int, n: int, inp, out: torch.Tensor,
                           stream=None) -> Prepared:
    L = load_library()
    c = echo_config(*(getattr(cfg, f) for f, _ in echo_config._fields_))
    return Prepared(L.echo_dequant_gather,
                    (ctypes.byref(c), P, n, _seg_table(P, inp), _ptr(out), _stream(stream)),
                    (c, list(inp), out), "echo_dequant_gather")
