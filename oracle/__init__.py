"""CPU oracle for the Echo all-reduce hot path -- TEST INFRASTRUCTURE ONLY.

Thin ctypes binding over ``echo_oracle.c`` (plain scalar C, binary32
arithmetic with no contraction, conversions written from the IEEE-754
definitions).  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package; the GPU library never does, and
this package imports nothing from it.

Pages followed (see the header of ``echo_oracle.c`` for the tags):
  * [JP-1] "Echoの仕組み①" -- all-to-all + owner high-precision sum +
    all-gather; only non-owned segments are quantized; the owner sum is
    requantized and sent to everyone; at most two quantizations per element.
  * [JP-2] "Echoの仕組み②" -- the residuals kept by the GPUs sum to the
    negated injected error; two moving averages (long and short memory) of
    it are added back into the next call's input.
  * [JP-T] "理論保証" -- with gain eta = 1 the accumulated error stays near
    2.1 q instead of N q.

``allreduce`` below strings the per-rank calls together for P simulated
ranks; it adds no arithmetic of its own.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import numpy as np

from .build import build, library_path

IN_BF16, IN_F16 = 0, 1
OUT_BF16, OUT_F32 = 0, 1
STATE_F32, STATE_BF16 = 0, 1

_LIB = None


def lib() -> ctypes.CDLL:
    global _LIB
    if _LIB is None:
        path = library_path()
        if not os.path.exists(path):
            build()
        L = ctypes.CDLL(path)
        P = ctypes.c_void_p
        i32, i64, f32 = ctypes.c_int, ctypes.c_int64, ctypes.c_float
        L.eo_f32_to_f16_array.argtypes = [P, P, i64]
        L.eo_f16_to_f32_array.argtypes = [P, P, i64]
        L.eo_f32_to_bf16_array.argtypes = [P, P, i64]
        L.eo_quantize_group.argtypes = [P, i32, i32, P, P, P, P]
        L.eo_quantize_feedback.argtypes = [i32, i32, i32, i32, f32, f32, f32, f32,
                                           i32, i32, i64, P, P, P, P, P, P]
        L.eo_owner_reduce_requant.argtypes = [i32, i32, i32, i32, i32, f32, f32, f32, f32,
                                              i32, i32, i64, P, P, P, P, P, P, P, P, P]
        L.eo_dequant_gather.argtypes = [i32, i32, i32, i32, i64, P, P, P]
        L.eo_state_reset.argtypes = [P, P, i32, i64]
        for name in ("eo_quantize_feedback", "eo_owner_reduce_requant",
                     "eo_dequant_gather", "eo_state_reset"):
            getattr(L, name).restype = ctypes.c_int
        _LIB = L
    return _LIB


@dataclass(frozen=True)
class Config:
    """Parameters of one call (the pages leave group size, decays and mix open;
    the defaults are the readings this repository uses)."""
    bits: int = 4
    group: int = 128
    eta: float = 1.0
    beta_short: float = 0.5
    beta_long: float = 0.9
    mix_long: float = 1.0 / 80.0
    in_dtype: int = IN_BF16
    out_dtype: int = OUT_BF16
    state_dtype: int = STATE_F32


def _ptr(a: np.ndarray | None) -> int | None:
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def _ptr_array(arrs):
    out = (ctypes.c_void_p * len(arrs))()
    for i, a in enumerate(arrs):
        out[i] = None if a is None else _ptr(a)
    return out


def codes_bytes(seg_len: int, bits: int) -> int:
    return seg_len * bits // 8


def segment_len(n: int, P: int, group: int) -> int:
    """Elements per segment: ceil(n/P) rounded up to whole groups; segment p is
    [p*seg_len, min((p+1)*seg_len, n)), so only the last non-empty segment can
    end in a partial group and trailing segments may be empty."""
    per = -(-n // P)
    return -(-per // group) * group


def segment_range(n: int, P: int, group: int, p: int):
    seg = segment_len(n, P, group)
    lo = min(p * seg, n)
    return lo, min(lo + seg, n) if p * seg < n else lo


def state_np_dtype(cfg: Config):
    return np.float32 if cfg.state_dtype == STATE_F32 else np.uint16


def _check(rc: int, what: str):
    if rc != 0:
        raise ValueError(f"oracle {what} rejected its arguments (code {rc})")


# ---------------------------------------------------------------- conversions
def f32_to_f16_bits(a: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.float32)
    out = np.empty(a.shape, np.uint16)
    lib().eo_f32_to_f16_array(_ptr(a), _ptr(out), a.size)
    return out


def f16_bits_to_f32(a: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.uint16)
    out = np.empty(a.shape, np.float32)
    lib().eo_f16_to_f32_array(_ptr(a), _ptr(out), a.size)
    return out


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.float32)
    out = np.empty(a.shape, np.uint16)
    lib().eo_f32_to_bf16_array(_ptr(a), _ptr(out), a.size)
    return out


# ---------------------------------------------------------------- quantizer
def quantize_group(v: np.ndarray, bits: int):
    """Q over one group -> (codes uint8[g], scale fp16 bits, zero fp16 bits, deq f32[g])."""
    v = np.ascontiguousarray(v, dtype=np.float32)
    g = v.size
    q = np.zeros(g, np.uint8)
    deq = np.zeros(g, np.float32)
    sb = np.zeros(1, np.uint16)
    zb = np.zeros(1, np.uint16)
    lib().eo_quantize_group(_ptr(v), g, bits, _ptr(q), _ptr(sb), _ptr(zb), _ptr(deq))
    return q, int(sb[0]), int(zb[0]), deq


# ---------------------------------------------------------------- the four calls
def state_reset(S: np.ndarray, L: np.ndarray, cfg: Config = Config(), n: int | None = None):
    """Empty both memories of the first n elements (default: all of S and L);
    S and L hold float32 (fp32 state) or uint16 bfloat16 bits (bf16 state)."""
    n = S.size if n is None else n
    assert S.dtype == state_np_dtype(cfg) and L.dtype == S.dtype
    assert 0 <= n <= min(S.size, L.size)
    _check(lib().eo_state_reset(_ptr(S), _ptr(L), cfg.state_dtype, n), "state_reset")


def quantize_feedback(cfg: Config, P: int, rank: int, x: np.ndarray, S: np.ndarray,
                      L: np.ndarray, codes, params, qpass: np.ndarray | None = None):
    """Entry pass of `rank`: fills codes[p], params[p] for p != rank; updates S, L."""
    n = x.size
    rc = lib().eo_quantize_feedback(cfg.bits, cfg.group, cfg.in_dtype, cfg.state_dtype,
                                    cfg.eta, cfg.beta_short, cfg.beta_long, cfg.mix_long,
                                    P, rank, n, _ptr(x), _ptr(S), _ptr(L),
                                    _ptr_array(codes), _ptr_array(params), _ptr(qpass))
    _check(rc, "quantize_feedback")


def owner_reduce_requant(cfg: Config, P: int, rank: int, x: np.ndarray, S: np.ndarray,
                         L: np.ndarray, in_codes, in_params, out_codes: np.ndarray,
                         out_params: np.ndarray, qpass: np.ndarray | None = None,
                         acc: np.ndarray | None = None):
    """Owner pass of `rank` over its segment: fills out_codes/out_params; updates S, L.
    acc (optional, float32, one per element of the segment) receives the fp32
    sum before requantization."""
    n = x.size
    if acc is not None:
        assert acc.dtype == np.float32 and acc.size >= segment_len(n, P, cfg.group)
    rc = lib().eo_owner_reduce_requant(cfg.bits, cfg.group, cfg.in_dtype, cfg.state_dtype,
                                       cfg.out_dtype, cfg.eta, cfg.beta_short,
                                       cfg.beta_long, cfg.mix_long, P, rank, n,
                                       _ptr(x), _ptr(S), _ptr(L), _ptr_array(in_codes),
                                       _ptr_array(in_params), _ptr(out_codes),
                                       _ptr(out_params), _ptr(qpass), _ptr(acc))
    _check(rc, "owner_reduce_requant")


def dequant_gather(cfg: Config, P: int, n: int, codes, params) -> np.ndarray:
    out = np.empty(n, np.uint16 if cfg.out_dtype == OUT_BF16 else np.float32)
    rc = lib().eo_dequant_gather(cfg.bits, cfg.group, cfg.out_dtype, P, n,
                                 _ptr_array(codes), _ptr_array(params), _ptr(out))
    _check(rc, "dequant_gather")
    return out


# ---------------------------------------------------------------- P simulated ranks
def new_payload(cfg: Config, seg_len: int):
    """Payload buffers for a segment of seg_len elements (whole groups)."""
    return (np.zeros(codes_bytes(seg_len, cfg.bits), np.uint8),
            np.zeros(-(-seg_len // cfg.group), np.uint32))


def allreduce(cfg: Config, xs, Ss, Ls, qpass=None):
    """One Echo all-reduce over P simulated ranks.

    xs[p]: uint16[n] input bits of rank p; Ss[p], Ls[p]: its error state
    (updated in place).  Returns (out, sent, owned): `out` is the gathered
    output (identical on every rank), sent[p][o] the payload rank p sent to
    owner o (None for o == p), owned[o] the requantized payload of owner o.
    qpass (optional): list of P uint32[n] counters, one per contributing
    rank, counting quantizer passes of that rank's contribution per element.
    """
    P = len(xs)
    n = xs[0].size
    seg = segment_len(n, P, cfg.group)
    sent = [[None if o == p else new_payload(cfg, seg) for o in range(P)] for p in range(P)]
    k1_counts = [np.zeros(n, np.uint32) for _ in range(P)] if qpass is not None else None
    for p in range(P):
        quantize_feedback(cfg, P, p, xs[p], Ss[p], Ls[p],
                          [None if o == p else sent[p][o][0] for o in range(P)],
                          [None if o == p else sent[p][o][1] for o in range(P)],
                          None if k1_counts is None else k1_counts[p])
    owned = [new_payload(cfg, seg) for _ in range(P)]
    k2_counts = [np.zeros(n, np.uint32) for _ in range(P)] if qpass is not None else None
    for o in range(P):
        in_codes = [None if p == o else sent[p][o][0] for p in range(P)]
        in_params = [None if p == o else sent[p][o][1] for p in range(P)]
        owner_reduce_requant(cfg, P, o, xs[o], Ss[o], Ls[o], in_codes,
                             in_params, owned[o][0], owned[o][1],
                             None if k2_counts is None else k2_counts[o])
    out = dequant_gather(cfg, P, n, [c for c, _ in owned], [q for _, q in owned])
    if qpass is not None:
        # the owner's requantization acts on the sum, hence on every rank's
        # contribution to the elements of its segment
        k2_all = np.zeros(n, np.uint32)
        for o in range(P):
            lo, hi = segment_range(n, P, cfg.group, o)
            k2_all[lo:hi] = k2_counts[o][lo:hi]
        for p in range(P):
            qpass[p][:] = k1_counts[p] + k2_all
    return out, sent, owned
