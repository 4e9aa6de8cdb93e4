"""Helpers shared by the GPU parity tests: config translation between the GPU
binding and the oracle, host copies, sampled mini-messages and comparisons.
No arithmetic of the method lives here."""
from __future__ import annotations

import numpy as np
import torch

import oracle as O
from error_compensated_bit_amd import binding as B

G = 128


def oracle_config(cfg: B.echo_config) -> O.Config:
    return O.Config(bits=cfg.bits, group=cfg.group, eta=cfg.eta, beta_short=cfg.beta_short,
                    beta_long=cfg.beta_long, mix_long=cfg.mix_long, in_dtype=cfg.in_dtype,
                    out_dtype=cfg.out_dtype, state_dtype=cfg.state_dtype)


def host(t: torch.Tensor) -> np.ndarray:
    """Host copy; 16-bit float tensors come back as their uint16 bits."""
    t = t.detach().contiguous()
    if t.dtype in (torch.bfloat16, torch.float16):
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    if t.dtype == torch.int32:
        return t.cpu().numpy().view(np.uint32)
    return t.cpu().numpy()


def device_bits16(a: np.ndarray, dtype: torch.dtype, device) -> torch.Tensor:
    return torch.from_numpy(a.view(np.int16).copy()).view(dtype).to(device)


def group_index(P: int, seg: int, groups: np.ndarray) -> np.ndarray:
    """Element indices of the sampled groups (same local groups in every
    segment), segment by segment: the layout of a mini-message."""
    starts = np.concatenate([o * seg + groups * G for o in range(P)])
    return (starts[:, None] + np.arange(G)).reshape(-1)


def gather_elems(t: torch.Tensor, idx: np.ndarray) -> np.ndarray:
    return host(t[torch.from_numpy(idx).to(t.device)])


def payload_groups(pay: B.Payload, groups: np.ndarray, bits: int):
    """Codes bytes and params of the given groups of one payload (host)."""
    cb = G * bits // 8
    idx = (groups[:, None] * cb + np.arange(cb)).reshape(-1)
    codes = host(pay.codes[torch.from_numpy(idx).to(pay.codes.device)])
    params = host(pay.params[torch.from_numpy(groups).to(pay.params.device)])
    return codes, params


def assert_bits_equal(a: np.ndarray, b: np.ndarray, what: str):
    a = np.ascontiguousarray(a)
    b = np.ascontiguousarray(b)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    if a.dtype.itemsize == 4:
        a, b = a.view(np.uint32), b.view(np.uint32)
    bad = np.nonzero(a != b)[0]
    assert bad.size == 0, f"{what}: {bad.size} mismatches, first at {bad[0]}: {a[bad[0]]:#x} vs {b[bad[0]]:#x}"


def assert_float_close(gpu: np.ndarray, ref: np.ndarray, what: str, rtol=1e-5):
    """Floating-point bar: within 1e-5 relative (absolute floor: 1e-5 of the
    array's largest magnitude, for values that cancel to near zero)."""
    g = gpu.astype(np.float64)
    r = ref.astype(np.float64)
    floor = rtol * max(np.abs(r).max(), 1e-30)
    bad = np.nonzero(np.abs(g - r) > rtol * np.abs(r) + floor)[0]
    assert bad.size == 0, f"{what}: {bad.size} values off, first at {bad[0]}: {g[bad[0]]} vs {r[bad[0]]}"


def state_as_f32(a: np.ndarray) -> np.ndarray:
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32)
    return a


def random_payload_host(rng, seg: int, bits: int, group: int = G):
    """Arbitrary codes and finite fp16 scale/zero pairs (including subnormal
    and zero scales) as incoming payload test data."""
    codes = rng.integers(0, 256, size=seg * bits // 8, dtype=np.uint8)
    ng = seg // group
    sb = rng.integers(0, 0x7800, size=ng).astype(np.uint32)        # finite, |s| < 32768
    sb[rng.random(ng) < 0.05] = 0
    sb[rng.random(ng) < 0.05] = rng.integers(1, 0x400)              # subnormal steps
    zb = rng.integers(0, 0x7800, size=ng).astype(np.uint32) | (rng.integers(0, 2, size=ng) << 15).astype(np.uint32)
    return codes, (sb | (zb << 16)).astype(np.uint32)


def to_device_payload(codes: np.ndarray, params: np.ndarray, device) -> B.Payload:
    return B.Payload(torch.from_numpy(codes.copy()).to(device),
                     torch.from_numpy(params.view(np.int32).copy()).to(device))


def interleave(S: np.ndarray, L: np.ndarray) -> np.ndarray:
    """Device state layout from the oracle's two arrays: state[2j] = S_j, state[2j+1] = L_j."""
    out = np.empty(2 * S.size, S.dtype)
    out[0::2] = S
    out[1::2] = L
    return out


def split_state(t: torch.Tensor):
    """(S, L) host arrays from a device state buffer."""
    h = host(t)
    return h[0::2].copy(), h[1::2].copy()


def gather_state(t: torch.Tensor, idx: np.ndarray):
    """(S, L) of the elements `idx` from a device state buffer."""
    both = np.stack([2 * idx, 2 * idx + 1], axis=1).reshape(-1)
    h = gather_elems(t, both)
    return h[0::2].copy(), h[1::2].copy()
