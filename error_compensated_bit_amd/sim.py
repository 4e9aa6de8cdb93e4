"""P simulated ranks of one Echo all-reduce on a single GPU.

The payload a rank sends to an owner is a device buffer the owner's pass reads
directly, which stands in for the all-to-all; the owners' requantized payloads
are read the same way by the dequantize pass, which stands in for the
all-gather.  Only the library's entry points run; nothing here computes.
"""
from __future__ import annotations

from dataclasses import dataclass

import torch

from . import binding as B


def state_torch_dtype(cfg: B.echo_config) -> torch.dtype:
    return torch.float32 if cfg.state_dtype == B.ECHO_STATE_F32 else torch.bfloat16


def out_torch_dtype(cfg: B.echo_config) -> torch.dtype:
    return torch.bfloat16 if cfg.out_dtype == B.ECHO_OUT_BF16 else torch.float32


@dataclass
class Ranks:
    """Error state and payload buffers of P ranks with n-element messages.
    state[p] holds rank p's short and long memories side by side (2n elements)."""
    P: int
    n: int
    state: list
    sent: list      # sent[p][o]: payload rank p sends to owner o (None for o == p)
    owned: list     # owned[o]: owner o's requantized payload
    out: torch.Tensor

    seg_len: int = 0


def alloc_ranks(cfg: B.echo_config, P: int, n: int, device, bits_max: int | None = None) -> Ranks:
    """Buffers for P ranks; payloads are sized for `bits_max` (default cfg.bits)
    so one set of buffers serves calls of different widths."""
    bits = bits_max or cfg.bits
    seg = B.echo_segment_len(n, P, cfg.group)
    sdt = state_torch_dtype(cfg)
    state = [torch.empty(2 * n, dtype=sdt, device=device) for _ in range(P)]
    sent = [[None if o == p else B.alloc_payload(seg, bits, device, group=cfg.group)
             for o in range(P)] for p in range(P)]
    owned = [B.alloc_payload(seg, bits, device, group=cfg.group) for _ in range(P)]
    out = torch.empty(n, dtype=out_torch_dtype(cfg), device=device)
    r = Ranks(P, n, state, sent, owned, out, seg)
    for p in range(P):
        B.echo_state_reset(cfg, state[p], n)
    return r


def entry(cfg, r: Ranks, p: int, x: torch.Tensor, stream=None):
    B.echo_quantize_feedback(cfg, r.P, p, r.n, x, r.state[p], r.sent[p], stream)


def owner(cfg, r: Ranks, o: int, x: torch.Tensor, stream=None):
    inp = [None if p == o else r.sent[p][o] for p in range(r.P)]
    B.echo_owner_reduce_requant(cfg, r.P, o, r.n, x, r.state[o], inp, r.owned[o], stream)


def gather(cfg, r: Ranks, stream=None):
    B.echo_dequant_gather(cfg, r.P, r.n, r.owned, r.out, stream)


def allreduce(cfg, r: Ranks, xs, stream=None) -> torch.Tensor:
    """One call over all P ranks: every entry pass, then every owner pass,
    then the dequantize pass (its output is the same on every rank)."""
    for p in range(r.P):
        entry(cfg, r, p, xs[p], stream)
    for o in range(r.P):
        owner(cfg, r, o, xs[o], stream)
    gather(cfg, r, stream)
    return r.out


def share(cfg, r: Ranks, rank: int, x: torch.Tensor, stream=None):
    """One rank's share of a call (what one GPU computes): its entry pass, its
    owner pass (reading the payloads the other ranks sent it) and the
    dequantize pass over the gathered payloads."""
    entry(cfg, r, rank, x, stream)
    owner(cfg, r, rank, x, stream)
    gather(cfg, r, stream)
