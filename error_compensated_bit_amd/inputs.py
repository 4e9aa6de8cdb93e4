"""Seeded synthetic inputs for the Echo all-reduce workloads.

This module holds no arithmetic of the method: it only draws the per-rank
16-bit input messages.  Both the GPU path and the CPU oracle are fed from it.

The pages measure on trained LLMs (Qwen3-8B, Llama-3-8B, Qwen3-0.6B) and public
benchmarks that are not available here; the synthetic activations below stand
in for them, with the shapes of those models' tensor-parallel all-reduce
sites.  Every value is drawn in fp32 and rounded to the 16-bit input type
(round to nearest even, by torch's cast).

Seeds: rank p of site s of workload w draws from seed(w, s, p); per-channel
scales use rank index 99 so that all ranks of a site share one vector.
Large messages are drawn on the device (torch's Philox generator) and copied
to the host when the oracle needs them; the bytes define the input.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    wid: int               # numeric id used in seeds
    P: int                 # simulated ranks
    shape: tuple           # per-rank message shape (tokens, hidden) or (n,)
    dist: str              # value distribution, see draw()
    sites: int             # chained calls with the error state carried
    bits_by_site: tuple = field(default=())   # (first_sites, bits_early, bits_late) or ()
    description: str = ""

    @property
    def n(self) -> int:
        return int(math.prod(self.shape))

    def bits(self, site: int) -> int:
        if not self.bits_by_site:
            return 4
        first, early, late = self.bits_by_site
        return early if site < first else late


WORKLOADS = {
    "single_p2_256k": Workload(
        "single_p2_256k", 1, 2, (262144,), "normal_outliers", 1,
        description="single call, P=2, 262144 bf16/rank ~N(0,1), 0.1% outliers x20"),
    "chain56_p4_512x1024": Workload(
        "chain56_p4_512x1024", 2, 4, (512, 1024), "t4_chan", 56,
        description="56 chained calls, P=4, 512 tokens x 1024 hidden, "
                    "Student-t(4) x per-channel lognormal(0,0.5)"),
    "llama8b_p8_8192x4096": Workload(
        "llama8b_p8_8192x4096", 3, 8, (8192, 4096), "t4_chan", 64,
        description="Llama-3-8B-like TP site, P=8, 8192 x 4096, 64 chained sites, "
                    "Student-t(4) x per-channel lognormal(0,0.5)"),
    "msg1gib_p8": Workload(
        "msg1gib_p8", 4, 8, (536870912,), "normal", 1,
        description="1 GiB bf16 message (536870912 elements) per rank, P=8, iid N(0,1)"),
    "mixed_p8_16384x5120": Workload(
        "mixed_p8_16384x5120", 5, 8, (16384, 5120), "t3", 80, (20, 8, 4),
        description="P=8, 16384 x 5120, 80 sites: first 20 INT8, rest INT4, Student-t(3)"),
}


def seed(wid: int, site: int, rank: int) -> int:
    return ((wid * 1000 + site) * 100 + rank) * 7919 + 12345


def _gen(device, s: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(s)
    return g


def draw(dist: str, shape, device, wid: int, site: int, rank: int) -> torch.Tensor:
    """fp32 values of one rank's message (before the 16-bit cast)."""
    g = _gen(device, seed(wid, site, rank))
    f32 = torch.float32
    if dist == "normal":
        return torch.randn(shape, generator=g, device=device, dtype=f32)
    if dist == "normal_outliers":
        x = torch.randn(shape, generator=g, device=device, dtype=f32)
        u = torch.rand(shape, generator=g, device=device, dtype=f32)
        return torch.where(u < 1e-3, x * 20.0, x)
    if dist in ("t4_chan", "t4"):
        z = torch.randn(shape, generator=g, device=device, dtype=f32)
        u1 = 1.0 - torch.rand(shape, generator=g, device=device, dtype=f32)
        u2 = 1.0 - torch.rand(shape, generator=g, device=device, dtype=f32)
        chi2_4 = -2.0 * torch.log(u1 * u2)          # chi-square with 4 degrees of freedom
        x = z / torch.sqrt(chi2_4 / 4.0)
        if dist == "t4_chan":
            gc = _gen(device, seed(wid, site, 99))
            ch = torch.exp(0.5 * torch.randn(shape[-1], generator=gc, device=device, dtype=f32))
            x = x * ch
        return x
    if dist == "t3":
        z = torch.randn((4,) + tuple(shape), generator=g, device=device, dtype=f32)
        chi2_3 = z[1] * z[1] + z[2] * z[2] + z[3] * z[3]
        return z[0] / torch.sqrt(chi2_3 / 3.0)
    raise ValueError(f"unknown distribution {dist}")


def make_x(w: Workload, site: int, rank: int, device="cpu",
           dtype: torch.dtype = torch.bfloat16) -> torch.Tensor:
    """One rank's flattened 16-bit message for site `site` of workload `w`."""
    return draw(w.dist, w.shape, device, w.wid, site, rank).to(dtype).reshape(-1)


def bits16_numpy(t: torch.Tensor):
    """Host uint16 view of a 16-bit tensor's bits (for the oracle)."""
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view("uint16")
