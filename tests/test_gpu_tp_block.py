"""Echo inside a tensor-parallel residual stream with random weights.

[JP] section '理論保証' bounds the accumulated error of Echo with gain 1 for
networks that do not keep amplifying perturbations; without the feedback the
error of N sites grows like N q ([JP] 'なぜ4bit通信は難しかったのか').  Here the
injected errors pass through real branches: at every site k each of P
simulated ranks computes a row-parallel partial product of the RMS-normalized
hidden state (its shard of the features times a random weight shard), the
all-reduce sums the P partials, and the sum is added to the residual stream:

    h_k = h_{k-1} + allreduce_p( rmsnorm(h_{k-1})[:, shard_p] @ W_k[shard_p, :] )

The same chain runs with the exact fp32 sum (the reference trajectory), with
a 16-bit all-reduce (fp32 sum, bf16 output: what a 16-bit NCCL all-reduce
delivers), and with Echo (INT4, feedback gain 1, and gain 0 = no feedback).
Each trajectory feeds its own h into its later branches.  Random weights only
(no trained model).

Every Echo call of the chain is also checked against the CPU oracle: the
same bf16 partials go to the oracle's all-reduce with its own error state
carried from site to site, and the output and every rank's short and long
memories must agree bit for bit at every site, for gain 1 and gain 0.

[JP] = 'テンソル並列の通信を4bitに圧縮する「Echo」——誤差補償で精度を保ちながら
分散LLMを高速化する仕組み'.
"""
import math

import numpy as np
import pytest
import torch

import oracle as O
from error_compensated_bit_amd import binding as B
from error_compensated_bit_amd import sim
from echo_testutil import assert_bits_equal, host, oracle_config, split_state

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def rmsnorm(h: torch.Tensor) -> torch.Tensor:
    return h * torch.rsqrt((h * h).mean(dim=-1, keepdim=True) + 1e-6)


def run_tp_chain(P=4, tokens=512, hidden=1024, sites=56, gain=1.0, norm=True, seed=0):
    """Residual-stream deviation from the exact trajectory after every site,
    for the 16-bit all-reduce and for Echo with feedback gain 1 and 0.
    Returns {name: [rms deviation after site k]} and the rms size of one
    Echo all-reduce's injected error at the first site."""
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    h0 = torch.randn(tokens, hidden, generator=g, device=DEV)
    weights = [torch.randn(hidden, hidden, generator=g, device=DEV) * (gain / math.sqrt(hidden))
               for _ in range(sites)]
    shard = hidden // P
    n = tokens * hidden

    def partials(h, W):
        a = rmsnorm(h) if norm else h
        return [(a[:, p * shard:(p + 1) * shard] @ W[p * shard:(p + 1) * shard, :]) for p in range(P)]

    runs = {"exact_fp32": None, "allreduce_bf16": None, "echo_eta1": 1.0, "echo_eta0": 0.0}
    hs = {k: h0.clone() for k in runs}
    ranks = {k: sim.alloc_ranks(B.make_config(eta=eta), P, n, DEV)
             for k, eta in runs.items() if eta is not None}
    # the oracle's error state of every rank, carried from site to site
    ostate = {k: ([np.zeros(n, np.float32) for _ in range(P)], [np.zeros(n, np.float32) for _ in range(P)])
              for k, eta in runs.items() if eta is not None}
    dev = {k: [] for k in runs if k != "exact_fp32"}
    first_error = None
    for k in range(sites):
        W = weights[k]
        ys = partials(hs["exact_fp32"], W)
        hs["exact_fp32"] = hs["exact_fp32"] + sum(ys)
        ys = [y.to(torch.bfloat16) for y in partials(hs["allreduce_bf16"], W)]
        hs["allreduce_bf16"] = hs["allreduce_bf16"] + sum(y.float() for y in ys).to(torch.bfloat16).float()
        for name in ("echo_eta1", "echo_eta0"):
            ys = [y.to(torch.bfloat16).contiguous().reshape(-1) for y in partials(hs[name], W)]
            cfg = B.make_config(eta=runs[name])
            r = ranks[name]
            got = sim.allreduce(cfg, r, ys)
            torch.cuda.synchronize()
            oS, oL = ostate[name]
            ref, _, _ = O.allreduce(oracle_config(cfg), [host(y) for y in ys], oS, oL)
            assert_bits_equal(host(got), ref, f"{name} site {k} output")
            for p in range(P):
                S, L = split_state(r.state[p])
                assert_bits_equal(S, oS[p], f"{name} site {k} rank {p} short memory")
                assert_bits_equal(L, oL[p], f"{name} site {k} rank {p} long memory")
            out = got.float().reshape(tokens, hidden)
            if first_error is None:
                first_error = (out - sum(y.float() for y in ys).reshape(tokens, hidden)).pow(2).mean().sqrt().item()
            hs[name] = hs[name] + out
        for name in dev:
            dev[name].append((hs[name] - hs["exact_fp32"]).pow(2).mean().sqrt().item())
    torch.cuda.synchronize()
    return dev, first_error


def report(tag, dev, q, sites):
    print(f"[tp] {tag}: every Echo call matched the oracle bit for bit; "
          f"one call's injected error (rms) q = {q:.4g}")
    for k in sorted({0, 3, 7, 15, sites - 1}):
        print(f"[tp]   after site {k + 1:2d}: echo eta=1 {dev['echo_eta1'][k] / q:9.3f} q   "
              f"eta=0 {dev['echo_eta0'][k] / q:9.3f} q   16-bit all-reduce "
              f"{dev['allreduce_bf16'][k] / q:8.3f} q")


def test_feedback_keeps_the_residual_stream_error_bounded():
    """Normalized branches with a small gain (little amplification): with
    feedback the deviation after 56 sites stays within a few single-call
    errors and several times below the chain without feedback, whose
    independent per-site errors keep adding up."""
    dev, q = run_tp_chain(gain=0.3)
    report("normalized, gain 0.3", dev, q, 56)
    e1, e0 = dev["echo_eta1"], dev["echo_eta0"]
    assert e1[-1] < 4 * q
    assert e1[-1] < e0[-1] / 3
    assert e0[-1] > 2 * e0[7]


def test_second_order_growth_with_unit_gain():
    """Unit-gain branches pass part of every earlier error into later
    branch inputs.  The feedback still removes most of the accumulation, and
    what remains grows like sqrt(N) (the second-order remainder the bound
    leaves, [JP] '理論保証')."""
    dev, q = run_tp_chain(gain=1.0)
    report("normalized, gain 1.0", dev, q, 56)
    e1, e0 = dev["echo_eta1"], dev["echo_eta0"]
    assert e1[-1] < e0[-1] / 2
    growth = e1[55] / e1[15]
    assert 0.75 * math.sqrt(56 / 16) < growth < 1.25 * math.sqrt(56 / 16)


def test_amplifying_branches_defeat_the_bound():
    """The bound excludes networks that keep amplifying perturbations ([JP]
    '理論保証').  Unnormalized unit-gain branches multiply every perturbation
    at every site: the deviation grows geometrically with or without the
    feedback."""
    dev, q = run_tp_chain(sites=20, gain=1.0, norm=False)
    report("unnormalized, gain 1.0", dev, q, 20)
    e1 = dev["echo_eta1"]
    assert e1[-1] > 100 * q
    assert e1[19] > 20 * e1[9]
