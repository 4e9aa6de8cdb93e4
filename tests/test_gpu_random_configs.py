"""Seeded random configurations of whole calls, bit-exact against the oracle.

Each case draws P (1..16), the group size, the code width, the input /
output / state types, the feedback gain, both decays and the long-memory
share, and a message length (a multiple of P*group or any length), then runs
two chained calls over all P simulated ranks through the C ABI.  Every
payload byte a segment holds, every rank's state and the output must equal
the oracle's.  The cases complement the structured parity tests with
combinations nobody picked by hand.
"""
import numpy as np
import pytest
import torch

import oracle as O
from error_compensated_bit_amd import binding as B
from error_compensated_bit_amd import sim
from echo_testutil import assert_bits_equal, device_bits16, host, oracle_config, split_state

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def draw_cases(count: int, seed: int):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(count):
        P = int(rng.integers(1, 17))
        group = int(rng.choice([32, 64, 128]))
        if rng.random() < 0.5:
            n = P * group * int(rng.integers(1, 12))
        else:
            n = int(rng.integers(1, P * group * 12))
        cases.append(dict(
            id=i, P=P, group=group, n=n, bits=int(rng.choice([4, 8])),
            in_dtype=int(rng.integers(0, 2)), out_dtype=int(rng.integers(0, 2)),
            state_dtype=int(rng.integers(0, 2)),
            eta=float(rng.choice([1.0, 0.5, 0.0, 1.75])),
            beta_short=float(np.float32(rng.uniform(0.0, 0.99))),
            beta_long=float(np.float32(rng.uniform(0.0, 0.99))),
            mix_long=float(np.float32(rng.choice([0.0, 1.0 / 80, rng.uniform(0, 1), 1.0]))),
            scale=float(10.0 ** rng.uniform(-3, 3)), seed=int(rng.integers(1 << 30))))
    return cases


CASES = draw_cases(256, 20261203)


def make_inputs(rng, n, in_dtype, scale):
    v = (rng.standard_t(3, size=n) * scale).astype(np.float32)
    if in_dtype == B.ECHO_IN_F16:
        return O.f32_to_f16_bits(np.clip(v, -65504, 65504)), torch.float16
    return O.f32_to_bf16_bits(v), torch.bfloat16


def valid_bytes(n, P, group, bits, p):
    lo, hi = O.segment_range(n, P, group, p)
    ln = hi - lo
    return -(-ln * bits // 8), -(-ln // group)


@pytest.mark.parametrize("case", CASES, ids=[f"case{c['id']}" for c in CASES])
def test_random_configuration_two_calls(case):
    c = case
    print(f"[gpu] random case {c}", flush=True)
    cfg = B.make_config(bits=c["bits"], group=c["group"], eta=c["eta"],
                        beta_short=c["beta_short"], beta_long=c["beta_long"],
                        mix_long=c["mix_long"], in_dtype=c["in_dtype"],
                        out_dtype=c["out_dtype"], state_dtype=c["state_dtype"])
    ocfg = oracle_config(cfg)
    P, n, group, bits = c["P"], c["n"], c["group"], c["bits"]
    rng = np.random.default_rng(c["seed"])
    r = sim.alloc_ranks(cfg, P, n, DEV)
    oS = [np.zeros(n, O.state_np_dtype(ocfg)) for _ in range(P)]
    oL = [np.zeros(n, O.state_np_dtype(ocfg)) for _ in range(P)]
    for call in range(2):
        xs = [make_inputs(rng, n, c["in_dtype"], c["scale"]) for _ in range(P)]
        sim.allreduce(cfg, r, [device_bits16(b, dt, DEV) for b, dt in xs])
        torch.cuda.synchronize()
        out, sent, owned = O.allreduce(ocfg, [b for b, _ in xs], oS, oL)
        for o in range(P):
            cb, pb = valid_bytes(n, P, group, bits, o)
            assert_bits_equal(host(r.owned[o].codes)[:cb], owned[o][0][:cb], f"call {call} owned {o} codes")
            assert_bits_equal(host(r.owned[o].params)[:pb], owned[o][1][:pb], f"call {call} owned {o} params")
            for p in range(P):
                if p != o:
                    assert_bits_equal(host(r.sent[p][o].codes)[:cb], sent[p][o][0][:cb],
                                      f"call {call} sent {p}->{o} codes")
                    assert_bits_equal(host(r.sent[p][o].params)[:pb], sent[p][o][1][:pb],
                                      f"call {call} sent {p}->{o} params")
        for p in range(P):
            S, L = split_state(r.state[p])
            assert_bits_equal(S, oS[p], f"call {call} rank {p} short memory")
            assert_bits_equal(L, oL[p], f"call {call} rank {p} long memory")
        assert_bits_equal(host(r.out), out, f"call {call} output")
