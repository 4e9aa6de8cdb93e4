"""A message longer than 2^32 elements, end to end through the C ABI.

Element indices past 2^32 and byte offsets past 2^34 (fp32 state) exercise
every kernel's 64-bit addressing; the bench's 1 GiB message stops at 2^29
elements.  P = 2, n = 2^32 + 2048 bf16 elements per rank (8 GiB), two
chained calls.  The GPU runs the whole message; the oracle runs the same
sampled groups of both segments -- the first, middle and last groups among
them -- as a mini-message (every group is independent of the others, also
across calls, because the state is per element), and the two must agree bit
for bit on output, payloads and state.  About 95 GB of device memory.
"""
import numpy as np
import pytest
import torch

import oracle as O
from error_compensated_bit_amd import binding as B
from error_compensated_bit_amd import sim
from echo_testutil import (G, assert_bits_equal, gather_elems, gather_state, group_index,
                           oracle_config, payload_groups)

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def random_bf16(n, seed, chunk=1 << 28):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    x = torch.empty(n, dtype=torch.bfloat16, device=DEV)
    for i in range(0, n, chunk):
        m = min(chunk, n - i)
        x[i:i + m] = torch.randn(m, generator=g, device=DEV).to(torch.bfloat16)
    return x


def test_message_past_32bit_indices():
    if torch.cuda.get_device_properties(0).total_memory < (140 << 30):
        pytest.skip("needs about 95 GB of device memory")
    P = 2
    n = (1 << 32) + P * G * 8
    seg = n // P
    gps = seg // G
    cfg = B.make_config()
    ocfg = oracle_config(cfg)
    rng = np.random.default_rng(4242)
    groups = np.unique(np.concatenate([[0, 1, gps // 2, gps - 2, gps - 1],
                                       rng.choice(gps, size=60, replace=False)])).astype(np.int64)
    idx = group_index(P, seg, groups)
    assert idx.max() > (1 << 32)
    print(f"[gpu] large message: n={n}, P={P}, {groups.size} groups per segment compared", flush=True)
    r = sim.alloc_ranks(cfg, P, n, DEV)
    oS = [np.zeros(idx.size, np.float32) for _ in range(P)]
    oL = [np.zeros(idx.size, np.float32) for _ in range(P)]
    try:
        for call in range(2):
            xs = [random_bf16(n, 1000 * call + p) for p in range(P)]
            sim.allreduce(cfg, r, xs)
            torch.cuda.synchronize()
            mini = [gather_elems(x, idx) for x in xs]
            del xs
            out, sent, owned = O.allreduce(ocfg, mini, oS, oL)
            tag = f"call {call}"
            assert_bits_equal(gather_elems(r.out, idx), out, f"{tag} output")
            for o in range(P):
                c, q = payload_groups(r.owned[o], groups, cfg.bits)
                assert_bits_equal(c, owned[o][0], f"{tag} owned codes {o}")
                assert_bits_equal(q, owned[o][1], f"{tag} owned params {o}")
                for p in range(P):
                    if p != o:
                        c, q = payload_groups(r.sent[p][o], groups, cfg.bits)
                        assert_bits_equal(c, sent[p][o][0], f"{tag} sent codes {p}->{o}")
                        assert_bits_equal(q, sent[p][o][1], f"{tag} sent params {p}->{o}")
            for p in range(P):
                S, L = gather_state(r.state[p], idx)
                assert_bits_equal(S, oS[p], f"{tag} S rank {p}")
                assert_bits_equal(L, oL[p], f"{tag} L rank {p}")
            print(f"[gpu] large message: call {call} matches", flush=True)
    finally:
        del r
        torch.cuda.empty_cache()
