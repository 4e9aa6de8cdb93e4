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


def free_device_bytes() -> int:
    """Free device memory once this process's cached blocks are released."""
    torch.cuda.empty_cache()
    return torch.cuda.mem_get_info(0)[0]


def random_bf16(n, seed, chunk=1 << 28):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    x = torch.empty(n, dtype=torch.bfloat16, device=DEV)
    for i in range(0, n, chunk):
        m = min(chunk, n - i)
        x[i:i + m] = torch.randn(m, generator=g, device=DEV).to(torch.bfloat16)
    return x


def test_message_past_32bit_indices():
    if free_device_bytes() < (110 << 30):
        pytest.skip("needs about 95 GB of free device memory")
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


# A dispatch holds at most 2^32 - 1 work-items along x.  The entry and owner
# passes put 2 elements on a lane with fp32 state (256-lane blocks), so a
# segment of more than (2^32 - 1) // 256 blocks * 512 elements, just under
# 2^33, goes out as two launches; the second starts at block 16,777,215 =
# group 67,108,860.
SPLIT_BLOCK = (2 ** 32 - 1) // 256
SPLIT_GROUP = SPLIT_BLOCK * 4
HUGE_SEG = (1 << 33) + (1 << 20)


def split_groups(gps, rng):
    """The first and last groups, the groups on both sides of the launch
    split, and random ones."""
    near = np.arange(SPLIT_GROUP - 6, SPLIT_GROUP + 6)
    return np.unique(np.concatenate([[0, 1, gps - 2, gps - 1], near,
                                     rng.choice(gps, size=40, replace=False)])).astype(np.int64)


def test_owner_pass_split_over_two_launches():
    """P = 1, n just above 2^33 elements: the owner pass (a requantizing
    round trip with the state update) runs as two launches; every sampled
    group -- both sides of the split among them -- matches the oracle over
    two chained calls, and so does the dequantized output.  About 100 GiB."""
    if free_device_bytes() < (110 << 30):
        pytest.skip("needs about 100 GiB of free device memory")
    P, n = 1, HUGE_SEG
    gps = n // G
    assert (gps + 3) // 4 > SPLIT_BLOCK
    cfg = B.make_config()
    ocfg = oracle_config(cfg)
    groups = split_groups(gps, np.random.default_rng(99))
    idx = group_index(P, n, groups)
    print(f"[gpu] owner pass over two launches: n={n}, {groups.size} groups compared", flush=True)
    r = None
    oS, oL = [np.zeros(idx.size, np.float32)], [np.zeros(idx.size, np.float32)]
    try:
        r = sim.alloc_ranks(cfg, P, n, DEV)
        for call in range(2):
            x = random_bf16(n, 5000 + call)
            sim.allreduce(cfg, r, [x])
            torch.cuda.synchronize()
            mini = [gather_elems(x, idx)]
            del x
            out, _, owned = O.allreduce(ocfg, mini, oS, oL)
            assert_bits_equal(gather_elems(r.out, idx), out, f"call {call} output")
            c, q = payload_groups(r.owned[0], groups, cfg.bits)
            assert_bits_equal(c, owned[0][0], f"call {call} codes")
            assert_bits_equal(q, owned[0][1], f"call {call} params")
            S, L = gather_state(r.state[0], idx)
            assert_bits_equal(S, oS[0], f"call {call} S")
            assert_bits_equal(L, oL[0], f"call {call} L")
            print(f"[gpu] owner pass over two launches: call {call} matches", flush=True)
    finally:
        del r
        torch.cuda.empty_cache()


def test_entry_pass_split_over_two_launches():
    """P = 2, segments just above 2^33 elements: rank 0's entry pass runs as
    two launches.  Its payload for owner 1 and its state match the oracle's
    entry pass on every sampled group of both segments (the owned segment's
    state stays empty).  About 170 GiB."""
    if free_device_bytes() < (175 << 30):
        pytest.skip("needs about 170 GiB of free device memory")
    P, seg = 2, HUGE_SEG
    n = P * seg
    gps = seg // G
    cfg = B.make_config()
    ocfg = oracle_config(cfg)
    groups = split_groups(gps, np.random.default_rng(98))
    idx = group_index(P, seg, groups)
    print(f"[gpu] entry pass over two launches: n={n}, {groups.size} groups per segment", flush=True)
    state = pay = None
    try:
        state = torch.empty(2 * n, dtype=torch.float32, device=DEV)
        pay = B.alloc_payload(seg, cfg.bits, DEV)
        B.echo_state_reset(cfg, state, n)
        x = random_bf16(n, 6000)
        B.echo_quantize_feedback(cfg, P, 0, n, x, state, [None, pay])
        torch.cuda.synchronize()
        mini = gather_elems(x, idx)
        del x
        oS, oL = np.zeros(idx.size, np.float32), np.zeros(idx.size, np.float32)
        sseg = groups.size * G
        ref = O.new_payload(ocfg, sseg)
        O.quantize_feedback(ocfg, P, 0, mini, oS, oL, [None, ref[0]], [None, ref[1]])
        c, q = payload_groups(pay, groups, cfg.bits)
        assert_bits_equal(c, ref[0], "codes for owner 1")
        assert_bits_equal(q, ref[1], "params for owner 1")
        S, L = gather_state(state, idx)
        assert_bits_equal(S, oS, "S")
        assert_bits_equal(L, oL, "L")
        assert not S[:sseg].any() and not L[:sseg].any()    # owned segment untouched
        print("[gpu] entry pass over two launches matches", flush=True)
    finally:
        del state, pay
        torch.cuda.empty_cache()
