"""GPU parity of each C-ABI entry point against the CPU oracle, at sizes the
oracle finishes in seconds: several 8-group tiles plus a ragged tail, every
supported type combination, the edge cases of the quantizer, P from 1 to 16,
and write-range checks with sentinel bytes.

Bar: codes and params bit-exact; state and outputs within 1e-5 relative
(they are expected, and checked, to be bit-exact as well).
"""
import numpy as np
import pytest
import torch

import oracle as O
from error_compensated_bit_amd import binding as B
from error_compensated_bit_amd import sim
from echo_testutil import (G, assert_bits_equal, assert_float_close, device_bits16, host,
                           interleave, oracle_config, random_payload_host, split_state,
                           state_as_f32, to_device_payload)

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

TYPES = [(B.ECHO_IN_BF16, B.ECHO_STATE_F32), (B.ECHO_IN_F16, B.ECHO_STATE_F32),
         (B.ECHO_IN_BF16, B.ECHO_STATE_BF16), (B.ECHO_IN_F16, B.ECHO_STATE_BF16)]


def banner(msg):
    print(f"[gpu] {msg}", flush=True)


def rand_input(rng, n, in_dtype, scale=1.0, special=False):
    v = rng.standard_t(4, size=n) * scale
    if special:
        k = n // 16
        v[:k] = 0.0
        v[k:2 * k] = -0.0
        v[2 * k:3 * k] = 0.375                               # constant groups
        v[3 * k:3 * k + 7] = [6e4, -6e4, 1e6, -1e6, 3e-6, -3e-6, 65504.0]
        v[4 * k:5 * k] = rng.normal(size=k) * 1e-6           # subnormal-fp16 steps
    v = v.astype(np.float32)
    if in_dtype == B.ECHO_IN_F16:
        v = np.clip(v, -65504, 65504)
        return O.f32_to_f16_bits(v), torch.float16
    return O.f32_to_bf16_bits(v), torch.bfloat16


def rand_state(rng, n, state_dtype, scale=0.05):
    v = (rng.normal(size=n) * scale).astype(np.float32)
    if state_dtype == B.ECHO_STATE_BF16:
        return O.f32_to_bf16_bits(v)
    return v


def state_dev(a):
    if a.dtype == np.uint16:
        return device_bits16(a, torch.bfloat16, DEV)
    return torch.from_numpy(a.copy()).to(DEV)


def cmp_arrays(g, ref, what):
    assert_float_close(state_as_f32(g), state_as_f32(ref), what)
    assert_bits_equal(g, ref, what + " (bits)")


def cmp_state(gpu_state, S_ref, L_ref, what):
    """Device state buffer (S_j, L_j pairs) against the oracle's S and L."""
    S, L = split_state(gpu_state)
    cmp_arrays(S, S_ref, what + " short memory")
    cmp_arrays(L, L_ref, what + " long memory")


# ------------------------------------------------------------------ entry pass
@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("in_dtype,state_dtype", TYPES)
@pytest.mark.parametrize("P,groups", [(2, 37), (3, 8), (4, 1), (8, 21), (16, 3)])
@pytest.mark.parametrize("group", [128, 64, 32])
def test_entry_pass(P, groups, bits, in_dtype, state_dtype, group):
    banner(f"entry P={P} groups={groups} bits={bits} in={in_dtype} state={state_dtype} group={group}")
    rng = np.random.default_rng(1000 * P + groups + bits + group)
    seg = groups * group
    n = P * seg
    cfg = B.make_config(bits=bits, group=group, in_dtype=in_dtype, state_dtype=state_dtype)
    ocfg = oracle_config(cfg)
    for rank in sorted({0, P - 1, P // 2}):
        xb, tdt = rand_input(rng, n, in_dtype, special=(rank == 0))
        s0, l0 = rand_state(rng, n, state_dtype), rand_state(rng, n, state_dtype, 0.2)
        x = device_bits16(xb, tdt, DEV)
        state = state_dev(interleave(s0, l0))
        out = [B.alloc_payload(seg, bits, DEV, fill=0xA5, group=group) for _ in range(P)]
        B.echo_quantize_feedback(cfg, P, rank, n, x, state, out)
        torch.cuda.synchronize()
        oc = [np.zeros(seg * bits // 8, np.uint8) if p != rank else None for p in range(P)]
        op = [np.zeros(groups, np.uint32) if p != rank else None for p in range(P)]   # groups per segment
        so, lo = s0.copy(), l0.copy()
        O.quantize_feedback(ocfg, P, rank, xb, so, lo, oc, op)
        for p in range(P):
            if p == rank:   # the owned slot is never written
                assert np.all(host(out[p].codes) == 0xA5)
                assert np.all(host(out[p].params.view(torch.uint8)) == 0xA5)
                continue
            assert_bits_equal(host(out[p].codes), oc[p], f"codes p={p}")
            assert_bits_equal(host(out[p].params), op[p], f"params p={p}")
        cmp_state(state, so, lo, "state")
        own = slice(rank * seg, (rank + 1) * seg)
        S, L = split_state(state)
        assert_bits_equal(S[own], s0[own], "owned S untouched")
        assert_bits_equal(L[own], l0[own], "owned L untouched")


# ------------------------------------------------------------------ owner pass
@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("out_dtype", [B.ECHO_OUT_BF16, B.ECHO_OUT_F32])
@pytest.mark.parametrize("in_dtype,state_dtype", TYPES)
@pytest.mark.parametrize("P,groups", [(1, 9), (2, 37), (3, 11), (5, 8), (6, 5), (8, 13), (11, 3),
                                      (16, 2)])
@pytest.mark.parametrize("group", [128, 64, 32])
def test_owner_pass(P, groups, bits, out_dtype, in_dtype, state_dtype, group):
    """Every slot count the owner kernel loads (P rounded up to 2, 4, 8, 16),
    with unused slots (P = 3, 5, 6, 11), for the first, a middle and the last
    rank."""
    banner(f"owner P={P} groups={groups} bits={bits} out={out_dtype} in={in_dtype} "
           f"state={state_dtype} group={group}")
    rng = np.random.default_rng(2000 * P + groups + bits + 10 * out_dtype + group)
    seg = groups * group
    n = P * seg
    cfg = B.make_config(bits=bits, group=group, in_dtype=in_dtype, out_dtype=out_dtype,
                        state_dtype=state_dtype)
    ocfg = oracle_config(cfg)
    for rank in sorted({0, P // 2, P - 1}):
        xb, tdt = rand_input(rng, n, in_dtype, special=(rank == 0))
        s0, l0 = rand_state(rng, n, state_dtype), rand_state(rng, n, state_dtype, 0.2)
        inc = [None if p == rank else random_payload_host(rng, seg, bits, group) for p in range(P)]
        if rank == 0 and P > 1:    # one sender of exactly representable integers
            k = rng.integers(0, 1 << bits, size=seg)
            c = k.astype(np.uint8) if bits == 8 else (k[0::2] | (k[1::2] << 4)).astype(np.uint8)
            inc[1] = (c, np.full(groups, 0x3C00, np.uint32))
        x = device_bits16(xb, tdt, DEV)
        state = state_dev(interleave(s0, l0))
        inp = [None if pl is None else to_device_payload(pl[0], pl[1], DEV) for pl in inc]
        out = B.alloc_payload(seg, bits, DEV, fill=0x5A, group=group)
        B.echo_owner_reduce_requant(cfg, P, rank, n, x, state, inp, out)
        torch.cuda.synchronize()
        oc = np.zeros(seg * bits // 8, np.uint8)
        op = np.zeros(groups, np.uint32)
        so, lo = s0.copy(), l0.copy()
        O.owner_reduce_requant(ocfg, P, rank, xb, so, lo,
                               [None if pl is None else pl[0] for pl in inc],
                               [None if pl is None else pl[1] for pl in inc], oc, op)
        assert_bits_equal(host(out.codes), oc, "owner codes")
        assert_bits_equal(host(out.params), op, "owner params")
        cmp_state(state, so, lo, "state")
        other = np.ones(n, bool)
        other[rank * seg:(rank + 1) * seg] = False
        S, L = split_state(state)
        assert_bits_equal(S[other], s0[other], "non-owned S untouched")
        assert_bits_equal(L[other], l0[other], "non-owned L untouched")


# ------------------------------------------------------------------ dequantize
@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("out_dtype", [B.ECHO_OUT_BF16, B.ECHO_OUT_F32])
@pytest.mark.parametrize("P,groups", [(1, 5), (2, 37), (8, 17), (16, 1), (3, 123)])
@pytest.mark.parametrize("group", [128, 64, 32])
def test_dequant_gather(P, groups, bits, out_dtype, group):
    banner(f"gather P={P} groups={groups} bits={bits} out={out_dtype} group={group}")
    rng = np.random.default_rng(3000 * P + groups + bits + out_dtype + group)
    seg = groups * group
    n = P * seg
    cfg = B.make_config(bits=bits, group=group, out_dtype=out_dtype)
    pls = [random_payload_host(rng, seg, bits, group) for _ in range(P)]
    inp = [to_device_payload(c, q, DEV) for c, q in pls]
    odt = torch.bfloat16 if out_dtype == B.ECHO_OUT_BF16 else torch.float32
    out = torch.empty(n + 64, dtype=odt, device=DEV)
    out.view(torch.uint8).fill_(0x77)
    B.echo_dequant_gather(cfg, P, n, inp, out[:n])
    torch.cuda.synchronize()
    ref = O.dequant_gather(oracle_config(cfg), P, n, [c for c, _ in pls], [q for _, q in pls])
    got = host(out)
    assert_bits_equal(got[:n], ref, "output")
    assert np.all(got[n:].view(np.uint8) == 0x77), "wrote past the output"


# ------------------------------------------------------------------ reset
@pytest.mark.parametrize("state_dtype", [B.ECHO_STATE_F32, B.ECHO_STATE_BF16])
@pytest.mark.parametrize("n", [1, 7, 8, 129, 4096, 1000003])
def test_state_reset(n, state_dtype):
    """The reset of a state holding garbage (NaN, Inf, -0, huge values)
    against the oracle's reset of the same garbage, interleaved into the
    device layout; the 16 elements past the 2n state words are sentinels."""
    cfg = B.make_config(state_dtype=state_dtype)
    ocfg = oracle_config(cfg)
    rng = np.random.default_rng(n + 7 * state_dtype)
    tail = 16
    v = (rng.normal(size=2 * n + tail) * 10.0).astype(np.float32)
    special = np.array([np.nan, np.inf, -np.inf, -0.0, 3e38, 1e-40], np.float32)
    v[rng.integers(0, v.size, v.size // 4)] = rng.choice(special, v.size // 4)
    garbage = O.f32_to_bf16_bits(v) if state_dtype == B.ECHO_STATE_BF16 else v
    S, L = garbage[0:2 * n:2].copy(), garbage[1:2 * n:2].copy()
    O.state_reset(S, L, ocfg)
    ref = garbage.copy()
    ref[:2 * n] = interleave(S, L)
    state = state_dev(garbage)
    assert B.echo_state_bytes(n, state_dtype) == 2 * n * state.element_size()
    B.echo_state_reset(cfg, state, n)
    torch.cuda.synchronize()
    assert_bits_equal(host(state), ref, "reset state (and the words past it)")
    assert not host(state)[:2 * n].view(np.uint32 if state_dtype == B.ECHO_STATE_F32 else np.uint16).any()


# ------------------------------------------------------------------ whole call
@pytest.mark.parametrize("P,groups,bits,out_dtype,state_dtype,group", [
    (1, 16, 4, B.ECHO_OUT_BF16, B.ECHO_STATE_F32, 128),
    (2, 1024, 4, B.ECHO_OUT_BF16, B.ECHO_STATE_F32, 128),     # the single-call 256k message
    (4, 77, 8, B.ECHO_OUT_F32, B.ECHO_STATE_F32, 128),
    (8, 29, 4, B.ECHO_OUT_BF16, B.ECHO_STATE_BF16, 128),
    (16, 5, 4, B.ECHO_OUT_F32, B.ECHO_STATE_BF16, 128),
    (4, 61, 4, B.ECHO_OUT_BF16, B.ECHO_STATE_F32, 64),
    (8, 45, 8, B.ECHO_OUT_BF16, B.ECHO_STATE_BF16, 64),
    (4, 99, 4, B.ECHO_OUT_BF16, B.ECHO_STATE_F32, 32),
    (8, 33, 4, B.ECHO_OUT_F32, B.ECHO_STATE_BF16, 32),
])
def test_allreduce_three_calls(P, groups, bits, out_dtype, state_dtype, group):
    """Three chained calls over P simulated ranks, state carried: every
    payload, the output and every rank's state against the oracle."""
    banner(f"allreduce P={P} groups={groups} bits={bits} group={group}")
    rng = np.random.default_rng(4000 + P + groups + group)
    seg = groups * group
    n = P * seg
    cfg = B.make_config(bits=bits, group=group, out_dtype=out_dtype, state_dtype=state_dtype)
    ocfg = oracle_config(cfg)
    r = sim.alloc_ranks(cfg, P, n, DEV)
    oS = [np.zeros(n, O.state_np_dtype(ocfg)) for _ in range(P)]
    oL = [np.zeros(n, O.state_np_dtype(ocfg)) for _ in range(P)]
    for site in range(3):
        xb = [rand_input(rng, n, B.ECHO_IN_BF16, scale=1.0 + site)[0] for _ in range(P)]
        xs = [device_bits16(a, torch.bfloat16, DEV) for a in xb]
        sim.allreduce(cfg, r, xs)
        torch.cuda.synchronize()
        out, sent, owned = O.allreduce(ocfg, xb, oS, oL)
        for p in range(P):
            for o in range(P):
                if o != p:
                    assert_bits_equal(host(r.sent[p][o].codes), sent[p][o][0], f"sent codes {p}->{o}")
                    assert_bits_equal(host(r.sent[p][o].params), sent[p][o][1], f"sent params {p}->{o}")
            assert_bits_equal(host(r.owned[p].codes), owned[p][0], f"owned codes {p}")
            assert_bits_equal(host(r.owned[p].params), owned[p][1], f"owned params {p}")
            cmp_state(r.state[p], oS[p], oL[p], f"rank {p} site {site}")
        got = host(r.out)
        if out_dtype == B.ECHO_OUT_F32:
            assert_float_close(got, out, "output")
        assert_bits_equal(got, out, "output bits")


def test_runs_on_the_callers_stream():
    P, seg = 4, 16 * G
    n = P * seg
    cfg = B.make_config()
    rng = np.random.default_rng(5)
    xb = [rand_input(rng, n, B.ECHO_IN_BF16)[0] for _ in range(P)]
    xs = [device_bits16(a, torch.bfloat16, DEV) for a in xb]
    r1 = sim.alloc_ranks(cfg, P, n, DEV)
    r2 = sim.alloc_ranks(cfg, P, n, DEV)
    sim.allreduce(cfg, r1, xs)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        sim.allreduce(cfg, r2, xs, stream=s)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    assert torch.equal(r1.out, r2.out)


@pytest.mark.parametrize("bits,in_dtype", [(4, B.ECHO_IN_BF16), (8, B.ECHO_IN_F16)])
@pytest.mark.parametrize("group", [128, 32])
def test_exact_ties_round_to_even(bits, in_dtype, group):
    """Groups built so that most elements sit exactly halfway between two
    codes: min 0 and max qmax * s with s a power of two, the rest at
    (k + 1/2) * s.  Codes must round half to even, as on the CPU."""
    P, groups = 2, 40
    seg = groups * group
    n = P * seg
    qmax = (1 << bits) - 1
    s = 2.0 if bits == 4 else 0.5
    rng = np.random.default_rng(17 + bits + group)
    v = ((rng.integers(0, qmax, size=n) + 0.5) * s).astype(np.float32)
    v[0::group] = 0.0
    v[1::group] = qmax * s
    xb = O.f32_to_f16_bits(v) if in_dtype == B.ECHO_IN_F16 else O.f32_to_bf16_bits(v)
    tdt = torch.float16 if in_dtype == B.ECHO_IN_F16 else torch.bfloat16
    back = (xb.astype(np.uint32) << 16).view(np.float32) if in_dtype == B.ECHO_IN_BF16 else \
        xb.view(np.float16).astype(np.float32)
    assert np.array_equal(back, v)                          # the ties survive the 16-bit input
    cfg = B.make_config(bits=bits, group=group, in_dtype=in_dtype)
    ocfg = oracle_config(cfg)
    x = device_bits16(xb, tdt, DEV)
    state = torch.zeros(2 * n, device=DEV)
    out = [None, B.alloc_payload(seg, bits, DEV, group=group)]
    B.echo_quantize_feedback(cfg, P, 0, n, x, state, out)
    torch.cuda.synchronize()
    oc = [None, np.zeros(seg * bits // 8, np.uint8)]
    op = [None, np.zeros(groups, np.uint32)]
    O.quantize_feedback(ocfg, P, 0, xb, np.zeros(n, np.float32), np.zeros(n, np.float32), oc, op)
    assert_bits_equal(host(out[1].codes), oc[1], "codes")
    assert_bits_equal(host(out[1].params), op[1], "params")
    codes = oc[1] if bits == 8 else np.stack([oc[1] & 15, oc[1] >> 4], axis=1).reshape(-1)
    k = np.rint(v[seg:] / s - 0.5).astype(np.int64)          # the tie lies between k and k + 1
    tie = np.ones(seg, bool)
    tie[0::group] = tie[1::group] = False
    assert np.all(codes[tie] % 2 == 0)
    assert np.all(codes[tie] == np.where(k[tie] % 2 == 0, k[tie], k[tie] + 1))


@pytest.mark.parametrize("bits", [4, 8])
def test_fp16_parameter_ties(bits):
    """Groups whose minimum lies exactly halfway between two fp16 values, and
    whose span / qmax is again exactly halfway between two fp16 values: both
    the zero point and the step must round half to even, as on the CPU.  The
    feedback term carries the values (x = 0, S = v, L = 0, gain 1), so any
    binary32 value can be placed in the group exactly."""
    P, groups, group = 2, 64, 128
    seg = groups * group
    n = P * seg
    qmax = (1 << bits) - 1
    rng = np.random.default_rng(23 + bits)
    h = rng.integers(0x0400, 0x5000, size=groups).astype(np.uint16)   # normal fp16, below 32
    lo = h.view(np.float16).astype(np.float32)
    hi = (h + 1).view(np.float16).astype(np.float32)
    mn = (lo + hi) / 2                                      # exact fp32 midpoints
    zf = mn.astype(np.float16).astype(np.float32)           # round half to even
    hs = rng.integers(0x2000, 0x4400, size=groups).astype(np.uint16)
    m = (hs.view(np.float16).astype(np.float32) + (hs + 1).view(np.float16).astype(np.float32)) / 2
    mx = zf + m * np.float32(qmax)
    assert np.all((mx - zf) / np.float32(qmax) == m)       # the quotient is the midpoint itself
    v = np.empty((groups, group), np.float32)
    for gi in range(groups):
        v[gi] = rng.uniform(mn[gi], mx[gi], size=group).astype(np.float32)
        v[gi, 0], v[gi, 1] = mn[gi], mx[gi]
        v[gi] = np.clip(v[gi], mn[gi], mx[gi])
    S = np.zeros(n, np.float32)
    S[seg:] = v.reshape(-1)
    cfg = B.make_config(bits=bits, group=group)
    ocfg = oracle_config(cfg)
    xb = np.zeros(n, np.uint16)
    x = device_bits16(xb, torch.bfloat16, DEV)
    state = state_dev(interleave(S, np.zeros(n, np.float32)))
    out = [None, B.alloc_payload(seg, bits, DEV, group=group)]
    B.echo_quantize_feedback(cfg, P, 0, n, x, state, out)
    torch.cuda.synchronize()
    oc = [None, np.zeros(seg * bits // 8, np.uint8)]
    op = [None, np.zeros(groups, np.uint32)]
    so, lo_ = S.copy(), np.zeros(n, np.float32)
    O.quantize_feedback(ocfg, P, 0, xb, so, lo_, oc, op)
    assert_bits_equal(host(out[1].params), op[1], "params")
    assert_bits_equal(host(out[1].codes), oc[1], "codes")
    cmp_state(state, so, lo_, "state")
    step_bits, zero_bits = op[1] & 0xFFFF, op[1] >> 16
    assert np.all(zero_bits & 1 == 0) and np.all(step_bits & 1 == 0)   # ties went to even


def test_reset_recovers_a_corrupted_state():
    """NaN and Inf in the error state are outside the contract and make the
    call's results undefined; echo_state_reset then restores a clean chain:
    two calls after the reset equal two calls from freshly allocated ranks."""
    P, seg = 4, 12 * G
    n = P * seg
    cfg = B.make_config()
    rng = np.random.default_rng(13)
    xs = [device_bits16(rand_input(rng, n, B.ECHO_IN_BF16)[0], torch.bfloat16, DEV) for _ in range(P)]
    fresh = sim.alloc_ranks(cfg, P, n, DEV)
    for _ in range(2):
        sim.allreduce(cfg, fresh, xs)
    r = sim.alloc_ranks(cfg, P, n, DEV)
    for st in r.state:
        st[0::7] = float("nan")
        st[3::11] = float("inf")
        st[5::13] = -float("inf")
    sim.allreduce(cfg, r, xs)                 # undefined results, but every kernel finishes
    for st in r.state:
        B.echo_state_reset(cfg, st, n)
    for _ in range(2):
        sim.allreduce(cfg, r, xs)
    torch.cuda.synchronize()
    assert torch.equal(r.out, fresh.out)
    for p in range(P):
        assert torch.equal(r.state[p], fresh.state[p])


def test_concurrent_host_threads_on_separate_streams():
    """The library keeps no state between calls: four host threads, each
    driving its own ranks on its own stream, produce what sequential calls
    produce (the binding releases the interpreter lock during each call)."""
    from concurrent.futures import ThreadPoolExecutor
    P, seg = 4, 24 * G
    n = P * seg
    cfg = B.make_config()
    rng = np.random.default_rng(11)
    inputs = [[device_bits16(rand_input(rng, n, B.ECHO_IN_BF16)[0], torch.bfloat16, DEV)
               for _ in range(P)] for _ in range(4)]
    ref = []
    for xs in inputs:
        r = sim.alloc_ranks(cfg, P, n, DEV)
        for _ in range(3):
            sim.allreduce(cfg, r, xs)
        ref.append((r.out.clone(), [st.clone() for st in r.state]))
    torch.cuda.synchronize()
    ranks = [sim.alloc_ranks(cfg, P, n, DEV) for _ in inputs]
    streams = [torch.cuda.Stream() for _ in inputs]
    torch.cuda.synchronize()

    def work(i):
        for _ in range(3):
            sim.allreduce(cfg, ranks[i], inputs[i], stream=streams[i])

    with ThreadPoolExecutor(max_workers=4) as pool:
        list(pool.map(work, range(len(inputs))))
    torch.cuda.synchronize()
    for i, (out, states) in enumerate(ref):
        assert torch.equal(ranks[i].out, out), f"thread {i} output"
        for p in range(P):
            assert torch.equal(ranks[i].state[p], states[p]), f"thread {i} rank {p} state"


def test_a_pending_error_of_the_caller_is_left_alone():
    """A HIP error the caller left pending (here a failed allocation, which
    touches no memory) neither fails a library call nor is cleared by it:
    each call checks its own launches' status."""
    import ctypes
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipMalloc.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_size_t]
    cfg = B.make_config()
    n = 4096
    state = torch.full((2 * n,), 7.0, device=DEV)
    torch.cuda.synchronize()
    hip.hipGetLastError()                                   # start from a clean slate
    ptr = ctypes.c_void_p()
    rc = hip.hipMalloc(ctypes.byref(ptr), ctypes.c_size_t(1 << 62))
    assert rc != 0
    B.echo_state_reset(cfg, state, n)                       # must not raise
    assert hip.hipGetLastError() == rc                      # still pending, then cleared
    torch.cuda.synchronize()
    assert torch.count_nonzero(state).item() == 0


def test_invalid_arguments_raise():
    cfg = B.make_config()
    x = torch.zeros(1024, dtype=torch.bfloat16, device=DEV)
    state = torch.zeros(2048, device=DEV)
    out = [B.alloc_payload(512, 4, DEV) for _ in range(2)]
    with pytest.raises(B.EchoError) as e:
        B.echo_quantize_feedback(cfg, 2, 0, 0, x, state, out)
    assert e.value.code == B.ECHO_ERR_SHAPE
    with pytest.raises(B.EchoError) as e:
        B.echo_quantize_feedback(cfg, 2, 0, 1024, x[1:], state, out)
    assert e.value.code == B.ECHO_ERR_ALIGN
    bad = B.make_config(bits=3)
    with pytest.raises(B.EchoError) as e:
        B.echo_dequant_gather(bad, 2, 1024, out, x)
    assert e.value.code == B.ECHO_ERR_ARG


# ------------------------------------------------------------------ ragged messages
def valid_payload_bytes(n, P, group, bits, p):
    """(code bytes, params) a segment holds: the rest of its buffer is never written."""
    lo, hi = O.segment_range(n, P, group, p)
    ln = hi - lo
    return -(-ln * bits // 8), -(-ln // group)


F16, BF16 = B.ECHO_IN_F16, B.ECHO_IN_BF16


@pytest.mark.parametrize("P,group,n,bits,state_dtype,out_dtype,in_dtype", [
    (4, 128, 1000, 4, B.ECHO_STATE_F32, B.ECHO_OUT_BF16, BF16),
    (3, 32, 1001, 4, B.ECHO_STATE_BF16, B.ECHO_OUT_BF16, F16),
    (8, 128, 300, 8, B.ECHO_STATE_F32, B.ECHO_OUT_F32, BF16),
    (2, 64, 7, 4, B.ECHO_STATE_F32, B.ECHO_OUT_BF16, BF16),
    (5, 32, 129, 8, B.ECHO_STATE_BF16, B.ECHO_OUT_F32, F16),
    (16, 128, 2049, 4, B.ECHO_STATE_BF16, B.ECHO_OUT_BF16, BF16),
    (1, 64, 1111, 4, B.ECHO_STATE_F32, B.ECHO_OUT_BF16, F16),
    (8, 128, 8 * 128 * 37 + 5, 4, B.ECHO_STATE_F32, B.ECHO_OUT_BF16, BF16),
    (6, 128, 6 * 128 * 11 + 6 * 128 - 1, 8, B.ECHO_STATE_F32, B.ECHO_OUT_BF16, F16),
])
def test_ragged_allreduce_two_calls(P, group, n, bits, state_dtype, out_dtype, in_dtype):
    """n not a multiple of P*group: the last non-empty segment ends in a
    partial group and later segments are empty.  Every payload byte a
    segment holds, the output and every state match the oracle; payload
    bytes past a segment's end keep their sentinel."""
    banner(f"ragged P={P} group={group} n={n} bits={bits}")
    rng = np.random.default_rng(n + P + group)
    cfg = B.make_config(bits=bits, group=group, state_dtype=state_dtype, out_dtype=out_dtype,
                        in_dtype=in_dtype)
    ocfg = oracle_config(cfg)
    seg = B.echo_segment_len(n, P, group)
    assert seg == O.segment_len(n, P, group)
    r = sim.alloc_ranks(cfg, P, n, DEV)
    for p in range(P):
        for pay in [r.owned[p]] + [r.sent[p][o] for o in range(P) if o != p]:
            pay.codes.fill_(0xA5)
            pay.params.view(torch.uint8).fill_(0xA5)
    oS = [np.zeros(n, O.state_np_dtype(ocfg)) for _ in range(P)]
    oL = [np.zeros(n, O.state_np_dtype(ocfg)) for _ in range(P)]
    for site in range(2):
        xb = [rand_input(rng, n, in_dtype, scale=1.0 + site)[0] for _ in range(P)]
        tdt = torch.float16 if in_dtype == F16 else torch.bfloat16
        sim.allreduce(cfg, r, [device_bits16(a, tdt, DEV) for a in xb])
        torch.cuda.synchronize()
        out, sent, owned = O.allreduce(ocfg, xb, oS, oL)
        for o in range(P):
            cb, pb = valid_payload_bytes(n, P, group, bits, o)
            pays = [(r.owned[o], owned[o], "owned")] + [(r.sent[p][o], sent[p][o], f"sent {p}")
                                                        for p in range(P) if p != o]
            for gpu_pay, ora_pay, tag in pays:
                c, q = host(gpu_pay.codes), host(gpu_pay.params)
                assert_bits_equal(c[:cb], ora_pay[0][:cb], f"{tag}->{o} codes")
                assert_bits_equal(q[:pb], ora_pay[1][:pb], f"{tag}->{o} params")
                assert np.all(c[cb:] == 0xA5), f"{tag}->{o}: codes written past the segment"
                assert np.all(q[pb:].view(np.uint8) == 0xA5), f"{tag}->{o}: params written past the segment"
        for p in range(P):
            cmp_state(r.state[p], oS[p], oL[p], f"rank {p} site {site}")
        assert_bits_equal(host(r.out), out, "output")


@pytest.mark.parametrize("group,n,P", [(128, 1000, 4), (32, 77, 2), (64, 65, 1)])
def test_ragged_gather_does_not_write_past_n(group, n, P):
    rng = np.random.default_rng(n)
    cfg = B.make_config(group=group)
    seg = B.echo_segment_len(n, P, group)
    pls = [random_payload_host(rng, seg, 4, group) for _ in range(P)]
    inp = [to_device_payload(c, q, DEV) for c, q in pls]
    out = torch.empty(n + 40, dtype=torch.bfloat16, device=DEV)
    out.view(torch.uint8).fill_(0x77)
    B.echo_dequant_gather(cfg, P, n, inp, out[:n])
    torch.cuda.synchronize()
    ref = O.dequant_gather(oracle_config(cfg), P, n, [c for c, _ in pls], [q for _, q in pls])
    got = host(out)
    assert_bits_equal(got[:n], ref, "output")
    assert np.all(got[n:].view(np.uint8) == 0x77)
