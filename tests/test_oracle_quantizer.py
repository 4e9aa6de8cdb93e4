"""Pins for the oracle's group quantizer Q and its payload layout.

Q is the zero-point-aware asymmetric quantizer of [JP] section 'Echoの仕組み①'
carrying 4-bit (or 8-bit) integers with half-precision parameters ([JP]
section 'よくある質問').  Nothing here re-implements the oracle's formula:
the checks are closed forms (groups whose grid is exact), exact rational
arithmetic on tiny groups (every code must be a nearest grid point, ties to
even), the parameters' definitions checked through numpy's float16 rounding,
order invariance, and the error bound of a nearest-point quantizer.

[JP] = 'テンソル並列の通信を4bitに圧縮する「Echo」——誤差補償で精度を保ちながら
分散LLMを高速化する仕組み'.
"""
import itertools
from fractions import Fraction as Fr

import numpy as np
import pytest

import oracle as O


def f16(bits: int) -> float:
    return float(np.array([bits], np.uint16).view(np.float16)[0])


def nearest_f16_bits(x: float) -> int:
    with np.errstate(over="ignore"):
        return int(np.array([x], np.float32).astype(np.float16).view(np.uint16)[0])


# --------------------------------------------------------------- closed forms
@pytest.mark.parametrize("bits", [4, 8])
def test_integer_group_is_lossless(bits):
    qmax = (1 << bits) - 1
    rng = np.random.default_rng(1)
    for _ in range(50):
        k = rng.integers(0, qmax + 1, size=128)
        k[rng.integers(128)] = 0
        k[rng.integers(128)] = qmax
        v = k.astype(np.float32)
        q, sb, zb, deq = O.quantize_group(v, bits)
        assert f16(sb) == 1.0 and zb == 0
        assert np.array_equal(q, k.astype(np.uint8))
        assert np.array_equal(deq, v)


def test_affine_grid_is_lossless():
    """v = z + k*s with fp16 z, s chosen so every grid point is exact in fp32:
    the quantizer must recover z, s and k exactly."""
    rng = np.random.default_rng(2)
    checked = 0
    while checked < 300:
        z = float(np.float16(rng.normal() * 4.0 ** rng.integers(-3, 4)))
        s = float(np.float16(abs(rng.normal()) * 4.0 ** rng.integers(-3, 3)))
        if s == 0.0 or z == 0.0:
            continue
        grid = [Fr(z) + k * Fr(s) for k in range(16)]
        if any(Fr(float(np.float32(float(g)))) != g for g in grid):
            continue                      # not exact in fp32: not a closed-form case
        k = rng.integers(0, 16, size=128)
        k[0], k[1] = 0, 15
        v = np.array([float(grid[i]) for i in k], np.float32)
        q, sb, zb, deq = O.quantize_group(v, 4)
        assert f16(zb) == z and f16(sb) == s
        assert np.array_equal(q, k.astype(np.uint8))
        assert np.array_equal(deq, v)
        checked += 1


# --------------------------------------------------------------- brute force
VALUES = [0.0, -0.0, 1.0, -1.0, 0.5, 2.5, -3.75, 7.0, 15.0, 0.1, -0.3, 1e-3,
          6e-8, -6e-8, 3e-5, 1000.0, -2048.0, 65504.0, -65504.0, 70000.0, -1e6,
          1.0 / 3.0, 7.5, 22.5]


def _check_group(v: np.ndarray, bits: int):
    qmax = (1 << bits) - 1
    q, sb, zb, deq = O.quantize_group(v, bits)
    mn, mx = float(v.min()), float(v.max())
    # zero point: nearest fp16 to the (range-clamped) minimum, never -0
    zexp = nearest_f16_bits(min(max(mn, -65504.0), 65504.0))
    if zexp == 0x8000:
        zexp = 0
    assert zb == zexp
    zf = f16(zb)
    # step: within half an fp16 spacing (plus the fp32 rounding of the
    # division) of the exact (max - zero) / qmax, clamped to [0, 65504]
    s_exact = (Fr(mx) - Fr(zf)) / qmax
    s_exact = min(max(s_exact, Fr(0)), Fr(65504))
    sf = f16(sb)
    assert sb < 0x7C00
    if s_exact > 0:
        ulp16 = Fr(f16(min(sb + 1, 0x7BFF)) - sf) if sb < 0x7BFF else Fr(32)
        assert abs(Fr(sf) - s_exact) <= ulp16 / 2 + s_exact * Fr(1, 1 << 22)
    else:
        assert sb == 0
    for i, vi in enumerate(v):
        vi = float(vi)
        if sf == 0.0:
            assert q[i] == 0
            assert float(deq[i]) == zf
            continue
        t = (Fr(vi) - Fr(zf)) / Fr(sf)     # exact position on the grid
        lo = max(0, min(qmax, int(np.floor(float(t)))))
        cands = {lo, max(0, min(qmax, lo + 1))}
        best = min(abs(t - c) for c in cands)
        nearest = {c for c in cands if abs(t - c) == best}
        if t < 0:
            nearest = {0}
        elif t > qmax:
            nearest = {qmax}
        near_tie = any(abs(abs(t - c) - Fr(1, 2)) < Fr(1, 1 << 17) for c in cands) and 0 <= t <= qmax
        if near_tie:
            # within fp32 rounding of a tie: either neighbour is a nearest point
            assert int(q[i]) in cands
        else:
            assert int(q[i]) in nearest, (v, i, t, q[i])
        # exact tie that fp32 reproduces exactly (power-of-two step): ties to even
        if t.denominator == 2 and 0 < t < qmax and (sf == 2.0 ** np.round(np.log2(sf))):
            assert int(q[i]) % 2 == 0
        # dequantized value: the grid point, rounded once to fp32
        g = Fr(int(q[i])) * Fr(sf) + Fr(zf)
        assert abs(Fr(float(deq[i])) - g) <= abs(g) * Fr(1, 1 << 24)
        # error bound of a nearest-point quantizer, inside the covered range
        if 0 <= t <= qmax:
            assert abs(Fr(float(deq[i])) - Fr(vi)) <= Fr(sf) / 2 * (1 + Fr(1, 1 << 16)) + abs(g) * Fr(1, 1 << 24)


@pytest.mark.parametrize("g", [2, 3, 4])
def test_brute_force_tiny_groups(g):
    for combo in itertools.product(VALUES[:12] if g == 4 else VALUES, repeat=g):
        v = np.array(combo, np.float32)
        _check_group(v, 4)
        if g == 2:
            _check_group(v, 8)


def test_random_groups_against_exact_rounding():
    rng = np.random.default_rng(3)
    for _ in range(400):
        scale = 10.0 ** rng.uniform(-6, 4)
        v = (rng.standard_t(4, size=128) * scale).astype(np.float32)
        _check_group(v, int(rng.choice([4, 8])))


def test_exact_ties_go_to_even():
    # step 1, zero 0: values k + 1/2 sit exactly between two codes
    v = np.array([0.0, 15.0, 0.5, 1.5, 2.5, 3.5, 12.5, 13.5, 14.5, 7.5], np.float32)
    q, sb, zb, deq = O.quantize_group(v, 4)
    assert f16(sb) == 1.0 and zb == 0
    assert list(q) == [0, 15, 0, 2, 2, 4, 12, 14, 14, 8]


def test_parameters_do_not_depend_on_element_order():
    rng = np.random.default_rng(4)
    for _ in range(100):
        v = rng.normal(size=128).astype(np.float32)
        perm = rng.permutation(128)
        q1, s1, z1, d1 = O.quantize_group(v, 4)
        q2, s2, z2, d2 = O.quantize_group(v[perm], 4)
        assert (s1, z1) == (s2, z2)
        assert np.array_equal(q1[perm], q2) and np.array_equal(d1[perm], d2)


# --------------------------------------------------------------- degenerate groups
def test_constant_group():
    # exactly representable: zero = value, no step, lossless
    q, sb, zb, deq = O.quantize_group(np.full(128, 0.5, np.float32), 4)
    assert sb == 0 and f16(zb) == 0.5 and not q.any() and np.all(deq == 0.5)
    # fp16 rounds the value up: the span above the zero point is negative,
    # so the step is 0 and every element decodes to the zero point
    up = np.float32(0.10002136)   # a quarter fp16 spacing below 0.10003662109375
    assert float(np.float16(up)) > float(up)
    q, sb, zb, deq = O.quantize_group(np.full(128, up, np.float32), 4)
    assert sb == 0 and not q.any() and np.all(deq == np.float32(np.float16(up)))
    # fp16 rounds the value down: a small (subnormal) step covers the gap,
    # every element gets the same code and the error shrinks below fp16's
    down = np.float32(0.1)
    assert float(np.float16(down)) < float(down)
    q, sb, zb, deq = O.quantize_group(np.full(128, down, np.float32), 4)
    assert 0 < sb < 0x0400 and np.all(q == q[0])
    assert abs(float(deq[0]) - float(down)) < abs(float(np.float16(down)) - float(down))


def test_zero_groups_have_all_zero_parameters():
    for v in (np.zeros(128, np.float32), np.full(128, -0.0, np.float32),
              np.array([0.0, -0.0] * 64, np.float32)):
        q, sb, zb, deq = O.quantize_group(v, 4)
        assert sb == 0 and zb == 0 and not q.any()
        assert np.all(deq.view(np.uint32) == 0)      # +0, not -0


def test_out_of_range_values_are_clamped_to_finite_fp16():
    v = np.array([-1e6, 1e6] + [0.0] * 126, np.float32)
    q, sb, zb, deq = O.quantize_group(v, 4)
    assert zb == 0xFBFF and sb == 0x7BFF          # -65504 and 65504
    assert np.all(np.isfinite(deq))
    assert q[0] == 0 and q[1] == 15


def test_tiny_ranges_use_fp16_subnormal_steps():
    v = (np.arange(16, dtype=np.float32) * np.float32(2.0 ** -24))
    q, sb, zb, deq = O.quantize_group(v, 4)
    assert zb == 0 and sb == 0x0001                 # step = smallest subnormal half
    assert np.array_equal(q, np.arange(16, dtype=np.uint8))


# --------------------------------------------------------------- payload layout
@pytest.mark.parametrize("bits", [4, 8])
def test_packed_payload_layout(bits):
    """Codes of a segment sit in element order; INT4 puts the even element in
    the low nibble; each group's parameters are scale | zero << 16."""
    qmax = (1 << bits) - 1
    P, rank, G = 2, 1, 128
    seg = 4 * G
    rng = np.random.default_rng(5)
    k = rng.integers(0, qmax + 1, size=seg)
    k[::G] = 0
    k[1::G] = qmax
    x = np.zeros(P * seg, np.float32)
    x[:seg] = k          # segment 0 is rank 1's non-owned segment
    xb = O.f32_to_bf16_bits(x)
    S = np.zeros(P * seg, np.float32)
    L = np.zeros(P * seg, np.float32)
    codes = [np.zeros(seg * bits // 8, np.uint8), None]
    params = [np.zeros(seg // G, np.uint32), None]
    O.quantize_feedback(O.Config(bits=bits), P, rank, xb, S, L, codes, params)
    if bits == 4:
        lo = codes[0] & 0x0F
        hi = codes[0] >> 4
        unpacked = np.stack([lo, hi], axis=1).reshape(-1)
    else:
        unpacked = codes[0]
    assert np.array_equal(unpacked, k.astype(np.uint8))
    assert np.all(params[0] == 0x3C00)   # scale 1.0 (0x3C00), zero 0.0
    assert not S.any() and not L.any()   # lossless: zero residual


def test_payload_bytes_do_not_depend_on_prior_buffer_contents():
    """The codes of a segment are fully written from scratch (INT4 bytes
    are rebuilt, not merged into old contents); an odd-length segment's last
    high nibble is 0."""
    P, rank, group, n = 2, 0, 32, 159       # segment 1 (rank 0 quantizes it) holds 63 elements
    rng = np.random.default_rng(8)
    x = O.f32_to_bf16_bits(rng.normal(size=n).astype(np.float32))
    seg = O.segment_len(n, P, group)
    assert seg == 96 and O.segment_range(n, P, group, 1) == (96, 159)
    outs = []
    for fill in (0x00, 0xFF, 0x5A):
        S = np.zeros(n, np.float32)
        L = np.zeros(n, np.float32)
        codes = [None, np.full(seg // 2, fill, np.uint8)]
        params = [None, np.full(seg // group, 0xFFFFFFFF, np.uint32)]
        O.quantize_feedback(O.Config(group=group), P, rank, x, S, L, codes, params)
        written = -(-63 // 2)                                  # bytes of 63 codes
        assert np.all(codes[1][written:] == fill)              # nothing past the segment
        outs.append((codes[1][:written].copy(), params[1][:2].copy()))
    for c, q in outs[1:]:
        assert np.array_equal(c, outs[0][0]) and np.array_equal(q, outs[0][1])
    assert outs[0][0][-1] >> 4 == 0                            # 63rd code: high nibble 0
