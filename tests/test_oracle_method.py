"""Pins for the oracle's whole all-reduce call and its error feedback.

What the pages fix about the method, checked on the oracle:
  * each value passes through the quantizer at most twice per call, for any
    number of GPUs ([EA] Abstract; [JP] 'Echoの仕組み①', 'まとめ');
  * the residuals the GPUs keep sum to the negated injected error ([JP]
    'Echoの仕組み②');
  * two moving averages of that error are added back into the next call's
    input, so the accumulated error follows a fixed linear filter of the
    injected errors; with gain 1 it stays within about 2.1 q instead of N q
    ([JP] '理論保証', 'なぜ4bit通信は難しかったのか');
  * closed forms: identical integer inputs sum exactly; zero stays zero;
    one rank reduces to one quantize round trip.

[EA] = 'Echo: Error-Compensated 4-Bit Tensor-Parallel Communication for LLM
Training and Inference' (abstract); [JP] = 'テンソル並列の通信を4bitに圧縮する
「Echo」——誤差補償で精度を保ちながら分散LLMを高速化する仕組み'.
"""
import json
import os

import numpy as np
import pytest

import oracle as O

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "echo_page_figures.json")))
G = 128


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def out_to_f64(out: np.ndarray, cfg: O.Config) -> np.ndarray:
    return bf16_to_f64(out) if cfg.out_dtype == O.OUT_BF16 else out.astype(np.float64)


def rand_bf16(rng, n, scale=1.0, t=None):
    v = rng.standard_t(t, size=n) if t else rng.normal(size=n)
    return O.f32_to_bf16_bits((v * scale).astype(np.float32))


def fresh_state(P, n, cfg=O.Config()):
    dt = O.state_np_dtype(cfg)
    return [np.zeros(n, dt) for _ in range(P)], [np.zeros(n, dt) for _ in range(P)]


# --------------------------------------------------------------- at most two quantizations
@pytest.mark.parametrize("P", [1, 2, 3, 4, 5, 8, 16])
def test_at_most_two_quantizations_for_any_P(P):
    fig = GOLDEN["max_quantizations_per_element"]
    n = P * G * 2
    rng = np.random.default_rng(P)
    xs = [rand_bf16(rng, n) for _ in range(P)]
    Ss, Ls = fresh_state(P, n)
    qpass = [np.zeros(n, np.uint32) for _ in range(P)]
    O.allreduce(O.Config(), xs, Ss, Ls, qpass=qpass)
    seg = n // P
    for p in range(P):
        assert qpass[p].max() <= fig["value"]
        own = slice(p * seg, (p + 1) * seg)
        assert np.all(qpass[p][own] == 1)          # own contribution: only the owner's requantization
        other = np.ones(n, bool)
        other[own] = False
        assert np.all(qpass[p][other] == 2)        # quantized once for the owner, once by it


# --------------------------------------------------------------- closed forms
@pytest.mark.parametrize("P", [1, 2, 4, 8])
def test_identical_integer_inputs_sum_exactly(P):
    """Every rank holds the same integers 0..15 (each group spans 0..15):
    the payloads are lossless and the owner's sum P*v requantizes exactly."""
    n = P * G * 4
    rng = np.random.default_rng(10 + P)
    k = rng.integers(0, 16, size=n)
    k[::G] = 0
    k[1::G] = 15
    x = O.f32_to_bf16_bits(k.astype(np.float32))
    xs = [x.copy() for _ in range(P)]
    Ss, Ls = fresh_state(P, n)
    out, _, _ = O.allreduce(O.Config(), xs, Ss, Ls)
    assert np.array_equal(out_to_f64(out, O.Config()), P * k.astype(np.float64))
    for p in range(P):
        assert not Ss[p].any() and not Ls[p].any()


def test_zero_message():
    P, n = 4, 4 * G * 2
    xs = [np.zeros(n, np.uint16) for _ in range(P)]
    Ss, Ls = fresh_state(P, n)
    out, sent, owned = O.allreduce(O.Config(), xs, Ss, Ls)
    assert not out.any()
    for o in range(P):
        assert not owned[o][0].any() and not owned[o][1].any()
    for p in range(P):
        assert not Ss[p].view(np.uint32).any() and not Ls[p].view(np.uint32).any()


@pytest.mark.parametrize("bits", [4, 8])
def test_single_rank_is_one_round_trip(bits):
    cfg = O.Config(bits=bits, out_dtype=O.OUT_F32)
    n = G * 8
    rng = np.random.default_rng(20)
    x = rand_bf16(rng, n, t=4)
    Ss, Ls = fresh_state(1, n)
    out, _, owned = O.allreduce(cfg, [x], Ss, Ls)
    xf = bf16_to_f64(x).astype(np.float32)
    for gi in range(n // G):
        sl = slice(gi * G, (gi + 1) * G)
        q, sb, zb, deq = O.quantize_group(xf[sl], bits)
        assert np.array_equal(out[sl], deq)
        assert owned[0][1][gi] == (sb | (zb << 16))


# --------------------------------------------------------------- residuals sum to -e
@pytest.mark.parametrize("P,bits,out_dtype", [(2, 4, O.OUT_BF16), (4, 4, O.OUT_BF16),
                                              (8, 4, O.OUT_F32), (8, 8, O.OUT_BF16),
                                              (16, 4, O.OUT_BF16)])
def test_residuals_sum_to_negated_injected_error(P, bits, out_dtype):
    """With the short memory taking the whole residual and no decay
    (beta_short = 0, mix = 0), S' = r exactly, so the residuals are visible.
    The injected error is e = o - sum_p x_p (state starts at zero, so the
    feedback-added input equals x).  Sum_p r_p must equal -e up to the fp32
    rounding of the owner's sum and of the residuals."""
    cfg = O.Config(bits=bits, out_dtype=out_dtype, beta_short=0.0, mix_long=0.0)
    n = P * G * 4
    rng = np.random.default_rng(30 + P + bits)
    xs = [rand_bf16(rng, n, t=4) for _ in range(P)]
    Ss, Ls = fresh_state(P, n)
    out, _, _ = O.allreduce(cfg, xs, Ss, Ls)
    xsum = sum(bf16_to_f64(x) for x in xs)
    e = out_to_f64(out, cfg) - xsum
    rsum = sum(S.astype(np.float64) for S in Ss)
    abs_terms = sum(np.abs(bf16_to_f64(x)) for x in xs) + np.abs(xsum) + np.abs(e)
    tol = (2 * P + 2) * 2.0 ** -24 * abs_terms
    assert np.all(np.abs(rsum + e) <= tol)
    assert np.abs(e).max() > 100 * tol.max()        # the identity is not trivially satisfied


# --------------------------------------------------------------- the owner's fp32 sum
def exact_dequant(codes: np.ndarray, params: np.ndarray, bits: int, count: int) -> np.ndarray:
    """code * step + zero for the first `count` elements of a payload, in
    fp64 (exact: an 8-bit code times an fp16 step plus an fp16 zero needs at
    most 51 significant bits), then rounded once to fp32 -- the value a
    single-rounding fused multiply-add gives."""
    if bits == 4:
        q = np.empty(codes.size * 2, np.uint8)
        q[0::2], q[1::2] = codes & 0xF, codes >> 4
    else:
        q = codes
    q = q[:count].astype(np.float64)
    grp = np.arange(count) // G
    step = (params[grp] & 0xFFFF).astype(np.uint16).view(np.float16).astype(np.float64)
    zero = (params[grp] >> 16).astype(np.uint16).view(np.float16).astype(np.float64)
    return (q * step + zero).astype(np.float32)


@pytest.mark.parametrize("P", [2, 3, 5, 8, 16])
@pytest.mark.parametrize("bits", [4, 8])
def test_owner_sum_within_recursive_summation_bound(P, bits):
    """The owner adds the P contributions in high precision ([JP]
    'Echoの仕組み①'; binary32 here).  For m terms added one by one in
    binary32, the computed sum s satisfies |s - exact| <= gamma_(m-1) *
    sum|terms|, gamma_k = k u / (1 - k u), u = 2^-24 (the classical bound of
    recursive summation).  Terms: the owner's own feedback-added input
    x + eta (S + L) (random fp32 state, so it carries a full 24-bit
    significand and most additions round) and the incoming payloads'
    dequantized codes, both computed here independently of the oracle.
    Magnitudes spread over four decades."""
    import math
    cfg = O.Config(bits=bits)
    n = P * G * 6
    rng = np.random.default_rng(70 + P + bits)
    xs = [O.f32_to_bf16_bits((rng.standard_t(3, n) * 10.0 ** rng.uniform(-2, 2, n)).astype(np.float32))
          for _ in range(P)]
    Ss = [rng.normal(size=n).astype(np.float32) for _ in range(P)]
    Ls = [(0.1 * rng.normal(size=n)).astype(np.float32) for _ in range(P)]
    seg = O.segment_len(n, P, G)
    # the owners' feedback-added inputs, before any pass touches the state
    v_own = [(bf16_to_f64(xs[o]).astype(np.float32)
              + np.float32(cfg.eta) * (Ss[o] + Ls[o]))[o * seg:(o + 1) * seg].astype(np.float64)
             for o in range(P)]
    sent = [[None if o == p else O.new_payload(cfg, seg) for o in range(P)] for p in range(P)]
    for p in range(P):
        O.quantize_feedback(cfg, P, p, xs[p], Ss[p], Ls[p],
                            [None if o == p else sent[p][o][0] for o in range(P)],
                            [None if o == p else sent[p][o][1] for o in range(P)])
    u = 2.0 ** -24
    gamma = (P - 1) * u / (1 - (P - 1) * u)
    for o in (0, P - 1):
        acc = np.zeros(seg, np.float32)
        out = O.new_payload(cfg, seg)
        O.owner_reduce_requant(cfg, P, o, xs[o], Ss[o], Ls[o],
                               [None if p == o else sent[p][o][0] for p in range(P)],
                               [None if p == o else sent[p][o][1] for p in range(P)],
                               out[0], out[1], acc=acc)
        terms = [v_own[o] if p == o else exact_dequant(sent[p][o][0], sent[p][o][1], bits, seg).astype(np.float64)
                 for p in range(P)]
        T = np.stack(terms)                                      # P x seg, rank order
        exact = np.array([math.fsum(T[:, k]) for k in range(seg)])
        bound = gamma * np.abs(T).sum(axis=0) * (1 + 1e-12)
        err = np.abs(acc.astype(np.float64) - exact)
        assert np.all(err <= bound), f"owner {o}: worst excess {np.max(err - bound)}"
        assert np.count_nonzero(err) > seg // 4                 # additions do round
        # a sum missing any one term lies far outside the bound
        for p in range(P):
            assert np.mean(np.abs(T[p]) > bound) > 0.9


# --------------------------------------------------------------- chained calls
def run_chain(cfg, P, n, sites, inputs):
    """Chain of `sites` calls with the state carried.  inputs(site) -> list of
    P bf16 arrays.  Returns per-site arrays (o - sum x, feedback sum F before
    the call), all in fp64."""
    Ss, Ls = fresh_state(P, n, cfg)
    d, F = [], []
    for k in range(sites):
        xs = inputs(k)
        F.append(sum(S.astype(np.float64) + Lm.astype(np.float64) for S, Lm in zip(Ss, Ls))
                 if cfg.state_dtype == O.STATE_F32 else
                 sum(bf16_to_f64(S) + bf16_to_f64(Lm) for S, Lm in zip(Ss, Ls)))
        out, _, _ = O.allreduce(cfg, xs, Ss, Ls)
        d.append(out_to_f64(out, cfg) - sum(bf16_to_f64(x) for x in xs))
    return np.array(d), np.array(F)


def filter_weights(cfg, m):
    """Share of an error injected m calls ago still present in the feedback:
    T_m = (1 - mix) bS^m + mix bL^m (the two memories are normalized moving
    averages that take shares 1 - mix and mix of each residual)."""
    return (1 - cfg.mix_long) * cfg.beta_short ** m + cfg.mix_long * cfg.beta_long ** m


@pytest.mark.parametrize("eta", [1.0, 0.5])
def test_accumulated_error_follows_the_feedback_filter(eta):
    """A_N = sum_k (o_k - sum_p x_pk) must equal sum_k [1 - eta(1 - T_{N-k})] e_k
    where e_k = o_k - sum_p v_pk is the error injected at call k."""
    cfg = O.Config(eta=eta)
    P, n, sites = 4, 4 * G * 8, 56
    rng = np.random.default_rng(40)
    seqs = [[rand_bf16(rng, n, t=4) for _ in range(P)] for _ in range(sites)]
    d, F = run_chain(cfg, P, n, sites, lambda k: seqs[k])
    e = d - eta * F                       # o_k - sum_p (x_pk + eta (S + L))
    A = np.cumsum(d, axis=0)
    scale = np.abs(e).max()
    for N in range(1, sites + 1):
        c = np.array([1 - eta * (1 - filter_weights(cfg, N - 1 - k)) for k in range(N)])
        pred = (c[:, None] * e[:N]).sum(axis=0)
        assert np.abs(A[N - 1] - pred).max() <= 1e-5 * scale, N


def chain_identity_residual(cfg, seqs, fault=None, at=None):
    """Run a chain of calls on the oracle, optionally with a fault at call
    `at`: "skip" discards that call's state update (the memories are put back
    as they were), "repeat" runs that call twice while counting its output
    once.  Returns the largest deviation of A_N from the filter prediction
    over all depths, relative to the largest injected error."""
    P, n = len(seqs[0]), seqs[0][0].size
    Ss, Ls = fresh_state(P, n, cfg)
    d, F = [], []
    for k, xs in enumerate(seqs):
        F.append(sum(S.astype(np.float64) + Lm.astype(np.float64) for S, Lm in zip(Ss, Ls)))
        keep = [(S.copy(), Lm.copy()) for S, Lm in zip(Ss, Ls)]
        if fault == "repeat" and k == at:
            O.allreduce(cfg, xs, Ss, Ls)
        out, _, _ = O.allreduce(cfg, xs, Ss, Ls)
        if fault == "skip" and k == at:
            for p, (S0, L0) in enumerate(keep):
                Ss[p][:] = S0
                Ls[p][:] = L0
        d.append(out_to_f64(out, cfg) - sum(bf16_to_f64(x) for x in xs))
    d, F = np.array(d), np.array(F)
    e = d - cfg.eta * F
    A = np.cumsum(d, axis=0)
    worst = 0.0
    for N in range(1, len(seqs) + 1):
        c = np.array([1 - cfg.eta * (1 - filter_weights(cfg, N - 1 - k)) for k in range(N)])
        worst = max(worst, np.abs(A[N - 1] - (c[:, None] * e[:N]).sum(axis=0)).max())
    return worst / np.abs(e).max()


@pytest.mark.parametrize("fault", ["skip", "repeat"])
def test_filter_identity_detects_a_skipped_or_repeated_call(fault):
    """The accumulated error follows the feedback filter only if every call
    updates the state exactly once ([JP] 'Echoの仕組み②'): a call whose state
    update is lost, or a call run twice, breaks the identity by far more than
    its rounding tolerance, so checking it detects either fault."""
    cfg = O.Config()
    P, n, sites = 4, 4 * G * 4, 12
    rng = np.random.default_rng(45)
    seqs = [[rand_bf16(rng, n, t=4) for _ in range(P)] for _ in range(sites)]
    assert chain_identity_residual(cfg, seqs) <= 1e-5
    assert chain_identity_residual(cfg, seqs, fault, at=5) > 1e-2


def test_bound_with_gain_one():
    """With eta = 1 the accumulated error stays within the stated factor of
    the per-call error at every depth; the filter's total weight
    (1-mix)/(1-bS) + mix/(1-bL) equals that factor under this repository's
    decays 0.5 / 0.9 and long-memory share 1/80."""
    fig = GOLDEN["accumulated_error_bound_factor_eta1"]
    cfg = O.Config(eta=fig["eta"])
    total = (1 - cfg.mix_long) / (1 - cfg.beta_short) + cfg.mix_long / (1 - cfg.beta_long)
    assert total == pytest.approx(fig["value"], abs=1e-12)
    P, n, sites = 4, 4 * G * 8, GOLDEN["depth_example_sites"]["value"]
    rng = np.random.default_rng(50)
    seqs = [[rand_bf16(rng, n, t=4) for _ in range(P)] for _ in range(sites)]
    d, F = run_chain(cfg, P, n, sites, lambda k: seqs[k])
    e = d - F
    A = np.cumsum(d, axis=0)
    q = np.abs(e).max(axis=0)             # per-element size of one call's error
    assert np.all(np.abs(A) <= fig["value"] * q * (1 + 1e-5))


def test_uncompensated_error_grows_as_N_q():
    """eta = 0 and the same input at every call: every call injects the same
    error, so A_N = N e_1 exactly; the improvement of the 2.1 q bound at the
    pages' depth of 56 is the stated ~27x."""
    P, n, sites = 4, 4 * G * 4, GOLDEN["depth_example_sites"]["value"]
    rng = np.random.default_rng(60)
    xs = [rand_bf16(rng, n, t=4) for _ in range(P)]
    d, F = run_chain(O.Config(eta=0.0), P, n, sites, lambda k: xs)
    assert np.all(d == d[0])                      # bit-identical outputs at every call
    A = np.cumsum(d, axis=0)
    assert np.array_equal(A[-1], sites * d[0])
    ratio = sites / GOLDEN["accumulated_error_bound_factor_eta1"]["value"]
    assert round(ratio) == GOLDEN["improvement_at_56_sites"]["value"]
    # with feedback the same repeated input stays bounded
    d1, F1 = run_chain(O.Config(eta=1.0), P, n, sites, lambda k: xs)
    e1 = d1 - F1
    A1 = np.cumsum(d1, axis=0)
    assert np.all(np.abs(A1) <= 2.1 * np.abs(e1).max(axis=0) * (1 + 1e-5))
    assert np.abs(A[-1]).mean() > 10 * np.abs(A1[-1]).mean()


def test_independent_errors_without_feedback_grow_as_sqrt_N():
    P, n, sites = 4, 4 * G * 16, 56
    rng = np.random.default_rng(70)
    seqs = [[rand_bf16(rng, n) for _ in range(P)] for _ in range(sites)]
    d, _ = run_chain(O.Config(eta=0.0), P, n, sites, lambda k: seqs[k])
    A = np.cumsum(d, axis=0)
    growth = np.sqrt((A[-1] ** 2).mean() / (d ** 2).mean())
    assert 0.8 * np.sqrt(sites) < growth < 1.2 * np.sqrt(sites)


# --------------------------------------------------------------- state reset
def garbage_state(rng, size, cfg):
    """Memories holding leftovers of anything: NaN, +-Inf, -0, huge, subnormal
    and ordinary values."""
    v = (rng.normal(size=size) * 10.0).astype(np.float32)
    special = np.array([np.nan, np.inf, -np.inf, -0.0, 3e38, -3e38, 1e-40, -1e-42], np.float32)
    v[rng.integers(0, size, size // 4)] = rng.choice(special, size // 4)
    if cfg.state_dtype == O.STATE_BF16:
        return O.f32_to_bf16_bits(v)
    return v


@pytest.mark.parametrize("state_dtype", [O.STATE_F32, O.STATE_BF16])
@pytest.mark.parametrize("n", [1, 7, 128, 1000])
def test_state_reset_empties_both_memories(state_dtype, n):
    """A chain of calls starts with both memories empty ([JP] 'Echoの仕組み②'
    carries each call's error into later calls; the chain start is this
    repository's reading): after the reset the first n elements of S and L
    are +0 bit patterns (numpy's zeros of the state type), whatever they held,
    and nothing past n is touched."""
    cfg = O.Config(state_dtype=state_dtype)
    rng = np.random.default_rng(n + 10 * state_dtype)
    S = garbage_state(rng, n + 64, cfg)
    L = garbage_state(rng, n + 64, cfg)
    S0, L0 = S.copy(), L.copy()
    O.state_reset(S, L, cfg, n)
    zeros = np.zeros(n, O.state_np_dtype(cfg))
    bits = np.uint32 if state_dtype == O.STATE_F32 else np.uint16
    assert np.array_equal(S[:n].view(bits), zeros.view(bits))
    assert np.array_equal(L[:n].view(bits), zeros.view(bits))
    assert np.array_equal(S[n:].view(bits), S0[n:].view(bits))
    assert np.array_equal(L[n:].view(bits), L0[n:].view(bits))


@pytest.mark.parametrize("state_dtype", [O.STATE_F32, O.STATE_BF16])
def test_reset_state_restarts_the_chain(state_dtype):
    """Ranks whose state was reset after arbitrary earlier traffic continue
    exactly like fresh ranks: every output, payload and state bit of three
    chained calls equals the chain started from numpy zeros."""
    cfg = O.Config(state_dtype=state_dtype)
    P, n = 4, 4 * G * 3 + 200                     # ragged: a partial last group
    rng = np.random.default_rng(77 + state_dtype)
    seqs = [[rand_bf16(rng, n, t=4) for _ in range(P)] for _ in range(3)]
    Sf, Lf = fresh_state(P, n, cfg)
    Sr = [garbage_state(rng, n, cfg) for _ in range(P)]
    Lr = [garbage_state(rng, n, cfg) for _ in range(P)]
    for _ in range(2):                            # earlier calls on the garbage
        O.allreduce(cfg, [rand_bf16(rng, n) for _ in range(P)], Sr, Lr)
    for p in range(P):
        O.state_reset(Sr[p], Lr[p], cfg)
    for xs in seqs:
        of, sf, wf = O.allreduce(cfg, xs, Sf, Lf)
        orr, sr, wr = O.allreduce(cfg, xs, Sr, Lr)
        assert np.array_equal(of, orr)
        for o in range(P):
            assert np.array_equal(wf[o][0], wr[o][0]) and np.array_equal(wf[o][1], wr[o][1])
            for p in range(P):
                if p != o:
                    assert np.array_equal(sf[p][o][0], sr[p][o][0])
                    assert np.array_equal(sf[p][o][1], sr[p][o][1])
        for p in range(P):
            assert np.array_equal(Sf[p].view(np.uint8), Sr[p].view(np.uint8))
            assert np.array_equal(Lf[p].view(np.uint8), Lr[p].view(np.uint8))


# --------------------------------------------------------------- storage variants
def test_bf16_state_stores_the_rounded_fp32_update():
    """A compact state keeps bf16(RNE) of the value the fp32 state would hold;
    from the same (bf16-representable) starting state one call agrees."""
    P, n = 4, 4 * G * 4
    rng = np.random.default_rng(80)
    xs = [rand_bf16(rng, n, t=4) for _ in range(P)]
    s0 = [O.f32_to_bf16_bits((0.05 * rng.normal(size=n)).astype(np.float32)) for _ in range(P)]
    l0 = [O.f32_to_bf16_bits((0.05 * rng.normal(size=n)).astype(np.float32)) for _ in range(P)]
    cf = O.Config()
    cb = O.Config(state_dtype=O.STATE_BF16)
    Sf = [bf16_to_f64(s).astype(np.float32) for s in s0]
    Lf = [bf16_to_f64(s).astype(np.float32) for s in l0]
    Sb = [s.copy() for s in s0]
    Lb = [s.copy() for s in l0]
    out_f, _, _ = O.allreduce(cf, xs, Sf, Lf)
    out_b, _, _ = O.allreduce(cb, xs, Sb, Lb)
    assert np.array_equal(out_f, out_b)
    for p in range(P):
        assert np.array_equal(Sb[p], O.f32_to_bf16_bits(Sf[p]))
        assert np.array_equal(Lb[p], O.f32_to_bf16_bits(Lf[p]))


def test_fp16_input_matches_bf16_input_on_common_values():
    """Values exact in both 16-bit formats give identical results."""
    P, n = 4, 4 * G * 4
    rng = np.random.default_rng(90)
    vals = [np.round(rng.normal(size=n) * 64) / 16 for _ in range(P)]   # multiples of 1/16, |v| < 64
    xb = [O.f32_to_bf16_bits(v.astype(np.float32)) for v in vals]
    xh = [O.f32_to_f16_bits(v.astype(np.float32)) for v in vals]
    for a, b in zip(xb, xh):
        assert np.array_equal(bf16_to_f64(a), O.f16_bits_to_f32(b).astype(np.float64))
    Sb, Lb = fresh_state(P, n)
    Sh, Lh = fresh_state(P, n)
    ob, _, _ = O.allreduce(O.Config(), xb, Sb, Lb)
    oh, _, _ = O.allreduce(O.Config(in_dtype=O.IN_F16), xh, Sh, Lh)
    assert np.array_equal(ob, oh)
    for p in range(P):
        assert np.array_equal(Sb[p], Sh[p]) and np.array_equal(Lb[p], Lh[p])


def test_payload_ratio_matches_the_stated_ceiling():
    """4-bit codes plus one fp16 scale and one fp16 zero per 128 elements
    carry 16 / (4 + 32/128) = 3.76x fewer bits than 16-bit values, the ~3.8x
    cap the pages state for the 4-bit gain."""
    fig = GOLDEN["speedup_ceiling_4bit"]
    payload_bits = 4 + 32 / G
    assert round(16 / payload_bits, 1) == fig["value"]
    # and the oracle's payload really is that size
    seg = G * 16
    codes, params = O.new_payload(O.Config(), seg)
    assert (codes.nbytes + params.nbytes) * 8 / seg == payload_bits


# --------------------------------------------------------------- ragged messages
# n not a multiple of P * group: segments of whole groups, the last non-empty
# one ends in a partial group, trailing ones may be empty (a reading of the
# pages, which fix no layout).
RAGGED = [(4, 128, 1000), (3, 32, 1000), (8, 128, 300), (2, 64, 7), (5, 32, 129), (16, 128, 2049)]


@pytest.mark.parametrize("P,group,n", RAGGED)
def test_ragged_at_most_two_quantizations(P, group, n):
    rng = np.random.default_rng(n + P)
    xs = [rand_bf16(rng, n) for _ in range(P)]
    Ss, Ls = fresh_state(P, n)
    qpass = [np.zeros(n, np.uint32) for _ in range(P)]
    O.allreduce(O.Config(group=group), xs, Ss, Ls, qpass=qpass)
    for p in range(P):
        lo, hi = O.segment_range(n, P, group, p)
        assert np.all(qpass[p][lo:hi] == 1)
        other = np.ones(n, bool)
        other[lo:hi] = False
        assert np.all(qpass[p][other] == 2)


@pytest.mark.parametrize("P,group,n", RAGGED)
def test_ragged_residuals_sum_to_negated_injected_error(P, group, n):
    cfg = O.Config(group=group, beta_short=0.0, mix_long=0.0)
    rng = np.random.default_rng(7 * n + P)
    xs = [rand_bf16(rng, n, t=4) for _ in range(P)]
    Ss, Ls = fresh_state(P, n)
    out, _, _ = O.allreduce(cfg, xs, Ss, Ls)
    xsum = sum(bf16_to_f64(x) for x in xs)
    e = out_to_f64(out, cfg) - xsum
    rsum = sum(S.astype(np.float64) for S in Ss)
    abs_terms = sum(np.abs(bf16_to_f64(x)) for x in xs) + np.abs(xsum) + np.abs(e)
    assert np.all(np.abs(rsum + e) <= (2 * P + 2) * 2.0 ** -24 * abs_terms)


@pytest.mark.parametrize("P,group,n", RAGGED)
def test_ragged_identical_integer_inputs_sum_exactly(P, group, n):
    rng = np.random.default_rng(3 * n)
    k = rng.integers(0, 16, size=n)
    seg = O.segment_len(n, P, group)
    for p in range(P):                      # every group, partial ones too, spans 0..15
        lo, hi = O.segment_range(n, P, group, p)
        for g0 in range(lo, hi, group):
            k[g0] = 0
            if g0 + 1 < hi:
                k[g0 + 1] = 15
    x = O.f32_to_bf16_bits(k.astype(np.float32))
    Ss, Ls = fresh_state(P, n)
    out, _, owned = O.allreduce(O.Config(group=group), [x.copy() for _ in range(P)], Ss, Ls)
    # (a one-element last group is a constant group: exact too, zero = the value)
    assert np.array_equal(out_to_f64(out, O.Config()), P * k.astype(np.float64))
    assert seg % group == 0


@pytest.mark.parametrize("group,n", [(128, 300), (32, 77), (64, 65)])
def test_ragged_single_rank_round_trip_per_group(group, n):
    cfg = O.Config(group=group, out_dtype=O.OUT_F32)
    rng = np.random.default_rng(n)
    x = rand_bf16(rng, n, t=4)
    Ss, Ls = fresh_state(1, n)
    out, _, owned = O.allreduce(cfg, [x], Ss, Ls)
    xf = bf16_to_f64(x).astype(np.float32)
    for gi, g0 in enumerate(range(0, n, group)):
        sl = slice(g0, min(g0 + group, n))
        q, sb, zb, deq = O.quantize_group(xf[sl], 4)
        assert np.array_equal(out[sl], deq)
        assert owned[0][1][gi] == (sb | (zb << 16))
        unpacked = np.stack([owned[0][0] & 0x0F, owned[0][0] >> 4], axis=1).reshape(-1)
        assert np.array_equal(unpacked[sl], q)
    # the unused high nibble of an odd-length INT4 segment is 0
    if n % 2:
        assert owned[0][0][n // 2] >> 4 == 0


def test_ragged_empty_segments():
    """n = 100 over P = 4 with groups of 128: only rank 0 owns elements."""
    P, group, n = 4, 128, 100
    assert [O.segment_range(n, P, group, p) for p in range(P)] == [(0, 100)] + [(100, 100)] * 3
    rng = np.random.default_rng(5)
    xs = [rand_bf16(rng, n) for _ in range(P)]
    Ss, Ls = fresh_state(P, n)
    out, sent, owned = O.allreduce(O.Config(group=group), xs, Ss, Ls)
    for o in range(1, P):
        assert not owned[o][0].any() and not owned[o][1].any()
    xsum = sum(bf16_to_f64(x) for x in xs)
    assert np.abs(out_to_f64(out, O.Config()) - xsum).max() < 0.5 * np.abs(xsum).max()
