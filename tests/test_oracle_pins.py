"""Pins of the CPU oracle against things other than itself.

Closed forms, brute force on tiny inputs, independent library routines
(torch's scaled_dot_product_attention, numpy's SVD-based matrix 2-norm,
Python's exact `statistics.pvariance` on Fractions) and hand-worked values.
Each test is chosen so that a plausible slip in the oracle (a dropped term,
a wrong sign or index, a transposed operand, the wrong causal side, the wrong
rounding mode) fails it.  CPU only.
"""
import itertools
import math
import statistics
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle as O


def _rng(seed):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------- stage 1

def _attention_matrix_sdpa(Qg, Kh):
    """A[g] = causal softmax(Q_g K^T / sqrt(d)) via torch SDPA with V = I (fp64, CPU)."""
    G, N, d = Qg.shape
    q = torch.from_numpy(Qg.astype(np.float64))[None]
    k = torch.from_numpy(np.broadcast_to(Kh.astype(np.float64), (G, N, d)).copy())[None]
    eye = torch.eye(N, dtype=torch.float64).expand(1, G, N, N).contiguous()
    return torch.nn.functional.scaled_dot_product_attention(q, k, eye, is_causal=True)[0].numpy()


@pytest.mark.parametrize("G,N", [(1, 7), (4, 33), (2, 130)])
def test_token_weights_match_sdpa_column_sums(G, N):
    r = _rng(1)
    Q = r.standard_normal((G, N, 128)).astype(np.float16)
    K = (r.standard_normal((N, 128)) * 1.5).astype(np.float16)
    A = _attention_matrix_sdpa(Q, K)
    ref = A.sum(axis=(0, 1))
    w = O.token_weights(Q, K, block=16)
    np.testing.assert_allclose(w, ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("N", [1, 9, 70])
def test_row_lse_normalises_the_sdpa_attention_rows(N):
    # exp(s - LSE) must reproduce torch's causal attention matrix row by row
    r = _rng(11)
    Q = r.standard_normal((1, N, 128)).astype(np.float16)
    K = r.standard_normal((N, 128)).astype(np.float16)
    lse = O.row_lse(Q[0], K, block=8)
    S = Q[0].astype(np.float64) @ K.astype(np.float64).T / math.sqrt(128)
    A = np.where(np.tril(np.ones((N, N), dtype=bool)), np.exp(S - lse[:, None]), 0.0)
    np.testing.assert_allclose(A, _attention_matrix_sdpa(Q, K)[0], rtol=1e-12, atol=1e-15)


def test_row_lse_closed_forms():
    # Q = 0: every visible score is 0, so LSE_tau = ln(tau + 1)
    N = 300
    K = _rng(12).standard_normal((N, 128)).astype(np.float16)
    lse = O.row_lse(np.zeros((N, 128), np.float16), K, block=64)
    np.testing.assert_allclose(lse, np.log(np.arange(1, N + 1)), rtol=0, atol=1e-12)
    # one visible key: row 0's LSE is its only score, and a key far above the
    # rest dominates later rows: LSE -> its score
    Q = np.zeros((3, 128), np.float16)
    Q[:, 0] = 1.0
    Kb = np.zeros((3, 128), np.float16)
    Kb[0, 0] = 2.0
    Kb[1, 0] = 300.0
    l3 = O.row_lse(Q, Kb)
    s0, s1 = 2.0 / math.sqrt(128), 300.0 / math.sqrt(128)   # row 2 also sees key 2, score 0
    assert l3[0] == pytest.approx(s0, abs=1e-14)
    assert l3[2] == pytest.approx(s1 + math.log1p(math.exp(s0 - s1) + math.exp(-s1)), abs=1e-12)


@pytest.mark.parametrize("G,N", [(1, 40), (4, 97)])
def test_token_weights_from_lse_agree_with_token_weights(G, N):
    r = _rng(13)
    Q = r.standard_normal((G, N, 128)).astype(np.float16)
    K = r.standard_normal((N, 128)).astype(np.float16)
    lse = np.stack([O.row_lse(Q[g], K, block=16) for g in range(G)])
    w = O.token_weights_from_lse(Q, K, lse, block=32)
    np.testing.assert_allclose(w, O.token_weights(Q, K, block=16), rtol=1e-12, atol=1e-14)
    assert w.sum() == pytest.approx(G * N, rel=1e-12)
    # a wrong normaliser scales each row's mass: LSE + ln 2 halves every weight
    np.testing.assert_allclose(O.token_weights_from_lse(Q, K, lse + math.log(2.0)), w / 2, rtol=1e-12)


def test_token_weights_sum_to_number_of_query_rows():
    r = _rng(2)
    G, N = 4, 300
    Q = r.standard_normal((G, N, 128)).astype(np.float16)
    K = r.standard_normal((N, 128)).astype(np.float16)
    K[:10, 0] = 60  # strong heavy hitters
    w = O.token_weights(Q, K, block=64)
    assert abs(w.sum() - G * N) < 1e-9 * G * N
    assert np.all(w > 0)


def test_token_weights_uniform_attention_harmonic_closed_form():
    # Q = 0: every row attends uniformly to its tau + 1 visible tokens, so
    # w_t = G * (H_N - H_t) with H_n the n-th harmonic number (t 0-indexed).
    G, N = 3, 257
    Q = np.zeros((G, N, 128), np.float16)
    K = _rng(3).standard_normal((N, 128)).astype(np.float16)
    w = O.token_weights(Q, K, block=100)
    H = [Fraction(0)]
    for i in range(1, N + 1):
        H.append(H[-1] + Fraction(1, i))
    ref = np.array([float(G * (H[N] - H[t])) for t in range(N)])
    np.testing.assert_allclose(w, ref, rtol=1e-13)
    # first token sees every row, last token only its own
    assert w[0] > w[1] > w[-1]


def test_token_weight_is_total_variation_of_eviction():
    # The page defines w_t as the total-variation distance of the attention
    # distribution after evicting t.  Brute force: for every row, remove t,
    # renormalise, measure TV; a row whose only visible token is t goes to the
    # empty distribution (TV 1).
    G, N = 2, 9
    r = _rng(4)
    Q = r.standard_normal((G, N, 128)).astype(np.float16)
    K = r.standard_normal((N, 128)).astype(np.float16)
    A = _attention_matrix_sdpa(Q, K)
    w = O.token_weights(Q, K)
    for t in range(N):
        tv = 0.0
        for g in range(G):
            for tau in range(N):
                p = A[g, tau, : tau + 1]
                if t > tau:
                    continue
                rest = np.delete(np.arange(tau + 1), t)
                if rest.size == 0:
                    tv += 1.0
                    continue
                pe = np.zeros(tau + 1)
                pe[rest] = p[rest] / p[rest].sum()
                tv += 0.5 * np.abs(p - pe).sum()
        assert abs(tv - w[t]) < 1e-12


def test_channel_weight_is_spectral_norm_of_logit_deviation():
    # Zeroing channel c changes the logits of the group by the rank-1 matrix
    # Q_{:,c} K_{:,c}^T / sqrt(d); its spectral norm is w_c.
    G, N = 4, 40
    r = _rng(5)
    Q = r.standard_normal((G, N, 128)).astype(np.float16)
    K = (r.standard_normal((N, 128)) * np.linspace(0.1, 3, 128)).astype(np.float16)
    w = O.channel_weights(Q, K)
    Qs = Q.astype(np.float64).reshape(G * N, 128)
    K64 = K.astype(np.float64)
    for c in [0, 1, 63, 127]:
        Qz, Kz = Qs.copy(), K64.copy()
        Qz[:, c] = 0
        dev = Qs @ K64.T / math.sqrt(128) - Qz @ K64.T / math.sqrt(128)
        assert abs(np.linalg.norm(dev, 2) - w[c]) < 1e-10 * w[c]
        Kz[:, c] = 0
        dev2 = Qs @ K64.T / math.sqrt(128) - Qs @ Kz.T / math.sqrt(128)
        assert abs(np.linalg.norm(dev2, 2) - w[c]) < 1e-10 * w[c]


def test_token_variance_matches_pvariance():
    V = _rng(6).standard_normal((5, 128)).astype(np.float16)
    got = O.token_variance(V)
    for t in range(5):
        ref = statistics.pvariance([Fraction(float(x)) for x in V[t]])
        assert abs(got[t] - float(ref)) < 1e-14


# ---------------------------------------------------------------- exact variance and rounding

def test_round_rational_to_f32_matches_numpy_away_from_ties():
    r = _rng(7)
    for _ in range(2000):
        num = int(r.integers(1, 1 << 62))
        den = int(r.integers(1, 1 << 40))
        got = O.round_rational_to_f32(num, den)
        assert got == np.float32(num / den) or abs(float(got) - num / den) <= abs(float(np.float32(num / den)) - num / den)
        # the result is the nearest fp32: neither neighbour is closer
        exact = Fraction(num, den)
        lo = np.nextafter(got, np.float32(0))
        hi = np.nextafter(got, np.float32(np.inf))
        d0 = abs(Fraction(float(got)) - exact)
        assert d0 <= abs(Fraction(float(lo)) - exact) and d0 <= abs(Fraction(float(hi)) - exact)


def test_round_rational_to_f32_ties_to_even():
    one = Fraction(1)
    ulp = Fraction(1, 1 << 23)
    # 1 + ulp/2 is a tie between 1 (even) and 1 + ulp (odd) -> 1
    t = one + ulp / 2
    assert O.round_rational_to_f32(t.numerator, t.denominator) == np.float32(1.0)
    # 1 + 3ulp/2 is a tie between 1 + ulp (odd) and 1 + 2ulp (even) -> 1 + 2ulp
    t = one + 3 * ulp / 2
    assert O.round_rational_to_f32(t.numerator, t.denominator) == np.float32(1 + 2 * 2.0 ** -23)
    # just above the tie rounds up
    t = one + ulp / 2 + Fraction(1, 1 << 60)
    assert O.round_rational_to_f32(t.numerator, t.denominator) == np.float32(1 + 2.0 ** -23)


def test_exact_variance_matches_statistics_pvariance():
    r = _rng(8)
    for n in [1, 2, 5, 64, 301]:
        x = (r.standard_normal(n) * r.choice([1e-3, 1, 300])).astype(np.float16)
        ref = statistics.pvariance([Fraction(float(v)) for v in x])
        assert O.exact_population_variance(x) == ref
    assert O.exact_population_variance(np.zeros(0, np.float16)) == 0
    assert O.exact_population_variance(np.full(7, 3.5, np.float16)) == 0


def test_masked_channel_variance_uses_kept_tokens_only():
    r = _rng(9)
    K = r.standard_normal((50, 128)).astype(np.float16)
    bits = np.zeros(50, np.uint8)
    bits[[3, 7, 8, 20, 49]] = [2, 16, 4, 8, 2]
    got = O.masked_channel_variance(K, bits)
    for c in [0, 5, 127]:
        ref = statistics.pvariance([Fraction(float(v)) for v in K[[3, 7, 8, 20, 49], c]])
        assert got[c] == O.round_rational_to_f32(ref.numerator, ref.denominator)
    assert np.all(O.masked_channel_variance(K, np.zeros(50, np.uint8)) == 0)


# ---------------------------------------------------------------- allocation

BITS = (0, 2, 4, 8, 16)


def _lagrangian_value(c, b, lam):
    return Fraction(float(c)) * Fraction(1, 1 << b) + lam * b


def _exact_argmin_bits(c, lam):
    """Per-unit argmin of c 2^-b + lam b over {0,2,4,8,16}, ties to the lower b (exact)."""
    out = []
    for cu in c:
        vals = [_lagrangian_value(cu, b, lam) for b in BITS]
        out.append(BITS[min(range(5), key=lambda i: (vals[i], i))])
    return np.array(out)


def test_step_slopes_are_the_exact_hull_slopes():
    exact = [Fraction(3, 8), Fraction(3, 32), Fraction(15, 1024), Fraction(255, 524288)]
    assert [Fraction(float(s)) for s in O.STEP_SLOPE] == exact
    assert list(O.STEP_BITS) == [2, 2, 4, 8]


@pytest.mark.parametrize("seed", range(60))
def test_allocation_is_lagrangian_and_hull_optimal_bruteforce(seed):
    r = _rng(100 + seed)
    n = int(r.integers(1, 6))
    c = np.exp(r.standard_normal(n) * 2).astype(np.float32)
    if seed % 5 == 0:
        c[0] = c[-1]            # equal costs
    if seed % 7 == 0:
        c[0] = 0                # a zero-cost unit
    B = int(r.integers(0, 16 * n + 4))
    bits, lam = O.lagrangian_allocate(c, B)
    R = int(bits.sum())
    assert R <= B
    lamf = Fraction(lam)
    # (1) every unit is at the exact per-unit Lagrangian argmin for lambda*
    assert np.array_equal(bits, _exact_argmin_bits(c, lamf))
    # (2) lambda* is minimal: any smaller candidate multiplier overshoots B
    cands = sorted({Fraction(float(cu)) * Fraction(s) for cu in c for s in
                    (Fraction(3, 8), Fraction(3, 32), Fraction(15, 1024), Fraction(255, 524288))} | {Fraction(0)})
    smaller = [x for x in cands if x < lamf]
    if smaller:
        assert int(_exact_argmin_bits(c, smaller[-1]).sum()) > B
    # (3) hull optimality: no assignment with rate <= R has lower distortion
    dist = sum(Fraction(float(cu)) / (1 << int(b)) for cu, b in zip(c, bits))
    best = min(sum(Fraction(float(cu)) / (1 << b) for cu, b in zip(c, a))
               for a in itertools.product(BITS, repeat=n) if sum(a) <= R)
    assert dist == best


def test_group_allocation_of_one_segment_is_the_segment_allocation():
    r = _rng(31)
    N = 200
    w = np.exp(r.standard_normal(N)).astype(np.float32)
    v = (r.chisquare(128, N) / 128).astype(np.float32)
    wc = np.exp(r.standard_normal(128)).astype(np.float32)
    K = r.standard_normal((N, 128)).astype(np.float16)
    g = O.allocate_group([w], [v], [wc], [K], 700, 150)
    s = O.allocate_segment(w, v, wc, K, 700, 150)
    assert np.array_equal(g["bits_tok"][0], s["bits_tok"]) and np.array_equal(g["bits_chan"][0], s["bits_chan"])
    assert g["lambda_v"] == s["lambda_v"] and g["lambda_k"] == s["lambda_k"]
    assert np.array_equal(g["var_chan"][0].view(np.uint32), s["var_chan"].view(np.uint32))


def test_group_allocation_pools_the_budget():
    r = _rng(32)
    n, N, B = 3, 150, 900
    w = [np.exp(r.standard_normal(N) * (1 + i)).astype(np.float32) for i in range(n)]
    v = [(r.chisquare(128, N) / 128).astype(np.float32) for _ in range(n)]
    wc = [np.exp(r.standard_normal(128)).astype(np.float32) for _ in range(n)]
    K = [r.standard_normal((N, 128)).astype(np.float16) for _ in range(n)]
    g = O.allocate_group(w, v, wc, K, B, 300)
    assert int(g["bits_tok"].astype(np.int64).sum()) <= B
    assert int(g["bits_chan"].astype(np.int64).sum()) <= 300

    def distortion(bits, costs):
        return float(sum(np.sum(c.astype(np.float64) * 2.0 ** -b.astype(np.float64)) for b, c in zip(bits, costs)))
    costs = [O.unit_costs(w[i], v[i]) for i in range(n)]
    split = [O.lagrangian_allocate(costs[i], B // n)[0] for i in range(n)]
    # one multiplier over the pooled units is at least as good as any split of the budget
    assert distortion(g["bits_tok"], costs) <= distortion(split, costs) + 1e-9
    # the bits follow the weights: the segment with the heaviest tail gets the most
    per_seg = g["bits_tok"].astype(np.int64).sum(axis=1)
    assert per_seg[2] > per_seg[0]
    # a segment with all-zero weights gets nothing; the others share the whole budget
    w0 = [np.zeros(N, np.float32)] + w[1:]
    g0 = O.allocate_group(w0, v, wc, K, B, 300)
    assert g0["bits_tok"][0].sum() == 0
    assert np.array_equal(g0["bits_tok"][1:].reshape(-1),
                          O.lagrangian_allocate(np.concatenate(costs[1:]), B)[0])


def test_unit_cost_is_rounded_once_to_fp32():
    """c_u = fl32(w_u * sigma_u) with both factors fp32: the one rounding that
    makes lambda* and the bits unique.  w1*s1 = 1 + 2^-22 + 2^-46 rounds to
    1 + 2^-22 = w2*s2, so the two units tie and a 2-bit budget (one step for
    one unit) leaves both at 0 bits (ties stay at the lower bitwidth).  With
    an unrounded fp64 product the first unit would be strictly dearer and
    take the 2 bits alone."""
    e = np.float32(2.0 ** -23)
    w = np.array([1 + e, np.float32(1 + 2 * e)], np.float32)
    s = np.array([1 + e, 1.0], np.float32)
    c = O.unit_costs(w, s)
    assert c.dtype == np.float32
    assert c[0] == c[1] == np.float32(1 + 2.0 ** -22)
    assert Fraction(float(w[0])) * Fraction(float(s[0])) > Fraction(float(w[1])) * Fraction(float(s[1]))
    bits, lam = O.lagrangian_allocate(c, 2)
    assert list(bits) == [0, 0] and lam == float(c[0]) * 3 / 8
    # the same through the whole segment allocation (V problem)
    K = np.zeros((2, 128), np.float16)
    a = O.allocate_segment(w, s, np.ones(128, np.float32), K, 2, 0)
    assert list(a["bits_tok"]) == [0, 0]
    # and the rounding is to nearest, not truncation: a product just above a
    # half ulp rounds up
    x = np.float32(1 + 2.0 ** -12)
    y = np.float32(1 + 2.0 ** -12 + 2.0 ** -23)
    ex = Fraction(float(x)) * Fraction(float(y))          # 1 + 2^-11 + 2^-23 + 2^-24 + 2^-35
    assert O.unit_costs(np.array([x]), np.array([y]))[0] == np.float32(1 + 2.0 ** -11 + 2.0 ** -22)
    assert ex > Fraction(1) + Fraction(1, 2 ** 11) + Fraction(1, 2 ** 23) + Fraction(1, 2 ** 24)


def test_allocation_special_cases():
    c = np.array([1.0, 2.0, 0.5, 3.0], np.float32)
    assert list(O.lagrangian_allocate(c, 64)[0]) == [16] * 4          # budget covers all 16
    assert O.lagrangian_allocate(c, 64)[1] == 0.0
    assert list(O.lagrangian_allocate(c, 1)[0]) == [0] * 4            # below one 2-bit step
    assert list(O.lagrangian_allocate(c, 0)[0]) == [0] * 4
    z = np.array([0.0, 1.0, -2.0, np.nan], np.float32)
    assert list(O.lagrangian_allocate(z, 1000)[0]) == [0, 16, 0, 0]   # non-positive units evicted
    e = np.full(6, 1.7, np.float32)
    b, _ = O.lagrangian_allocate(e, 25)                               # equal costs, equal bits
    assert len(set(b.tolist())) == 1
    with pytest.raises(ValueError):
        O.lagrangian_allocate(c, -1)


def test_allocation_invariances():
    r = _rng(11)
    c = np.exp(r.standard_normal(500) * 1.5).astype(np.float32)
    prev = None
    for B in range(0, 4000, 97):
        b, lam = O.lagrangian_allocate(c, B)
        assert b.sum() <= B
        if prev is not None:
            assert np.all(b >= prev)                                   # monotone in the budget
        prev = b
        b2, lam2 = O.lagrangian_allocate(c * np.float32(8), B)         # exact power-of-two scaling
        assert np.array_equal(b, b2) and lam2 == 8 * lam
    b, _ = O.lagrangian_allocate(c, 1000)
    order = np.argsort(c)
    assert np.all(np.diff(b[order].astype(int)) >= 0)                  # monotone in the cost


def test_allocation_mixes_eviction_and_quantization():
    # the pages' central claim: the optimum mixes zero-bit and finite-bit units
    w = np.exp(_rng(12).standard_normal(2000) * 2).astype(np.float32)
    b, _ = O.lagrangian_allocate(w, 2 * 2000)
    assert {0, 2, 4}.issubset(set(b.tolist()))


# ---------------------------------------------------------------- quantizer

def test_quantize_hand_worked_examples():
    # scale = (2 - (-1)) / 3 = 1, zero = -1: (x - zero) = 0, 1, 1.5, 3
    q, s, z = O.quantize(np.array([-1, 0, 0.5, 2], np.float16), 2)
    assert list(q) == [0, 1, 2, 3] and s == 1 and z == -1        # 1.5 rounds to even 2
    q, s, z = O.quantize(np.array([0, 0.5, 2.5, 3], np.float16), 2)
    assert list(q) == [0, 0, 2, 3]                                  # 0.5 -> 0, 2.5 -> 2 (half-even)
    q, s, z = O.quantize(np.array([5, 5, 5], np.float16), 4)
    assert list(q) == [0, 0, 0] and s == 0 and z == 5               # zero range
    # 8 bits over [0, 255]: identity codes
    x = np.arange(256).astype(np.float16)
    q, s, z = O.quantize(x, 8)
    assert s == 1 and z == 0 and np.array_equal(q, np.arange(256))


@pytest.mark.parametrize("b", [2, 4, 8])
def test_quantize_properties(b):
    r = _rng(20 + b)
    X = (r.standard_normal((200, 37)) * r.choice([0.01, 1, 100], (200, 1))).astype(np.float16)
    q, s, z = O.quantize(X, b)
    assert q.max() <= (1 << b) - 1
    assert np.all(q[np.arange(200), X.argmin(axis=1)] == 0)           # min maps to 0
    assert np.all(z == X.min(axis=1))
    xr = O.dequantize(q, s[:, None], z[:, None]).astype(np.float64)
    err = np.abs(xr - X.astype(np.float64))
    top = (z.astype(np.float64) + s.astype(np.float64) * ((1 << b) - 1))[:, None]
    unclamped = X.astype(np.float64) <= top
    bound = s.astype(np.float64)[:, None] / 2 * (1 + 1e-6) + np.abs(X.astype(np.float64)) * 2 ** -22
    assert np.all(err[unclamped] <= bound[unclamped])


def test_dequantize_is_single_rounding_fma():
    r = _rng(30)
    q = r.integers(0, 256, 3000)
    s = (np.abs(r.standard_normal(3000)) * r.choice([1e-4, 1, 300], 3000)).astype(np.float16)
    z = (r.standard_normal(3000) * 50).astype(np.float16)
    got = O.dequantize(q, s, z)
    for i in range(0, 3000, 7):
        ex = Fraction(int(q[i])) * Fraction(float(s[i])) + Fraction(float(z[i]))
        if ex >= 0:
            ref = O.round_rational_to_f32(ex.numerator, ex.denominator) if ex else np.float32(0)
        else:
            ref = -O.round_rational_to_f32((-ex).numerator, (-ex).denominator)
        assert got[i] == ref


def test_oracle_decode_path_emits_no_numpy_deprecation_warnings():
    """Every shape the decode path hands to dequantize (one row, a column of
    per-row scales) stays on supported numpy idioms, so a numpy release that
    turns today's deprecations into errors cannot break the oracle."""
    import warnings
    r = _rng(33)
    with warnings.catch_warnings(record=True) as caught:
        warnings.simplefilter("always")
        for shape in [(1,), (1, 1), (5, 1), ()]:
            s = np.asarray(np.abs(r.standard_normal(shape)) + 0.1, np.float16)
            z = np.asarray(r.standard_normal(shape), np.float16)
            O.dequantize(r.integers(0, 4, shape[:1] + (3,) if shape else (3,)), s, z)
        lay = O.Layout(1, 1, 2, 1, 128, 20, 40, 64, 2)
        K, V = r.standard_normal((2, 20, 128)).astype(np.float16)
        bt = np.array([2] * 10 + [0] * 10, np.uint8)
        bc = np.array([2] * 32 + [0] * 96, np.uint8)
        blob = O.pack_cache(lay, K[None, None, None], V[None, None, None], bt[None, None, None], bc[None, None, None])
        O.decode_step(blob, lay, r.standard_normal((1, 1, 2, 128)).astype(np.float16), 0,
                      r.standard_normal((1, 1, 1, 128)).astype(np.float16),
                      r.standard_normal((1, 1, 1, 128)).astype(np.float16))
    dep = [w for w in caught if issubclass(w.category, DeprecationWarning)]
    assert not dep, [str(w.message) for w in dep]


def test_pack_codes_bit_order():
    assert O.pack_codes(np.array([1, 2, 3, 0]), 2)[0] == 1 | (2 << 2) | (3 << 4)
    assert O.pack_codes(np.array([0xA, 0x5] + [0] * 6 + [0xF]), 4).tolist() == [0x5A, 0xF]
    assert O.pack_codes(np.array([1, 2, 3, 4, 5]), 8).tolist() == [0x04030201, 5]
    r = _rng(31)
    for b in (2, 4, 8):
        c = r.integers(0, 1 << b, (3, 77))
        assert np.array_equal(O.unpack_codes(O.pack_codes(c, b), b, 77), c)


# ---------------------------------------------------------------- format, decode

def _layout(N, budget_v=None, budget_k=512, cap=16, S=1, L=1, Hq=4, Hkv=1):
    return O.Layout(S, L, Hq, Hkv, 128, N, budget_v if budget_v is not None else 16 * N, budget_k, cap)


def _sdpa(q, K, V):
    """softmax(q K^T/sqrt(d)) V via torch SDPA in fp64 on the CPU."""
    qt = torch.from_numpy(np.asarray(q, np.float64))[None, :, None, :]
    kt = torch.from_numpy(np.asarray(K, np.float64))[None, None].expand(1, q.shape[0], -1, -1)
    vt = torch.from_numpy(np.asarray(V, np.float64))[None, None].expand(1, q.shape[0], -1, -1)
    return torch.nn.functional.scaled_dot_product_attention(qt, kt.contiguous(), vt.contiguous())[0, :, 0].numpy()


def test_all_16_bit_cache_is_exact_attention_and_exact_bytes():
    N = 70
    r = _rng(40)
    K = r.standard_normal((N, 128)).astype(np.float16)
    V = r.standard_normal((N, 128)).astype(np.float16)
    lay = _layout(N, budget_k=2048)
    bt = np.full(N, 16, np.uint8)
    bc = np.full(128, 16, np.uint8)
    blob = O.pack_cache(lay, K[None, None, None], V[None, None, None], bt[None, None, None], bc[None, None, None])
    Kh, Vh, pos, tb = O.unpack_segment(blob, lay, 0)
    assert np.array_equal(pos, np.arange(N)) and np.all(tb == 16)
    assert np.array_equal(Kh, K.astype(np.float32)) and np.array_equal(Vh, V.astype(np.float32))
    # fp16 bytes verbatim: the V rows and the K records are the fp16 cache
    ds = O.read_descriptor(blob, lay, 0)
    assert blob[ds["off_v"][3]:ds["off_v"][3] + N * 256].tobytes() == V.tobytes()
    assert blob[ds["off_krec"]:ds["off_krec"] + N * 256].tobytes() == K.tobytes()
    assert O.segment_decode_bytes(blob, lay, 0, 0) == 2 * N * 128 * 2
    q = r.standard_normal((1, 1, 4, 128)).astype(np.float16)
    out = O.decode_step(blob, lay, q, 0)
    np.testing.assert_allclose(out[0, 0], _sdpa(q[0, 0], K, V), rtol=1e-12, atol=1e-13)


def test_eviction_only_cache_is_attention_over_kept_tokens():
    N = 90
    r = _rng(41)
    K = r.standard_normal((N, 128)).astype(np.float16)
    V = r.standard_normal((N, 128)).astype(np.float16)
    bt = np.where(r.random(N) < 0.4, 16, 0).astype(np.uint8)
    lay = _layout(N, budget_k=2048)
    blob = O.pack_cache(lay, K[None, None, None], V[None, None, None], bt[None, None, None],
                        np.full((1, 1, 1, 128), 16, np.uint8))
    q = r.standard_normal((1, 1, 4, 128)).astype(np.float16)
    out = O.decode_step(blob, lay, q, 0)
    keep = np.nonzero(bt)[0]
    np.testing.assert_allclose(out[0, 0], _sdpa(q[0, 0], K[keep], V[keep]), rtol=1e-12, atol=1e-13)


def test_zero_bit_channels_contribute_nothing():
    N = 40
    r = _rng(42)
    K = r.standard_normal((N, 128)).astype(np.float16)
    V = r.standard_normal((N, 128)).astype(np.float16)
    bc = np.where(np.arange(128) % 3 == 0, 0, 16).astype(np.uint8)
    lay = _layout(N, budget_k=2048)
    blob = O.pack_cache(lay, K[None, None, None], V[None, None, None], np.full((1, 1, 1, N), 16, np.uint8),
                        bc[None, None, None])
    Kh, _, _, _ = O.unpack_segment(blob, lay, 0)
    Kz = K.astype(np.float32) * (bc > 0)
    assert np.array_equal(Kh, Kz)
    q = r.standard_normal((1, 1, 4, 128)).astype(np.float16)
    np.testing.assert_allclose(O.decode_step(blob, lay, q, 0)[0, 0], _sdpa(q[0, 0], Kz, V), rtol=1e-12, atol=1e-13)


def test_mixed_pack_roundtrip_and_group_order():
    N = 200
    r = _rng(43)
    K = (r.standard_normal((N, 128)) * 3).astype(np.float16)
    V = r.standard_normal((N, 128)).astype(np.float16)
    bt = r.choice(np.array([0, 2, 4, 8, 16], np.uint8), N)
    bc = r.choice(np.array([0, 2, 4, 8, 16], np.uint8), 128)
    lay = _layout(N, budget_v=int(bt.sum()), budget_k=int(bc.sum()))
    blob = O.pack_cache(lay, K[None, None, None], V[None, None, None], bt[None, None, None], bc[None, None, None])
    Kh, Vh, pos, tb = O.unpack_segment(blob, lay, 0)
    # kept order: bitwidth 2, 4, 8, 16, ascending positions inside each group
    exp_pos = np.concatenate([np.nonzero(bt == b)[0] for b in (2, 4, 8, 16)])
    assert np.array_equal(pos, exp_pos) and np.array_equal(tb, bt[exp_pos])
    for i, t in enumerate(pos):
        b = int(bt[t])
        if b == 16:
            assert np.array_equal(Vh[i], V[t].astype(np.float32))
        else:
            qv, s, z = O.quantize(V[t], b)
            assert np.array_equal(Vh[i], O.dequantize(qv, s, z))
        for cb in (8, 4, 2):
            ch = np.nonzero(bc == cb)[0]
            qk, s, z = O.quantize(K[t, ch], cb)
            assert np.array_equal(Kh[i, ch], O.dequantize(qk, s, z))
        assert np.array_equal(Kh[i, bc == 16], K[t, bc == 16].astype(np.float32))
        assert np.all(Kh[i, bc == 0] == 0)
    assert O.segment_payload_bytes(blob, lay, 0) * 8 == 128 * int(bt.sum()) + len(pos) * int(bc.sum())
    # regions stay inside the slot and the slot inside the blob
    ds = O.read_descriptor(blob, lay, 0)
    assert ds["off_pos"] + 4 * len(pos) <= lay.slot_base(0) + lay.slot_bytes <= lay.cache_bytes


def test_zone_c_append_and_zone_c_only_attention():
    N = 30
    r = _rng(44)
    K = r.standard_normal((N, 128)).astype(np.float16)
    V = r.standard_normal((N, 128)).astype(np.float16)
    lay = _layout(N, cap=4)
    blob = O.pack_cache(lay, K[None, None, None], V[None, None, None], np.zeros((1, 1, 1, N), np.uint8),
                        np.zeros((1, 1, 1, 128), np.uint8))
    q = r.standard_normal((1, 1, 4, 128)).astype(np.float16)
    assert np.all(O.decode_step(blob, lay, q, 0) == 0)                 # nothing to attend to
    kn = r.standard_normal((3, 1, 1, 1, 128)).astype(np.float16)
    vn = r.standard_normal((3, 1, 1, 1, 128)).astype(np.float16)
    for step in range(3):
        out = O.decode_step(blob, lay, q, step, kn[step], vn[step])
        ref = _sdpa(q[0, 0], kn[:step + 1, 0, 0, 0], vn[:step + 1, 0, 0, 0])
        np.testing.assert_allclose(out[0, 0], ref, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(O.decode_step(blob, lay, q, 3)[0, 0], ref, rtol=1e-12, atol=1e-13)
    with pytest.raises(ValueError):
        O.decode_step(blob, lay, q, 4, kn[0], vn[0])


def test_layout_bounds_hold_at_the_budget_extremes():
    # a maximal allocation must fit its slot: all kept tokens at 2 bits, K bits
    # spread to maximise padding
    N = 64
    for bk in (0, 1, 2, 3, 7, 30, 81, 100, 256, 2048, 5000):
        lay = _layout(N, budget_v=2 * N, budget_k=bk)
        bits_c = np.zeros(128, np.uint8)
        left = min(bk, 2048)
        for b in (16, 8, 4, 2):            # one channel of each width first, most padding
            if left >= b and np.sum(bits_c == 0):
                bits_c[np.nonzero(bits_c == 0)[0][0]] = b
                left -= b
        for i in np.nonzero(bits_c == 0)[0]:
            if left >= 2:
                bits_c[i] = 2
                left -= 2
        w16, w8, w4, w2, nm = O.record_words([int(np.sum(bits_c == b)) for b in (16, 8, 4, 2)])
        assert 4 * (w16 + w8 + w4 + w2 + nm + 1) <= lay.rec_max


def test_empty_segment_with_channel_bits_packs_and_decodes():
    N = 20
    lay = _layout(N, budget_v=64, budget_k=64, cap=2)
    r = _rng(45)
    K = r.standard_normal((N, 128)).astype(np.float16)
    V = r.standard_normal((N, 128)).astype(np.float16)
    bc = np.zeros(128, np.uint8)
    bc[:3] = [8, 4, 2]
    blob = O.pack_cache(lay, K[None, None, None], V[None, None, None], np.zeros((1, 1, 1, N), np.uint8),
                        bc[None, None, None])
    ds = O.read_descriptor(blob, lay, 0)
    assert ds["n_kept"] == 0 and ds["n_chan"] == [0, 1, 1, 1] and ds["rec"] == 4 * (3 + 3 + 1)
    Kh, Vh, pos, tb = O.unpack_segment(blob, lay, 0)
    assert Kh.shape == (0, 128) and pos.size == 0
    q = r.standard_normal((1, 1, 4, 128)).astype(np.float16)
    assert np.all(O.decode_step(blob, lay, q, 0) == 0)
