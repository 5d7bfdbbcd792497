"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Pages are cited by title and section:
  [Ch15] "Chapter 15: Decoding acceleration techniques" (zsc.github.io), 15.1.2
         (steps 2-4, Lemma 1, main theorem, distribution of the accepted count N,
         E[N] for a constant acceptance rate), 15.1.3 (geometric form of E[N]),
         exercises (basic exercise 2 vectors).
  [CSDN] devpress.csdn.net speculative-inference post, 2.1 (speculative_decode()).
  [HSD]  "LLM inference optimisation: hidden-state speculative decoding", 3.3 (bonus token).
None of these tests touches the GPU or the HIP library.
"""
import json
import math
import os
import subprocess
from fractions import Fraction

import numpy as np
import pytest
import scipy.special
import scipy.stats
import torch

import oracle
import workloads as W

HERE = os.path.dirname(os.path.abspath(__file__))


# ---------------------------------------------------------------------------
# Philox4x32-10
# ---------------------------------------------------------------------------
@pytest.fixture(scope="module")
def aten_philox(tmp_path_factory):
    """ATen's header-only Philox engine, compiled test-only (independent code)."""
    inc = os.path.join(os.path.dirname(torch.__file__), "include")
    exe = str(tmp_path_factory.mktemp("philox") / "aten_philox")
    src = os.path.join(HERE, "aten_philox_dump.cpp")
    subprocess.run(["g++", "-O1", "-std=c++17", "-I", inc, src, "-o", exe], check=True)
    return exe


def test_philox_matches_aten_engine(aten_philox):
    rng = np.random.default_rng(11)
    cases = [(0, 0, 0, 0, 0, 0), (0xFFFFFFFF, 0xFFFFFFFF, 0xFFFFFFFF, 0xFFFFFFFF, 0xFFFFFFFF, 0xFFFFFFFF)]
    for _ in range(300):
        k = rng.integers(0, 2**32, size=2)
        c = rng.integers(0, 2**32, size=4)
        cases.append((*k, *c))
    for b in range(8):                      # the counters the verifier uses: (b, i, purpose, 0)
        for i in range(9):
            for pu in (0, 1):
                cases.append((12345, 0, b, i, pu, 0))
    inp = "\n".join(" ".join(str(int(v)) for v in c) for c in cases) + "\n"
    out = subprocess.run([aten_philox], input=inp, capture_output=True, text=True, check=True).stdout
    ref = [tuple(int(x) for x in line.split()) for line in out.strip().splitlines()]
    assert len(ref) == len(cases)
    for c, r in zip(cases, ref):
        got = tuple(int(x) for x in oracle.philox(c[2:], c[:2]))
        assert got == r, (c, got, r)


def test_uniform_is_53_bit_from_words_x0_x1():
    # U53 = ((x1 << 32 | x0) >> 11) * 2^-53 over Philox words (counter (b, i, purpose, 0), key = seed)
    for seed in (0, 1, 0xDEADBEEFCAFEF00D):
        for (b, i, pu) in [(0, 0, 0), (3, 7, 1), (1000, 62, 0)]:
            x = oracle.philox([b, i, pu, 0], [seed & 0xFFFFFFFF, seed >> 32])
            bits = ((int(x[1]) << 32) | int(x[0])) >> 11
            u = oracle.uniform(seed, b, i, pu)
            assert u == bits / 2.0**53
            assert 0.0 <= u < 1.0


def test_uniform_chi_square():
    n = 1_000_000
    b = np.arange(n, dtype=np.uint32)
    u = oracle.uniforms(7, b, 3, 0)
    assert (u >= 0).all() and (u < 1).all()
    assert np.all(u * 2.0**53 == np.floor(u * 2.0**53))
    counts = np.bincount(np.minimum((u * 1000).astype(np.int64), 999), minlength=1000)
    assert scipy.stats.chisquare(counts).pvalue > 1e-3
    # distinct purposes and positions give unrelated streams
    u2 = oracle.uniforms(7, b, 3, 1)
    assert abs(np.corrcoef(u, u2)[0, 1]) < 5e-3


# ---------------------------------------------------------------------------
# Softmax statistics ([Ch15] 15.1.2 step 2; [CSDN] 2.1)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", [W.F32, W.BF16])
@pytest.mark.parametrize("T", [0.3, 0.8, 1.0, 2.5])
def test_softmax_matches_library(dtype, T):
    rng = np.random.default_rng(int(T * 100) + dtype)
    for V in (1, 7, 1000, 4099):
        l64 = rng.normal(0, 3, V) - 1.1 * np.log(rng.permutation(V) + 1)
        if V > 10:
            l64[rng.choice(V, 5, replace=False)] = -np.inf
        row = W.to_storage(l64, dtype)
        lw = W.storage_to_f64(row, dtype)
        ok, p, m, S = oracle.row_softmax(row, dtype, T)
        assert ok
        assert m == lw.max()
        ref = torch.softmax(torch.from_numpy(lw) / T, dim=0).numpy()
        np.testing.assert_allclose(p, ref, rtol=1e-13, atol=1e-300)
        lse = scipy.special.logsumexp(lw / T)
        assert abs(S - math.exp(lse - m / T)) <= 1e-13 * S


def test_softmax_unusable_rows():
    for bad in ([0.0, np.nan, 1.0], [0.0, np.inf, 1.0], [-np.inf, -np.inf]):
        row = np.array(bad, np.float32)
        ok, _, _, S = oracle.row_softmax(row, W.F32, 1.0)
        assert not ok and math.isnan(S)
    ok, p, m, S = oracle.row_softmax(np.array([-np.inf, 2.0, -np.inf], np.float32), W.F32, 1.0)
    assert ok and m == 2.0 and S == 1.0 and list(p) == [0.0, 1.0, 0.0]


# ---------------------------------------------------------------------------
# Lemma 1 ([Ch15] 15.1.2): sum min(p, q) + sum max(0, p - q) = 1
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("name", ["tiny_b1_g4_v1000_f32", "zipf_b8_g5_v32000_f32", W.HEADLINE])
def test_lemma1_on_workload_rows(name):
    wl = W.WORKLOADS[name]
    if wl.B > 8:
        wl = wl.scaled(B=2)
    inp = W.make_inputs(wl, 0)
    for b in range(wl.B):
        for i in range(wl.gamma):
            _, p, _, _ = oracle.row_softmax(inp.target[b, i], wl.dtype, wl.T)
            _, q, _, _ = oracle.row_softmax(inp.draft[b, i], wl.dtype, wl.T)
            s = np.minimum(p, q).sum() + np.maximum(0.0, p - q).sum()
            assert abs(s - 1.0) < 1e-12


# ---------------------------------------------------------------------------
# Worked example: exercise 2 vectors of [Ch15]
# ---------------------------------------------------------------------------
def test_worked_example_exercise2():
    g = json.load(open(os.path.join(HERE, "golden", "ex2_worked_vectors.json")))
    p, q = np.array(g["p"]), np.array(g["q"])
    lp, lq = W.log_probs(p), W.log_probs(q)
    t_row, d_row = lp.astype(np.float32), lq.astype(np.float32)
    # softmax of fp32 log-probabilities reproduces p to fp32 rounding
    _, pp, _, _ = oracle.row_softmax(t_row, W.F32, 1.0)
    _, qq, _, _ = oracle.row_softmax(d_row, W.F32, 1.0)
    np.testing.assert_allclose(pp, p, rtol=1e-6)
    np.testing.assert_allclose(np.minimum(pp, qq).sum(), g["accept_mass_num"] / g["accept_mass_den"], rtol=1e-6)
    Z, cdf = oracle.residual_cdf(t_row, d_row, W.F32, 1.0)
    assert abs(Z - g["Z_num"] / g["Z_den"]) < 1e-6
    np.testing.assert_array_equal(np.diff(np.concatenate([[0.0], cdf])) > 0, np.array(g["residual_normalised"]) > 0)
    assert cdf[-1] == 1.0
    # through the verifier (gamma = 1): draft token 0 has alpha = 5/6
    alpha0 = g["alpha_num"][0] / g["alpha_den"][0]
    target = np.stack([t_row, t_row])[None]          # row 0 scores the draft token, row 1 = bonus row
    draft = d_row[None, None]
    for u, accepted in ((alpha0 - 1e-3, True), (alpha0 + 1e-3, False)):
        for us in (0.0, 0.3, 0.999):
            r = oracle.verify_u(target, draft, np.array([[0]]), W.F32, 1.0,
                                np.array([[u]]), np.array([[us, us]]))
            if accepted:
                assert r.n[0] == 1 and r.tokens[0, 0] == 0
            else:
                assert r.n[0] == 0 and r.tokens[0, 0] == 2 and r.tokens[0, 1] == -1
            assert abs(r.alpha[0, 0] - alpha0) < 1e-6
    # tokens 1 and 2 have alpha = 1 (token 1 up to the fp32 rounding of its logits)
    for tok, u in ((1, 0.999), (2, 1 - 2.0**-53)):
        r = oracle.verify_u(target, draft, np.array([[tok]]), W.F32, 1.0,
                            np.array([[u]]), np.array([[0.5, 0.5]]))
        assert r.n[0] == 1 and r.tokens[0, 0] == tok


# ---------------------------------------------------------------------------
# Main theorem by exact enumeration ([Ch15] 15.1.2 main theorem and its proof)
# ---------------------------------------------------------------------------
def _enumerate_exact(P, Q, T, G):
    """Run the oracle over every draft string (weighted by prod q_i) and every
    grid point of the uniforms (u_i = (g + 1/2)/G, shared correction uniform).
    Probabilities are rationals whose alphas and residual CDF points are
    multiples of 1/G, so grid counts are exact. Returns the exact output
    distribution at each position (conditional on reaching it) and P(N = k)."""
    g1, V = len(P), len(P[0])
    g = g1 - 1
    Pf = [np.array([float(x) for x in row]) for row in P]
    Qf = [np.array([float(x) for x in row]) for row in Q]
    t_row = np.stack([T * W.log_probs(r) for r in Pf])
    d_row = np.stack([T * W.log_probs(r) for r in Qf])
    grid = (np.arange(G) + 0.5) / G
    strings = np.array(np.meshgrid(*[np.arange(V)] * g, indexing="ij")).reshape(g, -1).T
    ugrid = np.array(np.meshgrid(*[grid] * (g + 1), indexing="ij")).reshape(g + 1, -1).T
    S, U = len(strings), len(ugrid)
    tokens = np.repeat(strings, U, axis=0).astype(np.int32)
    ua = np.tile(ugrid[:, :g], (S, 1))
    us = np.repeat(np.tile(ugrid[:, g:], (S, 1)), g + 1, axis=1)
    B = S * U
    target = np.broadcast_to(t_row, (B, g1, V)).astype(np.float64)
    draft = np.broadcast_to(d_row, (B, g, V)).astype(np.float64)
    # fp64 logits are not a storage type: feed fp32 (log-probabilities of
    # small rationals lose < 1e-7 relative, far inside the 1/(2G) grid margin)
    r = oracle.verify_u(target.astype(np.float32), draft.astype(np.float32), tokens, W.F32, T, ua, us)
    w_string = [math.prod(Q[i][s[i]] for i in range(g)) for s in strings]
    dist = [[Fraction(0)] * V for _ in range(g1)]
    reach = [Fraction(0)] * g1
    pmf = [Fraction(0)] * g1
    unit = Fraction(1, U)
    for si in range(S):
        w = w_string[si] * unit
        if w == 0:
            continue
        n = r.n[si * U:(si + 1) * U]
        out = r.tokens[si * U:(si + 1) * U]
        for k in range(g1):
            pmf[k] += w * int((n == k).sum())
        for pos in range(g1):
            sel = n >= pos
            cnt = int(sel.sum())
            if cnt == 0:
                continue
            reach[pos] += w * cnt
            vals, c = np.unique(out[sel, pos], return_counts=True)
            for v, cc in zip(vals, c):
                assert 0 <= v < V
                dist[pos][v] += w * int(cc)
    cond = [[d / reach[pos] if reach[pos] else None for d in dist[pos]] for pos in range(g1)]
    return cond, pmf


@pytest.mark.parametrize("T", [1.0, 0.5])
def test_theorem_exact_enumeration_v4(T):
    F = Fraction
    # rows with a zero-probability token on each side; alphas and residual CDFs are multiples of 1/12
    P = [[F(1, 2), F(1, 4), F(1, 4), F(0)],
         [F(1, 3), F(1, 3), F(1, 6), F(1, 6)],
         [F(1, 4), F(1, 4), F(1, 4), F(1, 4)]]
    Q = [[F(1, 4), F(1, 2), F(1, 6), F(1, 12)],
         [F(1, 6), F(1, 2), F(1, 3), F(0)]]
    cond, pmf = _enumerate_exact(P, Q, T, 12)
    for pos in range(3):
        assert cond[pos] == P[pos], (pos, cond[pos])
    beta = [sum(min(a, b) for a, b in zip(P[i], Q[i])) for i in range(2)]
    # P(N = k) = prod_{i<=k} beta_i * (1 - beta_{k+1}),  P(N = gamma) = prod beta_i
    assert pmf == [1 - beta[0], beta[0] * (1 - beta[1]), beta[0] * beta[1]]


def test_residual_sampler_grid_mass():
    """The correction draw gives each token exactly r_j / Z of the uniform's range."""
    F = Fraction
    p = [F(3, 10), F(1, 5), F(1, 10), F(2, 5), F(0)]
    q = [F(1, 10), F(2, 5), F(0), F(3, 10), F(1, 5)]
    r = [max(F(0), a - b) for a, b in zip(p, q)]
    Z = sum(r)
    G = 200
    t = np.tile(W.log_probs([float(x) for x in p]).astype(np.float32), (2, 1))
    d = W.log_probs([float(x) for x in q]).astype(np.float32)[None]
    B = G
    u_s = (np.arange(G) + 0.5) / G
    res = oracle.verify_u(np.broadcast_to(t, (B, 2, 5)).copy(), np.broadcast_to(d, (B, 1, 5)).copy(),
                          np.full((B, 1), 1, np.int32), W.F32, 1.0,
                          np.full((B, 1), 0.99), np.stack([u_s, u_s], 1))
    assert (res.n == 0).all()          # token 1: alpha = 1/2 < 0.99 -> rejected
    counts = np.bincount(res.tokens[:, 0], minlength=5)
    assert [F(int(c), G) for c in counts] == [x / Z for x in r]


# ---------------------------------------------------------------------------
# Main theorem by chi-square through the whole oracle (Philox uniforms)
# ---------------------------------------------------------------------------
def test_theorem_chi_square_v16():
    V, g, B = 16, 3, 1_000_000
    rng = np.random.default_rng(5)
    t_rows = rng.normal(0, 1.5, (g + 1, V))
    d_rows = t_rows[:g] + rng.normal(0, 1.0, (g, V))
    inp = W.repeated_rows_inputs(t_rows, d_rows, B, 1.0, seed=3)
    res = oracle.verify(inp.target, inp.draft, inp.tokens, W.F32, 1.0, seed=99, diag=False)
    P = [oracle.row_softmax(inp.target[0, i], W.F32, 1.0)[1] for i in range(g + 1)]
    Q = [oracle.row_softmax(inp.draft[0, i], W.F32, 1.0)[1] for i in range(g)]
    for pos in range(g + 1):
        sel = res.n >= pos
        obs = np.bincount(res.tokens[sel, pos], minlength=V)
        exp = P[pos] * sel.sum()
        assert scipy.stats.chisquare(obs, exp).pvalue > 1e-3, pos
    beta = [np.minimum(P[i], Q[i]).sum() for i in range(g)]
    pmf = [np.prod(beta[:k]) * (1 - beta[k]) for k in range(g)] + [np.prod(beta)]
    obs = np.bincount(res.n, minlength=g + 1)
    assert scipy.stats.chisquare(obs, np.array(pmf) * B).pvalue > 1e-3


# ---------------------------------------------------------------------------
# E[N] for a constant acceptance rate ([Ch15] 15.1.2 sum form, 15.1.3 geometric form)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("alpha", [0.5, 0.7, 0.9])
@pytest.mark.parametrize("gamma", [1, 4, 8])
def test_expected_accepted_count(alpha, gamma):
    B = 1_000_000
    p = np.array([alpha / 2, 1 - alpha / 2])
    q = np.array([1 - alpha / 2, alpha / 2])          # sum min(p, q) = alpha
    t_rows = np.tile(np.log(p), (gamma + 1, 1))
    d_rows = np.tile(np.log(q), (gamma, 1))
    inp = W.repeated_rows_inputs(t_rows, d_rows, B, 1.0, seed=gamma * 10 + int(alpha * 10))
    res = oracle.verify(inp.target, inp.draft, inp.tokens, W.F32, 1.0, seed=17, diag=False)
    n = res.n.astype(np.float64)
    pmf = np.array([alpha**k * (1 - alpha) for k in range(gamma)] + [alpha**gamma])
    ks = np.arange(gamma + 1)
    mean = (ks * pmf).sum()
    # the two forms the pages give for the i.i.d. case agree with the PMF
    assert abs(mean - alpha * (1 - alpha**gamma) / (1 - alpha)) < 1e-12
    sd = math.sqrt(((ks - mean) ** 2 * pmf).sum() / B)
    assert abs(n.mean() - mean) < 5 * sd
    obs = np.bincount(res.n, minlength=gamma + 1)
    assert scipy.stats.chisquare(obs, pmf * B).pvalue > 1e-3
    # tokens emitted per call: E[N] + 1 = (1 - alpha^(gamma+1)) / (1 - alpha)
    assert abs((n + 1).mean() - (1 - alpha ** (gamma + 1)) / (1 - alpha)) < 5 * sd


def test_printed_closed_form_is_not_expected_count():
    """The 'closed form' printed after the generating-function step of [Ch15]
    15.1.2 equals sum_{k=0}^{gamma} k alpha^k, not E[N]; at alpha = 0.8, gamma = 4
    it exceeds gamma. E[N] is checked against the sum form and the geometric form."""
    a, g = Fraction(4, 5), 4
    printed = a * (1 - (g + 1) * a**g + g * a ** (g + 1)) / (1 - a) ** 2
    assert printed == sum(k * a**k for k in range(g + 1))
    assert printed > g
    en = sum(k * a**k * (1 - a) for k in range(g)) + g * a**g
    assert en == a * (1 - a**g) / (1 - a) == Fraction(2952, 1250)


# ---------------------------------------------------------------------------
# Special cases
# ---------------------------------------------------------------------------
def test_identical_models_accept_everything():
    inp = W.small_random_inputs(64, 5, 300, W.F32, 0.9, seed=1)
    draft = inp.target[:, :5].copy()
    for seed in range(5):
        r = oracle.verify(inp.target, draft, inp.tokens, W.F32, 0.9, seed=seed)
        assert (r.n == 5).all()
        np.testing.assert_array_equal(r.tokens[:, :5], inp.tokens)
        np.testing.assert_allclose(r.alpha, 1.0)


def test_masked_draft_token_is_rejected():
    inp = W.small_random_inputs(16, 4, 200, W.F32, 1.0, seed=2)
    tgt = inp.target.copy()
    for b in range(16):
        tgt[b, 2, inp.tokens[b, 2]] = -np.inf       # target gives the draft token zero mass
        tgt[b, 2, :10] = -np.inf
    r = oracle.verify(tgt, inp.draft, inp.tokens, W.F32, 1.0, seed=4)
    assert (r.n <= 2).all()
    for b in range(16):
        if r.n[b] == 2:
            assert r.alpha[b, 2] == 0.0
            assert r.tokens[b, 2] != inp.tokens[b, 2] and r.tokens[b, 2] >= 10


def test_single_token_vocabulary():
    B, g = 5, 6
    t = np.zeros((B, g + 1, 1), np.float32)
    d = np.full((B, g, 1), 3.0, np.float32)
    r = oracle.verify(t, d, np.zeros((B, g), np.int32), W.F32, 1.3, seed=0)
    assert (r.n == g).all() and (r.tokens == 0).all()


def _greedy_expected(t64, tokens):
    B, g1, V = t64.shape
    g = g1 - 1
    n = np.empty(B, np.int32)
    out = np.full((B, g1), -1, np.int32)
    a = np.argmax(t64, axis=2)                      # first index of the maximum
    for b in range(B):
        mism = np.nonzero(tokens[b] != a[b, :g])[0]
        k = int(mism[0]) if len(mism) else g
        n[b] = k
        out[b, :k] = tokens[b, :k]
        out[b, k] = a[b, k]
    return n, out


@pytest.mark.parametrize("dtype", [W.F32, W.BF16])
def test_greedy_matches_argmax(dtype):
    wl = W.WORKLOADS["greedy_b32_g8_v128256_f32"].scaled(B=6, V=5003, dtype=dtype)
    inp = W.make_inputs(wl, 3)
    t = inp.target.copy()
    t64 = W.storage_to_f64(t, dtype)
    # inject ties: duplicate each row maximum at a higher and a lower index
    for b in range(wl.B):
        for i in range(wl.gamma + 1):
            j = int(np.argmax(t64[b, i]))
            t[b, i, (j + 17) % wl.V] = t[b, i, j]
            if i % 2 == 0:
                t[b, i, (j + wl.V - 29) % wl.V] = t[b, i, j]
    t64 = W.storage_to_f64(t, dtype)
    r = oracle.verify(t, None, inp.tokens, dtype, 0.0)
    n, out = _greedy_expected(t64, inp.tokens)
    np.testing.assert_array_equal(r.n, n)
    np.testing.assert_array_equal(r.tokens, out)


def test_sampling_tends_to_greedy_as_T_goes_to_zero():
    rng = np.random.default_rng(8)
    B, g, V = 40, 4, 50
    t = rng.integers(-20, 20, (B, g + 1, V)).astype(np.float32)
    for b in range(B):
        for i in range(g + 1):
            t[b, i, rng.integers(0, V)] = 25.0       # unique maximum
    d = rng.integers(-20, 20, (B, g, V)).astype(np.float32)
    a = np.argmax(t, axis=2)
    tokens = np.where(rng.random((B, g)) < 0.7, a[:, :g], rng.integers(0, V, (B, g))).astype(np.int32)
    # at T = 1e-3 every target row is one-hot in fp64, so alpha is 0 or 1 and
    # the residual is one-hot on the argmax, for any draft distribution
    for dd in (d, t[:, :g].copy()):
        rs = oracle.verify(t, dd, tokens, W.F32, 1e-3, seed=12)
        rg = oracle.verify(t, None, tokens, W.F32, 0.0)
        np.testing.assert_array_equal(rs.n, rg.n)
        np.testing.assert_array_equal(rs.tokens, rg.tokens)


# ---------------------------------------------------------------------------
# Invalid inputs: reported in band as n = -1 when the loop reaches them
# ---------------------------------------------------------------------------
def test_invalid_inputs_positional_rule():
    inp = W.small_random_inputs(4, 4, 100, W.F32, 1.0, seed=6)
    base = oracle.verify(inp.target, inp.draft, inp.tokens, W.F32, 1.0, seed=0)
    # NaN / +inf / all -inf in target row 0 or in draft row 0: always reached
    for where, val in (("t", np.nan), ("t", np.inf), ("d", np.nan)):
        t, d = inp.target.copy(), inp.draft.copy()
        (t if where == "t" else d)[1, 0, 5] = val
        r = oracle.verify(t, d, inp.tokens, W.F32, 1.0, seed=0)
        assert r.n[1] == -1 and (r.tokens[1] == -1).all()
        np.testing.assert_array_equal(np.delete(r.n, 1), np.delete(base.n, 1))
    t = inp.target.copy(); t[2, 0, :] = -np.inf
    assert oracle.verify(t, inp.draft, inp.tokens, W.F32, 1.0, seed=0).n[2] == -1
    # out-of-range draft token at position 0
    tok = inp.tokens.copy(); tok[3, 0] = 100
    assert oracle.verify(inp.target, inp.draft, tok, W.F32, 1.0, seed=0).n[3] == -1
    tok[3, 0] = -1
    assert oracle.verify(inp.target, inp.draft, tok, W.F32, 1.0, seed=0).n[3] == -1
    # a bad row after the emitted position is never reached: no effect
    for b in range(4):
        k = base.n[b]
        if k < 3:
            t = inp.target.copy(); t[b, k + 1, 0] = np.nan
            tok = inp.tokens.copy(); tok[b, k + 1] = 10**6
            r = oracle.verify(t, inp.draft, tok, W.F32, 1.0, seed=0)
            assert r.n[b] == k and (r.tokens[b] == base.tokens[b]).all()


def test_bonus_row_checked_only_when_reached():
    inp = W.small_random_inputs(8, 3, 64, W.F32, 1.0, seed=9)
    d = inp.target[:, :3].copy()              # identical rows: always reaches the bonus
    t = inp.target.copy(); t[0, 3, 7] = np.nan
    r = oracle.verify(t, d, inp.tokens, W.F32, 1.0, seed=1)
    assert r.n[0] == -1 and (r.n[1:] == 3).all()
    r = oracle.verify(t, None, inp.tokens, W.F32, 0.0)
    a = np.argmax(inp.target[0, :3], axis=1)
    if (a == inp.tokens[0]).all():
        assert r.n[0] == -1


# ---------------------------------------------------------------------------
# Draft-side sampling ([Ch15] 15.1.2 step 1: each draft token is drawn from the
# draft distribution and its probability kept; [CSDN] 2.1 stage 1)
# ---------------------------------------------------------------------------
def _draft_u(seed, B, n, pos0=0, b_offset=0):
    b = np.repeat(np.arange(B, dtype=np.int64) + b_offset, n)
    t = np.tile(np.arange(n, dtype=np.int64) + pos0, B)
    return oracle.uniforms(seed, b.astype(np.uint32), t.astype(np.uint32), oracle.DRAFT).reshape(B, n)


@pytest.mark.parametrize("V", [1, 2, 3, 10, 1000, 4097])
def test_draft_uniform_row_is_floor_uV(V):
    # equal logits: p_j = 1/V, C_j = (j+1)/V, so the inverse CDF picks floor(u*V)
    B, n, seed = 40, 5, 99
    logits = np.full((B, n, V), 0.75, np.float32)
    r = oracle.draft_sample(logits, W.F32, 1.7, seed=seed, pos0=3, b_offset=11)
    u = _draft_u(seed, B, n, pos0=3, b_offset=11)
    want = np.floor(u * V).astype(np.int64)
    near = np.abs(u * V - np.round(u * V)) < 1e-9
    assert ((r.tokens == want) | near).all()
    np.testing.assert_allclose(r.q, 1.0 / V, rtol=1e-14)


@pytest.mark.parametrize("T", [0.4, 1.0, 2.3])
def test_draft_two_token_closed_form(T):
    # p_0 = 1 / (1 + exp((l_1 - l_0)/T)); the draw is token 0 exactly when u < p_0
    rng = np.random.default_rng(5)
    B, n, seed = 300, 4, 1234
    logits = rng.normal(0, 2, (B, n, 2)).astype(np.float32)
    r = oracle.draft_sample(logits, W.F32, T, seed=seed)
    u = _draft_u(seed, B, n)
    l = logits.astype(np.float64)
    p0 = 1.0 / (1.0 + np.exp((l[..., 1] - l[..., 0]) / T))
    clear = np.abs(u - p0) > 1e-12
    assert clear.sum() > 0.99 * B * n
    np.testing.assert_array_equal(r.tokens[clear], np.where(u < p0, 0, 1)[clear])
    np.testing.assert_allclose(r.q, np.where(r.tokens == 0, p0, 1.0 - p0), rtol=1e-12)


def test_draft_distribution_chi_square():
    # many draws of one row (distinct counters) against softmax(l/T) from scipy
    rng = np.random.default_rng(8)
    V, T = 16, 0.7
    row = rng.normal(0, 1.5, V).astype(np.float32)
    B, n = 25000, 8
    logits = np.broadcast_to(row, (B, n, V))
    r = oracle.draft_sample(logits, W.F32, T, seed=77)
    p = scipy.special.softmax(row.astype(np.float64) / T)
    counts = np.bincount(r.tokens.ravel(), minlength=V)
    assert scipy.stats.chisquare(counts, p * B * n).pvalue > 1e-3
    np.testing.assert_allclose(r.q.ravel(), p[r.tokens.ravel()], rtol=1e-12)


def test_draft_cdf_interval_holds_u():
    inp = W.small_random_inputs(6, 5, 3000, W.BF16, 0.9, seed=4)
    r = oracle.draft_sample(inp.draft, W.BF16, 0.9, seed=21, pos0=2, b_offset=7)
    u = _draft_u(21, 6, 5, pos0=2, b_offset=7)
    assert ((r.cdf_lo <= u) & (u < r.cdf_hi)).all()
    np.testing.assert_allclose(r.cdf_hi - r.cdf_lo, r.q, rtol=1e-9, atol=1e-15)


def test_draft_counters_split_across_calls():
    # positions pos0 + t and sequences b + b_offset name the counters: splitting
    # a call over positions or sequences changes nothing
    inp = W.small_random_inputs(6, 6, 500, W.F32, 1.0, seed=3)
    d = inp.draft
    whole = oracle.draft_sample(d, W.F32, 1.0, seed=5)
    left = oracle.draft_sample(d[:, :2], W.F32, 1.0, seed=5)
    right = oracle.draft_sample(d[:, 2:], W.F32, 1.0, seed=5, pos0=2)
    np.testing.assert_array_equal(whole.tokens, np.concatenate([left.tokens, right.tokens], axis=1))
    top = oracle.draft_sample(d[:4], W.F32, 1.0, seed=5)
    bot = oracle.draft_sample(d[4:], W.F32, 1.0, seed=5, b_offset=4)
    np.testing.assert_array_equal(whole.tokens, np.concatenate([top.tokens, bot.tokens], axis=0))
    assert len(np.unique(whole.tokens)) > 10


@pytest.mark.parametrize("dtype", [W.F32, W.BF16])
def test_draft_greedy_is_first_argmax(dtype):
    rng = np.random.default_rng(6)
    l64 = np.round(rng.normal(0, 1, (5, 3, 300)), 1)   # coarse values: many ties
    logits = W.to_storage(l64, dtype)
    r = oracle.draft_sample(logits, dtype, 0.0)
    np.testing.assert_array_equal(r.tokens, np.argmax(W.storage_to_f64(logits, dtype), axis=-1))
    assert (r.q == 1.0).all()


def test_draft_unusable_and_masked_rows():
    logits = np.zeros((1, 5, 6), np.float32)
    logits[0, 0, 2] = np.nan
    logits[0, 1, 4] = np.inf
    logits[0, 2, :] = -np.inf
    logits[0, 3, :] = -np.inf
    logits[0, 3, 5] = 1.0                                # one finite entry: always drawn, q = 1
    logits[0, 4, ::2] = -np.inf                          # masked entries are never drawn
    for T in (1.0, 0.0):
        r = oracle.draft_sample(logits, W.F32, T, seed=2)
        assert list(r.tokens[0, :3]) == [-1, -1, -1] and np.isnan(r.q[0, :3]).all()
        assert r.tokens[0, 3] == 5 and r.q[0, 3] == 1.0
        assert r.tokens[0, 4] % 2 == 1
    many = oracle.draft_sample(np.broadcast_to(logits[0, 4], (400, 1, 6)), W.F32, 1.0, seed=9)
    assert set(np.unique(many.tokens)) == {1, 3, 5}
    np.testing.assert_allclose(many.q, 1.0 / 3, rtol=1e-14)


# ---------------------------------------------------------------------------
# Diagnostics for the draft length ([Ch15] 15.1.4 dynamic strategy adjustment;
# 15.2.4 adaptive draft length from the prediction entropy; Lemma 1)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("V", [1, 2, 7, 1000])
def test_entropy_of_equal_logits_is_log_V(V):
    for T in (0.5, 1.0, 3.0):
        assert abs(oracle.row_entropy(np.full(V, -1.25, np.float32), W.F32, T) - math.log(V)) <= 1e-12 * max(1, math.log(V))


@pytest.mark.parametrize("dtype", [W.F32, W.BF16])
@pytest.mark.parametrize("T", [0.4, 1.0, 2.5])
def test_entropy_matches_scipy(dtype, T):
    rng = np.random.default_rng(int(T * 10) + dtype)
    for V in (2, 50, 3000):
        l64 = rng.normal(0, 3, V)
        if V > 10:
            l64[rng.choice(V, 4, replace=False)] = -np.inf
        row = W.to_storage(l64, dtype)
        p = scipy.special.softmax(W.storage_to_f64(row, dtype) / T)
        assert abs(oracle.row_entropy(row, dtype, T) - scipy.stats.entropy(p)) <= 1e-11


def test_entropy_special_rows():
    # two tokens: the binary entropy of p0 = 1 / (1 + e^((l1 - l0)/T))
    l0, l1, T = 0.3, -1.1, 0.7
    p0 = 1.0 / (1.0 + math.exp((float(np.float32(l1)) - float(np.float32(l0))) / T))
    want = -p0 * math.log(p0) - (1 - p0) * math.log(1 - p0)
    assert abs(oracle.row_entropy(np.array([l0, l1], np.float32), W.F32, T) - want) < 1e-14
    one = np.full(9, -np.inf, np.float32)
    one[4] = 2.0
    assert oracle.row_entropy(one, W.F32, 1.0) == 0.0
    assert oracle.row_entropy(np.array([1.0, 3.0, 3.0], np.float32), W.F32, 0.0) == 0.0
    for bad in ([0.0, np.nan], [np.inf, 0.0], [-np.inf, -np.inf]):
        for T in (1.0, 0.0):
            assert math.isnan(oracle.row_entropy(np.array(bad, np.float32), W.F32, T))


def test_expected_accept_worked_example():
    g = json.load(open(os.path.join(HERE, "golden", "ex2_worked_vectors.json")))
    t_row = W.log_probs(np.array(g["p"])).astype(np.float32)
    d_row = W.log_probs(np.array(g["q"])).astype(np.float32)
    beta = oracle.expected_accept(np.stack([t_row, t_row])[None], d_row[None, None], W.F32, 1.0)
    assert abs(beta[0, 0] - g["accept_mass_num"] / g["accept_mass_den"]) < 1e-6


def test_expected_accept_special_cases_and_lemma1():
    inp = W.small_random_inputs(3, 4, 500, W.F32, 1.0, seed=6)
    t = inp.target.copy()
    d = inp.draft.copy()
    d[0] = t[0, :4]                                  # identical rows: beta = 1
    t[1, 1, :250] = -np.inf                          # disjoint supports: beta = 0
    d[1, 1, 250:] = -np.inf
    t[2, 2, 7] = np.nan                              # unusable: NaN
    for T in (0.6, 1.0, 1.7):
        beta = oracle.expected_accept(t, d, W.F32, T)
        np.testing.assert_allclose(beta[0], 1.0, rtol=0, atol=1e-12)
        assert beta[1, 1] == 0.0
        assert math.isnan(beta[2, 2])
        for b, i in ((1, 0), (1, 3), (2, 0), (2, 3)):
            Z, _ = oracle.residual_cdf(t[b, i], d[b, i], W.F32, T)   # Lemma 1: sum min + sum max(0, p - q) = 1
            assert abs(beta[b, i] + Z - 1.0) < 1e-12
            p = scipy.special.softmax(t[b, i].astype(np.float64) / T)
            q = scipy.special.softmax(d[b, i].astype(np.float64) / T)
            assert abs(beta[b, i] - np.minimum(p, q).sum()) < 1e-12


# ---------------------------------------------------------------------------
# Token-tree verification, the labelled heuristic mode ([CSDN] 3.2
# TokenTreeVerifier.parallel_verify; [Ch15] 15.2.4)
# ---------------------------------------------------------------------------
def _hand_tree():
    # root (node 0) -> node 1 (token 1), node 2 (token 2); node 1 -> node 3 (token 3)
    p0, q0 = [0.1, 0.6, 0.2, 0.1], [0.3, 0.2, 0.4, 0.1]      # scores: node 1 min(1, .6/.2) = 1, node 2 .2/.4 = .5
    p1, q1 = [0.5, 0.25, 0.125, 0.125], [0.25] * 4           # node 3: .125/.25 = .5; argmax of p1 is token 0
    rows_t = np.stack([W.log_probs(p0), W.log_probs(p1), W.log_probs(p0), W.log_probs(p0)]).astype(np.float32)
    rows_d = np.stack([W.log_probs(q0), W.log_probs(q1), W.log_probs(q0), W.log_probs(q0)]).astype(np.float32)
    parent = np.array([[-1, 0, 0, 1]], np.int32)
    token = np.array([[-1, 1, 2, 3]], np.int32)
    return rows_t[None], rows_d[None], parent, token


@pytest.mark.parametrize("threshold,path", [(0.4, [1, 3]), (0.6, [1]), (1.0, [1]), (1.01, []), (0.0, [1, 3])])
def test_tree_hand_example(threshold, path):
    t, d, parent, token = _hand_tree()
    tok, nodes, n = oracle.tree_verify(t, d, parent, token, W.F32, 1.0, threshold)
    assert n[0] == len(path)
    assert list(nodes[0, :n[0]]) == path and (nodes[0, n[0]:] == -1).all()
    assert list(tok[0, :n[0]]) == [int(token[0, j]) for j in path]


def test_tree_hand_example_greedy_and_ties():
    t, d, parent, token = _hand_tree()
    tok, nodes, n = oracle.tree_verify(t, None, parent, token, W.F32, 0.0, 0.5)
    assert n[0] == 1 and nodes[0, 0] == 1                  # root argmax = token 1; node 1's argmax 0 is no child
    # two children with score 1: the first (lower index) is taken
    token2 = token.copy()
    token2[0, 2] = 3                                         # p0(3) = q0(3): score 1, like node 1
    tok, nodes, n = oracle.tree_verify(t, d, parent, token2, W.F32, 1.0, 0.9)
    assert nodes[0, 0] == 1
    parent2 = np.array([[-1, 0, 0, 0]], np.int32)            # three root children: tokens 2, 1, 1
    tok, nodes, n = oracle.tree_verify(t, d, parent2, np.array([[-1, 2, 1, 1]], np.int32), W.F32, 1.0, 0.9)
    assert nodes[0, 0] == 2 and n[0] == 1                    # scores .5, 1, 1 (exactly): node 2 first at 1


def test_tree_chain_equals_linear_verification():
    # a chain (one child per node) with threshold tau accepts exactly where the
    # linear rule with every accept uniform equal to tau does (alpha != tau)
    for seed, T in ((1, 1.0), (2, 0.7)):
        inp = W.small_random_inputs(40, 6, 300, W.F32, T, seed=seed)
        g = 6
        N = g + 1
        parent = np.tile(np.arange(-1, N - 1, dtype=np.int32), (40, 1))
        token = np.concatenate([np.full((40, 1), -1, np.int32), inp.tokens], axis=1)
        t = inp.target[:, :N]
        d = np.concatenate([inp.draft, inp.draft[:, -1:]], axis=1)   # row g has no child: unused
        for tau in (0.3, 0.8):
            tok, nodes, n = oracle.tree_verify(t, d, parent, token, W.F32, T, tau)
            lin = oracle.verify_u(inp.target, inp.draft, inp.tokens, W.F32, T, np.full((40, g), tau),
                                  np.full((40, g + 1), 0.5))
            assert (lin.alpha[np.isfinite(lin.alpha)] != tau).all()
            np.testing.assert_array_equal(n, lin.n)
            for b in range(40):
                assert list(tok[b, :n[b]]) == list(inp.tokens[b, :n[b]])
                assert list(nodes[b, :n[b]]) == list(range(1, n[b] + 1))


def test_tree_greedy_follows_argmax_and_zero_threshold_reaches_a_leaf():
    tr = W.tree_inputs(6, 3, 3, 40, W.BF16, 1.0, seed=4)
    t64 = W.storage_to_f64(tr.target, W.BF16)
    tok, nodes, n = oracle.tree_verify(tr.target, None, tr.parent, tr.token, W.BF16, 0.0, 0.5)
    for b in range(6):
        v, path = 0, []
        while True:
            kids = [c for c in range(1, tr.parent.shape[1]) if tr.parent[b, c] == v]
            a = int(np.argmax(t64[b, v]))
            hit = [c for c in kids if tr.token[b, c] == a]
            if not kids or not hit:
                break
            v = hit[0]
            path.append(v)
        assert list(nodes[b, :n[b]]) == path
    tok, nodes, n = oracle.tree_verify(tr.target, tr.draft, tr.parent, tr.token, W.BF16, 1.0, 0.0)
    assert (n == 3).all()


def test_tree_invalid_inputs():
    t, d, parent, token = _hand_tree()
    bad_parent = parent.copy()
    bad_parent[0, 2] = 2                                     # a parent must come before its child
    assert oracle.tree_verify(t, d, bad_parent, token, W.F32, 1.0, 0.4)[2][0] == -1
    bad_tok = token.copy()
    bad_tok[0, 3] = 4                                        # out of range, on the walk
    assert oracle.tree_verify(t, d, parent, bad_tok, W.F32, 1.0, 0.4)[2][0] == -1
    assert oracle.tree_verify(t, d, parent, bad_tok, W.F32, 1.0, 1.01)[2][0] == 0  # node 1's children never scored
    t2 = t.copy()
    t2[0, 1, 0] = np.nan                                     # node 1's row, on the walk
    assert oracle.tree_verify(t2, d, parent, token, W.F32, 1.0, 0.4)[2][0] == -1
    t3 = t.copy()
    t3[0, 2, 0] = np.nan                                     # node 2's row: never read
    assert oracle.tree_verify(t3, d, parent, token, W.F32, 1.0, 0.4)[2][0] == 2
