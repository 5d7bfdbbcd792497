"""Statistical checks through the HIP path itself: the theorem of [Ch15]
15.1.2 (emitted tokens are distributed as p) by chi-square over 10^6
sequences, and the accepted-count distribution and E[N] for a constant
acceptance rate ([Ch15] 15.1.2, 15.1.3).
[Ch15] = "Chapter 15: Decoding acceleration techniques" (zsc.github.io)."""
import math

import numpy as np
import pytest
import scipy.stats
import torch

import oracle
import workloads as W

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import gpu_helpers as G
    import speculative_sampling_verification_05_amd as sv


def _run(inp, seed):
    wl = inp.wl
    tgt = G.to_device(inp.target, wl.dtype)
    dft = G.to_device(inp.draft, wl.dtype)
    tok = torch.from_numpy(inp.tokens).to("cuda:0")
    out_t, out_n = sv.verify(tgt, dft, tok, wl.T, seed)
    torch.cuda.synchronize()
    return out_t.cpu().numpy(), out_n.cpu().numpy()


@pytest.mark.parametrize("dt", [W.F32, W.BF16])
def test_theorem_chi_square_v16(dt):
    V, g, B = 16, 3, 1_000_000
    rng = np.random.default_rng(6)
    t_rows = rng.normal(0, 1.5, (g + 1, V))
    d_rows = t_rows[:g] + rng.normal(0, 1.0, (g, V))
    inp = W.repeated_rows_inputs(t_rows, d_rows, B, 0.9, seed=4, dtype=dt)
    tokens, n = _run(inp, 2024)
    assert (n >= 0).all()
    P = [oracle.row_softmax(inp.target[0, i], dt, 0.9)[1] for i in range(g + 1)]
    Q = [oracle.row_softmax(inp.draft[0, i], dt, 0.9)[1] for i in range(g)]
    for pos in range(g + 1):
        sel = n >= pos
        obs = np.bincount(tokens[sel, pos], minlength=V)
        assert scipy.stats.chisquare(obs, P[pos] * sel.sum()).pvalue > 1e-3, pos
    beta = [np.minimum(P[i], Q[i]).sum() for i in range(g)]
    pmf = [np.prod(beta[:k]) * (1 - beta[k]) for k in range(g)] + [np.prod(beta)]
    assert scipy.stats.chisquare(np.bincount(n, minlength=g + 1), np.array(pmf) * B).pvalue > 1e-3


@pytest.mark.parametrize("alpha,gamma", [(0.5, 4), (0.7, 8), (0.9, 8), (0.8, 1)])
def test_expected_accepted_count(alpha, gamma):
    B = 1_000_000
    p = np.array([alpha / 2, 1 - alpha / 2])
    q = np.array([1 - alpha / 2, alpha / 2])
    inp = W.repeated_rows_inputs(np.tile(np.log(p), (gamma + 1, 1)), np.tile(np.log(q), (gamma, 1)),
                                 B, 1.0, seed=gamma + 100)
    _, n = _run(inp, 99)
    pmf = np.array([alpha**k * (1 - alpha) for k in range(gamma)] + [alpha**gamma])
    ks = np.arange(gamma + 1)
    mean = alpha * (1 - alpha**gamma) / (1 - alpha)
    sd = math.sqrt(((ks - mean) ** 2 * pmf).sum() / B)
    assert abs(n.mean() - mean) < 5 * sd
    assert scipy.stats.chisquare(np.bincount(n, minlength=gamma + 1), pmf * B).pvalue > 1e-3
