"""GPU parity of the draft-side sampler ([Ch15] 15.1.2 step 1; [CSDN] 2.1
stage 1) through the C ABI, against the fp64 oracle on the same seeded inputs.

Tolerances: tokens exact (T == 0 always; T > 0 except draws within 1e-6 of a
boundary of the oracle's CDF, pooled under 0.1% of draws, at least one allowed);
q relative 1e-5 (the fp32 exponentials against fp64); unusable rows -1 and NaN.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from oracle.compare import compare_draft

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import gpu_helpers as G
    import speculative_sampling_verification_05_amd as sv


def gpu_draft(logits, dtype, T, seed, pos0=0, b_offset=0, want_q=True):
    x = G.to_device(logits, dtype)
    print(f"draft_sample B={logits.shape[0]} n={logits.shape[1]} V={logits.shape[2]} dtype={dtype} T={T} "
          f"seed={seed} pos0={pos0} b_offset={b_offset}", flush=True)
    tok, q = sv.draft_sample(x, T, seed, pos0=pos0, b_offset=b_offset, want_q=want_q)
    torch.cuda.synchronize()
    return tok.cpu().numpy(), (q.cpu().numpy() if q is not None else None)


def check(logits, dtype, T, seed, pos0=0, b_offset=0):
    tok, q = gpu_draft(logits, dtype, T, seed, pos0, b_offset)
    orc = oracle.draft_sample(logits, dtype, T, seed=seed, pos0=pos0, b_offset=b_offset)
    rep = compare_draft(logits, dtype, T, orc, tok, q, seed, pos0, b_offset)
    print(rep)
    assert rep.ok(), str(rep) + " " + str(rep.hard_fail[:5])
    return tok, q, rep


# shapes spanning several ranges, blocks and a ragged last chunk; V * size not
# a multiple of 16 takes the scalar path
SHAPES = [
    (3, 4, 1000, W.F32), (5, 3, 3000, W.BF16), (2, 2, 1003, W.F32), (4, 2, 1001, W.BF16),
    (1, 1, 1, W.F32), (2, 3, 7, W.BF16), (3, 2, 40000, W.BF16), (2, 2, 70001, W.F32),
    (2, 1, 152064, W.BF16), (1, 2, 262144, W.F32),
    (1, 3, 131072, W.BF16), (1, 3, 131080, W.BF16),   # the largest one-block row, and the smallest split one
]


@pytest.mark.parametrize("B,n,V,dtype", SHAPES)
@pytest.mark.parametrize("T", [0.8, 1.0, 0.0])
def test_draft_shapes(B, n, V, dtype, T):
    inp = W.small_random_inputs(B, n, V, dtype, T if T > 0 else 1.0, seed=V % 97 + n)
    check(inp.draft, dtype, T, seed=V + 3, pos0=n, b_offset=B)


def test_draft_workload_rows_full_size():
    # every draft row of the 64 x 8 x 128256 bf16 workload, in the launch the benchmark times
    wl = W.WORKLOADS[W.HEADLINE]
    inp = W.make_inputs(wl, 0)
    tok, q, rep = check(inp.draft, wl.dtype, wl.T, seed=0)
    assert rep.draws == wl.B * wl.gamma


def test_draft_greedy_full_size():
    wl = W.WORKLOADS["greedy_b32_g8_v128256_f32"]
    inp = W.make_inputs(wl, 0)
    tok, q, _ = check(inp.target, wl.dtype, 0.0, seed=0)
    np.testing.assert_array_equal(tok, np.argmax(inp.target, axis=-1))


@pytest.mark.parametrize("dtype", [W.F32, W.BF16])
@pytest.mark.parametrize("T", [1.0, 0.0])
def test_draft_edge_rows(dtype, T):
    V = 5000
    rng = np.random.default_rng(3)
    l64 = rng.normal(0, 2, (2, 6, V))
    l64[0, 0, 4321] = np.nan
    l64[0, 1, 17] = np.inf
    l64[0, 2, :] = -np.inf
    l64[0, 3, :] = -np.inf
    l64[0, 3, V - 1] = 0.5                 # one finite entry, in the last (ragged) chunk
    l64[0, 4, ::2] = -np.inf               # masked half
    l64[0, 5, :] = 3.0                     # all ties
    l64[1, 0, :4096] = -np.inf             # mass only in the second range
    l64[1, 1, :] = -1e4                    # very negative but finite
    logits = W.to_storage(l64, dtype)
    tok, q, _ = check(logits, dtype, T, seed=5)
    assert list(tok[0, :3]) == [-1, -1, -1] and np.isnan(q[0, :3]).all()
    assert tok[0, 3] == V - 1 and q[0, 3] == 1.0
    assert tok[0, 4] % 2 == 1
    assert tok[1, 0] >= 4096
    if T == 0:
        assert tok[0, 5] == 0


def test_draft_split_calls_and_reuse():
    # splitting over positions or sequences gives the same tokens; calls of
    # other shapes, and a verification, in between leave nothing behind
    inp = W.small_random_inputs(6, 6, 30000, W.BF16, 1.0, seed=12)
    d = inp.draft
    whole, qw = gpu_draft(d, W.BF16, 1.0, seed=9)
    left, _ = gpu_draft(np.ascontiguousarray(d[:, :2]), W.BF16, 1.0, seed=9)
    vinp = W.small_random_inputs(5, 4, 3000, W.F32, 0.9, seed=2)
    G.run(vinp, seed=1)
    right, _ = gpu_draft(np.ascontiguousarray(d[:, 2:]), W.BF16, 1.0, seed=9, pos0=2)
    np.testing.assert_array_equal(whole, np.concatenate([left, right], axis=1))
    top, _ = gpu_draft(np.ascontiguousarray(d[:4]), W.BF16, 1.0, seed=9)
    bot, _ = gpu_draft(np.ascontiguousarray(d[4:]), W.BF16, 1.0, seed=9, b_offset=4)
    np.testing.assert_array_equal(whole, np.concatenate([top, bot], axis=0))
    again, qa = gpu_draft(d, W.BF16, 1.0, seed=9)
    np.testing.assert_array_equal(whole, again)
    np.testing.assert_array_equal(qw, qa)
    r = G.run(vinp, seed=1)
    o = oracle.verify(vinp.target, vinp.draft, vinp.tokens, W.F32, 0.9, seed=1)
    from oracle.compare import compare_tokens
    rep = compare_tokens(vinp, o, r.tokens, r.n, 1)
    assert rep.ok() and not rep.hard_fail, str(rep) + " " + str(rep.hard_fail[:5])


def test_draft_two_dim_input_and_no_q():
    inp = W.small_random_inputs(4, 1, 2048, W.F32, 1.0, seed=1)
    x = G.to_device(inp.draft[:, 0], W.F32)
    tok, q = sv.draft_sample(x, 1.0, 4, pos0=3, want_q=False)
    torch.cuda.synchronize()
    assert q is None and tuple(tok.shape) == (4,)
    orc = oracle.draft_sample(inp.draft, W.F32, 1.0, seed=4, pos0=3)
    rep = compare_draft(inp.draft, W.F32, 1.0, orc, tok.cpu().numpy()[:, None], None, 4, pos0=3)
    assert rep.ok(), str(rep) + " " + str(rep.hard_fail[:5])


@pytest.mark.parametrize("B,n,V,dtype", [(3, 4, 1000, W.F32), (2, 3, 40000, W.BF16), (2, 2, 1003, W.F32),
                                         (1, 2, 262144, W.F32), (2, 2, 128256, W.BF16)])
@pytest.mark.parametrize("T", [0.7, 1.3, 0.0])
def test_draft_entropy(B, n, V, dtype, T):
    # the entropy beside the draw ([Ch15] 15.2.4): the same tokens as without
    # it, and H within 1e-5 of the oracle's (absolute, plus 1e-5 relative)
    inp = W.small_random_inputs(B, n, V, dtype, 1.0, seed=V % 31 + n)
    l64 = W.storage_to_f64(inp.draft, dtype)
    l64[0, 0, : V // 2] = -np.inf                     # masked half
    logits = W.to_storage(l64, dtype)
    x = G.to_device(logits, dtype)
    tok, q, H = sv.draft_sample(x, T, 3, want_entropy=True)
    tok2, q2 = sv.draft_sample(x, T, 3)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(tok.cpu().numpy(), tok2.cpu().numpy())
    np.testing.assert_array_equal(q.cpu().numpy(), q2.cpu().numpy())
    want = oracle.entropies(logits, dtype, T)
    got = H.cpu().numpy()
    np.testing.assert_allclose(got, want, rtol=1e-5, atol=1e-5)


def test_draft_entropy_edge_rows():
    V = 3000
    l64 = np.random.default_rng(2).normal(0, 1, (1, 5, V))
    l64[0, 0, 5] = np.nan
    l64[0, 1, :] = -np.inf
    l64[0, 2, :] = -np.inf
    l64[0, 2, 2999] = 4.0                                # one token: H = 0
    l64[0, 3, :] = 0.25                                  # equal logits: H = ln V
    logits = W.to_storage(l64, W.BF16)
    for T in (1.0, 0.0):
        tok, q, H = sv.draft_sample(G.to_device(logits, W.BF16), T, 1, want_entropy=True)
        torch.cuda.synchronize()
        H = H.cpu().numpy()[0]
        assert np.isnan(H[0]) and np.isnan(H[1])
        assert abs(H[2]) < 1e-6
        assert abs(H[3] - (np.log(V) if T > 0 else 0.0)) < 1e-5



# ---------------------------------------------------------------------------
# Expected acceptance per position (Lemma 1): sum_x min(p_i(x), q_i(x))
# ---------------------------------------------------------------------------
def gpu_beta(target, draft, dtype, T):
    print(f"expected_accept B={target.shape[0]} gamma={draft.shape[1]} V={target.shape[2]} dtype={dtype} T={T}",
          flush=True)
    out = sv.expected_accept(G.to_device(target, dtype), G.to_device(draft, dtype), T)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("B,g,V,dtype", [(3, 4, 1000, W.F32), (2, 3, 40000, W.BF16), (2, 2, 1003, W.F32),
                                         (2, 2, 1001, W.BF16), (1, 1, 1, W.F32), (1, 2, 152064, W.BF16)])
@pytest.mark.parametrize("T", [0.6, 1.0, 1.8])
def test_expected_accept_shapes(B, g, V, dtype, T):
    inp = W.small_random_inputs(B, g, V, dtype, T, seed=V % 13 + g)
    got = gpu_beta(inp.target, inp.draft, dtype, T)
    want = oracle.expected_accept(inp.target, inp.draft, dtype, T)
    np.testing.assert_allclose(got, want, rtol=1e-5, atol=1e-6)


def test_expected_accept_edge_rows_and_workload():
    inp = W.small_random_inputs(3, 4, 5000, W.BF16, 1.0, seed=6)
    t, d = inp.target.copy(), inp.draft.copy()
    d[0] = t[0, :4]                                  # identical rows: 1
    t64 = W.storage_to_f64(t, W.BF16)
    d64 = W.storage_to_f64(d, W.BF16)
    t64[1, 1, :2500] = -np.inf                       # disjoint supports: 0
    d64[1, 1, 2500:] = -np.inf
    t64[2, 2, 77] = np.nan                           # unusable: NaN
    d64[2, 3, :] = -np.inf
    t, d = W.to_storage(t64, W.BF16), W.to_storage(d64, W.BF16)
    got = gpu_beta(t, d, W.BF16, 1.0)
    np.testing.assert_allclose(got[0], 1.0, atol=1e-6)
    assert got[1, 1] == 0.0
    assert np.isnan(got[2, 2]) and np.isnan(got[2, 3])
    want = oracle.expected_accept(t, d, W.BF16, 1.0)
    np.testing.assert_allclose(got, want, rtol=1e-5, atol=1e-6)
    # every position of the 64 x 8 x 128256 bf16 workload
    wl = W.WORKLOADS[W.HEADLINE]
    full = W.make_inputs(wl, 0)
    got = gpu_beta(full.target, full.draft, wl.dtype, wl.T)
    want = oracle.expected_accept(full.target, full.draft, wl.dtype, wl.T)
    np.testing.assert_allclose(got, want, rtol=1e-5, atol=1e-6)


def test_expected_accept_never_reads_the_bonus_rows():
    """beta needs target rows 0..gamma-1 only: NaN in every bonus row (row
    gamma of each sequence) leaves every beta finite and equal to the
    oracle's."""
    inp = W.small_random_inputs(5, 3, 3000, W.F32, 0.9, seed=12)
    t = inp.target.copy()
    t[:, -1, :] = np.nan
    got = gpu_beta(t, inp.draft, W.F32, 0.9)
    assert np.isfinite(got).all()
    np.testing.assert_allclose(got, oracle.expected_accept(inp.target, inp.draft, W.F32, 0.9), rtol=1e-5, atol=1e-6)


def test_expected_accept_alternating_with_verification_on_one_workspace():
    """The expected-acceptance launch keeps three sets of counters at once;
    calls of it alternate with verification calls (whose counters share those
    addresses) on one stream, and each call still matches the oracle."""
    from oracle.compare import compare_tokens
    a = W.small_random_inputs(16, 6, 2048, W.BF16, 0.8, seed=21)
    v = W.small_random_inputs(8, 5, 4000, W.F32, 1.0, seed=22)
    want = oracle.expected_accept(a.target, a.draft, W.BF16, 0.8)
    orc = oracle.verify(v.target, v.draft, v.tokens, W.F32, 1.0, 5)
    for _ in range(3):
        np.testing.assert_allclose(gpu_beta(a.target, a.draft, W.BF16, 0.8), want, rtol=1e-5, atol=1e-6)
        for schedule in (1, 2):
            gpu = G.run(v, 5, schedule=schedule)
            r = compare_tokens(v, orc, gpu.tokens, gpu.n, 5)
            assert not r.hard_fail, r.hard_fail[:5]
