"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle on the
same seeded inputs.

Tolerances:
  - row max: exact (it is an input value);
  - sum-exp, p(x_i), q(x_i), Z: relative 1e-5 (Z below 1e-3: absolute 1e-8);
  - accepted counts and tokens: exact, except draws within 1e-6 of the oracle's
    decision boundary, counted and pooled per workload under 0.1% of draws;
  - greedy (T == 0): exact, no exceptions.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from oracle.compare import TokenReport, compare_tokens, rel_err

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import gpu_helpers as G
    import speculative_sampling_verification_05_amd as sv


def check_values(inp, orc, gpu):
    wl = inp.wl
    g = wl.gamma
    if wl.T == 0.0:
        t64 = inp.target_f64
        np.testing.assert_array_equal(gpu.argmax, np.argmax(t64, axis=2))
        return
    ok = np.isfinite(orc.row_sumexp)
    assert np.array_equal(gpu.row_max[ok].astype(np.float64), orc.row_max[ok])
    assert np.isfinite(gpu.row_sumexp[ok]).all()
    assert rel_err(gpu.row_sumexp[ok], orc.row_sumexp[ok]).max() <= 1e-5
    reached = np.isfinite(orc.p_tok)
    assert rel_err(gpu.p[reached], orc.p_tok[reached]).max(initial=0) <= 1e-5
    assert rel_err(gpu.q[reached], orc.q_tok[reached]).max(initial=0) <= 1e-5
    valid = orc.n >= 0
    big = valid & (orc.Z >= 1e-3)
    small = valid & (orc.Z < 1e-3)
    assert rel_err(gpu.Z[big], orc.Z[big]).max(initial=0) <= 1e-5
    assert np.abs(gpu.Z[small] - orc.Z[small]).max(initial=0) <= 1e-8


# The grid orders, each as a leg (schedule, debug outputs):
#  group      the group-major order (T == 0: k_group in greedy mode) with every
#             debug output;
#  position   the position-major order reading every row, every debug output;
#  early      the position-major order with the early stop and no per-row
#             debug output, so that rows after a sequence's first rejection are
#             really skipped (the default call's path at T == 0 and at large B);
#  plain      the group-major order with no debug output (the default call's
#             path at small B): at T > 0 the bonus row is then read only by the
#             closing blocks of sequences that accept every draft token.
LEGS = {"group": (1, True), "position": (3, True), "early": (2, False), "plain": (1, False), "two_phase": (4, False)}


def parity(inp, seed, b_offset=0, report=None, schedule=0, debug=True):
    gpu = G.run(inp, seed, b_offset=b_offset, schedule=schedule, debug=debug)
    wl = inp.wl
    orc = oracle.verify(inp.target, inp.draft if wl.T > 0 else None, inp.tokens, wl.dtype, wl.T,
                        seed, b_offset=b_offset)
    if debug:
        check_values(inp, orc, gpu)
    rep = compare_tokens(inp, orc, gpu.tokens, gpu.n, seed, b_offset)
    assert not rep.hard_fail, rep.hard_fail[:5]
    if wl.T == 0.0:
        assert rep.mismatches == 0
    if report is not None:
        report.merge(rep)
    return gpu, orc, rep


# (seeds, batch override). Sampling pools hold >= ~2000 draws so that the
# 0.1% bound on near-boundary disagreements is a meaningful count.
POOL_SEEDS = {
    "tiny_b1_g4_v1000_f32": (range(500), None),
    "zipf_b8_g5_v32000_f32": (range(80), None),
    "zipf_b64_g8_v128256_bf16": (range(8), None),
    "greedy_b32_g8_v128256_f32": (range(3), 8),
    "zipf_b256_g8_v152064_bf16": (range(12), 64),
    # the headline recipe at 24 sequences: the group-major closing blocks then
    # take one residual subsegment per wavefront
    "zipf_b64_g8_v128256_bf16@24": (range(4), 24),
}


@pytest.mark.parametrize("name", list(POOL_SEEDS))
def test_workload_parity_pooled(name):
    """Several seeds per workload at a batch the oracle finishes quickly; the
    near-boundary count is pooled over the seeds, per leg. Every leg (both
    grid orders, and the early stop with its row skipping) runs on the same
    inputs."""
    seeds, B = POOL_SEEDS[name]
    wl = W.WORKLOADS[name.split("@")[0]]
    if B is not None:
        wl = wl.scaled(B=B)
    reps = {leg: TokenReport() for leg in LEGS}
    for s in seeds:
        inp = W.make_inputs(wl, s)
        for leg, (schedule, debug) in LEGS.items():
            parity(inp, seed=1000 + s, report=reps[leg], schedule=schedule, debug=debug)
    for leg, rep in reps.items():
        print(name, leg, rep)
        assert rep.ok(), f"{leg}: {rep}"


@pytest.mark.parametrize("B", [1, 2, 4])
@pytest.mark.parametrize("name", ["zipf_b64_g8_v128256_bf16", "greedy_b32_g8_v128256_f32"])
def test_small_batches_full_vocabulary(name, B):
    """One to four sequences at the full 128256-entry vocabulary: the ranges
    are then as short as a group's partial slots in the LDS stage (group-major)
    or one wavefront's worth of slots per row (position-major) allow. Every
    leg against the oracle, several seeds pooled per leg."""
    wl = W.WORKLOADS[name].scaled(B=B)
    reps = {leg: TokenReport() for leg in LEGS}
    for s in range(4):
        inp = W.make_inputs(wl, 50 + s)
        for leg, (schedule, debug) in LEGS.items():
            parity(inp, seed=70 + s, report=reps[leg], schedule=schedule, debug=debug)
    for leg, rep in reps.items():
        print(name, B, leg, rep)
        assert rep.mismatches <= 1, f"{leg}: {rep}"


@pytest.mark.parametrize("name,auto", [("greedy_b32_g8_v128256_f32", 2), ("zipf_b256_g8_v152064_bf16", 4)])
def test_full_size_parity(name, auto):
    """The full workload: every row's values against the oracle (the debug
    outputs read every row), and the call the benchmark times (the automatic
    schedule, no extras: the early stop for the greedy workload, two phases
    for the 256-sequence one) returning exactly the same tokens."""
    wl = W.WORKLOADS[name]
    inp = W.make_inputs(wl, 0)
    gpu, _, rep = parity(inp, seed=0)
    print(name, rep)
    assert rep.mismatches <= max(1, int(1e-3 * rep.draws)), str(rep)
    assert sv.auto_schedule(wl.B, wl.gamma, wl.V, wl.dtype, wl.T) == auto
    tgt, dft = G.to_device(inp.target, wl.dtype), G.to_device(inp.draft, wl.dtype)
    tok = torch.from_numpy(inp.tokens).to("cuda:0")
    out_t, out_n = sv.verify(tgt, dft if wl.T > 0 else None, tok, wl.T, 0)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out_n.cpu().numpy(), gpu.n)
    np.testing.assert_array_equal(out_t.cpu().numpy(), gpu.tokens)


EDGE_SHAPES = [
    # B, gamma, V, dtype  (vector path needs V*sizeof % 16 == 0)
    (1, 1, 1, W.F32),
    (3, 1, 7, W.BF16),
    (2, 63, 300, W.F32),
    (5, 7, 1003, W.BF16),      # scalar path, ragged
    (4, 4, 4097, W.F32),       # scalar path
    (2, 3, 520, W.BF16),       # vector path, one full chunk + ragged tail
    (3, 2, 8192, W.BF16),
    (7, 5, 33000, W.F32),
    (1, 8, 128256, W.BF16),
    (60, 2, 1003, W.BF16),     # more groups than the group-major lag: residual blocks interleaved
    (61, 1, 4096, W.F32),      #   with the stream (scalar and vector path)
    (70, 3, 1003, W.BF16),     # two phases with the deciders interleaved with the first phase
    (130, 3, 1003, W.BF16),    # two phases from 128 groups: second-phase ranges longer than the first's
    (128, 4, 4096, W.F32),     #   (scalar path: 12 chunks against 1; vector path: 48 against 16)
]


@pytest.mark.parametrize("leg", list(LEGS))
@pytest.mark.parametrize("shape", EDGE_SHAPES)
@pytest.mark.parametrize("T", [0.0, 0.6, 1.7])
def test_edge_shapes(shape, T, leg):
    B, g, V, dt = shape
    schedule, debug = LEGS[leg]
    rep = TokenReport()
    for s in range(3):
        inp = W.small_random_inputs(B, g, V, dt, T, seed=100 + s)
        parity(inp, seed=s, report=rep, schedule=schedule, debug=debug)
    assert rep.mismatches <= 1, str(rep)


@pytest.mark.parametrize("dt", [W.F32, W.BF16])
@pytest.mark.parametrize("T", [0.0, 0.8])
def test_unaligned_pointers_take_the_scalar_path(dt, T):
    inp = W.small_random_inputs(4, 3, 4096, dt, T, seed=7)
    wl = inp.wl
    es = 4 if dt == W.F32 else 2
    tdt = torch.float32 if dt == W.F32 else torch.bfloat16

    def shifted(a):
        flat = G.to_device(a.reshape(-1), dt)
        buf = torch.empty(flat.numel() + 1, dtype=tdt, device="cuda:0")
        buf[1:].copy_(flat)
        v = buf[1:].view(a.shape)
        assert v.data_ptr() % 16 == es
        return v

    tgt, dft = shifted(inp.target), shifted(inp.draft)
    tok = torch.from_numpy(inp.tokens).to("cuda:0")
    out_t, out_n = sv.verify(tgt, dft, tok, wl.T, 5)
    torch.cuda.synchronize()
    orc = oracle.verify(inp.target, inp.draft if T > 0 else None, inp.tokens, dt, T, 5)
    rep = compare_tokens(inp, orc, out_t.cpu().numpy(), out_n.cpu().numpy(), 5)
    assert not rep.hard_fail and rep.mismatches == 0


@pytest.mark.parametrize("leg", list(LEGS))
@pytest.mark.parametrize("T", [0.0, 1.0])
def test_invalid_inputs_reported_in_band(T, leg):
    """Unusable rows and out-of-range tokens, in every leg: rows the
    sequential loop reaches give -1, rows it never reaches (some of which the
    early stop skips) change nothing."""
    schedule, debug = LEGS[leg]
    inp = W.small_random_inputs(12, 4, 2048, W.BF16, T, seed=21)
    t, d, tok = inp.target.copy(), inp.draft.copy(), inp.tokens.copy()
    nan, inf, ninf = (W.f32_to_bf16_bits(np.array([v], np.float32))[0] for v in (np.nan, np.inf, -np.inf))
    t[0, 0, 17] = nan                 # target row 0: always reached
    t[1, 0, 5] = inf
    t[2, 0, :] = ninf                 # no finite entry
    d[3, 0, 9] = nan                  # draft row 0 (T > 0 only)
    tok[4, 0] = 2048                  # out of range
    tok[5, 0] = -3
    t[6, 3, 0] = nan                  # late row: only matters if reached
    t[7, 4, 1] = nan                  # bonus row
    d[8, 3, :] = ninf
    t[9, 2, 3] = inf                  # late rows of one sequence: +inf, NaN, none finite
    d[9, 3, 4] = nan
    t[10, 1, :] = ninf
    tok[11, 3] = 4096                 # late out-of-range token
    inp2 = W.Inputs(inp.wl, inp.seed, t, d, tok)
    gpu = G.run(inp2, 3, schedule=schedule, debug=debug)
    orc = oracle.verify(t, d if T > 0 else None, tok, W.BF16, T, 3)
    np.testing.assert_array_equal(gpu.n, orc.n)
    np.testing.assert_array_equal(gpu.tokens, orc.tokens)
    for b in (0, 1, 2, 4, 5):
        assert gpu.n[b] == -1 and (gpu.tokens[b] == -1).all()


def test_identical_models_accept_everything():
    inp = W.small_random_inputs(32, 6, 5000, W.BF16, 0.9, seed=4)
    same = W.Inputs(inp.wl, inp.seed, inp.target, inp.target[:, :6].copy(), inp.tokens)
    for s in range(3):
        gpu, orc, rep = parity(same, seed=s)
        assert (gpu.n == 6).all()


@pytest.mark.parametrize("leg", list(LEGS))
def test_greedy_ties_lowest_index(leg):
    schedule, debug = LEGS[leg]
    wl = W.WORKLOADS["greedy_b32_g8_v128256_f32"].scaled(B=8, V=20000)
    inp = W.make_inputs(wl, 5)
    t = inp.target.copy()
    for b in range(wl.B):
        for i in range(wl.gamma + 1):
            j = int(np.argmax(t[b, i]))
            t[b, i, (j + 4999) % wl.V] = t[b, i, j]
            if i % 2:
                t[b, i, (j + wl.V - 777) % wl.V] = t[b, i, j]
    inp2 = W.Inputs(wl, 5, t, inp.draft, inp.tokens)
    gpu = G.run(inp2, 0, schedule=schedule, debug=debug)
    orc = oracle.verify(t, None, inp.tokens, W.F32, 0.0)
    np.testing.assert_array_equal(gpu.n, orc.n)
    np.testing.assert_array_equal(gpu.tokens, orc.tokens)
    if debug:
        np.testing.assert_array_equal(gpu.argmax, np.argmax(t, axis=2))


def test_deterministic_run_to_run():
    inp = W.make_inputs(W.WORKLOADS["zipf_b64_g8_v128256_bf16"].scaled(B=8), 9)
    a = G.run(inp, 77)
    b = G.run(inp, 77)
    for f in ("tokens", "n", "row_max", "row_sumexp", "p", "q", "Z"):
        x, y = getattr(a, f), getattr(b, f)
        assert np.array_equal(x.view(np.uint8), y.view(np.uint8)), f


def test_batch_offset_shards_reproduce_the_whole_batch():
    inp = W.make_inputs(W.WORKLOADS["zipf_b8_g5_v32000_f32"], 2)
    whole = G.run(inp, 31)
    h = inp.wl.B // 2
    parts = []
    for lo, hi in ((0, h), (h, inp.wl.B)):
        sub = W.Inputs(inp.wl.scaled(B=hi - lo), 2, inp.target[lo:hi], inp.draft[lo:hi], inp.tokens[lo:hi])
        parts.append(G.run(sub, 31, b_offset=lo))
    np.testing.assert_array_equal(np.concatenate([p.tokens for p in parts]), whole.tokens)
    np.testing.assert_array_equal(np.concatenate([p.n for p in parts]), whole.n)


def test_side_stream():
    inp = W.small_random_inputs(16, 4, 6000, W.BF16, 1.1, seed=8)
    s = torch.cuda.Stream()
    tensors = (G.to_device(inp.target, W.BF16), G.to_device(inp.draft, W.BF16),
               torch.from_numpy(inp.tokens).to("cuda:0"))
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        gpu = G.run(inp, 12, tensors=tensors, stream=s)
    orc = oracle.verify(inp.target, inp.draft, inp.tokens, W.BF16, 1.1, 12)
    rep = compare_tokens(inp, orc, gpu.tokens, gpu.n, 12)
    assert not rep.hard_fail and rep.mismatches == 0


@pytest.mark.parametrize("dt", [W.F32, W.BF16])
def test_row_stats_entry_point(dt):
    rng = np.random.default_rng(3)
    rows, V = 37, 10001 if dt == W.F32 else 12288
    l64 = rng.normal(0, 2.5, (rows, V)) - 1.1 * np.log(rng.permuted(np.tile(np.arange(1, V + 1), (rows, 1)), axis=1))
    l64[3, :] = -np.inf
    l64[3, 100] = 1.0
    l64[5, 7] = np.nan
    st = W.to_storage(l64, dt)
    m, s = sv.row_stats(G.to_device(st, dt), 0.7)
    m, s = m.cpu().numpy(), s.cpu().numpy()
    for r in range(rows):
        ok, _, om, oS = oracle.row_softmax(st[r], dt, 0.7)
        if not ok:
            assert np.isnan(s[r])
            continue
        assert m[r] == om
        assert abs(s[r] - oS) <= 1e-5 * oS


def test_workspace_reuse_across_shapes_and_modes():
    """Calls of different shapes and modes, back to back on one stream, share
    the library's workspace (group counters are left at zero by every call):
    each still matches the oracle."""
    cases = [
        W.small_random_inputs(6, 4, 3000, W.BF16, 0.9, seed=31),
        W.small_random_inputs(5, 3, 1003, W.F32, 1.0, seed=32),
        W.small_random_inputs(9, 7, 4096, W.BF16, 0.0, seed=33),
        W.small_random_inputs(40, 2, 520, W.F32, 1.3, seed=34),
        W.small_random_inputs(3, 9, 9000, W.BF16, 0.7, seed=35),
        W.small_random_inputs(6, 4, 3000, W.BF16, 0.9, seed=31),
    ]
    for rep in range(2):
        for n, inp in enumerate(cases):
            parity(inp, seed=100 * rep + n)
        rng = np.random.default_rng(rep)
        logits = W.to_storage(rng.normal(0, 2, (7, 2048)), W.BF16)
        m, s = sv.row_stats(G.to_device(logits, W.BF16), 0.9)
        m, s = m.cpu().numpy(), s.cpu().numpy()
        for r in range(7):
            ok, _, om, oS = oracle.row_softmax(logits[r], W.BF16, 0.9)
            assert ok and m[r] == om and abs(s[r] - oS) <= 1e-5 * oS


@pytest.mark.parametrize("name", list(POOL_SEEDS))
def test_schedules_give_the_same_outputs(name):
    """Every schedule - group-major, position-major reading every row, and the
    early stop, which skips the rows of sequences already known to have
    stopped - returns exactly the same tokens and counts (and the oracle's)."""
    seeds, B = POOL_SEEDS[name]
    wl = W.WORKLOADS[name.split("@")[0]]
    if B is not None:
        wl = wl.scaled(B=B)
    for s in list(seeds)[:3]:
        inp = W.make_inputs(wl, s)
        full = G.run(inp, 1000 + s, schedule=sv.SCHEDULE_POSITION)
        tgt, dft = G.to_device(inp.target, wl.dtype), G.to_device(inp.draft, wl.dtype)
        tok = torch.from_numpy(inp.tokens).to("cuda:0")
        for sched in (sv.SCHEDULE_AUTO, sv.SCHEDULE_GROUP, sv.SCHEDULE_EARLY_STOP, sv.SCHEDULE_POSITION,
                      sv.SCHEDULE_GROUP_TWO_PHASE):
            ex = sv.Extras()
            ex.schedule = sched
            for rep_call in range(2):
                out_t, out_n = sv.verify(tgt, dft if wl.T > 0 else None, tok, wl.T, 1000 + s, extras=ex)
                torch.cuda.synchronize()
                np.testing.assert_array_equal(out_n.cpu().numpy(), full.n)
                np.testing.assert_array_equal(out_t.cpu().numpy(), full.tokens)
        orc = oracle.verify(inp.target, inp.draft if wl.T > 0 else None, inp.tokens, wl.dtype, wl.T, 1000 + s)
        rep = compare_tokens(inp, orc, full.tokens, full.n, 1000 + s)
        assert not rep.hard_fail, rep.hard_fail[:5]


def test_auto_schedule_rule():
    """The automatic choice: group-major in two phases for the B=64 headline
    shape (one phase at gamma = 1), the early stop once one position's row
    pairs come to 152 MiB (from 320 sequences of both recipes)."""
    assert sv.auto_schedule(64, 8, 128256, sv.SPEC_BF16, 0.8) == sv.SCHEDULE_GROUP_TWO_PHASE
    assert sv.auto_schedule(64, 1, 128256, sv.SPEC_BF16, 0.8) == sv.SCHEDULE_GROUP
    assert sv.auto_schedule(8, 5, 32000, sv.SPEC_F32, 1.0) == sv.SCHEDULE_GROUP  # (rows below 112 MiB)
    assert sv.auto_schedule(24, 8, 128256, sv.SPEC_BF16, 0.8) == sv.SCHEDULE_GROUP  # 98 MB
    assert sv.auto_schedule(32, 8, 128256, sv.SPEC_BF16, 0.8) == sv.SCHEDULE_GROUP_TWO_PHASE  # 131 MB
    assert sv.auto_schedule(96, 5, 32000, sv.SPEC_F32, 1.0) == sv.SCHEDULE_GROUP_TWO_PHASE  # 123 MB
    assert sv.auto_schedule(192, 8, 128256, sv.SPEC_BF16, 0.8) == sv.SCHEDULE_GROUP_TWO_PHASE
    # the early stop from 152 MiB of one position's row pairs (2 B V s)
    assert sv.auto_schedule(256, 8, 128256, sv.SPEC_BF16, 0.8) == sv.SCHEDULE_GROUP_TWO_PHASE  # 131 MB
    assert sv.auto_schedule(320, 8, 128256, sv.SPEC_BF16, 0.8) == sv.SCHEDULE_EARLY_STOP  # 164 MB
    assert sv.auto_schedule(384, 8, 128256, sv.SPEC_BF16, 0.8) == sv.SCHEDULE_EARLY_STOP
    assert sv.auto_schedule(256, 8, 152064, sv.SPEC_BF16, 0.7) == sv.SCHEDULE_GROUP_TWO_PHASE  # 156 MB
    assert sv.auto_schedule(320, 8, 152064, sv.SPEC_BF16, 0.7) == sv.SCHEDULE_EARLY_STOP  # 195 MB
    assert sv.auto_schedule(32, 8, 128256, sv.SPEC_F32, 0.0) == sv.SCHEDULE_EARLY_STOP
