"""Element-by-element comparison of a verification result with the oracle.

TEST INFRASTRUCTURE ONLY (tests, smoke check, benchmark validation). The GPU
result comes in as plain numpy arrays; nothing here imports the HIP path.

Token parity rule (the tolerance the contract states): accepted counts and
tokens are bit-exact, except for draws whose uniform lies within 1e-6 of a
boundary of the oracle's decision (alpha for an accept draw; the emitted
token's CDF interval for a correction or bonus draw). Such draws are counted,
and must stay under 0.1% of all draws the oracle consumes. Any other
disagreement fails outright. Greedy (T == 0) results must match exactly.
"""
from __future__ import annotations

import dataclasses
import numpy as np

from . import ACCEPT, SAMPLE, residual_cdf, uniform

BAND = 1e-6


@dataclasses.dataclass
class TokenReport:
    sequences: int = 0
    accept_draws: int = 0
    sample_draws: int = 0
    accept_mismatch: int = 0
    sample_mismatch: int = 0
    hard_fail: list = dataclasses.field(default_factory=list)
    max_boundary_dist: float = 0.0

    @property
    def draws(self):
        return self.accept_draws + self.sample_draws

    @property
    def mismatches(self):
        return self.accept_mismatch + self.sample_mismatch

    def merge(self, o: "TokenReport"):
        for f in ("sequences", "accept_draws", "sample_draws", "accept_mismatch", "sample_mismatch"):
            setattr(self, f, getattr(self, f) + getattr(o, f))
        self.hard_fail += o.hard_fail
        self.max_boundary_dist = max(self.max_boundary_dist, o.max_boundary_dist)

    def ok(self, max_rate=1e-3):
        return not self.hard_fail and self.mismatches <= max_rate * max(self.draws, 1)

    def __str__(self):
        return (f"seqs={self.sequences} draws={self.draws} (accept {self.accept_draws}, sample "
                f"{self.sample_draws}) near-boundary mismatches: accept {self.accept_mismatch}, "
                f"sample {self.sample_mismatch}; max dist {self.max_boundary_dist:.2e}; "
                f"hard failures {len(self.hard_fail)}")


def compare_tokens(inp, orc, gpu_tokens, gpu_n, seed, b_offset=0) -> TokenReport:
    """inp: workloads.Inputs; orc: oracle.Result with diagnostics."""
    wl = inp.wl
    g = wl.gamma
    rep = TokenReport()
    greedy = wl.T == 0.0
    for b in range(wl.B):
        ko, kg = int(orc.n[b]), int(gpu_n[b])
        rep.sequences += 1
        if ko >= 0 and not greedy:
            rep.accept_draws += min(ko + 1, g)
            rep.sample_draws += 1
        if ko == kg and np.array_equal(orc.tokens[b], gpu_tokens[b]):
            continue
        if greedy or ko < 0 or kg < 0:
            rep.hard_fail.append((b, "greedy/invalid mismatch", ko, kg))
            continue
        if ko != kg:
            f = min(ko, kg)
            u = uniform(seed, b + b_offset, f, ACCEPT)
            alpha = orc.alpha[b, f]
            dist = abs(u - alpha)
            same_prefix = np.array_equal(orc.tokens[b, :f], gpu_tokens[b, :f])
            if dist < BAND and same_prefix:
                rep.accept_mismatch += 1
                rep.max_boundary_dist = max(rep.max_boundary_dist, dist)
            else:
                rep.hard_fail.append((b, "accept", f, float(u), float(alpha), ko, kg))
            continue
        # same k: the accepted prefix must agree exactly; the drawn token may differ near a boundary
        k = ko
        if not np.array_equal(orc.tokens[b, :k], gpu_tokens[b, :k]) or \
                not np.array_equal(orc.tokens[b, k + 1:], gpu_tokens[b, k + 1:]):
            rep.hard_fail.append((b, "prefix/padding", k))
            continue
        j = int(gpu_tokens[b, k])
        if not (0 <= j < wl.V):
            rep.hard_fail.append((b, "token out of range", j))
            continue
        u = uniform(seed, b + b_offset, k, SAMPLE)
        q_row = inp.draft[b, k] if k < g else None
        _, cdf = residual_cdf(inp.target[b, k], q_row, wl.dtype, wl.T)
        lo = cdf[j - 1] if j > 0 else 0.0
        hi = cdf[j]
        dist = 0.0 if lo <= u < hi else min(abs(u - lo), abs(u - hi))
        if dist < BAND:
            rep.sample_mismatch += 1
            rep.max_boundary_dist = max(rep.max_boundary_dist, dist)
        else:
            rep.hard_fail.append((b, "sample", k, j, int(orc.tokens[b, k]), float(u), float(lo), float(hi)))
    return rep


def rel_err(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return np.abs(a - b) / np.maximum(np.abs(b), 1e-300)


@dataclasses.dataclass
class DraftReport:
    rows: int = 0
    draws: int = 0
    boundary: int = 0
    hard_fail: list = dataclasses.field(default_factory=list)
    max_q_rel: float = 0.0

    def ok(self, max_rate=1e-3):
        return not self.hard_fail and self.boundary <= max(1, int(max_rate * max(self.draws, 1)))

    def __str__(self):
        return (f"rows={self.rows} draws={self.draws} near-boundary {self.boundary}; max q rel err "
                f"{self.max_q_rel:.2e}; hard failures {len(self.hard_fail)}")


def compare_draft(logits, dtype, T, orc, gpu_tokens, gpu_q, seed, pos0=0, b_offset=0, q_rtol=1e-5) -> DraftReport:
    """Draft-side sampling against the oracle. logits [B, n, V] storage arrays;
    orc: oracle.DraftResult. Tokens are exact (T == 0: always; T > 0: except a
    draw whose uniform lies within BAND of the oracle's CDF interval of the GPU
    token, counted); q within q_rtol relative (exactly 1 at T == 0); unusable
    rows give -1 and NaN on both sides."""
    from . import DRAFT
    B, n, V = logits.shape
    rep = DraftReport()
    for b in range(B):
        for t in range(n):
            rep.rows += 1
            to, tg = int(orc.tokens[b, t]), int(gpu_tokens[b, t])
            qg = None if gpu_q is None else float(gpu_q[b, t])
            if to < 0:
                if tg != -1 or (qg is not None and not np.isnan(qg)):
                    rep.hard_fail.append((b, t, "unusable row", tg, qg))
                continue
            if T > 0:
                rep.draws += 1
            if tg == to:
                if qg is not None:
                    if T == 0:
                        if qg != 1.0:
                            rep.hard_fail.append((b, t, "greedy q", qg))
                    else:
                        e = abs(qg - orc.q[b, t]) / orc.q[b, t]
                        rep.max_q_rel = max(rep.max_q_rel, e)
                        if not e <= q_rtol:
                            rep.hard_fail.append((b, t, "q", qg, float(orc.q[b, t])))
                continue
            if T == 0 or not (0 <= tg < V):
                rep.hard_fail.append((b, t, "token", to, tg))
                continue
            u = uniform(seed, b + b_offset, pos0 + t, DRAFT)
            _, cdf = residual_cdf(logits[b, t], None, dtype, T)
            lo = cdf[tg - 1] if tg > 0 else 0.0
            hi = cdf[tg]
            dist = 0.0 if lo <= u < hi else min(abs(u - lo), abs(u - hi))
            if dist < BAND:
                rep.boundary += 1
            else:
                rep.hard_fail.append((b, t, "sample", to, tg, float(u), float(lo), float(hi)))
    return rep



def tree_scores(target, draft, parent, token, dtype, T, b, v):
    """The oracle's scores of node v's children in sequence b (index, score),
    T > 0: min(1, p/q) in fp64; T == 0: 1 for the argmax child, else -1."""
    from . import row_softmax
    kids = [j for j in range(v + 1, parent.shape[1]) if parent[b, j] == v]
    if T == 0:
        a = int(np.argmax(np.asarray(target[b, v]).astype(np.float64) if dtype == 0 else
                          (np.asarray(target[b, v]).astype(np.uint32) << 16).view(np.float32)))
        return [(j, 1.0 if token[b, j] == a else -1.0) for j in kids]
    _, p, _, _ = row_softmax(target[b, v], dtype, T)
    _, q, _, _ = row_softmax(draft[b, v], dtype, T)
    out = []
    for j in kids:
        pp, qq = p[token[b, j]], q[token[b, j]]
        out.append((j, 0.0 if pp == 0 else (1.0 if qq == 0 else min(1.0, pp / qq))))
    return out


def compare_tree(target, draft, parent, token, dtype, T, threshold, orc, gpu_nodes, gpu_n):
    """Tree walks against the oracle: identical paths, except where the first
    differing step was a decision within BAND (the best two children's scores,
    or the best score and the threshold). Returns (near, hard) lists."""
    o_tok, o_nodes, o_n = orc
    near, hard = [], []
    for b in range(parent.shape[0]):
        no, ng = int(o_n[b]), int(gpu_n[b])
        if no == ng and np.array_equal(o_nodes[b, :max(no, 0)], gpu_nodes[b, :max(ng, 0)]):
            continue
        if no < 0 or ng < 0:
            hard.append((b, "invalid", no, ng))
            continue
        k = 0
        while k < min(no, ng) and o_nodes[b, k] == gpu_nodes[b, k]:
            k += 1
        v = 0 if k == 0 else int(o_nodes[b, k - 1])
        sc = sorted((s_ for _, s_ in tree_scores(target, draft, parent, token, dtype, T, b, v)), reverse=True)
        margin = min([abs(sc[0] - threshold)] + ([sc[0] - sc[1]] if len(sc) > 1 else []))
        (near if T > 0 and margin < BAND else hard).append((b, k, margin))
    return near, hard
