"""Seeded synthetic inputs for batched speculative-sampling verification.

This module is shared by the oracle side and the HIP side of the tests and the
benchmark. It produces logits, draft tokens and seeds only: it contains none of
the verification arithmetic (no softmax, no acceptance ratio, no residual).
Draft tokens are drawn with the Gumbel-max identity, argmax_j(l_j/T + G_j) with
G_j standard Gumbel, which samples softmax(l/T) without forming it.

Sources of the shapes (pages are cited by title and section):
  [Ch15]  "Chapter 15: Decoding acceleration techniques" (zsc.github.io, LLM edge
          inference), section 15.1.2: notation (gamma draft tokens, typically 4-8;
          vocabulary V of 32K-128K; temperature T), draft-generation step 1.
  [CSDN]  devpress.csdn.net speculative-inference post, section 2.1: the
          speculative_decode() listing (draft tokens sampled from the draft
          softmax; target logits over gamma+1 positions).
The five workloads below restate the configurations the benchmark contract
names: a tiny fp32 case, a Zipf-biased 32K-vocabulary case, the bf16 headline
case (B=64, gamma=8, V=128256, T=0.8), a greedy fp32 case at T=0 and a large
low-acceptance bf16 case (B=256, V=152064, T=0.7).

Randomness: numpy Generator(Philox) keyed by the seed, one independent stream
per (seed, sequence) so that any sequence can be regenerated alone.
"""
from __future__ import annotations

import dataclasses
import numpy as np

F32 = 0
BF16 = 1
DTYPE_NAMES = {F32: "fp32", BF16: "bf16"}


# ---------------------------------------------------------------------------
# bf16 helpers (bit-level; round-to-nearest-even from fp32)
# ---------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (round to nearest, ties to even); return uint16 bits.
    NaN stays NaN (quiet), infinities stay infinities."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    b = x.view(np.uint32).astype(np.uint64)
    lsb = (b >> 16) & 1
    rounded = ((b + 0x7FFF + lsb) >> 16).astype(np.uint32)
    nan = np.isnan(x)
    if nan.any():
        rounded[nan] = ((b[nan] >> 16) | 0x40).astype(np.uint32)
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32)


def to_storage(x64: np.ndarray, dtype: int) -> np.ndarray:
    """fp64 -> storage array: float32 for F32, uint16 bf16 bits for BF16
    (fp64 -> fp32 -> bf16, each step round-to-nearest-even)."""
    x32 = np.asarray(x64, dtype=np.float32)
    if dtype == F32:
        return np.ascontiguousarray(x32)
    return f32_to_bf16_bits(x32)


def storage_to_f64(a: np.ndarray, dtype: int) -> np.ndarray:
    if dtype == F32:
        return np.asarray(a, dtype=np.float64)
    return bf16_bits_to_f32(a).astype(np.float64)


# ---------------------------------------------------------------------------
# Workload descriptions
# ---------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    gamma: int
    V: int
    dtype: int
    T: float
    kind: str              # "iid", "zipf" or "greedy"
    target_sd: float       # sd of the Gaussian part of the target logits
    zipf_s: float          # rank-bias exponent: -s * ln(rank); 0 = none
    draft_sd: float        # draft logits = target + N(0, draft_sd^2)
    greedy_p: float = 0.0  # greedy only: P(draft token = target argmax)

    @property
    def rows(self) -> int:
        return self.B * (2 * self.gamma + 1)

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == F32 else 2

    def compulsory_bytes(self) -> int:
        """Bytes the method must read once: every target and draft row at T > 0,
        the target rows alone at T == 0 (greedy verification never looks at q)."""
        rows = self.gamma + 1 if self.T == 0.0 else 2 * self.gamma + 1
        return rows * self.B * self.V * self.elem_bytes

    def bytes_read(self) -> int:
        """Bytes the statistics pass streams (the compulsory bytes)."""
        return self.compulsory_bytes()

    def scaled(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    # tiny fp32 case: i.i.d. N(0, 2^2) logits, draft = target + N(0, 0.5^2), T = 1
    "tiny_b1_g4_v1000_f32": Workload("tiny_b1_g4_v1000_f32", 1, 4, 1000, F32, 1.0,
                                     "iid", 2.0, 0.0, 0.5),
    # Zipf-biased fp32 case: N(0, 3^2) - 1.1 ln(rank), draft + N(0, 1), T = 1
    "zipf_b8_g5_v32000_f32": Workload("zipf_b8_g5_v32000_f32", 8, 5, 32000, F32, 1.0,
                                      "zipf", 3.0, 1.1, 1.0),
    # headline bf16 case: -1.1 ln(rank) + N(0, 1.5^2), draft + N(0, 0.7^2), T = 0.8
    "zipf_b64_g8_v128256_bf16": Workload("zipf_b64_g8_v128256_bf16", 64, 8, 128256, BF16, 0.8,
                                         "zipf", 1.5, 1.1, 0.7),
    # greedy fp32 case at T = 0 (target logits as the headline generator, in fp32)
    "greedy_b32_g8_v128256_f32": Workload("greedy_b32_g8_v128256_f32", 32, 8, 128256, F32, 0.0,
                                          "greedy", 1.5, 1.1, 0.7, greedy_p=0.8),
    # large low-acceptance bf16 case: -1.3 ln(rank) + N(0, 1), draft + N(0, 1.2^2), T = 0.7
    "zipf_b256_g8_v152064_bf16": Workload("zipf_b256_g8_v152064_bf16", 256, 8, 152064, BF16, 0.7,
                                          "zipf", 1.0, 1.3, 1.2),
}
WORKLOAD_ORDER = list(WORKLOADS)
HEADLINE = "zipf_b64_g8_v128256_bf16"


@dataclasses.dataclass
class Inputs:
    wl: Workload
    seed: int
    target: np.ndarray        # [B, gamma+1, V] float32 or uint16 (bf16 bits)
    draft: np.ndarray         # [B, gamma, V]
    tokens: np.ndarray        # [B, gamma] int32

    @property
    def target_f64(self) -> np.ndarray:
        return storage_to_f64(self.target, self.wl.dtype)

    @property
    def draft_f64(self) -> np.ndarray:
        return storage_to_f64(self.draft, self.wl.dtype)


def _seq_rng(seed: int, b: int, stream: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.Philox(key=[(seed & 0xFFFFFFFFFFFFFFFF), (b << 8) | stream]))


def gumbel_max_sample(rng: np.random.Generator, logits64: np.ndarray, T: float) -> int:
    """One draw from softmax(logits/T) by the Gumbel-max identity (T > 0).
    Entries equal to -inf are never drawn."""
    g = -np.log(-np.log(rng.random(logits64.shape[-1])))
    score = logits64 / T + g
    return int(np.argmax(score))


def _gen_sequence(wl: Workload, seed: int, b: int):
    """Target rows [gamma+1, V], draft rows [gamma, V] (fp64 before storage rounding)."""
    rng = _seq_rng(seed, b)
    G1, V = wl.gamma + 1, wl.V
    if wl.kind == "iid":
        t = rng.normal(0.0, wl.target_sd, size=(G1, V))
    else:
        t = np.empty((G1, V))
        logrank = np.log(np.arange(1, V + 1, dtype=np.float64))
        for i in range(G1):
            t[i] = -wl.zipf_s * logrank[rng.permutation(V)]
        t += rng.normal(0.0, wl.target_sd, size=(G1, V))
    d = t[: wl.gamma] + rng.normal(0.0, wl.draft_sd, size=(wl.gamma, V))
    return t, d, rng


def make_inputs(wl: Workload, seed: int = 0) -> Inputs:
    """Seeded synthetic inputs of workload `wl`.

    Draft token i of each sequence is drawn from softmax(draft row i / T) of the
    *stored* (rounded) draft logits, so that q is exactly the distribution the
    token came from. For the greedy workload it is the target row's argmax with
    probability greedy_p, else uniform over [0, V)."""
    B, g, V = wl.B, wl.gamma, wl.V
    if wl.dtype == F32:
        target = np.empty((B, g + 1, V), np.float32)
        draft = np.empty((B, g, V), np.float32)
    else:
        target = np.empty((B, g + 1, V), np.uint16)
        draft = np.empty((B, g, V), np.uint16)
    tokens = np.empty((B, g), np.int32)
    for b in range(B):
        t, d, rng = _gen_sequence(wl, seed, b)
        target[b] = to_storage(t, wl.dtype)
        draft[b] = to_storage(d, wl.dtype)
        t_st = storage_to_f64(target[b], wl.dtype)
        d_st = storage_to_f64(draft[b], wl.dtype)
        for i in range(g):
            if wl.kind == "greedy":
                if rng.random() < wl.greedy_p:
                    tokens[b, i] = int(np.argmax(t_st[i]))
                else:
                    tokens[b, i] = int(rng.integers(0, V))
            else:
                tokens[b, i] = gumbel_max_sample(rng, d_st[i], wl.T)
    return Inputs(wl, seed, target, draft, tokens)


# ---------------------------------------------------------------------------
# Constructed inputs for statistical checks
# ---------------------------------------------------------------------------
def log_probs(p) -> np.ndarray:
    """Logits whose softmax at T = 1 is p (zeros map to -inf)."""
    p = np.asarray(p, dtype=np.float64)
    with np.errstate(divide="ignore"):
        return np.where(p > 0, np.log(p), -np.inf)


def repeated_rows_inputs(target_rows64: np.ndarray, draft_rows64: np.ndarray, B: int,
                         T: float, seed: int, dtype: int = F32) -> Inputs:
    """B sequences that share the same target rows [gamma+1, V] and draft rows
    [gamma, V]; each sequence draws its own draft tokens x_i ~ softmax(draft_i/T).
    Used for the distribution (chi-square) and acceptance-count checks."""
    g1, V = target_rows64.shape
    g = g1 - 1
    assert draft_rows64.shape == (g, V)
    t_st = to_storage(target_rows64, dtype)
    d_st = to_storage(draft_rows64, dtype)
    target = np.broadcast_to(t_st, (B, g1, V)).copy()
    draft = np.broadcast_to(d_st, (B, g, V)).copy()
    d64 = storage_to_f64(d_st, dtype)
    rng = np.random.Generator(np.random.Philox(key=[seed & 0xFFFFFFFFFFFFFFFF, 0xD0]))
    tokens = np.empty((B, g), np.int32)
    for i in range(g):
        # vectorised Gumbel-max over the batch
        gmb = -np.log(-np.log(rng.random((B, V))))
        tokens[:, i] = np.argmax(d64[i][None, :] / T + gmb, axis=1)
    wl = Workload("constructed", B, g, V, dtype, T, "constructed", 0.0, 0.0, 0.0)
    return Inputs(wl, seed, target, draft, tokens)


def small_random_inputs(B: int, gamma: int, V: int, dtype: int, T: float, seed: int,
                        sd: float = 2.0, draft_sd: float = 0.7) -> Inputs:
    """Small i.i.d. Gaussian case of arbitrary shape (ragged V, odd gamma)."""
    wl = Workload(f"small_b{B}_g{gamma}_v{V}", B, gamma, V, dtype, T, "iid", sd, 0.0, draft_sd)
    return make_inputs(wl, seed)


# ---------------------------------------------------------------------------
# Token trees (the tree-verification mode's inputs)
# ---------------------------------------------------------------------------
@dataclasses.dataclass
class TreeInputs:
    target: np.ndarray   # [B, N, V] storage: row j = the target model's logits after the path to node j
    draft: np.ndarray    # [B, N, V] storage: the draft model's
    parent: np.ndarray   # [B, N] int32: node 0 is the root (-1), node j >= 1 has parent < j
    token: np.ndarray    # [B, N] int32: node j's token (-1 at the root)
    dtype: int
    T: float


def tree_inputs(B: int, depth: int, branch: int, V: int, dtype: int, T: float, seed: int,
                sd: float = 2.0, draft_sd: float = 0.7) -> TreeInputs:
    """Full trees of `depth` levels below the root with `branch` children per
    node, built level by level as a draft model's beam would: each node's
    children are `branch` distinct tokens drawn without replacement from
    softmax(draft row / T) (Gumbel top-k on the stored draft row). Rows are
    i.i.d. Gaussian logits (drawn in fp32), the draft row the target row plus
    noise."""
    N = sum(branch ** d for d in range(depth + 1))
    st = np.float32 if dtype == F32 else np.uint16
    target = np.empty((B, N, V), st)
    draft = np.empty((B, N, V), st)
    parent = np.full((B, N), -1, np.int32)
    token = np.full((B, N), -1, np.int32)
    for b in range(B):
        rng = _seq_rng(seed, b, stream=7)
        t = rng.standard_normal((N, V), dtype=np.float32) * np.float32(sd)
        d = t + rng.standard_normal((N, V), dtype=np.float32) * np.float32(draft_sd)
        target[b] = to_storage(t, dtype)
        draft[b] = to_storage(d, dtype)
        d_st = storage_to_f64(draft[b], dtype)
        nxt = 1
        level = [0]
        for _ in range(depth):
            new_level = []
            for v in level:
                g = -np.log(-np.log(rng.random(V)))
                score = d_st[v] / (T if T > 0 else 1.0) + g
                top = np.argpartition(-score, branch - 1)[:branch] if branch < V else np.arange(V)
                kids = top[np.argsort(-score[top], kind="stable")]
                for x in kids:
                    parent[b, nxt] = v
                    token[b, nxt] = int(x)
                    new_level.append(nxt)
                    nxt += 1
            level = new_level
        assert nxt == N
    return TreeInputs(target, draft, parent, token, dtype, T)
