"""Host-side choice of the draft length gamma between verification calls.

Two rules from "Chapter 15: Decoding acceleration techniques" (zsc.github.io):
  - 15.1.4, dynamic strategy adjustment, adaptive draft length: the mean
    acceptance rate over a sliding window of recent calls raises gamma by one
    above 0.85 and lowers it by one below 0.6, within [gamma_min, gamma_max];
  - 15.2.4, adaptive draft length from the prediction entropy: an entropy below
    0.5 allows up to 8 draft tokens, below 1.0 up to 4, otherwise 1.
Both are plain host logic; the inputs come from the GPU path (the accepted
counts spec_verify returns, the entropy spec_draft_sample_ex returns, or the
per-position expected acceptance of spec_expected_accept).
"""
from __future__ import annotations

import collections
import math

MAX_GAMMA = 63


class AcceptanceWindowGamma:
    """gamma from the acceptance rate of the last `window` calls.

    A call's acceptance rate is the mean over its valid sequences (n >= 0) of
    n_accepted / gamma. After each observed call the mean rate over the window
    (the calls seen so far while fewer than `window`) moves gamma by one step
    if it is above `hi` or below `lo`."""

    def __init__(self, gamma: int, gamma_min: int = 1, gamma_max: int = 16, window: int = 8,
                 hi: float = 0.85, lo: float = 0.6):
        if not (1 <= gamma_min <= gamma <= gamma_max <= MAX_GAMMA):
            raise ValueError("need 1 <= gamma_min <= gamma <= gamma_max <= 63")
        if window < 1 or not (0.0 <= lo <= hi <= 1.0):
            raise ValueError("need window >= 1 and 0 <= lo <= hi <= 1")
        self.gamma = gamma
        self.gamma_min, self.gamma_max = gamma_min, gamma_max
        self.hi, self.lo = hi, lo
        self.rates = collections.deque(maxlen=window)

    @staticmethod
    def call_rate(n_accepted, gamma: int) -> float:
        """Mean of n / gamma over the sequences with n >= 0 (NaN if none)."""
        valid = [int(n) for n in n_accepted if int(n) >= 0]
        if not valid:
            return math.nan
        return sum(valid) / (len(valid) * gamma)

    def observe(self, n_accepted, gamma_used: int | None = None) -> int:
        """Record one call's accepted counts (made with gamma_used, default the
        current gamma) and return the gamma for the next call."""
        g = self.gamma if gamma_used is None else gamma_used
        r = self.call_rate(n_accepted, g)
        if not math.isnan(r):
            self.rates.append(r)
        if self.rates:
            avg = sum(self.rates) / len(self.rates)
            if avg > self.hi:
                self.gamma = min(self.gamma + 1, self.gamma_max)
            elif avg < self.lo:
                self.gamma = max(self.gamma - 1, self.gamma_min)
        return self.gamma


def entropy_draft_length(entropy: float, k_predicted: int = 8,
                         thresholds=(0.5, 1.0), lengths=(8, 4, 1)) -> int:
    """Draft length from the prediction entropy (natural log): below
    thresholds[0] min(lengths[0], k), below thresholds[1] min(lengths[1], k),
    otherwise lengths[2] (a NaN entropy, an unusable row, gives lengths[2])."""
    if entropy < thresholds[0]:
        return max(1, min(lengths[0], k_predicted))
    if entropy < thresholds[1]:
        return max(1, min(lengths[1], k_predicted))
    return max(1, min(lengths[2], k_predicted))
