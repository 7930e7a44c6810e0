"""Diagnostics the pages reason with (oracle, CPU, fp64).

TEST INFRASTRUCTURE -- see the package docstring.

* Pruned softmax mass of a hard logit cut-off -- AnchorAttention review, referee major
  comment 3: with theta = 12, 100k keys sitting 13 logits under the anchor carry about
  100000 * exp(-13) of mass relative to a unit anchor term.
* Sparsity of a kept set -- AnchorAttention review, referee major comment 2 (Table 1
  arithmetic: kept keys over context keys).
* SALE's relative attention score in log form -- SALE review, referee major comment 1:
  exp(S - em) / el >= tau  <=>  S >= ln(tau * el) + em (the corrected Eq. 4).
"""
from __future__ import annotations

import numpy as np


def pruned_mass_fraction(logits, kept_mask) -> float:
    """Softmax mass of the logits outside ``kept_mask`` (fp64, max-shifted)."""
    z = np.asarray(logits, dtype=np.float64)
    m = z.max()
    p = np.exp(z - m)
    return float(p[~np.asarray(kept_mask, dtype=bool)].sum() / p.sum())


def sparsity_from_kept(kept_tokens: int, total_tokens: int) -> float:
    """1 - kept / total."""
    return 1.0 - float(kept_tokens) / float(total_tokens)


def sale_log_margin(s, em, el, tau) -> np.ndarray:
    """S - (ln(tau * el) + em): >= 0 exactly when the relative score exp(S - em)/el >= tau."""
    s = np.asarray(s, dtype=np.float64)
    return s - (np.log(tau * el) + em)
