"""Oracle for the step-predictor features of a request after one denoise step, float64.

Test infrastructure only (see the package docstring).

From [DiLaServe] (page "DiLaServe: High SLO Attainment Serving for Diffusion Language Models"),
§四 4.2 ③ (paper §3.2.3, Step Prediction): the remaining-step predictor is updated online from
progress features (the fraction of tokens already unmasked) and confidence features (quantiles of
the output tokens' confidence scores); its scalar inputs are the threshold, the output length, the
full and block progress, and the min / q25 / median / mean / q75 of the confidences.

Readings (the pages leave these open):
  * the page counts 11 features but names 9; the 9 named ones are computed, in this order:
    threshold, output length, full progress, block progress, min, q25, median, mean, q75;
  * output length = K * L (the request's blocks times the block length);
  * full progress = (b * L + unmasked slots of the current block after the step) / (K * L);
    block progress = unmasked slots of the current block after the step / L;
  * the confidences are those scored in this step (the block's masked slots on entry); quantiles
    interpolate linearly between order statistics (position q * (n - 1)); with no scored slot the
    five confidence features are NaN.
"""
from __future__ import annotations

import numpy as np

NAMES = ("threshold", "output_len", "full_progress", "block_progress", "conf_min", "conf_q25", "conf_median",
         "conf_mean", "conf_q75")


def row_features(conf_row, mask_after_row, tau, b: int, K: int, L: int) -> np.ndarray:
    """conf_row: float64 [L], -1 where not scored this step; mask_after_row: [L], 1 = still masked."""
    conf_row = np.asarray(conf_row, np.float64)
    unmasked = int(L - (np.asarray(mask_after_row) != 0).sum())
    f = np.empty(len(NAMES))
    f[0] = float(np.float32(tau))
    f[1] = K * L
    f[2] = (b * L + unmasked) / (K * L)
    f[3] = unmasked / L
    c = conf_row[conf_row >= 0]
    if c.size == 0:
        f[4:] = np.nan
    else:
        f[4] = c.min()
        f[5], f[6], f[8] = np.quantile(c, [0.25, 0.5, 0.75])
        f[7] = c.mean()
    return f


def features(conf, mask_after, threshold, b, K, L: int) -> np.ndarray:
    """[rows, 9] features for a box after a step (per-row threshold, b, K)."""
    rows = conf.shape[0]
    return np.stack([row_features(conf[r], mask_after[r], threshold[r], int(b[r]), int(K[r]), L)
                     for r in range(rows)]) if rows else np.zeros((0, len(NAMES)))
