"""Comparison rules between the GPU path and the oracle (test infrastructure).

The parity contract for one step:
  (i)   argmax equal bit for bit at every compared scored slot (a comparison of stored values);
  (ii)  |conf_gpu - conf_oracle| <= CONF_TOL at every compared scored slot;
  (iii) the GPU's unmask decision equals the rule applied to the GPU's own confidences, exactly;
  (iv)  the GPU's decision equals the rule applied to the oracle's confidences, except in
        ambiguous rows: a masked confidence within CONF_TOL of the row's threshold, or a fallback
        row whose two largest oracle confidences are within CONF_TOL.
Everything integer (ids, masks, done, accept, pack/compact layouts) is compared exactly.
"""
import numpy as np

from oracle import quota as oquota
from oracle import step as ostep

CONF_TOL = 1e-5


def ambiguous_row(conf_row, masked, tau):
    c = np.asarray(conf_row, np.float64)[masked]
    if c.size == 0:
        return False
    t = float(np.float32(tau))
    if np.any(np.abs(c - t) <= CONF_TOL):
        return True
    if not np.any(c > t) and c.size >= 2:
        top = np.sort(c)[-2:]
        return bool(top[1] - top[0] <= CONF_TOL)
    return False


def check_decisions(gpu_conf, oracle_conf, mask_in, mask_out_gpu, tau):
    """(iii) and (iv) for every row; returns the number of ambiguous rows."""
    rows = mask_in.shape[0]
    n_amb = 0
    for r in range(rows):
        masked = mask_in[r] != 0
        gpu_U = masked & (mask_out_gpu[r] == 0)
        own = ostep.decide(np.asarray(gpu_conf[r], np.float64), masked, tau[r])
        assert np.array_equal(gpu_U, own), f"row {r}: decision differs from the rule on the GPU's own confidences"
        if ambiguous_row(oracle_conf[r], masked, tau[r]):
            n_amb += 1
            continue
        ref = ostep.decide(np.asarray(oracle_conf[r], np.float64), masked, tau[r])
        assert np.array_equal(gpu_U, ref), f"row {r}: decision differs from the oracle's"
    return n_amb


def check_scores(gpu_conf, gpu_arg, oracle_conf, oracle_arg, where=None):
    """(i) and (ii) over the slots selected by `where` (default: all scored slots)."""
    sel = (oracle_arg >= 0) if where is None else where
    assert np.array_equal(gpu_arg[sel], oracle_arg[sel]), "argmax differs"
    err = np.abs(np.asarray(gpu_conf, np.float64)[sel] - oracle_conf[sel])
    assert err.size == 0 or err.max() <= CONF_TOL, f"conf error {err.max()}"
    return float(err.max()) if err.size else 0.0


def ambiguous_topk_row(conf_row, masked, k):
    """Quota rule: ambiguous when the k-th and (k+1)-th largest masked oracle confidences (the cut)
    are within CONF_TOL."""
    c = np.sort(np.asarray(conf_row, np.float64)[masked])[::-1]
    if k <= 0 or k >= c.size:
        return False
    return bool(c[k - 1] - c[k] <= CONF_TOL)


def check_quota_decisions(gpu_conf, oracle_conf, mask_in, mask_out_gpu, S):
    """(iii) and (iv) for the quota rule; returns the number of ambiguous rows."""
    rows, L = mask_in.shape
    n_amb = 0
    for r in range(rows):
        masked = mask_in[r] != 0
        k = oquota.quota_for_remaining(L, S, int(masked.sum()))
        gpu_U = masked & (mask_out_gpu[r] == 0)
        own = oquota.decide_topk(np.asarray(gpu_conf[r], np.float64), masked, k)
        assert np.array_equal(gpu_U, own), f"row {r}: decision differs from the quota rule on the GPU's confidences"
        if ambiguous_topk_row(oracle_conf[r], masked, k):
            n_amb += 1
            continue
        ref = oquota.decide_topk(np.asarray(oracle_conf[r], np.float64), masked, k)
        assert np.array_equal(gpu_U, ref), f"row {r}: quota decision differs from the oracle's"
    return n_amb
