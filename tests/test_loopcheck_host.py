"""The deferred loop checker on the CPU: it passes right results and reports planted wrong ones
(a wrong argmax, a confidence off by more than the tolerance, a decision the oracle would not
take), with the step, row and slot."""
import numpy as np
import pytest

from oracle import rows as orows
from oracle import step as ostep
from tests.loopcheck import DeferredChecker

torch = pytest.importorskip("torch")


def _job(seed, rows=3, L=4, V=300, dtype="bf16"):
    rng = np.random.default_rng(seed)
    x = rng.normal(0, 2, (rows, L, V)).astype(np.float32)
    x[..., 5] += 6.0                                       # a clear winner: decisions far from ties
    lg = torch.from_numpy(x).to(torch.bfloat16) if dtype == "bf16" else torch.from_numpy(x)
    masked = rng.random((rows, L)) < 0.7
    masked[:, 0] = True
    rr, jj = np.nonzero(masked)
    host = lg.reshape(-1, V)[torch.from_numpy(rr * L + jj)]
    hx = host.view(torch.int16).numpy().view(np.uint16) if dtype == "bf16" else host.numpy()
    a, c = orows.score_rows(hx, dtype)
    conf = np.full((rows, L), -1.0)
    conf[rr, jj] = c
    tau = np.float32(0.9)
    U = np.stack([ostep.decide(conf[r], masked[r], tau) for r in range(rows)])
    return lg, masked, rr, jj, a, c, tau, U


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("chunk", [1024, 3])
def test_checker_passes_the_oracle_own_results(dtype, chunk):
    lg, masked, rr, jj, a, c, tau, U = _job(1, dtype=dtype)
    ck = DeferredChecker(dtype, lg.shape[-1], threads=2)
    ck.CHUNK_ROWS = chunk
    host = ck.gather(lg, rr * masked.shape[1] + jj)
    rows_full = [(r, masked[r], tau, U[r]) for r in range(masked.shape[0])]
    ck.submit(1, host, list(zip(rr.tolist(), jj.tolist())), a, c.astype(np.float32), rows_full)
    st = ck.finish()
    assert st["slots"] == len(rr) and st["rows_full"] == masked.shape[0] and st["max_err"] <= 1e-7


@pytest.mark.parametrize("plant", ["argmax", "conf", "decision"])
def test_checker_reports_planted_mistakes(plant):
    lg, masked, rr, jj, a, c, tau, U = _job(2)
    ck = DeferredChecker("bf16", lg.shape[-1], threads=2)
    ck.CHUNK_ROWS = 4
    slots = list(zip(rr.tolist(), jj.tolist()))
    rows_full = [(r, masked[r], tau, U[r].copy()) for r in range(masked.shape[0])]
    # a first, correct step
    ck.submit(1, ck.gather(lg, rr * 4 + jj), slots, a, c, rows_full)
    a2, c2 = a.copy(), c.copy()
    if plant == "argmax":
        a2[3] += 1
    elif plant == "conf":
        c2[3] += 2e-5
    else:
        r = rows_full[1][0]
        wrong = rows_full[1][3].copy()
        j = int(np.flatnonzero(masked[r] & ~wrong)[0]) if (masked[r] & ~wrong).any() else int(np.flatnonzero(wrong)[0])
        wrong[j] = not wrong[j]
        rows_full[1] = (r, masked[r], tau, wrong)
    ck.submit(2, ck.gather(lg, rr * 4 + jj), slots, a2, c2, rows_full)
    with pytest.raises(AssertionError, match="step 2"):
        ck.finish()
