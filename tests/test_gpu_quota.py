"""GPU parity of the fixed per-step quota rule (dllm_step_quota) against the float64 oracle."""
import numpy as np
import pytest

from oracle import quota as oquota
from tests.parity import CONF_TOL, check_quota_decisions, check_scores
from tests.test_gpu_step import _rand_case, _to_dev_logits

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import confidence_block_unmasking_amd  # noqa: F401


def gpu_quota(logits_host, dtype, ids, mask, S, halves=False):
    from confidence_block_unmasking_amd import api
    rows, L, V = logits_host.shape
    lg = _to_dev_logits(logits_host, dtype)
    d_ids = torch.from_numpy(ids.astype(np.int32)).cuda()
    d_mask = torch.from_numpy(mask.astype(np.uint8)).cuda()
    d_out = torch.full_like(d_mask, 77)
    done = torch.full((rows,), 9, dtype=torch.uint8, device="cuda")
    acc = torch.full((rows,), -7, dtype=torch.int32, device="cuda")
    conf = torch.full((rows, L), 5.0, dtype=torch.float32, device="cuda")
    arg = torch.full((rows, L), -9, dtype=torch.int32, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    ws = api.new_workspace(rows, L, V, lg.dtype)
    if halves:
        api.dllm_step_score(lg, d_mask, ws, status)
        api.dllm_step_decide_quota(lg.dtype, rows, L, V, d_ids, d_mask, d_out, S, done, acc, ws, status, conf=conf,
                                   argmax=arg)
    else:
        api.dllm_step_quota(lg, d_ids, d_mask, d_out, S, done, acc, ws, status, conf=conf, argmax=arg)
    torch.cuda.synchronize()
    return dict(ids=d_ids.cpu().numpy(), mask=d_out.cpu().numpy(), done=done.cpu().numpy(),
                accept=acc.cpu().numpy(), conf=conf.cpu().numpy(), argmax=arg.cpu().numpy(), status=int(status.item()))


def check_quota_step(logits, dtype, ids, mask, S, g):
    o = oquota.step_quota(logits, dtype, ids, mask, S)
    check_scores(g["conf"], g["argmax"], o["conf"], o["argmax"])
    n_amb = check_quota_decisions(g["conf"], o["conf"], mask, g["mask"], S)
    lk = oquota.step_quota(logits, dtype, ids, mask, S, conf_override=g["conf"].astype(np.float64))
    for k in ("ids", "mask", "done", "accept"):
        assert np.array_equal(g[k], lk[k]), k
    if n_amb == 0:
        for k in ("ids", "mask", "done", "accept"):
            assert np.array_equal(g[k], o[k]), k
    return n_amb


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("rows,L,V,S", [(4, 32, 1024, 32), (3, 32, 5000, 10), (5, 64, 2051, 32), (2, 7, 300, 3),
                                        (6, 100, 777, 200), (2, 1024, 130, 32)])
def test_quota_parity_random(dtype, rows, L, V, S):
    rng = np.random.default_rng(rows * 100 + L + S)
    logits, ids, mask, _ = _rand_case(rng, rows, L, V, dtype, p_mask=0.7)
    mask[0, :] = 1                                   # a row at the start of its block
    print(f"quota rows={rows} L={L} V={V} S={S} {dtype}", flush=True)
    g = gpu_quota(logits, dtype, ids, mask, S)
    assert g["status"] == 0
    check_quota_step(logits, dtype, ids, mask, S, g)
    h = gpu_quota(logits, dtype, ids, mask, S, halves=True)
    for k in ("ids", "mask", "done", "accept", "conf", "argmax"):
        assert np.array_equal(g[k], h[k]), k


@pytest.mark.parametrize("case", range(32))
def test_quota_random_sweep(case):
    # seeded random shapes, dtypes, mask densities and steps per block (including S > L and S = 1),
    # through both the one-call step and its halves
    rng = np.random.default_rng(7000 + case)
    dtype = str(rng.choice(["fp32", "bf16"]))
    rows = int(rng.integers(1, 17))
    L = int(rng.choice([1, 3, 8, 16, 32, 33, 64, 65, 100]))
    V = int(rng.integers(1, 5000))
    V = max(1, min(V, 2_000_000 // (rows * L)))
    S = int(rng.choice([1, 2, 5, 8, 16, 32, 64, 200]))
    logits, ids, mask, _ = _rand_case(rng, rows, L, V, dtype, p_mask=float(rng.random()))
    if rng.random() < 0.3:
        mask[int(rng.integers(0, rows))] = 1
    if rng.random() < 0.3:
        mask[int(rng.integers(0, rows))] = 0
    halves = bool(rng.random() < 0.5)
    print(f"quota sweep case {case}: rows={rows} L={L} V={V} S={S} {dtype} halves={halves}", flush=True)
    g = gpu_quota(logits, dtype, ids, mask, S, halves=halves)
    assert g["status"] == 0
    check_quota_step(logits, dtype, ids, mask, S, g)


@pytest.mark.parametrize("L,S", [(32, 32), (32, 10), (7, 3), (64, 32), (5, 8), (40, 1), (65, 9), (100, 7)])
def test_quota_count_for_every_masked_count(L, S):
    # row m has m masked slots: it unmasks exactly quota_for_remaining(L, S, m)
    rng = np.random.default_rng(L * 7 + S)
    rows, V = L + 1, 64
    logits, ids, _, _ = _rand_case(rng, rows, L, V, "fp32")
    mask = np.zeros((rows, L), np.uint8)
    for m in range(rows):
        mask[m, rng.permutation(L)[:m]] = 1
    g = gpu_quota(logits, "fp32", ids, mask, S)
    for m in range(rows):
        unm = int((mask[m] != 0).sum() - (g["mask"][m] != 0).sum())
        assert unm == oquota.quota_for_remaining(L, S, m), m
    check_quota_step(logits, "fp32", ids, mask, S, g)


@pytest.mark.parametrize("L,S", [(32, 32), (32, 10), (16, 5)])
def test_quota_block_finishes_in_min_S_L_steps(L, S):
    # repeated steps from a fully masked block follow the schedule and finish in min(S, L) steps
    rng = np.random.default_rng(9)
    rows, V = 3, 500
    mask = np.ones((rows, L), np.uint8)
    ids = rng.integers(0, V, (rows, L + 2)).astype(np.int32)
    sched = oquota.quota_schedule(L, S)
    steps = 0
    while mask.any():
        logits, _, _, _ = _rand_case(rng, rows, L, V, "fp32")
        g = gpu_quota(logits, "fp32", ids, mask, S)
        check_quota_step(logits, "fp32", ids, mask, S, g)
        unm = (mask != 0).sum(1) - (g["mask"] != 0).sum(1)
        assert steps >= S or np.all(unm == sched[steps])
        ids, mask = g["ids"], g["mask"]
        steps += 1
        assert (g["done"] == (~mask.any(1))).all()
    assert steps == min(S, L)
