"""GPU parity of the vocabulary-sharded step (dllm_step_score_shard + dllm_step_decide_shards)."""
import numpy as np
import pytest

from oracle import shard as osh
from oracle import step as ostep
from tests.parity import CONF_TOL, check_decisions
from tests.test_gpu_step import _rand_case, _to_dev_logits, gpu_step

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import confidence_block_unmasking_amd  # noqa: F401


def gpu_sharded(logits_host, dtype, ids, mask, tau, T, order=None):
    from confidence_block_unmasking_amd import api
    rows, L, V = logits_host.shape
    lg = _to_dev_logits(logits_host, dtype).reshape(-1)
    pts = osh.split_points(V, T)
    d_ids = torch.from_numpy(ids.astype(np.int32)).cuda()
    d_mask = torch.from_numpy(mask.astype(np.uint8)).cuda()
    d_out = torch.full_like(d_mask, 77)
    d_tau = torch.from_numpy(np.asarray(tau, np.float32)).cuda()
    done = torch.full((rows,), 9, dtype=torch.uint8, device="cuda")
    acc = torch.full((rows,), -7, dtype=torch.int32, device="cuda")
    conf = torch.full((rows, L), 5.0, dtype=torch.float32, device="cuda")
    arg = torch.full((rows, L), -9, dtype=torch.int32, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    tri = api.new_triples(rows, L, T)
    for t in (order or range(T)):
        Vt = pts[t + 1] - pts[t]
        ws = api.new_workspace(rows, L, Vt, lg.dtype)
        api.dllm_step_score_shard(lg[pts[t]:], d_mask, ws, tri, t, T, pts[t], status, rows=rows, L=L, V_shard=Vt,
                                  pos_stride=V, row_stride=L * V)
    api.dllm_step_decide_shards(T, tri, rows, L, V, d_ids, d_mask, d_out, d_tau, done, acc, status, conf=conf,
                                argmax=arg)
    torch.cuda.synchronize()
    recs = tri.view(torch.float32).view(rows, L, T, 4).cpu().numpy()
    return dict(ids=d_ids.cpu().numpy(), mask=d_out.cpu().numpy(), done=done.cpu().numpy(),
                accept=acc.cpu().numpy(), conf=conf.cpu().numpy(), argmax=arg.cpu().numpy(),
                status=int(status.item()), records=recs)


@pytest.mark.parametrize("rows,L,V,T,dtype", [(3, 32, 152064, 8, "bf16"), (2, 16, 1001, 3, "bf16"),
                                              (2, 8, 5000, 1, "fp32"), (4, 32, 20011, 5, "fp32"),
                                              (2, 4, 70000, 64, "bf16")])
def test_sharded_step_parity(rows, L, V, T, dtype):
    rng = np.random.default_rng(V + T)
    logits, ids, mask, tau = _rand_case(rng, rows, L, V, dtype, p_mask=0.8)
    mask[0, 0] = 1
    print(f"shards rows={rows} L={L} V={V} T={T} {dtype}", flush=True)
    g = gpu_sharded(logits, dtype, ids, mask, tau, T)
    assert g["status"] == 0
    pts = osh.split_points(V, T)
    o = ostep.step(logits, dtype, ids, mask, tau)
    for r in range(rows):
        for j in range(L):
            if not mask[r, j]:
                continue
            x = ostep.widen(logits[r, j], dtype)
            trip = [osh.shard_triple(x[pts[t]:pts[t + 1]], pts[t]) for t in range(T)]
            for t in range(T):                     # each shard's record
                m, a, S = trip[t]
                rec = g["records"][r, j, t]
                assert rec[0] == np.float32(m) and rec[2].view(np.int32) == a
                assert abs(rec[1] - S) <= 1e-5 * S
            _, a, _, c = osh.combine(trip)          # the combination
            assert g["argmax"][r, j] == a == o["argmax"][r, j]
            assert abs(float(g["conf"][r, j]) - c) <= CONF_TOL
    n_amb = check_decisions(g["conf"], o["conf"], mask, g["mask"], tau)
    lk = ostep.step(logits, dtype, ids, mask, tau, conf_override=g["conf"].astype(np.float64))
    for k in ("ids", "mask", "done", "accept"):
        assert np.array_equal(g[k], lk[k]), k
    # against the unsharded GPU step: same argmax, confidences within rounding of each other
    u = gpu_step(logits, dtype, ids, mask, tau)
    assert np.array_equal(u["argmax"], g["argmax"])
    assert np.max(np.abs(u["conf"] - g["conf"])) <= 2e-6
    if n_amb == 0:
        for k in ("ids", "mask", "done", "accept"):
            assert np.array_equal(g[k], u[k]), k


def test_shard_order_does_not_change_bits():
    rng = np.random.default_rng(5)
    logits, ids, mask, tau = _rand_case(rng, 3, 16, 9000, "bf16", p_mask=0.9)
    a = gpu_sharded(logits, "bf16", ids, mask, tau, 4)
    b = gpu_sharded(logits, "bf16", ids, mask, tau, 4, order=[3, 1, 0, 2])
    for k in ("ids", "mask", "done", "accept", "argmax"):
        assert np.array_equal(a[k], b[k]), k
    assert np.array_equal(a["conf"].view(np.uint32), b["conf"].view(np.uint32))
