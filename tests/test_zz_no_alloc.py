"""dllm_step_noalloc, the step for callers that cannot allocate (its partials live in the library's
fixed per-GPU scratch array), against dllm_step with a caller workspace: two calls in a row, the
second on a smaller input, must give dllm_step's outputs bit for bit (the same kernels run)."""
import numpy as np
import pytest

from workload import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import confidence_block_unmasking_amd  # noqa: F401  (fails loudly if the library is missing)


def _case(rows, L, V, dtype, seed, W):
    """Device inputs: generator logits for every slot, a seeded mask, thresholds, p and b that fit."""
    rng = np.random.default_rng(seed)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    lg = torch.empty((rows, L, V), dtype=tdt, device="cuda")
    full = torch.ones(rows * L, dtype=torch.uint8, device="cuda")
    rr = torch.arange(rows, dtype=torch.int32, device="cuda")
    bb = torch.zeros(rows, dtype=torch.int32, device="cuda")
    synth.logits_gpu(lg, dtype, rows, L, V, rr, bb, full, 4242 + seed, 2, 14)
    mask = (rng.random((rows, L)) < 0.6).astype(np.uint8)
    mask[0] = 1
    mask[-1] = 0
    p = rng.integers(1, W - L + 1, rows).astype(np.int32)
    return dict(logits=lg, mask=mask, tau=rng.choice([0.5, 0.7, 0.9], rows).astype(np.float32),
                ids=rng.integers(0, V, (rows, W)).astype(np.int32), p=p, b=np.zeros(rows, np.int32))


def _run(c, noalloc):
    from confidence_block_unmasking_amd import api
    rows, L, V = c["logits"].shape
    out = dict(ids=torch.from_numpy(c["ids"]).cuda(),
               mask_in=torch.from_numpy(c["mask"]).cuda(),
               mask_out=torch.full(c["mask"].shape, 77, dtype=torch.uint8, device="cuda"),
               done=torch.full((rows,), 9, dtype=torch.uint8, device="cuda"),
               acc=torch.full((rows,), -7, dtype=torch.int32, device="cuda"),
               conf=torch.full((rows, L), 5.0, dtype=torch.float32, device="cuda"),
               arg=torch.full((rows, L), -9, dtype=torch.int32, device="cuda"),
               status=torch.zeros(1, dtype=torch.int32, device="cuda"))
    tau = torch.from_numpy(c["tau"]).cuda()
    p, b = torch.from_numpy(c["p"]).cuda(), torch.from_numpy(c["b"]).cuda()
    if noalloc:
        api.dllm_step_noalloc(c["logits"], out["ids"], out["mask_in"], out["mask_out"], tau, out["done"], out["acc"],
                              out["status"], p=p, b=b, conf=out["conf"], argmax=out["arg"])
    else:
        ws = api.new_workspace(rows, L, V, c["logits"].dtype)
        api.dllm_step(c["logits"], out["ids"], out["mask_in"], out["mask_out"], tau, out["done"], out["acc"], ws,
                      out["status"], p=p, b=b, conf=out["conf"], argmax=out["arg"])
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in out.items()}


def test_noalloc_step_equals_dllm_step_on_two_calls_in_a_row():
    """A Dream-shaped box (64 x 32 slots, V = 152064 bf16), then a smaller one (5 x 8, V = 1001 fp32,
    a ragged vocabulary): the second call finds the first call's partials in the scratch array."""
    from oracle import step as ostep
    for rows, L, V, dtype, W in ((64, 32, 152064, "bf16", 600), (5, 8, 1001, "fp32", 40)):
        print(f"noalloc: rows={rows} L={L} V={V} {dtype}", flush=True)
        c = _case(rows, L, V, dtype, rows, W)
        ref = _run(c, noalloc=False)
        got = _run(c, noalloc=True)
        assert int(got["status"][0]) == 0 and int(ref["status"][0]) == 0
        for k in ("ids", "mask_out", "done", "acc", "arg"):
            assert np.array_equal(got[k], ref[k]), k
        assert np.array_equal(got["conf"].view(np.uint32), ref["conf"].view(np.uint32)), "conf bits"
        # and a few rows against the oracle itself
        host = c["logits"].cpu()
        host = host.view(torch.int16).numpy().view(np.uint16) if dtype == "bf16" else host.numpy()
        for r in (0, rows - 2):
            o = ostep.step(host[r:r + 1], dtype, c["ids"][r:r + 1], c["mask"][r:r + 1], c["tau"][r:r + 1])
            assert np.array_equal(got["arg"][r:r + 1], o["argmax"])
            assert np.abs(got["conf"][r:r + 1].astype(np.float64) - o["conf"]).max() <= 1e-5
            assert np.array_equal(got["ids"][r:r + 1], o["ids"]) and np.array_equal(got["mask_out"][r:r + 1], o["mask"])


def test_noalloc_step_at_the_scratch_capacity():
    """The largest box the scratch array holds at V = 152064 bf16 (3942 x 7 = 27 594 slots of 38
    chunks: 16 777 056 bytes of partials, 160 short of 16 MiB), then the Dream-shaped box again:
    equal to dllm_step."""
    from confidence_block_unmasking_amd import _lib, api
    rows, L, V = 3942, 7, 152064
    assert api.dllm_step_workspace_bytes(rows, L, V) <= _lib.NOALLOC_SCRATCH_BYTES
    assert api.dllm_step_workspace_bytes(rows + 1, L, V) > _lib.NOALLOC_SCRATCH_BYTES
    for rows, L, W in ((3942, 7, 40), (64, 32, 600)):
        print(f"noalloc capacity: rows={rows} L={L} V={V} bf16", flush=True)
        c = _case(rows, L, V, "bf16", 7 + rows, W)
        ref = _run(c, noalloc=False)
        got = _run(c, noalloc=True)
        assert int(got["status"][0]) == 0 and int(ref["status"][0]) == 0
        for k in ("ids", "mask_out", "done", "acc", "arg"):
            assert np.array_equal(got[k], ref[k]), k
        assert np.array_equal(got["conf"].view(np.uint32), ref["conf"].view(np.uint32)), "conf bits"
        del c
        torch.cuda.empty_cache()
