"""GPU parity of dllm_step against the float64 oracle (element by element), through the C ABI."""
import numpy as np
import pytest

from oracle import pack as opack
from oracle import step as ostep
from tests.parity import CONF_TOL, check_decisions, check_scores
from workload import configs, synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import confidence_block_unmasking_amd  # noqa: F401  (fails loudly if the library is missing)


def _to_dev_logits(host, dtype):
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(host).view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(host)).cuda()


def gpu_step(logits_host, dtype, ids, mask, tau, p=None, b=None, pos_stride=None, row_stride=None, ws=None,
             offset=0, mask_offset=0, in_place=False):
    """Run dllm_step on host inputs; logits may be embedded in a larger strided buffer."""
    from confidence_block_unmasking_amd import api
    rows, L, V = logits_host.shape
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    if pos_stride is None and row_stride is None and offset == 0:
        lg = _to_dev_logits(logits_host, dtype)
        ps, rs = V, L * V
        base = lg
    else:
        ps = pos_stride or V
        rs = row_stride or L * ps
        total = offset + (rows - 1) * rs + (L - 1) * ps + V
        buf = np.full(total, 0x7FC0 if dtype == "bf16" else np.nan,
                      np.uint16 if dtype == "bf16" else np.float32)
        for r in range(rows):
            for j in range(L):
                s = offset + r * rs + j * ps
                buf[s:s + V] = logits_host[r, j]
        dev = _to_dev_logits(buf, dtype)
        base = dev[offset:]
    W = ids.shape[1]
    d_ids = torch.from_numpy(ids.astype(np.int32)).cuda()
    d_mask = torch.from_numpy(np.concatenate([np.full(mask_offset, 3, np.uint8),
                                              mask.astype(np.uint8).ravel()])).cuda()[mask_offset:].view(mask.shape)
    d_mask_out = d_mask if in_place else torch.full_like(d_mask, 77)
    d_tau = torch.from_numpy(np.asarray(tau, np.float32)).cuda()
    done = torch.full((rows,), 9, dtype=torch.uint8, device="cuda")
    acc = torch.full((rows,), -7, dtype=torch.int32, device="cuda")
    conf = torch.full((rows, L), 5.0, dtype=torch.float32, device="cuda")
    arg = torch.full((rows, L), -9, dtype=torch.int32, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    if ws is None:
        ws = api.new_workspace(rows, L, V, tdt)
    kw = {}
    if p is not None:
        kw = dict(p=torch.from_numpy(np.asarray(p, np.int32)).cuda(), b=torch.from_numpy(np.asarray(b, np.int32)).cuda())
    api.dllm_step(base, d_ids, d_mask, d_mask_out, d_tau, done, acc, ws, status, conf=conf, argmax=arg, rows=rows,
                  L=L, V=V, pos_stride=ps, row_stride=rs, **kw)
    torch.cuda.synchronize()
    return dict(ids=d_ids.cpu().numpy(), mask=d_mask_out.cpu().numpy(), done=done.cpu().numpy(),
                accept=acc.cpu().numpy(), conf=conf.cpu().numpy(), argmax=arg.cpu().numpy(),
                status=int(status.item()), mask_in_after=mask if in_place else d_mask.cpu().numpy())


def check_step(logits, dtype, ids, mask, tau, g, p=None, b=None):
    """Full element-by-element comparison of one GPU step with the oracle."""
    o = ostep.step(logits, dtype, ids, mask, tau, p, b)
    assert np.array_equal(g["mask_in_after"], mask), "mask_in was modified"
    err = check_scores(g["conf"], g["argmax"], o["conf"], o["argmax"])
    unscored = o["argmax"] < 0
    assert np.all(g["argmax"][unscored] == -1) and np.all(g["conf"][unscored] == -1.0)
    n_amb = check_decisions(g["conf"], o["conf"], mask, g["mask"], tau)
    # lockstep: the oracle's write-back with the GPU's decisions must give identical integers
    lk = ostep.step(logits, dtype, ids, mask, tau, conf_override=g["conf"].astype(np.float64))
    for k in ("ids", "mask", "done", "accept"):
        assert np.array_equal(g[k], lk[k]), k
    if n_amb == 0:
        for k in ("ids", "mask", "done", "accept"):
            assert np.array_equal(g[k], o[k]), k
    return err, n_amb


def _packed_step_inputs(w):
    W = opack.box_width(w.row_req, w.rows, w.p, w.b, w.L)
    pk = opack.pack(w.row_req, w.rows, w.L, W, w.pad_id, w.p, w.b, w.threshold, w.arena_off, w.arena, w.blk_mask)
    logits = synth.logits_cpu(w.rows, w.L, w.V, w.dtype, w.row_req, pk["b"], pk["mask"], w.logit_seed, w.sigma, w.umax)
    return pk, logits


@pytest.mark.parametrize("name", ["tiny-step", "llada-sync", "dream-dynamic-step"])
def test_step_parity_workloads(name):
    w = configs.make(name)
    pk, logits = _packed_step_inputs(w)
    print(f"{name}: rows={w.rows} L={w.L} V={w.V} masked={int(pk['mask'].sum())}", flush=True)
    g = gpu_step(logits, w.dtype, pk["box_ids"], pk["mask"], pk["threshold"], pk["p"], pk["b"])
    assert g["status"] == 0
    err, n_amb = check_step(logits, w.dtype, pk["box_ids"], pk["mask"], pk["threshold"], g, pk["p"], pk["b"])
    print(f"{name}: max conf error {err:.3g}, ambiguous rows {n_amb}")
    assert np.array_equal(g["ids"][:, :-w.L], pk["box_ids"][:, :-w.L])        # prompt columns untouched


def test_generator_gpu_matches_cpu():
    from confidence_block_unmasking_amd import api  # noqa: F401
    for name in ("tiny-step", "dream-dynamic-step"):
        w = configs.make(name)
        rows = min(w.rows, 8)
        rr = w.row_req[:rows]
        blk = w.b[rr].astype(np.int32)
        msk = w.blk_mask[rr]
        host = synth.logits_cpu(rows, w.L, w.V, w.dtype, rr, blk, msk, w.logit_seed, w.sigma, w.umax, fill_nan=True)
        tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
        dev = torch.empty((rows, w.L, w.V), dtype=tdt, device="cuda")
        synth.logits_gpu(dev, w.dtype, rows, w.L, w.V, torch.from_numpy(rr.astype(np.int32)).cuda(),
                         torch.from_numpy(blk).cuda(), torch.from_numpy(msk).cuda(), w.logit_seed, w.sigma, w.umax,
                         fill_nan=True)
        torch.cuda.synchronize()
        got = dev.view(torch.int16).cpu().numpy().view(np.uint16) if w.dtype == "bf16" else dev.cpu().numpy()
        if w.dtype == "bf16":
            assert np.array_equal(got, host)
        else:
            assert np.array_equal(got.view(np.uint32), host.view(np.uint32))


def _rand_case(rng, rows, L, V, dtype, p_mask=0.5, W_extra=3, scale=2.0, planted=12.0):
    x = rng.normal(0, scale, (rows, L, V)).astype(np.float32)
    for r in range(rows):
        for j in range(L):
            x[r, j, rng.integers(0, V)] += rng.uniform(0, planted)
    if dtype == "bf16":
        u = x.view(np.uint32).astype(np.uint64)
        logits = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    else:
        logits = x
    W = L + W_extra
    ids = rng.integers(0, V, (rows, W)).astype(np.int32)
    mask = (rng.random((rows, L)) < p_mask).astype(np.uint8)
    tau = rng.choice([0.5, 0.6, 0.7, 0.8, 0.9], rows).astype(np.float32)
    return logits, ids, mask, tau


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("rows,L,V", [(1, 1, 1), (3, 5, 7), (2, 32, 1000), (2, 32, 1001), (4, 64, 4099),
                                      (2, 100, 515), (1, 7, 65536), (5, 33, 8200), (2, 1024, 300)])
def test_step_shapes_and_ragged_tails(dtype, rows, L, V):
    rng = np.random.default_rng(rows * 1000 + L * 10 + V)
    logits, ids, mask, tau = _rand_case(rng, rows, L, V, dtype)
    mask[0, 0] = 1
    print(f"shape rows={rows} L={L} V={V} {dtype}", flush=True)
    g = gpu_step(logits, dtype, ids, mask, tau)
    assert g["status"] == 0
    check_step(logits, dtype, ids, mask, tau, g)


@pytest.mark.parametrize("case", range(64))
def test_step_random_sweep(case):
    # seeded random cases: shape, dtype, strides and offset, mask density, thresholds at the ends of
    # their range, in-place masks, a misaligned mask, p/b given or not; all against the oracle
    rng = np.random.default_rng(9000 + case)
    dtype = str(rng.choice(["fp32", "bf16"]))
    rows = int(rng.integers(1, 25))
    L = int(rng.choice([1, 2, 7, 16, 31, 32, 33, 64, 65, 100]))
    V = int(rng.integers(1, 6000))
    if rng.random() < 0.4:
        V = max(8, V - V % 8)                   # whole 16-byte vectors: the vector path
    V = max(1, min(V, 3_000_000 // (rows * L)))
    logits, ids, mask, tau = _rand_case(rng, rows, L, V, dtype, p_mask=float(rng.random()))
    if rng.random() < 0.3:
        mask[int(rng.integers(0, rows))] = 0    # a row with nothing masked
    if rng.random() < 0.3:
        mask[int(rng.integers(0, rows))] = 1    # a fully masked row
    tau = rng.choice([0.0, 0.2, 0.5, 0.9, 0.999, 1.0], rows).astype(np.float32)
    kw = {}
    if rng.random() < 0.5:
        ps = V + int(rng.integers(0, 9))
        kw = dict(pos_stride=ps, row_stride=L * ps + int(rng.integers(0, 9)), offset=int(rng.integers(0, 9)))
    in_place = bool(rng.random() < 0.3)
    moff = int(rng.integers(1, 16)) if rng.random() < 0.3 else 0
    pb = {}
    if rng.random() < 0.5:
        W = ids.shape[1]
        pb = dict(p=rng.integers(0, W - L + 1, rows).astype(np.int32), b=np.zeros(rows, np.int32))
    print(f"sweep case {case}: rows={rows} L={L} V={V} {dtype} {kw} in_place={in_place} mask_offset={moff} "
          f"pb={bool(pb)}", flush=True)
    g = gpu_step(logits, dtype, ids, mask.copy(), tau, in_place=in_place, mask_offset=moff, **kw, **pb)
    assert g["status"] == 0
    check_step(logits, dtype, ids, mask, tau, g, **pb)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_step_strided_and_unaligned(dtype):
    rng = np.random.default_rng(17)
    rows, L, V = 3, 6, 2051
    logits, ids, mask, tau = _rand_case(rng, rows, L, V, dtype)
    for ps, rs, off in [(V + 5, None, 0), (V, L * V + 3, 1), (2056, 2056 * L + 8, 8)]:
        print(f"strides pos={ps} row={rs} offset={off}", flush=True)
        g = gpu_step(logits, dtype, ids, mask, tau, pos_stride=ps, row_stride=rs, offset=off)
        check_step(logits, dtype, ids, mask, tau, g)


@pytest.mark.parametrize("rows,L,V,dtype,p_mask,moff", [(400, 40, 130, "fp32", 0.3, 0), (3000, 5, 64, "bf16", 0.9, 0),
                                                       (700, 24, 96, "bf16", 0.6, 1)])
def test_step_many_slots(rows, L, V, dtype, p_mask, moff):
    # boxes of more slots than one pass of the scoring prologue covers, rows shorter than the 16
    # mask bytes a thread reads, and a mask that is not 16-byte aligned (byte loads)
    rng = np.random.default_rng(rows + L)
    logits, ids, mask, tau = _rand_case(rng, rows, L, V, dtype, p_mask=p_mask)
    print(f"many slots rows={rows} L={L} V={V} {dtype} mask offset {moff}", flush=True)
    g = gpu_step(logits, dtype, ids, mask, tau, mask_offset=moff)
    assert g["status"] == 0
    check_step(logits, dtype, ids, mask, tau, g)


@pytest.mark.parametrize("per_cu", [24, 140])
@pytest.mark.parametrize("delta", [-32, 0, 32])
def test_step_at_the_grid_thresholds(per_cu, delta):
    # boxes of just under, at and just over 24 and 140 chunks per compute unit (one chunk per slot
    # here), where the scoring grid changes from one to two to four workgroups per unit
    cu = torch.cuda.get_device_properties(0).multi_processor_count
    S = per_cu * cu + delta
    L = 32
    rows = S // L
    rng = np.random.default_rng(per_cu * 100 + delta)
    logits, ids, mask, tau = _rand_case(rng, rows, L, 64, "bf16", p_mask=0.5)
    print(f"grid threshold {per_cu}/CU x {cu} CUs {delta:+d}: rows={rows} L={L}", flush=True)
    g = gpu_step(logits, "bf16", ids, mask, tau)
    assert g["status"] == 0
    check_step(logits, "bf16", ids, mask, tau, g)


def test_step_at_the_position_limit():
    # rows * L = DLLM_MAX_POSITIONS slots in one call (rows = DLLM_MAX_ROWS)
    from confidence_block_unmasking_amd import _lib
    rows = _lib.MAX_ROWS
    L = _lib.MAX_POSITIONS // rows
    rng = np.random.default_rng(5)
    logits, ids, mask, tau = _rand_case(rng, rows, L, 8, "bf16", p_mask=0.5)
    print(f"position limit rows={rows} L={L}", flush=True)
    g = gpu_step(logits, "bf16", ids, mask, tau)
    assert g["status"] == 0
    check_step(logits, "bf16", ids, mask, tau, g)


def test_binding_rejects_logits_smaller_than_the_shape():
    # the C ABI cannot see a tensor's extent; the binding refuses shapes and strides that would
    # read past the logits' storage, before anything is launched
    from confidence_block_unmasking_amd import api
    rows, L, V = 2, 4, 64
    lg = torch.zeros(rows * L * V - 1, dtype=torch.bfloat16, device="cuda")
    mask = torch.ones(rows * L, dtype=torch.uint8, device="cuda")
    ws = api.new_workspace(rows, L, V, torch.bfloat16)
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    with pytest.raises(ValueError, match="reach"):
        api.dllm_step_score(lg, mask, ws, st, rows=rows, L=L, V=V)
    full = torch.zeros(rows * L * V + 8, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError, match="reach"):
        api.dllm_step_score(full[9:], mask, ws, st, rows=rows, L=L, V=V)
    with pytest.raises(ValueError, match="reach"):
        api.dllm_step_score(full, mask, ws, st, rows=rows, L=L, V=V, pos_stride=V + 2)
    api.dllm_step_score(full[8:], mask, ws, st, rows=rows, L=L, V=V)   # exactly enough
    torch.cuda.synchronize()
    assert int(st.item()) == 0


def test_step_halves_equal_step():
    # dllm_step_score then dllm_step_decide gives dllm_step's outputs bit for bit
    from confidence_block_unmasking_amd import api
    w = configs.dream_step()
    pk, logits = _packed_step_inputs(w)
    a = gpu_step(logits, w.dtype, pk["box_ids"], pk["mask"], pk["threshold"])
    rows, L, V = logits.shape
    lg = _to_dev_logits(logits, w.dtype)
    ids = torch.from_numpy(pk["box_ids"].astype(np.int32)).cuda()
    mask = torch.from_numpy(pk["mask"].astype(np.uint8)).cuda()
    mout = torch.empty_like(mask)
    tau = torch.from_numpy(pk["threshold"].astype(np.float32)).cuda()
    done = torch.empty(rows, dtype=torch.uint8, device="cuda")
    acc = torch.empty(rows, dtype=torch.int32, device="cuda")
    conf = torch.empty((rows, L), dtype=torch.float32, device="cuda")
    arg = torch.empty((rows, L), dtype=torch.int32, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    ws = api.new_workspace(rows, L, V, torch.bfloat16)
    api.dllm_step_score(lg, mask, ws, status)
    api.dllm_step_decide(torch.bfloat16, rows, L, V, ids, mask, mout, tau, done, acc, ws, status, conf=conf,
                         argmax=arg)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    b = dict(ids=ids.cpu().numpy(), mask=mout.cpu().numpy(), done=done.cpu().numpy(), accept=acc.cpu().numpy(),
             conf=conf.cpu().numpy(), argmax=arg.cpu().numpy())
    for k in b:
        assert np.array_equal(a[k], b[k]), k
    # the kernel-bound timed launch leaves the same partials: the same decisions again
    ids.copy_(torch.from_numpy(pk["box_ids"].astype(np.int32)))
    ws.fill_(0xA5)
    ev = api.KernelEvents()
    api.dllm_step_score_timed(lg, mask, ws, status, ev)
    api.dllm_step_decide(torch.bfloat16, rows, L, V, ids, mask, mout, tau, done, acc, ws, status, conf=conf,
                         argmax=arg)
    ms = ev.elapsed_ms()
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    assert 0.0 < ms < 1000.0
    c = dict(ids=ids.cpu().numpy(), mask=mout.cpu().numpy(), done=done.cpu().numpy(), accept=acc.cpu().numpy(),
             conf=conf.cpu().numpy(), argmax=arg.cpu().numpy())
    for k in c:
        assert np.array_equal(a[k], c[k]), k
    # the whole step timed from the scoring kernel's start to the deciding kernel's end: same outputs,
    # and an interval that holds the scoring kernel's
    ids.copy_(torch.from_numpy(pk["box_ids"].astype(np.int32)))
    ws.fill_(0x5A)
    ev2 = api.KernelEvents()
    api.dllm_step_timed(lg, ids, mask, mout, tau, done, acc, ws, status, ev2, conf=conf, argmax=arg)
    ms2 = ev2.elapsed_ms()
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    assert 0.5 * ms < ms2 < 1000.0
    d = dict(ids=ids.cpu().numpy(), mask=mout.cpu().numpy(), done=done.cpu().numpy(), accept=acc.cpu().numpy(),
             conf=conf.cpu().numpy(), argmax=arg.cpu().numpy())
    for k in d:
        assert np.array_equal(a[k], d[k]), k


def test_step_in_place_mask_update():
    # mask_out = mask_in: the same results as with two buffers
    w = configs.dream_step()
    pk, logits = _packed_step_inputs(w)
    a = gpu_step(logits, w.dtype, pk["box_ids"], pk["mask"], pk["threshold"])
    b = gpu_step(logits, w.dtype, pk["box_ids"], pk["mask"], pk["threshold"], in_place=True)
    for k in ("ids", "mask", "done", "accept", "argmax", "conf"):
        assert np.array_equal(a[k], b[k]), k


def test_step_mask_patterns_and_ties():
    rows, L, V = 6, 8, 300
    logits = np.zeros((rows, L, V), np.float32)
    logits[1, :, 17] = 3.0                      # same value at one index: ties across slots
    logits[2, :, 5] = 9.0
    logits[2, :, 200] = 9.0                     # tie inside a row of the vocabulary: lowest index wins
    logits[3, 2, 10] = 50.0                     # one very confident slot
    logits[4] = np.random.default_rng(3).normal(0, 1, (L, V))
    ids = np.arange(rows * (L + 2), dtype=np.int32).reshape(rows, L + 2)
    mask = np.ones((rows, L), np.uint8)
    mask[0] = 0                                 # nothing masked: done, accept = L, untouched
    mask[5] = 0
    mask[5, 7] = 1                              # a single masked slot: the fallback finishes the block
    tau = np.array([0.9, 0.9, 0.4, 0.9, 0.99, 0.9], np.float32)
    g = gpu_step(logits, "fp32", ids, mask, tau)
    check_step(logits, "fp32", ids, mask, tau, g)
    assert g["done"].tolist() == [1, 0, 1, 0, 0, 1]           # row 2: every slot clears tau = 0.4
    assert g["accept"].tolist() == [L, 0, L, 0, 0, L]
    assert np.all(g["argmax"][2] == 5)
    assert g["mask"][3].tolist() == [1, 1, 0, 1, 1, 1, 1, 1]     # only the confident slot
    assert g["mask"][1].sum() == L - 1 and g["mask"][1, 0] == 0   # fallback tie across slots -> slot 0
    assert np.array_equal(g["ids"][0], ids[0])


def test_step_threshold_equal_is_not_above():
    # two slots with softmax confidence exactly 0.5 (logits (0, 0) over V = 2) and tau = 0.5
    logits = np.zeros((1, 2, 2), np.float32)
    ids = np.zeros((1, 2), np.int32)
    mask = np.ones((1, 2), np.uint8)
    g = gpu_step(logits, "fp32", ids, mask, np.array([0.5], np.float32))
    assert g["conf"][0].tolist() == [0.5, 0.5]
    assert g["mask"][0].tolist() == [0, 1]      # no slot exceeds: fallback to the lowest slot


def test_step_many_chunks_merge_path():
    # V large enough for more than 64 chunks per slot (the multi-block merge)
    rng = np.random.default_rng(8)
    logits, ids, mask, tau = _rand_case(rng, 1, 3, 300000, "bf16", p_mask=1.0)
    logits[0, 1, 299999] = 0x4200                 # max at the very last element
    g = gpu_step(logits, "bf16", ids, mask, tau)
    check_step(logits, "bf16", ids, mask, tau, g)


def test_step_never_reads_unmasked_slots():
    w = configs.tiny_step()
    pk, logits = _packed_step_inputs(w)           # unmasked slots hold NaN
    assert np.isnan(logits[pk["mask"] == 0]).all()
    g = gpu_step(logits, w.dtype, pk["box_ids"], pk["mask"], pk["threshold"])
    assert np.all(np.isfinite(g["conf"]))
    check_step(logits, w.dtype, pk["box_ids"], pk["mask"], pk["threshold"], g)


def test_step_status_for_row_that_does_not_fit():
    rng = np.random.default_rng(2)
    logits, ids, mask, tau = _rand_case(rng, 2, 4, 64, "fp32", W_extra=2)
    g = gpu_step(logits, "fp32", ids, mask, tau, p=[2, 3], b=[0, 0])   # row 1 needs 7 > W = 6
    assert g["status"] == 2
    check_step(logits, "fp32", ids, mask, tau, g)                      # the step still completes


def test_step_determinism_and_batch_invariance():
    w = configs.dream_step()
    pk, logits = _packed_step_inputs(w)
    a = gpu_step(logits, w.dtype, pk["box_ids"], pk["mask"], pk["threshold"])
    b = gpu_step(logits, w.dtype, pk["box_ids"], pk["mask"], pk["threshold"])
    for k in a:
        assert np.array_equal(np.asarray(a[k]), np.asarray(b[k])), k
    # the same rows in another order, with half of the batch removed: identical bits per row
    rng = np.random.default_rng(4)
    sel = rng.permutation(w.rows)[:w.rows // 2]
    c = gpu_step(logits[sel], w.dtype, pk["box_ids"][sel], pk["mask"][sel], pk["threshold"][sel])
    for k in ("ids", "mask", "done", "accept", "argmax"):
        assert np.array_equal(c[k], a[k][sel]), k
    assert np.array_equal(c["conf"].view(np.uint32), a["conf"][sel].view(np.uint32))


def test_workspace_reused_across_shapes():
    from confidence_block_unmasking_amd import api
    rng = np.random.default_rng(6)
    ws = api.new_workspace(64, 64, 70000, torch.bfloat16)
    for rows, L, V in [(5, 16, 70000), (64, 64, 3000), (2, 3, 65000), (17, 40, 9000)]:
        logits, ids, mask, tau = _rand_case(rng, rows, L, V, "bf16", p_mask=0.7)
        g = gpu_step(logits, "bf16", ids, mask, tau, ws=ws)
        check_step(logits, "bf16", ids, mask, tau, g)
    assert CONF_TOL == 1e-5


@pytest.mark.parametrize("case", range(6))
def test_decide_reports_unmasked_and_fallback(case):
    """dllm_step_decide's per-row report: the slots it unmasked and whether the single-slot fallback
    applied, against the oracle's (the Dream-shaped step, then random boxes with thresholds 0.5..1
    where some rows fall back and some have no masked slot)."""
    from confidence_block_unmasking_amd import api
    from tests.parity import ambiguous_row
    rng = np.random.default_rng(900 + case)
    if case == 0:
        w = configs.dream_step()
        pk, logits = _packed_step_inputs(w)
        ids, mask, tau, dtype = pk["box_ids"], pk["mask"], pk["threshold"], w.dtype
    else:
        rows, L, V = int(rng.integers(1, 40)), int(rng.choice([4, 16, 32, 64])), int(rng.integers(50, 3000))
        logits, ids, mask, tau = _rand_case(rng, rows, L, V, "fp32", p_mask=float(rng.uniform(0.1, 0.9)))
        tau = rng.choice([0.5, 0.9, 0.99, 1.0], rows).astype(np.float32)
        mask[0] = 0
        dtype = "fp32"
    rows, L, V = logits.shape
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    lg = _to_dev_logits(logits, dtype)
    d_ids = torch.from_numpy(ids.astype(np.int32)).cuda()
    d_mask = torch.from_numpy(mask.astype(np.uint8)).cuda()
    mout = torch.empty_like(d_mask)
    d_tau = torch.from_numpy(np.asarray(tau, np.float32)).cuda()
    done = torch.empty(rows, dtype=torch.uint8, device="cuda")
    acc = torch.empty(rows, dtype=torch.int32, device="cuda")
    conf = torch.empty((rows, L), dtype=torch.float32, device="cuda")
    unm = torch.full((rows,), -3, dtype=torch.int32, device="cuda")
    fb = torch.full((rows,), 7, dtype=torch.uint8, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    ws = api.new_workspace(rows, L, V, tdt)
    api.dllm_step_score(lg, d_mask, ws, status)
    api.dllm_step_decide(tdt, rows, L, V, d_ids, d_mask, mout, d_tau, done, acc, ws, status, conf=conf,
                         unmasked=unm, fallback=fb)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    g_unm, g_fb, g_conf = unm.cpu().numpy(), fb.cpu().numpy(), conf.cpu().numpy().astype(np.float64)
    o = ostep.step(logits, dtype, ids, mask, tau)
    n_amb = 0
    for r in range(rows):
        masked = mask[r] != 0
        own, own_fb = ostep.decide(g_conf[r], masked, tau[r], return_fallback=True)
        assert g_unm[r] == int(own.sum()) and g_fb[r] == int(own_fb), r
        if ambiguous_row(o["conf"][r], masked, tau[r]):
            n_amb += 1
            continue
        assert g_unm[r] == o["unmasked"][r] and g_fb[r] == o["fallback"][r], r
    assert g_fb[0] == 0 and g_unm[0] == 0 or case == 0
    print(f"case {case}: rows {rows}, fallback rows {int(g_fb.sum())}, ambiguous {n_amb}", flush=True)
