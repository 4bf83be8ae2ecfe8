"""Checks of the seeded input generators (workload package): determinism, laws, layouts."""
import numpy as np
import pytest

from workload import configs, synth


def _f(u16):
    return (u16.astype(np.uint32) << 16).view(np.float32)


def test_generator_is_deterministic_and_keyed():
    a = synth.row_cpu(4096, "fp32", 7, 3, 1, 5, 9, 2, 14)
    b = synth.row_cpu(4096, "fp32", 7, 3, 1, 5, 9, 2, 14)
    assert np.array_equal(a, b)
    for other in [(8, 3, 1, 5, 9), (7, 4, 1, 5, 9), (7, 3, 2, 5, 9), (7, 3, 1, 6, 9), (7, 3, 1, 5, 8)]:
        c = synth.row_cpu(4096, "fp32", *other, 2, 14)
        assert not np.array_equal(a, c)


def test_generator_noise_law_irwin_hall():
    # sigma = 1, no planted offset (umax = 0): mean 0, sd 1, support within +-6
    x = np.concatenate([synth.row_cpu(65536, "fp32", 11, q, 0, j, 5, 1, 0) for q in range(4) for j in range(4)])
    assert abs(x.mean()) < 0.01
    assert abs(x.std() - 1.0) < 0.01
    assert x.max() <= 6.0 and x.min() >= -6.0
    # values are multiples of 2^-20 * 16
    assert np.all(np.mod(x * 2**20, 16) == 0)


def test_generator_planted_token_and_offset():
    V = 2048
    seen = []
    for j in range(64):
        t = synth.planted_cpu(V, 5, 1, 0, j)
        assert 0 <= t < V
        seen.append(t)
        base = synth.row_cpu(V, "fp32", 5, 1, 0, j, 10, 2, 0)
        hot = synth.row_cpu(V, "fp32", 5, 1, 0, j, 10, 2, 14)
        diff = hot - base
        assert np.count_nonzero(diff) <= 1
        assert 0 <= diff[t] < 14 and np.all(np.delete(diff, t) == 0)
    assert len(set(seen)) > 50                                 # spread over the vocabulary


def test_generator_bf16_is_rne_of_fp32():
    f = synth.row_cpu(8192, "fp32", 3, 2, 1, 0, 4, 2, 14)
    h = synth.row_cpu(8192, "bf16", 3, 2, 1, 0, 4, 2, 14)
    u = f.view(np.uint32).astype(np.uint64)
    rne = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    assert np.array_equal(h, rne)
    assert np.all(np.abs(_f(h) - f) <= np.abs(f) * 2**-8 + 1e-30)


def test_logits_fill_masked_only_with_nan_elsewhere():
    w = configs.tiny_step()
    lg = synth.logits_cpu(w.rows, w.L, w.V, w.dtype, w.row_req, w.b[w.row_req[:w.rows]],
                          w.blk_mask[w.row_req[:w.rows]], w.logit_seed, w.sigma, w.umax)
    m = w.blk_mask[w.row_req[:w.rows]] != 0
    assert np.all(np.isfinite(lg[m]))
    assert np.all(np.isnan(lg[~m]))
    # row of one position equals the single-row generator with the row's masked count
    r, j = 1, int(np.flatnonzero(m[1])[0])
    one = synth.row_cpu(w.V, w.dtype, w.logit_seed, int(w.row_req[r]), int(w.b[w.row_req[r]]), j,
                        int(m[r].sum()), w.sigma, w.umax)
    assert np.array_equal(lg[r, j], one)


@pytest.mark.parametrize("name", list(configs.WORKLOADS))
def test_workload_shapes(name):
    w = configs.make(name)
    assert w.arena.shape[0] == int((w.p.astype(np.int64) + w.K.astype(np.int64) * w.L).sum())
    act = w.row_req[:w.rows]
    assert np.all(w.state[act] == configs.ACTIVE)
    assert len(w.queue) + w.rows == int(np.sum(w.state != configs.FINISHED))
    qp = [(int(w.p[q]), int(q)) for q in w.queue]
    assert qp == sorted(qp)
    assert np.all(np.isin(w.threshold, np.array(configs.TAU_SET, np.float32)))
    for q in range(w.n_req):
        o = int(w.arena_off[q]) + int(w.p[q]) + int(w.b[q]) * w.L
        blk = w.arena[o:o + w.L]
        assert np.array_equal(blk == w.mask_id, w.blk_mask[q] == 1)
    if name == "tiny-step":
        assert w.rows == 4 and np.all(w.blk_mask.sum(1) == 16) and w.b.tolist() == [0, 1, 0, 1]
    if name == "dream-dynamic-step":
        mf = w.blk_mask.sum(1)
        assert mf.min() >= 1 and mf.max() <= 32 and 900 < mf.sum() < 1350
    if name == "blockserve-mixed":
        W = int((w.p[act] + (w.b[act] + 1) * w.L).max())
        assert w.rows * W <= w.budget
        assert np.all(w.K == 8)
    if name == "large-fdfo":
        assert w.rows == 0 and len(w.queue) == 2048 and w.K.min() >= 2 and w.K.max() <= 16
