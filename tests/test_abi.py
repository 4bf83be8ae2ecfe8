"""C ABI checks that need no GPU: the library loads, exports every declared symbol, sizes its
workspace, and rejects bad arguments synchronously before touching a device."""
import ctypes
import os
import re

import pytest

from confidence_block_unmasking_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    names = set()
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            src = open(os.path.join(ROOT, "include", fn)).read()
            src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
            names |= set(re.findall(r"\b(dllm_\w+)\s*\(", src))
    return names


def test_library_exports_every_declared_symbol():
    L = _lib.lib()
    declared = _declared()
    assert declared == set(_lib.EXPORTS)
    for name in declared:
        assert hasattr(L, name), name


def test_workspace_bytes():
    L = _lib.lib()
    # V = 152064 bf16: 19008 vectors of 8, 38 chunks of <= 512 vectors
    pos = 64 * 32
    part = pos * 38 * 16
    n = L.dllm_step_workspace_bytes(64, 32, 152064, _lib.DLLM_BF16)
    assert n >= part and n % 256 == 0
    assert L.dllm_step_workspace_bytes(-1, 32, 1024, 0) == 0
    assert L.dllm_step_workspace_bytes(4, 0, 1024, 0) == 0
    assert L.dllm_step_workspace_bytes(4, 32, 1024, 9) == 0
    # fp32 V = 1024: 256 vectors, one chunk
    assert L.dllm_step_workspace_bytes(4, 32, 1024, _lib.DLLM_FP32) >= 128 * 16


FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: every call below fails validation first


def _step(**kw):
    a = dict(stream=None, logits=FAKE, dtype=1, pos_stride=1024, row_stride=32 * 1024, rows=4, L=32, V=1024,
             ids=FAKE, W=64, mask_in=FAKE, mask_out=ctypes.c_void_p(0x2000), tau=FAKE, p=None, b=None, conf=None,
             arg=None, done=FAKE, accept=FAKE, ws=FAKE, ws_bytes=0, status=FAKE)
    a.update(kw)
    return _lib.lib().dllm_step(a["stream"], a["logits"], a["dtype"], a["pos_stride"], a["row_stride"], a["rows"],
                                a["L"], a["V"], a["ids"], a["W"], a["mask_in"], a["mask_out"], a["tau"], a["p"],
                                a["b"], a["conf"], a["arg"], a["done"], a["accept"], a["ws"], a["ws_bytes"],
                                a["status"])


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=7), _lib.DLLM_ERR_DTYPE),
    (dict(rows=-1), _lib.DLLM_ERR_ARG),
    (dict(L=0), _lib.DLLM_ERR_SHAPE),
    (dict(L=1025, W=2000, row_stride=1025 * 1024), _lib.DLLM_ERR_SHAPE),
    (dict(V=0), _lib.DLLM_ERR_ARG),
    (dict(W=31), _lib.DLLM_ERR_SHAPE),
    (dict(rows=4097), _lib.DLLM_ERR_SHAPE),
    (dict(rows=4096, L=128, row_stride=128 * 1024, W=200), _lib.DLLM_ERR_SHAPE),
    (dict(pos_stride=1000), _lib.DLLM_ERR_ARG),
    (dict(row_stride=1024), _lib.DLLM_ERR_ARG),
    (dict(p=FAKE), _lib.DLLM_ERR_ARG),
    (dict(logits=None), _lib.DLLM_ERR_ARG),
    (dict(status=None), _lib.DLLM_ERR_ARG),
    (dict(mask_out=ctypes.c_void_p(0x1000 + 127)), _lib.DLLM_ERR_ARG),   # overlaps mask_in's last byte
    (dict(ws_bytes=10), _lib.DLLM_ERR_ARG),                 # workspace too small
])
def test_step_rejects_bad_arguments(kw, code):
    assert _step(**kw) == code
    assert _lib.last_error() != ""


def test_step_halves_reject_bad_arguments():
    L = _lib.lib()
    need = L.dllm_step_workspace_bytes(4, 32, 1024, 1)
    f, ws = FAKE, ctypes.c_void_p(0x10000)

    def score(**kw):
        a = dict(logits=f, dtype=1, ps=1024, rs=32 * 1024, rows=4, L=32, V=1024, mask=f, ws=ws, n=need, status=f)
        a.update(kw)
        return L.dllm_step_score(None, a["logits"], a["dtype"], a["ps"], a["rs"], a["rows"], a["L"], a["V"],
                                 a["mask"], a["ws"], a["n"], a["status"])

    def decide(**kw):
        a = dict(dtype=1, rows=4, L=32, V=1024, ids=f, W=40, mi=f, mo=ctypes.c_void_p(0x2000), tau=f, done=f,
                 acc=f, ws=ws, n=need, status=f)
        a.update(kw)
        return L.dllm_step_decide(None, a["dtype"], a["rows"], a["L"], a["V"], a["ids"], a["W"], a["mi"], a["mo"],
                                  a["tau"], None, None, None, None, a["done"], a["acc"], a["ws"], a["n"], a["status"],
                                  None, None)
    assert score(dtype=5) == _lib.DLLM_ERR_DTYPE
    assert score(logits=None) == _lib.DLLM_ERR_ARG
    assert score(ps=100) == _lib.DLLM_ERR_ARG
    assert score(n=need - 16) == _lib.DLLM_ERR_ARG
    assert score(L=0) == _lib.DLLM_ERR_SHAPE
    assert score(rows=0, logits=None, mask=None) == _lib.DLLM_OK
    assert decide(W=31) == _lib.DLLM_ERR_SHAPE
    assert decide(done=None) == _lib.DLLM_ERR_ARG
    assert decide(ws=None) == _lib.DLLM_ERR_ARG
    assert decide(mo=ctypes.c_void_p(0x1000 + 1)) == _lib.DLLM_ERR_ARG
    assert decide(rows=0, ids=None) == _lib.DLLM_OK


def test_timed_score_rejects_bad_arguments():
    # the same checks as dllm_step_score, plus the two events; all refused before any launch
    L = _lib.lib()
    need = L.dllm_step_workspace_bytes(4, 32, 1024, 1)
    f, ws, ev = FAKE, ctypes.c_void_p(0x10000), ctypes.c_void_p(0x3000)

    def timed(**kw):
        a = dict(logits=f, dtype=1, ps=1024, rs=32 * 1024, rows=4, L=32, V=1024, mask=f, ws=ws, n=need, status=f,
                 e0=ev, e1=ev)
        a.update(kw)
        return L.dllm_step_score_timed(None, a["logits"], a["dtype"], a["ps"], a["rs"], a["rows"], a["L"], a["V"],
                                       a["mask"], a["ws"], a["n"], a["status"], a["e0"], a["e1"])
    assert timed(e0=None) == _lib.DLLM_ERR_ARG
    assert timed(e1=None) == _lib.DLLM_ERR_ARG
    assert "event" in _lib.last_error()
    assert timed(dtype=5) == _lib.DLLM_ERR_DTYPE
    assert timed(logits=None) == _lib.DLLM_ERR_ARG
    assert timed(ps=100) == _lib.DLLM_ERR_ARG
    assert timed(n=need - 16) == _lib.DLLM_ERR_ARG
    assert timed(L=0) == _lib.DLLM_ERR_SHAPE
    assert timed(rows=0, logits=None, mask=None) == _lib.DLLM_OK


def test_timed_step_rejects_bad_arguments():
    L = _lib.lib()
    need = L.dllm_step_workspace_bytes(4, 32, 1024, 1)
    f, ws, ev = FAKE, ctypes.c_void_p(0x10000), ctypes.c_void_p(0x3000)

    def timed(**kw):
        a = dict(logits=f, dtype=1, rows=4, W=40, ws=ws, n=need, e0=ev, e1=ev, done=f)
        a.update(kw)
        return L.dllm_step_timed(None, a["logits"], a["dtype"], 1024, 32 * 1024, a["rows"], 32, 1024, f, a["W"], f,
                                 ctypes.c_void_p(0x2000), f, None, None, None, None, a["done"], f, a["ws"], a["n"], f,
                                 a["e0"], a["e1"])
    assert timed(e0=None) == _lib.DLLM_ERR_ARG
    assert timed(e1=None) == _lib.DLLM_ERR_ARG
    assert "event" in _lib.last_error()
    assert timed(dtype=7) == _lib.DLLM_ERR_DTYPE
    assert timed(W=31) == _lib.DLLM_ERR_SHAPE
    assert timed(done=None) == _lib.DLLM_ERR_ARG
    assert timed(n=need - 16) == _lib.DLLM_ERR_ARG
    assert timed(rows=0, logits=None) == _lib.DLLM_OK


def test_quota_rejects_bad_arguments():
    L = _lib.lib()
    need = L.dllm_step_workspace_bytes(4, 32, 1024, 1)
    f, ws = FAKE, ctypes.c_void_p(0x10000)

    def quota(S=32, done=f, W=40, rows=4):
        return L.dllm_step_quota(None, f, 1, 1024, 32 * 1024, rows, 32, 1024, f, W, f, ctypes.c_void_p(0x2000), S,
                                 None, None, None, None, done, f, ws, need, f)

    def dq(S=32, done=f):
        return L.dllm_step_decide_quota(None, 1, 4, 32, 1024, f, 40, f, ctypes.c_void_p(0x2000), S, None, None,
                                        None, None, done, f, ws, need, f)
    assert quota(S=0) == _lib.DLLM_ERR_ARG
    assert quota(S=-3) == _lib.DLLM_ERR_ARG
    assert quota(done=None) == _lib.DLLM_ERR_ARG
    assert quota(W=31) == _lib.DLLM_ERR_SHAPE
    assert quota(rows=0) == _lib.DLLM_OK
    assert dq(S=0) == _lib.DLLM_ERR_ARG
    assert dq(done=None) == _lib.DLLM_ERR_ARG


def test_features_rejects_bad_arguments():
    L = _lib.lib()
    r = _reqs()
    f = FAKE

    def call(rows=4, Lb=32, row_req=f, reqs=r, conf=f, mask=f, out=f, status=f):
        return L.dllm_step_features(None, rows, Lb, row_req, ctypes.byref(reqs) if reqs is not None else None, conf,
                                    mask, out, status)
    assert call(rows=-1) == _lib.DLLM_ERR_ARG
    assert call(Lb=0) == _lib.DLLM_ERR_SHAPE
    assert call(rows=5000) == _lib.DLLM_ERR_SHAPE
    assert call(conf=None) == _lib.DLLM_ERR_ARG
    assert call(reqs=None) == _lib.DLLM_ERR_ARG
    assert call(reqs=_lib.Reqs(4, 0x1000, 0, 0x1000, 0x1000, 0x1000, 0x1000, 0x1000, 0x1000)) == _lib.DLLM_ERR_ARG
    assert call(rows=0, row_req=None, conf=None) == _lib.DLLM_OK


def test_shards_reject_bad_arguments():
    L = _lib.lib()
    assert L.dllm_shard_triples_bytes(4, 32, 8) == 4 * 32 * 8 * 16
    assert L.dllm_shard_triples_bytes(4, 32, 0) == 0
    need = L.dllm_step_workspace_bytes(4, 32, 1000, 1)
    f, ws = FAKE, ctypes.c_void_p(0x10000)

    def sc(shard=0, n=2, off=0, tri=f, V=1000):
        return L.dllm_step_score_shard(None, f, 1, V, 32 * V, 4, 32, V, off, shard, n, f, ws, need, tri, f)

    def dc(n=2, tri=f, W=40):
        return L.dllm_step_decide_shards(None, n, tri, 4, 32, 2000, f, W, f, ctypes.c_void_p(0x2000), f, None, None,
                                         None, None, f, f, f)
    assert sc(shard=2) == _lib.DLLM_ERR_ARG
    assert sc(shard=-1) == _lib.DLLM_ERR_ARG
    assert sc(n=0) == _lib.DLLM_ERR_ARG
    assert sc(off=-5) == _lib.DLLM_ERR_ARG
    assert sc(tri=None) == _lib.DLLM_ERR_ARG
    assert dc(n=0) == _lib.DLLM_ERR_ARG
    assert dc(n=2000) == _lib.DLLM_ERR_ARG
    assert dc(tri=None) == _lib.DLLM_ERR_ARG
    assert dc(W=31) == _lib.DLLM_ERR_SHAPE


def test_step_rows_zero_is_noop():
    assert _step(rows=0, logits=None, ids=None) == _lib.DLLM_OK


def test_step_rejects_misaligned_workspace():
    L = _lib.lib()
    need = L.dllm_step_workspace_bytes(4, 32, 1024, 1)
    assert _step(ws=ctypes.c_void_p(0x1004), ws_bytes=need) == _lib.DLLM_ERR_ARG


def _reqs():
    return _lib.Reqs(4, 0x1000, 0x1000, 0x1000, 0x1000, 0x1000, 0x1000, 0x1000, 0x1000)


def test_pack_rejects_bad_arguments():
    L = _lib.lib()
    r = _reqs()
    f = FAKE
    assert L.dllm_pack(None, -1, 32, 64, 0, f, ctypes.byref(r), f, None, None, f, f, f, f, f) == _lib.DLLM_ERR_ARG
    assert L.dllm_pack(None, 2, 0, 64, 0, f, ctypes.byref(r), f, None, None, f, f, f, f, f) == _lib.DLLM_ERR_SHAPE
    assert L.dllm_pack(None, 2, 32, 16, 0, f, ctypes.byref(r), f, None, None, f, f, f, f, f) == _lib.DLLM_ERR_SHAPE
    assert L.dllm_pack(None, 5000, 32, 64, 0, f, ctypes.byref(r), f, None, None, f, f, f, f, f) == _lib.DLLM_ERR_SHAPE
    assert L.dllm_pack(None, 2, 32, 64, 0, None, ctypes.byref(r), f, None, None, f, f, f, f, f) == _lib.DLLM_ERR_ARG
    bad = _lib.Reqs(4, 0x1000, 0x1000, 0, 0x1000, 0x1000, 0x1000, 0x1000, 0x1000)
    assert L.dllm_pack(None, 2, 32, 64, 0, f, ctypes.byref(bad), f, None, None, f, f, f, f, f) == _lib.DLLM_ERR_ARG
    assert L.dllm_pack(None, 0, 32, 0, 0, None, None, None, None, None, None, None, None, None, None) == _lib.DLLM_OK


def test_compact_rejects_bad_arguments():
    L = _lib.lib()
    r = _reqs()
    q = _lib.Queue(0x1000, 0x1000, 4)
    f = FAKE

    def call(rows=2, Lb=32, W=64, box=f, mask=f, done=f, row_req=f, cap=4, reqs=r, queue=q, meta=f, status=f):
        return L.dllm_compact(None, rows, Lb, W, 0, -1, box, mask, done, row_req, cap,
                              ctypes.byref(reqs) if reqs is not None else None,
                              ctypes.byref(queue) if queue is not None else None, 0, meta, status)
    assert call(rows=-1) == _lib.DLLM_ERR_ARG
    assert call(rows=5, cap=4) == _lib.DLLM_ERR_ARG
    assert call(cap=5000) == _lib.DLLM_ERR_SHAPE
    assert call(Lb=0) == _lib.DLLM_ERR_SHAPE
    assert call(mask=None) == _lib.DLLM_ERR_ARG
    assert call(W=16) == _lib.DLLM_ERR_SHAPE
    assert call(meta=None) == _lib.DLLM_ERR_ARG
    assert call(queue=_lib.Queue(0x1000, 0x1000, 9000)) == _lib.DLLM_ERR_CAPACITY
    assert call(queue=_lib.Queue(0x1000, None, 4)) == _lib.DLLM_ERR_ARG
    bad = _lib.Reqs(4, 0x1000, 0, 0x1000, 0x1000, 0x1000, 0x1000, 0x1000, 0x1000)
    assert call(reqs=bad) == _lib.DLLM_ERR_ARG


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "absent.so"))
    monkeypatch.setattr(_lib, "_lib", None)
    with pytest.raises(RuntimeError, match="no fallback"):
        _lib.lib()


def test_binding_limits_match_the_header():
    text = open(os.path.join(ROOT, "include", "dllm.h")).read()
    got = {m.group(1): int(m.group(2)) for m in re.finditer(r"#define DLLM_(MAX_\w+)\s+(\d+)", text)}
    assert got["MAX_L"] == _lib.MAX_L and got["MAX_ROWS"] == _lib.MAX_ROWS
    assert got["MAX_POSITIONS"] == _lib.MAX_POSITIONS and got["MAX_QUEUE"] == _lib.MAX_QUEUE
    m = re.search(r"#define DLLM_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == _lib.NOALLOC_SCRATCH_BYTES


def test_binding_rejects_a_strided_vocabulary():
    """The kernels read each slot's vocabulary row as one contiguous run: a view whose last
    dimension is strided (x[..., ::2]) is refused before anything reaches the library."""
    torch = pytest.importorskip("torch")
    from confidence_block_unmasking_amd import api
    x = torch.zeros(2, 3, 16, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="unit stride"):
        api._logits_shape(x[..., ::2], None, None, None, None, None)
    with pytest.raises(ValueError, match="unit stride"):
        api._logits_shape(x.reshape(-1)[::2], 2, 3, 16, 16, 48)
    with pytest.raises(ValueError, match="device tensor"):          # a contiguous view passes the stride test
        api._logits_shape(x[..., :8], None, None, None, None, None)


def test_noalloc_step_rejects_bad_arguments_and_oversize():
    """dllm_step_noalloc checks what dllm_step checks, and refuses a shape whose workspace would not
    fit its fixed scratch array, all before touching a device."""
    L = _lib.lib()

    def na(**kw):
        a = dict(logits=FAKE, dtype=1, ps=152064, rs=64 * 152064, rows=256, L=64, V=152064, ids=FAKE, W=5000,
                 mi=FAKE, mo=ctypes.c_void_p(0x900000), tau=FAKE, done=FAKE, acc=FAKE, status=FAKE)
        a.update(kw)
        return L.dllm_step_noalloc(None, a["logits"], a["dtype"], a["ps"], a["rs"], a["rows"], a["L"], a["V"],
                                   a["ids"], a["W"], a["mi"], a["mo"], a["tau"], None, None, None, None, a["done"],
                                   a["acc"], a["status"])
    assert na(dtype=7) == _lib.DLLM_ERR_DTYPE
    assert na(logits=None) == _lib.DLLM_ERR_ARG
    assert na(ps=100) == _lib.DLLM_ERR_ARG
    assert na(W=63) == _lib.DLLM_ERR_SHAPE
    assert na(tau=None) == _lib.DLLM_ERR_ARG
    assert na(rows=0, logits=None, ids=None) == _lib.DLLM_OK
    # the largest batch of the large FDFO run (256 x 64 slots at V = 152064 bf16) fits; 4x as many rows do not
    assert L.dllm_step_workspace_bytes(256, 64, 152064, 1) <= _lib.NOALLOC_SCRATCH_BYTES
    big = dict(rows=1024, mo=ctypes.c_void_p(0x4000000))
    assert L.dllm_step_workspace_bytes(1024, 64, 152064, 1) > _lib.NOALLOC_SCRATCH_BYTES
    assert na(**big) == _lib.DLLM_ERR_CAPACITY
    assert "scratch" in _lib.last_error()
