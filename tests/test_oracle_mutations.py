"""The oracle's pins must catch plausible mistakes.

Each case plants one mistake (a flipped sign, an off-by-one index, a `>` turned into `>=`, a
reordered rule) in a scratch copy of `oracle/`, then runs the pin tests of that file against the
copy; they must fail.  A control run of the unmodified copy must pass.  Everything runs on the
CPU in subprocesses; the repository's own oracle is never modified.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

STEP = "tests/test_oracle_step.py"
PACK = "tests/test_oracle_pack_compact.py"
LOOP = "tests/test_oracle_loop.py"
QUOTA = "tests/test_oracle_quota.py"
FEAT = "tests/test_oracle_features.py"
SHARD = "tests/test_oracle_shard.py"
ROWS = "tests/test_oracle_rows.py"

MUTATIONS = [
    ("oracle/step.py", "S = float(np.sum(np.exp(x - m)))", "S = float(np.sum(np.exp(m - x)))", STEP),
    ("oracle/step.py", "a = int(np.flatnonzero(x == m)[0])", "a = int(np.flatnonzero(x == m)[-1])", STEP),
    ("oracle/step.py", "np.asarray(conf, np.float64) > t", "np.asarray(conf, np.float64) >= t", STEP),
    ("oracle/step.py", "if masked[j] and conf[j] > best_c", "if masked[j] and conf[j] >= best_c", STEP),
    ("oracle/step.py", "ids[r, W - L + j] = arg[r, j]", "ids[r, W - L + j - 1] = arg[r, j]", STEP),
    ("oracle/step.py", "accept[r] = L if done[r] else 0", "accept[r] = 1 if done[r] else 0", STEP),
    ("oracle/pack.py", "return int(p) + (int(b) + 1) * int(L)", "return int(p) + int(b) * int(L)", PACK),
    ("oracle/pack.py", "box_pos[r, pad:] = np.arange(w)", "box_pos[r, pad:] = np.arange(1, w + 1)", PACK),
    ("oracle/compact.py", "and queue_p[i] + L <= W_A:", "and queue_p[i] + L < W_A:", PACK),
    ("oracle/compact.py", "if best is None or queue_p[i] > queue_p[best]:",
     "if best is None or queue_p[i] >= queue_p[best]:", PACK),
    ("oracle/compact.py", "if budget > 0 and (n_active + 1) * new_W > budget:",
     "if budget > 0 and n_active * new_W > budget:", PACK),
    ("oracle/compact.py", "if b[q] >= K[q] or hit_eos:", "if b[q] > K[q] or hit_eos:", PACK),
    ("oracle/compact.py", "movers = sorted([r for r in occupied if r >= n_new], reverse=True)",
     "movers = sorted([r for r in occupied if r >= n_new])", PACK),
    ("oracle/compact.py", "slots = sorted(freed) + list(range(rows, rows_cap))",
     "slots = list(range(rows, rows_cap)) + sorted(freed)", PACK),
    ("oracle/loop.py", 'if mode == "sync" and out["done"].all():', 'if mode == "sync" and out["done"].any():', LOOP),
    ("oracle/loop.py", 'trace["request_steps"] += rows', 'trace["request_steps"] += 1', LOOP),
    ("oracle/quota.py", "return [base + (1 if t < rem else 0) for t in range(S)]",
     "return [base + (1 if t >= S - rem else 0) for t in range(S)]", QUOTA),
    ("oracle/quota.py", "js.sort(key=lambda j: (-float(conf[j]), j))", "js.sort(key=lambda j: (-float(conf[j]), -j))",
     QUOTA),
    ("oracle/quota.py", "while t < S and pre + ks[t] <= u:", "while t < S and pre + ks[t] < u:", QUOTA),
    ("oracle/features.py", "f[2] = (b * L + unmasked) / (K * L)", "f[2] = ((b + 1) * L + unmasked) / (K * L)", FEAT),
    ("oracle/features.py", "f[5], f[6], f[8] = np.quantile(c, [0.25, 0.5, 0.75])",
     "f[5], f[6], f[8] = np.quantile(c, [0.25, 0.5, 0.75], method='lower')", FEAT),
    ("oracle/shard.py", "a = min(t[1] for t in triples if t[0] == m)", "a = max(t[1] for t in triples if t[0] == m)",
     SHARD),
    ("oracle/shard.py", "S = sum(t[2] * np.exp(t[0] - m) for t in triples)", "S = sum(t[2] for t in triples)", SHARD),
    # a dropped term, a shifted or transposed index, a flipped test: one more of each kind per module
    ("oracle/step.py", "S = float(np.sum(np.exp(x - m)))", "S = float(np.sum(np.exp(x[1:] - m)))", STEP),
    ("oracle/pack.py", "box_valid[r, pad:] = 1", "box_valid[r, pad + 1:] = 1", PACK),
    ("oracle/pack.py", "tau[r] = threshold[q]", "tau[r] = threshold[r]", PACK),
    ("oracle/compact.py", "arena[block_slice(q, b[q])] = box_ids[r, W - L:W]",
     "arena[block_slice(q, b[q])] = box_ids[r, W - L - 1:W - 1]", PACK),
    ("oracle/compact.py", "hit_eos = eos_id >= 0 and bool(np.any(committed == eos_id))",
     "hit_eos = eos_id >= 0 and bool(np.all(committed == eos_id))", PACK),
    ("oracle/loop.py", 'trace["idle_request_steps"] += int(np.sum(~(msk != 0).any(axis=1)))',
     'trace["idle_request_steps"] += int(np.sum((msk != 0).any(axis=1)))', LOOP),
    ("oracle/features.py", "f[3] = unmasked / L", "f[3] = (L - unmasked) / L", FEAT),
    ("oracle/shard.py", "o += base + (1 if t < rem else 0)", "o += base + (1 if t <= rem else 0)", SHARD),
    ("oracle/quota.py", "return min(m, ks[t])", "return ks[t]", QUOTA),
    ("oracle/compact.py", "                arena[block_slice(q, b[q])] = mask_id\n                blk_mask[q] = 1",
     "                blk_mask[q] = 1", PACK),
    ("oracle/compact.py", "        state[q] = ACTIVE\n        b[q] = 0", "        state[q] = ACTIVE", PACK),
    ("oracle/features.py", "        f[7] = c.mean()", "        f[7] = np.median(c)", FEAT),
    ("oracle/loop.py", '            if mode == "fdfo" and out["done"].any():', '            if mode == "fdfo" and out["done"].all():',
     LOOP),
    ("oracle/shard.py", "    return m, offset + a, S", "    return m, a, S", SHARD),
    ("oracle/quota.py", "    for j in js[:max(0, int(k))]:", "    for j in js[:max(0, int(k) - 1)]:", QUOTA),
    # a row-index slip in the per-box wrapper of the features
    ("oracle/features.py", "threshold[r], int(b[r]), int(K[r]), L)", "threshold[0], int(b[r]), int(K[r]), L)", FEAT),
    ("oracle/features.py", "threshold[r], int(b[r]), int(K[r]), L)", "threshold[r], int(b[0]), int(K[r]), L)", FEAT),
    ("oracle/features.py", "threshold[r], int(b[r]), int(K[r]), L)", "threshold[r], int(b[r]), int(K[-1]), L)", FEAT),
    ("oracle/features.py", "row_features(conf[r], mask_after[r],", "row_features(conf[r], mask_after[0],", FEAT),
    ("oracle/step.py", "    fallback = not U.any() and masked.any()\n", "    fallback = not U.any()\n", STEP),
    ("oracle/step.py", "        unmasked[r] = int(U.sum())", "        unmasked[r] = int(masked.sum())", STEP),
    # the C row scorer (rebuilt from the planted source in the scratch copy)
    ("oracle/rows.c", "S += exp(buf[v] - m);", "S += exp(m - buf[v]);", ROWS),
    ("oracle/rows.c", "for (int64_t v = 0; v < V; ++v) S += exp", "for (int64_t v = 1; v < V; ++v) S += exp", ROWS),
    ("oracle/rows.c", "    int64_t a = 0;\n", "    int64_t a = 1;\n", ROWS),
    ("oracle/rows.c", "m = buf[v] > m ? buf[v] : m;", "m = buf[v] < m ? buf[v] : m;", ROWS),
    ("oracle/rows.c", "*conf = 1.0 / S;", "*conf = 1.0 / (S + 1.0);", ROWS),
    ("oracle/rows.c", "uint32_t u = (uint32_t)h[v] << 16;", "uint32_t u = (uint32_t)h[v] << 15;", ROWS),
    ("oracle/rows.c", "finite &= fabs(buf[v]) <= DBL_MAX;", "finite &= fabs(buf[v]) <= INFINITY;", ROWS),
    ("oracle/rows.c", "(size_t)i * (size_t)row_stride * es", "(size_t)i * (size_t)V * es", ROWS),
]


def _copy_tree(dst):
    for d in ("oracle", "workload", "tests"):
        shutil.copytree(os.path.join(ROOT, d), os.path.join(dst, d),
                        ignore=shutil.ignore_patterns("__pycache__", "golden_tmp*", "liboracle_*.so"))
    shutil.copy(os.path.join(ROOT, "pytest.ini"), dst)


def _run_pins(dst, pin_file):
    env = dict(os.environ, PYTHONDONTWRITEBYTECODE="1")
    return subprocess.run([sys.executable, "-m", "pytest", pin_file, "-x", "-q", "-m", "not gpu",
                           "-p", "no:cacheprovider"], cwd=dst, env=env, capture_output=True, text=True,
                          timeout=300)


def test_unmodified_copy_passes(tmp_path):
    _copy_tree(str(tmp_path))
    for pin in (STEP, PACK, LOOP, QUOTA, FEAT, SHARD, ROWS):
        r = _run_pins(str(tmp_path), pin)
        assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-2000:]


@pytest.mark.parametrize("path,old,new,pin", MUTATIONS, ids=[f"{m[0]}:{i}" for i, m in enumerate(MUTATIONS)])
def test_planted_mistake_is_caught(tmp_path, path, old, new, pin):
    _copy_tree(str(tmp_path))
    f = os.path.join(str(tmp_path), path)
    src = open(f).read()
    assert src.count(old) == 1, f"mutation site not found once in {path}: {old}"
    with open(f, "w") as fh:
        fh.write(src.replace(old, new))
    r = _run_pins(str(tmp_path), pin)
    assert r.returncode != 0, f"planted mistake survived the pins of {pin}: {path}: {old} -> {new}"
