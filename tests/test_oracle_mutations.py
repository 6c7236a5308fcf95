"""Mutation check of the oracle's pins.

Each mutation plants one plausible mistake in a copy of oracle/ (in a
temporary directory, on the CPU; the repository's oracle is never touched)
and runs the pin tests against that copy: at least one pin must fail.  The
unmutated copy must pass the same pins, so a failure is the mutation's.
Every mutation must match its source text exactly once, so the list follows
the oracle as it changes.
"""
import concurrent.futures
import os
import shutil
import subprocess
import sys

import pytest

TESTS = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(TESTS)
PIN_FILES = ["test_oracle_pins.py", "test_margin_pins.py"]

# (name, file under oracle/, text, replacement)
MUTATIONS = [
    # top-p cut and its margin
    ("topp-margin-before-index", "sampling.py",
     "before = csum[keep - 2] if keep >= 2 else 0.0", "before = csum[keep - 1] if keep >= 2 else 0.0"),
    ("topp-margin-including-index", "sampling.py",
     "including = csum[keep - 1]", "including = csum[min(keep, p.size - 1)]"),
    ("topp-margin-no-temperature", "sampling.py",
     "s = np.asarray(z, dtype=np.float64) / float(temperature)\n    e = np.exp(s - s.max())\n"
     "    p = e / e.sum()\n    order",
     "s = np.asarray(z, dtype=np.float64)\n    e = np.exp(s - s.max())\n    p = e / e.sum()\n    order"),
    ("topp-keeps-one-more", "sampling.py",
     "side=\"left\")) + 1, p.size)\n    kept", "side=\"left\")) + 2, p.size)\n    kept"),
    ("topp-ties-by-larger-id", "sampling.py",
     "np.lexsort((np.arange(p.shape[-1]), -p))", "np.lexsort((-np.arange(p.shape[-1]), -p))"),
    ("softmax-no-temperature", "sampling.py",
     "s = np.asarray(z, dtype=np.float64) / float(temperature)\n    e = np.exp(s - s.max())\n"
     "    p = e / e.sum()\n    if top_p",
     "s = np.asarray(z, dtype=np.float64)\n    e = np.exp(s - s.max())\n    p = e / e.sum()\n    if top_p"),
    ("argmax-last-on-ties", "sampling.py",
     "return np.argmax(np.asarray(z), axis=-1)",
     "return np.asarray(z).shape[-1] - 1 - np.argmax(np.asarray(z)[..., ::-1], axis=-1)"),
    # inverse CDF and its margins
    ("cdf-le", "sampling.py", "hits = np.nonzero(float(u) * W < c)[0]", "hits = np.nonzero(float(u) * W <= c)[0]"),
    ("cdf-margin-lower-bound", "sampling.py",
     "lo = c[y - 1] / W if y >= 1 else 0.0", "lo = c[y] / W if y >= 1 else 0.0"),
    ("cdf-margin-upper-bound", "sampling.py",
     "hi = c[y] / W\n    return y", "hi = c[min(y + 1, c.size - 1)] / W\n    return y"),
    ("cdf-rows-le", "sampling.py", "hit = (u * W)[..., None] < c", "hit = (u * W)[..., None] <= c"),
    ("cdf-rows-margin-lower-bound", "sampling.py",
     "np.take_along_axis(c, np.maximum(y - 1, 0)[..., None], axis=-1)",
     "np.take_along_axis(c, y[..., None], axis=-1)"),
    ("cdf-rows-margin-unnormalised", "sampling.py",
     "hi = np.take_along_axis(c, y[..., None], axis=-1)[..., 0] / W",
     "hi = np.take_along_axis(c, y[..., None], axis=-1)[..., 0]"),
    # acceptance, selection, final draw
    ("accept-wrong-parent-row", "verify.py",
     "pi = p_rows[bidx, par[:, i], tok[:, i]]", "pi = p_rows[bidx, i, tok[:, i]]"),
    ("accept-le", "verify.py",
     "(u_accept[:, i].astype(np.float64) < ratio)", "(u_accept[:, i].astype(np.float64) <= ratio)"),
    ("accept-margin-against-p", "verify.py",
     "np.abs(u_accept[:, i] - ratio)", "np.abs(u_accept[:, i] - pi)"),
    ("path-not-chained", "verify.py", "acc[:, i] = a[:, i] & acc[bidx, par[:, i]]", "acc[:, i] = a[:, i]"),
    ("vstar-last-on-ties", "verify.py",
     "vstar = np.argmax(key, axis=1)", "vstar = T - 1 - np.argmax(key[:, ::-1], axis=1)"),
    ("residual-q-minus-p", "verify.py", "resid = np.maximum(pv - qc, 0.0)", "resid = np.maximum(qc - pv, 0.0)"),
    ("no-residual", "verify.py", "w = np.where(use_resid[:, None], resid, pv)", "w = pv"),
    ("residual-last-child", "verify.py",
     "for i in range(T - 1, 0, -1):\n        first_child", "for i in range(1, T):\n        first_child"),
    ("near-topp-own-row", "verify.py", "(tmargin[bidx, par] < topp_band)", "(tmargin < topp_band)"),
    ("near-final-no-draft-row", "verify.py",
     "\n                  | ((fc >= 0) & (dmargin[b1, np.maximum(fc, 0)] < topp_band)))", ")"),
    ("near-final-no-target-row", "verify.py", "| (tmargin[b1, vstar] < topp_band)", ""),
    ("near-final-no-cdf", "verify.py", "final_near = ((out[\"cdf_margin\"] < cdf_band) | ", "final_near = (("),
    # attention and the tree
    ("sibling-visibility", "attention.py",
     "tail = [kv_len + j for j in ancestors(parent, i)]", "tail = [kv_len + j for j in range(i + 1)]"),
    ("node-does-not-see-itself", "attention.py",
     "tail = [kv_len + j for j in ancestors(parent, i)]", "tail = [kv_len + j for j in ancestors(parent, i)[:-1]]"),
    ("gqa-interleaved-heads", "attention.py", "kappa = (h * hkv) // hq", "kappa = h % hkv"),
    ("attention-scale-1-over-d", "attention.py", "scale = 1.0 / np.sqrt(d)", "scale = 1.0 / d"),
    ("depth-from-previous-node", "tree.py", "d[i] = d[int(parent[i])] + 1", "d[i] = d[i - 1] + 1"),
]


def _copy_tree(dst):
    for sub in ("oracle", "synth"):
        shutil.copytree(os.path.join(ROOT, sub), os.path.join(dst, sub),
                        ignore=shutil.ignore_patterns("__pycache__"))
    os.makedirs(os.path.join(dst, "tests"))
    shutil.copytree(os.path.join(TESTS, "golden"), os.path.join(dst, "tests", "golden"))
    for f in ["conftest.py"] + PIN_FILES:
        shutil.copy(os.path.join(TESTS, f), os.path.join(dst, "tests", f))


def _run_pins(dst):
    env = dict(os.environ, PYTHONDONTWRITEBYTECODE="1", OMP_NUM_THREADS="1", OPENBLAS_NUM_THREADS="1")
    cmd = [sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider"] + ["tests/" + f for f in PIN_FILES]
    r = subprocess.run(cmd, cwd=dst, env=env, capture_output=True, text=True, timeout=600)
    return r.returncode, (r.stdout + r.stderr)[-1500:]


def _mutant(base, m):
    name, fname, old, new = m
    dst = os.path.join(base, name)
    _copy_tree(dst)
    path = os.path.join(dst, "oracle", fname)
    src = open(path, encoding="utf-8").read()
    count = src.count(old)
    if count != 1:
        return name, None, "text found %d times in oracle/%s" % (count, fname)
    open(path, "w", encoding="utf-8").write(src.replace(old, new))
    rc, tail = _run_pins(dst)
    return name, rc, tail


def test_every_planted_mistake_fails_a_pin(tmp_path):
    control = os.path.join(str(tmp_path), "control")
    _copy_tree(control)
    rc, tail = _run_pins(control)
    assert rc == 0, "unmutated oracle copy fails its pins:\n" + tail
    with concurrent.futures.ThreadPoolExecutor(max_workers=6) as ex:
        results = list(ex.map(lambda m: _mutant(str(tmp_path), m), MUTATIONS))
    survivors = []
    for name, rc, tail in results:
        if rc is None:
            survivors.append("%s: %s" % (name, tail))
        elif rc != 1:       # 1 = some test failed; anything else (0 = all passed, 2+ = errors) is not a catch
            survivors.append("%s: pytest exit %d\n%s" % (name, rc, tail))
    assert not survivors, "mutations not caught:\n" + "\n".join(survivors)


@pytest.mark.parametrize("m", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_mutation_text_is_present_once(m):
    name, fname, old, new = m
    src = open(os.path.join(ROOT, "oracle", fname), encoding="utf-8").read()
    assert src.count(old) == 1, name
