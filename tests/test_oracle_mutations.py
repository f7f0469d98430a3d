"""The oracle's pins catch plausible mistakes.

Each case plants one mistake in a copy of the oracle (on the CPU only): a
dropped term, a wrong sign, a missing factor, a wrong count.  The pin suite
(tests/test_oracle.py) is run against that copy and must fail; against an
unchanged copy it must pass (so the copy, not the package, is what runs)."""

import os
import re
import shutil
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE = os.path.join(ROOT, "oracle")
PINS = os.path.join(ROOT, "tests", "test_oracle.py")

# name -> (text in oracle/fldce_oracle.py, replacement)
MUTATIONS = {
    "loss drops the smoothing term": (
        "out = ((1.0 - eps) * ce + eps * uni) / p", "out = ((1.0 - eps) * ce) / p"),
    "smoothing term not divided by V": (
        "uni = lse - z_sum / float(V)", "uni = lse - z_sum"),
    "lse drops the max": (
        "return m + np.log(np.exp(z - m[:, None]).sum(axis=1))",
        "return np.log(np.exp(z - m[:, None]).sum(axis=1))"),
    "logit scale not applied to the logits": (
        "return float(logit_scale) * a", "return a"),
    "gradient target term with the wrong sign": (
        "g[rows, tc[rows]] -= (1.0 - eps)", "g[rows, tc[rows]] += (1.0 - eps)"),
    "gradient misses the logit scale": (
        "c = float(logit_scale) / (p * D)", "c = 1.0 / (p * D)"),
    "gradient not divided by p_mask": (
        "c = float(logit_scale) / (p * D)", "c = float(logit_scale) / D"),
    "gradient smoothing term not divided by V": (
        "g = np.exp(z - _f64(lse)[:, None]) - eps / float(V_global)",
        "g = np.exp(z - _f64(lse)[:, None]) - eps"),
    "ignored rows keep a gradient": (
        "    g[~valid] = 0.0\n", ""),
    "mean divides by every row, ignored ones too": (
        "return float(n) if n > 0 else 1.0", "return float(len(valid))"),
    "end-of-block weight multiplies p_mask": (
        "p[eob] = p[eob] / float(eob_weight)", "p[eob] = p[eob] * float(eob_weight)"),
    "bias added after the logit scale": (
        "    return float(logit_scale) * a\n",
        "    return float(logit_scale) * (a - (0 if bias is None else _f64(bias)[None, :]))"
        " + (0 if bias is None else _f64(bias)[None, :])\n"),
    "dH takes the logit scale a second time": (
        "dH[r0:r1] = g @ W\n", "dH[r0:r1] = float(logit_scale) * (g @ W)\n"),
    "dW keeps only the last row block": (
        "            dW += g.T @ h[r0:r1]\n", "            dW = g.T @ h[r0:r1]\n"),
    "shard combine forgets to rescale the sums": (
        "lse = M + np.log((Ss * np.exp(ms - M[None, :])).sum(axis=0))",
        "lse = M + np.log(Ss.sum(axis=0))"),
    "upstream gradient applied twice": (
        "return tuple(None if g is None else _f64(g) * float(do) for g in grads)",
        "return tuple(None if g is None else _f64(g) * float(do) ** 2 for g in grads)"),
}


def _copy(dst, mutation=None):
    d = os.path.join(dst, "oracle")
    shutil.copytree(ORACLE, d, ignore=shutil.ignore_patterns("__pycache__"))
    if mutation is not None:
        p = os.path.join(d, "fldce_oracle.py")
        src = open(p).read()
        old, new = mutation
        assert src.count(old) == 1, f"mutation anchor not found exactly once: {old!r}"
        open(p, "w").write(src.replace(old, new))


def _start(cwd):
    # cwd (which holds the copy) comes first on sys.path; ROOT is on the path
    # already, so the tests' conftest does not put the package's oracle first
    env = dict(os.environ, PYTHONPATH=os.pathsep.join([cwd, ROOT]), PYTHONDONTWRITEBYTECODE="1",
               OMP_NUM_THREADS="1", OPENBLAS_NUM_THREADS="1", MKL_NUM_THREADS="1")
    return subprocess.Popen([sys.executable, "-m", "pytest", PINS, "-x", "-q", "-p",
                             "no:cacheprovider", "--rootdir", ROOT],
                            cwd=cwd, env=env, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                            text=True)


def test_pins_fail_on_planted_mistakes(tmp_path):
    runs = {}
    control = tmp_path / "control"
    control.mkdir()
    _copy(str(control))
    runs[None] = _start(str(control))
    for i, (name, m) in enumerate(MUTATIONS.items()):
        d = tmp_path / f"m{i}"
        d.mkdir()
        _copy(str(d), m)
        runs[name] = _start(str(d))
    out = {name: (p.wait(timeout=300), p.stdout.read()) for name, p in runs.items()}
    rc, log = out.pop(None)
    assert rc == 0, "the unchanged copy must pass the pins:\n" + log[-3000:]
    survived = [name for name, (rc, _) in out.items() if rc == 0]
    assert not survived, f"mistakes no pin catches: {survived}"
    # each copy failed a pin (an assertion), not at import or collection
    broken = [name for name, (rc, log) in out.items()
              if rc != 1 or not re.search(r"\b1 failed\b", log.strip().splitlines()[-1])]
    assert not broken, f"copies that did not fail on a pin: {broken}"
