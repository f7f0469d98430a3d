"""The stored expected values (tests/golden/rowstats_*.npz, written by
tests/golden/make_golden.py with the oracle) against the oracle recomputed
on sampled rows, and the vocabulary-shard file's stored combine of the other
shards against the full-vocabulary statistics (page 3 section 4: the shards'
partials combine to the whole softmax).  CPU only."""

import os

import numpy as np

import oracle as O
from lm_head_linear_bf16_amd import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _load(name):
    g = np.load(os.path.join(GOLDEN, f"rowstats_{name}.npz"))
    assert str(g["fingerprint"]) == synth.fingerprint(synth.WORKLOADS[name]), "stale golden file"
    return g


def _rows(N, n, seed):
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, N - 1], rng.choice(N, n, replace=False)]))


def test_headline_rowstats_match_the_oracle():
    w = synth.WORKLOADS["headline"]
    g = _load("headline")
    t, _ = synth.targets(w)
    rows = _rows(w.N, 14, seed=0)
    lse, zt, zs = O.row_stats(synth.hidden(w).values[rows], synth.weight(w).values, t[rows],
                              np.arange(len(rows)), w.logit_scale)
    np.testing.assert_allclose(g["lse"][rows], lse, rtol=1e-12)
    np.testing.assert_allclose(g["z_target"][rows], zt, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(g["z_sum"][rows], zs, rtol=1e-9, atol=1e-9)


def test_shard_rest_combine_gives_the_full_vocabulary():
    """Shard k's oracle partials combined with the stored combine of the other
    shards equal the stored full-vocabulary lse, target logit and row sum,
    for rows with and without a target."""
    w = synth.WORKLOADS["shard"]
    g = _load("shard")
    t, _ = synth.targets(w)
    rows = _rows(w.N, 30, seed=1)
    assert np.any(t[rows] == synth.IGNORE_INDEX) and np.any(t[rows] != synth.IGNORE_INDEX)
    hk = synth.hidden(w).values[rows]
    part = O.shard_partials(hk, synth.weight(w, shard=w.shard_k).values, t[rows], w.vocab_start,
                            w.logit_scale)
    rest = (g["rest_lse"][rows], np.ones(len(rows)), g["rest_target"][rows], g["rest_sum"][rows])
    lse, zt, zs = O.combine_shard_partials([part, rest])
    np.testing.assert_allclose(lse, g["lse"][rows], rtol=1e-12)
    np.testing.assert_allclose(zt, g["z_target"][rows], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(zs, g["z_sum"][rows], rtol=1e-9, atol=1e-9)
