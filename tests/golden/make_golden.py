"""Write the stored expected row statistics for the large workloads.

For every token row of the ``4b``, ``headline``, ``block`` and ``shard``
workloads (and ``4b_bias``: the ``4b`` inputs with the seeded bias) this
stores the oracle's float64 logsumexp over the FULL vocabulary, the target
logit and the row sum of the logits (``oracle.row_stats``).  For the
vocabulary-shard workload it also stores, for every row, the combine (lse,
target logit, row sum) of the partials of the other shards (``oracle.shard_partials`` of each shard but
the one the GPU computes, then ``oracle.combine_shard_partials``), so a test
can combine the GPU's shard partials with them and compare every row with
the full-vocabulary lse.  The parity tests finish the loss, dH and dW with
the oracle at test time; only these O(N*H*V) float64 GEMMs over the whole
vocabulary are too slow to redo there.  Inputs come from
``lm_head_linear_bf16_amd.synth``; nothing here touches the HIP library.

Usage:  python tests/golden/make_golden.py [workload ...]
"""

import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle as O  # noqa: E402
from lm_head_linear_bf16_amd import synth  # noqa: E402

HERE = os.path.dirname(os.path.abspath(__file__))


def path_for(name: str) -> str:
    return os.path.join(HERE, f"rowstats_{name}.npz")


def make(name: str) -> None:
    with_bias = name.endswith("_bias")
    w = synth.WORKLOADS[name[:-5] if with_bias else name]
    t0 = time.time()
    target, _ = synth.targets(w)
    h = synth.hidden(w).values
    W = synth.weight(w).values               # full vocabulary (all shards)
    b = synth.bias(w).values if with_bias else None
    lse, zt, zs = O.row_stats(h, W, target, np.arange(w.N), w.logit_scale, row_block=1024,
                              bias=b)
    extra = {}
    if w.shards > 1:  # the other shards' partials, combined (every row, ignored ones too)
        # (ignored rows have a target in no shard: their partials are those of every row)
        parts = [O.shard_partials(h, synth.weight(w, shard=j).values, target, j * w.V_local,
                                  w.logit_scale)
                 for j in range(w.shards) if j != w.shard_k]
        rl, rt, rs = O.combine_shard_partials(parts)
        extra = dict(rest_lse=rl, rest_target=rt, rest_sum=rs)
    np.savez(path_for(name), lse=lse, z_target=zt, z_sum=zs,
             fingerprint=np.array(synth.fingerprint(w)), **extra)
    print(f"{name}: N={w.N} H={w.H} V={w.V} in {time.time() - t0:.1f}s", flush=True)


if __name__ == "__main__":
    names = sys.argv[1:] or ["4b", "headline", "block", "shard", "4b_bias"]
    for n in names:
        make(n)
