"""Seeded synthetic inputs for the fused linear diffusion cross-entropy.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic, so both the GPU path's tests and the CPU oracle can take
their inputs from it.

Workloads (all shapes and distributions as stated for the masked-diffusion LM
head of the model page "fused_linear_diffusion_cross_entropy.py"):

* ``tiny``      B=2,  L=64,   H=64,   V=1000,   fp32, W ~ N(0, 1/H)
* ``4b``        B=4,  L=512,  H=2560, V=151936, bf16, W ~ N(0, 0.02^2)
* ``headline``  B=8,  L=1024, H=2560, V=151936, bf16, eps=0.1, s=0.5
* ``block``     B=16, L=1024, H=4096, V=151936, bf16, p_mask per 4-token
                 block, trailing 154 tokens of each sequence are padding
* ``shard``     B=16, L=2048, H=5120, vocab shard k=3 of 8 (18992 rows of a
                 151936 vocab), targets uniform over the full vocab

An optional bias b [V] ~ N(0, 1) can be drawn for any workload (``bias``).

Masking recipe (the masked-diffusion forward process): per sequence (or per
block) a masking probability t ~ U(0.05, 1) is drawn; each token is masked
when its own uniform draw u < t.  Masked tokens keep their token id as target,
unmasked tokens get ``ignore_index``; p_mask is t for every token of the
sequence (block).  Padding rows get ``ignore_index`` and p_mask = 1.

Every tensor has its own seed key ``[workload index, tensor id(, shard)]`` so
any tensor (or one vocab shard of W) can be generated without the others.
bf16 values are produced from float32 draws by round-to-nearest-even and are
returned both as raw uint16 bit patterns and as the exactly-representable
float32 values.
"""

from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

IGNORE_INDEX = -100

_T_ID, _TT_ID, _U_ID, _H_ID, _W_ID, _B_ID = 0, 1, 2, 3, 4, 5


@dataclasses.dataclass(frozen=True)
class Workload:
    index: int
    name: str
    B: int
    L: int
    H: int
    V: int                      # global vocabulary size
    dtype: str                  # "f32" or "bf16"
    w_std: float
    label_smoothing: float = 0.0
    logit_scale: float = 1.0
    reduction: str = "mean"     # "mean" or "sum"
    total_is_N: bool = True     # mean divisor = N ("sum/N"); False: count non-ignored
    p_block: int = 0            # >0: t drawn per block of this many tokens
    pad_tail: int = 0           # trailing padding tokens per sequence
    shards: int = 1             # vocab shards (only the shard workload)
    shard_k: int = 0

    @property
    def N(self) -> int:
        return self.B * self.L

    @property
    def V_local(self) -> int:
        return self.V // self.shards

    @property
    def vocab_start(self) -> int:
        return self.shard_k * self.V_local

    @property
    def total(self) -> int:
        """Divisor passed to the library: N for "sum/N", 0 for "count on device"."""
        return self.N if self.total_is_N else 0


WORKLOADS = {
    "tiny": Workload(0, "tiny", 2, 64, 64, 1000, "f32", 1.0 / 8.0),
    "4b": Workload(1, "4b", 4, 512, 2560, 151936, "bf16", 0.02),
    "headline": Workload(2, "headline", 8, 1024, 2560, 151936, "bf16", 0.02,
                         label_smoothing=0.1, logit_scale=0.5),
    "block": Workload(3, "block", 16, 1024, 4096, 151936, "bf16", 0.02,
                      total_is_N=False, p_block=4, pad_tail=154),
    "shard": Workload(4, "shard", 16, 2048, 5120, 151936, "bf16", 0.02,
                      shards=8, shard_k=3),
}


def custom(name: str, B: int, L: int, H: int, V: int, dtype: str = "bf16",
           w_std: Optional[float] = None, index: int = 100, **kw) -> Workload:
    """A workload with the same recipe at other sizes (parity cases, edges)."""
    if w_std is None:
        w_std = 0.02 if dtype == "bf16" else 1.0 / np.sqrt(H)
    return Workload(index, name, B, L, H, V, dtype, float(w_std), **kw)


def _rng(*key: int) -> np.random.Generator:
    return np.random.default_rng(list(key))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclasses.dataclass
class Tensor:
    """A generated tensor: exact float32 values, plus bf16 bits if bf16."""
    values: np.ndarray                  # float32, exactly the stored values
    bits: Optional[np.ndarray] = None   # uint16 bf16 bit patterns, or None for fp32


def _as_dtype(x32: np.ndarray, dtype: str) -> Tensor:
    if dtype == "bf16":
        bits = f32_to_bf16_bits(x32)
        return Tensor(bf16_bits_to_f32(bits), bits)
    return Tensor(np.ascontiguousarray(x32, dtype=np.float32), None)


def targets(w: Workload):
    """(target int64 [N], p_mask float32 [N]) for a workload."""
    N, L = w.N, w.L
    tok = _rng(w.index, _T_ID).integers(0, w.V, size=N, dtype=np.int64)
    if w.p_block:
        nblk = N // w.p_block
        t = _rng(w.index, _TT_ID).uniform(0.05, 1.0, size=nblk)
        p = np.repeat(t, w.p_block)
    else:
        t = _rng(w.index, _TT_ID).uniform(0.05, 1.0, size=w.B)
        p = np.repeat(t, L)
    u = _rng(w.index, _U_ID).uniform(0.0, 1.0, size=N)
    masked = u < p
    target = np.where(masked, tok, IGNORE_INDEX).astype(np.int64)
    p_mask = p.astype(np.float32)
    if w.pad_tail:
        pos = np.arange(N) % L
        pad = pos >= (L - w.pad_tail)
        target[pad] = IGNORE_INDEX
        p_mask[pad] = 1.0
    return target, p_mask


def hidden(w: Workload) -> Tensor:
    """h [N, H] ~ N(0, 1)."""
    x = _rng(w.index, _H_ID).standard_normal((w.N, w.H), dtype=np.float32)
    return _as_dtype(x, w.dtype)


def weight(w: Workload, shard: Optional[int] = None) -> Tensor:
    """W [V, H] ~ N(0, w_std^2); for a sharded workload, shard ``shard`` only
    ([V_local, H]) or, with shard=None, the concatenation of all shards."""
    if w.shards == 1:
        x = _rng(w.index, _W_ID).standard_normal((w.V, w.H), dtype=np.float32)
        x *= np.float32(w.w_std)
        return _as_dtype(x, w.dtype)
    ks = range(w.shards) if shard is None else [shard]
    parts = []
    for k in ks:
        x = _rng(w.index, _W_ID, k).standard_normal((w.V_local, w.H), dtype=np.float32)
        x *= np.float32(w.w_std)
        parts.append(x)
    x = parts[0] if len(parts) == 1 else np.concatenate(parts, axis=0)
    return _as_dtype(x, w.dtype)


def bias(w: Workload) -> Tensor:
    """b [V] ~ N(0, 1): an input for the optional bias of the LM head (the
    model page's functions accept one; its workloads use none)."""
    x = _rng(w.index, _B_ID).standard_normal(w.V, dtype=np.float32)
    return _as_dtype(x, w.dtype)


def fingerprint(w: Workload) -> str:
    """Short digest of the generated target/p_mask and a corner of h, W (used to
    detect stale stored expected values)."""
    import hashlib
    t, p = targets(w)
    d = hashlib.sha256()
    d.update(t.tobytes())
    d.update(p.tobytes())
    d.update(repr(dataclasses.astuple(w)).encode())
    return d.hexdigest()[:16]
