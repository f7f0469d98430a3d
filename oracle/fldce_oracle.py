"""Float64 CPU oracle of the fused linear diffusion cross-entropy.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the tests, the smoke check and the benchmark's
``cpu_baseline`` leg use it.  It shares no code with the HIP library.

It is the plain definition written out, in float64 NumPy, one step per
function, each following a passage of the pages:

* Page 1, "fused_linear_diffusion_cross_entropy.py" (a Hugging Face model
  file; Python + Triton).  Its ``fused_linear_cross_entropy_forward`` forms
  the logits with ``F.linear`` and a logit scale, ``logsumexp_fwd`` /
  ``logsumexp_fwd_kernel`` take a max-shifted row logsumexp,
  ``cross_entropy_kernel`` steps 4-6 give the per-row loss (divided by the
  per-token masking probability p_mask, the "diffusion scaled 1/t" rule),
  the label-smoothing term, and the gradient (softmax - eps/V, target entry
  minus (1 - eps), all scaled by logit_scale / p_mask / total), and the
  chunk loop turns that gradient into dx = g W and dw = g^T x.
* Page 3, the tensor-parallel tutorial (daliqc.cn developer article
  673292621566021), section 4 "output-layer embedding": a vocabulary split
  where each shard sums its own exp, the per-row denominators are combined,
  and each shard finishes its softmax locally.

Readings where the pages leave a step open (each listed in the design notes):

* The whole label-smoothed CE of a row is divided by p_i (the page's loss
  divides only the hard-label part, while its gradient divides every term;
  the gradient and the "unreduced_loss /= p_mask" guideline the module
  docstring cites fix the reading).  ``row_losses_literal`` keeps the
  page's literal loss for reference only.
* eps / V always uses the global vocabulary size, also inside one shard.
* Shard partials are max-shifted (page 1's two-stage logsumexp) rather than
  page 3's raw sum of exp; the combined result is the same number.
* The ``mean`` divisor D is the caller's ``total`` when given (> 0), else the
  number of non-ignored rows (page 1 counts them with ``target.ne``).  An
  all-ignored batch gives loss 0 and zero gradients.
* p_mask of an ignored row is never used (page 1 returns before using it).
* The optional bias enters the logits before the logit scale
  (z = s (h W^T + b): ``F.linear(c_x, weight, bias)`` then the kernels'
  scale), and db is the column sum of the same gradient g over the rows.
* The end-of-block weight w of the module's forward divides p_mask by w on
  the rows whose target is the EOB token (so their loss and gradient are
  multiplied by w); the oracle applies it exactly that way.

Rows are processed in blocks purely to bound memory; each row's arithmetic is
the same as with a single block.
"""

from __future__ import annotations

import math
from typing import Optional, Sequence

import numpy as np

__all__ = [
    "scaled_logits", "row_logsumexp", "valid_rows", "divisor", "row_losses",
    "row_losses_literal", "dlogits", "forward_backward", "row_stats",
    "dH_rows", "dW_rows", "shard_partials", "combine_shard_partials",
    "shard_backward", "loss_from_row_losses", "eob_p_mask", "forward",
    "scale_grads",
]

_F = np.float64


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=_F)


# -- step 1: logits --------------------------------------------------------
def scaled_logits(h, W, logit_scale: float, bias=None) -> np.ndarray:
    """z = s * (h W^T + b).  Page 1: ``F.linear(c_x, weight, bias)`` in the
    chunk loop, and the kernels multiply every loaded logit by
    ``logit_scale``.  ``bias`` is None (no bias) or [V]."""
    a = _f64(h) @ _f64(W).T
    if bias is not None:
        a = a + _f64(bias)[None, :]
    return float(logit_scale) * a


# -- step 2: per-row logsumexp ---------------------------------------------
def row_logsumexp(z) -> np.ndarray:
    """lse_i = m_i + log sum_j exp(z_ij - m_i), m_i = max_j z_ij.
    Page 1: ``logsumexp_fwd_kernel`` (max, then log of the shifted exp sum,
    plus the max) and its host combine ``z.logsumexp(-1)``."""
    z = _f64(z)
    m = z.max(axis=1)
    return m + np.log(np.exp(z - m[:, None]).sum(axis=1))


# -- step 0: which rows count, and the reduction divisor -------------------
def valid_rows(target, ignore_index: int) -> np.ndarray:
    """Page 1, ``cross_entropy_kernel`` step 2: a row whose target equals
    ``ignore_index`` contributes nothing."""
    return np.asarray(target) != ignore_index


def divisor(valid, reduction: str, total: Optional[int] = None) -> float:
    """D = 1 for "sum"; for "mean" the caller's total if > 0, else the number
    of non-ignored rows (page 1: ``total = target.ne(ignore_index).sum()``).
    D = 1 if that count is 0 (no row then contributes)."""
    if reduction == "sum":
        return 1.0
    if reduction != "mean":
        raise ValueError(f"reduction {reduction!r}")
    if total is not None and total > 0:
        return float(total)
    n = int(np.count_nonzero(valid))
    return float(n) if n > 0 else 1.0


def eob_p_mask(target, p_mask, eob_token_id: Optional[int], eob_weight: float):
    """Page 1, ``FusedLinearDiffusionCrossEntropyLoss.forward``: when an EOB
    token id is given and its weight is not 1, p_mask is copied and divided
    by the weight on the rows whose target is that token (the kernel divides
    each row's loss by p_mask, so their loss is multiplied by the weight)."""
    p = _f64(p_mask).copy()
    if eob_token_id is None or eob_weight == 1.0:
        return p
    eob = np.asarray(target) == eob_token_id
    with np.errstate(divide="ignore"):     # weight 0: p = inf, the rows add nothing
        p[eob] = p[eob] / float(eob_weight)
    return p


# -- step 3: per-row loss --------------------------------------------------
def row_losses(lse, z_target, z_sum, V: int, p_mask, valid,
               label_smoothing: float) -> np.ndarray:
    """l_i = [(1 - eps)(lse_i - z_{i,y_i}) + eps (lse_i - z_sum_i / V)] / p_i,
    and 0 on ignored rows.  Page 1, ``cross_entropy_kernel``: step 4 (hard
    label CE lse - z_y, divided by p_mask) and the label-smoothing combine
    after step 5 (eps * (lse - mean_j z_ij) is H(u, p)); whole CE divided by
    p_i as read above."""
    lse, z_target, z_sum = _f64(lse), _f64(z_target), _f64(z_sum)
    eps = float(label_smoothing)
    ce = lse - z_target
    uni = lse - z_sum / float(V)
    valid = np.asarray(valid, dtype=bool)
    p = np.where(valid, _f64(p_mask), 1.0)
    out = ((1.0 - eps) * ce + eps * uni) / p
    return np.where(valid, out, 0.0)


def row_losses_literal(lse, z_target, z_sum, V: int, p_mask, valid,
                       label_smoothing: float) -> np.ndarray:
    """The page's loss exactly as printed: only the hard-label term is divided
    by p_i, the smoothing term is added undivided.  Reference only: it is not
    the loss whose gradient the page computes when eps > 0 and p != 1."""
    lse, z_target, z_sum = _f64(lse), _f64(z_target), _f64(z_sum)
    eps = float(label_smoothing)
    valid = np.asarray(valid, dtype=bool)
    p = np.where(valid, _f64(p_mask), 1.0)
    out = (1.0 - eps) * (lse - z_target) / p + eps * (lse - z_sum / float(V))
    return np.where(valid, out, 0.0)


def loss_from_row_losses(row_loss, D: float) -> float:
    """loss = (sum_i l_i) / D (page 1: ``loss.sum()`` after the per-row division
    by total).  math.fsum keeps the sum exact to one rounding."""
    return math.fsum(np.asarray(row_loss, dtype=_F).ravel().tolist()) / D


# -- step 4: gradient w.r.t. the raw logits a = h W^T ----------------------
def dlogits(z, lse, target_col, p_mask, valid, D: float,
            label_smoothing: float, logit_scale: float,
            V_global: int) -> np.ndarray:
    """g_ij = s / (p_i D) * (exp(z_ij - lse_i) - eps / V - (1 - eps)[j = y_i]);
    g_i = 0 on ignored rows.  Page 1, ``cross_entropy_kernel`` step 5 (the
    softmax minus eps/V, times logit_scale, divided by p_mask and total) and
    step 6 (the target entry gets (eps - 1) * s / p / total added).

    ``target_col`` is the column of the target inside ``z`` (or -1 when the
    target is not among these columns: a vocabulary shard)."""
    z = _f64(z)
    eps = float(label_smoothing)
    valid = np.asarray(valid, dtype=bool)
    p = np.where(valid, _f64(p_mask), 1.0)
    c = float(logit_scale) / (p * D)
    g = np.exp(z - _f64(lse)[:, None]) - eps / float(V_global)
    tc = np.asarray(target_col)
    rows = np.nonzero(valid & (tc >= 0))[0]
    g[rows, tc[rows]] -= (1.0 - eps)
    g *= c[:, None]
    g[~valid] = 0.0
    return g


# -- full problem ----------------------------------------------------------
def forward_backward(h, W, target, p_mask=None, ignore_index: int = -100,
                     label_smoothing: float = 0.0, logit_scale: float = 1.0,
                     reduction: str = "mean", total: Optional[int] = None,
                     row_block: int = 1024, need_grads: bool = True, bias=None,
                     eob_token_id: Optional[int] = None, eob_weight: float = 1.0):
    """loss, dH = g W, dW = g^T h (page 1: the chunk loop's ``torch.mm`` and
    ``c_logits.t() @ c_x``) and, with a bias, db = sum_i g_i (the loop's
    ``c_logits.sum(0)``).  Returns a dict with loss, dH, dW, db (None without
    a bias), lse, row_loss, D and the literal-reading loss (reference only)."""
    h, W = _f64(h), _f64(W)
    target = np.asarray(target, dtype=np.int64)
    N, H = h.shape
    V = W.shape[0]
    if p_mask is None:                      # page 1 module: None -> ones
        p_mask = np.ones(N)
    p_mask = eob_p_mask(target, p_mask, eob_token_id, eob_weight)
    valid = valid_rows(target, ignore_index)
    if np.any(valid & ((target < 0) | (target >= V))):
        raise ValueError("target out of range")
    D = divisor(valid, reduction, total)
    lse = np.empty(N)
    rl = np.empty(N)
    rl_lit = np.empty(N)
    dH = np.zeros((N, H)) if need_grads else None
    dW = np.zeros((V, H)) if need_grads else None
    db = np.zeros(V) if (need_grads and bias is not None) else None
    tcol = np.where(valid, target, -1)
    for r0 in range(0, N, row_block):
        r1 = min(N, r0 + row_block)
        z = scaled_logits(h[r0:r1], W, logit_scale, bias)
        lse[r0:r1] = row_logsumexp(z)
        zt = np.where(valid[r0:r1], z[np.arange(r1 - r0), np.maximum(tcol[r0:r1], 0)], 0.0)
        zs = z.sum(axis=1)
        args = (lse[r0:r1], zt, zs, V, p_mask[r0:r1], valid[r0:r1], label_smoothing)
        rl[r0:r1] = row_losses(*args)
        rl_lit[r0:r1] = row_losses_literal(*args)
        if need_grads:
            g = dlogits(z, lse[r0:r1], tcol[r0:r1], p_mask[r0:r1], valid[r0:r1], D,
                        label_smoothing, logit_scale, V)
            dH[r0:r1] = g @ W
            dW += g.T @ h[r0:r1]
            if db is not None:
                db += g.sum(axis=0)
    return dict(loss=loss_from_row_losses(rl, D), dH=dH, dW=dW, db=db, lse=lse,
                row_loss=rl, D=D, loss_literal=loss_from_row_losses(rl_lit, D))


def forward(h, W, target, p_mask=None, **kw):
    """Loss, per-row lse and per-row loss without gradients (the forward half
    of page 1's chunk loop: ``F.linear``, ``logsumexp_fwd`` and the loss part
    of ``cross_entropy_kernel``)."""
    r = forward_backward(h, W, target, p_mask, need_grads=False, **kw)
    return dict(loss=r["loss"], lse=r["lse"], row_loss=r["row_loss"], D=r["D"])


def scale_grads(do: float, *grads):
    """Page 1, ``fused_linear_cross_entropy_backward``: the gradients computed
    in the forward pass are for d(loss) = 1; with an upstream gradient
    ``do`` != 1 each is multiplied by it (skipped when do == 1).  None
    entries stay None."""
    if do == 1.0:
        return tuple(grads)
    return tuple(None if g is None else _f64(g) * float(do) for g in grads)


# -- sampled pieces for large problems --------------------------------------
def row_stats(h, W, target, rows: Sequence[int], logit_scale: float,
              ignore_index: int = -100, row_block: int = 512, bias=None):
    """(lse, z_target, z_sum) of the given rows over the full vocabulary."""
    h, W = _f64(h), _f64(W)
    rows = np.asarray(rows, dtype=np.int64)
    target = np.asarray(target, dtype=np.int64)
    lse = np.empty(len(rows))
    zt = np.zeros(len(rows))
    zs = np.empty(len(rows))
    for b0 in range(0, len(rows), row_block):
        rr = rows[b0:b0 + row_block]
        z = scaled_logits(h[rr], W, logit_scale, bias)
        lse[b0:b0 + len(rr)] = row_logsumexp(z)
        zs[b0:b0 + len(rr)] = z.sum(axis=1)
        t = target[rr]
        ok = t != ignore_index
        zt[b0:b0 + len(rr)][ok] = z[np.nonzero(ok)[0], t[ok]]
    return lse, zt, zs


def dH_rows(h, W, target, p_mask, lse_rows, rows, D, label_smoothing,
            logit_scale, ignore_index=-100, V_global=None, vocab_start=0, bias=None):
    """dH for the given rows: g_rows W (needs only those rows' lse).  ``W`` may
    be a vocabulary shard starting at ``vocab_start`` of a ``V_global`` vocab
    (then this is the shard's dH_partial)."""
    h, W = _f64(h), _f64(W)
    rows = np.asarray(rows, dtype=np.int64)
    t = np.asarray(target, dtype=np.int64)[rows]
    V_global = W.shape[0] if V_global is None else V_global
    valid = t != ignore_index
    ins = valid & (t >= vocab_start) & (t < vocab_start + W.shape[0])
    z = scaled_logits(h[rows], W, logit_scale, bias)
    g = dlogits(z, lse_rows, np.where(ins, t - vocab_start, -1), np.asarray(p_mask)[rows],
                valid, D, label_smoothing, logit_scale, V_global)
    return g @ W


def dW_rows(h, W, target, p_mask, lse_all, vocab_rows, D, label_smoothing,
            logit_scale, ignore_index=-100, V_global=None, vocab_start=0, bias=None,
            with_db: bool = False):
    """dW for the given vocabulary rows (of ``W``, which may be a shard that
    starts at ``vocab_start`` in a vocabulary of ``V_global``): g[:, j]^T h
    over all token rows (needs every row's lse).  With ``with_db`` also returns
    db of those vocabulary rows (the column sums of g)."""
    h = _f64(h)
    vr = np.asarray(vocab_rows, dtype=np.int64)
    Wr = _f64(W)[vr]
    target = np.asarray(target, dtype=np.int64)
    V_global = W.shape[0] if V_global is None else V_global
    valid = target != ignore_index
    z = scaled_logits(h, Wr, logit_scale, None if bias is None else _f64(bias)[vr])
    # column index of the target among the selected vocab rows (or -1)
    gcol = vocab_start + vr
    pos = {int(v): i for i, v in enumerate(gcol)}
    tc = np.array([pos.get(int(y), -1) if ok else -1 for y, ok in zip(target, valid)])
    g = dlogits(z, lse_all, tc, p_mask, valid, D, label_smoothing, logit_scale, V_global)
    if with_db:
        return g.T @ h, g.sum(axis=0)
    return g.T @ h


# -- vocabulary shards (page 3, section 4) ---------------------------------
def shard_partials(h, W_local, target, vocab_start: int, logit_scale: float,
                   ignore_index: int = -100, row_block: int = 1024):
    """Per-row partials of one vocabulary shard [v0, v0 + V_local):
    m = max_j z_ij, S = sum_j exp(z_ij - m), t = z_{i,y_i} if y_i is in the
    shard (and the row is not ignored) else 0, r = sum_j z_ij.
    Page 3 section 4: each shard sums exp of its own logits; page 1's
    logsumexp kernel keeps the per-block max alongside the shifted sum."""
    h, W_local = _f64(h), _f64(W_local)
    target = np.asarray(target, dtype=np.int64)
    N = h.shape[0]
    Vl = W_local.shape[0]
    m = np.empty(N)
    S = np.empty(N)
    t = np.zeros(N)
    r = np.empty(N)
    for r0 in range(0, N, row_block):
        r1 = min(N, r0 + row_block)
        z = scaled_logits(h[r0:r1], W_local, logit_scale)
        m[r0:r1] = z.max(axis=1)
        S[r0:r1] = np.exp(z - m[r0:r1, None]).sum(axis=1)
        r[r0:r1] = z.sum(axis=1)
        y = target[r0:r1]
        ins = (y != ignore_index) & (y >= vocab_start) & (y < vocab_start + Vl)
        idx = np.nonzero(ins)[0]
        t[r0:r1][idx] = z[idx, y[idx] - vocab_start]
    return m, S, t, r


def combine_shard_partials(parts):
    """Combine shard partials [(m, S, t, r), ...] into (lse, z_target, z_sum):
    M = max_k m_k, lse = M + log sum_k S_k exp(m_k - M), z_target = sum_k t_k,
    z_sum = sum_k r_k.  Page 3 section 4: the per-row exp sums are added over
    the shards (the all-reduce of the softmax denominator)."""
    ms = np.stack([_f64(p[0]) for p in parts])
    Ss = np.stack([_f64(p[1]) for p in parts])
    M = ms.max(axis=0)
    lse = M + np.log((Ss * np.exp(ms - M[None, :])).sum(axis=0))
    zt = np.stack([_f64(p[2]) for p in parts]).sum(axis=0)
    zs = np.stack([_f64(p[3]) for p in parts]).sum(axis=0)
    return lse, zt, zs


def shard_backward(h, W_local, target, p_mask, lse, vocab_start: int,
                   V_global: int, D: float, label_smoothing: float,
                   logit_scale: float, ignore_index: int = -100,
                   row_block: int = 1024):
    """Given each row's global lse: dH_partial = g[:, shard] W_local and
    dW_local = g[:, shard]^T h, with eps / V over the global vocabulary and
    the target column y - v0 when it falls in the shard.  Summing dH_partial
    over shards gives dH (page 3 section 1.1: a row split of the product
    summed across devices); concatenating dW_local gives dW."""
    h, W_local = _f64(h), _f64(W_local)
    target = np.asarray(target, dtype=np.int64)
    N, H = h.shape
    Vl = W_local.shape[0]
    valid = target != ignore_index
    ins = valid & (target >= vocab_start) & (target < vocab_start + Vl)
    tcol = np.where(ins, target - vocab_start, -1)
    dH = np.zeros((N, H))
    dW = np.zeros((Vl, H))
    for r0 in range(0, N, row_block):
        r1 = min(N, r0 + row_block)
        z = scaled_logits(h[r0:r1], W_local, logit_scale)
        g = dlogits(z, _f64(lse)[r0:r1], tcol[r0:r1], np.asarray(p_mask)[r0:r1],
                    valid[r0:r1], D, label_smoothing, logit_scale, V_global)
        dH[r0:r1] = g @ W_local
        dW += g.T @ h[r0:r1]
    return dH, dW
