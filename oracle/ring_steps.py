"""The ring loop of the pages, in fp64 numpy -- TEST INFRASTRUCTURE (self-tests).

"Ring Attention" (Ultralytics glossary), section "How ring attention works":
the sequence is cut into N blocks, one per device; device i keeps query block i
for the whole computation and, at each of N steps, works on the key/value block
it currently holds -- the block that arrived from the previous device, i.e.
block (i - step) mod N -- while it forwards that block to the next device.  Each
device keeps running sums of the exponentiated scores (denominator) and of the
score-weighted values (numerator), and divides one by the other at the end.
The same passage notes that production kernels also subtract a running maximum
before exponentiating; ``ring_online`` is that variant, merging per-step
partials with the online softmax of flash attention.

These routines simulate the N devices as loop iterations on one CPU, as the
pages' own four-device demonstration does.  They exist to pin the claim
"ring result == full softmax attention" against the C oracle, for any visit
order, for the causal mask and for both token layouts.
"""
from __future__ import annotations

import numpy as np

from . import layout as _layout


def _visit(i, step, n, order):
    """Block held by device i at a step: (i - step) mod N, or a permuted step offset."""
    off = step if order is None else order[step]
    return (i - off) % n


def ring_no_max(q, k, v, n_dev, visit_order=None, scale=None, dtype=np.float64):
    """Non-causal ring over contiguous blocks, plain exp sums (no running max).

    What the ring computes, stated as one reduction: the sequence is cut into
    N equal blocks; after s hops device i holds key/value block (i - s) mod N
    (or the block a permuted step order puts there), so over N hops every
    device meets every block once.  Device i's output is the ratio of two sums
    over the blocks in the order they arrive: of the exp-weighted values
    exp(sigma q k^T) v and of the weights exp(sigma q k^T) themselves.  All
    devices and all hops are evaluated at once as a grid of score blocks
    [hop, device, query, key]; the sums over hops run in arrival order.

    q, k, v: [S, d] with S a multiple of n_dev.  Arithmetic in ``dtype`` (fp64
    by default; fp32 reproduces the pages' single-precision demonstration).
    Returns (out [S, d], shape of one device's score block).
    """
    q, k, v = (np.asarray(a, dtype=dtype) for a in (q, k, v))
    S, d = q.shape
    if S % n_dev:
        raise ValueError("the sequence must split into equal blocks")
    sig = dtype(scale or 1.0 / np.sqrt(d))
    qb, kb, vb = (a.reshape(n_dev, S // n_dev, d) for a in (q, k, v))
    offsets = np.arange(n_dev) if visit_order is None else np.asarray(visit_order)
    held = (np.arange(n_dev)[None, :] - offsets[:, None]) % n_dev  # [hop, device]: block held
    weights = np.exp(np.einsum("iqd,hikd->hiqk", qb, kb[held]) * sig)
    weighted = np.einsum("hiqk,hikd->hiqd", weights, vb[held])
    mass = weights.sum(axis=3)
    out = np.cumsum(weighted, axis=0)[-1] / np.cumsum(mass, axis=0)[-1][..., None]
    return out.reshape(S, d), weights.shape[2:]


def block_partial(qi, qpos, kj, vj, kpos, causal, sig):
    """(m, l, numerator) of one query block against one key/value block.

    m = row max of the allowed scaled scores (-inf if none), l = sum exp(s - m),
    numerator = sum exp(s - m) v.  Masked entries contribute nothing.
    """
    s = qi @ kj.T * sig
    if causal:
        s = np.where(kpos[None, :] <= qpos[:, None], s, -np.inf)
    m = s.max(axis=1)
    safe = np.where(np.isfinite(m), m, 0.0)
    p = np.exp(s - safe[:, None])
    return m, p.sum(axis=1), p @ vj


def merge(a, b):
    """Online-softmax merge of two partials (m, l, numerator); -inf rows weigh 0."""
    ma, la, na = a
    mb, lb, nb = b
    m = np.maximum(ma, mb)
    safe = np.where(np.isfinite(m), m, 0.0)
    wa = np.where(np.isfinite(ma), np.exp(ma - safe), 0.0)
    wb = np.where(np.isfinite(mb), np.exp(mb - safe), 0.0)
    return m, wa * la + wb * lb, wa[:, None] * na + wb[:, None] * nb


def ring_online(q, k, v, n_dev, causal=False, layout="contiguous", visit_order=None,
                scale=None):
    """Ring with a running max: per-step block partials merged online.

    q, k, v: [S, d] in global token order.  Tokens are assigned to devices by
    ``layout`` ("contiguous" chunks or "striped" round-robin); masking uses the
    tokens' global positions.  Returns (o [S, d], lse [S]) in global order.
    """
    q, k, v = (np.asarray(a, dtype=np.float64) for a in (q, k, v))
    S, d = q.shape
    sig = scale or 1.0 / np.sqrt(d)
    owner = [_layout.tokens_of(i, S, n_dev, layout) for i in range(n_dev)]
    o = np.zeros((S, d))
    lse = np.zeros(S)
    for i in range(n_dev):
        ti = owner[i]
        acc = (np.full(len(ti), -np.inf), np.zeros(len(ti)), np.zeros((len(ti), d)))
        for step in range(n_dev):
            j = _visit(i, step, n_dev, visit_order)
            tj = owner[j]
            part = block_partial(q[ti], ti, k[tj], v[tj], tj, causal, sig)
            acc = merge(acc, part)
        m, l, num = acc
        o[ti] = num / l[:, None]
        lse[ti] = m + np.log(l)
    return o, lse
