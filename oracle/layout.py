"""Token-to-device maps for the ring, written as plain loops -- TEST INFRASTRUCTURE.

* contiguous: the sequence is cut into N equal chunks, chunk i on device i
  ("Ring Attention" (Ultralytics glossary), section "How ring attention works",
  where the sequence is split into N blocks; "Context Parallelism" (freenetmedia),
  section "How context parallelism works": a length-S sequence becomes N pieces
  of S/N tokens).
* striped: the pages' fix for causal load imbalance gives every device tokens
  spread evenly along the sequence ("Ring Attention", same section).  Reading
  taken: round-robin, token t on device t mod N as its local row t div N.

Shard layout used by the GPU library: position-major [N, B, H, S/N, d].
"""
from __future__ import annotations

import numpy as np


def device_of(t, S, n, layout):
    """(device, local row) of global token t."""
    sb = S // n
    if layout == "contiguous":
        return t // sb, t % sb
    if layout == "striped":
        return t % n, t // n
    raise ValueError(layout)


def tokens_of(i, S, n, layout):
    """Global token positions held by device i, in local row order (int64 array)."""
    sb = S // n
    out = np.empty(sb, dtype=np.int64)
    for t in range(S):
        dev, row = device_of(t, S, n, layout)
        if dev == i:
            out[row] = t
    return out


def to_shards(x, n, layout):
    """[B, H, S, d] -> [N, B, H, S/N, d] by per-token copies."""
    B, H, S, d = x.shape
    if S % n:
        raise ValueError("sequence length must be a multiple of the ring size")
    y = np.empty((n, B, H, S // n, d), dtype=x.dtype)
    for t in range(S):
        dev, row = device_of(t, S, n, layout)
        y[dev, :, :, row, :] = x[:, :, t, :]
    return y


def from_shards(y, layout):
    """[N, B, H, S/N, d] -> [B, H, S, d], the inverse of ``to_shards``."""
    n, B, H, sb, d = y.shape
    S = n * sb
    x = np.empty((B, H, S, d), dtype=y.dtype)
    for t in range(S):
        dev, row = device_of(t, S, n, layout)
        x[:, :, t, :] = y[dev, :, :, row, :]
    return x
