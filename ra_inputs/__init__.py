"""Seeded synthetic inputs shared by the oracle side and the GPU side.

Holds no attention arithmetic: a counter-based normal generator (Philox4x32-10
plus Box-Muller, in ``gen.c``), bfloat16 widening, and the choice of sampled
query rows.  Tensors are numpy arrays; bfloat16 tensors are carried as their
raw ``uint16`` bit patterns so that both sides see exactly the same values.

Stream ids: Q = 0, K = 1, V = 2.  Default seed 0 (the pages' examples seed 0);
the sampled-row seed is 1.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "libra_inputs.so")
_lib = None

STREAM_Q, STREAM_K, STREAM_V = 0, 1, 2
F32, BF16 = 0, 1


def build() -> str:
    """Compile gen.c into libra_inputs.so (always recompiles)."""
    src = os.path.join(_HERE, "gen.c")
    tmp = _SO + ".tmp"
    subprocess.run(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-std=c11", src,
                    "-o", tmp, "-lm"], check=True)
    os.replace(tmp, _SO)
    global _lib
    _lib = None
    return _SO


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build()
        lib = ctypes.CDLL(_SO)
        lib.rin_normal_rows.restype = ctypes.c_int
        lib.rin_normal_rows.argtypes = [
            ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
            ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int,
            ctypes.c_float, ctypes.c_void_p]
        lib.rin_philox4x32_10.restype = None
        lib.rin_philox4x32_10.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        lib.rin_bf16_to_f32.restype = None
        lib.rin_bf16_to_f32.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64]
        lib.rin_f32_to_bf16_rne.restype = ctypes.c_uint16
        lib.rin_f32_to_bf16_rne.argtypes = [ctypes.c_float]
        _lib = lib
    return _lib


def philox4x32_10(ctr, key):
    """Raw Philox4x32-10 block (for known-answer tests)."""
    c = np.asarray(ctr, dtype=np.uint32).copy()
    k = np.asarray(key, dtype=np.uint32).copy()
    out = np.zeros(4, dtype=np.uint32)
    _load().rin_philox4x32_10(c.ctypes.data, k.ctypes.data, out.ctypes.data)
    return out


def normal(shape, stream_id, seed=0, dtype="bf16", t0=0, t_stride=1, n_rows=None,
           scale=1.0):
    """scale * N(0,1) values of the logical tensor ``shape = (B, H, S, d)``.

    Returns the token rows ``t = t0 + r * t_stride`` for r < n_rows (default: all S
    rows) as an array of shape (B, H, n_rows, d): float32, or uint16 bfloat16 bits.
    """
    B, H, S, d = (int(x) for x in shape)
    n = S if n_rows is None else int(n_rows)
    code = BF16 if dtype == "bf16" else F32
    out = np.empty((B, H, n, d), dtype=np.uint16 if code == BF16 else np.float32)
    rc = _load().rin_normal_rows(seed, stream_id, B, H, S, d, t0, t_stride, n, code,
                                 float(scale), out.ctypes.data)
    if rc != 0:
        raise ValueError("rin_normal_rows rejected its arguments")
    return out


def bf16_to_f32(x: np.ndarray) -> np.ndarray:
    """Widen uint16 bfloat16 bit patterns to float32 (exact)."""
    x = np.ascontiguousarray(x, dtype=np.uint16)
    y = np.empty(x.shape, dtype=np.float32)
    _load().rin_bf16_to_f32(x.ctypes.data, y.ctypes.data, x.size)
    return y


def f32_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 bits, nearest-even (vectorised numpy)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    return ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)


def sample_rows(seq_len, n_pos, n_samples, heads, seed=1, first_last_every=None, share=None,
                layout="contiguous"):
    """Seeded, stratified choice of exactly ``n_samples`` distinct (head, token)
    query rows to check.

    Rows are drawn from every token of the sequence, or with ``share = i`` only
    from ring position i's tokens under ``layout`` (contiguous: tokens
    [i Sb, (i + 1) Sb); striped: tokens i + r N), Sb = seq_len // n_pos.
    Always includes the first and last token of every block of
    ``first_last_every`` tokens (default Sb) that the choice may hold -- for a
    share its first and last token -- and token 0 when it may, each on a seeded
    head; the rest are drawn uniformly (seeded) until exactly n_samples
    distinct pairs are held.  Returns (heads, tokens) int64 arrays sorted by
    (head, token).
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    sb = max(1, seq_len // max(1, n_pos))
    if share is None:
        n_tok = seq_len

        def token(r):
            return r
        blk = first_last_every or sb
        forced_rows = {0, seq_len - 1} | set(range(0, seq_len, blk)) | \
            {min(seq_len - 1, b + blk - 1) for b in range(0, seq_len, blk)}
    else:
        if not 0 <= share < n_pos or seq_len % n_pos:
            raise ValueError("share must name a ring position of an evenly split sequence")
        n_tok = sb

        def token(r):
            return share + r * n_pos if layout == "striped" else share * sb + r
        forced_rows = {0, sb - 1}
    if n_samples > heads * n_tok:
        raise ValueError(f"{n_samples} distinct rows requested, only {heads * n_tok} exist")
    chosen = []
    seen = set()

    def add(h, t):
        if len(chosen) < n_samples and (h, t) not in seen:
            seen.add((h, t))
            chosen.append((h, t))

    forced = sorted(forced_rows)
    for r, h in zip(forced, rng.integers(0, heads, size=len(forced))):
        add(int(h), int(token(r)))
    while len(chosen) < n_samples:
        need = n_samples - len(chosen)
        hs = rng.integers(0, heads, size=need)
        rs = rng.integers(0, n_tok, size=need)
        for h, r in zip(hs, rs):
            add(int(h), int(token(int(r))))
    chosen.sort()
    h = np.array([c[0] for c in chosen], dtype=np.int64)
    t = np.array([c[1] for c in chosen], dtype=np.int64)
    return h, t
