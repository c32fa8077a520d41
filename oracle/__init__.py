"""CPU fp64 oracle for ring attention's blockwise forward -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the benchmark's ``cpu_baseline``
leg may import this package.  It shares no code with the GPU path
(``ring_attention_step_amd``) and imports nothing from it.

* ``rows``       -- the C routine ``ra_oracle_rows`` (attention_oracle.c): full
                    softmax attention of given query rows over a key set, fp64,
                    plus the (M, Z, numerator) partial of that key set.
* ``grads``      -- the C routine ``ra_oracle_grads``: dQ, dK, dV of that
                    attention for an upstream gradient dO (the backward pass the
                    pages run: "Context Parallelism", "Practical use and
                    trade-offs"), and one key block's share of them given the
                    rows' full-key-set lse and D = dO . O.
* ``attention``  -- [B, H, S, d] wrapper with the grouped-query head mapping.
* ``attention_grads`` -- [B, H, S, d] gradients, dK and dV summed over the
                    query heads that share a key/value head.
* ``ring_steps`` -- the ring loop of the pages, in fp64 numpy (self-tests only).
* ``layout``     -- contiguous / striped token maps, written as plain loops.

Sources: "Ring Attention" (Ultralytics glossary), section "How ring attention
works" (ring == full softmax attention; running max; striped layout), and
"Context Parallelism" (Ultralytics glossary), section "Practical use and
trade-offs" (causal masking, [B, H, S, d] with the sequence on dim 2).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# RA_ORACLE_LIBRARY names another build of attention_oracle.c (e.g. one with
# sanitizers); by default the in-tree libra_oracle.so
_SO = os.environ.get("RA_ORACLE_LIBRARY") or os.path.join(_HERE, "libra_oracle.so")
_lib = None

F32, BF16 = 0, 1


def build(src: str | None = None, out: str | None = None) -> str:
    """Compile the oracle C source into a shared library (always recompiles)."""
    src = src or os.path.join(_HERE, "attention_oracle.c")
    out = out or _SO
    tmp = out + ".tmp"
    subprocess.run(["gcc", "-O3", "-fopenmp", "-shared", "-fPIC", "-std=c11", src, "-o",
                    tmp, "-lm"], check=True)
    os.replace(tmp, out)
    global _lib
    if out == _SO:
        _lib = None
    return out


def load(path: str | None = None):
    """Load (and on first use build) the oracle library; returns the ctypes handle."""
    global _lib
    if path is None and _lib is not None:
        return _lib
    p = path or _SO
    if not os.path.exists(p):
        build(out=p)
    lib = ctypes.CDLL(p)
    f = lib.ra_oracle_rows
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_int64, ctypes.c_double, ctypes.c_int, ctypes.c_int, ctypes.c_int64,
                  ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                  ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                  ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    g = lib.ra_oracle_grads
    g.restype = ctypes.c_int
    g.argtypes = [ctypes.c_int64, ctypes.c_double, ctypes.c_int, ctypes.c_int, ctypes.c_int64,
                  ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                  ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                  ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    if path is None:
        _lib = lib
    return lib


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    raise TypeError(f"oracle inputs are float32 or uint16 bfloat16 bits, got {a.dtype}")


def _ptr(a):
    return None if a is None else a.ctypes.data


def rows(q, k, v, q_pos=None, k_pos=None, causal=False, scale=None, lib=None):
    """Attention of query rows q [n, d] over keys k, v [n_keys, d] (one head).

    q_pos / k_pos: int64 global positions (needed for causal; k_pos defaults to
    0..n_keys-1).  Returns a dict of fp64 arrays: o [n, d], lse [n], and the
    partial of this key set: m [n] (max scaled score), l [n] (sum of exp(s - m))
    and o_num [n, d] (sum of exp(s - m) v).
    """
    q = np.ascontiguousarray(q)
    k = np.ascontiguousarray(k)
    v = np.ascontiguousarray(v)
    code = _dtype_code(q)
    if _dtype_code(k) != code or _dtype_code(v) != code:
        raise TypeError("q, k, v must share a dtype")
    n, d = q.shape
    nk = k.shape[0]
    if k.shape != (nk, d) or v.shape != (nk, d):
        raise ValueError("k, v must be [n_keys, d]")
    qp = None if q_pos is None else np.ascontiguousarray(q_pos, dtype=np.int64)
    kp = None if k_pos is None else np.ascontiguousarray(k_pos, dtype=np.int64)
    if causal and qp is None:
        raise ValueError("causal attention needs query positions")
    out = {"o": np.empty((n, d)), "lse": np.empty(n), "m": np.empty(n), "l": np.empty(n),
           "o_num": np.empty((n, d))}
    rc = (lib or load()).ra_oracle_rows(
        d, float(scale) if scale else 0.0, int(bool(causal)), code, n, _ptr(q), _ptr(qp), nk,
        _ptr(k), _ptr(v), _ptr(kp), _ptr(out["o_num"]), _ptr(out["m"]), _ptr(out["l"]),
        _ptr(out["o"]), _ptr(out["lse"]))
    if rc != 0:
        raise RuntimeError(f"ra_oracle_rows failed ({rc})")
    return out


def attention(q, k, v, causal=False, scale=None, sel_b=None, sel_h=None, sel_t=None,
              lib=None):
    """Full attention for [B, Hq, S, d] q and [B, Hkv, S, d] k, v (global token order).

    Query head h reads key/value head h // (Hq // Hkv) (grouped-query attention,
    consecutive grouping).  With sel_* (equal-length int arrays) only those
    (b, h, t) rows are computed and o [n, d], lse [n] are returned; otherwise
    o [B, Hq, S, d] and lse [B, Hq, S].
    """
    B, Hq, S, d = q.shape
    Hkv = k.shape[1]
    if Hq % Hkv:
        raise ValueError("q heads must be a multiple of kv heads")
    g = Hq // Hkv
    if sel_t is None:
        o = np.empty((B, Hq, S, d))
        lse = np.empty((B, Hq, S))
        pos = np.arange(S, dtype=np.int64)
        for b in range(B):
            for h in range(Hq):
                r = rows(q[b, h], k[b, h // g], v[b, h // g], q_pos=pos, causal=causal,
                         scale=scale, lib=lib)
                o[b, h], lse[b, h] = r["o"], r["lse"]
        return o, lse
    sel_b = np.zeros_like(sel_t) if sel_b is None else np.asarray(sel_b)
    sel_h = np.asarray(sel_h)
    sel_t = np.asarray(sel_t)
    n = sel_t.shape[0]
    o = np.empty((n, d))
    lse = np.empty(n)
    for b in np.unique(sel_b):
        for h in np.unique(sel_h[sel_b == b]):
            idx = np.nonzero((sel_b == b) & (sel_h == h))[0]
            ts = sel_t[idx].astype(np.int64)
            r = rows(q[b, h][ts], k[b, h // g], v[b, h // g], q_pos=ts, causal=causal,
                     scale=scale, lib=lib)
            o[idx], lse[idx] = r["o"], r["lse"]
    return o, lse


def grads(q, k, v, dout, q_pos=None, k_pos=None, causal=False, scale=None, lse=None, delta=None,
          lib=None, key_grads=True):
    """Gradients of one head's attention of query rows q [n, d] over keys k, v [n_keys, d]
    for the upstream gradient dout [n, d] (dtype of q).

    lse / delta (fp64 [n], optional): the rows' log-sum-exp and D = dO . O over
    their full key set; given, the result is this key set's share of the
    gradients.  Returns a dict of fp64 arrays dq [n, d], dk, dv [n_keys, d],
    lse [n], delta [n]; with key_grads=False the per-key pass is skipped and
    dk, dv are None.
    """
    q, k, v, dout = (np.ascontiguousarray(x) for x in (q, k, v, dout))
    code = _dtype_code(q)
    if any(_dtype_code(x) != code for x in (k, v, dout)):
        raise TypeError("q, k, v, dout must share a dtype")
    n, d = q.shape
    nk = k.shape[0]
    if k.shape != (nk, d) or v.shape != (nk, d) or dout.shape != (n, d):
        raise ValueError("shapes: q, dout [n, d]; k, v [n_keys, d]")
    qp = None if q_pos is None else np.ascontiguousarray(q_pos, dtype=np.int64)
    kp = None if k_pos is None else np.ascontiguousarray(k_pos, dtype=np.int64)
    if causal and qp is None:
        raise ValueError("causal attention needs query positions")
    li = None if lse is None else np.ascontiguousarray(lse, dtype=np.float64)
    di = None if delta is None else np.ascontiguousarray(delta, dtype=np.float64)
    out = {"dq": np.empty((n, d)), "dk": np.empty((nk, d)) if key_grads else None,
           "dv": np.empty((nk, d)) if key_grads else None, "lse": np.empty(n), "delta": np.empty(n)}
    rc = (lib or load()).ra_oracle_grads(
        d, float(scale) if scale else 0.0, int(bool(causal)), code, n, _ptr(q), _ptr(qp), _ptr(dout),
        nk, _ptr(k), _ptr(v), _ptr(kp), _ptr(li), _ptr(di), _ptr(out["dq"]), _ptr(out["dk"]),
        _ptr(out["dv"]), _ptr(out["lse"]), _ptr(out["delta"]))
    if rc != 0:
        raise RuntimeError(f"ra_oracle_grads failed ({rc})")
    return out


def attention_grads(q, k, v, dout, causal=False, scale=None, lib=None):
    """dQ [B, Hq, S, d], dK, dV [B, Hkv, S, d] of full attention (global token order).

    Query head h reads key/value head h // (Hq // Hkv); a key/value head's
    gradients are the sum over the query heads that read it.
    """
    B, Hq, S, d = q.shape
    Hkv = k.shape[1]
    if Hq % Hkv:
        raise ValueError("q heads must be a multiple of kv heads")
    g = Hq // Hkv
    dq = np.empty((B, Hq, S, d))
    dk = np.zeros((B, Hkv, S, d))
    dv = np.zeros((B, Hkv, S, d))
    pos = np.arange(S, dtype=np.int64)
    for b in range(B):
        for h in range(Hq):
            r = grads(q[b, h], k[b, h // g], v[b, h // g], dout[b, h], q_pos=pos, causal=causal,
                      scale=scale, lib=lib)
            dq[b, h] = r["dq"]
            dk[b, h // g] += r["dk"]
            dv[b, h // g] += r["dv"]
    return dq, dk, dv
