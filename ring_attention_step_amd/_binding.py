"""ctypes binding of libra.so (include/ra.h): argument marshalling only.

Functions keep the C names.  Tensors are torch tensors on a ROCm device; the
binding reads shapes, strides and data pointers, passes the current HIP
stream, and turns a non-OK status into ``RAError``.  Every computation runs in
the library's HIP kernels; there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# RA_LIBRARY names another build of the same library (e.g. one with host-side
# sanitizers); by default the in-tree libra.so
LIB_PATH = os.environ.get("RA_LIBRARY") or os.path.join(_HERE, "libra.so")

RA_OK, RA_ERR_INVALID, RA_ERR_UNSUPPORTED, RA_ERR_HIP, RA_ERR_WORKSPACE = range(5)
RA_F32, RA_BF16 = 0, 1
RA_CONTIGUOUS, RA_STRIPED = 0, 1
RA_BLOCK_FORCE_SIMT = 1
RA_BLOCK_ACCUMULATE = 2
LAYOUTS = {"contiguous": RA_CONTIGUOUS, "striped": RA_STRIPED}


class RAError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"ra status {status}: {message}")
        self.status = status


class ra_block_desc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("q_heads", ctypes.c_int32), ("kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("q_len", ctypes.c_int64), ("kv_len", ctypes.c_int64),
                ("dtype", ctypes.c_int32), ("causal", ctypes.c_int32), ("scale", ctypes.c_float),
                ("flags", ctypes.c_uint32), ("q_pos0", ctypes.c_int64), ("k_pos0", ctypes.c_int64),
                ("pos_stride", ctypes.c_int64), ("q_strides", ctypes.c_int64 * 3),
                ("k_strides", ctypes.c_int64 * 3), ("v_strides", ctypes.c_int64 * 3)]


class ra_ring_stats(ctypes.Structure):
    _fields_ = [("block_ms", ctypes.c_double), ("merge_ms", ctypes.c_double), ("copy_ms", ctypes.c_double),
                ("block_launches", ctypes.c_int64), ("merge_launches", ctypes.c_int64),
                ("copy_launches", ctypes.c_int64), ("blocks_skipped", ctypes.c_int64),
                ("unmasked_pairs", ctypes.c_double), ("flops", ctypes.c_double), ("kv_splits", ctypes.c_int64)]


class ra_ring_desc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("q_heads", ctypes.c_int32), ("kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("n_pos", ctypes.c_int32), ("first_pos", ctypes.c_int32),
                ("n_run", ctypes.c_int32), ("layout", ctypes.c_int32), ("block_len", ctypes.c_int64),
                ("dtype", ctypes.c_int32), ("causal", ctypes.c_int32), ("scale", ctypes.c_float),
                ("emulate_copy", ctypes.c_int32), ("n_streams", ctypes.c_int32),
                ("separate_merge", ctypes.c_int32), ("kv_splits", ctypes.c_int32),
                ("visit_order", ctypes.POINTER(ctypes.c_int32)),
                ("stats", ctypes.POINTER(ra_ring_stats))]


EXPORTS = ["ra_block_attn_fwd", "ra_lse_merge", "ra_ring_workspace_size", "ra_ring_forward",
           "ra_stripe_permute", "ra_mask_offset", "ra_unmasked_pairs", "ra_ring_pair_offset",
           "ra_last_error", "ra_abi_version", "ra_release", "ra_attn_bwd_delta", "ra_block_attn_bwd",
           "ra_ring_bwd_workspace_size", "ra_ring_backward", "ra_block_attn_fwd_kernel",
           "ra_block_attn_bwd_kernel", "ra_ring_forward_noalloc", "ra_ring_noalloc_max_bytes"]

_lib = None


def load_library(path: str = LIB_PATH):
    """Load libra.so; raises if it has not been built (no fallback exists)."""
    global _lib
    if _lib is not None and path == LIB_PATH:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m ring_attention_step_amd.build` "
                          "(the HIP kernels are the only implementation)")
    lib = ctypes.CDLL(path)
    vp, i32, i64, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
    lib.ra_block_attn_fwd.argtypes = [ctypes.POINTER(ra_block_desc), vp, vp, vp, vp, vp, vp, vp]
    lib.ra_block_attn_fwd.restype = ctypes.c_int
    lib.ra_lse_merge.argtypes = [i64, i32, vp, vp, vp, vp, vp, vp, vp, i32, vp, vp]
    lib.ra_lse_merge.restype = ctypes.c_int
    lib.ra_ring_workspace_size.argtypes = [ctypes.POINTER(ra_ring_desc), ctypes.POINTER(ctypes.c_size_t)]
    lib.ra_ring_workspace_size.restype = ctypes.c_int
    lib.ra_ring_forward.argtypes = [ctypes.POINTER(ra_ring_desc), vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.ra_ring_forward.restype = ctypes.c_int
    lib.ra_stripe_permute.argtypes = [i32, i32, i32, i32, i32, i64, i32, i32, vp, vp, vp]
    lib.ra_stripe_permute.restype = ctypes.c_int
    lib.ra_mask_offset.argtypes = [i64, i64, i64]
    lib.ra_mask_offset.restype = i64
    lib.ra_unmasked_pairs.argtypes = [i64, i64, i32, i64]
    lib.ra_unmasked_pairs.restype = i64
    lib.ra_ring_pair_offset.argtypes = [i32, i32, i64, i32, i32]
    lib.ra_ring_pair_offset.restype = i64
    lib.ra_last_error.argtypes = []
    lib.ra_last_error.restype = ctypes.c_char_p
    lib.ra_abi_version.argtypes = []
    lib.ra_abi_version.restype = i32
    lib.ra_release.argtypes = []
    lib.ra_release.restype = None
    lib.ra_attn_bwd_delta.argtypes = [i64, i32, i32, vp, vp, vp, vp]
    lib.ra_attn_bwd_delta.restype = ctypes.c_int
    lib.ra_block_attn_bwd.argtypes = [ctypes.POINTER(ra_block_desc), vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.ra_block_attn_bwd.restype = ctypes.c_int
    lib.ra_ring_bwd_workspace_size.argtypes = [ctypes.POINTER(ra_ring_desc), ctypes.POINTER(ctypes.c_size_t)]
    lib.ra_ring_bwd_workspace_size.restype = ctypes.c_int
    lib.ra_ring_backward.argtypes = [ctypes.POINTER(ra_ring_desc), vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                     ctypes.c_size_t, vp]
    lib.ra_ring_backward.restype = ctypes.c_int
    lib.ra_block_attn_fwd_kernel.argtypes = [ctypes.POINTER(ra_block_desc), vp, vp, vp, vp, vp, vp]
    lib.ra_block_attn_fwd_kernel.restype = i32
    lib.ra_block_attn_bwd_kernel.argtypes = [ctypes.POINTER(ra_block_desc), vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.ra_block_attn_bwd_kernel.restype = i32
    lib.ra_ring_forward_noalloc.argtypes = [ctypes.POINTER(ra_ring_desc), vp, vp, vp, vp, vp, vp]
    lib.ra_ring_forward_noalloc.restype = ctypes.c_int
    lib.ra_ring_noalloc_max_bytes.argtypes = []
    lib.ra_ring_noalloc_max_bytes.restype = ctypes.c_size_t
    del f32
    if path == LIB_PATH:
        _lib = lib
    return lib


def _check(status):
    if status != RA_OK:
        raise RAError(status, load_library().ra_last_error().decode())


def _dtype(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return RA_F32
    if t.dtype == torch.bfloat16:
        return RA_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _need_dense(t, name, dtype=None):
    if t is not None:
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if dtype is not None and t.dtype != dtype:
            raise TypeError(f"{name} must be {dtype}")


# ------------------------------------------------------------------ host helpers
def ra_mask_offset(q_pos0: int, k_pos0: int, pos_stride: int) -> int:
    return load_library().ra_mask_offset(q_pos0, k_pos0, pos_stride)


def ra_unmasked_pairs(q_len: int, kv_len: int, causal: bool, offset: int) -> int:
    return load_library().ra_unmasked_pairs(q_len, kv_len, int(bool(causal)), offset)


def ra_ring_pair_offset(layout, n_pos: int, block_len: int, i: int, j: int) -> int:
    lay = LAYOUTS[layout] if isinstance(layout, str) else int(layout)
    return load_library().ra_ring_pair_offset(lay, n_pos, block_len, i, j)


def ra_abi_version() -> int:
    return load_library().ra_abi_version()


def ra_release() -> None:
    load_library().ra_release()


# ------------------------------------------------------------------ device calls
def block_desc(q, k, v, causal=False, scale=0.0, q_pos0=0, k_pos0=0, pos_stride=1, flags=0):
    """ra_block_desc for q [B, Hq, q_len, D] and k, v [B, Hkv, kv_len, D] (D contiguous)."""
    B, Hq, q_len, D = q.shape
    Bk, Hkv, kv_len, Dk = k.shape
    if (Bk, Dk) != (B, D) or tuple(v.shape) != tuple(k.shape):
        raise ValueError("q, k, v shapes disagree")
    for t, name in ((q, "q"), (k, "k"), (v, "v")):
        if t.stride(3) != 1 and t.shape[3] > 1:
            raise ValueError(f"{name}: head_dim must be contiguous")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k, v must share a dtype")
    d = ra_block_desc()
    d.batch, d.q_heads, d.kv_heads, d.head_dim = B, Hq, Hkv, D
    d.q_len, d.kv_len = q_len, kv_len
    d.dtype, d.causal, d.scale, d.flags = _dtype(q), int(bool(causal)), float(scale), int(flags)
    d.q_pos0, d.k_pos0, d.pos_stride = int(q_pos0), int(k_pos0), int(pos_stride)
    d.q_strides[:] = [q.stride(0), q.stride(1), q.stride(2)]
    d.k_strides[:] = [k.stride(0), k.stride(1), k.stride(2)]
    d.v_strides[:] = [v.stride(0), v.stride(1), v.stride(2)]
    return d


def ra_block_attn_fwd(q, k, v, o, m, l, *, causal=False, scale=0.0, q_pos0=0, k_pos0=0, pos_stride=1,
                      flags=0, stream=None):
    """Partial (o unnormalised [B,Hq,q_len,D], m, l [B,Hq,q_len]) of q against k, v."""
    for t, name in ((o, "o"), (m, "m"), (l, "l")):
        _need_dense(t, name, torch.float32)
    d = block_desc(q, k, v, causal, scale, q_pos0, k_pos0, pos_stride, flags)
    if tuple(o.shape) != tuple(q.shape) or tuple(m.shape) != tuple(q.shape[:3]) or m.shape != l.shape:
        raise ValueError("o must be shaped like q, m and l like q without head_dim")
    _check(load_library().ra_block_attn_fwd(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(m),
                                            _ptr(l), _stream(stream)))


def ra_lse_merge(o_acc, m_acc, l_acc, o_part=None, m_part=None, l_part=None, o_out=None, lse_out=None,
                 stream=None):
    """Fold a partial into (o_acc, m_acc, l_acc); finalise into o_out / lse_out when given."""
    for t, name in ((o_acc, "o_acc"), (m_acc, "m_acc"), (l_acc, "l_acc"), (o_part, "o_part"),
                    (m_part, "m_part"), (l_part, "l_part"), (lse_out, "lse_out")):
        _need_dense(t, name, torch.float32)
    _need_dense(o_out, "o_out")
    D = o_acc.shape[-1]
    rows = m_acc.numel()
    if o_acc.numel() != rows * D or l_acc.numel() != rows:
        raise ValueError("running state shapes disagree")
    for t in (o_part, o_out):
        if t is not None and t.numel() != rows * D:
            raise ValueError("o_part / o_out must match o_acc")
    for t in (m_part, l_part, lse_out):
        if t is not None and t.numel() != rows:
            raise ValueError("m_part / l_part / lse_out must have one value per row")
    out_dtype = _dtype(o_out) if o_out is not None else RA_F32
    _check(load_library().ra_lse_merge(rows, D, _ptr(o_acc), _ptr(m_acc), _ptr(l_acc), _ptr(o_part),
                                       _ptr(m_part), _ptr(l_part), _ptr(o_out), out_dtype, _ptr(lse_out),
                                       _stream(stream)))


def ring_desc(q, k, *, n_pos, first_pos=0, layout="contiguous", causal=False, scale=0.0, emulate_copy=False,
              n_streams=0, separate_merge=False, kv_splits=0, visit_order=None, stats=None):
    """ra_ring_desc for q [n_run, B, Hq, Sb, D] and k [n_pos, B, Hkv, Sb, D]."""
    n_run, B, Hq, Sb, D = q.shape
    if k.shape[0] != n_pos or k.shape[1] != B or k.shape[3] != Sb or k.shape[4] != D:
        raise ValueError("k must be [n_pos, B, Hkv, Sb, D] matching q")
    d = ra_ring_desc()
    d.batch, d.q_heads, d.kv_heads, d.head_dim = B, Hq, k.shape[2], D
    d.n_pos, d.first_pos, d.n_run = int(n_pos), int(first_pos), n_run
    d.layout = LAYOUTS[layout] if isinstance(layout, str) else int(layout)
    d.block_len, d.dtype, d.causal, d.scale = Sb, _dtype(q), int(bool(causal)), float(scale)
    d.emulate_copy, d.n_streams = int(bool(emulate_copy)), int(n_streams)
    d.separate_merge = int(bool(separate_merge))
    d.kv_splits = int(kv_splits)
    if visit_order is not None:
        arr = (ctypes.c_int32 * n_pos)(*[int(x) for x in visit_order])
        d._order_keepalive = arr
        d.visit_order = ctypes.cast(arr, ctypes.POINTER(ctypes.c_int32))
    if stats is not None:
        d.stats = ctypes.pointer(stats)
    return d


def ra_ring_workspace_size(desc) -> int:
    n = ctypes.c_size_t(0)
    _check(load_library().ra_ring_workspace_size(ctypes.byref(desc), ctypes.byref(n)))
    return n.value


def ra_ring_forward(q, k, v, o, lse=None, *, n_pos, first_pos=0, layout="contiguous", causal=False,
                    scale=0.0, emulate_copy=False, n_streams=0, separate_merge=False, kv_splits=0,
                    visit_order=None, workspace=None, stats=False, stream=None):
    """Run positions first_pos .. first_pos + n_run - 1 of an n_pos ring on one GPU.

    Returns a dict of ra_ring_stats when stats=True (the call then waits for its
    work), else None.
    """
    for t, name in ((q, "q"), (k, "k"), (v, "v"), (o, "o")):
        _need_dense(t, name)
    _need_dense(lse, "lse", torch.float32)
    if v.shape != k.shape or o.shape != q.shape or o.dtype != q.dtype:
        raise ValueError("v must match k and o must match q")
    st = ra_ring_stats() if stats else None
    d = ring_desc(q, k, n_pos=n_pos, first_pos=first_pos, layout=layout, causal=causal, scale=scale,
                  emulate_copy=emulate_copy, n_streams=n_streams, separate_merge=separate_merge,
                  kv_splits=kv_splits, visit_order=visit_order, stats=st)
    need = ra_ring_workspace_size(d)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    _check(load_library().ra_ring_forward(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                          _ptr(workspace), workspace.numel() * workspace.element_size(),
                                          _stream(stream)))
    if st is None:
        return None
    return {name: getattr(st, name) for name, _ in ra_ring_stats._fields_}


def ra_ring_forward_noalloc(q, k, v, o, lse=None, *, n_pos, first_pos=0, layout="contiguous", causal=False,
                            scale=0.0, separate_merge=False, kv_splits=0, visit_order=None, stream=None):
    """ra_ring_forward on one stream (the current one) with the library's own
    device scratch: the call allocates nothing, on the device or through torch."""
    for t, name in ((q, "q"), (k, "k"), (v, "v"), (o, "o")):
        _need_dense(t, name)
    _need_dense(lse, "lse", torch.float32)
    if v.shape != k.shape or o.shape != q.shape or o.dtype != q.dtype:
        raise ValueError("v must match k and o must match q")
    d = ring_desc(q, k, n_pos=n_pos, first_pos=first_pos, layout=layout, causal=causal, scale=scale,
                  n_streams=1, separate_merge=separate_merge, kv_splits=kv_splits, visit_order=visit_order)
    _check(load_library().ra_ring_forward_noalloc(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                                  _stream(stream)))


def ra_ring_noalloc_max_bytes() -> int:
    return load_library().ra_ring_noalloc_max_bytes()


def ra_stripe_permute(x, y, *, layout, inverse, n_pos, stream=None):
    """Forward: x [B, H, S, D] -> y [N, B, H, S/N, D]; inverse the other way."""
    _need_dense(x, "x")
    _need_dense(y, "y", x.dtype)
    if inverse:
        N, B, H, Sb, D = x.shape
        S = N * Sb
        if tuple(y.shape) != (B, H, S, D):
            raise ValueError("y must be [B, H, N*Sb, D]")
    else:
        B, H, S, D = x.shape
        if tuple(y.shape) != (n_pos, B, H, S // n_pos, D):
            raise ValueError("y must be [N, B, H, S/N, D]")
        N = n_pos
    lay = LAYOUTS[layout] if isinstance(layout, str) else int(layout)
    _check(load_library().ra_stripe_permute(lay, int(bool(inverse)), _dtype(x), B, H, S, D, N, _ptr(x), _ptr(y),
                                            _stream(stream)))


# ------------------------------------------------------------------ backward
def ra_attn_bwd_delta(o, dout, delta, stream=None):
    """delta [rows] = sum over head_dim of dout * o (o, dout [..., D] dense, same dtype)."""
    _need_dense(o, "o")
    _need_dense(dout, "dout", o.dtype)
    _need_dense(delta, "delta", torch.float32)
    D = o.shape[-1]
    rows = o.numel() // D if D else 0
    if dout.shape != o.shape or delta.numel() != rows:
        raise ValueError("dout must match o; delta needs one value per row")
    _check(load_library().ra_attn_bwd_delta(rows, D, _dtype(o), _ptr(o), _ptr(dout), _ptr(delta),
                                            _stream(stream)))


def ra_block_attn_bwd(q, k, v, dout, lse, delta, dq, dk, dv, *, causal=False, scale=0.0, q_pos0=0, k_pos0=0,
                      pos_stride=1, flags=0, stream=None):
    """Add one block pair's share of dQ [B,Hq,q_len,D], dK, dV [B,Hkv,kv_len,D] (fp32)."""
    if dout.shape != q.shape or dout.dtype != q.dtype or tuple(dout.stride()) != tuple(q.stride()):
        raise ValueError("dout must have q's shape, dtype and strides")
    for t, name in ((lse, "lse"), (delta, "delta"), (dq, "dq"), (dk, "dk"), (dv, "dv")):
        _need_dense(t, name, torch.float32)
    if tuple(dq.shape) != tuple(q.shape) or tuple(dk.shape) != tuple(k.shape) or dv.shape != dk.shape:
        raise ValueError("dq must be shaped like q, dk and dv like k")
    if tuple(lse.shape) != tuple(q.shape[:3]) or lse.shape != delta.shape:
        raise ValueError("lse and delta must be shaped like q without head_dim")
    d = block_desc(q, k, v, causal, scale, q_pos0, k_pos0, pos_stride, flags)
    _check(load_library().ra_block_attn_bwd(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(lse),
                                            _ptr(delta), _ptr(dq), _ptr(dk), _ptr(dv), _stream(stream)))


def ra_ring_bwd_workspace_size(desc) -> int:
    n = ctypes.c_size_t(0)
    _check(load_library().ra_ring_bwd_workspace_size(ctypes.byref(desc), ctypes.byref(n)))
    return n.value


def ra_ring_backward(q, k, v, o, dout, lse, dq, dk, dv, *, n_pos, first_pos=0, layout="contiguous",
                     causal=False, scale=0.0, visit_order=None, n_streams=0, workspace=None, stats=False,
                     stream=None):
    """Gradients of the ring: dq [n_run,B,Hq,Sb,D], dk, dv [n_pos,B,Hkv,Sb,D] (fp32, overwritten).

    Returns a dict of ra_ring_stats when stats=True, else None.
    """
    for t, name in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (dout, "dout")):
        _need_dense(t, name)
    for t, name in ((lse, "lse"), (dq, "dq"), (dk, "dk"), (dv, "dv")):
        _need_dense(t, name, torch.float32)
    if v.shape != k.shape or o.shape != q.shape or dout.shape != q.shape or dq.shape != q.shape:
        raise ValueError("v must match k; o, dout, dq must match q")
    if dk.shape != k.shape or dv.shape != k.shape or tuple(lse.shape) != tuple(q.shape[:4]):
        raise ValueError("dk, dv must match k; lse must be q's shape without head_dim")
    st = ra_ring_stats() if stats else None
    d = ring_desc(q, k, n_pos=n_pos, first_pos=first_pos, layout=layout, causal=causal, scale=scale,
                  visit_order=visit_order, n_streams=n_streams, stats=st)
    need = ra_ring_bwd_workspace_size(d)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _check(load_library().ra_ring_backward(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout),
                                           _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace),
                                           workspace.numel() * workspace.element_size(), _stream(stream)))
    if st is None:
        return None
    return {name: getattr(st, name) for name, _ in ra_ring_stats._fields_}
