"""The C-ABI library on the host (no GPU): exports, mask/work accounting,
argument validation.  Nothing here launches a kernel."""
import ctypes
import os
import re

import numpy as np
import pytest

from oracle import layout
from ring_attention_step_amd import _binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = ctypes.c_void_p(0x10000)  # never dereferenced: every call below fails validation first


@pytest.fixture(scope="module")
def lib():
    return B.load_library()


def declared_functions():
    text = open(os.path.join(ROOT, "include", "ra.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ra_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert len(names) >= 10
    for name in names:
        assert hasattr(lib, name), f"libra.so does not export {name}"
    assert set(names) == set(B.EXPORTS)
    assert lib.ra_abi_version() == 5


def test_mask_offset_is_floor_division(lib):
    rng = np.random.Generator(np.random.PCG64(0))
    for _ in range(2000):
        q0, k0 = (int(x) for x in rng.integers(-10**6, 10**6, size=2))
        s = int(rng.integers(1, 40))
        assert lib.ra_mask_offset(q0, k0, s) == (q0 - k0) // s


def test_unmasked_pairs_matches_enumeration(lib):
    for q_len in range(0, 9):
        for kv_len in range(0, 9):
            for off in range(-11, 12):
                r = np.arange(q_len)[:, None]
                c = np.arange(kv_len)[None, :]
                want = int(np.sum(c <= r + off)) if q_len and kv_len else 0
                assert lib.ra_unmasked_pairs(q_len, kv_len, 1, off) == want
                assert lib.ra_unmasked_pairs(q_len, kv_len, 0, off) == q_len * kv_len
    # large sizes stay exact (int64)
    assert lib.ra_unmasked_pairs(32768, 32768, 1, 0) == 32768 * 32769 // 2
    assert lib.ra_unmasked_pairs(32768, 32768, 1, -1) == 32768 * 32767 // 2


@pytest.mark.parametrize("lay", ["contiguous", "striped"])
def test_ring_pair_offset_matches_token_maps(lib, lay):
    """The per-(position, block) mask offset reproduces the global causal rule."""
    S = 48
    for n in (1, 2, 3, 4, 8):
        sb = S // n
        for i in range(n):
            ti = layout.tokens_of(i, S, n, lay)
            for j in range(n):
                tj = layout.tokens_of(j, S, n, lay)
                off = B.ra_ring_pair_offset(lay, n, sb, i, j)
                r = np.arange(sb)[:, None]
                c = np.arange(sb)[None, :]
                assert np.array_equal(c <= r + off, tj[None, :] <= ti[:, None])
                assert lib.ra_unmasked_pairs(sb, sb, 1, off) == int(np.sum(tj[None, :] <= ti[:, None]))


def _ring_flops(n, sb, heads, d, lay, causal, i):
    total = 0
    for j in range(n):
        off = B.ra_ring_pair_offset(lay, n, sb, i, j)
        total += B.ra_unmasked_pairs(sb, sb, causal, off)
    return 4 * d * heads * total


def test_causal_flop_accounting_of_the_benchmark_shapes():
    # striped, 8 positions of 32768 tokens, 8 heads, d 128: the last position's share
    assert _ring_flops(8, 32768, 8, 128, "striped", True, 7) == 4 * 128 * 8 * 8 * 32768 * 32769 // 2
    # striped 1M tokens over 32 positions, 32 query heads
    f = _ring_flops(32, 32768, 32, 128, "striped", True, 31)
    assert f == 4 * 128 * 32 * 32 * 32768 * 32769 // 2
    assert abs(f - 2.8148e14) / 2.8148e14 < 1e-4
    # contiguous 32768 tokens over 4 positions: the whole ring is the causal triangle
    full = sum(_ring_flops(4, 8192, 32, 128, "contiguous", True, i) for i in range(4))
    assert full == 4 * 128 * 32 * 32768 * 32769 // 2


def _block_desc(**kw):
    d = B.ra_block_desc()
    d.batch, d.q_heads, d.kv_heads, d.head_dim = 1, 4, 2, 64
    d.q_len, d.kv_len, d.dtype, d.causal, d.scale, d.flags = 16, 16, B.RA_BF16, 1, 0.0, 0
    d.q_pos0, d.k_pos0, d.pos_stride = 0, 0, 1
    d.q_strides[:] = [4 * 16 * 64, 16 * 64, 64]
    d.k_strides[:] = [2 * 16 * 64, 16 * 64, 64]
    d.v_strides[:] = [2 * 16 * 64, 16 * 64, 64]
    for k, v in kw.items():
        setattr(d, k, v)
    return d


@pytest.mark.parametrize("field,value,status", [
    ("q_heads", 3, B.RA_ERR_INVALID), ("kv_heads", 0, B.RA_ERR_INVALID), ("head_dim", 0, B.RA_ERR_INVALID),
    ("head_dim", 300, B.RA_ERR_UNSUPPORTED), ("dtype", 7, B.RA_ERR_UNSUPPORTED), ("causal", 2, B.RA_ERR_INVALID),
    ("flags", 0x80, B.RA_ERR_UNSUPPORTED), ("pos_stride", 0, B.RA_ERR_INVALID), ("q_len", -1, B.RA_ERR_INVALID),
    ("kv_len", 1 << 40, B.RA_ERR_INVALID), ("batch", 0, B.RA_ERR_INVALID), ("scale", float("nan"), B.RA_ERR_INVALID),
])
def test_block_validation(lib, field, value, status):
    d = _block_desc(**{field: value})
    st = lib.ra_block_attn_fwd(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None)
    assert st == status
    assert lib.ra_last_error()


def test_block_validation_pointers(lib):
    d = _block_desc()
    assert lib.ra_block_attn_fwd(None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == B.RA_ERR_INVALID
    assert lib.ra_block_attn_fwd(ctypes.byref(d), None, FAKE, FAKE, FAKE, FAKE, FAKE, None) == B.RA_ERR_INVALID
    assert lib.ra_block_attn_fwd(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, None, FAKE, None) == B.RA_ERR_INVALID
    odd = ctypes.c_void_p(0x10001)
    assert lib.ra_block_attn_fwd(ctypes.byref(d), odd, FAKE, FAKE, FAKE, FAKE, FAKE, None) == B.RA_ERR_INVALID
    # an empty query block is a no-op, even with null pointers
    e = _block_desc(q_len=0)
    assert lib.ra_block_attn_fwd(ctypes.byref(e), None, None, None, None, None, None, None) == B.RA_OK


def test_merge_and_permute_validation(lib):
    m = lib.ra_lse_merge
    assert m(-1, 64, FAKE, FAKE, FAKE, None, None, None, None, 0, None, None) == B.RA_ERR_INVALID
    assert m(8, 0, FAKE, FAKE, FAKE, None, None, None, None, 0, None, None) == B.RA_ERR_INVALID
    assert m(8, 64, FAKE, FAKE, FAKE, FAKE, None, None, None, 0, None, None) == B.RA_ERR_INVALID
    assert m(8, 64, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, 5, None, None) == B.RA_ERR_UNSUPPORTED
    assert m(8, 64, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, None, None) == B.RA_ERR_INVALID  # alias
    assert m(0, 64, None, None, None, None, None, None, None, 0, None, None) == B.RA_OK
    p = lib.ra_stripe_permute
    assert p(2, 0, 1, 1, 1, 64, 8, 4, FAKE, ctypes.c_void_p(0x900000), None) == B.RA_ERR_INVALID  # layout
    assert p(1, 0, 1, 1, 1, 63, 8, 4, FAKE, ctypes.c_void_p(0x900000), None) == B.RA_ERR_INVALID  # S % N
    assert p(1, 0, 1, 1, 1, 64, 8, 4, FAKE, ctypes.c_void_p(0x10010), None) == B.RA_ERR_INVALID   # overlap
    assert p(1, 0, 9, 1, 1, 64, 8, 4, FAKE, ctypes.c_void_p(0x900000), None) == B.RA_ERR_UNSUPPORTED


def _ring_desc(**kw):
    d = B.ra_ring_desc()
    d.batch, d.q_heads, d.kv_heads, d.head_dim = 1, 32, 8, 128
    d.n_pos, d.first_pos, d.n_run, d.layout = 32, 31, 1, B.RA_STRIPED
    d.block_len, d.dtype, d.causal, d.scale = 32768, B.RA_BF16, 1, 0.0
    d.emulate_copy, d.n_streams = 0, 0
    for k, v in kw.items():
        setattr(d, k, v)
    return d


QUEUE = 256  # bytes of tile-queue counters per stream of a ring call


def test_ring_workspace_and_validation(lib):
    n = ctypes.c_size_t()
    d = _ring_desc()
    assert lib.ra_ring_workspace_size(ctypes.byref(d), ctypes.byref(n)) == B.RA_OK
    rows = 32 * 32768
    state = rows * 128 * 4 + 2 * rows * 4  # fp32 O, m, l of the 32768 queries x 32 heads
    # a single position whose launches hold 8192 query tiles (>= 2 per compute
    # unit) keeps two running states (accumulation chains), one 256-byte block
    # of tile-queue counters per chain's stream
    assert n.value == 2 * state + 2 * QUEUE
    # n_streams = 1: one running state and one stream
    one = _ring_desc(n_streams=1)
    assert lib.ra_ring_workspace_size(ctypes.byref(one), ctypes.byref(n)) == B.RA_OK
    assert n.value == state + QUEUE
    # a single position of few query tiles (256) keeps one state with n_streams = 0
    small = _ring_desc(q_heads=8, kv_heads=8, block_len=4096, kv_splits=1)
    assert lib.ra_ring_workspace_size(ctypes.byref(small), ctypes.byref(n)) == B.RA_OK
    assert n.value == (8 * 4096) * 128 * 4 + 2 * (8 * 4096) * 4 + QUEUE
    s = _ring_desc(separate_merge=1)  # plus one partial per stream
    assert lib.ra_ring_workspace_size(ctypes.byref(s), ctypes.byref(n)) == B.RA_OK
    assert n.value == 2 * (rows * 128 * 4 + 2 * rows * 4) + QUEUE
    e = _ring_desc(emulate_copy=1)
    assert lib.ra_ring_workspace_size(ctypes.byref(e), ctypes.byref(n)) == B.RA_OK
    assert n.value == (rows * 128 * 4 + 2 * rows * 4) + 4 * (8 * 32768 * 128 * 2) + QUEUE
    for kw in ({"first_pos": 32}, {"n_run": 2}, {"layout": 3}, {"n_pos": 0}, {"block_len": 0},
               {"emulate_copy": 2}, {"kv_heads": 5}, {"n_streams": -1}, {"separate_merge": 2},
               {"kv_splits": -1}, {"kv_splits": 9}):
        bad = _ring_desc(**kw)
        assert lib.ra_ring_workspace_size(ctypes.byref(bad), ctypes.byref(n)) != B.RA_OK
    order = (ctypes.c_int32 * 32)(*([0] * 32))
    bad = _ring_desc()
    bad.visit_order = ctypes.cast(order, ctypes.POINTER(ctypes.c_int32))
    assert lib.ra_ring_workspace_size(ctypes.byref(bad), ctypes.byref(n)) == B.RA_ERR_INVALID
    # too small a workspace is refused before anything runs
    st = lib.ra_ring_forward(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, None, ctypes.c_void_p(0x100000), 1024, None)
    assert st == B.RA_ERR_WORKSPACE


def test_kv_split_workspace(lib):
    """Key splits: a ring whose block launches fill few workgroups keeps
    n_splits partials per stream (one per 128-key range); 0 chooses the count
    so that the launches of one step reach about 256 workgroups."""
    n = ctypes.c_size_t()
    # 2 positions of 2048 tokens, 4 heads, d 64: 8 query tiles x 4 heads x 2 streams = 64 workgroups
    kw = dict(q_heads=4, kv_heads=4, head_dim=64, n_pos=2, first_pos=0, n_run=2, block_len=2048, causal=0,
              layout=B.RA_CONTIGUOUS)
    rows = 4 * 2048
    state = rows * 64 * 4 + 2 * rows * 4  # fp32 O, m, l of one position (all 256-byte multiples)

    def size(**extra):
        d = _ring_desc(**kw, **extra)
        assert lib.ra_ring_workspace_size(ctypes.byref(d), ctypes.byref(n)) == B.RA_OK
        streams = extra.get("n_streams", 2)
        return n.value - streams * QUEUE  # the partials and running states alone

    assert size(kv_splits=1) == 2 * state
    assert size() == 2 * state + 2 * 4 * state  # automatic: 4 ranges of 4 tiles
    assert size(kv_splits=8) == 2 * state + 2 * 8 * state
    assert size(kv_splits=3) == 2 * state + 2 * 3 * state  # 6 + 6 + 4 tiles
    assert size(kv_splits=5) == 2 * state + 2 * 4 * state  # 4-tile ranges: the fifth would be empty
    assert size(separate_merge=1) == 2 * state + 2 * state  # one partial per stream, no splits
    assert size(n_streams=1) == 2 * state + 1 * 8 * state  # 32 workgroups per step: 8 ranges of 2 tiles
    assert size(dtype=B.RA_F32) == 2 * state  # the vector-ALU kernel has no key splits
    kw["block_len"] = 128  # one key tile: nothing to split
    rows = 4 * 128
    state = rows * 64 * 4 + 2 * rows * 4
    assert size() == 2 * state and size(kv_splits=4) == 2 * state


def test_backward_validation(lib):
    d = _block_desc()
    args = [FAKE] * 9
    assert lib.ra_block_attn_bwd(None, *args, None) == B.RA_ERR_INVALID
    bad = _block_desc(flags=B.RA_BLOCK_ACCUMULATE)  # the backward always accumulates; the flag is not accepted
    assert lib.ra_block_attn_bwd(ctypes.byref(bad), *args, None) == B.RA_ERR_UNSUPPORTED
    nulls = [FAKE] * 8 + [None]
    assert lib.ra_block_attn_bwd(ctypes.byref(d), *nulls, None) == B.RA_ERR_INVALID
    e = _block_desc(kv_len=0)
    assert lib.ra_block_attn_bwd(ctypes.byref(e), *([None] * 9), None) == B.RA_OK
    assert lib.ra_attn_bwd_delta(-1, 64, 0, FAKE, FAKE, FAKE, None) == B.RA_ERR_INVALID
    assert lib.ra_attn_bwd_delta(4, 64, 9, FAKE, FAKE, FAKE, None) == B.RA_ERR_UNSUPPORTED
    assert lib.ra_attn_bwd_delta(0, 64, 0, None, None, None, None) == B.RA_OK
    n = ctypes.c_size_t()
    r = _ring_desc()
    assert lib.ra_ring_bwd_workspace_size(ctypes.byref(r), ctypes.byref(n)) == B.RA_OK
    assert n.value == 32 * 32768 * 4  # one delta per row of the run position
    st = lib.ra_ring_backward(ctypes.byref(r), *([FAKE] * 9), ctypes.c_void_p(0x100000), 1024, None)
    assert st == B.RA_ERR_WORKSPACE


def _desc(D=128, dtype=B.RA_BF16, q_len=256, kv_len=256, kv_row_stride=None, flags=0):
    d = B.ra_block_desc()
    d.batch, d.q_heads, d.kv_heads, d.head_dim = 1, 2, 1, D
    d.q_len, d.kv_len = q_len, kv_len
    d.dtype, d.causal, d.scale, d.flags = dtype, 1, 0.0, flags
    d.q_pos0, d.k_pos0, d.pos_stride = 0, 0, 1
    rs = D if kv_row_stride is None else kv_row_stride
    d.q_strides[:] = [2 * q_len * D, q_len * D, D]
    d.k_strides[:] = [kv_len * rs, kv_len * rs, rs]
    d.v_strides[:] = [kv_len * rs, kv_len * rs, rs]
    return d


def test_block_kernel_selection_on_host(lib):
    """Which kernel a block call would run, decided on the host: bf16 with head_dim
    64 or 128 takes the MFMA kernels; fp32, other head_dims, the force flag,
    misalignment and key/value row strides of 2^24 elements or more (whose
    per-lane 32-bit copy offsets would wrap) take the vector-ALU kernels; invalid
    calls return -1.  No pointer is dereferenced (no kernel is launched)."""
    a16 = ctypes.c_void_p(0x100000)   # 16-byte aligned fake device addresses
    odd = ctypes.c_void_p(0x100008)   # 8-byte aligned only

    def fwd(d, q=a16, o=a16):
        return lib.ra_block_attn_fwd_kernel(ctypes.byref(d), q, a16, a16, o, a16, a16)

    def bwd(d, q=a16):
        return lib.ra_block_attn_bwd_kernel(ctypes.byref(d), q, a16, a16, a16, a16, a16, a16, a16, a16)

    assert fwd(_desc(128)) == 1 and bwd(_desc(128)) == 1
    assert fwd(_desc(64)) == 1 and bwd(_desc(64)) == 1
    assert fwd(_desc(96)) == 0 and bwd(_desc(96)) == 0
    assert fwd(_desc(128, dtype=B.RA_F32)) == 0 and bwd(_desc(128, dtype=B.RA_F32)) == 0
    assert fwd(_desc(128, flags=B.RA_BLOCK_FORCE_SIMT)) == 0
    assert bwd(_desc(128, flags=B.RA_BLOCK_FORCE_SIMT)) == 0
    assert fwd(_desc(128), q=odd) == 0 and bwd(_desc(128), q=odd) == 0
    # row strides: the largest that keeps 32-bit copy offsets, and the first that does not
    assert fwd(_desc(128, kv_row_stride=(1 << 24) - 8)) == 1
    assert fwd(_desc(128, kv_row_stride=1 << 24)) == 0
    assert bwd(_desc(128, kv_row_stride=(1 << 24) - 8)) == 1
    assert bwd(_desc(128, kv_row_stride=1 << 24)) == 0
    # a stride that is not a multiple of 8 elements (16-byte rows) stays off MFMA
    assert fwd(_desc(128, kv_row_stride=136 + 4)) == 0
    # empty calls are valid no-ops; invalid ones are rejected with a message
    assert fwd(_desc(128, q_len=0), q=FAKE) == 0
    assert bwd(_desc(128, kv_len=0)) == 0
    bad = _desc(128)
    bad.pos_stride = 0
    assert fwd(bad) == -1 and b"pos_stride" in lib.ra_last_error()
    assert bwd(bad) == -1
    assert lib.ra_block_attn_fwd_kernel(None, a16, a16, a16, a16, a16, a16) == -1
