"""GPU parity: every C-ABI entry point against the CPU fp64 oracle.

Element by element on seeded inputs at sizes that span several tiles and a
ragged tail; at the full benchmark sizes on 4096 seeded sampled query rows
(stratified to include the first and last row of every block and token 0).
Tolerances are written in tests/gpu_helpers.py: binary32 1e-5 abs (output and
log-sum-exp); bfloat16 2e-2 abs on the output, 1e-3 abs on the log-sum-exp.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import ra_inputs
import ring_attention_step_amd as ra
from oracle import layout as olayout
from tests import gpu_helpers as gh

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ra.load_library()
    yield
    torch.cuda.synchronize()


# ------------------------------------------------------------------ block kernel
BLOCK_CASES = [
    # (dtype, head_dim, flags) -- flags 1 forces the vector-ALU kernel
    ("f32", 16, 0), ("f32", 64, 0), ("f32", 100, 0), ("f32", 256, 0),
    ("bf16", 64, 0), ("bf16", 128, 0), ("bf16", 128, 1), ("bf16", 48, 0),
]
OFFSETS = [None, 0, -1, 37, -150, 400, -400]


def _oracle_partial(q, k, v, causal, off):
    """Oracle partial of one (b, h) block: rows r at position r + off, keys c at c."""
    n = q.shape[0]
    pos = np.arange(n, dtype=np.int64) + (off or 0)
    return oracle.rows(q, k, v, q_pos=pos, causal=causal)


@pytest.mark.parametrize("dtype,D,flags", BLOCK_CASES)
def test_block_partial_matches_oracle(dtype, D, flags):
    B, Hq, Hkv, q_len, kv_len = 2, 4, 2, 300, 333
    gh.say("ra_block_attn_fwd", dtype, D, flags)
    qn = ra_inputs.normal((B, Hq, q_len, D), 0, seed=3, dtype=dtype)
    kn = ra_inputs.normal((B, Hkv, kv_len, D), 1, seed=3, dtype=dtype)
    vn = ra_inputs.normal((B, Hkv, kv_len, D), 2, seed=3, dtype=dtype)
    # q as a strided view ([B, S, H, D] memory) to exercise the stride arguments
    q = gh.to_device(np.ascontiguousarray(qn.transpose(0, 2, 1, 3)), dtype).permute(0, 2, 1, 3)
    k, v = gh.to_device(kn, dtype), gh.to_device(vn, dtype)
    tol = gh.TOL[dtype]
    for off in OFFSETS:
        causal = off is not None
        o = torch.full((B, Hq, q_len, D), float("nan"), device="cuda")
        m = torch.full((B, Hq, q_len), float("nan"), device="cuda")
        l = torch.full((B, Hq, q_len), float("nan"), device="cuda")
        ra.ra_block_attn_fwd(q, k, v, o, m, l, causal=causal, q_pos0=(off or 0), k_pos0=0, flags=flags)
        torch.cuda.synchronize()
        o, m, l = gh.to_host_f64(o), gh.to_host_f64(m), gh.to_host_f64(l)
        for b in range(B):
            for h in range(Hq):
                r = _oracle_partial(qn[b, h], kn[b, h // 2], vn[b, h // 2], causal, off)
                empty = np.isneginf(r["m"])
                assert np.all(np.isneginf(m[b, h][empty])) and np.all(l[b, h][empty] == 0)
                assert np.all(o[b, h][empty] == 0)
                ok = ~empty
                if not ok.any():
                    continue
                assert np.max(np.abs(m[b, h][ok] - r["m"][ok])) <= 1e-4
                assert np.max(np.abs(l[b, h][ok] / r["l"][ok] - 1)) <= tol["lse"]
                lse = m[b, h][ok] + np.log(l[b, h][ok])
                assert np.max(np.abs(lse - r["lse"][ok])) <= tol["lse"]
                out = o[b, h][ok] / l[b, h][ok][:, None]
                assert np.max(np.abs(out - r["o"][ok])) <= tol["o"], (off, b, h)


def test_block_empty_cases():
    gh.say("ra_block_attn_fwd empty")
    q = torch.randn(1, 2, 5, 64, device="cuda").bfloat16()
    k = torch.randn(1, 2, 0, 64, device="cuda").bfloat16()
    o = torch.full((1, 2, 5, 64), 7.0, device="cuda")
    m = torch.zeros(1, 2, 5, device="cuda")
    l = torch.ones(1, 2, 5, device="cuda")
    ra.ra_block_attn_fwd(q, k, k, o, m, l)
    torch.cuda.synchronize()
    assert torch.all(torch.isneginf(m)) and torch.all(l == 0) and torch.all(o == 0)
    q0 = torch.randn(1, 2, 0, 64, device="cuda").bfloat16()
    e = torch.empty(1, 2, 0, 64, device="cuda")
    ra.ra_block_attn_fwd(q0, q0, q0, e, e[..., 0], e[..., 0])  # no-op


# ------------------------------------------------------------------ merge kernel
@pytest.mark.parametrize("dtype,D", [("f32", 16), ("bf16", 128), ("bf16", 64), ("f32", 37)])
def test_merge_matches_oracle(dtype, D):
    B, H, q_len, kv_len, split = 1, 3, 200, 333, 150
    gh.say("ra_lse_merge", dtype, D)
    qn = ra_inputs.normal((B, H, q_len, D), 0, seed=5, dtype=dtype)
    kn = ra_inputs.normal((B, H, kv_len, D), 1, seed=5, dtype=dtype)
    vn = ra_inputs.normal((B, H, kv_len, D), 2, seed=5, dtype=dtype)
    q, k, v = (gh.to_device(x, dtype) for x in (qn, kn, vn))
    off = 140  # rows < 10 see no key of the second part
    parts = []
    for lo, hi in ((0, split), (split, kv_len)):
        o = torch.empty(B, H, q_len, D, device="cuda")
        m = torch.empty(B, H, q_len, device="cuda")
        l = torch.empty(B, H, q_len, device="cuda")
        ra.ra_block_attn_fwd(q, k[:, :, lo:hi], v[:, :, lo:hi], o, m, l, causal=True, q_pos0=off, k_pos0=lo)
        parts.append((o, m, l))
    (oa, ma, la), (ob, mb, lb) = parts
    # commutativity and the -inf identity
    o1, m1, l1 = oa.clone(), ma.clone(), la.clone()
    ra.ra_lse_merge(o1, m1, l1, ob, mb, lb)
    o2, m2, l2 = ob.clone(), mb.clone(), lb.clone()
    ra.ra_lse_merge(o2, m2, l2, oa, ma, la)
    e_o, e_m, e_l = torch.zeros_like(ob), torch.full_like(mb, float("-inf")), torch.zeros_like(lb)
    ra.ra_lse_merge(e_o, e_m, e_l, ob, mb, lb)
    torch.cuda.synchronize()
    assert torch.equal(e_o, ob) and torch.equal(e_m, mb) and torch.equal(e_l, lb)
    assert torch.allclose(o1, o2, rtol=1e-6, atol=1e-6) and torch.equal(m1, m2)
    # finalise
    out = torch.empty(B, H, q_len, D, device="cuda", dtype=torch.bfloat16 if dtype == "bf16" else torch.float32)
    lse = torch.empty(B, H, q_len, device="cuda")
    before = (oa.clone(), ma.clone(), la.clone())
    ra.ra_lse_merge(oa, ma, la, ob, mb, lb, o_out=out, lse_out=lse)
    torch.cuda.synchronize()
    assert all(torch.equal(x, y) for x, y in zip(before, (oa, ma, la)))  # running state untouched
    out, lse, m1, l1, o1 = (gh.to_host_f64(x) for x in (out, lse, m1, l1, o1))
    tol = gh.TOL[dtype]
    for h in range(H):
        r = oracle.rows(qn[0, h], kn[0, h], vn[0, h], q_pos=np.arange(q_len) + off, causal=True)
        assert np.max(np.abs(m1[0, h] - r["m"])) <= 1e-4
        assert np.max(np.abs(o1[0, h] / l1[0, h][:, None] - r["o"])) <= tol["o"]
        assert np.max(np.abs(out[0, h] - r["o"])) <= tol["o"]
        assert np.max(np.abs(lse[0, h] - r["lse"])) <= tol["lse"]


# ------------------------------------------------------------------ permute
@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("bf16", 64), ("f32", 1), ("f32", 16), ("bf16", 3)])
@pytest.mark.parametrize("lay", ["contiguous", "striped"])
def test_stripe_permute_bit_exact(dtype, D, lay):
    gh.say("ra_stripe_permute", dtype, D, lay)
    for n in (1, 2, 4, 8):
        B, H, S = 2, 3, 16 * n
        xn = ra_inputs.normal((B, H, S, D), 0, seed=n, dtype=dtype)
        x = gh.to_device(xn, dtype)
        y = torch.empty((n, B, H, S // n, D), dtype=x.dtype, device="cuda")
        ra.ra_stripe_permute(x, y, layout=lay, inverse=False, n_pos=n)
        back = torch.empty_like(x)
        ra.ra_stripe_permute(y, back, layout=lay, inverse=True, n_pos=n)
        torch.cuda.synchronize()
        want = olayout.to_shards(xn, n, lay)
        got = y.view(torch.int16).cpu().numpy().view(np.uint16) if dtype == "bf16" else y.cpu().numpy()
        assert np.array_equal(got, want)
        assert torch.equal(back, x)


# ------------------------------------------------------------------ ring: configs
def test_config1_page_example_fp32():
    """4 positions x 8 tokens, d 16, fp32, non-causal: the pages' worked example."""
    gh.say("ra_ring_forward config1 fp32")
    for source in ("page", "seeded"):
        if source == "page":
            torch.manual_seed(0)
            qn, kn, vn = (t.numpy()[None, None] for t in torch.randn(3, 32, 16))
        else:
            qn, kn, vn = gh.qkv_global(1, 1, 1, 32, 16, "f32", seed=0)
        qs, ks, vs = (gh.shards_on_device(x, 4, "contiguous", "f32") for x in (qn, kn, vn))
        o, lse, _ = gh.run_ring(qs, ks, vs, 4, 0, "contiguous", False)
        full = torch.empty(1, 1, 32, 16, device="cuda")
        ra.ra_stripe_permute(o, full, layout="contiguous", inverse=True, n_pos=4)
        torch.cuda.synchronize()
        r = oracle.rows(qn[0, 0], kn[0, 0], vn[0, 0])
        got = gh.to_host_f64(full)[0, 0]
        assert np.max(np.abs(got - r["o"])) <= 1e-5
        assert np.max(np.abs(gh.to_host_f64(lse).reshape(32) - r["lse"])) <= 1e-5
        # the page's own criterion: allclose(atol=1e-5) with the default rtol
        assert np.allclose(got, r["o"], atol=1e-5)


def test_config2_noncausal_bf16_all_rows():
    B, H, S, D, N = 1, 4, 4096, 64, 2
    gh.say("ra_ring_forward config2")
    qn, kn, vn = gh.qkv_global(B, H, H, S, D, "bf16")
    qs, ks, vs = (gh.shards_on_device(x, N, "contiguous", "bf16") for x in (qn, kn, vn))
    hh, tt = np.meshgrid(np.arange(H), np.arange(S), indexing="ij")
    # 8 query tiles x 4 heads per launch: the automatic schedule splits each
    # block's keys into 4 ranges and folds them with one merge pass per step
    o, lse, st = gh.run_ring(qs, ks, vs, N, 0, "contiguous", False, stats=True)
    assert st["block_launches"] == 4 and st["merge_launches"] == 4 and st["blocks_skipped"] == 0
    assert st["kv_splits"] == 4
    assert st["flops"] == 4 * D * H * S * S
    gh.compare_rows(o, lse, qn, kn, vn, hh.ravel(), tt.ravel(), N, "contiguous", 0, False, "bf16")
    # without splits: the merge is fused into the block kernel, one finalise per position
    o, lse, st = gh.run_ring(qs, ks, vs, N, 0, "contiguous", False, kv_splits=1, stats=True)
    assert st["block_launches"] == 4 and st["merge_launches"] == 2
    gh.compare_rows(o, lse, qn, kn, vn, hh.ravel(), tt.ravel(), N, "contiguous", 0, False, "bf16")


@pytest.mark.timeout(600)
def test_config3_causal_contiguous_sampled():
    B, H, S, D, N = 1, 32, 32768, 128, 4
    gh.say("ra_ring_forward config3")
    qn, kn, vn = gh.qkv_global(B, H, H, S, D, "bf16")
    qs, ks, vs = (gh.shards_on_device(x, N, "contiguous", "bf16") for x in (qn, kn, vn))
    o, lse, st = gh.run_ring(qs, ks, vs, N, 0, "contiguous", True, stats=True)
    assert st["blocks_skipped"] == N * (N - 1) // 2
    assert st["flops"] == 4 * D * H * S * (S + 1) // 2
    sh, stt = ra_inputs.sample_rows(S, N, 4096, heads=H, seed=1)
    assert len(set(zip(sh.tolist(), stt.tolist()))) == 4096
    gh.compare_rows(o, lse, qn, kn, vn, sh, stt, N, "contiguous", 0, True, "bf16")


# ------------------------------------------------------------------ ring: invariants
def _small_ring_inputs(S=2048, H=4, Hkv=4, D=128, N=8, lay="striped", dtype="bf16", seed=7):
    qn, kn, vn = gh.qkv_global(1, H, Hkv, S, D, dtype, seed=seed)
    return (qn, kn, vn), tuple(gh.shards_on_device(x, N, lay, dtype) for x in (qn, kn, vn))


def test_visit_order_invariance():
    gh.say("ra_ring_forward visit orders")
    N, S, H = 8, 2048, 4
    (qn, kn, vn), (qs, ks, vs) = _small_ring_inputs(S=S, H=H, N=N)
    rng = np.random.Generator(np.random.PCG64(11))
    hh, tt = np.meshgrid(np.arange(H), np.arange(S), indexing="ij")
    outs = []
    for order in (None, list(range(N))[::-1], list(rng.permutation(N))):
        o, lse, _ = gh.run_ring(qs, ks, vs, N, 0, "striped", True, visit_order=order)
        gh.compare_rows(o, lse, qn, kn, vn, hh.ravel(), tt.ravel(), N, "striped", 0, True, "bf16")
        outs.append((o.float(), lse))
    for o, lse in outs[1:]:
        assert torch.max(torch.abs(o - outs[0][0])) <= 2e-2
        assert torch.max(torch.abs(lse - outs[0][1])) <= 1e-4


def test_emulated_copy_ring_and_streams_are_bitwise_identical():
    gh.say("ra_ring_forward emulate_copy / streams / determinism")
    N = 8
    _, (qs, ks, vs) = _small_ring_inputs(N=N)
    ref, ref_lse, _ = gh.run_ring(qs, ks, vs, N, 0, "striped", True)
    for kw in ({}, {"emulate_copy": True}, {"n_streams": 1}, {"n_streams": 3, "emulate_copy": True},
               {"visit_order": list(range(N))}):
        o, lse, _ = gh.run_ring(qs, ks, vs, N, 0, "striped", True, **kw)
        assert torch.equal(o, ref) and torch.equal(lse, ref_lse), kw
    # contiguous causal with skipped blocks through the copy path too
    (qn, kn, vn), (qc, kc, vc) = _small_ring_inputs(N=4, lay="contiguous")
    a, al, st = gh.run_ring(qc, kc, vc, 4, 0, "contiguous", True, stats=True)
    b, bl, stb = gh.run_ring(qc, kc, vc, 4, 0, "contiguous", True, emulate_copy=True, stats=True)
    assert torch.equal(a, b) and torch.equal(al, bl)
    assert st["blocks_skipped"] == 6 and stb["copy_launches"] == 4 * 4


def test_gqa_equals_repeated_kv_heads():
    gh.say("ra_ring_forward gqa")
    N, S, Hq, Hkv = 4, 1024, 8, 2
    (qn, kn, vn), (qs, ks, vs) = _small_ring_inputs(S=S, H=Hq, Hkv=Hkv, N=N)
    o, lse, _ = gh.run_ring(qs, ks, vs, N, 0, "striped", True)
    kr, vr = (x.repeat_interleave(Hq // Hkv, dim=2).contiguous() for x in (ks, vs))
    o2, lse2, _ = gh.run_ring(qs, kr, vr, N, 0, "striped", True)
    assert torch.equal(o, o2) and torch.equal(lse, lse2)
    hh, tt = np.meshgrid(np.arange(Hq), np.arange(S), indexing="ij")
    gh.compare_rows(o, lse, qn, kn, vn, hh.ravel(), tt.ravel(), N, "striped", 0, True, "bf16")


def test_striped_and_contiguous_agree_after_unpermuting():
    gh.say("ra_ring_forward striped vs contiguous")
    N, S, H, D = 4, 2048, 4, 64
    qn, kn, vn = gh.qkv_global(1, H, H, S, D, "bf16", seed=13)
    res = {}
    for lay in ("striped", "contiguous"):
        qs, ks, vs = (gh.shards_on_device(x, N, lay, "bf16") for x in (qn, kn, vn))
        o, lse, _ = gh.run_ring(qs, ks, vs, N, 0, lay, True)
        full = torch.empty(1, H, S, D, device="cuda", dtype=torch.bfloat16)
        ra.ra_stripe_permute(o, full, layout=lay, inverse=True, n_pos=N)
        lse_full = torch.empty(1, H, S, 1, device="cuda")
        ra.ra_stripe_permute(lse[..., None].contiguous(), lse_full, layout=lay, inverse=True, n_pos=N)
        torch.cuda.synchronize()
        res[lay] = (gh.to_host_f64(full)[0], gh.to_host_f64(lse_full)[0, ..., 0])
    assert np.max(np.abs(res["striped"][0] - res["contiguous"][0])) <= 2e-2
    assert np.max(np.abs(res["striped"][1] - res["contiguous"][1])) <= 1e-3
    o_ref, lse_ref = oracle.attention(qn, kn, vn, causal=True)
    assert np.max(np.abs(res["striped"][0] - o_ref[0])) <= 2e-2
    assert np.max(np.abs(res["striped"][1] - lse_ref[0])) <= 1e-3


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("lay", ["contiguous", "striped"])
def test_brute_force_causal_grid(dtype, lay):
    gh.say("ra_ring_forward causal grid", dtype, lay)
    grid = ([(S, N) for S in (1, 2, 3, 7, 8, 9, 16, 33) for N in (1, 2, 4, 8) if S % N == 0]
            if dtype == "f32" else [(S, N) for S in (128, 256, 512) for N in (1, 2, 4)])
    D = 16 if dtype == "f32" else 64
    for S, N in grid:
        qn, kn, vn = gh.qkv_global(1, 2, 1, S, D, dtype, seed=S * 10 + N)
        qs, ks, vs = (gh.shards_on_device(x, N, lay, dtype) for x in (qn, kn, vn))
        o, lse, _ = gh.run_ring(qs, ks, vs, N, 0, lay, True)
        hh, tt = np.meshgrid(np.arange(2), np.arange(S), indexing="ij")
        gh.compare_rows(o, lse, qn, kn, vn, hh.ravel(), tt.ravel(), N, lay, 0, True, dtype)


# ------------------------------------------------------------------ fused merge
@pytest.mark.parametrize("dtype,D,flags", [("bf16", 128, 0), ("bf16", 64, 0), ("f32", 40, 0), ("bf16", 128, 1)])
def test_block_accumulate_equals_separate_merge(dtype, D, flags):
    """RA_BLOCK_ACCUMULATE merges a block into a running state exactly like
    computing the partial and folding it in with ra_lse_merge."""
    B, H, q_len, kv_len, split = 1, 3, 300, 333, 150
    gh.say("ra_block_attn_fwd accumulate", dtype, D, flags)
    qn = ra_inputs.normal((B, H, q_len, D), 0, seed=6, dtype=dtype)
    kn = ra_inputs.normal((B, H, kv_len, D), 1, seed=6, dtype=dtype)
    vn = ra_inputs.normal((B, H, kv_len, D), 2, seed=6, dtype=dtype)
    q, k, v = (gh.to_device(x, dtype) for x in (qn, kn, vn))
    off = 140
    def part(lo, hi, o, m, l, extra=0):
        ra.ra_block_attn_fwd(q, k[:, :, lo:hi], v[:, :, lo:hi], o, m, l, causal=True, q_pos0=off, k_pos0=lo,
                             flags=flags | extra)
    new = lambda: (torch.empty(B, H, q_len, D, device="cuda"), torch.empty(B, H, q_len, device="cuda"),
                   torch.empty(B, H, q_len, device="cuda"))
    acc, pb, ref = new(), new(), new()
    part(0, split, *acc)
    part(0, split, *ref)
    part(split, kv_len, *pb)
    ra.ra_lse_merge(*ref, *pb)                           # separate: partial + fold
    part(split, kv_len, *acc, extra=ra.RA_BLOCK_ACCUMULATE)  # fused
    # an empty running state (m = -inf) is the identity
    emp = (torch.zeros(B, H, q_len, D, device="cuda"), torch.full((B, H, q_len), float("-inf"), device="cuda"),
           torch.zeros(B, H, q_len, device="cuda"))
    part(split, kv_len, *emp, extra=ra.RA_BLOCK_ACCUMULATE)
    torch.cuda.synchronize()
    assert torch.equal(acc[1], ref[1])
    assert torch.allclose(acc[2], ref[2], rtol=2e-6, atol=0)
    assert torch.allclose(acc[0], ref[0], rtol=2e-6, atol=1e-6)
    assert torch.equal(emp[1], pb[1]) and torch.allclose(emp[2], pb[2], rtol=1e-6, atol=0)
    assert torch.allclose(emp[0], pb[0], rtol=1e-6, atol=1e-7)
    o, m, l = (gh.to_host_f64(x) for x in acc)
    tol = gh.TOL[dtype]
    for h in range(H):
        r = oracle.rows(qn[0, h], kn[0, h], vn[0, h], q_pos=np.arange(q_len) + off, causal=True)
        assert np.max(np.abs(m[0, h] - r["m"])) <= 1e-4
        assert np.max(np.abs(o[0, h] / l[0, h][:, None] - r["o"])) <= tol["o"]
        assert np.max(np.abs(m[0, h] + np.log(l[0, h]) - r["lse"])) <= tol["lse"]


@pytest.mark.parametrize("lay,causal", [("striped", True), ("contiguous", True), ("contiguous", False)])
def test_fused_and_separate_merge_rings_agree(lay, causal):
    gh.say("ra_ring_forward fused vs separate", lay, causal)
    N, S, H = 4, 2048, 4
    (qn, kn, vn), (qs, ks, vs) = _small_ring_inputs(S=S, H=H, N=N, lay=lay)
    o1, l1, st1 = gh.run_ring(qs, ks, vs, N, 0, lay, causal, kv_splits=1, stats=True)
    o2, l2, st2 = gh.run_ring(qs, ks, vs, N, 0, lay, causal, separate_merge=True, stats=True)
    # fused: one finalising pass per position; separate: one fold per block after the
    # first (the last one also finalises), and one pass where a position has a single block
    singles = 1 if (lay == "contiguous" and causal) else 0
    assert st1["merge_launches"] == N
    assert st2["merge_launches"] == st2["block_launches"] - N + singles
    assert torch.max(torch.abs(o1.float() - o2.float())) <= 1e-2
    assert torch.max(torch.abs(l1 - l2)) <= 1e-5
    hh, tt = np.meshgrid(np.arange(H), np.arange(S), indexing="ij")
    for o, lse in ((o1, l1), (o2, l2)):
        gh.compare_rows(o, lse, qn, kn, vn, hh.ravel(), tt.ravel(), N, lay, 0, causal, "bf16")


@pytest.mark.parametrize("lay,causal,D,Sb,N,splits,used", [
    ("contiguous", True, 128, 1000, 2, 3, 3),  # ragged last range; diagonal block: early tiles see empty ranges
    ("contiguous", True, 64, 640, 3, 0, 2),    # automatic count over 5 tiles: 2 ranges of 3 and 2 tiles
    ("striped", True, 128, 1000, 2, 8, 8),     # 8 ranges of one tile
    ("striped", False, 64, 384, 4, 2, 2),
    ("striped", False, 64, 384, 4, 8, 3),      # capped at the block's 3 tiles
    ("contiguous", False, 128, 2048, 2, 8, 8),
])
def test_kv_split_ring_matches_oracle(lay, causal, D, Sb, N, splits, used):
    """Key-split schedule: each block's keys in ranges of whole 128-key tiles,
    one partial per range, folded by one multi-partial merge per step; every
    row against the oracle, and close to the unsplit schedule."""
    H = 2
    S = Sb * N
    gh.say("ra_ring_forward kv splits", lay, causal, D, Sb, N, splits)
    (qn, kn, vn), (qs, ks, vs) = _small_ring_inputs(S=S, H=H, Hkv=1, D=D, N=N, lay=lay, seed=5)
    o1, l1, st1 = gh.run_ring(qs, ks, vs, N, 0, lay, causal, kv_splits=splits, stats=True)
    o2, l2, st2 = gh.run_ring(qs, ks, vs, N, 0, lay, causal, kv_splits=1, stats=True)
    assert st1["kv_splits"] == used and st2["kv_splits"] == 1
    computed = st1["block_launches"]
    assert computed == st2["block_launches"] == N * N - st1["blocks_skipped"]
    assert st1["merge_launches"] == computed  # one fold per computed block, the last also finalises
    assert st2["merge_launches"] == N
    assert torch.max(torch.abs(o1.float() - o2.float())) <= 1e-2
    assert torch.max(torch.abs(l1 - l2)) <= 1e-4
    hh, tt = np.meshgrid(np.arange(H), np.arange(S), indexing="ij")
    gh.compare_rows(o1, l1, qn, kn, vn, hh.ravel(), tt.ravel(), N, lay, 0, causal, "bf16")
    # the same key ranges with blocks travelling through the emulated-transfer
    # slots on one stream: the same schedule, so bit-identical
    o3, l3, st3 = gh.run_ring(qs, ks, vs, N, 0, lay, causal, kv_splits=splits, emulate_copy=True, n_streams=1,
                              stats=True)
    assert st3["kv_splits"] == used
    assert torch.equal(o3, o1) and torch.equal(l3, l1)


@pytest.mark.parametrize("H,S,D,splits", [(4, 4096, 64, 0), (4, 4096, 64, 1), (32, 8192, 128, 0)],
                         ids=["key-splits", "no-splits", "work-queues"])
def test_ring_forward_graph_replay(H, S, D, splits):
    """A whole ring step (permute in, ra_ring_forward, permute out) captured
    into a HIP graph: every replay, with eager work and synchronisations
    between replays, reproduces the eager step bit for bit.  The small ring
    runs with key splits or without; the larger one (512 query tiles a
    launch) takes the block kernel's work queues, whose counters the call
    zeroes with a fill kernel and every launch leaves zeroed."""
    B, N = 1, 2
    gh.say("ra_ring_forward graph replay", H, S, D, splits)
    qn, kn, vn = gh.qkv_global(B, H, H, S, D, "bf16", seed=3)
    q_g, k_g, v_g = (gh.to_device(x, "bf16") for x in (qn, kn, vn))
    q_sh = torch.empty((N, B, H, S // N, D), dtype=torch.bfloat16, device="cuda")
    k_sh, v_sh, o_sh = torch.empty_like(q_sh), torch.empty_like(q_sh), torch.empty_like(q_sh)
    lse = torch.empty(q_sh.shape[:4], dtype=torch.float32, device="cuda")
    out = torch.empty_like(q_g)
    ws = torch.empty(ra.ra_ring_workspace_size(ra.ring_desc(q_sh, k_sh, n_pos=N, kv_splits=splits)),
                     dtype=torch.uint8, device="cuda")

    def step():
        for src, dst in ((q_g, q_sh), (k_g, k_sh), (v_g, v_sh)):
            ra.ra_stripe_permute(src, dst, layout="contiguous", inverse=False, n_pos=N)
        ra.ra_ring_forward(q_sh, k_sh, v_sh, o_sh, lse, n_pos=N, workspace=ws, kv_splits=splits)
        ra.ra_stripe_permute(o_sh, out, layout="contiguous", inverse=True, n_pos=N)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    ref_o, ref_l = out.clone(), lse.clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for _ in range(3):
        out.fill_(0)
        lse.fill_(0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_o) and torch.equal(lse, ref_l)
        step()  # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(out, ref_o)
    hh, tt = np.meshgrid(np.arange(H), np.arange(S), indexing="ij")
    sel = np.arange(0, H * S, 37)
    gh.compare_rows(o_sh, lse, qn, kn, vn, hh.ravel()[sel], tt.ravel()[sel], N, "contiguous", 0, False, "bf16")


@pytest.mark.parametrize("D", [128, 64])
@pytest.mark.parametrize("lay", ["striped", "contiguous"])
def test_work_queue_ring_equals_fixed_order_blocks(lay, D):
    """A ring whose block launches have many more query tiles than the GPU has
    compute units runs them through the kernel's work queues (persistent
    workgroups claiming tiles from per-XCD queues).  The same fused schedule
    composed from ra_block_attn_fwd calls (one workgroup per tile, fixed
    order) and a finalising ra_lse_merge must give bit-identical O and lse:
    every tile is then processed exactly once by the queues, with the same
    arithmetic, in every step of the ring (the counters each launch leaves for
    the next included)."""
    B, Hq, Hkv, N = 1, 32, 8, 4
    Sb = max(4096, 2 * torch.cuda.get_device_properties(0).multi_processor_count * 256 // Hq)
    S, i = Sb * N, N - 1
    gh.say("ra_ring_forward work queues vs fixed-order blocks", lay, D, Sb)
    qn, kn, vn = gh.qkv_global(B, Hq, Hkv, S, D, "bf16", seed=41)
    qs, ks, vs = (gh.shards_on_device(x, N, lay, "bf16") for x in (qn, kn, vn))
    del qn, kn, vn
    q_run = qs[i:i + 1].contiguous()
    # one stream: the steps fold into one running state in ring order
    o_ring, lse_ring, _ = gh.run_ring(q_run, ks, vs, N, i, lay, True, n_streams=1)

    o = torch.empty(B, Hq, Sb, D, device="cuda")
    m = torch.empty(B, Hq, Sb, device="cuda")
    l = torch.empty_like(m)
    for s in range(N):
        j = (i - s) % N
        if lay == "striped":  # token i + N r of position i, j + N c of block j
            pos = dict(q_pos0=i, k_pos0=j, pos_stride=N)
        else:
            pos = dict(q_pos0=i * Sb, k_pos0=j * Sb, pos_stride=1)
        if lay == "contiguous" and j > i:
            continue  # fully masked: the ring skips it too
        first = s == 0
        ra.ra_block_attn_fwd(q_run[0], ks[j], vs[j], o, m, l, causal=True,
                             flags=0 if first else ra.RA_BLOCK_ACCUMULATE, **pos)
    o_blk = torch.empty(B, Hq, Sb, D, dtype=torch.bfloat16, device="cuda")
    lse_blk = torch.empty(B, Hq, Sb, device="cuda")
    ra.ra_lse_merge(o, m, l, o_out=o_blk, lse_out=lse_blk)
    torch.cuda.synchronize()
    assert torch.equal(o_ring[0].view(torch.int16), o_blk.view(torch.int16))
    assert torch.equal(lse_ring[0], lse_blk)


@pytest.mark.parametrize("lay", ["striped", "contiguous"])
def test_single_position_accumulation_chains(lay):
    """One position whose block launches are large runs its computed steps
    alternately on two running states (two streams) that the finalising merge
    folds together.  Same launches and one merge pass as the one-stream
    schedule, agreement with it to rounding, and the oracle on 2048 rows."""
    B, Hq, Hkv, N, D = 1, 32, 8, 4, 128
    Sb = max(4096, 2 * torch.cuda.get_device_properties(0).multi_processor_count * 256 // Hq)
    S, i = Sb * N, N - 1
    gh.say("ra_ring_forward accumulation chains", lay, Sb)
    qn, kn, vn = gh.qkv_global(B, Hq, Hkv, S, D, "bf16", seed=45)
    qs, ks, vs = (gh.shards_on_device(x, N, lay, "bf16") for x in (qn, kn, vn))
    q_run = qs[i:i + 1].contiguous()
    desc1 = ra.ring_desc(q_run, ks, n_pos=N, first_pos=i, layout=lay, causal=True, n_streams=1)
    desc2 = ra.ring_desc(q_run, ks, n_pos=N, first_pos=i, layout=lay, causal=True)
    # the second chain's running state is the only extra workspace
    assert ra.ra_ring_workspace_size(desc2) - ra.ra_ring_workspace_size(desc1) >= B * Hq * Sb * (4 * D + 8)
    o1, l1, st1 = gh.run_ring(q_run, ks, vs, N, i, lay, True, n_streams=1, stats=True)
    o2, l2, st2 = gh.run_ring(q_run, ks, vs, N, i, lay, True, stats=True)
    assert st2["block_launches"] == st1["block_launches"] == N and st2["merge_launches"] == st1["merge_launches"] == 1
    assert torch.max(torch.abs(o1.float() - o2.float())) <= 1e-2
    assert torch.max(torch.abs(l1 - l2)) <= 1e-5
    sh, st = ra_inputs.sample_rows(S, N, 2048, heads=Hq, seed=1, share=i, layout=lay)
    gh.compare_rows(o2, l2, qn, kn, vn, sh, st, N, lay, i, True, "bf16")
    # deterministic: the same call twice gives the same bits
    o3, l3, _ = gh.run_ring(q_run, ks, vs, N, i, lay, True)
    assert torch.equal(o3, o2) and torch.equal(l3, l2)
