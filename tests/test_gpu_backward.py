"""GPU parity of the backward pass against the fp64 gradient oracle.

Block pairs: ra_block_attn_bwd adds one (query block, key block) share of dQ,
dK, dV given the rows' full-key-set lse and delta; the oracle computes the
same share (``oracle.grads`` with lse/delta).  Rings: ra_ring_backward's
gradients against ``oracle.attention_grads`` in global token order.

Tolerance: elementwise, |GPU - oracle| <= rtol (|oracle| + row RMS + 2^-4 RMS)
(tests/gpu_helpers.py grad_close), with rtol = 1e-4 for the fp32-arithmetic
kernels on binary32 inputs and 2^-5 where bfloat16 enters a gradient sum (the
MFMA kernels round P and dS to bfloat16; bfloat16 rings feed the forward's
bfloat16 output into delta).
"""
import numpy as np
import pytest
import torch

import oracle
import ra_inputs
import ring_attention_step_amd as ra
from tests import gpu_helpers as gh

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ra.load_library()
    yield
    torch.cuda.synchronize()


def _close(got, want, tol, what):
    err = float(np.max(np.abs(got - want))) if want.size else 0.0
    ref = max(1.0, float(np.max(np.abs(want)))) if want.size else 1.0
    assert err <= tol * ref, f"{what}: max |GPU - oracle| = {err:.3e} > {tol} * {ref:.3g}"
    return err / ref


def _dq_delta_extra(qn, kn, vn, gn, causal):
    """dq_delta_bound over whole [B, Hq, S, D] tensors: the oracle's O and P K."""
    o_ref, _ = oracle.attention(qn, kn, vn, causal=causal)
    pk_ref, _ = oracle.attention(qn, kn, kn, causal=causal)
    return gh.dq_delta_bound(o_ref, pk_ref, gn, 1.0 / np.sqrt(qn.shape[-1]))


def test_delta_kernel():
    for dtype, D in (("f32", 48), ("bf16", 128)):
        gh.say("ra_attn_bwd_delta", dtype, D)
        o = ra_inputs.normal((1, 3, 257, D), 0, seed=21, dtype=dtype)
        g = ra_inputs.normal((1, 3, 257, D), 1, seed=21, dtype=dtype)
        od, gd = gh.to_device(o, dtype), gh.to_device(g, dtype)
        delta = torch.empty(1, 3, 257, device="cuda")
        ra.ra_attn_bwd_delta(od, gd, delta)
        torch.cuda.synchronize()
        wid = (lambda x: ra_inputs.bf16_to_f32(x)) if dtype == "bf16" else (lambda x: x)
        want = np.sum(wid(o).astype(np.float64) * wid(g).astype(np.float64), axis=-1)
        _close(gh.to_host_f64(delta), want, 1e-5, "delta")


BLOCK_CASES = [("f32", 16, 1), ("f32", 64, 1), ("f32", 100, 1), ("f32", 256, 1), ("bf16", 64, 1),
               ("bf16", 128, 1), ("bf16", 128, 0), ("bf16", 64, 0), ("bf16", 48, 0)]
OFFSETS = [None, 0, -1, 37, -150, 400]


@pytest.mark.parametrize("dtype,D,force_simt", BLOCK_CASES)
def test_block_bwd_matches_oracle(dtype, D, force_simt):
    B, Hq, Hkv, q_len, kv_len = 1, 4, 2, 300, 333
    gh.say("ra_block_attn_bwd", dtype, D, force_simt)
    qn = ra_inputs.normal((B, Hq, q_len, D), 0, seed=31, dtype=dtype)
    kn = ra_inputs.normal((B, Hkv, kv_len, D), 1, seed=31, dtype=dtype)
    vn = ra_inputs.normal((B, Hkv, kv_len, D), 2, seed=31, dtype=dtype)
    gn = ra_inputs.normal((B, Hq, q_len, D), 3, seed=31, dtype=dtype)
    # q and dout as strided views ([B, S, H, D] memory)
    q = gh.to_device(np.ascontiguousarray(qn.transpose(0, 2, 1, 3)), dtype).permute(0, 2, 1, 3)
    g = gh.to_device(np.ascontiguousarray(gn.transpose(0, 2, 1, 3)), dtype).permute(0, 2, 1, 3)
    k, v = gh.to_device(kn, dtype), gh.to_device(vn, dtype)
    mfma = dtype == "bf16" and D in (64, 128) and not force_simt
    tol = gh.GRAD_RTOL["bf16"] if mfma else gh.GRAD_RTOL["fp32"]
    grp = Hq // Hkv
    for off in OFFSETS:
        causal = off is not None
        qpos = np.arange(q_len, dtype=np.int64) + (off or 0)
        # the rows' "full key set" for lse / delta: this block plus keys before it,
        # so that lse is not this block's own (exercises the share semantics)
        lse = np.empty((B, Hq, q_len))
        dlt = np.empty((B, Hq, q_len))
        want = {"dq": np.zeros((B, Hq, q_len, D)), "dk": np.zeros((B, Hkv, kv_len, D)),
                "dv": np.zeros((B, Hkv, kv_len, D))}
        extra = ra_inputs.normal((1, Hkv, 64, D), 1, seed=32, dtype=dtype)
        for h in range(Hq):
            kk = np.concatenate([extra[0, h // grp], kn[0, h // grp]])
            vv = np.concatenate([extra[0, h // grp], vn[0, h // grp]])
            kpos = np.concatenate([np.arange(-64, 0), np.arange(kv_len)])
            full = oracle.grads(qn[0, h], kk, vv, gn[0, h], q_pos=qpos, k_pos=kpos, causal=causal)
            lse[0, h], dlt[0, h] = full["lse"], full["delta"]
            part = oracle.grads(qn[0, h], kn[0, h // grp], vn[0, h // grp], gn[0, h], q_pos=qpos,
                                k_pos=np.arange(kv_len), causal=causal, lse=full["lse"], delta=full["delta"])
            want["dq"][0, h] = part["dq"]
            want["dk"][0, h // grp] += part["dk"]
            want["dv"][0, h // grp] += part["dv"]
        dq = torch.zeros(B, Hq, q_len, D, device="cuda")
        dk = torch.zeros(B, Hkv, kv_len, D, device="cuda")
        dv = torch.zeros(B, Hkv, kv_len, D, device="cuda")
        lse_d = torch.from_numpy(lse.astype(np.float32)).cuda()
        dlt_d = torch.from_numpy(dlt.astype(np.float32)).cuda()
        ra.ra_block_attn_bwd(q, k, v, g, lse_d, dlt_d, dq, dk, dv, causal=causal, q_pos0=(off or 0), k_pos0=0,
                             flags=ra.RA_BLOCK_FORCE_SIMT if force_simt else 0)
        torch.cuda.synchronize()
        for name, got in (("dq", dq), ("dk", dk), ("dv", dv)):
            gh.grad_close(gh.to_host_f64(got), want[name], tol, f"{name} off={off}")


def test_block_bwd_accumulates_and_empty_cases():
    gh.say("ra_block_attn_bwd accumulate / empty")
    D = 64
    q = torch.randn(1, 2, 40, D, device="cuda")
    k = torch.randn(1, 2, 50, D, device="cuda")
    lse = torch.full((1, 2, 40), 3.0, device="cuda")
    dlt = torch.zeros(1, 2, 40, device="cuda")
    dq = torch.full((1, 2, 40, D), 1.5, device="cuda")
    dk = torch.full((1, 2, 50, D), -2.0, device="cuda")
    dv = torch.full((1, 2, 50, D), 0.25, device="cuda")
    # every key after every query: nothing visible, outputs unchanged
    ra.ra_block_attn_bwd(q, k, k, q, lse, dlt, dq, dk, dv, causal=True, q_pos0=0, k_pos0=1000)
    torch.cuda.synchronize()
    assert torch.all(dq == 1.5) and torch.all(dk == -2.0) and torch.all(dv == 0.25)
    # rows without keys (lse = -inf) contribute nothing either
    ninf = torch.full((1, 2, 40), float("-inf"), device="cuda")
    ra.ra_block_attn_bwd(q, k, k, q, ninf, dlt, dq, dk, dv)
    torch.cuda.synchronize()
    assert torch.all(dq == 1.5) and torch.all(dk == -2.0) and torch.all(dv == 0.25)
    e = torch.empty(1, 2, 0, D, device="cuda")
    ra.ra_block_attn_bwd(e, k, k, e, e[..., 0], e[..., 0], e, dk, dv)  # no-op


@pytest.mark.parametrize("D", [128, 64])
def test_block_bwd_rows_without_keys_mfma(D):
    """bf16 MFMA kernels: rows whose lse is -inf contribute nothing, both where
    they share a query tile with rows that see keys (queries start 37 positions
    before the block's keys, lse over this block only) and where the caller
    passes -inf for every row of a non-causal block."""
    gh.say("ra_block_attn_bwd rows without keys", D)
    Hq, Hkv, q_len, kv_len, off = 2, 1, 200, 150, -37
    qn = ra_inputs.normal((1, Hq, q_len, D), 0, seed=37)
    kn = ra_inputs.normal((1, Hkv, kv_len, D), 1, seed=37)
    vn = ra_inputs.normal((1, Hkv, kv_len, D), 2, seed=37)
    gn = ra_inputs.normal((1, Hq, q_len, D), 3, seed=37)
    q, k, v, g = (gh.to_device(x, "bf16") for x in (qn, kn, vn, gn))
    qpos = np.arange(q_len, dtype=np.int64) + off
    want = {"dq": np.zeros((1, Hq, q_len, D)), "dk": np.zeros((1, Hkv, kv_len, D)),
            "dv": np.zeros((1, Hkv, kv_len, D))}
    lse = np.empty((1, Hq, q_len))
    dlt = np.empty((1, Hq, q_len))
    for h in range(Hq):
        r = oracle.grads(qn[0, h], kn[0, 0], vn[0, 0], gn[0, h], q_pos=qpos, causal=True)
        lse[0, h], dlt[0, h] = r["lse"], r["delta"]
        want["dq"][0, h] = r["dq"]
        want["dk"][0, 0] += r["dk"]
        want["dv"][0, 0] += r["dv"]
    assert np.isneginf(lse[0, :, :37]).all() and np.isfinite(lse[0, :, 37:]).all()
    dq = torch.zeros(1, Hq, q_len, D, device="cuda")
    dk = torch.zeros(1, Hkv, kv_len, D, device="cuda")
    dv = torch.zeros(1, Hkv, kv_len, D, device="cuda")
    lse_d = torch.from_numpy(lse.astype(np.float32)).cuda()
    dlt_d = torch.from_numpy(dlt.astype(np.float32)).cuda()
    ra.ra_block_attn_bwd(q, k, v, g, lse_d, dlt_d, dq, dk, dv, causal=True, q_pos0=off, k_pos0=0)
    torch.cuda.synchronize()
    for name, got in (("dq", dq), ("dk", dk), ("dv", dv)):
        gh.grad_close(gh.to_host_f64(got), want[name], gh.GRAD_RTOL["bf16"], name)
    # every row -inf on a non-causal block: nothing changes
    for x in (dq, dk, dv):
        x.fill_(0.5)
    ra.ra_block_attn_bwd(q, k, v, g, torch.full_like(lse_d, float("-inf")), dlt_d, dq, dk, dv)
    torch.cuda.synchronize()
    assert all(bool(torch.all(x == 0.5)) for x in (dq, dk, dv))


RING_CASES = [("striped", True, "f32", 16, 4, 64), ("contiguous", True, "f32", 16, 4, 64),
              ("contiguous", False, "f32", 32, 2, 96), ("striped", True, "bf16", 128, 4, 1024),
              ("contiguous", True, "bf16", 64, 2, 512)]


@pytest.mark.parametrize("lay,causal,dtype,D,N,S", RING_CASES)
def test_ring_backward_matches_oracle(lay, causal, dtype, D, N, S):
    gh.say("ra_ring_backward", lay, causal, dtype, D, N, S)
    Hq, Hkv = 4, 2
    qn, kn, vn = gh.qkv_global(1, Hq, Hkv, S, D, dtype, seed=41)
    gn = ra_inputs.normal((1, Hq, S, D), 3, seed=41, dtype=dtype)
    qs, ks, vs, gs = (gh.shards_on_device(x, N, lay, dtype) for x in (qn, kn, vn, gn))
    o, lse, _ = gh.run_ring(qs, ks, vs, N, 0, lay, causal)
    dq = torch.empty(qs.shape, device="cuda")
    dk = torch.empty(ks.shape, device="cuda")
    dv = torch.empty(ks.shape, device="cuda")
    st = ra.ra_ring_backward(qs, ks, vs, o, gs, lse, dq, dk, dv, n_pos=N, layout=lay, causal=causal, stats=True)
    torch.cuda.synchronize()
    assert st["block_launches"] == N * N - st["blocks_skipped"]
    dq_g, dk_g, dv_g = (torch.empty(1, t.shape[2], S, D, device="cuda") for t in (dq, dk, dv))
    for sh, full in ((dq, dq_g), (dk, dk_g), (dv, dv_g)):
        ra.ra_stripe_permute(sh, full, layout=lay, inverse=True, n_pos=N)
    torch.cuda.synchronize()
    want = oracle.attention_grads(qn, kn, vn, gn, causal=causal)
    # the backward consumes the GPU forward's bf16 output and fp32 lse, so bf16
    # rings carry that rounding too (in dQ through delta = dO . O)
    tol = gh.GRAD_RTOL["bf16"] if dtype == "bf16" else gh.GRAD_RTOL["fp32"]
    extra = _dq_delta_extra(qn, kn, vn, gn, causal) if dtype == "bf16" else None
    for name, got, ref, ex in (("dq", dq_g, want[0], extra), ("dk", dk_g, want[1], None),
                               ("dv", dv_g, want[2], None)):
        gh.grad_close(gh.to_host_f64(got), ref, tol, name, extra=ex)


@pytest.mark.parametrize("lay", ["contiguous", "striped"])
def test_ring_backward_streams_are_bit_identical_to_one_stream(lay):
    """The positions of a lockstep step run on several library streams, joined
    after every step, so every dK / dV block still accumulates its shares in
    step order: the gradients equal the one-stream run bit for bit."""
    gh.say("ra_ring_backward streams", lay)
    S, N, Hq, Hkv, D = 4096, 4, 4, 2, 128
    qn, kn, vn = gh.qkv_global(1, Hq, Hkv, S, D, "bf16", seed=43)
    gn = ra_inputs.normal((1, Hq, S, D), 3, seed=43)
    qs, ks, vs, gs = (gh.shards_on_device(x, N, lay, "bf16") for x in (qn, kn, vn, gn))
    o, lse, _ = gh.run_ring(qs, ks, vs, N, 0, lay, True)
    outs = []
    for n_streams in (1, 0, 3):
        grads = [torch.full(t.shape, float("nan"), device="cuda") for t in (qs, ks, ks)]
        ra.ra_ring_backward(qs, ks, vs, o, gs, lse, *grads, n_pos=N, layout=lay, causal=True, n_streams=n_streams)
        torch.cuda.synchronize()
        outs.append(grads)
    for other in outs[1:]:
        for a_, b_ in zip(outs[0], other):
            assert torch.equal(a_, b_)


def test_mfma_backward_runs_and_differs_from_vector_path():
    """bf16 head_dim 128 takes the MFMA kernels (P and dS rounded to bf16 for the
    products); the vector-ALU path keeps them in fp32.  Both match the oracle,
    and they are not bit-identical -- so the MFMA path really ran."""
    gh.say("ra_block_attn_bwd mfma vs simt")
    B, Hq, Hkv, n, D = 1, 2, 1, 256, 128
    qn = ra_inputs.normal((B, Hq, n, D), 0, seed=51)
    kn, vn = (ra_inputs.normal((B, Hkv, n, D), s, seed=51) for s in (1, 2))
    gn = ra_inputs.normal((B, Hq, n, D), 3, seed=51)
    q, k, v, g = (gh.to_device(x, "bf16") for x in (qn, kn, vn, gn))
    pos = np.arange(n)
    lse = np.empty((B, Hq, n))
    dlt = np.empty((B, Hq, n))
    for h in range(Hq):
        r = oracle.grads(qn[0, h], kn[0, 0], vn[0, 0], gn[0, h], q_pos=pos, causal=True, key_grads=False)
        lse[0, h], dlt[0, h] = r["lse"], r["delta"]
    lse_d = torch.from_numpy(lse.astype(np.float32)).cuda()
    dlt_d = torch.from_numpy(dlt.astype(np.float32)).cuda()
    outs = []
    for flags in (0, ra.RA_BLOCK_FORCE_SIMT):
        dq = torch.zeros(B, Hq, n, D, device="cuda")
        dk = torch.zeros(B, Hkv, n, D, device="cuda")
        dv = torch.zeros(B, Hkv, n, D, device="cuda")
        ra.ra_block_attn_bwd(q, k, v, g, lse_d, dlt_d, dq, dk, dv, causal=True, flags=flags)
        outs.append((dq, dk, dv))
    torch.cuda.synchronize()
    for a_, b_ in zip(*outs):
        assert not torch.equal(a_, b_)
        gh.grad_close(gh.to_host_f64(a_), gh.to_host_f64(b_), gh.GRAD_RTOL["bf16"], "mfma vs vector path")


def test_ring_backward_gqa_moderate_size_all_gradients():
    gh.say("ra_ring_backward gqa 4096")
    S, N, Hq, Hkv, D = 4096, 2, 4, 2, 128
    qn, kn, vn = gh.qkv_global(1, Hq, Hkv, S, D, "bf16", seed=61)
    gn = ra_inputs.normal((1, Hq, S, D), 3, seed=61)
    qs, ks, vs, gs = (gh.shards_on_device(x, N, "striped", "bf16") for x in (qn, kn, vn, gn))
    o, lse, _ = gh.run_ring(qs, ks, vs, N, 0, "striped", True)
    dq = torch.empty(qs.shape, device="cuda")
    dk = torch.empty(ks.shape, device="cuda")
    dv = torch.empty(ks.shape, device="cuda")
    ra.ra_ring_backward(qs, ks, vs, o, gs, lse, dq, dk, dv, n_pos=N, layout="striped", causal=True)
    outs = []
    for sh in (dq, dk, dv):
        full = torch.empty(1, sh.shape[2], S, D, device="cuda")
        ra.ra_stripe_permute(sh, full, layout="striped", inverse=True, n_pos=N)
        outs.append(full)
    torch.cuda.synchronize()
    want = oracle.attention_grads(qn, kn, vn, gn, causal=True)
    extras = (_dq_delta_extra(qn, kn, vn, gn, True), None, None)
    for name, got, ref, ex in zip(("dq", "dk", "dv"), outs, want, extras):
        gh.grad_close(gh.to_host_f64(got), ref, gh.GRAD_RTOL["bf16"], name, extra=ex)


@pytest.mark.timeout(900)
def test_backward_256k_share_sampled_rows_and_identities():
    """The causal 256K striped share at full size, elementwise against the oracle:
    dQ on 1024 distinct sampled rows of the share (all heads); dK and dV on 256
    sampled keys of two heads drawn from every key/value block, among the keys of
    the last 4096 tokens of the sequence -- the share's rows that see them are
    its last 512, whose full-key-set lse and delta the oracle computes (about
    1.3e8 visible pairs a head).  Plus identities that hold at any size: per
    key/value head, sum_c dK_c = 0, sum_c dV_c = sum_t dO_t (t over the share's
    rows), and <Q, dQ> over the group's query heads = <K, dK>."""
    gh.say("ra_ring_backward 256k share")
    B, H, S, D, N, i = 1, 8, 262144, 128, 8, 7
    sb = S // N
    kn = ra_inputs.normal((B, H, S, D), 1, seed=0)
    vn = ra_inputs.normal((B, H, S, D), 2, seed=0)
    qn = ra_inputs.normal((B, H, S, D), 0, seed=0, t0=i, t_stride=N, n_rows=sb)
    gn = ra_inputs.normal((B, H, S, D), 3, seed=0, t0=i, t_stride=N, n_rows=sb)
    ks, vs = (gh.shards_on_device(x, N, "striped", "bf16") for x in (kn, vn))
    q, g = gh.to_device(qn, "bf16")[None], gh.to_device(gn, "bf16")[None]
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:4], device="cuda")
    ra.ra_ring_forward(q, ks, vs, o, lse, n_pos=N, first_pos=i, layout="striped", causal=True)
    dq = torch.empty(q.shape, device="cuda")
    dk = torch.empty(ks.shape, device="cuda")
    dv = torch.empty(ks.shape, device="cuda")
    st = ra.ra_ring_backward(q, ks, vs, o, g, lse, dq, dk, dv, n_pos=N, first_pos=i, layout="striped",
                             causal=True, stats=True)
    torch.cuda.synchronize()
    assert st["block_launches"] == N and st["blocks_skipped"] == 0
    rtol = gh.GRAD_RTOL["bf16"]
    # dQ: 1024 distinct rows of the share
    sh, stt = ra_inputs.sample_rows(S, N, 1024, heads=H, seed=1, share=i, layout="striped")
    assert len(set(zip(sh.tolist(), stt.tolist()))) == 1024
    rr = (stt - i) // N
    got = gh.to_host_f64(dq[0, 0][torch.as_tensor(sh, device="cuda"), torch.as_tensor(rr, device="cuda")])
    want = np.empty_like(got)
    o_ref = np.empty_like(got)
    pk_ref = np.empty_like(got)
    for h in np.unique(sh):
        idx = np.nonzero(sh == h)[0]
        r = oracle.grads(qn[0, h][rr[idx]], kn[0, h], vn[0, h], gn[0, h][rr[idx]], q_pos=stt[idx], causal=True,
                         key_grads=False)
        want[idx] = r["dq"]
        o_ref[idx] = oracle.rows(qn[0, h][rr[idx]], kn[0, h], vn[0, h], q_pos=stt[idx], causal=True)["o"]
        pk_ref[idx] = oracle.rows(qn[0, h][rr[idx]], kn[0, h], kn[0, h], q_pos=stt[idx], causal=True)["o"]
    extra = gh.dq_delta_bound(o_ref, pk_ref, gn[0][sh, rr], 1.0 / np.sqrt(D))
    gh.grad_close(got, want, rtol, "dq, 1024 sampled share rows", extra=extra)
    # dK, dV: sampled keys of the last 4096 tokens, every block j (local rows c >= sb - 512)
    rows_late = np.arange(sb - 512, sb)
    t_late = i + N * rows_late
    rng = np.random.Generator(np.random.PCG64(2))
    for h in (0, 5):
        full = oracle.grads(qn[0, h][rows_late], kn[0, h], vn[0, h], gn[0, h][rows_late], q_pos=t_late, causal=True,
                            key_grads=False)
        flat = rng.choice(N * 512, size=256, replace=False)
        jj, cc = flat // 512, sb - 512 + flat % 512
        tok = jj + N * cc
        share = oracle.grads(qn[0, h][rows_late], kn[0, h][tok], vn[0, h][tok], gn[0, h][rows_late], q_pos=t_late,
                             k_pos=tok, causal=True, lse=full["lse"], delta=full["delta"])
        sel_j, sel_c = torch.as_tensor(jj, device="cuda"), torch.as_tensor(cc, device="cuda")
        gh.grad_close(gh.to_host_f64(dk[sel_j, 0, h, sel_c]), share["dk"], rtol, f"dk head {h}, 256 keys")
        gh.grad_close(gh.to_host_f64(dv[sel_j, 0, h, sel_c]), share["dv"], rtol, f"dv head {h}, 256 keys")
    # identities per head
    dk_h = dk.double().sum(dim=(0, 3))[0]  # [H, D]: sum over positions and key rows
    dv_h = dv.double().sum(dim=(0, 3))[0]
    g_h = g.double().sum(dim=3)[0, 0]      # [H, D]
    assert float(torch.max(torch.abs(dk_h))) <= 1e-2 * float(dk.abs().double().sum(dim=(0, 3)).max())
    assert float(torch.max(torch.abs(dv_h - g_h))) <= 1e-2 * float(torch.max(torch.abs(g_h)) + 1.0)
    qd = (q.double() * dq.double()).sum(dim=(0, 3, 4))[0]         # [H]
    kd = (ks.double() * dk.double()).sum(dim=(0, 3, 4))[0]        # [H]
    scale = float(torch.max(torch.abs(qd)).item()) + 1.0
    assert float(torch.max(torch.abs(qd - kd))) <= 2e-2 * scale


@pytest.mark.timeout(900)
def test_backward_gqa_1m_share_sampled_rows():
    """The Llama-3-8B-shaped GQA share at full size (32 query heads on 8
    key/value heads, d 128, 1M tokens striped over 32 positions, position 31's
    share: 32768 queries against 32 blocks), elementwise against the oracle:
    dQ on 1024 distinct sampled rows of the share (all heads); dK and dV on 256
    sampled keys of key/value head 5, drawn from every block among the keys of
    the last 16384 tokens -- the share rows that see them are its last 512 of
    the head's four query heads, whose full-key-set lse and delta the oracle
    computes, and whose shares add up in each key's gradient.  Plus, per
    key/value head, sum_c dK_c = 0 and sum_c dV_c = the sum of dO over the
    group's query heads and the share's rows."""
    gh.say("ra_ring_backward gqa 1m share inputs")
    Hq, Hkv, S, D, N, i = 32, 8, 1 << 20, 128, 32, 31
    grp, sb = Hq // Hkv, S // N
    kn = ra_inputs.normal((1, Hkv, S, D), 1, seed=0, dtype="bf16")
    vn = ra_inputs.normal((1, Hkv, S, D), 2, seed=0, dtype="bf16")
    qn = ra_inputs.normal((1, Hq, S, D), 0, seed=0, dtype="bf16", t0=i, t_stride=N, n_rows=sb)
    gn = ra_inputs.normal((1, Hq, S, D), 3, seed=0, dtype="bf16", t0=i, t_stride=N, n_rows=sb)
    ks, vs = (gh.shards_on_device(x, N, "striped", "bf16") for x in (kn, vn))
    q, g = gh.to_device(qn, "bf16")[None], gh.to_device(gn, "bf16")[None]
    gh.say("ra_ring_backward gqa 1m share")
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:4], device="cuda")
    ra.ra_ring_forward(q, ks, vs, o, lse, n_pos=N, first_pos=i, layout="striped", causal=True)
    dq = torch.empty(q.shape, device="cuda")
    dk = torch.empty(ks.shape, device="cuda")
    dv = torch.empty(ks.shape, device="cuda")
    st = ra.ra_ring_backward(q, ks, vs, o, g, lse, dq, dk, dv, n_pos=N, first_pos=i, layout="striped",
                             causal=True, stats=True)
    torch.cuda.synchronize()
    assert st["block_launches"] == N and st["blocks_skipped"] == 0
    rtol = gh.GRAD_RTOL["bf16"]
    gh.say("ra_ring_backward gqa 1m share: dq rows")
    sh, stt = ra_inputs.sample_rows(S, N, 1024, heads=Hq, seed=1, share=i, layout="striped")
    assert len(set(zip(sh.tolist(), stt.tolist()))) == 1024
    rr = (stt - i) // N
    got = gh.to_host_f64(dq[0, 0][torch.as_tensor(sh, device="cuda"), torch.as_tensor(rr, device="cuda")])
    want, o_ref, pk_ref = np.empty_like(got), np.empty_like(got), np.empty_like(got)
    for h in np.unique(sh):
        idx = np.nonzero(sh == h)[0]
        kv = h // grp
        r = oracle.grads(qn[0, h][rr[idx]], kn[0, kv], vn[0, kv], gn[0, h][rr[idx]], q_pos=stt[idx], causal=True,
                         key_grads=False)
        want[idx] = r["dq"]
        o_ref[idx] = oracle.rows(qn[0, h][rr[idx]], kn[0, kv], vn[0, kv], q_pos=stt[idx], causal=True)["o"]
        pk_ref[idx] = oracle.rows(qn[0, h][rr[idx]], kn[0, kv], kn[0, kv], q_pos=stt[idx], causal=True)["o"]
    extra = gh.dq_delta_bound(o_ref, pk_ref, gn[0][sh, rr], 1.0 / np.sqrt(D))
    gh.grad_close(got, want, rtol, "dq, 1024 sampled share rows", extra=extra)
    gh.say("ra_ring_backward gqa 1m share: dk, dv keys")
    kv = 5
    rows_late = np.arange(sb - 512, sb)
    t_late = i + N * rows_late
    rng = np.random.Generator(np.random.PCG64(2))
    flat = rng.choice(N * 512, size=256, replace=False)
    jj, cc = flat // 512, sb - 512 + flat % 512
    tok = jj + N * cc
    want_dk = np.zeros((256, D))
    want_dv = np.zeros((256, D))
    for h in range(kv * grp, (kv + 1) * grp):
        full = oracle.grads(qn[0, h][rows_late], kn[0, kv], vn[0, kv], gn[0, h][rows_late], q_pos=t_late,
                            causal=True, key_grads=False)
        part = oracle.grads(qn[0, h][rows_late], kn[0, kv][tok], vn[0, kv][tok], gn[0, h][rows_late], q_pos=t_late,
                            k_pos=tok, causal=True, lse=full["lse"], delta=full["delta"])
        want_dk += part["dk"]
        want_dv += part["dv"]
    sel_j, sel_c = torch.as_tensor(jj, device="cuda"), torch.as_tensor(cc, device="cuda")
    gh.grad_close(gh.to_host_f64(dk[sel_j, 0, kv, sel_c]), want_dk, rtol, f"dk kv head {kv}, 256 keys")
    gh.grad_close(gh.to_host_f64(dv[sel_j, 0, kv, sel_c]), want_dv, rtol, f"dv kv head {kv}, 256 keys")
    # identities per key/value head
    dk_h = dk.double().sum(dim=(0, 3))[0]  # [Hkv, D]: over blocks and key rows
    dv_h = dv.double().sum(dim=(0, 3))[0]
    g_h = g.double().sum(dim=3)[0, 0].view(Hkv, grp, D).sum(dim=1)  # over the group's heads and the share's rows
    assert float(torch.max(torch.abs(dk_h))) <= 1e-2 * float(dk.abs().double().sum(dim=(0, 3)).max())
    assert float(torch.max(torch.abs(dv_h - g_h))) <= 1e-2 * float(torch.max(torch.abs(g_h)) + 1.0)


@pytest.mark.parametrize("lay", ["striped", "contiguous"])
def test_batch2_gqa4_ring_forward_and_backward(lay):
    """Batch 2, 8 query heads on 2 key/value heads, d 64: forward output and lse
    on every row, and all three gradients, against the oracle."""
    gh.say("ring batch 2 gqa 4", lay)
    B, Hq, Hkv, S, D, N = 2, 8, 2, 512, 64, 4
    qn, kn, vn = gh.qkv_global(B, Hq, Hkv, S, D, "bf16", seed=71)
    gn = ra_inputs.normal((B, Hq, S, D), 3, seed=71)
    qs, ks, vs, gs = (gh.shards_on_device(x, N, lay, "bf16") for x in (qn, kn, vn, gn))
    o, lse, _ = gh.run_ring(qs, ks, vs, N, 0, lay, True)
    o_full = torch.empty(B, Hq, S, D, device="cuda", dtype=torch.bfloat16)
    ra.ra_stripe_permute(o, o_full, layout=lay, inverse=True, n_pos=N)
    lse_full = torch.empty(B, Hq, S, 1, device="cuda")
    ra.ra_stripe_permute(lse[..., None].contiguous(), lse_full, layout=lay, inverse=True, n_pos=N)
    dq = torch.empty(qs.shape, device="cuda")
    dk = torch.empty(ks.shape, device="cuda")
    dv = torch.empty(ks.shape, device="cuda")
    ra.ra_ring_backward(qs, ks, vs, o, gs, lse, dq, dk, dv, n_pos=N, layout=lay, causal=True)
    grads = []
    for sh in (dq, dk, dv):
        full = torch.empty(B, sh.shape[2], S, D, device="cuda")
        ra.ra_stripe_permute(sh, full, layout=lay, inverse=True, n_pos=N)
        grads.append(full)
    torch.cuda.synchronize()
    want_o, want_lse = oracle.attention(qn, kn, vn, causal=True)
    assert np.max(np.abs(gh.to_host_f64(o_full) - want_o)) <= gh.TOL["bf16"]["o"]
    assert np.max(np.abs(gh.to_host_f64(lse_full)[..., 0] - want_lse)) <= gh.TOL["bf16"]["lse"]
    want = oracle.attention_grads(qn, kn, vn, gn, causal=True)
    extras = (_dq_delta_extra(qn, kn, vn, gn, True), None, None)
    for name, got, ref, ex in zip(("dq", "dk", "dv"), grads, want, extras):
        gh.grad_close(gh.to_host_f64(got), ref, gh.GRAD_RTOL["bf16"], name, extra=ex)


@pytest.mark.timeout(900)
def test_backward_identical_keys_closed_form_at_scale():
    """Every key of a head equal (k_c = k0) over the 256K-token striped ring:
    the causal softmax of row t is uniform, p_tc = 1 / (t + 1) for c <= t, so
        dV_c = sum over t >= c of dO_t / (t + 1)     (every key, all heads),
    and dS_tc = p_tc dO_t . (v_c - O_t) sums to zero over c, so dQ_t = 0 up to
    rounding (every row).  The reference is a float64 suffix sum on the host."""
    B, H, S, D, N = 1, 8, 262144, 128, 8
    gh.say("ra_ring_backward identical keys 256k")
    qn = ra_inputs.normal((B, H, S, D), ra_inputs.STREAM_Q, seed=29, dtype="bf16")
    k0 = ra_inputs.normal((B, H, 1, D), ra_inputs.STREAM_K, seed=29, dtype="bf16")
    vn = ra_inputs.normal((B, H, S, D), ra_inputs.STREAM_V, seed=29, dtype="bf16")
    gn = ra_inputs.normal((B, H, S, D), 3, seed=29, dtype="bf16")
    kn = np.broadcast_to(k0, (B, H, S, D))
    qs, ks, vs, gs = (gh.shards_on_device(x, N, "striped", "bf16") for x in (qn, kn, vn, gn))
    o, lse, _ = gh.run_ring(qs, ks, vs, N, 0, "striped", True)
    dq = torch.empty(qs.shape, device="cuda")
    dk = torch.empty(ks.shape, device="cuda")
    dv = torch.empty(ks.shape, device="cuda")
    ra.ra_ring_backward(qs, ks, vs, o, gs, lse, dq, dk, dv, n_pos=N, layout="striped", causal=True)
    full = {}
    for name, sh in (("dq", dq), ("dv", dv)):
        full[name] = torch.empty(B, H, S, D, device="cuda")
        ra.ra_stripe_permute(sh, full[name], layout="striped", inverse=True, n_pos=N)
    torch.cuda.synchronize()
    inv = 1.0 / np.arange(1, S + 1, dtype=np.float64)
    for h in range(H):
        g = ra_inputs.bf16_to_f32(gn[0, h]).astype(np.float64) * inv[:, None]
        want_dv = np.cumsum(g[::-1], axis=0)[::-1]
        gh.grad_close(gh.to_host_f64(full["dv"][0, h]), want_dv, gh.GRAD_RTOL["bf16"], f"dv head {h}")
        # dQ is zero exactly; what remains is rounding noise of the dS terms,
        # each about 2^-8 of |dS| <= 12 / (t + 1) times scale |k0|: an absolute bound
        _close(gh.to_host_f64(full["dq"][0, h]), np.zeros((S, D)), 2e-2, f"dq head {h}")
