"""GPU parity for wide query-head groups and ragged shards.

Grouped-query attention maps query head h to key/value head h // (Hq / Hkv)
(one key/value head per group of consecutive query heads).  These cases take
groups of 8 (one key/value head for all 8 query heads, i.e. multi-query
attention, and 16 query heads over 2 key/value heads) with shard lengths
that are not whole query or key tiles, on both kernels of the forward path
and on the backward:

* forward, 16 query heads over 2 key/value heads, 16000 tokens striped over 2
  positions (8000 a shard: 31 whole 256-row query tiles and a ragged one,
  62 whole 128-key tiles and a ragged one), causal: 512 query tiles a block
  launch, so the launches take the per-XCD work queues; 4096 distinct sampled
  rows against the oracle;
* forward and backward, multi-query (8 query heads, one key/value head),
  2000 tokens over 2 positions (ragged 1000-token shards), causal, head_dim
  128 (striped) and 64 (contiguous): every output row against the oracle and
  every element of dQ, dK, dV against the gradient oracle.

Tolerances as in the other parity tests (tests/gpu_helpers.py): 2e-2 on the
bf16 output, 1e-3 on the log-sum-exp; gradients elementwise with the bf16
relative factor and the delta term for dQ.
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


def test_group8_ragged_ring_forward_on_work_queues():
    B, Hq, Hkv, S, D, N, lay = 1, 16, 2, 16000, 128, 2, "striped"
    gh.say("ra_ring_forward group 8, ragged shards, work queues")
    sb = S // N
    assert (sb + 255) // 256 * Hq * B >= 2 * 256, "the launch must hold two query tiles per compute unit"
    qn, kn, vn = gh.qkv_global(B, Hq, Hkv, S, D, "bf16", seed=71)
    qs, ks, vs = (gh.shards_on_device(x, N, lay, "bf16") for x in (qn, kn, vn))
    o, lse, st = gh.run_ring(qs, ks, vs, N, 0, lay, True, stats=True)
    assert st["kv_splits"] in (0, 1)
    assert st["flops"] == 4 * D * Hq * S * (S + 1) // 2
    sh, stt = ra_inputs.sample_rows(S, N, 4096, heads=Hq, seed=1, layout=lay)
    assert len(set(zip(sh.tolist(), stt.tolist()))) == 4096
    gh.compare_rows(o, lse, qn, kn, vn, sh, stt, N, lay, 0, True, "bf16")


@pytest.mark.parametrize("D,lay", [(128, "striped"), (64, "contiguous")])
def test_multi_query_ragged_ring_forward_and_backward(D, lay):
    B, Hq, Hkv, S, N = 1, 8, 1, 2000, 2
    gh.say("ra_ring_forward/backward multi-query", D, lay)
    qn, kn, vn = gh.qkv_global(B, Hq, Hkv, S, D, "bf16", seed=73)
    gn = ra_inputs.normal((B, Hq, S, D), 3, seed=73)
    qs, ks, vs, gs = (gh.shards_on_device(x, N, lay, "bf16") for x in (qn, kn, vn, gn))
    o, lse, _ = gh.run_ring(qs, ks, vs, N, 0, lay, True)
    hh, tt = np.meshgrid(np.arange(Hq), np.arange(S), indexing="ij")
    gh.compare_rows(o, lse, qn, kn, vn, hh.ravel(), tt.ravel(), N, lay, 0, True, "bf16")

    dq = torch.empty(qs.shape, device="cuda")
    dk = torch.empty(ks.shape, device="cuda")
    dv = torch.empty(ks.shape, device="cuda")
    ra.ra_ring_backward(qs, ks, vs, o, gs, lse, dq, dk, dv, n_pos=N, layout=lay, causal=True)
    outs = []
    for sh in (dq, dk, dv):
        full = torch.empty(B, sh.shape[2], S, D, device="cuda")
        ra.ra_stripe_permute(sh, full, layout=lay, inverse=True, n_pos=N)
        outs.append(full)
    torch.cuda.synchronize()
    want = oracle.attention_grads(qn, kn, vn, gn, causal=True)
    o_ref, _ = oracle.attention(qn, kn, vn, causal=True)
    pk_ref, _ = oracle.attention(qn, kn, kn, causal=True)
    extras = (gh.dq_delta_bound(o_ref, pk_ref, gn, 1.0 / np.sqrt(D)), None, None)
    for name, got, ref, ex in zip(("dq", "dk", "dv"), outs, want, extras):
        gh.grad_close(gh.to_host_f64(got), ref, gh.GRAD_RTOL["bf16"], name, extra=ex)
