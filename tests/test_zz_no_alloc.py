"""ra_ring_forward_noalloc: the ring forward with the library's own device
scratch, for callers that cannot allocate.  Two calls in a row, the second on
a smaller input, each against ra_ring_forward on one stream (same kernels, same
order: identical bits) and against the fp64 oracle; device memory in use does
not change across the calls."""
import numpy as np
import pytest
import torch

import ra_inputs
import ring_attention_step_amd as ra
from ring_attention_step_amd import _binding as B
from tests import gpu_helpers as gh

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ra.load_library()
    yield
    torch.cuda.synchronize()


def _case(B_, Hq, Hkv, S, D, N, lay, causal, first, n_run, seed):
    qn, kn, vn = gh.qkv_global(B_, Hq, Hkv, S, D, "bf16", seed=seed)
    qs_all = gh.shards_on_device(qn, N, lay, "bf16")
    ks = gh.shards_on_device(kn, N, lay, "bf16")
    vs = gh.shards_on_device(vn, N, lay, "bf16")
    return (qn, kn, vn), qs_all[first:first + n_run].contiguous(), ks, vs


@pytest.mark.timeout(600)
def test_noalloc_matches_ring_forward_twice_second_smaller():
    # first: one position's share of the causal 256K-token striped ring (8 heads,
    # head_dim 128): work queues and the fused running state, 130 MiB of scratch;
    # second, smaller: the non-causal 4K ring (head_dim 64, both positions), whose
    # launches split keys into ranges with partials in the scratch
    cases = [dict(B_=1, Hq=8, Hkv=8, S=262144, D=128, N=8, lay="striped", causal=True, first=7, n_run=1, seed=3),
             dict(B_=1, Hq=4, Hkv=4, S=4096, D=64, N=2, lay="contiguous", causal=False, first=0, n_run=2, seed=4)]
    # set-up: the first call on a device looks the scratch array up, and the
    # HIP runtime backs it with device memory then; later calls allocate nothing
    (_, qs0, ks0, vs0) = _case(1, 2, 2, 512, 64, 2, "contiguous", False, 0, 2, 5)
    B.ra_ring_forward_noalloc(qs0, ks0, vs0, torch.empty_like(qs0), None, n_pos=2)
    torch.cuda.synchronize()
    sizes = []
    for c in cases:
        gh.say("ra_ring_forward_noalloc", c)
        (qn, kn, vn), qs, ks, vs = _case(**c)
        kw = dict(n_pos=c["N"], first_pos=c["first"], layout=c["lay"], causal=c["causal"])
        desc = ra.ring_desc(qs, ks, n_streams=1, **kw)
        sizes.append(ra.ra_ring_workspace_size(desc))
        assert sizes[-1] <= B.ra_ring_noalloc_max_bytes()
        o_ref = torch.empty_like(qs)
        lse_ref = torch.empty(qs.shape[:4], device="cuda")
        ra.ra_ring_forward(qs, ks, vs, o_ref, lse_ref, n_streams=1, **kw)
        o = torch.full_like(qs, float("nan"))
        lse = torch.full(qs.shape[:4], float("nan"), device="cuda")
        torch.cuda.synchronize()
        free_before = torch.cuda.mem_get_info()[0]
        B.ra_ring_forward_noalloc(qs, ks, vs, o, lse, **kw)
        torch.cuda.synchronize()
        assert torch.cuda.mem_get_info()[0] == free_before  # nothing allocated on the device
        assert torch.equal(o, o_ref) and torch.equal(lse, lse_ref)
        # and the oracle, on 512 distinct rows of the computed positions
        if c["n_run"] == 1:
            sh, st = ra_inputs.sample_rows(c["S"], c["N"], 512, heads=c["Hq"], seed=1, share=c["first"],
                                           layout=c["lay"])
        else:
            sh, st = ra_inputs.sample_rows(c["S"], c["N"], 512, heads=c["Hq"], seed=1)
        gh.compare_rows(o, lse, qn, kn, vn, sh, st, c["N"], c["lay"], c["first"], c["causal"], "bf16")
        del qs, ks, vs, o_ref, o
    assert sizes[1] < sizes[0]


def test_noalloc_refusals():
    """Refused before anything is launched: shapes whose scratch exceeds the
    array, timing stats and emulated copies (they need library events)."""
    q = torch.empty(1, 1, 32, 32768, 128, dtype=torch.bfloat16, device="cuda")
    k = torch.empty(32, 1, 8, 32768, 128, dtype=torch.bfloat16, device="cuda")
    o = torch.empty_like(q)
    with pytest.raises(ra.RAError) as e:
        B.ra_ring_forward_noalloc(q, k, k, o, None, n_pos=32, first_pos=31, layout="striped", causal=True)
    assert e.value.status == B.RA_ERR_WORKSPACE
    q2 = torch.empty(1, 1, 2, 256, 64, dtype=torch.bfloat16, device="cuda")
    k2 = torch.empty(2, 1, 2, 256, 64, dtype=torch.bfloat16, device="cuda")
    d = ra.ring_desc(q2, k2, n_pos=2, emulate_copy=True)
    rc = B.load_library().ra_ring_forward_noalloc(d, B._ptr(q2), B._ptr(k2), B._ptr(k2), B._ptr(torch.empty_like(q2)),
                                                 None, None)
    assert rc == B.RA_ERR_UNSUPPORTED
