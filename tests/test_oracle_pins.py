"""Pins of the CPU fp64 oracle to facts outside itself (CPU only).

Each ``check_*`` takes an oracle library handle so that the same checks can be
run against deliberately broken copies of the oracle source (the mutation test
at the bottom): every planted mistake must make at least one pin fail.

Sources of the pins:
* the worked example printed by "Ring Attention" (Ultralytics glossary),
  section "How ring attention works" (tests/golden/page_ring_example.txt);
* special cases that reduce to a library routine (torch fp64 softmax /
  logsumexp), closed forms, and brute force on tiny inputs;
* the exactness claim of the same section (ring result == full attention for
  any visit order, causal or not, contiguous or striped).
"""
from __future__ import annotations

import os
import re
import shutil
import tempfile

import numpy as np
import pytest
import torch

import oracle
import ra_inputs
from oracle import layout, ring_steps
from tests.conftest import golden

TOL = 1e-12


def _rand(shape, seed, stream, dtype="f32", scale=1.0):
    return ra_inputs.normal(shape, stream, seed=seed, dtype=dtype, scale=scale)


def _torch_full(q, k, v, causal, scale=None):
    """Reference via torch fp64 library routines (softmax, logsumexp)."""
    q, k, v = (torch.from_numpy(np.asarray(a, dtype=np.float64)) for a in (q, k, v))
    sig = scale or 1.0 / np.sqrt(q.shape[-1])
    s = (q @ k.T) * sig
    if causal:
        S = s.shape[0]
        allowed = torch.ones(S, k.shape[0], dtype=torch.bool).tril()
        s = s.masked_fill(~allowed, float("-inf"))
    return (torch.softmax(s, dim=-1) @ v).numpy(), torch.logsumexp(s, dim=-1).numpy()


# --------------------------------------------------------------------------- checks
def check_page_example(lib):
    """The pages' four-device simulation: ring == full attention at atol 1e-5."""
    g = golden("page_ring_example.txt")
    n_dev, blk, dim = int(g["devices"]), int(g["block"]), int(g["dim"])
    torch.manual_seed(int(g["seed"]))
    q, k, v = (t.numpy() for t in torch.randn(3, n_dev * blk, dim))   # page-exact inputs
    ring32, biggest = ring_steps.ring_no_max(q, k, v, n_dev, dtype=np.float32)
    full = oracle.rows(q, k, v, lib=lib)["o"]
    assert f"{biggest[0]}x{biggest[1]}" == g["score_block_per_device"]
    assert f"{full.shape[0]}x{k.shape[0]}" == g["full_score_matrix"]
    matches = bool(np.all(np.abs(ring32 - full) <= float(g["allclose_atol"])))
    assert str(matches) == g["ring_matches_full_attention"]
    # the fp64 transcription of the same loop agrees to rounding
    r64, _ = ring_steps.ring_no_max(q, k, v, n_dev)
    assert np.max(np.abs(r64 - full)) <= TOL


def check_library_softmax(lib):
    """Equals torch fp64 softmax(q k^T / sqrt(d)) v and logsumexp, causal or not."""
    for causal in (False, True):
        for S, Sk, d in ((37, 37, 16), (5, 5, 64), (64, 64, 128)):
            q = _rand((1, 1, S, d), 11, 0)[0, 0]
            k = _rand((1, 1, Sk, d), 11, 1)[0, 0]
            v = _rand((1, 1, Sk, d), 11, 2)[0, 0]
            ref_o, ref_lse = _torch_full(q, k, v, causal)
            r = oracle.rows(q, k, v, q_pos=np.arange(S), causal=causal, lib=lib)
            assert np.max(np.abs(r["o"] - ref_o)) <= TOL
            assert np.max(np.abs(r["lse"] - ref_lse)) <= TOL
    # an explicit scale is honoured
    q, k, v = (_rand((1, 1, 9, 8), 3, s)[0, 0] for s in range(3))
    ref_o, ref_lse = _torch_full(q, k, v, False, scale=0.3)
    r = oracle.rows(q, k, v, scale=0.3, lib=lib)
    assert np.max(np.abs(r["o"] - ref_o)) <= TOL and np.max(np.abs(r["lse"] - ref_lse)) <= TOL


def check_bf16_inputs(lib):
    """bfloat16 bit patterns are widened exactly (same result as their f32 values)."""
    q, k, v = (_rand((1, 1, 20, 32), 5, s, dtype="bf16")[0, 0] for s in range(3))
    rb = oracle.rows(q, k, v, q_pos=np.arange(20), causal=True, lib=lib)
    qf, kf, vf = (ra_inputs.bf16_to_f32(a) for a in (q, k, v))
    ref_o, ref_lse = _torch_full(qf, kf, vf, True)
    assert np.max(np.abs(rb["o"] - ref_o)) <= TOL
    assert np.max(np.abs(rb["lse"] - ref_lse)) <= TOL


def check_rows_sum_to_one(lib):
    """With V = I (d = S) the output row is the softmax row: >= 0, sums to 1,
    and under the causal mask it is zero above the diagonal."""
    S = 24
    q = _rand((1, 1, S, S), 7, 0)[0, 0]
    k = _rand((1, 1, S, S), 7, 1)[0, 0]
    v = np.eye(S, dtype=np.float32)
    for causal in (False, True):
        p = oracle.rows(q, k, v, q_pos=np.arange(S), causal=causal, lib=lib)["o"]
        assert np.all(p >= 0)
        assert np.max(np.abs(p.sum(axis=1) - 1.0)) <= TOL
        if causal:
            assert np.all(np.triu(p, 1) == 0.0)
            assert p[0, 0] == 1.0


def check_identical_keys(lib):
    """All keys equal: uniform weights, O_t = mean of allowed v_c, lse = s + ln|C_t|."""
    S, d = 33, 16
    q = _rand((1, 1, S, d), 9, 0)[0, 0]
    k = np.repeat(_rand((1, 1, 1, d), 9, 1)[0, 0], S, axis=0)
    v = _rand((1, 1, S, d), 9, 2)[0, 0]
    s = (q.astype(np.float64) @ k[0].astype(np.float64)) / np.sqrt(d)
    for causal in (False, True):
        r = oracle.rows(q, k, v, q_pos=np.arange(S), causal=causal, lib=lib)
        n = np.arange(1, S + 1) if causal else np.full(S, S)
        mean = (np.cumsum(v.astype(np.float64), axis=0) / n[:, None] if causal
                else np.broadcast_to(v.astype(np.float64).mean(axis=0), (S, d)))
        assert np.max(np.abs(r["o"] - mean)) <= TOL
        assert np.max(np.abs(r["lse"] - (s + np.log(n)))) <= TOL


def check_zero_query_and_single_key(lib):
    """q = 0 gives lse_t = ln|C_t|; a single key gives O = v_0 and lse = s_00."""
    S, d = 17, 8
    q = np.zeros((S, d), dtype=np.float32)
    k, v = (_rand((1, 1, S, d), 4, s)[0, 0] for s in (1, 2))
    r = oracle.rows(q, k, v, q_pos=np.arange(S), causal=True, lib=lib)
    assert np.max(np.abs(r["lse"] - np.log(np.arange(1, S + 1)))) <= TOL
    q1, k1, v1 = (_rand((1, 1, 1, d), 4, s)[0, 0] for s in range(3))
    r1 = oracle.rows(q1, k1, v1, q_pos=np.zeros(1), causal=True, lib=lib)
    assert np.max(np.abs(r1["o"][0] - v1[0])) <= TOL
    s00 = float(q1[0].astype(np.float64) @ k1[0].astype(np.float64)) / np.sqrt(d)
    assert abs(r1["lse"][0] - s00) <= TOL
    assert r1["m"][0] == pytest.approx(s00, abs=TOL) and r1["l"][0] == 1.0


def check_brute_force_causal(lib):
    """Materialised S x S score matrix with -inf above the diagonal, tiny S."""
    for S in (1, 2, 3, 7, 8, 9, 16, 33):
        d = 8
        q, k, v = (_rand((1, 1, S, d), 100 + S, s)[0, 0].astype(np.float64) for s in range(3))
        o_bf = np.empty((S, d))
        lse_bf = np.empty(S)
        for t in range(S):
            row = np.array([(q[t] @ k[c]) / np.sqrt(d) if c <= t else -np.inf
                            for c in range(S)])
            mx = row.max()
            w = np.exp(row - mx)
            o_bf[t] = (w[:, None] * v).sum(axis=0) / w.sum()
            lse_bf[t] = mx + np.log(w.sum())
        r = oracle.rows(q.astype(np.float32), k.astype(np.float32), v.astype(np.float32),
                        q_pos=np.arange(S), causal=True, lib=lib)
        assert np.max(np.abs(r["o"] - o_bf)) <= TOL
        assert np.max(np.abs(r["lse"] - lse_bf)) <= TOL


def check_dominant_self_key(lib):
    """K = alpha * Q: the own key dominates, so causal O_t = v_t (pins the diagonal);
    with keys shifted by one the dominant key lies in the future and is masked."""
    S, d, alpha = 256, 64, 8.0
    shape = (1, 1, S, d)
    q = _rand(shape, 21, 0)[0, 0]
    k = _rand(shape, 21, 0, scale=alpha)[0, 0]             # same stream as q
    v = _rand(shape, 21, 2)[0, 0].astype(np.float64)
    pos = np.arange(S)
    r = oracle.rows(q, k, v.astype(np.float32), q_pos=pos, causal=True, lib=lib)
    assert np.max(np.abs(r["o"] - v)) <= 1e-4
    # shifted: key c is alpha * q_{c-1}, so row t's dominant key is c = t + 1
    ks = ra_inputs.normal(shape, 0, seed=21, dtype="f32", t0=-1, scale=alpha)[0, 0]
    rs = oracle.rows(q, ks, v.astype(np.float32), q_pos=pos, causal=False, lib=lib)
    assert np.max(np.abs(rs["o"][:-1] - v[1:])) <= 1e-4
    rc = oracle.rows(q, ks, v.astype(np.float32), q_pos=pos, causal=True, lib=lib)
    assert np.min(np.max(np.abs(rc["o"][1:-1] - v[2:]), axis=1)) > 0.1


def check_gqa(lib):
    """Grouped heads equal multi-head attention on repeat-interleaved K/V."""
    B, Hq, Hkv, S, d = 2, 4, 2, 12, 16
    q = _rand((B, Hq, S, d), 31, 0)
    k = _rand((B, Hkv, S, d), 31, 1)
    v = _rand((B, Hkv, S, d), 31, 2)
    o, lse = oracle.attention(q, k, v, causal=True, lib=lib)
    o2, lse2 = oracle.attention(q, np.repeat(k, 2, axis=1), np.repeat(v, 2, axis=1),
                                causal=True, lib=lib)
    assert np.max(np.abs(o - o2)) == 0.0 and np.max(np.abs(lse - lse2)) == 0.0
    for b in range(B):
        for h in range(Hq):
            ro, rl = _torch_full(q[b, h], k[b, h // 2], v[b, h // 2], True)
            assert np.max(np.abs(o[b, h] - ro)) <= TOL and np.max(np.abs(lse[b, h] - rl)) <= TOL
    # the row-sampled path gives the same rows
    sb, sh, st = np.array([0, 1, 1]), np.array([3, 0, 2]), np.array([0, 11, 5])
    os_, ls_ = oracle.attention(q, k, v, causal=True, sel_b=sb, sel_h=sh, sel_t=st, lib=lib)
    assert np.max(np.abs(os_ - o[sb, sh, st])) == 0.0 and np.max(np.abs(ls_ - lse[sb, sh, st])) == 0.0


def check_ring_equals_full(lib):
    """The ring (online max + merge) equals the oracle for any visit order,
    causal or not, contiguous or striped."""
    rng = np.random.Generator(np.random.PCG64(5))
    S, d = 48, 16
    q, k, v = (_rand((1, 1, S, d), 41, s)[0, 0] for s in range(3))
    for n_dev in (1, 2, 4, 8):
        for causal in (False, True):
            full = oracle.rows(q, k, v, q_pos=np.arange(S), causal=causal, lib=lib)
            for lay in ("contiguous", "striped"):
                for order in (None, list(rng.permutation(n_dev))):
                    o, lse = ring_steps.ring_online(q, k, v, n_dev, causal, lay, order)
                    assert np.max(np.abs(o - full["o"])) <= TOL
                    assert np.max(np.abs(lse - full["lse"])) <= TOL
        order = list(rng.permutation(n_dev))
        nm, _ = ring_steps.ring_no_max(q, k, v, n_dev, visit_order=order)
        assert np.max(np.abs(nm - oracle.rows(q, k, v, lib=lib)["o"])) <= TOL


def check_partial_and_merge(lib):
    """The (m, l, numerator) partial of a union of key sets is the merge of the
    partials of its parts; an empty key set is the merge identity."""
    S, d = 40, 16
    q, k, v = (_rand((1, 1, S, d), 51, s)[0, 0] for s in range(3))
    pos = np.arange(S)
    whole = oracle.rows(q, k, v, q_pos=pos, causal=True, lib=lib)
    a = oracle.rows(q, k[:13], v[:13], q_pos=pos, k_pos=pos[:13], causal=True, lib=lib)
    b = oracle.rows(q, k[13:], v[13:], q_pos=pos, k_pos=pos[13:], causal=True, lib=lib)
    m, l, num = ring_steps.merge((a["m"], a["l"], a["o_num"]), (b["m"], b["l"], b["o_num"]))
    assert np.array_equal(m, whole["m"])
    assert np.max(np.abs(l - whole["l"])) <= TOL and np.max(np.abs(num - whole["o_num"])) <= TOL
    # rows 0..12 see no key of part b: m = -inf, l = 0, numerator = 0
    assert np.all(np.isneginf(b["m"][:13])) and np.all(b["l"][:13] == 0)
    assert np.all(b["o_num"][:13] == 0) and np.all(np.isneginf(b["lse"][:13]))


CHECKS = [check_page_example, check_library_softmax, check_bf16_inputs, check_rows_sum_to_one,
          check_identical_keys, check_zero_query_and_single_key, check_brute_force_causal,
          check_dominant_self_key, check_gqa, check_ring_equals_full, check_partial_and_merge]


@pytest.mark.parametrize("check", CHECKS, ids=[c.__name__ for c in CHECKS])
def test_oracle_pin(check):
    check(oracle.load())


def test_layout_maps():
    """Contiguous: device i holds [i*Sb, (i+1)*Sb); striped: tokens i, i+N, ...;
    every token lands exactly once; shards -> tokens is the identity."""
    S, n = 24, 4
    for lay in ("contiguous", "striped"):
        seen = np.concatenate([layout.tokens_of(i, S, n, lay) for i in range(n)])
        assert sorted(seen.tolist()) == list(range(S))
    assert layout.tokens_of(2, S, n, "contiguous").tolist() == list(range(12, 18))
    assert layout.tokens_of(1, S, n, "striped").tolist() == list(range(1, S, n))
    x = np.arange(2 * 3 * S * 5).reshape(2, 3, S, 5)
    for lay in ("contiguous", "striped"):
        y = layout.to_shards(x, n, lay)
        assert np.array_equal(layout.from_shards(y, lay), x)
    y = layout.to_shards(x, n, "striped")
    assert np.array_equal(y[3, :, :, 2], x[:, :, 3 + 2 * n])


# --------------------------------------------------------------------------- mutations
MUTATIONS = {
    "dropped_scale": ("s[c] = scale * dot;", "s[c] = dot;"),
    "diagonal_excluded": ("pc <= q_pos[r]", "pc < q_pos[r]"),
    "future_allowed": ("pc <= q_pos[r]", "pc <= q_pos[r] + 1"),
    "wrong_exp_sign": ("const double w = exp(s[c] - M);", "const double w = exp(s[c] + M);"),
    "value_is_key": ("num[j] += w * load_elem(v,", "num[j] += w * load_elem(k,"),
    "lse_without_max": ("M + log(Z)", "log(Z)"),
    "max_is_min": ("if (s[c] > M) M = s[c];", "if (M == -INFINITY || s[c] < M) M = s[c];"),
    "bf16_widen_wrong": ("<< 16;", "<< 15;"),
    "unnormalised_output": ("num[j] / Z", "num[j]"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_oracle_mistake(name):
    """A plausible mistake planted in a copy of the oracle source must fail a pin."""
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    src = open(os.path.join(os.path.dirname(oracle.__file__), "attention_oracle.c")).read()
    old, new = MUTATIONS[name]
    assert src.count(old) >= 1, f"mutation anchor missing: {old}"
    mutated = src.replace(old, new)
    with tempfile.TemporaryDirectory() as tmp:
        path = os.path.join(tmp, "mutant.c")
        with open(path, "w") as f:
            f.write(mutated)
        lib = oracle.load(oracle.build(src=path, out=os.path.join(tmp, f"lib_{name}.so")))
        failures = 0
        for check in CHECKS:
            try:
                with np.errstate(all="ignore"):
                    check(lib)
            except (AssertionError, RuntimeError, ValueError, FloatingPointError):
                failures += 1
        assert failures > 0, f"no pin caught the planted mistake {name!r}"
