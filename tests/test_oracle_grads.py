"""Pins of the fp64 gradient oracle (``oracle.grads``) -- CPU only.

The pages run attention's backward pass: "Context Parallelism" (Ultralytics
glossary), section "Practical use and trade-offs", marks q, k, v as requiring
gradients and back-propagates mean(O^2) through the causal attention.  The
oracle evaluates the chain-rule definitions directly; these checks tie it to
things other than itself:

* torch autograd in fp64 on the same inputs (a library routine), causal and
  not, including the pages' own loss mean(O^2);
* central finite differences of the forward oracle (itself pinned in
  test_oracle_pins.py) -- independent of any derivative formula;
* identities that hold at any size: per head sum_c dK_c = 0,
  sum_c dV_c = sum_t dO_t, <Q, dQ> = <K, dK>;
* one key block's share given the full-key-set lse and D sums to the whole;
* grouped-query attention equals repeated key/value heads;
* and, as for the forward oracle, plausible mistakes planted in copies of the
  source must each fail at least one check.
"""
import os
import shutil
import tempfile

import numpy as np
import pytest
import torch

import oracle


def _rand(shape, seed, dtype=np.float32, scale=1.0):
    rng = np.random.default_rng(seed)
    return (scale * rng.standard_normal(shape)).astype(dtype)


def _torch_grads(q, k, v, dout, causal, loss="dot"):
    """fp64 autograd of O = softmax(q k^T / sqrt(d) masked) v; loss = sum(O * dout) or mean(O^2)."""
    qt, kt, vt = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    d = q.shape[-1]
    s = qt @ kt.transpose(-1, -2) / d ** 0.5
    if causal:
        n, m = s.shape[-2:]
        mask = torch.ones(n, m, dtype=torch.bool).tril()
        s = s.masked_fill(~mask, float("-inf"))
    o = torch.softmax(s, dim=-1) @ vt
    if loss == "dot":
        (o * torch.tensor(dout, dtype=torch.float64)).sum().backward()
    else:
        o.square().mean().backward()
    return o.detach().numpy(), qt.grad.numpy(), kt.grad.numpy(), vt.grad.numpy()


def check_torch_autograd(lib):
    for causal in (False, True):
        for n, d in ((13, 8), (32, 16)):
            q, k, v, do = (_rand((n, d), 10 * n + i) for i in range(4))
            _, gq, gk, gv = _torch_grads(q, k, v, do, causal)
            r = oracle.grads(q, k, v, do, q_pos=np.arange(n), causal=causal, lib=lib)
            for got, want in ((r["dq"], gq), (r["dk"], gk), (r["dv"], gv)):
                assert np.max(np.abs(got - want)) <= 1e-10 * max(1.0, np.max(np.abs(want)))


def check_page_loss(lib):
    """The pages' loss mean(O^2): dL/dO = 2 O / numel."""
    n, d = 24, 16
    q, k, v = (_rand((n, d), 70 + i) for i in range(3))
    o, gq, gk, gv = _torch_grads(q, k, v, None, True, loss="square_mean")
    fwd = oracle.rows(q, k, v, q_pos=np.arange(n), causal=True, lib=lib)
    assert np.max(np.abs(fwd["o"] - o)) < 1e-12
    do = (2.0 * fwd["o"] / o.size).astype(np.float32)  # the upstream gradient, in the inputs' dtype
    r = oracle.grads(q, k, v, do, q_pos=np.arange(n), causal=True, lib=lib)
    for got, want in ((r["dq"], gq), (r["dk"], gk), (r["dv"], gv)):
        assert np.max(np.abs(got - want)) <= 1e-6 * np.max(np.abs(want))


def check_finite_differences(lib):
    """d/dx of L = sum(O * dO) by central differences of the forward oracle."""
    n, d = 9, 6
    q, k, v, do = (_rand((n, d), 90 + i) for i in range(4))
    pos = np.arange(n)
    r = oracle.grads(q, k, v, do, q_pos=pos, causal=True, lib=lib)

    def loss(qq, kk, vv):
        f = oracle.rows(qq, kk, vv, q_pos=pos, causal=True, lib=lib)
        return float(np.sum(f["o"] * do.astype(np.float64)))

    rng = np.random.default_rng(5)
    for name, which in (("dq", 0), ("dk", 1), ("dv", 2)):
        for _ in range(6):
            i, j = int(rng.integers(0, n)), int(rng.integers(0, d))
            args = [q.copy(), k.copy(), v.copy()]
            x0 = args[which][i, j]
            plus, minus = [a.copy() for a in args], [a.copy() for a in args]
            plus[which][i, j] = np.float32(x0 + 1e-2)
            minus[which][i, j] = np.float32(x0 - 1e-2)
            h = float(plus[which][i, j]) - float(minus[which][i, j])  # the step actually taken
            fd = (loss(*plus) - loss(*minus)) / h
            assert abs(fd - r[name][i, j]) <= 2e-4 * max(1.0, abs(fd)), (name, i, j, fd, r[name][i, j])


def check_identities(lib):
    for causal in (False, True):
        n, d = 40, 16
        q, k, v, do = (_rand((n, d), 120 + i) for i in range(4))
        r = oracle.grads(q, k, v, do, q_pos=np.arange(n), causal=causal, lib=lib)
        assert np.max(np.abs(r["dk"].sum(0))) < 1e-11
        assert np.max(np.abs(r["dv"].sum(0) - do.astype(np.float64).sum(0))) < 1e-11
        lhs = np.sum(q.astype(np.float64) * r["dq"])
        rhs = np.sum(k.astype(np.float64) * r["dk"])
        assert abs(lhs - rhs) < 1e-10 * max(1.0, abs(lhs))
        # D = dO . O
        o = oracle.rows(q, k, v, q_pos=np.arange(n), causal=causal, lib=lib)["o"]
        assert np.max(np.abs(r["delta"] - np.sum(do.astype(np.float64) * o, axis=1))) < 1e-12


def check_block_shares(lib):
    """Sum over key blocks of each block's share (full-set lse, D) = the whole."""
    n, d, nb = 48, 8, 4
    q, k, v, do = (_rand((n, d), 150 + i) for i in range(4))
    pos = np.arange(n)
    for causal in (False, True):
        full = oracle.grads(q, k, v, do, q_pos=pos, causal=causal, lib=lib)
        dq = np.zeros_like(full["dq"])
        for b in range(nb):
            sl = slice(b * n // nb, (b + 1) * n // nb)
            part = oracle.grads(q, k[sl], v[sl], do, q_pos=pos, k_pos=pos[sl], causal=causal,
                                lse=full["lse"], delta=full["delta"], lib=lib)
            dq += part["dq"]
            assert np.max(np.abs(part["dk"] - full["dk"][sl])) < 1e-12
            assert np.max(np.abs(part["dv"] - full["dv"][sl])) < 1e-12
        assert np.max(np.abs(dq - full["dq"])) < 1e-12


def check_gqa(lib):
    B, Hq, Hkv, S, d = 1, 4, 2, 16, 8
    q, do = _rand((B, Hq, S, d), 180), _rand((B, Hq, S, d), 181)
    k, v = _rand((B, Hkv, S, d), 182), _rand((B, Hkv, S, d), 183)
    dq, dk, dv = oracle.attention_grads(q, k, v, do, causal=True, lib=lib)
    g = Hq // Hkv
    _, gq, gk, gv = _torch_grads(q[0], np.repeat(k[0], g, axis=0), np.repeat(v[0], g, axis=0), do[0], True)
    assert np.max(np.abs(dq[0] - gq)) < 1e-10
    assert np.max(np.abs(dk[0] - gk.reshape(Hkv, g, S, d).sum(1))) < 1e-10
    assert np.max(np.abs(dv[0] - gv.reshape(Hkv, g, S, d).sum(1))) < 1e-10


def check_bf16_and_empty_rows(lib):
    """bf16 inputs are widened exactly; a row with no allowed key has zero gradient."""
    n, d = 10, 8
    q32, k32, v32, do32 = (_rand((n, d), 200 + i) for i in range(4))
    to_bf = lambda x: (torch.tensor(x).bfloat16().view(torch.int16).numpy().view(np.uint16))
    qb, kb, vb, dob = (to_bf(x) for x in (q32, k32, v32, do32))
    wid = lambda x: torch.tensor(x.view(np.int16)).view(torch.bfloat16).float().numpy()
    r16 = oracle.grads(qb, kb, vb, dob, q_pos=np.arange(n), causal=True, lib=lib)
    r32 = oracle.grads(*(wid(x) for x in (qb, kb, vb, dob)), q_pos=np.arange(n), causal=True, lib=lib)
    for key in ("dq", "dk", "dv"):
        assert np.array_equal(r16[key], r32[key])
    # keys all after the queries: nothing allowed
    r = oracle.grads(q32, k32, v32, do32, q_pos=np.arange(n), k_pos=np.arange(n) + n, causal=True, lib=lib)
    assert np.all(r["dq"] == 0) and np.all(r["dk"] == 0) and np.all(r["dv"] == 0)
    assert np.all(np.isneginf(r["lse"]))


CHECKS = [check_torch_autograd, check_page_loss, check_finite_differences, check_identities,
          check_block_shares, check_gqa, check_bf16_and_empty_rows]


@pytest.mark.parametrize("check", CHECKS, ids=lambda c: c.__name__)
def test_grads_oracle_pin(check):
    check(oracle.load())


# --------------------------------------------------------------------------- mutations
# anchors lie inside ra_oracle_grads only
MUTATIONS = {
    "dq_dropped_scale": ("dq[r * d + j] = scale * acc[j];", "dq[r * d + j] = acc[j];"),
    "dk_dropped_scale": ("if (dk) dk[c * d + j] = scale * ak[j];", "if (dk) dk[c * d + j] = ak[j];"),
    "ds_sign": ("const double ds = p * (dp - delta[r]);", "const double ds = p * (dp + delta[r]);"),
    "dv_weighted_by_ds": ("av[j] += p * load_elem(dout,", "av[j] += ds * load_elem(dout,"),
    "dk_uses_dout": ("ak[j] += ds * load_elem(q,", "ak[j] += ds * load_elem(dout,"),
    "delta_unweighted": ("D += exp(s[c] - L) * dp;", "D += dp;"),
    "dq_unnormalised_p": ("const double p = exp(s[c] - L);", "const double p = exp(s[c] - M);"),
    "pass2_ignores_mask": ("if (causal && pc > q_pos[r]) continue;\n                    if (lse[r]",
                           "if (0 && causal && pc > q_pos[r]) continue;\n                    if (lse[r]"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_grad_pins_catch_planted_mistake(name):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    src = open(os.path.join(os.path.dirname(oracle.__file__), "attention_oracle.c")).read()
    old, new = MUTATIONS[name]
    assert src.count(old) == 1, f"mutation anchor must be unique: {old}"
    with tempfile.TemporaryDirectory() as tmp:
        path = os.path.join(tmp, "mutant.c")
        with open(path, "w") as f:
            f.write(src.replace(old, new))
        lib = oracle.load(oracle.build(src=path, out=os.path.join(tmp, f"lib_{name}.so")))
        failures = 0
        for check in CHECKS:
            try:
                with np.errstate(all="ignore"):
                    check(lib)
            except (AssertionError, RuntimeError, ValueError, FloatingPointError):
                failures += 1
        assert failures > 0, f"no pin caught the planted mistake {name!r}"
