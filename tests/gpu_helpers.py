"""Shared plumbing of the GPU parity tests: seeded inputs -> device tensors,
sampled-row comparison against the fp64 oracle, tolerances.

Tolerances (absolute): binary32 paths 1e-5 on the output and the log-sum-exp;
bfloat16 paths 2e-2 on the output (bf16-rounded) and 1e-3 on the log-sum-exp.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
import ra_inputs
import ring_attention_step_amd as ra

TOL = {"f32": {"o": 1e-5, "lse": 1e-5}, "bf16": {"o": 2e-2, "lse": 1e-3}}

# Gradient tolerances (relative factor of grad_close).  "bf16": the MFMA
# backward rounds P (for dV) and dS (for dQ, dK) to bfloat16, and bfloat16
# rings feed the forward's bf16-rounded output into delta = dO . O: every
# term of a gradient sum carries an independent relative error of at most
# 2^-8 (8 significant bits), so an element's error is about 2^-8/sqrt(3)
# times the root-sum-square of its terms, which the row's RMS over head_dim
# estimates; 2^-5 of the row RMS is above the largest such error over 10^8
# elements (about 6.5 sigma, 0.015 of the row RMS).  "fp32": products and
# probabilities kept in binary32.
GRAD_RTOL = {"bf16": 2.0 ** -5, "fp32": 1e-4}


def say(*args):
    """Name the GPU step about to run (flushed, so it survives a crash)."""
    print("[gpu-step]", *args, file=sys.stderr, flush=True)


def to_device(arr: np.ndarray, dtype: str) -> torch.Tensor:
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(arr)).cuda()


def to_host_f64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def qkv_global(B, Hq, Hkv, S, D, dtype, seed=0, k_from_q_scale=None):
    """Seeded q [B,Hq,S,D], k, v [B,Hkv,S,D] (numpy; uint16 bits for bf16)."""
    q = ra_inputs.normal((B, Hq, S, D), ra_inputs.STREAM_Q, seed=seed, dtype=dtype)
    if k_from_q_scale is None:
        k = ra_inputs.normal((B, Hkv, S, D), ra_inputs.STREAM_K, seed=seed, dtype=dtype)
    else:  # dominant self-key construction: k = alpha * q (same stream)
        k = ra_inputs.normal((B, Hkv, S, D), ra_inputs.STREAM_Q, seed=seed, dtype=dtype, scale=k_from_q_scale)
    v = ra_inputs.normal((B, Hkv, S, D), ra_inputs.STREAM_V, seed=seed, dtype=dtype)
    return q, k, v


def shards_on_device(x_np, n_pos, layout, dtype):
    """Global [B,H,S,D] host array -> [N,B,H,S/N,D] device tensor via ra_stripe_permute."""
    x = to_device(x_np, dtype)
    B, H, S, D = x.shape
    y = torch.empty((n_pos, B, H, S // n_pos, D), dtype=x.dtype, device=x.device)
    ra.ra_stripe_permute(x, y, layout=layout, inverse=False, n_pos=n_pos)
    del x
    return y


def local_of(t, S, n_pos, layout):
    sb = S // n_pos
    if layout == "contiguous":
        return t // sb, t % sb
    return t % n_pos, t // n_pos


def compare_rows(o_dev, lse_dev, q_np, k_np, v_np, sel_h, sel_t, n_pos, layout, first_pos, causal, dtype,
                 scale=None):
    """Check ring outputs o [n_run,B,Hq,Sb,D], lse [n_run,B,Hq,Sb] at (b=0, h, t) rows
    against the oracle.  q_np may be the global q or a callable (h, t) -> rows."""
    pos, row = local_of(sel_t, k_np.shape[2], n_pos, layout)
    assert np.all((pos >= first_pos) & (pos < first_pos + o_dev.shape[0])), "row outside the run positions"
    idx_p = torch.as_tensor(pos - first_pos, device=o_dev.device)
    idx_h = torch.as_tensor(sel_h, device=o_dev.device)
    idx_r = torch.as_tensor(row, device=o_dev.device)
    got_o = to_host_f64(o_dev[idx_p, 0, idx_h, idx_r])
    got_lse = to_host_f64(lse_dev[idx_p, 0, idx_h, idx_r])
    if callable(q_np):
        qrows = q_np(sel_h, sel_t)
    else:
        qrows = q_np[0][sel_h, sel_t]
    Hq, Hkv = int(o_dev.shape[2]), int(k_np.shape[1])
    g = Hq // Hkv
    want_o = np.empty_like(got_o)
    want_lse = np.empty_like(got_lse)
    for h in np.unique(sel_h):
        ii = np.nonzero(sel_h == h)[0]
        r = oracle.rows(qrows[ii], k_np[0, h // g], v_np[0, h // g], q_pos=sel_t[ii], causal=causal,
                        scale=scale)
        want_o[ii], want_lse[ii] = r["o"], r["lse"]
    err_o = float(np.max(np.abs(got_o - want_o)))
    err_lse = float(np.max(np.abs(got_lse - want_lse)))
    tol = TOL[dtype]
    assert err_o <= tol["o"], f"max |O - oracle| = {err_o:.3e} > {tol['o']}"
    assert err_lse <= tol["lse"], f"max |lse - oracle| = {err_lse:.3e} > {tol['lse']}"
    return err_o, err_lse, got_o


def run_ring(q_sh, k_sh, v_sh, n_pos, first_pos, layout, causal, **kw):
    n_run = q_sh.shape[0]
    o = torch.empty_like(q_sh)
    lse = torch.empty(q_sh.shape[:4], dtype=torch.float32, device=q_sh.device)
    stats = ra.ra_ring_forward(q_sh, k_sh, v_sh, o, lse, n_pos=n_pos, first_pos=first_pos, layout=layout,
                               causal=causal, **kw)
    torch.cuda.synchronize()
    assert n_run == o.shape[0]
    return o, lse, stats


def dq_delta_bound(o_ref, pk_ref, dout, scale):
    """Extra dQ error allowed where delta = dO . O is formed from a bfloat16
    output (the ring backward reads the forward's bf16 O).  Rounding O to bf16
    changes delta_r by eps_r = sum_e dO_re (O_re' - O_re), each term with an
    independent relative error of at most 2^-8, so eps_r has a standard
    deviation of at most 2^-8 / sqrt(3) * sqrt(sum_e (dO_re O_re)^2); since
    dS_rc = p_rc (dP_rc - delta_r), dQ_r moves by scale * eps_r * sum_c p_rc k_c,
    i.e. by scale * eps_r * (P K)_r.  Allowed: six standard deviations.
    o_ref, pk_ref: the rows' exact O and P K (attention with V replaced by K);
    dout: the rows' dO (float array or bf16 bits)."""
    g = ra_inputs.bf16_to_f32(dout) if np.asarray(dout).dtype == np.uint16 else np.asarray(dout)
    g = np.asarray(g, dtype=np.float64)
    spread = np.sqrt(np.sum((g * o_ref) ** 2, axis=-1, keepdims=True))
    return scale * np.abs(pk_ref) * 6.0 / np.sqrt(3.0) * 2.0 ** -8 * spread


def grad_close(got, want, rtol, what, extra=None):
    """Elementwise gradient check against the oracle:
        |got - want| <= rtol * (|want| + rms_row(want) + 2^-4 rms(want)) + extra
    rms_row is the RMS of the element's row over head_dim (the last axis), the
    scale of the rounding errors of the sums that form the row; the 2^-4 term
    is a floor for rows whose exact value is (near) zero; ``extra`` (optional,
    broadcastable) adds a bound for an error source the row scale does not
    describe (dq_delta_bound).  Returns the largest ratio of error to bound."""
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, (got.shape, want.shape)
    if want.size == 0:
        return 0.0
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    row_rms = np.sqrt(np.mean(want * want, axis=-1, keepdims=True))
    floor = 2.0 ** -4 * float(np.sqrt(np.mean(want * want)))
    bound = rtol * (np.abs(want) + row_rms + floor)
    if extra is not None:
        bound = bound + np.asarray(extra, dtype=np.float64)
    err = np.abs(got - want)
    zero = bound == 0
    assert not np.any(err[zero] > 0), f"{what}: nonzero error where the reference is exactly zero"
    ratio = np.where(zero, 0.0, err / np.where(zero, 1.0, bound))
    worst = float(np.max(ratio))
    at = np.unravel_index(int(np.argmax(ratio)), ratio.shape)
    assert worst <= 1.0, (f"{what}: |GPU - oracle| = {float(err[at]):.3e} at {tuple(int(i) for i in at)} exceeds "
                          f"{float(bound[at]):.3e} (ref {float(want[at]):.3e}, row rms {float(row_rms[at[:-1]][0]):.3e})")
    return worst
