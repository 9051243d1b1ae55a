"""Shared helpers for GPU-vs-oracle parity checks (test code only)."""

from __future__ import annotations

import math

import numpy as np
import torch

import oracle

# Max-abs bounds on O and P per compute dtype (the pages' f32/f16/bf16 bar),
# and on LSE (float32 row statistics from dtype-exact inputs).
TOL_OP = {torch.float32: 1e-5, torch.float16: 2e-3, torch.bfloat16: 8e-3}
TOL_LSE = {torch.float32: 1e-5, torch.float16: 1e-4, torch.bfloat16: 1e-4}

MANT_BITS = {torch.float32: 23, torch.float16: 10, torch.bfloat16: 7}


# frexp exponent of the smallest normal number of each dtype (x = m 2^e,
# m in [0.5, 1)): below it the spacing stays that of the subnormals
EMIN = {torch.float32: -125, torch.float16: -13, torch.bfloat16: -125}


def ulp(x, dtype):
    """Spacing of ``dtype`` at |x| (its unit in the last place there; the
    subnormal spacing below the smallest normal number, and at zero)."""
    x = np.abs(np.asarray(x, dtype=np.float64))
    _, e = np.frexp(x)
    e = np.where(x == 0, EMIN[dtype], np.maximum(e, EMIN[dtype]))
    return np.ldexp(1.0, e - 1 - MANT_BITS[dtype])


# Error of the kernels' float32 O before its final rounding, per unit of the
# largest |V| the row reads: P is carried as its rounded value plus the
# rounded residual (relative error at most 2^-16 in bf16, 2^-22 in fp16 per
# term), exp2 and its argument in float32 (a few 2^-24 relative), and the
# float32 accumulation of the products. 2^-13 covers all three with margin.
PRE_ROUND_SLACK = 2.0 ** -13


def bound(ref, dtype, vmax):
    """Element-wise max-abs bound on O: the stated per-dtype tolerance wherever
    a correctly rounded output can meet it (half an ulp of the dtype at the
    oracle value is at most the tolerance: bf16 |O| < 4, fp16 |O| < 8, fp32
    |O| < 256); elsewhere half an ulp plus the pre-rounding slack times the
    largest |V|. P never exceeds 1, so its bound is always the stated one."""
    tol = TOL_OP[dtype]
    half = 0.5 * ulp(ref, dtype)
    return np.where(half <= tol, tol, half + PRE_ROUND_SLACK * vmax)


# An oracle probability this small may legitimately come back as 0: below half
# the smallest subnormal of the output dtype it rounds to 0, and the kernel's
# float32 exp2 does not produce float32 subnormals.
UNDERFLOW = {torch.float32: 2.0 ** -126, torch.float16: 2.0 ** -25, torch.bfloat16: 2.0 ** -126}


def poisoned_outputs(B, Hq, Sq, Skv, Dv, dtype, device):
    """Output buffers filled with NaN so that an unwritten element cannot pass."""
    O = torch.full((B, Hq, Sq, Dv), float("nan"), dtype=dtype, device=device)
    P = torch.full((B, Hq, Sq, Skv), float("nan"), dtype=dtype, device=device)
    L = torch.full((B, Hq, Sq), float("nan"), dtype=torch.float32, device=device)
    return O, P, L


def compare(O, P, L, ref, dtype, label="", v=None):
    """Element-by-element comparison against the float64 oracle.

    ``v`` is the value tensor the call read (its largest magnitude scales the
    pre-rounding slack of the O bound where the stated tolerance is out of a
    correctly rounded output's reach). Returns a dict of the observed errors
    (``o_elems_relaxed``: O elements whose bound exceeds the stated one);
    raises AssertionError on failure.
    """
    if v is None:
        raise ValueError("compare needs the value tensor v")
    vmax = float(v.detach().abs().max()) if v.numel() else 0.0
    ro, rp, rl = ref
    o = O.detach().cpu().double().numpy()
    p = P.detach().cpu().double().numpy()
    lse = L.detach().cpu().double().numpy()
    assert o.shape == ro.shape and p.shape == rp.shape and lse.shape == rl.shape, label
    assert not np.isnan(o).any(), f"{label}: NaN in O"
    assert not np.isnan(p).any(), f"{label}: NaN in P"
    assert not np.isnan(lse).any(), f"{label}: NaN in LSE"
    err_o = float(np.abs(o - ro).max()) if o.size else 0.0
    err_p = float(np.abs(p - rp).max()) if p.size else 0.0
    tol = TOL_OP[dtype]
    bo = bound(ro, dtype, vmax)
    bad = np.abs(o - ro) > bo
    assert not bad.any(), (f"{label}: {int(bad.sum())} O elements beyond the bound; max|dO| = {err_o:.3e} "
                           f"(max|O_ref| = {np.abs(ro).max():.3f})")
    relaxed = int((bo > tol).sum())
    assert err_p <= tol, f"{label}: max|dP| = {err_p:.3e} > {tol}"
    # dead rows: LSE exactly -inf; live rows within tolerance
    dead = np.isneginf(rl)
    assert np.array_equal(np.isneginf(lse), dead), f"{label}: dead-row pattern of LSE differs"
    # LSE is float32 whatever the dtype: the stated bound, or four float32 ulps
    # at the oracle's |LSE| where that is larger (a large scale gives |LSE| of
    # tens, where float32 scores and their sum cannot hold 1e-5 absolute)
    dl = np.abs(lse[~dead] - rl[~dead])
    err_l = float(dl.max()) if dl.size else 0.0
    lb = np.maximum(TOL_LSE[dtype], 4 * ulp(rl[~dead], torch.float32))
    assert not (dl > lb).any(), f"{label}: max|dLSE| = {err_l:.3e} (max|LSE_ref| = {np.abs(rl[~dead]).max():.2f})"
    # masked-position pattern of P: bit-exact +0.0 where the oracle is exactly 0
    if P.numel():
        bits = P.detach().cpu().contiguous().view(torch.int16 if P.element_size() == 2 else torch.int32)
        zero_bits = (bits == 0).numpy()
        ref_zero = rp == 0
        assert np.array_equal(zero_bits & ref_zero, ref_zero), f"{label}: a removed position is not +0.0"
        unexpected = zero_bits & ~ref_zero & (rp >= UNDERFLOW[dtype])
        assert not unexpected.any(), f"{label}: {int(unexpected.sum())} live positions came back as 0"
    return {"err_o": err_o, "err_p": err_p, "err_lse": err_l, "o_elems_relaxed": relaxed,
            "max_abs_o_ref": float(np.abs(ro).max()) if ro.size else 0.0}


def run_oracle(q, k, v, mask, causal, scale, gqa, causal_alignment="top_left"):
    return oracle.sdpa_reference(q, k, v, mask, causal, scale, gqa, causal_alignment=causal_alignment)


def head_slice(q, k, v, mask, b, h):
    """Inputs restricted to batch b, query head h (and the KV head it reads)."""
    g = q.shape[1] // k.shape[1]
    hk = h // g
    qs, ks, vs = q[b:b + 1, h:h + 1], k[b:b + 1, hk:hk + 1], v[b:b + 1, hk:hk + 1]
    ms = None
    if mask is not None:
        m4 = mask
        while m4.dim() < 4:
            m4 = m4.unsqueeze(0)
        mb = m4[b:b + 1] if m4.shape[0] > 1 else m4
        ms = mb[:, h:h + 1] if mb.shape[1] > 1 else mb
    return qs, ks, vs, ms


def default_scale(D):
    return 1.0 / math.sqrt(D)


# Backward bound: per element, half an ulp of the dtype at the oracle
# gradient plus BWD_SLACK times the gradient's envelope, the sum of absolute
# values of the terms it adds up (float32 accumulation, exp2 of the
# recomputed probabilities, and the rounded residuals of P and dS in the
# 16-bit products all scale with it).
BWD_SLACK = 2.0 ** -12


# fp16 has subnormals below 2^-14: there the split of dS into rounded value
# plus rounded residual carries a term only to an absolute 2^-25, so fp16
# gradients built from dS (dq, dk) get a floor of 2^-24 per kept term.
BWD_FP16_FLOOR = 2.0 ** -24


def backward_envelopes(q, k, v, mask, causal, scale, gqa, dout, dprobs, causal_alignment="top_left"):
    """(env_dq, env_dk, env_dv) in float64 from the oracle's probabilities:
    env_dq_i = |scale| sum_j P_ij (|dP_ij| + |D_i|) |k_j|, env_dk_j the same
    summed over queries with |q_i|, env_dv_j = sum_i P_ij |dout_i|; for fp16
    inputs the dq and dk envelopes also carry the subnormal floor,
    BWD_FP16_FLOOR / BWD_SLACK * |scale| * sum over kept terms of |k_j| or
    |q_i|."""
    _, p, _ = oracle.sdpa_reference(q, k, v, mask, causal, scale, gqa, causal_alignment=causal_alignment)
    q, k, v = (x.double().numpy() for x in (q, k, v))
    do = dout.double().numpy()
    B, Hq, Sq, D = q.shape
    Hkv = k.shape[1]
    g = Hq // Hkv
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    kr = np.repeat(k, g, axis=1)
    vr = np.repeat(v, g, axis=1)
    dp = do @ vr.transpose(0, 1, 3, 2)
    if dprobs is not None:
        dp = dp + dprobs.double().numpy()
    dsum = (p * dp).sum(-1, keepdims=True)
    w = p * (np.abs(dp) + np.abs(dsum))
    env_dq = abs(scale) * (w @ np.abs(kr))
    env_dk = abs(scale) * (w.transpose(0, 1, 3, 2) @ np.abs(q))
    env_dv = p.transpose(0, 1, 3, 2) @ np.abs(do)
    if dout.dtype == torch.float16:
        kept = (p > 0).astype(np.float64)
        f = BWD_FP16_FLOOR / BWD_SLACK * abs(scale)
        env_dq = env_dq + f * (kept @ np.abs(kr))
        env_dk = env_dk + f * (kept.transpose(0, 1, 3, 2) @ np.abs(q))
    env_dk = env_dk.reshape(B, Hkv, g, *env_dk.shape[2:]).sum(2)
    env_dv = env_dv.reshape(B, Hkv, g, *env_dv.shape[2:]).sum(2)
    return env_dq, env_dk, env_dv


def compare_backward(got, ref, env, dtype, label=""):
    """Element-by-element check of (dq, dk, dv) against the oracle."""
    out = {}
    for name, g, r, e in zip(("dq", "dk", "dv"), got, ref, env):
        x = g.detach().cpu().double().numpy()
        assert x.shape == r.shape, (label, name)
        assert not np.isnan(x).any(), f"{label}: NaN in {name}"
        err = np.abs(x - r)
        bound = 0.5 * ulp(r, dtype) + BWD_SLACK * e
        bad = err > bound
        assert not bad.any(), (f"{label}: {int(bad.sum())} {name} elements beyond the bound; "
                               f"max|d{name}| = {float(err.max()):.3e}, worst ratio "
                               f"{float((err / np.maximum(bound, 1e-300)).max()):.2f}")
        out["err_" + name] = float(err.max()) if err.size else 0.0
        out["ratio_" + name] = float((err / np.maximum(bound, 1e-300)).max()) if err.size else 0.0
    return out
