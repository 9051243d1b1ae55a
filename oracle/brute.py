"""Pure-Python brute force of the materialised-probability SDPA forward.

TEST INFRASTRUCTURE ONLY (used to pin the C oracle on tiny inputs).

Written independently of ``sdpa_oracle.c``: the textbook softmax
``P_j = exp(s_j - m) / sum_k exp(s_k - m)`` with exact (``math.fsum``)
summation everywhere, the key/value head found by expanding the KV heads with
``repeat_interleave`` semantics, and the mask looked up by broadcasting
indices. Semantics as in the package docstring of ``oracle``.
"""

from __future__ import annotations

import math
from typing import Optional

import numpy as np


def _lookup(mask: np.ndarray, b: int, h: int, i: int, j: int):
    """Broadcast-index a mask of up to 4 dims at logical (b, h, i, j)."""
    idx = (b, h, i, j)[4 - mask.ndim:]
    idx = tuple(0 if n == 1 else x for x, n in zip(idx, mask.shape))
    return mask[idx]


def _array(x):
    if hasattr(x, "detach"):  # a torch tensor: widen first (numpy has no bfloat16)
        x = x.detach().cpu()
        x = x.numpy() if str(x.dtype) == "torch.bool" else x.double().numpy()
    return np.asarray(x)


def sdpa_brute(q, k, v, attn_mask=None, is_causal: bool = False,
               scale: Optional[float] = None, enable_gqa: bool = False,
               causal_alignment: str = "top_left", dropout_p: float = 0.0, dropout_mask=None,
               dropout_rule: str = "explicit"):
    """Brute-force (O, P, LSE). With ``dropout_mask`` (True keeps): rule
    "explicit" returns the kept probabilities as they are and divides O by
    (1 - p); rule "random" divides the kept probabilities by (1 - p) and O
    is their product with V."""
    q = _array(q).astype(np.float64)
    k = _array(k).astype(np.float64)
    v = _array(v).astype(np.float64)
    B, Hq, Sq, D = q.shape
    Hkv, Skv, Dv = k.shape[1], k.shape[2], v.shape[3]
    if Hkv == 0 or Hq % Hkv:
        raise ValueError("head counts do not divide")
    if Hq != Hkv and not enable_gqa:
        raise ValueError("Hq != Hkv requires enable_gqa")
    if is_causal and attn_mask is not None:
        raise ValueError("is_causal and attn_mask are mutually exclusive")
    if causal_alignment not in ("top_left", "bottom_right"):
        raise ValueError(f"unknown causal alignment {causal_alignment!r}")
    # the last key query i may see: i (top-left) or i + Skv - Sq (bottom-right)
    shift = Skv - Sq if causal_alignment == "bottom_right" else 0
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    mask = None if attn_mask is None else _array(attn_mask)
    keep = None if dropout_mask is None else _array(dropout_mask)
    if keep is not None and dropout_rule not in ("explicit", "random"):
        raise ValueError(f"unknown dropout rule {dropout_rule!r}")
    # KV heads expanded the way repeat_interleave(Hq // Hkv, dim=1) would.
    kv_head = [h * Hkv // Hq for h in range(Hq)]

    out = np.zeros((B, Hq, Sq, Dv))
    probs = np.zeros((B, Hq, Sq, Skv))
    lse = np.zeros((B, Hq, Sq))
    for b in range(B):
        for h in range(Hq):
            hk = kv_head[h]
            for i in range(Sq):
                s = []
                for j in range(Skv):
                    x = scale * math.fsum(float(q[b, h, i, d]) * float(k[b, hk, j, d])
                                          for d in range(D))
                    if is_causal and j > i + shift:
                        x = -math.inf
                    elif mask is not None:
                        mv = _lookup(mask, b, h, i, j)
                        if mask.dtype == np.bool_:
                            x = x if bool(mv) else -math.inf
                        else:
                            x = x + float(mv)
                    s.append(x)
                live = [x for x in s if x != -math.inf]
                if not live:
                    lse[b, h, i] = -math.inf
                    continue  # P row and O row stay zero
                m = max(live)
                e = [math.exp(x - m) if x != -math.inf else 0.0 for x in s]
                z = math.fsum(e)
                lse[b, h, i] = m + math.log(z)
                p = [x / z for x in e]
                oscale = 1.0
                if keep is not None:
                    p = [x if bool(_lookup(keep, b, h, i, j)) else 0.0 for j, x in enumerate(p)]
                    if dropout_rule == "random":
                        p = [x / (1.0 - dropout_p) for x in p]
                    else:
                        oscale = 1.0 / (1.0 - dropout_p)
                probs[b, h, i, :] = p
                for d in range(Dv):
                    out[b, h, i, d] = oscale * math.fsum(p[j] * float(v[b, hk, j, d]) for j in range(Skv))
    return out, probs, lse


def sdpa_backward_brute(q, k, v, attn_mask=None, is_causal: bool = False,
                        scale: Optional[float] = None, enable_gqa: bool = False,
                        dout=None, dprobs=None, causal_alignment: str = "top_left"):
    """Gradients (dq, dk, dv) of a loss with dL/dO = ``dout`` and dL/dP =
    ``dprobs`` (None: zero), by brute force: the probabilities from
    ``sdpa_brute``, then the full softmax Jacobian of each row,
    dP_ik/dS_ij = P_ik (delta_kj - P_ij), applied term by term with exact
    summation, and the key/value gradients of every query head added to the
    key/value head it reads (repeat_interleave expansion, summed back)."""
    _, probs, _ = sdpa_brute(q, k, v, attn_mask, is_causal, scale, enable_gqa, causal_alignment)
    q = _array(q).astype(np.float64)
    k = _array(k).astype(np.float64)
    v = _array(v).astype(np.float64)
    B, Hq, Sq, D = q.shape
    Hkv, Skv, Dv = k.shape[1], k.shape[2], v.shape[3]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    do = _array(dout).astype(np.float64)
    dpr = None if dprobs is None else _array(dprobs).astype(np.float64)
    kv_head = [h * Hkv // Hq for h in range(Hq)]
    dq = np.zeros((B, Hq, Sq, D))
    dk_terms = [[[[[] for _ in range(D)] for _ in range(Skv)] for _ in range(Hkv)] for _ in range(B)]
    dv_terms = [[[[[] for _ in range(Dv)] for _ in range(Skv)] for _ in range(Hkv)] for _ in range(B)]
    for b in range(B):
        for h in range(Hq):
            hk = kv_head[h]
            for i in range(Sq):
                p = probs[b, h, i]
                # dL/dP_ik: through O (dout . v_k) plus the direct gradient on P
                g = [math.fsum(float(do[b, h, i, d]) * float(v[b, hk, kk, d]) for d in range(Dv))
                     + (0.0 if dpr is None else float(dpr[b, h, i, kk])) for kk in range(Skv)]
                # dL/dS_ij = sum_k g_k P_ik (delta_kj - P_ij)
                ds = [math.fsum(g[kk] * float(p[kk]) * ((1.0 if kk == j else 0.0) - float(p[j]))
                                for kk in range(Skv)) for j in range(Skv)]
                for d in range(D):
                    dq[b, h, i, d] = scale * math.fsum(ds[j] * float(k[b, hk, j, d]) for j in range(Skv))
                for j in range(Skv):
                    for d in range(D):
                        dk_terms[b][hk][j][d].append(scale * ds[j] * float(q[b, h, i, d]))
                    for d in range(Dv):
                        dv_terms[b][hk][j][d].append(float(p[j]) * float(do[b, h, i, d]))
    dk = np.array([[[[math.fsum(dk_terms[b][hk][j][d]) for d in range(D)] for j in range(Skv)]
                    for hk in range(Hkv)] for b in range(B)]).reshape(B, Hkv, Skv, D)
    dv = np.array([[[[math.fsum(dv_terms[b][hk][j][d]) for d in range(Dv)] for j in range(Skv)]
                    for hk in range(Hkv)] for b in range(B)]).reshape(B, Hkv, Skv, Dv)
    return dq, dk, dv
