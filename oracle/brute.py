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
               causal_alignment: str = "top_left"):
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
                probs[b, h, i, :] = p
                for d in range(Dv):
                    out[b, h, i, d] = math.fsum(p[j] * float(v[b, hk, j, d]) for j in range(Skv))
    return out, probs, lse
