"""GPU parity of packed variable-length sequences (sdpa_math_fwd_varlen,
token-major [T, H, D] with device cu_seqlens) against the oracle applied
sequence by sequence: every element of O, P (including the zero padding past
each sequence's keys) and LSE, outputs NaN-poisoned beforehand; empty query
and key sequences, causal top-left and bottom-right, grouped heads, every
dtype and head dim, row lengths with and without 16-byte rows."""

import numpy as np
import pytest
import torch

import oracle
from parity import compare

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TD = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def _pack(seed, lq, lk, Hq, Hkv, D, dtype):
    g = np.random.default_rng(seed)
    cq = np.cumsum([0] + lq).astype(np.int32)
    ck = np.cumsum([0] + lk).astype(np.int32)
    dt = TD[dtype]
    q = torch.from_numpy(g.standard_normal((int(cq[-1]), Hq, D))).to(dt)
    k = torch.from_numpy(g.standard_normal((int(ck[-1]), Hkv, D))).to(dt)
    v = torch.from_numpy(g.standard_normal((int(ck[-1]), Hkv, D))).to(dt)
    return q, k, v, torch.from_numpy(cq), torch.from_numpy(ck)


CASES = [
    ("bf16-d128-causal-mixed", 501, [70, 0, 130, 1, 64], [70, 3, 130, 1, 64], 4, 4, 128, "bf16", True, "top_left"),
    ("f16-d64-br-chunks", 502, [16, 100, 37], [200, 100, 300], 4, 2, 64, "f16", True, "bottom_right"),
    ("f32-d32-noncausal", 503, [5, 9, 64, 33], [7, 0, 12, 96], 2, 2, 32, "f32", False, "top_left"),
    ("bf16-d64-odd-maxkv", 504, [40, 20], [201, 77], 2, 1, 64, "bf16", False, "top_left"),
    ("f16-d128-gqa-decode", 505, [1, 1, 1, 1], [1000, 17, 513, 64], 8, 2, 128, "f16", False, "top_left"),
]


@pytest.mark.parametrize("label,seed,lq,lk,Hq,Hkv,D,dtype,causal,align", CASES, ids=[c[0] for c in CASES])
def test_varlen(label, seed, lq, lk, Hq, Hkv, D, dtype, causal, align):
    import sdpa_forward_materialised_amd as S
    q, k, v, cq, ck = _pack(seed, lq, lk, Hq, Hkv, D, dtype)
    max_q, max_k = max(lq), max(lk)
    Tq = q.shape[0]
    dt = q.dtype
    out = (torch.full((Tq, Hq, D), float("nan"), dtype=dt, device=DEV),
           torch.full((Tq, Hq, max_k), float("nan"), dtype=dt, device=DEV),
           torch.full((Tq, Hq), float("nan"), dtype=torch.float32, device=DEV))
    print(f"[case] varlen {label}", flush=True)
    O, P, L = S.fwd_varlen(q.to(DEV), k.to(DEV), v.to(DEV), cq.to(DEV), ck.to(DEV), max_q, max_k, causal, None,
                           Hq != Hkv, align, out=out)
    torch.cuda.synchronize()
    ref = oracle.sdpa_varlen_reference(q, k, v, cq, ck, max_k, causal, None, Hq != Hkv, align)
    r = compare(O, P, L, ref, dt, f"varlen {label}", v=v)
    print(f"[result] varlen {label} {r}", flush=True)


def test_varlen_errors_before_launch():
    import sdpa_forward_materialised_amd as S
    q, k, v, cq, ck = _pack(506, [4, 4], [4, 4], 2, 2, 64, "f16")
    with pytest.raises(ValueError):
        S.fwd_varlen(q.to(DEV), k.to(DEV), v.to(DEV), cq.to(DEV).long(), ck.to(DEV), 4, 4)
    with pytest.raises(ValueError):
        S.fwd_varlen(q.to(DEV), k.to(DEV), v.to(DEV), cq.to(DEV), ck[:2].to(DEV), 4, 4)
    with pytest.raises(NotImplementedError):
        S.fwd_varlen(q[..., :48].contiguous().to(DEV), k[..., :48].contiguous().to(DEV),
                     v[..., :48].contiguous().to(DEV), cq.to(DEV), ck.to(DEV), 4, 4)
