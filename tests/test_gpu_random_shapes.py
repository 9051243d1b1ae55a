"""Seeded random shapes through the default plan, against the oracle element
by element: dtypes, head dims, masks (none, bool, additive, broadcast
shapes), causal alignments, grouped heads, query and key counts from one to
a few thousand (decode rows that take the one-sweep key ranges, short
queries that take the fused kernels, prefill blocks that take the two-pass
kernel, ragged tails everywhere). Each case prints its shape before it runs."""

import numpy as np
import pytest
import torch

import sdpa_workloads as W
from parity import compare, poisoned_outputs, run_oracle

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _cases(n=96, seed=2024):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        dtype = ["f32", "f16", "bf16"][rng.integers(3)]
        D = int([32, 64, 128][rng.integers(3)])
        group = int([1, 1, 2, 4, 8][rng.integers(5)])
        Hkv = int(rng.integers(1, 3))
        Hq = Hkv * group
        B = int(rng.integers(1, 3))
        kind = ["decode", "short", "prefill"][rng.integers(3)]
        if kind == "decode":
            Sq, Skv = int(rng.integers(1, 5)), int(rng.integers(64, 2600))
        elif kind == "short":
            Sq, Skv = int(rng.integers(5, 130)), int(rng.integers(16, 1300))
        else:
            Sq, Skv = int(rng.integers(130, 420)), int(rng.integers(130, 700))
        if rng.random() < 0.5:
            Skv = (Skv + 7) // 8 * 8  # the 16-byte layouts (ranges, staged tiles) need Skv % 8 == 0
        mask = ["none", "none", "bool", "add"][rng.integers(4)]
        causal = mask == "none" and rng.random() < 0.4
        align = "bottom_right" if causal and rng.random() < 0.5 else "top_left"
        mshape = None
        if mask != "none":
            mshape = [(B, Hq, Sq, Skv), (B, 1, Sq, Skv), (B, 1, 1, Skv), (1, Hq, Sq, Skv)][rng.integers(4)]
        out.append(dict(seed=500 + i, dtype=dtype, B=B, Hq=Hq, Hkv=Hkv, Sq=Sq, Skv=Skv, D=D, mask=mask,
                        mask_shape=mshape, causal=causal, p=0.15, align=align))
    return out


CASES = _cases()


@pytest.mark.parametrize("spec", CASES, ids=[f"r{i}" for i in range(len(CASES))])
def test_random_shape_matches_oracle(spec):
    import sdpa_forward_materialised_amd as S
    spec = dict(spec)
    align = spec.pop("align")
    c = W.make_case(**spec)
    q, k, v, m = c["q"], c["k"], c["v"], c["mask"]
    B, Hq, Sq, D = q.shape
    Skv = k.shape[2]
    gqa = Hq != k.shape[1]
    kernel = S.kernel_name(q, k, v, m, c["causal"], gqa, causal_alignment=align)
    print(f"[case] {spec} align={align} kernel={kernel}", flush=True)
    out = poisoned_outputs(B, Hq, Sq, Skv, D, q.dtype, DEV)
    O, P, L = S.fwd(q.to(DEV), k.to(DEV), v.to(DEV), None if m is None else m.to(DEV), c["causal"], None, gqa,
                    out=out, causal_alignment=align)
    torch.cuda.synchronize()
    ref = run_oracle(q, k, v, m, c["causal"], None, gqa, align)
    compare(O, P, L, ref, q.dtype, f"random {spec}", v=v)
