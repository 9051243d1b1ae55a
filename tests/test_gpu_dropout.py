"""GPU parity of dropout (sdpa_math_fwd_dropout through the C ABI) against
the float64 oracle: the explicit and the random rule with a seeded keep-mask,
every element of O, P and LSE, removed and dropped positions bit-exact +0.0,
across dtypes, head dims, attention masks, causal alignments, grouped heads,
broadcast and unaligned keep-masks; plus the binding's own random draw."""

import ctypes

import numpy as np
import pytest
import torch

import sdpa_workloads as W
from parity import TOL_OP, compare, poisoned_outputs, run_oracle
import oracle

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _keep(seed, shape, p):
    return torch.from_numpy(np.random.default_rng(seed).random(shape) >= p)


def _run(c, keep, p, rule, align="top_left", scale=None):
    from sdpa_forward_materialised_amd import _binding as Bd
    lib = Bd.load_library()
    q, k, v = (c[x].to(DEV) for x in ("q", "k", "v"))
    m = None if c["mask"] is None else c["mask"].to(DEV)
    B, Hq, Sq, D = q.shape
    Skv = k.shape[2]
    O, P, L = poisoned_outputs(B, Hq, Sq, Skv, D, q.dtype, DEV)
    gqa = int(q.shape[1] != k.shape[1])
    causal = (2 if align == "bottom_right" else 1) if c["causal"] else 0
    sc = 1.0 / D ** 0.5 if scale is None else scale
    gk = keep.to(DEV)
    rc = lib.sdpa_math_fwd_dropout(Bd._desc(q, 4), Bd._desc(k, 4), Bd._desc(v, 4), Bd._desc(m, 4), causal, sc, gqa,
                                   p, Bd._desc(gk, 4), rule, Bd._desc(O, 4), Bd._desc(P, 4), Bd._desc(L, 3),
                                   ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == 0, lib.sdpa_math_last_error()
    torch.cuda.synchronize()
    ref = oracle.sdpa_reference(c["q"], c["k"], c["v"], c["mask"], c["causal"], sc, bool(gqa),
                                causal_alignment=align, dropout_p=p, dropout_mask=keep,
                                dropout_rule="random" if rule else "explicit")
    return (O, P, L), ref


CASES = [
    ("bf16-d128-causal", dict(seed=401, dtype="bf16", B=1, Hq=2, Hkv=2, Sq=150, Skv=150, D=128, causal=True)),
    ("f16-d64-nomask", dict(seed=402, dtype="f16", B=2, Hq=2, Hkv=2, Sq=77, Skv=136, D=64)),
    ("f32-d32-bool", dict(seed=403, dtype="f32", B=1, Hq=2, Hkv=1, Sq=64, Skv=96, D=32, mask="bool")),
    ("f16-d128-gqa-keypad", dict(seed=404, dtype="f16", B=2, Hq=8, Hkv=2, Sq=96, Skv=192, D=128, mask="bool",
                                 mask_shape=(2, 1, 1, 192), p=0.3)),
    ("bf16-d64-add", dict(seed=405, dtype="bf16", B=1, Hq=3, Hkv=3, Sq=100, Skv=264, D=64, mask="add", p=0.1)),
    ("f16-d64-odd-skv", dict(seed=406, dtype="f16", B=1, Hq=2, Hkv=2, Sq=50, Skv=37, D=64)),
]


@pytest.mark.parametrize("rule", [0, 1])
@pytest.mark.parametrize("label,spec", CASES, ids=[x[0] for x in CASES])
def test_dropout_rules(label, spec, rule):
    c = W.make_case(**spec)
    B, Hq, Sq, _ = c["q"].shape
    Skv = c["k"].shape[2]
    keep = _keep(spec["seed"], (B, Hq, Sq, Skv), 0.2)
    print(f"[case] dropout {label} rule={rule}", flush=True)
    got, ref = _run(c, keep, 0.2, rule)
    r = compare(*got, ref, c["q"].dtype, f"dropout {label} rule={rule}", v=c["v"])
    print(f"[result] dropout {label} rule={rule} {r}", flush=True)


@pytest.mark.parametrize("shape", [(1, 1, 1, 200), (2, 1, 70, 200), (200,)])
def test_dropout_broadcast_keep(shape):
    c = W.make_case(seed=407, dtype="bf16", B=2, Hq=4, Hkv=4, Sq=70, Skv=200, D=64)
    keep = _keep(408, shape, 0.3)
    got, ref = _run(c, keep, 0.3, 1)
    compare(*got, ref, torch.bfloat16, f"dropout keep {shape}", v=c["v"])


def test_dropout_bottom_right_and_dead_rows():
    c = W.make_case(seed=409, dtype="f16", B=1, Hq=2, Hkv=2, Sq=150, Skv=90, D=32, causal=True)
    keep = _keep(410, (1, 2, 150, 90), 0.5)
    got, ref = _run(c, keep, 0.5, 0, align="bottom_right")
    compare(*got, ref, torch.float16, "dropout bottom-right", v=c["v"])
    assert torch.isneginf(got[2][0, :, :60]).all() and torch.all(got[1][0, :, :60] == 0)


def test_dropout_keep_all_p0_is_no_dropout():
    import sdpa_forward_materialised_amd as S
    c = W.make_case(seed=411, dtype="bf16", B=1, Hq=2, Hkv=2, Sq=130, Skv=130, D=128, causal=True)
    keep = torch.ones(1, 2, 130, 130, dtype=torch.bool)
    got, _ = _run(c, keep, 0.0, 0)
    ref = run_oracle(c["q"], c["k"], c["v"], None, True, None, False)
    compare(*got, ref, torch.bfloat16, "keep all, p = 0", v=c["v"])


def test_dropout_errors_before_launch():
    from sdpa_forward_materialised_amd import _binding as Bd
    lib = Bd.load_library()
    c = W.make_case(seed=412, dtype="f16", B=1, Hq=2, Hkv=2, Sq=16, Skv=16, D=64)
    q = c["q"].to(DEV)
    O, P, L = poisoned_outputs(1, 2, 16, 16, 64, q.dtype, DEV)
    keep = torch.ones(16, 16, dtype=torch.bool, device=DEV)
    def args(p, kp, rule):
        return (Bd._desc(q, 4), Bd._desc(q, 4), Bd._desc(q, 4), None, 0, 0.125, 0, p, kp, rule,
                Bd._desc(O, 4), Bd._desc(P, 4), Bd._desc(L, 3), None)
    assert lib.sdpa_math_fwd_dropout(*args(1.0, Bd._desc(keep, 4), 0)) == 1
    assert lib.sdpa_math_fwd_dropout(*args(0.1, Bd._desc(keep, 4), 2)) == 1
    assert lib.sdpa_math_fwd_dropout(*args(0.1, None, 0)) == 1
    assert lib.sdpa_math_fwd_dropout(*args(0.1, Bd._desc(keep.float(), 4), 0)) == 1
    torch.cuda.synchronize()
    assert torch.isnan(O).all() and torch.isnan(P).all()


def test_binding_random_rule_draws_its_own_keep_mask():
    """dropout_p without a mask: the binding draws keep with torch's generator
    and applies the random rule: every P entry is 0 or the undropped one
    divided by 1 - p, about p of the kept-by-softmax entries are dropped, and
    O = P V within the dtype's bound."""
    import sdpa_forward_materialised_amd as S
    c = W.make_case(seed=413, dtype="f32", B=2, Hq=4, Hkv=4, Sq=128, Skv=256, D=64)
    q, k, v = (c[x].to(DEV) for x in ("q", "k", "v"))
    torch.manual_seed(0)
    O, P, L = S.fwd(q, k, v, dropout_p=0.25)
    O0, P0, L0 = S.fwd(q, k, v)
    torch.cuda.synchronize()
    kept = P != 0
    frac = 1.0 - kept.float().mean().item()
    assert abs(frac - 0.25) < 0.01, frac
    assert torch.allclose(P[kept] * 0.75, P0[kept], rtol=1e-6, atol=1e-7)
    assert torch.equal(L, L0)
    ref_o = (P.double() @ v.double())
    assert (O.double() - ref_o).abs().max().item() <= TOL_OP[torch.float32]
