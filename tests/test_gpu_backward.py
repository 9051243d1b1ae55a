"""GPU parity of the backward (sdpa_math_bwd through the C ABI) against the
float64 oracle's sdpa_backward_reference: dq, dk, dv element by element on
seeded inputs (every dtype and head dim, causal top-left and bottom-right,
bool and additive masks, grouped heads, dead rows, ragged shapes, with and
without a gradient on P), outputs poisoned with NaN beforehand; and the
differentiable wrapper end to end through torch autograd."""

import numpy as np
import pytest
import torch

import oracle
import sdpa_workloads as W
from parity import backward_envelopes, compare_backward

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _lib():
    import sdpa_forward_materialised_amd as S
    S.load_library()
    return S


def _grads(c, seed, with_dp=True):
    g = np.random.default_rng(seed)
    B, Hq, Sq, _ = c["q"].shape
    Skv, Dv = c["k"].shape[2], c["v"].shape[3]
    to = W.TORCH_DTYPES
    dt = {torch.float32: "f32", torch.float16: "f16", torch.bfloat16: "bf16"}[c["q"].dtype]
    dout = W.to_dtype(g.standard_normal((B, Hq, Sq, Dv)), dt)
    dprobs = W.to_dtype(g.standard_normal((B, Hq, Sq, Skv)), dt) if with_dp else None
    return dout, dprobs


def _check(c, label, with_dp=True, scale=None, align="top_left"):
    S = _lib()
    q, k, v = c["q"], c["k"], c["v"]
    m = c["mask"]
    gqa = q.shape[1] != k.shape[1]
    dout, dprobs = _grads(c, 7 + q.shape[2], with_dp)
    dev = [x.to(DEV) for x in (q, k, v)]
    gm = None if m is None else m.to(DEV)
    print(f"[case] bwd {label} {tuple(q.shape)}x{tuple(k.shape)} dprobs={with_dp}", flush=True)
    O, P, L = S.fwd(*dev, gm, c["causal"], scale, gqa, causal_alignment=align)
    out = tuple(torch.full_like(x, float("nan")) for x in dev)
    got = S.bwd(*dev, L, dout.to(DEV), None if dprobs is None else dprobs.to(DEV), gm, c["causal"], scale, gqa,
                causal_alignment=align, out=out)
    torch.cuda.synchronize()
    ref = oracle.sdpa_backward_reference(q, k, v, m, c["causal"], scale, gqa, dout, dprobs,
                                         causal_alignment=align)
    env = backward_envelopes(q, k, v, m, c["causal"], scale, gqa, dout, dprobs, align)
    r = compare_backward(got, ref, env, q.dtype, label)
    print(f"[result] bwd {label} {r}", flush=True)
    return r


CASES = [
    ("bf16-d128-causal", dict(seed=201, dtype="bf16", B=1, Hq=2, Hkv=2, Sq=150, Skv=150, D=128, causal=True)),
    ("f16-d64-nomask-ragged", dict(seed=202, dtype="f16", B=2, Hq=2, Hkv=2, Sq=77, Skv=131, D=64)),
    ("f32-d32-causal", dict(seed=203, dtype="f32", B=1, Hq=2, Hkv=2, Sq=64, Skv=64, D=32, causal=True)),
    ("f32-d128-bool", dict(seed=204, dtype="f32", B=1, Hq=2, Hkv=1, Sq=40, Skv=70, D=128, mask="bool")),
    ("bf16-d64-gqa-keypad", dict(seed=205, dtype="bf16", B=2, Hq=8, Hkv=2, Sq=96, Skv=200, D=64, mask="bool",
                                 mask_shape=(2, 1, 1, 200), p=0.3)),
    ("f16-d32-add", dict(seed=206, dtype="f16", B=1, Hq=3, Hkv=3, Sq=65, Skv=100, D=32, mask="add", p=0.1)),
    ("f16-d128-neginf", dict(seed=207, dtype="f16", B=1, Hq=4, Hkv=2, Sq=33, Skv=257, D=128, mask="neginf", p=0.3)),
    ("bf16-d32-single", dict(seed=208, dtype="bf16", B=1, Hq=1, Hkv=1, Sq=1, Skv=1, D=32)),
    ("f16-d64-sq>skv-causal", dict(seed=209, dtype="f16", B=1, Hq=2, Hkv=1, Sq=130, Skv=70, D=64, causal=True)),
    ("f32-d64-add-odd-skv", dict(seed=210, dtype="f32", B=1, Hq=2, Hkv=2, Sq=50, Skv=37, D=64, mask="add", p=0.2)),
    # aligned masks (Skv a multiple of 8): the key side stages each step's mask tile in LDS
    ("f16-d128-add-aligned", dict(seed=218, dtype="f16", B=1, Hq=4, Hkv=2, Sq=75, Skv=264, D=128, mask="add", p=0.1)),
    ("f32-d64-add-aligned", dict(seed=219, dtype="f32", B=2, Hq=2, Hkv=1, Sq=41, Skv=136, D=64, mask="add", p=0.2)),
    ("bf16-d32-neginf-aligned", dict(seed=220, dtype="bf16", B=1, Hq=3, Hkv=3, Sq=97, Skv=200, D=32, mask="neginf",
                                     p=0.3)),
]


@pytest.mark.parametrize("with_dp", [True, False])
@pytest.mark.parametrize("label,spec", CASES, ids=[x[0] for x in CASES])
def test_backward_small(label, spec, with_dp):
    c = W.make_case(**spec)
    _check(c, label, with_dp)


def test_backward_dead_rows():
    c = W.make_case(seed=211, dtype="f16", B=2, Hq=4, Hkv=2, Sq=96, Skv=160, D=64, mask="bool",
                    mask_shape=(2, 4, 96, 160), p=0.2)
    c["mask"][0, 1, 5, :] = False
    c["mask"][1, 3, 40:72, :] = False
    _check(c, "dead rows")


@pytest.mark.parametrize("Sq,Skv", [(130, 520), (150, 90)])
def test_backward_bottom_right(Sq, Skv):
    c = W.make_case(seed=212, dtype="bf16", B=1, Hq=2, Hkv=2, Sq=Sq, Skv=Skv, D=64, causal=True)
    _check(c, f"bottom-right {Sq}x{Skv}", align="bottom_right")


@pytest.mark.parametrize("scale", [-0.125, 0.0, 2.0])
def test_backward_scales(scale):
    c = W.make_case(seed=213, dtype="bf16", B=1, Hq=2, Hkv=1, Sq=70, Skv=96, D=64, mask="bool", p=0.2)
    _check(c, f"scale={scale}", scale=scale)


# Causal calls with few key blocks split each key block's query steps over
# up to four workgroups (float32 partial dk, dv summed by a reduce launch):
# four ranges with ragged Sq and Skv and grouped heads, two ranges
# bottom-right with more keys than queries, and fp32.
@pytest.mark.parametrize("label,spec,align", [
    ("4-ranges-gqa", dict(seed=215, dtype="bf16", B=1, Hq=2, Hkv=1, Sq=600, Skv=700, D=64, causal=True), "top_left"),
    ("2-ranges-br", dict(seed=216, dtype="f16", B=1, Hq=2, Hkv=2, Sq=520, Skv=776, D=128, causal=True), "bottom_right"),
    ("f32-ranges", dict(seed=217, dtype="f32", B=1, Hq=1, Hkv=1, Sq=520, Skv=520, D=32, causal=True), "top_left"),
], ids=["4-ranges-gqa", "2-ranges-br", "f32-ranges"])
def test_backward_query_ranges(label, spec, align):
    c = W.make_case(**spec)
    _check(c, label, align=align)


def test_backward_deterministic():
    S = _lib()
    c = W.make_case(seed=214, dtype="bf16", B=1, Hq=4, Hkv=2, Sq=200, Skv=200, D=128, causal=True)
    dev = [c[x].to(DEV) for x in ("q", "k", "v")]
    O, P, L = S.fwd(*dev, None, True, None, True)
    dout, dprobs = _grads(c, 5)
    a = S.bwd(*dev, L, dout.to(DEV), dprobs.to(DEV), None, True, None, True)
    b = S.bwd(*dev, L, dout.to(DEV), dprobs.to(DEV), None, True, None, True)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_autograd_function_end_to_end():
    """loss = <O, W1> + <P, W2> through sdpa_math (torch autograd calls the
    library's backward): q.grad, k.grad, v.grad against the oracle."""
    S = _lib()
    c = W.make_case(seed=215, dtype="bf16", B=1, Hq=4, Hkv=2, Sq=80, Skv=120, D=64, mask="bool",
                    mask_shape=(1, 1, 80, 120), p=0.2)
    dout, dprobs = _grads(c, 9)
    q, k, v = (c[x].to(DEV).requires_grad_(True) for x in ("q", "k", "v"))
    O, P, L = S.sdpa_math(q, k, v, c["mask"].to(DEV), False, None, True)
    loss = (O.float() * dout.to(DEV).float()).sum() + (P.float() * dprobs.to(DEV).float()).sum()
    loss.backward()
    torch.cuda.synchronize()
    ref = oracle.sdpa_backward_reference(c["q"], c["k"], c["v"], c["mask"], False, None, True, dout, dprobs)
    env = backward_envelopes(c["q"], c["k"], c["v"], c["mask"], False, None, True, dout, dprobs)
    compare_backward((q.grad, k.grad, v.grad), ref, env, torch.bfloat16, "autograd")


def test_backward_workspace_errors():
    import ctypes
    from sdpa_forward_materialised_amd import _binding as Bd
    lib = Bd.load_library()
    c = W.make_case(seed=216, dtype="f16", B=1, Hq=2, Hkv=2, Sq=16, Skv=16, D=64)
    q, k, v = (c[x].to(DEV) for x in ("q", "k", "v"))
    L = torch.zeros(1, 2, 16, device=DEV)
    do = torch.zeros_like(q)
    dq, dk, dv = (torch.full_like(x, float("nan")) for x in (q, k, v))
    args = [Bd._desc(q, 4), Bd._desc(k, 4), Bd._desc(v, 4), None, 0, 0.125, 0, Bd._desc(L, 3), Bd._desc(do, 4), None,
            Bd._desc(dq, 4), Bd._desc(dk, 4), Bd._desc(dv, 4)]
    assert lib.sdpa_math_bwd(*args, None, 0, None) == 1 and b"workspace" in lib.sdpa_math_last_error()
    ws = torch.empty(64, dtype=torch.uint8, device=DEV)
    assert lib.sdpa_math_bwd(*args, ctypes.c_void_p(ws.data_ptr()), 64, None) == 1
    torch.cuda.synchronize()
    assert torch.isnan(dq).all() and torch.isnan(dk).all() and torch.isnan(dv).all()


@pytest.mark.parametrize("name", ["prefill_1k_d64_f16_causal", "prefill_2k_d128_bf16_causal",
                                  "gqa_1k_d128_f16_keypad"])
def test_backward_workload_full_size(name):
    """The backward at the timed workloads' full size, every element of dq,
    dk and dv against the oracle (upstream gradients N(0,1), seeded)."""
    w = W.BY_NAME[name]
    inp = W.make_inputs(w)
    c = dict(inp, causal=w.causal)
    r = _check(c, name, with_dp=True, scale=w.scale)
    print(f"[result] bwd full {name} {r}", flush=True)
