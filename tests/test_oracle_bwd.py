"""Pins for the backward of the CPU oracle (no GPU).

``oracle.sdpa_backward_reference`` gives (dq, dk, dv) for gradients dL/dO and
dL/dP of the forward's two outputs (the FlagOS-OP page's two-output
backward: Implementation section and "P800 fused backward" update). It is
tied to things other than itself:
  * an independent brute force (full softmax Jacobian, exact summation);
  * central finite differences of the forward oracle's own loss;
  * identities every softmax-attention gradient satisfies: the key gradients
    of a head sum to zero (scores of a row are shift invariant), the query and
    key gradients give the same derivative with respect to the scale, the
    value gradients of a head sum to the output gradient of its live rows, a
    dL/dP constant along each row has no effect;
  * closed forms (a single key; zero upstream gradients);
  * grouped heads equal repeated key/value heads with the gradients summed;
and a mutation test plants plausible mistakes in the C backward.
"""

import os

import numpy as np
import pytest
import torch

import oracle
from oracle.brute import sdpa_backward_brute
import sdpa_workloads as W

ORACLE_SRC = os.path.join(os.path.dirname(oracle.__file__), "sdpa_oracle.c")


def _case(seed, B=1, Hq=2, Hkv=2, Sq=4, Skv=5, D=3, mask="none", mask_shape=None, causal=False, Dv=None,
          p=0.3, dtype="f32", with_dprobs=True):
    c = W.make_case(seed, dtype, B, Hq, Hkv, Sq, Skv, D, mask, mask_shape, causal, Dv, p)
    g = np.random.default_rng(seed + 1000)
    dv_ = D if Dv is None else Dv
    c["dout"] = torch.from_numpy(g.standard_normal((B, Hq, Sq, dv_)))
    c["dprobs"] = torch.from_numpy(g.standard_normal((B, Hq, Sq, Skv))) if with_dprobs else None
    return c


def _bwd(fn, c, scale=None, align="top_left", **kw):
    gqa = c["q"].shape[1] != c["k"].shape[1]
    return fn(c["q"], c["k"], c["v"], c["mask"], c["causal"], scale, gqa, c["dout"], c["dprobs"],
              causal_alignment=align, **kw)


CASES = [
    dict(seed=1),
    dict(seed=2, causal=True),
    dict(seed=3, Sq=6, Skv=4, causal=True),
    dict(seed=4, Sq=3, Skv=7, causal=True),
    dict(seed=5, mask="bool"),
    dict(seed=6, mask="bool", mask_shape=(1, 1, 4, 5), p=0.6),
    dict(seed=7, mask="add"),
    dict(seed=8, mask="neginf", p=0.5),
    dict(seed=9, Hq=4, Hkv=2),
    dict(seed=10, Hq=4, Hkv=1, B=2, mask="bool"),
    dict(seed=11, D=2, Dv=4),
    dict(seed=12, Sq=1, Skv=1),
    dict(seed=13, with_dprobs=False),
    dict(seed=14, dtype="bf16", causal=True, Sq=5, Skv=5),
]


@pytest.mark.parametrize("spec", CASES, ids=lambda s: "-".join(f"{k}{v}" for k, v in s.items()))
def test_backward_matches_brute_force(spec):
    c = _case(**spec)
    a = _bwd(oracle.sdpa_backward_reference, c)
    b = _bwd(sdpa_backward_brute, c)
    for x, y in zip(a, b):
        assert x.shape == y.shape
        assert np.allclose(x, y, rtol=0, atol=1e-12)


@pytest.mark.parametrize("align", ["top_left", "bottom_right"])
def test_backward_causal_alignments_match_brute_force(align):
    c = _case(21, Sq=5, Skv=8, causal=True)
    a = _bwd(oracle.sdpa_backward_reference, c, align=align)
    b = _bwd(sdpa_backward_brute, c, align=align)
    for x, y in zip(a, b):
        assert np.allclose(x, y, rtol=0, atol=1e-12)


def _loss(c, q, k, v, scale, align="top_left"):
    """The scalar loss whose output gradients are dout and dprobs."""
    gqa = q.shape[1] != k.shape[1]
    o, p, _ = oracle.sdpa_reference(q, k, v, c["mask"], c["causal"], scale, gqa, causal_alignment=align)
    val = float(np.sum(o * c["dout"].numpy()))
    if c["dprobs"] is not None:
        val += float(np.sum(p * c["dprobs"].numpy()))
    return val


@pytest.mark.parametrize("spec", [dict(seed=31), dict(seed=32, causal=True, Sq=4, Skv=6),
                                  dict(seed=33, Hq=4, Hkv=2, mask="bool", p=0.4),
                                  dict(seed=34, mask="add", Dv=2), dict(seed=35, with_dprobs=False)],
                         ids=lambda s: "-".join(f"{k}{v}" for k, v in s.items()))
def test_backward_matches_finite_differences(spec):
    c = _case(**spec)
    scale = 0.7
    q, k, v = (c[x].double().numpy() for x in ("q", "k", "v"))
    dq, dk, dv = _bwd(oracle.sdpa_backward_reference, c, scale=scale)
    h = 1e-5
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args = {"q": q, "k": k, "v": v}
            args[name] = xp
            fp = _loss(c, args["q"], args["k"], args["v"], scale)
            args[name] = xm
            fm = _loss(c, args["q"], args["k"], args["v"], scale)
            num[idx] = (fp - fm) / (2 * h)
        assert np.allclose(g, num, rtol=0, atol=2e-7), name


@pytest.mark.parametrize("spec", [dict(seed=41, Sq=6, Skv=9), dict(seed=42, Hq=4, Hkv=2, causal=True, Sq=7, Skv=7),
                                  dict(seed=43, mask="bool", p=0.5, Sq=6), dict(seed=44, mask="add", B=2)])
def test_backward_identities(spec):
    c = _case(**spec)
    scale = 0.4
    dq, dk, dv = _bwd(oracle.sdpa_backward_reference, c, scale=scale)
    q, k = c["q"].double().numpy(), c["k"].double().numpy()
    B, Hq, Sq, _ = q.shape
    Hkv = k.shape[1]
    g = Hq // Hkv
    _, p, lse = oracle.sdpa_reference(c["q"], c["k"], c["v"], c["mask"], c["causal"], scale, Hq != Hkv)
    live = ~np.isneginf(lse)
    do = c["dout"].numpy()
    for b in range(B):
        for hk in range(Hkv):
            heads = slice(hk * g, (hk + 1) * g)
            # shift invariance of each row's scores: the key gradients sum to zero
            assert np.allclose(dk[b, hk].sum(0), 0.0, atol=1e-12)
            # d/d(scale) from the query side equals the key side
            lhs = float(np.sum(q[b, heads] * dq[b, heads]))
            rhs = float(np.sum(k[b, hk] * dk[b, hk]))
            assert abs(lhs - rhs) <= 1e-12 * max(1.0, abs(lhs))
            # rows of P sum to one: value gradients sum to the live rows' output gradients
            want = (do[b, heads] * live[b, heads][..., None]).sum((0, 1))
            assert np.allclose(dv[b, hk].sum(0), want, atol=1e-12)


def test_backward_row_constant_dprobs_has_no_effect():
    c = _case(51, Sq=5, Skv=6, mask="bool", p=0.3)
    base = _bwd(oracle.sdpa_backward_reference, dict(c, dprobs=None))
    rowc = torch.from_numpy(np.random.default_rng(5).standard_normal((1, 2, 5, 1))).expand(1, 2, 5, 6)
    got = _bwd(oracle.sdpa_backward_reference, dict(c, dprobs=rowc.contiguous()))
    for x, y in zip(base, got):
        assert np.allclose(x, y, atol=1e-12)


def test_backward_closed_forms():
    # a single key: P = 1 whatever the scores, so no gradient reaches q or k,
    # and dv is the sum of the output gradients
    c = _case(61, Sq=4, Skv=1)
    dq, dk, dv = _bwd(oracle.sdpa_backward_reference, c)
    assert np.all(dq == 0) and np.allclose(dk, 0, atol=1e-15)
    assert np.allclose(dv[0, :, 0], c["dout"].numpy()[0].sum(1), atol=1e-12)
    # zero upstream gradients give zero gradients
    c = _case(62)
    c["dout"] = torch.zeros_like(c["dout"])
    c["dprobs"] = torch.zeros_like(c["dprobs"])
    for x in _bwd(oracle.sdpa_backward_reference, c):
        assert np.all(x == 0)
    # a dead row (every key removed) receives and passes on nothing
    c = _case(63, mask="bool", p=0.2)
    c["mask"][0, 1, 2, :] = False
    dq, dk, dv = _bwd(oracle.sdpa_backward_reference, c)
    assert np.all(dq[0, 1, 2] == 0)
    c2 = dict(c)
    c2["dout"] = c["dout"].clone()
    c2["dout"][0, 1, 2] = 123.0
    c2["dprobs"] = c["dprobs"].clone()
    c2["dprobs"][0, 1, 2] = -7.0
    for x, y in zip((dq, dk, dv), _bwd(oracle.sdpa_backward_reference, c2)):
        assert np.array_equal(x, y)


def test_backward_gqa_equals_repeated_kv():
    c = _case(71, Hq=6, Hkv=2, Sq=4, Skv=5, mask="bool", mask_shape=(1, 1, 4, 5))
    dq, dk, dv = _bwd(oracle.sdpa_backward_reference, c)
    r = dict(c, k=c["k"].repeat_interleave(3, 1), v=c["v"].repeat_interleave(3, 1))
    rq, rk, rv = _bwd(oracle.sdpa_backward_reference, r)
    assert np.allclose(dq, rq, atol=1e-13)
    assert np.allclose(dk, rk.reshape(1, 2, 3, 5, 3).sum(2), atol=1e-13)
    assert np.allclose(dv, rv.reshape(1, 2, 3, 5, 3).sum(2), atol=1e-13)


def test_backward_errors():
    c = _case(81)
    with pytest.raises(ValueError):
        oracle.sdpa_backward_reference(c["q"], c["k"], c["v"], None, False, None, False, None)
    with pytest.raises(ValueError):
        oracle.sdpa_backward_reference(c["q"], c["k"], c["v"], None, False, None, False, c["dout"][..., :2])
    with pytest.raises(ValueError):
        oracle.sdpa_backward_reference(c["q"], c["k"], c["v"], torch.ones(4, 5, dtype=torch.bool), True, None,
                                       False, c["dout"])


# ---------------------------------------------------------------- mutation test

def _bwd_pins_pass(lib_path):
    ok = True
    for spec in (dict(seed=91, Hq=4, Hkv=2, causal=True, Sq=5, Skv=5), dict(seed=92, mask="bool", p=0.4),
                 dict(seed=93, mask="add", Dv=2), dict(seed=94, Sq=3, Skv=6, causal=True)):
        c = _case(**spec)
        al = "bottom_right" if spec["seed"] == 94 else "top_left"
        a = _bwd(oracle.sdpa_backward_reference, c, scale=0.6, align=al, lib_path=lib_path)
        b = _bwd(sdpa_backward_brute, c, scale=0.6, align=al)
        for x, y in zip(a, b):
            if not np.allclose(x, y, rtol=0, atol=1e-12):
                ok = False
    return ok


BWD_MUTANTS = [
    ("Jacobian row term dropped", "const double ds = p[j] * (dp[j] - dsum);", "const double ds = p[j] * dp[j];"),
    ("Jacobian sign", "const double ds = p[j] * (dp[j] - dsum);", "const double ds = p[j] * (dsum - dp[j]);"),
    ("dq without scale", "dqi[d] += scale * ds * kh[j * D + d];", "dqi[d] += ds * kh[j * D + d];"),
    ("dk from the wrong row", "dkh[j * D + d] += scale * ds * qi[d];", "dkh[j * D + d] += scale * ds * qi[(d + 1) % D];"),
    ("dv without P", "dvh[j * Dv + d] += p[j] * doi[d];", "dvh[j * Dv + d] += doi[d];"),
    ("dprobs ignored", "acc += dprobs[row * Skv + j];", "acc += 0.0;"),
    ("group heads not summed", "for (int64_t h = hk * group; h < (hk + 1) * group; ++h) {",
     "for (int64_t h = hk * group; h < hk * group + 1; ++h) {"),
]


@pytest.mark.parametrize("name,old,new", BWD_MUTANTS, ids=[m[0] for m in BWD_MUTANTS])
def test_backward_pins_catch_planted_mistakes(tmp_path, name, old, new):
    src = open(ORACLE_SRC).read()
    cut = src.index("int oracle_sdpa_bwd(")  # plant it in the backward only
    fwd, rest = src[:cut], src[cut:]
    assert rest.count(old) == 1, name
    mutant_src = tmp_path / "mutant.c"
    mutant_src.write_text(fwd + rest.replace(old, new))
    lib = str(tmp_path / "libmutant.so")
    oracle.build(force=True, src=str(mutant_src), out=lib)
    assert not _bwd_pins_pass(lib), f"planted mistake '{name}' went unnoticed"


def test_backward_pins_pass_on_unmutated_oracle():
    assert _bwd_pins_pass(oracle.build(force=False))
