"""Pins for the CPU oracle (no GPU).

The oracle is trusted only because these checks tie it to things other than
itself: an independent pure-Python brute force with exact summation, closed
forms, invariants every softmax-attention result must satisfy, equivalences
between differently-expressed masks, torch's own CPU math backend on float
masks, and the semantics rules of the FlagOS-OP ``sdpa_math`` pull request
(Implementation and Intentional-divergences sections). A mutation test
re-compiles the C oracle with plausible mistakes planted and checks that the
pins catch every one.
"""

import math
import os
import re
import subprocess

import numpy as np
import pytest
import torch

import oracle
from oracle.brute import sdpa_brute
import sdpa_workloads as W

ORACLE_SRC = os.path.join(os.path.dirname(oracle.__file__), "sdpa_oracle.c")


def _case(seed, dtype="f32", B=1, Hq=2, Hkv=2, Sq=5, Skv=7, D=8, mask="none",
          mask_shape=None, causal=False, Dv=None, p=0.3):
    return W.make_case(seed, dtype, B, Hq, Hkv, Sq, Skv, D, mask, mask_shape, causal, Dv, p)


TINY_CASES = [
    dict(seed=1),
    dict(seed=2, causal=True),
    dict(seed=3, Sq=9, Skv=4, causal=True),            # Sq > Skv, top-left causal
    dict(seed=4, Sq=3, Skv=9, causal=True),            # Sq < Skv
    dict(seed=5, mask="bool"),
    dict(seed=6, mask="bool", mask_shape=(1, 1, 5, 7)),
    dict(seed=7, mask="bool", mask_shape=(1, 2, 1, 7)),
    dict(seed=8, mask="add"),
    dict(seed=9, mask="add", mask_shape=(7,)),
    dict(seed=10, mask="neginf", p=0.6),
    dict(seed=11, Hq=4, Hkv=2),                        # GQA, 2 query heads per KV head
    dict(seed=12, Hq=4, Hkv=1, mask="bool", B=2),
    dict(seed=13, Hq=6, Hkv=2, causal=True, Sq=6, Skv=6, D=4),
    dict(seed=14, D=3, Dv=5),                          # D_v != D_qk
    dict(seed=15, Sq=1, Skv=1),
    dict(seed=16, mask="bool", p=0.9, Sq=6),           # some rows fully masked
    dict(seed=17, dtype="bf16", causal=True, Sq=8, Skv=8),
    dict(seed=18, dtype="f16", mask="add", Hq=4, Hkv=2),
]


def _call(fn, c, scale=None):
    gqa = c["q"].shape[1] != c["k"].shape[1]
    return fn(c["q"], c["k"], c["v"], c["mask"], c["causal"], scale, gqa)


@pytest.mark.parametrize("spec", TINY_CASES, ids=lambda s: "-".join(f"{k}{v}" for k, v in s.items()))
def test_oracle_matches_brute_force(spec):
    c = _case(**spec)
    for scale in (None, 0.37):
        o1, p1, l1 = _call(oracle.sdpa_reference, c, scale)
        o2, p2, l2 = _call(sdpa_brute, c, scale)
        np.testing.assert_allclose(p1, p2, rtol=0, atol=1e-13)
        np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-12)
        np.testing.assert_array_equal(np.isneginf(l1), np.isneginf(l2))
        fin = np.isfinite(l2)
        np.testing.assert_allclose(l1[fin], l2[fin], rtol=0, atol=1e-12)
        # masked positions are exactly zero in both
        np.testing.assert_array_equal(p1 == 0, p2 == 0)


def _scores(q, k, scale, gqa_group):
    q = np.asarray(q.to(torch.float64))
    k = np.asarray(k.to(torch.float64))
    k = np.repeat(k, gqa_group, axis=1)
    return scale * (q @ np.swapaxes(k, -1, -2))


def _masked_scores(c, scale):
    q, k, mask = c["q"], c["k"], c["mask"]
    g = q.shape[1] // k.shape[1]
    s = _scores(q, k, scale, g)
    Sq, Skv = s.shape[-2:]
    if c["causal"]:
        s = np.where(np.triu(np.ones((Sq, Skv), bool), 1), -np.inf, s)
    if mask is not None:
        m = np.asarray(mask) if mask.dtype == torch.bool else np.asarray(mask.to(torch.float64))
        s = np.where(m, s, -np.inf) if m.dtype == np.bool_ else s + m
    return s


def _check_invariants(c, o, p, lse, scale):
    from scipy.special import logsumexp
    g = c["q"].shape[1] // c["k"].shape[1]
    v = np.repeat(np.asarray(c["v"].to(torch.float64)), g, axis=1)
    s = _masked_scores(c, scale)
    dead = np.all(np.isneginf(s), axis=-1)
    rows = p.sum(-1)
    # rows of P sum to one, or are all zero when every key is removed
    np.testing.assert_allclose(rows[~dead], 1.0, rtol=0, atol=1e-12)
    assert np.all(p[dead] == 0) and np.all(o[dead] == 0) and np.all(np.isneginf(lse[dead]))
    # removed positions are exactly +0.0
    assert np.all(p[np.isneginf(s)] == 0)
    assert not np.any(np.signbit(p))
    # O = P V, recomputed with a library matmul
    np.testing.assert_allclose(o, p @ v, rtol=0, atol=1e-11)
    # LSE = log sum exp of the scaled, masked scores (library logsumexp)
    ref = logsumexp(s, axis=-1)
    np.testing.assert_allclose(lse[~dead], ref[~dead], rtol=0, atol=1e-11)
    # exact-P identity P = exp(s - LSE) on live rows
    live = ~dead
    np.testing.assert_allclose(p[live], np.exp(s[live] - lse[live][..., None]), rtol=0, atol=1e-13)


def _head_slice(inp, b, h0, nh):
    """Batch b, query heads h0..h0+nh-1 and the KV heads they read."""
    q, k, v, m = inp["q"], inp["k"], inp["v"], inp["mask"]
    g = q.shape[1] // k.shape[1]
    assert h0 % g == 0 and nh % g == 0
    out = {"q": q[b:b + 1, h0:h0 + nh], "k": k[b:b + 1, h0 // g:(h0 + nh) // g],
           "v": v[b:b + 1, h0 // g:(h0 + nh) // g], "mask": None}
    if m is not None:
        mb = m[b:b + 1] if m.shape[0] > 1 else m
        out["mask"] = mb[:, h0:h0 + nh] if mb.shape[1] > 1 else mb
    return out


@pytest.mark.parametrize("w", W.WORKLOADS, ids=lambda w: w.name)
def test_oracle_invariants_on_workloads(w):
    inp = W.make_inputs(w)
    g = w.Hq // w.Hkv
    nh = min(w.Hq, max(2, g))
    c = _head_slice(inp, 0, 0, nh)
    c["causal"] = w.causal
    o, p, lse = oracle.sdpa_reference(c["q"], c["k"], c["v"], c["mask"], w.causal, w.scale, w.gqa)
    _check_invariants(c, o, p, lse, w.scale)
    if w.causal:
        assert np.all(np.triu(p, 1) == 0)
    if w.mask == "keypad_bool":
        # batch 0, query rows 0-7 are fully masked: P = O = 0, LSE = -inf
        assert np.all(p[0, :, :8] == 0) and np.all(o[0, :, :8] == 0)
        assert np.all(np.isneginf(lse[0, :, :8]))


def test_workload_recipes():
    w4 = W.BY_NAME["gqa_1k_d128_f16_keypad"]
    m = W.make_inputs(w4)["mask"]
    assert m.shape == (4, 1, 1024, 1024) and m.dtype == torch.bool
    lens = m[:, 0, 100].sum(-1)
    assert torch.all((lens >= 512) & (lens <= 1024))
    assert not m[0, 0, :8].any() and m[0, 0, 8].any()
    w5 = W.BY_NAME["decode_100x1152_d64_f16_addmask"]
    m5 = W.make_inputs(w5)["mask"]
    frac = torch.isneginf(m5).double().mean().item()
    assert m5.dtype == torch.float16 and abs(frac - 0.10) < 0.002
    assert set(torch.unique(m5[torch.isfinite(m5)]).tolist()) == {0.0}
    # same seed, same numbers
    a, b = W.make_inputs(W.WORKLOADS[0]), W.make_inputs(W.WORKLOADS[0])
    assert torch.equal(a["q"], b["q"]) and torch.equal(a["v"], b["v"])


# ---------------------------------------------------------------- closed forms

def test_closed_form_worked_example():
    # One query (1,0), keys (0,0) and (ln 3, 0), scale 1: scores 0 and ln 3, so
    # P = (1/4, 3/4), LSE = ln 4, and with values 4 and 8, O = 1 + 6 = 7.
    q = np.array([[[[1.0, 0.0]]]])
    k = np.array([[[[0.0, 0.0], [math.log(3.0), 0.0]]]])
    v = np.array([[[[4.0], [8.0]]]])
    o, p, lse = oracle.sdpa_reference(q, k, v, scale=1.0)
    np.testing.assert_allclose(p[0, 0, 0], [0.25, 0.75], rtol=0, atol=1e-15)
    np.testing.assert_allclose(lse[0, 0, 0], math.log(4.0), rtol=0, atol=1e-15)
    np.testing.assert_allclose(o[0, 0, 0, 0], 7.0, rtol=0, atol=1e-14)


@pytest.mark.parametrize("mask", ["none", "bool", "neginf"])
def test_closed_form_zero_query_is_uniform(mask):
    c = _case(21, B=2, Hq=4, Hkv=2, Sq=6, Skv=9, D=8, mask=mask, p=0.4)
    c["q"] = torch.zeros_like(c["q"])
    o, p, lse = _call(oracle.sdpa_reference, c)
    s = _masked_scores(c, 1 / math.sqrt(8))
    keep = ~np.isneginf(s)
    n = keep.sum(-1)
    v = np.repeat(np.asarray(c["v"].double()), 2, axis=1)
    live = n > 0
    np.testing.assert_allclose(p[live], (keep / np.maximum(n, 1)[..., None])[live], rtol=0, atol=1e-15)
    np.testing.assert_allclose(lse[live], np.log(n[live]), rtol=0, atol=1e-14)
    mean_v = (keep[..., None] * v[:, :, None, :, :]).sum(-2) / np.maximum(n, 1)[..., None]
    np.testing.assert_allclose(o[live], mean_v[live], rtol=0, atol=1e-14)


def test_closed_form_equal_keys_is_uniform():
    c = _case(22, Sq=4, Skv=6, D=8)
    c["k"] = c["k"][:, :, :1].expand(-1, -1, 6, -1).contiguous()
    o, p, lse = _call(oracle.sdpa_reference, c)
    np.testing.assert_allclose(p, 1 / 6, rtol=0, atol=1e-15)
    s0 = _scores(c["q"], c["k"], 1 / math.sqrt(8), 1)[..., 0]
    np.testing.assert_allclose(lse, s0 + math.log(6), rtol=0, atol=1e-13)


def test_closed_form_single_key():
    c = _case(23, Sq=5, Skv=1, D=8)
    o, p, lse = _call(oracle.sdpa_reference, c)
    assert np.all(p == 1.0)
    np.testing.assert_array_equal(o, np.broadcast_to(np.asarray(c["v"].double()), o.shape))
    np.testing.assert_allclose(lse, _scores(c["q"], c["k"], 1 / math.sqrt(8), 1)[..., 0], atol=1e-14, rtol=0)


def test_closed_form_causal_first_row():
    c = _case(24, Sq=6, Skv=6, causal=True)
    o, p, lse = _call(oracle.sdpa_reference, c)
    assert np.all(p[:, :, 0, 0] == 1.0) and np.all(p[:, :, 0, 1:] == 0)
    np.testing.assert_array_equal(o[:, :, 0], np.asarray(c["v"].double())[:, :, 0])


def test_closed_form_two_keys_is_logistic():
    c = _case(25, Sq=7, Skv=2, D=8)
    o, p, lse = _call(oracle.sdpa_reference, c)
    s = _scores(c["q"], c["k"], 1 / math.sqrt(8), 1)
    sig = 1.0 / (1.0 + np.exp(s[..., 1] - s[..., 0]))
    np.testing.assert_allclose(p[..., 0], sig, rtol=0, atol=1e-15)


def test_dead_rows_and_empty_keys():
    c = _case(26, Sq=4, Skv=5, mask="bool", p=0.0)
    c["mask"][0, 1, 2, :] = False
    o, p, lse = _call(oracle.sdpa_reference, c)
    assert np.all(p[0, 1, 2] == 0) and np.all(o[0, 1, 2] == 0) and np.isneginf(lse[0, 1, 2])
    assert np.all(np.isfinite(np.delete(lse.reshape(-1), 1 * 4 + 2)))
    c0 = _case(27, Sq=3, Skv=0)
    o, p, lse = _call(oracle.sdpa_reference, c0)
    assert p.shape[-1] == 0 and np.all(o == 0) and np.all(np.isneginf(lse))


# ---------------------------------------------------------------- equivalences

def test_all_true_bool_mask_is_no_mask():
    c = _case(31, Sq=6, Skv=8)
    a = _call(oracle.sdpa_reference, c)
    c["mask"] = torch.ones(1, 1, 6, 8, dtype=torch.bool)
    b = _call(oracle.sdpa_reference, c)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)


def test_bool_mask_equals_neginf_float_mask():
    c = _case(32, Sq=6, Skv=8, mask="bool", p=0.4)
    a = _call(oracle.sdpa_reference, c)
    c["mask"] = torch.where(c["mask"], 0.0, -math.inf).double()
    b = _call(oracle.sdpa_reference, c)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)


# ---------------------------------------------------------------- bottom-right causal
# (query i keeps keys j <= i + Skv - Sq: the alignment of a query chunk against
# a longer key cache, cudnn-frontend merge-log notes)

@pytest.mark.parametrize("spec", [
    dict(seed=71, Sq=5, Skv=7), dict(seed=72, Sq=9, Skv=4), dict(seed=73, Sq=3, Skv=9),
    dict(seed=74, Sq=6, Skv=6), dict(seed=75, Hq=4, Hkv=2, Sq=4, Skv=10, D=5, Dv=3),
], ids=lambda s: "-".join(f"{k}{v}" for k, v in s.items()))
def test_bottom_right_matches_brute_force(spec):
    c = _case(causal=True, **spec)
    gqa = c["q"].shape[1] != c["k"].shape[1]
    a = oracle.sdpa_reference(c["q"], c["k"], c["v"], None, True, 0.41, gqa, causal_alignment="bottom_right")
    b = sdpa_brute(c["q"], c["k"], c["v"], None, True, 0.41, gqa, causal_alignment="bottom_right")
    np.testing.assert_allclose(a[1], b[1], rtol=0, atol=1e-13)
    np.testing.assert_allclose(a[0], b[0], rtol=0, atol=1e-12)
    np.testing.assert_array_equal(np.isneginf(a[2]), np.isneginf(b[2]))
    fin = np.isfinite(b[2])
    np.testing.assert_allclose(a[2][fin], b[2][fin], rtol=0, atol=1e-12)
    np.testing.assert_array_equal(a[1] == 0, b[1] == 0)


@pytest.mark.parametrize("sq,skv", [(6, 6), (9, 4), (3, 9), (1, 8)])
def test_bottom_right_equals_shifted_tril_bool_mask(sq, skv):
    c = _case(34, Sq=sq, Skv=skv, causal=True)
    a = oracle.sdpa_reference(c["q"], c["k"], c["v"], None, True, causal_alignment="bottom_right")
    keep = torch.ones(sq, skv, dtype=torch.bool).tril(diagonal=skv - sq)
    b = oracle.sdpa_reference(c["q"], c["k"], c["v"], keep, False)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)


def test_bottom_right_closed_forms():
    # square: the same as top-left
    c = _case(35, Sq=7, Skv=7, causal=True)
    a = oracle.sdpa_reference(c["q"], c["k"], c["v"], None, True, causal_alignment="bottom_right")
    b = oracle.sdpa_reference(c["q"], c["k"], c["v"], None, True)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)
    # a chunk against a longer cache: the last row keeps every key (the
    # non-causal row); row i keeps exactly i + Skv - Sq + 1 keys
    c = _case(36, Sq=3, Skv=8, causal=True)
    o, p, lse = oracle.sdpa_reference(c["q"], c["k"], c["v"], None, True, causal_alignment="bottom_right")
    on, pn, ln = oracle.sdpa_reference(c["q"], c["k"], c["v"], None, False)
    np.testing.assert_array_equal(p[:, :, -1], pn[:, :, -1])
    np.testing.assert_array_equal(o[:, :, -1], on[:, :, -1])
    for i in range(3):
        assert ((p[:, :, i] > 0).sum(axis=-1) == i + 5 + 1).all()
        assert (p[:, :, i, i + 6:] == 0).all()
    # more queries than keys: rows i < Sq - Skv keep no key (dead rows)
    c = _case(37, Sq=9, Skv=4, causal=True)
    o, p, lse = oracle.sdpa_reference(c["q"], c["k"], c["v"], None, True, causal_alignment="bottom_right")
    assert (p[:, :, :5] == 0).all() and (o[:, :, :5] == 0).all() and np.isneginf(lse[:, :, :5]).all()
    np.testing.assert_allclose(p[:, :, 5:].sum(-1), 1.0, rtol=0, atol=1e-12)
    with pytest.raises(ValueError):
        oracle.sdpa_reference(c["q"], c["k"], c["v"], None, True, causal_alignment="middle")


@pytest.mark.parametrize("sq,skv", [(6, 6), (9, 4), (3, 9)])
def test_causal_equals_tril_bool_mask(sq, skv):
    c = _case(33, Sq=sq, Skv=skv, causal=True)
    a = _call(oracle.sdpa_reference, c)
    c["causal"] = False
    c["mask"] = torch.ones(sq, skv, dtype=torch.bool).tril()
    b = _call(oracle.sdpa_reference, c)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)


def test_gqa_equals_repeated_kv():
    c = _case(34, B=2, Hq=6, Hkv=2, Sq=5, Skv=7, mask="bool")
    a = _call(oracle.sdpa_reference, c)
    c["k"] = c["k"].repeat_interleave(3, dim=1)
    c["v"] = c["v"].repeat_interleave(3, dim=1)
    b = _call(oracle.sdpa_reference, c)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)


# ---------------------------------------------------------------- library cross-check

@pytest.mark.parametrize("spec", [
    dict(seed=41, Sq=7, Skv=11, D=16),
    dict(seed=42, Sq=9, Skv=9, D=16, causal=True),
    dict(seed=43, Sq=5, Skv=13, D=16, mask="add", p=0.2),
    dict(seed=44, B=2, Hq=4, Hkv=2, Sq=6, Skv=10, D=8, mask="add", p=0.0),
])
def test_matches_torch_cpu_math_backend(spec):
    """torch's CPU math backend in float64, on float masks without dead rows
    (its direct call treats bool masks differently, which the FlagOS-OP page
    lists as an intentional divergence)."""
    c = _case(**spec)
    gqa = c["q"].shape[1] != c["k"].shape[1]
    mask = c["mask"]
    if mask is not None:
        assert not torch.isneginf(mask).all(-1).any()
    o, p, lse = _call(oracle.sdpa_reference, c)
    to, tp = torch.ops.aten._scaled_dot_product_attention_math(
        c["q"].double(), c["k"].double(), c["v"].double(),
        None if mask is None else mask.double(), 0.0, c["causal"], None, enable_gqa=gqa)
    np.testing.assert_allclose(p, tp.numpy(), rtol=0, atol=1e-13)
    np.testing.assert_allclose(o, to.numpy(), rtol=0, atol=1e-12)


# ---------------------------------------------------------------- error rules

def test_semantic_errors():
    c = _case(51, Hq=3, Hkv=2)
    with pytest.raises(ValueError):
        _call(oracle.sdpa_reference, c)
    c = _case(52, Hq=4, Hkv=2)
    with pytest.raises(ValueError):  # GQA layout without the flag
        oracle.sdpa_reference(c["q"], c["k"], c["v"], None, False, None, False)
    c = _case(53, mask="bool")
    with pytest.raises(ValueError):
        oracle.sdpa_reference(c["q"], c["k"], c["v"], c["mask"], True)
    for fn in (sdpa_brute,):
        with pytest.raises(ValueError):
            fn(c["q"], c["k"], c["v"], c["mask"], True)


# ---------------------------------------------------------------- mutation test

def _pins_pass(lib_path):
    """Run a compact set of the pins above against an oracle build."""
    ok = True
    for spec in (dict(seed=61, Hq=4, Hkv=2, Sq=6, Skv=6, causal=True),
                 dict(seed=62, Hq=4, Hkv=2, mask="bool", p=0.5, Sq=8),
                 dict(seed=63, mask="add"), dict(seed=64, Sq=4, Skv=9, D=6, Dv=3),
                 dict(seed=65, mask="bool", p=0.2),
                 dict(seed=66, Sq=4, Skv=9, causal=True, align="bottom_right")):
        c = _case(**{k: x for k, x in spec.items() if k != "align"})
        if spec["seed"] == 65:
            c["mask"][0, 1, 3, :] = False  # one dead row
        gqa = c["q"].shape[1] != c["k"].shape[1]
        al = spec.get("align", "top_left")
        a = oracle.sdpa_reference(c["q"], c["k"], c["v"], c["mask"], c["causal"], None, gqa,
                                  lib_path=lib_path, causal_alignment=al)
        b = sdpa_brute(c["q"], c["k"], c["v"], c["mask"], c["causal"], None, gqa, causal_alignment=al)
        for x, y in zip(a, b):
            same_inf = np.array_equal(np.isneginf(x), np.isneginf(y))
            fin = np.isfinite(y)
            if not same_inf or not np.allclose(x[fin], y[fin], rtol=0, atol=1e-12):
                ok = False
    return ok


MUTANTS = [
    ("dropped scale", "double s = scale * dot;", "double s = dot;"),
    ("GQA head index", "const int64_t hk = h / group;", "const int64_t hk = h % Hkv;"),
    ("causal diagonal", "if (is_causal && j > i + coff)", "if (is_causal && j >= i + coff)"),
    ("bottom-right offset sign", "is_causal == 2 ? Skv - Sq : 0;", "is_causal == 2 ? Sq - Skv : 0;"),
    ("bool polarity", "((const uint8_t*)mask)[off] == 0)", "((const uint8_t*)mask)[off] != 0)"),
    ("additive sign", "s += ((const double*)mask)[off];", "s -= ((const double*)mask)[off];"),
    ("LSE missing log-sum", "const double L = m + log(l);", "const double L = m;"),
    ("dead-row LSE", "lse[row] = -INFINITY;", "lse[row] = 0.0;"),
    ("transposed V index", "acc += p[j] * vh[j * Dv + d];", "acc += p[j] * vh[(j * Dv + d) % Dv];"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_planted_mistakes(tmp_path, name, old, new):
    src = open(ORACLE_SRC).read()
    cut = src.index("int oracle_sdpa_bwd(")  # plant it in the forward only
    fwd, rest = src[:cut], src[cut:]
    assert fwd.count(old) == 1, name
    mutant_src = tmp_path / "mutant.c"
    mutant_src.write_text(fwd.replace(old, new) + rest)
    lib = str(tmp_path / "libmutant.so")
    oracle.build(force=True, src=str(mutant_src), out=lib)
    assert not _pins_pass(lib), f"planted mistake '{name}' went unnoticed"


def test_pins_pass_on_unmutated_oracle():
    assert _pins_pass(oracle.build(force=False))
