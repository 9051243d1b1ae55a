"""Pins for the oracle's dropout (no GPU): the FlagOS-OP page's two dropout
rules (Implementation section: explicit and random; Intentional divergences:
with dropout the output is the dropped probabilities times V).

  explicit: P_out = keep * P,          O = (keep * P) V / (1 - p)
  random:   P_out = keep * P / (1 - p), O = P_out V

Tied to: an independent brute force; torch's CPU math backend, whose
dropout_mask argument applies the explicit rule; equivalences (both rules
give the same O; p = 0 with every key kept is no dropout; keeping nothing
zeroes P and O but not LSE); and planted mistakes in the C code.
"""

import os

import numpy as np
import pytest
import torch

import oracle
from oracle.brute import sdpa_brute
import sdpa_workloads as W

ORACLE_SRC = os.path.join(os.path.dirname(oracle.__file__), "sdpa_oracle.c")


def _case(seed, Sq=5, Skv=7, D=6, Hq=2, Hkv=2, B=1, mask="none", causal=False, keep_shape=None, keep_p=0.7):
    c = W.make_case(seed, "f32", B, Hq, Hkv, Sq, Skv, D, mask, None, causal)
    g = np.random.default_rng(seed + 500)
    shape = keep_shape or (B, Hq, Sq, Skv)
    c["keep"] = torch.from_numpy(g.random(shape) < keep_p)
    return c


def _ref(c, p, rule, fn=oracle.sdpa_reference, **kw):
    gqa = c["q"].shape[1] != c["k"].shape[1]
    return fn(c["q"], c["k"], c["v"], c["mask"], c["causal"], None, gqa, dropout_p=p, dropout_mask=c["keep"],
              dropout_rule=rule, **kw)


SPECS = [dict(seed=1), dict(seed=2, causal=True, Sq=6, Skv=6), dict(seed=3, mask="bool"), dict(seed=4, mask="add"),
         dict(seed=5, Hq=4, Hkv=2), dict(seed=6, keep_shape=(1, 1, 5, 7)), dict(seed=7, keep_shape=(7,)),
         dict(seed=8, keep_p=0.2, Sq=3, Skv=9)]


@pytest.mark.parametrize("rule", ["explicit", "random"])
@pytest.mark.parametrize("spec", SPECS, ids=lambda s: "-".join(f"{k}{v}" for k, v in s.items()))
def test_dropout_matches_brute_force(spec, rule):
    c = _case(**spec)
    for x, y in zip(_ref(c, 0.3, rule), _ref(c, 0.3, rule, sdpa_brute)):
        fin = np.isfinite(y)
        assert np.array_equal(np.isneginf(x), np.isneginf(y))
        assert np.allclose(x[fin], y[fin], rtol=0, atol=1e-12)


@pytest.mark.parametrize("spec", [dict(seed=11), dict(seed=12, causal=True, Sq=6, Skv=6), dict(seed=13, mask="add"),
                                  dict(seed=14, keep_p=0.5, Sq=8)])
def test_explicit_rule_matches_torch_math_backend(spec):
    c = _case(**spec)
    o, p, _ = _ref(c, 0.25, "explicit")
    m = c["mask"]
    if m is not None and m.dtype != torch.bool:
        m = m.double()
    to, tp = torch.ops.aten._scaled_dot_product_attention_math(
        c["q"].double(), c["k"].double(), c["v"].double(), m, 0.25, c["causal"], c["keep"])
    assert np.allclose(p, tp.numpy(), atol=1e-13) and np.allclose(o, to.numpy(), atol=1e-13)


def test_dropout_rules_and_special_cases():
    c = _case(21, mask="bool")
    o_e, p_e, l_e = _ref(c, 0.4, "explicit")
    o_r, p_r, l_r = _ref(c, 0.4, "random")
    o0, p0, l0 = oracle.sdpa_reference(c["q"], c["k"], c["v"], c["mask"])
    keep = c["keep"].numpy()
    # both rules: same O, P differing by the factor 1 / (1 - p), LSE of the undropped softmax
    assert np.allclose(o_e, o_r, atol=1e-13) and np.allclose(p_r, p_e / 0.6, atol=1e-13)
    assert np.array_equal(l_e, l0) and np.array_equal(l_r, l0)
    # explicit rule: the kept probabilities untouched, the removed ones exactly 0
    assert np.array_equal(p_e, np.where(keep, p0, 0.0))
    assert np.allclose(o_e, (p_e @ c["v"].double().numpy()) / 0.6, atol=1e-13)
    # p = 0 with every key kept is no dropout
    c1 = dict(c, keep=torch.ones_like(c["keep"]))
    for rule in ("explicit", "random"):
        for x, y in zip(_ref(c1, 0.0, rule), (o0, p0, l0)):
            assert np.array_equal(x, y)
    # keeping nothing: P = O = 0, LSE unchanged
    c2 = dict(c, keep=torch.zeros_like(c["keep"]))
    o2, p2, l2 = _ref(c2, 0.4, "random")
    assert np.all(p2 == 0) and np.all(o2 == 0) and np.array_equal(l2, l0)


def test_dropout_errors():
    c = _case(31)
    for bad_p in (1.0, -0.1):
        with pytest.raises(ValueError):
            _ref(c, bad_p, "explicit")
    with pytest.raises(ValueError):
        _ref(c, 0.1, "sometimes")


def _pins_pass(lib_path):
    ok = True
    for spec, rule in ((dict(seed=41, mask="bool"), "explicit"), (dict(seed=42, causal=True, Sq=6, Skv=6), "random"),
                       (dict(seed=43, keep_shape=(1, 2, 1, 7)), "explicit"), (dict(seed=44, Hq=4, Hkv=2), "random")):
        c = _case(**spec)
        for x, y in zip(_ref(c, 0.3, rule, lib_path=lib_path), _ref(c, 0.3, rule, sdpa_brute)):
            fin = np.isfinite(y)
            if not np.array_equal(np.isneginf(x), np.isneginf(y)) or not np.allclose(x[fin], y[fin], atol=1e-12):
                ok = False
    return ok


DROP_MUTANTS = [
    ("explicit O not rescaled", "                oscale = inv;", "                oscale = 1.0;"),
    ("random P not rescaled", "                    p[j] *= inv;", "                    p[j] *= 1.0;"),
    ("kept and removed swapped", "if (keep[off] == 0)", "if (keep[off] != 0)"),
    ("keep mask row index", "i * keep_strides[2] + j * keep_strides[3];", "(Sq - 1 - i) * keep_strides[2] + j * keep_strides[3];"),
]


@pytest.mark.parametrize("name,old,new", DROP_MUTANTS, ids=[m[0] for m in DROP_MUTANTS])
def test_dropout_pins_catch_planted_mistakes(tmp_path, name, old, new):
    src = open(ORACLE_SRC).read()
    assert src.count(old) == 1, name
    mutant = tmp_path / "mutant.c"
    mutant.write_text(src.replace(old, new))
    lib = str(tmp_path / "libmutant.so")
    oracle.build(force=True, src=str(mutant), out=lib)
    assert not _pins_pass(lib), f"planted mistake '{name}' went unnoticed"


def test_dropout_pins_pass_on_unmutated_oracle():
    assert _pins_pass(oracle.build(force=False))
