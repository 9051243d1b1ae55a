"""GPU parity: the HIP path through the C ABI against the float64 oracle.

Every case pre-poisons the outputs with NaN, runs ``sdpa_math_fwd_path`` on
the MI355X, and compares O, P and LSE element by element with the oracle on
the same seeded inputs (max-abs bounds per dtype, +0.0 bit pattern at every
removed position, LSE = -inf exactly on dead rows).
"""

import contextlib
import math
import os
import re

import numpy as np
import pytest
import torch

import sdpa_workloads as W
from parity import TOL_OP, compare, head_slice, poisoned_outputs, run_oracle

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
# "fused": the fused path as the planner configures it (its wide kernel
# wherever that fits); "fused1": the fused path held to its one-row-group
# kernel; "fusedw": held to the wide kernel (skipped where it cannot fit);
# "ranges": the default plan with the wide kernel's one-sweep key ranges
# forced wherever they fit (64-key ranges, one key group per row group, so
# that small calls span several ranges)
PATHS = ["twopass", "fused", "fused1", "ranges"]
_PATH_ENV = {"fused1": {"SDPA_MATH_FUSED_WIDE": "0"}, "fusedw": {"SDPA_MATH_FUSED_WIDE": "1"},
             "ranges": {"SDPA_MATH_RANGES": "1", "SDPA_MATH_RANGE_KEYS": "64", "SDPA_MATH_RANGE_WAVES": "1"}}
_BINDING_PATH = {"fused1": "fused", "fusedw": "fused", "ranges": "auto"}


@contextlib.contextmanager
def _path_env(path):
    """Environment of a test path name; yields the binding's path argument."""
    env = _PATH_ENV.get(path, {})
    saved = {k: os.environ.get(k) for k in env}
    os.environ.update(env)
    try:
        yield _BINDING_PATH.get(path, path)
    finally:
        for k, val in saved.items():
            if val is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = val


def _lib():
    import sdpa_forward_materialised_amd as S
    S.load_library()
    return S


def _fwd(path, *args, **kw):
    """S.fwd with a test path name (see PATHS)."""
    S = _lib()
    with _path_env(path) as p:
        return S.fwd(*args, path=p, **kw)


def _run(c, path, scale=None, gqa=None, label=""):
    S = _lib()
    q, k, v, m = c["q"], c["k"], c["v"], c["mask"]
    B, Hq, Sq, D = q.shape
    Skv, Dv = k.shape[2], v.shape[3]
    if gqa is None:
        gqa = q.shape[1] != k.shape[1]
    out = poisoned_outputs(B, Hq, Sq, Skv, Dv, q.dtype, DEV)
    print(f"[case] {label} path={path} shape={tuple(q.shape)}x{tuple(k.shape)} mask="
          f"{None if m is None else (tuple(m.shape), m.dtype)} causal={c['causal']}", flush=True)
    gm = None if m is None else m.to(DEV)
    try:
        with _path_env(path) as p:
            O, P, L = S.fwd(q.to(DEV), k.to(DEV), v.to(DEV), gm, c["causal"], scale, gqa, path=p, out=out,
                            causal_alignment=c.get("align", "top_left"))
    except NotImplementedError as e:
        if path.startswith("fused"):
            pytest.skip(f"the fused path cannot take this shape: {e}")
        raise
    torch.cuda.synchronize()
    return O, P, L


def _check(c, path, scale=None, label=""):
    O, P, L = _run(c, path, scale, label=label)
    gqa = c["q"].shape[1] != c["k"].shape[1]
    ref = run_oracle(c["q"], c["k"], c["v"], c["mask"], c["causal"], scale, gqa, c.get("align", "top_left"))
    return compare(O, P, L, ref, c["q"].dtype, label, v=c["v"])


# ------------------------------------------------------------ small cases, full oracle

SMALL = [
    # (label, make_case kwargs)
    ("f16-d64-causal-ragged", dict(seed=101, dtype="f16", B=2, Hq=3, Hkv=3, Sq=150, Skv=150, D=64, causal=True)),
    ("bf16-d128-causal-sq<skv", dict(seed=102, dtype="bf16", B=1, Hq=2, Hkv=2, Sq=70, Skv=200, D=128, causal=True)),
    ("bf16-d128-causal-sq>skv", dict(seed=103, dtype="bf16", B=1, Hq=2, Hkv=2, Sq=200, Skv=70, D=128, causal=True)),
    ("f32-d32-causal", dict(seed=104, dtype="f32", B=1, Hq=2, Hkv=2, Sq=64, Skv=64, D=32, causal=True)),
    ("f32-d64-nomask-ragged", dict(seed=105, dtype="f32", B=2, Hq=2, Hkv=2, Sq=77, Skv=131, D=64)),
    ("f32-d128-bool", dict(seed=106, dtype="f32", B=1, Hq=2, Hkv=1, Sq=96, Skv=100, D=128, mask="bool")),
    ("f16-d32-bool-bcast", dict(seed=107, dtype="f16", B=2, Hq=4, Hkv=2, Sq=65, Skv=129, D=32, mask="bool",
                                mask_shape=(1, 1, 65, 129))),
    ("f16-d128-keypad", dict(seed=108, dtype="f16", B=2, Hq=8, Hkv=2, Sq=128, Skv=192, D=128, mask="bool",
                             mask_shape=(2, 1, 1, 192), p=0.3)),
    ("bf16-d64-add", dict(seed=109, dtype="bf16", B=2, Hq=2, Hkv=2, Sq=100, Skv=300, D=64, mask="add", p=0.1)),
    ("f16-d64-neginf-heads", dict(seed=110, dtype="f16", B=1, Hq=4, Hkv=4, Sq=33, Skv=1152, D=64, mask="neginf",
                                  mask_shape=(1, 4, 33, 1152))),
    ("f32-d32-add-bcast-key", dict(seed=111, dtype="f32", B=2, Hq=2, Hkv=2, Sq=40, Skv=90, D=32, mask="add",
                                   mask_shape=(90,), p=0.2)),
    ("bf16-d32-single", dict(seed=112, dtype="bf16", B=1, Hq=1, Hkv=1, Sq=1, Skv=1, D=32)),
    ("f16-d128-decode-row", dict(seed=113, dtype="f16", B=3, Hq=8, Hkv=8, Sq=1, Skv=1025, D=128)),
    ("f16-d64-odd-skv", dict(seed=114, dtype="f16", B=1, Hq=2, Hkv=2, Sq=50, Skv=37, D=64, mask="bool")),
    ("f32-d64-add-staged", dict(seed=116, dtype="f32", B=1, Hq=2, Hkv=2, Sq=100, Skv=136, D=64, mask="add", p=0.1)),
    ("f32-d32-add-full-staged", dict(seed=117, dtype="f32", B=2, Hq=2, Hkv=1, Sq=70, Skv=200, D=32, mask="add", p=0.2)),
    ("bf16-d64-add-rows-shared", dict(seed=115, dtype="bf16", B=2, Hq=4, Hkv=2, Sq=150, Skv=264, D=64, mask="add",
                                      mask_shape=(2, 1, 1, 264), p=0.2)),
]


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("label,spec", SMALL, ids=[s[0] for s in SMALL])
def test_small_cases(label, spec, path):
    c = W.make_case(**spec)
    _check(c, path, label=label)


# The wide fused kernel with two and four 32-row groups per workgroup (grids
# of at least 256 workgroups), causal and GQA, ragged row groups, masks of
# each kind, and a layout without 16-byte rows (element loads and stores).
WIDE = [
    ("wide-rg2-f16-d64-add", dict(seed=201, dtype="f16", B=32, Hq=8, Hkv=8, Sq=64, Skv=300, D=64, mask="add", p=0.1)),
    ("wide-rg2-f16-d64-add-ragged", dict(seed=202, dtype="f16", B=16, Hq=8, Hkv=8, Sq=100, Skv=520, D=64,
                                         mask="neginf", p=0.1)),
    ("wide-rg4-bf16-d128", dict(seed=203, dtype="bf16", B=64, Hq=8, Hkv=8, Sq=128, Skv=160, D=128)),
    ("wide-rg2-f32-d32-causal", dict(seed=204, dtype="f32", B=32, Hq=8, Hkv=8, Sq=64, Skv=64, D=32, causal=True)),
    ("wide-rg2-bf16-d64-gqa-bool", dict(seed=205, dtype="bf16", B=16, Hq=32, Hkv=8, Sq=40, Skv=256, D=64,
                                        mask="bool", p=0.2)),
    ("wide-rg2-f16-d32-oddskv", dict(seed=206, dtype="f16", B=32, Hq=8, Hkv=8, Sq=50, Skv=97, D=32, mask="bool")),
    ("wide-rg2-f32-d64-add", dict(seed=207, dtype="f32", B=32, Hq=8, Hkv=8, Sq=64, Skv=200, D=64, mask="add",
                                  p=0.2)),
]


@pytest.mark.parametrize("label,spec", WIDE, ids=[s[0] for s in WIDE])
def test_fused_wide_row_groups(label, spec):
    c = W.make_case(**spec)
    _check(c, "fusedw", label=label)


# Bool key-padding masks whose tails remove whole 64-key tiles for every row a
# wave holds (those tiles are skipped), with some rows removed entirely, at
# each head dim and compute-wave count.
@pytest.mark.parametrize("waves", [2, 3, 4])
@pytest.mark.parametrize("D,dtype", [(32, "f16"), (64, "bf16"), (128, "f16")])
def test_key_padding_dead_tiles(D, dtype, waves, monkeypatch):
    monkeypatch.setenv("SDPA_MATH_TP_WAVES", str(waves))
    c = W.make_case(seed=150 + D, dtype=dtype, B=3, Hq=4, Hkv=2, Sq=200, Skv=512, D=D)
    keep = torch.zeros(3, 1, 200, 512, dtype=torch.bool)
    for b, n in enumerate((130, 300, 512)):
        keep[b, :, :, :n] = True
    keep[0, :, 40:75, :] = False   # rows with every key removed
    c["mask"] = keep
    _check(c, "twopass", label=f"keypad D={D} {dtype} waves={waves}")


# Head rows: grouped heads on the four-wave kernel without a loader wave take
# four query heads of one KV group per workgroup, on 32 shared rows. Group 4
# and 8, no mask / head-shared bool and additive masks (with dead tail tiles
# and dead rows), ragged Sq and Skv; against the oracle and bit for bit
# against the same call with head rows off (SDPA_MATH_HEAD_ROWS=0: with a
# head-shared 16-bit bool mask both take 64-key tiles with recorded classes,
# and a wave's classes depend only on its own rows). A mask with per-head
# rows keeps one head per workgroup.
HEAD_ROWS = [
    ("f16-d128-g4-keypad", dict(seed=190, dtype="f16", B=2, Hq=8, Hkv=2, Sq=200, Skv=320, D=128), "keypad"),
    ("bf16-d64-g8-none", dict(seed=191, dtype="bf16", B=1, Hq=16, Hkv=2, Sq=77, Skv=136, D=64), None),
    ("f16-d32-g4-add", dict(seed=192, dtype="f16", B=2, Hq=4, Hkv=1, Sq=65, Skv=256, D=32, mask="add",
                            mask_shape=(2, 1, 65, 256), p=0.2), None),
    ("f32-d64-g4-bool", dict(seed=193, dtype="f32", B=1, Hq=8, Hkv=2, Sq=96, Skv=200, D=64, mask="bool",
                             mask_shape=(1, 1, 96, 200), p=0.3), None),
    ("f16-d64-g4-perhead", dict(seed=194, dtype="f16", B=1, Hq=4, Hkv=1, Sq=70, Skv=128, D=64, mask="bool",
                                mask_shape=(1, 4, 70, 128), p=0.3), None),
]


@pytest.mark.parametrize("label,spec,kind", HEAD_ROWS, ids=[s[0] for s in HEAD_ROWS])
def test_head_rows(label, spec, kind, monkeypatch):
    monkeypatch.setenv("SDPA_MATH_TP_WAVES", "4")
    c = W.make_case(**spec)
    if kind == "keypad":
        B, Sq, Skv = spec["B"], spec["Sq"], spec["Skv"]
        keep = torch.zeros(B, 1, Sq, Skv, dtype=torch.bool)
        for b, nk in enumerate((100, Skv)):
            keep[b, :, :, :nk] = True
        keep[0, :, 30:41, :] = False  # dead rows
        c["mask"] = keep
    on = _check(c, "twopass", label=f"{label} head rows")
    S = _lib()
    q, k, v = (c[x].to(DEV) for x in ("q", "k", "v"))
    m = None if c["mask"] is None else c["mask"].to(DEV)
    a = S.fwd(q, k, v, m, False, None, True, path="twopass")
    monkeypatch.setenv("SDPA_MATH_HEAD_ROWS", "0")
    b = S.fwd(q, k, v, m, False, None, True, path="twopass")
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    print(f"[result] {label} {on}", flush=True)


# Bool masks that every query head shares, on the four-wave kernel without a
# loader wave (64-key tiles, tile classes recorded in the statistics sweep,
# the mask read from memory for mixed tiles in the probability sweep; with
# head rows also dead tiles' K/V loads skipped): random masks (every tile
# mixed), key padding with ragged tails, fully masked rows, more than 16 and
# more than 64 tiles (the class record spans several lanes); grouped heads
# (head rows) and one KV head per query head.
CLASS_CASES = [
    ("mha-random-ragged", dict(seed=186, dtype="bf16", B=2, Hq=3, Hkv=3, Sq=150, Skv=264, D=128, mask="bool",
                               mask_shape=(2, 1, 150, 264), p=0.3), None),
    ("mha-keypad-2104", dict(seed=187, dtype="f16", B=2, Hq=2, Hkv=2, Sq=130, Skv=2104, D=64), (900, 2097)),
    ("mha-broadcast-row", dict(seed=188, dtype="f16", B=1, Hq=2, Hkv=2, Sq=200, Skv=136, D=128, mask="bool",
                               mask_shape=(1, 1, 1, 136), p=0.5), None),
    ("random-ragged", dict(seed=196, dtype="f16", B=2, Hq=8, Hkv=2, Sq=77, Skv=200, D=64, mask="bool",
                           mask_shape=(2, 1, 77, 200), p=0.3), None),
    ("keypad-2000", dict(seed=197, dtype="bf16", B=2, Hq=4, Hkv=1, Sq=96, Skv=2000, D=128), (700, 1999)),
    ("keypad-4200", dict(seed=198, dtype="f16", B=1, Hq=8, Hkv=2, Sq=40, Skv=4200, D=32), (4100,)),
    ("broadcast-row", dict(seed=199, dtype="bf16", B=1, Hq=4, Hkv=1, Sq=64, Skv=328, D=64, mask="bool",
                           mask_shape=(1, 1, 1, 328), p=0.5), None),
]


@pytest.mark.parametrize("label,spec,lens", CLASS_CASES, ids=[s[0] for s in CLASS_CASES])
def test_head_rows_bool_classes(label, spec, lens, monkeypatch):
    monkeypatch.setenv("SDPA_MATH_TP_WAVES", "4")
    c = W.make_case(**spec)
    if lens is not None:
        B, Sq, Skv = spec["B"], spec["Sq"], spec["Skv"]
        keep = torch.zeros(B, 1, Sq, Skv, dtype=torch.bool)
        for b in range(B):
            keep[b, :, :, :lens[b]] = True
        keep[0, :, 3:9, :] = False  # dead rows
        c["mask"] = keep
    r = _check(c, "twopass", label=f"{label} head rows, bool classes")
    print(f"[result] {label} {r}", flush=True)


def test_head_rows_orders(monkeypatch):
    """Head rows under every non-causal workgroup order: 16 head sets of 4 query heads, 4 query
    blocks each (64 workgroups, 8 per XCD: whole head sets per XCD, so order 5 applies); the same
    bits in each order, and the oracle's values."""
    monkeypatch.setenv("SDPA_MATH_TP_WAVES", "4")
    c = W.make_case(195, "f16", 2, 32, 8, 100, 200, 64)
    keep = torch.zeros(2, 1, 100, 200, dtype=torch.bool)
    keep[0, :, :, :120] = True
    keep[1] = True
    c["mask"] = keep
    ref = run_oracle(c["q"], c["k"], c["v"], c["mask"], False, None, True)
    outs = {}
    for sched in ("0", "4", "5"):
        monkeypatch.setenv("SDPA_MATH_SCHED", sched)
        outs[sched] = _run(c, "twopass", label=f"head rows order {sched}")
        compare(*outs[sched], ref, torch.float16, f"head rows order {sched}", v=c["v"])
    for sched in ("0", "4"):
        for x, y in zip(outs["5"], outs[sched]):
            assert torch.equal(x, y), sched


# Bottom-right causal (query i keeps keys j <= i + Skv - Sq): a query chunk
# against a longer key cache, grouped heads, more queries than keys (leading
# dead rows), ragged float32, square, a few rows against a long cache, and a
# 512-row chunk against a 2048-key cache.
BOTTOM_RIGHT = [
    ("bf16-d128-chunk-vs-cache", dict(seed=160, dtype="bf16", B=1, Hq=2, Hkv=2, Sq=130, Skv=520, D=128)),
    ("f16-d64-chunk-gqa", dict(seed=161, dtype="f16", B=2, Hq=4, Hkv=2, Sq=64, Skv=1000, D=64)),
    ("f16-d32-more-queries", dict(seed=162, dtype="f16", B=1, Hq=2, Hkv=2, Sq=150, Skv=90, D=32)),
    ("f32-d64-ragged", dict(seed=163, dtype="f32", B=1, Hq=2, Hkv=2, Sq=37, Skv=101, D=64)),
    ("bf16-d128-square", dict(seed=164, dtype="bf16", B=1, Hq=2, Hkv=2, Sq=100, Skv=100, D=128)),
    ("f16-d128-few-rows", dict(seed=165, dtype="f16", B=2, Hq=4, Hkv=4, Sq=3, Skv=776, D=128)),
    ("bf16-d128-chunk512-cache2048", dict(seed=166, dtype="bf16", B=1, Hq=4, Hkv=4, Sq=512, Skv=2048, D=128)),
]


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("label,spec", BOTTOM_RIGHT, ids=[s[0] for s in BOTTOM_RIGHT])
def test_bottom_right_causal(label, spec, path):
    c = W.make_case(causal=True, **spec)
    c["align"] = "bottom_right"
    _check(c, path, label=f"{label} bottom-right")


@pytest.mark.parametrize("waves", [2, 3, 4])
def test_bottom_right_causal_wave_counts(waves, monkeypatch):
    monkeypatch.setenv("SDPA_MATH_TP_WAVES", str(waves))
    c = W.make_case(seed=167, dtype="bf16", B=1, Hq=2, Hkv=2, Sq=300, Skv=712, D=64, causal=True)
    c["align"] = "bottom_right"
    _check(c, "twopass", label=f"bottom-right waves={waves}")


# Keys split into ranges over workgroups (statistics launch, probability
# launch, output combine; forced range counts): causal with empty ranges in
# the light blocks, bottom-right chunk, additive-mask decode rows, bool key
# padding, float32 ragged causal, grouped heads.
SPLIT_CASES = [
    ("bf16-d128-causal-296", dict(seed=170, dtype="bf16", B=1, Hq=2, Hkv=2, Sq=296, Skv=296, D=128, causal=True), None),
    ("bf16-d128-chunk-br", dict(seed=171, dtype="bf16", B=1, Hq=2, Hkv=2, Sq=130, Skv=520, D=128, causal=True),
     "bottom_right"),
    ("f16-d64-decode-add", dict(seed=172, dtype="f16", B=2, Hq=4, Hkv=4, Sq=100, Skv=1152, D=64, mask="add", p=0.1),
     None),
    ("f16-d32-keypad", dict(seed=173, dtype="f16", B=2, Hq=2, Hkv=1, Sq=70, Skv=640, D=32, mask="bool",
                            mask_shape=(2, 1, 1, 640), p=0.4), None),
    ("f32-d64-causal-ragged", dict(seed=174, dtype="f32", B=1, Hq=2, Hkv=2, Sq=77, Skv=136, D=64, causal=True), None),
    ("bf16-d64-gqa", dict(seed=175, dtype="bf16", B=1, Hq=4, Hkv=2, Sq=64, Skv=1000, D=64), None),
]


@pytest.mark.parametrize("splits", [2, 3])
@pytest.mark.parametrize("label,spec,align", SPLIT_CASES, ids=[s[0] for s in SPLIT_CASES])
def test_key_ranges(label, spec, align, splits, monkeypatch):
    monkeypatch.setenv("SDPA_MATH_SPLITS", str(splits))
    c = W.make_case(**spec)
    if align:
        c["align"] = align
    _check(c, "twopass", label=f"{label} splits={splits}")


# Key ranges in one sweep on the wide fused kernel (forced with small ranges so
# that small calls span several, the last one ragged): each range's float32
# probabilities relative to its own row maximum, its (max, sum) and its float32
# partial O, folded into P, O and LSE by the combine launch. The same shapes
# as the two-pass ranges, plus rows that every key of a range (or of the whole
# row) removes.
RANGE_CASES = SPLIT_CASES + [
    ("f16-d64-neginf-heads", dict(seed=110, dtype="f16", B=1, Hq=4, Hkv=4, Sq=33, Skv=1152, D=64, mask="neginf",
                                  mask_shape=(1, 4, 33, 1152)), None),
    ("bf16-d128-bool-dead", dict(seed=179, dtype="bf16", B=2, Hq=2, Hkv=1, Sq=40, Skv=528, D=128, mask="bool",
                                 mask_shape=(2, 1, 40, 528), p=0.3), None),
]


def _dead_ranges(c):
    # batch 0 keeps no key past 200 (whole ranges removed), batch 1 rows 3..6
    # keep no key at all (dead rows: P = O = 0, LSE = -inf)
    m = c["mask"].clone()
    m[0, :, :, 200:] = False
    m[1, :, 3:7, :] = False
    c["mask"] = m
    return c


def _ran_ranges(capfd):
    # the launch itself (SDPA_MATH_DEBUG): the fused path over more than one key range
    err = capfd.readouterr().err
    m = re.search(r"path=fused .*splits=(\d+)", err)
    assert m and int(m.group(1)) > 1, err


@pytest.mark.parametrize("keys,waves", [(64, 2), (256, 8)])
@pytest.mark.parametrize("label,spec,align", RANGE_CASES, ids=[s[0] for s in RANGE_CASES])
def test_one_sweep_key_ranges(label, spec, align, keys, waves, monkeypatch, capfd):
    monkeypatch.setenv("SDPA_MATH_DEBUG", "1")
    monkeypatch.setenv("SDPA_MATH_RANGES", "1")
    # grouped heads are the workgroup's row groups: `waves` split into them
    group = spec["Hq"] // spec["Hkv"]
    monkeypatch.setenv("SDPA_MATH_RANGE_KEYS", str(keys))
    monkeypatch.setenv("SDPA_MATH_RANGE_WAVES", str(max(1, waves // group)))
    c = W.make_case(**spec)
    if label.endswith("-dead"):
        c = _dead_ranges(c)
    if align:
        c["align"] = align
    Sq, Skv = spec["Sq"], spec["Skv"]
    last = Skv if not spec.get("causal") else min(Skv, Sq + (Skv - Sq if align == "bottom_right" else 0))
    if last <= keys:
        pytest.skip(f"the last row keeps {last} keys: one range of {keys}")
    S = _lib()
    gqa = c["q"].shape[1] != c["k"].shape[1]
    assert S.kernel_name(c["q"], c["k"], c["v"], c["mask"], c["causal"], gqa,
                         causal_alignment=c.get("align", "top_left")) == "sdpa_fused_wide_kernel"
    _check(c, "auto", label=f"{label} one-sweep ranges of {keys} keys")
    _ran_ranges(capfd)


@pytest.mark.parametrize("spec", [
    dict(seed=180, dtype="bf16", B=1, Hq=4, Hkv=4, Sq=1, Skv=8192, D=128),
    dict(seed=181, dtype="f16", B=2, Hq=4, Hkv=4, Sq=2, Skv=4096, D=128, mask="add", p=0.1),
    dict(seed=182, dtype="f32", B=1, Hq=2, Hkv=2, Sq=3, Skv=3000, D=64),
    dict(seed=183, dtype="f16", B=2, Hq=8, Hkv=2, Sq=2, Skv=4096, D=128, mask="add", p=0.1),
    dict(seed=184, dtype="bf16", B=1, Hq=16, Hkv=2, Sq=3, Skv=4000, D=64, causal=True, align="bottom_right"),
    # batched decode: enough (batch, head) pairs to fill the chip unsplit
    dict(seed=185, dtype="bf16", B=64, Hq=8, Hkv=2, Sq=1, Skv=1024, D=128),
], ids=["bf16-decode", "f16-add", "f32-d64", "f16-gqa4-add", "bf16-gqa8-causal-br", "bf16-batched-gqa"])
def test_one_sweep_ranges_chosen_by_default(spec, monkeypatch, capfd):
    # decode rows against long keys: the default plan runs the keys as one-sweep
    # ranges on the wide kernel (grouped heads: the group's heads in one workgroup)
    for e in ("SDPA_MATH_RANGES", "SDPA_MATH_RANGE_KEYS", "SDPA_MATH_RANGE_WAVES", "SDPA_MATH_SPLITS"):
        monkeypatch.delenv(e, raising=False)
    monkeypatch.setenv("SDPA_MATH_DEBUG", "1")
    spec = dict(spec)
    align = spec.pop("align", "top_left")
    c = W.make_case(**spec)
    c["align"] = align
    S = _lib()
    gqa = c["q"].shape[1] != c["k"].shape[1]
    assert S.kernel_name(c["q"], c["k"], c["v"], c["mask"], c["causal"], gqa,
                         causal_alignment=align) == "sdpa_fused_wide_kernel"
    _check(c, "auto", label="default one-sweep ranges")
    _ran_ranges(capfd)


def test_key_ranges_chosen_by_default(monkeypatch):
    # few query rows against many keys: the default plan splits the keys
    monkeypatch.delenv("SDPA_MATH_SPLITS", raising=False)
    c = W.make_case(seed=176, dtype="bf16", B=1, Hq=2, Hkv=2, Sq=3, Skv=4096, D=64)
    _check(c, "auto", label="default key ranges")


def test_workspace_missing_short_or_misaligned_runs_unsplit(monkeypatch):
    # through the C ABI: with no workspace, too small a one or a misaligned one
    # the call runs unsplit; every variant matches the split call to the bound
    import ctypes
    from sdpa_forward_materialised_amd import _binding as Bd
    monkeypatch.delenv("SDPA_MATH_SPLITS", raising=False)
    S = _lib()
    lib = Bd.load_library()
    c = W.make_case(seed=177, dtype="f16", B=1, Hq=2, Hkv=2, Sq=5, Skv=4096, D=64)
    q, k, v = (c[x].to(DEV) for x in ("q", "k", "v"))
    dq, dk, dv = Bd._desc(q, 4), Bd._desc(k, 4), Bd._desc(v, 4)
    n = ctypes.c_size_t(0)
    assert lib.sdpa_math_workspace_bytes(dq, dk, dv, None, 0, 0, ctypes.byref(n)) == 0
    assert n.value > 0
    ws = torch.empty(n.value + 512, dtype=torch.uint8, device=DEV)
    ref = run_oracle(c["q"], c["k"], c["v"], None, False, None, False)
    for label, ptr, size in (("split", ws.data_ptr(), n.value), ("none", None, 0),
                             ("short", ws.data_ptr(), n.value - 256), ("misaligned", ws.data_ptr() + 16, n.value)):
        O, P, L = poisoned_outputs(1, 2, 5, 4096, 64, q.dtype, DEV)
        do, dp, dl = Bd._desc(O, 4), Bd._desc(P, 4), Bd._desc(L, 3)
        rc = lib.sdpa_math_fwd_ws(dq, dk, dv, None, 0, 0.125, 0, do, dp,
                                  dl, None if ptr is None else ctypes.c_void_p(ptr), size,
                                  ctypes.c_void_p(torch.cuda.current_stream().cuda_stream), 0)
        assert rc == 0, S.last_error()
        torch.cuda.synchronize()
        compare(O, P, L, ref, q.dtype, f"workspace {label}", v=c["v"])


@pytest.mark.parametrize("entry,path", [("sdpa_math_fwd", None), ("sdpa_math_fwd_path", 0),
                                        ("sdpa_math_fwd_path", 1), ("sdpa_math_fwd_path", 2)])
def test_entry_points_direct(entry, path):
    """sdpa_math_fwd and sdpa_math_fwd_path called straight through the C ABI
    (ctypes, no binding logic) on NaN-poisoned outputs, against the oracle; a
    bool key-padding mask with grouped heads and a dead row."""
    import ctypes
    from sdpa_forward_materialised_amd import _binding as Bd
    lib = Bd.load_library()
    c = W.make_case(seed=178, dtype="bf16", B=2, Hq=4, Hkv=2, Sq=96, Skv=200, D=64, mask="bool",
                    mask_shape=(2, 1, 96, 200), p=0.2)
    c["mask"][1, 0, 7, :] = False
    q, k, v, m = (c[x].to(DEV) for x in ("q", "k", "v", "mask"))
    O, P, L = poisoned_outputs(2, 4, 96, 200, 64, q.dtype, DEV)
    args = [Bd._desc(q, 4), Bd._desc(k, 4), Bd._desc(v, 4), Bd._desc(m, 4), 0, 0.125, 1,
            Bd._desc(O, 4), Bd._desc(P, 4), Bd._desc(L, 3),
            ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)]
    print(f"[case] {entry} path={path}", flush=True)
    rc = getattr(lib, entry)(*args) if path is None else getattr(lib, entry)(*args, path)
    assert rc == 0, lib.sdpa_math_last_error()
    assert lib.sdpa_math_last_error() == b""
    torch.cuda.synchronize()
    ref = run_oracle(c["q"], c["k"], c["v"], c["mask"], False, 0.125, True)
    r = compare(O, P, L, ref, q.dtype, f"{entry} path={path}", v=c["v"])
    assert torch.isneginf(L[1, :, 7]).all() and r["o_elems_relaxed"] == 0
    # an unknown path value is rejected before any launch
    if path is not None:
        O2, P2, L2 = poisoned_outputs(2, 4, 96, 200, 64, q.dtype, DEV)
        bad = args[:7] + [Bd._desc(O2, 4), Bd._desc(P2, 4), Bd._desc(L2, 3), args[10]]
        assert lib.sdpa_math_fwd_path(*bad, 7) == 1 and b"path" in lib.sdpa_math_last_error()
        torch.cuda.synchronize()
        assert torch.isnan(O2).all() and torch.isnan(P2).all() and torch.isnan(L2).all()


# Every compute-wave count the kernel is built for (a tuning knob read at each
# call): 2 or 3 compute waves plus a loader wave, or 4 compute waves sharing
# the tile loads (where their staged tiles fit in LDS; otherwise the request
# falls back to the default shape, which is then what is checked).
WAVE_CASES = [
    ("bf16-d128-causal", dict(seed=130, dtype="bf16", B=1, Hq=2, Hkv=2, Sq=300, Skv=300, D=128, causal=True)),
    ("f16-d64-bool-staged", dict(seed=131, dtype="f16", B=1, Hq=2, Hkv=1, Sq=257, Skv=320, D=64, mask="bool", p=0.2)),
    ("bf16-d32-add-staged", dict(seed=132, dtype="bf16", B=2, Hq=1, Hkv=1, Sq=200, Skv=136, D=32, mask="add", p=0.1)),
    ("f16-d128-causal-skv-ragged", dict(seed=133, dtype="f16", B=1, Hq=2, Hkv=2, Sq=190, Skv=250, D=128,
                                        causal=True)),
    ("f32-d64-causal", dict(seed=134, dtype="f32", B=1, Hq=2, Hkv=2, Sq=160, Skv=160, D=64, causal=True)),
]


@pytest.mark.parametrize("waves", [2, 3, 4])
@pytest.mark.parametrize("label,spec", WAVE_CASES, ids=[s[0] for s in WAVE_CASES])
def test_compute_wave_counts(label, spec, waves, monkeypatch):
    monkeypatch.setenv("SDPA_MATH_TP_WAVES", str(waves))
    c = W.make_case(**spec)
    _check(c, "twopass", label=f"{label} waves={waves}")


# A mask whose rows are all equal, passed as a full-size expanded view (sizes
# [B, Hq, Sq, Skv], row stride 0): every query row's mask tile reads the same
# bytes; every compute-wave count.
@pytest.mark.parametrize("waves", [2, 3, 4])
@pytest.mark.parametrize("kind,D", [("bool", 128), ("add", 64), ("neginf", 32)])
def test_shared_mask_rows_expanded(kind, D, waves, monkeypatch):
    monkeypatch.setenv("SDPA_MATH_TP_WAVES", str(waves))
    c = W.make_case(125, "f16", 2, 4, 4, 200, 136, D, mask=kind, mask_shape=(2, 4, 1, 136), p=0.25)
    S = _lib()
    gm = c["mask"].to(DEV).expand(2, 4, 200, 136)  # expanded on the device: row stride 0
    assert gm.stride(2) == 0
    out = poisoned_outputs(2, 4, 200, 136, D, torch.float16, DEV)
    print(f"[case] shared rows {kind} D={D} waves={waves}", flush=True)
    O, P, L = S.fwd(c["q"].to(DEV), c["k"].to(DEV), c["v"].to(DEV), gm, False, None, False, path="twopass", out=out)
    torch.cuda.synchronize()
    ref = run_oracle(c["q"], c["k"], c["v"], c["mask"], False, None, False)
    compare(O, P, L, ref, torch.float16, f"shared rows {kind} D={D} waves={waves}", v=c["v"])


@pytest.mark.parametrize("Sq,waves", [(384, None), (288, "3")])
def test_dispatch_orders_identical(Sq, waves, monkeypatch):
    """Every causal workgroup order (a permutation of the query blocks) gives the same bits, and
    each matches the oracle (so no block is skipped or run twice). 16 heads: whole head pairs per
    XCD, so order 3 applies; Sq = 288 on three compute waves gives an odd number of query blocks
    per head (3), where order 1 must not be taken."""
    if waves:
        monkeypatch.setenv("SDPA_MATH_TP_WAVES", waves)
    c = W.make_case(124, "bf16", 2, 8, 8, Sq, Sq, 64, causal=True)
    ref = run_oracle(c["q"], c["k"], c["v"], None, True, None, False)
    outs = {}
    for sched in ("0", "1", "2", "3", "4", "5"):
        monkeypatch.setenv("SDPA_MATH_SCHED", sched)
        outs[sched] = _run(c, "twopass", label=f"Sq={Sq} order {sched}")
        compare(*outs[sched], ref, torch.bfloat16, f"Sq={Sq} order {sched}", v=c["v"])
    monkeypatch.delenv("SDPA_MATH_SCHED")
    for sched in ("0", "1", "2", "4", "5"):
        for x, y in zip(outs["3"], outs[sched]):
            assert torch.equal(x, y), sched


@pytest.mark.parametrize("path", PATHS)
def test_fully_masked_rows(path):
    c = W.make_case(120, "f16", 2, 4, 2, 96, 160, 64, mask="bool", mask_shape=(2, 4, 96, 160), p=0.2)
    c["mask"][0, 1, 5, :] = False
    c["mask"][1, 3, 40:72, :] = False
    O, P, L = _run(c, path, label="dead rows")
    assert torch.all(P[0, 1, 5] == 0) and torch.all(O[0, 1, 5] == 0)
    assert torch.isneginf(L[0, 1, 5]) and torch.isneginf(L[1, 3, 40:72]).all()
    ref = run_oracle(c["q"], c["k"], c["v"], c["mask"], False, None, True)
    compare(O, P, L, ref, torch.float16, "dead rows", v=c["v"])


@pytest.mark.parametrize("path", PATHS)
def test_explicit_scale_and_strided_inputs(path):
    # physical [B, S, H, D] viewed as logical [B, H, S, D]: only the last dim is dense
    c = W.make_case(121, "bf16", 2, 4, 4, 80, 96, 64, causal=True)
    for key in ("q", "k", "v"):
        c[key] = c[key].transpose(1, 2).contiguous().transpose(1, 2)
    _check(c, path, scale=0.05, label="strided scale=0.05")


@pytest.mark.parametrize("path", PATHS)
def test_gqa_matches_repeated_kv_bitwise(path):
    c = W.make_case(122, "f16", 2, 8, 2, 70, 130, 64, mask="bool", mask_shape=(2, 1, 70, 130))
    S = _lib()
    q, k, v, m = (c[x].to(DEV) for x in ("q", "k", "v", "mask"))
    a = _fwd(path, q, k, v, m, False, None, True)
    b = _fwd(path, q, k.repeat_interleave(4, 1).contiguous(), v.repeat_interleave(4, 1).contiguous(), m, False,
             None, False)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


@pytest.mark.parametrize("path", PATHS)
def test_deterministic(path):
    c = W.make_case(123, "bf16", 1, 4, 4, 200, 200, 128, causal=True)
    S = _lib()
    q, k, v = (c[x].to(DEV) for x in ("q", "k", "v"))
    a = _fwd(path, q, k, v, None, True)
    b = _fwd(path, q, k, v, None, True)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_degenerate_shapes():
    S = _lib()
    q = torch.randn(2, 2, 0, 64, device=DEV, dtype=torch.float16)
    k = torch.randn(2, 2, 10, 64, device=DEV, dtype=torch.float16)
    O, P, L = S.fwd(q, k, k)
    assert O.shape == (2, 2, 0, 64) and P.shape == (2, 2, 0, 10) and L.shape == (2, 2, 0)
    # no keys at all: O = 0, LSE = -inf
    q = torch.randn(1, 2, 5, 32, device=DEV, dtype=torch.bfloat16)
    k = torch.randn(1, 2, 0, 32, device=DEV, dtype=torch.bfloat16)
    out = poisoned_outputs(1, 2, 5, 0, 32, torch.bfloat16, DEV)
    O, P, L = S.fwd(q, k, k, out=out)
    torch.cuda.synchronize()
    assert torch.all(O == 0) and torch.isneginf(L).all() and P.numel() == 0


def test_errors_leave_outputs_untouched():
    S = _lib()
    q = torch.randn(1, 3, 8, 64, device=DEV, dtype=torch.float16)
    k = torch.randn(1, 2, 8, 64, device=DEV, dtype=torch.float16)
    with pytest.raises(ValueError):
        S.fwd(q, k, k, enable_gqa=True)
    q = torch.randn(1, 2, 8, 48, device=DEV, dtype=torch.float16)
    with pytest.raises(NotImplementedError):
        S.fwd(q, q, q)
    q = torch.randn(1, 2, 8, 64, device=DEV, dtype=torch.float16)
    m = torch.ones(8, 8, dtype=torch.bool, device=DEV)
    with pytest.raises(ValueError):
        S.fwd(q, q, q, m, is_causal=True)


# ------------------------------------------------------------ the five workloads

def _workload_case(w):
    inp = W.make_inputs(w)
    inp["causal"] = w.causal
    return inp


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("w", [w for w in W.WORKLOADS if w.name.startswith(("tiny", "decode"))],
                         ids=lambda w: w.name)
def test_workload_full_oracle(w, path):
    """Workloads the oracle finishes in seconds: every output element checked."""
    c = _workload_case(w)
    r = _check(c, path, scale=w.scale, label=w.name)
    print(f"[result] {w.name} {path} {r}", flush=True)
    assert r["o_elems_relaxed"] == 0 and r["err_o"] <= TOL_OP[c["q"].dtype], r


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("w", [w for w in W.WORKLOADS if w.name.startswith(("prefill", "gqa"))],
                         ids=lambda w: w.name)
def test_workload_full_size(w, path):
    """Full-size workloads: every (batch, head) slice against the oracle,
    element by element, and every O element within the stated tolerance
    (none of these workloads reaches an |O| where correct rounding alone
    would exceed it)."""
    c = _workload_case(w)
    O, P, L = _run(c, path, scale=w.scale, label=w.name)
    dt = c["q"].dtype
    tol = TOL_OP[dt]
    worst = {"err_o": 0.0, "err_p": 0.0, "err_lse": 0.0, "max_abs_o_ref": 0.0}
    for b in range(w.B):
        for h in range(w.Hq):
            qs, ks, vs, ms = head_slice(c["q"], c["k"], c["v"], c["mask"], b, h)
            ref = run_oracle(qs, ks, vs, ms, w.causal, w.scale, False)
            r = compare(O[b:b + 1, h:h + 1], P[b:b + 1, h:h + 1], L[b:b + 1, h:h + 1], ref, dt,
                        f"{w.name} b{b} h{h}", v=vs)
            assert r["o_elems_relaxed"] == 0 and r["err_o"] <= tol, (w.name, b, h, r)
            for key in worst:
                worst[key] = max(worst[key], r[key])
    print(f"[result] {w.name} {path} every slice: {worst}", flush=True)
    dead = torch.isneginf(L)
    if w.mask == "keypad_bool":
        assert dead[0, :, :8].all() and (dead.sum().item() == 8 * w.Hq)


# ------------------------------------------------------------ bench's extra workloads

@pytest.mark.parametrize("w", list(W.EXTRA_WORKLOADS), ids=lambda w: w.name)
def test_extra_workload_full_size(w):
    """Chunked prefill (bottom-right causal), long-key decode and batched
    grouped-head decode at full size, with the default plan (key ranges where
    the planner picks them): sampled
    (batch, head) slices against the oracle, plus whole-output properties."""
    c = _workload_case(w)
    c["align"] = w.align
    O, P, L = _run(c, "auto", scale=w.scale, label=w.name)
    dt = c["q"].dtype
    for b, h in [(0, 0), (w.B - 1, w.Hq - 1), (w.B // 2, w.Hq // 2 + 1)]:
        qs, ks, vs, ms = head_slice(c["q"], c["k"], c["v"], c["mask"], b, h)
        ref = run_oracle(qs, ks, vs, ms, w.causal, w.scale, False, w.align)
        r = compare(O[b:b + 1, h:h + 1], P[b:b + 1, h:h + 1], L[b:b + 1, h:h + 1], ref, dt, f"{w.name} b{b} h{h}",
                    v=vs)
        print(f"[result] {w.name} b={b} h={h} {r}", flush=True)
    assert not torch.isnan(O).any() and not torch.isnan(P).any() and not torch.isnan(L).any()
    rows = P.float().sum(-1)
    assert torch.allclose(rows, torch.ones_like(rows), atol=1e-2)
    if w.causal:
        # bottom-right: query i keeps keys j <= i + Skv - Sq
        off = w.Skv - w.Sq if w.align == "bottom_right" else 0
        upper = torch.ones(w.Sq, w.Skv, dtype=torch.bool, device=DEV).triu(1 + off)
        assert torch.all(P[:, :, upper] == 0)


def test_launch_follows_current_stream():
    """The binding launches on torch's current stream (a side stream inside
    ``torch.cuda.stream``), and the results equal a default-stream call."""
    S = _lib()
    from sdpa_forward_materialised_amd import _binding as B
    dev = torch.device(DEV)
    c = W.make_case(seed=120, dtype="bf16", B=2, Hq=4, Hkv=4, Sq=200, Skv=200, D=64, causal=True)
    q, k, v = (c[x].to(DEV) for x in ("q", "k", "v"))
    print("[case] side stream bf16 2x4x200x64 causal", flush=True)
    ref = S.fwd(q, k, v, None, True)
    torch.cuda.synchronize()
    side = torch.cuda.Stream(device=dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        assert B._current_stream(dev) == side.cuda_stream
        got = S.fwd(q, k, v, None, True)
    assert B._current_stream(dev) == torch.cuda.current_stream(dev).cuda_stream
    side.synchronize()
    for x, y in zip(ref, got):
        assert torch.equal(x, y)


def test_largest_slice():
    """The largest square bf16 slice the kernels take (Sq = Skv = 23170, P just
    under 1 GiB), one head at D = 128, non-causal, default plan: sampled query
    rows (first, last, ragged tail, random) against the oracle, and every row
    of P summing to 1."""
    S = _lib()
    n = 23170
    c = W.make_case(seed=130, dtype="bf16", B=1, Hq=1, Hkv=1, Sq=n, Skv=n, D=128)
    print(f"[case] largest slice bf16 1x1x{n}x128", flush=True)
    O, P, L = S.fwd(c["q"].to(DEV), c["k"].to(DEV), c["v"].to(DEV))
    torch.cuda.synchronize()
    rows = sorted({0, 1, 95, 96, n - 35, n - 2, n - 1} |
                  set(np.random.default_rng(130).integers(0, n, 25).tolist()))
    idx = torch.tensor(rows)
    ref = run_oracle(c["q"][:, :, idx], c["k"], c["v"], None, False, None, False)
    r = compare(O[:, :, idx.to(DEV)], P[:, :, idx.to(DEV)], L[:, :, idx.to(DEV)], ref, torch.bfloat16,
                "largest slice", v=c["v"])
    print(f"[result] largest slice {r}", flush=True)
    sums = torch.cat([P[0, 0, i:i + 4096].float().sum(-1) for i in range(0, n, 4096)])
    assert sums.numel() == n and torch.allclose(sums, torch.ones_like(sums), atol=1e-2)
    assert not torch.isnan(O).any() and not torch.isnan(L).any()


SCALE_CASES = [
    ("bf16-d128-causal", dict(seed=140, dtype="bf16", B=1, Hq=2, Hkv=2, Sq=200, Skv=200, D=128, causal=True)),
    ("f16-d64-bool", dict(seed=141, dtype="f16", B=2, Hq=2, Hkv=1, Sq=100, Skv=300, D=64, mask="bool")),
    ("f16-d64-add", dict(seed=142, dtype="f16", B=1, Hq=2, Hkv=2, Sq=130, Skv=260, D=64, mask="add", p=0.1)),
    ("f32-d32-nomask", dict(seed=143, dtype="f32", B=1, Hq=2, Hkv=2, Sq=70, Skv=150, D=32)),
]


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("scale", [-0.125, 0.0, 3.0])
@pytest.mark.parametrize("label,spec", SCALE_CASES, ids=[s[0] for s in SCALE_CASES])
def test_nonpositive_and_large_scale(label, spec, scale, path):
    """A negative scale (the row maximum then comes from the smallest raw
    score), zero (P uniform over the kept keys) and a large one (nearly
    one-hot rows) against the oracle."""
    c = W.make_case(**spec)
    r = _check(c, path, scale=scale, label=f"{label} scale={scale}")
    print(f"[result] {label} scale={scale} {path} {r}", flush=True)


def test_concurrent_streams_independent():
    """Two calls in flight at once on two streams (one split over key ranges,
    with its own workspace; one unsplit), launched back to back with no
    synchronisation between them: each equals the same call made alone."""
    S = _lib()
    dev = torch.device(DEV)
    a = W.make_case(seed=150, dtype="bf16", B=2, Hq=4, Hkv=4, Sq=1, Skv=8192, D=128)
    b = W.make_case(seed=151, dtype="f16", B=1, Hq=8, Hkv=2, Sq=300, Skv=300, D=64, mask="bool",
                    mask_shape=(1, 1, 300, 300), causal=False)
    ga = [a[x].to(DEV) for x in ("q", "k", "v")]
    gb = [b[x].to(DEV) for x in ("q", "k", "v")] + [b["mask"].to(DEV)]
    print("[case] two streams: bf16 2x4x1x8192x128 (split) + f16 gqa 300x300 bool", flush=True)
    ref_a = S.fwd(*ga)
    ref_b = S.fwd(*gb, False, None, True)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(device=dev), torch.cuda.Stream(device=dev)
    for _ in range(3):
        with torch.cuda.stream(s1):
            got_a = S.fwd(*ga)
        with torch.cuda.stream(s2):
            got_b = S.fwd(*gb, False, None, True)
        torch.cuda.synchronize()
        for x, y in zip(ref_a + ref_b, got_a + got_b):
            assert torch.equal(x, y)


# ------------------------------------------------------------ prepared calls

@pytest.mark.parametrize("label,spec", [
    ("prepared-decode-key-ranges", dict(seed=301, dtype="bf16", B=2, Hq=8, Hkv=8, Sq=4, Skv=4096, D=128)),
    ("prepared-f16-bool", dict(seed=302, dtype="f16", B=2, Hq=4, Hkv=2, Sq=70, Skv=300, D=64, mask="bool")),
])
def test_prepared_call_matches_fwd(label, spec):
    """prepare_fwd binds the call to its tensors once; runs after refilling
    the inputs in place give fwd's bits on the new inputs, and the oracle's
    values."""
    S = _lib()
    c = W.make_case(**spec)
    c2 = W.make_case(**{**spec, "seed": spec["seed"] + 1000})
    q, k, v = (c[x].to(DEV) for x in ("q", "k", "v"))
    m = None if c["mask"] is None else c["mask"].to(DEV)
    gqa = q.shape[1] != k.shape[1]
    print(f"[case] {label}", flush=True)
    call = S.prepare_fwd(q, k, v, m, False, None, gqa)
    for cc in (c, c2):
        for t, x in zip((q, k, v), ("q", "k", "v")):
            t.copy_(cc[x].to(DEV))
        if m is not None:
            m.copy_(cc["mask"].to(DEV))
        O, P, L = call.run()
        torch.cuda.synchronize()
        want = S.fwd(q, k, v, m, False, None, gqa)
        for x, y in zip((O, P, L), want):
            assert torch.equal(x, y), label
        ref = run_oracle(cc["q"], cc["k"], cc["v"], cc["mask"], False, None, gqa)
        compare(O, P, L, ref, cc["q"].dtype, label, v=cc["v"])
