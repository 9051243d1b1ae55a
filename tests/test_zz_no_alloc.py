"""sdpa_math_fwd_noalloc (static per-device scratch, nothing allocated)
against sdpa_math_fwd_ws with a caller workspace, through the C ABI: two
calls in a row whose keys the planner splits into ranges, the second with a
smaller input; each output equal bit for bit to the workspace call's and
within the oracle's bounds. Also an unsplit call."""

import ctypes

import pytest
import torch

import sdpa_workloads as W
from parity import compare, poisoned_outputs, run_oracle

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _lib():
    from sdpa_forward_materialised_amd import _binding as Bd
    return Bd, Bd.load_library()


def _call(Bd, lib, entry, c, ws=None):
    q, k, v = (c[x].to(DEV) for x in ("q", "k", "v"))
    m = None if c["mask"] is None else c["mask"].to(DEV)
    B, Hq, Sq, D = q.shape
    Skv = k.shape[2]
    O, P, L = poisoned_outputs(B, Hq, Sq, Skv, D, q.dtype, DEV)
    gqa = int(q.shape[1] != k.shape[1])
    args = [Bd._desc(q, 4), Bd._desc(k, 4), Bd._desc(v, 4), Bd._desc(m, 4), 0, 1.0 / D ** 0.5, gqa,
            Bd._desc(O, 4), Bd._desc(P, 4), Bd._desc(L, 3)]
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if entry == "ws":
        n = ctypes.c_size_t(0)
        assert lib.sdpa_math_workspace_bytes(*args[:4], 0, gqa, ctypes.byref(n)) == 0
        buf = torch.empty(max(n.value, 1), dtype=torch.uint8, device=DEV)
        rc = lib.sdpa_math_fwd_ws(*args, ctypes.c_void_p(buf.data_ptr()), n.value, stream, 0)
    else:
        rc = lib.sdpa_math_fwd_noalloc(*args, stream, 0)
    assert rc == 0, lib.sdpa_math_last_error()
    torch.cuda.synchronize()
    return O, P, L


@pytest.mark.parametrize("cases", [
    # (first call, second smaller call): one query row against long keys, split into ranges
    (dict(seed=301, dtype="bf16", B=2, Hq=8, Hkv=8, Sq=1, Skv=16384, D=128),
     dict(seed=302, dtype="bf16", B=1, Hq=4, Hkv=4, Sq=1, Skv=4096, D=128)),
    # few query rows, bool key padding, grouped heads, fp16 D = 64
    (dict(seed=303, dtype="f16", B=2, Hq=8, Hkv=2, Sq=16, Skv=8192, D=64, mask="bool", mask_shape=(2, 1, 1, 8192),
          p=0.3),
     dict(seed=304, dtype="f16", B=1, Hq=4, Hkv=2, Sq=5, Skv=3000, D=64, mask="bool", mask_shape=(1, 1, 1, 3000),
          p=0.3)),
])
def test_noalloc_matches_workspace_call(cases):
    Bd, lib = _lib()
    for i, spec in enumerate(cases):
        c = W.make_case(**spec)
        print(f"[case] noalloc call {i}: {spec}", flush=True)
        ref_ws = _call(Bd, lib, "ws", c)
        got = _call(Bd, lib, "noalloc", c)
        for x, y in zip(ref_ws, got):
            assert torch.equal(x, y)
        gqa = c["q"].shape[1] != c["k"].shape[1]
        ref = run_oracle(c["q"], c["k"], c["v"], c["mask"], False, None, gqa)
        compare(*got, ref, c["q"].dtype, f"noalloc call {i}", v=c["v"])


def test_noalloc_unsplit():
    Bd, lib = _lib()
    # a full grid: no key ranges, no scratch used
    c = W.make_case(seed=305, dtype="bf16", B=2, Hq=8, Hkv=8, Sq=256, Skv=256, D=64, causal=False)
    print("[case] noalloc unsplit", flush=True)
    a = _call(Bd, lib, "ws", c)
    b = _call(Bd, lib, "noalloc", c)
    for x, y in zip(a, b):
        assert torch.equal(x, y)
