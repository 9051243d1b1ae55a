"""The C-ABI boundary on the CPU: the library loads, exports what the header
declares, validates arguments before touching the GPU, and counts score tiles
the way the FlagOS-OP page's path rule does (values printed on that page)."""

import ctypes
import json
import os
import re

import pytest
import torch

import sdpa_forward_materialised_amd as S
from sdpa_forward_materialised_amd import _binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GOLDEN = os.path.join(ROOT, "tests", "golden")


def _declared_functions():
    names = set()
    inc = os.path.join(ROOT, "include")
    for fn in os.listdir(inc):
        if not fn.endswith(".h"):
            continue
        text = open(os.path.join(inc, fn)).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for m in re.finditer(r"^[A-Za-z_][\w \*]*?\b(sdpa_\w+)\s*\(", text, flags=re.M):
            names.add(m.group(1))
    return names


def test_library_exports_every_declared_symbol():
    lib = S.load_library()
    declared = _declared_functions()
    assert {"sdpa_math_fwd", "sdpa_math_fwd_path", "sdpa_math_plan", "sdpa_math_last_error",
            "sdpa_math_version"} <= declared
    for name in declared:
        assert hasattr(lib, name), f"{name} declared in include/ but not exported"
    assert S.version() == 1


def test_tile_counts_match_page_values():
    g = json.load(open(os.path.join(GOLDEN, "page_tile_counts.json")))
    for case in g["cases"]:
        q = torch.zeros(1, 1, case["Sq"], 64, dtype=torch.float16)
        k = torch.zeros(1, 1, case["Skv"], 64, dtype=torch.float16)
        _, _, t64 = S.plan(q, k, k, is_causal=case["causal"])
        assert t64 == case["tiles"], case["cite"]


def _z(*shape, dtype=torch.float16):
    return torch.zeros(*shape, dtype=dtype)


@pytest.mark.parametrize("args,exc,frag", [
    ((_z(1, 3, 8, 64), _z(1, 2, 8, 64), _z(1, 2, 8, 64)), ValueError, "not a multiple"),
    ((_z(1, 4, 8, 64), _z(1, 2, 8, 64), _z(1, 2, 8, 64), None, False, False), ValueError, "enable_gqa"),
    ((_z(1, 2, 8, 64), _z(1, 2, 8, 64), _z(1, 2, 8, 64), torch.ones(8, 8, dtype=torch.bool), True), ValueError,
     "mutually exclusive"),
    ((_z(1, 2, 8, 64), _z(1, 2, 8, 64), _z(1, 2, 8, 64), torch.ones(3, 8, dtype=torch.bool)), ValueError,
     "broadcast"),
    ((_z(1, 2, 8, 64), _z(1, 2, 8, 64), _z(1, 2, 8, 64), torch.ones(8, 8, dtype=torch.float32)), ValueError,
     "mask dtype"),
    ((_z(1, 2, 8, 64), _z(1, 2, 8, 64, dtype=torch.bfloat16), _z(1, 2, 8, 64)), ValueError, "dtypes differ"),
    ((_z(2, 2, 8, 64), _z(1, 2, 8, 64), _z(1, 2, 8, 64)), ValueError, "batch"),
    ((_z(1, 2, 8, 48), _z(1, 2, 8, 48), _z(1, 2, 8, 48)), NotImplementedError, "head dim"),
    ((_z(1, 2, 8, 64), _z(1, 2, 8, 64), _z(1, 2, 8, 32)), NotImplementedError, "value head dim"),
    ((_z(1, 2, 8, 128)[..., ::2], _z(1, 2, 8, 64), _z(1, 2, 8, 64)), NotImplementedError, "last dim"),
    ((_z(1, 2, 8, 65)[..., 1:], _z(1, 2, 8, 64), _z(1, 2, 8, 64)), NotImplementedError, "aligned"),
    ((_z(1, 2, 8, 64, dtype=torch.int32),) * 3, ValueError, "unsupported dtype"),
])
def test_validation_errors(args, exc, frag):
    full = list(args) + [None, False, True][len(args) - 3:]
    q, k, v, m, causal, gqa = full[:6]
    with pytest.raises(exc) as ei:
        S.plan(q, k, v, m, causal, gqa)
    assert frag in str(ei.value)


def test_fwd_rejects_bad_outputs_before_launch():
    """Output descriptors are checked on the host; nothing reaches the GPU."""
    lib = S.load_library()
    q = _z(1, 2, 8, 64)
    o, p, lse = _z(1, 2, 8, 64), _z(1, 2, 8, 9), torch.zeros(1, 2, 8)
    d = [B._desc(t, 4) for t in (q, q, q, o, p)] + [B._desc(lse, 3)]
    rc = lib.sdpa_math_fwd(d[0], d[1], d[2], None, 0, 0.125, 0,
                           d[3], d[4], d[5], None)
    assert rc == 1 and "probs dim 3" in S.last_error()
    lse16 = B._desc(torch.zeros(1, 2, 8, dtype=torch.float16), 3)
    p_ok = B._desc(_z(1, 2, 8, 8), 4)
    rc = lib.sdpa_math_fwd(d[0], d[1], d[2], None, 0, 0.125, 0,
                           d[3], p_ok, lse16, None)
    assert rc == 1 and "lse must be f32" in S.last_error()
    rc = lib.sdpa_math_fwd(None, d[1], d[2], None, 0, 0.125, 0,
                           d[3], p_ok, d[5], None)
    assert rc == 1 and "q is NULL" in S.last_error()
    rc = lib.sdpa_math_fwd_path(d[0], d[1], d[2], None, 0, 0.125, 0,
                                d[3], p_ok, d[5], None, 7)
    assert rc == 1 and "unknown path" in S.last_error()


def test_binding_refuses_cpu_tensors():
    q = _z(1, 2, 8, 64)
    with pytest.raises(ValueError, match="GPU only"):
        S.fwd(q, q, q)


def test_plan_reports_paths_and_tiles():
    q = _z(2, 16, 2048, 128, dtype=torch.bfloat16)
    path, tiles, t64 = S.plan(q, q, q, is_causal=True)
    assert t64 == 528 and path == "twopass"
    q = _z(4, 32, 1024, 128)
    k = _z(4, 8, 1024, 128)
    m = torch.ones(4, 1, 1024, 1024, dtype=torch.bool)
    assert S.plan(q, k, k, m, False, True)[2] == 256


def test_plan_picks_fused_for_few_tiles():
    # decode-like: 100 queries x 1152 keys is 36 tiles of 64x64 per (b, h);
    # with a bool or an additive mask the wide fused kernel takes it, two
    # 32-row groups per workgroup (2 x 18 tiles of 64 rows x 64 keys)
    q, k = _z(16, 8, 100, 64), _z(16, 8, 1152, 64)
    mb = torch.ones(16, 8, 100, 1152, dtype=torch.bool)
    assert S.plan(q, k, k, mb) == ("fused", 2 * 18, 36)
    m = torch.zeros(16, 8, 100, 1152, dtype=torch.float16)
    assert S.plan(q, k, k, m) == ("fused", 2 * 18, 36)
    # 64 queries: one row group per workgroup (two would leave the grid at
    # 128 workgroups), 32-row blocks
    q64 = _z(16, 8, 64, 64)
    assert S.plan(q64, k, k, m[:, :, :64]) == ("fused", 2 * 18, 18)
    # no mask, 512 keys: two-pass
    k512 = _z(16, 8, 512, 64)
    assert S.plan(q, k512, k512)[0] == "twopass"
    q = _z(1, 2, 64, 32, dtype=torch.float32)
    assert S.plan(q, q, q, is_causal=True)[0] == "fused"
    # many tiles: two-pass
    q = _z(4, 8, 1024, 64)
    assert S.plan(q, q, q, is_causal=True)[0] == "twopass"
    # few tiles, but more keys than the fused waves hold at D=128: two-pass
    q, k = _z(1, 2, 1, 128), _z(1, 2, 1100, 128)
    assert S.plan(q, k, k) == ("twopass", 18, 18)


def _tiles64_brute(Sq, Skv, coff):
    """64x64 score tiles holding at least one key kept under causal offset coff."""
    n = 0
    for r0 in range(0, Sq, 64):
        for c0 in range(0, Skv, 64):
            last_row = min(Sq, r0 + 64) - 1
            if c0 <= last_row + coff:
                n += 1
    return n


@pytest.mark.parametrize("Sq,Skv", [(512, 2048), (100, 1152), (64, 64), (200, 100), (1, 300), (700, 700)])
def test_plan_bottom_right_tile_counts(Sq, Skv):
    q, k = _z(1, 2, Sq, 64), _z(1, 2, Skv, 64)
    _, _, t64 = S.plan(q, k, k, is_causal=True, causal_alignment="bottom_right")
    assert t64 == _tiles64_brute(Sq, Skv, Skv - Sq)
    _, _, t64_tl = S.plan(q, k, k, is_causal=True)
    assert t64_tl == _tiles64_brute(Sq, Skv, 0)
    if Sq == Skv:
        assert S.plan(q, k, k, is_causal=True, causal_alignment="bottom_right") == S.plan(q, k, k, is_causal=True)


def test_causal_codes_validated():
    q = _z(1, 2, 8, 64)
    with pytest.raises(ValueError, match="causal_alignment"):
        S.plan(q, q, q, is_causal=True, causal_alignment="middle")
    lib = S.load_library()
    d = B._desc(q, 4)
    out = (ctypes.c_int32(), ctypes.c_int64(), ctypes.c_int64())
    for code, want in ((0, 0), (1, 0), (2, 0), (3, 1), (-1, 1)):
        rc = lib.sdpa_math_plan(d, d, d, None, code, 0, *(ctypes.byref(x) for x in out))
        assert rc == want, (code, S.last_error())
    assert "is_causal" in (S.last_error() or "")


def _ws_bytes(q, k, mask=None, causal=0, gqa=0):
    lib = S.load_library()
    n = ctypes.c_size_t(123)
    rc = lib.sdpa_math_workspace_bytes(B._desc(q, 4), B._desc(k, 4), B._desc(k, 4),
                                       B._desc(mask, 4), causal, gqa, ctypes.byref(n))
    return rc, n.value


def test_workspace_query(monkeypatch):
    monkeypatch.delenv("SDPA_MATH_SPLITS", raising=False)
    # full grids or short key ranges: no split, no workspace
    assert _ws_bytes(_z(2, 16, 2048, 128, dtype=torch.bfloat16), _z(2, 16, 2048, 128, dtype=torch.bfloat16),
                     causal=1) == (0, 0)
    q, k = _z(16, 8, 100, 64), _z(16, 8, 1152, 64)
    assert _ws_bytes(q, k, torch.zeros(16, 8, 100, 1152, dtype=torch.float16)) == (0, 0)
    # one query row against 32768 keys, 32 heads: one-sweep ranges of 256 keys
    # on the wide kernel (128 ranges): per range and row (max, sum) and a float32
    # partial O, then every probability as float32
    q, k = _z(4, 8, 1, 128, dtype=torch.bfloat16), _z(4, 8, 32768, 128, dtype=torch.bfloat16)
    rc, n = _ws_bytes(q, k)
    rows = 4 * 8 * 1
    up = lambda x: -(-x // 256) * 256  # noqa: E731
    ml = up(128 * rows * 8)
    assert rc == 0 and n == up(ml + 128 * rows * 128 * 4) + rows * 32768 * 4
    # without them: the two-pass split, 16 ranges of 32 tiles (towards 512 workgroups)
    monkeypatch.setenv("SDPA_MATH_RANGES", "0")
    rc, n = _ws_bytes(q, k)
    assert rc == 0 and n == up(16 * rows * 8) + 16 * rows * 128 * 4
    monkeypatch.delenv("SDPA_MATH_RANGES")
    # forced ranges; a semantic error leaves the count at 0
    monkeypatch.setenv("SDPA_MATH_SPLITS", "3")
    assert _ws_bytes(_z(1, 2, 256, 64), _z(1, 2, 640, 64))[1] > 0  # two-pass shape (the fused path never splits)
    rc, n = _ws_bytes(_z(1, 3, 8, 64), _z(1, 2, 8, 64))
    assert rc == 1 and n == 0


def _bwd_ws_bytes(q, k, causal=0, gqa=0):
    lib = S.load_library()
    n = ctypes.c_size_t(123)
    rc = lib.sdpa_math_bwd_workspace_bytes(B._desc(q, 4), B._desc(k, 4), B._desc(k, 4), B._desc(None, 4),
                                           causal, gqa, ctypes.byref(n))
    return rc, n.value


def test_backward_workspace_query():
    up = lambda x: -(-x // 256) * 256  # noqa: E731
    # D_i per query row only: large grids, and any call without a causal mask
    q = _z(2, 16, 2048, 128, dtype=torch.bfloat16)
    assert _bwd_ws_bytes(q, q, causal=1) == (0, up(2 * 16 * 2048 * 4))
    q, k = _z(4, 32, 1024, 128), _z(4, 8, 1024, 128)
    assert _bwd_ws_bytes(q, k, causal=0, gqa=1) == (0, up(4 * 32 * 1024 * 4))
    # causal with 4 x 8 x 16 = 512 key blocks of 64 keys (under 1024): two query
    # ranges, each with float32 partial dk and dv
    q = _z(4, 8, 1024, 64)
    assert _bwd_ws_bytes(q, q, causal=1) == (0, up(4 * 8 * 1024 * 4) + 2 * 2 * 4 * 8 * 1024 * 64 * 4)
    # one key block: four ranges (at least 8 steps of 32 rows each: 2 heads x 19 tiles)
    q, k = _z(1, 2, 600, 64, dtype=torch.bfloat16), _z(1, 1, 64, 64, dtype=torch.bfloat16)
    assert _bwd_ws_bytes(q, k, causal=2, gqa=1) == (0, up(2 * 600 * 4) + 4 * 2 * 1 * 64 * 64 * 4)
    # too few steps for a range of 8: none
    q = _z(1, 1, 200, 32)
    assert _bwd_ws_bytes(q, q, causal=1) == (0, up(200 * 4))


@pytest.mark.parametrize("shape,ndim,view", [
    ((2, 3, 5, 32), 4, None),                 # contiguous 4-D
    ((2, 3, 7), 3, None),                     # LSE-like 3-D
    ((5, 9), 4, None),                        # mask with fewer dims: right-aligned
    ((9,), 4, None),
    ((2, 3, 0, 32), 4, None),                 # empty: null data pointer
    ((2, 6, 5, 32), 4, "transpose"),          # strided view
    ((2, 3, 5, 64), 4, "slice"),              # last-dim slice (offset pointer)
])
def test_descriptor_bytes_match_field_layout(shape, ndim, view):
    """The packed descriptor is byte-for-byte the sdpa_tensor_t that a
    field-by-field ctypes construction gives (pointer, dtype, ndim, sizes[4],
    strides[4], unused trailing entries zero)."""
    t = torch.randn(*shape, dtype=torch.float16)
    if view == "transpose":
        t = t.transpose(1, 2)
    elif view == "slice":
        t = t[..., 16:48]
    d = B._desc(t, ndim)
    u = t
    while u.dim() < ndim:
        u = u.unsqueeze(0)
    ref = B.SdpaTensor()
    ref.data = u.data_ptr() if u.numel() > 0 else None
    ref.dtype = B.SDPA_F16
    ref.ndim = ndim
    for i in range(ndim):
        ref.sizes[i] = u.shape[i]
        ref.strides[i] = u.stride(i)
    assert isinstance(d, bytes) and d == bytes(ref)
    dd = B.SdpaTensor.from_buffer_copy(d)
    assert (dd.data or 0) == (u.data_ptr() if u.numel() else 0)
    assert list(dd.sizes)[:ndim] == list(u.shape) and list(dd.strides)[:ndim] == list(u.stride())


def _fake_desc(shape, dtype_code, addr):
    """A dense sdpa_tensor_t at a made-up (16-byte aligned) address: only for
    calls that the library rejects before anything touches the device."""
    strides, s = [], 1
    for n in reversed(shape):
        strides.insert(0, s)
        s *= n
    nd = len(shape)
    return B._PACK[nd].pack(addr, dtype_code, nd, *shape, *strides)


def test_slice_extent_limit():
    """A (batch, head) slice of any tensor must span less than 1 GiB (the
    kernels' buffer descriptors hold 32-bit extents): a bf16 P slice of
    23171 x 23171 is the first square one past it, and is rejected on the host
    before any launch (23170 x 23170, just under, runs in the GPU parity tests)."""
    n = 23171
    assert (n - 1) * (n - 1) * 2 < (1 << 30) <= n * n * 2
    lib = S.load_library()
    q = _fake_desc((1, 1, n, 128), B.SDPA_BF16, 1 << 20)
    o = _fake_desc((1, 1, n, 128), B.SDPA_BF16, 1 << 21)
    p = _fake_desc((1, 1, n, n), B.SDPA_BF16, 1 << 22)
    lse = _fake_desc((1, 1, n), B.SDPA_F32, 1 << 23)
    rc = lib.sdpa_math_fwd(q, q, q, None, 0, 0.088, 0, o, p, lse, None)
    assert rc == 2 and "1 GiB" in S.last_error()


def test_noalloc_rejects_plans_beyond_its_scratch(monkeypatch):
    """sdpa_math_fwd_noalloc keeps key-range statistics in a static scratch of
    SDPA_MATH_NOALLOC_SCRATCH_BYTES; a plan that needs more (here 512 forced
    ranges over 8192 query rows: about 2 GB) is rejected on the host, before
    any launch (fake device addresses: nothing is touched)."""
    monkeypatch.setenv("SDPA_MATH_SPLITS", "512")
    lib = S.load_library()
    hdr = open(os.path.join(ROOT, "include", "sdpa_math.h")).read()
    m = re.search(r"#define SDPA_MATH_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", hdr)
    limit = int(m.group(1)) << int(m.group(2))
    n = 65536
    q = _fake_desc((1, 128, 64, 128), B.SDPA_BF16, 1 << 20)
    k = _fake_desc((1, 128, n, 128), B.SDPA_BF16, 1 << 30)
    o = _fake_desc((1, 128, 64, 128), B.SDPA_BF16, 1 << 21)
    p = _fake_desc((1, 128, 64, n), B.SDPA_BF16, 1 << 31)
    lse = _fake_desc((1, 128, 64), B.SDPA_F32, 1 << 22)
    ws = ctypes.c_size_t(0)
    assert lib.sdpa_math_workspace_bytes(q, k, k, None, 0, 0, ctypes.byref(ws)) == 0
    assert ws.value > limit
    rc = lib.sdpa_math_fwd_noalloc(q, k, k, None, 0, 0.088, 0, o, p, lse, None, 0)
    assert rc == 2 and "scratch" in S.last_error()
