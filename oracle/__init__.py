"""CPU oracle for the materialised-probability SDPA forward (float64).

TEST INFRASTRUCTURE ONLY. Only the tests, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package. The product (the
HIP library and its Python binding) never imports, links or calls it, and this
package imports nothing from the product.

``sdpa_reference`` is the plain definition written out in C (``sdpa_oracle.c``):
scores, masking, row maximum, log-sum-exp, probabilities, output, one query
row at a time in float64. ``brute.py`` is an independent pure-Python
implementation with exact summation used to pin it on tiny inputs.

Semantics (FlagOS-OP pull request "feat: add sdpa_math operator (Ascend Triton
+ P800 exact-P/A1)", sections Overview, Implementation and Intentional
divergences; its "P800 exact-P fast path" update for P = exp(scale*QK^T - LSE);
cudnn-frontend pull request "[SDPA] SM80 fwd: TemplateParams kernels,
plan-time compile, sym_int THD extents", merge-log notes on dead rows and the
LSE layout):
  * bool mask: True keeps a key, False removes it (score -inf);
  * additive mask: added to the scaled score;
  * causal: top-left, key j is removed for query i when j > i; with
    ``causal_alignment="bottom_right"`` when j > i + Skv - Sq (the chunked-
    prefill alignment named in the cudnn-frontend merge-log notes: the last
    query row keeps every key; rows i < Sq - Skv keep none and are dead);
  * causal together with a mask is an error; Hq not a multiple of Hkv is an
    error; Hq != Hkv without ``enable_gqa`` is an error;
  * a row with every key removed has P = 0, O = 0 and LSE = -inf.

Every function here is pinned: the forward by ``tests/test_oracle.py`` (brute
force, closed forms, invariants, equivalences, torch's CPU math backend on
float masks, planted mistakes), the backward ``sdpa_backward_reference`` by
``tests/test_oracle_bwd.py`` (brute force with the full softmax Jacobian,
finite differences of the forward, gradient identities, closed forms,
planted mistakes).
"""

from __future__ import annotations

import ctypes
import math
import os
import subprocess
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "sdpa_oracle.c")
_LIB = os.path.join(_HERE, "liboracle_sdpa.so")

MASK_NONE, MASK_BOOL, MASK_ADD = 0, 1, 2


def build(force: bool = True, src: str = _SRC, out: str = _LIB) -> str:
    """Compile the C oracle with gcc (float64, no FMA contraction, OpenMP)."""
    if force or not os.path.exists(out):
        cmd = ["gcc", "-O2", "-std=c99", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared",
               "-o", out, src, "-lm"]
        subprocess.run(cmd, check=True)
    return out


_lib_cache = {}


def load(path: str = _LIB) -> ctypes.CDLL:
    if path in _lib_cache:
        return _lib_cache[path]
    if not os.path.exists(path) or (path == _LIB and os.path.getmtime(_SRC) > os.path.getmtime(path)):
        build(force=True, out=path)  # missing, or older than its source
    lib = ctypes.CDLL(path)
    dp = ctypes.POINTER(ctypes.c_double)
    i64 = ctypes.c_int64
    lib.oracle_sdpa_fwd.restype = ctypes.c_int
    lib.oracle_sdpa_fwd.argtypes = [dp, dp, dp, i64, i64, i64, i64, i64, i64, i64,
                                    ctypes.c_int, ctypes.c_void_p, ctypes.POINTER(i64),
                                    ctypes.c_int, ctypes.c_double,
                                    ctypes.c_void_p, ctypes.POINTER(i64), ctypes.c_double, ctypes.c_int,
                                    dp, dp, dp]
    lib.oracle_sdpa_bwd.restype = ctypes.c_int
    lib.oracle_sdpa_bwd.argtypes = [dp, dp, dp, i64, i64, i64, i64, i64, i64, i64,
                                    ctypes.c_int, ctypes.c_void_p, ctypes.POINTER(i64),
                                    ctypes.c_int, ctypes.c_double, dp, dp, dp, dp, dp]
    lib.oracle_sdpa_threads.restype = ctypes.c_int
    lib.oracle_sdpa_threads.argtypes = []
    _lib_cache[path] = lib
    return lib


def threads() -> int:
    """OpenMP threads the oracle runs with."""
    return int(load().oracle_sdpa_threads())


def _f64(x) -> np.ndarray:
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().to("cpu", torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _mask_array(mask, full_shape):
    """Mask -> (kind, contiguous array, element strides over [B,Hq,Sq,Skv])."""
    try:
        import torch
        if isinstance(mask, torch.Tensor):
            mask = mask.detach().cpu()
            mask = mask.numpy() if mask.dtype == torch.bool else mask.to(torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    mask = np.asarray(mask)
    if mask.ndim > 4:
        raise ValueError("mask has more than 4 dims")
    shape = (1,) * (4 - mask.ndim) + tuple(mask.shape)
    for got, want in zip(shape, full_shape):
        if got != 1 and got != want:
            raise ValueError(f"mask shape {tuple(mask.shape)} does not broadcast to {full_shape}")
    if mask.dtype == np.bool_:
        kind, arr = MASK_BOOL, np.ascontiguousarray(mask.reshape(shape), dtype=np.uint8)
    else:
        kind, arr = MASK_ADD, np.ascontiguousarray(mask.reshape(shape), dtype=np.float64)
    strides = [0 if shape[d] == 1 else arr.strides[d] // arr.itemsize for d in range(4)]
    return kind, arr, strides


def causal_code(is_causal, causal_alignment: str = "top_left") -> int:
    """0 no causal mask, 1 top-left, 2 bottom-right."""
    if causal_alignment not in ("top_left", "bottom_right"):
        raise ValueError(f"unknown causal alignment {causal_alignment!r}")
    if not is_causal:
        return 0
    return 2 if causal_alignment == "bottom_right" else 1


DROPOUT_RULES = {"explicit": 0, "random": 1}


def sdpa_reference(q, k, v, attn_mask=None, is_causal: bool = False,
                   scale: Optional[float] = None, enable_gqa: bool = False,
                   lib_path: str = _LIB, causal_alignment: str = "top_left",
                   dropout_p: float = 0.0, dropout_mask=None, dropout_rule: str = "explicit"
                   ) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Return (O [B,Hq,Sq,Dv], P [B,Hq,Sq,Skv], LSE [B,Hq,Sq]) in float64.

    ``dropout_mask`` (bool, True keeps; broadcastable to [B,Hq,Sq,Skv]) with
    ``dropout_p`` applies the FlagOS-OP page's dropout rules: "explicit"
    returns keep * P and O = (keep * P) V / (1 - p); "random" returns
    keep * P / (1 - p) and O = that times V. LSE is the undropped one."""
    causal = causal_code(is_causal, causal_alignment)
    q, k, v = _f64(q), _f64(k), _f64(v)
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("q, k, v must be 4-D [B, H, S, D]")
    B, Hq, Sq, D = q.shape
    Bk, Hkv, Skv, Dk = k.shape
    Bv, Hv, Sv, Dv = v.shape
    if (Bk, Dk) != (B, D) or (Bv, Hv, Sv) != (B, Hkv, Skv):
        raise ValueError("q, k, v shapes disagree")
    if Hkv == 0 or Hq % Hkv != 0:
        raise ValueError(f"query heads {Hq} are not a multiple of key/value heads {Hkv}")
    if Hq != Hkv and not enable_gqa:
        raise ValueError("Hq != Hkv requires enable_gqa")
    if is_causal and attn_mask is not None:
        raise ValueError("is_causal and attn_mask are mutually exclusive")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    kind, marr, mstr = MASK_NONE, None, [0, 0, 0, 0]
    if attn_mask is not None:
        kind, marr, mstr = _mask_array(attn_mask, (B, Hq, Sq, Skv))
    karr, kstr = None, [0, 0, 0, 0]
    if dropout_mask is not None:
        kkind, karr, kstr = _mask_array(dropout_mask, (B, Hq, Sq, Skv))
        if kkind != MASK_BOOL:
            raise ValueError("dropout_mask must be bool")
        if dropout_rule not in DROPOUT_RULES:
            raise ValueError(f"dropout_rule must be one of {sorted(DROPOUT_RULES)}")
        if not 0.0 <= dropout_p < 1.0:
            raise ValueError("dropout_p must be in [0, 1)")
    out = np.empty((B, Hq, Sq, Dv), np.float64)
    probs = np.empty((B, Hq, Sq, Skv), np.float64)
    lse = np.empty((B, Hq, Sq), np.float64)
    dp = ctypes.POINTER(ctypes.c_double)
    st = (ctypes.c_int64 * 4)(*mstr)
    kst = (ctypes.c_int64 * 4)(*kstr)
    lib = load(lib_path)
    rc = lib.oracle_sdpa_fwd(q.ctypes.data_as(dp), k.ctypes.data_as(dp), v.ctypes.data_as(dp),
                             B, Hq, Hkv, Sq, Skv, D, Dv, kind,
                             None if marr is None else marr.ctypes.data_as(ctypes.c_void_p),
                             st, causal, float(scale),
                             None if karr is None else karr.ctypes.data_as(ctypes.c_void_p), kst,
                             float(dropout_p), DROPOUT_RULES.get(dropout_rule, 0),
                             out.ctypes.data_as(dp), probs.ctypes.data_as(dp), lse.ctypes.data_as(dp))
    if rc != 0:
        raise ValueError(f"oracle rejected the call (code {rc})")
    return out, probs, lse


def sdpa_backward_reference(q, k, v, attn_mask=None, is_causal: bool = False,
                            scale: Optional[float] = None, enable_gqa: bool = False,
                            dout=None, dprobs=None, lib_path: str = _LIB,
                            causal_alignment: str = "top_left"
                            ) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Return (dq [B,Hq,Sq,D], dk [B,Hkv,Skv,D], dv [B,Hkv,Skv,Dv]) in float64:
    the gradients of a loss whose gradients with respect to the forward's
    outputs are ``dout`` (dL/dO, required) and ``dprobs`` (dL/dP, or None).

    The plain chain rule through P = softmax(scale * Q K^T + mask) and
    O = P V (``oracle_sdpa_bwd`` in ``sdpa_oracle.c``), following the FlagOS-OP
    page's Implementation section (an autograd.Function with gradients from
    both outputs) and its "P800 fused backward" update (softmax Jacobian from
    the probability map; query-head gradients reduced back to the key/value
    heads). Removed keys and dead rows receive no gradient.
    """
    causal = causal_code(is_causal, causal_alignment)
    q, k, v = _f64(q), _f64(k), _f64(v)
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("q, k, v must be 4-D [B, H, S, D]")
    B, Hq, Sq, D = q.shape
    Bk, Hkv, Skv, Dk = k.shape
    Bv, Hv, Sv, Dv = v.shape
    if (Bk, Dk) != (B, D) or (Bv, Hv, Sv) != (B, Hkv, Skv):
        raise ValueError("q, k, v shapes disagree")
    if Hkv == 0 or Hq % Hkv != 0:
        raise ValueError(f"query heads {Hq} are not a multiple of key/value heads {Hkv}")
    if Hq != Hkv and not enable_gqa:
        raise ValueError("Hq != Hkv requires enable_gqa")
    if is_causal and attn_mask is not None:
        raise ValueError("is_causal and attn_mask are mutually exclusive")
    if dout is None:
        raise ValueError("dout is required")
    do = _f64(dout)
    if do.shape != (B, Hq, Sq, Dv):
        raise ValueError("dout must be [B, Hq, Sq, Dv]")
    dpr = None
    if dprobs is not None:
        dpr = _f64(dprobs)
        if dpr.shape != (B, Hq, Sq, Skv):
            raise ValueError("dprobs must be [B, Hq, Sq, Skv]")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    kind, marr, mstr = MASK_NONE, None, [0, 0, 0, 0]
    if attn_mask is not None:
        kind, marr, mstr = _mask_array(attn_mask, (B, Hq, Sq, Skv))
    dq = np.empty((B, Hq, Sq, D), np.float64)
    dk = np.empty((B, Hkv, Skv, D), np.float64)
    dv = np.empty((B, Hkv, Skv, Dv), np.float64)
    dp = ctypes.POINTER(ctypes.c_double)
    st = (ctypes.c_int64 * 4)(*mstr)
    lib = load(lib_path)
    rc = lib.oracle_sdpa_bwd(q.ctypes.data_as(dp), k.ctypes.data_as(dp), v.ctypes.data_as(dp),
                             B, Hq, Hkv, Sq, Skv, D, Dv, kind,
                             None if marr is None else marr.ctypes.data_as(ctypes.c_void_p),
                             st, causal, float(scale), do.ctypes.data_as(dp),
                             None if dpr is None else dpr.ctypes.data_as(dp),
                             dq.ctypes.data_as(dp), dk.ctypes.data_as(dp), dv.ctypes.data_as(dp))
    if rc != 0:
        raise ValueError(f"oracle rejected the call (code {rc})")
    return dq, dk, dv


def sdpa_varlen_reference(q, k, v, cu_seqlens_q, cu_seqlens_kv, max_seqlen_kv: int, is_causal: bool = False,
                          scale: Optional[float] = None, enable_gqa: bool = False,
                          causal_alignment: str = "top_left") -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Packed variable-length sequences (token-major q [Tq, Hq, D], k/v
    [Tkv, Hkv, D], cumulative offsets cu_seqlens_*; the THD layout of the
    cudnn-frontend pull request "[SDPA] SM80 fwd: TemplateParams kernels,
    plan-time compile, sym_int THD extents"): each sequence is an independent
    call of ``sdpa_reference`` on its own tokens. Returns O [Tq, Hq, Dv],
    P [Tq, Hq, max_seqlen_kv] (zeros past each sequence's keys) and
    LSE [Tq, Hq], float64. A token outside every sequence gets O = 0, P = 0 and
    LSE = -inf."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    cq = [int(x) for x in np.asarray(cu_seqlens_q.cpu() if hasattr(cu_seqlens_q, "cpu") else cu_seqlens_q)]
    ck = [int(x) for x in np.asarray(cu_seqlens_kv.cpu() if hasattr(cu_seqlens_kv, "cpu") else cu_seqlens_kv)]
    if len(cq) != len(ck) or len(cq) < 1:
        raise ValueError("cu_seqlens_q and cu_seqlens_kv must hold n_seqs + 1 offsets each")
    Tq, Hq, _ = q.shape
    Dv = v.shape[2]
    out = np.zeros((Tq, Hq, Dv))
    probs = np.zeros((Tq, Hq, max_seqlen_kv))
    lse = np.full((Tq, Hq), -np.inf)
    for b in range(len(cq) - 1):
        q0, q1, k0, k1 = cq[b], cq[b + 1], ck[b], ck[b + 1]
        if q1 <= q0:
            continue
        if k1 - k0 > max_seqlen_kv:
            raise ValueError("a sequence has more keys than max_seqlen_kv")
        qs = q[q0:q1].transpose(1, 0, 2)[None]
        ks = k[k0:k1].transpose(1, 0, 2)[None]
        vs = v[k0:k1].transpose(1, 0, 2)[None]
        o, p, l = sdpa_reference(qs, ks, vs, None, is_causal, scale, enable_gqa, causal_alignment=causal_alignment)
        out[q0:q1] = o[0].transpose(1, 0, 2)
        probs[q0:q1, :, :k1 - k0] = p[0].transpose(1, 0, 2)
        lse[q0:q1] = l[0].T
    return out, probs, lse
