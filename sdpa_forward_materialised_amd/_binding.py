"""ctypes binding of libsdpa_math.so (argument marshalling only).

Every step of the forward runs in the HIP library; this module only turns
torch tensors into ``sdpa_tensor_t`` descriptors, allocates the outputs with
torch's caching allocator and passes torch's current stream. There is no
fallback: if the library is missing or the device is not a GPU, calls fail.
"""

from __future__ import annotations

import ctypes
import math
import os
import struct
from typing import Optional, Tuple

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libsdpa_math.so")

SDPA_F32, SDPA_F16, SDPA_BF16, SDPA_BOOL = 0, 1, 2, 3
PATH_AUTO, PATH_FUSED, PATH_TWOPASS = 0, 1, 2
PATHS = {"auto": PATH_AUTO, "fused": PATH_FUSED, "twopass": PATH_TWOPASS}
PATH_FUSED_WIDE = 3  # reported by sdpa_math_plan: the fused path on its wide kernel
PATH_NAMES = {**{v: k for k, v in PATHS.items()}, PATH_FUSED_WIDE: "fused"}
KERNEL_NAMES = {PATH_FUSED: "sdpa_fused_kernel", PATH_FUSED_WIDE: "sdpa_fused_wide_kernel",
                PATH_TWOPASS: "sdpa_twopass_kernel"}
CAUSAL_ALIGNMENTS = {"top_left": 1, "bottom_right": 2}  # the C ABI's is_causal codes

_DTYPES = {torch.float32: SDPA_F32, torch.float16: SDPA_F16, torch.bfloat16: SDPA_BF16,
           torch.bool: SDPA_BOOL}

EXPORTS = ("sdpa_math_fwd", "sdpa_math_fwd_path", "sdpa_math_fwd_ws", "sdpa_math_workspace_bytes",
           "sdpa_math_fwd_noalloc", "sdpa_math_fwd_dropout", "sdpa_math_fwd_varlen", "sdpa_math_bwd", "sdpa_math_bwd_workspace_bytes", "sdpa_math_plan",
           "sdpa_math_last_error",
           "sdpa_math_version", "sdpa_probe_fill", "sdpa_probe_copy")


class SdpaTensor(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("ndim", ctypes.c_int32),
                ("sizes", ctypes.c_int64 * 4), ("strides", ctypes.c_int64 * 4)]


# sdpa_tensor_t byte layouts: pointer, dtype, ndim, sizes[4], strides[4]
# (unused trailing entries zero)
_PACK = {4: struct.Struct("<Qii4q4q"), 3: struct.Struct("<Qii3q8x3q8x"), 2: struct.Struct("<Qii2q16x2q16x")}
assert all(p.size == ctypes.sizeof(SdpaTensor) for p in _PACK.values())

_lib = None
_WS_BYTES = {}  # workspace bytes per call signature (shapes, dtypes, mask layout, flags)


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m sdpa_forward_materialised_amd.build` "
                           "(there is no CPU fallback)")
    lib = ctypes.CDLL(path)
    # tensor descriptors go in as the bytes of an sdpa_tensor_t (built by
    # _desc; the library only reads them), or None for NULL
    T = ctypes.c_char_p
    lib.sdpa_math_fwd.restype = ctypes.c_int
    lib.sdpa_math_fwd.argtypes = [T, T, T, T, ctypes.c_int, ctypes.c_float, ctypes.c_int, T, T, T, ctypes.c_void_p]
    lib.sdpa_math_fwd_path.restype = ctypes.c_int
    lib.sdpa_math_fwd_path.argtypes = lib.sdpa_math_fwd.argtypes + [ctypes.c_int]
    lib.sdpa_math_fwd_ws.restype = ctypes.c_int
    lib.sdpa_math_fwd_ws.argtypes = [T, T, T, T, ctypes.c_int, ctypes.c_float, ctypes.c_int, T, T, T,
                                     ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int]
    lib.sdpa_math_fwd_varlen.restype = ctypes.c_int
    lib.sdpa_math_fwd_varlen.argtypes = [T, T, T, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                         ctypes.c_int64, ctypes.c_int, ctypes.c_float, ctypes.c_int, T, T, T,
                                         ctypes.c_void_p]
    lib.sdpa_math_fwd_dropout.restype = ctypes.c_int
    lib.sdpa_math_fwd_dropout.argtypes = [T, T, T, T, ctypes.c_int, ctypes.c_float, ctypes.c_int, ctypes.c_float, T,
                                          ctypes.c_int, T, T, T, ctypes.c_void_p]
    lib.sdpa_math_fwd_noalloc.restype = ctypes.c_int
    lib.sdpa_math_fwd_noalloc.argtypes = lib.sdpa_math_fwd.argtypes + [ctypes.c_int]
    lib.sdpa_math_bwd.restype = ctypes.c_int
    lib.sdpa_math_bwd.argtypes = [T, T, T, T, ctypes.c_int, ctypes.c_float, ctypes.c_int, T, T, T, T, T, T,
                                  ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    lib.sdpa_math_bwd_workspace_bytes.restype = ctypes.c_int
    lib.sdpa_math_bwd_workspace_bytes.argtypes = [T, T, T, T, ctypes.c_int, ctypes.c_int,
                                                  ctypes.POINTER(ctypes.c_size_t)]
    lib.sdpa_math_workspace_bytes.restype = ctypes.c_int
    lib.sdpa_math_workspace_bytes.argtypes = [T, T, T, T, ctypes.c_int, ctypes.c_int, ctypes.POINTER(ctypes.c_size_t)]
    lib.sdpa_math_plan.restype = ctypes.c_int
    lib.sdpa_math_plan.argtypes = [T, T, T, T, ctypes.c_int, ctypes.c_int, ctypes.POINTER(ctypes.c_int32),
                                   ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int64)]
    lib.sdpa_math_last_error.restype = ctypes.c_char_p
    lib.sdpa_math_last_error.argtypes = []
    lib.sdpa_math_version.restype = ctypes.c_int
    lib.sdpa_math_version.argtypes = []
    lib.sdpa_probe_fill.restype = ctypes.c_int
    lib.sdpa_probe_fill.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_uint32, ctypes.c_void_p]
    lib.sdpa_probe_copy.restype = ctypes.c_int
    lib.sdpa_probe_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    _lib = lib
    return lib


def _desc(t: Optional[torch.Tensor], ndim: int) -> Optional[bytes]:
    if t is None:
        return None
    if t.dim() > ndim:
        raise ValueError(f"expected at most {ndim} dims, got {t.dim()}")
    while t.dim() < ndim:  # right-align (a mask may have fewer dims)
        t = t.unsqueeze(0)
    dt = _DTYPES.get(t.dtype)
    if dt is None:
        raise ValueError(f"unsupported dtype {t.dtype}")
    # the sdpa_tensor_t bytes, packed in one go (building a ctypes struct
    # costs a few microseconds more per call over the seven descriptors)
    return _PACK[ndim].pack(t.data_ptr() if t.numel() > 0 else 0, dt, ndim, *t.shape, *t.stride())


def _raise(code: int, lib) -> None:
    msg = lib.sdpa_math_last_error().decode()
    if code == 1:
        raise ValueError(msg)
    if code == 2:
        raise NotImplementedError(msg)
    raise RuntimeError(f"sdpa_math: {msg}")


def _check_devices(*ts):
    dev = None
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("sdpa_math runs on the GPU only: every tensor must be a cuda tensor")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"tensors on different devices ({dev} and {t.device})")
    return dev


# torch's current stream on a device, as the raw HIP handle (torch's own
# pointer query when it has one: no Stream object built per call)
_RAW_STREAM = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _current_stream(dev: torch.device) -> int:
    if _RAW_STREAM is not None:
        return _RAW_STREAM(dev.index)
    return torch.cuda.current_stream(dev).cuda_stream


def _causal_code(is_causal, causal_alignment: str) -> int:
    if causal_alignment not in CAUSAL_ALIGNMENTS:
        raise ValueError(f"causal_alignment must be one of {sorted(CAUSAL_ALIGNMENTS)}")
    return CAUSAL_ALIGNMENTS[causal_alignment] if is_causal else 0


DROPOUT_RULES = {"explicit": 0, "random": 1}


# planner overrides the workspace size depends on
_PLAN_ENV = ("SDPA_MATH_PATH", "SDPA_MATH_SPLITS", "SDPA_MATH_TP_WAVES", "SDPA_MATH_RANGES", "SDPA_MATH_RANGE_KEYS",
             "SDPA_MATH_RANGE_WAVES")


def fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, attn_mask: Optional[torch.Tensor] = None,
        is_causal: bool = False, scale: Optional[float] = None, enable_gqa: bool = False,
        path: str = "auto", out: Optional[Tuple[torch.Tensor, torch.Tensor, torch.Tensor]] = None,
        causal_alignment: str = "top_left", dropout_p: float = 0.0,
        dropout_mask: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """Return (O [B,Hq,Sq,Dv], P [B,Hq,Sq,Skv], LSE [B,Hq,Sq] float32).

    ``scale=None`` means 1/sqrt(D). ``path`` is "auto", "fused" or "twopass".
    ``causal_alignment`` ("top_left" or "bottom_right") places the causal
    diagonal when ``is_causal``: key j is removed for query i when j > i, or
    when j > i + Skv - Sq.
    ``out`` may pass preallocated (O, P, LSE) buffers (any strides with a
    contiguous last dim); by default P and O share one allocation.
    ``dropout_p > 0``: with ``dropout_mask`` (bool, True keeps) the explicit
    rule (P = keep * P, O divided by 1 - p); without one, the random rule on a
    keep-mask drawn here with torch's generator (P = keep * P / (1 - p)).
    """
    lib = load_library()
    dev = _check_devices(q, k, v, attn_mask)
    causal = _causal_code(is_causal, causal_alignment)
    if path not in PATHS:
        raise ValueError(f"path must be one of {sorted(PATHS)}")
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be 4-D [B, H, S, D]")
    B, Hq, Sq, D = q.shape
    Skv, Dv = k.shape[2], v.shape[3]
    if scale is None:
        scale = 1.0 / math.sqrt(D) if D > 0 else 1.0
    if out is None:
        n_p = B * Hq * Sq * Skv
        n_o = B * Hq * Sq * Dv
        pad = (-n_p) % 64  # keep O 128-byte aligned behind P
        buf = torch.empty(n_p + pad + n_o, dtype=q.dtype, device=dev)
        P = buf[:n_p].view(B, Hq, Sq, Skv)
        O = buf[n_p + pad:].view(B, Hq, Sq, Dv)
        L = torch.empty((B, Hq, Sq), dtype=torch.float32, device=dev)
    else:
        O, P, L = out
        _check_devices(q, O, P, L)
    dq, dk, dv = _desc(q, 4), _desc(k, 4), _desc(v, 4)
    dm = _desc(attn_mask, 4)
    do, dp, dl = _desc(O, 4), _desc(P, 4), _desc(L, 3)
    if dropout_p > 0 or dropout_mask is not None:
        if path == "fused":
            raise NotImplementedError("dropout runs on the two-pass path only")
        rule = DROPOUT_RULES["explicit"] if dropout_mask is not None else DROPOUT_RULES["random"]
        if dropout_mask is None:  # the random rule's keep draws
            dropout_mask = torch.rand((B, q.shape[1], Sq, Skv), device=dev) >= dropout_p
        _check_devices(q, dropout_mask)

        def launch_drop():
            return lib.sdpa_math_fwd_dropout(dq, dk, dv, dm, causal, float(scale), int(bool(enable_gqa)),
                                             float(dropout_p), _desc(dropout_mask, 4), rule, do, dp, dl,
                                             ctypes.c_void_p(_current_stream(dev)))
        if dev.index == torch.cuda.current_device():
            rc = launch_drop()
        else:
            with torch.cuda.device(dev):
                rc = launch_drop()
        if rc != 0:
            _raise(rc, lib)
        return O, P, L
    # workspace for key ranges, when the library would split this call
    # (the byte count depends on dtypes, shapes, mask layout and flags only:
    # remembered per signature, the descriptors' bytes past the data pointer)
    sig = (dq[8:], dk[8:], None if dm is None else dm[8:], causal, bool(enable_gqa),
           tuple(os.environ.get(e) for e in _PLAN_ENV))
    nbytes = _WS_BYTES.get(sig)
    if nbytes is None:
        n = ctypes.c_size_t(0)
        rc = lib.sdpa_math_workspace_bytes(dq, dk, dv, dm, causal, int(bool(enable_gqa)),
                                           ctypes.byref(n))
        if rc != 0:
            _raise(rc, lib)
        if len(_WS_BYTES) >= 4096:  # many distinct shapes: start over rather than grow
            _WS_BYTES.clear()
        nbytes = _WS_BYTES[sig] = n.value
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev) if nbytes > 0 else None

    def launch():
        stream = _current_stream(dev)
        return lib.sdpa_math_fwd_ws(dq, dk, dv, dm, causal,
                                    float(scale), int(bool(enable_gqa)), do, dp, dl,
                                    None if ws is None else ctypes.c_void_p(ws.data_ptr()), nbytes,
                                    ctypes.c_void_p(stream), PATHS[path])

    # the launch goes to the tensors' device (made current only when it is not)
    if dev.index == torch.cuda.current_device():
        rc = launch()
    else:
        with torch.cuda.device(dev):
            rc = launch()
    if rc != 0:
        _raise(rc, lib)
    return O, P, L


class PreparedFwd:
    """A forward call bound to fixed tensors: ``prepare_fwd`` validates the
    arguments, packs the tensor descriptors and sizes the key-range workspace
    once; each ``run()`` then launches with one C call (about a torch op
    launch of host time, where ``fwd`` also spends some microseconds on
    argument handling), for loops that refill the same buffers in place.
    The tensors must keep their storage, shapes and strides between runs
    (they are held here, so they stay alive)."""

    def __init__(self, q, k, v, attn_mask, is_causal, scale, enable_gqa, path, out, causal_alignment):
        self._lib = load_library()
        self._dev = _check_devices(q, k, v, attn_mask)
        if path not in PATHS:
            raise ValueError(f"path must be one of {sorted(PATHS)}")
        if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
            raise ValueError("q, k, v must be 4-D [B, H, S, D]")
        B, Hq, Sq, D = q.shape
        Skv, Dv = k.shape[2], v.shape[3]
        if out is None:
            out = (torch.empty((B, Hq, Sq, Dv), dtype=q.dtype, device=self._dev),
                   torch.empty((B, Hq, Sq, Skv), dtype=q.dtype, device=self._dev),
                   torch.empty((B, Hq, Sq), dtype=torch.float32, device=self._dev))
        _check_devices(q, *out)
        self.out = tuple(out)
        self._keep = (q, k, v, attn_mask)
        causal = _causal_code(is_causal, causal_alignment)
        dq, dk, dv, dm = _desc(q, 4), _desc(k, 4), _desc(v, 4), _desc(attn_mask, 4)
        n = ctypes.c_size_t(0)
        rc = self._lib.sdpa_math_workspace_bytes(dq, dk, dv, dm, causal, int(bool(enable_gqa)), ctypes.byref(n))
        if rc != 0:
            _raise(rc, self._lib)
        self._ws = torch.empty(n.value, dtype=torch.uint8, device=self._dev) if n.value > 0 else None
        if scale is None:
            scale = 1.0 / math.sqrt(D) if D > 0 else 1.0
        self._args = (dq, dk, dv, dm, causal, float(scale), int(bool(enable_gqa)),
                      _desc(self.out[0], 4), _desc(self.out[1], 4), _desc(self.out[2], 3),
                      None if self._ws is None else ctypes.c_void_p(self._ws.data_ptr()), n.value)
        self._path = PATHS[path]
        # validate everything once, on the current stream
        self.run()

    def run(self, stream: Optional[int] = None) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
        """Launch on ``stream`` (a raw HIP stream handle; default: the
        current stream of the tensors' device, which must be current)."""
        st = _current_stream(self._dev) if stream is None else stream
        rc = self._lib.sdpa_math_fwd_ws(*self._args, ctypes.c_void_p(st), self._path)
        if rc != 0:
            _raise(rc, self._lib)
        return self.out


def prepare_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, attn_mask: Optional[torch.Tensor] = None,
                is_causal: bool = False, scale: Optional[float] = None, enable_gqa: bool = False,
                path: str = "auto", out: Optional[Tuple[torch.Tensor, torch.Tensor, torch.Tensor]] = None,
                causal_alignment: str = "top_left") -> PreparedFwd:
    """``fwd`` bound to these tensors (see PreparedFwd); runs it once."""
    return PreparedFwd(q, k, v, attn_mask, is_causal, scale, enable_gqa, path, out, causal_alignment)


def fwd_varlen(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cu_seqlens_q: torch.Tensor,
               cu_seqlens_kv: torch.Tensor, max_seqlen_q: int, max_seqlen_kv: int, is_causal: bool = False,
               scale: Optional[float] = None, enable_gqa: bool = False, causal_alignment: str = "top_left",
               out: Optional[Tuple[torch.Tensor, torch.Tensor, torch.Tensor]] = None
               ) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """``sdpa_math_fwd_varlen``: packed sequences q [Tq, Hq, D], k/v [Tkv, Hkv, D]
    with int32 cu_seqlens on the device. Returns (O [Tq, Hq, Dv],
    P [Tq, Hq, max_seqlen_kv] (zeros past each sequence's keys), LSE [Tq, Hq])."""
    lib = load_library()
    dev = _check_devices(q, k, v, cu_seqlens_q, cu_seqlens_kv)
    for name, cu in (("cu_seqlens_q", cu_seqlens_q), ("cu_seqlens_kv", cu_seqlens_kv)):
        if cu.dtype != torch.int32 or cu.dim() != 1 or not cu.is_contiguous():
            raise ValueError(f"{name} must be a contiguous 1-D int32 tensor")
    if cu_seqlens_q.numel() != cu_seqlens_kv.numel() or cu_seqlens_q.numel() < 1:
        raise ValueError("cu_seqlens_q and cu_seqlens_kv must hold n_seqs + 1 offsets each")
    causal = _causal_code(is_causal, causal_alignment)
    if q.dim() != 3 or k.dim() != 3 or v.dim() != 3:
        raise ValueError("q, k, v must be 3-D [T, H, D]")
    Tq, Hq, D = q.shape
    Dv = v.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(D) if D > 0 else 1.0
    if out is None:
        O = torch.empty((Tq, Hq, Dv), dtype=q.dtype, device=dev)
        P = torch.empty((Tq, Hq, max_seqlen_kv), dtype=q.dtype, device=dev)
        L = torch.empty((Tq, Hq), dtype=torch.float32, device=dev)
    else:
        O, P, L = out
    args = (_desc(q, 3), _desc(k, 3), _desc(v, 3), ctypes.c_void_p(cu_seqlens_q.data_ptr()),
            ctypes.c_void_p(cu_seqlens_kv.data_ptr()), cu_seqlens_q.numel() - 1, int(max_seqlen_q),
            int(max_seqlen_kv), causal, float(scale), int(bool(enable_gqa)), _desc(O, 3), _desc(P, 3), _desc(L, 2))
    if dev.index == torch.cuda.current_device():
        rc = lib.sdpa_math_fwd_varlen(*args, ctypes.c_void_p(_current_stream(dev)))
    else:
        with torch.cuda.device(dev):
            rc = lib.sdpa_math_fwd_varlen(*args, ctypes.c_void_p(_current_stream(dev)))
    if rc != 0:
        _raise(rc, lib)
    return O, P, L


def fwd_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                out: Tuple[torch.Tensor, torch.Tensor, torch.Tensor],
                attn_mask: Optional[torch.Tensor] = None, is_causal: bool = False, scale: Optional[float] = None,
                enable_gqa: bool = False, path: str = "auto", causal_alignment: str = "top_left") -> None:
    """``sdpa_math_fwd_noalloc``: the forward into caller-provided (O, P, LSE)
    buffers with nothing allocated, neither by the library (its key-range
    scratch is a static per-device array) nor here. Calls that may overlap on
    one GPU share that scratch and must be ordered by the caller."""
    lib = load_library()
    O, P, L = out
    dev = _check_devices(q, k, v, attn_mask, O, P, L)
    causal = _causal_code(is_causal, causal_alignment)
    if path not in PATHS:
        raise ValueError(f"path must be one of {sorted(PATHS)}")
    if q.dim() != 4:
        raise ValueError("q, k, v must be 4-D [B, H, S, D]")
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[3]) if q.shape[3] > 0 else 1.0
    args = (_desc(q, 4), _desc(k, 4), _desc(v, 4), _desc(attn_mask, 4), causal, float(scale),
            int(bool(enable_gqa)), _desc(O, 4), _desc(P, 4), _desc(L, 3))
    if dev.index == torch.cuda.current_device():
        rc = lib.sdpa_math_fwd_noalloc(*args, ctypes.c_void_p(_current_stream(dev)), PATHS[path])
    else:
        with torch.cuda.device(dev):
            rc = lib.sdpa_math_fwd_noalloc(*args, ctypes.c_void_p(_current_stream(dev)), PATHS[path])
    if rc != 0:
        _raise(rc, lib)


def bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, lse: torch.Tensor, dout: torch.Tensor,
        dprobs: Optional[torch.Tensor] = None, attn_mask: Optional[torch.Tensor] = None, is_causal: bool = False,
        scale: Optional[float] = None, enable_gqa: bool = False, causal_alignment: str = "top_left",
        out: Optional[Tuple[torch.Tensor, torch.Tensor, torch.Tensor]] = None
        ) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """``sdpa_math_bwd``: (dq, dk, dv) for upstream gradients ``dout`` (dL/dO)
    and ``dprobs`` (dL/dP, or None). The other arguments are those of the
    forward call and its LSE. ``out`` may pass preallocated (dq, dk, dv)."""
    lib = load_library()
    dev = _check_devices(q, k, v, attn_mask, lse, dout, dprobs)
    causal = _causal_code(is_causal, causal_alignment)
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be 4-D [B, H, S, D]")
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[3]) if q.shape[3] > 0 else 1.0
    if out is None:
        dq, dk, dv = torch.empty_like(q, memory_format=torch.contiguous_format), \
            torch.empty_like(k, memory_format=torch.contiguous_format), \
            torch.empty_like(v, memory_format=torch.contiguous_format)
    else:
        dq, dk, dv = out
        _check_devices(q, dq, dk, dv)
    dq_, dk_, dv_ = _desc(q, 4), _desc(k, 4), _desc(v, 4)
    dm = _desc(attn_mask, 4)
    n = ctypes.c_size_t(0)
    rc = lib.sdpa_math_bwd_workspace_bytes(dq_, dk_, dv_, dm, causal, int(bool(enable_gqa)), ctypes.byref(n))
    if rc != 0:
        _raise(rc, lib)
    ws = torch.empty(max(n.value, 16), dtype=torch.uint8, device=dev)
    args = (dq_, dk_, dv_, dm, causal, float(scale), int(bool(enable_gqa)), _desc(lse, 3), _desc(dout, 4),
            _desc(dprobs, 4), _desc(dq, 4), _desc(dk, 4), _desc(dv, 4), ctypes.c_void_p(ws.data_ptr()), n.value)
    if dev.index == torch.cuda.current_device():
        rc = lib.sdpa_math_bwd(*args, ctypes.c_void_p(_current_stream(dev)))
    else:
        with torch.cuda.device(dev):
            rc = lib.sdpa_math_bwd(*args, ctypes.c_void_p(_current_stream(dev)))
    if rc != 0:
        _raise(rc, lib)
    return dq, dk, dv


class SdpaMathFunction(torch.autograd.Function):
    """(O, P) = sdpa_math(q, k, v, ...) with gradients from both outputs
    (the FlagOS-OP page's autograd.Function, Implementation section): the
    forward saves q, k, v, the mask and LSE; the backward calls
    ``sdpa_math_bwd`` with dL/dO and dL/dP. The mask gets no gradient."""

    @staticmethod
    def forward(ctx, q, k, v, attn_mask, is_causal, scale, enable_gqa, causal_alignment):
        O, P, L = fwd(q, k, v, attn_mask, is_causal, scale, enable_gqa, causal_alignment=causal_alignment)
        ctx.save_for_backward(q, k, v, attn_mask, L)
        ctx.args = (is_causal, scale, enable_gqa, causal_alignment)
        ctx.mark_non_differentiable(L)
        return O, P, L

    @staticmethod
    def backward(ctx, dO, dP, dL):
        q, k, v, m, L = ctx.saved_tensors
        is_causal, scale, gqa, align = ctx.args
        if dO is None:
            dO = torch.zeros(q.shape[:3] + (v.shape[3],), dtype=q.dtype, device=q.device)
        dq, dk, dv = bwd(q, k, v, L, dO.contiguous(), None if dP is None else dP.contiguous(), m, is_causal, scale,
                         gqa, align)
        return dq, dk, dv, None, None, None, None, None


def sdpa_math(q, k, v, attn_mask=None, is_causal=False, scale=None, enable_gqa=False, causal_alignment="top_left"):
    """Differentiable (O, P, LSE): ``fwd`` with ``sdpa_math_bwd`` as its
    backward (gradients reach q, k and v through both O and P)."""
    return SdpaMathFunction.apply(q, k, v, attn_mask, is_causal, scale, enable_gqa, causal_alignment)


def plan(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, attn_mask: Optional[torch.Tensor] = None,
         is_causal: bool = False, enable_gqa: bool = False, causal_alignment: str = "top_left"):
    """Validate like ``fwd`` and return (path name, tiles per (b,h), 64x64 tiles per (b,h)).

    Reads only shapes, strides, dtypes and pointers; works on CPU tensors too.
    """
    lib = load_library()
    path = ctypes.c_int32(-1)
    tiles = ctypes.c_int64(-1)
    tiles64 = ctypes.c_int64(-1)
    rc = lib.sdpa_math_plan(_desc(q, 4), _desc(k, 4), _desc(v, 4),
                            _desc(attn_mask, 4), _causal_code(is_causal, causal_alignment),
                            int(bool(enable_gqa)),
                            ctypes.byref(path), ctypes.byref(tiles), ctypes.byref(tiles64))
    if rc != 0:
        _raise(rc, lib)
    return PATH_NAMES[path.value], tiles.value, tiles64.value


def kernel_name(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, attn_mask: Optional[torch.Tensor] = None,
                is_causal: bool = False, enable_gqa: bool = False, causal_alignment: str = "top_left") -> str:
    """Name of the kernel that does the bulk of a call planned like ``plan``."""
    lib = load_library()
    path = ctypes.c_int32(-1)
    rc = lib.sdpa_math_plan(_desc(q, 4), _desc(k, 4), _desc(v, 4), _desc(attn_mask, 4),
                            _causal_code(is_causal, causal_alignment), int(bool(enable_gqa)),
                            ctypes.byref(path), None, None)
    if rc != 0:
        _raise(rc, lib)
    return KERNEL_NAMES[path.value]


def probe_fill(dst: torch.Tensor, value: int = 0) -> None:
    """Streaming write of `dst` (whole tensor) with the library's fill kernel."""
    lib = load_library()
    _check_devices(dst)
    with torch.cuda.device(dst.device):
        rc = lib.sdpa_probe_fill(ctypes.c_void_p(dst.data_ptr()), dst.numel() * dst.element_size(), value,
                                 ctypes.c_void_p(torch.cuda.current_stream(dst.device).cuda_stream))
    if rc != 0:
        raise RuntimeError(f"sdpa_probe_fill failed with hip error {rc}")


def probe_copy(dst: torch.Tensor, src: torch.Tensor) -> None:
    """Streaming copy src -> dst (same byte size) with the library's copy kernel."""
    lib = load_library()
    _check_devices(dst, src)
    nbytes = dst.numel() * dst.element_size()
    if nbytes != src.numel() * src.element_size():
        raise ValueError("probe_copy needs equal byte sizes")
    with torch.cuda.device(dst.device):
        rc = lib.sdpa_probe_copy(ctypes.c_void_p(dst.data_ptr()), ctypes.c_void_p(src.data_ptr()), nbytes,
                                 ctypes.c_void_p(torch.cuda.current_stream(dst.device).cuda_stream))
    if rc != 0:
        raise RuntimeError(f"sdpa_probe_copy failed with hip error {rc}")


def version() -> int:
    return int(load_library().sdpa_math_version())


def last_error() -> str:
    return load_library().sdpa_math_last_error().decode()
