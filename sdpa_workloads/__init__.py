"""Seeded synthetic inputs for the materialised-probability SDPA forward.

This module only draws numbers and names shapes. It holds none of the
attention arithmetic, so that the HIP path and the CPU oracle can both be fed
from it without sharing any of the method.

The five workloads follow the shapes the FlagOS-OP ``sdpa_math`` pull request
times (page "feat: add sdpa_math operator", performance tables: prefill 1k/2k
at D64/D128, GQA 1k D128, decode/tail with a KV cache), with batch and head
counts fixed here because the page never prints them.

Recipe (all inputs):
  * ``numpy.random.default_rng(seed)`` (PCG64), draws in the order Q, K, V,
    then whatever the mask needs;
  * Q, K, V are i.i.d. standard normal in float64, then rounded to the compute
    dtype with round-to-nearest-even (torch's CPU cast);
  * layouts are contiguous ``[B, H, S, D]``.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional, Sequence

import numpy as np
import torch

TORCH_DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic attention call: shapes, dtype, mask recipe and seed."""

    name: str
    dtype: str          # "f32" | "f16" | "bf16"
    B: int
    Hq: int
    Hkv: int
    Sq: int
    Skv: int
    D: int
    causal: bool
    mask: str           # "none" | "keypad_bool" | "random_neginf_add"
    seed: int
    Dv: Optional[int] = None
    align: str = "top_left"  # causal alignment: "top_left" | "bottom_right"

    @property
    def dv(self) -> int:
        return self.D if self.Dv is None else self.Dv

    @property
    def gqa(self) -> bool:
        return self.Hq != self.Hkv

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    def describe(self) -> str:
        return (f"{self.name}: {self.dtype} B={self.B} Hq={self.Hq} Hkv={self.Hkv} "
                f"Sq={self.Sq} Skv={self.Skv} D={self.D} causal={self.causal} mask={self.mask}")


# The five workloads (tiny check case, then the four timed shapes).
WORKLOADS: Sequence[Workload] = (
    Workload("tiny_f32_causal", "f32", 1, 2, 2, 64, 64, 32, True, "none", 1),
    Workload("prefill_1k_d64_f16_causal", "f16", 4, 8, 8, 1024, 1024, 64, True, "none", 2),
    Workload("prefill_2k_d128_bf16_causal", "bf16", 2, 16, 16, 2048, 2048, 128, True, "none", 3),
    Workload("gqa_1k_d128_f16_keypad", "f16", 4, 32, 8, 1024, 1024, 128, False, "keypad_bool", 4),
    Workload("decode_100x1152_d64_f16_addmask", "f16", 16, 8, 8, 100, 1152, 64, False,
             "random_neginf_add", 5),
)

# Measured beside them, not one of the five: a 512-query chunk of a prefill
# against a 2048-key cache with bottom-right causal alignment (the chunked-
# prefill shape the cudnn-frontend merge-log notes time), bf16, head dim 128.
EXTRA_WORKLOADS: Sequence[Workload] = (
    Workload("chunk_512x2048_d128_bf16_bottom_right", "bf16", 2, 16, 16, 512, 2048, 128, True, "none", 6,
             align="bottom_right"),
    # one query row per head against a long key cache: the keys are split over workgroups
    Workload("decode_1x32768_d128_bf16", "bf16", 4, 8, 8, 1, 32768, 128, False, "none", 7),
    # batched decode with grouped heads (4 query heads per KV head) against a 4096-key cache
    Workload("decode_gqa_16x32x8_1x4096_d128_bf16", "bf16", 16, 32, 8, 1, 4096, 128, False, "none", 8),
)

BY_NAME: Dict[str, Workload] = {w.name: w for w in (*WORKLOADS, *EXTRA_WORKLOADS)}


def to_dtype(x: np.ndarray, dtype: str) -> torch.Tensor:
    """float64 array -> CPU tensor of ``dtype`` (round to nearest even)."""
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float64)).to(TORCH_DTYPES[dtype])


def normal(rng: np.random.Generator, shape, dtype: str) -> torch.Tensor:
    return to_dtype(rng.standard_normal(shape), dtype)


def keypad_bool_mask(rng: np.random.Generator, B: int, Sq: int, Skv: int, lo: int, hi: int,
                     dead_rows: int = 0) -> torch.Tensor:
    """Key-padding mask ``[B, 1, Sq, Skv]``: True = attend.

    Batch b keeps keys ``j < L_b`` with ``L_b`` uniform on ``[lo, hi]``; in batch 0
    the first ``dead_rows`` query rows keep no key at all.
    """
    lens = rng.integers(lo, hi, size=B, endpoint=True)
    j = np.arange(Skv)
    m = np.broadcast_to(j[None, None, None, :] < lens[:, None, None, None], (B, 1, Sq, Skv)).copy()
    if dead_rows:
        m[0, 0, :dead_rows, :] = False
    return torch.from_numpy(m)


def random_neginf_add_mask(rng: np.random.Generator, shape, p: float, dtype: str) -> torch.Tensor:
    """Additive mask of zeros with ``-inf`` at an i.i.d. Bernoulli(p) subset."""
    hit = rng.random(shape) < p
    return to_dtype(np.where(hit, -np.inf, 0.0), dtype)


def random_bool_mask(rng: np.random.Generator, shape, p_true: float) -> torch.Tensor:
    return torch.from_numpy(rng.random(shape) < p_true)


def random_add_mask(rng: np.random.Generator, shape, dtype: str, p_neginf: float = 0.0) -> torch.Tensor:
    """Finite N(0,1) additive bias with an optional ``-inf`` subset."""
    x = rng.standard_normal(shape)
    if p_neginf > 0:
        x = np.where(rng.random(shape) < p_neginf, -np.inf, x)
    return to_dtype(x, dtype)


def make_inputs(w: Workload) -> Dict[str, Optional[torch.Tensor]]:
    """Q, K, V (and the mask, or None) of workload ``w`` as CPU tensors."""
    rng = np.random.default_rng(w.seed)
    q = normal(rng, (w.B, w.Hq, w.Sq, w.D), w.dtype)
    k = normal(rng, (w.B, w.Hkv, w.Skv, w.D), w.dtype)
    v = normal(rng, (w.B, w.Hkv, w.Skv, w.dv), w.dtype)
    mask = None
    if w.mask == "keypad_bool":
        mask = keypad_bool_mask(rng, w.B, w.Sq, w.Skv, w.Skv // 2, w.Skv, dead_rows=8)
    elif w.mask == "random_neginf_add":
        mask = random_neginf_add_mask(rng, (w.B, w.Hq, w.Sq, w.Skv), 0.10, w.dtype)
    elif w.mask != "none":
        raise ValueError(f"unknown mask recipe {w.mask!r}")
    return {"q": q, "k": k, "v": v, "mask": mask}


def make_case(seed: int, dtype: str, B: int, Hq: int, Hkv: int, Sq: int, Skv: int, D: int,
              mask: str = "none", mask_shape=None, causal: bool = False, Dv: Optional[int] = None,
              p: float = 0.1) -> Dict[str, Optional[torch.Tensor]]:
    """A free-form seeded case for ragged-shape and edge tests.

    ``mask`` is "none", "bool" (True with probability 1-p), "add" (N(0,1) bias
    with -inf at rate p) or "neginf" (0 with -inf at rate p); ``mask_shape``
    defaults to the full ``[B, Hq, Sq, Skv]`` and may use size-1 broadcast dims.
    """
    dv = D if Dv is None else Dv
    rng = np.random.default_rng(seed)
    q = normal(rng, (B, Hq, Sq, D), dtype)
    k = normal(rng, (B, Hkv, Skv, D), dtype)
    v = normal(rng, (B, Hkv, Skv, dv), dtype)
    shape = tuple(mask_shape) if mask_shape is not None else (B, Hq, Sq, Skv)
    m = None
    if mask == "bool":
        m = random_bool_mask(rng, shape, 1.0 - p)
    elif mask == "add":
        m = random_add_mask(rng, shape, dtype, p_neginf=p)
    elif mask == "neginf":
        m = random_neginf_add_mask(rng, shape, p, dtype)
    elif mask != "none":
        raise ValueError(f"unknown mask kind {mask!r}")
    return {"q": q, "k": k, "v": v, "mask": m, "causal": causal}
