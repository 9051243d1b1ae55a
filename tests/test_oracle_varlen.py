"""Pins for the oracle's packed variable-length helper (no GPU): one sequence
spanning every token equals the dense call, equal-length sequences equal the
dense batched call, and a mixed-length pack equals the brute force applied
sequence by sequence (with the probability rows zero past each sequence)."""

import numpy as np
import torch

import oracle
from oracle.brute import sdpa_brute
import sdpa_workloads as W


def _thd(x):  # [1, H, S, D] -> [S, H, D]
    return x[0].permute(1, 0, 2).contiguous()


def test_single_sequence_equals_dense():
    c = W.make_case(1, "f32", 1, 4, 2, 9, 13, 8, causal=True)
    o, p, l = oracle.sdpa_reference(c["q"], c["k"], c["v"], None, True, None, True, causal_alignment="bottom_right")
    vo, vp, vl = oracle.sdpa_varlen_reference(_thd(c["q"]), _thd(c["k"]), _thd(c["v"]), [0, 9], [0, 13], 16, True,
                                              None, True, "bottom_right")
    assert np.array_equal(vo, o[0].transpose(1, 0, 2)) and np.array_equal(vl, l[0].T)
    assert np.array_equal(vp[:, :, :13], p[0].transpose(1, 0, 2)) and np.all(vp[:, :, 13:] == 0)


def test_equal_lengths_equal_dense_batch():
    c = W.make_case(2, "f32", 3, 2, 2, 6, 6, 8)
    o, p, l = oracle.sdpa_reference(c["q"], c["k"], c["v"], None, True)
    def pack(x):
        return x.permute(0, 2, 1, 3).reshape(-1, x.shape[1], x.shape[3])

    vo, vp, vl = oracle.sdpa_varlen_reference(pack(c["q"]), pack(c["k"]), pack(c["v"]), [0, 6, 12, 18],
                                              [0, 6, 12, 18], 6, True)
    assert np.array_equal(vo, o.transpose(0, 2, 1, 3).reshape(18, 2, 8))
    assert np.array_equal(vp, p.transpose(0, 2, 1, 3).reshape(18, 2, 6))
    assert np.array_equal(vl, l.transpose(0, 2, 1).reshape(18, 2))


def test_mixed_lengths_match_brute_force_per_sequence():
    lq, lk = [3, 0, 5, 2], [4, 6, 0, 7]
    cq, ck = np.cumsum([0] + lq), np.cumsum([0] + lk)
    g = np.random.default_rng(3)
    q = torch.from_numpy(g.standard_normal((cq[-1], 4, 8)))
    k = torch.from_numpy(g.standard_normal((ck[-1], 2, 8)))
    v = torch.from_numpy(g.standard_normal((ck[-1], 2, 8)))
    vo, vp, vl = oracle.sdpa_varlen_reference(q, k, v, cq, ck, 8, True, None, True)
    for b in range(4):
        if lq[b] == 0:
            continue
        qs = q[cq[b]:cq[b + 1]].permute(1, 0, 2)[None]
        ks = k[ck[b]:ck[b + 1]].permute(1, 0, 2)[None]
        vs = v[ck[b]:ck[b + 1]].permute(1, 0, 2)[None]
        o, p, l = sdpa_brute(qs, ks, vs, None, True, None, True)
        sl = slice(cq[b], cq[b + 1])
        assert np.allclose(vo[sl], o[0].transpose(1, 0, 2), atol=1e-12)
        assert np.allclose(vp[sl, :, :lk[b]], p[0].transpose(1, 0, 2), atol=1e-12)
        assert np.all(vp[sl, :, lk[b]:] == 0)
        same = np.isneginf(vl[sl]) == np.isneginf(l[0].T)
        assert same.all() and np.allclose(vl[sl][np.isfinite(vl[sl])], l[0].T[np.isfinite(l[0].T)], atol=1e-12)
