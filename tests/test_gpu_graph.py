"""The forward recorded into a HIP graph (torch.cuda.CUDAGraph) and replayed:
each replay, after new inputs are copied into the captured buffers and with
eager calls and synchronisations in between, equals bit for bit an eager call
on the same inputs. Covers the two-pass kernel, the wide fused kernel, the
one-sweep key ranges with their combine launch (workspace allocated during
capture from the graph's pool), a prepared call and the allocation-free entry
point."""

import pytest
import torch

import sdpa_workloads as W

pytestmark = pytest.mark.gpu

DEV = "cuda:0"

CASES = [
    ("twopass-causal", dict(seed=401, dtype="bf16", B=1, Hq=4, Hkv=4, Sq=384, Skv=384, D=128, causal=True)),
    ("wide-decode-add", dict(seed=402, dtype="f16", B=2, Hq=4, Hkv=4, Sq=100, Skv=1152, D=64, mask="add", p=0.1)),
    ("ranges-gqa", dict(seed=403, dtype="bf16", B=2, Hq=8, Hkv=2, Sq=1, Skv=4096, D=128)),
]


def _inputs(spec, seed):
    c = W.make_case(**{**spec, "seed": seed})
    return tuple(None if c[x] is None else c[x].to(DEV) for x in ("q", "k", "v", "mask")), c["causal"]


def _eager(S, q, k, v, m, causal, gqa):
    out = S.fwd(q, k, v, m, causal, None, gqa)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("mode", ["fwd", "prepared", "noalloc"])
@pytest.mark.parametrize("label,spec", CASES, ids=[c[0] for c in CASES])
def test_graph_replays_match_eager(label, spec, mode):
    import sdpa_forward_materialised_amd as S
    (q, k, v, m), causal = _inputs(spec, spec["seed"])
    gqa = q.shape[1] != k.shape[1]
    B, Hq, Sq, D = q.shape
    Skv = k.shape[2]
    out = (torch.empty(B, Hq, Sq, D, dtype=q.dtype, device=DEV),
           torch.empty(B, Hq, Sq, Skv, dtype=q.dtype, device=DEV),
           torch.empty(B, Hq, Sq, dtype=torch.float32, device=DEV))
    print(f"[case] graph {label} {mode}", flush=True)
    if mode == "prepared":
        call = S.prepare_fwd(q, k, v, m, causal, None, gqa, out=out).run
    elif mode == "noalloc":
        def call():
            S.fwd_noalloc(q, k, v, out, m, causal, None, gqa)
    else:
        def call():
            S.fwd(q, k, v, m, causal, None, gqa, out=out)
    call()  # outside capture first: kernel attributes, workspace sizes
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    for it in range(3):
        (q2, k2, v2, m2), _ = _inputs(spec, spec["seed"] + 100 + it)
        q.copy_(q2)
        k.copy_(k2)
        v.copy_(v2)
        if m is not None:
            m.copy_(m2)
        torch.cuda.synchronize()
        for t in out:
            t.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        ref = _eager(S, q, k, v, m, causal, gqa)
        for name, a, b in zip(("O", "P", "LSE"), out, ref):
            assert torch.equal(a, b), f"{label} {mode} replay {it}: {name} differs from the eager call"
