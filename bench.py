"""Benchmark of the materialised-probability SDPA forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

One step = one ``sdpa_math_fwd`` call (validation, path choice, kernel launch)
on the 2k-token, head-dim-128, causal bf16 prefill workload (B=2, H=16,
Sq=Skv=2048) by default, inputs resident in HBM. Before each timed call the
caches are flushed (a 512 MiB write, outside the call's event interval: the
cudnn-frontend page's merge-log notes on measurement flush L2 per
iteration); the call's own events give its time. Prints one JSON line on
stdout; progress goes to stderr.

Accounting (the FlagOS-OP page's perf-gate convention, Validation table):
  flops = 2 * B * Hq * Sq * Skv * (D + Dv), halved when causal
  bytes = P + Q + K + V + O + LSE (+ mask), each once; P counts in full
          (its causal upper triangle is written as zeros).
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "ms, effective TFLOPS and P-write GB/s for SDPA fwd (out,P) prefill 2k D128 fp16"
HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "f16": 2500.0, "f32": 157.3}
ELT = {"f32": 4, "f16": 2, "bf16": 2}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic_flops(B, Hq, Sq, Skv, D, Dv, causal):
    f = 2.0 * B * Hq * Sq * Skv * (D + Dv)
    return f / 2 if causal else f


def algorithmic_bytes(w, mask_bytes=0):
    e = ELT[w.dtype]
    q = w.B * w.Hq * w.Sq * w.D * e
    k = w.B * w.Hkv * w.Skv * w.D * e
    v = w.B * w.Hkv * w.Skv * w.dv * e
    o = w.B * w.Hq * w.Sq * w.dv * e
    p = w.B * w.Hq * w.Sq * w.Skv * e
    lse = w.B * w.Hq * w.Sq * 4
    return {"total": q + k + v + o + p + lse + mask_bytes, "p": p}


FLUSH_BYTES = 512 << 20   # written before each timed call: more than L2 (8 x 4 MB) and the 256 MB MALL
_flush_buf = None


def flush_caches():
    """Stream-write a 512 MiB buffer (the library's fill kernel) so that the
    next call finds neither its inputs nor its outputs in L2 or the MALL."""
    import torch

    import sdpa_forward_materialised_amd as S

    global _flush_buf
    if _flush_buf is None:
        _flush_buf = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device="cuda:0")
    S.probe_fill(_flush_buf, 0)


def time_gpu(w, steps, warmup, path="auto", warm_ms=50.0, flush=True):
    """Time ``steps`` calls of workload ``w`` with inputs and preallocated
    outputs resident in HBM.

    Per call: a cache flush (outside the timed interval), then an event pair
    on the launch stream around the call alone; reported are the mean and
    median of those per-call times (device time of the call plus its launch
    gap). Before that, ``warmup`` calls and at least ``warm_ms`` of sustained
    work (the clock ramps up over tens of ms). Beside it, the same calls back
    to back without flushes, as one event interval / steps (labelled
    secondary: later calls may find data in the caches)."""
    import statistics

    import torch

    import sdpa_forward_materialised_amd as S
    import sdpa_workloads as W

    dev = torch.device("cuda:0")
    inp = W.make_inputs(w)
    q, k, v = (inp[x].to(dev) for x in ("q", "k", "v"))
    m = None if inp["mask"] is None else inp["mask"].to(dev)
    mask_bytes = 0 if m is None else m.numel() * m.element_size()
    B, Hq, Sq, D = q.shape
    Skv, Dv = k.shape[2], v.shape[3]
    O = torch.empty(B, Hq, Sq, Dv, dtype=q.dtype, device=dev)
    P = torch.empty(B, Hq, Sq, Skv, dtype=q.dtype, device=dev)
    L = torch.empty(B, Hq, Sq, dtype=torch.float32, device=dev)
    out = (O, P, L)
    chosen, tiles, tiles64 = S.plan(q, k, v, m, w.causal, w.gqa, causal_alignment=w.align)
    # the kernel doing the call's bulk (a forced path goes through the planner's override)
    if path != "auto":
        os.environ["SDPA_MATH_PATH"] = path
    try:
        kernel = S.kernel_name(q, k, v, m, w.causal, w.gqa, causal_alignment=w.align)
    finally:
        if path != "auto":
            os.environ.pop("SDPA_MATH_PATH", None)

    def call():
        S.fwd(q, k, v, m, w.causal, w.scale, w.gqa, path=path, out=out, causal_alignment=w.align)

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    t_w = time.perf_counter()
    while (time.perf_counter() - t_w) * 1e3 < warm_ms:
        for _ in range(20):
            call()
        torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        if flush:
            flush_caches()
        starts[i].record(stream)
        call()
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_call = [a.elapsed_time(b) for a, b in zip(starts, ends)]
    # secondary: back to back, no flushes
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    return {"ms": statistics.fmean(per_call), "ms_median": statistics.median(per_call), "ms_min": min(per_call),
            "ms_back_to_back": e0.elapsed_time(e1) / steps, "wall_ms": wall * 1e3 / steps,
            "mask_bytes": mask_bytes, "flushed": flush,
            "path": path if path != "auto" else chosen, "kernel": kernel, "tiles_per_bh": tiles,
            "tiles64_per_bh": tiles64}


# Sources whose change invalidates a stored counter measurement of the kernel.
KERNEL_SOURCES = ["sdpa_device.h", "sdpa_internal.h", "twopass.h", "twopass_bf16.hip", "twopass_f16.hip",
                  "twopass_f32.hip", "fused.hip", "sdpa_math_api.cpp"]


def profile_file(kernel, workload):
    return os.path.join(ROOT, "profiles", f"{kernel}.{workload}.txt")


def kernel_source_hash():
    import hashlib

    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "sdpa_forward_materialised_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def stored_traffic(kernel, workload):
    """HBM bytes per launch of ``kernel`` on ``workload`` from the committed
    rocprofv3 summary (FETCH_SIZE + WRITE_SIZE, each scaled by the copy-kernel
    calibration), or None when it is missing or was taken on other kernel
    sources."""
    try:
        with open(profile_file(kernel, workload)) as fh:
            kv = dict(ln.split(":", 1) for ln in fh if ":" in ln and not ln.startswith("#"))
    except OSError:
        return None
    kv = {k.strip(): v.strip() for k, v in kv.items()}
    if kv.get("kernel_source_sha256") != kernel_source_hash():
        return None
    val = kv.get(f"traffic_bytes_{kernel}")
    return int(val.split()[0]) if val else None


def probe_copy(mib, steps, warmup):
    """Time the library's streaming copy kernel over `mib` MiB (counter calibration)."""
    import torch

    import sdpa_forward_materialised_amd as S

    n = mib << 20
    src = torch.ones(n // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(warmup):
        S.probe_copy(dst, src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        S.probe_copy(dst, src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    assert torch.equal(dst, src)
    return {"probe": "copy", "bytes_read": n, "bytes_written": n, "ms": round(ms, 5),
            "gbps": round(2 * n / (ms * 1e-3) / 1e9, 1), "steps": steps}


def threshold_sweep(reps=15, warmup=3):
    """Both paths on a grid of shapes (fp16, B=4, H=16; D 64/128; causal or
    not; Sq 32..1024; Skv 128..2048): one JSON line per shape with the event
    time per call of each path (None where the fused path cannot take the
    shape). Run under ``rocprofv3 --kernel-trace`` for kernel-only times: the
    dispatches come in order, ``warmup + reps`` per shape and path."""
    import torch

    import sdpa_forward_materialised_amd as S

    dev = "cuda:0"
    g = torch.Generator(device="cpu").manual_seed(0)
    BH = (4, 16)
    for D in (64, 128):
        for causal in (False, True):
            for Sq in (32, 64, 128, 256, 512, 1024):
                for Skv in (128, 256, 512, 1024, 2048):
                    if causal and Skv < Sq:
                        continue
                    q = torch.randn(*BH, Sq, D, generator=g).to(dev, torch.float16)
                    k = torch.randn(*BH, Skv, D, generator=g).to(dev, torch.float16)
                    v = torch.randn(*BH, Skv, D, generator=g).to(dev, torch.float16)
                    out = (torch.empty_like(q), torch.empty(*BH, Sq, Skv, device=dev, dtype=torch.float16),
                           torch.empty(*BH, Sq, device=dev))
                    auto, _, t64 = S.plan(q, k, v, None, causal)
                    res = {"D": D, "causal": causal, "Sq": Sq, "Skv": Skv, "tiles64": t64, "auto": auto}
                    for path in ("twopass", "fused"):
                        def call():
                            S.fwd(q, k, v, None, causal, None, False, path=path, out=out)
                        try:
                            for _ in range(warmup):
                                call()
                        except NotImplementedError:
                            res[path + "_us"] = None
                            continue
                        torch.cuda.synchronize()
                        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                        e0.record()
                        for _ in range(reps):
                            call()
                        e1.record()
                        torch.cuda.synchronize()
                        res[path + "_us"] = round(e0.elapsed_time(e1) / reps * 1e3, 2)
                    print(json.dumps(res), flush=True)


def mask_sweep(reps=30, warmup=5):
    """Short-query shapes (fp16, B=16, H=8, non-causal; no mask, or a full
    [B,H,Sq,Skv] additive or bool mask removing 10 % of keys at random; Sq
    32..256, Skv 256..2048, D 64/128): flushed per-call median of the fused
    path's wide variant, its one-row-group kernel (SDPA_MATH_FUSED_WIDE=0)
    and the two-pass path; one text line per shape, with the path the
    planner picks ("-" where a variant cannot take the shape)."""
    import statistics

    import torch

    import sdpa_forward_materialised_amd as S

    dev = "cuda:0"
    g = torch.Generator(device="cpu").manual_seed(0)
    variants = (("fused", None), ("fused", "0"), ("twopass", None))
    print("B H Sq Skv D mask | fused-wide fused-1group twopass (us) | auto-plan", flush=True)
    for Sq in (32, 64, 100, 128, 256):
        for Skv in (256, 512, 1152, 2048):
            for D in (64, 128):
                for mk in ("none", "add", "bool"):
                    B, H = 16, 8
                    q = torch.randn(B, H, Sq, D, generator=g).half().to(dev)
                    k = torch.randn(B, H, Skv, D, generator=g).half().to(dev)
                    v = torch.randn(B, H, Skv, D, generator=g).half().to(dev)
                    drop = torch.rand(B, H, Sq, Skv, generator=g) < 0.1
                    m = None if mk == "none" else \
                        (torch.where(drop, float("-inf"), 0.0).half() if mk == "add" else ~drop).to(dev)
                    out = (torch.empty(B, H, Sq, D, dtype=q.dtype, device=dev),
                           torch.empty(B, H, Sq, Skv, dtype=q.dtype, device=dev),
                           torch.empty(B, H, Sq, dtype=torch.float32, device=dev))
                    res = []
                    for path, wide in variants:
                        os.environ.pop("SDPA_MATH_FUSED_WIDE", None)
                        if wide is not None:
                            os.environ["SDPA_MATH_FUSED_WIDE"] = wide
                        elif path == "fused":
                            os.environ["SDPA_MATH_FUSED_WIDE"] = "1"
                        try:
                            for _ in range(warmup):
                                S.fwd(q, k, v, m, False, None, False, path=path, out=out)
                        except NotImplementedError:
                            res.append(None)
                            continue
                        torch.cuda.synchronize()
                        st = [torch.cuda.Event(enable_timing=True) for _ in range(reps)]
                        en = [torch.cuda.Event(enable_timing=True) for _ in range(reps)]
                        for i in range(reps):
                            flush_caches()
                            st[i].record()
                            S.fwd(q, k, v, m, False, None, False, path=path, out=out)
                            en[i].record()
                        torch.cuda.synchronize()
                        res.append(statistics.median(x.elapsed_time(y) * 1e3 for x, y in zip(st, en)))
                    os.environ.pop("SDPA_MATH_FUSED_WIDE", None)
                    print(f"{B} {H} {Sq} {Skv} {D} {mk} | " +
                          " ".join("      -" if x is None else f"{x:7.2f}" for x in res) +
                          f" | {S.plan(q, k, v, m)[0]}", flush=True)


def host_path(n=2000):
    """Host time per call on the tiny workload (1x2 heads, 64x64, D=32, fp32
    causal): through the Python binding's fwd, through a prepared call (one C
    call per launch), and the GPU time per call back to back. Calls are issued
    without synchronising; the host time is the issuing loop's wall time."""
    import torch

    import sdpa_forward_materialised_amd as S
    import sdpa_workloads as W

    w = W.BY_NAME["tiny_f32_causal"]
    inp = W.make_inputs(w)
    q, k, v = (inp[x].to("cuda:0") for x in ("q", "k", "v"))
    out = S.fwd(q, k, v, None, True)
    call = S.prepare_fwd(q, k, v, None, True, out=out)

    def host(fn):
        fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(n):
            fn()
        t1 = time.perf_counter()
        torch.cuda.synchronize()
        return (t1 - t0) / n * 1e6

    r = {"workload": w.name, "fwd_host_us": round(host(lambda: S.fwd(q, k, v, None, True, out=out)), 2),
         "prepared_host_us": round(host(call.run), 2)}
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(n):
        call.run()
    e1.record()
    torch.cuda.synchronize()
    r["gpu_us_per_call_back_to_back"] = round(e0.elapsed_time(e1) / n * 1e3, 2)
    return r


def kept_pairs(Sq, Skv, align):
    """(query, key) pairs a causal mask keeps: query i keeps keys j <= i + c
    (c = 0 top-left, Skv - Sq bottom-right)."""
    c = Skv - Sq if align == "bottom_right" else 0
    return sum(max(0, min(Skv, i + c + 1)) for i in range(Sq))


def workload_row(w, r):
    """One table row: median per-call time with flushed caches, effective
    TFLOPS, P-write GB/s and the fraction of the HBM and MFMA rooflines. FLOPs
    follow the perf-gate convention (causal halves the square); a causal shape
    with Sq != Skv counts the (query, key) pairs its mask keeps."""
    by = algorithmic_bytes(w, r["mask_bytes"])
    sec = r["ms_median"] * 1e-3
    if w.causal and w.Sq != w.Skv:
        fl = 2.0 * w.B * w.Hq * kept_pairs(w.Sq, w.Skv, w.align) * (w.D + w.dv)
    else:
        fl = algorithmic_flops(w.B, w.Hq, w.Sq, w.Skv, w.D, w.dv, w.causal)
    return {"workload": w.name, "dtype": w.dtype, "path": r["path"], "kernel": r["kernel"], "ms": round(r["ms_median"], 5),
            "ms_mean": round(r["ms"], 5), "ms_back_to_back": round(r["ms_back_to_back"], 5),
            "tflops": round(fl / sec / 1e12, 2), "p_write_gbps": round(by["p"] / sec / 1e9, 1),
            "hbm_gbps": round(by["total"] / sec / 1e9, 1),
            "hbm_frac": round(by["total"] / sec / 1e9 / HBM_PEAK_GBPS, 4),
            "mfma_frac": round(fl / sec / 1e12 / MFMA_PEAK_TFLOPS[w.dtype], 4),
            "bytes": by["total"], "flops": fl}


def all_configs(path, workloads=None, reps=100, warmup=10):
    """Every seeded workload, ``reps`` flushed calls each (median reported)."""
    import sdpa_workloads as W

    rows = []
    for w in (W.WORKLOADS if workloads is None else workloads):
        r = time_gpu(w, reps, warmup, path, warm_ms=50.0)
        rows.append(workload_row(w, r))
        log(f"[bench] {w.name}: {r['ms_median']:.4f} ms median (flushed), {rows[-1]['hbm_frac'] * 100:.1f}% "
            f"of HBM roofline; back to back {r['ms_back_to_back']:.4f} ms")
    return rows


def time_backward(w, reps=50, warmup=10):
    """The backward (sdpa_math_bwd) on workload ``w`` with dL/dO and dL/dP
    both given: flushed per-call event time (median), effective TFLOPS over
    its four algorithmic products (dV, dP, dQ, dK: twice the forward's
    flops) and HBM bytes (q, k, v, dout, dprobs, lse read; dq, dk, dv
    written)."""
    import statistics

    import torch

    import sdpa_forward_materialised_amd as S
    import sdpa_workloads as W

    dev = torch.device("cuda:0")
    inp = W.make_inputs(w)
    q, k, v = (inp[x].to(dev) for x in ("q", "k", "v"))
    m = None if inp["mask"] is None else inp["mask"].to(dev)
    O, P, L = S.fwd(q, k, v, m, w.causal, w.scale, w.gqa, causal_alignment=w.align)
    g = torch.Generator(device="cpu").manual_seed(w.seed)
    dout = torch.randn(O.shape, generator=g).to(dev, q.dtype)
    dprobs = torch.randn(P.shape, generator=g).to(dev, q.dtype)
    out = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))

    def call():
        S.bwd(q, k, v, L, dout, dprobs, m, w.causal, w.scale, w.gqa, w.align, out=out)

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    st = [torch.cuda.Event(enable_timing=True) for _ in range(reps)]
    en = [torch.cuda.Event(enable_timing=True) for _ in range(reps)]
    for i in range(reps):
        flush_caches()
        st[i].record()
        call()
        en[i].record()
    torch.cuda.synchronize()
    ms = statistics.median(a.elapsed_time(b) for a, b in zip(st, en))
    fl = 2 * algorithmic_flops(w.B, w.Hq, w.Sq, w.Skv, w.D, w.dv, w.causal)
    e = ELT[w.dtype]
    nbytes = (2 * (q.numel() + k.numel() + v.numel()) + dout.numel() + dprobs.numel()) * e + L.numel() * 4 \
        + (0 if m is None else m.numel() * m.element_size())
    return {"workload": w.name, "ms": round(ms, 5), "tflops": round(fl / (ms * 1e-3) / 1e12, 2),
            "hbm_gbps": round(nbytes / (ms * 1e-3) / 1e9, 1),
            "hbm_frac": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
            "mfma_frac": round(fl / (ms * 1e-3) / 1e12 / MFMA_PEAK_TFLOPS[w.dtype], 4), "bytes": nbytes}


def cpu_baseline(w, budget_s=12.0):
    """The float64 oracle on whole (batch, head) slices of the same workload,
    taken in order (and again from the start once all were done) until about
    ``budget_s`` seconds of host time are used."""
    import oracle
    import sdpa_workloads as W

    inp = W.make_inputs(w)
    g = w.Hq // w.Hkv
    done, t_used = 0, 0.0
    heads = [(b, h) for b in range(w.B) for h in range(w.Hq)]
    while t_used < budget_s:
        b, h = heads[done % len(heads)]
        hk = h // g
        qs, ks, vs = inp["q"][b:b + 1, h:h + 1], inp["k"][b:b + 1, hk:hk + 1], inp["v"][b:b + 1, hk:hk + 1]
        ms = None
        if inp["mask"] is not None:
            mm = inp["mask"]
            ms = (mm[b:b + 1] if mm.shape[0] > 1 else mm)
            ms = ms[:, h:h + 1] if ms.shape[1] > 1 else ms
        t0 = time.perf_counter()
        oracle.sdpa_reference(qs, ks, vs, ms, w.causal, w.scale, False)
        t_used += time.perf_counter() - t0
        done += 1
    flops = algorithmic_flops(1, done, w.Sq, w.Skv, w.D, w.dv, w.causal)
    return {"value": flops / t_used / 1e12, "unit": "TFLOPS", "cores": oracle.threads(), "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"{done} (batch, head) slices of {w.name} (it has {len(heads)}), float64, "
                      f"{t_used:.1f} s ({t_used / done * 1e3:.0f} ms per slice)"}


def cpu_model():
    """The host CPU's model name (from /proc/cpuinfo), or None."""
    try:
        with open("/proc/cpuinfo") as fh:
            for ln in fh:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10,
                    help="untimed calls before the timed ones (plus at least 50 ms of sustained calls: "
                         "the clock ramps up over tens of ms)")
    ap.add_argument("--workload", default="prefill_2k_d128_bf16_causal",
                    help="the workload of the headline line (default: the 2k D128 bf16 causal prefill)")
    ap.add_argument("--path", default="auto", choices=["auto", "fused", "twopass"])
    ap.add_argument("--no-flush", action="store_true", help="no cache flush before each timed call")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-fp16", action="store_true", help="skip the same-shape fp16 line")
    ap.add_argument("--no-configs", action="store_true", help="skip the table over every seeded workload")
    ap.add_argument("--mask-sweep", action="store_true",
                    help="fused vs two-pass (2 and 3 compute waves) on masked short-query shapes, then exit")
    ap.add_argument("--threshold-sweep", action="store_true",
                    help="only time both paths over a grid of shapes (fused/two-pass switch)")
    ap.add_argument("--backward", action="store_true",
                    help="only time the backward (sdpa_math_bwd) of --workload and print its JSON line")
    ap.add_argument("--probe-copy-mib", type=int, default=0,
                    help="only time the streaming copy kernel over this many MiB (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch  # noqa: F401

    import sdpa_workloads as W

    if args.mask_sweep:
        mask_sweep()
        return
    if args.threshold_sweep:
        threshold_sweep()
        return
    if args.probe_copy_mib:
        print(json.dumps(probe_copy(args.probe_copy_mib, args.steps, args.warmup)), flush=True)
        return

    w = W.BY_NAME[args.workload]
    if args.backward:
        print(json.dumps(time_backward(w, reps=args.steps, warmup=args.warmup)), flush=True)
        return
    log(f"[bench] {w.describe()} steps={args.steps} warmup={args.warmup} flush={not args.no_flush}")
    r = time_gpu(w, args.steps, args.warmup, args.path, flush=not args.no_flush)
    row = workload_row(w, r)
    sec = r["ms"] * 1e-3  # mean per-call time: the roofline's average launch duration
    tflops = row["flops"] / sec / 1e12
    achieved = row["bytes"] / sec / 1e9
    p_gbps = algorithmic_bytes(w, r["mask_bytes"])["p"] / sec / 1e9
    log(f"[bench] {w.dtype}: {r['ms']:.4f} ms mean, {r['ms_median']:.4f} median per call (flushed); "
        f"{tflops:.1f} TFLOPS, {achieved:.0f} GB/s, P {p_gbps:.0f} GB/s; back to back {r['ms_back_to_back']:.4f} ms")

    extra = {}
    if not args.no_fp16 and w.name == "prefill_2k_d128_bf16_causal":
        w16 = W.Workload("prefill_2k_d128_f16_causal", "f16", 2, 16, 16, 2048, 2048, 128, True, "none", 3)
        r16 = time_gpu(w16, args.steps, args.warmup, args.path, flush=not args.no_flush)
        extra["fp16_same_shape"] = {"ms": round(r16["ms"], 5), "ms_median": round(r16["ms_median"], 5),
                                    "tflops": round(row["flops"] / (r16["ms"] * 1e-3) / 1e12, 2),
                                    "p_write_gbps": round(algorithmic_bytes(w16)["p"] / (r16["ms"] * 1e-3) / 1e9, 1)}
        log(f"[bench] fp16: {r16['ms']:.4f} ms mean per call")

    if not args.no_configs:
        extra["configs"] = all_configs(args.path)
        extra["extra_configs"] = all_configs(args.path, W.EXTRA_WORKLOADS)

    if not args.no_configs:
        extra["host_path"] = host_path()
        log(f"[bench] host path: {extra['host_path']}")
        extra["backward"] = []
        for name in ("prefill_2k_d128_bf16_causal", "gqa_1k_d128_f16_keypad"):
            rb = time_backward(W.BY_NAME[name])
            extra["backward"].append(rb)
            log(f"[bench] backward {name}: {rb['ms']:.4f} ms, {rb['tflops']} TFLOPS, {rb['hbm_frac'] * 100:.1f}% HBM")

    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] timing the float64 oracle on the host")
        cpu = cpu_baseline(w)
        log(f"[bench] cpu baseline: {cpu}")

    kernel = r["kernel"]
    line = {
        "metric": METRIC, "value": round(tflops, 3), "unit": "TFLOPS", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(r["ms"], 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "Sq": w.Sq, "Skv": w.Skv,
                   "D": w.D, "causal": w.causal, "mask": w.mask, "path": r["path"],
                   "tiles_per_bh": r["tiles_per_bh"], "tiles64_per_bh": r["tiles64_per_bh"]},
        "timing": {"per_call": "hip events on the launch stream around each call, caches flushed before it "
                               "(512 MiB write, outside the interval)" if r["flushed"] else
                               "hip events on the launch stream around each call, no flush",
                   "ms_mean": round(r["ms"], 5), "ms_median": round(r["ms_median"], 5),
                   "ms_min": round(r["ms_min"], 5),
                   "ms_back_to_back_secondary": round(r["ms_back_to_back"], 5)},
        "p_write_gbps": round(p_gbps, 1),
        "effective_tflops_frac_of_mfma_peak": round(tflops / MFMA_PEAK_TFLOPS[w.dtype], 4),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": stored_traffic(kernel, w.name),
                     "kernel": kernel, "bytes_per_launch": row["bytes"]},
        "cpu_baseline": cpu,
        "wall_ms_per_step": round(r["wall_ms"], 5),
    }
    line.update(extra)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
