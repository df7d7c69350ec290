"""Benchmark: causal Taylor-series linear attention on one MI355X.

One "step" is one taylor_attn_prefill call over the Based-style order-2
workload (B=4, H=16, N=4096, d=16 -> 153 symmetric features, dv=64, bf16 in
and out, fp32 accumulation, a = sqrt(d)): feature maps, score tiles,
read-out, intra-chunk term, state update and normalisation all run inside
that call. Inputs rotate over several resident replicas whose total exceeds
the 256 MiB last-level cache, so every step reads them from HBM.

Printed: ONE JSON line with the prefill throughput (tokens/s) and its MFMA
fraction, the decode state bandwidth of the order-2 decode workload (64 x 16
heads, states seeded by a 32768-token prefill) as a fraction of HBM peak, the
roofline of the dominant kernel and the fp64 CPU oracle timed beside it.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu]
       [--no-decode] [--no-native] [--only prefill|decode|copy]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_DENSE_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
FP32_DENSE_TFLOPS = 157.3
PREFILL = "based_order2_prefill"
DECODE = "order2_decode"
CHUNK = 32                      # tokens per chunk of the order-2 d=16 bf16 kernel
TRAFFIC = os.path.join(ROOT, "profiles", "traffic_based_order2_prefill.json")


# sources the timed order-2 d=16 bf16 prefill kernel is compiled from
TIMED_SOURCES = ("prefill_o2.hip", "internal.hpp", "mma.hpp")


def source_hash():
    """Hash of the timed kernel's HIP sources, to tell whether stored counter
    data still describes the kernel being timed."""
    import hashlib
    csrc = os.path.join(ROOT, "taylor_series_linear_amd", "csrc")
    h = hashlib.sha256()
    for name in TIMED_SOURCES:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def _pmc_rows(d):
    import csv
    import glob
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {d}")
    rows = []
    for fn in files:
        with open(fn) as f:
            rows += list(csv.DictReader(f))
    return rows


def pmc_summary(fetch_dir, write_dir, copy_fetch_dir, copy_write_dir, out_path):
    """Turn four rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE of the prefill
    bench; the same two counters over bench.py --only copy) into per-call HBM
    bytes. The counters report KiB per dispatch; each is scaled by the ratio
    of the plain copy's known bytes to what the same counter reads for it."""
    copy_bytes = 256 * 1024 * 1024

    def per_kernel(rows, counter):
        acc = {}
        for r in rows:
            if r["Counter_Name"] != counter:
                continue
            acc.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]) * 1024.0)
        return {k: sum(v) / len(v) for k, v in acc.items()}

    f_copy = per_kernel(_pmc_rows(copy_fetch_dir), "FETCH_SIZE")
    w_copy = per_kernel(_pmc_rows(copy_write_dir), "WRITE_SIZE")
    ck = max(f_copy, key=lambda k: f_copy[k])      # the 256 MiB copy kernel
    f_scale = copy_bytes / f_copy[ck]
    w_scale = copy_bytes / w_copy[max(w_copy, key=lambda k: w_copy[k])]
    fetch = per_kernel(_pmc_rows(fetch_dir), "FETCH_SIZE")
    write = per_kernel(_pmc_rows(write_dir), "WRITE_SIZE")
    kernels = {}
    for k in sorted(set(fetch) | set(write)):
        if "o2_" not in k and "prefill" not in k:
            continue
        kernels[k] = {"fetch_bytes": fetch.get(k, 0.0) * f_scale, "write_bytes": write.get(k, 0.0) * w_scale}
    total = sum(v["fetch_bytes"] + v["write_bytes"] for v in kernels.values())
    rec = {"workload": PREFILL, "source_hash": source_hash(), "fetch_scale": f_scale, "write_scale": w_scale,
           "copy_kernel": ck, "kernels": kernels, "bytes_per_call": total}
    with open(out_path, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec))


def stored_traffic():
    """HBM bytes per prefill call from the stored counter summary, or None if
    the kernels changed since it was taken."""
    try:
        with open(TRAFFIC) as f:
            rec = json.load(f)
    except OSError:
        return None
    return rec["bytes_per_call"] if rec.get("source_hash") == source_hash() else None


def feature_dim(d, n_terms):
    """Width of the symmetric basis: sum over orders m < n of C(d+m-1, m)."""
    return sum(math.comb(d + m - 1, m) for m in range(n_terms))


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic_prefill(w, chunk=CHUNK):
    """Per-call algorithmic bytes and flops.

    bytes: q, k, v read once and o written once: (2d + dv) * in + dv * out.
    flops: 4 F (dv+1) for state read-out and update (with the denominator
    column) + (min(c,256)+1)(d+dv+1) for the causal half of the diagonal block.
    """
    F = feature_dim(w.d, w.n_terms)
    esz = 2 if w.dtype == "bf16" else 4
    th = w.B * w.H * w.N
    bytes_ = th * ((2 * w.d + w.dv) * esz + w.dv * esz)
    flops = th * (4 * F * (w.dv + 1) + (min(chunk, 256) + 1) * (w.d + w.dv + 1))
    return bytes_, flops, F


def dev_tensor(arr, dtype, torch):
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).cuda()


def time_loop(fn, steps, torch):
    """Average ms per call over `steps` calls, with HIP events on the current stream."""
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(steps):
        fn(i)
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps


def bench_prefill(args, torch, tl, W):
    w = W.WORKLOADS[PREFILL]
    x = W.make_workload(w)
    reps = args.replicas
    qs = [dev_tensor(x["q"], w.dtype, torch) for _ in range(reps)]
    ks = [dev_tensor(x["k"], w.dtype, torch) for _ in range(reps)]
    vs = [dev_tensor(x["v"], w.dtype, torch) for _ in range(reps)]
    os_ = [torch.empty((w.B, w.H, w.N, w.dv), dtype=torch.bfloat16, device="cuda") for _ in range(reps)]
    ws_bytes = tl.prefill_workspace_bytes(w.B, w.H, w.N, w.d, w.dv, w.n_terms, torch.bfloat16)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")
    L = tl.lib()

    # every call's arguments are built before the timed loop, so the loop only
    # enqueues launches
    stream = tl._stream().value
    calls = [(qs[r].data_ptr(), ks[r].data_ptr(), vs[r].data_ptr(), tl.TAYLOR_BF16, w.B, w.H, w.N, w.d, w.dv,
              w.n_terms, w.a, None, None, os_[r].data_ptr(), tl.TAYLOR_BF16, None, None, ws.data_ptr(),
              ws_bytes, stream) for r in range(reps)]

    def step(i):
        st = L.taylor_attn_prefill(*calls[i % reps])
        if st != 0:
            tl.check(st)

    for i in range(args.warmup):
        step(i)
    ms = time_loop(step, args.steps, torch)
    bytes_, flops, F = algorithmic_prefill(w)
    return w, ms, bytes_, flops, F, reps, x


def bench_decode(args, torch, tl, W):
    w = W.WORKLOADS[DECODE]
    log("decode: generating the 32768-token seeding prefill and", w.steps, "steps")
    x = W.make_decode_inputs(w)
    pk = dev_tensor(x["prefill_k"], "f32", torch)
    pv = dev_tensor(x["prefill_v"], "f32", torch)
    _, S, z = tl.prefill(pk, pk, pv, w.n_terms, w.a, want_output=False, return_state=True)
    torch.cuda.synchronize()
    del pk, pv
    R = args.decode_replicas
    Ss = [S.clone() for _ in range(R)]
    zs = [z.clone() for _ in range(R)]
    sq = dev_tensor(np.moveaxis(x["step_q"], 2, 0), "f32", torch)
    sk = dev_tensor(np.moveaxis(x["step_k"], 2, 0), "f32", torch)
    sv = dev_tensor(np.moveaxis(x["step_v"], 2, 0), "f32", torch)
    o = torch.empty((w.B, w.H, w.dv), dtype=torch.float32, device="cuda")
    L = tl.lib()

    # every step's arguments are built before the timed loop, so the loop only
    # enqueues launches (step s takes token s of the 1024 and replica s % R_)
    stream = tl._stream().value

    def make_step(R_):
        calls = [(sq[s].data_ptr(), sk[s].data_ptr(), sv[s].data_ptr(), tl.TAYLOR_F32, w.B, w.H, w.d, w.dv,
                  w.n_terms, w.a, Ss[s % R_].data_ptr(), zs[s % R_].data_ptr(), o.data_ptr(), tl.TAYLOR_F32,
                  stream) for s in range(w.steps)]

        def step(i):
            st = L.taylor_attn_decode(*calls[i % w.steps])
            if st != 0:
                tl.check(st)
        return step

    cold = make_step(R)
    for i in range(min(args.warmup * 4, 64)):
        cold(i)
    ms_cold = time_loop(cold, w.steps, torch)
    hot = make_step(1)
    for i in range(16):
        hot(i)
    ms_hot = time_loop(hot, w.steps, torch)
    F = feature_dim(w.d, w.n_terms)
    state_bytes = 2 * F * (w.dv + 1) * 4 * w.B * w.H   # read + write of S and z
    flops = 4 * F * (w.dv + 1) * w.B * w.H / 2            # 2F(dv+1) per head-step
    return {
        "workload": DECODE, "heads": w.B * w.H, "features": F, "steps_timed": w.steps,
        "state_bytes_per_step": state_bytes,
        "us_per_step_cold": ms_cold * 1e3, "us_per_step_hot": ms_hot * 1e3,
        "state_GBps_cold": state_bytes / (ms_cold * 1e-3) / 1e9,
        "state_GBps_hot": state_bytes / (ms_hot * 1e-3) / 1e9,
        "hbm_frac_cold": state_bytes / (ms_cold * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "state_replicas_cold": R, "algorithmic_gflop_per_step": flops / 1e9,
        "kernel": "decode_kernel<16,64,3,fp32>",
    }


def native_c_abi():
    """Decode and prefill timed through the C ABI by a plain C++ host program
    (taylor_series_linear_amd/bench_native, built with the library), run as a
    child process with no Python or torch in it: a cross-check of the figures
    above with the library used the way a C or C++ caller would use it."""
    import subprocess
    exe = os.path.join(ROOT, "taylor_series_linear_amd", "bench_native")
    if not os.path.exists(exe):
        return {"skipped": "bench_native is not built"}
    log("native: timing decode and prefill through the C ABI in a child process")
    # a failure here is reported in this block and never stops the bench line
    try:
        r = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    except subprocess.TimeoutExpired:
        return {"error": "bench_native did not finish within 300 s"}
    if r.returncode != 0:
        return {"error": f"bench_native exited with {r.returncode}: {r.stderr.strip()[-500:]}"}
    try:
        res = json.loads(r.stdout.strip().splitlines()[-1])
    except (ValueError, IndexError):
        return {"error": "bench_native printed no JSON line"}
    res["note"] = ("same kernels and workloads, timed by HIP events in a C++ process; decode states seeded by a "
                   "256-token prefill (the state size does not depend on the context length)")
    return res


def _fit_exponent(ns, ts):
    """Least-squares slope of log t against log N."""
    x = np.log(np.asarray(ns, dtype=np.float64))
    y = np.log(np.asarray(ts, dtype=np.float64))
    return float(np.polyfit(x, y, 1)[0])


def _unit_rows(shape, gen, torch):
    x = torch.randn(shape, generator=gen, device="cuda", dtype=torch.float32)
    return x / x.norm(dim=-1, keepdim=True)


def sweep(args, torch, tl):
    """Growth of prefill time with N and of decode step time with the context
    length, at the defaults of "Expanding Attention" (d=16, dv=64, a=2,
    order 2, unit-sphere queries and keys). Prints one JSON line per point and
    one per fit; inputs are drawn on the device from a seeded generator."""
    d, dv, n_terms, a = 16, 64, 3, 2.0
    gen = torch.Generator(device="cuda")
    L = tl.lib()
    # prefill: 64 heads, N = 1024 .. 65536, fp32 and bf16 inputs
    H = 64
    ns = [1024 * 2 ** i for i in range(7)]
    for dt in ("f32", "bf16"):
        tdt = torch.float32 if dt == "f32" else torch.bfloat16
        code = tl.TAYLOR_F32 if dt == "f32" else tl.TAYLOR_BF16
        times = []
        for N in ns:
            gen.manual_seed(2000 + N)
            q = _unit_rows((1, H, N, d), gen, torch).to(tdt)
            k = _unit_rows((1, H, N, d), gen, torch).to(tdt)
            v = torch.randn((1, H, N, dv), generator=gen, device="cuda").to(tdt)
            o = torch.empty((1, H, N, dv), dtype=tdt, device="cuda")
            wsb = tl.prefill_workspace_bytes(1, H, N, d, dv, n_terms, tdt)
            ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device="cuda")

            def step(i):
                st = L.taylor_attn_prefill(tl._ptr(q), tl._ptr(k), tl._ptr(v), code, 1, H, N, d, dv, n_terms, a,
                                           None, None, tl._ptr(o), code, None, None, tl._ptr(ws), wsb,
                                           tl._stream())
                if st != 0:
                    tl.check(st)

            for i in range(3):
                step(i)
            ms = time_loop(step, 10, torch)
            times.append(ms)
            print(json.dumps({"sweep": "prefill", "dtype": dt, "heads": H, "N": N, "ms": ms,
                              "token_heads_per_s": H * N / (ms * 1e-3)}), flush=True)
            del q, k, v, o, ws
        big = [i for i, N in enumerate(ns) if N >= 8192]
        print(json.dumps({"sweep": "prefill_fit", "dtype": dt, "exponent_all": _fit_exponent(ns, times),
                          "exponent_N_ge_8192": _fit_exponent([ns[i] for i in big], [times[i] for i in big]),
                          "N": [ns[0], ns[-1]]}), flush=True)
    # decode: 1024 heads (64 sequences x 16), fp32, after contexts of 1024 .. 65536 tokens
    B, Hd, R, steps = 64, 16, 8, 256
    ctx = [1024, 4096, 16384, 65536]
    times = []
    for N in ctx:
        gen.manual_seed(3000 + N)
        k = _unit_rows((B, Hd, N, d), gen, torch)
        v = torch.randn((B, Hd, N, dv), generator=gen, device="cuda")
        _, S, z = tl.prefill(k, k, v, n_terms, a, want_output=False, return_state=True)
        del k, v
        Ss = [S.clone() for _ in range(R)]
        zs = [z.clone() for _ in range(R)]
        sq = _unit_rows((steps, B, Hd, d), gen, torch)
        sk = _unit_rows((steps, B, Hd, d), gen, torch)
        sv = torch.randn((steps, B, Hd, dv), generator=gen, device="cuda")
        o = torch.empty((B, Hd, dv), dtype=torch.float32, device="cuda")

        stream = tl._stream().value
        calls = [(sq[s].data_ptr(), sk[s].data_ptr(), sv[s].data_ptr(), tl.TAYLOR_F32, B, Hd, d, dv, n_terms, a,
                  Ss[s % R].data_ptr(), zs[s % R].data_ptr(), o.data_ptr(), tl.TAYLOR_F32, stream)
                 for s in range(steps)]

        def dstep(i):
            st = L.taylor_attn_decode(*calls[i % steps])
            if st != 0:
                tl.check(st)

        for i in range(32):
            dstep(i)
        ms = time_loop(dstep, steps, torch)
        times.append(ms)
        print(json.dumps({"sweep": "decode", "dtype": "f32", "heads": B * Hd, "context": N,
                          "us_per_step": ms * 1e3, "state_replicas": R}), flush=True)
        del Ss, zs, S, z, sq, sk, sv
    print(json.dumps({"sweep": "decode_fit", "exponent": _fit_exponent(ctx, times), "context": [ctx[0], ctx[-1]]}),
          flush=True)


def time_workloads(names, torch, tl, W, reps=20):
    """One prefill call per named workload (its own inputs, output in the input
    dtype), 3 warm-up and `reps` timed calls; one JSON line per workload."""
    for name in names:
        w = W.WORKLOADS[name]
        x = W.make_workload(w)
        q, k, v = (dev_tensor(x[s], w.dtype, torch) for s in "qkv")
        od = torch.bfloat16 if w.dtype == "bf16" else torch.float32
        wsb = tl.prefill_workspace_bytes(w.B, w.H, w.N, w.d, w.dv, w.n_terms, q.dtype)
        ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device="cuda")
        o = torch.empty((w.B, w.H, w.N, w.dv), dtype=od, device="cuda")
        L = tl.lib()
        code = tl.TAYLOR_BF16 if w.dtype == "bf16" else tl.TAYLOR_F32

        def step(i):
            st = L.taylor_attn_prefill(tl._ptr(q), tl._ptr(k), tl._ptr(v), code, w.B, w.H, w.N, w.d, w.dv,
                                       w.n_terms, w.a, None, None, tl._ptr(o), code, None, None, tl._ptr(ws), wsb,
                                       tl._stream())
            if st != 0:
                tl.check(st)

        for i in range(3):
            step(i)
        ms = time_loop(step, reps, torch)
        _, flops, F = algorithmic_prefill(w)  # both large-feature kernels use 32-token chunks
        print(json.dumps({"workload": name, "ms": round(ms, 4), "tokens_per_s": w.B * w.N / (ms * 1e-3),
                          "algorithmic_tflops": flops / (ms * 1e-3) / 1e12, "features": F,
                          "workspace_MB": wsb / 1e6}), flush=True)
        del q, k, v, o, ws


def cpu_baseline(w, x, budget_s):
    """fp64 oracle direct() on the first heads of the same inputs until ~budget_s."""
    from oracle import taylor_oracle as T
    try:
        import threadpoolctl
        threads = max(i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()) or 1
    except Exception:  # noqa: BLE001
        threads = os.cpu_count() or 1
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    done = 0
    t0 = time.perf_counter()
    for (b, h) in heads:
        T.direct(x["q64"][b, h], x["k64"][b, h], x["v64"][b, h], w.n_terms, w.a)
        done += 1
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    token_heads = done * w.N
    return {"value": token_heads / dt / w.H, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"first {done} of {len(heads)} heads, all {w.N} rows each, fp64 numpy direct(); "
                      f"tokens/s = token-heads/s / H; {dt:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--replicas", type=int, default=4)
    ap.add_argument("--decode-replicas", type=int, default=8)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-native", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--only", choices=["prefill", "decode", "copy"], default=None)
    ap.add_argument("--time", nargs="+", metavar="WORKLOAD",
                    help="time one prefill call of each named workload, then exit")
    ap.add_argument("--sweep", action="store_true",
                    help="growth of prefill time with N and of decode time with the context, then exit")
    ap.add_argument("--pmc-summary", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR", "COPY_WRITE_DIR"),
                    help="summarise rocprofv3 --pmc runs into the stored traffic record and exit")
    args = ap.parse_args()
    if args.pmc_summary:
        pmc_summary(*args.pmc_summary, TRAFFIC)
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(heads shard across GPUs with no communication). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import taylor_series_linear_amd as tl
    import workloads as W

    torch.cuda.set_device(0)
    if args.sweep:
        sweep(args, torch, tl)
        return
    if args.time:
        time_workloads(args.time, torch, tl, W)
        return
    if args.only == "copy":
        # plain copy of known size, for counter calibration (FETCH_SIZE / WRITE_SIZE)
        n = 256 * 1024 * 1024 // 4
        a = torch.ones(n, device="cuda")
        b = torch.empty_like(a)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_each_way": n * 4, "launches": 5}))
        return
    if args.only == "decode":
        print(json.dumps(bench_decode(args, torch, tl, W)))
        return

    w, ms, bytes_, flops, F, reps, x = bench_prefill(args, torch, tl, W)
    tokens = w.B * w.N
    gbs = bytes_ / (ms * 1e-3) / 1e9
    tflops = flops / (ms * 1e-3) / 1e12
    out = {
        "metric": "prefill tokens/s + MFMA % peak; decode state GB/s % HBM peak (1 GPU)",
        "value": tokens / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": PREFILL, "B": w.B, "H": w.H, "N": w.N, "d": w.d, "dv": w.dv,
                   "n_terms": w.n_terms, "a": w.a, "features": F, "in": "bf16", "out": "bf16",
                   "accumulate": "fp32", "input_replicas": reps, "seed": w.seed},
        "token_heads_per_s": w.B * w.H * w.N / (ms * 1e-3),
        "mfma": {"achieved_tflops": tflops, "peak_tflops": BF16_DENSE_TFLOPS,
                 "frac": tflops / BF16_DENSE_TFLOPS, "flops_per_step": flops,
                 "note": "algorithmic flops 4F(dv+1)+(c+1)(d+dv+1) per token-head, c=32"},
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs / HBM_PEAK_GBS, "traffic": stored_traffic(),
                     "kernel": "one taylor_attn_prefill call: flag reset + single-pass o2 kernel (2 launches)",
                     "launch_us": ms * 1e3, "algorithmic_bytes_per_launch": bytes_},
    }
    if args.only != "prefill" and not args.no_decode:
        out["decode"] = bench_decode(args, torch, tl, W)
    if not args.no_native and args.only is None:
        out["native_c_abi"] = native_c_abi()
    if not args.no_cpu and args.only is None:
        out["cpu_baseline"] = cpu_baseline(w, x, args.cpu_budget)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
