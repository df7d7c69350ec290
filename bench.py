"""Benchmark: causal Taylor-series linear attention on one MI355X.

One "step" is one taylor_attn_prefill call over the long-context order-2
workload (B=1, H=8, N=65536, d=64 -> 2145 symmetric features, dv=64, bf16 in
and out, fp32 accumulation, a = sqrt(d) = 8): feature maps, score tiles,
read-out, intra-chunk term, state update, segment prefix and normalisation
all run inside that call. It is the largest single-GPU configuration and the
one whose cost is matrix-core bound ("Expanding Attention", "Time"), so the
headline roofline is the bf16 MFMA peak. Inputs rotate over resident
replicas whose total exceeds the 256 MiB last-level cache, so every step
reads them from HBM.

Printed: ONE JSON line with the headline prefill (tokens/s, roofline against
the bf16 MFMA peak, HBM traffic from counters), extra blocks for the
Based-style order-2 prefill (HBM-bound), the order-4 prefill and the order-2
decode (state bandwidth against HBM peak), and the fp64 CPU oracle timed
beside it on all host cores and on one thread.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu]
       [--no-decode] [--no-extra] [--no-native] [--only prefill|decode|copy]
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
HEADLINE = "long_order2_prefill"
DECODE = "order2_decode"
CHUNK = 32                      # tokens per chunk of every timed bf16 prefill kernel

# Timed prefill workloads: the HIP sources their kernels are compiled from
# (a stored counter record is used only while these are unchanged), the
# roofline that binds them, and the input replicas that keep them out of the
# last-level cache.
PREFILLS = {
    "long_order2_prefill": dict(sources=("prefill_w2.hip", "internal.hpp", "mma.hpp", "sched.hpp"),
                                bound="mfma", replicas=2),
    "based_order2_prefill": dict(sources=("prefill_o2.hip", "internal.hpp", "mma.hpp", "sched.hpp"),
                                 bound="hbm", replicas=4),
    "order4_prefill": dict(sources=("prefill.hip", "features.hpp", "qarrange.hpp", "rank.hpp", "internal.hpp",
                                    "mma.hpp", "sched.hpp"),
                           bound="mfma", replicas=8),
}


def traffic_path(name):
    return os.path.join(ROOT, "profiles", f"traffic_{name}.json")


def source_hash(name=HEADLINE):
    """Hash of a timed kernel's HIP sources, to tell whether stored counter
    data still describes the kernel being timed."""
    import hashlib
    csrc = os.path.join(ROOT, "taylor_series_linear_amd", "csrc")
    h = hashlib.sha256()
    for fn in PREFILLS[name]["sources"]:
        with open(os.path.join(csrc, fn), "rb") as f:
            h.update(fn.encode() + b"\0" + f.read())
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


def pmc_summary(name, fetch_dir, write_dir, copy_fetch_dir, copy_write_dir, out_path):
    """Turn four rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE of one prefill
    workload's calls; the same two counters over bench.py --only copy) into
    per-call HBM bytes. The counters report KiB per dispatch; each is scaled
    by the ratio of the plain copy's known bytes to what the same counter
    reads for it. Every kernel of the library counts (all launches of one
    call), the copy and torch's own kernels do not."""
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
        if "tl::" not in k:
            continue
        kernels[k] = {"fetch_bytes": fetch.get(k, 0.0) * f_scale, "write_bytes": write.get(k, 0.0) * w_scale}
    total = sum(v["fetch_bytes"] + v["write_bytes"] for v in kernels.values())
    rec = {"workload": name, "source_hash": source_hash(name), "fetch_scale": f_scale, "write_scale": w_scale,
           "copy_kernel": ck, "kernels": kernels, "bytes_per_call": total}
    with open(out_path, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec))


def stored_traffic(name=HEADLINE):
    """HBM bytes per prefill call from the stored counter summary, or None if
    the kernels changed since it was taken."""
    try:
        with open(traffic_path(name)) as f:
            rec = json.load(f)
    except OSError:
        return None
    return rec["bytes_per_call"] if rec.get("source_hash") == source_hash(name) else None


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


def bench_prefill(name, steps, warmup, torch, tl, W, replicas=None):
    """Time `steps` taylor_attn_prefill calls of a named workload (bf16 or
    fp32 in, output in the input dtype), inputs rotating over resident
    replicas. Returns the workload, ms per call, algorithmic bytes and flops
    per call, the feature width, the replica count and the host inputs."""
    w = W.WORKLOADS[name]
    x = W.make_workload(w)
    reps = replicas or PREFILLS[name]["replicas"]
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    code = tl.TAYLOR_BF16 if w.dtype == "bf16" else tl.TAYLOR_F32
    qs = [dev_tensor(x["q"], w.dtype, torch) for _ in range(reps)]
    ks = [dev_tensor(x["k"], w.dtype, torch) for _ in range(reps)]
    vs = [dev_tensor(x["v"], w.dtype, torch) for _ in range(reps)]
    os_ = [torch.empty((w.B, w.H, w.N, w.dv), dtype=tdt, device="cuda") for _ in range(reps)]
    ws_bytes = tl.prefill_workspace_bytes(w.B, w.H, w.N, w.d, w.dv, w.n_terms, tdt)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")
    L = tl.lib()

    # every call's arguments are built before the timed loop, so the loop only
    # enqueues launches (on torch's current stream, which the events time)
    stream = tl._stream().value
    calls = [(qs[r].data_ptr(), ks[r].data_ptr(), vs[r].data_ptr(), code, w.B, w.H, w.N, w.d, w.dv,
              w.n_terms, w.a, None, None, os_[r].data_ptr(), code, None, None, ws.data_ptr(),
              ws_bytes, stream) for r in range(reps)]

    def step(i):
        st = L.taylor_attn_prefill(*calls[i % reps])
        if st != 0:
            tl.check(st)

    for i in range(warmup):
        step(i)
    ms = time_loop(step, steps, torch)
    bytes_, flops, F = algorithmic_prefill(w)
    del qs, ks, vs, os_, ws
    return w, ms, bytes_, flops, F, reps, x


def prefill_block(name, w, ms, bytes_, flops, F, reps, steps):
    """Figures of one timed prefill workload: throughput, both roofs, counter
    traffic (null unless the stored record matches the kernel's sources)."""
    gbs = bytes_ / (ms * 1e-3) / 1e9
    tflops = flops / (ms * 1e-3) / 1e12
    traffic = stored_traffic(name)
    return {
        "workload": name, "B": w.B, "H": w.H, "N": w.N, "d": w.d, "dv": w.dv, "n_terms": w.n_terms, "a": w.a,
        "features": F, "dtype": w.dtype, "steps_timed": steps, "input_replicas": reps,
        "ms_per_call": ms, "tokens_per_s": w.B * w.N / (ms * 1e-3),
        "token_heads_per_s": w.B * w.H * w.N / (ms * 1e-3),
        "mfma_tflops": tflops, "mfma_frac": tflops / BF16_DENSE_TFLOPS,
        "hbm_GBps": gbs, "hbm_frac": gbs / HBM_PEAK_GBS,
        "bound": PREFILLS[name]["bound"],
        "traffic_bytes_per_call": traffic,
        "traffic_over_algorithmic": None if traffic is None else traffic / bytes_,
        "note": f"algorithmic flops 4F(dv+1)+(c+1)(d+dv+1) per token-head with c={CHUNK}; "
                "bytes (2d+dv)*in+dv*out per token-head",
    }


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
    # Same-shape read-modify-write ceiling: torch's in-place add over buffers
    # of the state's size, round-robin over the same number of replicas and
    # timed the same way; it reads and writes exactly the bytes a decode step
    # moves, with no feature map or read-out.
    del Ss, zs
    bufs = [torch.empty(state_bytes // 8, dtype=torch.float32, device="cuda").fill_(1.0) for _ in range(R)]
    for i in range(16):
        bufs[i % R].add_(1.0)
    ms_rmw = time_loop(lambda i: bufs[i % R].add_(1.0), w.steps, torch)
    del bufs
    flops = 4 * F * (w.dv + 1) * w.B * w.H / 2            # 2F(dv+1) per head-step
    return {
        "workload": DECODE, "heads": w.B * w.H, "features": F, "steps_timed": w.steps,
        "state_bytes_per_step": state_bytes,
        "us_per_step_cold": ms_cold * 1e3, "us_per_step_hot": ms_hot * 1e3,
        "state_GBps_cold": state_bytes / (ms_cold * 1e-3) / 1e9,
        "state_GBps_hot": state_bytes / (ms_hot * 1e-3) / 1e9,
        "hbm_frac_cold": state_bytes / (ms_cold * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "state_replicas_cold": R, "algorithmic_gflop_per_step": flops / 1e9,
        "rmw_ceiling": {"us_per_step": ms_rmw * 1e3, "GBps": state_bytes / (ms_rmw * 1e-3) / 1e9,
                        "hbm_frac": state_bytes / (ms_rmw * 1e-3) / 1e9 / HBM_PEAK_GBS,
                        "what": "torch in-place add over buffers of the state's size, same replicas and timing"},
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


def _van_der_corput_blocks(nb):
    """Block indices 0..nb-1 in base-2 radical-inverse order: every prefix of
    the list spreads over the whole sequence, so a sample cut short anywhere
    covers early and late rows alike."""
    order, seen = [], set()
    bits = max(1, (nb - 1).bit_length())
    for i in range(1 << bits):
        r = int(format(i, f"0{bits}b")[::-1], 2)
        if r < nb and r not in seen:
            seen.add(r)
            order.append(r)
    return order


def _oracle_leg(w, x, budget_s, block=256):
    """fp64 oracle direct() over 256-row query blocks of the workload's own
    inputs (blocks in radical-inverse order, heads in turn) until budget_s.
    Row t costs t + 1 key columns, so the rate is converted to whole-workload
    rows by work: equivalent token-heads = sum over sampled rows of (t + 1)
    divided by the workload's mean (N + 1) / 2."""
    from oracle import taylor_oracle as T
    nb = (w.N + block - 1) // block
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    work = 0
    blocks = 0
    t0 = time.perf_counter()
    for i, blk in enumerate(_van_der_corput_blocks(nb) * len(heads)):
        b, h = heads[i % len(heads)]
        rows = np.arange(blk * block, min(w.N, (blk + 1) * block))
        T.direct(x["q64"][b, h], x["k64"][b, h], x["v64"][b, h], w.n_terms, w.a, rows=rows)
        work += int(np.sum(rows + 1))
        blocks += 1
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    token_heads = work / ((w.N + 1) / 2.0)
    return token_heads / dt / w.H, dt, blocks


def cpu_baseline(w, x, budget_s):
    """The fp64 oracle on the host cores, over a bounded sample of the same
    workload: all cores (BLAS threads as configured), then one thread, as the
    pages' own implementation runs ("Expanding Attention", defaults
    paragraph: single-threaded NumPy)."""
    try:
        import threadpoolctl
        threads = max(i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()) or 1
    except Exception:  # noqa: BLE001
        threadpoolctl = None
        threads = os.cpu_count() or 1
    sample = ("256-row query blocks of the same inputs in radical-inverse order over the sequence, heads in turn, "
              "fp64 numpy direct(); rate converted to whole-workload rows by work (row t costs t+1 keys); "
              "tokens/s = token-heads/s / H")
    v, dt, nblk = _oracle_leg(w, x, budget_s)
    out = {"value": v, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
           "sample": f"{sample}; {nblk} blocks in {dt:.1f} s"}
    if threadpoolctl is not None:
        with threadpoolctl.threadpool_limits(1):
            v1, dt1, nb1 = _oracle_leg(w, x, budget_s)
        out["single_thread"] = {"value": v1, "unit": "tokens/s", "cores": 1, "kind": "oracle",
                                "sample": f"same recipe on one BLAS thread; {nb1} blocks in {dt1:.1f} s"}
    return out


def time_ext(torch, tl, W):
    """Plain prefill against the extended entry point with a decay (0.999) and
    with q/k normalisation plus scales (2, 2), on the shapes of the two order-2
    bf16 workloads (the options run on the generic kernels). Prints one JSON
    line per shape."""
    for name in ("based_order2_prefill", "long_order2_prefill"):
        w = W.WORKLOADS[name]
        g = torch.Generator(device="cuda")
        g.manual_seed(3)
        q, k = (torch.randn(w.B, w.H, w.N, w.d, device="cuda", generator=g).bfloat16() for _ in range(2))
        v = torch.randn(w.B, w.H, w.N, w.dv, device="cuda", generator=g).bfloat16()
        res = {"workload": name}
        for label, kw in (("plain", {}), ("decay_0.999", {"gamma": 0.999}),
                          ("qk_norm_scales_2", {"qk_norm": True, "q_scale": 2.0, "k_scale": 2.0})):
            nb = tl.prefill_workspace_bytes(w.B, w.H, w.N, w.d, w.dv, w.n_terms, q.dtype, decayed=bool(kw))
            ws = torch.empty(max(nb, 1), dtype=torch.uint8, device="cuda")
            call = lambda i: tl.prefill(q, k, v, w.n_terms, w.a, workspace=ws, **kw)
            for i in range(3):
                call(i)
            res[label + "_ms"] = time_loop(call, 10, torch)
        print(json.dumps(res), flush=True)


def bench_order6(torch, tl):
    """Order 6 (n_terms = 7, d = 16, dv = 64, F = 74,613; the generic kernels):
    one prefill shape and one decode shape, random bf16 / fp32 inputs with
    q and k rows at norm 2 (as in the order-4 workload). Algorithmic flops
    and state bytes as for the other workloads."""
    d, dv, n, a = 16, 64, 7, 4.0
    F = feature_dim(d, n)
    g = torch.Generator(device="cuda")
    g.manual_seed(7)

    def rows(shape, dt):
        x = torch.randn(*shape, device="cuda", generator=g)
        return (2.0 * x / x.norm(dim=-1, keepdim=True)).to(dt)
    B, H, N = 2, 8, 2048
    q, k = rows((B, H, N, d), torch.bfloat16), rows((B, H, N, d), torch.bfloat16)
    v = torch.randn(B, H, N, dv, device="cuda", generator=g).bfloat16()
    ws = torch.empty(max(tl.prefill_workspace_bytes(B, H, N, d, dv, n, q.dtype), 1), dtype=torch.uint8,
                     device="cuda")
    call = lambda i: tl.prefill(q, k, v, n, a, workspace=ws)
    for i in range(2):
        call(i)
    ms = time_loop(call, 5, torch)
    flops = B * H * N * (4 * F * (dv + 1) + (CHUNK + 1) * (d + dv + 1))
    out = {"prefill": {"B": B, "H": H, "N": N, "dtype": "bf16", "ms_per_call": ms,
                       "tokens_per_s": B * N / (ms * 1e-3), "mfma_tflops": flops / (ms * 1e-3) / 1e12,
                       "mfma_frac": flops / (ms * 1e-3) / 1e12 / BF16_DENSE_TFLOPS}}
    del q, k, v, ws
    Bd, Hd = 8, 16
    S = torch.randn(Bd, Hd, F, dv, device="cuda", generator=g) * 0.01
    z = torch.rand(Bd, Hd, F, device="cuda", generator=g) + 1.0
    qd, kd = rows((8, Bd, Hd, d), torch.float32), rows((8, Bd, Hd, d), torch.float32)
    vd = torch.randn(8, Bd, Hd, dv, device="cuda", generator=g)
    step = lambda i: tl.decode(qd[i % 8], kd[i % 8], vd[i % 8], S, z, n, a)
    for i in range(2):
        step(i)
    msd = time_loop(step, 16, torch)
    nbytes = 2 * F * (dv + 1) * 4 * Bd * Hd
    out["decode"] = {"heads": Bd * Hd, "us_per_step": msd * 1e3, "state_bytes_per_step": nbytes,
                     "state_GBps": nbytes / (msd * 1e-3) / 1e9,
                     "hbm_frac": nbytes / (msd * 1e-3) / 1e9 / HBM_PEAK_GBS}
    out["features"] = F
    return out


def time_fmap(torch, tl):
    """The standalone feature map: rows of bf16 inputs -> [rows, F] fp32. It
    is bound by the HBM write of the output (4F bytes per row; the input adds
    2d). Prints one JSON line per (d, n_terms)."""
    g = torch.Generator(device="cuda")
    g.manual_seed(5)
    for d, n, rows in ((16, 3, 1 << 20), (16, 5, 1 << 16), (64, 3, 1 << 17), (16, 7, 1 << 12)):
        x = torch.randn(rows, d, device="cuda", generator=g).bfloat16()
        F = feature_dim(d, n)
        call = lambda i: tl.feature_map(x, n, a=math.sqrt(d))
        for i in range(2):
            call(i)
        ms = time_loop(call, 10, torch)
        nbytes = rows * (4 * F + 2 * d)
        print(json.dumps({"d": d, "n_terms": n, "features": F, "rows": rows, "ms": ms,
                          "GBps": nbytes / (ms * 1e-3) / 1e9, "hbm_frac": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}),
              flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--replicas", type=int, default=None)
    ap.add_argument("--decode-replicas", type=int, default=8)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip the order-2 d=16 and order-4 prefill blocks")
    ap.add_argument("--no-native", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=10.0)
    ap.add_argument("--only", choices=["prefill", "decode", "copy"], default=None)
    ap.add_argument("--workload", default=HEADLINE, choices=sorted(PREFILLS),
                    help="prefill workload of --only prefill")
    ap.add_argument("--time", nargs="+", metavar="WORKLOAD",
                    help="time one prefill call of each named workload, then exit")
    ap.add_argument("--sweep", action="store_true",
                    help="growth of prefill time with N and of decode time with the context, then exit")
    ap.add_argument("--fmap", action="store_true",
                    help="time the standalone feature map (taylor_feature_map) on a few widths, then exit")
    ap.add_argument("--ext", action="store_true",
                    help="time the extended entry point (decay, q/k preprocessing) against the plain one on the "
                         "two order-2 workload shapes, then exit")
    ap.add_argument("--pmc-summary", nargs=5,
                    metavar=("WORKLOAD", "FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR", "COPY_WRITE_DIR"),
                    help="summarise rocprofv3 --pmc runs into the workload's stored traffic record and exit")
    args = ap.parse_args()
    if args.pmc_summary:
        name = args.pmc_summary[0]
        pmc_summary(name, *args.pmc_summary[1:], traffic_path(name))
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
    if args.ext:
        time_ext(torch, tl, W)
        return
    if args.fmap:
        time_fmap(torch, tl)
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
    if args.only == "prefill":
        r = bench_prefill(args.workload, args.steps, args.warmup, torch, tl, W, args.replicas)
        print(json.dumps(prefill_block(args.workload, *r[:6], args.steps)))
        return

    log(f"prefill: {HEADLINE}, {args.steps} timed calls")
    w, ms, bytes_, flops, F, reps, x = bench_prefill(HEADLINE, args.steps, args.warmup, torch, tl, W,
                                                     args.replicas)
    tflops = flops / (ms * 1e-3) / 1e12
    gbs = bytes_ / (ms * 1e-3) / 1e9
    out = {
        "metric": "prefill tokens/s + MFMA % peak; decode state GB/s % HBM peak (1 GPU)",
        "value": w.B * w.N / (ms * 1e-3),
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
        "config": {"workload": HEADLINE, "B": w.B, "H": w.H, "N": w.N, "d": w.d, "dv": w.dv,
                   "n_terms": w.n_terms, "a": w.a, "features": F, "in": "bf16", "out": "bf16",
                   "accumulate": "fp32", "input_replicas": reps, "seed": w.seed},
        "token_heads_per_s": w.B * w.H * w.N / (ms * 1e-3),
        "roofline": {"bound": "mfma", "achieved": tflops, "peak": BF16_DENSE_TFLOPS, "unit": "TFLOP/s",
                     "frac": tflops / BF16_DENSE_TFLOPS, "traffic": stored_traffic(HEADLINE),
                     "kernel": "one taylor_attn_prefill call (all its launches), timed by HIP events on the "
                               "stream the library launches on",
                     "launch_us": ms * 1e3, "algorithmic_flops_per_launch": flops,
                     "algorithmic_bytes_per_launch": bytes_,
                     "note": f"algorithmic flops 4F(dv+1)+(c+1)(d+dv+1) per token-head, c={CHUNK}; traffic = "
                             "HBM bytes per call from FETCH_SIZE/WRITE_SIZE scaled by a plain copy"},
        "hbm": {"achieved_GBps": gbs, "frac": gbs / HBM_PEAK_GBS},
    }
    if not args.no_extra:
        for name in ("based_order2_prefill", "order4_prefill"):
            log(f"prefill: {name}")
            st = max(args.steps, 50) if name == "based_order2_prefill" else args.steps
            r = bench_prefill(name, st, args.warmup, torch, tl, W)
            out[name] = prefill_block(name, *r[:6], st)
            del r
        log("order 6: prefill and decode")
        out["order6"] = bench_order6(torch, tl)
    if not args.no_decode:
        out["decode"] = bench_decode(args, torch, tl, W)
    if not args.no_native:
        out["native_c_abi"] = native_c_abi()
    if not args.no_cpu:
        log("cpu oracle: all cores, then one thread")
        out["cpu_baseline"] = cpu_baseline(w, x, args.cpu_budget)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
