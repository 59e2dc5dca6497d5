"""Benchmark of the prefix-KV chunk attention hot path on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic input:
chunk_attn_fwd_append (the forward and the append of the chunk's K/V to the cache,
one launch) and chunk_attn_bwd (delta, dQ, chunk-only dK/dV), on the 8B-like
workload by default (4 windows, 32 query / 8 KV heads, head_dim 128, bf16 prefix
cache, P = 16384, C = 512).

Prints one JSON line. `value` is fwd+bwd algorithmic TFLOP/s of the whole step
(forward: 2 contractions over every allowed (query, key) pair; backward: 3 over
prefix pairs and 5 over chunk pairs; S recompute counted, avoided prefix dK/dV
not). `roofline` is for the dominant kernel (bwd_dq), timed live with HIP events
around each of its launches inside the timed region. `cpu_baseline` times the
fp64 oracle on a bounded sample of the same workload.

After the step, and outside its timing, the calls of the rows beyond the step are
timed on their own (skip them all with --no-next): the prefix gradient within a
horizon (`prefix_kv_grad`, H = 4096), the fused forward + cache append against the two
separate calls (`decode`), and the row-sparse linear backward of the projections next
to attention ("stop-gradient through context tokens", Mechanism) for one 1.7B-class
layer at 2048 tokens with half the rows kept (`row_sparse`).

Warm-up: the --warmup steps, then more untimed steps until --warmup-ms (250) has
passed. From idle, the GPU's clocks take some tens of ms of load to settle (a
kernel trace shows the forward at 650 us early on and 456 us from ~50 ms on), so a
short warm-up would time the ramp instead of the steady state.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
METRIC = "chunk attn fwd+bwd TFLOP/s + prefix-KV GB/s (%roofline) at P=16384,C=512"


def pairs(w):
    prefix = w.chunk_len * w.prefix_len
    chunk = w.chunk_len * (w.chunk_len + 1) // 2
    return prefix, chunk


def flops(w):
    """Algorithmic FLOPs of forward and backward."""
    pp, cp = pairs(w)
    unit = 2 * w.batch * w.n_heads_q * w.head_dim   # FLOPs of one contraction per pair
    fwd = 2 * unit * (pp + cp)
    bwd = unit * (3 * pp + 5 * cp)
    dq = 3 * unit * (pp + cp)                       # S, dP, dQ over every pair
    return fwd, bwd, dq


def prefix_bytes(w):
    rows = w.batch * w.n_heads_kv * w.prefix_len
    if w.cache_type == "q8_0":
        per_row = w.head_dim + 2 * (w.head_dim // 32)
    else:
        per_row = 2 * w.head_dim
    return 2 * rows * per_row   # K and V


def code_text(src):
    """C/C++ source with comments removed and whitespace runs collapsed to one space, so
    that an edit of comments or layout leaves it unchanged (string and character
    literals are kept as written)."""
    out, i, n = [], 0, len(src)
    while i < n:
        c = src[i]
        if c in "\"'":
            j = i + 1
            while j < n and src[j] != c:
                j += 2 if src[j] == "\\" else 1
            out.append(src[i:j + 1])
            i = j + 1
        elif src.startswith("//", i):
            j = src.find("\n", i)
            i = n if j < 0 else j
        elif src.startswith("/*", i):
            j = src.find("*/", i + 2)
            out.append(" ")
            i = n if j < 0 else j + 2
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def source_digest(files):
    """First 16 hex digits of the SHA-256 of the code (comments and layout aside) of the
    kernel sources a figure was taken on."""
    import hashlib
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "prefix_kv_attention_amd", "csrc", f), "r") as fh:
            h.update(code_text(fh.read()).encode())
    return h.hexdigest()[:16]


TRAFFIC_SOURCES = ("attn_bwd.hip", "pka_device.hpp", "pka_internal.hpp")


def read_traffic(kernel_name):
    """HBM bytes per launch from the committed counter summary, if still current."""
    path = os.path.join(ROOT, "profiles", f"{kernel_name}_traffic.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    try:
        files = [f.strip() for f in vals["source_files"].split(",")]
        if source_digest(files) != vals["source_sha256_16"]:
            return None
        return float(vals["bytes_per_launch"])
    except (KeyError, OSError, ValueError):
        return None


def cpu_model():
    """The host CPU's model name from /proc/cpuinfo (None if not readable)."""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def _oracle_group_worker(args):
    """One (window, KV head) group through the fp64 oracle, forward then backward, in a
    pool worker with one BLAS thread. args: (path of the group's .npz inputs, softmax
    scale); the arrays travel through a file because the pool's pipe moves ~100 MB/s
    and would serialise the workers' start. Returns its outputs and seconds."""
    import numpy as np
    import oracle
    path, sc = args
    with np.load(path) as z:
        q, kc, vc, kp, vp, do = (z[k] for k in ("q", "kc", "vc", "kp", "vp", "do"))
    t0 = time.perf_counter()
    o, lse = oracle.group_fwd(q, kc, vc, kp, vp, sc)
    dq, dk, dv, _ = oracle.group_bwd(q, kc, vc, kp, vp, sc, do)
    return (o, lse, dq, dk, dv), time.perf_counter() - t0


def _pool_init():
    import oracle  # noqa: F401  (imported before the timed tasks)
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:  # noqa: BLE001
        pass


def _start(x):
    time.sleep(0.5)   # long enough that every worker of the pool takes one
    return x


def cpu_workers():
    """Workers of the oracle's process pool: the host's cores, at most 16 (a GPU machine
    gives one GPU's job a 16-core share whatever os.cpu_count() shows)."""
    return max(1, min(os.cpu_count() or 1, 16))


def cpu_baseline(w, inputs, budget_s=15.0, gpu_out=None):
    """Time the fp64 oracle (forward + backward) over the workload's (window, KV head)
    groups with a process pool of cpu_workers() workers, one BLAS thread each, in
    whole rounds of the pool until the groups are done or about budget_s of wall
    time is spent (the first round sizes the rest); also the oracle's
    conversion of the chunk's K/V rows into the cache (the append) for the workload's
    cache type and for q8_0. With gpu_out (host copies of the step's O, LSE, dQ, dK,
    dV) it also reports the GPU's errors against the oracle on the groups computed."""
    import multiprocessing as mp
    from concurrent.futures import ProcessPoolExecutor
    import numpy as np
    import oracle
    from oracle.cache import from_torch_bf16
    G = w.group
    sc = w.softmax_scale
    fwd_f, bwd_f, _ = flops(w)
    per_group = (fwd_f + bwd_f) / (w.batch * w.n_heads_kv)
    groups = [(b, kv) for b in range(w.batch) for kv in range(w.n_heads_kv)]
    f = lambda t: from_torch_bf16(t).astype(np.float64)
    workers = cpu_workers()

    import tempfile
    tmp_root = "/dev/shm" if os.path.isdir("/dev/shm") else None
    tmp = tempfile.TemporaryDirectory(prefix="pka_oracle_", dir=tmp_root)

    def args_of(b, kv):
        hs = slice(kv * G, (kv + 1) * G)
        kp = oracle.build_prefix(from_torch_bf16(inputs["kp"][b, kv]), w.cache_type)["values"]
        vp = oracle.build_prefix(from_torch_bf16(inputs["vp"][b, kv]), w.cache_type)["values"]
        path = os.path.join(tmp.name, f"g{b}_{kv}.npz")
        np.savez(path, q=f(inputs["q"][b, hs]), kc=f(inputs["kc"][b, kv]),
                 vc=f(inputs["vc"][b, kv]), kp=kp, vp=vp, do=f(inputs["do"][b, hs]))
        return path, sc

    ctx = mp.get_context("spawn")   # fresh interpreters: the parent holds the GPU
    with tmp, ProcessPoolExecutor(max_workers=workers, mp_context=ctx,
                                  initializer=_pool_init) as ex:
        list(ex.map(_start, range(workers)))         # start every worker, untimed
        # a first round of the pool sizes the sample to the budget
        first = groups[:workers]
        args = [args_of(b, kv) for b, kv in first]    # cache conversion, untimed
        t0 = time.perf_counter()
        res = list(ex.map(_oracle_group_worker, args))
        wall = time.perf_counter() - t0
        cpu_s = sum(r[1] for r in res)
        done = list(zip(first, res))
        rest = groups[workers:]
        if rest and wall < budget_s:
            rounds = int((budget_s - wall) / max(wall, 1e-9))
            more = rest[:max(0, rounds) * workers]
            if more:
                args = [args_of(b, kv) for b, kv in more]
                t0 = time.perf_counter()
                res2 = list(ex.map(_oracle_group_worker, args))
                wall += time.perf_counter() - t0
                cpu_s += sum(r[1] for r in res2)
                done += list(zip(more, res2))
    n = len(done)
    out = {"value": per_group * n / wall / 1e12, "unit": "TFLOP/s", "cores": workers,
           "kind": "oracle",
           "sample": f"{n} of {len(groups)} (window, KV head) groups of {w.name} "
                     f"({G} query heads x {w.chunk_len} rows vs {w.prefix_len + w.chunk_len} "
                     f"keys each), fp64 forward + backward, a pool of {workers} processes "
                     f"with one BLAS thread each: {wall:.1f} s wall, {cpu_s:.1f} s summed over the workers",
           "workers": workers, "blas_threads_per_worker": 1,
           "os_cpu_count": os.cpu_count(), "cpu_model": cpu_model(),
           "wall_s": round(wall, 3), "worker_s": round(cpu_s, 3)}
    # The append: the oracle's conversion of the chunk's K and V rows of every
    # (window, KV head) into the cache's storage, in one process.
    kc, vc = from_torch_bf16(inputs["kc"]), from_torch_bf16(inputs["vc"])
    app = {}
    for ct in dict.fromkeys((w.cache_type, "q8_0")):
        t0 = time.perf_counter()
        oracle.append_rows(kc, ct)
        oracle.append_rows(vc, ct)
        app[ct] = round((time.perf_counter() - t0) * 1e3, 3)
    out["append_ms"] = app
    out["append_rows"] = int(2 * kc.shape[0] * kc.shape[1] * kc.shape[2])
    if gpu_out is not None:
        acc, lse_err = {}, 0.0
        for (b, kv), ((ro, rl, rdq, rdk, rdv), _) in done:
            hs = slice(kv * G, (kv + 1) * G)
            pairs_ = (("o", gpu_out["o"][b, hs], ro), ("dq", gpu_out["dq"][b, hs], rdq),
                      ("dk", gpu_out["dk"][b, kv], rdk), ("dv", gpu_out["dv"][b, kv], rdv))
            for name, got, ref in pairs_:
                acc.setdefault(name, [[], []])
                acc[name][0].append(f(got).ravel())
                acc[name][1].append(ref.ravel())
            lse_err = max(lse_err, float(np.abs(gpu_out["lse"][b, hs].double().numpy()
                                                - rl).max()))
        err = {}
        for name, (a, r) in acc.items():
            a, r = np.concatenate(a), np.concatenate(r)
            err[name] = float(np.linalg.norm(a - r) / np.linalg.norm(r))
        err["lse_abs"] = lse_err
        out["parity_vs_gpu"] = {k: round(v, 6) for k, v in err.items()}
        out["parity_vs_gpu"]["groups"] = n
    return out


class StepSetup:
    """Device buffers and the calls of one chunk step of workload w: the prefix cache
    built by one append of the raw rows, then chunk_attn_fwd_append (forward and the
    append of the chunk's K/V to cache rows [P, P + C), one launch: the backward reads
    cache rows [0, P) only, so the step's outputs are those of forward, backward, then
    append) and chunk_attn_bwd."""

    def __init__(self, pka, w, inputs, dev):
        import torch
        d = {k: v.to(dev) for k, v in inputs.items()}
        B, Hq, Hkv, D, P, C = (w.batch, w.n_heads_q, w.n_heads_kv, w.head_dim, w.prefix_len,
                               w.chunk_len)
        self.cache = pka.PrefixCache.empty(w.cache_type, B, Hkv, P + C, D, dev)
        if P > 0:
            pka.kv_append(d["kp"], d["vp"], self.cache, 0)
        del d["kp"], d["vp"]
        self.q, self.kc, self.vc, self.do = d["q"], d["kc"], d["vc"], d["do"]
        sc = w.softmax_scale
        self.o = torch.empty_like(self.q)
        self.lse = torch.empty((B, Hq, C), dtype=torch.float32, device=dev)
        self.dq = torch.empty_like(self.q)
        self.dk, self.dv = torch.empty_like(self.kc), torch.empty_like(self.vc)
        dims = pka.make_dims(B, Hq, Hkv, D, P, C, sc)
        wsf, wsb = pka.fwd_workspace_bytes(dims), pka.bwd_workspace_bytes(dims)
        self.ws_f = torch.empty(wsf, dtype=torch.uint8, device=dev) if wsf else None
        self.ws_b = torch.empty(wsb, dtype=torch.uint8, device=dev)
        q, kc, vc, do, o, lse, cache = self.q, self.kc, self.vc, self.do, self.o, self.lse, \
            self.cache
        dq, dk, dv, ws_f, ws_b = self.dq, self.dk, self.dv, self.ws_f, self.ws_b

        def fwd_append():
            pka.chunk_attn_fwd_append(q, kc, vc, cache, P, sc, o=o, lse=lse, ws=ws_f)

        def bwd():
            pka.chunk_attn_bwd(q, kc, vc, cache, P, sc, o, lse, do, dq=dq, dk=dk, dv=dv,
                               ws=ws_b)

        def step():
            fwd_append()
            bwd()

        self.fwd_append, self.bwd, self.step = fwd_append, bwd, step


def time_workloads(pka, names, steps, warmup, warmup_ms):
    """The step of each named workload, timed like the headline (untimed warm-up, then
    `steps` back-to-back steps between two synchronisations), one after another and
    after the headline's timed loop. Per workload: ms per step, fwd + bwd algorithmic
    TFLOP/s and its fraction of the bf16 MFMA peak, prefix-cache GB/s (two reads of
    the prefix per step) and its fraction of HBM bandwidth, and the per-kernel
    averages of a short pass with every kernel bracketed by HIP events."""
    import torch
    import synthetic
    out = {}
    for name in names:
        w = synthetic.WORKLOAD_BY_NAME[name]
        st = StepSetup(pka, w, synthetic.make_inputs(w), "cuda:0")
        warm_up(st.step, warmup, warmup_ms)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            st.step()
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / steps
        fwd_f, bwd_f, _ = flops(w)
        tf = (fwd_f + bwd_f) / (ms * 1e-3) / 1e12
        gbs = 2 * prefix_bytes(w) / (ms * 1e-3) / 1e9
        pka.profile_reset()
        pka.profile_select(None)
        pka.profile_enable(True)
        for _ in range(min(steps, 20)):
            st.step()
        torch.cuda.synchronize()
        pka.profile_enable(False)
        kern = {}
        for k in ("fwd", "fwd_combine", "bwd_dq", "bwd_dkdv", "bwd_dq_reduce"):
            tot, n, _ = pka.profile_read(k)
            if n:
                kern[k] = round(tot / n, 5)
        out[name] = {"ms_per_step": round(ms, 5), "tflops": round(tf, 2),
                     "mfma_frac": round(tf / PEAK_BF16_TFLOPS, 4),
                     "prefix_kv_gbs": round(gbs, 1),
                     "prefix_kv_hbm_frac": round(gbs / PEAK_HBM_GBS, 4),
                     "flop_per_step": fwd_f + bwd_f, "steps": steps,
                     "config": {"batch": w.batch, "n_heads_q": w.n_heads_q,
                                "n_heads_kv": w.n_heads_kv, "head_dim": w.head_dim,
                                "prefix_len": w.prefix_len, "chunk_len": w.chunk_len,
                                "cache": w.cache_type},
                     "kernel_ms": kern}
        del st
        torch.cuda.empty_cache()
    return out


def time_prefix_kv_grad(pka, w, t, cache, horizon, steps, warmup):
    """Time pka_prefix_kv_grad (dK/dV of the last H prefix rows from the chunk queries)
    over `steps` launches with HIP events around each launch. Work: 4 contractions (S
    and dP recomputed, dK, dV) of 2*D FLOP per (chunk query, horizon key) pair."""
    import torch
    P, sc = w.prefix_len, w.softmax_scale
    H = min(int(horizon), P)
    q, kc, vc, o, lse, do = t["q"], t["kc"], t["vc"], t["o"], t["lse"], t["do"]
    delta = torch.empty(lse.shape, dtype=torch.float32, device=q.device)
    pka.chunk_attn_fwd(q, kc, vc, cache, P, sc, o=o, lse=lse)
    pka.chunk_attn_bwd(q, kc, vc, cache, P, sc, o, lse, do, delta=delta)
    shape = (w.batch, w.n_heads_kv, H, w.head_dim)
    dkp = torch.empty(shape, dtype=torch.float32, device=q.device)
    dvp = torch.empty(shape, dtype=torch.float32, device=q.device)
    dims = pka.make_dims(w.batch, w.n_heads_q, w.n_heads_kv, w.head_dim, P, w.chunk_len, sc)
    nws = pka.prefix_kv_grad_workspace_bytes(dims, H)
    ws = torch.empty(nws, dtype=torch.uint8, device=q.device) if nws else None

    def run():
        pka.prefix_kv_grad(q, cache, P, sc, lse, do, delta, H, dk=dkp, dv=dvp, ws=ws)

    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    pka.profile_reset()
    pka.profile_select(["prefix_kv", "prefix_kv_reduce"])
    pka.profile_enable(True)
    for _ in range(steps):
        run()
    torch.cuda.synchronize()
    pka.profile_enable(False)
    tot, n, _ = pka.profile_read("prefix_kv")
    ms = tot / n
    red_tot, red_n, _ = pka.profile_read("prefix_kv_reduce")
    flop = 4 * 2 * w.head_dim * w.batch * w.n_heads_q * w.chunk_len * H
    return {"horizon": H, "kernel_ms": round(ms, 5),
            "reduce_ms": round(red_tot / red_n, 5) if red_n else 0.0,
            "flop_per_launch": flop, "achieved": round(flop / (ms * 1e-3) / 1e12, 2),
            "unit": "TFLOP/s", "frac": round(flop / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}


def time_row_sparse(pka, frac, steps, warmup, n_rows=2048, seed=11):
    """Row-sparse linear backward of one decoder layer's projections ("stop-gradient
    through context tokens", Mechanism and its microbenchmark: a 1.7B dense model at
    sequence length 2048): q, o (2048 -> 2048), gate, up (2048 -> 6144) and down
    (6144 -> 2048), with round(frac * 2048) kept rows in reply spans. Kernel times
    from HIP events around each launch (zero fill, dX product, its split reduction when
    split, dW product); work 2 * K * in * out FLOP for dW and the same for dX. Also timed, as context: the same two products with torch on the GPU
    (index_select of the kept rows, two hipBLASLt matmuls, zero and index_copy of
    dX), and the fp64 oracle on the host for q_proj."""
    import numpy as np
    import torch
    import oracle
    import synthetic
    dev = "cuda:0"
    out = {"n_rows": n_rows, "keep_frac": frac, "projections": {}}
    tot_k = tot_t = 0.0
    tot_f = 0
    for proj in synthetic.LAYER_1_7B:
        inp = synthetic.row_sparse_inputs(n_rows, proj.in_features, proj.out_features, frac,
                                          seed)
        x, w, dy, keep = (inp[k].to(dev) for k in ("x", "w", "dy", "keep"))
        dw = torch.empty((proj.out_features, proj.in_features), dtype=torch.float32,
                         device=dev)
        dx = torch.empty_like(x)
        K = keep.numel()

        def run():
            pka.row_sparse_linear_bwd(x, w, dy, keep, dw=dw, dx=dx)

        for _ in range(warmup):
            run()
        torch.cuda.synchronize()
        pka.profile_reset()
        pka.profile_select(["rs_zero", "rs_dx", "rs_dx_reduce", "rs_dw"])
        pka.profile_enable(True)
        for _ in range(steps):
            run()
        torch.cuda.synchronize()
        pka.profile_enable(False)
        t = {k: pka.profile_read(k)[0] / steps
             for k in ("rs_zero", "rs_dx", "rs_dx_reduce", "rs_dw")}
        kl = keep.long()

        def ref():
            xk, dyk = x.index_select(0, kl), dy.index_select(0, kl)
            torch.matmul(dyk.t(), xk)
            dx.zero_()
            dx.index_copy_(0, kl, torch.matmul(dyk, w))

        for _ in range(warmup):
            ref()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record()
        for _ in range(steps):
            ref()
        ev[1].record()
        torch.cuda.synchronize()
        t_ref = ev[0].elapsed_time(ev[1]) / steps
        f = 2 * K * proj.in_features * proj.out_features
        k_ms = t["rs_zero"] + t["rs_dx"] + t["rs_dx_reduce"] + t["rs_dw"]
        tot_k += k_ms
        tot_t += t_ref
        tot_f += 2 * f
        out["projections"][proj.name] = {
            "in": proj.in_features, "out": proj.out_features, "n_keep": K,
            "zero_ms": round(t["rs_zero"], 5), "dx_ms": round(t["rs_dx"], 5),
            "dx_reduce_ms": round(t["rs_dx_reduce"], 5), "dw_ms": round(t["rs_dw"], 5),
            "ws_bytes": pka.row_sparse_workspace_bytes(n_rows, K, proj.in_features,
                                                      proj.out_features),
            "dx_tflops": round(f / (t["rs_dx"] * 1e-3) / 1e12, 1),
            "dw_tflops": round(f / (t["rs_dw"] * 1e-3) / 1e12, 1),
            "torch_ms": round(t_ref, 5)}
    out["layer_kernel_ms"] = round(tot_k, 5)
    out["flop"] = tot_f
    out["achieved"] = round(tot_f / (tot_k * 1e-3) / 1e12, 1)
    out["unit"] = "TFLOP/s"
    out["frac"] = round(tot_f / (tot_k * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)
    out["torch_layer_ms"] = round(tot_t, 5)
    # the fp64 oracle on the host, q_proj
    inp = synthetic.row_sparse_inputs(n_rows, 2048, 2048, frac, seed)
    xs, ws_, dys = (inp[k].to(torch.float64).numpy() for k in ("x", "w", "dy"))
    kp = inp["keep"].numpy().astype(np.int64)
    t0 = time.perf_counter()
    oracle.row_sparse_linear_bwd(xs, ws_, dys, kp)
    sec = time.perf_counter() - t0
    f = 4 * len(kp) * 2048 * 2048
    out["cpu_baseline"] = {"value": round(f / sec / 1e12, 4), "unit": "TFLOP/s",
                           "cores": torch.get_num_threads(), "kind": "oracle",
                           "sample": "q_proj (2048 -> 2048), fp64 numpy, one call"}
    return out


def _pct(xs):
    import numpy as np
    a = np.asarray(xs)
    return {"median": round(float(np.median(a)), 5), "p10": round(float(np.percentile(a, 10)), 5),
            "p90": round(float(np.percentile(a, 90)), 5)}


def time_phases(parts, n, scratch=None):
    """ms of each part of the step (fwd_append, bwd) and of the whole step over n
    iterations, torch events on the current stream (the one the library launches on).
    scratch: a large device buffer rewritten before each iteration (evicts L2 and the
    last-level cache: cold runs)."""
    import torch
    names = list(parts) + ["step"]
    times = {k: [] for k in names}
    for i in range(n):
        if scratch is not None:
            scratch.fill_(i & 0xFF)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(parts) + 1)]
        ev[0].record()
        for j, fn in enumerate(parts.values()):
            fn()
            ev[j + 1].record()
        torch.cuda.synchronize()
        for j, k in enumerate(parts):
            times[k].append(ev[j].elapsed_time(ev[j + 1]))
        times["step"].append(ev[0].elapsed_time(ev[-1]))
    return {k: _pct(v) for k, v in times.items()}


def time_graph(step, steps, warmup):
    """ms per step replayed from a HIP graph of one captured step (the library makes
    no allocation, memset or sync inside its calls), after `warmup` replays."""
    import torch
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        g.replay()
    torch.cuda.synchronize()
    return round((time.perf_counter() - t0) * 1e3 / steps, 5)


def time_decode(pka, w, t, cache, steps, warmup):
    """Time the re-decode of a chunk into the cache two ways: one fused launch
    (pka_chunk_attn_fwd_append) against pka_chunk_attn_fwd followed by
    pka_kv_append_*. Both write the same O, LSE and cache rows [P, P + C); wall time
    per call over `steps` calls, synchronised on both sides."""
    import torch
    P, sc = w.prefix_len, w.softmax_scale
    q, kc, vc, o, lse = t["q"], t["kc"], t["vc"], t["o"], t["lse"]

    def fused():
        pka.chunk_attn_fwd_append(q, kc, vc, cache, P, sc, o=o, lse=lse)

    def separate():
        pka.chunk_attn_fwd(q, kc, vc, cache, P, sc, o=o, lse=lse)
        pka.kv_append(kc, vc, cache, P)

    res = {}
    for name, fn in (("separate_ms", separate), ("fused_ms", fused)):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            fn()
        torch.cuda.synchronize()
        res[name] = round((time.perf_counter() - t0) * 1e3 / steps, 5)
    return res


def warm_up(step, n_min, ms_min):
    """At least n_min untimed steps, continued until ms_min of wall time has passed
    (checked at a synchronisation every 8 steps, so the time is the GPU's, not the
    launch queue's). Returns (steps run, milliseconds)."""
    import torch
    t0 = time.perf_counter()
    n = 0
    while True:
        if n >= n_min and (n % 8 == 0 or n_min == n):
            torch.cuda.synchronize()
            if (time.perf_counter() - t0) * 1e3 >= ms_min:
                break
        step()
        n += 1
    return n, round((time.perf_counter() - t0) * 1e3, 1)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--warmup-ms", type=float, default=250.0,
                    help="after the --warmup steps, keep running untimed steps until this "
                         "much time has passed since the warm-up began: under load the "
                         "GPU's clocks take tens of ms to settle, and a step timed before "
                         "that runs up to 25 %% slower")
    ap.add_argument("--workload", default="8b-16k")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-kernel-events", action="store_true",
                    help="time the step without the per-kernel HIP events")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--prefix-horizon", type=int, default=4096,
                    help="also time pka_prefix_kv_grad (dK/dV of the last H prefix rows) "
                         "on the same inputs, outside the step (0: skip)")
    ap.add_argument("--no-phases", action="store_true",
                    help="skip the untimed warm / cold passes that time fwd_append and bwd "
                         "separately")
    ap.add_argument("--graph", action="store_true",
                    help="also time the step replayed from a captured HIP graph")
    ap.add_argument("--no-decode", action="store_true",
                    help="skip timing the fused forward + cache append against the two "
                         "separate calls (outside the step)")
    ap.add_argument("--row-sparse", type=float, default=0.5, metavar="FRAC",
                    help="kept fraction for timing the row-sparse linear backward of one "
                         "1.7B-class layer's projections at 2048 tokens (< 0: skip)")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip timing the other four workloads' steps (the `configs` "
                         "object, after the headline's timed loop)")
    ap.add_argument("--no-next", action="store_true",
                    help="skip the prefix-gradient, decode and row-sparse legs")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy 3 times (scales the HBM "
                         "byte counters of a profiler run)")
    args = ap.parse_args()

    if args.copy_calibration:
        import torch
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda:0")   # 1 GiB
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": src.numel() * 4, "copy_bytes_written":
                          dst.numel() * 4, "launches": 3}), flush=True)
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the hot path here is one GPU's share at its real "
              "shape and has no cross-GPU step; run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import prefix_kv_attention_amd as pka
    import synthetic

    w = synthetic.WORKLOAD_BY_NAME[args.workload]
    dev = "cuda:0"
    inputs = synthetic.make_inputs(w)
    st = StepSetup(pka, w, inputs, dev)
    B, Hq, Hkv, D, P, C = w.batch, w.n_heads_q, w.n_heads_kv, w.head_dim, w.prefix_len, w.chunk_len
    q, kc, vc, do, o, lse, dq, dk, dv, cache = (st.q, st.kc, st.vc, st.do, st.o, st.lse, st.dq,
                                                st.dk, st.dv, st.cache)
    fwd_append, bwd, step = st.fwd_append, st.bwd, st.step

    warm = warm_up(step, args.warmup, args.warmup_ms)

    # Inside the timed loop only the dominant kernel (bwd_dq) is bracketed by HIP
    # events (two per step); the per-kernel breakdown comes from a short untimed
    # pass afterwards with every kernel bracketed.
    kernel_events = not args.no_kernel_events
    pka.profile_reset()
    pka.profile_select(["bwd_dq"])
    pka.profile_enable(kernel_events)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    pka.profile_enable(False)
    dq_timed = pka.profile_read("bwd_dq") if kernel_events else (0.0, 0, 0)

    ms_step = elapsed * 1e3 / args.steps
    fwd_f, bwd_f, dq_f = flops(w)
    tflops = (fwd_f + bwd_f) / (ms_step * 1e-3) / 1e12
    pbytes = prefix_bytes(w)
    prefix_gbs = 2 * pbytes / (ms_step * 1e-3) / 1e9

    kernels = {}
    if kernel_events:
        n_bd = min(args.steps, 20)
        pka.profile_reset()
        pka.profile_select(None)
        pka.profile_enable(True)
        for _ in range(n_bd):
            step()
        torch.cuda.synchronize()
        pka.profile_enable(False)
        for name in ("fwd", "fwd_combine", "bwd_prep", "bwd_dq", "bwd_dkdv", "bwd_dq_reduce",
                     "bwd_dkdv_reduce", "append"):
            tot, n, _ = pka.profile_read(name)
            if n:
                kernels[name] = round(tot / n, 5)
    roofline = None
    if dq_timed[1]:
        dq_ms = dq_timed[0] / dq_timed[1]
        achieved = dq_f / (dq_ms * 1e-3) / 1e12
        roofline = {"bound": "mfma", "kernel": "bwd_dq", "achieved": round(achieved, 2),
                    "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                    "traffic": read_traffic("bwd_dq"),
                    "flop_per_launch": dq_f, "avg_launch_ms": round(dq_ms, 5),
                    "launches_timed": dq_timed[1]}
    out = {
        "metric": METRIC, "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "warmup_steps_run": warm[0],
        "warmup_ms": warm[1], "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": B, "n_heads_q": Hq, "n_heads_kv": Hkv,
                   "head_dim": D, "prefix_len": P, "chunk_len": C, "cache": w.cache_type,
                   "step": "chunk_attn_fwd_append + chunk_attn_bwd"},
        "prefix_kv_gbs": round(prefix_gbs, 1),
        "prefix_kv_hbm_frac": round(prefix_gbs / PEAK_HBM_GBS, 4),
        "mfma_frac_step": round(tflops / PEAK_BF16_TFLOPS, 4),
        "kernel_ms": kernels,
        "roofline": roofline,
        "cpu_baseline": None,
    }
    if not args.no_phases:
        # Untimed passes after the timed loop: the parts of the step, warm (back to back)
        # and cold (a 1 GiB device write before each step evicts L2 and the MALL).
        n_ph = min(args.steps, 30)
        parts = {"fwd_append": fwd_append, "bwd": bwd}
        scratch = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        out["phases_ms"] = {"iterations": n_ph, "warm": time_phases(parts, n_ph),
                            "cold": time_phases(parts, n_ph, scratch)}
        del scratch
    if args.graph:
        g_ms = time_graph(step, args.steps, args.warmup)
        out["graph"] = {"ms_per_step": g_ms, "value": round((fwd_f + bwd_f) / (g_ms * 1e-3)
                                                            / 1e12, 2)}
    # The calls of the NEXT rows, each outside the step and after it. A failure is
    # reported in its own object and does not lose the step's line.
    def leg(name, fn):
        try:
            out[name] = fn()
        except Exception as e:  # noqa: BLE001
            out[name] = {"error": f"{type(e).__name__}: {e}"}

    if not args.no_configs:
        others = [x.name for x in synthetic.WORKLOADS if x.name != w.name]
        leg("configs", lambda: time_workloads(pka, others, args.steps, args.warmup,
                                              min(args.warmup_ms, 150.0)))
        if isinstance(out.get("configs"), dict) and "error" not in out["configs"]:
            out["configs"][w.name] = {"ms_per_step": round(ms_step, 5),
                                      "tflops": round(tflops, 2),
                                      "mfma_frac": round(tflops / PEAK_BF16_TFLOPS, 4),
                                      "prefix_kv_gbs": round(prefix_gbs, 1),
                                      "prefix_kv_hbm_frac": round(prefix_gbs / PEAK_HBM_GBS, 4),
                                      "headline": True}
    if not args.no_next and args.prefix_horizon > 0:
        leg("prefix_kv_grad", lambda: time_prefix_kv_grad(
            pka, w, dict(q=q, kc=kc, vc=vc, o=o, lse=lse, do=do), cache, args.prefix_horizon,
            args.steps, args.warmup))
    if not args.no_next and not args.no_decode:
        leg("decode", lambda: time_decode(pka, w, dict(q=q, kc=kc, vc=vc, o=o, lse=lse),
                                          cache, args.steps, args.warmup))
    if not args.no_next and args.row_sparse >= 0:
        leg("row_sparse", lambda: time_row_sparse(pka, args.row_sparse, args.steps,
                                                  args.warmup))
    if not args.no_cpu_baseline:
        # The step is deterministic: one more recomputes the outputs the oracle checks.
        fwd_append()
        bwd()
        torch.cuda.synchronize()
        gpu_out = {"o": o.cpu(), "lse": lse.cpu(), "dq": dq.cpu(), "dk": dk.cpu(),
                   "dv": dv.cpu()}
        out["cpu_baseline"] = cpu_baseline(w, inputs, args.cpu_budget, gpu_out)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
