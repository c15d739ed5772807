"""Benchmark of the libfa355 hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input:
the causal bf16 prefill at sequence 8192 (B4 H16 D64) through ``fa_fwd``,
then the bf16 split-KV decode (B64 H32 D128, cache lengths U[4096, 32768],
256-key chunks) through ``fa_decode_splitkv``.  Inputs are resident in HBM
before the timed region starts.  Each call is bracketed by HIP events on the
stream it is launched on (torch's current stream), so the per-kernel times
are measured live; the wall clock over the K steps gives ms_per_step.

The printed JSON line carries:
* value     prefill throughput, algorithmic TFLOP/s (4*D per visible
            query/key pair; masked and skipped pairs are not credited);
* roofline  the prefill kernel against the dense bf16 MFMA peak;
* decode    the decode call's algorithmic GB/s (real K/V rows read once,
            plus q, o and lse) against the 8 TB/s HBM peak;
* cpu_baseline the float64 CPU oracle timed on a bounded sample of the same
            prefill workload (test infrastructure; reported, not a target).

``--config N`` times one workload of the table alone instead (add
``--cpu-baseline`` to time the oracle on a sample of that workload too).

``traffic`` comes from committed rocprofv3 counter summaries under
``profiles/`` and is reported only while the kernel source they were taken
on is unchanged (a hash of the source files is stored with them).
"""

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA (fp16 the same)
PEAK_F32_TFLOPS = 157.3     # MI355X dense fp32 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
KERNEL_SOURCES = ["exact_tiled_attention_11_amd/csrc/fwd.hip",
                  "exact_tiled_attention_11_amd/csrc/decode.hip",
                  "exact_tiled_attention_11_amd/csrc/bwd.hip",
                  "exact_tiled_attention_11_amd/csrc/fa_device.h"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_hash():
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def counters(name):
    """Per-launch HBM bytes from a committed counter summary, if still current."""
    path = os.path.join(ROOT, "profiles", name)
    if not name or not os.path.exists(path):
        return None
    try:
        with open(path) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    if d.get("source_hash") != source_hash():
        return None
    return d.get("hbm_bytes_per_launch")


def make_prefill(w, dev):
    import workloads as wl
    q, k, v = wl.prefill_inputs(w)
    return q.to(dev), k.to(dev), v.to(dev)


def make_decode(w, dev):
    """Device caches filled entry by entry (only the real rows are drawn)."""
    import torch
    import workloads as wl
    lens = w.lengths()
    dt = torch.bfloat16
    q = wl.decode_query(w).to(dev)
    kc = torch.empty((w.B, w.Nk, w.H, w.D), dtype=dt, device=dev)
    vc = torch.empty((w.B, w.Nk, w.H, w.D), dtype=dt, device=dev)
    for b in range(w.B):
        L = int(lens[b])
        kc[b, :L].copy_(wl.decode_cache_rows(w, 1, b, L))
        vc[b, :L].copy_(wl.decode_cache_rows(w, 2, b, L))
    sl = torch.tensor(lens, dtype=torch.int32, device=dev)
    return q, kc, vc, sl


def cpu_baseline(w, budget_s=20.0):
    """The oracle on whole (batch, head) slices of the prefill workload until
    the time budget is spent; returns algorithmic TFLOP/s of the sample."""
    import numpy as np
    import oracle
    import workloads as wl
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:
        cores = 1
    q, k, v = wl.prefill_inputs(w)
    q64, k64, v64 = wl.to_f64(q), wl.to_f64(k), wl.to_f64(v)
    per_head_flops = 4.0 * w.D * (w.Nq * (w.Nq + 1) // 2 if w.causal else w.Nq * w.Nk)
    done, t0 = 0, time.perf_counter()
    pairs = [(b, h) for b in range(w.B) for h in range(w.H)]
    for b, h in pairs:
        oracle.attention(q64[b:b + 1, :, h:h + 1], k64[b:b + 1, :, h:h + 1],
                         v64[b:b + 1, :, h:h + 1], w.scale, w.causal)
        done += 1
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    return {
        "value": done * per_head_flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": cores,
        "kind": "oracle",
        "sample": "%d of %d (batch, head) slices of %s, %.1f s of float64 numpy (BLAS "
                  "threads = cores; exp single-threaded)" % (done, len(pairs), w.name, dt),
    }


def cpu_baseline_config(w, budget_s=20.0):
    """The oracle on a bounded sample of one table workload, in that
    workload's unit: whole (batch, head) slices of a prefill, whole
    (sequence, head) pairs of a packed batch, whole batch entries (all heads)
    of a decode.  Input generation is outside the timed region."""
    import numpy as np
    import oracle
    import workloads as wl
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:
        cores = 1
    done, work, spent = 0, 0.0, 0.0
    wall0 = time.perf_counter()  # input generation counts against 3x the budget
    if w.kind == "prefill":
        if w.backward or w.dropout or w.prefix or w.alibi:
            return None
        return cpu_baseline(w, budget_s)
    if w.kind == "varlen":
        q, k, v, cu = wl.varlen_inputs(w)
        units = [(s, h) for s in range(len(cu) - 1) for h in range(w.H)]
        for s, h in units:
            a, b = int(cu[s]), int(cu[s + 1])
            qs, ks, vs = (wl.to_f64(t[a:b, h:h + 1])[None] for t in (q, k, v))
            t0 = time.perf_counter()
            oracle.attention(qs, ks, vs, w.scale, w.causal)
            spent += time.perf_counter() - t0
            L = b - a
            work += 4.0 * w.D * (L * (L + 1) // 2 if w.causal else L * L)
            done += 1
            if spent > budget_s or time.perf_counter() - wall0 > 3 * budget_s:
                break
        what = "(sequence, head) pairs"
        value, unit = work / spent / 1e12, "TFLOP/s"
    elif w.kind == "decode":
        lens = w.lengths()
        q = wl.to_f64(wl.decode_query(w))
        units = list(range(w.B))
        es = 2 if w.dtype in ("bf16", "f16") else 4
        for b in units:
            L = int(lens[b])
            kc = wl.to_f64(wl.decode_cache_rows(w, 1, b, L))[None]
            vc = wl.to_f64(wl.decode_cache_rows(w, 2, b, L))[None]
            t0 = time.perf_counter()
            oracle.decode(q[b:b + 1], kc, vc, np.array([L]), w.scale)
            spent += time.perf_counter() - t0
            work += 2.0 * L * w.H * w.D * es
            done += 1
            if spent > budget_s or time.perf_counter() - wall0 > 3 * budget_s:
                break
        what = "batch entries (all heads)"
        value, unit = work / spent / 1e9, "GB/s"
    else:
        return None
    return {
        "value": value,
        "unit": unit,
        "cores": cores,
        "kind": "oracle",
        "sample": "%d of %d %s of %s, %.1f s of float64 numpy (BLAS threads = cores)"
                  % (done, len(units), what, w.name, spent),
    }


def run_config(n, args, dev):
    """Time the library call of one workload of the benchmark table alone
    (the parity-test configurations) and print one JSON line for it."""
    import torch
    import workloads as wl
    import numpy as np
    import exact_tiled_attention_11_amd as fa
    w = wl.CFG[n]
    log("generating inputs for %s" % w.name)
    if w.kind == "prefill" and w.backward:
        q, k, v = make_prefill(w, dev)
        do = wl.tensor(w, 3, (w.B, w.Nq, w.H, w.D)).to(dev)
        sd = torch.from_numpy(wl.alibi_slopes(w.H)).to(dev) if w.alibi else None
        if w.dropout and (w.prefix or w.alibi):
            o, lse = fa.fwd_ex(q, k, v, causal=w.causal, scale=w.scale, prefix=w.prefix,
                               alibi_slopes=sd, dropout_p=w.dropout, seed=w.seed)
        elif w.dropout:
            o, lse = fa.fwd_dropout(q, k, v, dropout_p=w.dropout, seed=w.seed, causal=w.causal,
                                    scale=w.scale)
        elif w.prefix or w.alibi:
            o, lse = fa.fwd_masked(q, k, v, causal=w.causal, scale=w.scale, prefix=w.prefix,
                                   alibi_slopes=sd)
        else:
            o, lse = fa.fwd(q, k, v, causal=w.causal, scale=w.scale)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        ws = torch.empty(fa.fa_bwd_workspace_bytes(w.B, w.H, w.Nq), dtype=torch.uint8, device=dev)
        call = lambda: fa.bwd(q, k, v, o, lse, do, causal=w.causal, scale=w.scale, dq=dq, dk=dk,
                              dv=dv, dropout_p=w.dropout, seed=w.seed, prefix=w.prefix,
                              alibi_slopes=sd, workspace=ws)
    elif w.kind == "prefill":
        q, k, v = make_prefill(w, dev)
        o = torch.empty_like(q)
        lse = torch.empty((w.B, w.H, w.Nq), dtype=torch.float32, device=dev)
        if w.dropout and (w.prefix or w.alibi):
            sd = torch.from_numpy(wl.alibi_slopes(w.H)).to(dev) if w.alibi else None
            call = lambda: fa.fwd_ex(q, k, v, causal=w.causal, scale=w.scale, prefix=w.prefix,
                                     alibi_slopes=sd, dropout_p=w.dropout, seed=w.seed, out=o,
                                     lse=lse)
        elif w.dropout:
            call = lambda: fa.fwd_dropout(q, k, v, dropout_p=w.dropout, seed=w.seed,
                                          causal=w.causal, scale=w.scale, out=o, lse=lse)
        elif w.prefix or w.alibi:
            sd = torch.from_numpy(wl.alibi_slopes(w.H)).to(dev) if w.alibi else None
            call = lambda: fa.fwd_masked(q, k, v, causal=w.causal, scale=w.scale, prefix=w.prefix,
                                         alibi_slopes=sd, out=o, lse=lse)
        else:
            call = lambda: fa.fwd(q, k, v, causal=w.causal, scale=w.scale, out=o, lse=lse)
    elif w.kind == "varlen" and w.backward:
        q, k, v, cu = wl.varlen_inputs(w)
        q, k, v = q.to(dev), k.to(dev), v.to(dev)
        do = wl.tensor(w, 3, tuple(q.shape)).to(dev)
        cud = torch.from_numpy(cu).to(dev)
        mx = int(np.diff(cu).max())
        sd = torch.from_numpy(wl.alibi_slopes(w.H)).to(dev) if w.alibi else None
        opts = dict(prefix=w.prefix, alibi_slopes=sd, dropout_p=w.dropout, seed=w.seed)
        o, lse = fa.fwd_varlen(q, k, v, cud, cud, causal=w.causal, scale=w.scale, **opts)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        ws = torch.empty(fa.fa_bwd_workspace_bytes(1, w.H, q.shape[0]), dtype=torch.uint8,
                         device=dev)
        call = lambda: fa.bwd_varlen(q, k, v, o, lse, do, cud, cud, causal=w.causal,
                                     scale=w.scale, max_seqlen_q=mx, max_seqlen_k=mx, dq=dq,
                                     dk=dk, dv=dv, workspace=ws, **opts)
    elif w.kind == "varlen":
        q, k, v, cu = wl.varlen_inputs(w)
        q, k, v = q.to(dev), k.to(dev), v.to(dev)
        cud = torch.from_numpy(cu).to(dev)
        o = torch.empty_like(q)
        lse = torch.empty((w.H, q.shape[0]), dtype=torch.float32, device=dev)
        ws = torch.empty(fa.fa_fwd_varlen_workspace_bytes(len(cu) - 1, q.shape[0]),
                         dtype=torch.uint8, device=dev)
        sd = torch.from_numpy(wl.alibi_slopes(w.H)).to(dev) if w.alibi else None
        call = lambda: fa.fwd_varlen(q, k, v, cud, cud, causal=w.causal, scale=w.scale, out=o,
                                     lse=lse, workspace=ws, prefix=w.prefix, alibi_slopes=sd,
                                     dropout_p=w.dropout, seed=w.seed)
    elif w.kind == "paged":
        dq, kc, vc, sl = make_decode(w, dev)
        table, num_pages = wl.page_layout(w, w.page_size)
        bt = torch.from_numpy(table).to(dev)
        pool = (num_pages, w.page_size, w.H, w.D)
        idx = bt.flatten().long()
        kp = torch.empty(pool, dtype=kc.dtype, device=dev)
        kp[idx] = kc.view(-1, *pool[1:])
        del kc
        vp = torch.empty(pool, dtype=vc.dtype, device=dev)
        vp[idx] = vc.view(-1, *pool[1:])
        del vc
        o = torch.empty_like(dq)
        lse = torch.empty((w.B, w.H), dtype=torch.float32, device=dev)
        ws = torch.empty(fa.fa_decode_workspace_bytes(w.B, w.H, table.shape[1] * w.page_size, w.D,
                                                      w.chunk), dtype=torch.uint8, device=dev)
        call = lambda: fa.decode_splitkv_paged(dq, kp, vp, sl, bt, scale=w.scale, chunk=w.chunk,
                                               out=o, lse=lse, workspace=ws)
    else:
        dq, kc, vc, sl = make_decode(w, dev)
        o = torch.empty_like(dq)
        lse = torch.empty((w.B, w.H), dtype=torch.float32, device=dev)
        ws = torch.empty(fa.fa_decode_workspace_bytes(w.B, w.H, w.Nk, w.D, w.chunk),
                         dtype=torch.uint8, device=dev)
        call = lambda: fa.decode_splitkv(dq, kc, vc, sl, scale=w.scale, chunk=w.chunk, out=o,
                                         lse=lse, workspace=ws)
    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    for e0, e1 in evs:
        e0.record()
        call()
        e1.record()
    torch.cuda.synchronize()
    t = sorted(e0.elapsed_time(e1) for e0, e1 in evs)
    ms, med = sum(t) / len(t), t[len(t) // 2]
    if w.kind in ("decode", "paged"):
        val, unit, peak, bound = w.bytes_moved() / (ms * 1e-3) / 1e9, "GB/s", PEAK_HBM_GBS, "hbm"
    else:
        peak = PEAK_F32_TFLOPS if w.dtype == "f32" else PEAK_BF16_TFLOPS
        val, unit, bound = w.flops() / (ms * 1e-3) / 1e12, "TFLOP/s", "mfma"
    # HBM-side bytes per call from a committed counter summary, where one
    # exists for this workload and the kernel sources are unchanged since
    traffic = counters({9: "fa_bwd_causal_bf16_b4h16n8192d64.counters.json"}.get(n, ""))
    line = {"config": w.name, "kind": w.kind, "dtype": w.dtype, "value": val, "unit": unit,
            "ms_per_call": ms, "ms_median": med, "ms_min": t[0], "steps": args.steps,
            "roofline": {"bound": bound, "achieved": val, "peak": peak, "unit": unit,
                         "frac": val / peak, "traffic": traffic}}
    if args.cpu_baseline:
        log("timing the CPU oracle on a sample of %s" % w.name)
        line["cpu_baseline"] = cpu_baseline_config(w, args.cpu_budget)
    print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-baseline", action="store_true",
                    help="with --config: also time the CPU oracle on a bounded sample of that "
                         "workload (forward prefill, varlen and decode workloads)")
    ap.add_argument("--cpu-budget", type=float, default=20.0)
    ap.add_argument("--only", choices=["prefill", "decode", "copy"], default=None,
                    help="time one call only (for profiling runs); 'copy' runs a plain "
                         "1 GiB device-to-device copy, the reference for HBM byte counters")
    ap.add_argument("--config", type=int, choices=list(range(1, 19)), default=None,
                    help="time one workload alone (its library call only) and print a JSON "
                         "line for it instead of the bench line: 1-5 the benchmark table, "
                         "6 its decode over a paged cache, 7 / 8 its N8192 causal prefill "
                         "with a 2048-key prefix mask / with ALiBi, 9 the gradients of "
                         "that prefill (fa_bwd), 10 / 11 that prefill / its gradients with "
                         "attention dropout 0.1, 12 / 13 the gradients with the prefix mask / "
                         "with ALiBi, 14 the gradients of the varlen workload, 15 / 16 the "
                         "varlen workload with ALiBi and dropout 0.1 / its gradients, 17 / 18 "
                         "the N8192 causal prefill with the prefix, ALiBi and dropout 0.1 / its "
                         "gradients")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: libfa355 has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    import workloads as wl
    import exact_tiled_attention_11_amd as fa

    fa.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.config is not None:
        run_config(args.config, args, dev)
        return
    if args.only == "copy":
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(args.warmup + args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_each_way": src.numel() * 4, "calls": args.warmup + args.steps}))
        return
    wp, wd = wl.CFG[3], wl.CFG[5]
    do_p = args.only in (None, "prefill")
    do_d = args.only in (None, "decode")

    log("generating inputs")
    if do_p:
        q, k, v = make_prefill(wp, dev)
        o = torch.empty_like(q)
        lse = torch.empty((wp.B, wp.H, wp.Nq), dtype=torch.float32, device=dev)
    if do_d:
        dq, kc, vc, sl = make_decode(wd, dev)
        do_ = torch.empty_like(dq)
        dlse = torch.empty((wd.B, wd.H), dtype=torch.float32, device=dev)
        ws = torch.empty(fa.fa_decode_workspace_bytes(wd.B, wd.H, wd.Nk, wd.D, wd.chunk),
                         dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    def step(ev=None):
        if do_p:
            if ev: ev[0].record()
            fa.fwd(q, k, v, causal=True, scale=wp.scale, out=o, lse=lse)
            if ev: ev[1].record()
        if do_d:
            if ev: ev[2].record()
            fa.decode_splitkv(dq, kc, vc, sl, scale=wd.scale, chunk=wd.chunk, out=do_, lse=dlse,
                              workspace=ws)
            if ev: ev[3].record()

    log("warmup %d" % args.warmup)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    log("timing %d steps" % args.steps)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    tp = [e[0].elapsed_time(e[1]) for e in evs] if do_p else []
    td = [e[2].elapsed_time(e[3]) for e in evs] if do_d else []

    out = {
        "metric": "attention fwd TFLOP/s (prefill) & decode HBM GB/s, % of MI355X roofline",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall * 1e3 / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
    }
    cfg = {"workload": ""}
    if do_p:
        pm = sum(tp) / len(tp)
        pflops = wp.flops()
        achieved = pflops / (pm * 1e-3) / 1e12
        traffic = counters("fa_fwd_causal_bf16_b4h16n8192d64.counters.json")
        out["value"] = achieved
        out["unit"] = "TFLOP/s"
        out["roofline"] = {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS,
                           "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS,
                           "traffic": traffic, "kernel": "fwd_pipe_kernel<bf16,64,causal>",
                           "ms_per_launch": pm, "ms_min": min(tp),
                           "algorithmic_flops_per_launch": pflops}
        cfg["workload"] = "prefill: %s" % wp.name
        cfg["prefill"] = {"B": wp.B, "H": wp.H, "Nq": wp.Nq, "Nk": wp.Nk, "D": wp.D,
                          "causal": True, "scale": wp.scale, "seed": wp.seed}
    if do_d:
        dm = sum(td) / len(td)
        dbytes = wd.bytes_moved()
        gbs = dbytes / (dm * 1e-3) / 1e9
        traffic = counters("fa_decode_bf16_b64h32d128.counters.json")
        out["decode"] = {"value": gbs, "unit": "GB/s", "ms_per_call": dm, "ms_min": min(td),
                         "roofline": {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS,
                                      "unit": "GB/s", "frac": gbs / PEAK_HBM_GBS,
                                      "traffic": traffic,
                                      "kernel": "decode_partial + decode_combine (one call)",
                                      "algorithmic_bytes_per_call": dbytes}}
        cfg["workload"] = (cfg["workload"] + " + " if cfg["workload"] else "") + "decode: %s" % wd.name
        cfg["decode"] = {"B": wd.B, "H": wd.H, "D": wd.D, "Nk_max": wd.Nk, "chunk": wd.chunk,
                         "sum_Lk": int(wd.lengths().sum()), "scale": wd.scale, "seed": wd.seed}
        if not do_p:
            out["value"], out["unit"] = gbs, "GB/s"
            out["roofline"] = out["decode"]["roofline"]
    out["config"] = cfg
    if do_p and not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        out["cpu_baseline"] = cpu_baseline(wp, args.cpu_budget)
    order = ["metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
             "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
             "roofline", "decode", "cpu_baseline"]
    print(json.dumps({k: out[k] for k in order if k in out}), flush=True)


if __name__ == "__main__":
    main()
