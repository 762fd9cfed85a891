"""Benchmark of the TileMix fused prefill path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--template T] [--coverage BP] [--no-cpu-baseline]

One step = one pass of the device hot path over one packed batch: the
blockwise K quantiser followed by the fused mixed-precision prefill kernel,
which quantises each work unit's Q block in its prologue (one work unit is
exactly one Q block).  ``breakdown.split_path`` times the same step as two
passes over Q (the Q/K quantiser writing Q's INT8 codes, then the prefill
reading them); both give bit-identical outputs.
Routing words and the work plan are static per batch shape (the pages reuse
one template across layers, batch entries and KV heads) and are built once,
outside the timed region; their host build time is reported separately.

Prints ONE JSON line.  ``value`` is whole-job attention tokens/s with inputs
resident in HBM.  ``roofline`` refers to the fused prefill kernel: achieved
fp16-equivalent TFLOP/s (INT8 operations weighted by the fp16/int8 peak
ratio) against the published MI355X dense fp16 MFMA peak, i.e. ``frac`` is
the coverage-weighted MFMA roofline time over the measured kernel time.

Every prefill time below, as in the headline, is taken in the path's order
(each attention call follows its quantiser; HIP events on the launch stream
bracket only the attention call) after 20 untimed calls: the host work
between configurations lets the GPU clock drop, and with 3 warm-up calls the
same kernel measured up to 10% slower.  ``breakdown.prefill_ms_after_legs``
re-times the headline kernel once the legs have run.

``fp8`` (skip with --no-fp8) times the three-path prefill (FP16 / FP8 / INT8
groups from the same template) at two coverage mixes, against the
three-precision MFMA roofline.

``adaptive`` (skip with --no-adaptive) times the content-dependent routing
statistic, the host ranking, and the prefill under the resulting words at the
same coverage.

``sweep_headline`` and ``sweep`` (skip with --no-sweep) time the fused
prefill (the better of two passes) at INT8 coverages 0, 10, 25, 50, 75 and 100% -- the headline
workload's template, then every template at L=8192 -- with tokens/s, the
roofline fraction, whether tokens/s is non-decreasing in coverage, and
MAD(c), the mean absolute difference of all fp16 outputs from the same
kernel at 0%.

``depth`` (skip with --no-depth) runs a synthetic stack of attention +
residual layers (random weights, one template for every layer) at 0%, 25% and
the headline coverage side by side: the mean absolute deviation of the hidden
state from the stack without INT8 groups at every depth, and the time of one
layer and of each of its kernels against their rooflines.

``decode`` (skip with --no-decode) times one decode step per sequence against
an INT8 key/value cache holding the same workload's K and V: tokens/s is new
tokens per second, and its roofline is HBM bandwidth over the step's
algorithmic bytes.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_F16 = 2.5e15   # MI355X dense fp16 MFMA, FLOP/s (published)
PEAK_I8 = 5.0e15    # MI355X dense int8 MFMA, OP/s (published)
PEAK_F8 = 5.0e15    # MI355X dense fp8 MFMA, FLOP/s (published)
PEAK_HBM = 8.0e12   # MI355X HBM3E, bytes/s (published)
METRIC = "prefill attn tokens/s + % of MFMA roofline, 3B shape L=4k B=8 SpTrans75"
KERNEL_SRC = os.path.join(ROOT, "mixed_precision_attention_amd", "csrc", "tilemix_kernels.hip")


def legal_pair_counts(cu, words, hq, hkv):
    """(P, P8): legal causal (query, key) pairs over all query heads, and the
    ones lying in INT8-routed groups -- counted exactly from each KV head's
    words (query head h uses the words of KV head h // (Hq/Hkv))."""
    import numpy as np
    P = 0
    P8 = [0] * hkv
    row_off = 0
    for s in range(len(cu) - 1):
        L = int(cu[s + 1] - cu[s])
        Tm, Tn = -(-L // 128), -(-L // 64)
        g = max(1, -(-Tn // 64))
        for r in range(Tm):
            q = np.arange(128 * r, min(128 * r + 128, L))
            last_t = int(q[-1]) // 64
            t = np.arange(last_t + 1)
            # keys of tile t visible to query q: clip(q - 64 t + 1, 0, 64)
            cnt = np.clip(q[:, None] - 64 * t[None, :] + 1, 0, 64).sum(axis=0)
            P += int(cnt.sum())
            for kv in range(hkv):
                w = np.uint64(words[kv, row_off + r])
                bits = ((w >> (t // g).astype(np.uint64)) & np.uint64(1)).astype(np.int64)
                P8[kv] += int((cnt * bits).sum())
        row_off += Tm
    return P * hq, sum(P8) * (hq // hkv)


def traffic_record(path):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when the summary is missing or the kernel source changed since."""
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    sha = hashlib.sha256(open(KERNEL_SRC, "rb").read()).hexdigest()
    if rec.get("kernel_source_sha256") != sha:
        return None
    return rec


def _counter_mean_kib(path, kernel_substr):
    """Mean per-dispatch value (KiB) of the one counter in a rocprofv3
    counter_collection.csv, over dispatches whose name contains the text
    (every piece of it, when it is a tuple)."""
    import csv
    parts = kernel_substr if isinstance(kernel_substr, tuple) else (kernel_substr,)
    per = {}
    for r in csv.DictReader(open(path)):
        if all(p in r["Kernel_Name"] for p in parts):
            per[r["Dispatch_Id"]] = per.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    if not per:
        raise SystemExit(f"no dispatch of {kernel_substr!r} in {path}")
    return sum(per.values()) / len(per), len(per)


def write_traffic(args):
    """HBM bytes per prefill launch: FETCH_SIZE and WRITE_SIZE scaled by what
    the same counters read for a plain copy of known size."""
    fetch_csv, write_csv, cfetch_csv, cwrite_csv = args.write_traffic
    # the step's prefill kernel, prefill_kernel<d, false, true> (two-path,
    # Q quantised inline)
    kname = "tilemix::prefill_kernel"
    fetch, nf = _counter_mean_kib(fetch_csv, (kname + "<", ", false, true>"))
    write, nw = _counter_mean_kib(write_csv, (kname + "<", ", false, true>"))
    cfetch, _ = _counter_mean_kib(cfetch_csv, "copyBuffer")
    cwrite, _ = _counter_mean_kib(cwrite_csv, "copyBuffer")
    f_scale = args.copy_size / (cfetch * 1024)
    w_scale = args.copy_size / (cwrite * 1024)
    rec = {
        "kernel": kname,
        "workload": args.workload,
        "kernel_source_sha256": hashlib.sha256(open(KERNEL_SRC, "rb").read()).hexdigest(),
        "fetch_kib_per_dispatch": fetch, "write_kib_per_dispatch": write, "dispatches": [nf, nw],
        "copy_bytes": args.copy_size, "copy_fetch_kib": cfetch, "copy_write_kib": cwrite,
        "fetch_scale": f_scale, "write_scale": w_scale,
        "hbm_bytes_per_launch": fetch * 1024 * f_scale + write * 1024 * w_scale,
        "command": args.profile_command,
    }
    out = os.path.join(ROOT, "profiles", f"prefill_{args.workload}_traffic.json")
    with open(out, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(json.dumps(rec))
    return 0


def time_in_pipeline(prep, attend, steps, warmup=20):
    """Mean time (ms) of ``attend`` when each call follows ``prep`` (the
    quantiser), as in the path: HIP events on the launch stream bracket
    only the attention call of every step."""
    import torch
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        prep()
        attend()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    for a, b in ev:
        prep()
        a.record(stream)
        attend()
        b.record(stream)
    torch.cuda.synchronize()
    return sum(a.elapsed_time(b) for a, b in ev) / steps


def bench_adaptive(tp, qd, kd, vd, cu, hq, hkv, d, coverage, steps):
    """Adaptive routing at the same coverage: the device importance statistic
    (timed with events), the whole routing step with the host ranking and
    word upload (wall clock) and with the selection on the device (events),
    and the prefill under the adaptive words."""
    import numpy as np
    import torch
    stream = torch.cuda.current_stream()
    tp.quantize(qd, kd)
    tp.set_routing_adaptive(coverage)          # warm-up and buffers
    torch.cuda.synchronize()
    import mixed_precision_attention_amd as tm
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        tm.tilemix_routing_importance(tp.plan_h, tp.plan_d, tp.q_i8, tp.k_i8, tp.q_scale, tp.k_scale,
                                      tp.imp_ws, tp.importance)
    e1.record(stream)
    torch.cuda.synchronize()
    imp_us = e0.elapsed_time(e1) * 1e3 / steps
    # the whole routing step with the host ranking (wall clock: statistic,
    # copy, ranking, upload), then with the selection on the device (events:
    # statistic + selection, nothing leaves the GPU)
    t0 = time.perf_counter()
    tp.set_routing_adaptive(coverage, on_device=False)
    torch.cuda.synchronize()
    route_ms = (time.perf_counter() - t0) * 1e3
    host_words = tp.words.copy()
    tp.set_routing_adaptive(coverage)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        tp.set_routing_adaptive(coverage)
    e1.record(stream)
    torch.cuda.synchronize()
    route_dev_us = e0.elapsed_time(e1) * 1e3 / steps
    if not np.array_equal(tp.words_host(), host_words):
        raise SystemExit("device-selected adaptive words differ from the host ranking")
    out = torch.empty_like(qd)
    attn_ms = time_in_pipeline(lambda: tp.quantize_k(kd), lambda: tp.attend_qinline(qd, kd, vd, out), steps)
    P, P8 = legal_pair_counts(cu, tp.words_host(), hq, hkv)
    t_roof = 2 * d * (P - P8) / PEAK_F16 + 2 * d * P / PEAK_F16 + 2 * d * P8 / PEAK_I8
    lens = np.diff(np.asarray(cu, dtype=np.int64))
    tq, tk = sum(-(-int(L) // 128) for L in lens), sum(-(-int(L) // 64) for L in lens)
    imp_bytes = int(lens.sum()) * (hq + hkv) * d + (hq * tq + hkv * tk) * d * 4 * 2 + hkv * tq * 64 * 4
    return {"coverage_bp": coverage, "importance_us": imp_us,
            "importance_roofline": {"bound": "hbm", "achieved": imp_bytes / (imp_us * 1e-6) / 1e9,
                                    "peak": PEAK_HBM / 1e9, "unit": "GB/s",
                                    "frac": imp_bytes / (imp_us * 1e-6) / PEAK_HBM,
                                    "algorithmic_bytes": imp_bytes},
            "route_total_ms": route_ms, "route_on_device_us": route_dev_us,
            "prefill_ms": attn_ms, "frac": t_roof / (attn_ms * 1e-3),
            "int8_pair_share": P8 / P}


def bench_exposure(coverages=(2500, 5000, 7500), tau=0.5):
    """Importance exposure of the SpTrans template and of the adaptive words
    ([Explainer, 第二步] importance): per query row, the fewest keys holding a
    share tau of the exact causal softmax's mass are its high-importance keys;
    the figure is their mass inside INT8 groups over their whole mass, summed
    over rows and heads.  On synthetic inputs with locality and a sink (one
    2048-token sequence, 2 query heads over 1 KV head); routing words from the
    library (the adaptive ones from its device importance statistic),
    probabilities in float64 with torch on the GPU."""
    import math
    import numpy as np
    import torch
    import mixed_precision_attention_amd as tm
    import synth
    lens, hq, hkv, d = [2048], 2, 1, 128
    q, k, v, cu = synth.make_qkv_local(lens, hq, hkv, d, seed=7)
    qd, kd = (torch.from_numpy(x).cuda() for x in (q, k))
    L = lens[0]
    tp = tm.TileMixPrefill(cu, hq, hkv, d, "sptrans", coverages[0])
    tp.quantize(qd, kd)
    causal = torch.ones(L, L, dtype=torch.bool, device="cuda").triu(1)
    probs = []
    for h in range(hq):
        kv = h // (hq // hkv)
        S = (qd[:, h, :].double() @ kd[:, kv, :].double().T) / math.sqrt(d)
        P = torch.softmax(S.masked_fill(causal, float("-inf")), dim=1)
        sp, idx = torch.sort(P, dim=1, descending=True, stable=True)
        cum = torch.cumsum(sp, dim=1)
        n = (cum < tau).sum(dim=1, keepdim=True) + 1
        sel = torch.arange(L, device="cuda")[None, :] < n
        probs.append((kv, sp, idx, sel))
    g = int(np.asarray(tp.g).ravel()[0])
    rows = torch.arange(L, device="cuda") // 128

    def exposure(words):
        w = torch.from_numpy(np.ascontiguousarray(words).view(np.int64)).cuda()
        inside = total = 0.0
        for kv, sp, idx, sel in probs:
            grp = (idx // 64) // g
            bits = (w[kv, rows][:, None] >> grp) & 1
            m = sp * sel
            inside += float((m * bits).sum())
            total += float(m.sum())
        return inside / total

    out = {"workload": "one 2048-token sequence with locality and a sink, hq 2, hkv 1, d 128", "tau": tau,
           "sptrans": {}, "adaptive": {}}
    for cov in coverages:
        tp.set_routing("sptrans", cov)
        out["sptrans"][str(cov)] = round(exposure(tp.words), 4)
        tp.set_routing_adaptive(cov)
        out["adaptive"][str(cov)] = round(exposure(tp.words_host()), 4)
    return out


def bench_fp8(qd, kd, vd, cu, hq, hkv, d, template, mixes, steps):
    """Three-path prefill (FP16 / FP8 / INT8 groups) at the given (INT8, FP8)
    coverages against the three-precision MFMA roofline (FP8 at the published
    dense peak), as a step like the headline's (both key quantisers, then the
    prefill making Q's INT8 and FP8 codes in its prologue) and as
    ``split_path`` (both Q/K quantisers, then the prefill reading Q's codes)."""
    import torch
    import mixed_precision_attention_amd as tm
    stream = torch.cuda.current_stream()
    out = torch.empty_like(qd)

    def timed(fn):
        for _ in range(3):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / steps

    rows = []
    for c8, cf in mixes:
        tp = tm.TileMixPrefill3(cu, hq, hkv, d, template, c8, cf)
        kq_us = timed(lambda: tp.quantize_k(kd))
        qk_us = timed(lambda: tp.quantize(qd, kd))
        ms = time_in_pipeline(lambda: tp.quantize_k(kd), lambda: tp.attend_qinline(qd, kd, vd, out), steps)
        ms_split = time_in_pipeline(lambda: tp.quantize(qd, kd), lambda: tp.attend(qd, kd, vd, out), steps)
        P, P8 = legal_pair_counts(cu, tp.words, hq, hkv)
        _, Pf = legal_pair_counts(cu, tp.words_f8, hq, hkv)
        t_roof = 2 * d * (P - P8 - Pf) / PEAK_F16 + 2 * d * P8 / PEAK_I8 + 2 * d * Pf / PEAK_F8 \
            + 2 * d * P / PEAK_F16
        rows.append({"int8_bp": c8, "fp8_bp": cf, "prefill_ms": ms, "frac": t_roof / (ms * 1e-3),
                     "key_quantize_us": kq_us, "step_ms": ms + kq_us * 1e-3,
                     "int8_pair_share": P8 / P, "fp8_pair_share": Pf / P,
                     "split_path": {"prefill_ms": ms_split, "frac": t_roof / (ms_split * 1e-3),
                                    "quantize_us": qk_us, "step_ms": ms_split + qk_us * 1e-3}})
    return {"template": template, "runs": rows}


def bench_depth(cu, hq, hkv, d, template, coverages, n_layers, seed=0, reps=10):
    """Synthetic stack of attention + residual layers (random weights, one
    routing template for every layer): the deviation of the hidden state
    from the stack without INT8 groups at every depth, the time of one layer
    and of each of its kernels, and their rooflines."""
    import numpy as np
    import torch
    import mixed_precision_attention_amd as tm
    import synth
    stream = torch.cuda.current_stream()
    T = int(cu[-1])
    C = hq * d
    W = (hq // hkv) * d
    wqkv, wo = synth.stack_weights(n_layers, hq, hkv, d, seed=seed)
    wqkv_d, wo_d = torch.from_numpy(wqkv).cuda(), torch.from_numpy(wo).cuda()
    x0 = torch.from_numpy(synth.stack_input(T, hq, d, seed=seed + 1)).cuda()
    covs = [0] + [c for c in coverages if c != 0]
    stacks = {}
    for c in covs:
        st = tm.TileMixStack(cu, hq, hkv, d, template, c)
        st.set_weights(wqkv_d, wo_d)
        stacks[c] = st
    xw = x0.clone()
    for l in range(2):
        stacks[covs[-1]].layer(xw, l)
    del xw
    xs = {c: x0.clone() for c in covs}
    ev = {c: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(n_layers)] for c in covs}
    dev = {c: [] for c in covs[1:]}
    mag = []
    torch.cuda.synchronize()
    for l in range(n_layers):
        for c in covs:
            ev[c][l][0].record(stream)
            stacks[c].layer(xs[c], l)
            ev[c][l][1].record(stream)
        for c in covs[1:]:
            dev[c].append((xs[c] - xs[0]).abs().mean())
        mag.append(xs[0].abs().mean())
    torch.cuda.synchronize()
    layer_ms = {c: sum(a.elapsed_time(b) for a, b in ev[c]) / n_layers for c in covs}
    dev = {c: [float(t) for t in v] for c, v in dev.items()}
    mag = [float(t) for t in mag]

    # one layer's kernels, timed one by one at the last coverage
    cmain = covs[-1]
    tp = tm.TileMixPrefill(cu, hq, hkv, d, template, cmain)
    u = torch.empty((T, C), dtype=torch.float16, device="cuda")
    q = torch.empty((T, hq, d), dtype=torch.float16, device="cuda")
    k = torch.empty((T, hkv, d), dtype=torch.float16, device="cuda")
    v = torch.empty_like(k)
    o = torch.empty_like(q)
    xt = x0.clone()

    def timed(fn):
        fn()
        fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    ms = {
        "rms_norm": timed(lambda: tm.tilemix_stack_rms_norm(xt, u, hq, hkv, d, 1e-6)),
        "qkv_projection": timed(lambda: tm.tilemix_stack_qkv(u, wqkv_d[0], q, k, v, hq, hkv, d)),
        "quantize": timed(lambda: tp.quantize_k(k)),
        "prefill": timed(lambda: tp.attend_qinline(q, k, v, o)),
        "out_projection_residual": timed(lambda: tm.tilemix_stack_out_residual(o, wo_d[0], xt, hq, hkv, d)),
    }
    # algorithmic bytes and flops of each kernel
    norm_b = T * C * (4 + 2)
    qkv_f = 2 * T * W * (W + 2 * d) * hkv
    qkv_b = T * C * 2 + (T * C + 2 * T * hkv * d) * 2 + hkv * (W + 2 * d) * W * 2
    out_f = 2 * T * W * W * hkv
    out_b = T * C * 2 + T * C * 8 + hkv * W * W * 2
    quant_b = 3 * T * hkv * d + 4 * hkv * tp.tk  # K only: Q is quantised inside the prefill
    P, P8 = legal_pair_counts(cu, tp.words, hq, hkv)
    attn_roof = 2 * d * (P - P8) / PEAK_F16 + 2 * d * P / PEAK_F16 + 2 * d * P8 / PEAK_I8
    roof = {"rms_norm": norm_b / PEAK_HBM,
            "qkv_projection": max(qkv_f / PEAK_F16, qkv_b / PEAK_HBM),
            "quantize": quant_b / PEAK_HBM,
            "prefill": attn_roof,
            "out_projection_residual": max(out_f / PEAK_F16, out_b / PEAK_HBM)}
    kernels = {}
    for name, f, b in (("rms_norm", 0, norm_b), ("qkv_projection", qkv_f, qkv_b), ("quantize", 0, quant_b),
                       ("out_projection_residual", out_f, out_b)):
        t = ms[name] * 1e-3
        kernels[name] = {"ms": ms[name], "bound": "hbm", "achieved_GBps": b / t / 1e9,
                         "frac": roof[name] / t, "algorithmic_bytes": b}
        if f:
            kernels[name]["tflops"] = f / t / 1e12
            kernels[name]["flop_bound_frac"] = f / PEAK_F16 / t
    kernels["prefill"] = {"ms": ms["prefill"], "bound": "mfma", "frac": attn_roof / (ms["prefill"] * 1e-3)}
    t_roof = sum(roof.values())
    depths = [1, 2, 4, 8, 12, 16, 24, 32]
    return {
        "workload": f"synthetic stack, {n_layers} layers of attention + residual, streams of width {W}",
        "template": template, "layers": n_layers,
        "deviation": {str(c): [round(x, 7) for x in v] for c, v in dev.items()},
        "hidden_mean_abs": [round(x, 5) for x in mag],
        "deviation_at": {str(c): {str(l): v[l - 1] for l in depths if l <= n_layers} for c, v in dev.items()},
        "layer_ms": {str(c): t for c, t in layer_ms.items()},
        "layer_roofline_us": t_roof * 1e6,
        "layer_frac": t_roof / (layer_ms[cmain] * 1e-3),
        "kernels": kernels,
    }


SWEEP_TEMPLATES = ("band", "global", "rowrandom", "alignedsparse", "bigbird", "sptrans")
SWEEP_COVERAGES = (0, 1000, 2500, 5000, 7500, 10000)


def bench_sweep(workload, templates, coverages, steps=20):
    """Coverage sweep of the fused prefill over every template on one
    workload: kernel time, tokens/s, its monotonicity in coverage, and
    MAD(c) = mean |O_c - O_0%| over all fp16 outputs against the same kernel
    without INT8 groups (the analogue of the pages' deviation-by-coverage
    measurement)."""
    import torch
    import mixed_precision_attention_amd as tm
    import synth
    q, k, v, cu, spec = synth.make_workload(workload)
    hq, hkv, d = spec["hq"], spec["hkv"], spec["d"]
    qd, kd, vd = (torch.from_numpy(x).cuda() for x in (q, k, v))
    del q, k, v
    tp = tm.TileMixPrefill(cu, hq, hkv, d, templates[0], 0)
    tp.quantize_k(kd)
    o_ref = torch.empty_like(qd)
    tp.attend_qinline(qd, kd, vd, o_ref)  # 0%: no INT8 group, the same for every template
    out = torch.empty_like(qd)
    tokens = int(cu[-1])
    res = {}
    for template in templates:
        rows = []
        # two passes over the coverages, the better time of each kept:
        # consecutive configurations differ by a few percent, about the
        # spread of one timing
        best = {}
        for _ in range(2):
            for cov in coverages:
                tp.set_routing(template, cov)
                ms = time_in_pipeline(lambda: tp.quantize_k(kd), lambda: tp.attend_qinline(qd, kd, vd, out), steps)
                best[cov] = min(best.get(cov, ms), ms)
        for cov in coverages:
            tp.set_routing(template, cov)
            tp.quantize_k(kd)
            tp.attend_qinline(qd, kd, vd, out)
            ms = best[cov]
            mad = float((out.float() - o_ref.float()).abs().mean())
            P, P8 = legal_pair_counts(cu, tp.words, hq, hkv)
            t_roof = 2 * d * (P - P8) / PEAK_F16 + 2 * d * P / PEAK_F16 + 2 * d * P8 / PEAK_I8
            rows.append({"coverage_bp": cov, "prefill_ms": round(ms, 4), "tokens_per_s": tokens / (ms * 1e-3),
                         "frac": round(t_roof / (ms * 1e-3), 4), "int8_pair_share": round(P8 / P, 4),
                         "mad_vs_0": mad})
        tps = [r["tokens_per_s"] for r in rows]
        res[template] = {"runs": rows,
                         "monotone": all(b >= a for a, b in zip(tps, tps[1:])),
                         "monotone_within_1pct": all(b >= 0.99 * a for a, b in zip(tps, tps[1:])),
                         "mad_monotone": all(b["mad_vs_0"] >= a["mad_vs_0"] for a, b in zip(rows, rows[1:]))}
    return {"workload": workload, "steps": steps, "templates": res}


def bench_lengths(shapes=((32, 1024), (16, 2048), (8, 4096), (4, 8192), (2, 16384)), template="sptrans",
                  coverage=7500, steps=20):
    """Prefill at a fixed 32,768 tokens split into B sequences of L (3B head
    shape: Hq 24, Hkv 8, d 128, outlier channels, SpTrans 75%, Q quantised in
    the kernel): time per attention call in the path's order and the
    coverage-weighted MFMA roofline fraction, to show how the per-unit
    prologue and epilogue weigh at short sequences."""
    import torch
    import mixed_precision_attention_amd as tm
    import synth
    hq, hkv, d = 24, 8, 128
    rows = []
    for B, L in shapes:
        q, k, v, cu = synth.make_qkv([L] * B, hq, hkv, d, outliers=True, seed=0)
        qd, kd, vd = (torch.from_numpy(x).cuda() for x in (q, k, v))
        del q, k, v
        tp = tm.TileMixPrefill(cu, hq, hkv, d, template, coverage)
        out = torch.empty_like(qd)
        ms = min(time_in_pipeline(lambda: tp.quantize_k(kd), lambda: tp.attend_qinline(qd, kd, vd, out), steps)
                 for _ in range(2))
        P, P8 = legal_pair_counts(cu, tp.words, hq, hkv)
        t_roof = 2 * d * (P - P8) / PEAK_F16 + 2 * d * P / PEAK_F16 + 2 * d * P8 / PEAK_I8
        rows.append({"batch": B, "seq_len": L, "prefill_ms": round(ms, 4),
                     "tokens_per_s": B * L / (ms * 1e-3), "frac": round(t_roof / (ms * 1e-3), 4)})
        del qd, kd, vd, out, tp
        torch.cuda.empty_cache()
    return {"tokens": 32768, "hq": hq, "hkv": hkv, "head_dim": d, "template": template,
            "coverage_bp": coverage, "steps": steps, "runs": rows}


def decode_bytes(cu, hq, hkv, d, tq, tk):
    """Algorithmic HBM bytes of one decode step: the INT8 cache (K and V) and
    its scales read once, the routing words, the queries read and the output
    written once, and the split-key workspace written and read once."""
    import numpy as np
    lens = np.diff(np.asarray(cu, dtype=np.int64))
    tokens = int(lens.sum())
    chunks = int(sum(-(-int(L) // 256) for L in lens))
    B = len(lens)
    # `chunks` already sums over the sequences: one record per (chunk, head)
    return (2 * tokens * hkv * d + 2 * hkv * tk * 4 + hkv * tq * 8 + 2 * B * hq * d * 2
            + 2 * hq * chunks * (d + 2) * 4)


def bench_decode(q, k, v, cu, spec, template, coverage, steps, warmup, cpu):
    """One decode step per sequence against the INT8 cache of the workload's
    K and V (the newest token of each sequence is the query)."""
    import numpy as np
    import torch
    import mixed_precision_attention_amd as tm
    import synth
    hq, hkv, d = spec["hq"], spec["hkv"], spec["d"]
    td = tm.TileMixDecode(cu, hq, hkv, d, template, coverage)
    kd, vd = torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda()
    q_new = synth.decode_queries(q, cu)
    qd = torch.from_numpy(q_new).cuda()
    td.fill_cache(kd, vd)
    out = torch.empty((len(cu) - 1, hq, d), dtype=torch.float16, device="cuda")
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        td.step(qd, out)
    torch.cuda.synchronize()
    ref = out.clone()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        td.step(qd, out)
    e1.record(stream)
    torch.cuda.synchronize()
    us_eager = e0.elapsed_time(e1) * 1e3 / steps
    # A step is two short launches; issued one by one from Python the host
    # cannot keep the GPU busy, so the timed figure replays a HIP graph of
    # `per_graph` steps (no memset nodes; each replay is checked against the
    # eager output).
    per_graph = 20
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            for _ in range(per_graph):
                td.step(qd, out)
    stream.wait_stream(side)
    replays = max(1, steps // per_graph)
    for _ in range(2):
        out.zero_()
        graph.replay()
        torch.cuda.synchronize()
        if not torch.equal(out, ref):
            raise SystemExit("decode graph replay differs from the eager step")
    e0.record(stream)
    for _ in range(replays):
        graph.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    if not torch.equal(out, ref):
        raise SystemExit("decode graph replay differs from the eager step")
    us = e0.elapsed_time(e1) * 1e3 / (replays * per_graph)
    steps = replays * per_graph
    nbytes = decode_bytes(cu, hq, hkv, d, td.tq, td.tk)
    achieved = nbytes / (us * 1e-6) / 1e9
    rec = {
        "metric": "decode tokens/s (one new token per sequence, INT8 key/value cache)",
        "value": (len(cu) - 1) / (us * 1e-6), "unit": "tokens/s", "us_per_step": us,
        "us_per_step_eager": us_eager, "steps": steps, "warmup": warmup,
        "config": {"workload": f"decode_{spec['name']}_{template}{coverage // 100}",
                   "cache_lengths": f"{len(cu) - 1}x{int(cu[1] - cu[0])}"
                   if len(set(np.diff(cu))) == 1 else np.diff(cu).tolist(),
                   "hq": hq, "hkv": hkv, "head_dim": d},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM / 1e9, "unit": "GB/s",
                     "frac": achieved * 1e9 / PEAK_HBM, "traffic": None,
                     "algorithmic_bytes": nbytes, "launches": "decode_partial + decode_merge"},
    }
    if cpu:
        import oracle
        t0 = time.perf_counter()
        k_i8, ks, v_i8, vs = oracle.quantize_kv_cache(k, v, cu)
        t_q = time.perf_counter() - t0
        n = min(2, len(cu) - 1)
        sub = np.asarray(cu[:n + 1])
        t1 = time.perf_counter()
        oracle.decode_attention(q_new[:n], k_i8[:sub[-1]], ks, v_i8[:sub[-1]], vs, td.words, sub, hq, hkv)
        t_d = (time.perf_counter() - t1) * int(cu[-1]) / int(sub[-1])
        rec["cpu_baseline"] = {"value": (len(cu) - 1) / t_d, "unit": "tokens/s", "cores": _blas_threads(),
                               "kind": "oracle",
                               "sample": f"decode of the first {n} sequences ({int(sub[-1])} cached "
                                         f"tokens), extrapolated by cached tokens; the cache "
                                         f"quantiser ({t_q:.1f}s) is outside the step"}
    return rec


def _cpu_info():
    """CPUs this process may run on, and the host CPU model."""
    try:
        cpus = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        cpus = os.cpu_count() or 1
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:  # pragma: no cover
        pass
    return cpus, model


def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        return 1


def cpu_baseline(q, k, v, cu, spec, template, coverage, budget_s=20.0, full_headline=False):
    """The oracle, as it stands, on a bounded sample of the workload: the
    full quantiser pass plus sampled work units of the attention,
    extrapolated to the whole batch by legal-pair count."""
    import numpy as np
    import oracle
    threads = _blas_threads()
    t0 = time.perf_counter()
    words, g, n8, nl = oracle.routing_words(np.diff(cu).tolist(), spec["hkv"], template, coverage, 0)
    q_i8, q_s = oracle.quantize_blocks(q, cu, oracle.BLOCK_M)
    k_i8, k_s = oracle.quantize_blocks(k, cu, oracle.BLOCK_N)
    t_prep = time.perf_counter() - t0
    lens = np.diff(cu)
    rng = np.random.default_rng(0)
    units = [(s, h, r) for s in range(len(lens)) for h in range(spec["hq"])
             for r in range(-(-int(lens[s]) // 128))]
    order = rng.permutation(len(units))
    done, pairs, t_attn = [], 0, 0.0
    for i in order:
        s, h, r = units[i]
        t1 = time.perf_counter()
        oracle.prefill_attention(q, k, v, q_i8, k_i8, q_s, k_s, words, cu, spec["hq"], spec["hkv"],
                                 rows=[(s, h, r)])
        t_attn += time.perf_counter() - t1
        L = int(lens[s])
        qpos = np.arange(128 * r, min(128 * r + 128, L))
        pairs += int((qpos + 1).sum())
        done.append((s, h, r))
        if t_attn + t_prep > budget_s:
            break
    total_pairs = sum(int(L) * (int(L) + 1) // 2 for L in lens) * spec["hq"]
    t_total = t_prep + t_attn * total_pairs / pairs
    tokens = int(cu[-1])
    # the whole oracle, unsampled, on the two small configurations
    full = {}
    import synth
    for name in ("tiny", "llama3b_l1k"):
        qs_, ks_, vs_, cs_, sp = synth.make_workload(name)
        t1 = time.perf_counter()
        oracle.run(qs_, ks_, vs_, cs_, sp["hq"], sp["hkv"], sp["template"], sp["coverage_bp"])
        dt = time.perf_counter() - t1
        full[name] = {"seconds": round(dt, 3), "tokens_per_s": int(cs_[-1]) / dt}
    if full_headline:
        # the headline workload's whole oracle, unsampled (minutes of CPU time)
        print("cpu_baseline: the whole headline oracle, unsampled ...", file=sys.stderr, flush=True)
        t1 = time.perf_counter()
        oracle.run(q, k, v, cu, spec["hq"], spec["hkv"], template, coverage)
        dt = time.perf_counter() - t1
        print(f"cpu_baseline: whole headline oracle {dt:.1f} s", file=sys.stderr, flush=True)
        full[spec.get("name", "headline")] = {"seconds": round(dt, 3), "tokens_per_s": tokens / dt}
    cpus, model = _cpu_info()
    # numpy's BLAS pool runs the oracle's matrix products; the rest is one thread
    return {"value": tokens / t_total, "unit": "tokens/s", "cores": int(min(threads, cpus)), "kind": "oracle",
            "cpus_available": cpus, "cpu_model": model, "blas_threads": int(threads),
            "sample": (f"routing + full quantiser pass ({t_prep:.1f}s) + {len(done)} of {len(units)} "
                       f"(sequence, head, query-tile) units of attention ({t_attn:.1f}s, "
                       f"{pairs / total_pairs:.2%} of legal pairs), extrapolated by legal-pair count"),
            "full_oracle": full}


def hw_probes(reps=7):
    """Hardware-rate probes (libtilemix_probes.so, timing-only kernels) behind
    the kernels' cost model: shader clock, vector-ALU issue per wave count,
    the matrix pipe beside the vector ALU, direct HBM/L2->LDS copies, LDS
    reads, and the decode step's HBM read patterns.  Median of `reps` timed
    launches (events on the current stream) after two untimed ones."""
    import ctypes
    import statistics

    import torch

    from mixed_precision_attention_amd import build as _b

    if not os.path.exists(_b.PROBES_PATH):
        raise SystemExit("libtilemix_probes.so is not built (run __graft_entry__.build())")
    lib = ctypes.CDLL(_b.PROBES_PATH)
    vp, ci = ctypes.c_void_p, ctypes.c_int
    lib.tilemix_probe_valu.argtypes = [ci, ci, ci, vp, vp]
    lib.tilemix_probe_coexec.argtypes = [ci, ci, ci, vp, vp]
    lib.tilemix_probe_copy.argtypes = [vp, ci, ci, ci, ci, vp, vp]
    lib.tilemix_probe_lds.argtypes = [ci, ci, ci, vp, vp]
    lib.tilemix_probe_clock.argtypes = [ci, ci, vp, vp]
    lib.tilemix_probe_skeleton.argtypes = [ci, ci, ci, vp, vp]
    lib.tilemix_probe_read.argtypes = [ci, vp, vp, vp, vp]
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    cus = 256

    def timed(launch):
        ts = []
        for r in range(reps + 2):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            rc = launch()
            e1.record()
            if rc != 0:
                raise RuntimeError(f"probe launch failed ({rc})")
            torch.cuda.synchronize()
            if r >= 2:
                ts.append(e0.elapsed_time(e1) * 1e3)
        return statistics.median(ts)

    out = torch.zeros(2048 * 512, dtype=torch.int32, device="cuda")
    res = {}
    # shader clock under an all-CU FMA load
    stamps = torch.zeros(4, dtype=torch.int64, device="cuda")
    if lib.tilemix_probe_clock(cus * 4, 200000, stamps.data_ptr(), stream) != 0:
        raise RuntimeError("clock probe launch failed")
    torch.cuda.synchronize()
    t0, t1, r0, r1 = stamps.tolist()
    clk = (t1 - t0) / max(r1 - r0, 1) * 1e8
    res["shader_clock_ghz"] = round(clk / 1e9, 3)
    # vector-ALU issue: SIMD cycles per instruction, and each wave's issue interval
    iters = 4000
    valu = {}
    for op, name in ((0, "fma"), (1, "exp")):
        for w in (1, 2, 3, 4, 8):
            us = timed(lambda: lib.tilemix_probe_valu(op, cus * w, iters, out.data_ptr(), stream))
            per = us * 1e-6 * clk / (w * iters * 16)
            valu[f"{name}_{w}w"] = {"us": round(us, 1), "simd_cycles_per_instr": round(per, 2),
                                    "wave_issue_interval": round(per * w, 2)}
    res["valu_16_chains"] = valu
    # matrix pipe beside the vector ALU (one wave of each kind per SIMD)
    iters = 4000
    co = {name: round(timed(lambda: lib.tilemix_probe_coexec(mode, cus, iters, out.data_ptr(), stream)), 1)
          for mode, name in ((1, "mfma_only_us"), (2, "fma_only_us"), (0, "both_us"))}
    co["serial_us"] = round(co["mfma_only_us"] + co["fma_only_us"], 1)
    res["mfma_beside_valu"] = co
    # the prefill wave-tile's matrix skeleton (QK int8 -> convert -> pack -> PV f16), no loads:
    # matrix-pipe utilisation at the published peaks (768 cycles per iteration)
    iters = 2000
    sk = {}
    for w in (1, 2):
        for extra in (0, 64, 128):
            us = timed(lambda: lib.tilemix_probe_skeleton(extra, cus * w, iters, out.data_ptr(), stream))
            sk[f"{w}w_extra{extra}"] = round(768 * iters * w / (us * 1e-6 * clk), 3)
    res["skeleton_mfma_utilisation"] = sk
    # direct copies into LDS: bytes per clock per CU with 1..16 1-KB copies in flight per wave
    cp = {}
    for src_mb in (2, 256):
        src = torch.randint(-127, 127, (src_mb << 20,), dtype=torch.int8, device="cuda")
        for batch in (1, 2, 4, 8, 16):
            it = 512 // batch
            us = timed(lambda: lib.tilemix_probe_copy(src.data_ptr(), src_mb * 1024, cus, it, batch,
                                                      out.data_ptr(), stream))
            total = cus * 8 * it * batch * 1024
            cp[f"src{src_mb}MB_batch{batch}"] = round(total / cus / (us * 1e-6 * clk), 1)
        del src
    res["copy_to_lds_bytes_per_clk_per_cu"] = cp
    # LDS reads (8 waves per CU, conflict-free)
    iters = 200
    ld = {}
    for op, name in ((0, "ds_read_b128"), (1, "ds_read_b64_tr_b16")):
        us = timed(lambda: lib.tilemix_probe_lds(op, cus, iters, out.data_ptr(), stream))
        ld[name] = round(8 * 16384 * iters / (us * 1e-6 * clk), 1)
    res["lds_read_bytes_per_clk_per_cu"] = ld
    # the decode step's HBM read patterns over a 2 x 32 MiB int8 cache
    n = 32768 * 8 * 128
    kbuf = torch.randint(-127, 127, (n,), dtype=torch.int8, device="cuda")
    vbuf = torch.randint(-127, 127, (n,), dtype=torch.int8, device="cuda")
    rd = {}
    for pat, name in ((0, "contiguous"), (1, "key_row_per_lane"), (2, "8_lanes_per_key_row"),
                      (3, "8_lanes_per_key_row_head_fastest")):
        us = timed(lambda: lib.tilemix_probe_read(pat, kbuf.data_ptr(), vbuf.data_ptr(), out.data_ptr(), stream))
        rd[name] = {"us": round(us, 2), "tb_per_s": round(2 * n / us / 1e6, 2)}
    res["decode_read_patterns_64MiB"] = rd
    res["note"] = ("cycles at the measured shader clock; launches timed with events, so each time "
                   "includes a few microseconds of launch latency")
    return res


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="llama3b_l4k")
    ap.add_argument("--template", default=None)
    ap.add_argument("--coverage", type=int, default=None, help="INT8 coverage in basis points")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true",
                    help="skip the decode step over the INT8 key/value cache")
    ap.add_argument("--decode-steps", type=int, default=200)
    ap.add_argument("--no-fp8", action="store_true",
                    help="skip the three-path (FP16/FP8/INT8) prefill leg")
    ap.add_argument("--no-adaptive", action="store_true",
                    help="skip the adaptive-routing leg (importance statistic + prefill under its words)")
    ap.add_argument("--no-sweep", action="store_true",
                    help="skip the coverage sweep over every template at L=8192 (time and MAD by coverage)")
    ap.add_argument("--sweep-workload", default="llama3b_l8k")
    ap.add_argument("--no-depth", action="store_true",
                    help="skip the synthetic multi-layer stack (deviation by depth)")
    ap.add_argument("--depth-layers", type=int, default=32)
    ap.add_argument("--cpu-budget", type=float, default=20.0)
    ap.add_argument("--cpu-full", action="store_true",
                    help="also time the headline workload's whole oracle, unsampled (minutes of CPU time)")
    ap.add_argument("--no-exposure", action="store_true",
                    help="skip the importance-exposure probe of the SpTrans and adaptive layouts")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="only run a plain device-to-device copy of this many bytes 5 times "
                         "(calibrates rocprofv3 FETCH_SIZE / WRITE_SIZE) and exit")
    ap.add_argument("--write-traffic", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV",
                                                          "COPY_WRITE_CSV"),
                    help="no GPU: turn four rocprofv3 --pmc counter_collection.csv files (the prefill "
                         "run's FETCH_SIZE and WRITE_SIZE, then the --copy-bytes run's) into "
                         "profiles/prefill_<workload>_traffic.json and exit")
    ap.add_argument("--copy-size", type=int, default=512 << 20,
                    help="bytes the --copy-bytes run copied (for --write-traffic)")
    ap.add_argument("--length-sweep", action="store_true",
                    help="run only the sequence-length sweep (32,768 tokens as 32x1k ... 2x16k) and print it "
                         "as one JSON line")
    ap.add_argument("--hw-probes", action="store_true",
                    help="run only the hardware-rate probes (libtilemix_probes.so) and print their "
                         "results as one JSON line")
    ap.add_argument("--profile-command", default="",
                    help="command line recorded in the --write-traffic summary")
    args = ap.parse_args(argv)

    if args.write_traffic:
        return write_traffic(args)

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): the TileMix path has no "
              "cross-GPU work; splitting it across GPUs by KV head (or by query-tile rows for one long "
              "sequence) is a design note, not implemented.", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import mixed_precision_attention_amd as tm
    import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1

    if args.hw_probes:
        print(json.dumps({"hw_probes": hw_probes()}), flush=True)
        return 0

    if args.length_sweep:
        print(json.dumps({"length_sweep": bench_lengths()}), flush=True)
        return 0

    if args.copy_bytes:
        n = args.copy_bytes // 16 * 16
        src = torch.ones(n // 4, dtype=torch.int32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n, "launches": 5}), flush=True)
        return 0

    q, k, v, cu, spec = synth.make_workload(args.workload)
    template = args.template or spec["template"]
    coverage = spec["coverage_bp"] if args.coverage is None else args.coverage
    hq, hkv, d = spec["hq"], spec["hkv"], spec["d"]

    t0 = time.perf_counter()
    tp = tm.TileMixPrefill(cu, hq, hkv, d, template, coverage)
    host_build_ms = (time.perf_counter() - t0) * 1e3
    qd, kd, vd = (torch.from_numpy(x).cuda() for x in (q, k, v))
    out = torch.empty_like(qd)
    stream = torch.cuda.current_stream()

    for _ in range(args.warmup):
        tp.quantize_k(kd)
        tp.attend_qinline(qd, kd, vd, out)
    torch.cuda.synchronize()

    K = args.steps
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    start.record(stream)
    for _ in range(K):
        tp.quantize_k(kd)
        tp.attend_qinline(qd, kd, vd, out)
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = start.elapsed_time(end)
    # the same K steps again with an event around each kernel, for the
    # breakdown (kept out of the loop above so that they add nothing to it)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    for i in range(K):
        ev[i][0].record(stream)
        tp.quantize_k(kd)
        ev[i][1].record(stream)
        tp.attend_qinline(qd, kd, vd, out)
        ev[i][2].record(stream)
    torch.cuda.synchronize()
    quant_ms = sum(e[0].elapsed_time(e[1]) for e in ev) / K
    attn_ms = sum(e[1].elapsed_time(e[2]) for e in ev) / K
    ms_per_step = total_ms / K
    tokens = int(cu[-1])
    value = tokens / (ms_per_step * 1e-3)

    P, P8 = legal_pair_counts(cu, tp.words, hq, hkv)
    t_roof = 2 * d * (P - P8) / PEAK_F16 + 2 * d * P / PEAK_F16 + 2 * d * P8 / PEAK_I8
    frac = t_roof / (attn_ms * 1e-3)
    flops_eq = t_roof * PEAK_F16
    achieved = flops_eq / (attn_ms * 1e-3) / 1e12
    # the same step as two passes over Q (quantiser for Q and K, then the
    # prefill reading Q's INT8 codes), timed right after
    split_prefill_ms = time_in_pipeline(lambda: tp.quantize(qd, kd), lambda: tp.attend(qd, kd, vd, out), K)
    split_quant_ms = time_in_pipeline(lambda: None, lambda: tp.quantize(qd, kd), K)
    traffic = None
    rec = traffic_record(os.path.join(ROOT, "profiles", f"prefill_{args.workload}_traffic.json"))
    if rec is not None:
        traffic = rec["hbm_bytes_per_launch"]

    result = {
        "metric": METRIC,
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16+i8",
        "data": "synthetic",
        "config": {"workload": f"{args.workload}_{template}{coverage // 100}",
                   "seqlens": spec["seqlens"] if len(set(spec["seqlens"])) > 1 else
                   f"{len(spec['seqlens'])}x{spec['seqlens'][0]}",
                   "hq": hq, "hkv": hkv, "head_dim": d, "template": template,
                   "coverage_bp": coverage, "tokens": tokens},
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": PEAK_F16 / 1e12,
                     "unit": "TFLOP/s", "frac": frac, "traffic": traffic},
        "breakdown": {"quantize_ms": quant_ms, "prefill_ms": attn_ms,
                      "legal_pairs": P, "int8_pairs": P8, "int8_pair_share": P8 / P,
                      "int8_tops": 2 * d * P8 / (attn_ms * 1e-3) / 1e12,
                      "fp16_tflops": 2 * d * (2 * P - P8) / (attn_ms * 1e-3) / 1e12,
                      "roofline_us": t_roof * 1e6, "host_build_ms": host_build_ms,
                      "wall_s": wall,
                      "split_path": {"quantize_ms": split_quant_ms, "prefill_ms": split_prefill_ms,
                                     "ms_per_step": split_quant_ms + split_prefill_ms,
                                     "prefill_frac": t_roof / (split_prefill_ms * 1e-3)}},
    }
    if not args.no_fp8:
        result["fp8"] = bench_fp8(qd, kd, vd, cu, hq, hkv, d, template, [(5000, 2500), (0, 7500)], 20)
    if not args.no_adaptive:
        result["adaptive"] = bench_adaptive(tp, qd, kd, vd, cu, hq, hkv, d, coverage, 20)
    if not args.no_sweep:
        # the headline workload's SpTrans sweep, then every template at L=8192
        result["sweep_headline"] = bench_sweep(args.workload, (template,), SWEEP_COVERAGES)
        result["sweep"] = bench_sweep(args.sweep_workload, SWEEP_TEMPLATES, SWEEP_COVERAGES)
    if not args.no_depth:
        result["depth"] = bench_depth(cu, hq, hkv, d, template, [2500, coverage], args.depth_layers)
    if not args.no_exposure:
        result["exposure_probe"] = bench_exposure()
    if not args.no_decode:
        spec_named = dict(spec, name=args.workload)
        result["decode"] = bench_decode(q, k, v, cu, spec_named, template, coverage, args.decode_steps,
                                        20, not args.no_cpu_baseline)
    if any(k in result for k in ("fp8", "adaptive", "sweep", "depth", "decode", "exposure_probe")):
        # the headline kernel again, after the legs' seconds of sustained load
        tp.set_routing(template, coverage)  # the adaptive leg leaves its own words
        result["breakdown"]["prefill_ms_after_legs"] = time_in_pipeline(
            lambda: tp.quantize_k(kd), lambda: tp.attend_qinline(qd, kd, vd, out), K)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(q, k, v, cu, dict(spec, name=args.workload), template, coverage,
                                              args.cpu_budget, args.cpu_full)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
