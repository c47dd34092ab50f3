"""Benchmark of the int4 KV-cache hot path on one MI355X.

One step = the whole hot path over one batch of synthetic input:
  1. encode  the Qwen2.5-1.5B-shaped prefix (28 layers x {K,V} x 2 KV heads x
             4096 tokens, D=128: 458,752 vectors) with SRFT;
  2. decode  those codes back to fp16;
  3. a decode step on the int4 cache (batch 64, 8 query heads over 2 KV
     heads, D=128, 32768 cached tokens): append one token per sequence for K
     and V with kvq_encode, then int4 decode-step attention over 32769 tokens.
Steps rotate over four prefix batches and two int4 caches, so the working
set (about 1.8 GB) is far beyond the 256 MB Infinity Cache.  The fp16-cache
comparator (same attention over an unquantized cache) is timed in its own
loop right after the timed region, and so is the D=256 leg: encode and
decode of the Gemma-3-1B-shaped prefix (212,992 vectors) with SRFT and SRHT
(field "d256"), the code-format variants (field "formats": int4 in groups
of 16, int8 in groups of 32 and 16; encode and decode of the Qwen prefix and
the decode-step attention over a cache in that format), and the head sizes
that are not powers of two (field "mixed_radix": encode and decode of the
same prefix shape at D=96 and D=80 with the mixed-radix SRFT).

Prints ONE JSON line.  `value` is the encode throughput (Mvec/s) over the
timed region, measured with HIP events at the phase boundaries on the stream
the kernels run on; ns/vec, GB/s and the attention microseconds per step are
extra fields.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0       # MI355X HBM3E, 8 TB/s

# HBM bytes per launch from rocprofv3 FETCH_SIZE / WRITE_SIZE passes of this
# bench, scaled by what the same counters read for a 512 MiB copy (FETCH_SIZE
# reads half the bytes fetched, WRITE_SIZE all bytes written).  Valid only for
# the kernel sources they were taken on (sha256 prefix of the listed files);
# reported as null once those change.
TRAFFIC = {
    "attn": {"files": ("kvq_attn.hip", "kvq_attn_kernels.hpp", "kvq_device.hpp"), "sha256": "ede60afeb8f82f6d",
             "bytes": (295661.2 + 2130.0) * 2 * 1024 + (4362.1 + 128.0) * 1024},
    "encode": {"files": ("kvq_codec.hip", "kvq_device.hpp"), "sha256": "6bc5d18ba8a893be",
               "bytes": 57688.2 * 2 * 1024 + 32256.0 * 1024},
    "decode": {"files": ("kvq_codec.hip", "kvq_device.hpp"), "sha256": "6bc5d18ba8a893be",
               "bytes": 16451.5 * 2 * 1024 + 114715.9 * 1024},
}


def measured_traffic(which: str):
    """Counter-measured HBM bytes of one launch, or None if the kernel's
    sources changed since the counters were taken."""
    import hashlib
    t = TRAFFIC[which]
    h = hashlib.sha256()
    for f in t["files"]:
        with open(os.path.join(ROOT, "kv_cache_int4_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return round(t["bytes"]) if h.hexdigest()[:16] == t["sha256"] else None


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-bulk", action="store_true", help="skip the Mistral-shaped bulk leg (39 GB of HBM)")
    ap.add_argument("--sets", type=int, default=4, help="prefix batches rotated over")
    ap.add_argument("--profile-marks", action="store_true",
                    help="bracket the timed steps with marker kernels and add a calibration copy "
                         "of known size, for --trace-summary of a rocprofv3 run")
    ap.add_argument("--clock-windows", type=int, default=0, metavar="N",
                    help="after an idle pause, time N windows of 20 decode-step attention calls, read the "
                         "shader clock after each, print them as a Markdown table, then exit")
    ap.add_argument("--trace-summary", metavar="CSV",
                    help="summarize a rocprofv3 kernel_trace.csv or counter_collection.csv written "
                         "by a --profile-marks run, then exit")
    return ap.parse_args()


CALIB_BYTES = 512 << 20      # calibration copy: 512 MiB read + 512 MiB written
MARK_CYCLES = 1000           # marker kernel length (torch.cuda._sleep)


def trace_summary(path: str) -> str:
    """Per-kernel rows of the dispatches between the two marker kernels of a
    --profile-marks run, as a Markdown table.

    A kernel trace gives calls and durations (us) per (kernel, grid); a
    counter collection gives the mean per dispatch of each counter (FETCH_SIZE
    and WRITE_SIZE are KiB), and for the calibration copy the ratio of the
    counter to the bytes it moves."""
    import csv
    rows = list(csv.DictReader(open(path)))
    if not rows:
        return "(empty)"
    key = "Dispatch_Id" if "Dispatch_Id" in rows[0] else "Correlation_Id"
    rows.sort(key=lambda r: int(r[key]))
    # a counter collection has a row per (dispatch, counter[, partial]): the
    # window is taken by dispatch id, strictly between the first and the
    # last marker dispatch
    marks = sorted({int(r[key]) for r in rows if "sleep" in r["Kernel_Name"] or "spin" in r["Kernel_Name"]})
    if len(marks) < 2:
        raise SystemExit(f"{path}: fewer than two marker dispatches")
    lo, hi = marks[0], marks[-1]
    gk = "Grid_Size" if "Grid_Size" in rows[0] else "Grid_Size_X"
    window = [r for r in rows if lo < int(r[key]) < hi]
    # the calibration copy is the last kernel before the closing marker
    calib_id = max(int(r[key]) for r in window)

    def short(r):
        if int(r[key]) == calib_id:
            return "calibration copy (512 MiB)"
        n = r["Kernel_Name"].replace("(anonymous namespace)::", "")
        n = n[5:] if n.startswith("void ") else n
        return n.split("(")[0].replace("kvq::", "")

    out = []
    if "Counter_Name" in rows[0]:
        acc = {}
        for r in window:
            k = (short(r), int(r[gk]), r["Counter_Name"])
            d = acc.setdefault(k, {})
            d.setdefault(int(r[key]), 0.0)
            d[int(r[key])] += float(r["Counter_Value"])
        out.append("| kernel | grid | counter | dispatches | mean per dispatch | calibration ratio |")
        out.append("|---|---|---|---|---|---|")
        for (name, grid, ctr), d in sorted(acc.items()):
            mean = sum(d.values()) / len(d)
            ratio = ""
            if name.startswith("calibration") and ctr in ("FETCH_SIZE", "WRITE_SIZE"):
                ratio = f"{mean * 1024 / CALIB_BYTES:.4f}"
            out.append(f"| {name} | {grid} | {ctr} | {len(d)} | {mean:.1f} | {ratio} |")
    else:
        acc = {}
        for r in window:
            k = (short(r), int(r[gk]))
            acc.setdefault(k, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
        out.append("| kernel | grid (work-items) | calls | avg us | min us | max us |")
        out.append("|---|---|---|---|---|---|")
        for (name, grid), v in sorted(acc.items(), key=lambda kv: -sum(kv[1])):
            out.append(f"| {name} | {grid} | {len(v)} | {sum(v) / len(v):.2f} | {min(v):.2f} | {max(v):.2f} |")
    return "\n".join(out)


def host_info() -> dict:
    """CPU model and core counts of the host the oracle runs on."""
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_model": model, "nproc": os.cpu_count(),
            "cpus_allowed": len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else None}


def cpu_baseline(n_vec: int = 458752):
    """The CPU oracle as it stands, pinned to one host core (numpy with one
    BLAS/OpenMP thread; pocketfft is single-threaded): encode and decode of
    the Qwen prefix workload (by default all 458,752 vectors of one step),
    and the decode-step attention over the int4 cache for one sequence of
    the batch of 64 (D=128, 8 query heads over 2 KV heads, 32769 tokens),
    extrapolated to the batch.  About 5-10 s of work."""
    import numpy as np
    import oracle as O
    from kv_cache_int4_amd import workloads as W
    host = host_info()
    pinned = None
    if hasattr(os, "sched_setaffinity"):
        allowed = sorted(os.sched_getaffinity(0))
        pinned = allowed[0]
        os.sched_setaffinity(0, {pinned})
    cfg = W.CONFIGS["qwen"]
    T = 4096
    nb = min(cfg.B, max(1, -(-n_vec // (cfg.H * T))))
    x, lam = W.prefix_inputs(W.Config(cfg.name, cfg.D, nb, cfg.H, T, cfg.law, cfg.index))
    xs = x.numpy().reshape(-1, cfg.D)[:n_vec]
    lv = np.repeat(lam.numpy()[:, :, None, :], T, axis=2).reshape(-1, cfg.D)[:n_vec]
    signs = O.plan_signs(cfg.D, O.SRFT, cfg.sign_seed)
    t0 = time.perf_counter()
    codes, scales, _ = O.encode(xs, lv, O.SRFT, signs)
    t1 = time.perf_counter()
    O.decode(codes, scales, lv, O.SRFT, signs)
    t2 = time.perf_counter()
    # decode-step attention, one sequence: its K and V caches encoded by the
    # oracle, then attention over all 32769 tokens (timed), times 64
    dc = W.CONFIGS["decode"]
    L = dc.T + 1
    k16, v16, lam_k, lam_v, q = W.decode_inputs(1, dc.H, dc.Hq, L, dc.D, dc.data_seed)
    ks = O.plan_signs(dc.D, O.SRFT, dc.sign_seed)
    kc, ksc, _ = O.encode(k16.numpy(), lam_k.numpy()[None, :, None, :], O.SRFT, ks)
    vc, vsc, _ = O.encode(v16.numpy(), lam_v.numpy()[None, :, None, :], O.SRFT, ks)
    t3 = time.perf_counter()
    O.attention_int4(q.numpy(), kc, ksc, lam_k.numpy(), vc, vsc, lam_v.numpy(), L, 1 / math.sqrt(dc.D), O.SRFT,
                     ks)
    t4 = time.perf_counter()
    if pinned is not None:
        os.sched_setaffinity(0, set(allowed))
    return {
        "value": n_vec / (t1 - t0) / 1e6,
        "unit": "Mvec/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"{n_vec} vectors of the Qwen2.5-1.5B prefix workload (D=128, SRFT), numpy float64 oracle "
                  f"pinned to host core {pinned}: encode {(t1 - t0):.2f} s, decode {(t2 - t1):.2f} s; "
                  f"decode-step attention over the int4 cache for 1 of the 64 sequences "
                  f"({(t4 - t3):.2f} s), times 64",
        "decode_Mvec_s": n_vec / (t2 - t1) / 1e6,
        "attn_us_per_step_extrapolated": round((t4 - t3) * 64 * 1e6, 1),
        "host": host,
    }


def timed_loop(torch, stream, fn, n, warm=3, reps=3):
    """Microseconds per call of fn(i) over n back-to-back calls, with HIP
    events on the kernels' stream: the median of reps such windows (a window
    of a few hundred microseconds moves by 5-10% with the clock the power
    manager picks for it)."""
    for i in range(warm):
        fn(i)
    out = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(n):
            fn(i)
        e1.record(stream)
        torch.cuda.synchronize()
        out.append(e0.elapsed_time(e1) / n * 1e3)
    return sorted(out)[len(out) // 2]


def graph_loop(torch, stream, fn, n_calls=20, reps=10):
    """GPU microseconds per call of fn(): n_calls calls captured in one HIP
    graph, replayed reps times (the median replay), so that the host's own
    per-call work does not pace the launches."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(n_calls):
            fn()
    torch.cuda.synchronize()
    return timed_loop(torch, stream, lambda i: g.replay(), 1, warm=2, reps=reps) / n_calls


def small_leg(K, W, torch, stream, dev, n):
    """The single-K-tensor round trip (2 KV heads x 256 tokens, D=128, 512
    vectors): latency bound, reported as microseconds per call, both as
    back-to-back calls from Python (paced by the host's per-call work) and
    from a captured graph (the GPU's time per call, launch gaps included)."""
    cfg = W.CONFIGS["small"]
    x, lam = W.prefix_inputs(cfg, dev)
    plan = K.Plan(cfg.D, 32, "srft", cfg.sign_seed)
    B, H, T, D = x.shape
    codes = torch.empty((B, H, T, D // 2), dtype=torch.uint8, device=dev)
    scales = torch.empty((B, H, T, D // 32), dtype=torch.float16, device=dev)
    y = torch.empty_like(x)
    enc = timed_loop(torch, stream, lambda i: K.encode(plan, x, lam, codes, scales), n)
    dec = timed_loop(torch, stream, lambda i: K.decode(plan, codes, scales, lam, y), n)
    rt = timed_loop(torch, stream, lambda i: (K.encode(plan, x, lam, codes, scales),
                                              K.decode(plan, codes, scales, lam, y)), n)
    enc_g = graph_loop(torch, stream, lambda: K.encode(plan, x, lam, codes, scales))
    dec_g = graph_loop(torch, stream, lambda: K.decode(plan, codes, scales, lam, y))
    rt_g = graph_loop(torch, stream, lambda: (K.encode(plan, x, lam, codes, scales),
                                              K.decode(plan, codes, scales, lam, y)), n_calls=10)
    return {"workload": "single K tensor, 2 KV heads x 256 tokens, D=128, SRFT (512 vectors)",
            "encode_us": round(enc, 2), "decode_us": round(dec, 2), "round_trip_us": round(rt, 2),
            "graph_encode_us": round(enc_g, 2), "graph_decode_us": round(dec_g, 2),
            "graph_round_trip_us": round(rt_g, 2)}


def mistral_leg(K, W, torch, stream, dev, n_rep):
    """The Mistral-7B-shaped bulk path: 64 full-size calls (32 layers x {K,V};
    each B=16, H=8, T=8192, D=128, Student-t(3) values: 1,048,576 vectors and
    268 MB of fp16 per call, 17.2 GB in all), encoded into 64 caches, then the
    whole cache decoded back to fp16 with 64 calls.  Each pass of 64 calls is
    timed with HIP events, n_rep times; the caches and outputs (39 GB in all)
    stay in HBM."""
    cfg = W.CONFIGS["mistral"]
    D, B, H, T = cfg.D, cfg.B, cfg.H, cfg.T
    plan = K.Plan(D, 32, "srft", cfg.sign_seed)
    xs, lams, cs, ss, ys = [], [], [], [], []
    for call in range(64):
        layer, kv = divmod(call, 2)
        # the batch of 16 sequences as 16 x 8 heads of the law, seeded per call
        xs.append(W.student_t3(B * H, T, D, cfg.data_seed, dev, layer, kv).view(B, H, T, D))
        lams.append(W.lognormal_lambda((H, D), cfg.lambda_seed, dev, 0.3, layer, kv))
        cs.append(torch.empty((B, H, T, D // 2), dtype=torch.uint8, device=dev))
        ss.append(torch.empty((B, H, T, D // 32), dtype=torch.float16, device=dev))
        ys.append(torch.empty((B, H, T, D), dtype=torch.float16, device=dev))
    torch.cuda.synchronize()
    nvec = 64 * B * H * T
    nbytes = nvec * (2 * D + D // 2 + 2 * (D // 32))

    def enc_all(_):
        for c in range(64):
            K.encode(plan, xs[c], lams[c], cs[c], ss[c])

    def dec_all(_):
        for c in range(64):
            K.decode(plan, cs[c], ss[c], lams[c], ys[c])

    enc = timed_loop(torch, stream, enc_all, n_rep, warm=1)
    dec = timed_loop(torch, stream, dec_all, n_rep, warm=1)
    res = {
        "workload": "Mistral-7B-shaped bulk path: 64 calls (32 layers x {K,V}) of B=16, H=8, T=8192, D=128, "
                    "Student-t(3), SRFT, group 32; encode all, then decode the whole cache",
        "vectors": nvec, "bytes_per_pass": nbytes,
        "encode_ms_per_64_calls": round(enc / 1e3, 4), "encode_frac_hbm": round(nbytes / enc / 1e3 / HBM_PEAK_GBS, 4),
        "encode_Gvec_s": round(nvec / enc / 1e3, 2),
        "decode_ms_per_64_calls": round(dec / 1e3, 4), "decode_frac_hbm": round(nbytes / dec / 1e3 / HBM_PEAK_GBS, 4),
        "decode_Gvec_s": round(nvec / dec / 1e3, 2),
    }
    del xs, cs, ss, ys
    torch.cuda.synchronize()
    return res


def attn256_leg(K, W, torch, stream, dev, n):
    """The decode step at Gemma-3 1B's head shape: batch 64, 4 query heads
    over 1 KV head, D=256, 32768 cached tokens; append one token (K and V in
    one call over the stacked [2B, 1, Tcap] caches), then int4 attention over
    32769 tokens, timed as whole steps back to back, against the same
    attention over the fp16 cache."""
    dc = W.CONFIGS["decode256"]
    B, Hkv, Hq, D, T0 = dc.B, dc.H, dc.Hq, dc.D, dc.T
    L, Tcap = T0 + 1, T0 + 256
    plan = K.Plan(D, 32, "srft", dc.sign_seed)
    k16, v16, lam_k, lam_v, q = W.decode_inputs(B, Hkv, Hq, Tcap, D, dc.data_seed, dev)
    kvc = torch.empty((2 * B, Hkv, Tcap, D // 2), dtype=torch.uint8, device=dev)
    kvs = torch.empty((2 * B, Hkv, Tcap, D // 32), dtype=torch.float16, device=dev)
    K.encode(plan, k16[:, :, :T0], lam_k, kvc[:B], kvs[:B], 0)
    K.encode(plan, v16[:, :, :T0], lam_v, kvc[B:], kvs[B:], 0)
    kv_new = torch.cat([k16[:, :, T0:T0 + 1], v16[:, :, T0:T0 + 1]]).contiguous()
    lam_kv = torch.cat([lam_k.expand(B, Hkv, D), lam_v.expand(B, Hkv, D)]).contiguous()
    ws = torch.empty(K.attn_workspace_size(D, B, Hq, L), dtype=torch.uint8, device=dev)
    out = torch.empty((B, Hq, D), dtype=torch.float16, device=dev)
    sm = 1.0 / math.sqrt(D)
    kc, ks, vc, vs = kvc[:B], kvs[:B], kvc[B:], kvs[B:]

    def attn(i):
        K.attn_decode(plan, q, kc, ks, lam_k, vc, vs, lam_v, L, sm, out, ws)

    def step(i):
        K.encode(plan, kv_new, lam_kv, kvc, kvs, T0)
        attn(i)

    # whole steps back to back (the host queues the next append while the
    # attention runs, as in a decode loop); the append's share of a step is
    # the step less the attention alone.  An append timed on its own from
    # Python is paced by the host (about 10 us per call), not the GPU.
    stp = timed_loop(torch, stream, step, n)
    att = timed_loop(torch, stream, attn, n)
    app = max(stp - att, 0.0)
    app_g = graph_loop(torch, stream, lambda: K.encode(plan, kv_new, lam_kv, kvc, kvs, T0))
    f16 = timed_loop(torch, stream, lambda i: K.attn_decode_f16(q, k16, v16, L, sm, out, ws), max(5, n // 2))
    ab = B * Hkv * L * 2 * (D // 2 + 2 * (D // 32))
    fb = B * Hkv * L * 2 * 2 * D
    return {
        "workload": "decode step at Gemma-3-1B head shape: batch 64, Hq 4 / Hkv 1, D=256, 32768 cached tokens + 1 "
                    "appended, SRFT, group 32",
        "append_us": round(app, 2), "append_graph_us": round(app_g, 2), "int4_attn_us": round(att, 2),
        "int4_us_per_step": round(stp, 2),
        "int4_attn_bytes": ab, "int4_attn_frac_hbm": round(ab / att / 1e3 / HBM_PEAK_GBS, 4),
        "fp16_us_per_step": round(f16, 2), "fp16_frac_hbm": round(fb / f16 / 1e3 / HBM_PEAK_GBS, 4),
        "int4_over_fp16": round(stp / f16, 4),
    }


def d256_setup(K, W, torch, dev, n_sets):
    """Input batches of the Gemma-3-1B-shaped prefix (26 layers x {K,V} x 1
    KV head x 4096 tokens, D=256: 212,992 vectors), with code, scale and
    output buffers."""
    cfg = W.CONFIGS["gemma"]
    D = cfg.D
    sets = []
    for i in range(n_sets):
        c = W.Config(cfg.name, D, cfg.B, cfg.H, cfg.T, cfg.law, cfg.index + 10 * i)
        x, lam = W.prefix_inputs(c, dev)
        codes = torch.empty((cfg.B, cfg.H, cfg.T, D // 2), dtype=torch.uint8, device=dev)
        scales = torch.empty((cfg.B, cfg.H, cfg.T, D // 32), dtype=torch.float16, device=dev)
        sets.append((x, lam, codes, scales, torch.empty_like(x)))
    return cfg, sets


def d256_leg(K, torch, stream, cfg, sets, n):
    """Encode and decode of the D=256 batches with SRFT and with SRHT, each
    timed over n launches with HIP events on the kernels' stream, rotating
    over the batches (beyond the Infinity Cache)."""
    D = cfg.D
    nbytes = cfg.vectors * (2 * D + D // 2 + 2 * (D // 32))         # 656 B / vector
    ns = len(sets)

    def timed(fn):
        return timed_loop(torch, stream, fn, n)

    res = {"workload": "Gemma-3-1B-shaped prefix (26 layers x {K,V} x 1 KV head x 4096 tokens, D=256, "
                       "group 32)", "vectors": cfg.vectors, "bytes_per_call": nbytes}
    for rot in ("srft", "srht"):
        plan = K.Plan(D, 32, rot, cfg.sign_seed)
        enc = timed(lambda i: K.encode(plan, *sets[i % ns][:4]))
        dec = timed(lambda i: K.decode(plan, sets[i % ns][2], sets[i % ns][3], sets[i % ns][1], sets[i % ns][4]))
        res[rot] = {
            "encode_us": round(enc, 2), "encode_GB_s": round(nbytes / enc / 1e3, 1),
            "encode_frac_hbm": round(nbytes / enc / 1e3 / HBM_PEAK_GBS, 4),
            "decode_us": round(dec, 2), "decode_GB_s": round(nbytes / dec / 1e3, 1),
            "decode_frac_hbm": round(nbytes / dec / 1e3 / HBM_PEAK_GBS, 4),
        }
    return res


FORMATS = (("int4-g16", 4, 16), ("int8-g32", 8, 32), ("int8-g16", 8, 16))


def formats_leg(K, torch, stream, cfg, sets, dc, k16, v16, lam_k, lam_v, q, L, sm, n):
    """The code-format variants (int4 in groups of 16, int8 in groups of 32
    and 16) on the same work: encode and decode of the Qwen prefix batches,
    and the decode-step attention over a cache in that format, each timed
    over n launches with HIP events on the kernels' stream."""
    D = cfg.D
    B, Hkv, Hq = dc.B, dc.H, q.shape[1]
    T0, Tcap = L - 1, k16.shape[2]
    ns = len(sets)
    out = torch.empty((B, Hq, D), dtype=torch.float16, device=q.device)
    ws = torch.empty(K.attn_workspace_size(D, B, Hq, L), dtype=torch.uint8, device=q.device)

    def timed(fn):
        return timed_loop(torch, stream, fn, n)

    res = {}
    for name, bits, G in FORMATS:
        plan = K.Plan(D, G, "srft", cfg.sign_seed, bits=bits)
        cb, nsc = plan.code_bytes, D // G
        bufs = [(torch.empty((cfg.B, cfg.H, cfg.T, cb), dtype=torch.uint8, device=q.device),
                 torch.empty((cfg.B, cfg.H, cfg.T, nsc), dtype=torch.float16, device=q.device)) for _ in range(ns)]
        enc = timed(lambda i: K.encode(plan, sets[i % ns][0], sets[i % ns][1], *bufs[i % ns]))
        dec = timed(lambda i: K.decode(plan, *bufs[i % ns], sets[i % ns][1], sets[i % ns][4]))
        del bufs
        kc = torch.empty((B, Hkv, Tcap, cb), dtype=torch.uint8, device=q.device)
        ksc = torch.empty((B, Hkv, Tcap, nsc), dtype=torch.float16, device=q.device)
        vc, vsc = torch.empty_like(kc), torch.empty_like(ksc)
        K.encode(plan, k16[:, :, :L], lam_k, kc, ksc, 0)
        K.encode(plan, v16[:, :, :L], lam_v, vc, vsc, 0)
        att = timed(lambda i: K.attn_decode(plan, q, kc, ksc, lam_k, vc, vsc, lam_v, L, sm, out, ws))
        del kc, ksc, vc, vsc
        vb = 2 * D + cb + 2 * nsc                    # bytes per vector, encode or decode
        ab = B * Hkv * L * 2 * (cb + 2 * nsc)        # K and V codes + scales per step
        nv = cfg.vectors
        res[name] = {
            "encode_us": round(enc, 2), "encode_frac_hbm": round(nv * vb / enc / 1e3 / HBM_PEAK_GBS, 4),
            "decode_us": round(dec, 2), "decode_frac_hbm": round(nv * vb / dec / 1e3 / HBM_PEAK_GBS, 4),
            "attn_us": round(att, 2), "attn_bytes": ab, "attn_frac_hbm": round(ab / att / 1e3 / HBM_PEAK_GBS, 4),
        }
    torch.cuda.synchronize()
    return res


MIXED = (("d96", "int4-g32", 4, 32), ("d96", "int4-g16", 4, 16), ("d80", "int4-g16", 4, 16),
         ("d96", "int8-g32", 8, 32), ("d80", "int8-g16", 8, 16))


def mfma_leg(K, torch, stream, cfg, sets, n):
    """The D=128 SRFT encoder with its DFT on the matrix cores (plan option)
    against the VALU encoder, on the same Qwen prefix batches, each timed
    over n launches with HIP events on the kernels' stream."""
    D = cfg.D
    ns = len(sets)
    nbytes = cfg.vectors * (2 * D + D // 2 + 2 * (D // 32))
    res = {"workload": "Qwen2.5-1.5B-shaped prefix encode (458,752 vectors, D=128, SRFT, group 32)"}
    for name, mfma in (("valu_fft", False), ("mfma_dft", True)):
        plan = K.Plan(D, 32, "srft", cfg.sign_seed, mfma=mfma)
        us = timed_loop(torch, stream, lambda i: K.encode(plan, *sets[i % ns][:4]), n)
        res[name] = {"encode_us": round(us, 2), "encode_frac_hbm": round(nbytes / us / 1e3 / HBM_PEAK_GBS, 4)}
    return res


def mixed_leg(K, W, torch, stream, dev, n_sets, n):
    """Head sizes that are not powers of two (the mixed-radix SRFT): encode
    and decode of the 28-layer prefix shape (28 layers x {K,V} x 2 KV heads x
    4096 tokens = 458,752 vectors) at D=96 and D=80, per code format, each
    timed over n launches with HIP events on the kernels' stream, rotating
    over n_sets input batches."""

    def timed(fn):
        return timed_loop(torch, stream, fn, n)

    res = {"workload": "prefix shape 28 layers x {K,V} x 2 KV heads x 4096 tokens at D=96 and D=80, SRFT"}
    for key in ("d96", "d80"):
        cfg = W.CONFIGS[key]
        D = cfg.D
        sets = []
        for i in range(n_sets):
            c = W.Config(cfg.name, D, cfg.B, cfg.H, cfg.T, cfg.law, cfg.index + 10 * i)
            x, lam = W.prefix_inputs(c, dev)
            sets.append((x, lam, torch.empty_like(x)))
        for k2, name, bits, G in MIXED:
            if k2 != key:
                continue
            plan = K.Plan(D, G, "srft", cfg.sign_seed, bits=bits)
            cb, nsc = plan.code_bytes, D // G
            bufs = [(torch.empty((cfg.B, cfg.H, cfg.T, cb), dtype=torch.uint8, device=dev),
                     torch.empty((cfg.B, cfg.H, cfg.T, nsc), dtype=torch.float16, device=dev))
                    for _ in range(n_sets)]
            enc = timed(lambda i: K.encode(plan, sets[i % n_sets][0], sets[i % n_sets][1], *bufs[i % n_sets]))
            dec = timed(lambda i: K.decode(plan, *bufs[i % n_sets], sets[i % n_sets][1], sets[i % n_sets][2]))
            del bufs
            vb = 2 * D + cb + 2 * nsc                 # bytes per vector, encode or decode
            nb = cfg.vectors * vb
            res[f"D{D}-{name}"] = {
                "bytes_per_call": nb,
                "encode_us": round(enc, 2), "encode_GB_s": round(nb / enc / 1e3, 1),
                "encode_frac_hbm": round(nb / enc / 1e3 / HBM_PEAK_GBS, 4),
                "decode_us": round(dec, 2), "decode_GB_s": round(nb / dec / 1e3, 1),
                "decode_frac_hbm": round(nb / dec / 1e3 / HBM_PEAK_GBS, 4),
            }
        del sets
    torch.cuda.synchronize()
    return res


def graph_leg(K, torch, stream, plan, kv_new, lam_kv, lam_k, lam_v, cache, T0, q, L, sm, out, ws, n):
    """The decode step (append K and V, then attention) captured once in a
    HIP graph and replayed n times: us per replayed step.  Capture and
    replay go through torch's graph API; the library calls allocate,
    free, synchronize and memset nothing, so the step captures as is."""
    kc, ks, vc, vs, kvc, kvs = cache

    def step():
        K.encode(plan, kv_new, lam_kv, kvc, kvs, T0)
        K.attn_decode(plan, q, kc, ks, lam_k, vc, vs, lam_v, L, sm, out, ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(2):
            step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    return timed_loop(torch, stream, lambda i: g.replay(), n)


def clock_windows(K, torch, stream, dev, n_windows, call, encode_burst):
    """The decode-step attention call against the shader clock: n_windows
    windows of 20 calls each, the clock read right after every window;
    first from an idle GPU, then right after a burst of 40 prefix encodes."""
    import statistics
    khz = K.diag_wall_clock_khz()
    clk = torch.zeros((2 * n_windows, 3), dtype=torch.int64, device=dev)
    rows = []
    for phase in ("after 0.3 s idle", "after 40 prefix encodes"):
        torch.cuda.synchronize()
        if phase.startswith("after 0.3"):
            time.sleep(0.3)
        else:
            encode_burst(40)
        evs = []
        for w in range(n_windows):
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(21)]
            ev[0].record(stream)
            for i in range(20):
                call(i)
                ev[i + 1].record(stream)
            K.diag_shader_clock(clk[len(rows) + w])
            evs.append(ev)
        torch.cuda.synchronize()
        for w, ev in enumerate(evs):
            ts = [ev[i].elapsed_time(ev[i + 1]) * 1e3 for i in range(20)]
            rows.append((phase, w, statistics.median(ts), min(ts), max(ts)))
    ck = clk.cpu().tolist()
    out = ["| start | window | median us | min us | max us | shader clock after (GHz) |", "|---|---|---|---|---|---|"]
    for j, (phase, w, med, lo, hi) in enumerate(rows):
        c = ck[j]
        out.append(f"| {phase} | {w} | {med:.1f} | {lo:.1f} | {hi:.1f} | {c[0] / c[1] * khz / 1e6:.3f} |")
    return "\n".join(out)


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def main():
    args = parse()
    if args.trace_summary:
        print(trace_summary(args.trace_summary))
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); "
              "the int4 KV-cache path is per-GPU work with no collectives", file=sys.stderr)
        sys.exit(2)
    # single-threaded numpy for the oracle leg
    os.environ.setdefault("OMP_NUM_THREADS", "1")
    os.environ.setdefault("OPENBLAS_NUM_THREADS", "1")
    import torch
    import kv_cache_int4_amd as K
    from kv_cache_int4_amd import workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()

    # ---- prefix batches (Qwen2.5-1.5B shape) ----
    cfg = W.CONFIGS["qwen"]
    D = cfg.D
    plan = K.Plan(D, 32, "srft", cfg.sign_seed)
    sets = []
    for i in range(args.sets):
        c = W.Config(cfg.name, D, cfg.B, cfg.H, cfg.T, cfg.law, cfg.index + 10 * i)
        x, lam = W.prefix_inputs(c, dev)
        codes = torch.empty((cfg.B, cfg.H, cfg.T, D // 2), dtype=torch.uint8, device=dev)
        scales = torch.empty((cfg.B, cfg.H, cfg.T, D // 32), dtype=torch.float16, device=dev)
        y = torch.empty_like(x)
        sets.append((x, lam, codes, scales, y))
    n_vec = cfg.vectors
    log(f"prefix batches ready ({args.sets} x {n_vec} vectors)")

    # ---- decode step (batch 64, Hq 8, Hkv 2, 32768 cached tokens) ----
    dc = W.CONFIGS["decode"]
    B, Hkv, Hq, T0 = dc.B, dc.H, 8, dc.T
    L = T0 + 1
    Tcap = T0 + 256
    aplan = K.Plan(D, 32, "srft", dc.sign_seed)
    k16, v16, lam_k, lam_v, q = W.decode_inputs(B, Hkv, Hq, Tcap, D, dc.data_seed, dev)
    # A layer's K and V caches are one allocation [2B, Hkv, Tcap, ...], K rows
    # first: the new token's K and V go in with one kvq_encode call over the
    # 2B rows, lambda_K / lambda_V given per row.
    caches = []
    for _ in range(2):
        kvc = torch.empty((2 * B, Hkv, Tcap, D // 2), dtype=torch.uint8, device=dev)
        kvs = torch.empty((2 * B, Hkv, Tcap, D // 32), dtype=torch.float16, device=dev)
        K.encode(aplan, k16[:, :, :T0], lam_k, kvc[:B], kvs[:B], 0)
        K.encode(aplan, v16[:, :, :T0], lam_v, kvc[B:], kvs[B:], 0)
        caches.append((kvc[:B], kvs[:B], kvc[B:], kvs[B:], kvc, kvs))
    kv_new = torch.cat([k16[:, :, T0:T0 + 1], v16[:, :, T0:T0 + 1]]).contiguous()        # [2B, Hkv, 1, D]
    lam_kv = torch.cat([lam_k.expand(B, Hkv, D), lam_v.expand(B, Hkv, D)]).contiguous()  # [2B, Hkv, D]
    ws = torch.empty(K.attn_workspace_size(D, B, Hq, L), dtype=torch.uint8, device=dev)
    out = torch.empty((B, Hq, D), dtype=torch.float16, device=dev)
    sm = 1.0 / math.sqrt(D)
    if args.clock_windows:
        kc, ks, vc, vs, _, _ = caches[0]

        def call(i):
            K.attn_decode(aplan, q, kc, ks, lam_k, vc, vs, lam_v, L, sm, out, ws)

        def encode_burst(n):
            for i in range(n):
                x, lam, codes, scales, _ = sets[i % len(sets)]
                K.encode(plan, x, lam, codes, scales)

        for i in range(5):
            call(i)
        print(clock_windows(K, torch, stream, dev, args.clock_windows, call, encode_burst), flush=True)
        return
    g_cfg, g_sets = d256_setup(K, W, torch, dev, args.sets)
    torch.cuda.synchronize()
    log("decode-step caches and D=256 batches ready")

    phases = ("encode", "decode", "append", "attn")

    def run_phase(p, i):
        x, lam, codes, scales, y = sets[i % len(sets)]
        kc, ks, vc, vs, kvc, kvs = caches[i % 2]
        if p == "encode":
            K.encode(plan, x, lam, codes, scales)
        elif p == "decode":
            K.decode(plan, codes, scales, lam, y)
        elif p == "append":
            K.encode(aplan, kv_new, lam_kv, kvc, kvs, T0)
        else:
            K.attn_decode(aplan, q, kc, ks, lam_k, vc, vs, lam_v, L, sm, out, ws)

    for i in range(args.warmup):
        for p in phases:
            run_phase(p, i)
    torch.cuda.synchronize()

    # The K steps run phase-major (K encodes, K decodes, K appends, K
    # attention steps: the same work as K passes of the whole path, each
    # decode reading codes its set's encode wrote), with a pair of events
    # around each phase, so per-launch times are not padded by event records
    # between launches.
    # After each phase (outside its events) a one-wave probe reads the shader
    # clock: the power manager lowers it under sustained load, and the
    # attention kernel, half bound by its arithmetic, slows with it.
    ev_start = [torch.cuda.Event(enable_timing=True) for _ in phases]
    ev_end = [torch.cuda.Event(enable_timing=True) for _ in phases]
    clk = torch.zeros((len(phases) + 1, 3), dtype=torch.int64, device=dev)
    torch.cuda.synchronize()
    if args.profile_marks:
        torch.cuda._sleep(MARK_CYCLES)
        torch.cuda.synchronize()
    t_start = time.perf_counter()
    K.diag_shader_clock(clk[0])
    for j, p in enumerate(phases):
        ev_start[j].record(stream)
        for i in range(args.steps):
            run_phase(p, i)
        ev_end[j].record(stream)
        K.diag_shader_clock(clk[j + 1])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    log(f"timed {args.steps} steps in {wall:.3f} s")

    ms = {p: ev_start[j].elapsed_time(ev_end[j]) / args.steps for j, p in enumerate(phases)}
    khz = K.diag_wall_clock_khz()
    ck = clk.cpu().tolist()
    sclk = {name: round(c[0] / c[1] * khz / 1e6, 3) if c[1] > 0 else None
            for name, c in zip(("start",) + tuple(f"after_{p}" for p in phases), ck)}

    # ---- fp16-cache comparator, same shape ----
    f16_us = timed_loop(torch, stream, lambda i: K.attn_decode_f16(q, k16, v16, L, sm, out, ws),
                        max(5, args.steps // 2))
    # ---- the same decode step replayed from a captured HIP graph ----
    append_g = graph_loop(torch, stream, lambda: K.encode(aplan, kv_new, lam_kv, caches[0][4], caches[0][5], T0))
    graph_us = graph_leg(K, torch, stream, aplan, kv_new, lam_kv, lam_k, lam_v, caches[0], T0, q, L, sm, out, ws,
                         max(10, args.steps))
    # ---- D=256 (Gemma-3-1B-shaped prefix), both rotations, timed apart ----
    gemma = d256_leg(K, torch, stream, g_cfg, g_sets, max(10, args.steps))
    del g_sets
    # ---- code formats (int4 G16, int8 G32 / G16), timed apart ----
    fmts = formats_leg(K, torch, stream, cfg, sets, dc, k16, v16, lam_k, lam_v, q, L, sm, max(10, args.steps))
    # ---- the encoder with its DFT on the matrix cores, timed apart ----
    mfma = mfma_leg(K, torch, stream, cfg, sets, max(10, args.steps))
    # ---- D=96 and D=80 (mixed-radix SRFT), timed apart ----
    mixed = mixed_leg(K, W, torch, stream, dev, args.sets, max(10, args.steps))
    # ---- D=256 decode step (Gemma-3 1B head shape), timed apart ----
    att256 = attn256_leg(K, W, torch, stream, dev, max(10, args.steps))
    # ---- the 512-vector round trip (latency) ----
    small = small_leg(K, W, torch, stream, dev, max(20, args.steps))
    # ---- Mistral-7B-shaped bulk encode and full-cache decode ----
    del sets
    torch.cuda.empty_cache()
    mistral = None if args.no_bulk else mistral_leg(K, W, torch, stream, dev, 3)
    if args.profile_marks:
        src = torch.empty(CALIB_BYTES // 2, dtype=torch.float16, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        torch.cuda._sleep(MARK_CYCLES)
        torch.cuda.synchronize()
        del src, dst

    # ---- algorithmic bytes ----
    enc_bytes = n_vec * (2 * D + D // 2 + 2 * (D // 32))          # 328 B / vector
    attn_bytes = B * Hkv * L * 2 * (D // 2 + 2 * (D // 32))        # K and V codes + scales
    attn16_bytes = B * Hkv * L * 2 * 2 * D
    enc_s = ms["encode"] / 1e3
    dec_s = ms["decode"] / 1e3
    attn_us = (ms["append"] + ms["attn"]) * 1e3
    enc_gbs = enc_bytes / enc_s / 1e9
    dec_gbs = enc_bytes / dec_s / 1e9
    attn_gbs = attn_bytes / (ms["attn"] / 1e3) / 1e9

    # dominant launch of the step: the one with the largest share of step time
    shares = {"attn": ms["attn"], "encode": ms["encode"], "decode": ms["decode"]}
    dom = max(shares, key=shares.get)
    if dom == "attn":
        rl = {"kernel": "kvq_attn_decode (split-K stream with query rotation + combine)", "bytes": attn_bytes,
              "seconds": ms["attn"] / 1e3, "traffic": measured_traffic("attn")}
    elif dom == "encode":
        rl = {"kernel": "kvq_encode", "bytes": enc_bytes, "seconds": enc_s,
              "traffic": measured_traffic("encode")}
    else:
        rl = {"kernel": "kvq_decode", "bytes": enc_bytes, "seconds": dec_s,
              "traffic": measured_traffic("decode")}
    achieved = rl["bytes"] / rl["seconds"] / 1e9
    roofline = {
        "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
        "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": rl["traffic"],
        "kernel": rl["kernel"], "algorithmic_bytes_per_launch": rl["bytes"],
        "avg_launch_us": round(rl["seconds"] * 1e6, 2),
    }

    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        cpu = cpu_baseline()

    res = {
        "metric": "encode Mvec/s + ns/vec and HBM GB/s at D=128; int4 vs fp16 decode-attn µs/step",
        "value": round(n_vec / enc_s / 1e6, 2),
        "unit": "Mvec/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": "Qwen2.5-1.5B-shaped prefix encode+decode (28 layers x {K,V} x 2 KV heads x 4096 "
                        "tokens, D=128, SRFT, group 32) + GQA decode step on the int4 cache (batch 64, "
                        "Hq 8 / Hkv 2, D=128, 32768 cached tokens + 1 appended)",
            "vectors_per_step": n_vec, "D": D, "group": 32, "rotation": "srft",
            "decode_step": {"B": B, "Hq": Hq, "Hkv": Hkv, "seq_len": L},
        },
        "roofline": roofline,
        "cpu_baseline": cpu,
        "sclk_ghz": sclk,
        "encode": {"us": round(ms["encode"] * 1e3, 2), "Mvec_s": round(n_vec / enc_s / 1e6, 1),
                   "ns_per_vec": round(enc_s / n_vec * 1e9, 4), "GB_s": round(enc_gbs, 1),
                   "frac_hbm": round(enc_gbs / HBM_PEAK_GBS, 4),
                   "GFLOPS_5MlogM": round(n_vec * 5 * (D // 2) * math.log2(D // 2) / enc_s / 1e9, 1)},
        "decode": {"us": round(ms["decode"] * 1e3, 2), "Mvec_s": round(n_vec / dec_s / 1e6, 1),
                   "ns_per_vec": round(dec_s / n_vec * 1e9, 4), "GB_s": round(dec_gbs, 1),
                   "frac_hbm": round(dec_gbs / HBM_PEAK_GBS, 4)},
        "attention": {"int4_us_per_step": round(attn_us, 2), "append_us": round(ms["append"] * 1e3, 2),
                      "int4_attn_us": round(ms["attn"] * 1e3, 2), "int4_attn_GB_s": round(attn_gbs, 1),
                      "fp16_us_per_step": round(f16_us, 2),
                      "fp16_GB_s": round(attn16_bytes / (f16_us / 1e6) / 1e9, 1),
                      "int4_over_fp16": round(attn_us / f16_us, 4),
                      "graph_us_per_step": round(graph_us, 2), "append_graph_us": round(append_g, 2)},
        "d256": gemma,
        "attention_d256": att256,
        "formats": fmts,
        "mixed_radix": mixed,
        "mfma_rotation": mfma,
        "small_round_trip": small,
        "mistral_bulk": mistral,
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
