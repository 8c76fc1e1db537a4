"""Benchmark: exact attention forward (TFLOP/s) and decode (HBM GB/s) on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic input:
  * prefill: causal GQA with RoPE, B=2, Hq=32, Hkv=8, N=8192, d=128, bf16
    (the two launches of attn_fwd: K rotation pass + tiled attention kernel,
    made through attn_rope_apply and attn_prefill_cached so that each launch
    has its own events), and
  * decode: GQA, B=32, Hq=32, Hkv=8, d=128, bf16 cache, KV lengths ~ U[1024, 32768]
    (split kernel + merge kernel).
Inputs are resident in device memory before timing starts.  Each call is
bracketed by HIP events on the stream it runs on; the step time is the wall
time of the timed steps between two device synchronisations.

Printed: one JSON line.  ``value`` is the prefill TFLOP/s (algorithmic FLOPs:
4 * d per visible (query, key) pair per query head), ``decode.value`` the decode
GB/s (algorithmic bytes: every valid cached K/V row once, plus q, o, lse, lens).
``roofline`` is for the prefill attention kernel alone (MFMA-bound, bf16 dense
peak 2516.6 TFLOP/s), timed by events around its launch; ``decode.roofline``
for the decode call (HBM-bound, 8 TB/s).
``cpu_baseline`` times the fp64 oracle on a bounded sample of the same
workload on the host cores.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads as W  # noqa: E402

PEAK_BF16_TFLOPS = 2516.6
PEAK_HBM_GBS = 8000.0
TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "traffic.json")
CLOCK_RECORD = os.path.join(ROOT, "profiles", "clock.json")
CSRC = os.path.join(ROOT, "exact_scaled_dot_amd", "csrc")


def strip_comments(src: str) -> str:
    """C/C++ source without its comments (string and character literals kept
    whole) and without trailing blanks, so that editing a comment leaves the
    code's hash alone."""
    out = []
    i, n = 0, len(src)
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
            i = n if j < 0 else j + 2
        else:
            out.append(c)
            i += 1
    lines = [ln.rstrip() for ln in "".join(out).split("\n")]
    return "\n".join(ln for ln in lines if ln)


def source_hash() -> str:
    """Hash of the kernel sources' code (comments left out), to tell whether
    recorded counters still apply."""
    import hashlib
    h = hashlib.sha256()
    for f in sorted(os.listdir(CSRC)):
        if f.endswith((".hip", ".h", ".cpp")):
            h.update(f.encode())
            with open(os.path.join(CSRC, f), encoding="utf-8") as fh:
                h.update(strip_comments(fh.read()).encode())
    return h.hexdigest()[:16]


def recorded_traffic(kernel: str):
    """HBM bytes per launch of ``kernel`` from the committed counter record
    (FETCH_SIZE and WRITE_SIZE, each scaled by the copy-kernel calibration), or
    None when the record is missing or was taken on other kernel sources."""
    try:
        import json as _json
        with open(TRAFFIC_RECORD) as f:
            rec = _json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_hash") != source_hash():
        return None
    k = rec.get("kernels", {}).get(kernel)
    if not k:
        return None
    cal = rec["calibration"]
    return (k["fetch_kib"] * cal["fetch_factor"] + k["write_kib"] * cal["write_factor"]) * 1024.0


def recorded_clock(kernel: str):
    """Shader clock (GHz) under ``kernel`` from the committed counter record:
    GPU-active cycles per dispatch (from MfmaUtil = MFMA busy cycles / (active
    cycles x SIMDs)) over the dispatch time of the same profiled run; None when
    the record is missing or was taken on other kernel sources."""
    try:
        import json as _json
        with open(CLOCK_RECORD) as f:
            rec = _json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_hash") != source_hash():
        return None
    k = rec.get("kernels", {}).get(kernel)
    return None if not k else float(k["sclk_ghz"])


METRIC = "attn fwd TFLOP/s (causal GQA N=8192 d=128 bf16) + decode HBM GB/s"

# ---- writing the counter records from rocprofv3 output (CSV)
XCDS = 8  # MI355X: GRBM_GUI_ACTIVE arrives summed over its eight dies


def short_kernel_name(full: str) -> str:
    """'void attn::(anonymous namespace)::k<128, true>(int, ...)' -> 'k<128, true>'."""
    s = full
    for p in ("void ", "attn::", "(anonymous namespace)::"):
        s = s.replace(p, "")
    depth = 0
    for i, ch in enumerate(s):
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0:
            return s[:i]
    return s


def read_counters(path: str):
    """Per dispatch: kernel name, grid size, duration (ns) and each counter
    summed over the rows rocprofv3 wrote for it (one per die or instance)."""
    import csv
    import collections
    out = collections.OrderedDict()
    with open(path) as f:
        for r in csv.DictReader(f):
            d = int(r["Dispatch_Id"])
            e = out.setdefault(d, {"name": short_kernel_name(r["Kernel_Name"]),
                                   "grid": int(r["Grid_Size"]),
                                   "ns": int(r["End_Timestamp"]) - int(r["Start_Timestamp"]),
                                   "c": collections.defaultdict(float)})
            e["c"][r["Counter_Name"]] += float(r["Counter_Value"])
    return list(out.values())


def _counter_csv(d: str) -> str:
    import glob
    hits = sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True))
    if not hits:
        raise SystemExit(f"no counter_collection.csv under {d}")
    return hits[0]


def _mean_by(dispatches, counter, key):
    import collections
    acc = collections.defaultdict(list)
    for e in dispatches:
        if counter in e["c"]:
            acc[key(e)].append(e["c"][counter])
    return {k: sum(v) / len(v) for k, v in acc.items()}


def write_traffic_record(d: str):
    """profiles/traffic.json from rocprofv3 --pmc runs under ``d``: fetch/ and
    write/ (FETCH_SIZE, WRITE_SIZE over 'bench.py --steps 1 --warmup 0
    --no-cpu-baseline --no-extra'), xfetch/ and xwrite/ (the same without
    --no-extra, optional), cal_fetch/ and cal_write/ ('bench.py
    --calibrate-copy')."""
    def load(sub):
        p = os.path.join(d, sub)
        return read_counters(_counter_csv(p)) if os.path.isdir(p) else None
    f, w_ = load("fetch"), load("write")
    cf, cw = load("cal_fetch"), load("cal_write")
    name = lambda e: e["name"]
    copy = "__amd_rocclr_copyBuffer"
    cfk = _mean_by(cf, "FETCH_SIZE", name)[copy]
    cwk = _mean_by(cw, "WRITE_SIZE", name)[copy]
    nbytes = 1 << 30
    fk, wk = _mean_by(f, "FETCH_SIZE", name), _mean_by(w_, "WRITE_SIZE", name)
    rec = {
        "source_hash": source_hash(),
        "note": "per-dispatch FETCH_SIZE and WRITE_SIZE (KiB, mean over dispatches) from two "
                "rocprofv3 --pmc passes over 'python3 bench.py --steps 1 --warmup 0 --no-cpu-baseline "
                "--no-extra' (kernels of the headline step); 'extras' from the same passes without "
                "--no-extra, keyed by kernel and grid size; calibration: a 1 GiB device copy "
                "('python3 bench.py --calibrate-copy') reads as the counts below",
        "calibration": {"copy_bytes": nbytes, "copy_fetch_kib": cfk, "copy_write_kib": cwk,
                        "fetch_factor": nbytes / (cfk * 1024.0), "write_factor": nbytes / (cwk * 1024.0)},
        "kernels": {k: {"fetch_kib": fk[k], "write_kib": wk[k]} for k in sorted(fk)
                    if k in wk and not k.startswith("__amd")},
    }
    xf, xw = load("xfetch"), load("xwrite")
    if xf and xw:
        key = lambda e: f"{e['name']} @grid {e['grid']}"
        a, b = _mean_by(xf, "FETCH_SIZE", key), _mean_by(xw, "WRITE_SIZE", key)
        rec["extras"] = {k: {"fetch_kib": a[k], "write_kib": b[k]} for k in sorted(a)
                         if k in b and not k.startswith("__amd")}
    with open(TRAFFIC_RECORD, "w") as fh:
        json.dump(rec, fh, indent=1)
    print(f"wrote {TRAFFIC_RECORD}")


def write_clock_record(d: str):
    """profiles/clock.json from a rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES
    GRBM_GUI_ACTIVE run under ``d`` over the headline step: the shader clock is
    GPU-active cycles per die over the dispatch time; the matrix-core busy
    fraction is MFMA-busy cycles over active cycles x 1024 SIMDs."""
    ds = read_counters(_counter_csv(d))
    import collections
    per = collections.defaultdict(list)
    for e in ds:
        c = e["c"]
        # a short dispatch's active count takes in cycles outside it: only
        # kernels of 100 us and more are kept
        if "GRBM_GUI_ACTIVE" in c and "SQ_VALU_MFMA_BUSY_CYCLES" in c and e["ns"] >= 100000:
            act = c["GRBM_GUI_ACTIVE"] / XCDS
            per[e["name"]].append((act / e["ns"], 100.0 * c["SQ_VALU_MFMA_BUSY_CYCLES"] / (act * 1024)))
    rec = {
        "source_hash": source_hash(),
        "note": "shader clock under each kernel: GRBM_GUI_ACTIVE (summed over the 8 dies, so divided by 8) "
                "per dispatch over its duration, mean over dispatches (kernels of 100 us and more); mfma_util_pct = "
                "SQ_VALU_MFMA_BUSY_CYCLES / (active cycles x 1024 SIMDs); from rocprofv3 --pmc "
                "SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE over 'python3 bench.py --steps 2 --warmup 1 "
                "--no-cpu-baseline --no-extra'",
        "kernels": {k: {"sclk_ghz": sum(x[0] for x in v) / len(v),
                        "mfma_util_pct": sum(x[1] for x in v) / len(v)} for k, v in sorted(per.items())},
    }
    with open(CLOCK_RECORD, "w") as fh:
        json.dump(rec, fh, indent=1)
    print(f"wrote {CLOCK_RECORD}")


def visible_pairs(Nq, Nk, causal, window=0):
    if not causal:
        return Nq * Nk
    off = Nk - Nq
    if window:
        # query i (position off+i) sees keys max(0, off+i-w+1) .. off+i
        return int(np.minimum(np.arange(Nq, dtype=np.int64) + off + 1, window).sum())
    # query i sees keys 0..off+i
    return Nq * (off + 1) + Nq * (Nq - 1) // 2


def fwd_flops(w, window=0):
    return 4.0 * w.d * visible_pairs(w.Nq, w.Nk, w.causal, window) * w.B * w.Hq


def decode_bytes(w, lens, T=1):
    kv = int(np.sum(lens.astype(np.int64))) * w.Hkv * w.d * 2 * 2
    q = w.B * w.Hq * T * w.d * 2
    o = w.B * w.Hq * T * w.d * 4
    lse = w.B * w.Hq * T * 4
    return kv + q + o + lse + w.B * 4


def dev(x):
    import torch
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(x).cuda()


_CPU = {}  # inputs the oracle workers read (set before the pool forks)


def _blas_one_thread():
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:  # pragma: no cover
        pass


def _oracle_head(bh):
    """Oracle O and lse of every row of one query head of the prefill workload."""
    import oracle.dense as oa
    w3, q, k, v = _CPU["pf"]
    b, h = divmod(bh, w3.Hq)
    kc = _CPU.setdefault("kc", {})
    oa.attention_rows(q, k, v, b, h, np.arange(w3.Nq), causal=True, scale=w3.scale,
                      rope_base=w3.rope_base, dtype="bf16", _kcache=kc)
    return bh


def _oracle_seq(i):
    """Oracle decode of one sequence of the decode workload."""
    import oracle.dense as oa
    w4, lens, qd, kcache, vcache = _CPU["dec"]
    oa.decode(qd[i:i + 1], kcache[i:i + 1], vcache[i:i + 1], lens[i:i + 1], scale=w4.scale)
    return i


def cpu_baseline(w3, w4, budget_s=20.0):
    """Time the fp64 oracle on bounded samples of both workloads on the host.

    One worker process per available core (at most 16), each with one BLAS
    thread; the work unit is a whole query head of the causal GQA N=8192
    workload (all 8192 rows) for prefill, a whole sequence of the decode
    workload for decode.  Heads are handed out a round (one per worker) at a
    time until about half the budget is used; the prefill rate over those heads
    stands for the whole workload (extrapolated: the oracle's work per head is
    the same for every head).  Run before the process touches the GPU, so the
    forked workers inherit no device state.  The oracle runs as it is.
    """
    import multiprocessing as mp
    cores = max(1, min(len(os.sched_getaffinity(0)), 16))
    q, k, v = W.fwd_inputs(w3)
    _CPU["pf"] = (w3, q, k, v)
    lens = W.decode_lens(w4)[:8]
    qd, kcache, vcache = W.decode_inputs(w4, lens, max_len=int(lens.max()))
    _CPU["dec"] = (w4, lens, qd, kcache, vcache)
    total = w3.B * w3.Hq
    per_head_pairs = int(np.sum(np.arange(w3.Nq) + (w3.Nk - w3.Nq) + 1))
    ctx = mp.get_context("fork")
    with ctx.Pool(cores, initializer=_blas_one_thread) as pool:
        t0 = time.perf_counter()
        heads = 0
        while heads < total and time.perf_counter() - t0 < budget_s * 0.5:
            n = min(cores, total - heads)
            list(pool.imap_unordered(_oracle_head, range(heads, heads + n)))
            heads += n
        t_pf = time.perf_counter() - t0
        t0 = time.perf_counter()
        list(pool.imap_unordered(_oracle_seq, range(len(lens))))
        t_dec = time.perf_counter() - t0
    _CPU.clear()
    tflops = 4.0 * w3.d * per_head_pairs * heads / t_pf / 1e12
    nbytes = int(np.sum(lens.astype(np.int64))) * w4.Hkv * w4.d * 2 * 2
    return {
        "value": tflops, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
        "sample": f"prefill: {heads} of {total} whole query heads (8192 rows each) of the causal "
                  f"GQA RoPE N=8192 workload in {t_pf:.1f} s on {cores} worker processes of one "
                  f"BLAS thread each (fp64 NumPy, RoPE rounding model, dense score rows)"
                  + ("" if heads == total else "; the rate over those heads stands for the workload")
                  + f"; decode: {len(lens)} of the {w4.B} sequences of the decode workload in "
                  f"{t_dec:.1f} s, the rate over them standing for the workload",
        "extrapolated": heads < total,
        "prefill_seconds": t_pf, "prefill_heads": heads,
        "prefill_seconds_whole_workload": t_pf * total / heads,
        "decode_value": nbytes / t_dec / 1e9, "decode_unit": "GB/s", "decode_seconds": t_dec,
    }


EXTRA = (("mha_d64_n2048", 0), ("gqa_rope_n32768", 0), ("gqa_rope_n8192", 4096), ("gqa_rope_n32768", 4096))


PREWARM_S = 0.25  # set from --prewarm-s


def timed_calls(torch, stream, call, reps):
    """Untimed calls for PREWARM_S seconds (the clock settles under load), then
    ``reps`` calls timed one by one with events on ``stream``; mean ms."""
    t0 = time.perf_counter()
    call()
    torch.cuda.synchronize()
    while time.perf_counter() - t0 < PREWARM_S:
        call()
        torch.cuda.synchronize()
    ms = []
    for _ in range(reps):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        call()
        b.record(stream)
        torch.cuda.synchronize()
        ms.append(a.elapsed_time(b))
    return float(np.mean(ms))


def extra_prefill(torch, esd, stream, reps=5):
    """TFLOP/s of the other prefill workloads (same entry points, same timing):
    MHA d=64 N=2048, long-context GQA N=32768, and the causal sliding window
    (w=4096) on the GQA N=8192 and N=32768 shapes; flops count visible pairs."""
    out = {}
    for name, win in EXTRA:
        w = W.WORKLOADS[name]
        label = f"{name}_w{win}" if win else name
        note = f"{w.note}, sliding window {win}" if win else w.note
        print(f"[bench] extra workload {label}: {note}", file=sys.stderr, flush=True)
        q, k, v = W.fwd_inputs(w)
        dq, dk, dv = dev(q), dev(k), dev(v)
        del q, k, v
        o = torch.empty((w.B, w.Hq, w.Nq, w.d), dtype=torch.float32, device="cuda")
        lse = torch.empty((w.B, w.Hq, w.Nq), dtype=torch.float32, device="cuda")
        nws = esd.fwd_workspace_bytes(w.B, w.Hkv, w.Nk, w.d, w.rope_base, esd.ATTN_BF16)
        ws = torch.empty(max(nws, 1), dtype=torch.uint8, device="cuda") if nws else None
        call = lambda: esd.fwd(dq, dk, dv, causal=w.causal, scale=w.scale, rope_base=w.rope_base,
                               out=o, lse=lse, workspace=ws, window=win)
        ms = timed_calls(torch, stream, call, reps)
        fl = fwd_flops(w, win)
        out[label] = {"workload": note, "flops": fl, "ms": ms, "tflops": fl / (ms * 1e-3) / 1e12}
        del dq, dk, dv, o, lse, ws
        torch.cuda.empty_cache()
    return out


def extra_decode_evicted(torch, esd, stream, w, nbytes, dq, dkc, dvc, dlens, o, lse, ws, reps=10):
    """GB/s of the headline decode call with the 256 MB last-level cache
    (Infinity Cache) evicted before each call, outside the events, in two ways
    on the same stream: a 1 GiB write (which leaves that cache full of dirty
    lines for the call to write back as it streams) and a 1 GiB read.  The
    back-to-back timing of the headline line may find the tail of the
    previous call's cache rows still there."""
    print("[bench] extra workload decode with the last-level cache evicted", file=sys.stderr,
          flush=True)
    junk = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    junk.fill_(1)
    sink = torch.empty((), dtype=torch.int64, device="cuda")
    call = lambda: esd.decode(dq, dkc, dvc, dlens, scale=w.scale, out=o, lse=lse, workspace=ws)
    call()
    out = {"workload": f"{w.note}, a 1 GiB write or read between calls (outside the timed region)",
           "bytes": nbytes}
    for how in ("write", "read"):
        ms = []
        for r in range(reps):
            if how == "write":
                junk.fill_(r & 0xFF)
            else:
                torch.sum(junk.view(torch.int32), dim=0, out=sink)
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            call()
            b.record(stream)
            torch.cuda.synchronize()
            ms.append(a.elapsed_time(b))
        m = float(np.mean(ms))
        out[f"{how}_evict"] = {"ms": m, "ms_min": float(np.min(ms)), "gbs": nbytes / (m * 1e-3) / 1e9}
    del junk, sink
    torch.cuda.empty_cache()
    return out


def extra_decode_multi(torch, esd, stream, w, lens, dkc, dvc, dlens, T=4, reps=10):
    """GB/s of multi-token decode on the decode batch: T = 4 new tokens per
    sequence (verifying drafted tokens), so 16 queries per KV head."""
    print(f"[bench] extra workload decode_multi T={T}", file=sys.stderr, flush=True)
    q = dev(W.normal((w.B, w.Hq, T, w.d), 9700, 1.0, "bf16"))
    o = torch.empty((w.B, w.Hq, T, w.d), dtype=torch.float32, device="cuda")
    lse = torch.empty((w.B, w.Hq, T), dtype=torch.float32, device="cuda")
    ws = torch.empty(esd.decode_multi_workspace_bytes(w.B, w.Hq, w.Hkv, T, w.max_len, w.d),
                     dtype=torch.uint8, device="cuda")
    call = lambda: esd.decode_multi(q, dkc, dvc, dlens, scale=w.scale, out=o, lse=lse, workspace=ws)
    ms = timed_calls(torch, stream, call, reps)
    nb = decode_bytes(w, lens, T)
    return {"workload": f"{w.note}, T={T} new tokens per sequence (bottom-right causal)",
            "bytes": nb, "ms": ms, "gbs": nb / (ms * 1e-3) / 1e9}


def extra_decode_paged(torch, esd, stream, w, lens, reps=10):
    """GB/s of single-token decode on the decode batch with its cache in
    16-token blocks scattered over a pool (bytes as for the contiguous cache)."""
    print("[bench] extra workload decode_paged bs=16", file=sys.stderr, flush=True)
    q, kp, vp, table = W.paged_inputs(w, lens, block_size=16)
    dq, dkp, dvp, dt, dl = dev(q), dev(kp), dev(vp), dev(table), dev(lens)
    del q, kp, vp
    o = torch.empty((w.B, w.Hq, 1, w.d), dtype=torch.float32, device="cuda")
    lse = torch.empty((w.B, w.Hq, 1), dtype=torch.float32, device="cuda")
    ws = torch.empty(esd.decode_paged_workspace_bytes(w.B, w.Hq, w.Hkv, 1, table.shape[1], 16, w.d),
                     dtype=torch.uint8, device="cuda")
    call = lambda: esd.decode_paged(dq, dkp, dvp, dt, dl, scale=w.scale, out=o, lse=lse, workspace=ws)
    ms = timed_calls(torch, stream, call, reps)
    nb = decode_bytes(w, lens) + table.size * 4
    del dq, dkp, dvp, dt, dl, o, lse, ws
    torch.cuda.empty_cache()
    return {"workload": f"{w.note}, paged cache in blocks of 16 tokens", "bytes": nb,
            "ms": ms, "gbs": nb / (ms * 1e-3) / 1e9}


def extra_backward(torch, esd, stream, w, reps=5):
    """TFLOP/s of the backward pass (attn_bwd after attn_fwd) on a prefill
    workload.  Flops: the five products of the gradient (S, dP, dV, dQ, dK)
    over the visible pairs, 2.5x the forward's two; the recomputation of S and
    dP in the dQ kernel is not counted."""
    print(f"[bench] extra workload backward {w.name}", file=sys.stderr, flush=True)
    q, k, v = W.fwd_inputs(w)
    dq_, dk_, dv_ = dev(q), dev(k), dev(v)
    del q, k, v
    do = dev(W.normal((w.B, w.Hq, w.Nq, w.d), 11500, 1.0, "f32"))
    o, lse = esd.fwd(dq_, dk_, dv_, causal=w.causal, scale=w.scale, rope_base=w.rope_base)
    gq = torch.empty((w.B, w.Hq, w.Nq, w.d), dtype=torch.float32, device="cuda")
    gk = torch.empty((w.B, w.Hkv, w.Nk, w.d), dtype=torch.float32, device="cuda")
    gv = torch.empty_like(gk)
    ws = torch.empty(esd.bwd_workspace_bytes(w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.d, w.rope_base,
                                             esd.ATTN_BF16), dtype=torch.uint8, device="cuda")
    call = lambda: esd.bwd(dq_, dk_, dv_, o, lse, do, causal=w.causal, scale=w.scale,
                           rope_base=w.rope_base, dq=gq, dk=gk, dv=gv, workspace=ws)
    ms = timed_calls(torch, stream, call, reps)
    fl = 2.5 * fwd_flops(w)
    del dq_, dk_, dv_, do, o, lse, gq, gk, gv, ws
    torch.cuda.empty_cache()
    return {"workload": f"{w.note}, backward (dQ, dK, dV)", "flops": fl, "ms": ms,
            "tflops": fl / (ms * 1e-3) / 1e12}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", choices=["prefill", "decode", "backward"], default=None,
                    help="time one leg only, or the backward pass alone (for profiling)")
    ap.add_argument("--prewarm-s", type=float, default=0.25,
                    help="seconds of untimed steps before the warmup steps: under load the GPU's "
                         "clock settles over ~50 ms, and steps taken before that run up to 25%% slower")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the extra prefill workloads (MHA d=64 N=2048, GQA N=32768, sliding window)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run a plain 1 GiB device copy three times (counter calibration)")
    ap.add_argument("--write-traffic-record", metavar="DIR",
                    help="write profiles/traffic.json from rocprofv3 --pmc output under DIR (no GPU)")
    ap.add_argument("--write-clock-record", metavar="DIR",
                    help="write profiles/clock.json from rocprofv3 --pmc output under DIR (no GPU)")
    args = ap.parse_args()
    global PREWARM_S
    PREWARM_S = args.prewarm_s
    if args.write_traffic_record or args.write_clock_record:
        if args.write_traffic_record:
            write_traffic_record(args.write_traffic_record)
        if args.write_clock_record:
            write_clock_record(args.write_clock_record)
        return
    if args.calibrate_copy:
        import torch
        n = (1 << 30) // 4
        a = torch.ones(n, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": 1 << 30, "copy_bytes_written": 1 << 30, "copies": 3}))
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the library has no "
              "multi-GPU path", file=sys.stderr)
        sys.exit(2)

    w3 = W.WORKLOADS["gqa_rope_n8192"]
    w4 = W.WORKLOADS["decode_b32"]
    cpu = None
    if not args.no_cpu_baseline and args.only is None:
        # before anything touches the GPU: the oracle workers are forked
        print("[bench] cpu baseline", file=sys.stderr, flush=True)
        cpu = cpu_baseline(w3, w4)

    import torch
    import exact_scaled_dot_amd as esd

    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    if args.only == "backward":
        # attn_bwd on the prefill workload alone (for profiling): one untimed
        # call, then --steps timed calls
        rec = extra_backward(torch, esd, stream, w3, reps=args.steps)
        print(json.dumps({"only": "backward", **rec}), flush=True)
        return

    do_pf = args.only in (None, "prefill")
    do_dec = args.only in (None, "decode")

    print("[bench] generating inputs", file=sys.stderr, flush=True)
    flops = fwd_flops(w3)
    lens = W.decode_lens(w4)
    nbytes = decode_bytes(w4, lens)
    if do_pf:
        q, k, v = W.fwd_inputs(w3)
        dq, dk, dv = dev(q), dev(k), dev(v)
        del q, k, v
        o3 = torch.empty((w3.B, w3.Hq, w3.Nq, w3.d), dtype=torch.float32, device="cuda")
        l3 = torch.empty((w3.B, w3.Hq, w3.Nq), dtype=torch.float32, device="cuda")
        kr3 = torch.empty_like(dk)
    if do_dec:
        qd, kc, vc = W.decode_inputs(w4, lens)
        dqd, dkc, dvc, dlens = dev(qd), dev(kc), dev(vc), dev(lens)
        del qd, kc, vc
        o4 = torch.empty((w4.B, w4.Hq, w4.d), dtype=torch.float32, device="cuda")
        l4 = torch.empty((w4.B, w4.Hq), dtype=torch.float32, device="cuda")
        ws4 = torch.empty(esd.decode_workspace_bytes(w4.B, w4.Hq, w4.Hkv, w4.max_len, w4.d),
                          dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()

    def step(evs=None):
        if do_pf:
            # attn_fwd's two launches made as two calls, so that the attention
            # kernel has events of its own: the K rotation pass (attn_rope_apply,
            # the pass attn_fwd runs into its workspace), then the attention
            # kernel on the rotated keys (attn_prefill_cached: the same kernel
            # and launch; bit-identical to attn_fwd, tested)
            if evs: evs[0].record(stream)
            esd.rope_apply(dk, w3.rope_base, 0, out=kr3)
            if evs: evs[4].record(stream)
            esd.prefill_cached(dq, kr3, dv, scale=w3.scale, rope_base=w3.rope_base, out=o3, lse=l3)
            if evs: evs[1].record(stream)
        if do_dec:
            if evs: evs[2].record(stream)
            esd.decode(dqd, dkc, dvc, dlens, scale=w4.scale, out=o4, lse=l4, workspace=ws4)
            if evs: evs[3].record(stream)

    print("[bench] prewarm", file=sys.stderr, flush=True)
    t_pre = time.perf_counter()
    n_pre = 0
    while time.perf_counter() - t_pre < args.prewarm_s:
        step()
        torch.cuda.synchronize()
        n_pre += 1
    print("[bench] warmup", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(args.steps)]
    print("[bench] timing", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(evs[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    pf_ms = [e[0].elapsed_time(e[1]) for e in evs] if do_pf else [float("nan")]
    rope_ms = [e[0].elapsed_time(e[4]) for e in evs] if do_pf else [float("nan")]
    attn_ms_all = [e[4].elapsed_time(e[1]) for e in evs] if do_pf else [float("nan")]
    dec_ms = [e[2].elapsed_time(e[3]) for e in evs] if do_dec else [float("nan")]
    pf_avg = float(np.mean(pf_ms))
    dec_avg = float(np.mean(dec_ms))

    rope_avg = float(np.mean(rope_ms))
    attn_ms = float(np.mean(attn_ms_all))
    tflops = flops / (pf_avg * 1e-3) / 1e12 if do_pf else None
    kern_tflops = flops / (attn_ms * 1e-3) / 1e12 if do_pf else None
    gbs = nbytes / (dec_avg * 1e-3) / 1e9 if do_dec else None
    pf_traffic = recorded_traffic("prefill_bf16_kernel<128, true, true, false>")
    pf_sclk = recorded_clock("prefill_bf16_kernel<128, true, true, false>")
    dec_split = recorded_traffic("decode_split_kernel<128, 4, false>")
    dec_merge = recorded_traffic("decode_merge_kernel<128>")
    dec_traffic = dec_split + dec_merge if dec_split is not None and dec_merge is not None else None

    rec = {
        "metric": METRIC,
        "value": tflops,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall * 1e3 / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "prefill: causal GQA + RoPE 1e4, B=2 Hq=32 Hkv=8 N=8192 d=128 bf16; "
                        "decode: GQA B=32 Hq=32 Hkv=8 d=128 bf16, lens ~ U[1024,32768] seed 4004",
            "prefill_flops": flops, "prefill_ms": pf_avg, "prefill_ms_min": float(np.min(pf_ms)),
            "prefill_rope_k_ms": rope_avg, "prefill_attention_kernel_ms": attn_ms,
            "prefill_attention_kernel_ms_min": float(np.min(attn_ms_all)),
            "prefill_attention_kernel_ms_median": float(np.median(attn_ms_all)),
            "decode_bytes": nbytes, "decode_ms": dec_avg, "decode_ms_min": float(np.min(dec_ms)),
            "decode_ms_median": float(np.median(dec_ms)),
            "prewarm_steps": n_pre,
        },
        "roofline": {
            # events around the attention kernel's own launch
            "kernel": "prefill_bf16_kernel<128, true, true, false>",
            "bound": "mfma", "achieved": kern_tflops, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": (kern_tflops / PEAK_BF16_TFLOPS) if kern_tflops else None,
            "traffic": pf_traffic,
            # context only: the shader clock the counters measured under this
            # kernel in the profiled session (the clock sags under this load),
            # and the fraction of the peak scaled to that clock
            "sclk_ghz": pf_sclk,
            "frac_at_sclk": (kern_tflops / (PEAK_BF16_TFLOPS * pf_sclk / 2.4))
                            if (kern_tflops and pf_sclk) else None,
        },
        "decode": {
            "value": gbs, "unit": "GB/s",
            "roofline": {"kernel": "decode_split_kernel<128, 4, false> + decode_merge_kernel<128>",
                         "bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": (gbs / PEAK_HBM_GBS) if gbs else None, "traffic": dec_traffic},
        },
        "source_hash": source_hash(),
        "context": {
            "a100_roofline": "312 TFLOPS FP16, 1555 GB/s, ~200 FLOP/B",
            "materialised_scores_fp16_n8192_per_head_MB": 8192 * 8192 * 2 / 2 ** 20,
        },
    }
    if not args.no_extra and args.only is None:
        rec["extra_decode"] = {"decode_evicted": extra_decode_evicted(torch, esd, stream, w4, nbytes,
                                                                      dqd, dkc, dvc, dlens, o4, l4,
                                                                      ws4)}
        rec["extra_decode"]["decode_multi_T4"] = extra_decode_multi(torch, esd, stream, w4, lens,
                                                                    dkc, dvc, dlens)
        del dkc, dvc
        torch.cuda.empty_cache()
        rec["extra_decode"]["decode_paged_bs16"] = extra_decode_paged(torch, esd, stream, w4, lens)
        # free the headline workloads' buffers before the long-context one
        del dq, dk, dv, o3, l3, kr3, dqd, o4, l4, ws4
        torch.cuda.empty_cache()
        rec["extra"] = extra_prefill(torch, esd, stream)
        rec["extra"]["gqa_rope_n8192_backward"] = extra_backward(torch, esd, stream, w3)
    if cpu is not None:
        # the GPU figures over the oracle's on the same workloads (context only)
        cpu["gpu_speedup"] = {"prefill": tflops / cpu["value"] if tflops else None,
                              "decode": gbs / cpu["decode_value"] if gbs else None}
        rec["cpu_baseline"] = cpu
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
