"""Benchmark: exact attention forward (TFLOP/s) and decode (HBM GB/s) on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic input:
  * prefill: causal GQA with RoPE, B=2, Hq=32, Hkv=8, N=8192, d=128, bf16
    (K rotation pass + tiled attention kernel), and
  * decode: GQA, B=32, Hq=32, Hkv=8, d=128, bf16 cache, KV lengths ~ U[1024, 32768]
    (split kernel + merge kernel).
Inputs are resident in device memory before timing starts.  Each call is
bracketed by HIP events on the stream it runs on; the step time is the wall
time of the timed steps between two device synchronisations.

Printed: one JSON line.  ``value`` is the prefill TFLOP/s (algorithmic FLOPs:
4 * d per visible (query, key) pair per query head), ``decode.value`` the decode
GB/s (algorithmic bytes: every valid cached K/V row once, plus q, o, lse, lens).
``roofline`` is for the prefill attention call (MFMA-bound, bf16 dense peak
2516.6 TFLOP/s), ``decode.roofline`` for the decode call (HBM-bound, 8 TB/s).
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


def source_hash() -> str:
    """Hash of the kernel sources, to tell whether recorded counters still apply."""
    import hashlib
    h = hashlib.sha256()
    for f in sorted(os.listdir(CSRC)):
        if f.endswith((".hip", ".h", ".cpp")):
            h.update(f.encode())
            with open(os.path.join(CSRC, f), "rb") as fh:
                h.update(fh.read())
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


def cpu_baseline(w3, w4, budget_s=20.0):
    """Time the fp64 oracle on bounded samples of both workloads on the host.

    Prefill: whole query heads of the causal GQA N=8192 workload (all 8192 rows
    of head 0, then head 1, ...) until half the budget is used; decode: whole
    sequences of the decode workload until the other half is used.  The oracle
    runs as it is (NumPy fp64, BLAS threads as configured on the host).
    """
    import oracle.dense as oa
    try:
        from threadpoolctl import threadpool_info
        cores = max([int(p.get("num_threads", 1)) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    q, k, v = W.fwd_inputs(w3)
    t0 = time.perf_counter()
    heads = 0
    pairs = 0
    kc = {}
    rows = np.arange(w3.Nq)
    per_head_pairs = int(np.sum(rows + (w3.Nk - w3.Nq) + 1))
    while time.perf_counter() - t0 < budget_s * 0.5 and heads < w3.B * w3.Hq:
        b, h = divmod(heads, w3.Hq)
        oa.attention_rows(q, k, v, b, h, rows, causal=True, scale=w3.scale,
                          rope_base=w3.rope_base, dtype="bf16", _kcache=kc)
        pairs += per_head_pairs
        heads += 1
    t_pf = time.perf_counter() - t0
    tflops = 4.0 * w3.d * pairs / t_pf / 1e12
    del q, k, v
    lens = W.decode_lens(w4)[:8]
    qd, kcache, vcache = W.decode_inputs(w4, lens, max_len=int(lens.max()))
    t0 = time.perf_counter()
    nb = 0
    nbytes = 0
    while time.perf_counter() - t0 < budget_s * 0.5 and nb < len(lens):
        oa.decode(qd[nb:nb + 1], kcache[nb:nb + 1], vcache[nb:nb + 1], lens[nb:nb + 1], scale=w4.scale)
        nbytes += int(lens[nb]) * w4.Hkv * w4.d * 2 * 2
        nb += 1
    t_dec = time.perf_counter() - t0
    return {
        "value": tflops, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
        "sample": f"prefill: {heads} whole query heads (8192 rows each) of the causal GQA RoPE "
                  f"N=8192 workload in {t_pf:.1f} s (fp64 NumPy, RoPE rounding model, dense "
                  f"score rows); decode: {nb} whole sequences of the decode workload in "
                  f"{t_dec:.1f} s",
        "decode_value": nbytes / t_dec / 1e9, "decode_unit": "GB/s",
    }


EXTRA = (("mha_d64_n2048", 0), ("gqa_rope_n32768", 0), ("gqa_rope_n8192", 4096), ("gqa_rope_n32768", 4096))


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
        fl = fwd_flops(w, win)
        out[label] = {"workload": note, "flops": fl, "ms": float(np.mean(ms)),
                     "tflops": fl / (float(np.mean(ms)) * 1e-3) / 1e12}
        del dq, dk, dv, o, lse, ws
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
    nb = decode_bytes(w, lens, T)
    return {"workload": f"{w.note}, T={T} new tokens per sequence (bottom-right causal)",
            "bytes": nb, "ms": float(np.mean(ms)), "gbs": nb / (float(np.mean(ms)) * 1e-3) / 1e9}


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
    nb = decode_bytes(w, lens) + table.size * 4
    del dq, dkp, dvp, dt, dl, o, lse, ws
    torch.cuda.empty_cache()
    return {"workload": f"{w.note}, paged cache in blocks of 16 tokens", "bytes": nb,
            "ms": float(np.mean(ms)), "gbs": nb / (float(np.mean(ms)) * 1e-3) / 1e9}


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
    fl = 2.5 * fwd_flops(w)
    del dq_, dk_, dv_, do, o, lse, gq, gk, gv, ws
    torch.cuda.empty_cache()
    return {"workload": f"{w.note}, backward (dQ, dK, dV)", "flops": fl, "ms": float(np.mean(ms)),
            "tflops": fl / (float(np.mean(ms)) * 1e-3) / 1e12}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", choices=["prefill", "decode", "backward"], default=None,
                    help="time one leg only, or the backward pass alone (for profiling)")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the extra prefill workloads (MHA d=64 N=2048, GQA N=32768, sliding window)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run a plain 1 GiB device copy three times (counter calibration)")
    args = ap.parse_args()
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

    import torch
    import exact_scaled_dot_amd as esd

    w3 = W.WORKLOADS["gqa_rope_n8192"]
    w4 = W.WORKLOADS["decode_b32"]
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
        ws3 = torch.empty(esd.fwd_workspace_bytes(w3.B, w3.Hkv, w3.Nk, w3.d, w3.rope_base,
                                                  esd.ATTN_BF16), dtype=torch.uint8, device="cuda")
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
            if evs: evs[0].record(stream)
            esd.fwd(dq, dk, dv, causal=True, scale=w3.scale, rope_base=w3.rope_base, out=o3, lse=l3,
                    workspace=ws3)
            if evs: evs[1].record(stream)
            if evs:
                # the same K rotation pass attn_fwd runs first, timed on its own so
                # the attention kernel's share of the call is known
                evs[4].record(stream)
                esd.rope_apply(dk, w3.rope_base, 0, out=kr3)
                evs[5].record(stream)
        if do_dec:
            if evs: evs[2].record(stream)
            esd.decode(dqd, dkc, dvc, dlens, scale=w4.scale, out=o4, lse=l4, workspace=ws4)
            if evs: evs[3].record(stream)

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
    rope_ms = [e[4].elapsed_time(e[5]) for e in evs] if do_pf else [float("nan")]
    dec_ms = [e[2].elapsed_time(e[3]) for e in evs] if do_dec else [float("nan")]
    pf_avg = float(np.mean(pf_ms))
    dec_avg = float(np.mean(dec_ms))

    rope_avg = float(np.mean(rope_ms))
    tflops = flops / (pf_avg * 1e-3) / 1e12 if do_pf else None
    attn_ms = pf_avg - rope_avg
    kern_tflops = flops / (attn_ms * 1e-3) / 1e12 if do_pf else None
    gbs = nbytes / (dec_avg * 1e-3) / 1e9 if do_dec else None
    # the time of the step is the wall time; the K rotation timed separately is
    # not part of it
    wall -= float(np.sum(rope_ms)) * 1e-3 if do_pf else 0.0
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
            "decode_bytes": nbytes, "decode_ms": dec_avg, "decode_ms_min": float(np.min(dec_ms)),
        },
        "roofline": {
            "kernel": "prefill_bf16_kernel<128, true, true, false>",
            "bound": "mfma", "achieved": kern_tflops, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": (kern_tflops / PEAK_BF16_TFLOPS) if kern_tflops else None,
            "traffic": pf_traffic,
            # the clock sags under this load: the fraction of the peak at the
            # shader clock the counters measured under this kernel
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
        rec["extra_decode"] = {"decode_multi_T4": extra_decode_multi(torch, esd, stream, w4, lens,
                                                                     dkc, dvc, dlens)}
        del dkc, dvc
        torch.cuda.empty_cache()
        rec["extra_decode"]["decode_paged_bs16"] = extra_decode_paged(torch, esd, stream, w4, lens)
        # free the headline workloads' buffers before the long-context one
        del dq, dk, dv, o3, l3, ws3, kr3, dqd, o4, l4, ws4
        torch.cuda.empty_cache()
        rec["extra"] = extra_prefill(torch, esd, stream)
        rec["extra"]["gqa_rope_n8192_backward"] = extra_backward(torch, esd, stream, w3)
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline", file=sys.stderr, flush=True)
        rec["cpu_baseline"] = cpu_baseline(w3, w4)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
