"""Benchmark of the GDN chunked prefill on one MI355X.

One step = the whole hot path on one batch of seeded synthetic inputs:
forward (gate cumsum, decay matrix and its inverse, intra-GPU context-parallel
state recurrence and output, returning A and the final state) followed by the
backward (state recompute, reverse state-gradient recurrence, local gradients)
at the headline shape H_v = 64, T = 8192 (B = 1, H_q = 32, K = V = 128, bf16
inputs, fp32 state).  Inputs are resident in HBM before timing starts.

Prints ONE JSON line.  Besides the contract keys it carries:
  roofline      the dominant kernel's achieved rate against MI355X's peak,
                from per-kernel HIP-event timing of a second timed region
  cpu_baseline  the fp64 oracle (forward + reverse mode) timed on the host
                cores on a bounded sample of the same workload
  fwd / bwd     per-direction times, tokens/s, TFLOP/s and % of bf16 peak
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16 = 2.5e15      # dense bf16 MFMA, FLOP/s
PEAK_F32 = 157.3e12     # dense fp32 matrix, FLOP/s
PEAK_HBM = 8.0e12       # HBM3E, B/s
CHUNK = 64
FWD_FLOP_PER_TOKEN_HEAD = None  # computed from the chunked algorithm below
METRIC = "GDN chunk fwd/bwd tokens/s + TFLOP/s (% MFMA peak), H_v=64, T=8192"


def chunk_flops(K, V, n=CHUNK):
    """Algorithmic FLOPs of the chunked algorithm per full chunk per v-head.

    fwd = 2n^2(3K+2V) + 6nKV + n^3/3  (K K^T, Q K^T, w, u, w S, Q S, P Vn,
    K^T Vn and the triangular inverse);  bwd = 2n^2(8K+5V) + 16nKV + 4n^3 +
    n^3/3 (the recomputed K K^T, Q K^T, w, u, w S, Q S and inverse, plus
    every gradient product: dVn, dK~, dP, dQ (two), dS (two), dw, dT (two),
    dVb, dKb, dA (two n^3), dK (three)).  Every product is one the chunked
    form performs; the inverse counts n^3/3."""
    fwd = 2 * n * n * (3 * K + 2 * V) + 6 * n * K * V + n ** 3 / 3
    bwd = 2 * n * n * (8 * K + 5 * V) + 16 * n * K * V + 4 * n ** 3 + n ** 3 / 3
    return fwd, bwd


def kernel_model(name, w, nchunks, es):
    """Algorithmic (bytes, flops) of one launch of a library kernel.

    Per-unit figures (unit = one chunk of one v-head, 'cv'; or one chunk of one
    q/k head, 'cq'); q/k bytes are counted once per q/k head."""
    Hq, Hv, K, V = w.Hq, w.Hv, w.K, w.V
    ntok = w.B * w.T
    cv = nchunks * Hv
    cq = nchunks * Hq
    qk = ntok * Hq * K * es
    vbytes = ntok * Hv * V * es
    gb = ntok * Hv * (4 + es)
    tm = cv * 64 * 64 * es
    st = cv * K * V * es  # per-chunk states (backward's internal copy: element type)
    n = CHUNK
    if name == "fwd_main":
        byts = 2 * qk + 2 * vbytes + tm + gb
        fl = cv * (2 * n * n * K + 4 * n * K * V + 2 * 2 * n * n * V + 2 * n * K * V)
    elif name == "prep":
        byts = qk + gb + tm + ntok * Hv * (64 * 4 + 4)
        fl = cq * 2 * n * n * K + cv * n ** 3 / 3
    elif name == "state_main":
        byts = qk + vbytes + tm + gb + st
        fl = cv * (2 * n * K * V + 2 * n * n * V + 2 * n * K * V)
    elif name == "rev_main":
        byts = 2 * qk + vbytes + tm + gb + st
        fl = cv * (2 * n * K * V + 2 * n * n * K + 2 * 2 * n * n * V + 4 * n * K * V)
    elif name == "local_grad":
        byts = 2 * qk + 2 * vbytes + tm + gb + 2 * st + 2 * qk + vbytes + ntok * Hv * (es + 4)
        fl = cv * (4 * n * K * V + 2 * n * n * V + 2 * n * K * V + 2 * n * n * V
                   + 2 * n * V * K + 2 * n * n * V + 4 * n * n * V + 4 * n * V * K
                   + 6 * n * n * K) + cq * 4 * n * n * K
    else:
        return None
    return float(byts), float(fl)


def source_hash():
    d = os.path.join(ROOT, "gated_deltanet_chunked_gdn_amd", "csrc")
    h = hashlib.sha256()
    for f in sorted(os.listdir(d)):
        with open(os.path.join(d, f), "rb") as fh:
            h.update(f.encode())
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_from_profile(kernel, workload):
    """HBM bytes per launch from the committed counter summary, if it was
    taken on the current kernel sources (else None)."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path))
    except (OSError, ValueError):
        return None
    if rec.get("source_hash") != source_hash() or rec.get("workload") != workload:
        return None
    k = rec.get("kernels", {}).get(kernel)
    return None if k is None else k.get("hbm_bytes_per_launch")


def cpu_baseline(w, p, threads_hint=0, l2=False):
    """fp64 oracle forward + reverse mode on a sample of whole q/k groups."""
    import numpy as np
    from oracle import token
    nthr = token.max_threads() if threads_hint <= 0 else threads_hint
    grp = w.Hv // w.Hq
    units = min(w.Hv, max(grp, ((2 * nthr) // grp) * grp))
    mask = np.zeros((w.B, w.Hv), dtype=bool)
    mask[0, :units] = True
    t0 = time.perf_counter()
    token.fwd(p["q"], p["k"], p["v"], p["g"], p["beta"], scale=p["scale"], unit_mask=mask,
              threads=nthr, qk_l2norm=l2)
    token.bwd(p["q"], p["k"], p["v"], p["g"], p["beta"], p["do"], p["dht"], scale=p["scale"],
              unit_mask=mask, threads=nthr, qk_l2norm=l2)
    dt = time.perf_counter() - t0
    toks = w.T * units / w.Hv  # token-equivalents of the full-head workload
    return {"value": toks / dt, "unit": "tokens/s", "cores": int(nthr), "kind": "oracle",
            "sample": f"fwd+bwd of {units} of {w.Hv} v-heads (batch row 0, whole q/k "
                      f"groups), T={w.T}, fp64 token recurrence; {dt:.1f} s wall"}


def _timer(torch):
    def timed(fn, n):
        torch.cuda.synchronize()
        s = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(n):
            fn()
        e.record()
        torch.cuda.synchronize()
        return s.elapsed_time(e) / n
    return timed


def sweep(gdn, synth, torch, dev, args):
    """Head-count sweep (the pages' TP1..TP8 axis): per H_v, the fwd+bwd step
    with the automatic segment length, and fwd / bwd alone for a range of
    forced segment lengths (cp_mode n = n chunks per segment, 0 = no split),
    which is what the automatic choice is checked against."""
    timed = _timer(torch)
    out = []
    for hv in synth.SWEEP_HV:
        w = synth.sweep_workload(hv)
        p = synth.make(w)
        d = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in p.items()}

        def fwd(cp):
            return gdn.chunk_gated_delta_rule_fwd(
                d["q"], d["k"], d["v"], d["g"], d["beta"], scale=d["scale"],
                output_final_state=True, cp_mode=cp, return_states=False)

        def bwd(A, cp):
            return gdn.chunk_gated_delta_rule_bwd(
                d["q"], d["k"], d["v"], d["g"], d["beta"], A, d["do"], dht=d["dht"],
                scale=d["scale"], cp_mode=cp)

        A = fwd(-1)[1]
        for _ in range(args.warmup):
            bwd(fwd(-1)[1], -1)
        rec = {"H_v": hv, "H_q": w.Hq, "T": w.T,
               "auto_segments_per_head": gdn.plan_segments(d["q"], d["k"], d["v"], cp_mode=-1)}
        ms = timed(lambda: bwd(fwd(-1)[1], -1), args.steps)
        rec["step_ms"] = ms
        rec["step_tokens_per_s"] = w.T / (ms * 1e-3)
        by_cp = {}
        for cp in (-1, 0, 4, 8, 13, 16, 26, 32, 64):
            f = timed(lambda: fwd(cp), max(3, args.steps // 2))
            b = timed(lambda: bwd(A, cp), max(3, args.steps // 2))
            by_cp[str(cp)] = {"fwd_ms": round(f, 4), "bwd_ms": round(b, 4)}
        rec["by_cp_mode"] = by_cp
        out.append(rec)
        del d, p
        torch.cuda.empty_cache()
    return {"metric": "GDN chunk fwd/bwd head-count sweep (tokens/s per H_v, T=8192)",
            "unit": "tokens/s", "dtype": "bf16", "data": "synthetic (seeded)",
            "steps": args.steps, "warmup": args.warmup, "sweep": out}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="hv64_t8192")
    ap.add_argument("--cp", type=int, default=-1, help="cp_mode (-1 automatic)")
    ap.add_argument("--fwd-only", action="store_true",
                    help="time the inference forward alone (o and the final state)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-state-cache", action="store_true",
                    help="the backward recomputes the per-chunk states instead of taking "
                         "the forward's state cache")
    ap.add_argument("--calib-copy", action="store_true",
                    help="run only a 1 GiB device copy (counter calibration)")
    ap.add_argument("--qk-l2norm", action="store_true",
                    help="raw q, k inputs, L2-normalised inside the library")
    ap.add_argument("--sweep", action="store_true",
                    help="head-count sweep H_v in 64,48,32,24,16,8 at T=8192 (H_q = H_v/2): "
                         "fwd / bwd / step times per head count and per context-parallel "
                         "segment length; prints one JSON line")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path; "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import gated_deltanet_chunked_gdn_amd as gdn
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.calib_copy:
        a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"calib_copy_bytes": 1 << 30}))
        return

    if args.sweep:
        print(json.dumps(sweep(gdn, synth, torch, dev, args)), flush=True)
        return

    w = synth.WORKLOADS[args.workload]
    p = synth.make(w, with_grads=True, normalize_qk=not args.qk_l2norm)
    l2 = bool(args.qk_l2norm)
    d = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in p.items()}
    torch.cuda.synchronize()

    # training keeps the per-chunk states from the forward for the backward
    # (one buffer, reused every step like an activation buffer)
    use_cache = not args.no_state_cache and not args.fwd_only
    cache = (gdn.state_cache_empty(d["q"], d["v"], cu_seqlens=d["cu_seqlens"], cp_mode=args.cp)
             if use_cache else None)

    def fwd(with_cache=use_cache):
        # with the cache the backward needs neither A nor g_cum (T and the
        # states come from the cache), so the forward does not write them;
        # the forward alone is the inference forward (o and the final state)
        return gdn.chunk_gated_delta_rule_fwd(
            d["q"], d["k"], d["v"], d["g"], d["beta"], scale=d["scale"],
            initial_state=d["initial_state"], cu_seqlens=d["cu_seqlens"],
            output_final_state=True, cp_mode=args.cp, return_states=False,
            return_intermediates=not with_cache and not args.fwd_only,
            use_qk_l2norm_in_kernel=l2, state_cache=cache if with_cache else None)

    def bwd(A, with_cache=use_cache):
        return gdn.chunk_gated_delta_rule_bwd(
            d["q"], d["k"], d["v"], d["g"], d["beta"], A, d["do"], dht=d["dht"],
            scale=d["scale"], initial_state=d["initial_state"], cu_seqlens=d["cu_seqlens"],
            cp_mode=args.cp, use_qk_l2norm_in_kernel=l2,
            state_cache=cache if with_cache else None)

    def step():
        out = fwd()
        if not args.fwd_only:
            bwd(out[1])

    def step_recompute():
        bwd(fwd(False)[1], False)

    def timed(fn, n):
        torch.cuda.synchronize()
        s = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(n):
            fn()
        e.record()
        torch.cuda.synchronize()
        return s.elapsed_time(e) / n

    for _ in range(args.warmup):
        step()
    ms_step = timed(step, args.steps)
    ms_step_recompute = None
    if use_cache:
        for _ in range(2):
            step_recompute()
        ms_step_recompute = timed(step_recompute, args.steps)
    ms_fwd = timed(fwd, args.steps)
    if not args.fwd_only:
        A = fwd()[1]
        ms_bwd = timed(lambda: bwd(A), args.steps)
    # second region: per-kernel HIP events (roofline of the dominant kernel)
    gdn.timing_enable(True)
    timed(step, args.steps)
    gdn.timing_enable(False)
    kern = gdn.timing_collect()

    ntok = w.B * w.T
    nchunks = w.B * ((w.T + CHUNK - 1) // CHUNK)
    es = 2 if w.dtype == "bf16" else 4
    fpc, bpc = chunk_flops(w.K, w.V)
    fl_fwd = fpc * nchunks * w.Hv
    fl_bwd = bpc * nchunks * w.Hv
    peak_mm = PEAK_BF16 if w.dtype == "bf16" else PEAK_F32

    def direction(ms, fl):
        return {"ms": round(ms, 4), "tokens_per_s": ntok / (ms * 1e-3),
                "tflops": fl / (ms * 1e-3) / 1e12,
                "pct_mfma_peak": 100.0 * fl / (ms * 1e-3) / peak_mm}

    # dominant kernel by total time
    dom = max(kern.items(), key=lambda kv: kv[1][1])
    dname, (dcount, dms) = dom
    avg_s = dms / dcount * 1e-3
    model = kernel_model(dname, w, nchunks, es)
    roof = None
    if model is not None:
        byts, fl = model
        ai = fl / byts
        if ai < peak_mm / PEAK_HBM:
            roof = {"bound": "hbm", "achieved": byts / avg_s / 1e9, "peak": PEAK_HBM / 1e9,
                    "unit": "GB/s"}
        else:
            roof = {"bound": "mfma", "achieved": fl / avg_s / 1e12, "peak": peak_mm / 1e12,
                    "unit": "TFLOP/s"}
        roof["frac"] = roof["achieved"] / roof["peak"]
        traffic = traffic_from_profile(dname, w.name)
        roof["traffic"] = traffic
        roof.update({"kernel": dname, "avg_us": avg_s * 1e6, "launches_timed": dcount,
                     "algorithmic_bytes": byts, "algorithmic_flops": fl,
                     "arithmetic_intensity": ai})

    res = {
        "metric": METRIC,
        "value": ntok / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded; q,k L2-normalised N(0,1), v N(0,1), "
                "g=-softplus(N(0,1)), beta=sigmoid(N(0,1)), do N(0,1), dht N(0,0.1))",
        "config": {"workload": w.name + (" fwd only" if args.fwd_only else " fwd+bwd")
                   + (" (q/k L2-normalised in the library)" if l2 else ""),
                   "B": w.B, "T": w.T, "H_q": w.Hq, "H_v": w.Hv, "K": w.K, "V": w.V,
                   "chunk": CHUNK, "cp_mode": args.cp, "state": "fp32",
                   "state_cache": use_cache},
        "roofline": roof,
        "fwd": direction(ms_fwd, fl_fwd),
        "kernels_us": {k: round(v[1] / v[0] * 1e3, 2) for k, v in kern.items()},
    }
    if ms_step_recompute is not None:
        # the same step with the backward recomputing the per-chunk states
        res["ms_per_step_recompute_states"] = ms_step_recompute
    if not args.fwd_only:
        res["bwd"] = direction(ms_bwd, fl_bwd)
        res["step_tflops"] = (fl_fwd + fl_bwd) / (ms_step * 1e-3) / 1e12
        res["step_pct_mfma_peak"] = 100 * (fl_fwd + fl_bwd) / (ms_step * 1e-3) / peak_mm
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, p, l2=l2)
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
