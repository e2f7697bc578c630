"""Benchmark of the GDN chunked prefill on one MI355X.

One step = the whole hot path on one batch of seeded synthetic inputs: the
training forward (gate cumsum, decay matrix and its inverse, context-parallel
state recurrence and output, filling the state cache) followed by the
backward (reverse state-gradient recurrence and local gradients) at the
headline shape H_v = 64, T = 8192 (B = 1, H_q = 32, K = V = 128, bf16 inputs,
fp32 state).  Inputs are resident in HBM before timing starts.

Timing: every timed call is bracketed by its own pair of HIP events on the
launch stream; reports give the median over the repetitions ("warm": back to
back; "cold": a 512 MB scratch write before each repetition evicts the L2
and the MALL).  The contract keys value / ms_per_step come from the warm
median of the step; the region of K steps is still bracketed by device
synchronisation on both sides.

Prints ONE JSON line.  Besides the contract keys it carries:
  roofline      the dominant kernel of the step (largest total time from
                per-kernel HIP events): its algorithmic MFMA FLOPs per launch
                over its average duration against the bf16 dense peak (the
                bound the counters show: MFMA-bound products, latency-limited),
                with its HBM side (the method's minimum bytes and the
                counter-measured traffic) alongside
  fwd, fwd_train, bwd   per-direction medians, tokens/s, TFLOP/s, % of peak
  configs       the other workloads: the long small-head forward (automatic
                context parallelism), the packed variable-length forward and
                the backward configuration
  cpu_baseline  the fp64 oracle (forward + reverse mode) timed on the host
                cores on a bounded sample of the same workload, with the CPU
                model and a single-thread time
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


def kernel_flops(name, w, nchunks):
    """Algorithmic MFMA FLOPs of one launch of a library kernel, from the
    chunked algorithm's products that kernel performs (per chunk of n = 64
    tokens and v-head, dense tiles; shared Q K^T / K K^T counted per v-head):

      prep        K K^T (F2) and the triangular inverse (F3): 2n^2K + n^3/3
      fwd_main    w, u (F4), Q K^T (F5), w S and K^T Vn (F6), Q S and P Vn
                  (F7): 2n^2(2K + 2V) + 6nKV
      rev_main    the reverse state-gradient products (B3): 2n^2V + 6nKV
      state_main  the backward's state recompute (B2): 2n^2(K + V) + 4nKV
      local_grad  the chunk-local gradients (B4, B5, B6):
                  2n^2(6K + 4V) + 12nKV + 4n^3
    The fix-up and serial passes are implementation overhead (no
    algorithmic FLOPs)."""
    K, V, n = w.K, w.V, CHUNK
    per = {"prep": 2 * n * n * K + n ** 3 / 3,
           "fwd_main": 2 * n * n * (2 * K + 2 * V) + 6 * n * K * V,
           "rev_main": 2 * n * n * V + 6 * n * K * V,
           "state_main": 2 * n * n * (K + V) + 4 * n * K * V,
           "local_grad": 2 * n * n * (6 * K + 4 * V) + 12 * n * K * V + 4 * n ** 3}
    if name not in per:
        return None
    return float(per[name] * nchunks * w.Hv)


def min_bytes(w, ntok, nseq, direction, es, with_A=False, with_h0=False):
    """The method's minimum HBM bytes of one call: every input read once and
    every output written once (q/k once per q/k head), plus the saved A for
    the pages' backward; nothing for intermediates."""
    qk = ntok * w.Hq * w.K * es
    vv = ntok * w.Hv * w.V * es
    gb = ntok * w.Hv * (4 + es)
    st = nseq * w.Hv * w.K * w.V * 4
    if direction == "fwd":
        return 2 * qk + vv + gb + (st if with_h0 else 0) + vv + st
    A = ntok * w.Hv * CHUNK * 4 if with_A else 0
    # reads q k v g beta (A) do dht (h0); writes dq dk dv dbeta dg dh0
    return (2 * qk + vv + gb + A + vv + st + (st if with_h0 else 0)
            + 2 * qk + vv + ntok * w.Hv * (es + 4) + st)


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


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, p, threads_hint=0, l2=False):
    """fp64 oracle forward + reverse mode on a sample of whole q/k groups
    (all host threads), and one v-head on one thread."""
    import numpy as np
    from oracle import token
    nthr = token.max_threads() if threads_hint <= 0 else threads_hint
    grp = w.Hv // w.Hq
    units = min(w.Hv, max(grp, ((2 * nthr) // grp) * grp))

    def run(nunits, threads):
        mask = np.zeros((w.B, w.Hv), dtype=bool)
        mask[0, :nunits] = True
        t0 = time.perf_counter()
        token.fwd(p["q"], p["k"], p["v"], p["g"], p["beta"], scale=p["scale"], unit_mask=mask,
                  threads=threads, qk_l2norm=l2)
        token.bwd(p["q"], p["k"], p["v"], p["g"], p["beta"], p["do"], p["dht"],
                  scale=p["scale"], unit_mask=mask, threads=threads, qk_l2norm=l2)
        return time.perf_counter() - t0

    dt = run(units, nthr)
    dt1 = run(1, 1)
    toks = w.T * units / w.Hv  # token-equivalents of the full-head workload
    return {"value": toks / dt, "unit": "tokens/s", "cores": int(nthr), "kind": "oracle",
            "cpu_model": cpu_model(), "host_cpus": os.cpu_count(),
            "sample": f"fwd+bwd of {units} of {w.Hv} v-heads (batch row 0, whole q/k "
                      f"groups), T={w.T}, fp64 token recurrence on {nthr} threads; "
                      f"{dt:.1f} s wall",
            "single_thread": {"value": w.T / w.Hv / dt1, "unit": "tokens/s",
                              "sample": f"fwd+bwd of 1 v-head, T={w.T}, 1 thread; "
                                        f"{dt1:.1f} s wall"}}


def rep_times(torch, fn, reps, cold=None):
    """Per-call durations (ms) from a pair of events around each call on the
    current stream; `cold` (a large buffer) is overwritten before each call."""
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(reps)]
    stops = [torch.cuda.Event(enable_timing=True) for _ in range(reps)]
    torch.cuda.synchronize()
    for i in range(reps):
        if cold is not None:
            cold.zero_()
        starts[i].record()
        fn()
        stops[i].record()
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in zip(starts, stops)]


def median(xs):
    xs = sorted(xs)
    n = len(xs)
    return xs[n // 2] if n % 2 else 0.5 * (xs[n // 2 - 1] + xs[n // 2])


def timing(torch, fn, reps, cold_buf, ntok, flops, peak_mm, mbytes=None, warmup=3):
    """Warm and cold medians of one call, with its rates."""
    for _ in range(warmup):
        fn()
    warm = rep_times(torch, fn, reps)
    cold = rep_times(torch, fn, reps, cold_buf)
    ms = median(warm)
    out = {"ms": round(ms, 4), "ms_cold": round(median(cold), 4),
           "ms_min": round(min(warm), 4), "reps": reps,
           "tokens_per_s": ntok / (ms * 1e-3), "tflops": flops / (ms * 1e-3) / 1e12,
           "pct_mfma_peak": 100.0 * flops / (ms * 1e-3) / peak_mm,
           "pct_mfma_peak_cold": 100.0 * flops / (median(cold) * 1e-3) / peak_mm}
    if mbytes is not None:
        out["min_bytes"] = mbytes
        out["min_bytes_gbps"] = mbytes / (ms * 1e-3) / 1e9
        out["min_bytes_pct_hbm"] = 100.0 * mbytes / (ms * 1e-3) / PEAK_HBM
    return out


def _timer(torch):
    def timed(fn, n):
        return median(rep_times(torch, fn, n))
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


def nchunks_of(w, p):
    if p.get("cu_seqlens") is not None:
        return sum((L + CHUNK - 1) // CHUNK for L in p["lengths"])
    return w.B * ((w.T + CHUNK - 1) // CHUNK)


def config_entries(gdn, synth, torch, dev, args, cold_buf):
    """The other workloads of the benchmark, each timed warm and cold."""
    out = {}
    fpc, bpc = chunk_flops(128, 128)
    es = 2

    def load(name, **kw):
        w = synth.WORKLOADS[name]
        p = synth.make(w, **kw)
        d = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in p.items()}
        return w, p, d

    # long sequence, few heads: the automatic context-parallel split
    for name in ("hv8_t65536", "varlen16_hv32"):
        w, p, d = load(name)
        nch = nchunks_of(w, p)
        ntok = int(d["q"].shape[0] * d["q"].shape[1])
        nseq = len(p["lengths"]) if "lengths" in p else w.B

        def f():
            gdn.chunk_gated_delta_rule(d["q"], d["k"], d["v"], d["g"], d["beta"],
                                       scale=d["scale"], initial_state=d["initial_state"],
                                       output_final_state=True, cu_seqlens=d["cu_seqlens"])
        ent = timing(torch, f, args.reps, cold_buf, ntok, fpc * nch * w.Hv, PEAK_BF16,
                     min_bytes(w, ntok, nseq, "fwd", es, with_h0=d["initial_state"] is not None))
        ent.update({"direction": "fwd (inference)", "B": w.B, "T_total": ntok, "H_q": w.Hq,
                    "H_v": w.Hv, "K": w.K, "V": w.V, "chunks_per_head": nch,
                    "segments": gdn.plan_segments(d["q"], d["k"], d["v"],
                                                  cu_seqlens=d["cu_seqlens"])})
        if "lengths" in p:
            ent["lengths"] = p["lengths"]
        out[name] = ent
        del d, p
        torch.cuda.empty_cache()
    # the backward configuration: the pages' dataflow (the forward returns A,
    # the backward takes it) and the training step with the state cache
    w, p, d = load("bwd_b2_t16384_hv16")
    nch = nchunks_of(w, p)
    ntok = w.B * w.T
    kw = dict(scale=d["scale"], initial_state=d["initial_state"], cu_seqlens=d["cu_seqlens"])
    A = gdn.chunk_gated_delta_rule_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"],
                                       return_states=False, **kw)[1]

    def b():
        gdn.chunk_gated_delta_rule_bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], A, d["do"],
                                       dht=d["dht"], **kw)
    ent = timing(torch, b, args.reps, cold_buf, ntok, bpc * nch * w.Hv, PEAK_BF16,
                 min_bytes(w, ntok, w.B, "bwd", es, with_A=True))
    cache = gdn.state_cache_empty(d["q"], d["v"])

    def step():
        gdn.chunk_gated_delta_rule_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"],
                                       return_intermediates=False, state_cache=cache, **kw)
        gdn.chunk_gated_delta_rule_bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], None,
                                       d["do"], dht=d["dht"], state_cache=cache, **kw)
    st = timing(torch, step, args.reps, cold_buf, ntok, (fpc + bpc) * nch * w.Hv, PEAK_BF16)
    ent.update({"direction": "bwd (given A)", "B": w.B, "T": w.T, "H_q": w.Hq, "H_v": w.Hv,
                "K": w.K, "V": w.V, "step_with_state_cache": st})
    out["bwd_b2_t16384_hv16"] = ent
    del d, p, A, cache
    torch.cuda.empty_cache()
    # the pages' benchmark axis: head counts 48 .. 8 (TP2 .. TP8 of the
    # headline's 64; H_q = H_v / 2, T = 8192), the inference forward and the
    # cached training step (fwd + bwd) at each
    sw = {}
    for hv in synth.SWEEP_HV:
        if hv == 64:
            continue  # the headline line itself
        w = synth.sweep_workload(hv)
        p = synth.make(w)
        d = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in p.items()}
        nch = nchunks_of(w, p)
        ntok = w.B * w.T
        kw = dict(scale=d["scale"], initial_state=d["initial_state"])

        def f():
            gdn.chunk_gated_delta_rule(d["q"], d["k"], d["v"], d["g"], d["beta"],
                                       output_final_state=True, **kw)
        fe = timing(torch, f, args.reps, cold_buf, ntok, fpc * nch * w.Hv, PEAK_BF16)
        cache = gdn.state_cache_empty(d["q"], d["v"])

        def step():
            gdn.chunk_gated_delta_rule_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"],
                                           output_final_state=True, return_intermediates=False,
                                           return_states=False, state_cache=cache, **kw)
            gdn.chunk_gated_delta_rule_bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], None,
                                           d["do"], dht=d["dht"], state_cache=cache, **kw)
        se = timing(torch, step, args.reps, cold_buf, ntok, (fpc + bpc) * nch * w.Hv, PEAK_BF16)
        sw[str(hv)] = {"H_q": w.Hq, "T": w.T,
                       "segments": gdn.plan_segments(d["q"], d["k"], d["v"]),
                       "fwd_ms": fe["ms"], "fwd_pct_mfma_peak": round(fe["pct_mfma_peak"], 2),
                       "step_ms": se["ms"], "step_tokens_per_s": se["tokens_per_s"],
                       "step_pct_mfma_peak": round(se["pct_mfma_peak"], 2)}
        del d, p, cache
        torch.cuda.empty_cache()
    out["head_sweep_t8192"] = sw
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--reps", type=int, default=20,
                    help="repetitions per median for the per-direction and per-config entries")
    ap.add_argument("--workload", default="hv64_t8192")
    ap.add_argument("--cp", type=int, default=-1, help="cp_mode (-1 automatic)")
    ap.add_argument("--fwd-only", action="store_true",
                    help="time the inference forward alone (o and the final state)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the other workloads (quick and profiling runs)")
    ap.add_argument("--no-state-cache", action="store_true",
                    help="the backward recomputes the per-chunk states instead of taking "
                         "the forward's state cache")
    ap.add_argument("--calib-copy", action="store_true",
                    help="run only a 1 GiB device copy (counter calibration)")
    ap.add_argument("--calib-read", action="store_true",
                    help="run only a 1 GiB read-only reduction (counter calibration)")
    ap.add_argument("--qk-l2norm", action="store_true",
                    help="raw q, k inputs, L2-normalised inside the library")
    ap.add_argument("--sweep", action="store_true",
                    help="head-count sweep H_v in 64,48,32,24,16,8 at T=8192 (H_q = H_v/2): "
                         "fwd / bwd / step times per head count and per context-parallel "
                         "segment length; prints one JSON line")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path; "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import gated_deltanet_chunked_gdn_amd as gdn
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.calib_copy or args.calib_read:
        a = torch.ones(1 << 28, dtype=torch.float32, device=dev)  # 1 GiB
        if args.calib_copy:
            b = torch.empty_like(a)
            for _ in range(3):
                b.copy_(a)
        else:
            for _ in range(3):
                torch.sum(a)
        torch.cuda.synchronize()
        print(json.dumps({"calib_bytes": 1 << 30, "kind": "copy" if args.calib_copy else "read"}))
        return

    if args.sweep:
        print(json.dumps(sweep(gdn, synth, torch, dev, args)), flush=True)
        return

    w = synth.WORKLOADS[args.workload]
    p = synth.make(w, with_grads=True, normalize_qk=not args.qk_l2norm)
    l2 = bool(args.qk_l2norm)
    d = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in p.items()}
    torch.cuda.synchronize()
    cold_buf = torch.empty(512 << 20, dtype=torch.uint8, device=dev)

    # training keeps the per-chunk states from the forward for the backward
    # (one buffer, reused every step like an activation buffer)
    use_cache = not args.no_state_cache and not args.fwd_only
    cache = (gdn.state_cache_empty(d["q"], d["v"], cu_seqlens=d["cu_seqlens"], cp_mode=args.cp,
                                   use_qk_l2norm_in_kernel=l2)
             if use_cache else None)

    def fwd(with_cache=use_cache, inference=False):
        # with the cache the backward needs neither A nor g_cum (T and the
        # states come from the cache), so the forward does not write them
        return gdn.chunk_gated_delta_rule_fwd(
            d["q"], d["k"], d["v"], d["g"], d["beta"], scale=d["scale"],
            initial_state=d["initial_state"], cu_seqlens=d["cu_seqlens"],
            output_final_state=True, cp_mode=args.cp, return_states=False,
            return_intermediates=not with_cache and not inference,
            use_qk_l2norm_in_kernel=l2, state_cache=cache if with_cache else None)

    def bwd(A, with_cache=use_cache):
        return gdn.chunk_gated_delta_rule_bwd(
            d["q"], d["k"], d["v"], d["g"], d["beta"], A, d["do"], dht=d["dht"],
            scale=d["scale"], initial_state=d["initial_state"], cu_seqlens=d["cu_seqlens"],
            cp_mode=args.cp, use_qk_l2norm_in_kernel=l2,
            state_cache=cache if with_cache else None)

    def step():
        if args.fwd_only:
            fwd(False, inference=True)
        else:
            bwd(fwd()[1])

    def step_recompute():
        bwd(fwd(False)[1], False)

    ntok = w.B * w.T
    nchunks = w.B * ((w.T + CHUNK - 1) // CHUNK)
    es = 2 if w.dtype == "bf16" else 4
    fpc, bpc = chunk_flops(w.K, w.V)
    fl_fwd = fpc * nchunks * w.Hv
    fl_bwd = bpc * nchunks * w.Hv
    peak_mm = PEAK_BF16 if w.dtype == "bf16" else PEAK_F32
    has_h0 = d["initial_state"] is not None

    # the contract's region: W warm-up steps, then K steps between device
    # synchronisations, each step bracketed by its own events
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    step_ms = rep_times(torch, step, args.steps)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    ms_step = median(step_ms)
    step_cold = median(rep_times(torch, step, args.reps, cold_buf))

    res_dirs = {}
    res_dirs["fwd"] = timing(torch, lambda: fwd(False, inference=True), args.reps, cold_buf,
                             ntok, fl_fwd, peak_mm, min_bytes(w, ntok, w.B, "fwd", es, with_h0=has_h0))
    ms_step_recompute = None
    if not args.fwd_only:
        if use_cache:
            res_dirs["fwd_train"] = timing(torch, fwd, args.reps, cold_buf, ntok, fl_fwd, peak_mm)
            ms_step_recompute = median(rep_times(torch, step_recompute, args.reps))
        A = fwd()[1]
        res_dirs["bwd"] = timing(torch, lambda: bwd(A), args.reps, cold_buf, ntok, fl_bwd, peak_mm,
                                 min_bytes(w, ntok, w.B, "bwd", es, with_A=not use_cache,
                                           with_h0=has_h0))
    # per-kernel HIP events over one more region of the step
    gdn.timing_enable(True)
    rep_times(torch, step, args.steps)
    gdn.timing_enable(False)
    kern = gdn.timing_collect()

    dom = max(kern.items(), key=lambda kv: kv[1][1])
    dname, (dcount, dms) = dom
    avg_s = dms / dcount * 1e-3
    fl = kernel_flops(dname, w, nchunks)
    roof = None
    if fl is not None:
        traffic = traffic_from_profile(dname, w.name)
        roof = {"bound": "mfma", "achieved": fl / avg_s / 1e12, "peak": peak_mm / 1e12,
                "unit": "TFLOP/s", "frac": fl / avg_s / peak_mm, "traffic": traffic,
                "kernel": dname, "avg_us": avg_s * 1e6, "launches_timed": dcount,
                "algorithmic_flops": fl}
        if traffic is not None:
            roof["traffic_gbps"] = traffic / avg_s / 1e9
            roof["traffic_frac_hbm"] = traffic / avg_s / PEAK_HBM

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
        "ms_per_step_cold": step_cold,
        "ms_per_step_wall_mean": wall_ms,
        "kernels_us": {k: round(v[1] / v[0] * 1e3, 2) for k, v in kern.items()},
    }
    res.update(res_dirs)
    if ms_step_recompute is not None:
        # the same step with the backward recomputing the per-chunk states
        res["ms_per_step_recompute_states"] = ms_step_recompute
    if not args.fwd_only:
        res["step_tflops"] = (fl_fwd + fl_bwd) / (ms_step * 1e-3) / 1e12
        res["step_pct_mfma_peak"] = 100 * (fl_fwd + fl_bwd) / (ms_step * 1e-3) / peak_mm
    del d, cache
    torch.cuda.empty_cache()
    if not args.no_configs and not args.fwd_only and args.workload == "hv64_t8192":
        res["configs"] = config_entries(gdn, synth, torch, dev, args, cold_buf)
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, p, l2=l2)
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
