#!/usr/bin/env python3
"""Benchmark of the attention hot path on one MI355X.

One step = attn_fwd + attn_bwd on the 181M-style GQA workload (B=16, T=2048, 8 query / 4 KV
heads, d=96, causal, RoPE, QK-norm, soft-cap 50), inputs resident in HBM.  The printed JSON
line's `value` is that step's algorithmic throughput in TFLOP/s (14 d flops per visible
(query, key) pair).  The same line also reports:
  * decode: KV-cache decode of 64 sequences (cache lengths U{256..2048}, 8/4 heads, d=96,
    RoPE, soft-cap 50) in GB/s of active K/V read, rotating over several cache copies so the
    last-level cache cannot serve them;
  * the flaxchat-style d=128 workloads (full causal and window 512) fwd+bwd;
  * roofline: the dominant kernel's algorithmic rate against the MI355X bf16 dense peak,
    from per-kernel HIP events recorded by the library's trace on the launch stream;
  * cpu_baseline: the fp64 numpy oracle on a bounded sample of the same workload.
Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
METRIC = "causal attn fwd+bwd TFLOP/s (% bf16 MFMA peak); decode KV GB/s"


# Counter summaries (FETCH_SIZE / WRITE_SIZE runs, calibrated on a plain copy) and the sources
# whose hash each one is valid for.
TRAFFIC_FILES = {
    "bwd_dkdv_d96": ("hbm_traffic_bwd_dkdv_gqa181m_train.md", ["bwd.hip", "device_common.h", "launch.h"]),
    "decode_split_d96": ("hbm_traffic_decode_gqa181m_decode.md",
                         ["decode.hip", "device_common.h", "launch.h"]),
}


def kernel_sources_sha256(names):
    import hashlib
    h = hashlib.sha256()
    for name in names:
        with open(os.path.join(ROOT, "causal_attention_02_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(kernel):
    """HBM bytes per launch of `kernel` from its committed counter summary, or None when there
    is none for this kernel or its sources changed since the counters were taken."""
    if kernel not in TRAFFIC_FILES:
        return None
    fname, sources = TRAFFIC_FILES[kernel]
    try:
        with open(os.path.join(ROOT, "profiles", fname)) as f:
            for line in f:
                if line.startswith("bench-traffic:"):
                    rec = json.loads(line.split(":", 1)[1])
                    break
            else:
                return None
    except OSError:
        return None
    if rec.get("kernel") != kernel or rec.get("sources_sha256") != kernel_sources_sha256(sources):
        return None
    return rec.get("bytes_per_launch", rec.get("bytes_per_call"))


def visible_tiles32(T, window):
    """32 x 32 (query, key) tiles that meet the causal / window band of one head."""
    n = 0
    for qt in range((T + 31) // 32):
        lo = max(0, qt * 32 - window + 1) // 32 if window > 0 else 0
        n += qt - lo + 1
    return n


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--decode-iters", type=int, default=200)
    ap.add_argument("--decode-copies", type=int, default=4)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--only", choices=["train", "decode", "all"], default="all")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="also run a plain device copy of this many MiB (3 times) so HBM byte "
                         "counters can be calibrated against a known size")
    ap.add_argument("--profile-workload", default=None,
                    help="run only this workload's step (a training workload's fwd+bwd, or a "
                         "decode workload's call) --steps times after --warmup, for a profiler; "
                         "prints one line and skips everything else")
    ap.add_argument("--profile-split", action="store_true",
                    help="with --profile-workload: time attn_bwd_split instead of attn_bwd")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the attention path has no "
              "multi-GPU mode", file=sys.stderr)
        sys.exit(2)

    import ctypes

    import torch

    from causal_attention_02_amd import binding as bd
    from causal_attention_02_amd.inputs import (WORKLOADS, decode_bytes, make_decode_inputs,
                                                extend_flops, make_extend_inputs,
                                                make_segment_ids, packed_flops,
                                                make_train_inputs, train_flops, visible_pairs,
                                                make_leftpad_decode_inputs)

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    bd.lib()  # fails loudly when the HIP library is missing
    dev = torch.device("cuda:0")
    props = torch.cuda.get_device_properties(dev)
    stream = torch.cuda.current_stream()
    dinfo = bd.device_info(0)
    log(f"[bench] device: {dinfo['compute_units']} CUs at {dinfo['clock_khz'] / 1e3:.0f} MHz -> "
        f"dense bf16 {dinfo['bf16_dense_tflops']:.0f} TFLOP/s; memory clock "
        f"{dinfo['mem_clock_khz'] / 1e3:.0f} MHz x {dinfo['mem_bus_bits']} bits")

    def opts_of(w):
        return bd.AttnOptions(window=w.window, softcap=w.softcap, rope=w.rope,
                              rope_base=w.rope_base, qk_norm=w.qk_norm, norm_eps=w.norm_eps)

    def calibration_copy():
        nb = args.copy_mib << 20
        src = torch.empty(nb, dtype=torch.uint8, device=dev)
        dst = torch.empty(nb, dtype=torch.uint8, device=dev)
        src.fill_(1)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] calibration copy: 3 x {args.copy_mib} MiB device-to-device")
        del src, dst
        torch.cuda.empty_cache()

    def to_dev(x):
        return torch.from_numpy(x).to(dev).to(torch.bfloat16).contiguous()

    # ------------------------------------------------------------------------------------
    # fwd + bwd
    # ------------------------------------------------------------------------------------
    def timed(fn, n):
        """Milliseconds for n back-to-back calls of fn: one HIP event pair on the launch stream
        around all of them, synchronised on both sides (no marker between the calls)."""
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for i in range(n):
            fn(i)
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b)

    def per_call_ms(fn, n):
        """Per-call times from an event after every call (a separate pass: the markers between
        calls add their own cost, so these are for the spread, not the rate)."""
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
        ev[0].record(stream)
        for i in range(n):
            fn(i)
            ev[i + 1].record(stream)
        torch.cuda.synchronize()
        return np.array([ev[i].elapsed_time(ev[i + 1]) for i in range(n)])

    def settle(fn, seconds=0.5):
        """Run fn back to back for `seconds` before any warm-up or timing: a cold GPU takes some
        tens of milliseconds of load to reach its steady clocks, and the first workload timed
        would otherwise run partly below them.  Untimed."""
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < seconds:
            for i in range(4):
                fn(i)
            torch.cuda.synchronize()

    def train_case(w, steps, warmup, trace=False, ids=None, split=False):
        """Time fwd + bwd; with w.dropout > 0 each step also draws a fresh keep mask; split:
        the backward is attn_bwd_split."""
        q, k, v, dO = make_train_inputs(w)
        tids = None if ids is None else torch.from_numpy(ids).to(dev)
        tq, tk, tv, tdo = to_dev(q), to_dev(k), to_dev(v), to_dev(dO)
        del q, k, v, dO
        o = torch.empty_like(tq)
        lse = torch.empty(tq.shape[:3], dtype=torch.float32, device=dev)
        dq, dk, dv = torch.empty_like(tq), torch.empty_like(tk), torch.empty_like(tv)
        opts = opts_of(w)
        B, Hq, T, D = tq.shape
        Hkv = tk.shape[1]
        cfg = bd.make_cfg(B, T, Hq, Hkv, D, opts, bd.ATTN_BF16)
        if tids is None:
            nf = bd.lib().attn_fwd_workspace_bytes(ctypes.byref(cfg))
            nb = (bd.lib().attn_bwd_split_workspace_bytes if split else
                  bd.lib().attn_bwd_workspace_bytes)(ctypes.byref(cfg))
        else:
            nf = bd.lib().attn_fwd_packed_workspace_bytes(ctypes.byref(cfg))
            nb = bd.lib().attn_bwd_packed_workspace_bytes(ctypes.byref(cfg))
        wsf = torch.empty(max(int(nf), 1), dtype=torch.uint8, device=dev)
        wsb = torch.empty(max(int(nb), 1), dtype=torch.uint8, device=dev)
        p = w.dropout
        mask = None
        if p > 0:
            nm = bd.lib().attn_dropout_mask_bytes(ctypes.byref(cfg))
            mask = torch.empty(max(int(nm), 1), dtype=torch.uint8, device=dev)
        calls = [0]
        # The backward takes k after RoPE / QK-norm from the forward's workspace (a training
        # step keeps it from the forward to the backward, as it keeps o and lse).
        khat = wsf if ((w.rope or w.qk_norm) and tids is None and mask is None and not split) \
            else None

        def step(_i=0):
            if mask is not None:
                bd.attn_dropout_mask(tq, tk, p, w.seed, calls[0], opts, out=mask)
                calls[0] += 1
            bd.attn_fwd(tq, tk, tv, opts, out=o, lse=lse, workspace=wsf, segment_ids=tids,
                        dropout_p=p, dropout_mask=mask)
            bd.attn_bwd(tq, tk, tv, o, tdo, lse, opts, dq=dq, dk=dk, dv=dv, workspace=wsb,
                        segment_ids=tids, dropout_p=p, dropout_mask=mask, khat=khat, split=split)

        settle(step)
        for _ in range(warmup):
            step()
        total_ms = timed(step, steps)
        per = per_call_ms(step, steps)
        kern = None
        if trace:
            bd.trace_enable(True)
            for _ in range(steps):
                step()
            torch.cuda.synchronize()
            kern = bd.trace_read()
            bd.trace_enable(False)
        return total_ms / steps, per, kern

    if args.profile_workload:
        # One workload only, for a profiler: a training step (fwd + bwd) or a decode call over
        # --decode-copies cache copies.
        w = WORKLOADS[args.profile_workload]
        if args.copy_mib > 0:
            calibration_copy()
        if w.decode:
            qd, kc, vc, lens = make_decode_inputs(w)
            tq = to_dev(qd)
            tk0, tv0 = to_dev(kc), to_dev(vc)
            del kc, vc
            cps = [(tk0, tv0)] + [(tk0.clone(), tv0.clone()) for _ in range(args.decode_copies - 1)]
            tl = torch.from_numpy(lens).to(dev)
            od = torch.empty_like(tq)
            wsp = bd.decode_workspace(w.B, w.Hq, w.Hkv, w.D, w.T, opts_of(w))

            def one(i):
                kk, vv = cps[i % len(cps)]
                bd.attn_decode(tq, kk, vv, tl, opts_of(w), out=od, workspace=wsp)

            settle(one)
            for i in range(args.warmup):
                one(i)
            ms = timed(one, args.steps) / args.steps
            log(f"[bench] profile {w.name}: {ms * 1e3:.1f} us/call over {args.steps} calls, "
                f"{decode_bytes(w, lens) / 1e6:.1f} MB of active K/V per call")
        else:
            ids = make_segment_ids(w) if w.seg_lo > 0 else None
            ms, _, _ = train_case(w, args.steps, args.warmup, ids=ids, split=args.profile_split)
            log(f"[bench] profile {w.name}: {ms:.3f} ms/step over {args.steps} steps")
        print(json.dumps({"profile_workload": w.name, "ms": ms, "steps": args.steps}), flush=True)
        return

    result = {}
    extra = {}
    main_w = WORKLOADS["gqa181m_train"]
    if args.only in ("train", "all"):
        log(f"[bench] fwd+bwd {main_w.name}: steps={args.steps} warmup={args.warmup}")
        ms, per, kern = train_case(main_w, args.steps, args.warmup, trace=True)
        flops = train_flops(main_w)
        tflops = flops / (ms * 1e-3) / 1e12
        result.update(value=tflops, ms_per_step=ms)
        extra["gqa181m_train"] = dict(marker_ms_median=float(np.median(per)),
                                      marker_ms_p90=float(np.percentile(per, 90)),
                                      tflops=tflops, pct_peak=100 * tflops / PEAK_BF16_TFLOPS)
        log(f"[bench] {main_w.name}: {ms:.3f} ms/step  {tflops:.1f} TFLOP/s")
        # Dominant kernel and its algorithmic rate.
        pairs = visible_pairs(main_w.T, main_w.window) * main_w.B * main_w.Hq
        algo_per_pair = {"fwd_bf16": 4 * main_w.D, "bwd_dkdv": 8 * main_w.D, "bwd_dq": 2 * main_w.D}
        kern_ms = {n: (c, t / c) for n, (c, t) in kern.items()}
        extra["kernels_ms"] = {n: round(a, 4) for n, (c, a) in kern_ms.items()}
        dom = max(kern.items(), key=lambda kv: kv[1][1])[0]
        fam = next((f for f in algo_per_pair if dom.startswith(f)), None)
        avg_ms = kern_ms[dom][1]
        roof = {"kernel": dom, "avg_ms": avg_ms}
        if fam is not None:
            achieved = algo_per_pair[fam] * pairs / (avg_ms * 1e-3) / 1e12
            roof.update(bound="mfma", achieved=achieved, peak=PEAK_BF16_TFLOPS, unit="TFLOP/s",
                        frac=achieved / PEAK_BF16_TFLOPS, traffic=measured_traffic(dom),
                        algorithmic_flops_per_launch=algo_per_pair[fam] * pairs)
        result["roofline"] = roof
        # The same step with the split backward (dS stored by dK/dV, dQ from it), for the
        # comparison of the two backward designs.
        log(f"[bench] fwd+bwd {main_w.name} with attn_bwd_split")
        ms_s, per_s, kern_s = train_case(main_w, max(args.steps // 2, 3), 2, trace=True,
                                         split=True)
        extra["gqa181m_train_split_bwd"] = dict(
            ms_per_step=ms_s, tflops=train_flops(main_w) / (ms_s * 1e-3) / 1e12,
            kernels_ms={n: round(t / c, 4) for n, (c, t) in kern_s.items()})
        log(f"[bench] {main_w.name} split backward: {ms_s:.3f} ms/step")
        # MiniGPT shapes: the fp32 forward (B=2, T=128, 6 heads, d=32) and the bf16 training
        # batch (B=32) -- both far too small to fill the GPU; reported per call.
        w1 = WORKLOADS["minigpt_fwd_f32"]
        q1, k1, v1, _ = make_train_inputs(w1)
        t1 = [torch.from_numpy(x).to(dev).contiguous() for x in (q1, k1, v1)]
        o1 = torch.empty_like(t1[0])
        l1 = torch.empty(t1[0].shape[:3], dtype=torch.float32, device=dev)
        opts1 = opts_of(w1)

        def fwd32(_i=0):
            bd.attn_fwd(t1[0], t1[1], t1[2], opts1, out=o1, lse=l1)

        settle(fwd32, 0.2)
        n1 = 200
        us1 = timed(fwd32, n1) / n1 * 1e3
        f1 = 4 * w1.D * visible_pairs(w1.T, w1.window) * w1.B * w1.Hq
        extra["minigpt_fwd_f32"] = dict(us_per_call=us1, tflops=f1 / (us1 * 1e-6) / 1e12,
                                        note="fp32 forward, 12 (b, h) units: launch-bound")
        log(f"[bench] minigpt_fwd_f32: {us1:.1f} us/call")
        w2 = WORKLOADS["minigpt_train_bf16"]
        log(f"[bench] fwd+bwd {w2.name}")
        ms2_, per2_, _ = train_case(w2, max(args.steps, 20), 5)
        tf2_ = train_flops(w2) / (ms2_ * 1e-3) / 1e12
        extra[w2.name] = dict(ms_per_step=ms2_, marker_ms_median=float(np.median(per2_)),
                              tflops=tf2_, pct_peak=100 * tf2_ / PEAK_BF16_TFLOPS,
                              note="192 (b, h) units of T=128: launch-bound")
        log(f"[bench] {w2.name}: {ms2_ * 1e3:.1f} us/step  {tf2_:.1f} TFLOP/s")
        for name in ("flaxchat_full", "flaxchat_w512", "gpt_pretrain_train",
                     "gpt_pretrain_train_dropout", "gpt2xl_instruct_train"):
            w = WORKLOADS[name]
            log(f"[bench] fwd+bwd {name}")
            drop = w.dropout > 0
            ms2, per2, k2 = train_case(w, max(args.steps // 2, 3), 2, trace=drop)
            tf2 = train_flops(w) / (ms2 * 1e-3) / 1e12
            extra[name] = dict(ms_per_step=ms2, marker_ms_median=float(np.median(per2)), tflops=tf2,
                               pct_peak=100 * tf2 / PEAK_BF16_TFLOPS)
            if drop:
                # The mask kernel is integer-ALU work: report its rate in keep decisions per second
                # over the 32 x 32 tiles it fills.
                ktimes = {n: t / c for n, (c, t) in k2.items()}
                tiles = visible_tiles32(w.T, w.window) * w.B * w.Hq
                extra[name].update(
                    dropout=w.dropout, kernels_ms={n: round(a, 4) for n, a in ktimes.items()},
                    mask_gdecisions_per_s=tiles * 1024 / (ktimes["dropout_mask"] * 1e-3) / 1e9)
            log(f"[bench] {name}: {ms2:.3f} ms/step  {tf2:.1f} TFLOP/s")
        # flaxchat's layer pattern: three sliding-window layers per global one.
        wf, ww = WORKLOADS["flaxchat_full"], WORKLOADS["flaxchat_w512"]
        ms_mix = (3 * extra["flaxchat_w512"]["ms_per_step"] + extra["flaxchat_full"]["ms_per_step"]) / 4
        tf_mix = (3 * train_flops(ww) + train_flops(wf)) / 4 / (ms_mix * 1e-3) / 1e12
        extra["flaxchat_sssl_mix"] = dict(ms_per_layer=ms_mix, tflops=tf_mix,
                                          pct_peak=100 * tf_mix / PEAK_BF16_TFLOPS)
        # SFT-style packed rows (segment ids) on the 181M shapes.
        wp = WORKLOADS["gqa181m_sft_packed"]
        ids = make_segment_ids(wp)
        log(f"[bench] fwd+bwd {wp.name}")
        msp, perp, _ = train_case(wp, max(args.steps // 2, 3), 2, ids=ids)
        tfp = packed_flops(wp, ids) / (msp * 1e-3) / 1e12
        extra[wp.name] = dict(ms_per_step=msp, marker_ms_median=float(np.median(perp)), tflops=tfp,
                              pct_peak=100 * tfp / PEAK_BF16_TFLOPS)
        log(f"[bench] {wp.name}: {msp:.3f} ms/step  {tfp:.1f} TFLOP/s")
        torch.cuda.empty_cache()

    if args.copy_mib > 0:
        calibration_copy()

    # ------------------------------------------------------------------------------------
    # decode
    # ------------------------------------------------------------------------------------
    if args.only in ("decode", "all"):
        wd = WORKLOADS["gqa181m_decode"]
        log(f"[bench] decode {wd.name}: {args.decode_iters} calls over {args.decode_copies} cache copies")
        qd, kc, vc, lens = make_decode_inputs(wd)
        tq = to_dev(qd)
        tkc0, tvc0 = to_dev(kc), to_dev(vc)
        del kc, vc
        copies = [(tkc0, tvc0)] + [(tkc0.clone(), tvc0.clone()) for _ in range(args.decode_copies - 1)]
        tl = torch.from_numpy(lens).to(dev)
        od = torch.empty_like(tq)
        opts = opts_of(wd)
        cfg = bd.make_decode_cfg(wd.B, wd.Hq, wd.Hkv, wd.D, wd.T, opts)
        wsd = bd.decode_workspace(wd.B, wd.Hq, wd.Hkv, wd.D, wd.T, opts)
        n = args.decode_iters

        def dec(i):
            kcc, vcc = copies[i % len(copies)]
            bd.attn_decode(tq, kcc, vcc, tl, opts, out=od, workspace=wsd)

        settle(dec)
        for i in range(10):
            dec(i)

        ms_d = timed(dec, n) / n
        per = per_call_ms(dec, n)
        nbytes = decode_bytes(wd, lens)
        gbs = nbytes / (ms_d * 1e-3) / 1e9
        bd.trace_enable(True)
        for i in range(n):
            kcc, vcc = copies[i % len(copies)]
            bd.attn_decode(tq, kcc, vcc, tl, opts, out=od, workspace=wsd)
        torch.cuda.synchronize()
        dk = bd.trace_read()
        bd.trace_enable(False)
        split = {k: round(t / c, 5) for k, (c, t) in dk.items()}
        extra["decode"] = dict(ms_per_call=ms_d, marker_ms_median=float(np.median(per)),
                               marker_ms_p90=float(np.percentile(per, 90)), GBps=gbs,
                               pct_hbm_peak=100 * gbs / PEAK_HBM_GBS, bytes_per_call=nbytes,
                               measured_hbm_bytes_per_call=measured_traffic("decode_split_d96"),
                               kernels_ms=split)
        log(f"[bench] decode: {ms_d * 1e3:.1f} us/call  {gbs:.0f} GB/s")
        # The GPT pretraining page's KV-cache shape (one sequence, 256 cached rows, 12 heads,
        # d 64): latency-bound, reported per call.
        ws = WORKLOADS["gpt_pretrain_decode"]
        qs, kcs, vcs, lens_s = make_decode_inputs(ws)
        tqs, tks, tvs = to_dev(qs), to_dev(kcs), to_dev(vcs)
        tls = torch.from_numpy(lens_s).to(dev)
        os_ = torch.empty_like(tqs)
        opts_s = opts_of(ws)
        cfg_s = bd.make_decode_cfg(ws.B, ws.Hq, ws.Hkv, ws.D, ws.T, opts_s)
        wss = bd.decode_workspace(ws.B, ws.Hq, ws.Hkv, ws.D, ws.T, opts_s)
        for _ in range(10):
            bd.attn_decode(tqs, tks, tvs, tls, opts_s, out=os_, workspace=wss)
        torch.cuda.synchronize()
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        evs[0].record(stream)
        for _ in range(n):
            bd.attn_decode(tqs, tks, tvs, tls, opts_s, out=os_, workspace=wss)
        evs[1].record(stream)
        torch.cuda.synchronize()
        us_s = evs[0].elapsed_time(evs[1]) / n * 1e3
        extra["gpt_pretrain_decode"] = dict(us_per_call=us_s,
                                            GBps=decode_bytes(ws, lens_s) / (us_s * 1e-6) / 1e9)
        log(f"[bench] gpt_pretrain_decode: {us_s:.1f} us/call")
        # Left-padded batch (right-aligned caches of 2048 rows, U{256..2048} real rows each),
        # over the same number of cache copies as the plain decode.
        wl = WORKLOADS["gqa181m_decode_leftpad"]
        ql, kcl, vcl, starts_l, lens_l = make_leftpad_decode_inputs(wl)
        tql = to_dev(ql)
        tkl0, tvl0 = to_dev(kcl), to_dev(vcl)
        del kcl, vcl
        copies_l = [(tkl0, tvl0)] + [(tkl0.clone(), tvl0.clone())
                                     for _ in range(args.decode_copies - 1)]
        tll, tsl = torch.from_numpy(lens_l).to(dev), torch.from_numpy(starts_l).to(dev)
        ol = torch.empty_like(tql)
        opts_l = opts_of(wl)
        cfg_l = bd.make_decode_cfg(wl.B, wl.Hq, wl.Hkv, wl.D, wl.T, opts_l)
        wsl = bd.decode_workspace(wl.B, wl.Hq, wl.Hkv, wl.D, wl.T, opts_l)

        def dec_l(i):
            kcc, vcc = copies_l[i % len(copies_l)]
            bd.attn_decode(tql, kcc, vcc, tll, opts_l, out=ol, workspace=wsl, cache_start=tsl)

        for i in range(10):
            dec_l(i)
        torch.cuda.synchronize()
        evl = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        evl[0].record(stream)
        for i in range(n):
            dec_l(i)
        evl[1].record(stream)
        torch.cuda.synchronize()
        ms_l = evl[0].elapsed_time(evl[1]) / n
        gbs_l = decode_bytes(wl, lens_l - starts_l) / (ms_l * 1e-3) / 1e9
        extra[wl.name] = dict(us_per_call=ms_l * 1e3, GBps=gbs_l,
                              pct_hbm_peak=100 * gbs_l / PEAK_HBM_GBS)
        log(f"[bench] {wl.name}: {ms_l * 1e3:.1f} us/call  {gbs_l:.0f} GB/s")
        del copies_l, tkl0, tvl0
        torch.cuda.empty_cache()
        # Multi-token step (append + attend) on decode-sized caches.
        we = WORKLOADS["gqa181m_extend"]
        qe, kne, vne, kce, vce, lens_e = make_extend_inputs(we)
        tqe, tkne, tvne, tkce, tvce = (to_dev(x) for x in (qe, kne, vne, kce, vce))
        tle = torch.from_numpy(lens_e).to(dev)
        oe = torch.empty_like(tqe)
        opts_e = opts_of(we)
        for _ in range(5):
            bd.attn_extend(tqe, tkne, tvne, tkce, tvce, tle, opts_e, out=oe)
        torch.cuda.synchronize()
        evs[0].record(stream)
        for _ in range(n):
            bd.attn_extend(tqe, tkne, tvne, tkce, tvce, tle, opts_e, out=oe)
        evs[1].record(stream)
        torch.cuda.synchronize()
        us_e = evs[0].elapsed_time(evs[1]) / n * 1e3
        tf_e = extend_flops(we, lens_e) / (us_e * 1e-6) / 1e12
        extra["gqa181m_extend"] = dict(us_per_call=us_e, tflops=tf_e,
                                       pct_peak=100 * tf_e / PEAK_BF16_TFLOPS)
        log(f"[bench] gqa181m_extend: {us_e:.1f} us/call  {tf_e:.1f} TFLOP/s")
        if "value" not in result:
            result.update(value=gbs, ms_per_step=ms_d)

    # ------------------------------------------------------------------------------------
    # CPU oracle on a bounded sample
    # ------------------------------------------------------------------------------------
    cpu = None
    if not args.no_cpu_baseline and args.only in ("train", "all"):
        from oracle import attention_backward, attention_decode, attention_forward
        try:
            from threadpoolctl import threadpool_info, threadpool_limits
            pools = [d for d in threadpool_info() if d.get("user_api") == "blas"]
        except Exception:  # threadpoolctl missing: no BLAS metadata, no single-core leg
            threadpool_limits, pools = None, []
        threads = max([d.get("num_threads", 1) for d in pools] or [1])
        blas = [{"library": d.get("internal_api"), "version": d.get("version"),
                 "threads": d.get("num_threads")} for d in pools]

        def okw(w):
            return dict(window=w.window, softcap=w.softcap, rope=w.rope, rope_base=w.rope_base,
                        qk_norm=w.qk_norm, norm_eps=w.norm_eps)

        def run_for(seconds, fn):
            """Call fn(i) for i = 0, 1, ... until `seconds` have passed; (calls, elapsed)."""
            t0, n = time.perf_counter(), 0
            while True:
                fn(n)
                n += 1
                el = time.perf_counter() - t0
                if el >= seconds:
                    return n, el

        # The 181M workload: (batch, KV-group) slices, fwd + bwd.
        w = main_w
        q, k, v, dO = make_train_inputs(w)
        G = w.Hq // w.Hkv
        kw = okw(w)

        def slice_181m(i):
            b, g = i % w.B, (i // w.B) % w.Hkv
            hs = slice(g * G, (g + 1) * G)
            attention_forward(q[b:b + 1, hs], k[b:b + 1, g:g + 1], v[b:b + 1, g:g + 1], **kw)
            attention_backward(q[b:b + 1, hs], k[b:b + 1, g:g + 1], v[b:b + 1, g:g + 1],
                               dO[b:b + 1, hs], **kw)

        units, el = run_for(args.cpu_seconds, slice_181m)
        slice_flops = train_flops(w.with_(B=1, Hq=G, Hkv=1))
        cpu = {"value": slice_flops * units / el / 1e12, "unit": "TFLOP/s", "cores": int(threads),
               "kind": "oracle",
               "sample": f"{units} (batch, KV-group) slices of {w.name} (1 x {G} query heads x "
                         f"T={w.T} x d={w.D}) fwd+bwd in {el:.1f} s",
               "host": {"os_cpu_count": os.cpu_count(), "blas": blas,
                        "threads_used": int(threads),
                        "note": "numpy fp64; the BLAS pool's threads run the matrix products, "
                                "the rest of the oracle is one Python thread"}}
        if threadpool_limits is not None:
            with threadpool_limits(limits=1):
                n1, el1 = run_for(args.cpu_seconds / 3, slice_181m)
            cpu["single_core"] = {"value": slice_flops * n1 / el1 / 1e12, "unit": "TFLOP/s",
                                  "cores": 1, "sample": f"{n1} slices in {el1:.1f} s"}
        log(f"[bench] cpu oracle: {cpu['value'] * 1e3:.3f} GFLOP/s over {units} slices")

        # The other configurations, whole, beside their GPU lines (all host threads).
        per = {}
        w1 = WORKLOADS["minigpt_fwd_f32"]
        a1 = make_train_inputs(w1)
        n, el = run_for(1.0, lambda i: attention_forward(*a1[:3], **okw(w1)))
        f1 = 4 * w1.D * visible_pairs(w1.T, w1.window) * w1.B * w1.Hq
        per[w1.name] = {"us_per_call": el / n * 1e6, "TFLOP/s": f1 * n / el / 1e12,
                        "sample": f"{n} whole forwards in {el:.1f} s"}
        w2 = WORKLOADS["minigpt_train_bf16"]
        a2 = make_train_inputs(w2)

        def fb2(i):
            attention_forward(*a2[:3], **okw(w2))
            attention_backward(*a2, **okw(w2))

        n, el = run_for(3.0, fb2)
        per[w2.name] = {"ms_per_step": el / n * 1e3, "TFLOP/s": train_flops(w2) * n / el / 1e12,
                        "sample": f"{n} whole fwd+bwd steps in {el:.1f} s"}
        wdec = WORKLOADS["gqa181m_decode"]
        qdd, kcd, vcd, lensd = make_decode_inputs(wdec)
        dkw = {x: y for x, y in okw(wdec).items() if x != "window"}
        n, el = run_for(3.0, lambda i: attention_decode(qdd, kcd, vcd, lensd, **dkw))
        per[wdec.name] = {"us_per_call": el / n * 1e6,
                        "GB/s": decode_bytes(wdec, lensd) * n / el / 1e9,
                        "sample": f"{n} whole decode calls (64 sequences) in {el:.1f} s"}
        cpu["per_config"] = per
        log(f"[bench] cpu oracle per config: {per}")

    line = {
        "metric": METRIC,
        "value": result.get("value"),
        "unit": "TFLOP/s" if args.only in ("train", "all") else "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": result.get("ms_per_step"),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{main_w.name}: fwd+bwd, B={main_w.B} T={main_w.T} Hq={main_w.Hq} "
                               f"Hkv={main_w.Hkv} d={main_w.D} causal RoPE QK-norm softcap "
                               f"{main_w.softcap:g}",
                   "global_batch": main_w.B, "seq_len": main_w.T, "parallelism": "single GPU"},
        "pct_of_peak": (100 * result["value"] / PEAK_BF16_TFLOPS
                        if args.only in ("train", "all") and result.get("value") else None),
        "device": {"name": props.name, "arch": getattr(props, "gcnArchName", None),
                   "cu": dinfo["compute_units"], "clock_mhz": dinfo["clock_khz"] / 1e3,
                   "bf16_dense_tflops_from_device": dinfo["bf16_dense_tflops"],
                   "mem_clock_mhz": dinfo["mem_clock_khz"] / 1e3,
                   "mem_bus_bits": dinfo["mem_bus_bits"]},
        "peaks_used": {"bf16_tflops": PEAK_BF16_TFLOPS, "hbm_gbs": PEAK_HBM_GBS,
                       "source": "MI355X published dense figures"},
        "roofline": result.get("roofline"),
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
