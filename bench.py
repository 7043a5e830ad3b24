#!/usr/bin/env python3
"""Benchmark of the ALiBi attention hot path on one MI355X.

One step = one pass over both hot-path kernels on resident inputs:
  * the fused causal ALiBi forward, bf16, B=8 H=16 N=4096 d=128 (the N=4096,
    d=128 performance shape), and
  * the split-KV decode, bf16, B=32 H=32 L=32768 d=128.
`value` is the forward's TFLOP/s (algorithmic causal flops including the
diagonal, 4 d B H N (N+1) / 2, divided by the forward's own HIP-event time over
the timed steps); the decode's GB/s (K + V + q + out bytes over its own event
time) is reported under "decode". Both carry a roofline object against the
MI355X datasheet peaks (bf16 dense MFMA 2.5 PFLOP/s, HBM 8 TB/s). Beside
the forward's peak, `roofline.mfma_ceiling` reports the matrix rate the part
sustains (back-to-back register-fed bf16 MFMAs, measured in the same run): the
shader clock drops under sustained matrix load, so this is below the datasheet
figure, and the forward's fraction of it is reported too;
`roofline.mfma_valu_ceiling` adds the forward's per-MFMA softmax vector work to
those MFMAs (the forward's instruction mix, without memory or stalls).

After the timed steps, "next" reports the forward's other forms on the same
inputs, each timed on its own (HIP events, after its own warmup): the Sec. 3.4
mitigations of "When Attention Goes Blind" (bias floor -87, ln(D + 1)
distances, soft cap 50; singly and all together), the symmetric non-causal
bias, a chunked prefill (the last 512 query rows against the 4096-key
cache through position offsets), hard per-head windows (Sec. 5.2-5.3; each
head's window is where its bias reaches the fp32 denormal limit, rated on the
in-window flops), and the exact underflow skipping (its rate
counts the unskipped causal flops, so it is an effective rate, reported apart
from the headline; the same skipping in the decode, rated on the whole
cache's bytes), and the backward pass (dq, dk, dv from the forward's
log-sum-exp; 2.5x the forward's flops: five GEMMs of the causal triangle). Their flops are the algorithmic ones of each
form: the causal triangle for the mitigations, N^2 without the mask, and the
visible keys of the 512 rows for the prefill.

"configs" reports the plain causal forward at the other configurations of the
workload table (B8 H8 N1024 d64, B4 H12 N2048 d64, B1 H16 N16384 d128), each
over back-to-back launches of the C entry point, with the form the library
picks (alibi_debug_fwd_form: waves per workgroup, or the key-range split).

The CPU baseline is the fp64 oracle itself, timed on this host's cores on a
bounded sample (whole heads of the same forward, whole (b, h) pairs of the
same decode), scaled to the same units.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
    python bench.py --only fwd|decode|copy|bwd|mfma|mfma_valu [--steps K] [--warmup W]
    python bench.py --only underflow     (CPU only: the bf16 underflow diagnostic
                                          of the 16384-token workload, fp64 oracle)

`--only` runs a single kernel (`bwd`: the three backward kernels; `copy`: a
plain device-to-device copy of
a 1 GiB bf16 tensor; `mfma`, `mfma_valu`: the register-fed MFMA-rate kernel,
alone or with the forward's per-MFMA vector mix) so that
hardware-counter runs see one kernel; it prints a
short JSON line and no CPU baseline. The copy calibrates the HBM byte counters.
"""
import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)
sys.path.insert(0, os.path.join(ROOT, "tests"))

PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0


def fwd_flops(B, H, N, d):
    return 4.0 * d * B * H * N * (N + 1) / 2.0


def decode_bytes(B, H, L, d):
    return 2.0 * B * H * L * d * 2 + 2.0 * B * H * d * 2


def fwd_kernel_name(alibi, B, H, N, d):
    """The forward instantiation the library launches for the plain causal call."""
    f = alibi.fwd_form(B, H, N, N, d)
    return f"fwd_mfma_kernel<{d},8,true,0,false,2>" if f == 2 else f"fwd_mfma_kernel<{d},{f},true,0,false,1>"


def traffic_bytes(profile_md, sources, root=ROOT):
    """HBM bytes per launch from a committed counter summary, or None.

    The summary under profiles/ carries a `traffic_record` line with the kernel
    source hash it was measured on; a changed kernel gets None.
    """
    import hashlib
    path = os.path.join(root, "profiles", profile_md)
    try:
        rec = None
        for line in open(path):
            if line.strip().startswith("traffic_record:"):
                rec = json.loads(line.split("traffic_record:", 1)[1])
        if rec is None:
            return None
        h = hashlib.sha256()
        for f in sources:
            h.update(open(os.path.join(root, "alibi_linear_position_amd", "csrc", f), "rb").read())
        return rec["traffic_bytes"] if h.hexdigest()[:16] == rec["source_sha256_16"] else None
    except (OSError, ValueError, KeyError):
        return None


def cpu_baseline(q, k, v, kc, vc, qd, fwd_wl, dec_wl, budget_s=12.0):
    """Time the oracle on whole heads / (b, h) pairs of the bench workloads."""
    import numpy as np
    import torch
    import oracle
    threads = len(os.sched_getaffinity(0))
    s_f = oracle.slopes_ref(fwd_wl.H)
    heads = 0
    t_f = 0.0
    while t_f < budget_s and heads < fwd_wl.B * fwd_wl.H:
        b, h = divmod(heads, fwd_wl.H)
        qq, kk, vv = (x[b, h].to(torch.float64).numpy() for x in (q, k, v))
        t0 = time.perf_counter()
        oracle.attn_head_ref(qq, kk, vv, float(s_f[h]), causal=True)
        t_f += time.perf_counter() - t0
        heads += 1
    fwd_rate = fwd_flops(1, heads, fwd_wl.N, fwd_wl.d) / t_f / 1e12
    s_d = oracle.slopes_ref(dec_wl.H)
    pairs = 0
    t_d = 0.0
    while t_d < budget_s / 2 and pairs < dec_wl.B * dec_wl.H:
        b, h = divmod(pairs, dec_wl.H)
        qq = qd[b:b + 1, h:h + 1].cpu()
        kk = kc[b:b + 1, h:h + 1].cpu()
        vv = vc[b:b + 1, h:h + 1].cpu()
        t0 = time.perf_counter()
        oracle.decode_ref(qq, kk, vv, s_d[h:h + 1])
        t_d += time.perf_counter() - t0
        pairs += 1
    dec_rate = decode_bytes(1, pairs, dec_wl.L, dec_wl.d) / t_d / 1e9
    return {
        "value": fwd_rate, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
        "sample": f"{heads} of {fwd_wl.B * fwd_wl.H} (b,h) heads of the N={fwd_wl.N} d={fwd_wl.d} "
                  f"causal forward, fp64 numpy, {t_f:.1f} s",
        "decode": {"value": dec_rate, "unit": "GB/s",
                   "sample": f"{pairs} of {dec_wl.B * dec_wl.H} (b,h) pairs of the L={dec_wl.L} decode, "
                             f"{t_d:.1f} s (host copies excluded)"},
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", choices=["fwd", "fwd16k", "c1", "c2", "c3", "decode", "copy", "bwd", "bwd_skip", "mfma",
                                       "mfma_valu", "oracle", "underflow"], default=None)
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the library has no multi-GPU path)", file=sys.stderr)
        sys.exit(2)

    import workloads as W
    if args.only == "underflow":  # the oracle's diagnostic: CPU only, no library
        return underflow_report(W)
    import torch
    import alibi_linear_position_amd as alibi

    alibi.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    fw = W.FWD_B8_H16_N4096_D128
    dw = W.DECODE_B32_H32_L32768_D128
    if args.only is not None:
        return run_only(args, alibi, W, fw, dw, dev)

    q, k, v = W.gaussian_qkv_bf16(fw.shape, seed=fw.seed)
    qg, kg, vg = (x.to(dev) for x in (q, k, v))
    out = torch.empty_like(qg)
    s_f = alibi.slopes(fw.H).to(dev)
    kc = W.device_gaussian_bf16((dw.B, dw.H, dw.L, dw.d), seed=dw.seed)
    vc = W.device_gaussian_bf16((dw.B, dw.H, dw.L, dw.d), seed=dw.seed + 1)
    qd = W.device_gaussian_bf16((dw.B, dw.H, dw.d), seed=dw.seed + 2)
    od = torch.empty_like(qd)
    s_d = alibi.slopes(dw.H).to(dev)
    torch.cuda.synchronize()

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        alibi.attn_fwd(qg, kg, vg, s_f, causal=True, out=out)
        if ev is not None:
            ev[1].record()
        alibi.attn_decode(qd, kc, vc, s_d, out=od)
        if ev is not None:
            ev[2].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    t_fwd = sum(e[0].elapsed_time(e[1]) for e in events) / args.steps / 1e3  # s per launch
    t_dec = sum(e[1].elapsed_time(e[2]) for e in events) / args.steps / 1e3
    flops = fwd_flops(fw.B, fw.H, fw.N, fw.d)
    nbytes = decode_bytes(dw.B, dw.H, dw.L, dw.d)
    tflops = flops / t_fwd / 1e12
    gbs = nbytes / t_dec / 1e9
    assert torch.isfinite(out.float()).all() and torch.isfinite(od.float()).all()
    read_gbs = read_ceiling(alibi, (kc, vc), dev)
    mfma_tflops = mfma_ceiling(alibi, dev, lambda: alibi.attn_decode(qd, kc, vc, s_d, out=od))
    mix_tflops = mfma_ceiling(alibi, dev, lambda: alibi.attn_decode(qd, kc, vc, s_d, out=od), valu=1)

    res = {
        "metric": "causal ALiBi attn fwd TFLOP/s (bf16) + decode HBM GB/s, 1xMI355X",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{fw.name} + {dw.name}", "fwd": {"B": fw.B, "H": fw.H, "N": fw.N, "d": fw.d,
                                                                "causal": True},
                   "decode": {"B": dw.B, "H": dw.H, "L": dw.L, "d": dw.d}},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic_bytes("fwd_mfma_B8_H16_N4096_d128.md", ["fwd_mfma.hip", "device_common.h"]),
                     "kernel": fwd_kernel_name(alibi, fw.B, fw.H, fw.N, fw.d),
                     "ms_per_launch": round(t_fwd * 1e3, 4),
                     "per_launch": f"{flops:.4e} flop",
                     "mfma_ceiling": {"value": round(mfma_tflops, 1), "unit": "TFLOP/s",
                                      "kernel": "mfma_rate_kernel",
                                      "frac": round(tflops / mfma_tflops, 4),
                                      "note": "back-to-back register-fed 32x32x16 bf16 MFMAs on every SIMD "
                                              "(two waves per SIMD, random N(0,1) operands, no memory "
                                              "traffic), timed in ~0.5 ms launches each followed by the "
                                              "decode, as the forward runs in the step: the rate the part "
                                              "sustains, below the datasheet peak because the shader clock "
                                              "drops under sustained matrix load; context, not the peak"},
                     "mfma_valu_ceiling": {"value": round(mix_tflops, 1), "unit": "TFLOP/s",
                                           "kernel": "mfma_rate_kernel (valu)",
                                           "frac": round(tflops / mix_tflops, 4),
                                           "note": "the same MFMAs, each joined by the vector work the "
                                                   "forward's softmax issues per MFMA (fma, exponential, half "
                                                   "a bf16 pack, half a bf16 dot, an add) on independent data: "
                                                   "the forward's instruction mix without its memory traffic "
                                                   "or dependency stalls; context, not the peak"}},
        "decode": {"value": round(gbs, 1), "unit": "GB/s",
                   "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                                "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                                "traffic": traffic_bytes("decode_split_B32_H32_L32768_d128.md",
                                                         ["decode.hip", "device_common.h"]),
                                "kernel": "decode_split_kernel<16>", "ms_per_launch": round(t_dec * 1e3, 4),
                                "per_launch": f"{nbytes:.4e} B",
                                "read_ceiling": {"value": round(read_gbs, 1), "unit": "GB/s",
                                                 "kernel": "stream_read_kernel",
                                                 "note": "plain streaming read of the same K and V caches the "
                                                         "way the decode reads them (a contiguous slab per "
                                                         "workgroup, non-temporal 16-byte loads, 8 in flight "
                                                         "per thread); context, not the peak"}}},
        "cpu_baseline": None,
    }
    res["next"] = next_forms(alibi, qg, kg, vg, s_f, fw)
    res["next"]["decode_skip_underflow"] = decode_skip_rate(alibi, qd, kc, vc, s_d, dw)
    res["configs"] = config_rates(alibi, W, dev, (qg, kg, vg, s_f))
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(q, k, v, kc, vc, qd, fw, dw)
    print(json.dumps(res), flush=True)


def config_rates(alibi, W, dev, warm_args):
    """The plain forward at the other configurations of the workload table, each
    timed over back-to-back launches of the C entry point (HIP events), with the
    form the library picks for it. The headline forward runs between them so the
    clock stays up."""
    import ctypes
    import torch
    lib = alibi.load_library()
    P = ctypes.c_void_p
    st = P(torch.cuda.current_stream(dev).cuda_stream)
    res = {}
    for wl, reps in ((W.FWD_B8_H8_N1024_D64, 400), (W.FWD_B4_H12_N2048_D64, 200), (W.FWD_B1_H16_N16384_D128, 20)):
        q, k, v = (x.to(dev) for x in W.gaussian_qkv_bf16(wl.shape, seed=wl.seed))
        out = torch.empty_like(q)
        s = alibi.slopes(wl.H).to(dev)
        args = (P(q.data_ptr()), P(k.data_ptr()), P(v.data_ptr()), P(out.data_ptr()), wl.B, wl.H, wl.N, wl.d,
                P(s.data_ptr()), 1, st)
        for _ in range(20):  # clock up
            alibi.attn_fwd(*warm_args[:3], warm_args[3], causal=True)
        for _ in range(10):
            assert lib.alibi_attn_fwd(*args) == 0
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            lib.alibi_attn_fwd(*args)
        e1.record()
        torch.cuda.synchronize()
        assert torch.isfinite(out.float()).all()
        ms = e0.elapsed_time(e1) / reps
        flops = fwd_flops(wl.B, wl.H, wl.N, wl.d)
        f = alibi.fwd_form(wl.B, wl.H, wl.N, wl.N, wl.d)
        form = "key-range split, 8 waves" if f == 2 else f"{f} waves"
        res[wl.name] = {"value": round(flops / ms / 1e9, 1), "unit": "TFLOP/s", "ms_per_launch": round(ms, 5),
                        "frac": round(flops / ms / 1e9 / PEAK_BF16_TFLOPS, 4), "form": form,
                        "launches": reps}
        del q, k, v, out
    return res


def time_launches(fn, warmup=10, reps=10):
    """Mean ms per call of fn over `reps` calls after `warmup` calls (HIP events)."""
    import torch
    for _ in range(warmup):
        fn()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def next_forms(alibi, q, k, v, s, fw):
    """TFLOP/s of the forward's mitigation, non-causal and chunked-prefill forms."""
    import torch
    B, H, N, d = fw.B, fw.H, fw.N, fw.d
    causal_flops = fwd_flops(B, H, N, d)
    out = torch.empty_like(q)
    forms = {
        "clamp": dict(clamp=-87.0),
        "log_distance": dict(log_distance=True),
        "softcap": dict(softcap=50.0),
        "clamp+log+softcap": dict(clamp=-87.0, log_distance=True, softcap=50.0),
    }
    res = {}
    for name, kw in forms.items():
        ms = time_launches(lambda: alibi.attn_fwd_ex(q, k, v, s, True, out=out, **kw))
        res[name] = {"value": round(causal_flops / ms / 1e9, 1), "unit": "TFLOP/s", "ms": round(ms, 4)}
    ms = time_launches(lambda: alibi.attn_fwd(q, k, v, s, causal=False, out=out))
    res["non_causal"] = {"value": round(4.0 * d * B * H * N * N / ms / 1e9, 1), "unit": "TFLOP/s",
                         "ms": round(ms, 4)}
    ms = time_launches(lambda: alibi.attn_fwd_ex(q, k, v, s, False, skip_underflow=True, out=out))
    res["non_causal_skip_underflow"] = {"value": round(4.0 * d * B * H * N * N / ms / 1e9, 1),
                                        "unit": "TFLOP/s (unskipped flops)", "ms": round(ms, 4),
                                        "note": "the symmetric bias -m|i-j| with exact skipping on both sides of "
                                                "each query block; key-norm pass included"}
    ms = time_launches(lambda: alibi.attn_fwd_ex(q, k, v, s, True, skip_underflow=True, out=out))
    res["skip_underflow"] = {"value": round(causal_flops / ms / 1e9, 1), "unit": "TFLOP/s (causal flops)",
                             "ms": round(ms, 4),
                             "note": "exact skipping of all-underflow key tiles; key-norm pass included; "
                                     "flops are the unskipped causal count, so this is not the headline"}
    # hard per-head windows of "When Attention Goes Blind", Sec. 5.2-5.3: each
    # head's window is the distance at which its bias alone reaches the fp32
    # denormal limit, ceil(126 ln 2 / m_h) tokens (124 for the steepest head)
    sl = s.detach().cpu().double().tolist()
    wins = [min(N, int(math.ceil(126.0 * math.log(2.0) / m))) for m in sl]
    wt = torch.tensor(wins, dtype=torch.int32, device=q.device)
    ms = time_launches(lambda: alibi.attn_fwd_ex(q, k, v, s, True, out=out, window=wt))
    vis = sum(sum(min(i + 1, w) for i in range(N)) for w in wins) * B
    res["window_blindness"] = {"value": round(4.0 * d * vis / ms / 1e9, 1), "unit": "TFLOP/s (in-window flops)",
                               "ms": round(ms, 4), "causal_equivalent": round(causal_flops / ms / 1e9, 1),
                               "windows": wins,
                               "note": "hard per-head windows (changes results: weights outside the window are "
                                       "dropped); key tiles wholly out of a wave's window are skipped"}
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    alibi.attn_fwd_ex(q, k, v, s, True, out=out, lse=lse)
    dout = torch.randn(q.shape, generator=torch.Generator(device=q.device).manual_seed(7), device=q.device,
                       dtype=torch.float32).to(torch.bfloat16)
    ms = time_launches(lambda: alibi.attn_bwd(q, k, v, out, dout, lse, s, True), warmup=5, reps=10)
    res["backward"] = {"value": round(2.5 * causal_flops / ms / 1e9, 1), "unit": "TFLOP/s", "ms": round(ms, 4),
                       "note": "dq, dk, dv; flops = 5 causal GEMMs (S, dP, dV, dK, dQ) = 2.5x the forward's"}
    grads = []

    def bwd_skip():
        grads[:] = alibi.attn_bwd(q, k, v, out, dout, lse, s, True, skip_underflow=True)

    ms = time_launches(bwd_skip, warmup=5, reps=10)
    ref = alibi.attn_bwd(q, k, v, out, dout, lse, s, True)
    torch.cuda.synchronize()
    same = all(bool(torch.equal(a.view(torch.int16), b.view(torch.int16))) for a, b in zip(grads, ref))
    res["backward_skip_underflow"] = {
        "value": round(2.5 * causal_flops / ms / 1e9, 1), "unit": "TFLOP/s (unskipped causal flops)",
        "ms": round(ms, 4), "bitwise_equal_to_backward": same,
        "note": "exact skipping of query-key tiles whose every P rounds to zero (bound from the per-(b,h) "
                "maxima of |q| and |k|, whose pass is included); flops are the unskipped count, so this is "
                "an effective rate"}
    lse2 = torch.empty_like(lse)
    out2 = torch.empty_like(q)
    alibi.attn_fwd_ex(q, k, v, s, True, out=out2, lse=lse2, clamp=-87.0, log_distance=True)
    ms = time_launches(lambda: alibi.attn_bwd(q, k, v, out2, dout, lse2, s, True, clamp=-87.0, log_distance=True),
                       warmup=5, reps=10)
    res["backward_clamp+log"] = {"value": round(2.5 * causal_flops / ms / 1e9, 1), "unit": "TFLOP/s",
                                 "ms": round(ms, 4),
                                 "note": "the backward of the clamp (-87) with log-scaled distances; bias per score"}
    alibi.attn_fwd_ex(q, k, v, s, True, out=out2, lse=lse2, softcap=50.0)
    ms = time_launches(lambda: alibi.attn_bwd(q, k, v, out2, dout, lse2, s, True, softcap=50.0), warmup=5, reps=10)
    res["backward_softcap"] = {"value": round(2.5 * causal_flops / ms / 1e9, 1), "unit": "TFLOP/s",
                               "ms": round(ms, 4),
                               "note": "the backward of the soft cap z = 50: tanh per score, dS scaled by 1 - tanh^2"}
    nq = 512
    qc = q[:, :, N - nq:].contiguous()
    oc = torch.empty_like(qc)
    ms = time_launches(lambda: alibi.attn_fwd_ex(qc, k, v, s, True, q_offset=N - nq, out=oc))
    vis = sum(N - nq + r + 1 for r in range(nq))
    res["chunked_prefill_512_of_4096"] = {"value": round(4.0 * d * B * H * vis / ms / 1e9, 1),
                                          "unit": "TFLOP/s", "ms": round(ms, 4)}
    return res


def decode_skip_rate(alibi, qd, kc, vc, s_d, dw, warmup=5, steps=20):
    """The decode with exact underflow skipping at the decode workload: its
    effective rate (the unskipped K + V + q + out bytes over its time), the
    key-norm pass that supplies the bound timed apart (a serving cache keeps the
    bound as it appends keys), and a bitwise check against the plain decode."""
    import torch
    kn = alibi.key_norm_max(kc)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    kn = alibi.key_norm_max(kc)
    e1.record()
    torch.cuda.synchronize()
    t_norm = e0.elapsed_time(e1) * 1e-3
    out = torch.empty_like(qd)
    fn = lambda: alibi.attn_decode_ex(qd, kc, vc, s_d, skip_underflow=True, key_norm_max=kn, out=out)
    ms = time_launches(fn, warmup=warmup, reps=steps)
    ref = alibi.attn_decode(qd, kc, vc, s_d)
    torch.cuda.synchronize()
    same = bool(torch.equal(out.view(torch.int16), ref.view(torch.int16)))
    nbytes = decode_bytes(dw.B, dw.H, dw.L, dw.d)
    return {"value": round(nbytes / (ms * 1e-3) / 1e9, 1), "unit": "GB/s (unskipped bytes)", "ms": round(ms, 4),
            "bitwise_equal_to_decode": same, "key_norm_pass_ms": round(t_norm * 1e3, 4),
            "note": "exact skipping of cached keys whose weights round to zero (Cauchy-Schwarz bound with a "
                    "per-(b,h) key-norm bound from alibi_key_norm_max, computed once outside the timed "
                    "calls); the rate counts every cached byte, so it is an effective rate, not the headline"}


def read_ceiling(alibi, tensors, dev, workgroups=4096, warmup=2, steps=5):
    """GB/s of a plain streaming read (16-byte loads, every byte once) over the
    given device tensors: the practical read ceiling beside the decode's rate."""
    import torch
    lib = alibi.load_library()
    sink = torch.empty(workgroups, dtype=torch.int32, device=dev)
    st = torch.cuda.current_stream().cuda_stream
    nbytes = sum(t.numel() * t.element_size() for t in tensors)

    def once():
        for t in tensors:
            rc = lib.alibi_debug_stream_read(t.data_ptr(), t.numel() * t.element_size(), sink.data_ptr(),
                                             workgroups, st)
            assert rc == 0, rc

    for _ in range(warmup):
        once()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        once()
    e1.record()
    torch.cuda.synchronize()
    return nbytes * steps / (e0.elapsed_time(e1) * 1e-3) / 1e9


def mfma_ceiling(alibi, dev, between, valu=0, workgroups=1024, iters=160, warmup=5, steps=20):
    """TFLOP/s of back-to-back register-fed bf16 MFMAs on every SIMD (two waves
    per SIMD, random N(0, 1) operands like the forward's): the matrix rate the
    part sustains, beside the forward's rate; with valu=1 each MFMA is joined by
    the forward's per-MFMA softmax vector work on independent data. Timed the
    way the benchmark step runs the forward: launches of ~0.5 ms, each followed
    by `between` (the decode), only the MFMA launches inside the events."""
    import torch
    lib = alibi.load_library()
    g = torch.Generator(device=dev)
    g.manual_seed(7)
    frags = torch.randn(8 * 64 * 8, generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
    sink = torch.empty(8 * workgroups, dtype=torch.float32, device=dev)
    st = torch.cuda.current_stream().cuda_stream

    def once():
        rc = lib.alibi_debug_mfma_rate(frags.data_ptr(), iters, valu, sink.data_ptr(), workgroups, st)
        assert rc == 0, rc

    for _ in range(warmup):
        once()
        between()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for e0, e1 in ev:
        e0.record()
        once()
        e1.record()
        between()
    torch.cuda.synchronize()
    secs = sum(e0.elapsed_time(e1) for e0, e1 in ev) * 1e-3
    flops = float(workgroups) * 8 * iters * 16 * 32768.0
    return flops * steps / secs / 1e12


def oracle_timing(W, dw, dev):
    """The fp64 oracle timed per configuration on this host's cores (a reported
    baseline, not the target): the tiny fp32 case and the two d = 64 forwards
    (also single-threaded), the 16384-token forward and the decode (host copies
    excluded), each whole."""
    import numpy as np
    import torch
    import oracle
    from threadpoolctl import threadpool_limits
    threads = len(os.sched_getaffinity(0))
    model = "unknown"
    with open("/proc/cpuinfo") as f:
        for line in f:
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    res = {"only": "oracle", "cpu": model, "threads": threads, "cases": []}

    def timed(fn, reps):
        ts = []
        for _ in range(reps):
            t0 = time.perf_counter()
            fn()
            ts.append(time.perf_counter() - t0)
        return float(np.median(ts))

    def record(name, seconds, work, unit, nthreads, note):
        rate = work / seconds / (1e9 if unit == "GB/s" else 1e9)
        res["cases"].append({"case": name, "seconds": round(seconds, 4), "rate": round(rate, 4), "unit": unit,
                             "threads": nthreads, "note": note})
        print(f"[oracle] {name}: {seconds:.3f} s, {rate:.4g} {unit}, {nthreads} threads", flush=True)

    q, k, v = W.tiny_example_qkv()
    s4 = oracle.slopes_ref(4)
    for nt in (threads, 1):
        with threadpool_limits(nt):
            t = timed(lambda: oracle.attn_ref(q[None], k[None], v[None], s4, causal=True), 3)
        record("tiny fp32 B1 H4 N8 d16", t, fwd_flops(1, 4, 8, 16), "GFLOP/s", nt, "median of 3")
    for wl, reps1 in ((W.FWD_B8_H8_N1024_D64, 3), (W.FWD_B4_H12_N2048_D64, 1)):
        qq, kk, vv = (x.to(torch.float64).numpy() for x in W.gaussian_qkv_bf16(wl.shape, seed=wl.seed))
        sl = oracle.slopes_ref(wl.H)
        for nt, reps in ((threads, 3), (1, reps1)):
            with threadpool_limits(nt):
                t = timed(lambda: oracle.attn_ref(qq, kk, vv, sl, causal=True), reps)
            record(wl.name, t, fwd_flops(wl.B, wl.H, wl.N, wl.d), "GFLOP/s", nt, f"median of {reps}")
    wl = W.FWD_B1_H16_N16384_D128
    qq, kk, vv = (x[0].to(torch.float64).numpy() for x in W.gaussian_qkv_bf16(wl.shape, seed=wl.seed))
    sl = oracle.slopes_ref(wl.H)
    total = 0.0
    for h in range(wl.H):  # one head at a time: each materialises 16384 x 16384 fp64 matrices
        t0 = time.perf_counter()
        oracle.attn_head_ref(qq[h], kk[h], vv[h], float(sl[h]), causal=True)
        total += time.perf_counter() - t0
        print(f"[oracle] {wl.name} head {h}: {time.perf_counter() - t0:.2f} s", flush=True)
    record(wl.name, total, fwd_flops(wl.B, wl.H, wl.N, wl.d), "GFLOP/s", threads, "1 run")
    kc = W.device_gaussian_bf16((dw.B, dw.H, dw.L, dw.d), seed=dw.seed)
    vc = W.device_gaussian_bf16((dw.B, dw.H, dw.L, dw.d), seed=dw.seed + 1)
    qd = W.device_gaussian_bf16((dw.B, dw.H, dw.d), seed=dw.seed + 2)
    sd = oracle.slopes_ref(dw.H)
    total = 0.0
    for b in range(dw.B):
        for h in range(dw.H):
            qh, kh, vh = qd[b:b + 1, h:h + 1].cpu(), kc[b:b + 1, h:h + 1].cpu(), vc[b:b + 1, h:h + 1].cpu()
            t0 = time.perf_counter()
            oracle.decode_ref(qh, kh, vh, sd[h:h + 1])
            total += time.perf_counter() - t0
        print(f"[oracle] {dw.name} batch {b} done, {total:.1f} s so far", flush=True)
    record(dw.name, total, decode_bytes(dw.B, dw.H, dw.L, dw.d), "GB/s", threads,
           "1 run, host copies excluded")
    print(json.dumps(res), flush=True)


def underflow_report(W):
    """The bf16 underflow diagnostic of the 16384-token, 16-head workload (CPU only).

    Per head, for the two thresholds tau_u = ln(smallest bf16 subnormal) and
    tau_d = ln(smallest normal) ("When Attention Goes Blind", Sec. 3.2 and App. A
    Table 4): the share of weights whose stable-softmax exponent lies at or below
    the threshold, analytic (content scores 0: bias alone, -m d <= tau) and on the
    seeded bf16 inputs (x_ij = s_ij - max_j s_ij <= tau), over the causal triangle
    (Sec. 5.2's convention) and over the last row (Fig. 1b's per-distance
    convention). The two steepest heads are flagged. Computed by the fp64 oracle.
    """
    import numpy as np
    import oracle
    wl = W.FWD_B1_H16_N16384_D128
    q, k, _ = W.gaussian_qkv_bf16(wl.shape, seed=wl.seed)
    slopes = oracle.slopes_ref(wl.H).astype(np.float64)
    th = oracle.format_thresholds("bf16")
    taus = {"tau_u": th["tau_u"], "tau_d": th["tau_d"]}
    steep = set(int(x) for x in np.argsort(-slopes)[:2])
    heads = []
    t_all = time.perf_counter()
    for h in range(wl.H):
        m = float(slopes[h])
        t0 = time.perf_counter()
        data = oracle.underflow_fraction_data(q[0, h], k[0, h], m, [taus["tau_u"], taus["tau_d"]])
        row = {"head": h, "slope": m, "steepest_two": h in steep}
        for (name, tau), dd in zip(taus.items(), data):
            row[name] = {
                "analytic_triangle": oracle.underflow_fraction_causal(m, wl.N, tau),
                "analytic_last_row": oracle.underflow_fraction_by_distance([m], wl.N, tau),
                "data_triangle": dd["share"],
                "data_last_row": dd["last_row_share"],
            }
        heads.append(row)
        print(f"[underflow] head {h:2d} m={m:.6g}{' (steep)' if h in steep else ''}: "
              f"tau_u tri {row['tau_u']['data_triangle']:.5f}/{row['tau_u']['analytic_triangle']:.5f} "
              f"last {row['tau_u']['data_last_row']:.5f}/{row['tau_u']['analytic_last_row']:.5f}; "
              f"tau_d tri {row['tau_d']['data_triangle']:.5f}/{row['tau_d']['analytic_triangle']:.5f} "
              f"last {row['tau_d']['data_last_row']:.5f}/{row['tau_d']['analytic_last_row']:.5f} "
              f"(data/analytic, {time.perf_counter() - t0:.1f} s)", flush=True)
    print(json.dumps({"only": "underflow", "workload": wl.name, "thresholds": taus, "heads": heads,
                      "seconds": round(time.perf_counter() - t_all, 1)}), flush=True)


def run_only(args, alibi, W, fw, dw, dev):
    """One kernel, W + K launches, HIP-event timed; for counter runs."""
    import torch
    if args.only == "oracle":
        return oracle_timing(W, dw, dev)
    if args.only in ("fwd", "fwd16k", "c2", "c3"):
        wl = {"fwd": fw, "fwd16k": W.FWD_B1_H16_N16384_D128, "c2": W.FWD_B8_H8_N1024_D64,
              "c3": W.FWD_B4_H12_N2048_D64}[args.only]
        q, k, v = (x.to(dev) for x in W.gaussian_qkv_bf16(wl.shape, seed=wl.seed))
        out = torch.empty_like(q)
        s = alibi.slopes(wl.H).to(dev)
        fn = lambda: alibi.attn_fwd(q, k, v, s, causal=True, out=out)
        work, unit = fwd_flops(wl.B, wl.H, wl.N, wl.d), "flop"
    elif args.only == "c1":
        wl = W.TINY_FP32
        q, k, v = (torch.from_numpy(x).reshape(wl.shape).to(dev) for x in W.tiny_example_qkv())
        out = torch.empty_like(q)
        s = alibi.slopes(wl.H).to(dev)
        fn = lambda: alibi.attn_fwd_f32(q, k, v, s, causal=True, out=out)
        work, unit = fwd_flops(wl.B, wl.H, wl.N, wl.d), "flop"
    elif args.only == "decode":
        kc = W.device_gaussian_bf16((dw.B, dw.H, dw.L, dw.d), seed=dw.seed)
        vc = W.device_gaussian_bf16((dw.B, dw.H, dw.L, dw.d), seed=dw.seed + 1)
        qd = W.device_gaussian_bf16((dw.B, dw.H, dw.d), seed=dw.seed + 2)
        od = torch.empty_like(qd)
        s = alibi.slopes(dw.H).to(dev)
        fn = lambda: alibi.attn_decode(qd, kc, vc, s, out=od)
        work, unit = decode_bytes(dw.B, dw.H, dw.L, dw.d), "B"
    elif args.only in ("bwd", "bwd_skip"):
        q, k, v = (x.to(dev) for x in W.gaussian_qkv_bf16(fw.shape, seed=fw.seed))
        s = alibi.slopes(fw.H).to(dev)
        out, lse = alibi.attn_fwd_train(q, k, v, s, True)
        dout = torch.randn(q.shape, generator=torch.Generator(device=dev).manual_seed(7), device=dev,
                           dtype=torch.float32).to(torch.bfloat16)
        skip = args.only == "bwd_skip"
        fn = lambda: alibi.attn_bwd(q, k, v, out, dout, lse, s, True, skip_underflow=skip)
        work, unit = 2.5 * fwd_flops(fw.B, fw.H, fw.N, fw.d), "flop"
    elif args.only in ("mfma", "mfma_valu"):
        lib = alibi.load_library()
        valu = int(args.only == "mfma_valu")
        wgs, iters = 1024, 160
        frags = torch.randn(8 * 64 * 8, generator=torch.Generator(device=dev).manual_seed(7), device=dev,
                            dtype=torch.float32).to(torch.bfloat16)
        sink = torch.empty(8 * wgs, dtype=torch.float32, device=dev)
        st = torch.cuda.current_stream().cuda_stream
        fn = lambda: lib.alibi_debug_mfma_rate(frags.data_ptr(), iters, valu, sink.data_ptr(), wgs, st)
        work, unit = float(wgs) * 8 * iters * 16 * 32768.0, "flop"
    else:
        src = torch.ones(1 << 29, dtype=torch.bfloat16, device=dev)  # 1 GiB
        dst = torch.empty_like(src)
        fn = lambda: dst.copy_(src)
        work, unit = 2.0 * src.numel() * 2, "B (read + write)"
    for _ in range(args.warmup):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    print(json.dumps({"only": args.only, "ms_per_launch": round(ms, 4), "work_per_launch": work,
                      "unit": unit, "rate": work / ms / 1e9}), flush=True)


if __name__ == "__main__":
    main()
