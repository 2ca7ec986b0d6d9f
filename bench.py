"""Benchmark of the ThriftAttention forward path on one MI355X.

One step = the whole path on one batch of seeded synthetic input already in
HBM: block selection (means, scores, per-query-block top-k), FP4
quantisation of Q, K and V, and the mixed FP4/FP16 attention forward.
Prints one JSON line (rank 0) with the throughput of the step in attention
TFLOP/s, the roofline of the attention kernel (the dominant one) and the CPU
oracle timed on a bounded sample of the same workload.
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# committed profiler counters, per (workload, format) that has them
TRAFFIC_FILES = {("long", "mx"): os.path.join(ROOT, "profiles", "attn_fwd_kernel_long_mx_traffic.txt"),
                 ("decode", "mx"): os.path.join(ROOT, "profiles", "decode_kernels_decode_mx_traffic.txt"),
                 ("prefill_bwd", "mx"): os.path.join(ROOT, "profiles", "backward_kernels_prefill_mx_traffic.txt")}
# committed rocprofv3 --pmc utilisation summaries of the attention kernel
PMC_FILES = {("long", "mx"): os.path.join(ROOT, "profiles", "attn_fwd_kernel_long_mx_pmc.txt"),
             ("long", "nvfp4"): os.path.join(ROOT, "profiles", "attn_fwd_kernel_long_nvfp4_pmc.txt")}
CSRC = os.path.join(ROOT, "fp16_attention_amd", "csrc")
# the sources a profiled kernel is built from (their hash dates the counters)
KERNEL_SRC = (os.path.join(CSRC, "attention.hip"), os.path.join(CSRC, "common.h"))
BWD_SRC = (os.path.join(CSRC, "backward.hip"), os.path.join(CSRC, "common.h"))

P_FP4 = 10.1e15   # MI355X dense MXFP4 MFMA, FLOP/s
P_FP16 = 2.5e15   # MI355X dense FP16 MFMA, FLOP/s
HBM = 8.0e12      # bytes/s


def unmasked_pairs(S, causal, r0=0, r1=None):
    """Number of (query, key) pairs with key <= query (causal) for rows [r0, r1)."""
    r1 = S if r1 is None else r1
    if not causal:
        return (r1 - r0) * S
    return (r1 * (r1 + 1) - r0 * (r0 + 1)) // 2


def promoted_pairs(idx, cnt, S, bq, bk, causal):
    """Unmasked (query, key) pairs inside promoted tiles (host, from idx/cnt)."""
    B, H, nq, _ = idx.shape
    total = 0
    for i in range(nq):
        r0, r1 = i * bq, min(S, (i + 1) * bq)
        rows = np.arange(r0, r1)
        sel = idx[:, :, i]
        c = cnt[:, :, i]
        for jj in range(sel.shape[-1]):
            j = sel[..., jj]
            on = (jj < c) & (j >= 0)
            if not on.any():
                continue
            for jv in np.unique(j[on]):
                n_here = int(np.sum(on & (j == jv)))
                k0, k1 = int(jv) * bk, min(S, (int(jv) + 1) * bk)
                if causal:  # keys k0.. up to each row
                    per = int(np.sum(np.clip(rows + 1 - k0, 0, k1 - k0)))
                else:
                    per = len(rows) * (k1 - k0)
                total += n_here * per
    return total


def measured_traffic(workload, fmt_name, src=KERNEL_SRC):
    """HBM bytes per forward from the committed profiler counters
    (FETCH_SIZE + WRITE_SIZE, each scaled by its reading on a copy kernel of
    known size), or None when none were taken on this workload or they were
    taken on an attention kernel source other than the one built now."""
    rec = _counter_file(TRAFFIC_FILES.get((workload, fmt_name)), src)
    return None if rec is None else int(rec["traffic_bytes_per_launch"])


def _counter_file(path, src):
    """The machine-readable "key: value" lines of a committed profiler summary,
    or None when it is missing or was taken on sources other than the ones
    built now (kernel_source_sha256 over src)."""
    import hashlib

    if path is None or not os.path.exists(path):
        return None
    rec = {}
    with open(path) as f:
        for ln in f:
            if ":" in ln and not ln.startswith((" ", "#", "|")):
                k, v = ln.split(":", 1)
                rec[k.strip()] = v.strip()
    h = hashlib.sha256()
    for p in src:
        with open(p, "rb") as f:
            h.update(f.read())
    return rec if rec.get("kernel_source_sha256") == h.hexdigest() else None


def measured_utilisation(workload, fmt_name, scores, src=KERNEL_SRC):
    """MFMA busy fraction and VALU wave-instructions per score of the attention
    kernel from the committed rocprofv3 --pmc summary of this workload and
    format (SQ_VALU_MFMA_BUSY_CYCLES over SQ_BUSY_CYCLES scaled to SIMDs;
    SQ_INSTS_VALU per launch over 64 lanes' worth of scores), or {} when none
    was taken on the kernel source built now."""
    rec = _counter_file(PMC_FILES.get((workload, fmt_name)), src)
    if rec is None:
        return {}
    valu = float(rec["sq_insts_valu_per_launch"])
    return {"mfma_busy": float(rec["mfma_busy_frac"]), "valu_busy_est": float(rec["valu_busy_frac_est"]),
            "valu_insts_per_score": round(valu * 64 / scores, 3)}


def copy_calibration(torch, dev, mib):
    """One plain device copy of mib MiB: a kernel whose HBM traffic is known."""
    src = torch.empty(mib << 18, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def algorithmic_bytes(w, p16_tiles_q, fmt):
    """Bytes one attention launch must move at least: FP4 Q/K/V (codes +
    scales) once, the FP16 Q rows of query blocks with promoted tiles and the
    FP16 K/V of promoted key blocks once each, and the fp16 output."""
    g = 16 if fmt == 0 else 32
    fp4_row = w.D // 2 + w.D // g
    b = w.B * (w.Hq + 2 * w.Hkv) * w.S * fp4_row
    b += p16_tiles_q * w.bq * w.D * 2
    b += w.B * w.Hkv * w.S * w.D * 2 * 2  # every key block may be promoted by some query block
    b += w.B * w.Hq * w.S * w.D * 2        # output
    return b


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=None, help="default: long (forward), prefill (--pass bwd)")
    ap.add_argument("--pass", dest="pass_", default="fwd", choices=["fwd", "bwd"],
                    help="fwd: the forward path (default); bwd: the Attn-QAT backward pass")
    ap.add_argument("--fmt", default="mx", choices=["mx", "nvfp4", "nvfp4_mxp"],
                    help="nvfp4_mxp: NVFP4 Q/K/V with P quantised MX-style (forward only)")
    ap.add_argument("--topk-bp", type=int, default=None)
    ap.add_argument("--budget", default="block", choices=["block", "head"],
                    help="top-k per query block (default) or one budget per query head")
    ap.add_argument("--tier8-bp", type=int, default=0,
                    help="the three-tier variant (MX format, forward): this many basis points of the "
                         "valid pairs beyond the FP16 tier's run on the MXFP8 middle tier")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-nvfp4", action="store_true",
                    help="skip the NVFP4 forward that the default (MX) line reports beside its own")
    ap.add_argument("--all-configs", action="store_true",
                    help="one line per workload, format and top-k of the benchmark's configurations "
                         "(forward, no CPU baseline) instead of the single line")
    ap.add_argument("--out", default=None, help="also append the JSON line to this file")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="run one plain device copy of this many MiB before the steps (a "
                         "kernel of known traffic, to calibrate profiler byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: the path is measured on one GPU only; --gpus above 1 is not supported "
              "(the path shards by independent (batch, head) slices, nothing to measure across GPUs)",
              file=sys.stderr)
        sys.exit(2)

    import torch

    from fp16_attention_amd import api
    from fp16_attention_amd import workloads as W

    if args.workload is None:
        args.workload = "prefill" if args.pass_ == "bwd" else "long"
    w = W.WORKLOADS[args.workload]
    if args.topk_bp is not None:
        w = w.with_(topk_count=-1, topk_bp=args.topk_bp)
    fmt = api.THRIFT_MXFP4 if args.fmt == "mx" else api.THRIFT_NVFP4
    p_fmt = api.THRIFT_MXFP4 if args.fmt == "nvfp4_mxp" else None
    if p_fmt is not None and (args.pass_ == "bwd" or W.WORKLOADS[args.workload].Sq):
        print("bench.py: nvfp4_mxp is a forward variant (prefill shape only)", file=sys.stderr)
        sys.exit(2)
    tier8 = args.tier8_bp
    if tier8 and (args.pass_ == "bwd" or W.WORKLOADS[args.workload].Sq or fmt != api.THRIFT_MXFP4
                  or args.budget != "block" or w.topk_count >= 0):
        print("bench.py: --tier8-bp is a forward variant of the MX format with per-query-block budgets "
              "in basis points (prefill shape only)", file=sys.stderr)
        sys.exit(2)
    if args.all_configs:
        return run_all_configs(args)
    t0 = time.time()
    d = W.generate(w)
    gen_s = time.time() - t0
    if w.Sq:
        return run_decode(args, w, d, gen_s)
    if args.pass_ == "bwd":
        return run_backward(args, w, d, gen_s)
    m = measure_forward(args, w, d, fmt, p_fmt, tier8, args.budget, args.steps, args.warmup, args.copy_mib)
    line = forward_line(args, w, m, fmt, p_fmt, tier8, gen_s)
    if fmt == api.THRIFT_MXFP4 and not tier8 and args.budget == "block" and not args.no_nvfp4:
        # the pages' own format on the same input: its FP4 path runs on the fp16
        # matrix cores (decoded operands), so its bound is F_alg / fp16 peak
        mn = measure_forward(args, w, d, api.THRIFT_NVFP4, None, 0, "block", args.steps, args.warmup, 0)
        line["nvfp4"] = {"ms_per_step": round(mn["ms_step"], 4), "attention_fwd_ms": round(mn["fwd_ms"], 4),
                         "attention_fwd_tflops": round(mn["f_alg"] / mn["fwd_ms"] / 1e9, 2),
                         "frac_of_fp16_bound": round(mn["f_alg"] / P_FP16 / (mn["fwd_ms"] * 1e-3), 4),
                         "fp16_pair_share": round(mn["p16"] / mn["pairs"], 5)}
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, d, fmt, args.budget, p_fmt, tier8)
    emit(line, args.out)


WARM_S = 0.3  # --all-configs: each line's warm-up runs at least this long


def warm_up(step, n, torch, min_s=0.0):
    """n untimed steps, continued until min_s seconds have passed (the GPU
    raises its clocks over the first tens of milliseconds of work, which a
    few steps of a small workload do not cover)."""
    t0 = time.perf_counter()
    done = 0
    while done < n or time.perf_counter() - t0 < min_s:
        step()
        done += 1
        if done >= n:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    return done


def emit(line, out=None):
    s = json.dumps(line)
    print(s, flush=True)
    if out:
        with open(out, "a") as f:
            f.write(s + "\n")


def measure_forward(args, w, d, fmt, p_fmt, tier8, budget, steps, warmup, copy_mib, min_warm_s=0.0):
    """Time `steps` forward steps (after `warmup`) of workload w on input d:
    means + FP4 codes of Q and K in one pass, V's codes, selection, the
    attention forward.  Returns the timings (ms) and pair counts."""
    import torch

    from fp16_attention_amd import api

    dev = torch.device("cuda:0")
    q, k, v = (torch.from_numpy(d[n]).to(dev) for n in ("q", "k", "v"))
    if budget == "head":
        select = api.thrift_select_blocks_head
        kmax = api._lib.load().thrift_select_head_kmax(w.S, w.S, w.bq, w.bk, int(w.causal))
    else:
        select = api.thrift_select_blocks_means
        kmax = max(1, api.thrift_select_kmax(w.S, w.bq, w.bk, w.causal, w.topk_count, w.topk_bp))
    kmax2 = max(1, api.thrift_select_kmax(w.S, w.bq, w.bk, w.causal, -1, w.topk_bp + tier8)) if tier8 else 0
    o = torch.empty_like(q)

    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    if copy_mib:
        copy_calibration(torch, dev, copy_mib)

    def step(rec=None):
        # Q and K each read once for their block means and FP4 codes; V
        # quantised; selection from the means; the mixed forward
        if rec:
            rec[0].record()
        q4, qbar = api.thrift_quantize_fp4_means(q, fmt, w.bq)
        k4, kbar = api.thrift_quantize_fp4_means(k, fmt, w.bk)
        v4 = api.thrift_quantize_fp4(v, api.THRIFT_GROUP_S, fmt)
        if tier8:
            q8, k8 = api.thrift_quantize_fp8(q, api.THRIFT_GROUP_D), api.thrift_quantize_fp8(k, api.THRIFT_GROUP_D)
            v8 = api.thrift_quantize_fp8(v, api.THRIFT_GROUP_S)
        if rec:
            rec[1].record()
        idx, cnt = select(qbar, kbar, w.S, w.S, w.bq, w.bk, w.causal, w.topk_count, w.topk_bp, kmax)
        if tier8:
            idx2, cnt2 = select(qbar, kbar, w.S, w.S, w.bq, w.bk, w.causal, -1, w.topk_bp + tier8, kmax2)
        if rec:
            rec[2].record()
        if tier8:
            api.thrift_attention_fwd_tiered(q, k, v, q4, k4, v4, q8, k8, v8, idx, cnt, idx2, cnt2, w.bq, w.bk,
                                            w.causal, out=o)
        else:
            api.thrift_attention_fwd(q, k, v, q4, k4, v4, idx, cnt, w.bq, w.bk, w.causal, out=o, p_fmt=p_fmt)
        if rec:
            rec[3].record()
        return (idx, cnt, idx2, cnt2) if tier8 else (idx, cnt, None, None)

    nwarm = warm_up(step, warmup, torch, min_warm_s)
    recs = [[ev() for _ in range(4)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for r in recs:
        idx, cnt, idx2, cnt2 = step(r)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    idx_h, cnt_h = idx.cpu().numpy(), cnt.cpu().numpy()
    pairs = w.B * w.Hq * unmasked_pairs(w.S, w.causal)
    p16 = promoted_pairs(idx_h, cnt_h, w.S, w.bq, w.bk, w.causal)
    p8 = 0
    if tier8:  # the middle tier's pairs: in the joint list, not in the FP16 one
        p8 = promoted_pairs(idx2.cpu().numpy(), cnt2.cpu().numpy(), w.S, w.bq, w.bk, w.causal) - p16
    return {"ms_step": 1e3 * wall / steps,
            "q_ms": float(np.mean([r[0].elapsed_time(r[1]) for r in recs])),
            "sel_ms": float(np.mean([r[1].elapsed_time(r[2]) for r in recs])),
            "fwd_ms": float(np.mean([r[2].elapsed_time(r[3]) for r in recs])),
            "pairs": pairs, "p16": p16, "p8": p8, "f_alg": 4.0 * w.D * pairs,
            "qblocks_with_fp16": int((cnt_h > 0).sum()), "steps": steps, "warmup": warmup, "warmup_run": nwarm}


def fmt_name(api, fmt, p_fmt):
    return "mx" if fmt == api.THRIFT_MXFP4 else "nvfp4_mxp" if p_fmt is not None else "nvfp4"


def forward_line(args, w, m, fmt, p_fmt, tier8, gen_s):
    """The JSON line of one forward measurement m (measure_forward)."""
    from fp16_attention_amd import api

    name = fmt_name(api, fmt, p_fmt)
    f_alg = m["f_alg"]
    f16, f8 = 4.0 * w.D * m["p16"], 4.0 * w.D * m["p8"]
    f4 = f_alg - f16 - f8
    if fmt == api.THRIFT_MXFP4:
        # the middle tier runs on the fp16 matrix cores (MXFP8 decoded exactly to fp16)
        t_roof = f4 / P_FP4 + (f16 + f8) / P_FP16
        note = ("F_alg / (F_fp4 / 10.1 PF + (F_fp8 + F_fp16) / 2.5 PF): the middle tier runs on the "
                "fp16 matrix cores" if tier8 else
                "F_alg / (F_fp4 / 10.1 PF + F_fp16 / 2.5 PF) for this launch's FP16 share")
    else:
        t_roof = f_alg / P_FP16
        note = "F_alg / 2.5 PF: the NVFP4 FP4 path runs on the fp16 matrix cores (operands decoded exactly)"
    peak = f_alg / t_roof
    achieved = f_alg / (m["fwd_ms"] * 1e-3)
    value = f_alg / (m["ms_step"] * 1e-3) / 1e12
    roof = {
        "bound": "mfma",
        "achieved": round(achieved / 1e12, 2),
        "peak": round(peak / 1e12, 2),
        "unit": "TFLOP/s",
        "frac": round(achieved / peak, 4),
        "traffic": None if tier8 else measured_traffic(w.name, name),
        "traffic_algorithmic": algorithmic_bytes(w, m["qblocks_with_fp16"], fmt),
        "kernel": "attn_fwd_kernel",
        "peak_note": note,
    }
    if not tier8 and p_fmt is None:
        roof.update(measured_utilisation(w.name, name, m["pairs"]))
    return {
        "metric": "attention-fwd TFLOPS + % of mixed FP4/FP16 MFMA roofline at S=32K, D=128, 5% top-k",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": m["steps"],
        "warmup": m["warmup"],
        "ms_per_step": round(m["ms_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("mxfp4+mxfp8(fp16 math)+fp16" if tier8 else "mxfp4+fp16" if fmt == api.THRIFT_MXFP4 else
                  "nvfp4 q/k/v, mx p (fp16 math)+fp16" if p_fmt is not None else "nvfp4(fp16 math)+fp16"),
        "data": "synthetic",
        "config": {
            "workload": f"{w.name}: B{w.B} Hq{w.Hq} Hkv{w.Hkv} S{w.S} D{w.D} "
                        f"{'causal' if w.causal else 'non-causal'} blocks {w.bq}x{w.bk} "
                        f"top-k {w.topk_bp / 100 if w.topk_count < 0 else w.topk_count}"
                        f"{'%' if w.topk_count < 0 else ' per query block'} {name}"
                        f"{', one budget per query head' if args.budget == 'head' else ''}"
                        f"{f', MXFP8 middle tier {tier8 / 100}% more' if tier8 else ''}",
            "global_batch": w.B, "seq_len": w.S, "parallelism": "none (1 GPU)",
        },
        "roofline": roof,
        "breakdown_ms": {"means_and_quantize_qkv": round(m["q_ms"], 4), "select_from_means": round(m["sel_ms"], 4),
                         "attention_fwd": round(m["fwd_ms"], 4)},
        "fp16_pair_share": round(m["p16"] / m["pairs"], 5),
        **({"fp8_pair_share": round(m["p8"] / m["pairs"], 5)} if tier8 else {}),
        "attention_fwd_tflops": round(achieved / 1e12, 2),
        "input_gen_s": round(gen_s, 1),
    }


# (workload, top-k basis points or None for the workload's own, formats): one
# line each in --all-configs mode
ALL_CONFIGS = [("tiny", None), ("prefill", None)] + [("sweep", bp) for bp in (0, 100, 500, 2500, 10000)] + \
              [("long", None), ("verylong", None), ("dit", None)]


def run_all_configs(args):
    """One JSON line per workload, format and top-k of the benchmark's
    configurations (tiny, prefill, the top-k sweep at 0/1/5/25/100%, long,
    very long, DiT-shaped), both FP4 formats; no CPU baseline."""
    from fp16_attention_amd import api
    from fp16_attention_amd import workloads as W

    data = {}
    for wname, bp in ALL_CONFIGS:
        if wname not in data:  # one input set in host memory at a time (the sweep shares one)
            data.clear()
            t0 = time.time()
            data[wname] = (W.generate(W.WORKLOADS[wname]), time.time() - t0)
        d, gen_s = data[wname]
        w = W.WORKLOADS[wname]
        if bp is not None:
            w = w.with_(topk_count=-1, topk_bp=bp)
        for fmt in (api.THRIFT_MXFP4, api.THRIFT_NVFP4):
            m = measure_forward(args, w, d, fmt, None, 0, "block", args.steps, args.warmup, 0, WARM_S)
            line = forward_line(args, w, m, fmt, None, 0, gen_s)
            line["warmup_run"] = m["warmup_run"]  # at least WARM_S seconds of warm-up steps
            emit(line, args.out)


def run_decode(args, w, d, gen_s):
    """Decode step for Sq new tokens per sequence, written at the end of a
    Sk-key cache: update of the cache's derived state for the new positions
    (the key-block mean of their block, the MXFP4 codes of their K rows and V
    groups), the new query rows' block mean and FP4 codes in one pass,
    selection from the means, decode forward.  The derived state of the rest of the cache
    is built once before timing.  HBM-bound: the roofline is 8 TB/s on the
    algorithmic bytes of the decode forward."""
    import torch

    from fp16_attention_amd import api

    fmt = api.THRIFT_MXFP4 if args.fmt == "mx" else api.THRIFT_NVFP4
    dev = torch.device("cuda:0")
    q, k, v = (torch.from_numpy(d[n]).to(dev) for n in ("q", "k", "v"))
    k4 = api.thrift_quantize_fp4(k, api.THRIFT_GROUP_D, fmt)
    v4 = api.thrift_quantize_fp4(v, api.THRIFT_GROUP_S, fmt)
    kbar = api.thrift_block_means(k, w.bk)
    if args.copy_mib:
        copy_calibration(torch, dev, args.copy_mib)
    s0 = w.S - w.Sq
    kmax = max(1, api.thrift_select_kmax(w.Sq, w.bq, w.bk, w.causal, w.topk_count, w.topk_bp, w.S))
    o = torch.empty_like(q)
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731

    def step(rec=None):
        if rec:
            rec[0].record()
        api.thrift_cache_update(k, v, kbar, k4, v4, s0, w.S, w.bk)
        q4, qbar = api.thrift_quantize_fp4_means(q, fmt, w.bq)
        idx, cnt = api.thrift_select_blocks_means(qbar, kbar, w.Sq, w.S, w.bq, w.bk, w.causal, w.topk_count,
                                                  w.topk_bp, kmax)
        if rec:
            rec[1].record()
        api.thrift_attention_decode(q, k, v, q4, k4, v4, idx, cnt, w.bk, w.causal, out=o)
        if rec:
            rec[2].record()
        return idx, cnt

    warm_up(step, args.warmup, torch)
    recs = [[ev() for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for r in recs:
        idx, cnt = step(r)
    torch.cuda.synchronize()
    ms_step = 1e3 * (time.perf_counter() - t0) / args.steps
    prep_ms = float(np.mean([r[0].elapsed_time(r[1]) for r in recs]))
    fwd_ms = float(np.mean([r[1].elapsed_time(r[2]) for r in recs]))
    idx_h, cnt_h = idx.cpu().numpy(), cnt.cpu().numpy()
    # algorithmic bytes: the FP4 cache (codes + E8M0 scales) of every valid key block once,
    # the fp16 K/V of each distinct promoted block of a key head once, Q (fp16 + FP4), O fp16
    G = w.Hq // w.Hkv
    nkb = -(-w.S // w.bk)
    g = 32 if fmt == api.THRIFT_MXFP4 else 16
    fp4_cache = w.B * w.Hkv * nkb * w.bk * (w.D // 2 + w.D // g) * 2
    distinct = 0
    for b in range(w.B):
        for hk in range(w.Hkv):
            sel = set()
            for g in range(G):
                c = int(cnt_h[b, hk * G + g, 0])
                sel.update(int(j) for j in idx_h[b, hk * G + g, 0, :c])
            distinct += len(sel)
    fp16_tiles = distinct * w.bk * w.D * 2 * 2
    qo = w.B * w.Hq * w.Sq * w.D * (2 + 0.5 + 1 / g + 2)
    alg = fp4_cache + fp16_tiles + qo
    achieved = alg / (fwd_ms * 1e-3)
    rows = w.B * w.Hq * w.Sq
    line = {
        "metric": "decode query rows/s (new tokens x query heads) against a 32K dual FP16/FP4 cache, D=128, 5% top-k",
        "value": round(rows / (ms_step * 1e-3), 1),
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp4+fp16" if fmt == api.THRIFT_MXFP4 else "nvfp4(fp16 math)+fp16",
        "data": "synthetic",
        "config": {"workload": f"{w.name}: B{w.B} Hq{w.Hq} Hkv{w.Hkv} Sq{w.Sq} Sk{w.S} D{w.D} "
                               f"{'causal' if w.causal else 'non-causal'} top-k {w.topk_bp / 100}% {args.fmt}",
                   "global_batch": w.B, "seq_len": w.S, "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "hbm", "achieved": round(achieved / 1e9, 1), "peak": HBM / 1e9, "unit": "GB/s",
                     "frac": round(achieved / HBM, 4), "traffic": measured_traffic(w.name, args.fmt),
                     "traffic_algorithmic": int(alg),
                     "kernel": ("decode_mx_fused_kernel" if fmt == api.THRIFT_MXFP4
                                else "decode_nv4_kernel + decode_f16_kernel") + " + decode_merge_kernel"},
        "breakdown_ms": {"cache_update_select_quantize_q": round(prep_ms, 4), "attention_decode": round(fwd_ms, 4)},
        "bytes": {"fp4_cache": int(fp4_cache), "fp16_promoted_tiles": int(fp16_tiles), "q_and_o": int(qo)},
        "input_gen_s": round(gen_s, 1),
    }
    if not args.no_cpu_baseline:
        from oracle import oracle as O

        nthreads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
        O.lib()
        sec = 0.0
        for b in range(w.B):  # the whole workload, one batch element at a time
            qb, kb, vb = (np.ascontiguousarray(d[n][b:b + 1]) for n in ("q", "k", "v"))
            k4b = O.quantize(kb, O.AXIS_D, fmt)  # the cache's FP4 copy: outside the step, as on the GPU
            v4b = O.quantize(vb, O.AXIS_S, fmt)
            t0 = time.perf_counter()
            ib, cb, _ = O.select(qb, kb, w.bq, w.bk, w.causal, w.topk_count, w.topk_bp)
            q4b = O.quantize(qb, O.AXIS_D, fmt)
            O.attention(qb, kb, vb, q4b, k4b, v4b, ib, cb, w.bq, w.bk, w.causal)
            sec += time.perf_counter() - t0
        line["cpu_baseline"] = {"value": round(rows / sec, 2), "unit": "rows/s", "cores": nthreads,
                                "kind": "oracle", "seconds": round(sec, 3),
                                "sample": f"the whole workload ({w.B} batch elements x {w.Hq} query heads "
                                          f"against the {w.S}-key cache), one batch element at a time: "
                                          f"selection (the oracle recomputes every key-block mean), FP4 "
                                          f"quantisation of the rows, forward, fp64; the cache's FP4 copy "
                                          f"built outside the timer"}
    s = json.dumps(line)
    print(s, flush=True)
    if args.out:
        with open(args.out, "a") as f:
            f.write(s + "\n")


def run_backward(args, w, d, gen_s):
    """Attn-QAT backward.  One step = thrift_attention_bwd on resident inputs
    (Q, K, V, their FP4 copies, the selection, the forward's lse and O', and
    an output gradient dO ~ N(0, 1)).  Algorithmic flops: five products of
    2 D flops per unmasked pair (recomputed scores, dP, dV, dK, dQ), all on the
    fp16 matrix cores (FP4-decoded operands are exact in fp16; NVFP4's slice
    scales enter as fp32 factors).  roofline: the whole backward call (operand
    preparation and its kernels) against the fp16 peak; traffic: the HBM bytes
    of all its kernels."""
    import torch

    from fp16_attention_amd import api

    fmt = api.THRIFT_MXFP4 if args.fmt == "mx" else api.THRIFT_NVFP4
    dev = torch.device("cuda:0")
    q, k, v = (torch.from_numpy(d[n]).to(dev) for n in ("q", "k", "v"))
    rng = np.random.default_rng(w.seed + 1)
    do_h = rng.standard_normal((w.B, w.Hq, w.S, w.D)).astype(np.float16)
    do = torch.from_numpy(do_h).to(dev)
    idx, cnt = api.thrift_select_blocks(q, k, w.bq, w.bk, w.causal, w.topk_count, w.topk_bp)
    q4 = api.thrift_quantize_fp4(q, api.THRIFT_GROUP_D, fmt)
    k4 = api.thrift_quantize_fp4(k, api.THRIFT_GROUP_D, fmt)
    v4 = api.thrift_quantize_fp4(v, api.THRIFT_GROUP_S, fmt)
    _, lse = api.thrift_attention_fwd(q, k, v, q4, k4, v4, idx, cnt, w.bq, w.bk, w.causal, with_lse=True)
    ws = api.thrift_attention_bwd_workspace(w.B, w.Hq, w.Hkv, w.S, w.D, w.bq, dev)
    ohp = torch.empty((w.B, w.Hq, w.S, w.D), dtype=torch.float32, device=dev)
    if args.copy_mib:
        copy_calibration(torch, dev, args.copy_mib)
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731

    def hp():
        api.thrift_attention_fwd_hp(q, k, v, q4, k4, v4, idx, cnt, lse, w.bq, w.bk, w.causal, workspace=ws,
                                    out=ohp)

    def step(rec=None):
        if rec:
            rec[0].record()
        grads = api.thrift_attention_bwd(q, k, v, q4, k4, v4, idx, cnt, lse, ohp, do, w.bq, w.bk, w.causal,
                                         workspace=ws)
        if rec:
            rec[1].record()
        return grads

    hp()
    warm_up(step, args.warmup, torch)
    hp_recs = [[ev(), ev()] for _ in range(3)]
    for r in hp_recs:
        r[0].record()
        hp()
        r[1].record()
    recs = [[ev(), ev()] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for r in recs:
        step(r)
    torch.cuda.synchronize()
    ms_step = 1e3 * (time.perf_counter() - t0) / args.steps
    bwd_ms = float(np.mean([r[0].elapsed_time(r[1]) for r in recs]))
    hp_ms = float(np.mean([r[0].elapsed_time(r[1]) for r in hp_recs]))
    pairs = w.B * w.Hq * unmasked_pairs(w.S, w.causal)
    f_bwd = 10.0 * w.D * pairs
    achieved = f_bwd / (bwd_ms * 1e-3)
    line = {
        "metric": "attention-bwd (Attn-QAT) TFLOPS + % of the fp16 MFMA roofline",
        "value": round(f_bwd / (ms_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16 (FP4-decoded operands)",
        "data": "synthetic",
        "config": {"workload": f"{w.name}: B{w.B} Hq{w.Hq} Hkv{w.Hkv} S{w.S} D{w.D} "
                               f"{'causal' if w.causal else 'non-causal'} blocks {w.bq}x{w.bk} "
                               f"top-k {w.topk_bp / 100}% {args.fmt}, backward",
                   "global_batch": w.B, "seq_len": w.S, "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "mfma", "achieved": round(achieved / 1e12, 2), "peak": P_FP16 / 1e12,
                     "unit": "TFLOP/s", "frac": round(achieved / P_FP16, 4),
                     "traffic": measured_traffic(w.name + "_bwd", args.fmt, BWD_SRC),
                     "kernel": "thrift_attention_bwd (operand preparation, bwd_row_kernel, bwd_key_kernel)"},
        "breakdown_ms": {"attention_bwd": round(bwd_ms, 4), "fwd_hp_O_prime": round(hp_ms, 4)},
        "input_gen_s": round(gen_s, 1),
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline_bwd(w, d, do_h, fmt)
    s = json.dumps(line)
    print(s, flush=True)
    if args.out:
        with open(args.out, "a") as f:
            f.write(s + "\n")


def cpu_baseline_bwd(w, d, do_h, fmt):
    """The oracle's backward of query head 0 and its key head (one head per key
    head in this workload): selection, quantisation, the forward with O' and
    the backward over every query and key block of that head."""
    from oracle import oracle as O

    nthreads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    G = w.Hq // w.Hkv
    q1 = np.ascontiguousarray(d["q"][:1, :G])
    k1 = np.ascontiguousarray(d["k"][:1, :1])
    v1 = np.ascontiguousarray(d["v"][:1, :1])
    do1 = np.ascontiguousarray(do_h[:1, :G])
    O.lib()
    t0 = time.perf_counter()
    idx, cnt, _ = O.select(q1, k1, w.bq, w.bk, w.causal, w.topk_count, w.topk_bp)
    q4, k4, v4 = (O.quantize(x, ax, fmt) for x, ax in ((q1, O.AXIS_D), (k1, O.AXIS_D), (v1, O.AXIS_S)))
    _, lse, ohp = O.attention_hp(q1, k1, v1, q4, k4, v4, idx, cnt, w.bq, w.bk, w.causal)
    O.attention_bwd(q1, k1, v1, q4, k4, v4, idx, cnt, w.bq, w.bk, w.causal, lse, ohp, do1)
    sec = time.perf_counter() - t0
    f = 10.0 * w.D * G * unmasked_pairs(w.S, w.causal)
    return {"value": round(f / sec / 1e12, 5), "unit": "TFLOP/s", "cores": nthreads, "kind": "oracle",
            "seconds": round(sec, 2),
            "sample": f"key head 0 of batch 0 with its {G} query head(s): selection, FP4 quantisation, the forward "
                      f"with O' and the backward over all query and key blocks ({f / 1e9:.1f} GFLOP of backward), "
                      f"fp64"}


def cpu_baseline(w, d, fmt, budget="block", p_fmt=None, tier8=0):
    """The oracle on one query head (and its key head) of the same workload:
    selection, quantisation of that head's Q, K, V and the forward pass."""
    from oracle import oracle as O

    nthreads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    q1 = np.ascontiguousarray(d["q"][:1, :1])
    k1 = np.ascontiguousarray(d["k"][:1, :1])
    v1 = np.ascontiguousarray(d["v"][:1, :1])
    O.lib()
    t0 = time.perf_counter()
    if tier8:
        O.pipeline_tiers(q1, k1, v1, w.bq, w.bk, w.causal, w.topk_bp, tier8, with_amb=False)
    elif budget == "head":
        idx, cnt = O.select_head(q1, k1, w.bq, w.bk, w.causal, w.topk_count, w.topk_bp)
        q4, k4, v4 = (O.quantize(x, ax, fmt) for x, ax in ((q1, O.AXIS_D), (k1, O.AXIS_D), (v1, O.AXIS_S)))
        O.attention(q1, k1, v1, q4, k4, v4, idx, cnt, w.bq, w.bk, w.causal, p_fmt=p_fmt)
    else:
        O.pipeline(q1, k1, v1, fmt, w.bq, w.bk, w.causal, w.topk_count, w.topk_bp, p_fmt=p_fmt, with_amb=False)
    sec = time.perf_counter() - t0
    f = 4.0 * w.D * unmasked_pairs(w.S, w.causal)
    return {"value": round(f / sec / 1e12, 5), "unit": "TFLOP/s", "cores": nthreads,
            "kind": "oracle", "seconds": round(sec, 2),
            "sample": f"query head 0 of batch 0 with its key head: selection ({budget} budget"
                      f"{', twice: FP16 tier and both tiers' if tier8 else ''}), FP4 "
                      f"{'and MXFP8 ' if tier8 else ''}quantisation of "
                      f"its Q/K/V and the forward pass over all {-(-w.S // w.bq)} query blocks "
                      f"({f / 1e9:.1f} GFLOP of attention), fp64"}


if __name__ == "__main__":
    main()
