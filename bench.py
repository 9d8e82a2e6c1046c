#!/usr/bin/env python3
"""Benchmark of the MLA prolog on one MI355X.

One step is one ``mla_prolog_run`` over one batch of synthetic tokens: the
down-projection, norms/RoPE/cache scatter, up-projection with q-RoPE and
W^UK product (one kernel up to 32 tokens, three or four above).  Inputs are
resident in HBM before timing starts; the
weights rotate over enough replicas that consecutive steps cannot find them
in the 256 MB Infinity Cache, so every step streams its weights from HBM.

Prints one JSON line: tokens/s, the roofline of the dominant kernel (the
whole step up to 32 tokens, else the up-projection) from HIP events
recorded around each kernel, the roofline of
the whole step, and the CPU oracle timed on the host cores on a bounded
sample of the same workload.
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MLA-prolog tokens/s; % HBM roofline (decode), % MFMA peak (prefill)"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
INT8_PEAK_TOPS = 5000.0
MALL_BYTES = 256 << 20


def algorithmic(inp, T):
    """Bytes and flops each kernel must move / do at minimum for T tokens."""
    d = inp["dims"]
    q8 = bool(inp["quant"])                   # int8 x, W^DQ, W^DkvKr (and W^UqQr)
    st = bool(inp.get("preprocess", False))   # bf16 x quantised here, int8 weights, biases
    u8 = q8 or st or bool(inp.get("partial", False))   # int8 W^UqQr and c^Q
    sm = inp.get("smooth_scales_cq") is not None
    kv8 = bool(inp.get("kv_quant", False))            # int8 kv cache rows
    kr8 = kv8 and bool(inp.get("partial", False))    # int8 kr cache rows
    cache = T * (d.Hckv * (1 if kv8 else 2) + d.Dr * (1 if kr8 else 2)) + (kv8 and d.Hckv * 4) + (kr8 and d.Dr * 4)
    ed = 1 if q8 or st else 2                 # bytes of W^DQ, W^DkvKr elements
    ex = 1 if q8 else 2                       # bytes of x elements
    eu = 1 if u8 else 2                       # bytes of W^UqQr and c^Q elements
    W = d.N * (d.D + d.Dr)
    Nkr = d.Hckv + d.Dr
    qo = 1 if q8 else 2
    # the static scenario's extra parameters: deScale0 + bias0, deScale1 +
    # bias1, gamma0 + beta0, beta1
    st_dq = st and (d.Hcq + Nkr) * 8 + d.He * 4
    st_uq = st and W * 8
    k1_bytes = d.He * (d.Hcq + Nkr) * ed + T * d.He * ex + (q8 and (d.Hcq + Nkr + T) * 4) + st_dq
    k1_flop = 2 * T * d.He * (d.Hcq + Nkr)
    k2_bytes = (cache + T * d.Hcq * eu + T * 2 * d.Dr * 2 + T * 8
                + (u8 and T * 4) + (sm and d.Hcq * 4) + (st and d.Hcq * 2))
    k3_bytes = (d.Hcq * W * eu + T * d.Hcq * eu + T * d.N * d.D * 2
                + T * d.N * d.Dr * 2 + T * 2 * d.Dr * 2 + (u8 and W * 4 + T * 4) + (st and W * 4))
    k3_flop = 2 * T * d.Hcq * W
    k4_bytes = d.N * d.D * d.Hckv * 2 + T * d.N * d.D * 2 + T * d.N * d.Hckv * qo + (q8 and T * d.N * 4)
    k4_flop = 2 * T * d.N * d.D * d.Hckv
    weights = d.He * (d.Hcq + Nkr) * ed + d.Hcq * W * eu + d.N * d.D * d.Hckv * 2
    # inputs read once, outputs written once, the scales of the scenario
    step_bytes = (weights + T * d.He * ex + T * 2 * d.Dr * 2 + T * 8 + T * d.N * d.Hckv * qo
                  + T * d.N * d.Dr * 2 + cache
                  + (q8 and (T + d.Hcq + Nkr + T * d.N) * 4) + (u8 and not st and W * 4)
                  + (sm and d.Hcq * 4) + st_dq + st_uq + (st and d.Hcq * 2))
    return dict(k1_bytes=k1_bytes, k1_flop=k1_flop, k2_bytes=k2_bytes, k3_bytes=k3_bytes,
                k3_flop=k3_flop, k4_bytes=k4_bytes, k4_flop=k4_flop, weights=weights,
                step_bytes=step_bytes, step_flop=k1_flop + k3_flop + k4_flop)


def measured_traffic(workload, kernel, source="mla_prolog.hip"):
    """HBM bytes per launch of the dominant kernel (per step of the listed
    kernels) from the committed counter summary
    profiles/traffic_<workload>.json (FETCH_SIZE and WRITE_SIZE per dispatch,
    each scaled by what the counter reads for a plain copy of known size), or
    None when there is none or the kernel source has changed since the
    counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    src = os.path.join(ROOT, "head_latent_attention_amd", "csrc", source)
    with open(src, "rb") as f:
        digest = hashlib.sha256(f.read()).hexdigest()
    if t.get("source_sha256") != digest or t.get("bench_kernel") != kernel:
        return None
    return t["traffic_bytes"]


def cpu_baseline(inp, seconds):
    """The oracle, as it is, over repeated passes of the workload's first
    tokens until about ``seconds`` of host time are spent."""
    import oracle
    T = int(inp["T"])
    cores = len(os.sched_getaffinity(0))
    per_pass = min(T, 64)
    rows = list(range(per_pass))
    oracle.run(inp, tokens=rows[:1], caches=False, nthreads=cores)   # load + warm
    done, t0 = 0, time.perf_counter()
    while True:
        oracle.run(inp, tokens=rows, caches=False, nthreads=cores)
        done += per_pass
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    return {"value": done / el, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{done} tokens ({done // per_pass} passes over the first {per_pass} tokens "
                      f"of {inp['workload']}) in {el:.1f} s"}


SFA_METRIC = "sparse flash attention (MLA-absorb) decode tokens/s; % HBM roofline"


def sfa_bytes(inp, T):
    """Bytes a sparse attention step must move at minimum: the selected cache
    rows (each read once), the queries, the outputs, indices and tables."""
    N, D, Dr, K, sbs = (int(inp[k]) for k in ("N", "D", "Dr", "K", "sparse_block_size"))
    return (T * K * sbs * (D + Dr) * 2 + T * N * (D + Dr) * 2 + T * N * D * 2 + T * N * 8
            + T * K * 4 + T * int(inp["max_blocks"]) * 4 + T * 4)


def bench_sfa(args, workload):
    """One step = one mla_sfa_run over the workload's tokens.  The caches
    (filled on the device) are several times the Infinity Cache and each
    step takes the next of several index sets, so the selected rows come
    from HBM."""
    import torch
    import head_latent_attention_amd as mla
    from dataclasses import replace
    from synth.sfa import make_sfa_inputs, sfa_workload
    wl = sfa_workload(workload)
    # longer sequences than the parity workload: a 2 GB cache
    wl = replace(wl, len_lo=49152, len_hi=65536)
    sets = 8
    inps = [make_sfa_inputs(replace(wl, seed=wl.seed + 1000 * r), caches=False) for r in range(sets)]
    inp = inps[0]
    T, N, D, Dr = int(inp["T"]), int(inp["N"]), int(inp["D"]), int(inp["Dr"])
    block_num = max(int(i["block_num"]) for i in inps)
    gen = torch.Generator(device="cuda:0")
    gen.manual_seed(wl.seed)
    kv = torch.randn((block_num, int(inp["block_size"]), 1, D), generator=gen, device="cuda:0").to(torch.bfloat16)
    kr = torch.randn((block_num, int(inp["block_size"]), 1, Dr), generator=gen, device="cuda:0").to(torch.bfloat16)
    dev_sets = []
    for i in inps:
        dev_sets.append({
            "query": torch.from_numpy(i["query"].view(np.int16)).to("cuda:0").view(torch.bfloat16),
            "query_rope": torch.from_numpy(i["query_rope"].view(np.int16)).to("cuda:0").view(torch.bfloat16),
            "kv_cache": kv, "kr_cache": kr,
            "sparse_indices": torch.from_numpy(i["indices"]).to("cuda:0"),
            "block_table": torch.from_numpy(i["block_table"]).to("cuda:0"),
            "seq_lens_kv": torch.from_numpy(i["seq_lens"]).to("cuda:0")})
    out = torch.empty((T, N, D), dtype=torch.bfloat16, device="cuda:0")
    smax = torch.empty((T, N), dtype=torch.float32, device="cuda:0")
    ssum = torch.empty((T, N), dtype=torch.float32, device="cuda:0")
    for d in dev_sets:
        d.update(attention_out=out, softmax_max=smax, softmax_sum=ssum)
    desc = mla.make_sfa_desc(N=N, D=D, Dr=Dr, block_num=block_num, block_size=int(inp["block_size"]),
                             max_blocks=int(inp["max_blocks"]), sparse_size=int(inp["K"]),
                             sparse_block_size=int(inp["sparse_block_size"]), max_tokens=T,
                             scale=float(inp["scale"]))
    h = mla.MlaSfa(desc)
    stream = torch.cuda.current_stream()
    for i in range(args.warmup):
        h.run(dev_sets[i % sets], T, stream)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for i in range(args.steps):
        h.run(dev_sets[i % sets], T, stream)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = e0.elapsed_time(e1) / args.steps
    h.close()
    nbytes = sfa_bytes(inp, T)
    achieved = nbytes / (ms_step * 1e-3) / 1e9
    res = {
        "metric": SFA_METRIC, "value": T / (ms_step * 1e-3), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": wl.name, "T": T, "N": N, "D": D, "Dr": Dr, "sparse_size": int(inp["K"]),
                   "sparse_block_size": int(inp["sparse_block_size"]), "block_size": int(inp["block_size"]),
                   "kv_len": [wl.len_lo, wl.len_hi], "cache_bytes": int(kv.numel() * 2 + kr.numel() * 2),
                   "index_sets": sets},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS,
                     "traffic": measured_traffic(wl.name, "k_sfa + k_sfa_combine", "mla_sfa.hip"),
                     "kernel": "k_sfa + k_sfa_combine", "per_launch": f"{nbytes} B"},
        "wall_s": wall,
    }
    if not args.no_cpu_baseline:
        import oracle
        small = make_sfa_inputs(replace(sfa_workload(workload), T=2, len_lo=4096, len_hi=8192))
        cores = len(os.sched_getaffinity(0))
        oracle.sfa(small, tokens=[0], nthreads=cores)
        done, t0 = 0, time.perf_counter()
        while True:
            oracle.sfa(small, nthreads=cores)
            done += 2
            el = time.perf_counter() - t0
            if el >= args.cpu_seconds:
                break
        res["cpu_baseline"] = {"value": done / el, "unit": "tokens/s", "cores": cores, "kind": "oracle",
                               "sample": f"{done} tokens (passes over a 2-token instance of the workload's "
                                         f"shapes, same sparse_size) in {el:.1f} s"}
    del dev_sets, kv, kr
    torch.cuda.empty_cache()
    return res


WORKLOADS = ["decode_t32", "decode_t256", "prefill_t8192", "int8_decode_t128", "partial_decode_t32",
             "int8_kvq_decode_t128", "pre_decode_t32", "pre_f16_decode_t32", "tiny_t4", "sfa_decode_t32"]
#: measured after the headline workload in a default run (one line per run
#: of bench.py, so the other configurations ride along in it)
OTHERS = ["decode_t256", "int8_decode_t128", "prefill_t8192", "int8_kvq_decode_t128", "partial_decode_t32",
          "pre_decode_t32", "pre_f16_decode_t32", "sfa_decode_t32"]


def summary(res):
    """The compact record of a secondary workload in the default run's line."""
    out = {k: res[k] for k in ("value", "unit", "ms_per_step", "steps", "warmup", "dtype") if k in res}
    out["roofline"] = {k: res["roofline"][k] for k in ("bound", "achieved", "peak", "unit", "frac", "traffic",
                                                       "kernel") if k in res["roofline"]}
    if "path_roofline" in res:
        out["path_roofline_frac"] = res["path_roofline"]["frac"]
    if "kernel_us" in res:
        out["kernel_us"] = res["kernel_us"]
    out["config"] = res["config"]
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=None, choices=WORKLOADS,
                    help="one workload; without it, decode_t32 (the line's metric) and then the other "
                         "configurations at --other-steps steps each, recorded in the same line")
    ap.add_argument("--other-steps", type=int, default=50)
    ap.add_argument("--other-warmup", type=int, default=10)
    ap.add_argument("--replicas", type=int, default=0, help="weight replicas (0 = enough to "
                    "exceed twice the Infinity Cache)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--row-major", action="store_true",
                    help="run on the row-major weights only (no packed copy)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run five device-to-device copies of MIB MiB (the known-size copy "
                         "that scales the FETCH_SIZE / WRITE_SIZE counters) and exit")
    args = ap.parse_args()
    if args.copy_calibration:
        import torch
        n = args.copy_calibration << 20
        a = torch.full((n,), 1, dtype=torch.uint8, device="cuda:0")
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n, "copies": 5}), flush=True)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the prolog shards by tokens, or by heads, with no exchange between GPUs, so one "
              "GPU's share at the full shapes is what is measured)",
              file=sys.stderr)
        sys.exit(2)

    if args.workload is not None:
        res = (bench_sfa if args.workload.startswith("sfa_") else bench_prolog)(args, args.workload)
        print(json.dumps(res), flush=True)
        return
    # the CPU oracle's leg runs after every GPU leg: ten seconds of host work
    # with the GPU idle would leave the next workload's warmup on a cold clock
    first = argparse.Namespace(**vars(args))
    first.no_cpu_baseline = True
    res = bench_prolog(first, "decode_t32")
    others = {}
    sub = argparse.Namespace(**vars(args))
    sub.steps, sub.warmup, sub.no_cpu_baseline = args.other_steps, args.other_warmup, True
    for name in OTHERS:
        try:
            r = (bench_sfa if name.startswith("sfa_") else bench_prolog)(sub, name)
            others[name] = summary(r)
        except Exception as e:   # a failure of one configuration is recorded, not fatal
            others[name] = {"error": f"{type(e).__name__}: {e}"}
        print(f"bench: {name} done", file=sys.stderr, flush=True)
    if not args.no_cpu_baseline:
        import synth
        res["cpu_baseline"] = cpu_baseline(synth.make_inputs(synth.workload("decode_t32")), args.cpu_seconds)
    res["other_workloads"] = others
    print(json.dumps(res), flush=True)


def bench_prolog(args, workload):
    """One prolog workload: returns its bench record."""
    import torch
    import head_latent_attention_amd as mla
    import synth
    from synth import device as dev

    wl = synth.workload(workload)
    inp = synth.make_inputs(wl)
    T = int(inp["T"])
    d = inp["dims"]
    alg = algorithmic(inp, T)
    R = args.replicas or max(1, -(-2 * MALL_BYTES // alg["weights"]) + 1)

    base = dev.upload(inp, device="cuda:0")
    wnames = ("weight_dq", "weight_uq_qr", "weight_uk", "weight_dkv_kr")
    sets = [base]
    for _ in range(R - 1):
        s = dict(base)
        for k in wnames:
            s[k] = base[k].clone()
        sets.append(s)
    desc = mla.make_desc(**dev.desc_args(inp))
    h = mla.MlaProlog(desc)
    stream = torch.cuda.current_stream()
    if not args.row_major:
        # the one-time conversion of every weight replica to the packed layout
        for s in sets:
            s["packed_weights"] = torch.empty(mla.packed_weights_bytes(desc), dtype=torch.uint8,
                                              device="cuda:0")
            h.pack_weights(s, s["packed_weights"], stream)
        torch.cuda.synchronize()

    for i in range(args.warmup):
        h.run(sets[i % R], T, stream)
    torch.cuda.synchronize()

    # timed region 1: throughput
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for i in range(args.steps):
        h.run(sets[i % R], T, stream)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_total = e0.elapsed_time(e1)
    ms_step = ms_total / args.steps

    # timed region 2: the same steps with HIP events around every kernel
    h.profile(True)
    torch.cuda.synchronize()
    p0, p1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    p0.record(stream)
    for i in range(args.steps):
        h.run(sets[i % R], T, stream)
    p1.record(stream)
    torch.cuda.synchronize()
    kms, runs = h.profile_read()
    ms_step_profiled = p0.elapsed_time(p1) / args.steps
    h.profile(False)
    kernel_us = {k: 1000.0 * v / runs for k, v in kms.items()}
    h.close()

    decode = T < 1024
    k3_us = kernel_us["up_proj"]
    # small-T runs are one kernel (the profile books it to up_proj and the
    # others read 0): the dominant kernel then moves the whole step's bytes.
    # Otherwise the up-projection and the W^UK product may be one kernel
    # (uk reads 0), which neither writes nor reads q^C.
    one = kernel_us["down_proj"] == 0.0 and kernel_us["norm_rope_cache"] == 0.0
    fused = kernel_us["uk"] == 0.0
    if one:
        # one launch per step (two in the static scenario, whose x quantiser
        # comes first): the timed region's per-step time (HIP events around
        # back-to-back launches on the run's stream) is the kernel's average
        # duration, free of the per-kernel events' dispatch delay
        alg["k3_bytes"] = alg["step_bytes"]
        alg["k3_flop"] = alg["step_flop"]
        k3_us = ms_step * 1000.0
    elif fused:
        alg["k3_bytes"] += alg["k4_bytes"] - 2 * T * d.N * d.D * 2
        alg["k3_flop"] += alg["k4_flop"]
    if decode:
        achieved = alg["k3_bytes"] / (k3_us * 1e-6) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS, "traffic": None}
        path_ach = alg["step_bytes"] / (ms_step * 1e-3) / 1e9
        path = {"bound": "hbm", "achieved": path_ach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": path_ach / HBM_PEAK_GBS, "bytes_per_step": alg["step_bytes"]}
    else:
        peak = INT8_PEAK_TOPS if (inp["quant"] or inp.get("partial", False)) else BF16_PEAK_TFLOPS
        achieved = alg["k3_flop"] / (k3_us * 1e-6) / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
                "frac": achieved / peak, "traffic": None}
        path_ach = alg["step_flop"] / (ms_step * 1e-3) / 1e12
        path = {"bound": "mfma", "achieved": path_ach, "peak": BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": path_ach / BF16_PEAK_TFLOPS,
                "flop_per_step": alg["step_flop"]}
    # (the static scenario's one-kernel runs have the x quantiser in front)
    roof["kernel"] = (("x quantiser + prolog (one kernel)" if inp.get("preprocess", False) else "prolog (one kernel)")
                      if one else "up_proj+uk (fused)" if fused else "up_proj")
    if not args.row_major:
        roof["traffic"] = measured_traffic(wl.name, roof["kernel"])
    roof["per_launch"] = (f"{alg['k3_bytes']} B" if decode else f"{alg['k3_flop']} FLOP")

    out = {
        "metric": METRIC, "value": T * args.steps / (ms_total * 1e-3), "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": ("int8+fp16" if inp.get("fp16", False) else "int8" if inp["quant"] or inp.get("preprocess", False)
                  else "bf16+int8" if inp.get("partial", False) else "bf16"),
        "data": "synthetic",
        "config": {"workload": wl.name, "T": T, "He": d.He, "Hcq": d.Hcq, "Hckv": d.Hckv,
                   "N": d.N, "D": d.D, "Dr": d.Dr, "block_num": wl.block_num,
                   "block_size": wl.block_size, "weight_replicas": R,
                   "query_out": "int8" if inp["quant"] else "bf16",
                   "kv_cache": "int8" if inp.get("kv_quant", False) else "bf16",
                   "weights": "row-major" if args.row_major else "packed",
                   "scenario": ("static int8 (preprocess), fp16 tensors" if inp.get("fp16", False) else
                                "static int8 (preprocess)" if inp.get("preprocess", False) else
                                "int8" if inp["quant"] else "partial int8" if inp.get("partial", False)
                                else "bf16"),
                   "layout": "concatenated" if inp.get("concat", False) else "separate",
                   "weights_given": "(n, k)" if inp.get("weight_nk", False) else "(k, n)"},
        "roofline": roof,
        "path_roofline": path,
        "kernel_us": kernel_us,
        "ms_per_step_profiled": ms_step_profiled,
        "wall_s": wall,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(inp, args.cpu_seconds)
    del sets, base
    torch.cuda.empty_cache()
    return out


if __name__ == "__main__":
    main()
