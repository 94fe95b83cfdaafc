"""KDA hot-path benchmark on one MI355X.

One step = one pass of the whole hot path at Kimi-K3 head scale (96 KDA heads
x 128, bf16 inputs, fp32 state):
  * chunked prefill of one 32,768-token sequence (final state requested), and
  * one recurrent decode step for 256 sequences (state carried across steps).
`value` is the step's whole-job throughput, (32,768 + 256) tokens / step time.
The timed step runs the two on one stream, so each kernel's figures are its
own; the two parts are independent, and an extra pass reports the same step
with the decode on a second stream beside the prefill.

    python bench.py [--gpus 1] [--steps 20] [--warmup 3] [--no-cpu-baseline]

Prints one JSON line.  Inputs are synthetic and seeded (see
gated_delta_rule_04_amd/inputs.py) and resident in HBM before timing starts.
"""

import argparse
import hashlib
import json
import os
import resource
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "KDA chunked-prefill tokens/s + decode tokens/s; % MFMA peak, % HBM GB/s"
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, GB/s
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, TFLOP/s
CSRC = os.path.join(ROOT, "gated_delta_rule_04_amd", "csrc")
# Sources of each measured kernel (the bf16 prefill kernel is the pipelined one).
# what a kernel is built from: its sources and the build script (compile flags)
BUILD_PY = os.path.join(os.path.dirname(CSRC), "build.py")
PREFILL_SRCS = [os.path.join(CSRC, f) for f in ("kda_common.h", "kda_prefill_common.h", "kda_prefill.hip",
                                                "kda_prefill_pipe.hip")] + [BUILD_PY]
DECODE_SRCS = [os.path.join(CSRC, f) for f in ("kda_common.h", "kda_decode.hip")] + [BUILD_PY]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_counters.txt")


def alg_prefill(B, T, H, dk, dv, g_group, elem=2, final_state=True, C=64, N=None):
    """Algorithmic bytes and flops of one prefill call.
    Bytes per head-token: q, k, v, g in, o out (elem bytes each), beta in;
    plus the final fp32 state once per (sequence, head) (N sequences, default B).
    Flops per head-token: 6 dk dv (state pass: Kt S, Qt S, Kb^T U) + (C-1) dk
    (k-k block) + (C+1) dk (q-k block) + 2 (C+1) dv (P U, Tm R) + C^2/3
    (triangular solve), masked triangles counted at half."""
    ht = B * T * H
    per_tok_bytes = elem * (2 * dk + dv + dk // g_group + 1 + dv)
    nbytes = ht * per_tok_bytes + ((B if N is None else N) * H * dk * dv * 4 if final_state else 0)
    flops = ht * (6 * dk * dv + (C - 1) * dk + (C + 1) * dk + 2 * (C + 1) * dv + C * C / 3.0)
    return nbytes, flops


def alg_decode(N, H, dk, dv, g_group, elem=2):
    """Bytes of one decode step: fp32 state read and written, inputs and o."""
    per = 8 * dk * dv + elem * (2 * dk + dv + dk // g_group + 1 + dv)
    return N * H * per


def alg_decode_pool(N, H, dk, dv, g_group, state_elem=2, elem=2):
    """Bytes of one serving-pool decode step with a state of state_elem bytes
    per value (bf16: 2), read and written, plus the inputs and o."""
    per = 2 * state_elem * dk * dv + elem * (2 * dk + dv + dk // g_group + 1 + dv)
    return N * H * per


def alg_backward(B, T, H, dk, dv, g_group, N=None, elem=2):
    """Algorithmic bytes of one backward call: per head-token q, k, v, g,
    beta and do read, dq, dk, dv, dg, dbeta written (elem bytes each); per
    (sequence, head) the fp32 dht read and dh0 written."""
    N = B if N is None else N
    per_in = elem * (2 * dk + dv + dk // g_group + 1 + dv)
    per_out = elem * (2 * dk + dv + dk // g_group + 1)
    return B * T * H * (per_in + per_out) + N * H * dk * dv * 8


def pct(xs, p):
    """p-th percentile of a list of timings (linear interpolation)."""
    ys = sorted(xs)
    if not ys:
        return float("nan")
    x = (len(ys) - 1) * p / 100.0
    i = int(x)
    j = min(i + 1, len(ys) - 1)
    return ys[i] + (ys[j] - ys[i]) * (x - i)


def sha256_files(paths):
    """sha256 of the concatenated contents of paths (in order)."""
    h = hashlib.sha256()
    for p in paths:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def read_traffic(kernel):
    """HBM bytes per launch measured with rocprofv3 FETCH_SIZE/WRITE_SIZE,
    valid only while the kernel source is unchanged since the counters."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    want = sha256_files(PREFILL_SRCS if kernel == "prefill" else DECODE_SRCS)
    rec = {}
    with open(TRAFFIC_FILE) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#") or ":" not in line:
                continue
            k, v = line.split(":", 1)
            rec[k.strip()] = v.strip()
    if rec.get(kernel + "_source_sha256") != want:
        return None
    try:
        return float(rec[kernel + "_traffic_bytes"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(pre, dec, budget_s=12.0):
    """Time the CPU oracle (as it stands) on a bounded sample of the same
    workload and scale to the step's tokens/s."""
    import numpy as np
    import oracle.kda_oracle as orc

    f64 = lambda t: t.double().numpy()
    wall0 = time.perf_counter()
    cpu0 = time.process_time()
    # prefill sample: the first 8 heads, tokens until about half the budget
    Hs = 8
    q, k, v, g, beta = (pre[n][0, :, :Hs] for n in ("q", "k", "v", "g", "beta"))
    S = np.zeros((Hs, q.shape[-1], v.shape[-1]))
    t0 = time.perf_counter()
    ntok = 0
    blk = 256
    while ntok < q.shape[0] and time.perf_counter() - t0 < budget_s / 2:
        sl = slice(ntok, ntok + blk)
        _, S = orc.kda_sequence(f64(q[sl]), f64(k[sl]), f64(v[sl]), f64(g[sl]), f64(beta[sl]), S)
        ntok += min(blk, q.shape[0] - ntok)
    t_pre = time.perf_counter() - t0
    pre_headtok_s = ntok * Hs / t_pre
    # decode sample: 16 sequences x all heads, repeated steps
    st = dec["steps"][0]
    Ns = 16
    Sd = f64(dec["state"][:Ns])
    t0 = time.perf_counter()
    nstep = 0
    while time.perf_counter() - t0 < budget_s / 2:
        Sd, _ = orc.kda_decode_step(Sd, *(f64(st[n][:Ns]) for n in ("q", "k", "v", "g", "beta")))
        nstep += 1
    t_dec = time.perf_counter() - t0
    dec_pairs_s = nstep * Ns * Sd.shape[1] / t_dec
    wall = time.perf_counter() - wall0
    cores = max(1, round((time.process_time() - cpu0) / wall))
    B, T, H = pre["q"].shape[:3]
    N = dec["state"].shape[0]
    t_step = B * T * H / pre_headtok_s + N * H / dec_pairs_s
    try:  # BLAS threads the oracle's numpy could use
        import threadpoolctl
        blas = [p.get("num_threads") for p in threadpoolctl.threadpool_info() if p.get("user_api") == "blas"]
    except Exception:
        blas = []
    return {
        "value": (B * T + N) / t_step,
        "unit": "tokens/s",
        "cores": cores,
        "affinity_cpus": len(os.sched_getaffinity(0)),
        "blas_threads": blas[0] if blas else None,
        "kind": "oracle",
        "sample": ("fp64 numpy oracle: prefill on %d of %d heads x %d tokens (%.1f s), decode step on %d of %d "
                   "sequences x %d heads x %d steps (%.1f s); step time scaled to all heads and sequences"
                   % (Hs, H, ntok, t_pre, Ns, N, H, nstep, t_dec)),
        "prefill_tokens_per_s": pre_headtok_s / H,
        "decode_tokens_per_s": dec_pairs_s / H,
    }


CONFIGS = (("0", "tiny_f32"), ("1", "minikimi_bf16"), ("2", "mini1h_g64_bf16"), ("3", "varlen_bf16"),
           ("4a", "k3_prefill_bf16"))


def run_configs(warmup, steps):
    """Per-configuration figures (not the bench line): every prefill workload
    timed on its own (median of `steps` calls with final states, after
    `warmup`), the decode workload's 64 consecutive steps, and the CPU oracle
    on a bounded sample of each.  One JSON line per configuration."""
    import numpy as np
    import torch
    import oracle.kda_oracle as orc
    from gated_delta_rule_04_amd import inputs, kda

    f64 = lambda t: t.double().numpy()
    for cfg, name in CONFIGS:
        d = inputs.workload_prefill(name)
        P = {n: d[n].cuda() for n in ("q", "k", "v", "g", "beta")}
        cu = None if d.get("cu_seqlens") is None else d["cu_seqlens"].cuda()
        B, T, H, dk = d["q"].shape
        dv, gg = d["v"].shape[-1], d["g_group"]
        N = B if cu is None else cu.numel() - 1
        call = lambda: kda.chunk_fwd(P["q"], P["k"], P["v"], P["g"], P["beta"], output_final_state=True,
                                     cu_seqlens=cu)
        for _ in range(warmup):
            call()
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
        for e in ev:
            e[0].record()
            call()
            e[1].record()
        torch.cuda.synchronize()
        ms = pct([e[0].elapsed_time(e[1]) for e in ev], 50)
        elem = d["q"].element_size()
        nbytes, flops = alg_prefill(B, T, H, dk, dv, gg, elem=elem, N=N)
        # the oracle on a bounded sample: head 0 of the first sequence, about 2 s
        q, k, v, g, beta = (f64(d[n][0, :, :1]) for n in ("q", "k", "v", "g", "beta"))
        S = np.zeros((1, dk, dv))
        t0, ntok = time.perf_counter(), 0
        while ntok < q.shape[0] and time.perf_counter() - t0 < 2.0:
            sl = slice(ntok, ntok + 128)
            _, S = orc.kda_sequence(q[sl], k[sl], v[sl], orc.expand_decay(g[sl], dk, gg), beta[sl], S)
            ntok += min(128, q.shape[0] - ntok)
        orc_headtok_s = ntok / (time.perf_counter() - t0)
        print(json.dumps({"config": cfg, "workload": name, "B": B, "T": T, "H": H, "dk": dk, "dv": dv,
                          "g_group": gg, "num_seqs": N, "dtype": str(d["q"].dtype).replace("torch.", ""),
                          "ms_median": ms, "tokens_per_s": B * T / (ms * 1e-3),
                          "alg_bytes": nbytes, "alg_gbs": nbytes / (ms * 1e-3) / 1e9,
                          "hbm_frac": nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                          "alg_tflops": flops / (ms * 1e-3) / 1e12,
                          "mfma_frac": flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                          "oracle_tokens_per_s": orc_headtok_s / H, "oracle_sample": "%d tokens of one head" % ntok}),
              flush=True)
        del P, cu, d
    dec = inputs.workload_decode("k3_decode_bf16")
    state = dec["state"].cuda()
    Nd, H, dk, dv = state.shape
    D = [{n: st[n].cuda() for n in st} for st in dec["steps"]]
    od = torch.empty((Nd, H, dv), dtype=torch.bfloat16, device="cuda")
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(D) + 1)]
    ev[0].record()
    for i, s in enumerate(D):
        kda.recurrent_step(s["q"], s["k"], s["v"], s["g"], s["beta"], state, out=od)
        ev[i + 1].record()
    torch.cuda.synchronize()
    ms = pct([ev[i].elapsed_time(ev[i + 1]) for i in range(len(D))], 50)
    nbytes = alg_decode(Nd, H, dk, dv, 1)
    Sd = f64(dec["state"][:4])
    t0, nstep = time.perf_counter(), 0
    while time.perf_counter() - t0 < 2.0:
        Sd, _ = orc.kda_decode_step(Sd, *(f64(dec["steps"][0][n][:4]) for n in ("q", "k", "v", "g", "beta")))
        nstep += 1
    print(json.dumps({"config": "4b", "workload": "k3_decode_bf16", "N": Nd, "H": H, "dk": dk, "dv": dv,
                      "steps": len(D), "ms_median_per_step": ms, "tokens_per_s": Nd / (ms * 1e-3),
                      "alg_bytes_per_step": nbytes, "alg_gbs": nbytes / (ms * 1e-3) / 1e9,
                      "hbm_frac": nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                      "oracle_tokens_per_s": nstep * 4 / (time.perf_counter() - t0),
                      "oracle_sample": "4 sequences x %d heads, %d steps" % (H, nstep)}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=10)  # the clocks settle within the first ~8 prefill calls
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--configs", action="store_true",
                    help="only print per-configuration figures (one JSON line per configuration)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="only run one plain device copy of this many MiB (scale for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: the KDA hot path shards by sequences and heads with no exchange, "
              "so only --gpus 1 is supported", file=sys.stderr)
        sys.exit(2)

    if args.configs:
        run_configs(args.warmup, args.steps)
        return

    import torch
    from gated_delta_rule_04_amd import inputs, kda

    if args.copy_calibration_mib:
        n = args.copy_calibration_mib << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "read_bytes": n, "write_bytes": n}), flush=True)
        return

    t_gen = time.perf_counter()
    pre = inputs.workload_prefill("k3_prefill_bf16")
    dec = inputs.workload_decode("k3_decode_bf16")
    t_gen = time.perf_counter() - t_gen
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    P = {n: pre[n].to(dev) for n in ("q", "k", "v", "g", "beta")}
    B, T, H, dk = pre["q"].shape
    dv = pre["v"].shape[-1]
    g_group = pre["g_group"]
    o = torch.empty((B, T, H, dv), dtype=torch.bfloat16, device=dev)
    ht = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    state = dec["state"].to(dev)
    N = state.shape[0]
    D = [{n: st[n].to(dev) for n in st} for st in dec["steps"]]
    od = torch.empty((N, H, dv), dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()

    def step(i, ev=None):
        if ev is not None:
            ev[0].record()
        kda.chunk_fwd(P["q"], P["k"], P["v"], P["g"], P["beta"], output_final_state=True, out=o, final_state=ht)
        if ev is not None:
            ev[1].record()
        s = D[i % len(D)]
        kda.recurrent_step(s["q"], s["k"], s["v"], s["g"], s["beta"], state, out=od)
        if ev is not None:
            ev[2].record()

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i, evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    pre_ms = [e[0].elapsed_time(e[1]) for e in evs]
    dec_ms = [e[1].elapsed_time(e[2]) for e in evs]
    step_ms = [e[0].elapsed_time(e[2]) for e in evs]
    mean = lambda x: sum(x) / len(x)
    ms_step = wall * 1e3 / args.steps
    pre_avg, dec_avg = mean(pre_ms), mean(dec_ms)

    # Overlapped pass (outside the timed region).  The prefill of one sequence
    # and the decode step of 256 others are independent; the prefill's
    # workgroups hold 192 of the 256 CUs (one per CU: 157 KB of LDS) and use
    # under a third of HBM, so the decode step can run beside it on a second
    # stream (default priority), joined at the end of the step.
    main = torch.cuda.current_stream()
    side = torch.cuda.Stream()

    def step_overlapped(i, ev=None):
        # ev: prefill start/end (main stream), decode start/end (side stream)
        fork = torch.cuda.Event()
        fork.record(main)
        side.wait_event(fork)
        with torch.cuda.stream(side):
            if ev is not None:
                ev[2].record(side)
            s = D[i % len(D)]
            kda.recurrent_step(s["q"], s["k"], s["v"], s["g"], s["beta"], state, out=od)
            if ev is not None:
                ev[3].record(side)
        if ev is not None:
            ev[0].record(main)
        kda.chunk_fwd(P["q"], P["k"], P["v"], P["g"], P["beta"], output_final_state=True, out=o, final_state=ht)
        if ev is not None:
            ev[1].record(main)
        join = torch.cuda.Event()
        join.record(side)
        main.wait_event(join)

    for i in range(args.warmup):
        step_overlapped(i)
    oev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for i in range(args.steps):
        step_overlapped(args.warmup + args.steps + i, oev[i])
    torch.cuda.synchronize()
    ms_step_ovl = (time.perf_counter() - t1) * 1e3 / args.steps
    pre_ovl_ms = [e[0].elapsed_time(e[1]) for e in oev]
    dec_ovl_ms = [e[2].elapsed_time(e[3]) for e in oev]

    pre_bytes, pre_flops = alg_prefill(B, T, H, dk, dv, g_group)
    dec_bytes = alg_decode(N, H, dk, dv, g_group)
    pre_gbs = pre_bytes / (pre_avg * 1e-3) / 1e9
    dec_gbs = dec_bytes / (dec_avg * 1e-3) / 1e9
    pre_tfs = pre_flops / (pre_avg * 1e-3) / 1e12
    tokens = B * T + N
    traffic_p = read_traffic("prefill")
    traffic_d = read_traffic("decode")

    line = {
        "metric": METRIC,
        "value": tokens / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "kimi_k3_heads: prefill B=1 T=32768 H=96 dk=dv=128 + decode N=256 H=96 dk=dv=128",
            "prefill": {"B": B, "T": T, "H": H, "dk": dk, "dv": dv, "g_group": g_group, "final_state": True},
            "decode": {"N": N, "H": H, "dk": dk, "dv": dv, "g_group": g_group, "state": "fp32"},
            "io_dtype": "bf16", "state_dtype": "fp32", "accumulate": "fp32",
        },
        "roofline": {
            "kernel": "chunk_fwd_pipe_kernel (prefill, bf16)",
            "bound": "hbm",
            "achieved": pre_gbs,
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": pre_gbs / PEAK_HBM_GBS,
            "traffic": traffic_p,
            "alg_bytes_per_launch": pre_bytes,
            "avg_launch_ms": pre_avg,
        },
        # MFMA beside HBM for the prefill: algorithmic flops against the bf16
        # dense peak (the prefill's arithmetic intensity, ~104 flop/B at d=128,
        # is below the MI355X ridge of ~315 flop/B, so HBM is the binding roof)
        "roofline_prefill_mfma": {
            "kernel": "chunk_fwd_pipe_kernel (prefill, bf16)",
            "bound": "mfma",
            "achieved": pre_tfs,
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": pre_tfs / PEAK_BF16_TFLOPS,
            "alg_flops_per_launch": pre_flops,
            "avg_launch_ms": pre_avg,
        },
        "roofline_decode": {
            "kernel": "decode_step_kernel",
            "bound": "hbm",
            "achieved": dec_gbs,
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": dec_gbs / PEAK_HBM_GBS,
            "traffic": traffic_d,
            "alg_bytes_per_launch": dec_bytes,
            "avg_launch_ms": dec_avg,
        },
        "prefill": {
            "tokens_per_s": B * T / (pre_avg * 1e-3),
            "head_tokens_per_s": B * T * H / (pre_avg * 1e-3),
            "ms": pre_avg,
            "ms_min": min(pre_ms),
            "ms_median": pct(pre_ms, 50),
            "ms_p10": pct(pre_ms, 10),
            "ms_p90": pct(pre_ms, 90),
            "alg_tflops": pre_tfs,
            "mfma_frac_alg": pre_tfs / PEAK_BF16_TFLOPS,
            "hbm_frac_alg": pre_gbs / PEAK_HBM_GBS,
        },
        "decode": {
            "tokens_per_s": N / (dec_avg * 1e-3),
            "head_tokens_per_s": N * H / (dec_avg * 1e-3),
            "ms_per_step": dec_avg,
            "ms_min": min(dec_ms),
            "ms_median": pct(dec_ms, 50),
            "ms_p10": pct(dec_ms, 10),
            "ms_p90": pct(dec_ms, 90),
            "hbm_frac_alg": dec_gbs / PEAK_HBM_GBS,
        },
        "overlapped_step": {
            "what": "the same step with the decode on a second stream beside the prefill (outside the timed region)",
            "ms_per_step": ms_step_ovl,
            "tokens_per_s": tokens / (ms_step_ovl * 1e-3),
            "prefill_ms": mean(pre_ovl_ms),
            "decode_ms": mean(dec_ovl_ms),
        },
        "event_ms_per_step": mean(step_ms),
        "input_gen_s": t_gen,
    }
    # The decode workload as stated: its consecutive steps from the initial
    # state (carried), each step timed on its own (outside the timed region).
    st_run = dec["state"].to(dev)
    ev_run = [torch.cuda.Event(enable_timing=True) for _ in range(len(D) + 1)]
    ev_run[0].record()
    for i, s in enumerate(D):
        kda.recurrent_step(s["q"], s["k"], s["v"], s["g"], s["beta"], st_run, out=od)
        ev_run[i + 1].record()
    torch.cuda.synchronize()
    run_ms = [ev_run[i].elapsed_time(ev_run[i + 1]) for i in range(len(D))]
    run_med = pct(run_ms, 50)
    line["decode"]["consecutive_steps"] = {
        "steps": len(D),
        "ms_total": sum(run_ms),
        "ms_median": run_med,
        "ms_p10": pct(run_ms, 10),
        "ms_p90": pct(run_ms, 90),
        "tokens_per_s": N / (run_med * 1e-3),
        "hbm_frac_alg": dec_bytes / (run_med * 1e-3) / 1e9 / PEAK_HBM_GBS,
    }
    # the decode workload as stated (64 back-to-back steps): its own roofline
    # line, beside the step timed between prefill calls above
    line["roofline_decode_consecutive"] = {
        "kernel": "decode_step_kernel (64 consecutive steps, median step)",
        "bound": "hbm",
        "achieved": dec_bytes / (run_med * 1e-3) / 1e9,
        "peak": PEAK_HBM_GBS,
        "unit": "GB/s",
        "frac": dec_bytes / (run_med * 1e-3) / 1e9 / PEAK_HBM_GBS,
        "alg_bytes_per_launch": dec_bytes,
        "median_launch_ms": run_med,
    }
    del st_run
    # Serving form (outside the timed step above): the same decode inputs over a
    # bf16 state pool, sequences in shuffled slots of a larger pool.
    ns = N + N // 4
    slots = torch.randperm(ns, generator=torch.Generator().manual_seed(17))[:N].to(torch.int32).to(dev)
    pool = torch.zeros((ns, H, dk, dv), dtype=torch.bfloat16, device=dev)
    pool[slots.long()] = state.to(torch.bfloat16)
    for i in range(args.warmup):
        s = D[i % len(D)]
        kda.recurrent_step_pool(s["q"], s["k"], s["v"], s["g"], s["beta"], pool, slots, out=od)
    pev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    for i in range(args.steps):
        s = D[i % len(D)]
        pev[i][0].record()
        kda.recurrent_step_pool(s["q"], s["k"], s["v"], s["g"], s["beta"], pool, slots, out=od)
        pev[i][1].record()
    torch.cuda.synchronize()
    pool_ms = [e[0].elapsed_time(e[1]) for e in pev]
    pool_avg = mean(pool_ms)
    pool_bytes = alg_decode_pool(N, H, dk, dv, g_group)
    line["decode_pool_bf16"] = {
        "kernel": "decode_step_kernel (bf16 state pool, slot indirection)",
        "config": {"N": N, "H": H, "dk": dk, "dv": dv, "num_slots": ns, "state": "bf16"},
        "tokens_per_s": N / (pool_avg * 1e-3),
        "ms_per_step": pool_avg,
        "ms_min": min(pool_ms),
        "alg_bytes_per_launch": pool_bytes,
        "hbm_frac_alg": pool_bytes / (pool_avg * 1e-3) / 1e9 / PEAK_HBM_GBS,
    }

    # The same pool step with the output gate (logits [N, H, dv]), and over a
    # float16 state pool of the same bytes.
    def time_pool(p, gate):
        for i in range(args.warmup):
            s = D[i % len(D)]
            kda.recurrent_step_pool(s["q"], s["k"], s["v"], s["g"], s["beta"], p, slots, out=od, o_gate=gate)
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
        for i in range(args.steps):
            s = D[i % len(D)]
            ev[i][0].record()
            kda.recurrent_step_pool(s["q"], s["k"], s["v"], s["g"], s["beta"], p, slots, out=od, o_gate=gate)
            ev[i][1].record()
        torch.cuda.synchronize()
        return mean([e[0].elapsed_time(e[1]) for e in ev])

    zg = torch.randn((N, H, dv), generator=torch.Generator().manual_seed(18)).to(torch.bfloat16).to(dev)
    gated_ms = time_pool(pool, zg)
    del pool
    pool16 = torch.zeros((ns, H, dk, dv), dtype=torch.float16, device=dev)
    pool16[slots.long()] = state.to(torch.float16)
    f16_ms = time_pool(pool16, None)
    del pool16
    gate_bytes = N * H * dv * 2
    line["decode_pool_bf16"]["with_output_gate"] = {
        "ms_per_step": gated_ms,
        "hbm_frac_alg": (pool_bytes + gate_bytes) / (gated_ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
    }
    line["decode_pool_bf16"]["f16_state"] = {
        "ms_per_step": f16_ms,
        "hbm_frac_alg": pool_bytes / (f16_ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
    }
    # Short causal convolution (outside the timed step): one K3 projection's
    # width over the prefill tokens, W = 4.
    Cc, Wc = H * dk, 4
    gc = torch.Generator().manual_seed(19)
    xc = torch.randn((B, T, Cc), generator=gc).to(torch.bfloat16).to(dev)
    wc = (0.5 * torch.randn((Cc, Wc), generator=gc)).to(torch.bfloat16).to(dev)
    yc = torch.empty_like(xc)
    for _ in range(args.warmup):
        kda.short_conv_fwd(xc, wc, out=yc)
    cev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    for i in range(args.steps):
        cev[i][0].record()
        kda.short_conv_fwd(xc, wc, out=yc)
        cev[i][1].record()
    torch.cuda.synchronize()
    conv_ms = [e[0].elapsed_time(e[1]) for e in cev]
    conv_avg = mean(conv_ms)
    conv_bytes = 2 * (2 * B * T * Cc) + 2 * Cc * Wc
    line["short_conv_bf16"] = {
        "kernel": "short_conv_fwd_kernel",
        "config": {"B": B, "T": T, "C": Cc, "W": Wc},
        "tokens_per_s": B * T / (conv_avg * 1e-3),
        "ms": conv_avg,
        "ms_min": min(conv_ms),
        "alg_bytes_per_launch": conv_bytes,
        "hbm_frac_alg": conv_bytes / (conv_avg * 1e-3) / 1e9 / PEAK_HBM_GBS,
    }
    # its backward (dx, dweight), with a seeded cotangent
    dyc = torch.randn((B, T, Cc), generator=gc).to(torch.bfloat16).to(dev)
    cws = torch.empty(kda.lib().kda_short_conv_bwd_workspace_bytes(B, T, Cc, Wc), dtype=torch.uint8, device=dev)
    for _ in range(args.warmup):
        kda.short_conv_bwd(xc, wc, dyc, workspace=cws)
    cbev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    for i in range(args.steps):
        cbev[i][0].record()
        kda.short_conv_bwd(xc, wc, dyc, workspace=cws)
        cbev[i][1].record()
    torch.cuda.synchronize()
    cb_avg = mean([e[0].elapsed_time(e[1]) for e in cbev])
    cb_bytes = 2 * (3 * B * T * Cc) + 2 * Cc * Wc + 4 * Cc * Wc
    line["short_conv_bf16"]["backward"] = {
        "kernels": "short_conv_bwd_kernel, short_conv_bwd_weight_kernel",
        "ms": cb_avg,
        "alg_bytes_per_call": cb_bytes,
        "hbm_frac_alg": cb_bytes / (cb_avg * 1e-3) / 1e9 / PEAK_HBM_GBS,
    }
    # A plain device copy of the same bytes (torch's copy kernel; outside the
    # timed step): the rate a streaming read-and-write kernel reaches on this
    # GPU, context for the HBM fractions (all of which are against 8 TB/s).
    for _ in range(args.warmup):
        yc.copy_(xc)
    yev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    for i in range(args.steps):
        yev[i][0].record()
        yc.copy_(xc)
        yev[i][1].record()
    torch.cuda.synchronize()
    cp_avg = mean([e[0].elapsed_time(e[1]) for e in yev])
    cp_bytes = 2 * (2 * B * T * Cc)
    line["copy_reference"] = {
        "what": "torch copy_ of a bf16 [T, C] tensor (read once, written once), the short conv's bytes",
        "bytes": cp_bytes,
        "ms": cp_avg,
        "gbs": cp_bytes / (cp_avg * 1e-3) / 1e9,
        "hbm_frac": cp_bytes / (cp_avg * 1e-3) / 1e9 / PEAK_HBM_GBS,
    }
    del xc, yc, dyc, cws
    # Prefill with the fused gate/normalisation prologue (outside the timed
    # step): the same tensors taken as raw projections (q, k rows, gate logits
    # f = g, write logits b = beta), A_log = 0 and dt_bias = -2 per channel.
    A_log = torch.zeros((H, dk // g_group), dtype=torch.float32, device=dev)
    dt_bias = torch.full((H, dk // g_group), -2.0, dtype=torch.float32, device=dev)
    for _ in range(args.warmup):
        kda.chunk_fwd_prologue(P["q"], P["k"], P["v"], P["g"], P["beta"], A_log, dt_bias, output_final_state=True,
                               out=o, final_state=ht)
    rev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    for i in range(args.steps):
        rev[i][0].record()
        kda.chunk_fwd_prologue(P["q"], P["k"], P["v"], P["g"], P["beta"], A_log, dt_bias, output_final_state=True,
                               out=o, final_state=ht)
        rev[i][1].record()
    torch.cuda.synchronize()
    pro_ms = [e[0].elapsed_time(e[1]) for e in rev]
    pro_avg = mean(pro_ms)
    pro_bytes = pre_bytes + 2 * H * (dk // g_group) * 4
    line["prefill_prologue_bf16"] = {
        "kernel": "chunk_fwd_pipe_kernel with the fused prologue",
        "config": {"B": B, "T": T, "H": H, "dk": dk, "dv": dv, "g_group": g_group, "final_state": True},
        "tokens_per_s": B * T / (pro_avg * 1e-3),
        "ms": pro_avg,
        "ms_min": min(pro_ms),
        "alg_bytes_per_launch": pro_bytes,
        "hbm_frac_alg": pro_bytes / (pro_avg * 1e-3) / 1e9 / PEAK_HBM_GBS,
        "separate_pass_bytes_avoided": 2 * 2 * B * T * H * (2 * dk + dk // g_group + 1),
    }
    # the backward through the prologue (prepare, chunked backward, chain rule)
    gp = torch.Generator().manual_seed(29)
    dop = torch.randn((B, T, H, dv), generator=gp).to(torch.bfloat16).to(dev)
    dhtp = torch.randn((B, H, dk, dv), generator=gp).to(dev)
    pws = torch.empty(kda.lib().kda_chunk_bwd_prologue_workspace_bytes(B, T, H, dk, dv, B, 0, g_group, kda.KDA_BF16),
                      dtype=torch.uint8, device=dev)
    pout = None  # the gradients' buffers, allocated by the first call and reused (no allocation inside the timing)
    for _ in range(min(args.warmup, 3)):
        pout = kda.chunk_bwd_prologue(P["q"], P["k"], P["v"], P["g"], P["beta"], A_log, dt_bias, dop, dht=dhtp,
                                      workspace=pws, out=pout)
    pbev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(min(args.steps, 5))]
    for e in pbev:
        e[0].record()
        pout = kda.chunk_bwd_prologue(P["q"], P["k"], P["v"], P["g"], P["beta"], A_log, dt_bias, dop, dht=dhtp,
                                      workspace=pws, out=pout)
        e[1].record()
    torch.cuda.synchronize()
    pb_avg = mean([e[0].elapsed_time(e[1]) for e in pbev])
    line["prefill_prologue_bf16"]["backward"] = {
        "entry_point": "kda_chunk_bwd_prologue",
        "ms": pb_avg,
        "tokens_per_s": B * T / (pb_avg * 1e-3),
        "alg_bytes_per_call": alg_backward(B, T, H, dk, dv, g_group) + 2 * 2 * H * (dk // g_group) * 4,
    }
    line["prefill_prologue_bf16"]["backward"]["hbm_frac_alg"] = (
        line["prefill_prologue_bf16"]["backward"]["alg_bytes_per_call"] / (pb_avg * 1e-3) / 1e9 / PEAK_HBM_GBS)
    del A_log, dt_bias, dop, dhtp, pws, pout
    # Backward pass of the prefill (outside the timed step): the same inputs,
    # seeded cotangents of o and of the final state.
    gb = torch.Generator().manual_seed(23)
    dob = torch.randn((B, T, H, dv), generator=gb).to(torch.bfloat16).to(dev)
    dhtb = torch.randn((B, H, dk, dv), generator=gb).to(dev)
    wsb = torch.empty(kda.bwd_workspace_bytes(B, T, H, dk, dv, B, False, torch.bfloat16), dtype=torch.uint8,
                      device=dev)
    gout = None
    for _ in range(args.warmup):
        gout = kda.chunk_bwd(P["q"], P["k"], P["v"], P["g"], P["beta"], dob, dht=dhtb, workspace=wsb, out=gout)
    bev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    for i in range(args.steps):
        bev[i][0].record()
        gout = kda.chunk_bwd(P["q"], P["k"], P["v"], P["g"], P["beta"], dob, dht=dhtb, workspace=wsb, out=gout)
        bev[i][1].record()
    torch.cuda.synchronize()
    bwd_ms = [e[0].elapsed_time(e[1]) for e in bev]
    bwd_avg = mean(bwd_ms)
    bwd_bytes = alg_backward(B, T, H, dk, dv, g_group)
    line["chunk_bwd_bf16"] = {
        "kernels": "chunk_fwd_pipe_kernel (keeping chunk states), chunk_bwd_prep_kernel, chunk_bwd_dh_kernel, "
                   "chunk_bwd_local_kernel",
        "config": {"B": B, "T": T, "H": H, "dk": dk, "dv": dv, "g_group": g_group, "dht": True},
        "tokens_per_s": B * T / (bwd_avg * 1e-3),
        "ms": bwd_avg,
        "ms_min": min(bwd_ms),
        "alg_bytes_per_call": bwd_bytes,
        "hbm_frac_alg": bwd_bytes / (bwd_avg * 1e-3) / 1e9 / PEAK_HBM_GBS,
        "workspace_bytes": wsb.numel(),
    }
    # Training pair: the forward keeps its chunk states in the workspace and
    # the backward reads them instead of recomputing them.
    fo = fh = None

    def fwd_save():
        return kda.chunk_fwd_save(P["q"], P["k"], P["v"], P["g"], P["beta"], output_final_state=True, out=fo,
                                  final_state=fh, workspace=wsb)[:2]

    def bwd_saved():
        return kda.chunk_bwd(P["q"], P["k"], P["v"], P["g"], P["beta"], dob, dht=dhtb, workspace=wsb, out=gout,
                             states_saved=True)

    for _ in range(args.warmup):
        fo, fh = fwd_save()
        gout = bwd_saved()
    tev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    for i in range(args.steps):
        tev[i][0].record()
        fo, fh = fwd_save()
        tev[i][1].record()
        gout = bwd_saved()
        tev[i][2].record()
    torch.cuda.synchronize()
    fs_ms = [e[0].elapsed_time(e[1]) for e in tev]
    bs_ms = [e[1].elapsed_time(e[2]) for e in tev]
    line["chunk_bwd_bf16"]["training_pair"] = {
        "entry_points": "kda_chunk_fwd_save, kda_chunk_bwd_saved",
        "fwd_save_ms": mean(fs_ms),
        "bwd_saved_ms": mean(bs_ms),
        "bwd_saved_ms_min": min(bs_ms),
        "fwd_plus_bwd_ms": mean(fs_ms) + mean(bs_ms),
    }
    del dob, dhtb, wsb, gout, fo, fh
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(pre, dec)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
