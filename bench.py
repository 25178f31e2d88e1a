"""Benchmark of the VC-Attention hot path on one MI355X.

A step is one pass of the whole path over one batch of the Wan2.2-shaped synthetic
workload (B=1, H=40, N=70,400, d=128): warm-started k-means (550 clusters, 2
iterations) -> fused quantiser -> VC-Attention (V-Smooth + ExpCast-FP8). Inputs are
resident in HBM before the timed region. `value` is attention-equivalent TFLOPS of the
whole step, 4*B*H*N^2*d / t_step; the per-stage times and the attention kernel's own
TFLOPS (from HIP events on the launch stream) are reported beside it.

Usage: python bench.py [--steps K] [--warmup W] [--gpus 1] [--workload wan|sweepN|schedule|balance|oracle]
                       [--no-cpu-baseline] [--attention-only [--attn-mode vc|vc_e5m2|expcast|exp]]
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

METRIC = "FP8 VC-attention TFLOPS & % FP8 MFMA peak at N=70,400,H=40,d=128"
FP8_PEAK_TFLOPS = 5000.0       # MI355X dense FP8 MFMA (published)
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense BF16 MFMA (published)
HBM_PEAK_GBS = 8000.0
BETA = -0.35
BETA_E5M2 = -0.17              # minimax offset of the E5M2 ExpCast code


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def make_inputs(kind, B, H, N, d, seed):
    import numpy as np
    import torch
    import synth
    t0 = time.time()
    w = synth.gen(kind, seed=seed, B=B, H=H, N=N, d=d)
    log("[bench] generated %s inputs B=%d H=%d N=%d d=%d in %.1fs" % (kind, B, H, N, d, time.time() - t0))

    def dev(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    out = {k: dev(v) for k, v in w.items() if k != "meta"}
    return out, w


def profiled_traffic():
    """HBM bytes per attention launch from the committed rocprofv3 PMC summary, valid only
    while the kernel sources are the ones that were profiled (else None)."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "attn_fwd_wan_traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    csrc = os.path.join(ROOT, "bit_attention_video_online_amd", "csrc")
    src = b"".join(open(os.path.join(csrc, f), "rb").read() for f in ("vc_attention.hip", "vc_device.h"))
    if hashlib.sha256(src).hexdigest() != rec.get("source_sha256"):
        return None
    return round((rec["fetch_bytes"] + rec["write_bytes"]) / 1e9, 3)


def cpu_baseline(host, K_clusters, sample_rows, threads, gpu=None):
    """Time the oracle on a bounded sample of the same workload (head 0), and compare the GPU's
    head 0 with what the oracle computed: mismatch counts of every bit-exact output (k-means
    centroids, labels and permutation; quantiser codes, scales and means; the in-kernel ExpCast
    bytes of the last key block on sampled rows) and the output's relative L2 distance from the
    emulation on those rows (scores in the matrix core's precision, output rounded to bf16)."""
    import numpy as np
    import oracle
    Q, K, V, Vp = (host[k][0, 0] for k in ("Q", "K", "V", "V_prev"))
    N, d = Q.shape
    t0 = time.time()
    _, _, Cw = oracle.kmeans(Vp, K_clusters, 4, cold=True)          # warm-start state (not timed)
    t1 = time.time()
    labels, perm, C = oracle.kmeans(V, K_clusters, 2, cold=False, C=Cw)
    t2 = time.time()
    q = oracle.quantize(Q, K, V, perm, oracle.FLAG_KSMOOTH | oracle.FLAG_VSMOOTH)
    t3 = time.time()
    rows = np.linspace(0, N - 1, sample_rows).astype(np.int32)
    oracle.attention_emul(q, rows, beta=BETA, mode=oracle.MODE_EXPCAST)
    t4 = time.time()
    t_head = (t2 - t1) + (t3 - t2) + (t4 - t3) * N / sample_rows
    flops_head = 4.0 * N * N * d
    cpu = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    res = dict(value=flops_head / t_head / 1e12, unit="TFLOPS", cores=threads, kind="oracle", cpu=cpu,
               sample="head 0 of the workload: k-means (2 warm iterations, 550 clusters) and quantiser in full, "
                      "attention emulation on %d of %d query rows extrapolated x%.0f; per-head time %.1f s "
                      "(kmeans %.1f s, quantise %.1f s, attention %.1f s measured)"
                      % (sample_rows, N, N / sample_rows, t_head, t2 - t1, t3 - t2, t4 - t3),
               seconds_measured=round(t4 - t1, 2), warm_start_seconds=round(t1 - t0, 2))
    if gpu is not None:
        nb = N // 128
        g = gpu["q"]
        vq = g["Vq"].reshape(nb, d, 128).transpose(0, 2, 1).reshape(N, d)   # block-transposed -> row-major
        mis = {"centroids": int(np.count_nonzero(gpu["C"] != C)), "labels": int(np.count_nonzero(gpu["labels"] != labels)),
               "perm": int(np.count_nonzero(gpu["perm"] != perm))}
        for k in ("Qq", "sQ", "Kq", "sK", "sV", "mu", "mu_scaled"):
            mis[k] = int(np.count_nonzero(g[k] != q[k]))
        mis["Vq"] = int(np.count_nonzero(vq != q["Vq"]))
        prow = gpu["rows"]
        O_em, codes = oracle.attention_emul(q, prow, beta=BETA, mode=oracle.MODE_EXPCAST, dump_block=nb - 1,
                                            score="gfx950", out_bf16=True)
        mis["expcast_bytes_block_%d" % (nb - 1)] = int(np.count_nonzero(gpu["codes"] != codes))
        Og = gpu["O"].astype(np.float64)
        res["parity"] = {"mismatches": mis,
                         "elements_compared": {"centroids": int(C.size), "labels": int(N), "codes_per_tensor": int(N * d),
                                               "expcast_bytes": int(codes.size)},
                         "attention_rows": int(prow.size),
                         "attention_rel_l2_vs_emulation": float(np.linalg.norm(Og - O_em) / np.linalg.norm(O_em)),
                         "tolerance": 2e-3}
    return res


def exact_attention_rows(Qr, K, V):
    """softmax(Q K^T / sqrt(d)) V in binary64 for a few query rows (torch, on the device)."""
    import torch
    s = torch.mm(Qr, K.t().contiguous()) / (Qr.shape[1] ** 0.5)
    p = torch.softmax(s, dim=1)
    return p @ V


def error_columns(args, vc, torch, B, H, N, d, Kc, Qd, Kd, Vd, lab, perm, C, q, O, flags_q):
    """After the timed steps (the buffers hold the last step's results): the error of every path
    against binary64 exact attention (softmax(Q K^T / sqrt(d)) V from the bf16 inputs, torch on
    the device) on sampled rows of two heads, rMSE = ||O - O_exact||_F / ||O_exact||_F over the
    sampled rows. Paths: vc (V-Smooth + ExpCast, the timed output), vsmooth (V-Smooth, exp then
    cast), plain (no V-Smooth, exp then cast), expcast (no V-Smooth, ExpCast). Also returns the
    GPU's head-0 results for the oracle comparison of the CPU-baseline leg."""
    import numpy as np
    heads = (0, min(23, H - 1))
    rows = np.linspace(0, N - 1, args.error_rows).astype(np.int64)
    rows_t = torch.from_numpy(rows).cuda()
    Ovs = torch.empty_like(O)
    vc.vc_attention(q, Ovs, beta=BETA, flags=0)
    qp = vc.quantize_outputs(B, H, N, d)
    vc.vc_quantize(Qd, Kd, Vd, None, vc.VC_F_KSMOOTH, qp)
    Op = torch.empty_like(O)
    vc.vc_attention(qp, Op, beta=BETA, flags=0, restore_mean=False)
    Oe = torch.empty_like(O)
    vc.vc_attention(qp, Oe, beta=BETA, flags=vc.VC_F_EXPCAST, restore_mean=False)
    codes = torch.empty((B, H, N, 128), dtype=torch.uint8, device="cuda")
    Od = torch.empty_like(O)
    vc.vc_attention_dump(q, Od, N // 128 - 1, codes, beta=BETA, flags=vc.VC_F_EXPCAST)
    torch.cuda.synchronize()
    err = {k: [0.0, 0.0] for k in ("vc", "vsmooth", "plain", "expcast")}
    for h in heads:
        ex = exact_attention_rows(Qd[0, h][rows_t].double(), Kd[0, h].double(), Vd[0, h].double())
        for k, X in (("vc", O), ("vsmooth", Ovs), ("plain", Op), ("expcast", Oe)):
            diff = X[0, h][rows_t].double() - ex
            err[k][0] += float((diff * diff).sum())
            err[k][1] += float((ex * ex).sum())
    rmse = {k: round((a / b) ** 0.5, 6) for k, (a, b) in err.items()}
    errors = {"rmse_vs_fp64": rmse, "vc_below_plain_fp8": rmse["vc"] < rmse["plain"],
              "rows": "%d evenly spaced rows x heads %s, binary64 softmax(Q K^T / sqrt(d)) V from the bf16 inputs"
                      % (rows.size, list(heads)),
              "dump_output_identical": bool(torch.equal(Od, O))}
    prow = np.linspace(0, N - 1, 128).astype(np.int32)
    gpu = {"labels": lab[0, 0].cpu().numpy(), "perm": perm[0, 0].cpu().numpy(), "C": C[0, 0].cpu().numpy(),
           "q": {k: (v[0, 0].contiguous().view(torch.int16).cpu().numpy().view(np.uint16) if v.dtype == torch.bfloat16
                     else v[0, 0].cpu().numpy()) for k, v in q.items() if k != "mu_pack"},
           "rows": prow, "codes": codes[0, 0][torch.from_numpy(prow).long().cuda()].cpu().numpy(),
           "O": O[0, 0][torch.from_numpy(prow).long().cuda()].float().cpu().numpy()}
    del Ovs, qp, Op, Oe, codes, Od
    torch.cuda.empty_cache()
    log("[bench] rMSE vs binary64 exact attention: %s" % rmse)
    return errors, gpu


def device_info():
    """Name, compute units and the maximum shader clock the runtime reports for device 0."""
    import ctypes
    import torch
    prop = torch.cuda.get_device_properties(0)
    info = {"name": prop.name, "arch": getattr(prop, "gcnArchName", None), "compute_units": prop.multi_processor_count}
    try:
        hip = ctypes.CDLL("libamdhip64.so")
        v = ctypes.c_int(0)
        if hip.hipDeviceGetAttribute(ctypes.byref(v), 5, 0) == 0:  # hipDeviceAttributeClockRate (kHz)
            info["max_clock_mhz"] = v.value / 1000.0
    except OSError:
        pass
    return info


def measure_mfma_peak(grid=2048, iters=20000, reps=3):
    """Sustained rate of the attention kernel's FP8 matrix-core instruction (32x32x64, 131072
    FLOPs per wave instruction) with register operands and no memory traffic: best of `reps`
    timed launches each for fixed and pseudo-random operand bits (TFLOP/s)."""
    import torch
    import bit_attention_video_online_amd as vc
    out = torch.empty(grid * 256, dtype=torch.float32, device="cuda")
    flops = grid * 4.0 * iters * 4 * 131072
    res = {}
    for name, rnd in (("fixed_operands", 0), ("random_operands", 1)):
        vc.vc_debug_mfma_peak(grid, 200, rnd, out)
        best = None
        for _ in range(reps):
            e0 = torch.cuda.Event(enable_timing=True); e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            vc.vc_debug_mfma_peak(grid, iters, rnd, out)
            e1.record()
            e1.synchronize()
            t = e0.elapsed_time(e1) / 1e3
            best = t if best is None else min(best, t)
        res[name] = round(flops / best / 1e12, 1)
    return res


def exactness_spans(vc, torch, Kd, Vd, Cw, C1, N, d):
    """Exponent spans (largest exponent minus lowest significand bit, per (b,h), maximum over
    heads) of the step's inputs, against the sufficient conditions under which the k-means and
    quantiser sums are exact: sums of N terms need span <= 103 - 2 ceil(log2 N); the squared
    distances need the span of V together with the bf16-rounded centroids each assignment
    reads (the warm state Cw, then C1 after the first update) <= 50 - log2 d."""
    sv, sk = vc.vc_exponent_span(Vd), vc.vc_exponent_span(Kd)
    sc = [vc.vc_exponent_span(c, as_bf16=True) for c in (Cw, C1)]
    span = lambda s: int((s[..., 0] - s[..., 1]).max())
    dist = max(int((torch.maximum(sv[..., 0], c[..., 0]) - torch.minimum(sv[..., 1], c[..., 1])).max()) for c in sc)
    lim_sum = 103 - 2 * int(math.ceil(math.log2(N)))
    lim_dist = 50 - int(math.log2(d))
    out = {"V_span": span(sv), "K_span": span(sk), "V_with_centroids_span": dist, "sum_span_limit": lim_sum,
           "distance_span_limit": lim_dist}
    out["inside"] = out["V_span"] <= lim_sum and out["K_span"] <= lim_sum and dist <= lim_dist
    return out


def stage_rates(B, H, N, d, Kc, iters, avg):
    """Algorithmic bytes (and k-means FLOPs) per stage launch and the rates they give.

    quantiser, single-pass minimum: read Q, K, V (bf16) and the permutation; write the three
    code tensors, the Q/K block scales, the channel scales, mu (bf16), mu / s_V (fp32) and
    the matrix-core mean operand (bf16 hi/lo). The two-pass design re-reads K and V.
    k-means, per iteration: V read by the assignment and again by the centroid update,
    labels and permutation written once and read once, centroids read and written;
    assignment FLOPs 2 N K d per head (bf16 matrix core)."""
    nb = N // 128
    e = B * H * N * d
    quant = 3 * e * 2 + B * H * N * 4 + 3 * e + 2 * B * H * nb * 4 + B * H * d * 4 + B * H * nb * d * (2 + 4) \
        + B * H * ((nb + 7) // 8) * d * 2 * 2 * 2 * 8
    quant_two_pass = quant + 2 * e * 2
    clus = iters * (2 * e * 2 + 2 * 2 * B * H * N * 4 + 2 * B * H * Kc * d * 4)
    clus_flops = iters * 2.0 * B * H * N * Kc * d
    out = {}
    if avg.get("quantize"):
        t = avg["quantize"] / 1e3
        out["quantize"] = {"algorithmic_bytes": quant, "gbps": round(quant / t / 1e9, 1),
                           "two_pass_bytes": quant_two_pass, "two_pass_gbps": round(quant_two_pass / t / 1e9, 1),
                           "frac_hbm_peak": round(quant / t / 1e9 / HBM_PEAK_GBS, 4)}
    if avg.get("cluster"):
        t = avg["cluster"] / 1e3
        out["cluster"] = {"algorithmic_bytes": clus, "gbps": round(clus / t / 1e9, 1),
                          "frac_hbm_peak": round(clus / t / 1e9 / HBM_PEAK_GBS, 4),
                          "assign_flops": clus_flops, "assign_tflops": round(clus_flops / t / 1e12, 2),
                          "frac_bf16_peak": round(clus_flops / t / 1e12 / BF16_PEAK_TFLOPS, 4)}
    return out


def _oracle_c0():
    """The tiny configuration through the oracle in full: k-means (8 clusters, 4 cold
    iterations), quantiser, ExpCast attention emulation on all 1024 rows. Seconds per stage."""
    import numpy as np
    import synth
    import oracle
    w = synth.gen("tiny")
    Q, K, V = (w[k][0, 0] for k in ("Q", "K", "V"))
    t0 = time.perf_counter()
    _, perm, _ = oracle.kmeans(V, 8, 4, cold=True)
    t1 = time.perf_counter()
    q = oracle.quantize(Q, K, V, perm, oracle.FLAG_KSMOOTH | oracle.FLAG_VSMOOTH)
    t2 = time.perf_counter()
    oracle.attention_emul(q, np.arange(Q.shape[0], dtype=np.int32), beta=BETA, mode=oracle.MODE_EXPCAST)
    t3 = time.perf_counter()
    return {"kmeans_s": round(t1 - t0, 4), "quantize_s": round(t2 - t1, 4), "attention_s": round(t3 - t2, 4),
            "total_s": round(t3 - t0, 4), "threads": oracle.num_threads()}


def run_oracle_timing(args):
    """Oracle (CPU, not tuned) timings on the small configurations in full: tiny (B=1 H=1
    N=1024 d=128, whole VC path) with all host threads and with one thread, and the
    ExpCast-only configuration (B=1 H=8 N=8192 d=128: K smoothing, no V-Smooth, identity
    permutation) with all host threads. A reported baseline, not a target."""
    import subprocess
    import numpy as np
    import synth
    import oracle
    if args.workload == "oracle-c0":
        print(json.dumps(_oracle_c0()), flush=True)
        return
    cpu = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    res = {"workload": "oracle timing on the tiny and ExpCast-only configurations in full", "cpu": cpu,
           "nproc": os.cpu_count(), "omp_threads": oracle.num_threads()}
    c0 = _oracle_c0()
    c0["tflops_equiv"] = round(4.0 * 1024 * 1024 * 128 / c0["total_s"] / 1e12, 6)
    res["tiny_all_threads"] = c0
    env = dict(os.environ, OMP_NUM_THREADS="1")
    out = subprocess.run([sys.executable, os.path.abspath(__file__), "--workload", "oracle-c0"], env=env,
                         capture_output=True, text=True, check=True)
    c0s = json.loads(out.stdout.strip().splitlines()[-1])
    c0s["tflops_equiv"] = round(4.0 * 1024 * 1024 * 128 / c0s["total_s"] / 1e12, 6)
    res["tiny_one_thread"] = c0s
    w = synth.WORKLOADS["expcast"]
    H, N, d = w["H"], w["N"], w["d"]
    tq = ta = 0.0
    for h in range(H):
        g = synth.gen("expcast", heads=[h])
        Q, K, V = (g[k][0, 0] for k in ("Q", "K", "V"))
        t0 = time.perf_counter()
        q = oracle.quantize(Q, K, V, None, oracle.FLAG_KSMOOTH)
        t1 = time.perf_counter()
        oracle.attention_emul(q, np.arange(N, dtype=np.int32), beta=BETA, mode=oracle.MODE_EXPCAST)
        t2 = time.perf_counter()
        tq += t1 - t0
        ta += t2 - t1
        log("[oracle] expcast head %d: quantise %.2f s, attention %.2f s" % (h, t1 - t0, t2 - t1))
    res["expcast_all_threads"] = {"quantize_s": round(tq, 3), "attention_s": round(ta, 3),
                                  "total_s": round(tq + ta, 3),
                                  "tflops_equiv": round(4.0 * H * N * N * d / (tq + ta) / 1e12, 6),
                                  "threads": oracle.num_threads()}
    print(json.dumps(res), flush=True)


def run_schedule(args):
    """The 20-step amortised schedule on Wan-shaped inputs (seed 3): Q and K fixed, V drifts
    each step as V_s = bf16(V_{s-1} + xi * |V_{s-1}|), xi ~ N(0, 0.05^2) drawn with a seeded
    CUDA generator (stream state per step). Clustering runs at steps 0-4 (step 0 cold with 4
    iterations, steps 1-4 warm with 2) and steps 5-19 reuse step 4's permutation; every step
    quantises and runs attention. Reports per-step stage times, the clustering share
    sum t(cluster) / sum [t(quantize) + t(attention)], and the error against binary64 exact
    attention (computed with torch on the device) on sampled rows of head 0."""
    import numpy as np
    import torch
    import synth
    import bit_attention_video_online_amd as vc

    w = synth.WORKLOADS["schedule"]
    B, H, N, d, Kc, seed, S = 1, w["H"], w["N"], w["d"], w["clusters"], w["seed"], w["steps"]
    torch.cuda.set_device(0)
    dev, host = make_inputs("schedule", B, H, N, d, seed)
    Qd, Kd, V = dev["Q"], dev["K"], dev["V"].clone()
    C = torch.zeros((B, H, Kc, d), dtype=torch.float32, device="cuda")
    lab = torch.empty((B, H, N), dtype=torch.int32, device="cuda")
    perm = torch.empty((B, H, N), dtype=torch.int32, device="cuda")
    ws_c = vc.workspace(vc.vc_cluster_workspace_bytes(B, H, N, d, Kc))
    q = vc.quantize_outputs(B, H, N, d)
    ws_q = vc.workspace(vc.vc_quantize_workspace_bytes(B, H, N, d))
    O = torch.empty((B, H, N, d), dtype=torch.bfloat16, device="cuda")
    flags_q = vc.VC_F_KSMOOTH | vc.VC_F_VSMOOTH
    rows = np.linspace(0, N - 1, args.schedule_rows).astype(np.int32)
    rows_t = torch.from_numpy(rows).long().cuda()
    Qr = Qd[0, 0][rows_t].double()
    Kh = Kd[0, 0].double()
    gen = torch.Generator(device="cuda")
    cost = torch.empty((B, H), dtype=torch.float64, device="cuda")
    ws_cost = vc.workspace(int(vc.lib().vc_cluster_cost_workspace_bytes(B, H, N, d)))
    cost_ref = None
    mass = torch.zeros((B, H, Kc), dtype=torch.float32, device="cuda")
    steps = []
    for s in range(S):
        if s > 0:
            gen.manual_seed(seed * 1000 + s)
            xi = torch.randn(V.shape, generator=gen, device="cuda", dtype=torch.float32) * 0.05
            Vf = V.float()
            V = (Vf + xi * Vf.abs()).to(torch.bfloat16)
            del xi, Vf
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        ev[0].record()
        clustered, drift = False, None
        if args.refresh == "incremental":
            # cross-step incremental centroids: step 0 is the fixed schedule's cold 4-iteration
            # k-means (3 iterations, then a decay-0 incremental step = the 4th iteration, which
            # also sets every cluster's mass to its size); every later step re-assigns once
            # and folds the new members into the decayed running mean
            if s == 0:
                vc.vc_cluster(V, Kc, 3, True, C, lab, perm, ws=ws_c)
                vc.vc_cluster_incremental(V, 0.0, True, C, mass, lab, perm, ws=ws_c)
            else:
                vc.vc_cluster_incremental(V, args.decay, True, C, mass, lab, perm, ws=ws_c)
            clustered = True
        elif args.refresh == "fixed":
            if s == 0:
                vc.vc_cluster(V, Kc, 4, True, C, lab, perm, ws=ws_c)
            elif s <= 4:
                vc.vc_cluster(V, Kc, 2, False, C, lab, perm, ws=ws_c)
            clustered = s <= 4
        else:
            # drift-triggered refresh: the k-means objective of the current values under the
            # kept clustering, relative to its value right after the last clustering; the host
            # reads it back, so the decision's latency counts as clustering time
            if s == 0:
                vc.vc_cluster(V, Kc, 4, True, C, lab, perm, ws=ws_c)
                clustered = True
            else:
                vc.vc_cluster_cost(V, C, lab, cost, ws=ws_cost)
                drift = float((cost.cpu().numpy() / cost_ref).mean()) - 1.0
                if drift > args.drift_threshold:
                    vc.vc_cluster(V, Kc, 2, False, C, lab, perm, ws=ws_c)
                    clustered = True
            if clustered:
                vc.vc_cluster_cost(V, C, lab, cost, ws=ws_cost)
                cost_ref = cost.cpu().numpy()
        ev[1].record()
        vc.vc_quantize(Qd, Kd, V, perm, flags_q, q, ws=ws_q)
        ev[2].record()
        vc.vc_attention(q, O, beta=BETA, flags=vc.VC_F_EXPCAST)
        ev[3].record()
        torch.cuda.synchronize()
        tc, tq, ta = (ev[i].elapsed_time(ev[i + 1]) for i in range(3))
        O_ex = exact_attention_rows(Qr, Kh, V[0, 0].double())
        rmse = float(torch.linalg.norm(O[0, 0][rows_t].double() - O_ex) / torch.linalg.norm(O_ex))
        steps.append(dict(step=s, cluster_ms=round(tc, 3), quantize_ms=round(tq, 3), attention_ms=round(ta, 3),
                          rmse=round(rmse, 6), clustered=clustered,
                          drift=None if drift is None else round(drift, 5)))
        log("[schedule] step %2d: cluster %.3f ms%s, quantize %.3f ms, attention %.3f ms, rMSE %.4f%%%s"
            % (s, tc, " (clustered)" if clustered else "", tq, ta, 100 * rmse,
               "" if drift is None else ", drift %.4f" % drift))
    t_c = sum(x["cluster_ms"] for x in steps)
    t_qa = sum(x["quantize_ms"] + x["attention_ms"] for x in steps)
    sched = {"fixed": "cluster at steps 0-4 (cold x4, then warm x2), permutation of step 4 reused for steps 5-19",
             "drift": "cluster cold x4 at step 0; afterwards re-cluster (warm x2) whenever the mean over heads of "
                      "the k-means objective under the kept clustering exceeds its post-clustering value by more "
                      "than %g" % args.drift_threshold,
             "incremental": "cluster cold x4 at step 0; every later step one cross-step incremental update "
                            "(re-assignment, then centroids = decayed running member mean, decay %g)" % args.decay
             }[args.refresh]
    res = {"workload": "20-step amortised schedule, B=%d H=%d N=%d d=%d, %d clusters; %s" % (B, H, N, d, Kc, sched),
           "clusterings": sum(1 for x in steps if x["clustered"]),
           "clustering_share": round(t_c / t_qa, 5), "cluster_ms_total": round(t_c, 3),
           "quantize_attention_ms_total": round(t_qa, 3),
           "rmse_rows": "head 0, %d rows evenly spaced, vs binary64 softmax(Q K^T / sqrt(d)) V from the bf16 "
                        "inputs" % rows.size,
           "steps": steps}
    print(json.dumps(res), flush=True)


def run_balance(args):
    """Size-penalised (balanced) clustering against plain k-means on the Wan-shaped step:
    from the same warm state (cold 4-iteration k-means on the previous step's values and
    its cluster sizes), 2 warm iterations with lambda = kappa * J / (N/K), J the mean
    squared assignment distance of the current values under the warm clustering. Reports
    per kappa: k-means time, cluster-size spread, the share of 128-token key blocks that
    hold one cluster only, the k-means objective, and the attention error (V-Smooth +
    ExpCast) against binary64 exact attention on sampled rows of several heads."""
    import numpy as np
    import torch
    import bit_attention_video_online_amd as vc

    torch.cuda.set_device(0)
    B, H, N, d, Kc, seed = 1, 40, 70400, 128, 550, 2
    dev, _ = make_inputs("wan", B, H, N, d, seed)
    Qd, Kd, Vd, Vpd = dev["Q"], dev["K"], dev["V"], dev["V_prev"]
    Cw = torch.zeros((B, H, Kc, d), dtype=torch.float32, device="cuda")
    lab = torch.empty((B, H, N), dtype=torch.int32, device="cuda")
    perm = torch.empty((B, H, N), dtype=torch.int32, device="cuda")
    ws_c = vc.workspace(vc.vc_cluster_workspace_bytes(B, H, N, d, Kc))
    vc.vc_cluster(Vpd, Kc, 4, True, Cw, lab, perm, ws=ws_c)
    cnt_w = torch.stack([torch.bincount(lab[0, h].long(), minlength=Kc) for h in range(H)]).int().view(B, H, Kc)
    cost = torch.empty((B, H), dtype=torch.float64, device="cuda")
    ws_cost = vc.workspace(int(vc.lib().vc_cluster_cost_workspace_bytes(B, H, N, d)))
    vc.vc_cluster_cost(Vd, Cw, lab, cost, ws=ws_cost)
    J = float(cost.mean())
    q = vc.quantize_outputs(B, H, N, d)
    ws_q = vc.workspace(vc.vc_quantize_workspace_bytes(B, H, N, d))
    O = torch.empty((B, H, N, d), dtype=torch.bfloat16, device="cuda")
    heads = list(range(0, H, max(1, H // args.balance_heads)))[:args.balance_heads]
    rows_t = torch.from_numpy(np.linspace(0, N - 1, args.schedule_rows).astype(np.int64)).cuda()
    exact = {h: exact_attention_rows(Qd[0, h][rows_t].double(), Kd[0, h].double(), Vd[0, h].double()) for h in heads}
    C = torch.empty_like(Cw)
    cnt = torch.empty_like(cnt_w)
    out = []
    for kappa in [float(x) for x in args.kappas.split(",")]:
        lam = kappa * J * Kc / N

        def run():
            C.copy_(Cw)
            cnt.copy_(cnt_w)
            if kappa == 0.0:
                vc.vc_cluster(Vd, Kc, 2, False, C, lab, perm, ws=ws_c)
            else:
                vc.vc_cluster_balanced(Vd, Kc, 2, False, lam, cnt, C, lab, perm, ws=ws_c)
        run()
        times = []
        for _ in range(5):
            C.copy_(Cw)
            cnt.copy_(cnt_w)
            e0 = torch.cuda.Event(enable_timing=True); e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            if kappa == 0.0:
                vc.vc_cluster(Vd, Kc, 2, False, C, lab, perm, ws=ws_c)
            else:
                vc.vc_cluster_balanced(Vd, Kc, 2, False, lam, cnt, C, lab, perm, ws=ws_c)
            e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        sizes = torch.stack([torch.bincount(lab[0, h].long(), minlength=Kc) for h in range(H)]).double()
        ls = torch.gather(lab, 2, perm.long()).view(B, H, N // 128, 128)
        pure = float((ls.amin(-1) == ls.amax(-1)).double().mean())
        vc.vc_cluster_cost(Vd, C, lab, cost, ws=ws_cost)
        vc.vc_quantize(Qd, Kd, Vd, perm, vc.VC_F_KSMOOTH | vc.VC_F_VSMOOTH, q, ws=ws_q)
        vc.vc_attention(q, O, beta=BETA, flags=vc.VC_F_EXPCAST)
        torch.cuda.synchronize()
        num = den = 0.0
        for h in heads:
            diff = O[0, h][rows_t].double() - exact[h]
            num += float((diff * diff).sum())
            den += float((exact[h] * exact[h]).sum())
        row = dict(kappa=kappa, lam=lam, kmeans_ms=round(min(times), 3),
                   size_cv=round(float((sizes.std(1) / sizes.mean(1)).mean()), 4),
                   size_max=int(sizes.max()), empty_clusters=int((sizes == 0).sum()),
                   single_cluster_blocks=round(pure, 4), kmeans_objective=round(float(cost.mean()), 4),
                   rmse=round((num / den) ** 0.5, 6))
        log("[balance] %s" % row)
        out.append(row)
    res = {"workload": "balanced vs plain k-means on the wan2.2-shaped step, B=%d H=%d N=%d d=%d, %d clusters, "
                       "2 warm iterations; error on %d rows x heads %s" % (B, H, N, d, Kc, args.schedule_rows, heads),
           "J_warm": J, "rows": out}
    print(json.dumps(res), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="wan")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=12288,
                    help="attention rows of the oracle sample (about 10 s of CPU work with the k-means and quantiser)")
    ap.add_argument("--attention-only", action="store_true", help="time only vc_attention (profiling aid)")
    ap.add_argument("--attn-mode", default="vc", choices=["vc", "vc_e5m2", "expcast", "exp", "vs_mx4", "vc_mx4"],
                    help="with --attention-only: vc = V-Smooth + ExpCast (the path); vc_e5m2 = the same with "
                         "E5M2 probability bytes; expcast = ExpCast bytes without mean restoration; exp = "
                         "exp-then-cast probabilities without mean restoration (instruction-count comparison of "
                         "the probability stage); vs_mx4 / vc_mx4 = the 4-bit (MXFP4) value residual with V-Smooth "
                         "and exp-then-cast / ExpCast probabilities")
    ap.add_argument("--schedule-rows", type=int, default=64, help="sampled rows of head 0 for the schedule's rMSE")
    ap.add_argument("--error-rows", type=int, default=64,
                    help="rows per head (two heads) for the error columns of the default workload (0: no error columns)")
    ap.add_argument("--refresh", default="fixed", choices=["fixed", "drift", "incremental"],
                    help="schedule workload: fixed clustering steps 0-4, drift-triggered refresh, or a cross-step "
                         "incremental centroid update at every step")
    ap.add_argument("--decay", type=float, default=0.5,
                    help="schedule workload with --refresh incremental: weight of a cluster's past members")
    ap.add_argument("--drift-threshold", type=float, default=0.05,
                    help="relative growth of the k-means objective that triggers a refresh")
    ap.add_argument("--kappas", default="0,0.003,0.01,0.03,0.1",
                    help="balance workload: penalty scales, lambda = kappa * J / (N/K)")
    ap.add_argument("--balance-heads", type=int, default=8, help="balance workload: heads sampled for the error")
    ap.add_argument("--quant-prep", default="none", choices=["none", "rope", "hadamard", "rope_hadamard"],
                    help="preprocessing fused into the quantiser: RoPE on the video grid and/or the Q/K Hadamard "
                         "rotation")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (HBM counter calibration) and exit")
    args = ap.parse_args()
    if args.calibrate_copy:
        import torch
        x = torch.ones(args.calibrate_copy << 20, dtype=torch.uint8, device="cuda")
        y = torch.empty_like(x)
        torch.cuda.synchronize()
        y.copy_(x)
        torch.cuda.synchronize()
        print(json.dumps({"calibration_copy_bytes": x.numel()}), flush=True)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: runs on exactly one GPU; the path shards by (batch, head) with no exchange, "
              "but multi-GPU runs are not part of it (use --gpus 1)", file=sys.stderr)
        sys.exit(2)

    if args.workload == "schedule":
        run_schedule(args)
        return
    if args.workload == "balance":
        run_balance(args)
        return
    if args.workload in ("oracle", "oracle-c0"):
        run_oracle_timing(args)
        return

    import torch
    import bit_attention_video_online_amd as vc

    torch.cuda.set_device(0)
    if args.workload == "wan":
        B, H, N, d, Kc, seed, kind = 1, 40, 70400, 128, 550, 2, "wan"
    elif args.workload.startswith("sweep"):
        import synth
        i = int(args.workload[5:])
        s = synth.SWEEP[i]
        B, H, N, d, seed, kind = s["B"], s["H"], s["N"], s["d"], s["seed"], "sweep"
        Kc = N // 128
    else:
        raise SystemExit("unknown workload %s" % args.workload)
    dev, host = make_inputs(kind, B, H, N, d, seed)
    Qd, Kd, Vd, Vpd = dev["Q"], dev["K"], dev["V"], dev["V_prev"]

    # warm-start state: cold 4-iteration k-means on the previous step's values (untimed)
    Cw = torch.zeros((B, H, Kc, d), dtype=torch.float32, device="cuda")
    lab = torch.empty((B, H, N), dtype=torch.int32, device="cuda")
    perm = torch.empty((B, H, N), dtype=torch.int32, device="cuda")
    ws_c = vc.workspace(vc.vc_cluster_workspace_bytes(B, H, N, d, Kc))
    vc.vc_cluster(Vpd, Kc, 4, True, Cw, lab, perm, ws=ws_c)
    C = torch.empty_like(Cw)
    q = vc.quantize_outputs(B, H, N, d)
    ws_q = vc.workspace(vc.vc_quantize_workspace_bytes(B, H, N, d))
    O = torch.empty((B, H, N, d), dtype=torch.bfloat16, device="cuda")
    flags_q = vc.VC_F_KSMOOTH | vc.VC_F_VSMOOTH
    rope_c = rope_s = None
    if "rope" in args.quant_prep:
        import synth
        grid = synth.WAN_GRID if N == 70400 else None
        rope_c, rope_s = (torch.from_numpy(t).cuda() for t in synth.rope_tables(N, d, grid))
    if "hadamard" in args.quant_prep:
        flags_q |= vc.VC_F_HADAMARD
    torch.cuda.synchronize()

    ev = {k: [] for k in ("cluster", "quantize", "attention")}

    mode = args.attn_mode if args.attention_only else "vc"
    attn_flags = {"vc": vc.VC_F_EXPCAST, "vc_e5m2": vc.VC_F_EXPCAST | vc.VC_F_E5M2, "expcast": vc.VC_F_EXPCAST,
                  "exp": 0, "vs_mx4": vc.VC_F_MXFP4, "vc_mx4": vc.VC_F_EXPCAST | vc.VC_F_MXFP4}[mode]
    attn_beta = BETA_E5M2 if mode == "vc_e5m2" else BETA
    attn_restore = mode in ("vc", "vc_e5m2", "vs_mx4", "vc_mx4")
    if mode in ("vs_mx4", "vc_mx4"):
        flags_q |= vc.VC_F_MXFP4

    def step(record):
        if args.attention_only:
            if record:
                e0 = torch.cuda.Event(enable_timing=True); e1 = torch.cuda.Event(enable_timing=True)
                e0.record()
            vc.vc_attention(q, O, beta=attn_beta, flags=attn_flags, restore_mean=attn_restore)
            if record:
                e1.record(); ev["attention"].append((e0, e1))
            return
        es = [torch.cuda.Event(enable_timing=True) for _ in range(4)] if record else None
        C.copy_(Cw)
        if record: es[0].record()
        vc.vc_cluster(Vd, Kc, 2, False, C, lab, perm, ws=ws_c)
        if record: es[1].record()
        vc.vc_quantize(Qd, Kd, Vd, perm, flags_q, q, ws=ws_q, rope_cos=rope_c, rope_sin=rope_s)
        if record: es[2].record()
        vc.vc_attention(q, O, beta=BETA, flags=vc.VC_F_EXPCAST)
        if record:
            es[3].record()
            ev["cluster"].append((es[0], es[1])); ev["quantize"].append((es[1], es[2])); ev["attention"].append((es[2], es[3]))

    if args.attention_only:
        C.copy_(Cw)
        vc.vc_cluster(Vd, Kc, 2, False, C, lab, perm, ws=ws_c)
        vc.vc_quantize(Qd, Kd, Vd, perm, flags_q, q, ws=ws_q, rope_cos=rope_c, rope_sin=rope_s)
    for i in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    log("[bench] warmup done (%d steps)" % args.warmup)
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps
    avg = {k: (sum(a.elapsed_time(b) for a, b in v) / len(v) if v else None) for k, v in ev.items()}
    log("[bench] timed %d steps: %.3f ms/step; stage ms %s" % (args.steps, ms_step, avg))

    mfma = measure_mfma_peak()
    log("[bench] sustained FP8 matrix-core rate (TFLOP/s): %s" % mfma)

    exactness = None
    if not args.attention_only and args.quant_prep == "none":
        C1 = Cw.clone()
        vc.vc_cluster(Vd, Kc, 1, False, C1, lab, perm, ws=ws_c)  # what the second assignment reads
        exactness = exactness_spans(vc, torch, Kd, Vd, Cw, C1, N, d)
        del C1
        vc.vc_cluster(Vd, Kc, 2, False, C.copy_(Cw), lab, perm, ws=ws_c)  # the step's labels again
        torch.cuda.synchronize()

    errors = gpu_head0 = None
    if not args.attention_only and args.error_rows > 0:
        errors, gpu_head0 = error_columns(args, vc, torch, B, H, N, d, Kc, Qd, Kd, Vd, lab, perm, C, q, O, flags_q)

    flops = 4.0 * B * H * N * N * d
    t_att = avg["attention"] / 1e3
    att_tflops = flops / t_att / 1e12
    value = flops / (ms_step / 1e3) / 1e12
    res = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOPS", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 3), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "fp8_e4m3", "data": "synthetic",
        "config": {"workload": ("wan2.2-shaped VC-Attention step: B=%d H=%d N=%d d=%d, k-means %d clusters x 2 warm "
                                "iterations, block 128, beta=-0.35, V-Smooth + ExpCast-FP8" % (B, H, N, d, Kc)),
                   "global_batch": B, "seq_len": N, "heads": H, "head_dim": d, "clusters": Kc,
                   "parallelism": "single GPU"},
        "stage_ms": {k: (round(v, 3) if v is not None else None) for k, v in avg.items()},
        "attention_tflops": round(att_tflops, 2),
        "quantize_attention_tflops": (round(flops / ((avg["quantize"] + avg["attention"]) / 1e3) / 1e12, 2)
                                      if avg["quantize"] else None),
        "stage_rates": stage_rates(B, H, N, d, Kc, 2, avg),
        "device": device_info(),
        "attention_pct_fp8_peak": round(100.0 * att_tflops / FP8_PEAK_TFLOPS, 2),
        "fp8_mfma_sustained_tflops": mfma,
        "attention_pct_fp8_sustained": round(100.0 * att_tflops / mfma["random_operands"], 2),
        "roofline": {"bound": "mfma", "achieved": round(att_tflops, 2), "peak": FP8_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(att_tflops / FP8_PEAK_TFLOPS, 4), "traffic": profiled_traffic(),
                     "traffic_unit": "GB per launch (rocprofv3 FETCH_SIZE+WRITE_SIZE, copy-calibrated)",
                     "kernel": "attn_fwd<128,ExpCast,restore>", "algorithmic_flops_per_launch": flops},
    }
    if errors is not None:
        res["errors"] = errors
    if exactness is not None:
        res["exactness_spans"] = exactness
    if args.quant_prep != "none":
        res["config"]["workload"] += " (quantiser with %s%s)" % (
            {"rope": "RoPE", "hadamard": "the Q/K Hadamard rotation",
             "rope_hadamard": "RoPE and the Q/K Hadamard rotation"}[args.quant_prep],
            " on the 22x40x80 video grid" if "rope" in args.quant_prep and N == 70400 else "")
    if args.attention_only:
        res["config"]["workload"] += " (attention kernel only%s)" % {
            "vc": "", "vc_e5m2": ", E5M2 ExpCast bytes (beta -0.17)", "expcast": ", ExpCast without mean restoration",
            "exp": ", exp-then-cast probabilities, no mean restoration",
            "vs_mx4": ", 4-bit MXFP4 value residual with V-Smooth, exp-then-cast probabilities",
            "vc_mx4": ", 4-bit MXFP4 value residual with V-Smooth, ExpCast probabilities"}[mode]
        res["roofline"]["kernel"] = {"vc": "attn_fwd<128,ExpCast,restore>", "vc_e5m2": "attn_fwd<128,ExpCast-E5M2,restore>",
                                     "expcast": "attn_fwd<128,ExpCast>", "exp": "attn_fwd<128,exp-then-cast>",
                                     "vs_mx4": "attn_fwd<128,exp-then-cast,restore,MXFP4>",
                                     "vc_mx4": "attn_fwd<128,ExpCast,restore,MXFP4>"}[mode]
    if not args.no_cpu_baseline and not args.attention_only:
        import oracle
        log("[bench] timing the CPU oracle on a bounded sample ...")
        res["cpu_baseline"] = cpu_baseline(host, Kc, args.cpu_rows, oracle.num_threads(), gpu=gpu_head0)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
