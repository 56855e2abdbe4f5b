#!/usr/bin/env python3
"""Verify-step throughput on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

One step = one pass of the whole verify path (copy retrieval + probe gate, block-
triangular verify attention, full LM head, rejection sampling) over one batch of
seeded synthetic inputs shaped like Llama-3.1-8B (d=4096, 32/8 heads, hd=128,
prefix 4096, W=4 candidates x D=20 tokens, V=128256, bf16).  Inputs are resident
in HBM before timing starts.  Each timed step reads a different one of 32 KV
buffers (a Llama-8B has 32 layers) and alternates between 2 copies of the head,
so that no step is served from the 256 MB Infinity Cache left warm by the last.

Prints ONE JSON line.  Two timed passes of K steps each, both bracketed by
synchronisation and HIP events on the step's stream:
  * pass 1 (the headline value): the steps back to back, no events inside;
  * pass 2 (stage durations and the roofline): the same steps with an event between
    every two stages.  Each event costs the stream a few microseconds of idle time,
    which is why the headline pass carries none; the kernels themselves run the same.
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

METRIC = "verify steps/sec & candidate tokens/sec (Llama-8B shape); % of HBM/MFMA roofline"
HBM_PEAK_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "lm_head_llama8b_traffic.json")
HEAD_SRC = os.path.join(ROOT, "verification_step_amd", "csrc", "head.hip")


def head_bytes(M, d, V):
    """Algorithmic bytes of one full-head launch: W (bf16) + H (bf16) + fp32 logits."""
    return V * d * 2 + M * d * 2 + M * V * 4


def attn_bytes(B, M, Hq, Hkv, hd, sum_p):
    return 2 * sum_p * Hkv * hd * 2 + B * M * Hq * hd * 2 * 2 + 2 * B * M * Hkv * hd * 2


def attn_flops(B, W, D, Hq, hd, sum_p):
    return 4 * Hq * W * D * hd * sum_p + B * 4 * Hq * hd * W * D * (D + 1) // 2


def upload(case):
    import numpy as np
    import torch
    bf = case.shape.dtype == "bf16"
    model = {"probe_h", "q", "k_cand", "v_cand", "k_pool", "v_pool", "w_full"}
    out = {}
    for k, v in case.arrays.items():
        if k in ("w_down", "w_up", "draft_h", "u_draft"):
            continue
        t = torch.from_numpy(np.ascontiguousarray(v))
        if bf and k in model:
            t = t.view(torch.bfloat16)
        out[k] = t.cuda()
    return out


def cpu_baseline(case, shape, min_seconds=10.0):
    """The CPU oracle, as it stands, on full steps of the same inputs, repeated until at
    least `min_seconds` of CPU work have been timed."""
    import oracle
    threads = None
    try:
        import threadpoolctl
        info = threadpoolctl.threadpool_info()
        threads = max((i.get("num_threads", 0) for i in info), default=None)
    except Exception:
        pass
    if not threads:
        threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    n = 0
    t0 = time.perf_counter()
    while True:
        oracle.verify_step(case.arrays, shape)
        n += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds:
            break
    return {"value": n / dt, "unit": "verify steps/s", "cores": int(threads), "kind": "oracle",
            "sample": "%d full Llama-8B-shaped verify steps (retrieval, probe, attention over "
                      "4096 prefix keys, 128256x4096 head, sampler) on the same inputs, fp64 "
                      "NumPy/BLAS; %.1f s" % (n, dt),
            "seconds_per_step": dt / n,
            "host_cpus": len(os.sched_getaffinity(0))}


def traffic_entry():
    """HBM traffic of the head GEMM from committed rocprofv3 counter runs, or None if
    the kernel source changed since they were taken."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    try:
        rec = json.load(open(TRAFFIC_FILE))
        h = hashlib.sha256(open(HEAD_SRC, "rb").read()).hexdigest()
        if rec.get("head_src_sha256") != h:
            return None
        return rec.get("bytes_per_launch")
    except Exception:
        return None


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--kv-buffers", type=int, default=32)
    ap.add_argument("--head-copies", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calib", type=int, default=0,
                    help="only run N plain copies of 1 GiB (counter calibration) and exit")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(the verify step of one batch runs on one MI355X)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from verification_step_amd import _lib, api
    from verification_step_amd import workloads as wl

    _lib.load()       # fail loudly without the HIP library
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)

    if args.copy_calib:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(args.copy_calib):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calib_bytes": 1 << 30, "copies": args.copy_calib}))
        return

    sh = wl.config(2)
    case = wl.make_case(sh, wl.CONFIG_SEED[2], "measure")
    I = upload(case)
    B, W, D, M = sh.B, sh.W, sh.D, sh.M
    step = api.VerifyStep(I, B=B, W=W, D=D, Hq=sh.Hq, Hkv=sh.Hkv, hd=sh.hd, V=sh.V, tau=sh.tau,
                          temperature=sh.temperature, kappa=sh.kappa)

    # distinct KV buffers (layers) and head copies; buffer 0 / copy 0 are the seeded inputs
    g = torch.Generator(device=dev)
    g.manual_seed(1234)
    pools = [(I["k_pool"], I["v_pool"])]
    for _ in range(args.kv_buffers - 1):
        pools.append((torch.randn(I["k_pool"].shape, generator=g, device=dev).to(torch.bfloat16),
                      torch.randn(I["v_pool"].shape, generator=g, device=dev).to(torch.bfloat16)))
    heads = [step.w_packed]           # the head is prepacked once into MFMA tiles
    for _ in range(args.head_copies - 1):
        w = (torch.randn(I["w_full"].shape, generator=g, device=dev)
             * (1.0 / np.sqrt(sh.d))).to(torch.bfloat16)
        heads.append(api.pack_weight(w))
        del w
    torch.cuda.synchronize()

    def bind(k):
        kp, vp = pools[k % len(pools)]
        step.io.k_pool = kp.data_ptr()
        step.io.v_pool = vp.data_ptr()
        step.io.w_full = heads[k % len(heads)].data_ptr()

    K, Wm = args.steps, args.warmup
    for k in range(Wm):
        bind(k)
        step()
    torch.cuda.synchronize()

    # events on the step's stream (torch's current stream is the one VerifyStep uses)
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)

    # pass 1: the headline, K steps back to back
    torch.cuda.synchronize()
    t0.record()
    for k in range(K):
        bind(Wm + k)
        step()
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / K

    # pass 2: the same K steps with stage events (6 per step, made beforehand)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(K)]
    ev_ptrs = [step.event_array(e) for e in ev]
    torch.cuda.synchronize()
    t0.record()
    for k in range(K):
        bind(Wm + k)
        step.use_events(ev_ptrs[k])
        step()
    t1.record()
    torch.cuda.synchronize()
    step.use_events(None)
    ms_staged = t0.elapsed_time(t1) / K

    names = ["retrieval_gate", "attention", "head_gemm", "lse_tests", "sampler"]
    stage_ms = {n: float(np.mean([ev[k][i].elapsed_time(ev[k][i + 1]) for k in range(K)]))
                for i, n in enumerate(names)}

    steps_per_s = 1000.0 / ms
    hb = head_bytes(M, sh.d, sh.V)
    head_s = stage_ms["head_gemm"] * 1e-3
    achieved = hb / head_s / 1e9
    sum_p = int(sum(sh.P))
    ab = attn_bytes(B, M, sh.Hq, sh.Hkv, sh.hd, sum_p)
    af = attn_flops(B, W, D, sh.Hq, sh.hd, sum_p)
    att_s = stage_ms["attention"] * 1e-3
    out = step.out
    rec = {
        "metric": METRIC,
        "value": steps_per_s,
        "unit": "verify steps/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": Wm,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "llama8b_verify_step", "B": B, "W": W, "D": D,
                   "prefix": sh.P[0], "d": sh.d, "Hq": sh.Hq, "Hkv": sh.Hkv, "head_dim": sh.hd,
                   "V": sh.V, "kv_buffers": len(pools), "head_copies": len(heads),
                   "timing": "hip events on the step stream, no graph; value from a pass "
                             "without stage events, stages from a second pass with them"},
        "candidate_tokens_per_s": steps_per_s * B * W * D,
        "stages_us": {k: v * 1e3 for k, v in stage_ms.items()},
        "ms_per_step_with_stage_events": ms_staged,
        "roofline": {"kernel": "vs::head_lds_kernel<5> (full LM head GEMM + tile statistics)",
                     "bound": "hbm",
                     "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic_entry(),
                     "algorithmic_bytes": hb},
        "attention_roofline": {"achieved_GBs": ab / att_s / 1e9,
                               "achieved_TFLOPs": af / att_s / 1e12,
                               "t_hbm_us": ab / HBM_PEAK_GBS / 1e3,
                               "t_mfma_us": af / 2.5e15 * 1e6,
                               "frac_of_max_bound": max(ab / (HBM_PEAK_GBS * 1e9),
                                                        af / 2.5e15) / att_s},
        "accepted": int(out["n_acc"][0].item()),
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(case, sh)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
