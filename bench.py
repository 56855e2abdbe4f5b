#!/usr/bin/env python3
"""Verify-step throughput on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step = one pass of the whole verify path (copy retrieval + probe gate, block-
triangular verify attention, full LM head, rejection sampling) over one batch of
seeded synthetic inputs.  The default workload (the headline line) is shaped like
Llama-3.1-8B (d=4096, 32/8 heads, hd=128, prefix 4096, W=4 candidates x D=20 tokens,
V=128256, bf16).  Inputs are resident in HBM before timing starts.  Each timed step
reads a different one of 32 KV buffers (a Llama-8B has 32 layers) and alternates
between 2 copies of the head, so that no step is served from the 256 MB Infinity
Cache left warm by the last.

Other workloads (--workload): tiny (fp32, V=512), slimspec (the low-rank draft head
r=512 writing q for 7 drafts, the draft tokens drawn from q, then a W=1, D=7 verify
step of those drafts), llama70b
(d=8192, 64/8 heads, prefix 16384, W=8, D=20) and ragged (32 sequences, prefixes
U[512, 8192], randomly ordered pages, W=4, D=8, point-mass drafts).

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



def rho_tps(nu: float, rho_tau: float, kappa: float) -> float:
    """SlimSpec's acceptance-cost model ("SlimSpec: Low-Rank Draft LM-Head ...",
    gist.science, "이론적 프레임워크"): the end-to-end speed-up of a draft head that
    takes nu times the full head's time and keeps rho_tau of the acceptance length,
    when the full head takes kappa times the rest of the drafting pipeline.  Reported
    beside the measured nu; the verify path itself never evaluates it."""
    return rho_tau * (1.0 + kappa) / (1.0 + nu * kappa)

def head_bytes(M, d, V, esz=2):
    """Algorithmic bytes of one full-head launch: W + H (esz bytes each) + fp32 logits."""
    return V * d * esz + M * d * esz + M * V * 4


def attn_bytes(B, M, Hq, Hkv, hd, sum_p, esz=2):
    """Prefix K and V once, Q in and O out, the candidates' own K and V."""
    return (2 * sum_p * Hkv * hd + B * M * Hq * hd * 2 + 2 * B * M * Hkv * hd) * esz


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


def cpu_baseline(case, shape, min_seconds=10.0, accept="longest"):
    """The CPU oracle, as it stands, on full steps of the same inputs, repeated until at
    least `min_seconds` of CPU work have been timed.  With external drafts a step is the
    oracle's low-rank draft head, its draft sampling and its verify step over those
    drafts."""
    import numpy as np
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
    A = case.arrays
    sh = shape
    n = 0
    t0 = time.perf_counter()
    while True:
        if sh.external_drafts:
            z, l, _ = oracle.lm_head_lowrank(oracle.as_f64(A["draft_h"], "bf16"), A["w_down"],
                                             A["w_up"])
            A2 = dict(A)
            A2["q_draft"] = oracle.head_softmax(z, l).astype(np.float32)
            tok, _ = oracle.draft_sample(A2["q_draft"], A["u_draft"][0, 0, :sh.D])
            drafts = (tok.reshape(1, 1, sh.D), np.array([[sh.D]], dtype=np.int32))
            oracle.verify_step(A2, sh, drafts=drafts, accept=accept)
        else:
            oracle.verify_step(A, sh, accept=accept)
        n += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds:
            break
    what = ("low-rank draft head (r=%d), draft sampling + " % sh.rank) if sh.external_drafts else \
        "retrieval, probe, "
    return {"value": n / dt, "unit": "verify steps/s", "cores": int(threads), "kind": "oracle",
            "sample": "%d full %s verify steps (%sattention over %d prefix keys in all, "
                      "%dx%d head over %d rows, sampler) on the same inputs, fp64 "
                      "NumPy/BLAS; %.1f s" % (n, sh.name, what, int(sum(sh.P)), sh.V, sh.d,
                                              sh.B * sh.M, dt),
            "seconds_per_step": dt / n, **host_info()}


def measure_peaks(lib, dev):
    """What this GPU sustains, timed with HIP events on the current stream: a 1 GiB
    read stream (16-byte vector loads, eight in flight per thread; grid-strided over
    1,024, 4,096 and 16,384 workgroups, and one contiguous slice per workgroup over 1, 2,
    4 and 8 workgroups per CU) and back-to-back MFMA 32x32x16 bf16 products on register
    operands (two workgroups of four waves per CU).  Best of five launches each, after
    two warm-ups; the read ceiling is the best pattern."""
    import ctypes as C
    import torch
    stream = C.c_void_p(torch.cuda.current_stream().cuda_stream)
    nbytes = 1 << 30
    buf = torch.ones(nbytes // 4, dtype=torch.int32, device=dev)
    sink = torch.zeros(1024, dtype=torch.int32, device=dev)
    fsink = torch.zeros(4096, dtype=torch.float32, device=dev)
    n_cu = torch.cuda.get_device_properties(dev).multi_processor_count
    n_wg_mfma, iters = 2 * n_cu, 2000

    def best(launch):
        for _ in range(2):
            launch()
        times = []
        for _ in range(5):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            launch()
            e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1) * 1e-3)
        return min(times)

    def rd(n_wg, pattern):
        def go():
            assert lib.vs_measure_read(C.c_void_p(buf.data_ptr()), nbytes,
                                       C.c_void_p(sink.data_ptr()), n_wg, pattern, stream) == 0
        return go

    def mm():
        assert lib.vs_measure_mfma(n_wg_mfma, iters, C.c_void_p(fsink.data_ptr()), stream) == 0

    t_strided = min(best(rd(n, 0)) for n in (1024, 4096, 16384))
    t_slices = min(best(rd(n, 1)) for n in (n_cu, 2 * n_cu, 4 * n_cu, 8 * n_cu))
    t_rd = min(t_strided, t_slices)
    t_mm = best(mm)
    flops = n_wg_mfma * 4 * iters * 8 * 32768.0
    del buf
    return {"read_stream_GBs": nbytes / t_rd / 1e9, "mfma_bf16_TFLOPs": flops / t_mm / 1e12,
            "read_grid_strided_GBs": nbytes / t_strided / 1e9,
            "read_slice_per_workgroup_GBs": nbytes / t_slices / 1e9,
            "how": "1 GiB read once per launch, 16-byte loads, eight in flight per thread, "
                   "grid-strided (1,024 / 4,096 / 16,384 workgroups) or one contiguous slice "
                   "per workgroup (1 / 2 / 4 / 8 per CU), the faster pattern; %d "
                   "workgroups x 4 waves x %d x 8 independent MFMA 32x32x16 bf16; best of 5 "
                   "event-timed launches" % (n_wg_mfma, iters), "cus": n_cu}


def vendor_gemm_reference(api, dev, reps=20):
    """The head's product beside the vendor GEMM on the same shapes: this library's
    bound LM head (bf16 GEMM, fp32 logits, tile statistics and the row normalisers)
    against torch.mm with an fp32 output (bf16 operands; hipBLASLt on ROCm), which
    computes the product alone.  Two weight copies alternate so that the Infinity
    Cache does not serve the weight; mean of `reps` event-timed calls after warm-up."""
    import torch
    out = []
    V = 128256
    for name, M, K in (("slimspec verify head", 7, 4096), ("llama8b", 80, 4096),
                       ("llama70b", 160, 8192), ("ragged", 1024, 4096)):
        g = torch.Generator(device=dev).manual_seed(M)
        h = (torch.randn(M, K, device=dev, generator=g) * 0.05).to(torch.bfloat16)
        Ws = [(torch.randn(V, K, device=dev, generator=g) / K ** 0.5).to(torch.bfloat16)
              for _ in range(2)]
        heads = [api.LmHead(h, w_full=w) for w in Ws]
        Wt = [w.t() for w in Ws]

        def timed(fn):
            for i in range(4):
                fn(i)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for i in range(reps):
                fn(i)
            e1.record()
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) * 1000.0 / reps

        ours = timed(lambda i: heads[i % 2]())
        vendor = timed(lambda i: torch.mm(h, Wt[i % 2], out_dtype=torch.float32))
        flops = 2.0 * M * K * V
        out.append({"shape": name, "M": M, "K": K, "V": V, "ours_us": ours,
                    "vendor_us": vendor, "ours_TFLOPs": flops / ours / 1e6,
                    "vendor_TFLOPs": flops / vendor / 1e6})
        del heads, Ws, Wt
        torch.cuda.empty_cache()
    return {"vendor_gemm_reference": out,
            "how": "ours: vs_lm_head (GEMM + fp32 logits + tile statistics + normalisers); "
                   "vendor: torch.mm(h, W^T, out_dtype=float32), the product only; "
                   "bf16 operands, two weight copies alternating, mean of %d event-timed "
                   "calls" % reps}


def host_info():
    """The host the oracle baseline runs on: CPU model, cores the process may use,
    os.cpu_count() and the BLAS thread count."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = None
    try:
        import threadpoolctl
        info = threadpoolctl.threadpool_info()
        blas = max((i.get("num_threads", 0) for i in info if i.get("user_api") == "blas"),
                   default=None)
    except Exception:
        pass
    return {"cpu_model": model, "affinity_cpus": len(os.sched_getaffinity(0)),
            "os_cpu_count": os.cpu_count(), "blas_threads": blas}


def trace_summary(path):
    """Markdown table of a rocprofv3 kernel trace (run_kernel_trace.csv): calls, mean,
    median, p10, p90, min and max duration per kernel, in microseconds."""
    import csv
    import numpy as np
    durs = {}
    with open(path) as f:
        for row in csv.DictReader(f):
            name = row.get("Kernel_Name") or row.get("KernelName") or row.get("Name")
            t0 = int(row.get("Start_Timestamp") or row.get("BeginNs"))
            t1 = int(row.get("End_Timestamp") or row.get("EndNs"))
            durs.setdefault(name, []).append((t1 - t0) / 1e3)
    lines = ["| kernel | calls | mean | median | p10 | p90 | min | max |",
             "|---|---:|---:|---:|---:|---:|---:|---:|"]
    for name, d in sorted(durs.items(), key=lambda kv: -sum(kv[1])):
        d = np.asarray(d)
        short = name.replace("(anonymous namespace)::", "")
        short = short.split("(")[0] if short.startswith("vs::") or short.startswith("void vs::") else short[:60]
        lines.append("| `%s` | %d | %.2f | %.2f | %.2f | %.2f | %.2f | %.2f |" % (
            short, len(d), d.mean(), np.median(d), np.percentile(d, 10), np.percentile(d, 90),
            d.min(), d.max()))
    return "\n".join(lines)


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


# workload name -> (config index, KV buffers, head copies).  KV buffers and head copies
# are sized so that consecutive steps do not find their inputs in the 256 MB MALL.
WORKLOADS = {
    "llama8b": (2, 32, 2),      # the headline line
    "tiny": (1, 1, 1),
    "slimspec": (3, 32, 2),
    "llama70b": (4, 8, 2),
    "ragged": (5, 2, 2),
}
WORKLOAD_NAMES = {"llama8b": "llama8b_verify_step", "tiny": "tiny_verify_step",
                  "slimspec": "slimspec_draft_head_and_verify_step",
                  "llama70b": "llama70b_verify_step", "ragged": "ragged_batch32_verify_step"}
MFMA_PEAK = {"bf16": 2.5e15, "f32": 157.3e12}   # dense bf16 MFMA; fp32 vector (the f32 head)


def slimspec_drafts(api, sh, case, I, dev):
    """The SlimSpec side of the workload, on the GPU in every step: the low-rank draft
    head, bound so that it writes its probabilities straight into the verify step's q
    input, then the draft tokens drawn from them by inverse CDF straight into the
    step's candidate buffer."""
    import numpy as np
    import torch
    A = case.arrays
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a)).view(torch.bfloat16).to(dev)
    qbuf = torch.empty((sh.M, sh.V), dtype=torch.float32, device=dev)
    head = api.LmHead(bf(A["draft_h"]), w_down=bf(A["w_down"]), w_up=bf(A["w_up"]),
                      write_probs=True, probs=qbuf)
    u = torch.from_numpy(np.ascontiguousarray(A["u_draft"][0, 0, :sh.D])).to(dev)
    tok = torch.empty((1, 1, sh.D), dtype=torch.int32, device=dev)
    dflags = torch.empty(sh.D, dtype=torch.int32, device=dev)
    tok_flat = tok.view(-1)

    def draft():
        head()
        api.draft_sample(qbuf, u, tok_flat, dflags)

    I["q_draft"] = qbuf
    I["cand_tok"] = tok
    I["cand_len"] = torch.full((1, 1), sh.D, dtype=torch.int32, device=dev)
    return draft


def draft_head_tradeoff(api, sh, case, step, dev, K, Wm):
    """nu = low-rank draft head time / full-vocabulary draft head time on the same gamma
    draft states, both measured here, and SlimSpec's rho_TPS for it at the pages'
    rho_tau = 0.99 (r = d/8) over a range of kappa (full head time / rest of the
    drafting pipeline, which has no stand-in here)."""
    import numpy as np
    import torch
    A = case.arrays
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a)).view(torch.bfloat16).to(dev)
    h = bf(A["draft_h"])
    heads = {"full": api.LmHead(h, w_full=step.w_packed, V=sh.V, write_probs=True),
             "lowrank": api.LmHead(h, w_down=bf(A["w_down"]), w_up=bf(A["w_up"]),
                                   write_probs=True)}
    t = {}
    for name, hd in heads.items():
        for _ in range(Wm):
            hd()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(K):
            hd()
        e1.record()
        torch.cuda.synchronize()
        t[name] = e0.elapsed_time(e1) / K * 1e3
    nu = t["lowrank"] / t["full"]
    return {"t_full_head_us": t["full"], "t_lowrank_head_us": t["lowrank"], "nu": nu,
            "rho_tau": 0.99,
            "rho_tps": {str(k): rho_tps(nu, 0.99, k) for k in (0.25, 0.5, 1.0, 2.0)},
            "note": "heads with probabilities on gamma=%d rows, r=%d; the same head weights "
                    "serve as the full draft head" % (sh.gamma, sh.rank)}


def run_labels(args, api, wl, dev):
    """Copy-mode labels over one long context (Zipf ids, 5% of positions in planted
    5..40-token repeats): tokens labelled per second, the oracle timed on the same
    context."""
    import numpy as np
    import torch
    import oracle
    n = args.label_tokens
    ctx, _, _ = wl.make_context(np.random.default_rng(11), np.random.default_rng(12), n, 128256,
                                0.05, (5, 40), 4, 20, 5, False)
    off = np.array([0, n], dtype=np.int32)
    c, o = torch.from_numpy(ctx).to(dev), torch.from_numpy(off).to(dev)
    labels = torch.zeros(n, dtype=torch.uint8, device=dev)
    K, Wm = args.steps, args.warmup
    for _ in range(Wm):
        api.copy_labels(c, o, 5, labels)
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(K):
        api.copy_labels(c, o, 5, labels)
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / K
    alg = 5.0 * n                      # 4 B of token id read + 1 B of label written per position
    rec = {"metric": "copy_labels_tokens_per_s", "value": n / (ms * 1e-3),
           "unit": "tokens/s", "n_gpus": 1, "steps": K, "warmup": Wm, "ms_per_step": ms,
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "int32",
           "data": "synthetic",
           "config": {"workload": "copy_labels_long_context", "tokens": n, "kappa": 5,
                      "context": "Zipf s=1.1 over 128256 ids, 5% planted 5..40-token repeats"},
           "roofline": {"bound": "hbm", "achieved": alg / (ms * 1e-3) / 1e9,
                        "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, "traffic": None,
                        "kernel": "labels_{init,insert,query,mark}_kernel (whole call)",
                        "algorithmic_bytes": alg},
           "labelled_fraction": float(labels.float().mean().item())}
    if not args.no_cpu_baseline:
        t = time.perf_counter()
        oracle.copy_labels(ctx, off, 5)
        dt = time.perf_counter() - t
        rec["cpu_baseline"] = {"value": n / dt, "unit": "tokens/s", "cores": 1,
                               "kind": "oracle", "sample": "the same %d-token context, one "
                               "call, %.1f s" % (n, dt)}
    print(json.dumps(rec), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", choices=list(WORKLOADS), default="llama8b")
    ap.add_argument("--kv-buffers", type=int, default=0, help="0: the workload's default")
    ap.add_argument("--layers", type=int, default=1,
                    help="attention layers per step, in one launch over one shared block "
                         "table (per-layer synthetic q, candidate K/V and pools; the head "
                         "reads the last layer)")
    ap.add_argument("--head-copies", type=int, default=0, help="0: the workload's default")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--accept", choices=["longest", "multi", "greedy"], default="longest",
                    help="longest verified run (default), lossless multi-candidate "
                         "acceptance (over the workload's own drafts: dense q where it has "
                         "one, point masses for copy drafts) or greedy")
    ap.add_argument("--commit", action="store_true",
                    help="after each step, commit the accepted rows to the paged KV cache and "
                         "roll back to the old lengths (times the decode loop's cache update)")
    ap.add_argument("--graph", action="store_true",
                    help="also time the K steps as HIP graph replays (one graph per KV "
                         "buffer / head copy binding, captured after the warmup)")
    ap.add_argument("--labels", action="store_true",
                    help="time the copy-mode label kernel over one long Zipf context instead "
                         "of the verify step")
    ap.add_argument("--label-tokens", type=int, default=1 << 20)
    ap.add_argument("--copy-calib", type=int, default=0,
                    help="only run N plain copies of 1 GiB (counter calibration) and exit")
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip the read-stream and MFMA ceilings measured on this GPU")
    ap.add_argument("--vendor-gemm", action="store_true",
                    help="time the LM head beside the vendor GEMM on the four head shapes")
    ap.add_argument("--trace-summary", metavar="CSV",
                    help="print a markdown summary (mean, median, p10, p90) of a rocprofv3 "
                         "kernel trace and exit (no GPU needed)")
    args = ap.parse_args()

    if args.trace_summary:
        print(trace_summary(args.trace_summary))
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: there is no multi-GPU path "
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

    if args.labels:
        run_labels(args, api, wl, dev)
        return

    if args.vendor_gemm:
        print(json.dumps(vendor_gemm_reference(api, dev)))
        return

    peaks = None if args.no_peaks else measure_peaks(_lib.load(), dev)

    cfg, n_kv, n_head = WORKLOADS[args.workload]
    n_kv = args.kv_buffers or n_kv
    n_head = args.head_copies or n_head
    sh = wl.config(cfg)
    case = wl.make_case(sh, wl.CONFIG_SEED[cfg], "measure")
    I = upload(case)
    B, W, D, M = sh.B, sh.W, sh.D, sh.M
    draft = slimspec_drafts(api, sh, case, I, dev) if sh.external_drafts else None
    kv = None
    if args.commit and not sh.external_drafts:
        # room for a full accepted run per sequence: spare pool pages on a free stack and
        # page-table columns past the longest prefix
        extra_cols = (D + 15) // 16 + 1
        n_spare = B * extra_cols
        n0 = I["k_pool"].shape[0]
        for name in ("k_pool", "v_pool"):
            t = I[name]
            I[name] = torch.cat([t, torch.zeros((n_spare,) + tuple(t.shape[1:]), dtype=t.dtype,
                                                device=dev)])
        I["page_table"] = torch.cat([I["page_table"],
                                     torch.full((B, extra_cols), -1, dtype=torch.int32,
                                                device=dev)], dim=1).contiguous()
        free = torch.zeros(n0 + n_spare, dtype=torch.int32, device=dev)   # room for every page
        free[:n_spare] = torch.arange(n0, n0 + n_spare, dtype=torch.int32, device=dev)
        kv = dict(free=free, n_free=torch.tensor([n_spare], dtype=torch.int32, device=dev),
                  P0=I["prefix_len"].clone(), n_pages=n0 + n_spare)
    if args.accept == "greedy":
        for k in ("q_draft", "u_acc", "u_res"):  # argmax tests: nothing random is read
            I[k] = None
    n_layers = max(1, args.layers)
    g = torch.Generator(device=dev)
    g.manual_seed(1234)
    if n_layers > 1:
        # layer 0 is the seeded case; the other layers are N(0, 1) tensors made on the
        # device; every layer reads its own pools through the one page table.  The KV of
        # a step is then n_layers one-layer caches: two such sets alternate between
        # steps (more for few layers), so the KV read per step is never the last step's
        n_kv = args.kv_buffers or max(2, 32 // n_layers)
        for k in ("q", "k_cand", "v_cand", "k_pool", "v_pool"):
            t = I[k]
            rest = torch.randn((n_layers - 1,) + tuple(t.shape), generator=g, device=dev)
            I[k] = torch.cat([t.unsqueeze(0), rest.to(t.dtype)]).contiguous()
            del rest
    step = api.VerifyStep(I, B=B, W=W, D=D, Hq=sh.Hq, Hkv=sh.Hkv, hd=sh.hd, V=sh.V, tau=sh.tau,
                          temperature=sh.temperature, kappa=sh.kappa,
                          external_drafts=sh.external_drafts, accept=args.accept)
    mdt = I["q"].dtype
    esz = I["q"].element_size()

    # distinct KV buffers (layers) and head copies; buffer 0 / copy 0 are the seeded inputs
    pools = [(I["k_pool"], I["v_pool"])]
    for _ in range(n_kv - 1):
        pools.append((torch.randn(I["k_pool"].shape, generator=g, device=dev).to(mdt),
                      torch.randn(I["v_pool"].shape, generator=g, device=dev).to(mdt)))
    heads = [step.w_packed]           # a bf16 head is prepacked once into MFMA tiles
    for _ in range(n_head - 1):
        w = (torch.randn(I["w_full"].shape, generator=g, device=dev)
             * (1.0 / np.sqrt(sh.d))).to(mdt)
        heads.append(api.pack_weight(w) if mdt == torch.bfloat16 else w)
        del w
    torch.cuda.synchronize()

    def bind(k):
        kp, vp = pools[k % len(pools)]
        step.io.k_pool = kp.data_ptr()
        step.io.v_pool = vp.data_ptr()
        step.io.w_full = heads[k % len(heads)].data_ptr()

    def commit(k):
        kp, vp = pools[k % len(pools)]
        o = step.out
        api.kv_commit(I["k_cand"], I["v_cand"], o["best"], o["n_acc"], kp, vp, I["page_table"],
                      I["prefix_len"], kv["free"], kv["n_free"], W, D)
        api.kv_truncate(kv["P0"], I["page_table"], I["prefix_len"], kv["free"], kv["n_free"],
                        kv["n_pages"])

    def run(k):
        bind(k)
        if draft is not None:
            draft()
        step()
        if kv is not None:
            commit(k)

    K, Wm = args.steps, args.warmup
    for k in range(Wm):
        run(k)
    torch.cuda.synchronize()

    # events on the step's stream (torch's current stream is the one VerifyStep uses)
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)

    # pass 1: the headline, K steps back to back
    torch.cuda.synchronize()
    t0.record()
    for k in range(K):
        run(Wm + k)
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / K

    ms_graph = None
    if args.graph:
        # one graph per binding (KV buffer, head copy), each a whole step as captured
        period = int(np.lcm(len(pools), len(heads)))
        graphs = []
        for k in range(period):
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gr):
                run(k)
            graphs.append(gr)
        for k in range(Wm):
            graphs[k % period].replay()
        torch.cuda.synchronize()
        t0.record()
        for k in range(K):
            graphs[(Wm + k) % period].replay()
        t1.record()
        torch.cuda.synchronize()
        ms_graph = t0.elapsed_time(t1) / K

    # pass 2: the same K steps with stage events (6 per step, made beforehand; one more
    # before the draft head where there is one)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(K)]
    ev_d = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
    ev_ptrs = [step.event_array(e) for e in ev]
    torch.cuda.synchronize()
    t0.record()
    for k in range(K):
        bind(Wm + k)
        step.use_events(ev_ptrs[k])
        if draft is not None:
            ev_d[k].record()
            draft()
        step()
    t1.record()
    torch.cuda.synchronize()
    step.use_events(None)
    ms_staged = t0.elapsed_time(t1) / K
    commit_ms = None
    if kv is not None:
        # pass 3: the cache update alone (commit + rollback) after each step
        tc = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(K)]
        for k in range(K):
            bind(Wm + k)
            step()
            tc[k][0].record()
            commit(Wm + k)
            tc[k][1].record()
        torch.cuda.synchronize()
        commit_ms = float(np.mean([a.elapsed_time(b) for a, b in tc]))

    names = ["retrieval_gate", "attention", "head_gemm", "lse_tests", "sampler"]
    stage_ms = {}
    if draft is not None:
        stage_ms["draft_head_lowrank_and_sampling"] = float(
            np.mean([ev_d[k].elapsed_time(ev[k][0]) for k in range(K)]))
    for i, n in enumerate(names):
        stage_ms[n] = float(np.mean([ev[k][i].elapsed_time(ev[k][i + 1]) for k in range(K)]))

    steps_per_s = 1000.0 / ms
    dt_name = "bf16" if mdt == torch.bfloat16 else "f32"
    # the dominant kernel is the full LM head: HBM- or matrix-bound, whichever takes longer
    MR = B * M                        # head rows over the whole batch
    hb = head_bytes(MR, sh.d, sh.V, esz)
    hf = 2.0 * MR * sh.V * sh.d
    head_s = stage_ms["head_gemm"] * 1e-3
    t_hbm, t_mm = hb / (HBM_PEAK_GBS * 1e9), hf / MFMA_PEAK[dt_name]
    if t_hbm >= t_mm:
        roof = {"bound": "hbm", "achieved": hb / head_s / 1e9, "peak": HBM_PEAK_GBS,
                "unit": "GB/s"}
    else:
        roof = {"bound": "mfma" if dt_name == "bf16" else "alu",
                "achieved": hf / head_s / 1e12, "peak": MFMA_PEAK[dt_name] / 1e12,
                "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    if peaks is not None:
        roof["peak_measured"] = (peaks["read_stream_GBs"] if roof["bound"] == "hbm"
                                 else peaks["mfma_bf16_TFLOPs"] if roof["bound"] == "mfma" else None)
        if roof["peak_measured"]:
            roof["frac_measured"] = roof["achieved"] / roof["peak_measured"]
    roof["traffic"] = traffic_entry() if args.workload == "llama8b" else None
    kname = "vs::head_lds_kernel" if dt_name == "bf16" else "vs::gemm_f32_kernel"
    roof.update({"kernel": kname + " (full LM head GEMM + tile statistics), M=%d" % MR,
                 "algorithmic_bytes": hb, "algorithmic_flops": hf,
                 "t_hbm_us": t_hbm * 1e6, "t_mfma_us": t_mm * 1e6})
    sum_p = int(sum(sh.P))
    ab = attn_bytes(B, M, sh.Hq, sh.Hkv, sh.hd, sum_p, esz) * n_layers
    af = attn_flops(B, W, D, sh.Hq, sh.hd, sum_p) * n_layers
    att_s = stage_ms["attention"] * 1e-3
    out = step.out
    config = {"workload": WORKLOAD_NAMES[args.workload], "B": B, "W": W, "D": D,
              "prefix": sh.P[0] if B == 1 else {"sum": sum_p, "min": min(sh.P),
                                                "max": max(sh.P)},
              "d": sh.d, "Hq": sh.Hq, "Hkv": sh.Hkv, "head_dim": sh.hd, "V": sh.V,
              "kv_buffers": len(pools), "head_copies": len(heads), "layers": n_layers,
              "timing": "hip events on the step stream, no graph; value from a pass "
                        "without stage events, stages from a second pass with them"}
    if args.accept != "longest":
        config["accept"] = args.accept
    if kv is not None:
        config["commit"] = "accepted rows committed to the paged cache, then rolled back"
    if draft is not None:
        config.update({"draft_head": "low-rank r=%d, gamma=%d, probabilities into q"
                                     % (sh.rank, sh.gamma),
                       "drafts": "drawn on the GPU from q by inverse CDF in every step"})
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
        "dtype": dt_name,
        "data": "synthetic",
        "config": config,
        "candidate_tokens_per_s": steps_per_s * B * W * D,
        "stages_us": {k: v * 1e3 for k, v in stage_ms.items()},
        "ms_per_step_with_stage_events": ms_staged,
        "roofline": roof,
        "attention_roofline": {"achieved_GBs": ab / att_s / 1e9,
                               "achieved_TFLOPs": af / att_s / 1e12,
                               "t_hbm_us": ab / HBM_PEAK_GBS / 1e3,
                               "t_mfma_us": af / MFMA_PEAK[dt_name] * 1e6,
                               "frac_of_max_bound": max(ab / (HBM_PEAK_GBS * 1e9),
                                                        af / MFMA_PEAK[dt_name]) / att_s},
        "accepted": [int(x) for x in out["n_acc"].cpu().tolist()][:4],
    }
    if peaks is not None:
        rec["peaks_measured"] = peaks
        ar = rec["attention_roofline"]
        t_hbm_m = ab / (peaks["read_stream_GBs"] * 1e9)
        t_mm_m = af / (peaks["mfma_bf16_TFLOPs"] * 1e12) if dt_name == "bf16" else 0.0
        ar["frac_of_max_measured_bound"] = max(t_hbm_m, t_mm_m) / att_s
    if commit_ms is not None:
        rec["kv_commit_rollback_us"] = commit_ms * 1e3
    if ms_graph is not None:
        rec["ms_per_step_graph_replay"] = ms_graph
    if draft is not None:
        rec["slimspec_tradeoff"] = draft_head_tradeoff(api, sh, case, step, dev, K, Wm)
    if not args.no_cpu_baseline and n_layers == 1:
        # (the oracle's step is one layer: no CPU figure for a layered step)
        rec["cpu_baseline"] = cpu_baseline(case, sh, accept=args.accept)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
