"""Helpers for the GPU parity tests (not collected by pytest)."""
from __future__ import annotations

import sys

import numpy as np
import pytest

import oracle


def require_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    from verification_step_amd import _lib
    _lib.load()          # raises if the HIP library is missing: no silent fallback


def say(*a):
    """Name the case before each GPU step (flushed), so a failing run is attributable."""
    print("[gpu-case]", *a, flush=True)
    sys.stdout.flush()


def to_dev(arr: np.ndarray, bf16: bool = False):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(arr))
    if bf16:
        t = t.view(torch.bfloat16)
    return t.cuda()


def case_to_dev(case, keys=None):
    """Upload a workloads.Case: model tensors as bf16 (bit views) or fp32."""
    sh = case.shape
    bf = sh.dtype == "bf16"
    model = {"probe_h", "q", "k_cand", "v_cand", "k_pool", "v_pool", "w_full", "w_down", "w_up",
             "draft_h"}
    out = {}
    for k, v in case.arrays.items():
        if keys is not None and k not in keys:
            continue
        out[k] = to_dev(v, bf16=(bf and k in model))
    return out


def rel_err(x, y) -> float:
    """max_i |x_i - y_i| / max(|y_i|, rms(y)): elementwise relative error with an RMS floor."""
    x = np.asarray(x, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    rms = np.sqrt(np.mean(y * y)) if y.size else 0.0
    den = np.maximum(np.abs(y), rms)
    den = np.where(den == 0, 1.0, den)
    return float(np.max(np.abs(x - y) / den)) if y.size else 0.0


def bf16_tensor_to_f64(t) -> np.ndarray:
    import torch
    return t.view(torch.int16).cpu().numpy().view(np.uint16).astype(np.uint32).__lshift__(16) \
        .view(np.float32).astype(np.float64)


def tensor_np(t):
    import torch
    if t.dtype == torch.bfloat16:
        return bf16_tensor_to_f64(t)
    return t.cpu().numpy()


# sampler comparison: decisions bit-exact unless a near tie is flagged on either side
DECISIVE_FLAGS = oracle.FLAG_ACCEPT_TIE | oracle.FLAG_CDF_TIE | oracle.FLAG_PROBE_TIE


def compare_sampler(gpu: dict, orc: dict, B: int):
    """Returns (n_compared, n_excluded); asserts equality on compared sequences."""
    n_cmp = n_exc = 0
    g = {k: tensor_np(v) for k, v in gpu.items()}
    for b in range(B):
        if (int(orc["flags"][b]) | int(g["flags"][b])) & DECISIVE_FLAGS:
            n_exc += 1
            continue
        n_cmp += 1
        assert g["n_acc"][b] == orc["n_acc"][b], (b, g["n_acc"][b], orc["n_acc"][b])
        assert g["best"][b] == orc["best"][b], b
        assert g["n_out"][b] == orc["n_out"][b], b
        assert (g["out_tok"][b] == orc["out_tok"][b]).all(), (b, g["out_tok"][b], orc["out_tok"][b])
        assert (g["acc_per_cand"][b] == orc["acc_per_cand"][b]).all(), b
        other = 0xFF & ~DECISIVE_FLAGS
        assert (int(g["flags"][b]) & other) == (int(orc["flags"][b]) & other), b
    return n_cmp, n_exc
