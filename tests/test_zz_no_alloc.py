"""The verify step's no-allocation entry point (vs_verify_step_noalloc, the library's
fixed per-GPU scratch area instead of a workspace) against vs_verify_step on the same
inputs: every output bit-identical, over consecutive calls of different sizes (each
call finds what the previous one left in the scratch)."""
import numpy as np
import pytest

from gpu_util import case_to_dev, require_gpu, say, tensor_np
from verification_step_amd import workloads as wl

pytestmark = pytest.mark.gpu


def _inputs(case):
    keys = {"ctx", "ctx_off", "probe_h", "probe_w", "q", "k_cand", "v_cand", "k_pool", "v_pool",
            "page_table", "prefix_len", "w_full", "root_logits", "q_draft", "u_acc", "u_res"}
    return case_to_dev(case, keys)


def _pair(api, case, accept="longest"):
    sh = case.shape
    I = _inputs(case)
    kw = dict(B=sh.B, W=sh.W, D=sh.D, Hq=sh.Hq, Hkv=sh.Hkv, hd=sh.hd, V=sh.V, tau=sh.tau,
              temperature=sh.temperature, kappa=sh.kappa, accept=accept)
    if accept == "multi":
        I["q_draft"] = None
    ref = api.VerifyStep(I, **kw)
    na = api.VerifyStep(I, noalloc=True, **kw)
    assert na.ws is None
    return ref, na


def _same(ref_np, na_out):
    """ref_np: host copies of the workspace step's outputs; na_out: device outputs."""
    for k, a in ref_np.items():
        b = tensor_np(na_out[k])
        assert np.array_equal(a, b), k


def test_noalloc_matches_workspace_entry_point():
    require_gpu()
    import torch
    from verification_step_amd import api
    big = wl.make_case(wl.Shape(name="small", dtype="bf16", B=3, W=3, D=7, Hq=8, Hkv=2, hd=128,
                                d=1024, V=1000, P=(300, 777, 64), paged_random=True), 11)
    small = wl.make_case(wl.config(1), 1000)          # fp32, one sequence
    cases = [("bf16 B=3", big, "longest"), ("fp32 tiny", small, "longest"),
             ("bf16 B=3 multi", big, "multi"), ("fp32 tiny", small, "longest")]
    for name, case, accept in cases:
        say("noalloc vs workspace step:", name, accept)
        ref, na = _pair(api, case, accept)
        r = {k: tensor_np(v).copy() for k, v in ref().items()}
        torch.cuda.synchronize()
        g = na()
        torch.cuda.synchronize()
        _same(r, g)
        # twice in a row on the same scratch
        g = na()
        torch.cuda.synchronize()
        _same(r, g)
