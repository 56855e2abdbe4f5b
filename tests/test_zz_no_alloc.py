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


def _pair(api, case, accept="longest", layers=1):
    sh = case.shape
    I = _inputs(case)
    if layers > 1:
        from gpu_util import to_dev
        for k, v in wl.layer_inputs(case, layers, 404).items():
            I[k] = to_dev(v, bf16=sh.dtype == "bf16")
    dense = accept == "multi_dense"
    accept = "multi" if dense else accept
    kw = dict(B=sh.B, W=sh.W, D=sh.D, Hq=sh.Hq, Hkv=sh.Hkv, hd=sh.hd, V=sh.V, tau=sh.tau,
              temperature=sh.temperature, kappa=sh.kappa, accept=accept)
    if accept == "multi" and not dense:
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
    cases = [("bf16 B=3", big, "longest", 1), ("fp32 tiny", small, "longest", 1),
             ("bf16 B=3 multi", big, "multi", 1), ("bf16 B=3 multi, dense drafts", big, "multi_dense", 1),
             ("bf16 B=3, 3 layers", big, "longest", 3), ("fp32 tiny", small, "longest", 1)]
    for name, case, accept, layers in cases:
        say("noalloc vs workspace step:", name, accept, layers)
        ref, na = _pair(api, case, accept, layers)
        r = {k: tensor_np(v).copy() for k, v in ref().items()}
        torch.cuda.synchronize()
        g = na()
        torch.cuda.synchronize()
        _same(r, g)
        # twice in a row on the same scratch
        g = na()
        torch.cuda.synchronize()
        _same(r, g)
