"""ctypes view of libvstep.so (the C ABI declared in include/vstep.h).

Loading fails loudly when the library has not been built: there is no other
implementation of these calls in this package.
"""
from __future__ import annotations

import ctypes as C
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libvstep.so")

VS_OK, VS_ERR_INVALID_ARG, VS_ERR_UNSUPPORTED, VS_ERR_WORKSPACE, VS_ERR_HIP = 0, -1, -2, -3, -4
VS_F32, VS_BF16 = 0, 1
VS_ACCEPT_LONGEST, VS_ACCEPT_MULTI, VS_ACCEPT_GREEDY = 0, 1, 2
VS_NOALLOC_SCRATCH_BYTES = 64 << 20

FLAG_PROBE_TIE = 1
FLAG_ACCEPT_TIE = 2
FLAG_CDF_TIE = 4
FLAG_DEGENERATE_RESIDUAL = 8
FLAG_NO_CANDIDATE = 16
FLAG_BAD_PAGE = 32
FLAG_BAD_CTX = 64
FLAG_BAD_TOKEN = 128
FLAG_POOL_EMPTY = 256

EXPORTED = [
    "vs_abi_version", "vs_status_str", "vs_copy_match", "vs_probe_gate",
    "vs_attention_workspace_bytes", "vs_verify_attention", "vs_head_workspace_bytes",
    "vs_lm_head", "vs_sample_workspace_bytes", "vs_reject_sample",
    "vs_step_workspace_bytes", "vs_verify_step", "vs_verify_step_noalloc",
    "vs_packed_weight_bytes", "vs_pack_weight",
    "vs_kv_workspace_bytes", "vs_kv_commit", "vs_kv_truncate", "vs_kv_pack_pages",
    "vs_copy_labels_workspace_bytes", "vs_copy_labels",
    "vs_draft_sample_workspace_bytes", "vs_draft_sample",
    "vs_measure_read", "vs_measure_mfma",
]

P = C.c_void_p
I32 = C.c_int32
ABI_VERSION = 5      # VS_ABI_VERSION of the descriptor layouts below


class AttnDesc(C.Structure):
    _fields_ = [("B", I32), ("W", I32), ("D", I32), ("Hq", I32), ("Hkv", I32),
                ("head_dim", I32), ("page_size", I32), ("max_pages", I32),
                ("n_pool_pages", I32), ("dtype", I32), ("scale", C.c_float),
                ("n_layers", I32)]


class HeadDesc(C.Structure):
    _fields_ = [("M", I32), ("d", I32), ("V", I32), ("rank", I32), ("dtype", I32),
                ("temperature", C.c_float), ("write_probs", I32)]


class SampleDesc(C.Structure):
    _fields_ = [("B", I32), ("W", I32), ("D", I32), ("V", I32), ("temperature", C.c_float),
                ("accept_mode", I32)]


class StepDesc(C.Structure):
    _fields_ = [("B", I32), ("W", I32), ("D", I32), ("kappa", I32), ("Hq", I32), ("Hkv", I32),
                ("head_dim", I32), ("page_size", I32), ("max_pages", I32),
                ("n_pool_pages", I32), ("d", I32), ("V", I32), ("dtype", I32),
                ("scale", C.c_float), ("tau", C.c_float), ("temperature", C.c_float),
                ("external_drafts", I32), ("ctx_total", C.c_int64), ("accept_mode", I32),
                ("n_layers", I32)]


class KvDesc(C.Structure):
    _fields_ = [("B", I32), ("W", I32), ("D", I32), ("Hkv", I32), ("head_dim", I32),
                ("page_size", I32), ("max_pages", I32), ("n_pool_pages", I32), ("dtype", I32),
                ("n_layers", I32)]


class StepIO(C.Structure):
    _fields_ = [(n, P) for n in (
        "ctx", "ctx_off", "probe_h", "probe_w",
        "q", "k_cand", "v_cand", "k_pool", "v_pool", "page_table", "prefix_len",
        "w_full", "root_logits", "q_draft", "u_acc", "u_res",
        "cand_tok", "cand_len", "cand_pos", "n_found", "score", "gate",
        "attn_out", "logits", "row_lse",
        "n_acc", "best", "out_tok", "n_out", "acc_per_cand", "flags", "stage_events",
        "aux_stream", "fork_event", "join_event")]


_lib = None


def load(path: str = LIB_PATH):
    """Load libvstep.so once; raise if it is missing (build it first)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"libvstep.so not found at {path}: build it with "
            "`python -m verification_step_amd.build` (hipcc, gfx950)")
    lib = C.CDLL(path)
    lib.vs_abi_version.restype = C.c_int
    if lib.vs_abi_version() != ABI_VERSION:
        raise RuntimeError(f"{path} has ABI version {lib.vs_abi_version()}, this binding "
                           f"expects {ABI_VERSION}: rebuild it")
    lib.vs_status_str.restype = C.c_char_p
    lib.vs_status_str.argtypes = [C.c_int]
    lib.vs_copy_match.argtypes = [P, C.c_int64, P, C.c_int, C.c_int, C.c_int, C.c_int, P, P, P,
                                  P, P, P]
    lib.vs_probe_gate.argtypes = [P, C.c_int, P, C.c_int, C.c_int, C.c_float, P, P, P, P, P]
    lib.vs_attention_workspace_bytes.restype = C.c_size_t
    lib.vs_attention_workspace_bytes.argtypes = [C.POINTER(AttnDesc)]
    lib.vs_verify_attention.argtypes = [C.POINTER(AttnDesc), P, P, P, P, P, P, P, P, P, P,
                                        C.c_size_t, P]
    lib.vs_head_workspace_bytes.restype = C.c_size_t
    lib.vs_head_workspace_bytes.argtypes = [C.POINTER(HeadDesc)]
    lib.vs_lm_head.argtypes = [C.POINTER(HeadDesc), P, P, P, P, P, P, P, P, C.c_size_t, P]
    lib.vs_sample_workspace_bytes.restype = C.c_size_t
    lib.vs_sample_workspace_bytes.argtypes = [C.POINTER(SampleDesc)]
    lib.vs_reject_sample.argtypes = [C.POINTER(SampleDesc)] + [P] * 16 + [C.c_size_t, P]
    lib.vs_step_workspace_bytes.restype = C.c_size_t
    lib.vs_step_workspace_bytes.argtypes = [C.POINTER(StepDesc)]
    lib.vs_verify_step.argtypes = [C.POINTER(StepDesc), C.POINTER(StepIO), P, C.c_size_t, P]
    lib.vs_verify_step_noalloc.argtypes = [C.POINTER(StepDesc), C.POINTER(StepIO), P]
    lib.vs_packed_weight_bytes.restype = C.c_size_t
    lib.vs_packed_weight_bytes.argtypes = [C.c_int, C.c_int]
    lib.vs_pack_weight.argtypes = [P, P, C.c_int, C.c_int, P]
    lib.vs_kv_workspace_bytes.restype = C.c_size_t
    lib.vs_kv_workspace_bytes.argtypes = [C.POINTER(KvDesc)]
    lib.vs_kv_commit.argtypes = [C.POINTER(KvDesc)] + [P] * 12 + [C.c_size_t, P]
    lib.vs_kv_truncate.argtypes = [C.POINTER(KvDesc)] + [P] * 7
    lib.vs_kv_pack_pages.argtypes = [P, P, C.c_int64, C.c_int, C.c_int, C.c_int, P, P, P]
    lib.vs_copy_labels_workspace_bytes.restype = C.c_size_t
    lib.vs_copy_labels_workspace_bytes.argtypes = [C.c_int64]
    lib.vs_copy_labels.argtypes = [P, C.c_int64, P, C.c_int, C.c_int, P, P, P, C.c_size_t, P]
    lib.vs_draft_sample_workspace_bytes.restype = C.c_size_t
    lib.vs_draft_sample_workspace_bytes.argtypes = [C.c_int, C.c_int]
    lib.vs_draft_sample.argtypes = [P, C.c_int, C.c_int, P, P, P, P, C.c_size_t, P]
    lib.vs_measure_read.argtypes = [P, C.c_size_t, P, C.c_int, C.c_int, P]
    lib.vs_measure_mfma.argtypes = [C.c_int, C.c_int, P, P]
    for fn in EXPORTED:
        if fn not in ("vs_abi_version", "vs_status_str") and not fn.endswith("_bytes"):
            getattr(lib, fn).restype = C.c_int
    _lib = lib
    return lib
