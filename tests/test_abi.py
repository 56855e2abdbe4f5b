"""C-ABI checks that need no GPU: the library loads, exports every entry point
declared in include/vstep.h, and rejects bad arguments on the host before
anything is launched (a failing call enqueues nothing, so these calls never
touch a device)."""
import ctypes as C
import os
import re
import subprocess

import pytest

from verification_step_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "vstep.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(L.LIB_PATH):
        pytest.fail("libvstep.so is not built (run `python -m verification_step_amd.build`)")
    return L.load()


def declared_functions():
    inc = os.path.dirname(HEADER)
    src = "".join(open(os.path.join(inc, f)).read() for f in sorted(os.listdir(inc))
                  if f.endswith(".h"))
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(vs_[a-z_]+)\s*\(", src)))


def test_header_declares_expected_calls():
    names = declared_functions()
    for n in ("vs_copy_match", "vs_probe_gate", "vs_verify_attention", "vs_lm_head",
              "vs_reject_sample", "vs_verify_step"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", L.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\s[TW]\s+(vs_\w+)", out))
    missing = [n for n in declared_functions() if n not in exported]
    assert not missing, missing
    for n in declared_functions():
        assert hasattr(lib, n)


def test_version_and_status_strings(lib):
    assert lib.vs_abi_version() == 5
    assert lib.vs_status_str(0) == b"ok"
    assert b"workspace" in lib.vs_status_str(-3)
    assert lib.vs_status_str(99) == b"unknown status"


def test_struct_layouts_match_header():
    # int32 fields, int64 ctx_total at its natural alignment, int32 accept_mode and
    # n_layers in what was the tail padding
    assert C.sizeof(L.StepDesc) == 88
    assert L.StepDesc.ctx_total.offset == 72
    assert L.StepDesc.accept_mode.offset == 80
    assert L.StepDesc.n_layers.offset == 84
    assert C.sizeof(L.StepIO) == 35 * 8
    assert C.sizeof(L.AttnDesc) == 48
    assert C.sizeof(L.HeadDesc) == 28
    assert C.sizeof(L.SampleDesc) == 24
    assert C.sizeof(L.KvDesc) == 40


def test_struct_layouts_match_the_c_compiler(tmp_path):
    """Every descriptor's size and field offsets as the C compiler lays out the header
    (gcc on this host) equal the binding's ctypes view."""
    import shutil
    import subprocess
    if shutil.which("gcc") is None:
        pytest.skip("no C compiler")
    structs = {"vs_attn_desc": L.AttnDesc, "vs_head_desc": L.HeadDesc,
               "vs_sample_desc": L.SampleDesc, "vs_step_desc": L.StepDesc,
               "vs_step_io": L.StepIO, "vs_kv_desc": L.KvDesc}
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "vstep.h"', 'int main(void){']
    for cname, cls in structs.items():
        lines.append(f'printf("{cname} size %zu\\n", sizeof({cname}));')
        for f in cls._fields_:
            lines.append(f'printf("{cname} {f[0]} %zu\\n", offsetof({cname}, {f[0]}));')
    lines.append("return 0;}")
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines))
    exe = tmp_path / "layout"
    inc = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include")
    subprocess.run(["gcc", "-std=c11", "-I", inc, str(src), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split("\n")
    seen = 0
    for line in out:
        if not line:
            continue
        cname, field, val = line.split()
        cls = structs[cname]
        want = C.sizeof(cls) if field == "size" else getattr(cls, field).offset
        assert int(val) == want, (cname, field)
        seen += 1
    assert seen == sum(len(c._fields_) + 1 for c in structs.values())


def test_copy_match_validation(lib):
    nul = None
    fake = C.c_void_p(16)   # never dereferenced: validation fails first
    # null outputs
    assert lib.vs_copy_match(fake, 10, fake, 1, 5, 2, 2, nul, fake, fake, fake, nul, nul) == -1
    # kappa outside 1..16
    assert lib.vs_copy_match(fake, 10, fake, 1, 17, 2, 2, fake, fake, fake, fake, nul, nul) == -2
    assert lib.vs_copy_match(fake, 10, fake, 1, 0, 2, 2, fake, fake, fake, fake, nul, nul) == -2
    # W*D beyond 1024 rows, B <= 0
    assert lib.vs_copy_match(fake, 10, fake, 1, 5, 64, 17, fake, fake, fake, fake, nul, nul) == -1
    assert lib.vs_copy_match(fake, 10, fake, 0, 5, 2, 2, fake, fake, fake, fake, nul, nul) == -1


def test_probe_validation(lib):
    fake = C.c_void_p(16)
    assert lib.vs_probe_gate(None, 1, fake, 1, 8, 0.4, None, fake, fake, None, None) == -1
    assert lib.vs_probe_gate(fake, 7, fake, 1, 8, 0.4, None, fake, fake, None, None) == -2
    assert lib.vs_probe_gate(fake, 1, fake, 1, 8, float("nan"), None, fake, fake, None, None) == -1


def test_attention_validation(lib):
    fake = C.c_void_p(16)
    ok = dict(B=1, W=4, D=20, Hq=32, Hkv=8, head_dim=128, page_size=16, max_pages=256,
              n_pool_pages=256, dtype=1, scale=0.0)

    def call(**over):
        d = L.AttnDesc(**{**ok, **over})
        return lib.vs_verify_attention(C.byref(d), fake, fake, fake, fake, fake, fake, fake, fake,
                                       None, fake, 0, None)

    assert call(Hq=30) == -1                 # Hq % Hkv != 0
    assert call(head_dim=64) == -2           # bf16 path is head_dim 128
    assert call(dtype=0, head_dim=128) == -2
    assert call(page_size=32) == -2
    assert call(W=0) == -1
    assert call(W=64, D=20) == -1            # more than 1024 rows per sequence
    assert call() == -3                      # workspace too small
    assert call(n_layers=-1) == -1
    assert call(n_layers=1025) == -2         # beyond the layer limit
    assert call(n_layers=32) == -3           # 32 layers: valid, needs its workspace
    d = L.AttnDesc(**ok)
    assert lib.vs_attention_workspace_bytes(C.byref(d)) > 0
    # one layer: n_layers 0 and 1 are the same request
    d1 = L.AttnDesc(**{**ok, "n_layers": 1})
    assert lib.vs_attention_workspace_bytes(C.byref(d1)) == lib.vs_attention_workspace_bytes(C.byref(d))
    assert lib.vs_verify_attention(C.byref(d), None, fake, fake, fake, fake, fake, fake, fake,
                                   None, fake, 1 << 30, None) == -1


def test_head_validation(lib):
    fake = C.c_void_p(16)
    ok = dict(M=80, d=4096, V=128256, rank=0, dtype=1, temperature=1.0, write_probs=0)

    def call(w_full=fake, w_down=None, w_up=None, probs=None, ws=fake, nbytes=1 << 30, **over):
        d = L.HeadDesc(**{**ok, **over})
        return lib.vs_lm_head(C.byref(d), fake, w_full, w_down, w_up, fake, fake, probs, ws,
                              nbytes, None)

    assert call(d=4001) == -2                # bf16 needs d % 32 == 0
    assert call(temperature=0.0) == -1
    assert call(w_full=None) == -1
    assert call(rank=512, w_down=fake, w_up=fake) == -1   # both heads given
    assert call(rank=500, w_full=None, w_down=fake, w_up=fake) == -2
    assert call(write_probs=1) == -1         # probs requested but null
    assert call(nbytes=16) == -3
    d = L.HeadDesc(**ok)
    assert lib.vs_head_workspace_bytes(C.byref(d)) >= 80 * 501 * 8      # (max, sum) per row and 256-row tile


def test_sample_validation(lib):
    fake = C.c_void_p(16)
    d = L.SampleDesc(1, 4, 20, 128256, 1.0)
    args = [fake] * 15
    assert lib.vs_reject_sample(C.byref(L.SampleDesc(1, 4, 20, 128256, -1.0)), *args, None, 0,
                                None) == -1
    assert lib.vs_reject_sample(C.byref(L.SampleDesc(1, 4, 20, 1 << 20, 1.0)), *args, None, 0,
                                None) == -2
    bad = list(args)
    bad[0] = None
    assert lib.vs_reject_sample(C.byref(d), *bad, None, 0, None) == -1
    # accept modes: unknown (3) -> invalid; multi with more than 64 candidates, or copy
    # drafts (q NULL) with too many p values for LDS -> unsupported; multi with dense
    # drafts (any W) gets as far as the workspace check, whose size holds two fp64
    # residual rows per sequence
    def samp(W, D, mode, q=fake):
        a = list(args)
        a[3] = q
        return lib.vs_reject_sample(C.byref(L.SampleDesc(2, W, D, 1000, 1.0, mode)), *a, None,
                                    0, None)
    assert samp(4, 20, 3) == -1
    assert samp(4, 20, L.VS_ACCEPT_MULTI) == -3
    assert samp(65, 1, L.VS_ACCEPT_MULTI) == -2
    assert samp(16, 40, L.VS_ACCEPT_MULTI) == -3             # dense: no LDS bound on W*D
    assert samp(4, 20, L.VS_ACCEPT_MULTI, q=None) == -3
    assert (lib.vs_sample_workspace_bytes(C.byref(L.SampleDesc(2, 4, 20, 1000, 1.0, 1)))
            >= 2 * 2 * 1000 * 8)
    assert samp(65, 1, L.VS_ACCEPT_MULTI, q=None) == -2
    assert samp(16, 40, L.VS_ACCEPT_MULTI, q=None) == -2     # (640+1)*16 + 640 > 4096
    assert samp(8, 20, L.VS_ACCEPT_MULTI, q=None) == -3      # (160+1)*8 + 160 fits
    assert samp(1, 20, L.VS_ACCEPT_MULTI) == -3
    assert lib.vs_sample_workspace_bytes(C.byref(L.SampleDesc(2, 4, 20, 1000, 1.0, 3))) == 0
    # greedy: the uniforms and q are not read (NULL passes validation); its workspace
    # also holds the tile statistics of the given logits
    g = list(args)
    g[3] = g[6] = g[7] = None
    gd = L.SampleDesc(2, 4, 20, 1000, 1.0, L.VS_ACCEPT_GREEDY)
    assert lib.vs_reject_sample(C.byref(gd), *g, None, 0, None) == -3
    g[6] = None
    assert lib.vs_reject_sample(C.byref(L.SampleDesc(2, 4, 20, 1000, 1.0, 0)), *g, None, 0,
                                None) == -1
    assert (lib.vs_sample_workspace_bytes(C.byref(gd))
            >= lib.vs_sample_workspace_bytes(C.byref(L.SampleDesc(2, 4, 20, 1000, 1.0, 0)))
            + 2 * 80 * 4 * 8)


def test_pack_validation(lib):
    fake = C.c_void_p(16)
    assert lib.vs_packed_weight_bytes(1000, 96) == 1008 * 96 * 2      # rows padded to 16
    assert lib.vs_packed_weight_bytes(1000, 100) == 0
    assert lib.vs_pack_weight(fake, fake, 1000, 100, None) == -2      # K % 32 != 0
    assert lib.vs_pack_weight(None, fake, 1000, 96, None) == -1
    assert lib.vs_pack_weight(fake, fake, 0, 96, None) == -1


def test_step_validation(lib):
    fake = C.c_void_p(16)
    base = dict(B=1, W=4, D=20, kappa=5, Hq=32, Hkv=8, head_dim=128, page_size=16, max_pages=256,
                n_pool_pages=256, d=4096, V=128256, dtype=1, scale=0.0, tau=0.4, temperature=1.0,
                external_drafts=0, ctx_total=4096)
    d = L.StepDesc(**base)
    assert lib.vs_step_workspace_bytes(C.byref(d)) > 0
    io = L.StepIO()
    assert lib.vs_verify_step(C.byref(d), C.byref(io), fake, 1 << 40, None) == -1
    for f in io._fields_:
        if f[0] != "stage_events":
            setattr(io, f[0], 16)
    assert lib.vs_verify_step(C.byref(d), C.byref(io), fake, 16, None) == -3
    d2 = L.StepDesc(**{**base, "d": 4000})
    assert lib.vs_verify_step(C.byref(d2), C.byref(io), fake, 1 << 40, None) == -1
    d3 = L.StepDesc(**{**base, "kappa": 20})
    assert lib.vs_verify_step(C.byref(d3), C.byref(io), fake, 1 << 40, None) == -2
    # multi-candidate acceptance takes dense drafts (q_draft given) and copy drafts alike;
    # both get as far as the workspace check
    d4 = L.StepDesc(**{**base, "accept_mode": L.VS_ACCEPT_MULTI})
    assert lib.vs_step_workspace_bytes(C.byref(d4)) > 0
    assert lib.vs_verify_step(C.byref(d4), C.byref(io), fake, 16, None) == -3
    io.q_draft = None
    assert lib.vs_verify_step(C.byref(d4), C.byref(io), fake, 16, None) == -3
    d5 = L.StepDesc(**{**base, "accept_mode": 7})
    assert lib.vs_step_workspace_bytes(C.byref(d5)) == 0
    # layers: negative is invalid, beyond 1,024 unsupported; 0 and 1 are one layer
    assert lib.vs_step_workspace_bytes(C.byref(L.StepDesc(**{**base, "n_layers": -2}))) == 0
    assert lib.vs_verify_step(C.byref(L.StepDesc(**{**base, "n_layers": -2})), C.byref(io), fake,
                              1 << 40, None) == -1
    assert lib.vs_verify_step(C.byref(L.StepDesc(**{**base, "n_layers": 2000})), C.byref(io), fake,
                              1 << 40, None) == -2
    one = lib.vs_step_workspace_bytes(C.byref(L.StepDesc(**{**base, "n_layers": 1})))
    assert one == lib.vs_step_workspace_bytes(C.byref(d))
    assert lib.vs_step_workspace_bytes(C.byref(L.StepDesc(**{**base, "n_layers": 32}))) > 0


def test_step_noalloc_validation(lib):
    """The no-allocation step validates like the workspace step and refuses, before any
    device call, a request whose workspace would exceed the fixed scratch area."""
    base = dict(B=1, W=4, D=20, kappa=5, Hq=32, Hkv=8, head_dim=128, page_size=16, max_pages=256,
                n_pool_pages=256, d=4096, V=128256, dtype=1, scale=0.0, tau=0.4, temperature=1.0,
                external_drafts=0, ctx_total=4096)
    d = L.StepDesc(**base)
    assert 0 < lib.vs_step_workspace_bytes(C.byref(d)) <= L.VS_NOALLOC_SCRATCH_BYTES
    assert lib.vs_verify_step_noalloc(C.byref(d), None, None) == -1
    io = L.StepIO()
    for f in io._fields_:
        if f[0] != "stage_events":
            setattr(io, f[0], 16)
    d2 = L.StepDesc(**{**base, "d": 4000})
    assert lib.vs_verify_step_noalloc(C.byref(d2), C.byref(io), None) == -1
    # 32 sequences of up to 32768 prefix tokens: far beyond the scratch area
    big = L.StepDesc(**{**base, "B": 32, "max_pages": 2048, "n_pool_pages": 65536})
    assert lib.vs_step_workspace_bytes(C.byref(big)) > L.VS_NOALLOC_SCRATCH_BYTES
    assert lib.vs_verify_step_noalloc(C.byref(big), C.byref(io), None) == -2


def test_kv_validation(lib):
    fake = C.c_void_p(16)
    ok = dict(B=4, W=4, D=20, Hkv=8, head_dim=128, page_size=16, max_pages=64, n_pool_pages=300,
              dtype=1)
    d = L.KvDesc(**ok)
    assert lib.vs_kv_workspace_bytes(C.byref(d)) >= 4 * 3 * 4
    args = [fake] * 11

    def commit(desc, a=args, nbytes=1 << 20):
        return lib.vs_kv_commit(C.byref(desc), *a, fake, nbytes, None)

    assert commit(L.KvDesc(**{**ok, "n_layers": -1})) == -1
    assert commit(L.KvDesc(**{**ok, "n_layers": 70000})) == -2

    assert commit(L.KvDesc(**{**ok, "page_size": 8})) == -2
    assert commit(L.KvDesc(**{**ok, "B": 0})) == -1
    assert commit(L.KvDesc(**{**ok, "B": 2049})) == -2
    assert commit(L.KvDesc(**{**ok, "dtype": 5})) == -2
    assert commit(L.KvDesc(**{**ok, "W": 0})) == -1
    assert commit(d, nbytes=8) == -3
    bad = list(args)
    bad[9] = None                               # n_free
    assert commit(d, bad) == -1
    assert lib.vs_kv_workspace_bytes(C.byref(L.KvDesc(**{**ok, "max_pages": 0}))) == 0
    # truncate reads only B, page_size, max_pages, n_pool_pages
    tr = L.KvDesc(**{**ok, "W": 0, "D": 0, "Hkv": 0, "head_dim": 0, "dtype": 9})
    assert lib.vs_kv_truncate(C.byref(tr), fake, fake, fake, fake, None, None, None) == -1
    assert lib.vs_kv_truncate(C.byref(L.KvDesc(**{**ok, "page_size": 32})), *([fake] * 6),
                              None) == -2


def test_copy_labels_validation(lib):
    fake = C.c_void_p(16)
    nb = lib.vs_copy_labels_workspace_bytes(1000)
    assert nb >= 2048 * 12 + 1000
    assert lib.vs_copy_labels_workspace_bytes(-1) == 0
    assert lib.vs_copy_labels(fake, 1000, None, 2, 5, fake, None, fake, nb, None) == -1
    assert lib.vs_copy_labels(fake, 1000, fake, 2, 0, fake, None, fake, nb, None) == -2
    assert lib.vs_copy_labels(fake, 1000, fake, 2, 17, fake, None, fake, nb, None) == -2
    assert lib.vs_copy_labels(fake, 1000, fake, 2, 5, fake, None, fake, nb - 1, None) == -3
    assert lib.vs_copy_labels(fake, 1 << 31, fake, 2, 5, fake, None, fake, 1 << 40, None) == -2


def test_draft_sample_validation(lib):
    fake = C.c_void_p(16)
    nb = lib.vs_draft_sample_workspace_bytes(7, 128256)
    assert nb >= 7 * 63 * 8                 # one fp64 sum per 2048-id chunk and row
    assert lib.vs_draft_sample_workspace_bytes(7, 1 << 20) == 0
    assert lib.vs_draft_sample(None, 7, 1000, fake, fake, None, fake, nb, None) == -1
    assert lib.vs_draft_sample(fake, 7, 1 << 20, fake, fake, None, fake, 1 << 40, None) == -2
    assert lib.vs_draft_sample(fake, 7, 128256, fake, fake, None, fake, nb - 1, None) == -3


def test_bench_rho_tps_matches_the_oracle():
    import bench
    import oracle
    for nu in (0.05, 0.19, 0.5, 1.0):
        for k in (0.25, 1.0, 4.0):
            assert bench.rho_tps(nu, 0.99, k) == oracle.rho_tps(nu, 0.99, k)


def test_binding_computes_nothing():
    """The binding only marshals: no arithmetic helper of the method lives in it."""
    from verification_step_amd import api
    assert not hasattr(api, "rho_tps")


def test_kv_pack_validation(lib):
    fake = C.c_void_p(16)
    assert lib.vs_kv_pack_pages(None, fake, 100, 8, 128, 1, fake, fake, None) == -1
    assert lib.vs_kv_pack_pages(fake, fake, 0, 8, 128, 1, fake, fake, None) == -1
    assert lib.vs_kv_pack_pages(fake, fake, 100, 8, 128, 7, fake, fake, None) == -2
    assert lib.vs_kv_pack_pages(fake, fake, 100, 8, 512, 1, fake, fake, None) == -2


def test_binding_rejects_inconsistent_shapes(lib):
    """The binding stops tensors whose sizes disagree with the launch sizes on the host
    (meta tensors: no device needed)."""
    import torch
    from verification_step_amd import api
    m = lambda *s: torch.empty(*s, device="meta", dtype=torch.bfloat16)
    packed = torch.empty(lib.vs_packed_weight_bytes(1000, 64) // 2, device="meta",
                         dtype=torch.bfloat16)
    api.head_weight_sizes(lib, True, 64, 1000, 0, packed, None, None)
    api.head_weight_sizes(lib, True, 64, 1000, 0, m(1000, 64), None, None)
    for bad in (torch.empty(packed.numel() - 8, device="meta", dtype=torch.bfloat16),
                m(1000, 32)):
        with pytest.raises(ValueError):
            api.head_weight_sizes(lib, True, 64, 1000, 0, bad, None, None)
    # the flat packed full weight of a Llama-8B head is not a [V, d] tensor for V=7
    with pytest.raises(ValueError):
        api.head_weight_sizes(lib, True, 4096, 7, 0, packed, None, None)
    with pytest.raises(ValueError):
        api._expect(m(3, 4), (3, 5), "x")


def test_measure_validation(lib):
    fake = C.c_void_p(16)
    assert lib.vs_measure_read(None, 1 << 20, fake, 64, 0, None) == -1
    assert lib.vs_measure_read(fake, 8, fake, 64, 0, None) == -1          # under 16 bytes
    assert lib.vs_measure_read(fake, 1 << 20, fake, 0, 0, None) == -1     # no workgroups
    assert lib.vs_measure_read(fake, 1 << 20, fake, 64, 2, None) == -1    # no such pattern
    assert lib.vs_measure_read(fake, 64, fake, 64, 1, None) == -1         # slices under 16 B
    assert lib.vs_measure_mfma(0, 10, fake, None) == -1
    assert lib.vs_measure_mfma(4, 0, fake, None) == -1
