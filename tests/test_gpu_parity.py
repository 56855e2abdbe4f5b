"""GPU parity: every C-ABI call against the CPU oracle on the same seeded inputs.

Matching rules: integer outputs (retrieval, gate, accepted lengths, chosen
candidate, emitted tokens) bit-exact except sequences where either side flags a
near tie; attention outputs and logits within 1e-2 of the oracle in the
elementwise relative error with an RMS floor (max |x-y| / max(|y|, rms(y))).
Shapes span several tiles with ragged tails; the full-size workloads run in the
configuration the bench times.
"""
import numpy as np
import pytest
import scipy.special

import oracle
from gpu_util import (case_to_dev, compare_sampler, rel_err, require_gpu, say, tensor_np,
                      to_dev)
from verification_step_amd import workloads as wl

pytestmark = pytest.mark.gpu

TOL = 1e-2


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _api():
    from verification_step_amd import api
    return api


_cache = {}


def get_case(key, maker):
    if key not in _cache:
        _cache[key] = maker()
    return _cache[key]


def small_shape(**kw):
    base = dict(name="small", dtype="bf16", B=2, W=3, D=7, Hq=8, Hkv=2, hd=128, d=1024, V=1000,
                P=(300, 777), paged_random=True)
    base.update(kw)
    return wl.Shape(**base)


# =============================================================================== copy + probe

@pytest.mark.parametrize("c,variant", [(1, "measure"), (2, "measure"), (2, "natural"),
                                       (4, "measure"), (5, "measure"), (5, "natural")])
def test_copy_match_workloads(c, variant):
    api = _api()
    sh = wl.config(c)
    case = wl.make_case(sh.with_(V=min(sh.V, 4096)) if c != 1 else sh, 100 + c, variant,
                        with_head=False, with_q=False)
    A = case.arrays
    say("copy_match", c, variant)
    g = api.copy_match(to_dev(A["ctx"]), to_dev(A["ctx_off"]), sh.kappa, sh.W, sh.D)
    o = oracle.copy_match(A["ctx"], A["ctx_off"], sh.kappa, sh.W, sh.D)
    for k in ("cand_tok", "cand_len", "cand_pos", "n_found", "flags"):
        assert np.array_equal(tensor_np(g[k]), o[k]), k


def test_copy_match_random_batches():
    api = _api()
    for seed in range(6):
        rng = np.random.default_rng(seed)
        kappa = int(rng.integers(1, 9))
        W = int(rng.integers(1, 9))
        D = int(rng.integers(1, 21))
        lens = rng.integers(0, 400, size=64)
        lens[:3] = [0, kappa, kappa + 1]
        seqs = [rng.integers(0, 3, size=int(n)).astype(np.int32) for n in lens]
        ctx = np.concatenate(seqs).astype(np.int32)
        off = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        say("copy_match random", seed, kappa, W, D)
        g = api.copy_match(to_dev(ctx), to_dev(off), kappa, W, D)
        o = oracle.copy_match(ctx, off, kappa, W, D)
        for k in ("cand_tok", "cand_len", "cand_pos", "n_found", "flags"):
            assert np.array_equal(tensor_np(g[k]), o[k]), (seed, k)


def test_copy_match_long_contexts_and_bad_offsets():
    """Occurrences far from the current token (several LDS segments), none at all,
    one straddling a segment boundary, and invalid offsets."""
    api = _api()
    rng = np.random.default_rng(9)
    L = 20000
    seqs = []
    a = rng.integers(10, 1000, size=L).astype(np.int32)
    a[-5:] = [1, 2, 3, 4, 5]
    a[3:8] = [1, 2, 3, 4, 5]
    seqs.append(a)                                            # only match near the start
    b = rng.integers(10, 1000, size=L).astype(np.int32)
    seqs.append(b)                                            # no match
    c = rng.integers(10, 1000, size=L).astype(np.int32)
    c[-5:] = [7, 7, 8, 8, 9]
    j = L - 2 - 8192 + 2                                      # window crosses a segment edge
    c[j - 4:j + 1] = [7, 7, 8, 8, 9]
    seqs.append(c)
    ctx = np.concatenate(seqs).astype(np.int32)
    off = np.array([0, L, 2 * L, 3 * L], dtype=np.int32)
    say("copy_match long")
    g = api.copy_match(to_dev(ctx), to_dev(off), 5, 4, 20)
    o = oracle.copy_match(ctx, off, 5, 4, 20)
    for k in ("cand_tok", "cand_len", "cand_pos", "n_found", "flags"):
        assert np.array_equal(tensor_np(g[k]), o[k]), k
    assert tensor_np(g["n_found"]).tolist() == [1, 0, 1]
    bad = np.array([0, 50, 40, 3 * L + 5], dtype=np.int32)   # decreasing, past the end
    g = api.copy_match(to_dev(ctx), to_dev(bad), 5, 2, 4)
    o = oracle.copy_match(ctx, bad, 5, 2, 4)
    for k in ("cand_tok", "cand_len", "cand_pos", "n_found", "flags"):
        assert np.array_equal(tensor_np(g[k]), o[k]), k
    assert (tensor_np(g["flags"])[1:] & oracle.FLAG_BAD_CTX).all()


@pytest.mark.parametrize("d,dtype", [(64, "f32"), (4096, "bf16"), (8192, "bf16")])
def test_probe_gate(d, dtype):
    api = _api()
    rng = np.random.default_rng(d)
    B = 64
    w = (rng.standard_normal(d) / np.sqrt(d)).astype(np.float32)
    h32 = rng.standard_normal((B, d)).astype(np.float32)
    h = wl.f32_to_bf16_bits(h32) if dtype == "bf16" else h32
    n_found = rng.integers(0, 3, size=B).astype(np.int32)
    say("probe", d, dtype)
    g = api.probe_gate(to_dev(h, dtype == "bf16"), to_dev(w), 0.4, to_dev(n_found))
    o = oracle.probe_gate(oracle.as_f64(h, dtype), w, 0.4, n_found)
    score = tensor_np(g["score"])
    assert np.abs(score - o["score"]).max() < 1e-5
    ok = o["flags"] == 0
    assert ok.sum() >= B - 2
    assert np.array_equal(tensor_np(g["gate"])[ok], o["gate"][ok])
    assert np.array_equal(tensor_np(g["flags"])[ok], o["flags"][ok])


# =============================================================================== attention

def _run_attention(case):
    api = _api()
    sh = case.shape
    T = case_to_dev(case, {"q", "k_cand", "v_cand", "k_pool", "v_pool", "page_table",
                           "prefix_len"})
    out, flags = api.verify_attention(T["q"], T["k_cand"], T["v_cand"], T["k_pool"],
                                      T["v_pool"], T["page_table"], T["prefix_len"], sh.W, sh.D)
    return tensor_np(out), tensor_np(flags)


def _oracle_attention(case, seqs=None):
    sh = case.shape
    A = case.arrays
    f = lambda k: oracle.as_f64(A[k], sh.dtype)
    return oracle.verify_attention(f("q"), f("k_cand"), f("v_cand"), f("k_pool"), f("v_pool"),
                                   A["page_table"], A["prefix_len"], sh.B, sh.W, sh.D, sh.Hq,
                                   sh.Hkv, out_dtype=sh.dtype)


@pytest.mark.parametrize("shape", [
    small_shape(),
    small_shape(B=3, P=(0, 16, 1000), W=2, D=5, Hq=16, Hkv=4),    # empty prefix, one page
    small_shape(B=1, P=(4096,), W=4, D=20, Hq=32, Hkv=8, d=4096),  # Llama-8B attention shape
    small_shape(B=2, P=(513, 2047), W=1, D=7, Hq=4, Hkv=4, d=512), # MHA, gamma=7 drafts
    small_shape(B=1, P=(100,), W=8, D=20, Hq=64, Hkv=8, d=8192),   # 70B rows, short prefix
], ids=["small", "edge_prefixes", "llama8b_attn", "mha_w1", "70b_rows"])
def test_attention_bf16(shape):
    case = wl.make_case(shape, 7, with_head=False, with_q=False)
    say("attention", shape)
    g, gf = _run_attention(case)
    _, o_r, of = _oracle_attention(case)
    assert np.array_equal(gf, of)
    err = rel_err(g, o_r)
    print(f"rel_err={err:.3e}")
    assert err <= TOL


@pytest.mark.parametrize("plan", ["", "1,256", "2,512", "4,256", "5,512", "8,1024"])
def test_attention_repeatable(plan, monkeypatch):
    """Repeated calls give the same bits for every row-block width (waves per workgroup)
    and split length, and match the oracle.  Operand registers of an MFMA that are
    overwritten while the product is still in the matrix pipe corrupt it depending on
    timing, so a kernel change that provokes that shows up here as differing repeats."""
    api = _api()
    sh = small_shape(B=2, P=(3000, 1100), W=4, D=20, Hq=32, Hkv=8, d=4096)
    case = get_case(("attn", "repeat"), lambda: wl.make_case(sh, 91, with_head=False, with_q=False))
    if plan:
        monkeypatch.setenv("VSTEP_ATTN_PLAN", plan)
    say("attention repeatable", plan or "default")
    outs = [_run_attention(case)[0] for _ in range(4)]
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])
    _, o_r, _ = _oracle_attention(case)
    err = rel_err(outs[0], o_r)
    print(f"rel_err={err:.3e}")
    assert err <= TOL


@pytest.mark.parametrize("B", [64, 65])
def test_attention_batch_orders(B, monkeypatch):
    """A batch of ragged prefixes (empty, one key, one key short of a split, exact
    multiples of the split, the longest, two out of range) through every order of
    workgroups to XCDs -- contiguous ranges, split-major, group-major and longest first
    (taken up to 64 sequences; 65 fall back to group-major) -- gives the same bits,
    matches the oracle, and flags the out-of-range lengths."""
    api = _api()
    rng = np.random.default_rng(B)
    P = rng.integers(0, 2049, size=B)
    P[:6] = [0, 1, 511, 512, 1024, 2048]
    sh = small_shape(B=B, P=tuple(int(x) for x in P), W=2, D=3, Hq=4, Hkv=2, d=512)
    case = wl.make_case(sh, 5 + B, with_head=False, with_q=False)
    case.arrays["prefix_len"][7] = -5
    case.arrays["prefix_len"][9] = 10 ** 6
    outs = {}
    for m in ("3", "2", "1", "0"):
        monkeypatch.setenv("VSTEP_ATTN_MAP", m)
        say("attention batch order", B, m)
        outs[m] = _run_attention(case)
    for m in ("2", "1", "0"):
        assert np.array_equal(outs[m][0], outs["3"][0]), m
        assert np.array_equal(outs[m][1], outs["3"][1]), m
    _, o_r, of = _oracle_attention(case)
    assert np.array_equal(outs["3"][1], of)
    assert (of[[7, 9]] & oracle.FLAG_BAD_PAGE).all()
    err = rel_err(outs["3"][0], o_r)
    print(f"rel_err={err:.3e}")
    assert err <= TOL


def test_attention_nan_in_page_tails():
    """The unused tail of each sequence's last page holds NaN in K and V: the masked
    keys must not reach the output (a zero probability times NaN would)."""
    sh = small_shape(B=3, P=(300, 777, 33), W=3, D=7, Hq=8, Hkv=2, d=1024)
    case = wl.make_case(sh, 23, with_head=False, with_q=False)
    A = case.arrays
    nan = np.uint16(0x7FC0)
    for b, P in enumerate(sh.P):
        if P % 16:
            pg = A["page_table"][b, (P - 1) // 16]
            A["k_pool"][pg, :, P % 16:, :] = nan
            A["v_pool"][pg, :, :, P % 16:] = nan
    say("attention NaN page tails")
    g, _ = _run_attention(case)
    assert np.isfinite(g).all()
    _, o_r, _ = _oracle_attention(case)
    err = rel_err(g, o_r)
    print(f"rel_err={err:.3e}")
    assert err <= TOL


@pytest.mark.parametrize("where", ["prefix", "candidates", "both"])
def test_attention_values_beyond_fp16(where):
    """Values of 2^16 and more (outside the fp16 range): a few huge entries in the
    paged prefix and/or in the candidates' own values, against the oracle, and
    repeated calls bit-identical."""
    sh = small_shape(B=2, P=(700, 1500), W=3, D=7, Hq=8, Hkv=2, d=1024)
    case = wl.make_case(sh, 17, with_head=False, with_q=False)
    A = case.arrays
    rng = np.random.default_rng(5)
    big = wl.f32_to_bf16_bits(np.array([2.0 ** 20, -3.0 * 2 ** 17, 1.5 * 2 ** 16, 2.0 ** 30],
                                       dtype=np.float32))
    if where in ("prefix", "both"):
        vp = A["v_pool"]
        for k in range(6):
            idx = tuple(int(rng.integers(0, n)) for n in vp.shape)
            vp[idx] = big[k % 4]
    if where in ("candidates", "both"):
        vc = A["v_cand"]
        for k in range(4):
            idx = tuple(int(rng.integers(0, n)) for n in vc.shape)
            vc[idx] = big[k % 4]
    say("attention values beyond fp16", where)
    outs = [_run_attention(case)[0] for _ in range(2)]
    assert np.array_equal(outs[0], outs[1])
    _, o_r, _ = _oracle_attention(case)
    err = rel_err(outs[0], o_r)
    print(f"rel_err={err:.3e}")
    assert err <= TOL


def test_attention_f32_tiny():
    case = wl.make_case(wl.config(1), 1000, with_head=False, with_q=False)
    say("attention tiny f32")
    g, gf = _run_attention(case)
    O, _, of = _oracle_attention(case)
    assert rel_err(g, O) < 1e-5 and np.array_equal(gf, of)


def test_attention_bad_page_flagged():
    sh = small_shape(B=2, P=(64, 64), paged_random=False)
    case = wl.make_case(sh, 3, with_head=False, with_q=False)
    case.arrays["page_table"][1, 2] = 10 ** 6            # out of the pool: skipped and flagged
    say("attention bad page")
    g, gf = _run_attention(case)
    _, o_r, of = _oracle_attention(case)
    assert gf.tolist() == of.tolist() and (gf[1] & oracle.FLAG_BAD_PAGE) and gf[0] == 0
    assert rel_err(g, o_r) <= TOL


@pytest.mark.parametrize("c", [2, 4, 5])
def test_attention_full_size(c):
    sh = wl.config(c)
    case = get_case(("attn", c), lambda: wl.make_case(sh.with_(V=1024), 1000 * c, with_head=False,
                                                       with_q=False))
    say("attention full", c)
    g, gf = _run_attention(case)
    _, o_r, of = _oracle_attention(case)
    assert np.array_equal(gf, of)
    err = rel_err(g, o_r)
    print(f"rel_err={err:.3e}")
    assert err <= TOL


def _layers_dev(LI, bf16):
    return {k: to_dev(v, bf16=bf16) for k, v in LI.items()}


@pytest.mark.parametrize("shape,L,plan", [
    (small_shape(), 3, ""),                                                  # split-K
    (small_shape(B=3, P=(0, 16, 1000), W=2, D=5, Hq=16, Hkv=4), 2, "0,8192"),  # one split
    (small_shape(B=1, P=(4096,), W=4, D=20, Hq=32, Hkv=8, d=4096), 4, ""),   # Llama-8B layers
    (wl.config(1), 3, ""),                                                   # fp32 path
], ids=["small_split", "one_split", "llama8b_4", "tiny_f32"])
def test_attention_layers(shape, L, plan, monkeypatch):
    """L layers in one launch, sharing the page table and prefix lengths: every layer
    against the oracle's layered attention; layer 0 also bit-identical to a one-layer
    call where both use the same plan (same splits)."""
    api = _api()
    case = wl.make_case(shape, 31, with_head=False, with_q=False)
    LI = wl.layer_inputs(case, L, 77)
    bf = shape.dtype == "bf16"
    T = _layers_dev(LI, bf)
    pt, plen = to_dev(case.arrays["page_table"]), to_dev(case.arrays["prefix_len"])
    if plan:
        monkeypatch.setenv("VSTEP_ATTN_PLAN", plan)
    say("attention layers", shape.name, L, plan or "default")
    out, fl = api.verify_attention(T["q"], T["k_cand"], T["v_cand"], T["k_pool"], T["v_pool"],
                                   pt, plen, shape.W, shape.D)
    g = tensor_np(out)
    f = lambda k: oracle.as_f64(LI[k], shape.dtype)
    O, o_r, of = oracle.verify_attention_layers(f("q"), f("k_cand"), f("v_cand"), f("k_pool"),
                                                f("v_pool"), case.arrays["page_table"],
                                                case.arrays["prefix_len"], shape.B, shape.W,
                                                shape.D, shape.Hq, shape.Hkv, out_dtype=shape.dtype)
    assert np.array_equal(tensor_np(fl), of)
    errs = [rel_err(g[l], (o_r if bf else O)[l]) for l in range(L)]
    print("rel_err per layer", ["%.2e" % e for e in errs])
    assert max(errs) <= (TOL if bf else 1e-5)
    if plan:
        one, _ = api.verify_attention(T["q"][0], T["k_cand"][0], T["v_cand"][0], T["k_pool"][0],
                                      T["v_pool"][0], pt, plen, shape.W, shape.D)
        assert np.array_equal(tensor_np(one), g[0])


def test_attention_layers_llama8b_32_sampled():
    """The 32 layers of a Llama-8B-shaped step (prefix 4096) in one launch, in the
    configuration the layered bench times; layers 0, 13 and 31 against the oracle."""
    api = _api()
    sh = small_shape(B=1, P=(4096,), W=4, D=20, Hq=32, Hkv=8, d=4096)
    case = wl.make_case(sh, 2000, with_head=False, with_q=False)
    L = 32
    LI = wl.layer_inputs(case, L, 5)
    T = _layers_dev(LI, True)
    say("attention layers llama8b 32")
    out, fl = api.verify_attention(T["q"], T["k_cand"], T["v_cand"], T["k_pool"], T["v_pool"],
                                   to_dev(case.arrays["page_table"]),
                                   to_dev(case.arrays["prefix_len"]), sh.W, sh.D)
    g = tensor_np(out)
    assert (tensor_np(fl) == 0).all()
    for l in (0, 13, 31):
        f = lambda k: oracle.as_f64(LI[k][l], "bf16")
        _, o_r, _ = oracle.verify_attention(f("q"), f("k_cand"), f("v_cand"), f("k_pool"),
                                            f("v_pool"), case.arrays["page_table"],
                                            case.arrays["prefix_len"], sh.B, sh.W, sh.D, sh.Hq,
                                            sh.Hkv, out_dtype="bf16")
        err = rel_err(g[l], o_r)
        print(f"layer {l}: rel_err={err:.3e}")
        assert err <= TOL


# =============================================================================== head

def _head_case(M, d, V, dtype="bf16", rank=0, seed=0):
    rng = np.random.default_rng(seed)
    h32 = rng.standard_normal((M, d)).astype(np.float32) * 0.05
    if rank == 0:
        w32 = (rng.standard_normal((V, d)) / np.sqrt(d)).astype(np.float32)
        ws = dict(w_full=w32)
    else:
        ws = dict(w_down=(rng.standard_normal((rank, d)) / np.sqrt(d)).astype(np.float32),
                  w_up=(rng.standard_normal((V, rank)) / np.sqrt(rank)).astype(np.float32))
        h32 = rng.standard_normal((M, d)).astype(np.float32)
    if dtype == "bf16":
        h = wl.f32_to_bf16_bits(h32)
        ws = {k: wl.f32_to_bf16_bits(v) for k, v in ws.items()}
    else:
        h = h32
    return h, ws


def test_pack_weight_layout():
    """Packed tile (t, s), lane l holds row 16t + l%16, columns 32s + 8(l//16) .. +7
    (rows past N zero) -- checked against numpy indexing of the row-major matrix."""
    api = _api()
    rng = np.random.default_rng(0)
    for N, K in ((1000, 96), (64, 32), (17, 256)):
        w = wl.f32_to_bf16_bits(rng.standard_normal((N, K)).astype(np.float32))
        say("pack", N, K)
        g = api.pack_weight(to_dev(w, True)).view(__import__("torch").int16).cpu().numpy()
        g = g.view(np.uint16).reshape(-1, K // 32, 64, 8)
        T = -(-N // 16)
        wp = np.zeros((T * 16, K), dtype=np.uint16)
        wp[:N] = w
        exp = wp.reshape(T, 16, K // 32, 4, 8).transpose(0, 2, 3, 1, 4).reshape(T, K // 32, 64, 8)
        assert np.array_equal(g, exp)


@pytest.mark.parametrize("M,d,V,dtype,T", [
    (37, 256, 1000, "bf16", 1.0), (100, 512, 2000, "bf16", 0.7), (8, 64, 512, "f32", 1.0),
    (160, 1024, 777, "bf16", 1.0), (1024, 256, 300, "bf16", 1.0), (200, 512, 1500, "bf16", 1.0),
    (192, 384, 900, "bf16", 0.8), (160, 8192, 2100, "bf16", 1.0), (144, 256, 1000, "bf16", 1.0),
    (176, 128, 513, "bf16", 1.2), (13, 300, 700, "f32", 0.9), (40, 512, 1000, "f32", 1.0),
    (640, 256, 700, "bf16", 1.0), (480, 128, 513, "bf16", 0.9), (448, 256, 1000, "bf16", 1.0),
    (400, 384, 300, "bf16", 1.0)])
def test_head_full(M, d, V, dtype, T):
    api = _api()
    h, ws = _head_case(M, d, V, dtype, seed=M + V)
    bf = dtype == "bf16"
    say("head", M, d, V, dtype)
    lg, lse, _ = api.lm_head(to_dev(h, bf), w_full=to_dev(ws["w_full"], bf), temperature=T)
    z, l = oracle.lm_head_full(oracle.as_f64(h, dtype), ws["w_full"], T, dtype)
    assert rel_err(tensor_np(lg), z) <= (TOL if bf else 1e-5)
    assert np.abs(tensor_np(lse) - l).max() < 1e-5


@pytest.mark.parametrize("env,M,d,V", [
    ("VSTEP_HEAD_STREAM=1", 80, 512, 1000),    # register-streaming kernel (the large-H path)
    ("VSTEP_HEAD_STREAM=1", 300, 256, 700),    # ... over several row blocks
    ("", 50, 160, 900),                        # d not a multiple of 128: streaming kernel
    ("VSTEP_HEAD_NG=1", 80, 512, 1000),        # one vocabulary tile per workgroup
    ("VSTEP_HEAD_TALL=0", 160, 256, 777),      # 160 rows as two row blocks
    ("", 777, 320, 1030),                      # many ragged rows, d % 128 != 0: streaming kernel
    ("", 600, 384, 900),                       # many rows through row blocks, ragged vocabulary
])
def test_head_kernel_variants(env, M, d, V, monkeypatch):
    """Every head kernel the launcher can choose, against the oracle: the streaming
    kernel (taken for d % 128 != 0 and for H of 2^31 elements or more) and the tuning
    variants."""
    api = _api()
    if env:
        k, v = env.split("=")
        monkeypatch.setenv(k, v)
    h, ws = _head_case(M, d, V, "bf16", seed=M + d)
    say("head variant", env or "default", M, d, V)
    hd, wd = to_dev(h, True), to_dev(ws["w_full"], True)
    lg, lse, _ = api.lm_head(hd, w_full=wd, temperature=0.9)
    z, l = oracle.lm_head_full(oracle.as_f64(h, "bf16"), ws["w_full"], 0.9, "bf16")
    err = rel_err(tensor_np(lg), z)
    print(f"rel_err={err:.3e}")
    assert err <= TOL
    assert np.abs(tensor_np(lse) - l).max() < 1e-5
    # repeated calls give the same bits (an MFMA operand overwritten while in flight
    # would show up as run-to-run differences)
    for _ in range(3):
        lg2, lse2, _ = api.lm_head(hd, w_full=wd, temperature=0.9)
        assert np.array_equal(tensor_np(lg2), tensor_np(lg))
        assert np.array_equal(tensor_np(lse2), tensor_np(lse))


def test_head_full_llama70b_size_sampled():
    """The full head at the Llama-70B shape (M = 160 rows, d = 8192, V = 128,256; two row
    blocks per vocabulary tile): 4,096 sampled vocabulary rows against the oracle's
    fp64 product, and every row's normaliser against the logsumexp of the kernel's own
    logits (a property at any size)."""
    import torch
    api = _api()
    M, d, V = 160, 8192, 128256
    rng = np.random.default_rng(70)
    h = wl.f32_to_bf16_bits((rng.standard_normal((M, d)) * 0.05).astype(np.float32))
    w = np.empty((V, d), dtype=np.uint16)
    for i in range(0, V, 8192):
        n = min(8192, V - i)
        w[i:i + n] = wl.f32_to_bf16_bits((rng.standard_normal((n, d)) / np.sqrt(d)).astype(np.float32))
    say("head 70b size")
    lg, lse, _ = api.lm_head(to_dev(h, True), w_full=to_dev(w, True))
    rows = np.sort(rng.choice(V, 4096, replace=False))
    g = tensor_np(lg)
    z = oracle.as_f64(h, "bf16") @ oracle.bf16_bits_to_f64(w[rows]).T
    assert rel_err(g[:, rows], z) <= TOL
    own = torch.logsumexp(lg.double(), dim=1).cpu().numpy()
    assert np.abs(tensor_np(lse) - own).max() < 1e-6


@pytest.mark.parametrize("M,d,r,V,dtype", [(7, 256, 64, 1000, "bf16"), (5, 512, 32, 3000, "bf16"),
                                           (9, 130, 21, 600, "f32")])
def test_head_lowrank_small(M, d, r, V, dtype):
    api = _api()
    bf = dtype == "bf16"
    h, ws = _head_case(M, d, V, dtype, rank=r, seed=r)
    say("head lowrank", M, d, r, V, dtype)
    lg, lse, pr = api.lm_head(to_dev(h, bf), w_down=to_dev(ws["w_down"], bf),
                              w_up=to_dev(ws["w_up"], bf), write_probs=True)
    z, l, _ = oracle.lm_head_lowrank(oracle.as_f64(h, dtype), ws["w_down"], ws["w_up"], 1.0,
                                     dtype)
    assert rel_err(tensor_np(lg), z) <= (TOL if bf else 1e-5)
    assert np.abs(tensor_np(lse) - l).max() < 1e-5
    p = oracle.head_softmax(z, l)
    assert rel_err(tensor_np(pr), p) <= TOL
    assert np.abs(tensor_np(pr).astype(np.float64).sum(axis=1) - 1).max() < 1e-4


def test_head_lowrank_slimspec_full():
    """SlimSpec draft head at r = d/8 = 512 over the full vocabulary; also checked
    against the dense product (W_up W_down) h on sampled vocabulary rows."""
    api = _api()
    sh = wl.config(3)
    case = get_case(("slim",), lambda: wl.make_case(sh, 3000, with_head=False, with_q=False))
    A = case.arrays
    say("head lowrank slimspec full")
    lg, lse, pr = api.lm_head(to_dev(A["draft_h"], True), w_down=to_dev(A["w_down"], True),
                              w_up=to_dev(A["w_up"], True), write_probs=True)
    z, l, t = oracle.lm_head_lowrank(oracle.as_f64(A["draft_h"], "bf16"), A["w_down"], A["w_up"])
    g = tensor_np(lg)
    assert rel_err(g, z) <= TOL
    assert np.abs(tensor_np(lse) - l).max() < 1e-5
    assert rel_err(tensor_np(pr), oracle.head_softmax(z, l)) <= TOL
    rows = np.random.default_rng(0).choice(sh.V, 8192, replace=False)
    dense = oracle.bf16_bits_to_f64(A["w_up"][rows]) @ oracle.bf16_bits_to_f64(A["w_down"])
    zd = oracle.as_f64(A["draft_h"], "bf16") @ dense.T
    assert rel_err(g[:, rows], zd) <= TOL


# =============================================================================== sampler

@pytest.mark.parametrize("qmode,T", [("dense", 1.0), ("point", 1.0), ("dense", 0.6)])
def test_reject_sample_synthetic(qmode, T):
    """Sampler alone on generator-made logits; its row normaliser input is scipy's
    logsumexp of those logits."""
    api = _api()
    rng = np.random.default_rng(5)
    B, W, D, V = 64, 3, 5, 1000
    M = W * D
    root = (rng.standard_normal((B, V)) * 1.5).astype(np.float32)
    logits = (rng.standard_normal((B * M, V)) * 1.5).astype(np.float32)
    lse = scipy.special.logsumexp(logits.astype(np.float64) / T, axis=1)
    q = wl.draft_probs_from_logits(rng, (B * M, V), 1.5) if qmode == "dense" else None
    # drafts: mostly high-probability tokens so that runs are long and varied
    cand = rng.integers(0, 20, size=(B, W, D)).astype(np.int32)
    clen = rng.integers(0, D + 1, size=(B, W)).astype(np.int32)
    clen[0] = 0                                   # no candidate
    for b in range(B):
        for i in range(W):
            cand[b, i, clen[b, i]:] = -1
    ua = rng.random((B, W, D))
    ur = rng.random((B, W))
    gate = np.ones(B, dtype=np.int32)
    gate[1] = 0                                   # closed gate
    say("reject_sample", qmode, T)
    g = api.reject_sample(to_dev(root), to_dev(logits), to_dev(lse),
                          to_dev(q) if q is not None else None, to_dev(cand), to_dev(clen),
                          to_dev(ua), to_dev(ur), T, to_dev(gate))
    o = oracle.reject_sample(root, logits, q, cand, clen, ua, ur, T, gate)
    n_cmp, n_exc = compare_sampler(g, o, B)
    assert n_exc <= 2 and n_cmp >= B - 2
    assert (tensor_np(g["flags"])[:2] & oracle.FLAG_NO_CANDIDATE).all()


@pytest.mark.parametrize("qmode", ["dense", "point"])
def test_reject_sample_fused_and_two_launch_agree(qmode, monkeypatch):
    """The sampler's two ways to reach the draw (last workgroup of a fused launch, or a
    second launch) give the same bits, on a batch where the vocabulary spans several
    chunks and the sequences' chunks outnumber the CUs; both match the oracle."""
    api = _api()
    rng = np.random.default_rng(21)
    B, W, D, V = 40, 2, 4, 9000
    M = W * D
    root = (rng.standard_normal((B, V)) * 1.5).astype(np.float32)
    logits = (rng.standard_normal((B * M, V)) * 1.5).astype(np.float32)
    lse = scipy.special.logsumexp(logits.astype(np.float64), axis=1)
    q = wl.draft_probs_from_logits(rng, (B * M, V), 1.5) if qmode == "dense" else None
    cand = rng.integers(0, 30, size=(B, W, D)).astype(np.int32)
    clen = rng.integers(0, D + 1, size=(B, W)).astype(np.int32)
    for b in range(B):
        for i in range(W):
            cand[b, i, clen[b, i]:] = -1
    ua = rng.random((B, W, D))
    ur = rng.random((B, W))
    args = (to_dev(root), to_dev(logits), to_dev(lse), to_dev(q) if q is not None else None,
            to_dev(cand), to_dev(clen), to_dev(ua), to_dev(ur), 1.0)
    got = {}
    for mode in ("0", "1", "0", "1"):
        monkeypatch.setenv("VSTEP_SAMPLER_TWO_PASS", mode)
        say("reject_sample two-launch", qmode, mode)
        g = api.reject_sample(*args)
        g = {k: tensor_np(v).copy() for k, v in g.items()}
        if mode in got:
            for k in g:
                assert np.array_equal(g[k], got[mode][k]), (mode, k)
        got[mode] = g
    for k in got["0"]:
        assert np.array_equal(got["0"][k], got["1"][k]), k
    o = oracle.reject_sample(root, logits, q, cand, clen, ua, ur, 1.0, None)
    import torch
    n_cmp, n_exc = compare_sampler({k: torch.from_numpy(v) for k, v in got["1"].items()}, o, B)
    assert n_exc <= 1 and n_cmp >= B - 1


def _multi_case(rng, B, W, D, V, boost=8.0, n_hot=2):
    """Logits with n_hot tokens boosted in every row (so acceptances are frequent) and
    copy candidates over those tokens that share prefixes: candidate i copies a prefix
    of an earlier candidate and then goes its own way, as copy candidates of one
    context do.  Some tokens are out of range, some lengths are zero."""
    M = W * D
    hot = np.arange(1, 1 + n_hot)
    root = rng.standard_normal((B, V)).astype(np.float32)
    logits = rng.standard_normal((B * M, V)).astype(np.float32)
    root[:, hot] += boost
    logits[:, hot] += boost
    cand = rng.choice(hot, size=(B, W, D)).astype(np.int32)
    for b in range(B):
        for i in range(1, W):
            j = rng.integers(0, i)
            k = rng.integers(0, D + 1)
            cand[b, i, :k] = cand[b, j, :k]
    rare = rng.random((B, W, D)) < 0.03
    cand[rare] = rng.integers(0, V, size=rare.sum())
    cand[rng.random((B, W, D)) < 0.01] = V + 3               # out of range: rejected
    clen = rng.integers(0, D + 1, size=(B, W)).astype(np.int32)
    clen[rng.random((B, W)) < 0.5] = D
    for b in range(B):
        for i in range(W):
            cand[b, i, clen[b, i]:] = -1
    return root, logits, cand, clen


@pytest.mark.parametrize("B,W,D,V,T", [(96, 4, 6, 1000, 1.0), (64, 8, 20, 3000, 0.8),
                                       (48, 3, 2, 2100, 1.0)])
def test_reject_sample_multi(B, W, D, V, T):
    """Lossless multi-candidate acceptance against the oracle's rule on candidates that
    branch from shared prefixes (siblings with equal, distinct and invalid tokens)."""
    api = _api()
    rng = np.random.default_rng(31 + W)
    root, logits, cand, clen = _multi_case(rng, B, W, D, V)
    clen[0] = 0
    lse = scipy.special.logsumexp(logits.astype(np.float64) / T, axis=1)
    ua = rng.random((B, W, D))
    ur = rng.random((B, W))
    gate = np.ones(B, dtype=np.int32)
    gate[1] = 0
    say("reject_sample multi", B, W, D, V, T)
    g = api.reject_sample(to_dev(root), to_dev(logits), to_dev(lse), None, to_dev(cand),
                          to_dev(clen), to_dev(ua), to_dev(ur), T, to_dev(gate), accept="multi")
    o = oracle.reject_sample_multi(root, logits, None, cand, clen, ua, ur, T, gate)
    n_cmp, n_exc = compare_sampler(g, o, B)
    assert n_exc <= 2 and n_cmp >= B - 2
    # the chains did branch: sequences whose final reference is not candidate 0
    assert (o["best"] > 0).sum() >= 3 and (o["n_acc"] >= 2).sum() >= 3
    assert (tensor_np(g["flags"])[:2] & oracle.FLAG_NO_CANDIDATE).all()


@pytest.mark.parametrize("B,W,D,V,T", [(48, 4, 6, 1000, 1.0), (16, 8, 20, 3000, 0.8),
                                       (6, 2, 5, 128256, 1.0)])
def test_reject_sample_multi_dense(B, W, D, V, T):
    """Lossless multi-candidate acceptance with dense draft distributions (each
    rejection removes the sibling's whole q row from the residual) against the
    oracle's rule, up to the full vocabulary."""
    api = _api()
    rng = np.random.default_rng(53 + W + V)
    root, logits, cand, clen = _multi_case(rng, B, W, D, V)
    clen[0] = 0
    M = W * D
    # draft distributions favouring the same hot tokens, less sharply than the target
    ql = rng.standard_normal((B * M, V))
    ql[:, 1:3] += 6.0
    ql -= ql.max(axis=1, keepdims=True)
    q = np.exp(ql)
    q = (q / q.sum(axis=1, keepdims=True)).astype(np.float32)
    lse = scipy.special.logsumexp(logits.astype(np.float64) / T, axis=1)
    ua = rng.random((B, W, D))
    ur = rng.random((B, W))
    gate = np.ones(B, dtype=np.int32)
    gate[1] = 0
    say("reject_sample multi dense", B, W, D, V, T)
    g = api.reject_sample(to_dev(root), to_dev(logits), to_dev(lse), to_dev(q), to_dev(cand),
                          to_dev(clen), to_dev(ua), to_dev(ur), T, to_dev(gate), accept="multi")
    o = oracle.reject_sample_multi(root, logits, q, cand, clen, ua, ur, T, gate)
    n_cmp, n_exc = compare_sampler(g, o, B)
    print(f"compared {n_cmp}/{B}, excluded {n_exc}; n_acc {o['n_acc'].tolist()[:12]}")
    assert n_exc <= max(1, B // 16) and n_cmp >= B - max(1, B // 16)
    # chains that accepted tokens, and chains that ended on a rejection
    ln = clen.max(axis=1)
    assert (o["n_acc"][2:] >= 1).any() and (o["n_acc"][2:] < ln[2:]).any()
    assert (tensor_np(g["flags"])[:2] & oracle.FLAG_NO_CANDIDATE).all()


def test_reject_sample_multi_dense_widths(monkeypatch):
    """The dense chain gives the same bits whether a sequence's vocabulary passes are
    shared by 1, 3 or 16 workgroups (each chunk's sum is formed the same way whatever
    workgroup owns it), with several rejections per sequence at V = 128,256."""
    api = _api()
    rng = np.random.default_rng(808)
    B, W, D, V, T = 5, 6, 3, 128256, 1.0
    root, logits, cand, clen = _multi_case(rng, B, W, D, V)
    M = W * D
    ql = rng.standard_normal((B * M, V))
    ql[:, 1:3] += 6.0
    ql -= ql.max(axis=1, keepdims=True)
    q = np.exp(ql)
    q = (q / q.sum(axis=1, keepdims=True)).astype(np.float32)
    lse = scipy.special.logsumexp(logits.astype(np.float64) / T, axis=1)
    ua = rng.random((B, W, D))
    ur = rng.random((B, W))
    outs = []
    for wg in ("1", "3", "16"):
        monkeypatch.setenv("VSTEP_DENSE_WG", wg)
        say("reject_sample multi dense widths", wg)
        g = api.reject_sample(to_dev(root), to_dev(logits), to_dev(lse), to_dev(q), to_dev(cand),
                              to_dev(clen), to_dev(ua), to_dev(ur), T, None, accept="multi")
        outs.append({k: tensor_np(v) for k, v in g.items()})
    for o in outs[1:]:
        for k in outs[0]:
            assert np.array_equal(o[k], outs[0][k]), k
    orc = oracle.reject_sample_multi(root, logits, q, cand, clen, ua, ur, T, None)
    n_cmp, n_exc = compare_sampler({k: to_dev(v) for k, v in outs[0].items()}, orc, B)
    print(f"compared {n_cmp}/{B}, excluded {n_exc}; n_acc {orc['n_acc'].tolist()}")
    assert n_cmp >= B - 1
    assert not (outs[0]["flags"] & 512).any()      # no wait gave up


@pytest.mark.parametrize("mode", ["0", "1"])
def test_reject_sample_multi_launch_modes(mode, monkeypatch):
    """Multi-candidate acceptance through both ways to reach the draw, with more
    sequence chunks than CUs, against the oracle."""
    api = _api()
    rng = np.random.default_rng(77)
    B, W, D, V = 40, 4, 8, 9000
    root, logits, cand, clen = _multi_case(rng, B, W, D, V)
    lse = scipy.special.logsumexp(logits.astype(np.float64), axis=1)
    ua = rng.random((B, W, D))
    ur = rng.random((B, W))
    monkeypatch.setenv("VSTEP_SAMPLER_TWO_PASS", mode)
    say("reject_sample multi launch mode", mode)
    g = api.reject_sample(to_dev(root), to_dev(logits), to_dev(lse), None, to_dev(cand),
                          to_dev(clen), to_dev(ua), to_dev(ur), 1.0, accept="multi")
    o = oracle.reject_sample_multi(root, logits, None, cand, clen, ua, ur, 1.0, None)
    n_cmp, n_exc = compare_sampler(g, o, B)
    assert n_exc <= 1 and n_cmp >= B - 1


def test_reject_sample_multi_single_candidate_is_literal():
    """With one candidate the multi rule is the single-chain rule: same bits, dense or
    point-mass drafts."""
    api = _api()
    rng = np.random.default_rng(8)
    B, W, D, V = 32, 1, 7, 5000
    root, logits, cand, clen = _multi_case(rng, B, W, D, V)
    lse = scipy.special.logsumexp(logits.astype(np.float64), axis=1)
    q = wl.draft_probs_from_logits(rng, (B * W * D, V), 1.5)
    ua = rng.random((B, W, D))
    ur = rng.random((B, W))
    for qq in (q, None):
        args = (to_dev(root), to_dev(logits), to_dev(lse), None if qq is None else to_dev(qq),
                to_dev(cand), to_dev(clen), to_dev(ua), to_dev(ur), 1.0)
        say("reject_sample multi W=1", qq is None)
        a = api.reject_sample(*args, accept="multi")
        b = api.reject_sample(*args, accept="longest")
        for k in a:
            assert np.array_equal(tensor_np(a[k]), tensor_np(b[k])), k


def test_reject_sample_workspace_reused_across_shapes(monkeypatch):
    """The binding's cached workspace is zeroed when the shape changes: a two-launch
    call on a small batch leaves chunk sums where a larger batch keeps its counters,
    and the larger batch still completes every sequence."""
    api = _api()
    rng = np.random.default_rng(4)
    for B, V, two in ((40, 9000, "1"), (96, 1000, "0")):
        W, D = 4, 6
        root, logits, cand, clen = _multi_case(rng, B, W, D, V)
        lse = scipy.special.logsumexp(logits.astype(np.float64), axis=1)
        ua = rng.random((B, W, D))
        ur = rng.random((B, W))
        monkeypatch.setenv("VSTEP_SAMPLER_TWO_PASS", two)
        say("reject_sample workspace reuse", B, V)
        g = api.reject_sample(to_dev(root), to_dev(logits), to_dev(lse), None, to_dev(cand),
                              to_dev(clen), to_dev(ua), to_dev(ur), 1.0)
        o = oracle.reject_sample(root, logits, None, cand, clen, ua, ur, 1.0, None)
        n_cmp, n_exc = compare_sampler(g, o, B)
        assert n_exc <= 1 and n_cmp >= B - 1


def _greedy_case(rng, B, W, D, V):
    """Random logits; draft tokens that are mostly the argmax of their preceding row
    (so runs are long); rows with exact ties (inside a tile and across tiles), a row
    of equal logits (every tile holds the maximum), out-of-range tokens, a closed
    gate and a sequence without candidates."""
    M = W * D
    root = rng.standard_normal((B, V)).astype(np.float32)
    logits = rng.standard_normal((B * M, V)).astype(np.float32)
    for r in rng.choice(B * M, size=B * M // 6, replace=False):
        k = int(np.argmax(logits[r]))
        j = int(rng.integers(0, V))
        logits[r, j] = logits[r, k]                 # exact tie, possibly in another tile
    logits[5] = 0.25                                 # all equal: argmax is token 0
    t = min(3, B - 1)
    root[t, :] = root[t, int(np.argmax(root[t]))]
    cand = rng.integers(0, V, size=(B, W, D)).astype(np.int32)
    for b in range(B):
        for i in range(W):
            for o in range(D):
                if rng.random() < 0.8:
                    row = root[b] if o == 0 else logits[b * M + i * D + o - 1]
                    cand[b, i, o] = int(np.argmax(row))
    cand[rng.random((B, W, D)) < 0.01] = V + 7
    clen = rng.integers(0, D + 1, size=(B, W)).astype(np.int32)
    clen[rng.random((B, W)) < 0.5] = D
    clen[0] = 0
    gate = np.ones(B, dtype=np.int32)
    gate[1] = 0
    return root, logits, cand, clen, gate


@pytest.mark.parametrize("B,W,D,V,T", [(64, 4, 6, 3000, 1.0), (40, 3, 5, 1000, 0.7),
                                       (16, 8, 20, 128256, 1.0)])
def test_reject_sample_greedy(B, W, D, V, T):
    """Greedy verification against the oracle on the same fp32 logits: every output and
    every flag equal, near and exact ties included (both sides decide on the same
    values; exact ties take the first index)."""
    api = _api()
    rng = np.random.default_rng(60 + W)
    root, logits, cand, clen, gate = _greedy_case(rng, B, W, D, V)
    lse = scipy.special.logsumexp(logits.astype(np.float64) / T, axis=1)
    say("reject_sample greedy", B, W, D, V, T)
    g = api.reject_sample(to_dev(root), to_dev(logits), to_dev(lse), None, to_dev(cand),
                          to_dev(clen), None, None, T, to_dev(gate), accept="greedy")
    o = oracle.reject_sample_greedy(root, logits, cand, clen, gate)
    for k in ("n_acc", "best", "out_tok", "n_out", "acc_per_cand", "flags"):
        assert np.array_equal(tensor_np(g[k]), o[k]), (k, np.nonzero(
            (tensor_np(g[k]) != o[k]).reshape(B, -1).any(axis=1))[0][:5])
    assert (o["n_acc"] >= 3).sum() > B // 4
    assert (o["flags"] & oracle.FLAG_CDF_TIE).any() or (o["flags"] & oracle.FLAG_ACCEPT_TIE).any()


# =============================================================================== limits

def test_limits_max_rows_per_sequence():
    """W*D = 1024 draft rows per sequence (the largest the ABI takes): retrieval with 32
    candidates x 32 tokens, attention of 4096 query rows per KV head, and the sampler
    (longest run and greedy) over 1024 rows, each against the oracle."""
    api = _api()
    rng = np.random.default_rng(99)
    # retrieval: a context made of many repeats of the trailing 5-gram
    W, D, kappa = 32, 32, 5
    base = rng.integers(0, 50, size=2000).astype(np.int32)
    key = base[-kappa:]
    for j in rng.choice(np.arange(10, 1900), size=60, replace=False):
        base[j:j + kappa] = key
    off = np.array([0, len(base)], np.int32)
    say("limits copy_match")
    g = api.copy_match(to_dev(base), to_dev(off), kappa, W, D)
    o = oracle.copy_match(base, off, kappa, W, D)
    for k in ("cand_tok", "cand_len", "cand_pos", "n_found", "flags"):
        assert np.array_equal(tensor_np(g[k]), o[k]), k
    assert o["n_found"][0] == W
    # attention: 1 sequence x 1024 rows, 2 KV heads of 4 query heads, prefix 200
    sh = small_shape(B=1, W=16, D=64, Hq=8, Hkv=2, P=(200,), V=600)
    case = get_case(("limits", "attn"),
                    lambda: wl.make_case(sh, 77, with_head=False, with_q=False))
    say("limits attention")
    ga, gf = _run_attention(case)
    _, o_r, of = _oracle_attention(case)
    assert np.array_equal(gf, of)
    assert rel_err(ga, o_r) <= TOL
    # sampler over 1024 rows (longest run and greedy)
    B, W, D, V = 2, 32, 32, 3000
    root, logits, cand, clen, gate = _greedy_case(rng, B, W, D, V)
    gate[:] = 1
    clen[0] = D
    lse = scipy.special.logsumexp(logits.astype(np.float64), axis=1)
    ua = rng.random((B, W, D))
    ur = rng.random((B, W))
    say("limits sampler")
    g = api.reject_sample(to_dev(root), to_dev(logits), to_dev(lse), None, to_dev(cand),
                          to_dev(clen), to_dev(ua), to_dev(ur), 1.0)
    o = oracle.reject_sample(root, logits, None, cand, clen, ua, ur, 1.0)
    n_cmp, n_exc = compare_sampler(g, o, B)
    assert n_cmp >= 1
    g = api.reject_sample(to_dev(root), to_dev(logits), to_dev(lse), None, to_dev(cand),
                          to_dev(clen), None, None, 1.0, accept="greedy")
    o = oracle.reject_sample_greedy(root, logits, cand, clen)
    for k in ("n_acc", "best", "out_tok", "n_out", "acc_per_cand", "flags"):
        assert np.array_equal(tensor_np(g[k]), o[k]), k


def test_limits_multi_lds_bound():
    """Multi-candidate acceptance at the largest LDS footprint it takes (W = 8, D = 50:
    401 x 8 + 400 doubles), against the oracle."""
    api = _api()
    rng = np.random.default_rng(5)
    B, W, D, V = 6, 8, 50, 2000
    root, logits, cand, clen = _multi_case(rng, B, W, D, V)
    lse = scipy.special.logsumexp(logits.astype(np.float64), axis=1)
    ua = rng.random((B, W, D))
    ur = rng.random((B, W))
    say("limits multi")
    g = api.reject_sample(to_dev(root), to_dev(logits), to_dev(lse), None, to_dev(cand),
                          to_dev(clen), to_dev(ua), to_dev(ur), 1.0, accept="multi")
    o = oracle.reject_sample_multi(root, logits, None, cand, clen, ua, ur, 1.0)
    n_cmp, n_exc = compare_sampler(g, o, B)
    assert n_exc <= 1 and n_cmp >= B - 1


# =============================================================================== draft tokens

@pytest.mark.parametrize("rows,V", [(64, 1000), (33, 3001), (16, 128256)])
def test_draft_sample(rows, V):
    """Draft tokens by inverse CDF of stored probabilities, against the oracle on the same
    fp32 rows (zero-probability ids included); near ties flagged on either side are
    left out."""
    api = _api()
    rng = np.random.default_rng(V)
    q = wl.draft_probs_from_logits(rng, (rows, V), 2.0)
    q[:, rng.choice(V, size=V // 5, replace=False)] = 0.0
    u = rng.random(rows)
    say("draft sample", rows, V)
    tok, f = api.draft_sample(to_dev(q), to_dev(u))
    to, fo = oracle.draft_sample(q, u)
    tg, fg = tensor_np(tok), tensor_np(f)
    ok = (fg | fo) == 0
    assert ok.sum() >= rows - 1
    assert np.array_equal(tg[ok], to[ok])
    assert (q[np.arange(rows), tg] > 0).all()


def test_draft_sample_slimspec_pipeline():
    """The SlimSpec draft side on the GPU: the low-rank head's probabilities, then the
    draft tokens drawn from them.  Each token's CDF interval under those probabilities
    (summed in fp64 on the host) holds u * S."""
    api = _api()
    sh = wl.config(3)
    case = get_case(("slim",), lambda: wl.make_case(sh, 3000, with_head=False, with_q=False))
    A = case.arrays
    say("slimspec draft pipeline")
    _, _, pr = api.lm_head(to_dev(A["draft_h"], True), w_down=to_dev(A["w_down"], True),
                           w_up=to_dev(A["w_up"], True), write_probs=True)
    u = A["u_draft"][0, 0, :sh.D]
    tok, f = api.draft_sample(pr, to_dev(u))
    q = tensor_np(pr).astype(np.float64)
    for r, k in enumerate(tensor_np(tok)):
        c = np.cumsum(q[r])
        x = u[r] * c[-1]
        lo = c[k - 1] if k > 0 else 0.0
        assert q[r, k] > 0 and lo - 1e-9 * c[-1] <= x < c[k] + 1e-9 * c[-1]


# =============================================================================== copy labels

@pytest.mark.parametrize("kappa", [1, 3, 5, 7, 16])
def test_copy_labels_random(kappa):
    """Small-alphabet contexts with planted repeats (empty, shorter-than-kappa and long
    sequences, and a buffer with room before and after the sequences): every label
    equal to the oracle's, untouched positions keep their value."""
    api = _api()
    rng = np.random.default_rng(kappa)
    lens = rng.integers(0, 700, size=23)
    lens[[0, 5]] = 0
    lens[7] = max(kappa - 1, 0)
    parts = []
    for n in lens:
        c = rng.integers(0, {1: 500, 3: 8, 5: 3, 7: 3, 16: 2}[kappa], size=n)
        for _ in range(int(n) // 60):
            L = int(rng.integers(kappa, 3 * kappa + 2))
            if n > 2 * L:
                a, d = sorted(rng.choice(n - L, size=2, replace=False))
                c[d:d + L] = c[a:a + L]
        parts.append(c)
    body = np.concatenate(parts).astype(np.int32)
    ctx = np.concatenate([np.full(17, 1, np.int32), body, np.full(9, 1, np.int32)])
    off = (17 + np.concatenate([[0], np.cumsum(lens)])).astype(np.int32)
    init = np.full(len(ctx), 7, np.uint8)
    say("copy labels", kappa)
    y, f = api.copy_labels(to_dev(ctx), to_dev(off), kappa, to_dev(init))
    yo, fo = oracle.copy_labels(ctx, off, kappa, init)
    assert np.array_equal(tensor_np(f), fo)
    assert np.array_equal(tensor_np(y), yo)
    assert 0.05 < yo[17:-9].mean() < 0.95


def test_copy_labels_bad_offsets():
    api = _api()
    ctx = (np.arange(300) % 7).astype(np.int32)
    init = np.full(300, 7, np.uint8)
    for off in ([0, 120, 80, 300], [-3, 100, 300], [0, 100, 301]):
        say("copy labels bad offsets", off)
        y, f = api.copy_labels(to_dev(ctx), to_dev(np.array(off, np.int32)), 5, to_dev(init))
        assert (tensor_np(f) == oracle.FLAG_BAD_CTX).all()
        assert (tensor_np(y) == 7).all()


@pytest.mark.parametrize("name", ["ragged", "llama70b", "long"])
def test_copy_labels_full_contexts(name):
    """The workloads' own contexts: 32 Zipf contexts of 512..8192 tokens with 5% planted
    repeats, one of 16,384 with 5..60-token plants, and one of 262,144 tokens."""
    api = _api()
    if name == "long":
        rng = np.random.default_rng(3)
        ctx, _, _ = wl.make_context(rng, np.random.default_rng(4), 1 << 18, 128256, 0.05,
                                    (5, 40), 4, 20, 5, False)
        off = np.array([0, len(ctx)], np.int32)
    else:
        sh, seed = (wl.config(5), 5000) if name == "ragged" else (wl.config(4), 4000)
        case = get_case(("labels", name), lambda: wl.make_case(sh, seed, with_head=False))
        ctx, off = case.arrays["ctx"], case.arrays["ctx_off"]
    say("copy labels", name, len(ctx))
    y, f = api.copy_labels(to_dev(ctx), to_dev(off), 5)
    yo, fo = oracle.copy_labels(ctx, off, 5)
    assert not tensor_np(f).any() and not fo.any()
    assert np.array_equal(tensor_np(y), yo)
    assert 0.02 < yo.mean() < 0.5


# =============================================================================== KV commit

def _kv_dev(A, dtype):
    import torch
    out = {}
    for k, v in A.items():
        if isinstance(v, np.ndarray):
            t = torch.from_numpy(np.ascontiguousarray(v))
            if dtype == "bf16" and v.dtype == np.uint16:
                t = t.view(torch.bfloat16)
            out[k] = t.cuda()
    import torch as _t
    out["n_free"] = _t.tensor([A["n_free"]], dtype=_t.int32, device="cuda")
    return out


def _kv_host(G):
    import torch
    out = {}
    for k, t in G.items():
        if t.dtype == torch.bfloat16:
            out[k] = t.view(torch.int16).cpu().numpy().view(np.uint16)
        else:
            out[k] = t.cpu().numpy()
    out["n_free"] = int(out["n_free"][0])
    return out


def _kv_check(G, A, flags_g, flags_o):
    H = _kv_host(G)
    assert np.array_equal(flags_g, flags_o)
    for k in ("page_table", "prefix_len", "k_pool", "v_pool"):
        assert np.array_equal(H[k], A[k]), k
    assert H["n_free"] == A["n_free"]
    nf = min(max(A["n_free"], 0), len(A["free_list"]))
    assert np.array_equal(H["free_list"][:nf], A["free_list"][:nf])


@pytest.mark.parametrize("dtype,Hkv,hd", [("bf16", 8, 128), ("f32", 2, 64)])
def test_kv_commit_and_truncate_rounds(dtype, Hkv, hd):
    """Rounds of commit (fresh candidates and accepted runs each round) and random
    rollbacks: pools, page tables, lengths, the free stack and the flags equal the
    oracle's bit for bit after every call."""
    api = _api()
    B, W, D = 7, 3, 9
    A = wl.make_kv_case(3, B, W, D, Hkv, hd, [0, 1, 15, 16, 17, 40, 100], n_spare=30,
                        max_pages=16, dtype=dtype)
    G = _kv_dev(A, dtype)
    rng = np.random.default_rng(12)
    for rnd in range(5):
        fresh = wl.make_kv_case(50 + rnd, B, W, D, Hkv, hd, [0] * B, 0, 16, dtype)
        if rnd == 3:
            # full runs against a stack cut down to one page: refusals
            fresh["n_acc"][:] = D
            A["n_free"] = 1
            G["n_free"].fill_(1)
        for k in ("k_cand", "v_cand", "best", "n_acc"):
            A[k] = fresh[k]
            G[k] = _kv_dev({k: fresh[k], "n_free": 0}, dtype)[k]
        say("kv commit", dtype, rnd)
        fg = api.kv_commit(G["k_cand"], G["v_cand"], G["best"], G["n_acc"], G["k_pool"],
                           G["v_pool"], G["page_table"], G["prefix_len"], G["free_list"],
                           G["n_free"], W, D)
        k, v, pt, P, fl, nf, fo = oracle.kv_commit(
            A["k_pool"], A["v_pool"], A["page_table"], A["prefix_len"], A["free_list"],
            A["n_free"], A["k_cand"], A["v_cand"], A["best"], A["n_acc"], W, D)
        A.update(k_pool=k, v_pool=v, page_table=pt, prefix_len=P, free_list=fl, n_free=nf)
        _kv_check(G, A, tensor_np(fg), fo)
        if rnd == 3:
            assert (fo == oracle.FLAG_POOL_EMPTY).any()
        cut = np.array([rng.integers(0, int(p) + 1) if rng.random() < 0.5 else int(p)
                        for p in A["prefix_len"]], dtype=np.int32)
        cut[0] = int(A["prefix_len"][0]) + 1    # above the length: refused
        say("kv truncate", dtype, rnd)
        fg = api.kv_truncate(to_dev(cut), G["page_table"], G["prefix_len"], G["free_list"],
                             G["n_free"], A["k_pool"].shape[0])
        pt, P, fl, nf, fo = oracle.kv_truncate(A["page_table"], A["prefix_len"], cut,
                                               A["free_list"], A["n_free"], A["k_pool"].shape[0])
        A.update(page_table=pt, prefix_len=P, free_list=fl, n_free=nf)
        _kv_check(G, A, tensor_np(fg), fo)
    assert (fo == oracle.FLAG_BAD_PAGE).sum() == 1


@pytest.mark.parametrize("dtype,L", [("bf16", 4), ("f32", 3)])
def test_kv_commit_layers_then_truncate(dtype, L):
    """One commit over L layer pools that share the page table: every layer's pool,
    the table, lengths, stack and flags equal the oracle's bit for bit; then one
    rollback (the table is shared, so one call rolls back every layer) and a second
    commit into the pages it freed."""
    import torch
    api = _api()
    B, W, D, Hkv, hd = 6, 3, 9, 2, 128 if dtype == "bf16" else 64
    A = wl.make_kv_case(8, B, W, D, Hkv, hd, [0, 1, 15, 16, 40, 100], n_spare=24,
                        max_pages=16, dtype=dtype)
    rng = np.random.default_rng(3)
    extra = lambda a: np.stack([a] + [wl._normal_model(rng, a.shape, 1.0, dtype)
                                      for _ in range(L - 1)])
    A["k_pool"], A["v_pool"] = extra(A["k_pool"]), extra(A["v_pool"])
    for rnd in range(2):
        fresh = wl.make_kv_case(60 + rnd, B, W, D, Hkv, hd, [0] * B, 0, 16, dtype)
        A["k_cand"], A["v_cand"] = extra(fresh["k_cand"]), extra(fresh["v_cand"])
        A["best"], A["n_acc"] = fresh["best"], fresh["n_acc"]
        G = _kv_dev(A, dtype)
        say("kv commit layers", dtype, L, rnd)
        fg = api.kv_commit(G["k_cand"], G["v_cand"], G["best"], G["n_acc"], G["k_pool"],
                           G["v_pool"], G["page_table"], G["prefix_len"], G["free_list"],
                           G["n_free"], W, D)
        k, v, pt, P, fl, nf, fo = oracle.kv_commit_layers(
            A["k_pool"], A["v_pool"], A["page_table"], A["prefix_len"], A["free_list"],
            A["n_free"], A["k_cand"], A["v_cand"], A["best"], A["n_acc"], W, D)
        A.update(k_pool=k, v_pool=v, page_table=pt, prefix_len=P, free_list=fl, n_free=nf)
        _kv_check(G, A, tensor_np(fg), fo)
        assert (A["prefix_len"] > 0).any()
        cut = (A["prefix_len"] // 2).astype(np.int32)
        say("kv truncate layers", dtype, L, rnd)
        fg = api.kv_truncate(to_dev(cut), G["page_table"], G["prefix_len"], G["free_list"],
                             G["n_free"], A["k_pool"].shape[1])
        pt, P, fl, nf, fo = oracle.kv_truncate(A["page_table"], A["prefix_len"], cut,
                                               A["free_list"], A["n_free"], A["k_pool"].shape[1])
        A.update(page_table=pt, prefix_len=P, free_list=fl, n_free=nf)
        _kv_check(G, A, tensor_np(fg), fo)
        torch.cuda.synchronize()


@pytest.mark.parametrize("dtype,P", [("bf16", 300), ("bf16", 4096), ("f32", 77)])
def test_kv_pack_token_major(dtype, P):
    """A contiguous token-major cache [P, Hkv, hd] packed into the verify step's pages
    equals the same data rearranged on the host (bit for bit, zero tail), and verify
    attention over it with the identity page table matches the oracle on that data."""
    import torch
    api = _api()
    Hkv, hd = (8, 128) if dtype == "bf16" else (2, 64)
    Hq = 4 * Hkv
    rng = np.random.default_rng(31 + P)
    if dtype == "bf16":
        k_tm = wl.f32_to_bf16_bits(rng.standard_normal((P, Hkv, hd)).astype(np.float32))
        v_tm = wl.f32_to_bf16_bits(rng.standard_normal((P, Hkv, hd)).astype(np.float32))
    else:
        k_tm = rng.standard_normal((P, Hkv, hd)).astype(np.float32)
        v_tm = rng.standard_normal((P, Hkv, hd)).astype(np.float32)
    n_pages = (P + 15) // 16
    pad = np.zeros((n_pages * 16 - P, Hkv, hd), dtype=k_tm.dtype)
    kp = np.concatenate([k_tm, pad]).reshape(n_pages, 16, Hkv, hd)
    vp = np.concatenate([v_tm, pad]).reshape(n_pages, 16, Hkv, hd)
    k_ref = np.ascontiguousarray(kp.transpose(0, 2, 1, 3))     # [page, head, 16, hd]
    v_ref = np.ascontiguousarray(vp.transpose(0, 2, 3, 1))     # [page, head, hd, 16]
    bf = dtype == "bf16"
    say("kv pack token-major", dtype, P)
    gk, gv = api.kv_pack_pages(to_dev(k_tm, bf16=bf), to_dev(v_tm, bf16=bf))
    torch.cuda.synchronize()
    as_bits = lambda t: t.view(torch.int16).cpu().numpy().view(np.uint16) if bf else t.cpu().numpy()
    assert np.array_equal(as_bits(gk), k_ref) and np.array_equal(as_bits(gv), v_ref)
    # attention over the packed cache (identity page table) against the oracle
    W, D = 2, 5
    M = W * D
    mk = (lambda sh_: wl.f32_to_bf16_bits(rng.standard_normal(sh_).astype(np.float32))) if bf else \
        (lambda sh_: rng.standard_normal(sh_).astype(np.float32))
    q, kc, vc = mk((M, Hq, hd)), mk((M, Hkv, hd)), mk((M, Hkv, hd))
    pt = np.arange(n_pages, dtype=np.int32)[None, :]
    pl = np.array([P], dtype=np.int32)
    out, fl = api.verify_attention(to_dev(q, bf16=bf), to_dev(kc, bf16=bf), to_dev(vc, bf16=bf),
                                   gk, gv, to_dev(pt), to_dev(pl), W, D)
    f = lambda x: oracle.as_f64(x, dtype)
    _, o_r, _ = oracle.verify_attention(f(q), f(kc), f(vc), f(k_ref), f(v_ref), pt, pl, 1, W, D,
                                        Hq, Hkv, out_dtype=dtype)
    err = rel_err(tensor_np(out), o_r)
    print(f"rel_err={err:.3e}")
    assert err <= (TOL if bf else 1e-5)


def test_kv_bad_stack_count():
    """A free-stack count outside [0, n_pool_pages] is not read from: every request is
    refused, as in the oracle."""
    api = _api()
    B, W, D = 3, 2, 4
    A = wl.make_kv_case(7, B, W, D, 2, 64, [3, 20, 0], n_spare=4, max_pages=6, dtype="f32")
    A["best"][:] = [0, 1, 0]
    A["n_acc"][:] = [4, 4, 0]
    for nf in (-1, A["k_pool"].shape[0] + 1):
        A2 = dict(A, n_free=nf)
        G = _kv_dev(A2, "f32")
        say("kv bad stack", nf)
        fg = api.kv_commit(G["k_cand"], G["v_cand"], G["best"], G["n_acc"], G["k_pool"],
                           G["v_pool"], G["page_table"], G["prefix_len"], G["free_list"],
                           G["n_free"], W, D)
        k, v, pt, P, fl, n2, fo = oracle.kv_commit(
            A2["k_pool"], A2["v_pool"], A2["page_table"], A2["prefix_len"], A2["free_list"], nf,
            A2["k_cand"], A2["v_cand"], A2["best"], A2["n_acc"], W, D)
        _kv_check(G, dict(A2, k_pool=k, v_pool=v, page_table=pt, prefix_len=P, free_list=fl,
                          n_free=n2), tensor_np(fg), fo)
        fg = api.kv_truncate(to_dev(np.zeros(B, np.int32)), G["page_table"], G["prefix_len"],
                             G["free_list"], G["n_free"], A["k_pool"].shape[0])
        assert (tensor_np(fg) == oracle.FLAG_BAD_PAGE).all()
        assert int(tensor_np(G["n_free"])[0]) == nf


def test_kv_commit_ragged_batch_full_size():
    """The batched ragged shape (32 sequences, 4 x 8 candidates, 8 KV heads of 128, 16-token
    pages in random order, prefixes 512..2048): one commit of the accepted runs and one
    rollback to the old lengths, against the oracle; the rollback restores the stack's
    page set and the page tables."""
    api = _api()
    rng = np.random.default_rng(77)
    B, W, D = 32, 4, 8
    prefix = rng.integers(512, 2049, size=B)
    A = wl.make_kv_case(8, B, W, D, 8, 128, prefix, n_spare=64, max_pages=160)
    G = _kv_dev(A, "bf16")
    say("kv commit ragged")
    fg = api.kv_commit(G["k_cand"], G["v_cand"], G["best"], G["n_acc"], G["k_pool"], G["v_pool"],
                       G["page_table"], G["prefix_len"], G["free_list"], G["n_free"], W, D)
    k, v, pt, P, fl, nf, fo = oracle.kv_commit(
        A["k_pool"], A["v_pool"], A["page_table"], A["prefix_len"], A["free_list"], A["n_free"],
        A["k_cand"], A["v_cand"], A["best"], A["n_acc"], W, D)
    C = dict(A, k_pool=k, v_pool=v, page_table=pt, prefix_len=P, free_list=fl, n_free=nf)
    _kv_check(G, C, tensor_np(fg), fo)
    say("kv truncate ragged")
    fg = api.kv_truncate(to_dev(A["prefix_len"]), G["page_table"], G["prefix_len"],
                         G["free_list"], G["n_free"], A["k_pool"].shape[0])
    H = _kv_host(G)
    assert not tensor_np(fg).any()
    assert np.array_equal(H["page_table"], A["page_table"])
    assert np.array_equal(H["prefix_len"], A["prefix_len"])
    assert sorted(H["free_list"][:H["n_free"]]) == sorted(A["free_list"][:A["n_free"]])


# =============================================================================== whole step

def _step_inputs(case, T, external=None):
    sh = case.shape
    keys = {"ctx", "ctx_off", "probe_h", "probe_w", "q", "k_cand", "v_cand", "k_pool", "v_pool",
            "page_table", "prefix_len", "w_full", "root_logits", "q_draft", "u_acc", "u_res"}
    I = case_to_dev(case, keys)
    if external is not None:
        I["cand_tok"] = to_dev(external[0])
        I["cand_len"] = to_dev(external[1])
    return I


def _check_step(case, g, o, external=False):
    """Stage outputs against the oracle's step; returns (compared, excluded) sequences
    of the bit-exact sampler comparison.  The sampler sides start from their own logits
    (an oracle input never comes from the GPU).  Their logits differ where the two
    attention outputs round to neighbouring bf16 values (one ulp of O moves a logit by
    about |w| 2^-8 |h|: ~1e-5 at d = 4096, ~1e-4 at d = 1024), which is the size of the
    acceptance tie band (1e-4 relative on p, i.e. on z/T - lse); the differences are
    printed with the oracle's decision margins and bounded at 2e-4."""
    sh = case.shape
    if not external:
        for k in ("cand_tok", "cand_len", "cand_pos", "n_found"):
            assert np.array_equal(tensor_np(g[k]), o["copy"][k]), k
        ok = o["probe"]["flags"] == 0
        assert np.array_equal(tensor_np(g["gate"])[ok], o["gate"][ok])
    ga = tensor_np(g["attn_out"])
    e_attn = rel_err(ga, o["attn"].reshape(ga.shape))
    gl = tensor_np(g["logits"])
    e_logits = rel_err(gl, o["logits"])
    dz = float(np.abs(gl.astype(np.float64) - o["logits"].astype(np.float64)).max())
    dlse = float(np.abs(tensor_np(g["row_lse"]) - o["lse"]).max())
    print(f"attn rel_err={e_attn:.3e} logits rel_err={e_logits:.3e} "
          f"max|dz|={dz:.2e} max|dlse|={dlse:.2e}")
    assert e_attn <= TOL and e_logits <= TOL
    assert dz / sh.temperature <= 2e-4 and dlse <= 2e-4
    n_cmp, n_exc = compare_sampler({k: g[k] for k in ("n_acc", "best", "out_tok", "n_out",
                                                      "acc_per_cand", "flags")},
                                   o["sample"], sh.B)
    return n_cmp, n_exc


def _assert_compared(name, B, n_cmp, n_exc, o_sample=None, gpu=None):
    """Every sequence of a small batch is compared (a seed whose decision is a flagged
    near tie is replaced by another in the test, never excluded); a batch may exclude
    at most one in sixteen."""
    msg = f"{name}: compared {n_cmp}/{B}, excluded {n_exc}"
    if o_sample is not None and "accept_margin" in o_sample:
        msg += (f"; min accept margin {float(np.min(o_sample['accept_margin'])):.2e}, "
                f"min cdf margin {float(np.min(o_sample['cdf_margin'])):.2e}")
    if gpu is not None:
        na = tensor_np(gpu["n_acc"])
        msg += f"; n_acc {na.tolist() if B <= 4 else (int(na.min()), int(na.max()))}"
    print(msg)
    if B <= 2:
        assert n_cmp == B, msg
    else:
        assert n_exc <= max(1, B // 16) and n_cmp >= B - max(1, B // 16), msg


@pytest.mark.parametrize("name", ["tiny", "small", "llama8b", "llama70b", "ragged"])
def test_verify_step_end_to_end(name):
    api = _api()
    if name == "tiny":
        sh, seed = wl.config(1), 1000
    elif name == "small":
        sh, seed = small_shape(B=3, P=(300, 777, 64)), 11
    elif name == "llama8b":
        sh, seed = wl.config(2), 2000
    elif name == "llama70b":
        sh, seed = wl.config(4), 4000
    else:
        sh, seed = wl.config(5), 5000
    case = get_case(("step", name), lambda: wl.make_case(sh, seed))
    I = _step_inputs(case, sh.temperature)
    say("verify_step", name)
    step = api.VerifyStep(I, B=sh.B, W=sh.W, D=sh.D, Hq=sh.Hq, Hkv=sh.Hkv, hd=sh.hd, V=sh.V,
                          tau=sh.tau, temperature=sh.temperature, kappa=sh.kappa)
    g = step()
    o = oracle.verify_step(case.arrays, sh)
    n_cmp, n_exc = _check_step(case, g, o)
    _assert_compared(f"step {name}", sh.B, n_cmp, n_exc, o["sample"], g)


@pytest.mark.parametrize("name,L", [("small", 3), ("llama8b", 32)])
def test_verify_step_layers(name, L):
    """A step whose attention covers L layers in one launch (shared block table): every
    layer's output against the oracle (all of them for the small shape, three for
    Llama-8B), and the head and sampler, which read the last layer, against the
    oracle's step on a case whose attention tensors are that layer's."""
    api = _api()
    if name == "small":
        sh, seed = small_shape(B=3, P=(300, 777, 64)), 11
    else:
        sh, seed = wl.config(2), 2000
    case = get_case(("step", name), lambda: wl.make_case(sh, seed))
    LI = wl.layer_inputs(case, L, 99)
    I = _step_inputs(case, sh.temperature)
    I.update(_layers_dev(LI, sh.dtype == "bf16"))
    say("verify_step layers", name, L)
    step = api.VerifyStep(I, B=sh.B, W=sh.W, D=sh.D, Hq=sh.Hq, Hkv=sh.Hkv, hd=sh.hd, V=sh.V,
                          tau=sh.tau, temperature=sh.temperature, kappa=sh.kappa)
    g = step()
    ga = tensor_np(g["attn_out"])
    assert ga.shape[0] == L
    for l in (range(L) if L <= 4 else (0, 13, L - 1)):
        f = lambda k: oracle.as_f64(LI[k][l], sh.dtype)
        _, o_r, _ = oracle.verify_attention(f("q"), f("k_cand"), f("v_cand"), f("k_pool"),
                                            f("v_pool"), case.arrays["page_table"],
                                            case.arrays["prefix_len"], sh.B, sh.W, sh.D, sh.Hq,
                                            sh.Hkv, out_dtype=sh.dtype)
        err = rel_err(ga[l], o_r)
        print(f"layer {l}: rel_err={err:.3e}")
        assert err <= TOL
    last = wl.Case(shape=case.shape, variant=case.variant, seed=case.seed,
                   arrays={**case.arrays, **{k: LI[k][L - 1] for k in LI}}, meta=case.meta)
    o = oracle.verify_step(last.arrays, sh)
    g_last = dict(g)
    g_last["attn_out"] = g["attn_out"][L - 1]
    n_cmp, n_exc = _check_step(last, g_last, o)
    _assert_compared(f"step layers {name}", sh.B, n_cmp, n_exc, o["sample"], g)


@pytest.mark.parametrize("name", ["small", "llama8b", "ragged"])
def test_verify_step_multi(name):
    """The whole step with multi-candidate acceptance of the copy candidates (point-mass
    drafts: the case's dense q is not passed) against the oracle's step."""
    api = _api()
    if name == "small":
        sh, seed = small_shape(B=3, P=(300, 777, 64)), 11
    elif name == "llama8b":
        sh, seed = wl.config(2), 2000
    else:
        sh, seed = wl.config(5), 5000
    case = get_case(("step", name), lambda: wl.make_case(sh, seed))
    I = _step_inputs(case, sh.temperature)
    I["q_draft"] = None
    say("verify_step multi", name)
    step = api.VerifyStep(I, B=sh.B, W=sh.W, D=sh.D, Hq=sh.Hq, Hkv=sh.Hkv, hd=sh.hd, V=sh.V,
                          tau=sh.tau, temperature=sh.temperature, kappa=sh.kappa,
                          accept="multi")
    g = step()
    A = {k: v for k, v in case.arrays.items() if k != "q_draft"}
    o = oracle.verify_step(A, sh, accept="multi")
    n_cmp, n_exc = _check_step(case, g, o)
    _assert_compared(f"step multi {name}", sh.B, n_cmp, n_exc, gpu=g)


@pytest.mark.parametrize("name", ["small", "llama8b"])
def test_verify_step_multi_dense(name):
    """The whole step with multi-candidate acceptance over the workload's own dense
    draft distributions (N(0, 2^2) draft logits at V = 128,256 for the Llama-8B shape)."""
    api = _api()
    if name == "small":
        sh, seed = small_shape(B=3, P=(300, 777, 64)), 11
    else:
        sh, seed = wl.config(2), 2000
    case = get_case(("step", name), lambda: wl.make_case(sh, seed))
    I = _step_inputs(case, sh.temperature)
    say("verify_step multi dense", name)
    step = api.VerifyStep(I, B=sh.B, W=sh.W, D=sh.D, Hq=sh.Hq, Hkv=sh.Hkv, hd=sh.hd, V=sh.V,
                          tau=sh.tau, temperature=sh.temperature, kappa=sh.kappa,
                          accept="multi")
    g = step()
    o = oracle.verify_step(case.arrays, sh, accept="multi")
    n_cmp, n_exc = _check_step(case, g, o)
    _assert_compared(f"step multi dense {name}", sh.B, n_cmp, n_exc, o["sample"], g)


@pytest.mark.parametrize("name", ["small", "llama8b", "ragged"])
def test_verify_step_greedy(name):
    """The whole step with greedy verification (no uniforms, no draft distribution)
    against the oracle's step; sequences whose decisions are near ties are left out."""
    api = _api()
    if name == "small":
        sh, seed = small_shape(B=3, P=(300, 777, 64)), 11
    elif name == "llama8b":
        sh, seed = wl.config(2), 2000
    else:
        sh, seed = wl.config(5), 5000
    case = get_case(("step", name), lambda: wl.make_case(sh, seed))
    I = _step_inputs(case, sh.temperature)
    for k in ("q_draft", "u_acc", "u_res"):
        I[k] = None
    say("verify_step greedy", name)
    step = api.VerifyStep(I, B=sh.B, W=sh.W, D=sh.D, Hq=sh.Hq, Hkv=sh.Hkv, hd=sh.hd, V=sh.V,
                          tau=sh.tau, temperature=sh.temperature, kappa=sh.kappa,
                          accept="greedy")
    g = step()
    o = oracle.verify_step(case.arrays, sh, accept="greedy")
    n_cmp, n_exc = _check_step(case, g, o)
    _assert_compared(f"step greedy {name}", sh.B, n_cmp, n_exc, gpu=g)


def _ragged_mixed_case():
    """The 32-sequence ragged batch with its gating mixed sequence by sequence: from
    the forced-open inputs, sequences 0 mod 4 get their probe input negated (gate
    closed), 1 mod 4 keep 1 .. W-1 of their W planted occurrences of the current
    kappa-gram (the others broken by changing their last token), 2 mod 4 keep none,
    and 3 mod 4 stay as they are.  Both sides receive the modified arrays."""
    sh = wl.config(5)
    case = wl.make_case(sh, 5000, "measure")
    A = case.arrays
    off = A["ctx_off"]
    for b in range(sh.B):
        ends = case.meta["forced_ends"][b]
        if b % 4 == 0:
            A["probe_h"][b] ^= np.uint16(0x8000)          # w.h < 0: sigma < tau
        elif b % 4 in (1, 2):
            keep = (1 + b // 4) % sh.W if b % 4 == 1 else 0
            for j in ends[keep:]:
                k = off[b] + j
                A["ctx"][k] = (A["ctx"][k] + 1) % sh.V
    return case


@pytest.mark.parametrize("accept", ["longest", "multi", "greedy"])
def test_verify_step_ragged_mixed_gating(accept):
    """One batched step in which closed gates, sequences with fewer than W candidates
    and sequences with none meet (the ragged batch's correctness variant)."""
    api = _api()
    sh = wl.config(5)
    case = get_case(("step", "ragged_mixed"), _ragged_mixed_case)
    A = case.arrays
    I = _step_inputs(case, sh.temperature)
    if accept != "longest":
        I["q_draft"] = None
    if accept == "greedy":
        I["u_acc"] = I["u_res"] = None
    say("verify_step ragged mixed gating", accept)
    step = api.VerifyStep(I, B=sh.B, W=sh.W, D=sh.D, Hq=sh.Hq, Hkv=sh.Hkv, hd=sh.hd, V=sh.V,
                          tau=sh.tau, temperature=sh.temperature, kappa=sh.kappa, accept=accept)
    g = step()
    o = oracle.verify_step(A, sh, accept=accept)
    gates = o["gate"]
    nf = o["copy"]["n_found"]
    print(f"gates open {int(gates.sum())}/{sh.B}, n_found histogram "
          f"{np.bincount(nf, minlength=sh.W + 1).tolist()}")
    assert (gates == 0).any() and (gates == 1).any()
    assert ((nf > 0) & (nf < sh.W)).any() and (nf == 0).any()
    n_cmp, n_exc = _check_step(case, g, o)
    _assert_compared(f"step ragged mixed {accept}", sh.B, n_cmp, n_exc, gpu=g)
    fl = tensor_np(g["flags"])
    assert (fl[gates == 0] & oracle.FLAG_NO_CANDIDATE).all()


def test_verify_step_dense_rejection_mid_run():
    """Dense draft distributions at the full vocabulary (V = 128,256, Llama-8B shapes)
    with rejections inside the runs (0 < accepted < length): each candidate token's
    draft probability is set to a seeded multiple (1.2 to 3) of its target probability
    under the oracle's logits, so each test accepts with probability 1/multiple and the
    residual max(0, p - q) over the whole vocabulary is drawn from."""
    api = _api()
    sh = wl.config(2)
    case = get_case(("step", "llama8b"), lambda: wl.make_case(sh, 2000))
    A = dict(case.arrays)
    o0 = oracle.verify_step(A, sh)
    z = o0["logits"].astype(np.float64) / sh.temperature
    lse = o0["lse"]
    root = A["root_logits"].astype(np.float64) / sh.temperature
    root_lse = scipy.special.logsumexp(root, axis=1)
    q = A["q_draft"].copy()
    rng = np.random.default_rng(77)
    ct, cl = o0["cand_tok"], o0["cand_len"]
    M = sh.M
    for i in range(sh.W):
        for oo in range(int(cl[0, i])):
            x = int(ct[0, i, oo])
            p = np.exp(root[0, x] - root_lse[0]) if oo == 0 else np.exp(z[i * sh.D + oo - 1, x] - lse[i * sh.D + oo - 1])
            row = q[i * sh.D + oo].astype(np.float64)
            qx = min(0.5, float(p) * rng.uniform(1.2, 3.0))
            rest = row.sum() - row[x]
            row *= (1.0 - qx) / rest
            row[x] = qx
            q[i * sh.D + oo] = row.astype(np.float32)
    A["q_draft"] = q
    case2 = wl.Case(shape=sh, variant=case.variant, seed=case.seed, arrays=A, meta=case.meta)
    I = _step_inputs(case2, sh.temperature)
    say("verify_step dense rejection mid-run")
    g = api.VerifyStep(I, B=1, W=sh.W, D=sh.D, Hq=sh.Hq, Hkv=sh.Hkv, hd=sh.hd, V=sh.V,
                       tau=sh.tau, temperature=sh.temperature, kappa=sh.kappa)()
    o = oracle.verify_step(A, sh)
    n_cmp, n_exc = _check_step(case2, g, o)
    _assert_compared("step dense mid-run", 1, n_cmp, n_exc, o["sample"], g)
    a = int(o["sample"]["n_acc"][0])
    best = int(o["sample"]["best"][0])
    assert 0 < a < int(cl[0, best]), (a, cl[0].tolist())


def test_verify_step_external_drafts_slimspec():
    """Neural-draft path: the SlimSpec low-rank head makes q for gamma=7 drafts, the
    drafts are sampled from the oracle's q by inverse CDF (the drafter's job), then
    the step verifies them with W=1."""
    api = _api()
    sh = wl.config(3)
    case = get_case(("slim_step",), lambda: wl.make_case(sh, 3000))
    A = case.arrays
    z, l, _ = oracle.lm_head_lowrank(oracle.as_f64(A["draft_h"], "bf16"), A["w_down"], A["w_up"])
    q = oracle.head_softmax(z, l).astype(np.float32)              # [gamma, V]
    drafts = np.zeros((1, 1, sh.D), dtype=np.int32)
    for o_ in range(sh.D):
        c = np.cumsum(q[o_].astype(np.float64))
        drafts[0, 0, o_] = min(int(np.searchsorted(c, A["u_draft"][0, 0, o_] * c[-1], "right")),
                               sh.V - 1)
    lens = np.array([[sh.D]], dtype=np.int32)
    A2 = dict(A)
    A2["q_draft"] = q
    case.arrays = A2
    I = _step_inputs(case, 1.0, external=(drafts, lens))
    say("verify_step slimspec external drafts")
    step = api.VerifyStep(I, B=1, W=1, D=sh.D, Hq=sh.Hq, Hkv=sh.Hkv, hd=sh.hd, V=sh.V,
                          external_drafts=True)
    g = step()
    o = oracle.verify_step(A2, sh, drafts=(drafts, lens))
    n_cmp, n_exc = _check_step(case, g, o, external=True)
    _assert_compared("step slimspec", 1, n_cmp, n_exc, o["sample"], g)


def test_verify_step_equals_its_calls():
    """The fused step gives the same bits as its five calls made one by one."""
    api = _api()
    sh = small_shape(B=3, P=(300, 777, 64))
    case = get_case(("step", "small"), lambda: wl.make_case(sh, 11))
    I = _step_inputs(case, 1.0)
    say("verify_step vs calls")
    g = api.VerifyStep(I, B=sh.B, W=sh.W, D=sh.D, Hq=sh.Hq, Hkv=sh.Hkv, hd=sh.hd, V=sh.V)()
    cm = api.copy_match(I["ctx"], I["ctx_off"], 5, sh.W, sh.D)
    pg = api.probe_gate(I["probe_h"], I["probe_w"], 0.4, cm["n_found"])
    att, _ = api.verify_attention(I["q"], I["k_cand"], I["v_cand"], I["k_pool"], I["v_pool"],
                                  I["page_table"], I["prefix_len"], sh.W, sh.D)
    lg, lse, _ = api.lm_head(att.reshape(att.shape[0], -1), w_full=I["w_full"])
    rs = api.reject_sample(I["root_logits"], lg, lse, I["q_draft"], cm["cand_tok"],
                           cm["cand_len"], I["u_acc"], I["u_res"], 1.0, pg["gate"])
    for k in ("cand_tok", "cand_len", "cand_pos", "n_found"):
        assert np.array_equal(tensor_np(g[k]), tensor_np(cm[k])), k
    assert np.array_equal(tensor_np(g["gate"]), tensor_np(pg["gate"]))
    assert np.array_equal(tensor_np(g["attn_out"]), tensor_np(att))
    assert np.array_equal(tensor_np(g["logits"]), tensor_np(lg))
    assert np.array_equal(tensor_np(g["row_lse"]), tensor_np(lse))
    for k in ("n_acc", "best", "out_tok", "n_out", "acc_per_cand"):
        assert np.array_equal(tensor_np(g[k]), tensor_np(rs[k])), k


def test_verify_step_overlap_and_flag_reset():
    """Retrieval on the auxiliary stream gives the same bits as the serial step; a bad
    page raised inside attention reaches `flags` on every call (the workspace word it
    goes through is reset by the sampler), and only for the sequence that has it."""
    api = _api()
    sh = small_shape(B=2, P=(64, 64), paged_random=False)
    case = get_case(("step", "badpage"), lambda: wl.make_case(sh, 13))
    case.arrays["page_table"][1, 2] = 10 ** 6
    I = _step_inputs(case, 1.0)
    say("verify_step overlap vs serial, bad page")
    kw = dict(B=sh.B, W=sh.W, D=sh.D, Hq=sh.Hq, Hkv=sh.Hkv, hd=sh.hd, V=sh.V)
    serial = api.VerifyStep(I, overlap=False, **kw)
    over = api.VerifyStep(I, overlap=True, **kw)
    ref = None
    for step in (serial, over, serial, over):
        g = step()
        got = {k: tensor_np(v).copy() for k, v in g.items()}
        assert got["flags"][1] & oracle.FLAG_BAD_PAGE and not got["flags"][0] & oracle.FLAG_BAD_PAGE
        if ref is None:
            ref = got
        for k in ref:
            assert np.array_equal(got[k], ref[k]), k
