"""Pins for the oracle's block-triangular verify attention (CPU only).

SwitchSD summary (onedev.kr/papers/87), 'How it differs': every candidate token
attends to the whole prefix and to the earlier tokens of its own candidate, and
is isolated from the other candidates, so W hypotheses are verified in one pass.
The pins: (1) the block-triangular result equals running each candidate on its
own through ordinary causal attention over [prefix | candidate] (computed here
with torch's scaled_dot_product_attention in fp64, a library routine, with an
explicit causal mask); (2)-(6) special cases with closed forms.
"""
import numpy as np
import pytest
import torch

import oracle


def _rand_case(rng, B, W, D, Hq, Hkv, hd, P, page=16, shuffle=True):
    M = W * D
    maxp = max(-(-p // page) for p in P) if P else 1
    pages = [-(-p // page) for p in P]
    n_pages = max(1, sum(pages))
    q = rng.standard_normal((B * M, Hq, hd))
    kc = rng.standard_normal((B * M, Hkv, hd))
    vc = rng.standard_normal((B * M, Hkv, hd))
    kp = rng.standard_normal((n_pages, Hkv, page, hd))          # K pages: token rows
    vp = rng.standard_normal((n_pages, Hkv, hd, page))          # V pages: transposed
    perm = rng.permutation(n_pages) if shuffle else np.arange(n_pages)
    pt = np.full((B, max(maxp, 1)), -1, dtype=np.int32)
    o = 0
    for b in range(B):
        pt[b, :pages[b]] = perm[o:o + pages[b]]
        o += pages[b]
    return q, kc, vc, kp, vp, pt, np.asarray(P, dtype=np.int32)


def _contiguous_prefix(pool, pt, b, P, page=16, kind="k"):
    """Prefix rows [P, Hkv, hd] read element by element from the paged layout."""
    Hkv = pool.shape[1]
    hd = pool.shape[3] if kind == "k" else pool.shape[2]
    out = np.zeros((P, Hkv, hd))
    for pos in range(P):
        pg, off = pt[b, pos // page], pos % page
        for h in range(Hkv):
            out[pos, h] = pool[pg, h, off, :] if kind == "k" else pool[pg, h, :, off]
    return out


def causal_per_candidate(q, kc, vc, kp, vp, pt, plen, B, W, D, Hq, Hkv):
    """Each candidate alone: sequence = prefix followed by candidate i; causal
    attention over it (position p sees keys 0..p); keep the candidate rows."""
    M = W * D
    hd = q.shape[-1]
    g = Hq // Hkv
    out = np.zeros_like(q)
    for b in range(B):
        P = int(plen[b])
        Kp = _contiguous_prefix(kp, pt, b, P, kind="k")
        Vp = _contiguous_prefix(vp, pt, b, P, kind="v")
        for i in range(W):
            rows = slice(b * M + i * D, b * M + (i + 1) * D)
            K = np.concatenate([Kp, kc[rows]], axis=0)            # [P+D, Hkv, hd]
            Vv = np.concatenate([Vp, vc[rows]], axis=0)
            n = P + D
            mask = torch.tril(torch.ones(n, n, dtype=torch.bool))[P:]   # rows P..P+D-1
            for hq in range(Hq):
                kv = hq // g
                Qt = torch.from_numpy(q[rows, hq, :]).reshape(1, 1, D, hd)
                Kt = torch.from_numpy(np.ascontiguousarray(K[:, kv, :])).reshape(1, 1, n, hd)
                Vt = torch.from_numpy(np.ascontiguousarray(Vv[:, kv, :])).reshape(1, 1, n, hd)
                o = torch.nn.functional.scaled_dot_product_attention(Qt, Kt, Vt, attn_mask=mask)
                out[rows, hq, :] = o.reshape(D, hd).numpy()
    return out


@pytest.mark.parametrize("B,W,D,Hq,Hkv,hd,P", [
    (1, 2, 4, 4, 2, 16, (128,)),        # the tiny workload's shape
    (2, 3, 5, 6, 3, 8, (37, 50)),       # ragged prefixes, partial last pages
    (3, 4, 3, 4, 4, 8, (16, 0, 33)),    # MHA (g=1), an empty prefix
    (1, 1, 6, 8, 1, 4, (20,)),          # W=1, MQA
])
def test_equals_per_candidate_causal(B, W, D, Hq, Hkv, hd, P):
    rng = np.random.default_rng(sum(P) + 7 * W + D)
    q, kc, vc, kp, vp, pt, plen = _rand_case(rng, B, W, D, Hq, Hkv, hd, P)
    O, _, fl = oracle.verify_attention(q, kc, vc, kp, vp, pt, plen, B, W, D, Hq, Hkv,
                                       out_dtype="f32")
    ref = causal_per_candidate(q, kc, vc, kp, vp, pt, plen, B, W, D, Hq, Hkv)
    assert np.abs(O - ref).max() < 1e-12
    assert (fl == 0).all()


def test_zero_query_gives_mean_of_visible_values():
    rng = np.random.default_rng(1)
    B, W, D, Hq, Hkv, hd, P = 1, 2, 3, 2, 1, 4, (21,)
    q, kc, vc, kp, vp, pt, plen = _rand_case(rng, B, W, D, Hq, Hkv, hd, P)
    q[:] = 0.0
    O, _, _ = oracle.verify_attention(q, kc, vc, kp, vp, pt, plen, B, W, D, Hq, Hkv)
    Vp = _contiguous_prefix(vp, pt, 0, 21, kind="v")[:, 0, :]
    for i in range(W):
        for o in range(D):
            vis = np.concatenate([Vp, vc[i * D:i * D + o + 1, 0, :]])
            assert np.abs(O[i * D + o, 0] - vis.mean(axis=0)).max() < 1e-13


def test_constant_values_pass_through():
    rng = np.random.default_rng(2)
    B, W, D, Hq, Hkv, hd, P = 2, 2, 2, 4, 2, 8, (5, 40)
    q, kc, vc, kp, vp, pt, plen = _rand_case(rng, B, W, D, Hq, Hkv, hd, P)
    c = rng.standard_normal(hd)
    vc[:] = c
    vp[:] = c[None, None, :, None]                          # V pages hold hd on axis 2
    O, _, _ = oracle.verify_attention(q, kc, vc, kp, vp, pt, plen, B, W, D, Hq, Hkv)
    assert np.abs(O - c).max() < 1e-13


def test_no_prefix_single_candidate_is_causal_attention():
    rng = np.random.default_rng(3)
    D, hd = 7, 8
    q, kc, vc, kp, vp, pt, plen = _rand_case(rng, 1, 1, D, 1, 1, hd, (0,))
    O, _, _ = oracle.verify_attention(q, kc, vc, kp, vp, pt, plen, 1, 1, D, 1, 1)
    Qt = torch.from_numpy(q[:, 0, :]).reshape(1, 1, D, hd)
    Kt = torch.from_numpy(kc[:, 0, :]).reshape(1, 1, D, hd)
    Vt = torch.from_numpy(vc[:, 0, :]).reshape(1, 1, D, hd)
    ref = torch.nn.functional.scaled_dot_product_attention(Qt, Kt, Vt, is_causal=True)
    assert np.abs(O[:, 0, :] - ref.reshape(D, hd).numpy()).max() < 1e-12


def test_single_token_candidates_are_decode_attention():
    """D=1: each row sees the prefix and itself only."""
    rng = np.random.default_rng(4)
    W, hd, P = 3, 8, (30,)
    q, kc, vc, kp, vp, pt, plen = _rand_case(rng, 1, W, 1, 2, 1, hd, P)
    O, _, _ = oracle.verify_attention(q, kc, vc, kp, vp, pt, plen, 1, W, 1, 2, 1)
    Kp = _contiguous_prefix(kp, pt, 0, 30, kind="k")[:, 0, :]
    Vp = _contiguous_prefix(vp, pt, 0, 30, kind="v")[:, 0, :]
    for i in range(W):
        K = np.concatenate([Kp, kc[i:i + 1, 0, :]])
        Vv = np.concatenate([Vp, vc[i:i + 1, 0, :]])
        for hq in range(2):
            s = K @ q[i, hq] / np.sqrt(hd)
            a = np.exp(s - s.max())
            a /= a.sum()
            assert np.abs(O[i, hq] - a @ Vv).max() < 1e-12


def test_bf16_output_rounding_is_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -7, -3.0000001, 0.0])
    r = oracle.round_f64_to_bf16(x)
    # ties go to the even neighbour: 1+2^-8 -> 1, 1+3*2^-8 -> 1+2^-6
    assert r.tolist() == [1.0, 1.0, 1.0 + 2 ** -6, 1.0 + 2 ** -7, -3.0, 0.0]
    # every rounded value is a bf16 value: its low 16 fp32 bits are zero
    rng = np.random.default_rng(0)
    x = rng.standard_normal(1000)
    y = oracle.round_f64_to_bf16(x)
    assert (y.astype(np.float32).view(np.uint32) & 0xFFFF == 0).all()
    assert (np.abs(y - x) <= 2.0 ** -8 * np.abs(x)).all()      # half an ulp of 8 significant bits


def test_bad_page_is_flagged_and_masked():
    rng = np.random.default_rng(5)
    q, kc, vc, kp, vp, pt, plen = _rand_case(rng, 1, 1, 2, 1, 1, 4, (32,))
    pt[0, 1] = 999
    _, _, fl = oracle.verify_attention(q, kc, vc, kp, vp, pt, plen, 1, 1, 2, 1, 1)
    assert fl[0] & oracle.FLAG_BAD_PAGE


def test_layers_share_the_block_table():
    """Several layers over one block table [SD6: a paged cache per layer].  Layer 0 is
    a random layer pinned per candidate against causal attention (library routine);
    layer 1 has zero queries (mean of the visible values, read element by element
    from its own pool through the common table); layer 2 has constant values (they
    pass through); a page entry out of the pool is flagged once for the sequence
    and masked in every layer."""
    rng = np.random.default_rng(11)
    B, W, D, Hq, Hkv, hd, P = 2, 2, 3, 4, 2, 8, (37, 20)
    layers = [_rand_case(rng, B, W, D, Hq, Hkv, hd, P, shuffle=False) for _ in range(3)]
    pt, plen = layers[0][5], layers[0][6]
    q, kc, vc, kp, vp = (np.stack([L_[j] for L_ in layers]) for j in range(5))
    q[1] = 0.0
    c = rng.standard_normal(hd)
    vc[2] = c
    vp[2] = c[None, None, :, None]
    O, _, fl = oracle.verify_attention_layers(q, kc, vc, kp, vp, pt, plen, B, W, D, Hq, Hkv,
                                              out_dtype="f32")
    assert O.shape == (3,) + q.shape[1:] and (fl == 0).all()
    ref0 = causal_per_candidate(q[0], kc[0], vc[0], kp[0], vp[0], pt, plen, B, W, D, Hq, Hkv)
    assert np.abs(O[0] - ref0).max() < 1e-12
    M = W * D
    g = Hq // Hkv
    for b in range(B):
        Vp = _contiguous_prefix(vp[1], pt, b, int(plen[b]), kind="v")
        for i in range(W):
            for o in range(D):
                r = b * M + i * D + o
                for hq in range(Hq):
                    vis = np.concatenate([Vp[:, hq // g, :], vc[1, b * M + i * D:r + 1, hq // g, :]])
                    assert np.abs(O[1, r, hq] - vis.mean(axis=0)).max() < 1e-13
    assert np.abs(O[2] - c).max() < 1e-13
    # a bad page entry: flagged, and the same keys are dropped in every layer
    pt_bad = pt.copy()
    pt_bad[0, 1] = 10 ** 6
    Ob, _, fb = oracle.verify_attention_layers(q, kc, vc, kp, vp, pt_bad, plen, B, W, D, Hq,
                                               Hkv, out_dtype="f32")
    assert fb.tolist() == [oracle.FLAG_BAD_PAGE, 0]
    for l in range(3):
        keep = np.ones(int(plen[0]), dtype=bool)
        keep[16:32] = False
        Kp = _contiguous_prefix(kp[l], pt, 0, int(plen[0]), kind="k")[keep]
        Vp = _contiguous_prefix(vp[l], pt, 0, int(plen[0]), kind="v")[keep]
        r, hq = 2, 3                       # candidate 0, offset 2, query head 3
        K = np.concatenate([Kp[:, hq // g], kc[l, 0:3, hq // g]])
        Vv = np.concatenate([Vp[:, hq // g], vc[l, 0:3, hq // g]])
        s = K @ q[l, r, hq] / np.sqrt(hd)
        a = np.exp(s - s.max())
        a /= a.sum()
        assert np.abs(Ob[l, r, hq] - a @ Vv).max() < 1e-12
