"""Pins for the oracle's KV commit and rollback (CPU only).

Rejection-sampling blog (blog.huny.dev), section 6: after verification the KV
blocks of rejected tokens go back to the paged pool at once, and none may leak.
The commit appends the accepted rows; the rollback frees what lies past a new
length.  Pinned against a plain list-of-rows model of each sequence's cache and
against page conservation (every pool page is in exactly one page table or on the
free stack)."""
import numpy as np
import pytest

import oracle
from verification_step_amd import workloads as wl

PAGE = 16


def rows_of(A, b, P):
    """Token-major rows 0..P-1 of sequence b, through the page table."""
    kt = oracle.token_major(A["k_pool"], "k")
    vt = oracle.token_major(A["v_pool"], "v")
    k, vk = oracle.gather_prefix(kt, A["page_table"], b, P, PAGE)
    v, vv = oracle.gather_prefix(vt, A["page_table"], b, P, PAGE)
    assert vk.all() and vv.all()
    return k, v


def conserved(A, n_pages):
    pt, P = A["page_table"], A["prefix_len"]
    used = [int(pt[b, j]) for b in range(pt.shape[0]) for j in range((int(P[b]) + PAGE - 1) // PAGE)]
    free = [int(x) for x in A["free_list"][:A["n_free"]]]
    return sorted(used + free) == list(range(n_pages))


def commit(A, W, D):
    k, v, pt, P, fl, nf, flags = oracle.kv_commit(
        A["k_pool"], A["v_pool"], A["page_table"], A["prefix_len"], A["free_list"], A["n_free"],
        A["k_cand"], A["v_cand"], A["best"], A["n_acc"], W, D)
    B2 = dict(A)
    B2.update(k_pool=k, v_pool=v, page_table=pt, prefix_len=P, free_list=fl, n_free=nf)
    return B2, flags


def truncate(A, new_len):
    pt, P, fl, nf, flags = oracle.kv_truncate(A["page_table"], A["prefix_len"], new_len,
                                              A["free_list"], A["n_free"], A["k_pool"].shape[0])
    B2 = dict(A)
    B2.update(page_table=pt, prefix_len=P, free_list=fl, n_free=nf)
    return B2, flags


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_commit_matches_list_model_over_rounds(dtype):
    """Several rounds of commit (new candidates each round) and random rollbacks: each
    sequence's cache read through its page table equals a list model that appends
    the accepted candidate's rows and cuts at the rollback length."""
    B, W, D, Hkv, hd = 6, 3, 7, 2, 8
    A = wl.make_kv_case(3, B, W, D, Hkv, hd, [0, 1, 15, 16, 17, 40], n_spare=40, max_pages=12,
                        dtype=dtype)
    n_pages = A["k_pool"].shape[0]
    model = [list(zip(*rows_of(A, b, int(A["prefix_len"][b])))) for b in range(B)]
    rng = np.random.default_rng(9)
    for rnd in range(6):
        fresh = wl.make_kv_case(100 + rnd, B, W, D, Hkv, hd, [0] * B, 0, 12, dtype)
        A.update(k_cand=fresh["k_cand"], v_cand=fresh["v_cand"], best=fresh["best"],
                 n_acc=fresh["n_acc"])
        A, flags = commit(A, W, D)
        assert not flags.any()
        for b in range(B):
            i, a = int(A["best"][b]), int(A["n_acc"][b])
            if i >= 0:
                for o in range(a):
                    r = b * W * D + i * D + o
                    model[b].append((A["k_cand"][r], A["v_cand"][r]))
        assert conserved(A, n_pages)
        cut = np.array([rng.integers(0, int(p) + 1) if rng.random() < 0.4 else int(p)
                        for p in A["prefix_len"]], dtype=np.int32)
        A, flags = truncate(A, cut)
        assert not flags.any()
        for b in range(B):
            del model[b][int(cut[b]):]
        assert conserved(A, n_pages)
        for b in range(B):
            P = int(A["prefix_len"][b])
            assert P == len(model[b])
            if P:
                k, v = rows_of(A, b, P)
                assert np.array_equal(k, np.stack([r[0] for r in model[b]]))
                assert np.array_equal(v, np.stack([r[1] for r in model[b]]))
            # no page table entry past the length
            assert (A["page_table"][b, (P + PAGE - 1) // PAGE:] == -1).all()


def test_commit_page_boundaries_and_pop_order():
    """A prefix ending on a page boundary takes a new page for its first accepted row;
    one ending a row short of it fills it first; pages come off the top of the stack
    in sequence order."""
    B, W, D = 3, 1, 20
    A = wl.make_kv_case(4, B, W, D, 1, 4, [32, 31, 5], n_spare=5, max_pages=8, dtype="f32")
    A["best"][:] = 0
    A["n_acc"][:] = [1, 2, 12]
    top = [int(x) for x in A["free_list"][:5]][::-1]       # pop order
    C, flags = commit(A, W, D)
    assert not flags.any()
    assert C["page_table"][0, 2] == top[0]                   # 32 -> page 2 is new
    assert C["page_table"][1, 2] == top[1]                   # 31 + 2 spills into page 2
    assert C["page_table"][2, 1] == top[2]                   # 5 + 12 = 17: one new page
    assert (C["page_table"][2, 2:] == -1).all()
    assert C["n_free"] == 2 and list(C["prefix_len"]) == [33, 33, 17]
    # 5 + 11 = 16 rows fill the first page exactly: no page taken
    A["n_acc"][:] = [0, 0, 11]
    C, _ = commit(A, W, D)
    assert C["n_free"] == 5 and C["prefix_len"][2] == 16 and C["page_table"][2, 1] == -1


def test_commit_pool_exhaustion_and_bad_inputs():
    B, W, D = 5, 2, 40
    A = wl.make_kv_case(5, B, W, D, 1, 4, [16, 16, 16, 16, 120], n_spare=2, max_pages=8,
                        dtype="f32")
    A["best"][:] = [0, 1, 0, -1, 1]
    A["n_acc"][:] = [17, 20, 3, 5, 40]   # needs 2, 2, 1, -, (120 + 40 > 128: bad)
    C, flags = commit(A, W, D)
    # sequence 0 takes both free pages; 1 finds the stack empty; 2 needs one: empty too
    assert flags.tolist() == [0, oracle.FLAG_POOL_EMPTY, oracle.FLAG_POOL_EMPTY, 0,
                              oracle.FLAG_BAD_PAGE]
    assert list(C["prefix_len"]) == [33, 16, 16, 16, 120] and C["n_free"] == 0
    # a later sequence that fits still commits after an earlier one was refused
    A["n_acc"][:] = [40, 0, 3, 0, 0]            # 0 needs 3 pages (> 2): refused; 2 needs 1
    C, flags = commit(A, W, D)
    assert flags.tolist() == [oracle.FLAG_POOL_EMPTY, 0, 0, 0, 0]
    assert list(C["prefix_len"]) == [16, 16, 19, 16, 120] and C["n_free"] == 1
    # a free-stack entry that is not a pool page: the sequence is refused, nothing taken
    A["free_list"][1] = 10 ** 6
    A["n_acc"][:] = [17, 0, 0, 0, 0]
    C, flags = commit(A, W, D)
    assert flags[0] == oracle.FLAG_BAD_PAGE and C["n_free"] == 2 and C["prefix_len"][0] == 16


def test_truncate_round_trip_and_bad_lengths():
    B, W, D = 4, 2, 9
    A = wl.make_kv_case(6, B, W, D, 2, 8, [0, 16, 23, 64], n_spare=12, max_pages=10)
    A["best"][:] = [0, 1, 1, 0]
    A["n_acc"][:] = [9, 1, 9, 8]
    C, flags = commit(A, W, D)
    assert not flags.any()
    R, flags = truncate(C, A["prefix_len"])
    assert not flags.any()
    assert np.array_equal(R["prefix_len"], A["prefix_len"])
    assert R["n_free"] == A["n_free"]
    assert sorted(R["free_list"][:R["n_free"]]) == sorted(A["free_list"][:A["n_free"]])
    assert np.array_equal(R["page_table"], A["page_table"])
    # rollback to zero frees every page; a length above the current one is refused
    Z, flags = truncate(R, np.array([0, 0, 30, -1], np.int32))
    assert flags.tolist() == [0, 0, oracle.FLAG_BAD_PAGE, oracle.FLAG_BAD_PAGE]
    assert list(Z["prefix_len"]) == [0, 0, 23, 64]
    assert (Z["page_table"][:2] == -1).all()
    assert conserved(Z, A["k_pool"].shape[0])


def test_bad_stack_count_refuses_everything():
    B, W, D = 3, 2, 4
    A = wl.make_kv_case(7, B, W, D, 1, 4, [3, 20, 0], n_spare=4, max_pages=6, dtype="f32")
    A["best"][:] = [0, 1, 0]
    A["n_acc"][:] = [4, 4, 0]
    for nf in (-1, A["k_pool"].shape[0] + 1):
        A2 = dict(A, n_free=nf)
        C, flags = commit(A2, W, D)
        assert flags.tolist() == [oracle.FLAG_BAD_PAGE, oracle.FLAG_BAD_PAGE, 0]
        assert C["n_free"] == nf and np.array_equal(C["prefix_len"], A["prefix_len"])
        R, flags = truncate(A2, np.zeros(B, np.int32))
        assert (flags == oracle.FLAG_BAD_PAGE).all() and R["n_free"] == nf


def test_commit_layers_write_every_layer_at_the_same_slots():
    """Layers sharing one block table [SD6]: one commit takes each sequence's pages
    once, and every layer's accepted rows are found through the new table in that
    layer's own pool (read element by element from the raw head-major layout), the
    rows before them untouched and every other pool entry unchanged."""
    B, W, D, Hkv, hd, L = 5, 3, 6, 2, 8, 3
    base = wl.make_kv_case(21, B, W, D, Hkv, hd, [0, 15, 16, 17, 33], n_spare=20,
                           max_pages=8, dtype="f32")
    rng = np.random.default_rng(4)
    kp = np.stack([base["k_pool"]] + [rng.standard_normal(base["k_pool"].shape).astype(np.float32)
                                      for _ in range(L - 1)])
    vp = np.stack([base["v_pool"]] + [rng.standard_normal(base["v_pool"].shape).astype(np.float32)
                                      for _ in range(L - 1)])
    kc = np.stack([base["k_cand"]] + [rng.standard_normal(base["k_cand"].shape).astype(np.float32)
                                      for _ in range(L - 1)])
    vc = np.stack([base["v_cand"]] + [rng.standard_normal(base["v_cand"].shape).astype(np.float32)
                                      for _ in range(L - 1)])
    k2, v2, pt, P, fl, nf, flags = oracle.kv_commit_layers(
        kp, vp, base["page_table"], base["prefix_len"], base["free_list"], base["n_free"],
        kc, vc, base["best"], base["n_acc"], W, D)
    assert not flags.any()
    written = np.zeros(kp.shape, dtype=bool)
    written_v = np.zeros(vp.shape, dtype=bool)
    for b in range(B):
        P0, i, a = int(base["prefix_len"][b]), int(base["best"][b]), int(base["n_acc"][b])
        a = a if i >= 0 else 0
        assert int(P[b]) == P0 + a
        # the table keeps its old pages and takes new ones only past them
        old = (P0 + PAGE - 1) // PAGE
        assert np.array_equal(pt[b, :old], base["page_table"][b, :old])
        for o in range(a):
            pos = P0 + o
            pg, t = int(pt[b, pos // PAGE]), pos % PAGE
            row = b * W * D + i * D + o
            for l in range(L):
                for h in range(Hkv):
                    assert np.array_equal(k2[l, pg, h, t, :], kc[l, row, h])
                    assert np.array_equal(v2[l, pg, h, :, t], vc[l, row, h])
                    written[l, pg, h, t, :] = True
                    written_v[l, pg, h, :, t] = True
    assert np.array_equal(k2[~written], kp[~written])
    assert np.array_equal(v2[~written_v], vp[~written_v])
    # the pages taken are the ones a one-layer commit takes
    one = oracle.kv_commit(kp[0], vp[0], base["page_table"], base["prefix_len"], base["free_list"],
                           base["n_free"], kc[0], vc[0], base["best"], base["n_acc"], W, D)
    assert np.array_equal(one[2], pt) and one[5] == nf
