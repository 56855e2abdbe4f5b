"""Pins for the oracle's rejection sampler (CPU only).

Rejection-sampling blog (blog.huny.dev), sections 2-3: accept draft x with
probability alpha = min(1, p(x)/q(x)); on rejection draw from
p' = max(0, p-q)/sum max(0, p-q); all drafts accepted -> a bonus token from the
next position's p; identity P_final = min(p,q) + max(0,p-q) = p (lossless).
Section 5's five checks are mirrored with our own values (the page's numbers
were lost in extraction).  SwitchSD summary, 'How it differs': among W
candidates keep the longest verified continuation.

The exact-law pins compute the law of the oracle *implementation's* output by
locating, by bisection on the oracle itself, the thresholds in each uniform at
which its decision changes; the law is then compared with the closed form.
"""
import itertools
import json
import os

import numpy as np
import pytest

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _logits_of(p):
    return np.log(np.asarray(p, dtype=np.float64)).astype(np.float32)


def _stored_p(p):
    """Target probabilities as the sampler sees them: softmax of the fp32 logits."""
    z = _logits_of(p).astype(np.float64)
    e = np.exp(z - z.max())
    return e / e.sum()


def run(root_p, rows_p, q, toks, lens, u_acc, u_res, W, D):
    V = len(root_p)
    root = _logits_of(root_p)[None, :]
    logits = np.stack([_logits_of(r) for r in rows_p]) if rows_p else np.zeros((W * D, V), np.float32)
    return oracle.reject_sample(root, logits, q, np.asarray(toks, np.int32).reshape(1, W, D),
                                np.asarray(lens, np.int32).reshape(1, W),
                                np.asarray(u_acc, np.float64).reshape(1, W, D),
                                np.asarray(u_res, np.float64).reshape(1, W))


# ----------------------------------------------------------------- section 5 cases

def test_case1_target_dominates_always_accepts():
    p = [0.1, 0.6, 0.3]
    q = np.array([[0.3, 0.4, 0.3]], dtype=np.float32)      # p(1)=0.6 >= q(1)=0.4
    for u in (0.01, 0.25, 0.5, 0.75, 0.9999):
        r = run(p, [p], q, [1], [1], [u], [0.5], 1, 1)
        assert r["n_acc"][0] == 1 and r["out_tok"][0, 0] == 1


def test_case2_threshold():
    g = json.load(open(os.path.join(GOLD, "sampler_cases.json")))["threshold_case"]
    p = [g["p_x"], 1 - g["p_x"]]
    q = np.array([[g["q_x"], 1 - g["q_x"]]], dtype=np.float32)
    ra = run(p, [p], q, [0], [1], [g["u_accept"]], [0.5], 1, 1)
    rr = run(p, [p], q, [0], [1], [g["u_reject"]], [0.5], 1, 1)
    assert ra["n_acc"][0] == 1 and rr["n_acc"][0] == 0


def test_case3_residual_normalised_and_zero_where_draft_overproposes():
    p = np.array([0.1, 0.2, 0.3, 0.4])
    qd = np.array([0.4, 0.3, 0.2, 0.1])
    q = qd.astype(np.float32)[None, :]
    # rejection of token 0 (q > p there); scan the residual draw over u_res
    emitted = []
    for u in np.linspace(0.0005, 0.9995, 2000):
        r = run(p, [p], q, [0], [1], [0.999], [u], 1, 1)
        assert r["n_acc"][0] == 0
        emitted.append(int(r["out_tok"][0, 0]))
    emitted = np.array(emitted)
    freq = np.bincount(emitted, minlength=4) / len(emitted)
    resid = np.maximum(0.0, _stored_p(p) - qd.astype(np.float32))
    resid /= resid.sum()
    assert freq[0] == 0 and freq[1] == 0                  # over-proposed tokens get nothing
    assert np.abs(freq - resid).max() < 2e-3              # grid resolution 1/2000
    assert abs(resid.sum() - 1) < 1e-15


def test_case4_all_accepted_gives_bonus_from_last_row():
    V, K = 5, 3
    toks = [2, 0, 4]
    near_one = lambda k: [0.996 if j == k else 0.001 for j in range(V)]
    rows = [near_one(0), near_one(4), near_one(3)]          # rows judge toks[1], toks[2], bonus
    q = np.full((K, V), 0.2, dtype=np.float32)
    r = run(near_one(2), rows, q, toks, [K], [0.5] * K, [0.5], 1, K)
    assert r["n_acc"][0] == 3 and r["n_out"][0] == 4
    assert r["out_tok"][0].tolist() == [2, 0, 4, 3]         # bonus = argmax of row K-1


# ----------------------------------------------------------------- exact laws

def _threshold(f, lo=0.0, hi=1.0, it=64):
    """sup{u in [lo,hi): f(u)} for a predicate true on [lo, theta) and false after."""
    if not f(lo):
        return lo
    if f(np.nextafter(hi, 0)):
        return hi
    for _ in range(it):
        mid = 0.5 * (lo + hi)
        if f(mid):
            lo = mid
        else:
            hi = mid
    return lo


def exact_law(root_p, rows_p, qrows, D, V, W=1):
    """Law of (first token, second token | n_out >= 2) of the oracle's output with
    drafts x_o ~ q_o independently, for W=1.  Uses bisection on the oracle only."""
    first = np.zeros(V)
    second = np.zeros(V)
    p_second_mass = 0.0
    q = np.asarray(qrows, dtype=np.float32)
    for path in itertools.product(range(V), repeat=D):
        w_path = float(np.prod([float(q[o, path[o]]) for o in range(D)]))
        if w_path == 0.0:
            continue
        # threshold of each acceptance test (earlier tests forced to accept with u=0)
        th = []
        for o in range(D):
            def acc(u, o=o):
                ua = [0.0] * D
                ua[o] = u
                if o + 1 < D:
                    ua[o + 1] = np.nextafter(1.0, 0)
                r = run(root_p, rows_p, q, list(path), [D], ua, [0.5], 1, D)
                return r["n_acc"][0] >= o + 1
            th.append(_threshold(acc))
        for a in range(D + 1):
            pa = np.prod(th[:a]) * ((1 - th[a]) if a < D else 1.0)
            if pa == 0.0:
                continue
            ua = [t * 0.5 for t in th[:a]] + ([(1 + th[a]) * 0.5] if a < D else [])
            ua = (ua + [0.5] * D)[:D]

            def tok_le(k, u):
                r = run(root_p, rows_p, q, list(path), [D], ua, [u], 1, D)
                assert r["n_acc"][0] == a
                return r["out_tok"][0, a] <= k
            F = [_threshold(lambda u, k=k: tok_le(k, u)) for k in range(V)]
            law_y = np.diff(np.concatenate([[0.0], F]))
            if a == 0:
                first += w_path * pa * law_y
            else:
                first[path[0]] += w_path * pa
                p_second_mass += w_path * pa
                if a == 1:
                    second += w_path * pa * law_y
                else:
                    second[path[1]] += w_path * pa
    return first, second / max(p_second_mass, 1e-300), p_second_mass


def _dyadic(p, bits=20):
    """Probabilities k/2^bits summing to exactly one (exact in fp32), so the draft
    law sums to one in the exact arithmetic of the identity."""
    k = np.floor(np.asarray(p) * 2 ** bits).astype(np.int64)
    k[np.argmax(k)] += 2 ** bits - k.sum()
    return k / 2.0 ** bits


@pytest.mark.parametrize("seed,V,D", [(0, 3, 1), (1, 4, 1), (2, 5, 1), (3, 3, 2), (4, 4, 2)])
def test_emitted_law_equals_target_exactly(seed, V, D):
    """Identity P_final = p: the first emitted token follows the root target
    distribution, and given a second token it follows row 0's distribution."""
    rng = np.random.default_rng(seed)
    root_p = rng.dirichlet(np.ones(V))
    rows_p = [rng.dirichlet(np.ones(V)) for _ in range(D)]
    qrows = [_dyadic(rng.dirichlet(np.ones(V))) for _ in range(D)]
    first, second, m2 = exact_law(root_p, rows_p, qrows, D, V)
    assert np.abs(first - _stored_p(root_p)).max() < 1e-9
    assert np.abs(second - _stored_p(rows_p[0])).max() < 1e-9
    # acceptance law: P(a >= 1) = beta_0 = sum_x min(p_0(x), q_0(x))
    beta0 = np.minimum(_stored_p(root_p), np.asarray(qrows[0], np.float32)).sum()
    assert abs(m2 - beta0) < 1e-9


def test_monte_carlo_50k_within_4_sigma():
    """Section 5, case 5: 50,000 trials with strongly mismatched p and q."""
    rng = np.random.default_rng(11)
    V, N = 4, 50000
    p = np.array([0.7, 0.1, 0.1, 0.1])
    qd = np.array([0.05, 0.05, 0.1, 0.8], dtype=np.float32)
    root = _logits_of(p)[None, :]
    row = _logits_of(np.full(V, 0.25))[None, :]
    counts = np.zeros(V)
    xs = rng.choice(V, size=N, p=qd.astype(np.float64) / qd.sum())
    ua = rng.random(N)
    ur = rng.random(N)
    for n in range(N):
        r = oracle.reject_sample(root, row, qd[None, :], np.array([[[xs[n]]]], np.int32),
                                 np.array([[1]], np.int32), np.array([[[ua[n]]]]),
                                 np.array([[ur[n]]]))
        counts[r["out_tok"][0, 0]] += 1
    f = counts / N
    ps = _stored_p(p)
    assert (np.abs(f - ps) <= 4 * np.sqrt(ps * (1 - ps) / N)).all()


def test_greedy_limit_any_W():
    """One-hot target rows: the result is the longest prefix agreeing with the
    argmax chain, then the argmax, for any number of candidates."""
    V, W, D = 6, 3, 3
    hot = lambda k: [1 - 1e-30 * (V - 1) if j == k else 1e-30 for j in range(V)]
    greedy = [4, 1, 5, 2]                        # argmax at root, rows (.,0), (.,1), (.,2)
    toks = [[4, 1, 0], [4, 1, 5], [3, 1, 5]]
    rows = []
    for i in range(W):
        rows += [hot(greedy[1]), hot(greedy[2]), hot(greedy[3])]
    q = np.full((W * D, V), 1.0 / V, dtype=np.float32)
    r = run(hot(greedy[0]), rows, q, toks, [D] * W, [0.3] * (W * D), [0.7] * W, W, D)
    assert r["acc_per_cand"][0].tolist() == [2, 3, 0]
    assert r["best"][0] == 1 and r["out_tok"][0].tolist() == greedy


def test_multi_candidate_counterexample_law():
    g = json.load(open(os.path.join(GOLD, "sampler_cases.json")))["multi_candidate_counterexample"]
    p = np.array(g["p"])
    # enumerate the 2 acceptance uniforms on thresholds and the residual uniform
    law = np.zeros(2)
    q = np.array([g["q"], g["q"]], dtype=np.float32)
    for ua0, w0 in ((0.25, 0.5), (0.75, 0.5)):
        for ua1, w1 in ((0.25, 0.5), (0.75, 0.5)):
            for ur, wr in ((0.25, 0.5), (0.75, 0.5)):
                r = run(p, [p, p], q, [0, 0], [1, 1], [ua0, ua1], [ur, ur], 2, 1)
                law[r["out_tok"][0, 0]] += w0 * w1 * wr
    assert np.allclose(law, g["first_token_law"], atol=1e-12)


def test_point_mass_drafts():
    g = json.load(open(os.path.join(GOLD, "sampler_cases.json")))["point_mass_case"]
    p = g["p"]
    x = g["x"]
    th = _threshold(lambda u: run(p, [p], None, [x], [1], [u], [0.5], 1, 1)["n_acc"][0] == 1)
    assert abs(th - g["accept_prob"]) < 1e-7
    law = np.zeros(3)
    F = [_threshold(lambda u, k=k: run(p, [p], None, [x], [1], [0.99], [u], 1, 1)["out_tok"][0, 0] <= k)
         for k in range(3)]
    law = np.diff(np.concatenate([[0.0], F]))
    assert np.allclose(law, g["replacement_law"], atol=1e-7)


def test_no_candidate_samples_root_and_flags():
    p = [0.25, 0.5, 0.25]
    r = run(p, [p, p], None, [0, 1], [0, 0], [0.1, 0.1], [0.6, 0.1], 2, 1)
    assert r["n_out"][0] == 1 and r["best"][0] == -1 and r["out_tok"][0, 0] == 1
    assert r["flags"][0] & oracle.FLAG_NO_CANDIDATE
    # closed gate behaves the same even with candidates present
    root = _logits_of(p)[None, :]
    rr = oracle.reject_sample(root, np.stack([_logits_of(p)] * 2), None,
                              np.array([[[0], [1]]], np.int32), np.array([[1, 1]], np.int32),
                              np.array([[[0.1], [0.1]]]), np.array([[0.6, 0.1]]), gate=[0])
    assert rr["n_out"][0] == 1 and rr["flags"][0] & oracle.FLAG_NO_CANDIDATE


def test_degenerate_residual_falls_back_to_target():
    p = [0.5, 0.5]
    q = np.array([[0.9, 0.6]], dtype=np.float32)           # q >= p everywhere (unnormalised input)
    r = run(p, [p], q, [0], [1], [0.99], [0.75], 1, 1)
    assert r["n_acc"][0] == 0 and r["flags"][0] & oracle.FLAG_DEGENERATE
    assert r["out_tok"][0, 0] == 1


def test_ties_choose_smallest_candidate_and_bad_token_rejects():
    p = [0.5, 0.5]
    r = run(p, [p, p], None, [0, 1], [1, 1], [0.1, 0.1], [0.3, 0.3], 2, 1)
    assert r["acc_per_cand"][0].tolist() == [1, 1] and r["best"][0] == 0
    r = run(p, [p], None, [7], [1], [0.0], [0.3], 1, 1)
    assert r["n_acc"][0] == 0 and r["flags"][0] & oracle.FLAG_BAD_TOKEN


# ----------------------------------------------------------------- lossless multi-candidate
# (recursive residual across sibling candidates)

def run_multi(root_p, rows_p, q, toks, lens, u_acc, u_res, W, D):
    V = len(root_p)
    root = _logits_of(root_p)[None, :]
    logits = np.stack([_logits_of(r) for r in rows_p]) if rows_p else np.zeros((W * D, V), np.float32)
    return oracle.reject_sample_multi(root, logits, q, np.asarray(toks, np.int32).reshape(1, W, D),
                                      np.asarray(lens, np.int32).reshape(1, W),
                                      np.asarray(u_acc, np.float64).reshape(1, W, D),
                                      np.asarray(u_res, np.float64).reshape(1, W))


@pytest.mark.parametrize("dense", [False, True])
def test_multi_equals_literal_for_one_candidate(dense):
    """With W = 1 there are no siblings: the rule is section 3's chain exactly."""
    rng = np.random.default_rng(3)
    B, D, V = 40, 5, 12
    root = rng.standard_normal((B, V)).astype(np.float32)
    lg = (rng.standard_normal((B * D, V)) * 2).astype(np.float32)
    tok = rng.integers(0, 4, (B, 1, D)).astype(np.int32)
    ln = rng.integers(0, D + 1, (B, 1)).astype(np.int32)
    ua, ur = rng.random((B, 1, D)), rng.random((B, 1))
    q = None
    if dense:
        q = rng.dirichlet(np.ones(V), size=B * D).astype(np.float32)
    a = oracle.reject_sample_multi(root, lg, q, tok, ln, ua, ur)
    b = oracle.reject_sample(root, lg, q, tok, ln, ua, ur)
    for k in ("n_acc", "best", "out_tok", "n_out", "acc_per_cand", "flags"):
        assert np.array_equal(a[k], b[k]), k


def multi_first_law(root_p, qrows, W, V):
    """Law of the first emitted token of the multi rule with sibling drafts x_i ~
    q_i drawn independently (D = 1), from thresholds located by bisection on the
    oracle's uniforms only."""
    q = np.asarray(qrows, dtype=np.float32)
    rows_p = [root_p] * W                      # D = 1: rows are never used
    hi = np.nextafter(1.0, 0)
    law = np.zeros(V)
    for xs in itertools.product(range(V), repeat=W):
        w = float(np.prod([float(q[i, xs[i]]) for i in range(W)]))
        if w == 0.0:
            continue
        reach = 1.0
        for i in range(W):
            # sibling i's acceptance threshold: earlier siblings pushed to rejection
            # (u just below 1), later ones given an out-of-range token (always rejected)
            def acc(u, i=i):
                ua = [hi] * W
                ua[i] = u
                xs_i = list(xs[:i + 1]) + [V] * (W - i - 1)
                return run_multi(root_p, rows_p, q, xs_i, [1] * W, ua, [0.5] * W, W, 1)["n_acc"][0] == 1
            th = _threshold(acc)
            law[xs[i]] += w * reach * th
            reach *= 1.0 - th
        if reach == 0.0:
            continue

        def tok_le(k, u):
            r = run_multi(root_p, rows_p, q, list(xs), [1] * W, [hi] * W, [u] * W, W, 1)
            assert r["n_acc"][0] == 0
            return r["out_tok"][0, 0] <= k
        F = [_threshold(lambda u, k=k: tok_le(k, u)) for k in range(V)]
        law += w * reach * np.diff(np.concatenate([[0.0], F]))
    return law


@pytest.mark.parametrize("seed,W,V", [(0, 2, 3), (1, 2, 4), (2, 3, 3)])
def test_multi_first_token_law_is_target(seed, W, V):
    """Dense sibling drafts drawn independently from their own q: the emitted token
    follows the target exactly (the literal longest-run rule does not, see the
    counterexample above)."""
    rng = np.random.default_rng(seed)
    root_p = rng.dirichlet(np.ones(V))
    qrows = [_dyadic(rng.dirichlet(np.ones(V) * 0.7)) for _ in range(W)]
    law = multi_first_law(root_p, qrows, W, V)
    assert np.abs(law - _stored_p(root_p)).max() < 1e-9


def test_multi_counterexample_is_lossless():
    """The W = 2 counterexample of the literal rule (law (3/4, 1/4) for p = (1/2, 1/2))
    gives p under the multi rule."""
    g = json.load(open(os.path.join(GOLD, "sampler_cases.json")))["multi_candidate_counterexample"]
    law = multi_first_law(np.array(g["p"]), [g["q"], g["q"]], 2, 2)
    assert np.abs(law - _stored_p(g["p"])).max() < 1e-12


def test_multi_point_mass_siblings_law_is_target():
    """Copy drafts (point masses) at one depth, with a repeated token: trying x1, x2,
    x3 in turn and removing each rejected token's mass, then drawing from what is
    left, emits exactly the target law."""
    V = 5
    p = np.array([0.05, 0.3, 0.15, 0.4, 0.1])
    ps = _stored_p(p)
    hi = np.nextafter(1.0, 0)
    for xs in ([1, 3, 0], [3, 3, 2], [4, 4, 4]):
        W = len(xs)
        law = np.zeros(V)
        reach = 1.0
        for i in range(W):
            def acc(u, i=i):
                ua = [hi] * W
                ua[i] = u
                return run_multi(p, [p] * W, None, xs, [1] * W, ua, [0.5] * W, W, 1)["n_acc"][0] == 1
            th = _threshold(acc)
            law[xs[i]] += reach * th
            reach *= 1.0 - th

        def tok_le(k, u):
            return run_multi(p, [p] * W, None, xs, [1] * W, [hi] * W, [u] * W, W, 1)["out_tok"][0, 0] <= k
        F = [_threshold(lambda u, k=k: tok_le(k, u)) for k in range(V)]
        law += reach * np.diff(np.concatenate([[0.0], F]))
        assert np.abs(law - ps).max() < 1e-9, xs


def test_multi_second_depth_follows_reference_row():
    """Two copy candidates sharing their first token a: after a is accepted both
    survive, the second depth is judged by the reference candidate's row (0, 0) and
    the second emitted token follows that row exactly; candidate 1's own row is not
    used."""
    V = 4
    root_p = np.array([0.4, 0.3, 0.2, 0.1])
    row00 = np.array([0.1, 0.2, 0.3, 0.4])       # judges depth 1 for candidate 0
    row10 = np.array([0.7, 0.1, 0.1, 0.1])       # candidate 1's own row: never used
    rows_p = [row00, root_p, row10, root_p]       # rows (0,0), (0,1), (1,0), (1,1)
    toks = [0, 2, 0, 3]                           # cand 0 = (0, 2), cand 1 = (0, 3)
    hi = np.nextafter(1.0, 0)
    W, D = 2, 2
    law = np.zeros(V)
    reach = 1.0
    for i, x in ((0, 2), (1, 3)):
        def acc(u, i=i):
            ua = [0.0, hi, 0.0, hi]               # depth 0 accepted by candidate 0
            ua[i * D + 1] = u
            return run_multi(root_p, rows_p, None, toks, [2, 2], ua, [0.5, 0.5], W, D)["n_acc"][0] == 2
        th = _threshold(acc)
        law[x] += reach * th
        reach *= 1.0 - th

    def tok_le(k, u):
        r = run_multi(root_p, rows_p, None, toks, [2, 2], [0.0, hi, 0.0, hi], [u, u], W, D)
        assert r["n_acc"][0] == 1 and r["out_tok"][0, 0] == 0 and r["best"][0] == 0
        return r["out_tok"][0, 1] <= k
    F = [_threshold(lambda u, k=k: tok_le(k, u)) for k in range(V)]
    law += reach * np.diff(np.concatenate([[0.0], F]))
    assert np.abs(law - _stored_p(row00)).max() < 1e-9
    # both candidates survive depth 0: their common prefix with the accepted tokens
    r = run_multi(root_p, rows_p, None, toks, [2, 2], [0.0, hi, 0.0, hi], [0.5, 0.5], W, D)
    assert r["acc_per_cand"][0].tolist() == [1, 1]


def test_multi_greedy_limit():
    """One-hot targets: the multi rule emits the argmax chain as long as some
    candidate proposes it, then the argmax."""
    V, W, D = 6, 3, 3
    hot = lambda k: [1 - 1e-30 * (V - 1) if j == k else 1e-30 for j in range(V)]
    greedy = [4, 1, 5, 2]
    toks = [[4, 0, 0], [4, 1, 0], [3, 1, 5]]
    rows = [hot(greedy[1]), hot(greedy[2]), hot(greedy[3])] * W
    r = run_multi(hot(greedy[0]), rows, None, toks, [D] * W, [0.3] * (W * D), [0.7] * W, W, D)
    # depth 0: candidates 0, 1 propose 4 (accepted); depth 1: candidate 1 proposes 1
    # (accepted, judged by row (0, 0)); depth 2: candidate 1 proposes 0 -> residual
    assert r["n_acc"][0] == 2 and r["best"][0] == 1
    assert r["out_tok"][0].tolist() == [4, 1, 5, -1]
    assert r["acc_per_cand"][0].tolist() == [1, 2, 0]


# ----------------------------------------------------------------- greedy (T = 0)

def _spread_rows(rng, n, V, gap=0.05):
    """Random logits whose largest value leads the next by at least `gap`."""
    z = rng.standard_normal((n, V))
    k = z.argmax(axis=1)
    second = np.partition(z, V - 2, axis=1)[:, -2]
    z[np.arange(n), k] = np.maximum(z[np.arange(n), k], second + gap)
    return z.astype(np.float32)


@pytest.mark.parametrize("qmode", ["point", "dense"])
def test_greedy_is_the_zero_temperature_limit(qmode):
    """reject_sample at T = 1e-3 on rows whose top two logits are >= 0.05 apart gives
    every p(non-argmax) < exp(-50): whatever the uniforms and the draft distribution,
    it must emit what the greedy rule emits."""
    rng = np.random.default_rng(40)
    B, W, D, V = 60, 3, 4, 50
    M = W * D
    root = _spread_rows(rng, B, V)
    logits = _spread_rows(rng, B * M, V)
    cand = rng.integers(0, V, size=(B, W, D)).astype(np.int32)
    # make many tokens the argmax of their preceding row, so that runs are long
    for b in range(B):
        for i in range(W):
            for o in range(D):
                if rng.random() < 0.7:
                    r = root[b] if o == 0 else logits[b * M + i * D + o - 1]
                    cand[b, i, o] = int(np.argmax(r))
    clen = rng.integers(0, D + 1, size=(B, W)).astype(np.int32)
    q = None
    if qmode == "dense":
        q = rng.dirichlet(np.ones(V), size=B * M).astype(np.float32)
    ua = rng.random((B, W, D))
    ur = rng.random((B, W))
    s = oracle.reject_sample(root, logits, q, cand, clen, ua, ur, 1e-3)
    g = oracle.reject_sample_greedy(root, logits, cand, clen)
    for k in ("n_acc", "best", "out_tok", "n_out", "acc_per_cand"):
        assert np.array_equal(s[k], g[k]), k
    assert (g["n_acc"] >= 2).sum() > B // 4
    assert not (g["flags"] & (oracle.FLAG_ACCEPT_TIE | oracle.FLAG_CDF_TIE)).any()


def _tree_model(V, seed):
    """A toy deterministic model: the logits after a context depend only on the
    context's tokens."""
    def f(prefix):
        h = (seed * 1000003 + len(prefix)) & 0xFFFFFFFF
        for t in prefix:
            h = (h * 2654435761 + int(t) + 1) & 0xFFFFFFFF
        return np.random.default_rng(h).standard_normal(V).astype(np.float32)
    return f


@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_greedy_equals_plain_greedy_decoding(seed):
    """Under a model whose logits depend only on the context, greedy verification of W
    candidates emits a prefix of plain greedy decoding, as long as the longest
    candidate agreement plus one; the multi-candidate rule at T -> 0 emits the same."""
    V, W, D = 12, 4, 6
    f = _tree_model(V, seed)
    gd = []
    for _ in range(D + 1):
        gd.append(int(np.argmax(f(gd))))
    rng = np.random.default_rng(seed)
    cand = np.zeros((1, W, D), dtype=np.int32)
    for i in range(W):
        k = int(rng.integers(0, D + 1))              # agree with greedy for k tokens
        cand[0, i, :k] = gd[:k]
        for o in range(k, D):
            cand[0, i, o] = int(rng.integers(0, V))
    clen = rng.integers(1, D + 1, size=(1, W)).astype(np.int32)
    root = f([])[None, :]
    logits = np.stack([f(cand[0, i, :o + 1]) for i in range(W) for o in range(D)])
    g = oracle.reject_sample_greedy(root, logits, cand, clen)
    agree = []
    for i in range(W):
        k = 0
        while k < clen[0, i] and cand[0, i, k] == gd[k]:
            k += 1
        agree.append(k)
    n = g["n_out"][0]
    assert g["n_acc"][0] == max(agree) and n == max(agree) + 1
    assert g["out_tok"][0, :n].tolist() == gd[:n]
    assert g["acc_per_cand"][0].tolist() == agree
    m = oracle.reject_sample_multi(root, logits, None, cand, clen, np.full((1, W, D), 0.5),
                                   np.full((1, W), 0.5), 1e-3)
    assert m["n_acc"][0] == g["n_acc"][0]
    assert m["out_tok"][0].tolist() == g["out_tok"][0].tolist()


def test_greedy_ties_take_first_index_and_flag():
    V, W, D = 8, 2, 2
    z = np.zeros(V, np.float32)
    z[[2, 5]] = 3.0                                   # exact tie: argmax is 2
    zc = np.zeros(V, np.float32)
    zc[6] = 1.0
    zc[1] = 1.0 - 5e-4                                # near tie (within 1e-3)
    root = z[None, :]
    logits = np.stack([zc, zc, zc, zc])
    # candidate 0 proposes 5 (rejected against the tie), candidate 1 proposes 2 then 6
    cand = np.array([[[5, 0], [2, 6]]], np.int32)
    g = oracle.reject_sample_greedy(root, logits, cand, np.array([[2, 2]], np.int32))
    assert g["acc_per_cand"][0].tolist() == [0, 2]
    assert g["best"][0] == 1 and g["out_tok"][0].tolist() == [2, 6, 6]
    assert g["flags"][0] & oracle.FLAG_ACCEPT_TIE and g["flags"][0] & oracle.FLAG_CDF_TIE
    # no tie anywhere: no flags
    g2 = oracle.reject_sample_greedy(np.eye(V, dtype=np.float32)[3][None, :] * 4,
                                     np.tile(np.eye(V, dtype=np.float32)[7] * 4, (4, 1)),
                                     np.array([[[3, 7], [3, 1]]], np.int32),
                                     np.array([[2, 2]], np.int32))
    assert g2["flags"][0] == 0 and g2["out_tok"][0].tolist() == [3, 7, 7]
    assert g2["acc_per_cand"][0].tolist() == [2, 1]


def test_greedy_no_candidate_and_bad_token():
    V, W, D = 6, 2, 3
    root = np.array([[0, 1, 0, 4, 0, 0]], np.float32)
    logits = np.tile(np.array([5, 0, 0, 0, 0, 0], np.float32), (W * D, 1))
    cand = np.array([[[3, 0, 0], [3, 99, 0]]], np.int32)
    clen = np.array([[3, 3]], np.int32)
    g = oracle.reject_sample_greedy(root, logits, cand, clen, gate=np.array([0]))
    assert g["n_acc"][0] == 0 and g["best"][0] == -1 and g["out_tok"][0, 0] == 3
    assert g["flags"][0] == oracle.FLAG_NO_CANDIDATE
    g = oracle.reject_sample_greedy(root, logits, cand, clen)
    assert g["acc_per_cand"][0].tolist() == [3, 1]
    assert g["flags"][0] == oracle.FLAG_BAD_TOKEN
    assert g["out_tok"][0].tolist() == [3, 0, 0, 0]


# ----------------------------------------------------------------- draft sampling, rho_TPS

def test_draft_sample_worked_cases():
    q = np.array([[0.0, 0.5, 0.0, 0.5]] * 4, np.float32)
    tok, flags = oracle.draft_sample(q, np.array([0.25, 0.75, 0.0, 0.4999]))
    assert tok.tolist() == [1, 3, 1, 1]
    assert flags.tolist() == [0, 0, oracle.FLAG_CDF_TIE, 0]      # u = 0 sits on the first step
    # exactly on a step: flagged
    tok, flags = oracle.draft_sample(q[:1], np.array([0.5]))
    assert tok[0] == 3 and flags[0] == oracle.FLAG_CDF_TIE


def test_draft_sample_law_on_a_stratified_grid():
    """With u on the grid (k + 1/2)/N, token frequencies equal q / sum(q) within 1/N."""
    rng = np.random.default_rng(2)
    V, N = 37, 20000
    q = rng.dirichlet(np.ones(V) * 0.3).astype(np.float32)
    q[[3, 17]] = 0.0
    u = (np.arange(N) + 0.5) / N
    tok, _ = oracle.draft_sample(np.tile(q, (N, 1)), u)
    freq = np.bincount(tok, minlength=V) / N
    p = q.astype(np.float64) / q.astype(np.float64).sum()
    assert np.abs(freq - p).max() <= 1.0 / N + 1e-12
    assert freq[3] == 0 and freq[17] == 0


def test_rho_tps_special_cases():
    assert oracle.rho_tps(1.0, 0.97, 3.0) == pytest.approx(0.97)        # same head: acceptance only
    assert oracle.rho_tps(0.2, 0.99, 0.0) == pytest.approx(0.99)        # head costs nothing
    assert oracle.rho_tps(0.0, 1.0, 2.5) == pytest.approx(3.5)          # free head: 1 + kappa
    assert oracle.rho_tps(0.25, 1.0, 1.0) == pytest.approx(2.0 / 1.25)
    v = [oracle.rho_tps(nu, 0.99, 1.5) for nu in (0.1, 0.3, 0.6, 1.0)]
    assert all(a > b for a, b in zip(v, v[1:]))
