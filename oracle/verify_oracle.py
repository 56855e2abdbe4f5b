"""Plain, slow, fp64 CPU oracle of the speculative-decoding verify step.

TEST INFRASTRUCTURE ONLY -- imported by the tests, the smoke check and the
bench's cpu_baseline leg, never by the GPU library.  It shares no code with the
GPU path: it decodes bf16 itself, rounds stage outputs itself and reads only
host numpy arrays.

Sources (web pages; cited by title and section):
  [SW]  "SwitchSD는 LLM 내부 표현으로 추측 디코딩의 복사 모드를 판별한다"
        (onedev.kr/papers/87): sections "어떻게 동작하나" (how it works) and
        "무엇과 다른가" (how it differs).
  [SD]  "LLM 투기적 디코딩(Speculative Decoding) 해부 ..." (blog.huny.dev):
        section 2 (pipeline: drafting, parallel verification, rejection sampler,
        bonus token) and section 3 (equations for alpha(x), p'(x), P_final).
  [EX]  "추측 디코딩은 왜 빨라지면서 답은 바뀌지 않나" (jl917.github.io):
        step 2 (batch verify, cut at the first mismatch).
  [SL]  "SlimSpec: Low-Rank Draft LM-Head for Accelerated Speculative Decoding"
        (gist.science/ko/paper/2605.10453): "방법론 / 아키텍처", z = W_up W_down h.
  [SD6] the same blog's section 6 (production checklist): KV-cache rollback with a
        paged memory pool -- the KV blocks of rejected tokens go back to the pool
        at once, and no block may leak.

Every function below is the plain definition of its step; the readings taken
where the pages are silent or garbled are listed next to the code that uses them.
Parity pins: every function here is pinned by tests that do not call it to
produce the expected value (brute force, closed forms, library routines,
hand-derived values); see tests/test_oracle_*.py.

Parity unpinned: the law of the emitted token when W > 1 candidates are sampled
(not greedy).  The pages state only "keep the longest verified run"; they give no
distribution for it, and the literal rule is not lossless for W > 1 (a W = 2
counterexample gives (3/4, 1/4) for p = (1/2, 1/2)).  reject_sample follows the
literal rule; for W > 1 it is pinned only against the enumerated law of that same
rule and against the greedy limit, where it reduces to plain greedy decoding.
"""
from __future__ import annotations

import numpy as np

# Flag bits, shared in meaning (not in code) with the GPU library's header.
FLAG_PROBE_TIE = 1          # |score - tau| < 1e-5
FLAG_ACCEPT_TIE = 2         # a decisive acceptance test is a near tie
FLAG_CDF_TIE = 4            # the categorical draw lands within eps of a CDF step
FLAG_DEGENERATE = 8         # residual mass <= 0: fell back to the target distribution
FLAG_NO_CANDIDATE = 16      # no candidate (gate closed or nothing found): root sample only
FLAG_BAD_PAGE = 32          # page-table entry or prefix length out of range
FLAG_BAD_CTX = 64           # context offsets out of range
FLAG_BAD_TOKEN = 128        # candidate token id outside [0, V)
FLAG_POOL_EMPTY = 256       # KV commit: not enough free pages for the accepted rows

PROBE_TIE_EPS = 1e-5
ACCEPT_TIE_REL = 1e-4
CDF_TIE_EPS = 1e-8
GREEDY_TIE_REL = 1e-3       # greedy: top two logits of a row closer than this (x max(1, |top|))


# ----------------------------------------------------------------------------------
# number formats (own implementation; the GPU library has its own)

def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bf16 bit patterns: the 16 bits are the top half of an fp32."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def as_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return bf16_bits_to_f64(x)
    return np.asarray(x, dtype=np.float32).astype(np.float64)


def round_f64_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round fp64 values to the nearest bf16 value (ties to even), returned as fp64.
    bf16 keeps 7 explicit mantissa bits; fp64 has 52, so the rounding point is bit 45."""
    u = np.ascontiguousarray(x, dtype=np.float64).view(np.uint64)
    lsb = (u >> np.uint64(45)) & np.uint64(1)
    r = (u + lsb + np.uint64((1 << 44) - 1)) >> np.uint64(45) << np.uint64(45)
    return r.view(np.float64)


def round_stage(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round a stage output to the ABI dtype (bf16 RNE, or fp32)."""
    if dtype == "bf16":
        return round_f64_to_bf16(x)
    return x.astype(np.float32).astype(np.float64)


# ----------------------------------------------------------------------------------
# a1: copy-candidate retrieval  [SW, "무엇과 다른가"]

def copy_match(ctx: np.ndarray, ctx_off: np.ndarray, kappa: int, W: int, D: int):
    """For each sequence (context ctx[off[b]:off[b+1]], current token t = L-1):
    the key is the kappa-gram ending at t.  Every earlier end position j
    (kappa-1 <= j <= t-1) whose kappa-gram equals the key is an occurrence;
    occurrences may overlap.  Up to W occurrences are kept, most recent (largest j)
    first; candidate i continues the context after its occurrence:
    ctx[j+1 .. j+len], len = min(D, t-j) (readings: exact id equality, truncation
    at the end of the context, no de-duplication).  Missing candidates have len 0
    and position -1; token slots past len hold -1."""
    ctx = np.asarray(ctx, dtype=np.int64)
    off = np.asarray(ctx_off, dtype=np.int64)
    B = len(off) - 1
    cand_tok = np.full((B, W, D), -1, dtype=np.int32)
    cand_len = np.zeros((B, W), dtype=np.int32)
    cand_pos = np.full((B, W), -1, dtype=np.int32)
    n_found = np.zeros(B, dtype=np.int32)
    flags = np.zeros(B, dtype=np.int32)
    for b in range(B):
        lo, hi = off[b], off[b + 1]
        if not (0 <= lo <= hi <= len(ctx)):
            flags[b] |= FLAG_BAD_CTX
            continue
        c = ctx[lo:hi]
        L = len(c)
        t = L - 1
        if L < kappa + 1:
            continue
        key = c[t - kappa + 1:t + 1]
        i = 0
        for j in range(t - 1, kappa - 2, -1):
            if i == W:
                break
            if np.array_equal(c[j - kappa + 1:j + 1], key):
                ln = min(D, t - j)
                cand_pos[b, i] = j
                cand_len[b, i] = ln
                cand_tok[b, i, :ln] = c[j + 1:j + 1 + ln]
                i += 1
        n_found[b] = i
    return dict(cand_tok=cand_tok, cand_len=cand_len, cand_pos=cand_pos,
                n_found=n_found, flags=flags)


def copy_labels(ctx: np.ndarray, ctx_off: np.ndarray, kappa: int = 5, labels_init=None):
    """Copy-mode labels [SW "어떻게 동작하나"]: a token position is labelled Y = 1 when it
    lies inside a verbatim run of at least kappa tokens that already appeared earlier
    in the same context.

    Readings: "earlier" means the earlier occurrence starts at a smaller position (it
    may overlap the later one, as copy_match's occurrences may); every run of length
    L >= kappa holds a kappa-gram at each of its offsets, each of which also occurs
    earlier, so a position is labelled iff some kappa-gram window [s, s+kappa) that
    covers it occurs at a start t < s.  Written that way here: R[s] marks a repeated
    kappa-gram start, Y[p] = OR of R over the windows covering p.

    The offsets must be non-decreasing with ctx_off[0] >= 0 and ctx_off[B] <= len(ctx);
    otherwise every sequence gets FLAG_BAD_CTX and nothing is written.  Positions
    outside [ctx_off[0], ctx_off[B]) keep labels_init (0 by default).  Returns
    (labels uint8 [len(ctx)], flags int32 [B])."""
    ctx = np.asarray(ctx, dtype=np.int64)
    off = np.asarray(ctx_off, dtype=np.int64)
    B = len(off) - 1
    labels = (np.zeros(len(ctx), dtype=np.uint8) if labels_init is None
              else np.array(labels_init, dtype=np.uint8, copy=True))
    flags = np.zeros(B, dtype=np.int32)
    if off[0] < 0 or off[B] > len(ctx) or (np.diff(off) < 0).any():
        flags[:] = FLAG_BAD_CTX
        return labels, flags
    for b in range(B):
        lo, hi = int(off[b]), int(off[b + 1])
        first = {}
        R = np.zeros(max(hi - lo, 0), dtype=bool)
        for s in range(lo, hi - kappa + 1):
            g = tuple(ctx[s:s + kappa])
            if g in first:
                R[s - lo] = True
            else:
                first[g] = s
        for p in range(lo, hi):
            s0, s1 = max(lo, p - kappa + 1), min(p, hi - kappa)
            labels[p] = 1 if any(R[s - lo] for s in range(s0, s1 + 1)) else 0
    return labels, flags


# ----------------------------------------------------------------------------------
# a2: probe gate  [SW, "어떻게 동작하나" (bias-free probe) and "무엇과 다른가" (dual gate)]

def probe_gate(h: np.ndarray, w: np.ndarray, tau: float, n_found=None):
    """score = sigma(w . h) with no bias; the probe fires when score >= tau
    ("tau or above"); the copy path opens when the probe fires AND the kappa-gram
    has a prior occurrence (n_found >= 1).  h: [B, d] fp64 values, w: [d]."""
    h = np.asarray(h, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    x = h @ w
    score = 1.0 / (1.0 + np.exp(-x))
    probe = score >= tau
    if n_found is None:
        gate = probe
    else:
        gate = probe & (np.asarray(n_found) >= 1)
    flags = np.where(np.abs(score - tau) < PROBE_TIE_EPS, FLAG_PROBE_TIE, 0).astype(np.int32)
    return dict(score=score, probe=probe.astype(np.int32), gate=gate.astype(np.int32),
                flags=flags)


# ----------------------------------------------------------------------------------
# a3: block-triangular verify attention  [SW, "무엇과 다른가"]

def token_major(pool: np.ndarray, kind: str) -> np.ndarray:
    """View a paged pool as [n_pages, page, Hkv, hd].  K pages are stored
    [n_pages, Hkv, page, hd]; V pages transposed, [n_pages, Hkv, hd, page]."""
    if kind == "k":
        return np.transpose(pool, (0, 2, 1, 3))
    return np.transpose(pool, (0, 3, 1, 2))


def gather_prefix(pool: np.ndarray, page_table: np.ndarray, b: int, P: int, page: int):
    """Rows 0..P-1 of sequence b's prefix from a token-major paged view
    [n_pages, page, Hkv, hd].  Returns (rows [P, Hkv, hd], valid mask [P]) -- rows of
    out-of-range pages are marked invalid."""
    n_pages = pool.shape[0]
    rows = np.zeros((P,) + pool.shape[2:], dtype=pool.dtype)
    valid = np.zeros(P, dtype=bool)
    for pos in range(0, P, page):
        pg = int(page_table[b, pos // page])
        n = min(page, P - pos)
        if 0 <= pg < n_pages:
            rows[pos:pos + n] = pool[pg, :n]
            valid[pos:pos + n] = True
    return rows, valid


def verify_attention(q, k_cand, v_cand, k_pool, v_pool, page_table, prefix_len,
                     B, W, D, Hq, Hkv, scale=None, page=16, out_dtype="bf16"):
    """Attention of every candidate row over the prefix and its own candidate.

    Row r = i*D + o of sequence b holds candidate token (i, o).  Its query head hq
    (KV head hq // (Hq/Hkv)) attends to every prefix key 0..P_b-1 and to the keys
    of its own candidate at offsets 0..o (itself included); keys of other candidates
    are invisible.  Scores are (q . k) * scale with scale = 1/sqrt(hd); weights are
    the softmax of the visible scores; the output is the weighted sum of values.

    Inputs are fp64 arrays (decoded): q [B*M, Hq, hd], k_cand/v_cand [B*M, Hkv, hd],
    k_pool [n_pages, Hkv, page, hd], v_pool [n_pages, Hkv, hd, page].  Returns (O exact fp64, O rounded to out_dtype,
    flags [B])."""
    M = W * D
    hd = q.shape[-1]
    g = Hq // Hkv
    if scale is None:
        scale = 1.0 / np.sqrt(hd)
    O = np.zeros(q.shape, dtype=np.float64)
    flags = np.zeros(B, dtype=np.int32)
    max_keys = page_table.shape[1] * page
    for b in range(B):
        P = int(prefix_len[b])
        if P < 0 or P > max_keys:
            flags[b] |= FLAG_BAD_PAGE
            P = min(max(P, 0), max_keys)
        kp, valid = gather_prefix(token_major(k_pool, "k"), page_table, b, P, page)
        vp, _ = gather_prefix(token_major(v_pool, "v"), page_table, b, P, page)
        if not valid.all():
            flags[b] |= FLAG_BAD_PAGE
        for i in range(W):
            rows = slice(b * M + i * D, b * M + (i + 1) * D)
            for hq in range(Hq):
                kv = hq // g
                keys = np.concatenate([kp[:, kv, :], k_cand[rows, kv, :]], axis=0)   # [P+D, hd]
                vals = np.concatenate([vp[:, kv, :], v_cand[rows, kv, :]], axis=0)
                s = (q[rows, hq, :] @ keys.T) * scale                                  # [D, P+D]
                vis = np.zeros((D, P + D), dtype=bool)
                vis[:, :P] = valid[None, :]
                for o in range(D):
                    vis[o, P:P + o + 1] = True
                s = np.where(vis, s, -np.inf)
                m = s.max(axis=1, keepdims=True)
                e = np.where(vis, np.exp(s - m), 0.0)
                a = e / e.sum(axis=1, keepdims=True)
                O[rows, hq, :] = a @ vals
    return O, round_stage(O, out_dtype), flags


def verify_attention_layers(q, k_cand, v_cand, k_pool, v_pool, page_table, prefix_len,
                            B, W, D, Hq, Hkv, scale=None, page=16, out_dtype="bf16"):
    """The verify attention of L layers of one model [SW, "무엇과 다른가"; SD6: a paged
    cache per layer].  Reading: every layer keeps its own cache in pages, and the
    block table -- which page holds which 16 positions of a sequence, and how long the
    sequence is -- is the same for all layers, since every layer stores the same
    positions.  So layer l is verify_attention on that layer's queries, candidate
    keys/values and pools (each array here has a leading layer axis) with the common
    page_table and prefix_len.  Returns (O exact [L, ...], O rounded, flags [B]: the
    OR over layers, which all see the same table)."""
    L = q.shape[0]
    res = [verify_attention(q[l], k_cand[l], v_cand[l], k_pool[l], v_pool[l], page_table,
                            prefix_len, B, W, D, Hq, Hkv, scale, page, out_dtype)
           for l in range(L)]
    flags = np.zeros(B, dtype=np.int32)
    for r in res:
        flags |= r[2]
    return np.stack([r[0] for r in res]), np.stack([r[1] for r in res]), flags


# ----------------------------------------------------------------------------------
# a4/a5: vocabulary projection  [SL, "방법론 / 아키텍처"]; softmax rows [SD, section 3]

def _logsumexp_rows(z: np.ndarray) -> np.ndarray:
    m = z.max(axis=1, keepdims=True)
    return (m + np.log(np.exp(z - m).sum(axis=1, keepdims=True)))[:, 0]


def lm_head_full(H: np.ndarray, W_full, temperature: float = 1.0, dtype: str = "bf16",
                 block: int = 8192):
    """Full-rank head z = W_full h for every row h of H (z[r, v] = sum_k W[v,k] H[r,k]).
    W_full may be bf16 bits (decoded here block by block).  Logits are stored as
    fp32 (stage boundary); lse[r] = log sum_v exp(z[r,v]/T) is taken in fp64 from
    the stored fp32 logits.  Returns (logits fp32 [M, V], lse fp64 [M])."""
    H = np.asarray(H, dtype=np.float64)
    V = W_full.shape[0]
    z = np.empty((H.shape[0], V), dtype=np.float32)
    for s in range(0, V, block):
        Wb = as_f64(W_full[s:s + block], dtype)
        z[:, s:s + block] = (H @ Wb.T).astype(np.float32)
    lse = _logsumexp_rows(z.astype(np.float64) / temperature)
    return z, lse


def lm_head_lowrank(H: np.ndarray, W_down, W_up, temperature: float = 1.0,
                    dtype: str = "bf16", block: int = 16384):
    """SlimSpec head z = W_up (W_down h): the rank-r intermediate t = W_down h is kept
    unrounded, then projected to the vocabulary.  Returns (logits fp32, lse fp64, t)."""
    H = np.asarray(H, dtype=np.float64)
    Wd = as_f64(W_down, dtype)
    t = H @ Wd.T                                      # [M, r]
    V = W_up.shape[0]
    z = np.empty((H.shape[0], V), dtype=np.float32)
    for s in range(0, V, block):
        Wu = as_f64(W_up[s:s + block], dtype)
        z[:, s:s + block] = (t @ Wu.T).astype(np.float32)
    lse = _logsumexp_rows(z.astype(np.float64) / temperature)
    return z, lse, t


def head_softmax(logits: np.ndarray, lse: np.ndarray, temperature: float = 1.0):
    """Row softmax exp(z/T - lse) in fp64 (the head's probability output)."""
    return np.exp(logits.astype(np.float64) / temperature - lse[:, None])


# ----------------------------------------------------------------------------------
# a6: rejection sampling  [SD, sections 2-3]; longest verified continuation [SW]

def _draw(r: np.ndarray, u: float):
    """Categorical draw by inverse CDF over ascending token id:
    k = min{k : C_k > u * S}, with C the running sum of r and S its total.
    Returns (k, tie, margin): tie marks u*S within CDF_TIE_EPS*S of a CDF step;
    margin is the distance to the nearest step as a fraction of S."""
    C = np.cumsum(r)
    S = C[-1]
    x = u * S
    k = int(np.searchsorted(C, x, side="right"))
    k = min(k, len(r) - 1)
    lo = C[k - 1] if k > 0 else 0.0
    margin = min(abs(x - lo), abs(C[k] - x)) / S
    tie = margin < CDF_TIE_EPS
    return k, tie, margin


def draft_sample(q: np.ndarray, u: np.ndarray):
    """Draft tokens drawn from the drafter's distributions [SD section 2: each draft
    token is sampled from the draft model's q; SL: q = softmax of the low-rank head's
    logits]: row r gives _draw(q[r], u[r]) -- inverse CDF over ascending ids of the
    stored fp32 probabilities (not renormalised; S is their sum).  Returns (tok int32
    [rows], flags int32 [rows]: FLAG_CDF_TIE on a near tie)."""
    q = np.asarray(q, dtype=np.float32)
    rows = q.shape[0]
    tok = np.zeros(rows, dtype=np.int32)
    flags = np.zeros(rows, dtype=np.int32)
    for r in range(rows):
        k, tie, _ = _draw(q[r].astype(np.float64), float(u[r]))
        tok[r] = k
        flags[r] = FLAG_CDF_TIE if tie else 0
    return tok, flags


def rho_tps(nu: float, rho_tau: float, kappa: float) -> float:
    """End-to-end speed-up of a faster draft head [SL, "이론적 프레임워크"]:
    rho_TPS = rho_tau * (1 + kappa) / (1 + nu * kappa), with nu = new head time /
    full head time, rho_tau = acceptance-length ratio, kappa = full head time / time
    of the rest of the drafting pipeline."""
    return rho_tau * (1.0 + kappa) / (1.0 + nu * kappa)


def reject_sample(root_logits, logits, q, cand_tok, cand_len, u_acc, u_res,
                  temperature: float = 1.0, gate=None):
    """Leviathan/Chen acceptance over W independent candidate chains, keeping the
    longest accepted run.

    p at a position is softmax(z/T) of the row that precedes it: the root logits for
    offset 0, row (i, o-1) of the verify pass otherwise (row (i, o) holds token
    (i, o) and judges token (i, o+1)).  Draft token x at (i, o) is accepted iff
    u_acc[i,o] * Q < p(x), with Q = q[(i,o)][x] (dense drafts) or 1 (q is None:
    deterministic copy drafts, a point mass on x).  This is alpha = min(1, p/q) of
    section 3, written so that p >= q always accepts.  The chain stops at the first
    rejection.  a_i = accepted length of candidate i; the chosen candidate is the
    one with the longest run, ties to the smallest index.  After its a accepted
    tokens one more token is drawn:
      rejection at offset a: residual max(0, P - Qd), Qd the draft distribution at
                             (i*, a) (a point mass on the draft token for copy drafts)
      all accepted:          the bonus distribution softmax(row (i*, len-1))
    by inverse CDF with u_res[i*].  Uniforms are indexed by position, not consumed.
    Returns a dict of per-sequence results."""
    root_logits = np.asarray(root_logits, dtype=np.float32)
    logits = np.asarray(logits, dtype=np.float32)
    B, W, D = cand_tok.shape
    V = root_logits.shape[1]
    M = W * D
    T = float(temperature)
    z_root = root_logits.astype(np.float64) / T
    lse_root = _logsumexp_rows(z_root)
    out = dict(
        n_acc=np.zeros(B, dtype=np.int32), best=np.full(B, -1, dtype=np.int32),
        out_tok=np.full((B, D + 1), -1, dtype=np.int32), n_out=np.zeros(B, dtype=np.int32),
        acc_per_cand=np.zeros((B, W), dtype=np.int32), flags=np.zeros(B, dtype=np.int32),
        abs_tie=np.zeros(B, dtype=bool),
        # diagnostics: smallest relative distance of a decisive acceptance test from its
        # threshold, and of the final draw from the nearest CDF step (fraction of S)
        accept_margin=np.full(B, np.inf), cdf_margin=np.full(B, np.inf),
    )
    lse_cache = {}

    def row_p(b, prow):
        """Target distribution (fp64) at the row that judges the next token."""
        if prow < 0:
            return np.exp(z_root[b] - lse_root[b])
        r = b * M + prow
        if r not in lse_cache:
            zz = logits[r].astype(np.float64) / T
            m = zz.max()
            lse_cache[r] = (zz, m + np.log(np.exp(zz - m).sum()))
        zz, l = lse_cache[r]
        return np.exp(zz - l)

    for b in range(B):
        flags = 0
        lens = np.asarray(cand_len[b]).copy()
        if gate is not None and not gate[b]:
            lens[:] = 0
        a = np.zeros(W, dtype=np.int64)
        for i in range(W):
            if lens[i] < 1:
                continue
            a[i] = lens[i]
            for o in range(lens[i]):
                x = int(cand_tok[b, i, o])
                prow = -1 if o == 0 else i * D + o - 1
                if 0 <= x < V:
                    p = row_p(b, prow)[x]
                    Q = 1.0 if q is None else float(q[b * M + i * D + o, x])
                else:
                    flags |= FLAG_BAD_TOKEN
                    p, Q = 0.0, 1.0
                lhs = u_acc[b, i, o] * Q
                if max(p, lhs) > 0:
                    out["accept_margin"][b] = min(out["accept_margin"][b],
                                                  abs(lhs - p) / max(p, lhs))
                if abs(lhs - p) < ACCEPT_TIE_REL * max(p, lhs):
                    flags |= FLAG_ACCEPT_TIE
                if abs(lhs - p) < 1e-4:
                    out["abs_tie"][b] = True
                if not (lhs < p):
                    a[i] = o
                    break
        out["acc_per_cand"][b] = a
        have = np.nonzero(lens >= 1)[0]
        if len(have) == 0:
            # no candidate: one token from the target distribution at the current token
            r = row_p(b, -1)
            y, tie, out["cdf_margin"][b] = _draw(r, u_res[b, 0])
            out["out_tok"][b, 0] = y
            out["n_out"][b] = 1
            out["n_acc"][b] = 0
            out["best"][b] = -1
            out["flags"][b] = flags | FLAG_NO_CANDIDATE | (FLAG_CDF_TIE if tie else 0)
            continue
        best = int(have[np.argmax(a[have])])          # argmax returns the first maximum
        ab = int(a[best])
        out["best"][b] = best
        out["n_acc"][b] = ab
        out["out_tok"][b, :ab] = cand_tok[b, best, :ab]
        prow = -1 if ab == 0 else best * D + ab - 1
        P = row_p(b, prow)
        if ab < lens[best]:
            x = int(cand_tok[b, best, ab])
            if q is None:
                Qd = np.zeros(V)
                if 0 <= x < V:
                    Qd[x] = 1.0
            else:
                Qd = q[b * M + best * D + ab].astype(np.float64)
            r = np.maximum(0.0, P - Qd)
        else:
            r = P
        if not (r.sum() > 0.0):
            r = P
            flags |= FLAG_DEGENERATE
        y, tie, out["cdf_margin"][b] = _draw(r, u_res[b, best])
        if tie:
            flags |= FLAG_CDF_TIE
        out["out_tok"][b, ab] = y
        out["n_out"][b] = ab + 1
        out["flags"][b] = flags
    return out


def reject_sample_multi(root_logits, logits, q, cand_tok, cand_len, u_acc, u_res,
                        temperature: float = 1.0, gate=None):
    """Lossless acceptance over W candidates: recursive residual across the sibling
    candidates at each depth (built from [SD] section 3's single-draft rule and its
    residual).

    Depth a starts from the target distribution P of the reference row: the root for
    a = 0, else row (ref, a-1), ref being the smallest surviving candidate.  The
    siblings at depth a are the surviving candidates i with len_i > a, in index
    order; candidate i proposes x_i = cand[i, a] with draft distribution Q_i =
    q[(i, a)] (a point mass on x_i when q is None).  With the current residual p'
    (initially P), sibling i is accepted iff u_acc[i, a] * Q_i(x_i) < p'(x_i) -- the
    min(1, p'/q) rule -- and otherwise p' <- max(0, p' - Q_i), renormalised (if that
    leaves no mass, p' is kept and DEGENERATE flagged).  An accepted x is emitted and
    the survivors become the siblings whose token at depth a is x.  If every sibling
    is rejected, one token is drawn from p' with u_res[i_last] (the last sibling
    tested); if no survivor has a token at depth a, a bonus token is drawn from P
    with u_res[ref].  Each rejection removes exactly the mass the draft claimed, so
    the emitted token follows P at every depth whenever the drafts are independent
    draws from their Q (for copy drafts Q is the point mass they are).

    best = the final reference candidate; acc_per_cand[i] = the length of the
    common prefix of candidate i with the accepted tokens.  Same outputs and flags
    as reject_sample."""
    root_logits = np.asarray(root_logits, dtype=np.float32)
    logits = np.asarray(logits, dtype=np.float32)
    B, W, D = cand_tok.shape
    V = root_logits.shape[1]
    M = W * D
    T = float(temperature)
    z_root = root_logits.astype(np.float64) / T
    lse_root = _logsumexp_rows(z_root)
    out = dict(
        n_acc=np.zeros(B, dtype=np.int32), best=np.full(B, -1, dtype=np.int32),
        out_tok=np.full((B, D + 1), -1, dtype=np.int32), n_out=np.zeros(B, dtype=np.int32),
        acc_per_cand=np.zeros((B, W), dtype=np.int32), flags=np.zeros(B, dtype=np.int32),
        accept_margin=np.full(B, np.inf), cdf_margin=np.full(B, np.inf),
    )

    def row_p(b, prow):
        if prow < 0:
            return np.exp(z_root[b] - lse_root[b])
        zz = logits[b * M + prow].astype(np.float64) / T
        m = zz.max()
        return np.exp(zz - (m + np.log(np.exp(zz - m).sum())))

    for b in range(B):
        flags = 0
        lens = np.clip(np.asarray(cand_len[b]).copy(), 0, D)
        if gate is not None and not gate[b]:
            lens[:] = 0
        surv = [i for i in range(W) if lens[i] >= 1]
        if not surv:
            y, tie, out["cdf_margin"][b] = _draw(row_p(b, -1), u_res[b, 0])
            out["out_tok"][b, 0] = y
            out["n_out"][b] = 1
            out["flags"][b] = FLAG_NO_CANDIDATE | (FLAG_CDF_TIE if tie else 0)
            continue
        a = 0
        acc = []
        y = None
        while True:
            ref = surv[0]
            P = row_p(b, -1 if a == 0 else ref * D + a - 1)
            sib = [i for i in surv if lens[i] > a]
            if not sib:
                y, tie, out["cdf_margin"][b] = _draw(P, u_res[b, ref])
                break
            r = P.copy()
            accepted = None
            last = sib[0]
            for i in sib:
                last = i
                x = int(cand_tok[b, i, a])
                if q is None:
                    Qi = np.zeros(V)
                    if 0 <= x < V:
                        Qi[x] = 1.0
                else:
                    Qi = q[b * M + i * D + a].astype(np.float64)
                if 0 <= x < V:
                    pp = r[x] / r.sum()
                    Qx = Qi[x] if q is not None else 1.0
                else:
                    flags |= FLAG_BAD_TOKEN
                    pp, Qx = 0.0, 1.0
                lhs = u_acc[b, i, a] * Qx
                if max(pp, lhs) > 0:
                    out["accept_margin"][b] = min(out["accept_margin"][b],
                                                  abs(lhs - pp) / max(pp, lhs))
                if abs(lhs - pp) < ACCEPT_TIE_REL * max(pp, lhs):
                    flags |= FLAG_ACCEPT_TIE
                if lhs < pp:
                    accepted = x
                    break
                rn = np.maximum(0.0, r / r.sum() - Qi)
                if rn.sum() > 0.0:
                    r = rn
                else:
                    flags |= FLAG_DEGENERATE
            if accepted is None:
                y, tie, out["cdf_margin"][b] = _draw(r, u_res[b, last])
                break
            acc.append(accepted)
            surv = [i for i in sib if int(cand_tok[b, i, a]) == accepted]
            a += 1
        if tie:
            flags |= FLAG_CDF_TIE
        out["best"][b] = surv[0]
        out["n_acc"][b] = a
        out["out_tok"][b, :a] = acc
        out["out_tok"][b, a] = y
        out["n_out"][b] = a + 1
        for i in range(W):
            k = 0
            while k < min(lens[i], a) and int(cand_tok[b, i, k]) == acc[k]:
                k += 1
            out["acc_per_cand"][b, i] = k
        out["flags"][b] = flags
    return out


def _row_argmax(z: np.ndarray):
    """First index of the largest value, and whether the two largest values are within
    GREEDY_TIE_REL * max(1, |largest|) of each other (a near tie)."""
    z = np.asarray(z, dtype=np.float64)
    k = int(np.argmax(z))
    if z.size < 2:
        return k, False
    top2 = np.partition(z, z.size - 2)[-2:]
    gap = float(top2[1] - top2[0])
    return k, gap < GREEDY_TIE_REL * max(1.0, abs(float(top2[1])))


def reject_sample_greedy(root_logits, logits, cand_tok, cand_len, gate=None):
    """Greedy verification (temperature 0).

    The limit T -> 0 of section 3's rule [SD], where every target p becomes the point
    mass on its row's argmax: a draft token is accepted iff it is the argmax of the
    preceding row (root for offset 0, row (i, o-1) otherwise), a candidate's run
    stops at its first other token ([EX] step 2: cut at the first mismatch), and the
    extra token is the argmax of the row after the run (the residual of a point mass
    p against any rejected draft is that same point mass, and so is the bonus p).
    The draft distribution and the uniforms play no part.  Over W candidates the
    longest run is kept (ties: smallest index), and since every p is a point mass
    this emits exactly what plain greedy decoding emits, for any W.

    argmax is taken over the fp32 logits as given, first index among equal maxima.
    A tested position whose row has a near tie (_row_argmax) flags ACCEPT_TIE; a near
    tie in the row of the extra token flags CDF_TIE.  Same outputs as reject_sample."""
    root_logits = np.asarray(root_logits, dtype=np.float32)
    logits = np.asarray(logits, dtype=np.float32)
    B, W, D = cand_tok.shape
    V = root_logits.shape[1]
    M = W * D
    out = dict(
        n_acc=np.zeros(B, dtype=np.int32), best=np.full(B, -1, dtype=np.int32),
        out_tok=np.full((B, D + 1), -1, dtype=np.int32), n_out=np.zeros(B, dtype=np.int32),
        acc_per_cand=np.zeros((B, W), dtype=np.int32), flags=np.zeros(B, dtype=np.int32),
    )

    def row(b, prow):
        return root_logits[b] if prow < 0 else logits[b * M + prow]

    for b in range(B):
        flags = 0
        lens = np.clip(np.asarray(cand_len[b]).copy(), 0, D)
        if gate is not None and not gate[b]:
            lens[:] = 0
        a = np.zeros(W, dtype=np.int64)
        for i in range(W):
            a[i] = lens[i]
            for o in range(lens[i]):
                x = int(cand_tok[b, i, o])
                g, tie = _row_argmax(row(b, -1 if o == 0 else i * D + o - 1))
                if tie:
                    flags |= FLAG_ACCEPT_TIE
                if not (0 <= x < V):
                    flags |= FLAG_BAD_TOKEN
                if x != g:
                    a[i] = o
                    break
        out["acc_per_cand"][b] = a
        have = [i for i in range(W) if lens[i] >= 1]
        if not have:
            y, tie = _row_argmax(row(b, -1))
            out["out_tok"][b, 0] = y
            out["n_out"][b] = 1
            out["flags"][b] = FLAG_NO_CANDIDATE | (FLAG_CDF_TIE if tie else 0)
            continue
        best = have[0]
        for i in have:
            if a[i] > a[best]:
                best = i
        ab = int(a[best])
        y, tie = _row_argmax(row(b, -1 if ab == 0 else best * D + ab - 1))
        if tie:
            flags |= FLAG_CDF_TIE
        out["best"][b] = best
        out["n_acc"][b] = ab
        out["out_tok"][b, :ab] = cand_tok[b, best, :ab]
        out["out_tok"][b, ab] = y
        out["n_out"][b] = ab + 1
        out["flags"][b] = flags
    return out


# ----------------------------------------------------------------------------------
# KV commit and rollback over the paged pool  [SD6]
#
# Pool model: pages of `page` tokens, K pages [n_pages, Hkv, page, hd] and V pages
# transposed [n_pages, Hkv, hd, page] (token_major gives the token-major view);
# page_table[b, j] = pool page of tokens j*page .. j*page+page-1 of sequence b; a
# free-page stack free_list[0 .. n_free) whose top is free_list[n_free - 1].

def _pages_for(n_tokens: int, page: int) -> int:
    return (n_tokens + page - 1) // page


def kv_commit(k_pool, v_pool, page_table, prefix_len, free_list, n_free, k_cand, v_cand,
              best, n_acc, W, D, page=16):
    """Append each sequence's accepted rows to its paged KV cache.

    Sequence b's accepted rows are rows (best[b], 0 .. a-1), a = n_acc[b] clipped to
    [0, D], of the candidate K/V buffers ([B*W*D, Hkv, hd], row (b, i, o) at
    b*W*D + i*D + o); they become tokens P .. P+a-1, P = prefix_len[b].  Pages
    beyond the ones the prefix already holds are popped from the free stack, in
    sequence order and, within a sequence, in page order.  Nothing happens for a
    sequence with best < 0 or a = 0.  A sequence is skipped (nothing written, no
    page taken) with FLAG_BAD_PAGE when P + a exceeds the page table, when P is out
    of range, when a page it would write (its partly filled last page, or a popped
    one) is not a pool page, or when n_free itself is outside [0, n_pages] (the
    stack is then not read); with FLAG_POOL_EMPTY when the stack holds fewer pages
    than it needs.  Returns copies: (k_pool, v_pool, page_table, prefix_len,
    free_list, n_free, flags)."""
    k_pool = np.array(k_pool, copy=True)
    v_pool = np.array(v_pool, copy=True)
    page_table = np.array(page_table, dtype=np.int32, copy=True)
    prefix_len = np.array(prefix_len, dtype=np.int32, copy=True)
    free_list = np.array(free_list, dtype=np.int32, copy=True)
    n_free = int(n_free)
    B, max_pages = page_table.shape
    n_pages = k_pool.shape[0]
    M = W * D
    Kt, Vt = token_major(k_pool, "k"), token_major(v_pool, "v")   # views: writes land in the pools
    flags = np.zeros(B, dtype=np.int32)
    stack_ok = 0 <= n_free <= n_pages
    for b in range(B):
        i = int(best[b])
        a = min(max(int(n_acc[b]), 0), D)
        if i < 0 or i >= W or a == 0:
            continue
        P = int(prefix_len[b])
        if not stack_ok or P < 0 or P + a > max_pages * page:
            flags[b] |= FLAG_BAD_PAGE
            continue
        have = _pages_for(P, page)
        need = _pages_for(P + a, page) - have
        if P % page and not (0 <= page_table[b, have - 1] < n_pages):
            flags[b] |= FLAG_BAD_PAGE
            continue
        if need > n_free:
            flags[b] |= FLAG_POOL_EMPTY
            continue
        new = [int(free_list[n_free - 1 - k]) for k in range(need)]
        if any(not (0 <= pg < n_pages) for pg in new):
            flags[b] |= FLAG_BAD_PAGE
            continue
        n_free -= need
        page_table[b, have:have + need] = new
        for o in range(a):
            pos = P + o
            pg = page_table[b, pos // page]
            Kt[pg, pos % page] = k_cand[b * M + i * D + o]
            Vt[pg, pos % page] = v_cand[b * M + i * D + o]
        prefix_len[b] = P + a
    return k_pool, v_pool, page_table, prefix_len, free_list, n_free, flags


def kv_commit_layers(k_pools, v_pools, page_table, prefix_len, free_list, n_free, k_cands,
                     v_cands, best, n_acc, W, D, page=16):
    """kv_commit for L layers that share one block table [SD6].  Reading: the decision
    which pages a sequence takes is made once (it depends only on the table, the
    lengths and the free stack), and every layer's accepted rows are then written at
    the same (page, slot) of that layer's pool.  Equivalently: kv_commit applied to
    each layer alone from the same table and stack gives the same new table, lengths,
    stack and flags for every layer, and the layers' pools.  Arrays with a leading
    layer axis: k_pools/v_pools [L, n_pages, ...], k_cands/v_cands [L, B*W*D, Hkv, hd].
    Returns copies: (k_pools, v_pools, page_table, prefix_len, free_list, n_free,
    flags)."""
    L = k_pools.shape[0]
    ks, vs = [], []
    res = None
    for l in range(L):
        r = kv_commit(k_pools[l], v_pools[l], page_table, prefix_len, free_list, n_free,
                      k_cands[l], v_cands[l], best, n_acc, W, D, page)
        ks.append(r[0])
        vs.append(r[1])
        res = r
    return (np.stack(ks), np.stack(vs)) + tuple(res[2:])


def kv_truncate(page_table, prefix_len, new_len, free_list, n_free, n_pages, page=16):
    """Roll sequences back to new_len[b] tokens: the pages past the ones new_len needs
    return to the free stack (sequence order, ascending page index within a sequence,
    so the last page pushed is the sequence's highest) and their page-table entries
    become -1.  Token data is not touched.  A sequence is skipped with FLAG_BAD_PAGE
    when new_len is outside [0, prefix_len[b]], when prefix_len is out of range,
    when a page to free is not a pool page, when the stack would overflow, or (all
    sequences) when n_free itself is outside [0, n_pages].  Returns copies: (page_table, prefix_len,
    free_list, n_free, flags)."""
    page_table = np.array(page_table, dtype=np.int32, copy=True)
    prefix_len = np.array(prefix_len, dtype=np.int32, copy=True)
    free_list = np.array(free_list, dtype=np.int32, copy=True)
    n_free = int(n_free)
    B, max_pages = page_table.shape
    flags = np.zeros(B, dtype=np.int32)
    stack_ok = 0 <= n_free <= n_pages
    for b in range(B):
        P, L = int(prefix_len[b]), int(new_len[b])
        if not stack_ok or P < 0 or P > max_pages * page or L < 0 or L > P:
            flags[b] |= FLAG_BAD_PAGE
            continue
        keep, have = _pages_for(L, page), _pages_for(P, page)
        freed = [int(page_table[b, j]) for j in range(keep, have)]
        if any(not (0 <= pg < n_pages) for pg in freed) or n_free + len(freed) > n_pages:
            flags[b] |= FLAG_BAD_PAGE
            continue
        for pg in freed:
            free_list[n_free] = pg
            n_free += 1
        page_table[b, keep:have] = -1
        prefix_len[b] = L
    return page_table, prefix_len, free_list, n_free, flags


# ----------------------------------------------------------------------------------
# a7: the whole verify step

def verify_step(case_arrays: dict, shape, drafts=None, q_override=None, accept: str = "longest"):
    """copy_match -> probe_gate -> verify_attention -> lm_head -> reject_sample on one
    batch.  `drafts` = (cand_tok, cand_len) for the neural-draft path (copy retrieval
    skipped, gate open).  accept = "longest" (the pages' longest verified run),
    "multi" (reject_sample_multi) or "greedy" (reject_sample_greedy).  Returns every
    stage's outputs."""
    A = case_arrays
    sh = shape
    res = {}
    if drafts is None:
        cm = copy_match(A["ctx"], A["ctx_off"], sh.kappa, sh.W, sh.D)
        pg = probe_gate(as_f64(A["probe_h"], sh.dtype), A["probe_w"], sh.tau, cm["n_found"])
        cand_tok, cand_len, gate = cm["cand_tok"], cm["cand_len"], pg["gate"]
        res.update(copy=cm, probe=pg)
    else:
        cand_tok, cand_len = drafts
        gate = np.ones(sh.B, dtype=np.int32)
    O, O_r, aflags = verify_attention(
        as_f64(A["q"], sh.dtype), as_f64(A["k_cand"], sh.dtype), as_f64(A["v_cand"], sh.dtype),
        as_f64(A["k_pool"], sh.dtype), as_f64(A["v_pool"], sh.dtype), A["page_table"],
        A["prefix_len"], sh.B, sh.W, sh.D, sh.Hq, sh.Hkv, out_dtype=sh.dtype)
    H = O_r.reshape(O_r.shape[0], -1)
    logits, lse = lm_head_full(H, A["w_full"], sh.temperature, sh.dtype)
    q = q_override if q_override is not None else A.get("q_draft")
    if accept == "greedy":
        rs = reject_sample_greedy(A["root_logits"], logits, cand_tok, cand_len, gate)
    else:
        rule = reject_sample_multi if accept == "multi" else reject_sample
        rs = rule(A["root_logits"], logits, q, cand_tok, cand_len, A["u_acc"], A["u_res"],
                  sh.temperature, gate)
    res.update(attn=O_r, attn_exact=O, attn_flags=aflags, logits=logits, lse=lse, sample=rs,
               cand_tok=cand_tok, cand_len=cand_len, gate=gate)
    return res
