"""Seeded synthetic inputs for the speculative-decoding verify step.

This module only *makes data*: it holds none of the verify step's arithmetic
(no attention, no head projection, no probe score, no acceptance test).  Both
the CPU oracle's tests and the GPU path read the arrays it returns; neither
side imports the other.

Workloads follow the pages' model shapes:
  * tiny        -- fp32 toy verify step (d=64, 4/2 heads, hd=16, P=128, W=2, D=4, V=512)
  * llama8b     -- Llama-3.1-8B shape (d=4096, 32/8 heads, hd=128, P=4096, W=4, D=20,
                   V=128256); D=20 is the 20-token speculation maximum of the SwitchSD
                   summary ("Assumptions & limits", its section 4.2)
  * slimspec    -- SlimSpec low-rank draft head (d=4096, r=d/8=512, V=128256, gamma=7
                   drafts) followed by a Llama-8B-shaped verify with W=1, D=7
  * llama70b    -- Llama-3.3-70B shape (d=8192, 64/8 heads, P=16384, W=8, D=20)
  * ragged      -- 32 sequences, prefix U{512..8192}, W=4, D=8, paged KV (16-token
                   pages) in random page order, point-mass copy drafts

Token contexts are finite-Zipf(1.1) ids with planted verbatim repeats, standing in
for the repetition-heavy benchmark prompts of the SwitchSD summary (the copy label
is a verbatim run of >= 5 earlier tokens, "How it works").  No dataset items are used.

Random numbers: numpy ``default_rng(SeedSequence(seed))`` with child streams
spawned in a fixed order (see ``_STREAMS``).  bf16 tensors are produced by
round-to-nearest-even of fp32 draws and are handed out as raw uint16 bit
patterns; the consumer decodes them itself.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

# Child-stream order (fixed; appending new streams at the end keeps old data stable).
_STREAMS = (
    "ctx", "plants", "probe_h", "probe_w", "q", "kv_prefix", "kv_cand", "head",
    "w_down", "w_up", "draft_h", "q_logits", "root", "u_acc", "u_res", "u_draft",
    "prefix_len", "page_perm",
)

PAGE = 16          # KV page size in tokens
KAPPA = 5          # kappa-gram length of the copy trigger
TAU = 0.4          # probe threshold reported for Llama-3.1-8B


@dataclass(frozen=True)
class Shape:
    """All sizes of one verify-step workload.  Every field is a runtime value."""
    name: str
    dtype: str                 # "f32" or "bf16": model tensors (Q/K/V, head, probe h)
    B: int                     # sequences
    W: int                     # copy candidates per sequence
    D: int                     # tokens per candidate
    Hq: int
    Hkv: int
    hd: int
    d: int                     # hidden size (= Hq*hd: the attention output feeds the head)
    V: int                     # vocabulary
    P: tuple                   # prefix length per sequence (= context length)
    rank: int = 0              # >0: low-rank draft head of this rank (SlimSpec)
    gamma: int = 0             # drafts produced by the low-rank head
    q_mode: str = "dense"      # "dense" fp32 draft probabilities, or "point" (copy drafts)
    q_sigma: float = 2.0       # std of the draft logits behind dense q
    copy_density: float = 0.10 # fraction of context positions covered by planted repeats
    plant_len: tuple = (5, 40) # planted repeat length range (inclusive)
    paged_random: bool = False # random page order (else identity page table)
    external_drafts: bool = False  # drafts come from a neural drafter, not copy_match
    root_sigma: float = 1.0    # std of the root (previous-step) target logits
    temperature: float = 1.0
    tau: float = TAU
    kappa: int = KAPPA

    @property
    def M(self) -> int:
        return self.W * self.D

    @property
    def g(self) -> int:
        return self.Hq // self.Hkv

    def with_(self, **kw) -> "Shape":
        return dataclasses.replace(self, **kw)


def _cfg_tiny() -> Shape:
    return Shape("tiny", "f32", B=1, W=2, D=4, Hq=4, Hkv=2, hd=16, d=64, V=512,
                 P=(128,), q_sigma=1.0)


def _cfg_llama8b() -> Shape:
    return Shape("llama8b", "bf16", B=1, W=4, D=20, Hq=32, Hkv=8, hd=128, d=4096,
                 V=128256, P=(4096,))


def _cfg_slimspec() -> Shape:
    return Shape("slimspec", "bf16", B=1, W=1, D=7, Hq=32, Hkv=8, hd=128, d=4096,
                 V=128256, P=(4096,), rank=512, gamma=7, external_drafts=True)


def _cfg_llama70b() -> Shape:
    return Shape("llama70b", "bf16", B=1, W=8, D=20, Hq=64, Hkv=8, hd=128, d=8192,
                 V=128256, P=(16384,), plant_len=(5, 60))


def _cfg_ragged(seed: int = 5000) -> Shape:
    rng = np.random.default_rng(np.random.SeedSequence(seed).spawn(len(_STREAMS))[
        _STREAMS.index("prefix_len")])
    P = tuple(int(x) for x in rng.integers(512, 8192, size=32, endpoint=True))
    return Shape("ragged", "bf16", B=32, W=4, D=8, Hq=32, Hkv=8, hd=128, d=4096,
                 V=128256, P=P, q_mode="point", copy_density=0.05, paged_random=True)


CONFIGS = {
    1: _cfg_tiny,
    2: _cfg_llama8b,
    3: _cfg_slimspec,
    4: _cfg_llama70b,
    5: _cfg_ragged,
}
CONFIG_SEED = {c: 1000 * c for c in CONFIGS}


def config(c: int) -> Shape:
    return CONFIGS[c]()


# ----------------------------------------------------------------------------------
# data-format helpers (not arithmetic of the method)

def f32_to_bf16_bits(x: np.ndarray, block: int = 1 << 24) -> np.ndarray:
    """Round fp32 values to bf16 (round to nearest, ties to even); return uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    xf = x.reshape(-1)
    of = out.reshape(-1)
    for s in range(0, xf.size, block):
        u = xf[s:s + block].view(np.uint32)
        bias = ((u >> 16) & 1) + np.uint32(0x7FFF)
        of[s:s + block] = ((u + bias) >> 16).astype(np.uint16)
    return out


def _normal_bf16(rng: np.random.Generator, shape, std: float, block: int = 1 << 24):
    """N(0, std^2) draws in fp32, rounded to bf16 bits, generated in blocks."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    for s in range(0, n, block):
        m = min(block, n - s)
        v = rng.standard_normal(m, dtype=np.float32)
        if std != 1.0:
            v *= np.float32(std)
        out[s:s + m] = f32_to_bf16_bits(v)
    return out.reshape(shape)


def _normal_model(rng, shape, std, dtype):
    if dtype == "bf16":
        return _normal_bf16(rng, shape, std)
    v = rng.standard_normal(int(np.prod(shape)), dtype=np.float32).reshape(shape)
    if std != 1.0:
        v *= np.float32(std)
    return v


def zipf_table(V: int, s: float = 1.1) -> np.ndarray:
    """Finite Zipf law P(k) ~ k^-s over ranks k = 1..V (token id = k-1)."""
    w = np.arange(1, V + 1, dtype=np.float64) ** (-s)
    return w / w.sum()


# ----------------------------------------------------------------------------------
# contexts with planted repeats

def _plant_repeats(rng, ctx: np.ndarray, density: float, plant_len, limit: int, kappa: int):
    """Copy earlier spans of ctx onto later positions until `density` of the
    positions in [0, limit) are covered.  Returns the list of (src, dst, length)."""
    L = limit
    covered = np.zeros(len(ctx), dtype=bool)
    plants = []
    lo, hi = plant_len
    target = int(round(density * L))
    tries = 0
    while covered[:L].sum() < target and tries < 100000:
        tries += 1
        ln = int(rng.integers(lo, hi, endpoint=True))
        if L < 2 * ln + 1:
            break
        dst = int(rng.integers(ln, L - ln + 1))
        src = int(rng.integers(0, dst - ln + 1))
        if covered[dst:dst + ln].any():
            continue
        ctx[dst:dst + ln] = ctx[src:src + ln]
        covered[dst:dst + ln] = True
        plants.append((src, dst, ln))
    return plants


def _forced_trailing_plant(rng, ctx: np.ndarray, W: int, D: int, kappa: int):
    """Copy the trailing kappa-gram (the current token's key) to W earlier end
    positions, each followed by at least D tokens, spaced kappa+D apart.
    Returns the planted end positions, most recent first."""
    L = len(ctx)
    t = L - 1
    key = ctx[t - kappa + 1:t + 1].copy()
    ends = []
    stride = kappa + D
    for w in range(W):
        j = t - D - 1 - w * stride
        if j - kappa + 1 < 0:
            break
        ctx[j - kappa + 1:j + 1] = key
        ends.append(j)
    return ends


def make_context(rng_ctx, rng_plants, L: int, V: int, density: float, plant_len, W: int,
                 D: int, kappa: int, forced: bool, zipf: Optional[np.ndarray] = None,
                 uniform: bool = False):
    if uniform:
        ctx = rng_ctx.integers(0, V, size=L).astype(np.int32)
    else:
        p = zipf if zipf is not None else zipf_table(V)
        ctx = rng_ctx.choice(V, size=L, p=p).astype(np.int32)
    reserve = (W + 1) * (kappa + D) + kappa if forced else 0
    limit = max(0, L - reserve)
    plants = _plant_repeats(rng_plants, ctx, density, plant_len, limit, kappa) if density > 0 else []
    ends = _forced_trailing_plant(rng_plants, ctx, W, D, kappa) if forced else []
    return ctx, plants, ends


# ----------------------------------------------------------------------------------

@dataclass
class Case:
    shape: Shape
    variant: str
    seed: int
    arrays: dict = field(default_factory=dict)
    meta: dict = field(default_factory=dict)

    def __getitem__(self, k):
        return self.arrays[k]


def make_case(shape: Shape, seed: int, variant: str = "measure",
              with_head: bool = True, with_q: bool = True) -> Case:
    """Build every input of one verify step.

    variant:
      "measure" -- forced-open gate: the trailing kappa-gram is planted W times with
                   full-length continuations and the probe input is sign-matched to w
                   (so w.h > 0 and the probe fires without evaluating it here).
      "natural" -- no forced plant; probe input h ~ N(0,1).

    Arrays (model tensors are uint16 bf16 bits when shape.dtype == "bf16"):
      ctx int32 [sum P], ctx_off int32 [B+1]
      probe_h [B,d], probe_w f32 [d]
      q [B*M, Hq, hd], k_cand/v_cand [B*M, Hkv, hd]
      k_pool [n_pages, Hkv, 16, hd], v_pool [n_pages, Hkv, hd, 16] (V transposed in a page),
      page_table int32 [B, max_pages], prefix_len int32 [B]
      w_full [V, d]   (with_head)
      w_down [r, d], w_up [V, r], draft_h [gamma, d]  (rank > 0)
      q_draft f32 [B*M, V]  (q_mode == "dense" and with_q)
      root_logits f32 [B, V]
      u_acc f64 [B, W, D], u_res f64 [B, W], u_draft f64 [B, W, D]
    """
    sh = shape
    ss = np.random.SeedSequence(seed)
    kids = ss.spawn(len(_STREAMS))
    R = {name: np.random.default_rng(k) for name, k in zip(_STREAMS, kids)}
    A = {}
    meta = {}
    B, W, D, M = sh.B, sh.W, sh.D, sh.M
    forced = variant == "measure"

    # --- contexts (one per sequence, CSR) ---
    zipf = None if sh.name == "tiny" else zipf_table(sh.V)
    ctxs, plants, ends = [], [], []
    for b in range(B):
        if sh.name == "tiny":
            # uniform ids with exactly one planted 5-token repeat ending before t
            L = sh.P[b]
            c = R["ctx"].integers(0, sh.V, size=L).astype(np.int32)
            s = int(R["plants"].integers(0, L - 2 * sh.kappa, endpoint=True))  # s in [0, L-10]
            c[L - sh.kappa:L] = c[s:s + sh.kappa]
            ctxs.append(c)
            plants.append([(s, L - sh.kappa, sh.kappa)])
            ends.append([s + sh.kappa - 1])
        else:
            c, pl, en = make_context(R["ctx"], R["plants"], sh.P[b], sh.V, sh.copy_density,
                                     sh.plant_len, W, D, sh.kappa, forced, zipf)
            ctxs.append(c)
            plants.append(pl)
            ends.append(en)
    A["ctx"] = np.concatenate(ctxs).astype(np.int32)
    A["ctx_off"] = np.concatenate([[0], np.cumsum([len(c) for c in ctxs])]).astype(np.int32)
    meta["plants"] = plants
    meta["forced_ends"] = ends

    # --- probe ---
    w = (R["probe_w"].standard_normal(sh.d) / np.sqrt(sh.d)).astype(np.float32)
    h = R["probe_h"].standard_normal((B, sh.d)).astype(np.float32)
    if forced:
        h = np.abs(h) * np.where(w >= 0, 1.0, -1.0).astype(np.float32)[None, :]
    A["probe_w"] = w
    A["probe_h"] = f32_to_bf16_bits(h) if sh.dtype == "bf16" else h

    # --- attention tensors ---
    A["q"] = _normal_model(R["q"], (B * M, sh.Hq, sh.hd), 1.0, sh.dtype)
    A["k_cand"] = _normal_model(R["kv_cand"], (B * M, sh.Hkv, sh.hd), 1.0, sh.dtype)
    A["v_cand"] = _normal_model(R["kv_cand"], (B * M, sh.Hkv, sh.hd), 1.0, sh.dtype)
    pages_per = [-(-p // PAGE) for p in sh.P]
    n_pages = int(sum(pages_per))
    max_pages = int(max(pages_per))
    # paged cache, head-major pages: K [page, kv head, token, hd]; V [page, kv head, hd, token]
    A["k_pool"] = _normal_model(R["kv_prefix"], (n_pages, sh.Hkv, PAGE, sh.hd), 1.0, sh.dtype)
    A["v_pool"] = _normal_model(R["kv_prefix"], (n_pages, sh.Hkv, sh.hd, PAGE), 1.0, sh.dtype)
    if sh.paged_random:
        perm = R["page_perm"].permutation(n_pages).astype(np.int32)
    else:
        perm = np.arange(n_pages, dtype=np.int32)
    pt = np.full((B, max_pages), -1, dtype=np.int32)
    o = 0
    for b in range(B):
        pt[b, :pages_per[b]] = perm[o:o + pages_per[b]]
        o += pages_per[b]
    A["page_table"] = pt
    A["prefix_len"] = np.asarray(sh.P, dtype=np.int32)
    meta["n_pages"] = n_pages
    meta["max_pages"] = max_pages

    # --- heads ---
    if with_head:
        A["w_full"] = _normal_model(R["head"], (sh.V, sh.d), 1.0 / np.sqrt(sh.d), sh.dtype)
    if sh.rank > 0:
        A["w_down"] = _normal_model(R["w_down"], (sh.rank, sh.d), 1.0 / np.sqrt(sh.d), sh.dtype)
        A["w_up"] = _normal_model(R["w_up"], (sh.V, sh.rank), 1.0 / np.sqrt(sh.rank), sh.dtype)
        A["draft_h"] = _normal_model(R["draft_h"], (sh.gamma, sh.d), 1.0, sh.dtype)

    # --- draft distribution q (the draft model's output, an input of the verify step) ---
    if sh.q_mode == "dense" and with_q and not sh.external_drafts:
        A["q_draft"] = draft_probs_from_logits(R["q_logits"], (B * M, sh.V), sh.q_sigma)

    # --- root target logits: the previous step's output at the current token ---
    A["root_logits"] = (R["root"].standard_normal((B, sh.V)) * sh.root_sigma).astype(np.float32)

    # --- uniforms, indexed by position ---
    A["u_acc"] = R["u_acc"].random((B, W, D))
    A["u_res"] = R["u_res"].random((B, W))
    A["u_draft"] = R["u_draft"].random((B, W, D))
    return Case(shape=sh, variant=variant, seed=seed, arrays=A, meta=meta)


def draft_probs_from_logits(rng, shape, sigma: float, block_rows: int = 64) -> np.ndarray:
    """Dense draft distribution: the draft model's softmax over N(0, sigma^2) logits,
    formed in fp64 and stored as fp32 probabilities (not renormalised after rounding).
    This stands in for the drafter, which is not part of the verify step."""
    n, V = shape
    out = np.empty(shape, dtype=np.float32)
    for s in range(0, n, block_rows):
        m = min(block_rows, n - s)
        z = rng.standard_normal((m, V)) * sigma
        z -= z.max(axis=1, keepdims=True)
        e = np.exp(z)
        out[s:s + m] = (e / e.sum(axis=1, keepdims=True)).astype(np.float32)
    return out


LAYER_TENSORS = ("q", "k_cand", "v_cand", "k_pool", "v_pool")


def layer_inputs(case: Case, n_layers: int, seed: int) -> dict:
    """The attention tensors of a model with n_layers layers that share the case's block
    table (page_table, prefix_len): q, k_cand, v_cand, k_pool and v_pool stacked on a
    leading layer axis.  Layer 0 is the case's own; layers 1.. are fresh N(0, 1)
    tensors of the same shapes and dtype, one generator stream per layer."""
    sh = case.shape
    kids = np.random.SeedSequence(seed).spawn(max(n_layers - 1, 0))
    out = {k: [case.arrays[k]] for k in LAYER_TENSORS}
    for kid in kids:
        rng = np.random.default_rng(kid)
        for k in LAYER_TENSORS:
            out[k].append(_normal_model(rng, case.arrays[k].shape, 1.0, sh.dtype))
    return {k: np.stack(v) for k, v in out.items()}


def make_kv_case(seed: int, B: int, W: int, D: int, Hkv: int, hd: int, prefix, n_spare: int,
                 max_pages: int, dtype: str = "bf16"):
    """Inputs of a KV commit / rollback: a paged pool whose first pages hold the
    sequences' prefixes (pages in random order), `n_spare` further pages on a free
    stack (random order), candidate K/V rows and a random accepted candidate and run
    length per sequence.  Model tensors are bf16 bits (uint16) or float32.

    Arrays: k_pool [n_pages, Hkv, 16, hd], v_pool [n_pages, Hkv, hd, 16],
    page_table int32 [B, max_pages] (-1 past the prefix), prefix_len int32 [B],
    free_list int32 [n_pages] (the stack in its first n_free entries), n_free,
    k_cand/v_cand [B*W*D, Hkv, hd], best int32 [B] (-1 = none), n_acc int32 [B]."""
    rng = np.random.default_rng(seed)
    prefix = np.asarray(prefix, dtype=np.int64)
    used = [(int(p) + PAGE - 1) // PAGE for p in prefix]
    n_pages = int(sum(used)) + int(n_spare)
    perm = rng.permutation(n_pages).astype(np.int32)
    pt = np.full((B, max_pages), -1, dtype=np.int32)
    k = 0
    for b in range(B):
        pt[b, :used[b]] = perm[k:k + used[b]]
        k += used[b]
    free = np.zeros(n_pages, dtype=np.int32)
    free[:n_spare] = perm[k:]
    if dtype == "bf16":
        mk = lambda shp: f32_to_bf16_bits(rng.standard_normal(shp).astype(np.float32))
    else:
        mk = lambda shp: rng.standard_normal(shp).astype(np.float32)
    M = W * D
    return dict(
        k_pool=mk((n_pages, Hkv, PAGE, hd)), v_pool=mk((n_pages, Hkv, hd, PAGE)),
        page_table=pt, prefix_len=prefix.astype(np.int32), free_list=free,
        n_free=int(n_spare), k_cand=mk((B * M, Hkv, hd)), v_cand=mk((B * M, Hkv, hd)),
        best=rng.integers(-1, W, size=B).astype(np.int32),
        n_acc=rng.integers(0, D + 1, size=B).astype(np.int32))
