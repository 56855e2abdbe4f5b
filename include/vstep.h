/* vstep.h -- C ABI of the speculative-decoding verify step for AMD MI355X (gfx950).
 *
 * The verify step of speculative decoding, on one GPU:
 *   copy retrieval  -> probe gate -> block-triangular verify attention
 *   -> vocabulary projection (full or low-rank) -> rejection sampling.
 *
 * Sources (web pages, cited by title and section):
 *   [SW] "SwitchSD는 LLM 내부 표현으로 추측 디코딩의 복사 모드를 판별한다" (onedev.kr/papers/87),
 *        sections "어떻게 동작하나" (how it works) and "무엇과 다른가" (how it differs).
 *   [SD] "LLM 투기적 디코딩(Speculative Decoding) 해부 ..." (blog.huny.dev), section 2
 *        (draft / parallel verify / rejection sampler / bonus token) and section 3
 *        (alpha(x) = min(1, p/q), residual p'(x), P_final identity).
 *   [SL] "SlimSpec: Low-Rank Draft LM-Head for Accelerated Speculative Decoding"
 *        (gist.science/ko/paper/2605.10453), "방법론 / 아키텍처": z = W_up W_down h.
 *
 * Conventions (every entry point):
 *   - Every array pointer is a DEVICE pointer owned by the caller.  The library
 *     never allocates or frees memory and keeps no state between calls other than
 *     its loaded code object (which includes the fixed scratch area that only
 *     vs_verify_step_noalloc uses, and the per-device address of it that call looks up).
 *   - Every call only ENQUEUES work on `stream` (a hipStream_t; NULL = the default
 *     stream) and returns at once; outputs are valid after the stream is synchronised.
 *   - The return value reports host-side validation (checked before anything is
 *     launched: nothing is enqueued when a call fails validation) and launch errors.
 *     Conditions that only the device can see (bad page index, bad token id, near
 *     ties) come back in per-sequence `flags` outputs (VS_FLAG_*).
 *   - Workspace: calls that take `workspace` need at least the size reported by the
 *     matching vs_*_workspace_bytes function.  The workspace must be filled with
 *     zeros before its first use; every call leaves its counters at zero again, so a
 *     workspace can be reused by later calls on the same stream.  Calls that share a
 *     workspace must not run concurrently (on different streams).
 *   - Thread-safe and re-entrant as long as concurrent calls use distinct outputs and
 *     workspaces.  No C++ exception crosses this interface.
 *   - Layouts are row-major (C order).  "bf16" is the 16-bit brain float (top half of
 *     an IEEE fp32), rounded to nearest-even wherever the library writes it.
 */
#ifndef VSTEP_H
#define VSTEP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define VS_ABI_VERSION 5

typedef enum {
    VS_OK = 0,
    VS_ERR_INVALID_ARG = -1,   /* null required pointer, non-positive or inconsistent size */
    VS_ERR_UNSUPPORTED = -2,   /* valid request outside what the kernels implement */
    VS_ERR_WORKSPACE = -3,     /* workspace null or smaller than required */
    VS_ERR_HIP = -4            /* a HIP launch or runtime call failed */
} vs_status;

typedef enum { VS_F32 = 0, VS_BF16 = 1 } vs_dtype;

/* How the sampler chooses among W candidates (vs_sample_desc / vs_step_desc). */
typedef enum {
    VS_ACCEPT_LONGEST = 0,   /* each candidate judged alone; the longest accepted run wins */
    VS_ACCEPT_MULTI = 1,     /* lossless multi-candidate acceptance (see vs_reject_sample) */
    VS_ACCEPT_GREEDY = 2     /* greedy verification, temperature 0 (see vs_reject_sample) */
} vs_accept_mode;

/* Per-sequence device flags (bitwise OR). */
enum {
    VS_FLAG_PROBE_TIE = 1,            /* |score - tau| < 1e-5: probe decision is a near tie */
    VS_FLAG_ACCEPT_TIE = 2,           /* a decisive acceptance test has |u*Q - p| < 1e-4*max(p, u*Q) */
    VS_FLAG_CDF_TIE = 4,              /* the final draw lies within 1e-8*S of a CDF step */
    VS_FLAG_DEGENERATE_RESIDUAL = 8,  /* residual mass <= 0: drew from the target p instead
                                         (multi: also a removal that would leave no mass,
                                         which is then skipped) */
    VS_FLAG_NO_CANDIDATE = 16,        /* gate closed or no candidate: one token from the root p */
    VS_FLAG_BAD_PAGE = 32,            /* page index outside the pool, or prefix_len out of range */
    VS_FLAG_BAD_CTX = 64,             /* context offsets outside [0, ctx_total] or decreasing */
    VS_FLAG_BAD_TOKEN = 128,          /* a tested candidate token id is outside [0, V): rejected */
    VS_FLAG_POOL_EMPTY = 256,         /* kv commit: fewer free pages than a sequence needs */
    VS_FLAG_SYNC_TIMEOUT = 512        /* multi with dense drafts: a wait for the sequence's other
                                         workgroups gave up (cannot happen when the launch
                                         succeeds; the outputs are then not valid) */
};

int         vs_abi_version(void);
const char *vs_status_str(int status);

/* ---------------------------------------------------------------------------------
 * Copy-candidate retrieval [SW "무엇과 다른가"].
 * For each sequence b, the context is ctx[ctx_off[b] .. ctx_off[b+1]) (token ids),
 * its last token is the current token t.  The key is the kappa-gram ending at t.
 * Every earlier end position j (kappa-1 <= j <= t-1) whose kappa ids equal the key
 * is an occurrence (overlaps allowed).  The W largest j are kept, most recent
 * first; candidate i is ctx[j+1 .. j+len], len = min(D, t-j).
 *   ctx       int32 [ctx_total]
 *   ctx_off   int32 [B+1]     (device; checked on the device: bad offsets -> VS_FLAG_BAD_CTX)
 *   cand_tok  int32 [B, W, D] out: candidate ids, -1 past len
 *   cand_len  int32 [B, W]    out: 0 for missing candidates
 *   cand_pos  int32 [B, W]    out: end position j of the occurrence, or -1
 *   n_found   int32 [B]       out: number of candidates returned (<= W)
 *   flags     int32 [B]       out (may be NULL)
 * Limits: 1 <= kappa <= 16, 1 <= W, 1 <= D, W*D <= 1024, B >= 1.  Bit-exact. */
int vs_copy_match(const int32_t *ctx, int64_t ctx_total, const int32_t *ctx_off, int B,
                  int kappa, int W, int D, int32_t *cand_tok, int32_t *cand_len,
                  int32_t *cand_pos, int32_t *n_found, int32_t *flags, void *stream);

/* ---------------------------------------------------------------------------------
 * Probe gate [SW "어떻게 동작하나": bias-free linear probe; "무엇과 다른가": dual gate].
 * score[b] = sigmoid(sum_k w[k] h[b,k]) (fp32 products and accumulation, sigmoid in
 * fp64, stored fp32); gate[b] = (score >= tau) && (n_found == NULL || n_found[b] >= 1).
 *   h      [B, d] of h_dtype (VS_F32 or VS_BF16)
 *   w      fp32 [d]
 *   n_found int32 [B] or NULL
 *   score  fp32 [B] out;  gate int32 [B] out;  flags int32 [B] out or NULL (VS_FLAG_PROBE_TIE) */
int vs_probe_gate(const void *h, int h_dtype, const float *w, int B, int d, float tau,
                  const int32_t *n_found, float *score, int32_t *gate, int32_t *flags,
                  void *stream);

/* ---------------------------------------------------------------------------------
 * Block-triangular verify attention [SW "무엇과 다른가"].
 * Row r = i*D + o of sequence b holds candidate token (i, o).  For query head hq
 * (KV head hq / (Hq/Hkv)), the row attends to prefix keys 0..prefix_len[b]-1 and to
 * the keys of its own candidate at offsets 0..o (itself included); other candidates
 * are invisible.  softmax(scale * q.k) over the visible keys, weighted sum of values.
 *   q             [B*W*D, Hq, hd]   dtype
 *   k_cand/v_cand [B*W*D, Hkv, hd]  dtype (the candidates' own keys/values)
 *   k_pool        [n_pool_pages, Hkv, page_size, hd] dtype (paged prefix keys)
 *   v_pool        [n_pool_pages, Hkv, hd, page_size] dtype (paged prefix values,
 *                 transposed within each page: the page_size tokens of one head-dim
 *                 coordinate are contiguous)
 *   page_table    int32 [B, max_pages]: page of prefix positions 16p..16p+15
 *   prefix_len    int32 [B]
 *   out           [B*W*D, Hq, hd] dtype (bf16 rounded to nearest even, or fp32)
 *   flags         int32 [B] out or NULL (VS_FLAG_BAD_PAGE: keys of a bad page are skipped)
 * Supported: VS_BF16 with head_dim 128 (MFMA path); VS_F32 with head_dim 16, 32 or 64.
 * page_size must be 16; max_pages > 0 requires n_pool_pages >= 1.  scale <= 0 selects
 * 1/sqrt(head_dim).  Accumulation in fp32.
 * Layers [SD section 6: one paged cache per layer, the same block table for all]:
 * n_layers = L >= 1 (0 reads as 1) runs L independent layers in one launch.  q,
 * k_cand, v_cand, k_pool, v_pool and out are then L copies of the shapes above,
 * stacked (layer l at l times the one-layer size); page_table and prefix_len are
 * shared (a page id names the same slot in every layer's pool); flags are as for one
 * layer.  L <= 1024 and at most 2^30 workgroups (VS_ERR_UNSUPPORTED beyond). */
typedef struct {
    int32_t B, W, D, Hq, Hkv, head_dim, page_size, max_pages, n_pool_pages;
    int32_t dtype;          /* vs_dtype */
    float scale;
    int32_t n_layers;       /* 0 or 1: one layer */
} vs_attn_desc;

size_t vs_attention_workspace_bytes(const vs_attn_desc *desc);
int vs_verify_attention(const vs_attn_desc *desc, const void *q, const void *k_cand,
                        const void *v_cand, const void *k_pool, const void *v_pool,
                        const int32_t *page_table, const int32_t *prefix_len, void *out,
                        int32_t *flags, void *workspace, size_t ws_bytes, void *stream);

/* ---------------------------------------------------------------------------------
 * Weight prepacking for the bf16 vocabulary projection (data movement only).
 * A row-major bf16 matrix src [N, K] (K % 32 == 0) is rearranged into MFMA operand
 * tiles: tile (t, s) covers rows 16t..16t+15 and columns 32s..32s+31 and holds 64
 * lane slots of 8 values; slot l = row 16t + (l % 16), columns 32s + 8*(l / 16) .. +7.
 * Tiles are ordered t-major ([ceil(N/16)][K/32][64][8]); rows past N are zero.
 * dst must hold vs_packed_weight_bytes(N, K) bytes.  Done once per weight. */
size_t vs_packed_weight_bytes(int N, int K);
int vs_pack_weight(const void *src, void *dst, int N, int K, void *stream);

/* ---------------------------------------------------------------------------------
 * Vocabulary projection [SL "방법론 / 아키텍처"].
 *   rank == 0: z = W_full h            (w_full [V, d])
 *   rank  > 0: z = W_up (W_down h)     (w_down [rank, d], w_up [V, rank]; the rank-r
 *              intermediate is kept in fp32, not rounded to dtype)
 * VS_BF16 weights are passed PACKED (vs_pack_weight); VS_F32 weights row-major.
 * for every row h of `h` [M, d] (dtype).  Outputs:
 *   logits  fp32 [M, V] (required)
 *   row_lse fp64 [M]    (required): log sum_v exp(z[r,v] / temperature), from the fp32 logits
 *   probs   fp32 [M, V] or NULL: exp(z/temperature - lse) when write_probs != 0
 * Supported: VS_BF16 (MFMA path, d % 32 == 0, rank % 32 == 0) and VS_F32 (any d). */
typedef struct {
    int32_t M, d, V, rank;  /* rank 0 = full-rank head */
    int32_t dtype;          /* vs_dtype */
    float temperature;      /* > 0 */
    int32_t write_probs;
} vs_head_desc;

size_t vs_head_workspace_bytes(const vs_head_desc *desc);
int vs_lm_head(const vs_head_desc *desc, const void *h, const void *w_full,
               const void *w_down, const void *w_up, float *logits, double *row_lse,
               float *probs, void *workspace, size_t ws_bytes, void *stream);

/* ---------------------------------------------------------------------------------
 * Rejection sampling [SD sections 2-3] keeping the longest verified run [SW].
 * Candidate i of sequence b is judged token by token: draft x at offset o is
 * accepted iff u_acc[b,i,o] * Q < p(x), where p = softmax(z/T) of the preceding row
 * (root_logits[b] for o = 0, row (b, i, o-1) of `logits` otherwise) and
 * Q = q[(b,i,o)][x] (dense drafts) or 1 (q == NULL: copy drafts, a point mass on x).
 * The scan stops at the first rejection; a_i = accepted length.  The candidate
 * with the largest a_i wins (ties: smallest i).  Its a tokens are emitted, then one
 * more token drawn by inverse CDF over ascending ids with u_res[b, best]:
 *   rejection at offset a -> residual max(0, p - Qd) (Qd = q row (b,i,a), or the
 *                            point mass on the draft token);
 *   all accepted          -> bonus softmax(row (b, i, len-1)/T).
 * No candidate (all cand_len 0, or gate[b] == 0): one token from softmax(root/T)
 * drawn with u_res[b, 0], VS_FLAG_NO_CANDIDATE.  All sampler arithmetic is fp64.
 *   root_logits fp32 [B, V]; logits fp32 [B*W*D, V]; row_lse fp64 [B*W*D] (from vs_lm_head)
 *   q fp32 [B*W*D, V] or NULL; cand_tok int32 [B,W,D]; cand_len int32 [B,W]
 *   u_acc fp64 [B,W,D]; u_res fp64 [B,W]  (uniforms in [0,1), indexed by position)
 *   gate int32 [B] or NULL (NULL = open)
 * Outputs: n_acc [B], best [B] (-1 if none), out_tok [B, D+1] (-1 padded),
 *   n_out [B] (= n_acc + 1), acc_per_cand [B, W], flags [B] (may be NULL).
 *
 * accept_mode VS_ACCEPT_MULTI: lossless acceptance over the W candidates, built from
 * the single-draft rule and its residual [SD section 3] applied across sibling
 * drafts.  Depth a (from 0) starts from the target p of the reference row -- the
 * root for a = 0, else row (b, ref, a-1), ref = the smallest surviving candidate
 * (all candidates with cand_len >= 1 survive at a = 0).  The survivors with
 * cand_len > a are tried in index order: with p' the current residual (initially p),
 * candidate i's token x is accepted iff u_acc[b,i,a] * Q_i(x) < p'(x) with Q_i the
 * draft row q[b, i, a] (the point mass on x when q == NULL); a rejection sets
 * p' <- normalise(max(0, p' - Q_i)) over the whole vocabulary (a removal that would
 * leave no mass is skipped and flagged DEGENERATE).  An accepted x is emitted and the
 * survivors become the tried candidates whose token at depth a is x.  If all are
 * rejected, one token is drawn from p' with u_res[b, last candidate tried]; if no
 * survivor has a token at depth a, a bonus token is drawn from p with
 * u_res[b, ref].  Outputs as above with best = the final reference candidate and
 * acc_per_cand[b,i] = the length of candidate i's common prefix with the accepted
 * tokens.  At most 64 candidates (else VS_ERR_UNSUPPORTED).  Copy drafts also need
 * (W*D+1)*W + W*D <= 4096 (else VS_ERR_UNSUPPORTED); dense drafts with W > 1 keep
 * fp64 residual rows in the workspace and share each sequence's vocabulary passes
 * among up to 32 workgroups of a cooperative launch (one workgroup per sequence when
 * the device or the grid does not allow one; the results are the same bits).  With
 * W == 1 the rule is the single-chain rule above, which is what runs.
 *
 * accept_mode VS_ACCEPT_GREEDY: greedy verification, the temperature -> 0 limit of
 * the rule above [SD section 3] (every p becomes the point mass on its row's argmax):
 * draft x at offset o is accepted iff x is the argmax of the preceding row, a
 * candidate's run stops at its first other token, the longest run wins (ties:
 * smallest i) and the extra token is the argmax of the row after the run (root for
 * a = 0).  argmax = first index of the largest fp32 logit.  q, u_acc and u_res are
 * not read (may be NULL); temperature (> 0) only scales the normalisers computed on
 * the way.  A tested row, or the extra token's row, whose two largest logits are
 * within 1e-3 * max(1, |largest|) raises VS_FLAG_ACCEPT_TIE, resp. VS_FLAG_CDF_TIE. */
typedef struct {
    int32_t B, W, D, V;
    float temperature;
    int32_t accept_mode;      /* vs_accept_mode */
} vs_sample_desc;

size_t vs_sample_workspace_bytes(const vs_sample_desc *desc);
int vs_reject_sample(const vs_sample_desc *desc, const float *root_logits,
                     const float *logits, const double *row_lse, const float *q,
                     const int32_t *cand_tok, const int32_t *cand_len, const double *u_acc,
                     const double *u_res, const int32_t *gate, int32_t *n_acc, int32_t *best,
                     int32_t *out_tok, int32_t *n_out, int32_t *acc_per_cand, int32_t *flags,
                     void *workspace, size_t ws_bytes, void *stream);

/* ---------------------------------------------------------------------------------
 * Draft tokens [SD section 2: each draft token is sampled from the draft model's q]
 * from stored draft probabilities, e.g. the low-rank head's (vs_lm_head with
 * write_probs): tok[r] = min{k : C_k > u[r] * S} over the running sum C of q[r, 0..V)
 * in ascending id order, S its total (the probabilities are not renormalised); sums
 * in fp64.  A draw within 1e-8 * S of a CDF step raises VS_FLAG_CDF_TIE in flags[r].
 *   q fp32 [rows, V]; u fp64 [rows] in [0, 1); tok int32 [rows]; flags int32 [rows]
 *   or NULL.  V <= 524288 (VS_ERR_UNSUPPORTED beyond). */
size_t vs_draft_sample_workspace_bytes(int rows, int V);
int vs_draft_sample(const float *q, int rows, int V, const double *u, int32_t *tok,
                    int32_t *flags, void *workspace, size_t ws_bytes, void *stream);

/* ---------------------------------------------------------------------------------
 * The whole verify step, enqueued on one stream with no host synchronisation:
 *   copy_match + probe_gate (one fused launch; skipped when external_drafts != 0, in
 *   which case cand_tok/cand_len are INPUTS from a neural drafter and the gate is open)
 *   -> verify_attention -> lm_head (full rank, head input = attention output viewed
 *   as [B*W*D, Hq*hd], so d must equal Hq*head_dim) -> reject_sample.
 * stage_events: NULL, or 6 hipEvent_t handles recorded on `stream` before stage 1
 * and after each of the 5 stages (retrieval+gate, attention, head GEMM, normalisers
 * and acceptance tests, sampler) -- for timing only.
 * aux_stream, fork_event, join_event: NULL, or a second stream (default priority)
 * and two events owned by the caller.  Then retrieval + gate, when they have a launch
 * of their own (bf16 attention with fewer than four waves per row block; otherwise
 * they ride in the attention launch), run on aux_stream concurrently with attention
 * and the head: fork_event is recorded on `stream` and waited for on aux_stream before the
 * retrieval; join_event is recorded on aux_stream after it and waited for on
 * `stream` before the tests.  Stage event 1 then follows event 0 directly (the
 * retrieval is off the main stream). */
typedef struct {
    int32_t B, W, D, kappa;
    int32_t Hq, Hkv, head_dim, page_size, max_pages, n_pool_pages;
    int32_t d, V;
    int32_t dtype;            /* vs_dtype of q/k/v/pools/head/probe h/attention output */
    float scale;              /* <= 0: 1/sqrt(head_dim) */
    float tau;                /* probe threshold */
    float temperature;
    int32_t external_drafts;
    int64_t ctx_total;
    int32_t accept_mode;      /* vs_accept_mode of the sampler (same limits as vs_reject_sample;
                                 greedy: u_acc, u_res and q_draft are not read) */
    int32_t n_layers;         /* attention layers (0 or 1: one): q, k_cand, v_cand, the
                                 pools and attn_out stacked as for vs_verify_attention;
                                 the head reads the last layer's output */
} vs_step_desc;

typedef struct {
    /* copy retrieval and gate (unused when external_drafts) */
    const int32_t *ctx, *ctx_off;
    const void *probe_h;        /* [B, d] dtype */
    const float *probe_w;       /* [d] */
    /* attention */
    const void *q, *k_cand, *v_cand, *k_pool, *v_pool;
    const int32_t *page_table, *prefix_len;
    /* head */
    const void *w_full;         /* [V, d]: packed (vs_pack_weight) for bf16, row-major fp32 */
    /* sampler */
    const float *root_logits;   /* [B, V] */
    const float *q_draft;       /* [B*W*D, V] or NULL (copy drafts: point mass) */
    const double *u_acc, *u_res;
    /* retrieval outputs (inputs when external_drafts) */
    int32_t *cand_tok, *cand_len;
    int32_t *cand_pos, *n_found;            /* may be NULL when external_drafts */
    float *score; int32_t *gate;            /* may be NULL when external_drafts */
    /* stage outputs */
    void *attn_out;                         /* [n_layers][B*W*D, Hq, hd] dtype */
    float *logits;                          /* [B*W*D, V] */
    double *row_lse;                        /* [B*W*D] */
    int32_t *n_acc, *best, *out_tok, *n_out, *acc_per_cand;
    int32_t *flags;                         /* [B]: OR of every stage's flags */
    void **stage_events;                    /* NULL or 6 hipEvent_t */
    void *aux_stream;                       /* NULL or hipStream_t (see above) */
    void *fork_event, *join_event;          /* hipEvent_t, required with aux_stream */
} vs_step_io;

size_t vs_step_workspace_bytes(const vs_step_desc *desc);
int vs_verify_step(const vs_step_desc *desc, const vs_step_io *io, void *workspace,
                   size_t ws_bytes, void *stream);

/* ---------------------------------------------------------------------------------
 * The verify step without a workspace argument and without any allocation, for
 * callers that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc.  Same descriptor, pointers,
 * outputs, flags and results as vs_verify_step; the workspace is instead a fixed
 * scratch area of VS_NOALLOC_SCRATCH_BYTES inside the library, one per GPU, which
 * that GPU holds from the library's load until the process ends.
 *   - A request whose vs_step_workspace_bytes(desc) exceeds VS_NOALLOC_SCRATCH_BYTES
 *     returns VS_ERR_UNSUPPORTED before anything is enqueued.
 *   - `stream` must belong to the current device (else VS_ERR_INVALID_ARG); NULL is
 *     the current device's default stream.
 *   - The call makes no hipMalloc, hipFree, hipMemset or other allocating call.  It
 *     enqueues one small fill kernel first that clears the scratch words that must
 *     start at zero (the scratch keeps whatever the previous call on that GPU left).
 *   - Every call on one GPU shares that GPU's scratch: calls that overlap in time on
 *     one GPU (different streams, or different host threads) race and must be
 *     serialised by the caller. */
#define VS_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int vs_verify_step_noalloc(const vs_step_desc *desc, const vs_step_io *io, void *stream);

/* ---------------------------------------------------------------------------------
 * Copy-mode labels [SW "어떻게 동작하나"]: labels[p] = 1 when position p lies inside a
 * verbatim run of at least kappa tokens that already appeared earlier in the same
 * context (the earlier occurrence starts earlier; it may overlap), else 0.
 * Equivalently: some kappa-gram window [s, s+kappa) covering p also occurs at a start
 * t < s of the same sequence.  The training labels of the copy-intent probe.
 *   ctx int32 [ctx_total] (token ids, compared for equality only), ctx_off int32 [B+1]
 *   (sequence b = ctx[ctx_off[b] .. ctx_off[b+1])), labels uint8 [ctx_total],
 *   flags int32 [B] or NULL.
 * The offsets must be non-decreasing with ctx_off[0] >= 0 and ctx_off[B] <= ctx_total,
 * else every sequence gets VS_FLAG_BAD_CTX and no label is written; labels outside
 * [ctx_off[0], ctx_off[B]) are never written.  1 <= kappa <= 16; ctx_total < 2^31
 * (VS_ERR_UNSUPPORTED beyond). */
size_t vs_copy_labels_workspace_bytes(int64_t ctx_total);
int vs_copy_labels(const int32_t *ctx, int64_t ctx_total, const int32_t *ctx_off, int B,
                   int kappa, uint8_t *labels, int32_t *flags, void *workspace,
                   size_t ws_bytes, void *stream);

/* ---------------------------------------------------------------------------------
 * KV commit and rollback over the paged cache [SD section 6: the KV blocks of rejected
 * tokens go back to the paged pool at once, and none may leak].  The verify step
 * reads the candidates' K/V from their own buffers and leaves the cache untouched;
 * these calls then keep what was accepted.
 *
 * Cache model (as vs_verify_attention reads it): pages of 16 tokens, k_pool
 * [n_pool_pages, Hkv, 16, head_dim], v_pool [n_pool_pages, Hkv, head_dim, 16];
 * page_table int32 [B, max_pages], entry j = the pool page of tokens 16j .. 16j+15;
 * prefix_len int32 [B] (the cache length of each sequence); a free-page stack:
 * free_list int32 [n_pool_pages] (room for every page) whose first *n_free entries
 * are the free pages, top of the stack = free_list[*n_free - 1]; n_free is one int32
 * in device memory.  Page ids are taken and returned in a fixed order -- sequence
 * order, then page order -- so they do not depend on scheduling.
 * flags int32 [B] (may be NULL) is written whole: 0, VS_FLAG_POOL_EMPTY or
 * VS_FLAG_BAD_PAGE for a sequence that was refused (and left untouched).
 * At most 2048 sequences per call (VS_ERR_UNSUPPORTED beyond). */

typedef struct {
    int32_t B, W, D, Hkv, head_dim, page_size, max_pages, n_pool_pages;
    int32_t dtype;            /* vs_dtype of k_cand/v_cand and the pools (element copy) */
    int32_t n_layers;         /* commit: layers (0 or 1: one; stacked as for attention) */
} vs_kv_desc;

size_t vs_kv_workspace_bytes(const vs_kv_desc *desc);

/* Commit: for each sequence b with best[b] in [0, W) and a = min(n_acc[b], D) > 0,
 * rows (b, best[b], 0 .. a-1) of k_cand/v_cand ([B*W*D, Hkv, head_dim], the verify
 * step's candidate layout) become tokens P .. P+a-1, P = prefix_len[b]; the pages it
 * needs beyond ceil(P/16) are popped off the stack; prefix_len[b] becomes P + a.
 * With n_layers = L > 1, k_cand/v_cand and the pools are L stacked layers (as for
 * vs_verify_attention) and the same rows of every layer go to the same page slots:
 * the pages are taken once, for all layers (L <= 65535).
 * Refused with VS_FLAG_BAD_PAGE when P < 0 or P + a > 16*max_pages or when its
 * partly filled last page or a page it would pop is not in [0, n_pool_pages); with
 * VS_FLAG_POOL_EMPTY when the stack holds fewer pages than it needs (later
 * sequences may still be served).  best and n_acc are the sampler's outputs. */
int vs_kv_commit(const vs_kv_desc *desc, const void *k_cand, const void *v_cand,
                 const int32_t *best, const int32_t *n_acc, void *k_pool, void *v_pool,
                 int32_t *page_table, int32_t *prefix_len, int32_t *free_list, int32_t *n_free,
                 int32_t *flags, void *workspace, size_t ws_bytes, void *stream);

/* Token-major K/V into the pages above (data movement only).  k_src, v_src [n_tokens,
 * Hkv, head_dim] of dtype are a cache in token order: a contiguous cache [P, Hkv, hd]
 * (n_tokens = P), or token-major pages [n_pages, 16, Hkv, hd] (n_tokens = 16 n_pages;
 * the same bytes).  Writes k_pool [ceil(n_tokens/16), Hkv, 16, hd] and v_pool
 * [ceil(n_tokens/16), Hkv, hd, 16]; page p holds tokens 16p .. 16p+15 (positions past
 * n_tokens are zero), so the identity page table (entry j = j) serves the contiguous
 * cache.  k_pool/v_pool must not overlap the sources.  head_dim <= 256. */
int vs_kv_pack_pages(const void *k_src, const void *v_src, int64_t n_tokens, int Hkv,
                     int head_dim, int dtype, void *k_pool, void *v_pool, void *stream);

/* Rollback: sequence b keeps its first new_len[b] tokens; the pages past
 * ceil(new_len[b]/16) are pushed onto the stack in ascending page order and their
 * page-table entries set to -1; prefix_len[b] = new_len[b].  Token data is not
 * touched.  Refused with VS_FLAG_BAD_PAGE when new_len[b] is outside
 * [0, prefix_len[b]], prefix_len[b] is out of range, a page to free is not a pool
 * page, or the stack would overflow.  Only B, page_size, max_pages and n_pool_pages
 * of the descriptor are read: the page table is shared by all layers, so one call
 * rolls back every layer's cache. */
int vs_kv_truncate(const vs_kv_desc *desc, const int32_t *new_len, int32_t *page_table,
                   int32_t *prefix_len, int32_t *free_list, int32_t *n_free, int32_t *flags,
                   void *stream);

#ifdef __cplusplus
}
#endif
#endif /* VSTEP_H */
