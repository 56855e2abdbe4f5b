// Rejection sampling of the verify step.
//
// Leviathan/Chen acceptance as laid out in the rejection-sampling blog
// (blog.huny.dev), sections 2-3: draft x is kept with probability min(1, p(x)/q(x))
// -- here: kept iff u * q(x) < p(x) -- the chain stops at the first rejection, the
// rejected slot is refilled from the residual max(0, p - q) renormalised, and a
// fully accepted chain earns a bonus token from the next position's p.  Over W
// copy candidates the longest accepted run is kept (SwitchSD summary,
// onedev.kr/papers/87, "무엇과 다른가"); ties go to the smallest candidate index.
//
// All sampler arithmetic is fp64: p = exp(z/T - lse) from fp32 logits and fp64
// normalisers, the acceptance comparison, and the inverse-CDF draw over ascending
// token ids.
//
// Lossless multi-candidate acceptance (accept mode MULTI, copy drafts): at each depth
// the surviving candidates' tokens are tried in index order against one target
// distribution (the reference candidate's row) with the single-draft rule, each
// rejection removing the rejected token's mass; the normaliser kernel computes p of
// every candidate's token under every row, the chain itself is a short serial walk in
// LDS, and the draw excludes the rejected tokens.
//
// Greedy verification (accept mode GREEDY, temperature 0): a draft token is kept iff
// it is the argmax of the preceding row and the extra token is the argmax of the row
// after the run.  The normaliser kernel finds each row's argmax from the per-tile
// maxima (only the tiles holding the row maximum are read again) and writes the tests;
// one workgroup per sequence then picks the longest run.
//
// Layout of the work: grid (vocabulary chunks, sequences).  Every workgroup of a
// sequence repeats the (cheap) acceptance tests and the choice of candidate, then
// sums the residual weights of its own vocabulary chunk with coalesced loads.  The
// draw then adds the chunk sums in chunk order, finds the chunk holding u*S, finds
// the thread range holding it with an ordered block scan of that chunk's per-thread
// sums (recomputed from the logits by the drawing workgroup: the same arithmetic in the
// same order gives the same bits, and the owning thread then holds its ids' weights)
// and writes the outputs.  Two ways to reach the draw:
//   * fused: the last workgroup of the sequence to finish (atomic counter in the
//     workspace, reset afterwards) does it.  Each workgroup publishes its sums with
//     agent-scope atomic stores followed by an agent-scope acquire-release increment of
//     the counter (the release writes back its XCD's L2); with a few dozen workgroups
//     that is cheap;
//   * two launches: the chunk sums kernel ends, and a second kernel of one workgroup
//     per sequence draws.  With thousands of workgroups (large batches) the releases
//     of the fused form queue up behind each other and this is faster.

#include "vs_internal.hpp"

#include <limits.h>
#include <stdlib.h>

#include <mutex>

namespace vs {

namespace {

constexpr int kST = 256;              // threads per workgroup
constexpr int kPer = 8;               // vocabulary entries per thread per chunk
constexpr int kChunk = kST * kPer;    // 2048
constexpr int kMaxRows = 1024;
constexpr int kMaxCChunks = 128;      // dense multi-candidate chain: 4,096-id chunks, V <= 524,288

// Acceptance codes per draft position, written by the normaliser kernel and read by
// the sampler.
enum : uint8_t { CODE_ACCEPT = 1, CODE_TIE = 2, CODE_BAD = 4 };

__device__ __forceinline__ double warp_sum(double v) {
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

__device__ __forceinline__ double warp_max(double v) {
  for (int off = 32; off > 0; off >>= 1) v = fmax(v, __shfl_xor(v, off));
  return v;
}

// ---------------------------------------------------------------------------------
// Normalisers and acceptance tests.  One workgroup per distribution row: rows
// [0, B*M) are the verify rows (row (b, i, o) is the target distribution after draft
// token o of candidate i), rows [B*M, B*M + B) are the root distributions.  The
// workgroup forms lse = max + log(sum_t s_t exp(m_t - max)) in fp64 from the head's
// per-tile (max, sumexp) statistics, then tests the draft tokens this row scores:
// token o+1 of candidate i for a verify row, token 0 of every candidate for a root
// row.  A token x is kept iff u * q(x) < p(x) with p(x) = exp(z_x/T - lse).
struct TestArgs {
  int B, W, D, V, n_vt;
  double inv_t;
  const float2 *row_stats;    // [B*M][n_vt], or null: row_lse is an input
  const float2 *root_stats;   // [B][n_vt]
  double *row_lse;            // [B*M]
  double *root_lse;           // [B]
  const float *root_logits, *logits, *q;
  const int32_t *cand_tok, *cand_len, *gate;
  const double *u_acc;
  uint8_t *code;              // [B*W*D], or null: normalisers only
  double *pv;                 // MULTI: [B][M+1 rows][W] p of every candidate's token
  int greedy;                 // GREEDY: argmax tests instead of the probability tests
  const float2 *am_stats;     // GREEDY: tile maxima of the verify rows [B*M][n_vt]
  int32_t *amax;              // GREEDY: [B*M + B] argmax of every row (root rows last)
  uint8_t *amax_tie;          // GREEDY: [B*M + B] near tie between the two largest logits
};

__device__ double lse_of_stats(const float2 *st, int n_vt, double *red) {
  const int tid = threadIdx.x;
  double mx = -INFINITY;
  for (int t = tid; t < n_vt; t += 256) mx = fmax(mx, (double)st[t].x);
  mx = warp_max(mx);
  if ((tid & 63) == 0) red[tid >> 6] = mx;
  __syncthreads();
  mx = fmax(fmax(red[0], red[1]), fmax(red[2], red[3]));
  __syncthreads();
  double sm = 0.0;
  for (int t = tid; t < n_vt; t += 256) {
    const float2 v = st[t];
    if (v.x != -INFINITY) sm += (double)v.y * exp((double)v.x - mx);
  }
  sm = warp_sum(sm);
  if ((tid & 63) == 0) red[tid >> 6] = sm;
  __syncthreads();
  return mx + log((red[0] + red[1]) + (red[2] + red[3]));
}

// lse_of_stats for n_vt <= 512 from the two entries t = tid and t = tid + 256 a thread
// reads there, loaded beforehand by the caller: the same operations in the same order
__device__ double lse_of_stats2(float2 a0, float2 a1, int n_vt, double *red) {
  const int tid = threadIdx.x;
  double mx = -INFINITY;
  if (tid < n_vt) mx = fmax(mx, (double)a0.x);
  if (tid + 256 < n_vt) mx = fmax(mx, (double)a1.x);
  mx = warp_max(mx);
  if ((tid & 63) == 0) red[tid >> 6] = mx;
  __syncthreads();
  mx = fmax(fmax(red[0], red[1]), fmax(red[2], red[3]));
  __syncthreads();
  double sm = 0.0;
  if (tid < n_vt && a0.x != -INFINITY) sm += (double)a0.y * exp((double)a0.x - mx);
  if (tid + 256 < n_vt && a1.x != -INFINITY) sm += (double)a1.y * exp((double)a1.x - mx);
  sm = warp_sum(sm);
  if ((tid & 63) == 0) red[tid >> 6] = sm;
  __syncthreads();
  return mx + log((red[0] + red[1]) + (red[2] + red[3]));
}

struct PosIn {
  int x, len;
  double u, Q;
  float z;
};

// inputs of the test at draft position (b, i, oo) scored by row r (r < 0: root row)
__device__ __forceinline__ PosIn load_pos(const TestArgs &a, int b, int r, int i, int oo) {
  PosIn in{-1, 0, 0.0, 1.0, 0.f};
  const bool open = (a.gate == nullptr) || a.gate[b] != 0;
  const int ln = open ? a.cand_len[(int64_t)b * a.W + i] : 0;
  in.len = ln < 0 ? 0 : (ln > a.D ? a.D : ln);
  const int64_t pos = ((int64_t)b * a.W + i) * a.D + oo;
  if (oo < in.len) {
    in.x = a.cand_tok[pos];
    if (a.u_acc) in.u = a.u_acc[pos];
    if (in.x >= 0 && in.x < a.V) {
      in.z = (r < 0) ? a.root_logits[(int64_t)b * a.V + in.x] : a.logits[(int64_t)r * a.V + in.x];
      if (a.q) in.Q = (double)a.q[pos * a.V + in.x];
    }
  }
  return in;
}

__device__ __forceinline__ void store_test(const TestArgs &a, const PosIn &in, int b, int i,
                                           int oo, double lse) {
  uint8_t c = 0;
  if (oo < in.len) {
    if (in.x >= 0 && in.x < a.V) {
      const double p = exp((double)in.z * a.inv_t - lse);
      const double lhs = in.u * in.Q;
      if (lhs < p) c |= CODE_ACCEPT;
      if (fabs(lhs - p) < 1e-4 * fmax(p, lhs)) c |= CODE_TIE;
    } else {
      c = CODE_BAD;
    }
  }
  a.code[((int64_t)b * a.W + i) * a.D + oo] = c;
}

// ---- greedy: the argmax of a row from its tile maxima
constexpr int kTieTiles = 16;
constexpr double kGreedyTieRel = 1e-3;   // near tie: top two within this x max(1, |top|)

struct ArgmaxShared {
  float v1[4], v2[4];
  int i1[4];
  int n_list;
  int list[kTieTiles];
};

// (largest value, its first index, second largest value) of a multiset, merged with
// another such summary
__device__ __forceinline__ void am_merge(float &v1, int &i1, float &v2, float ov1, int oi1,
                                         float ov2) {
  if (ov1 > v1 || (ov1 == v1 && oi1 < i1)) {
    v2 = fmaxf(v1, ov2);
    v1 = ov1;
    i1 = oi1;
  } else {
    v2 = fmaxf(v2, ov1);
  }
}

// First index of the largest logit of row z[0, V) and whether the two largest are a
// near tie.  st[t].x is the maximum of fl(z * inv_t) over tile t; fl is monotone, so
// the argmax lies in a tile whose maximum equals the row's, and only those tiles
// (usually one; all of them if more than kTieTiles) are read.  The second largest
// logit outside them is estimated from their maxima (for the tie test only).
__device__ void row_argmax(const float2 *st, int n_vt, const float *z, int V, float inv_t,
                           ArgmaxShared &s, int &am, bool &tie) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  float g = -INFINITY;
  for (int t = tid; t < n_vt; t += 256) g = fmaxf(g, st[t].x);
  for (int off = 32; off > 0; off >>= 1) g = fmaxf(g, __shfl_xor(g, off));
  if (lane == 0) s.v1[wv] = g;
  if (tid == 0) s.n_list = 0;
  __syncthreads();
  g = fmaxf(fmaxf(s.v1[0], s.v1[1]), fmaxf(s.v1[2], s.v1[3]));
  float s2 = -INFINITY;
  for (int t = tid; t < n_vt; t += 256) {
    const float x = st[t].x;
    if (x == g) {
      const int k = atomicAdd(&s.n_list, 1);
      if (k < kTieTiles) s.list[k] = t;
    } else {
      s2 = fmaxf(s2, x);
    }
  }
  for (int off = 32; off > 0; off >>= 1) s2 = fmaxf(s2, __shfl_xor(s2, off));
  if (lane == 0) s.v2[wv] = s2;
  __syncthreads();
  s2 = fmaxf(fmaxf(s.v2[0], s.v2[1]), fmaxf(s.v2[2], s.v2[3]));
  const int nl = s.n_list;
  const bool all = nl > kTieTiles;
  const int nscan = all ? n_vt : nl;
  float v1 = -INFINITY, v2 = -INFINITY;
  int i1 = INT_MAX;
  for (int l = 0; l < nscan; ++l) {
    const int k = (all ? l : s.list[l]) * kHeadVocabTile + tid;
    if (k < V) am_merge(v1, i1, v2, z[k], k, -INFINITY);
  }
  for (int off = 32; off > 0; off >>= 1) {
    const float ov1 = __shfl_xor(v1, off), ov2 = __shfl_xor(v2, off);
    const int oi1 = __shfl_xor(i1, off);
    am_merge(v1, i1, v2, ov1, oi1, ov2);
  }
  __syncthreads();
  if (lane == 0) {
    s.v1[wv] = v1;
    s.i1[wv] = i1;
    s.v2[wv] = v2;
  }
  __syncthreads();
  v1 = s.v1[0];
  i1 = s.i1[0];
  v2 = s.v2[0];
  for (int w2 = 1; w2 < 4; ++w2) am_merge(v1, i1, v2, s.v1[w2], s.i1[w2], s.v2[w2]);
  am = i1;
  const double zm = v1;
  const double z2 = fmax((double)v2, (double)s2 / (double)inv_t);
  tie = (zm - z2) < kGreedyTieRel * fmax(1.0, fabs(zm));
}

__device__ __forceinline__ void store_test_greedy(const TestArgs &a, const PosIn &in, int b,
                                                  int i, int oo, int am, bool tie) {
  uint8_t c = 0;
  if (oo < in.len) {
    if (in.x >= 0 && in.x < a.V) {
      if (in.x == am) c |= CODE_ACCEPT;
    } else {
      c = CODE_BAD;
    }
    if (tie) c |= CODE_TIE;
  }
  a.code[((int64_t)b * a.W + i) * a.D + oo] = c;
}

__global__ void __launch_bounds__(256)
lse_tests_kernel(TestArgs a) {
  __shared__ double red[4];
  const int tid = threadIdx.x;
  const int M = a.W * a.D;
  const int r = blockIdx.x;
  const bool root = r >= a.B * M;
  const int b = root ? r - a.B * M : r / M;

  // positions scored by this row (their loads are issued before the reduction)
  int i0 = 0, oo = 0, npos = 0;
  if (a.code != nullptr) {
    if (root) {
      npos = a.W;
    } else {
      const int rr = r % M;
      i0 = rr / a.D;
      oo = rr % a.D + 1;
      npos = (oo < a.D) ? 1 : 0;
    }
  }
  const int rrow = root ? -1 : r;
  // this row's tile statistics first (up to 512 tiles: two per thread, in registers),
  // so that the draft token's dependent loads overlap the reduction
  const float2 *stp = root ? a.root_stats + (int64_t)b * a.n_vt
                           : (a.row_stats != nullptr ? a.row_stats + (int64_t)r * a.n_vt : nullptr);
  const bool pre = stp != nullptr && a.n_vt <= 512;
  float2 s0 = make_float2(0.f, 0.f), s1 = make_float2(0.f, 0.f);
  if (pre) {
    if (tid < a.n_vt) s0 = stp[tid];
    if (tid + 256 < a.n_vt) s1 = stp[tid + 256];
  }
  PosIn first{-1, 0, 0.0, 1.0, 0.f};
  if (tid < npos) first = load_pos(a, b, rrow, root ? tid : i0, oo);

  double lse;
  if (stp != nullptr) {
    lse = pre ? lse_of_stats2(s0, s1, a.n_vt, red) : lse_of_stats(stp, a.n_vt, red);
    if (tid == 0) {
      if (root) a.root_lse[b] = lse;
      else a.row_lse[r] = lse;
    }
  } else {
    lse = a.row_lse[r];
  }

  if (a.greedy) {
    __shared__ ArgmaxShared ash;
    const float *zr = root ? a.root_logits + (int64_t)b * a.V : a.logits + (int64_t)r * a.V;
    const float2 *st = root ? a.root_stats + (int64_t)b * a.n_vt : a.am_stats + (int64_t)r * a.n_vt;
    int am;
    bool tie;
    row_argmax(st, a.n_vt, zr, a.V, (float)a.inv_t, ash, am, tie);
    const int64_t gr = root ? (int64_t)a.B * M + b : r;
    if (tid == 0) {
      a.amax[gr] = am;
      a.amax_tie[gr] = tie ? 1 : 0;
    }
    if (tid < npos) store_test_greedy(a, first, b, root ? tid : i0, oo, am, tie);
    for (int t = tid + 256; t < npos; t += 256)
      store_test_greedy(a, load_pos(a, b, rrow, t, oo), b, t, oo, am, tie);
    return;
  }
  if (a.pv != nullptr) {
    // MULTI: p under this row of every candidate's token at the depth the row judges
    // (0 for the root row, o+1 for verify row (i, o)); -1 marks an out-of-range token,
    // 0 a candidate without a token there
    const int M = a.W * a.D;
    const int depth = root ? 0 : (r % M) % a.D + 1;
    const int rowidx = root ? M : r % M;
    for (int j = tid; j < a.W; j += 256) {
      double v = 0.0;
      const bool open = (a.gate == nullptr) || a.gate[b] != 0;
      int ln = open ? a.cand_len[(int64_t)b * a.W + j] : 0;
      ln = ln < 0 ? 0 : (ln > a.D ? a.D : ln);
      if (depth < ln) {
        const int x = a.cand_tok[((int64_t)b * a.W + j) * a.D + depth];
        if (x >= 0 && x < a.V) {
          const float z = root ? a.root_logits[(int64_t)b * a.V + x] : a.logits[(int64_t)r * a.V + x];
          v = exp((double)z * a.inv_t - lse);
        } else {
          v = -1.0;
        }
      }
      a.pv[((int64_t)b * (M + 1) + rowidx) * a.W + j] = v;
    }
    return;
  }
  if (tid < npos) store_test(a, first, b, root ? tid : i0, oo, lse);
  for (int t = tid + 256; t < npos; t += 256) store_test(a, load_pos(a, b, rrow, t, oo), b, t, oo, lse);
}

// ---------------------------------------------------------------------------------
struct SampShared {
  int a_len[kMaxRows];
  int lens[kMaxRows];
  int tok[kMaxRows];
  double rlse[kMaxRows];
  double ures[kMaxRows];
  uint8_t code[kMaxRows];
  double red[kST / 64];
  double red2[kST / 64];
  int flags;
  int best, ab, mode, xpt, is_last, owner, last_pos, tstar;
  int64_t prow, qrow;
  double lse, u, excl, tot, xs;
};

enum { MODE_ROOT = 0, MODE_RESID = 1, MODE_BONUS = 2, MODE_TARGET = 3 };

// MULTI: at most kMaxWMulti candidates; the p values [M+1][W] and the acceptance
// uniforms [M] sit in dynamic LDS, at most kMaxMultiLds doubles
constexpr int kMaxWMulti = 64;
constexpr int kMaxMultiLds = 4096;

__host__ __device__ constexpr int multi_lds_doubles(int W, int D) { return (W * D + 1) * W + W * D; }

template <bool MULTI> struct SampSharedT : SampShared {};
template <> struct SampSharedT<true> : SampShared {
  int excl_tok[kMaxWMulti];           // tokens rejected at the final depth (mass removed)
  int surv[kMaxWMulti];               // surviving candidates, ascending
  int sib[kMaxWMulti];
  int n_excl;
};

// fixed-order block sum of two values (every thread receives the totals)
__device__ void block_sum2(SampShared &sh, double &a, double &b) {
  const int tid = threadIdx.x;
  a = warp_sum(a);
  b = warp_sum(b);
  if ((tid & 63) == 0) {
    sh.red[tid >> 6] = a;
    sh.red2[tid >> 6] = b;
  }
  __syncthreads();
  a = (sh.red[0] + sh.red[1]) + (sh.red[2] + sh.red[3]);
  b = (sh.red2[0] + sh.red2[1]) + (sh.red2[2] + sh.red2[3]);
  __syncthreads();
}

// inclusive prefix sum over the block in thread order, in a fixed order: a shuffle
// scan inside each wave, then the totals of the earlier waves
__device__ double block_incl_scan(SampShared &sh, double v) {
  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const double y = __shfl_up(v, off);
    if (lane >= off) v += y;
  }
  if (lane == 63) sh.red[wv] = v;
  __syncthreads();
  double base = 0.0;
  for (int w2 = 0; w2 < wv; ++w2) base += sh.red[w2];
  __syncthreads();
  return base + v;
}

struct SampArgs {
  int B, W, D, V, nch;
  double inv_t;
  const float *root_logits, *logits;
  const double *row_lse, *root_lse;
  const float *q;
  const int32_t *cand_tok, *cand_len;
  const double *u_res;
  const int32_t *gate;
  const uint8_t *code;
  const double *pv;      // MULTI: [B][M+1][W] (see TestArgs)
  const double *u_acc;   // MULTI: [B, W, D]
  const int32_t *amax;   // GREEDY: [B*M + B] (see TestArgs)
  const uint8_t *amax_tie;
  int32_t *n_acc, *best, *out_tok, *n_out, *acc_per_cand, *flags;
  int flags_accumulate;
  int32_t *attn_flags;   // [B] or null: flags raised by attention, folded and reset here
  double2 *chunk_sums;   // [B][nch]: (residual-or-bonus weight sum, target p sum)
  uint32_t *counters;    // [B]
};

enum { SAMP_FUSED = 0, SAMP_SUMS = 1, SAMP_DRAW = 2 };
enum { RULE_LONGEST = 0, RULE_MULTI = 1, RULE_GREEDY = 2 };

// the per-sequence scalar outputs and the flags (with attention's, which are reset)
__device__ void store_scalars(const SampArgs &a, int b, int ab, int best, int f) {
  a.n_acc[b] = ab;
  a.best[b] = best;
  a.n_out[b] = ab + 1;
  if (a.attn_flags) {
    f |= a.attn_flags[b];
    a.attn_flags[b] = 0;      // ready for the next call on this workspace
  }
  if (a.flags) {
    if (a.flags_accumulate) atomicOr(&a.flags[b], f);
    else a.flags[b] = f;
  }
}

template <int PHASE, int RULE>
__global__ void __launch_bounds__(kST)
sampler_kernel(SampArgs a) {
  constexpr bool MULTI = RULE == RULE_MULTI;
  __shared__ SampSharedT<MULTI> sh;
  const int c = blockIdx.x;
  const int b = blockIdx.y;
  const int tid = threadIdx.x;
  const int W = a.W, D = a.D, V = a.V, M = W * D;
  const float *root = a.root_logits + (int64_t)b * V;

  if constexpr (MULTI) {
    extern __shared__ double multi_lds[];
    double *pv = multi_lds;                      // [M+1][W]
    double *uacc = multi_lds + (M + 1) * W;      // [M]
    // ---- one round of loads: lengths, tokens, uniforms, normalisers, p values
    const bool open = (a.gate == nullptr) || a.gate[b] != 0;
    if (tid == 0) sh.flags = 0;
    for (int i = tid; i < W; i += kST) {
      int ln = open ? a.cand_len[(int64_t)b * W + i] : 0;
      ln = ln < 0 ? 0 : (ln > D ? D : ln);
      sh.lens[i] = ln;
      sh.ures[i] = a.u_res ? a.u_res[(int64_t)b * W + i] : 0.0;   // greedy: not given
    }
    for (int idx = tid; idx < M; idx += kST) {
      sh.tok[idx] = a.cand_tok[(int64_t)b * M + idx];
      sh.rlse[idx] = a.row_lse[(int64_t)b * M + idx];
      uacc[idx] = a.u_acc[(int64_t)b * M + idx];
    }
    for (int k = tid; k < (M + 1) * W; k += kST) pv[k] = a.pv[(int64_t)b * (M + 1) * W + k];
    const double lse_root = a.root_lse[b];
    __syncthreads();
    // ---- the chain (one thread): depth by depth, siblings in index order against the
    //      reference row; each rejection removes its token's mass
    if (tid == 0) {
      int fl = 0;
      int ns = 0;
      for (int i = 0; i < W; ++i)
        if (sh.lens[i] >= 1) sh.surv[ns++] = i;
      sh.qrow = -1;
      sh.xpt = -1;
      sh.n_excl = 0;
      int depth = 0, row = M;      // row M: the root distribution
      if (ns == 0) {
        sh.best = -1;
        sh.mode = MODE_ROOT;
        sh.u = sh.ures[0];
        fl |= FLAG_NO_CANDIDATE;
      } else {
        while (true) {
          const int ref = sh.surv[0];
          row = (depth == 0) ? M : ref * D + depth - 1;
          int nsib = 0;
          for (int k = 0; k < ns; ++k)
            if (sh.lens[sh.surv[k]] > depth) sh.sib[nsib++] = sh.surv[k];
          if (nsib == 0) {
            sh.mode = MODE_BONUS;
            sh.u = sh.ures[ref];
            break;
          }
          double removed = 0.0;
          int n_excl = 0, last = sh.sib[0], acc = -1;
          for (int k = 0; k < nsib; ++k) {
            const int i = sh.sib[k];
            last = i;
            const int x = sh.tok[i * D + depth];
            const double pvv = pv[row * W + i];
            const bool valid = pvv >= 0.0;
            bool dup = false;
            for (int e = 0; e < n_excl; ++e) dup |= (sh.excl_tok[e] == x);
            if (!valid) fl |= FLAG_BAD_TOKEN;
            const double pp = (valid && !dup) ? pvv / (1.0 - removed) : 0.0;
            const double lhs = uacc[i * D + depth];
            if (fabs(lhs - pp) < 1e-4 * fmax(pp, lhs)) fl |= FLAG_ACCEPT_TIE;
            if (lhs < pp) {
              acc = x;
              break;
            }
            if (valid && !dup) {
              if (1.0 - (removed + pvv) > 0.0) {
                removed += pvv;
                sh.excl_tok[n_excl++] = x;
              } else {
                fl |= FLAG_DEGENERATE;
              }
            }
          }
          if (acc < 0) {
            sh.mode = MODE_RESID;
            sh.u = sh.ures[last];
            sh.n_excl = n_excl;
            break;
          }
          ns = 0;
          for (int k = 0; k < nsib; ++k)
            if (sh.tok[sh.sib[k] * D + depth] == acc) sh.surv[ns++] = sh.sib[k];
          ++depth;
        }
        sh.best = sh.surv[0];
      }
      sh.ab = depth;
      sh.prow = (row == M) ? -1 : (int64_t)b * M + row;
      sh.lse = (row == M) ? lse_root : sh.rlse[row];
      if (fl) atomicOr(&sh.flags, fl);
    }
  } else {
    // ---- one round of independent loads: lengths, acceptance codes, draft tokens, the
    //      residual uniforms and the normalisers of every row
    const bool open = (a.gate == nullptr) || a.gate[b] != 0;
    if (tid == 0) sh.flags = 0;
    for (int i = tid; i < W; i += kST) {
      int ln = open ? a.cand_len[(int64_t)b * W + i] : 0;
      ln = ln < 0 ? 0 : (ln > D ? D : ln);
      sh.lens[i] = ln;
      sh.a_len[i] = ln;
      sh.ures[i] = a.u_res ? a.u_res[(int64_t)b * W + i] : 0.0;   // greedy: not given
    }
    for (int idx = tid; idx < M; idx += kST) {
      sh.code[idx] = a.code[(int64_t)b * M + idx];
      sh.tok[idx] = a.cand_tok[(int64_t)b * M + idx];
      sh.rlse[idx] = a.row_lse[(int64_t)b * M + idx];
    }
    const double lse_root = a.root_lse[b];
    __syncthreads();
    // accepted run of each candidate: up to its first rejected position
    for (int idx = tid; idx < M; idx += kST) {
      const int i = idx / D, o = idx % D;
      if (o < sh.lens[i] && !(sh.code[idx] & CODE_ACCEPT)) atomicMin(&sh.a_len[i], o);
    }
    __syncthreads();
    int fl = 0;
    for (int idx = tid; idx < M; idx += kST) {
      const int i = idx / D, o = idx % D;
      if (o >= sh.lens[i]) continue;
      // only the tested positions (up to the first rejection) raise flags
      if (o > sh.a_len[i]) continue;
      const uint8_t cd = sh.code[idx];
      if (cd & CODE_BAD) fl |= FLAG_BAD_TOKEN;
      if (cd & CODE_TIE) fl |= FLAG_ACCEPT_TIE;
    }
    if (fl) atomicOr(&sh.flags, fl);

    // ---- the chosen candidate and the distribution of the extra token
    if (tid == 0) {
      int best = -1;
      for (int i = 0; i < W; ++i)
        if (sh.lens[i] >= 1 && (best < 0 || sh.a_len[i] > sh.a_len[best])) best = i;
      sh.best = best;
      sh.qrow = -1;
      sh.xpt = -1;
      int prow_local = -1;
      if (best < 0) {
        sh.ab = 0;
        sh.mode = MODE_ROOT;
        sh.u = sh.ures[0];
        atomicOr(&sh.flags, FLAG_NO_CANDIDATE);
      } else {
        const int ab = sh.a_len[best];
        sh.ab = ab;
        sh.u = sh.ures[best];
        prow_local = (ab == 0) ? -1 : best * D + ab - 1;
        if (ab < sh.lens[best]) {
          sh.mode = MODE_RESID;
          if (a.q) sh.qrow = (int64_t)b * M + best * D + ab;
          else sh.xpt = sh.tok[best * D + ab];
        } else {
          sh.mode = MODE_BONUS;
        }
      }
      sh.prow = (prow_local < 0) ? -1 : (int64_t)b * M + prow_local;
      sh.lse = (prow_local < 0) ? lse_root : sh.rlse[prow_local];
    }

  }
  __syncthreads();
  if constexpr (RULE == RULE_GREEDY) {
    // the extra token: the argmax of the row after the run, found with the tests
    const int64_t frow = (sh.prow < 0) ? (int64_t)a.B * M + b : sh.prow;
    const int best = sh.best, ab = sh.ab;
    if (tid == 0) store_scalars(a, b, ab, best, sh.flags | (a.amax_tie[frow] ? FLAG_CDF_TIE : 0));
    const int yy = a.amax[frow];
    int32_t *ot = a.out_tok + (int64_t)b * (D + 1);
    for (int o = tid; o <= D; o += kST)
      ot[o] = (o < ab) ? sh.tok[best * D + o] : (o == ab ? yy : -1);
    for (int i = tid; i < W; i += kST)
      a.acc_per_cand[(int64_t)b * W + i] = (sh.lens[i] >= 1) ? sh.a_len[i] : 0;
    return;
  }
  const float *zrow = (sh.prow < 0) ? root : a.logits + sh.prow * V;
  const double lse = sh.lse;
  const float *qrow = (sh.qrow < 0) ? nullptr : a.q + sh.qrow * V;
  const int xpt = sh.xpt;
  const bool resid = sh.mode == MODE_RESID;
  int n_excl = 0;
  if constexpr (MULTI) n_excl = sh.n_excl;

  // target probability and residual weight of the kPer ids k0 .. k0+kPer-1 (ids at or
  // past V weigh nothing)
  auto weights = [&](int k0, double *pk, double *rk) {
    float z[kPer], qv[kPer];
    // MULTI: the rejected tokens among k0 .. k0+kPer-1 (their point masses are removed)
    unsigned exm = 0;
    if constexpr (MULTI) {
      for (int e = 0; e < n_excl; ++e) {
        const unsigned j = (unsigned)(sh.excl_tok[e] - k0);
        if (j < (unsigned)kPer) exm |= 1u << j;
      }
    }
    if (k0 + kPer <= V) {
      const f32x4 z0 = *(const f32x4 *)(zrow + k0), z1 = *(const f32x4 *)(zrow + k0 + 4);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        z[j] = z0[j];
        z[4 + j] = z1[j];
      }
      if (qrow) {
        const f32x4 q0 = *(const f32x4 *)(qrow + k0), q1 = *(const f32x4 *)(qrow + k0 + 4);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          qv[j] = q0[j];
          qv[4 + j] = q1[j];
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < kPer; ++j) {
        z[j] = (k0 + j < V) ? zrow[k0 + j] : 0.f;
        qv[j] = (qrow && k0 + j < V) ? qrow[k0 + j] : 0.f;
      }
    }
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int k = k0 + j;
      if (k >= V) {
        pk[j] = 0.0;
        rk[j] = 0.0;
        continue;
      }
      pk[j] = exp((double)z[j] * a.inv_t - lse);
      if (resid) {
        double qk;
        if constexpr (MULTI) {
          qk = ((exm >> j) & 1u) ? 1.0 : 0.0;
        } else {
          qk = qrow ? (double)qv[j] : (k == xpt ? 1.0 : 0.0);
        }
        rk[j] = fmax(0.0, pk[j] - qk);
      } else {
        rk[j] = pk[j];
      }
    }
  };

  // ---- this chunk's sums: thread t owns the kPer consecutive ids c*kChunk + t*kPer ..
  //      (vector loads; 8 KB contiguous per chunk); its sums are kept for the draw
  double2 own = make_double2(0.0, 0.0);   // this workgroup's chunk sums (fused, nch == 1)
  if constexpr (PHASE != SAMP_DRAW) {
    double sr = 0.0, sp = 0.0;
    {
      double pk[kPer], rk[kPer];
      weights(c * kChunk + tid * kPer, pk, rk);
#pragma unroll
      for (int j = 0; j < kPer; ++j) {
        sr += rk[j];
        sp += pk[j];
      }
    }
    block_sum2(sh, sr, sp);
    if constexpr (PHASE == SAMP_SUMS) {
      if (tid == 0) a.chunk_sums[(int64_t)b * a.nch + c] = make_double2(sr, sp);
      return;
    } else if (a.nch == 1) {
      own = make_double2(sr, sp);   // the sequence's only workgroup: its sums are the totals
    } else {
      if (tid == 0) {
        // Publication: the sums are agent-scope atomic stores, and the counter increment
        // is an agent-scope acquire-release read-modify-write.  Its release half orders
        // this workgroup's sums before the increment; its acquire half, in the
        // workgroup that reads the final count, orders every other workgroup's sums
        // before the loads that follow.  (Only the few dozen workgroups of a small batch
        // take this path; large batches draw in a second launch.)
        uint64_t *cp = reinterpret_cast<uint64_t *>(a.chunk_sums + (int64_t)b * a.nch + c);
        __hip_atomic_store(cp, (uint64_t)__double_as_longlong(sr), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(cp + 1, (uint64_t)__double_as_longlong(sp), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
        const uint32_t old = __hip_atomic_fetch_add(&a.counters[b], 1u, __ATOMIC_ACQ_REL,
                                                    __HIP_MEMORY_SCOPE_AGENT);
        sh.is_last = (old == (uint32_t)(a.nch - 1));
      }
      __syncthreads();
      if (!sh.is_last) return;
    }
  }

  // ---- last workgroup of the sequence: total, owner chunk, owner thread, draw
  // chunk k's sums on thread k (nch <= kST)
  double2 cs = make_double2(0.0, 0.0);
  if (PHASE == SAMP_FUSED && a.nch == 1) {
    if (tid == 0) cs = own;
  } else if (tid < a.nch) {
    const uint64_t *cp = reinterpret_cast<const uint64_t *>(a.chunk_sums + (int64_t)b * a.nch + tid);
    cs.x = __longlong_as_double((long long)__hip_atomic_load(cp, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
    cs.y = __longlong_as_double((long long)__hip_atomic_load(cp + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
  }
  double S, xs;
  // the owner chunk: first with weight whose inclusive sum passes u*S; if rounding
  // leaves u*S at or past the total, the last chunk with weight
  if (a.nch <= 64) {
    // the chunk sums lie in wave 0: its shuffles and ballots replace the block's
    // reductions and scans (the other waves would add zeros: the same numbers)
    if (tid < 64) {
      const double Sx = warp_sum(cs.x), Sy = warp_sum(cs.y);
      const bool use_target = !(Sx > 0.0);
      const double St = use_target ? Sy : Sx;
      const double xt = sh.u * St;
      const double v = use_target ? cs.y : cs.x;
      double incl = v;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const double y = __shfl_up(incl, off);
        if (tid >= off) incl += y;
      }
      const bool has = tid < a.nch && v > 0.0;
      const uint64_t passed = __ballot(has && incl > xt);
      const uint64_t weighted = __ballot(has);
      int own = passed ? __builtin_ctzll(passed) : (weighted ? 63 - __builtin_clzll(weighted) : a.nch - 1);
      const double ex = __shfl(incl - v, own);
      if (tid == 0) {
        sh.owner = own;
        sh.excl = ex;
        sh.tot = St;
        sh.xs = xt;
        sh.tstar = INT_MAX;
        if (use_target) {
          sh.mode = MODE_TARGET;
          atomicOr(&sh.flags, FLAG_DEGENERATE);
        }
        if (PHASE == SAMP_FUSED) a.counters[b] = 0u;   // ready for the next call on this workspace
      }
    }
    __syncthreads();
    S = sh.tot;
    xs = sh.xs;
  } else {
    double Sx = cs.x, Sy = cs.y;
    block_sum2(sh, Sx, Sy);
    const bool use_target = !(Sx > 0.0);
    S = use_target ? Sy : Sx;
    xs = sh.u * S;
    const double v = use_target ? cs.y : cs.x;
    const double incl = block_incl_scan(sh, v);
    if (tid == 0) {
      sh.owner = INT_MAX;
      sh.last_pos = -1;
      sh.tstar = INT_MAX;
      if (use_target) {
        sh.mode = MODE_TARGET;
        atomicOr(&sh.flags, FLAG_DEGENERATE);
      }
      if (PHASE == SAMP_FUSED) a.counters[b] = 0u;   // ready for the next call on this workspace
    }
    __syncthreads();
    if (tid < a.nch && v > 0.0) {
      if (incl > xs) atomicMin(&sh.owner, tid);
      atomicMax(&sh.last_pos, tid);
    }
    __syncthreads();
    if (sh.owner == INT_MAX && tid == 0) sh.owner = sh.last_pos >= 0 ? sh.last_pos : a.nch - 1;
    __syncthreads();
    if (tid == sh.owner) sh.excl = incl - v;
    __syncthreads();
  }
  const int owner = sh.owner;
  const bool use_p = sh.mode == MODE_TARGET;
  // the owner chunk's per-thread sums, recomputed (same arithmetic, same order as its
  // workgroup's): the thread whose range holds u*S
  double pk[kPer], rk[kPer];
  weights(owner * kChunk + tid * kPer, pk, rk);
  double tv = 0.0;
#pragma unroll
  for (int j = 0; j < kPer; ++j) tv += use_p ? pk[j] : rk[j];
  const double tincl = block_incl_scan(sh, tv);
  const double texcl = sh.excl + (tincl - tv);
  if (tv > 0.0 && sh.excl + tincl > xs) atomicMin(&sh.tstar, tid);
  __syncthreads();
  const int best = sh.best, ab = sh.ab;
  __shared__ int y_sh;
  if (tid == sh.tstar || (sh.tstar == INT_MAX && tid == 0)) {
    int f = sh.flags;
    int yy = -1;
    if (sh.tstar != INT_MAX) {
      double run = texcl;
      double lo = 0.0, hi = 0.0;
      int last_w = -1;
      for (int j = 0; j < kPer; ++j) {
        const double w = use_p ? pk[j] : rk[j];
        const double prev = run;
        run += w;
        if (w > 0.0) last_w = owner * kChunk + tid * kPer + j;
        if (yy < 0 && w > 0.0 && run > xs) {
          yy = owner * kChunk + tid * kPer + j;
          lo = prev;
          hi = run;
        }
      }
      if (yy >= 0 && (fabs(xs - lo) < 1e-8 * S || fabs(hi - xs) < 1e-8 * S)) f |= FLAG_CDF_TIE;
      if (yy < 0) {
        // the sequential re-sum fell a rounding step short of the scan: last weighted id
        yy = last_w;
        f |= FLAG_CDF_TIE;
      }
    }
    if (yy < 0) {
      // rounding at a chunk or thread edge left u*S past the scan: last id of the chunk
      yy = min(V, (owner + 1) * kChunk) - 1;
      f |= FLAG_CDF_TIE;
    }
    y_sh = yy;
    store_scalars(a, b, ab, best, f);
  }
  __syncthreads();
  const int yy = y_sh;
  int32_t *ot = a.out_tok + (int64_t)b * (D + 1);
  for (int o = tid; o <= D; o += kST)
    ot[o] = (o < ab) ? sh.tok[best * D + o] : (o == ab ? yy : -1);
  for (int i = tid; i < W; i += kST) {
    int k = 0;
    if constexpr (MULTI) {
      // common prefix with the emitted accepted tokens (those of the final reference)
      const int lim = min(sh.lens[i], ab);
      while (k < lim && sh.tok[i * D + k] == sh.tok[best * D + k]) ++k;
    } else {
      k = (sh.lens[i] >= 1) ? sh.a_len[i] : 0;
    }
    a.acc_per_cand[(int64_t)b * W + i] = k;
  }
}

// (max, sum exp(x - max)) of x = logits/T over one vocabulary tile, for B rows;
// stats layout [B][n_vt].
__global__ void __launch_bounds__(256)
root_stats_kernel(const float *root_logits, int B, int V, float inv_t, float2 *stats) {
  const int vt = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int n_vt = (V + kHeadVocabTile - 1) / kHeadVocabTile;
  for (int b = blockIdx.y * 4 + wv; b < B; b += 4 * gridDim.y) {
    const float *row = root_logits + (int64_t)b * V;
    float x[kHeadVocabTile / 64];
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < kHeadVocabTile / 64; ++j) {
      const int k = vt * kHeadVocabTile + j * 64 + lane;
      x[j] = (k < V) ? row[k] * inv_t : -INFINITY;
      mx = fmaxf(mx, x[j]);
    }
    for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < kHeadVocabTile / 64; ++j)
      if (x[j] != -INFINITY) s += expf(x[j] - mx);
    for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
    if (lane == 0) stats[(int64_t)b * n_vt + vt] = make_float2(mx, s);
  }
}

// ---------------------------------------------------------------------------------
// Draft tokens: row r of stored draft probabilities q (fp32, as the low-rank head
// writes them) gives the id k = min{k : C_k > u_r * S} of its running sum C over
// ascending ids, S = C_{V-1} -- the sampler's inverse-CDF draw with the same chunk
// structure: per-chunk and per-thread fp64 sums, then one workgroup per row scans the
// chunk sums, the owner chunk's thread sums and one thread's 8 ids.
struct DraftArgs {
  const float *q;
  const double *u;
  int rows, V, nch;
  int32_t *tok, *flags;
  double *chunk_sums;    // [rows][nch]
};

__device__ __forceinline__ void draft_vals(const DraftArgs &a, int r, int k0, double *w) {
  const float *row = a.q + (int64_t)r * a.V;
#pragma unroll
  for (int j = 0; j < kPer; ++j) w[j] = (k0 + j < a.V) ? (double)row[k0 + j] : 0.0;
}

__global__ void __launch_bounds__(kST)
draft_sums_kernel(DraftArgs a) {
  __shared__ double red[kST / 64];
  const int c = blockIdx.x, r = blockIdx.y, tid = threadIdx.x;
  double w[kPer];
  draft_vals(a, r, c * kChunk + tid * kPer, w);
  double s = 0.0;
#pragma unroll
  for (int j = 0; j < kPer; ++j) s += w[j];
  s = warp_sum(s);
  if ((tid & 63) == 0) red[tid >> 6] = s;
  __syncthreads();
  if (tid == 0) a.chunk_sums[(int64_t)r * a.nch + c] = (red[0] + red[1]) + (red[2] + red[3]);
}

__global__ void __launch_bounds__(kST)
draft_draw_kernel(DraftArgs a) {
  __shared__ SampShared sh;
  const int r = blockIdx.x, tid = threadIdx.x;
  const double cs = (tid < a.nch) ? a.chunk_sums[(int64_t)r * a.nch + tid] : 0.0;
  double S = cs, unused = 0.0;
  block_sum2(sh, S, unused);
  const double xs = a.u[r] * S;
  const double incl = block_incl_scan(sh, cs);
  if (tid == 0) {
    sh.owner = INT_MAX;
    sh.last_pos = -1;
    sh.tstar = INT_MAX;
    sh.flags = 0;
  }
  __syncthreads();
  if (tid < a.nch && cs > 0.0) {
    if (incl > xs) atomicMin(&sh.owner, tid);
    atomicMax(&sh.last_pos, tid);
  }
  __syncthreads();
  if (tid == 0 && sh.owner == INT_MAX) {
    // rounding left u*S at or past the total (or a row without mass): last chunk with mass
    sh.owner = sh.last_pos >= 0 ? sh.last_pos : a.nch - 1;
    sh.flags = FLAG_CDF_TIE;
  }
  __syncthreads();
  if (tid == sh.owner) sh.excl = incl - cs;
  __syncthreads();
  const int owner = sh.owner;
  // the owner chunk's per-thread sums, recomputed in the sums kernel's order
  double w[kPer];
  const int k0 = owner * kChunk + tid * kPer;
  draft_vals(a, r, k0, w);
  double tv = 0.0;
#pragma unroll
  for (int j = 0; j < kPer; ++j) tv += w[j];
  const double tincl = block_incl_scan(sh, tv);
  const double texcl = sh.excl + (tincl - tv);
  if (tv > 0.0 && sh.excl + tincl > xs) atomicMin(&sh.tstar, tid);
  __syncthreads();
  if (tid == sh.tstar || (sh.tstar == INT_MAX && tid == 0)) {
    int f = sh.flags;
    int yy = -1;
    if (sh.tstar != INT_MAX) {
      double run = texcl, lo = 0.0, hi = 0.0;
      int last_w = -1;
      for (int j = 0; j < kPer; ++j) {
        const double prev = run;
        run += w[j];
        if (w[j] > 0.0) last_w = k0 + j;
        if (yy < 0 && w[j] > 0.0 && run > xs) {
          yy = k0 + j;
          lo = prev;
          hi = run;
        }
      }
      if (yy >= 0 && (fabs(xs - lo) < 1e-8 * S || fabs(hi - xs) < 1e-8 * S)) f |= FLAG_CDF_TIE;
      if (yy < 0) {
        yy = last_w;
        f |= FLAG_CDF_TIE;
      }
    }
    if (yy < 0) {
      yy = min(a.V, (owner + 1) * kChunk) - 1;
      f |= FLAG_CDF_TIE;
    }
    a.tok[r] = yy;
    if (a.flags) a.flags[r] = f;
  }
}

}  // namespace

size_t draft_workspace_bytes(int rows, int V) {
  const int nch = (V + kChunk - 1) / kChunk;
  return (((size_t)rows * nch * sizeof(double)) + 255) & ~(size_t)255;
}

hipError_t launch_draft_sample(const float *q, int rows, int V, const double *u, int32_t *tok,
                               int32_t *flags, void *ws, hipStream_t st) {
  DraftArgs a;
  a.q = q;
  a.u = u;
  a.rows = rows;
  a.V = V;
  a.nch = (V + kChunk - 1) / kChunk;
  a.tok = tok;
  a.flags = flags;
  a.chunk_sums = (double *)ws;
  hipLaunchKernelGGL(draft_sums_kernel, dim3(a.nch, rows), dim3(kST), 0, st, a);
  if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  hipLaunchKernelGGL(draft_draw_kernel, dim3(rows), dim3(kST), 0, st, a);
  return hipGetLastError();
}

SampleWs sample_ws(void *ws, int B, int W, int D, int V, bool row_stats) {
  SampleWs w;
  const int n_vt = (V + kHeadVocabTile - 1) / kHeadVocabTile;
  const int nch = (V + kChunk - 1) / kChunk;
  char *p = (char *)ws;
  size_t off = 0;
  w.counters = (uint32_t *)(p + off);
  off += ((size_t)B * sizeof(uint32_t) + 255) & ~(size_t)255;
  w.chunk_sums = (double2 *)(p + off);
  off += ((size_t)B * nch * sizeof(double2) + 255) & ~(size_t)255;
  w.root_stats = (float2 *)(p + off);
  off += ((size_t)B * n_vt * sizeof(float2) + 255) & ~(size_t)255;
  w.root_lse = (double *)(p + off);
  off += ((size_t)B * sizeof(double) + 255) & ~(size_t)255;
  w.code = (uint8_t *)(p + off);
  off += ((size_t)B * W * D + 255) & ~(size_t)255;
  w.attn_flags = (int32_t *)(p + off);
  off += ((size_t)B * sizeof(int32_t) + 255) & ~(size_t)255;
  w.pv = (double *)(p + off);
  off += ((size_t)B * (W * D + 1) * W * sizeof(double) + 255) & ~(size_t)255;
  w.amax = (int32_t *)(p + off);
  off += ((size_t)B * (W * D + 1) * sizeof(int32_t) + 255) & ~(size_t)255;
  w.amax_tie = (uint8_t *)(p + off);
  off += ((size_t)B * (W * D + 1) + 255) & ~(size_t)255;
  // lossless multi-candidate acceptance with dense drafts: two fp64 residual rows per
  // sequence
  w.resid = (double *)(p + off);
  off += ((size_t)B * 2 * V * sizeof(double) + 255) & ~(size_t)255;
  w.dpart = (double *)(p + off);
  off += ((size_t)B * 2 * kMaxCChunks * sizeof(double) + 255) & ~(size_t)255;
  w.row_stats = nullptr;
  if (row_stats) {
    w.row_stats = (float2 *)(p + off);
    off += ((size_t)B * W * D * n_vt * sizeof(float2) + 255) & ~(size_t)255;
  }
  w.bytes = off;
  return w;
}

bool sampler_multi_fits(int W, int D) {
  return W <= kMaxWMulti && multi_lds_doubles(W, D) <= kMaxMultiLds;
}

size_t sample_workspace_bytes(int B, int W, int D, int V, bool row_stats) {
  return sample_ws(nullptr, B, W, D, V, row_stats).bytes;
}

hipError_t launch_root_stats(const float *root_logits, int B, int V, float temperature,
                             float2 *stats, hipStream_t st) {
  const int n_vt = (V + kHeadVocabTile - 1) / kHeadVocabTile;
  hipLaunchKernelGGL(root_stats_kernel, dim3(n_vt), dim3(256), 0, st, root_logits, B, V,
                     1.0f / temperature, stats);
  return hipGetLastError();
}

hipError_t launch_row_stats(const float *logits, int rows, int V, float temperature,
                            float2 *stats, hipStream_t st) {
  const int n_vt = (V + kHeadVocabTile - 1) / kHeadVocabTile;
  const int gy = min((rows + 3) / 4, 256);
  hipLaunchKernelGGL(root_stats_kernel, dim3(n_vt, gy), dim3(256), 0, st, logits, rows, V,
                     1.0f / temperature, stats);
  return hipGetLastError();
}

hipError_t launch_lse_from_stats(const float2 *stats, int rows, int V, double *lse,
                                 hipStream_t st) {
  TestArgs a{};
  a.B = rows;
  a.W = 1;
  a.D = 1;
  a.V = V;
  a.n_vt = (V + kHeadVocabTile - 1) / kHeadVocabTile;
  a.row_stats = stats;
  a.row_lse = lse;
  hipLaunchKernelGGL(lse_tests_kernel, dim3(rows), dim3(256), 0, st, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------
// Lossless multi-candidate acceptance with dense drafts (accept mode MULTI, q given).
// The single-draft rule and its residual (rejection-sampling blog, section 3) applied
// across the sibling candidates at each depth: with the current residual p' (the
// target p of the reference row at first), sibling i is kept iff u * Q_i(x_i) <
// p'(x_i) / sum p', and a rejection sets p' <- max(0, p' / sum p' - Q_i) over the whole
// vocabulary.  The chain itself is serial: every rejection needs the new residual's
// total before the next sibling is tested.
//
// G workgroups per sequence share the vocabulary passes: the ids are cut into chunks of
// kCChunk (thread t of a workgroup holds ids 8t .. 8t+7 of a chunk) and workgroup c of
// the sequence owns chunks c, c+G, c+2G, ...  Every workgroup repeats the (cheap)
// decisions of the chain; a pass over the vocabulary (the exact total of a target row,
// a new residual, the sums of a draw) has each workgroup sum its own chunks in a fixed
// order and publish the chunk sums, then a barrier of the sequence's G workgroups (a
// counter in the workspace, agent-scope release on arrival and acquire while waiting),
// after which every workgroup adds all chunk sums in chunk order -- the same total, bit
// for bit, everywhere.  Residual rows live in the workspace (two fp64 rows per sequence,
// written alternately); a workgroup only ever reads back its own chunks of them.  The
// residual at a sibling's token, which may lie in another workgroup's chunk, is
// replayed from the target row and the removals made so far at this depth -- the same
// operations in the same order as the pass that stored it, so the same bits.  The draw
// is the inverse CDF over ascending ids: the chunk holding u * S is found from the
// chunk sums by every workgroup, and its owner scans it and writes the outputs.
//
// The G workgroups of a sequence must be resident together: with G > 1 the kernel goes
// out as a cooperative launch (which fails rather than oversubscribe); G = 1 needs
// nothing.  A wait gives up after kSpinLimit polls (FLAG_SYNC_TIMEOUT), so a kernel
// always ends.
constexpr int kCT = 512;
constexpr int kCPer = 8;
constexpr int kCChunk = kCT * kCPer;     // 4,096 ids
constexpr int kMaxCoopWg = 32;           // workgroups per sequence
constexpr int kSpinLimit = 1 << 20;
constexpr int kPvCache = 1024;           // p of the candidates' tokens, kept in LDS when it fits

struct DenseShared {
  double red[kCT / 64];
  double csum[kMaxCChunks];              // chunk sums of the last pass, all chunks
  double hist_s[kMaxWMulti];             // removals at this depth: the total before each
  int hist_q[kMaxWMulti];                // and the draft row it removed
  int lens[kMaxWMulti];
  double ures[kMaxWMulti];
  int tok[kMaxRows];
  double uacc[kMaxRows];
  double rlse[kMaxRows];
  float qx[kMaxRows];                    // Q of each candidate token at its own depth
  double pvc[kPvCache];                  // copy of pv when (W*D+1)*W fits
  int acc[kMaxRows];
  int surv[kMaxWMulti], sib[kMaxWMulti];
  int flags, owner, tstar, y;
  double excl;
};

struct DenseArgs {
  int B, W, D, V, G;
  double inv_t;
  const float *root_logits, *logits, *q;
  const double *row_lse, *root_lse;
  const double *pv;       // [B][W*D+1][W] p of every candidate's token under each row
  const int32_t *cand_tok, *cand_len, *gate;
  const double *u_acc, *u_res;
  double *resid;          // [B][2][V]
  double *part;           // [B][2][kMaxCChunks] published chunk sums (two pass parities)
  uint32_t *bar;          // [B] barrier counters, zero between calls
  int32_t *n_acc, *best, *out_tok, *n_out, *acc_per_cand, *flags;
  int flags_accumulate;
  int32_t *attn_flags;
};

// fixed-order block sum over kCT threads (every thread receives the total)
__device__ double dense_sum(DenseShared &sh, double v) {
  const int tid = threadIdx.x;
  v = warp_sum(v);
  if ((tid & 63) == 0) sh.red[tid >> 6] = v;
  __syncthreads();
  double t = 0.0;
#pragma unroll
  for (int w = 0; w < kCT / 64; ++w) t += sh.red[w];
  __syncthreads();
  return t;
}

__device__ double dense_incl_scan(DenseShared &sh, double v) {
  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const double y = __shfl_up(v, off);
    if (lane >= off) v += y;
  }
  if (lane == 63) sh.red[wv] = v;
  __syncthreads();
  double base = 0.0;
  for (int w = 0; w < wv; ++w) base += sh.red[w];
  __syncthreads();
  return base + v;
}

// (four waves per SIMD, i.e. at most 128 VGPRs: the runtime's occupancy check for a
// cooperative launch finds no room for a 512-thread workgroup above that)
__global__ void __launch_bounds__(kCT, 4)
multi_dense_kernel(DenseArgs a) {
  __shared__ DenseShared sh;
  const int c0 = blockIdx.x;          // this workgroup's place among the sequence's G
  const int b = blockIdx.y;
  const int tid = threadIdx.x;
  const int G = a.G;
  const int W = a.W, D = a.D, V = a.V, M = W * D;
  const int nch = (V + kCChunk - 1) / kCChunk;
  const bool open = (a.gate == nullptr) || a.gate[b] != 0;
  for (int i = tid; i < W; i += kCT) {
    int ln = open ? a.cand_len[(int64_t)b * W + i] : 0;
    sh.lens[i] = ln < 0 ? 0 : (ln > D ? D : ln);
    sh.ures[i] = a.u_res[(int64_t)b * W + i];
  }
  // everything the acceptance tests read, loaded at once: an accepted depth then needs
  // no memory access (p of the tokens comes from the normaliser pass, pv, formed there
  // with the same arithmetic as p_at below)
  const bool pv_lds = (M + 1) * W <= kPvCache;
  for (int k = tid; k < M; k += kCT) {
    const int x = a.cand_tok[(int64_t)b * M + k];
    sh.tok[k] = x;
    sh.uacc[k] = a.u_acc[(int64_t)b * M + k];
    sh.rlse[k] = a.row_lse[(int64_t)b * M + k];
    sh.qx[k] = (x >= 0 && x < V) ? a.q[((int64_t)b * M + k) * V + x] : 1.0f;
  }
  if (pv_lds)
    for (int k = tid; k < (M + 1) * W; k += kCT) sh.pvc[k] = a.pv[(int64_t)b * (M + 1) * W + k];
  if (tid == 0) sh.flags = 0;
  __syncthreads();
  double *rbuf[2] = {a.resid + (int64_t)b * 2 * V, a.resid + ((int64_t)b * 2 + 1) * V};
  uint32_t *bar = a.bar + b;
  double *part = a.part + (int64_t)b * 2 * kMaxCChunks;
  int n_bar = 0, par = 0;

  // barrier of the sequence's G workgroups, then every workgroup reads all chunk sums
  // of the pass (published in parity `par`) into LDS and returns their total
  auto sync_sums = [&]() -> double {
    __syncthreads();
    ++n_bar;
    if (tid < 64) {
      if (tid == 0) __hip_atomic_fetch_add(bar, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
      const uint32_t target = (uint32_t)n_bar * (uint32_t)G;
      // poll with plain atomic loads, then one acquire (an acquiring load in the loop
      // would invalidate this XCD's L2 on every poll, under the other workgroups' feet)
      int spins = 0;
      while (__hip_atomic_load(bar, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
        __builtin_amdgcn_s_sleep(1);
        if (++spins > kSpinLimit) {
          if (tid == 0) atomicOr(&sh.flags, FLAG_SYNC_TIMEOUT);
          break;
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      for (int c = tid; c < nch; c += 64)
        sh.csum[c] = __hip_atomic_load(part + par * kMaxCChunks + c, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    double S = 0.0;
    for (int c = 0; c < nch; ++c) S += sh.csum[c];
    par ^= 1;
    return S;
  };
  auto publish = [&](int c, double v) {
    if (tid == 0)
      __hip_atomic_store(part + par * kMaxCChunks + c, v, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
  };

  // the distribution a pass reads: p of row prow (kind 0), or the residual in rbuf[cur]
  // (kind 1, this workgroup's chunks only); lse of that row
  const float *zrow = nullptr;
  double lse = 0.0;
  int kind = 0, cur = 0;
  auto p_at = [&](int k) -> double { return exp((double)zrow[k] * a.inv_t - lse); };
  auto weight = [&](int k) -> double {
    if (k >= V) return 0.0;
    if (kind == 0) return p_at(k);
    return rbuf[cur][k];
  };
  auto set_row = [&](int prow) {
    kind = 0;
    zrow = prow < 0 ? a.root_logits + (int64_t)b * V : a.logits + ((int64_t)b * M + prow) * V;
    lse = prow < 0 ? a.root_lse[b] : sh.rlse[prow];
  };
  // chunk sums of the current distribution (this workgroup's chunks), then everyone's
  auto sum_pass = [&]() -> double {
    for (int c = c0; c < nch; c += G) {
      const int k0 = c * kCChunk + tid * kCPer;
      double v = 0.0;
#pragma unroll
      for (int j = 0; j < kCPer; ++j) v += weight(k0 + j);
      publish(c, dense_sum(sh, v));
    }
    return sync_sums();
  };
  // the current distribution at candidate j's token x, whichever workgroup owns it: the
  // target row's p(x) followed by this depth's removals, as the passes that stored them
  // computed it
  int n_hist = 0, pvrow = M;
  auto value_at = [&](int j0, int x) -> double {
    const int idx = pvrow * W + j0;
    double w = pv_lds ? sh.pvc[idx] : a.pv[(int64_t)b * (M + 1) * W + idx];
    for (int j = 0; j < n_hist; ++j) {
      const float *qr = a.q + ((int64_t)b * M + sh.hist_q[j]) * V;
      w = fmax(0.0, w / sh.hist_s[j] - (double)qr[x]);
    }
    return w;
  };
  // inverse-CDF draw with uniform u from the distribution whose chunk sums are in
  // sh.csum (total S); only the owner of the chunk holding u*S finds the token
  auto draw = [&](double u, double S) -> int {
    const double xs = u * S;
    if (tid == 0) {
      // the chunk holding u*S (the last chunk with weight if rounding leaves u*S past)
      double run = 0.0;
      int own = -1, last = nch - 1;
      for (int c = 0; c < nch; ++c) {
        if (sh.csum[c] > 0.0) last = c;
        if (own < 0 && sh.csum[c] > 0.0 && run + sh.csum[c] > xs) own = c;
        if (own < 0) run += sh.csum[c];
      }
      if (own < 0) {
        own = last;
        run = 0.0;
        for (int c = 0; c < last; ++c) run += sh.csum[c];
      }
      sh.owner = own;
      sh.excl = run;
      sh.tstar = INT_MAX;
      sh.y = -1;
    }
    __syncthreads();
    if (sh.owner % G != c0) return -1;
    const int k0 = sh.owner * kCChunk + tid * kCPer;
    double w[kCPer], tv = 0.0;
#pragma unroll
    for (int j = 0; j < kCPer; ++j) {
      w[j] = weight(k0 + j);
      tv += w[j];
    }
    const double incl = dense_incl_scan(sh, tv);
    const double texcl = sh.excl + (incl - tv);
    if (tv > 0.0 && sh.excl + incl > xs) atomicMin(&sh.tstar, tid);
    __syncthreads();
    if (tid == sh.tstar || (sh.tstar == INT_MAX && tid == 0)) {
      int yy = -1, last_w = -1;
      double run = texcl, lo = 0.0, hi = 0.0;
      if (sh.tstar != INT_MAX) {
        for (int j = 0; j < kCPer; ++j) {
          if (w[j] <= 0.0) continue;
          last_w = k0 + j;
          if (run + w[j] > xs) {
            yy = k0 + j;
            lo = run;
            hi = run + w[j];
            break;
          }
          run += w[j];
        }
        if (yy < 0) {
          yy = last_w;
          lo = run;
          hi = run;
        }
      } else {
        yy = V - 1;
        lo = hi = S;
      }
      if (fmin(fabs(xs - lo), fabs(hi - xs)) < 1e-8 * S) atomicOr(&sh.flags, FLAG_CDF_TIE);
      sh.y = yy;
    }
    __syncthreads();
    return sh.y;
  };

  if (tid == 0) {
    int n = 0;
    for (int i = 0; i < W; ++i)
      if (sh.lens[i] >= 1) sh.surv[n++] = i;
  }
  __syncthreads();
  int ns = 0;   // survivors (every thread keeps the same count)
  for (int i = 0; i < W; ++i) ns += sh.lens[i] >= 1;
  int depth = 0, y = -1, best = -1;
  if (ns == 0) {
    set_row(-1);
    y = draw(sh.ures[0], sum_pass());
    if (tid == 0) atomicOr(&sh.flags, FLAG_NO_CANDIDATE);
  } else {
    while (true) {
      const int ref = sh.surv[0];
      set_row(depth == 0 ? -1 : ref * D + depth - 1);
      pvrow = depth == 0 ? M : ref * D + depth - 1;
      n_hist = 0;
      int nsib = 0;
      for (int k = 0; k < ns; ++k)
        if (sh.lens[sh.surv[k]] > depth) {
          if (tid == 0) sh.sib[nsib] = sh.surv[k];
          ++nsib;
        }
      __syncthreads();
      if (nsib == 0) {
        y = draw(sh.ures[ref], sum_pass());
        break;
      }
      // a target row sums to one up to the rounding of its lse, which moves p' by about
      // 1e-7 relative: close enough for the acceptance tests, whose tie band is 1e-4;
      // its exact total is taken only before the first rejection builds a residual
      double S = 1.0;
      bool exact = false;
      bool sums_valid = false;   // sh.csum holds the current distribution's chunk sums
      int accepted = -1, last = sh.sib[0];
      for (int k = 0; k < nsib; ++k) {
        const int i = sh.sib[k];
        last = i;
        const int x = sh.tok[i * D + depth];
        const int qr = i * D + depth;
        const float *qrow = a.q + ((int64_t)b * M + qr) * V;
        const bool valid = x >= 0 && x < V;
        const double pp = valid ? value_at(i, x) / S : 0.0;
        const double Qx = valid ? (double)sh.qx[qr] : 1.0;
        const double lhs = sh.uacc[i * D + depth] * Qx;
        if (tid == 0) {
          int f = 0;
          if (!valid) f |= FLAG_BAD_TOKEN;
          if (fabs(lhs - pp) < 1e-4 * fmax(pp, lhs)) f |= FLAG_ACCEPT_TIE;
          if (f) atomicOr(&sh.flags, f);
        }
        if (lhs < pp) {
          accepted = x;
          break;
        }
        // rejected: p' <- max(0, p' / S - Q_i) into the residual row not being read
        if (!exact) {
          S = sum_pass();
          exact = true;
        }
        const int nxt = (kind == 1) ? (cur ^ 1) : 0;
        double *dst = rbuf[nxt];
        for (int c = c0; c < nch; c += G) {
          const int k0 = c * kCChunk + tid * kCPer;
          // all loads first: the stores below may alias them as far as the compiler
          // knows, and would otherwise serialise every load behind the previous store
          double wv[kCPer];
          float qv[kCPer];
#pragma unroll
          for (int j = 0; j < kCPer; ++j) {
            const int kk = k0 + j;
            wv[j] = weight(kk);
            qv[j] = kk < V ? qrow[kk] : 0.0f;
          }
          double v = 0.0;
#pragma unroll
          for (int j = 0; j < kCPer; ++j) {
            const int kk = k0 + j;
            if (kk < V) {
              const double r = fmax(0.0, wv[j] / S - (double)qv[j]);
              dst[kk] = r;
              v += r;
            }
          }
          publish(c, dense_sum(sh, v));
        }
        const double part_s = sync_sums();
        if (part_s > 0.0) {
          if (tid == 0) {
            sh.hist_s[n_hist] = S;
            sh.hist_q[n_hist] = qr;
          }
          ++n_hist;
          cur = nxt;
          kind = 1;
          S = part_s;   // exact: summed in the pass that wrote the row
          sums_valid = true;
        } else {
          if (tid == 0) atomicOr(&sh.flags, FLAG_DEGENERATE);   // no mass left: p' is kept
          sums_valid = false;
        }
        __syncthreads();   // the row and the history are complete before they are read
      }
      if (accepted < 0) {
        // every sibling rejected: draw from p' (its chunk sums are the last pass's
        // unless that removal was skipped)
        const double Sd = sums_valid ? S : sum_pass();
        y = draw(sh.ures[last], Sd);
        break;
      }
      if (tid == 0) {
        sh.acc[depth] = accepted;
        int n2 = 0;
        for (int k = 0; k < nsib; ++k)
          if (sh.tok[sh.sib[k] * D + depth] == accepted) sh.surv[n2++] = sh.sib[k];
      }
      __syncthreads();
      int n2 = 0;
      for (int k = 0; k < nsib; ++k) n2 += sh.tok[sh.sib[k] * D + depth] == accepted;
      ns = n2;
      ++depth;
    }
    best = sh.surv[0];
  }
  // ---- outputs, from the workgroup that drew the token
  if (y >= 0) {
    int32_t *ot = a.out_tok + (int64_t)b * (D + 1);
    for (int o = tid; o <= D; o += kCT) ot[o] = (o < depth) ? sh.acc[o] : (o == depth ? y : -1);
    for (int i = tid; i < W; i += kCT) {
      int k = 0;
      const int lim = min(sh.lens[i], depth);
      while (k < lim && sh.tok[i * D + k] == sh.acc[k]) ++k;
      a.acc_per_cand[(int64_t)b * W + i] = k;
    }
    if (tid == 0) {
      a.n_acc[b] = depth;
      a.best[b] = best;
      a.n_out[b] = depth + 1;
      int f = sh.flags;
      if (a.attn_flags) {
        f |= a.attn_flags[b];
        a.attn_flags[b] = 0;
      }
      if (a.flags) {
        if (a.flags_accumulate) atomicOr(&a.flags[b], f);
        else a.flags[b] = f;
      }
    }
  }
  // the last workgroup of the sequence to leave puts the counter back to zero
  if (tid == 0) {
    const uint32_t old = __hip_atomic_fetch_add(bar, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (old == (uint32_t)(n_bar + 1) * (uint32_t)G - 1u)
      __hip_atomic_store(bar, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Workgroups per sequence for the dense multi-candidate chain: up to kMaxCoopWg, no more
// than the vocabulary has chunks, and all B*G of them resident at once (the device's
// cooperative-launch support and the kernel's occupancy, looked up once per device).
// VSTEP_DENSE_WG=n caps it (1: one workgroup per sequence, a plain launch).
int dense_width(int B, int nch) {
  static std::mutex mu;
  static int cap[64], coop[64];
  static bool known[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 1;
  {
    std::lock_guard<std::mutex> lock(mu);
    if (!known[dev]) {
      int cus = 0, per_cu = 0, c = 0;
      if (hipDeviceGetAttribute(&c, hipDeviceAttributeCooperativeLaunch, dev) != hipSuccess) c = 0;
      if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        cus = 0;
      if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, multi_dense_kernel, kCT, 0) !=
          hipSuccess)
        per_cu = 0;
      cap[dev] = cus * per_cu;
      coop[dev] = c;
      known[dev] = true;
    }
  }
  int g = kMaxCoopWg;
  if (const char *e = getenv("VSTEP_DENSE_WG")) {
    const int v = atoi(e);
    if (v >= 1 && v < g) g = v;
  }
  g = g < nch ? g : nch;
  if (!coop[dev] || B <= 0) return 1;
  const int fit = cap[dev] / B;
  g = g < fit ? g : fit;
  return g < 1 ? 1 : g;
}

hipError_t launch_lse_tests(int B, int W, int D, int V, float temperature,
                            const float2 *row_stats, double *row_lse, const float *root_logits,
                            const float *logits, const float *q, const int32_t *cand_tok,
                            const int32_t *cand_len, const int32_t *gate, const double *u_acc,
                            const SampleWs &ws, hipStream_t st, int rule,
                            const float2 *am_stats) {
  const bool multi = rule == 1, greedy = rule == 2;
  TestArgs a{};
  a.B = B;
  a.W = W;
  a.D = D;
  a.V = V;
  a.n_vt = (V + kHeadVocabTile - 1) / kHeadVocabTile;
  a.inv_t = 1.0 / (double)temperature;
  a.row_stats = row_stats;
  a.root_stats = ws.root_stats;
  a.row_lse = row_lse;
  a.root_lse = ws.root_lse;
  a.root_logits = root_logits;
  a.logits = logits;
  a.q = q;
  a.cand_tok = cand_tok;
  a.cand_len = cand_len;
  a.gate = gate;
  a.u_acc = u_acc;
  a.code = multi ? nullptr : ws.code;
  a.pv = multi ? ws.pv : nullptr;
  if (greedy) {
    a.q = nullptr;                 // draft probabilities play no part
    a.greedy = 1;
    a.am_stats = am_stats;
    a.amax = ws.amax;
    a.amax_tie = ws.amax_tie;
  }
  hipLaunchKernelGGL(lse_tests_kernel, dim3(B * W * D + B), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_sampler(int B, int W, int D, int V, float temperature, const float *root_logits,
                          const float *logits, const double *row_lse, const float *q,
                          const int32_t *cand_tok, const int32_t *cand_len, const double *u_res,
                          const int32_t *gate, int32_t *n_acc, int32_t *best, int32_t *out_tok,
                          int32_t *n_out, int32_t *acc_per_cand, int32_t *flags,
                          int flags_accumulate, const SampleWs &ws, hipStream_t st,
                          int32_t *attn_flags, int rule, const double *u_acc) {
  const bool multi = rule == 1;
  SampArgs a;
  a.B = B;
  a.W = W;
  a.D = D;
  a.V = V;
  a.nch = (V + kChunk - 1) / kChunk;
  a.inv_t = 1.0 / (double)temperature;
  a.root_logits = root_logits;
  a.logits = logits;
  a.row_lse = row_lse;
  a.root_lse = ws.root_lse;
  a.q = q;
  a.cand_tok = cand_tok;
  a.cand_len = cand_len;
  a.u_res = u_res;
  a.gate = gate;
  a.code = ws.code;
  a.pv = ws.pv;
  a.u_acc = u_acc;
  a.amax = ws.amax;
  a.amax_tie = ws.amax_tie;
  a.n_acc = n_acc;
  a.best = best;
  a.out_tok = out_tok;
  a.n_out = n_out;
  a.acc_per_cand = acc_per_cand;
  a.flags = flags;
  a.flags_accumulate = flags_accumulate;
  a.attn_flags = attn_flags;
  a.chunk_sums = ws.chunk_sums;
  a.counters = ws.counters;
  // fused while the workgroups number about one per CU or fewer (measured: B = 1 at
  // V = 128256 is faster fused, B = 32 far faster in two launches)
  bool two = (int64_t)a.nch * B > 256;
  if (const char *ov = getenv("VSTEP_SAMPLER_TWO_PASS")) two = atoi(ov) != 0;
  if (rule == 2) {
    // greedy: no vocabulary sweep, one workgroup per sequence
    hipLaunchKernelGGL((sampler_kernel<SAMP_DRAW, RULE_GREEDY>), dim3(1, B), dim3(kST), 0, st, a);
    return hipGetLastError();
  }
  if (multi && q != nullptr) {
    // dense drafts: the residual chain over the whole vocabulary, G workgroups per
    // sequence (a cooperative launch when G > 1)
    DenseArgs d{};
    d.B = B;
    d.W = W;
    d.D = D;
    d.V = V;
    d.inv_t = a.inv_t;
    d.root_logits = root_logits;
    d.logits = logits;
    d.q = q;
    d.row_lse = row_lse;
    d.root_lse = ws.root_lse;
    d.pv = ws.pv;
    d.cand_tok = cand_tok;
    d.cand_len = cand_len;
    d.gate = gate;
    d.u_acc = u_acc;
    d.u_res = u_res;
    d.resid = ws.resid;
    d.part = ws.dpart;
    d.bar = ws.counters;
    d.n_acc = n_acc;
    d.best = best;
    d.out_tok = out_tok;
    d.n_out = n_out;
    d.acc_per_cand = acc_per_cand;
    d.flags = flags;
    d.flags_accumulate = flags_accumulate;
    d.attn_flags = attn_flags;
    d.G = dense_width(B, (V + kCChunk - 1) / kCChunk);
    if (d.G == 1) {
      hipLaunchKernelGGL(multi_dense_kernel, dim3(1, B), dim3(kCT), 0, st, d);
      return hipGetLastError();
    }
    void *args[] = {&d};
    if (hipLaunchCooperativeKernel((const void *)multi_dense_kernel, dim3(d.G, B), dim3(kCT), args,
                                   0, st) == hipSuccess)
      return hipSuccess;
    // refused (the grid would not be resident at once): one workgroup per sequence
    (void)hipGetLastError();
    d.G = 1;
    hipLaunchKernelGGL(multi_dense_kernel, dim3(1, B), dim3(kCT), 0, st, d);
    return hipGetLastError();
  }
  if (multi) {
    const size_t lds = (size_t)multi_lds_doubles(W, D) * sizeof(double);
    if (!two) {
      hipLaunchKernelGGL((sampler_kernel<SAMP_FUSED, RULE_MULTI>), dim3(a.nch, B), dim3(kST), lds, st, a);
      return hipGetLastError();
    }
    hipLaunchKernelGGL((sampler_kernel<SAMP_SUMS, RULE_MULTI>), dim3(a.nch, B), dim3(kST), lds, st, a);
    if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
    hipLaunchKernelGGL((sampler_kernel<SAMP_DRAW, RULE_MULTI>), dim3(1, B), dim3(kST), lds, st, a);
    return hipGetLastError();
  }
  if (!two) {
    hipLaunchKernelGGL((sampler_kernel<SAMP_FUSED, RULE_LONGEST>), dim3(a.nch, B), dim3(kST), 0, st, a);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((sampler_kernel<SAMP_SUMS, RULE_LONGEST>), dim3(a.nch, B), dim3(kST), 0, st, a);
  if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  hipLaunchKernelGGL((sampler_kernel<SAMP_DRAW, RULE_LONGEST>), dim3(1, B), dim3(kST), 0, st, a);
  return hipGetLastError();
}

}  // namespace vs
