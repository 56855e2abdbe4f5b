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
// Layout of the work: grid (vocabulary chunks, sequences).  Every workgroup of a
// sequence repeats the (cheap) acceptance tests and the choice of candidate, then
// sums the residual weights of its own vocabulary chunk with coalesced loads.  The
// last workgroup of the sequence to finish (atomic counter in the workspace) adds
// the chunk sums in chunk order, finds the chunk holding u*S, rescans that chunk
// with an ordered block scan and writes the outputs; it then resets the counter.

#include "vs_internal.hpp"

#include <limits.h>

namespace vs {

namespace {

constexpr int kST = 256;              // threads per workgroup
constexpr int kPer = 8;               // vocabulary entries per thread per chunk
constexpr int kChunk = kST * kPer;    // 2048
constexpr int kMaxRows = 1024;

struct SampShared {
  int a_len[kMaxRows];
  int lens[kMaxRows];
  unsigned char tie[kMaxRows];
  double red[kST / 64];
  double red2[kST / 64];
  double scan[kST];
  int flags;
  int best, ab, mode, xpt, is_last, owner, y;
  int64_t prow, qrow;
  double lse, u, S, excl, lo, hi;
};

enum { MODE_ROOT = 0, MODE_RESID = 1, MODE_BONUS = 2, MODE_TARGET = 3 };

__device__ __forceinline__ double warp_sum(double v) {
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

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
  double ra = 0.0, rb = 0.0;
  for (int w = 0; w < kST / 64; ++w) {
    ra += sh.red[w];
    rb += sh.red2[w];
  }
  __syncthreads();
  a = ra;
  b = rb;
}

struct SampArgs {
  int B, W, D, V, nch;
  double inv_t;
  const float *root_logits, *logits;
  const double *row_lse, *root_lse;
  const float *q;
  const int32_t *cand_tok, *cand_len;
  const double *u_acc, *u_res;
  const int32_t *gate;
  int32_t *n_acc, *best, *out_tok, *n_out, *acc_per_cand, *flags;
  int flags_accumulate;
  double2 *chunk_sums;   // [B][nch]: (residual-or-bonus weight sum, target p sum)
  uint32_t *counters;    // [B]
};

__global__ void __launch_bounds__(kST)
sampler_kernel(SampArgs a) {
  __shared__ SampShared sh;
  const int c = blockIdx.x;
  const int b = blockIdx.y;
  const int tid = threadIdx.x;
  const int W = a.W, D = a.D, V = a.V, M = W * D;
  const float *root = a.root_logits + (int64_t)b * V;
  const double lse_root = a.root_lse[b];

  // ---- acceptance tests (repeated by every chunk workgroup of the sequence)
  const bool open = (a.gate == nullptr) || a.gate[b] != 0;
  if (tid == 0) sh.flags = 0;
  for (int i = tid; i < W; i += kST) {
    int ln = open ? a.cand_len[(int64_t)b * W + i] : 0;
    ln = ln < 0 ? 0 : (ln > D ? D : ln);
    sh.lens[i] = ln;
    sh.a_len[i] = ln;
  }
  __syncthreads();
  for (int idx = tid; idx < M; idx += kST) {
    const int i = idx / D, o = idx % D;
    sh.tie[idx] = 0;
    if (o >= sh.lens[i]) continue;
    const int x = a.cand_tok[((int64_t)b * W + i) * D + o];
    double p = 0.0, Q = 1.0;
    if (x >= 0 && x < V) {
      double z, l;
      if (o == 0) {
        z = (double)root[x];
        l = lse_root;
      } else {
        const int64_t r = (int64_t)b * M + i * D + o - 1;
        z = (double)a.logits[r * V + x];
        l = a.row_lse[r];
      }
      p = exp(z * a.inv_t - l);
      if (a.q) Q = (double)a.q[((int64_t)b * M + idx) * V + x];
    } else {
      atomicOr(&sh.flags, FLAG_BAD_TOKEN);
    }
    const double lhs = a.u_acc[((int64_t)b * W + i) * D + o] * Q;
    if (fabs(lhs - p) < 1e-4 * fmax(p, lhs)) sh.tie[idx] = 1;
    if (!(lhs < p)) atomicMin(&sh.a_len[i], o);
  }
  __syncthreads();
  for (int idx = tid; idx < M; idx += kST) {
    const int i = idx / D, o = idx % D;
    if (o < sh.lens[i] && o <= sh.a_len[i] && sh.tie[idx]) atomicOr(&sh.flags, FLAG_ACCEPT_TIE);
  }
  __syncthreads();

  // ---- the chosen candidate and the distribution of the extra token
  if (tid == 0) {
    int best = -1;
    for (int i = 0; i < W; ++i)
      if (sh.lens[i] >= 1 && (best < 0 || sh.a_len[i] > sh.a_len[best])) best = i;
    sh.best = best;
    sh.qrow = -1;
    sh.xpt = -1;
    if (best < 0) {
      sh.ab = 0;
      sh.mode = MODE_ROOT;
      sh.prow = -1;
      sh.u = a.u_res[(int64_t)b * W];
      sh.flags |= FLAG_NO_CANDIDATE;
    } else {
      const int ab = sh.a_len[best];
      sh.ab = ab;
      sh.u = a.u_res[(int64_t)b * W + best];
      sh.prow = (ab == 0) ? -1 : (int64_t)b * M + best * D + ab - 1;
      if (ab < sh.lens[best]) {
        sh.mode = MODE_RESID;
        if (a.q) sh.qrow = (int64_t)b * M + best * D + ab;
        else sh.xpt = a.cand_tok[((int64_t)b * W + best) * D + ab];
      } else {
        sh.mode = MODE_BONUS;
      }
    }
    sh.lse = (sh.prow < 0) ? lse_root : a.row_lse[sh.prow];
  }
  __syncthreads();
  const float *zrow = (sh.prow < 0) ? root : a.logits + sh.prow * V;
  const double lse = sh.lse;
  const float *qrow = (sh.qrow < 0) ? nullptr : a.q + sh.qrow * V;
  const int xpt = sh.xpt;
  const bool resid = sh.mode == MODE_RESID;

  // target probability and residual weight of token k
  auto weights = [&](int k, double &pk, double &rk) {
    pk = exp((double)zrow[k] * a.inv_t - lse);
    if (resid) {
      const double qk = qrow ? (double)qrow[k] : (k == xpt ? 1.0 : 0.0);
      rk = fmax(0.0, pk - qk);
    } else {
      rk = pk;
    }
  };

  // ---- this chunk's sums (coalesced: entry c*kChunk + j*kST + tid)
  double sr = 0.0, sp = 0.0;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int k = c * kChunk + j * kST + tid;
    if (k < V) {
      double pk, rk;
      weights(k, pk, rk);
      sr += rk;
      sp += pk;
    }
  }
  block_sum2(sh, sr, sp);
  if (tid == 0) {
    a.chunk_sums[(int64_t)b * a.nch + c] = make_double2(sr, sp);
    __threadfence();
    const uint32_t old = atomicAdd(&a.counters[b], 1u);
    sh.is_last = (old == (uint32_t)(a.nch - 1));
  }
  __syncthreads();
  if (!sh.is_last) return;
  __threadfence();

  // ---- last workgroup of the sequence: total, owner chunk, ordered scan, outputs
  if (tid == 0) {
    const double2 *cs = a.chunk_sums + (int64_t)b * a.nch;
    double S = 0.0;
    for (int k = 0; k < a.nch; ++k) S += cs[k].x;
    bool use_target = false;
    if (!(S > 0.0)) {
      use_target = true;
      sh.flags |= FLAG_DEGENERATE;
      S = 0.0;
      for (int k = 0; k < a.nch; ++k) S += cs[k].y;
    }
    const double xs = sh.u * S;
    double run = 0.0;
    int owner = -1;
    double excl = 0.0;
    for (int k = 0; k < a.nch; ++k) {
      const double v = use_target ? cs[k].y : cs[k].x;
      if (run + v > xs && v > 0.0) {
        owner = k;
        excl = run;
        break;
      }
      run += v;
    }
    if (owner < 0) {
      // u*S at or (by rounding) past the total: the last chunk with weight
      owner = a.nch - 1;
      for (int k = a.nch - 1; k >= 0; --k)
        if ((use_target ? cs[k].y : cs[k].x) > 0.0) {
          owner = k;
          break;
        }
      excl = 0.0;
      for (int k = 0; k < owner; ++k) excl += use_target ? cs[k].y : cs[k].x;
    }
    sh.owner = owner;
    sh.excl = excl;
    sh.S = S;
    if (use_target) sh.mode = MODE_TARGET;
    sh.y = INT_MAX;
    a.counters[b] = 0u;   // ready for the next call on this workspace
  }
  __syncthreads();
  const bool use_p = sh.mode == MODE_TARGET;
  const double S = sh.S;
  const double xs = sh.u * S;
  // ordered scan of the owner chunk: thread t owns entries t*kPer .. t*kPer+kPer-1
  double vals[kPer];
  double tsum = 0.0;
  const int base = sh.owner * kChunk + tid * kPer;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int k = base + j;
    double pk = 0.0, rk = 0.0;
    if (k < V) weights(k, pk, rk);
    vals[j] = use_p ? pk : rk;
    tsum += vals[j];
  }
  // inclusive prefix of thread sums in thread order (Hillis-Steele, fixed order)
  sh.scan[tid] = tsum;
  __syncthreads();
  for (int off = 1; off < kST; off <<= 1) {
    const double add = (tid >= off) ? sh.scan[tid - off] : 0.0;
    __syncthreads();
    sh.scan[tid] += add;
    __syncthreads();
  }
  double run = sh.excl + (sh.scan[tid] - tsum);
  int y = -1;
  double lo = 0.0, hi = 0.0;
  for (int j = 0; j < kPer; ++j) {
    const double prev = run;
    run += vals[j];
    if (y < 0 && vals[j] > 0.0 && run > xs) {
      y = base + j;
      lo = prev;
      hi = run;
    }
  }
  if (y >= 0) atomicMin(&sh.y, y);
  __syncthreads();
  if (y >= 0 && y == sh.y) {
    sh.lo = lo;
    sh.hi = hi;
  }
  __syncthreads();
  if (tid == 0) {
    int yy = sh.y;
    int fl = sh.flags;
    if (yy == INT_MAX) {
      // rounding at the chunk edge left u*S past this chunk's scan: last weighted entry
      yy = min(V, (sh.owner + 1) * kChunk) - 1;
      fl |= FLAG_CDF_TIE;
    } else if (fabs(xs - sh.lo) < 1e-8 * S || fabs(sh.hi - xs) < 1e-8 * S) {
      fl |= FLAG_CDF_TIE;
    }
    const int best = sh.best, ab = sh.ab;
    int32_t *ot = a.out_tok + (int64_t)b * (D + 1);
    for (int o = 0; o < ab; ++o) ot[o] = a.cand_tok[((int64_t)b * W + best) * D + o];
    ot[ab] = yy;
    for (int o = ab + 1; o <= D; ++o) ot[o] = -1;
    a.n_acc[b] = ab;
    a.best[b] = best;
    a.n_out[b] = ab + 1;
    if (a.flags) {
      if (a.flags_accumulate) atomicOr(&a.flags[b], fl);
      else a.flags[b] = fl;
    }
  }
  for (int i = tid; i < W; i += kST)
    a.acc_per_cand[(int64_t)b * W + i] = (sh.lens[i] >= 1) ? sh.a_len[i] : 0;
}

// (max, sum exp(x - max)) of x = logits/T over one vocabulary tile, for B rows;
// stats layout [B][n_vt].
__global__ void __launch_bounds__(256)
root_stats_kernel(const float *root_logits, int B, int V, float inv_t, float2 *stats) {
  const int vt = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int n_vt = (V + kHeadVocabTile - 1) / kHeadVocabTile;
  for (int b = wv; b < B; b += 4) {
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

// Row normalisers lse = max + log(sum_t s_t exp(m_t - max)) in fp64 from tile
// statistics [rows][n_vt].  One workgroup per row.
__global__ void __launch_bounds__(256)
lse_from_stats_kernel(const float2 *stats, int n_vt, double *lse) {
  const int r = blockIdx.x;
  __shared__ double red[4];
  const float2 *st = stats + (int64_t)r * n_vt;
  double mx = -INFINITY;
  for (int t = threadIdx.x; t < n_vt; t += 256) mx = fmax(mx, (double)st[t].x);
  for (int off = 32; off > 0; off >>= 1) mx = fmax(mx, __shfl_xor(mx, off));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = mx;
  __syncthreads();
  mx = fmax(fmax(red[0], red[1]), fmax(red[2], red[3]));
  __syncthreads();
  double s = 0.0;
  for (int t = threadIdx.x; t < n_vt; t += 256) {
    const float2 v = st[t];
    if (v.x != -INFINITY) s += (double)v.y * exp((double)v.x - mx);
  }
  for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = s;
  __syncthreads();
  if (threadIdx.x == 0) lse[r] = mx + log(red[0] + red[1] + red[2] + red[3]);
}

}  // namespace

SampleWs sample_ws(void *ws, int B, int V) {
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
  w.bytes = off;
  return w;
}

size_t sample_workspace_bytes(int B, int W, int D, int V) {
  (void)W;
  (void)D;
  return sample_ws(nullptr, B, V).bytes;
}

hipError_t launch_root_stats(const float *root_logits, int B, int V, float temperature,
                             float2 *stats, hipStream_t st) {
  const int n_vt = (V + kHeadVocabTile - 1) / kHeadVocabTile;
  hipLaunchKernelGGL(root_stats_kernel, dim3(n_vt), dim3(256), 0, st, root_logits, B, V,
                     1.0f / temperature, stats);
  return hipGetLastError();
}

hipError_t launch_lse_from_stats(const float2 *stats, int rows, int V, double *lse,
                                 hipStream_t st) {
  const int n_vt = (V + kHeadVocabTile - 1) / kHeadVocabTile;
  hipLaunchKernelGGL(lse_from_stats_kernel, dim3(rows), dim3(256), 0, st, stats, n_vt, lse);
  return hipGetLastError();
}

hipError_t launch_sampler(int B, int W, int D, int V, float temperature, const float *root_logits,
                          const float *logits, const double *row_lse, const double *root_lse,
                          const float *q, const int32_t *cand_tok, const int32_t *cand_len,
                          const double *u_acc, const double *u_res, const int32_t *gate,
                          int32_t *n_acc, int32_t *best, int32_t *out_tok, int32_t *n_out,
                          int32_t *acc_per_cand, int32_t *flags, int flags_accumulate,
                          const SampleWs &ws, hipStream_t st) {
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
  a.root_lse = root_lse;
  a.q = q;
  a.cand_tok = cand_tok;
  a.cand_len = cand_len;
  a.u_acc = u_acc;
  a.u_res = u_res;
  a.gate = gate;
  a.n_acc = n_acc;
  a.best = best;
  a.out_tok = out_tok;
  a.n_out = n_out;
  a.acc_per_cand = acc_per_cand;
  a.flags = flags;
  a.flags_accumulate = flags_accumulate;
  a.chunk_sums = ws.chunk_sums;
  a.counters = ws.counters;
  hipLaunchKernelGGL(sampler_kernel, dim3(a.nch, B), dim3(kST), 0, st, a);
  return hipGetLastError();
}

}  // namespace vs
