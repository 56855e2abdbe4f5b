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
// All sampler arithmetic is fp64: p = exp(z/T - lse) from fp32 logits and the head's
// fp64 normaliser, the acceptance comparison, and the inverse-CDF draw over
// ascending token ids.  One workgroup of 1024 threads per sequence: every thread
// owns a contiguous slice of the vocabulary for the normaliser and the residual
// sums; slice sums are prefix-summed in a fixed order, the slice holding u*S is
// re-expanded in LDS and scanned to find the token.

#include "vs_internal.hpp"

namespace vs {

namespace {

constexpr int kST = 1024;
constexpr int kMaxSlice = 512;   // vocabulary slice per thread: V <= kST * kMaxSlice

struct SampShared {
  double red[kST];
  double slice_val[kMaxSlice];
  int a_len[1024];
  int lens[1024];
  unsigned char tie[1024];
  int flags;
  int best, ab, mode, xpt, owner;
  int64_t prow;      // -1: root row
  int64_t qrow;      // -1: no dense q row
  double lse, u, S, excl;
};

enum { MODE_ROOT = 0, MODE_RESID = 1, MODE_BONUS = 2 };

// fixed-order block reduction (sum or max) over kST doubles
template <bool MAX>
__device__ double block_reduce(SampShared &sh, double v) {
  sh.red[threadIdx.x] = v;
  __syncthreads();
  for (int off = kST / 2; off > 0; off >>= 1) {
    if ((int)threadIdx.x < off) {
      const double o = sh.red[threadIdx.x + off];
      sh.red[threadIdx.x] = MAX ? fmax(sh.red[threadIdx.x], o) : sh.red[threadIdx.x] + o;
    }
    __syncthreads();
  }
  const double r = sh.red[0];
  __syncthreads();
  return r;
}

__global__ void __launch_bounds__(kST)
sampler_kernel(int W, int D, int V, double inv_t, const float *root_logits, const float *logits,
               const double *row_lse, const float *q, const int32_t *cand_tok,
               const int32_t *cand_len, const double *u_acc, const double *u_res,
               const int32_t *gate, int32_t *n_acc, int32_t *best_out, int32_t *out_tok,
               int32_t *n_out, int32_t *acc_per_cand, int32_t *flags, int flags_accumulate) {
  __shared__ SampShared sh;
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int M = W * D;
  const float *root = root_logits + (int64_t)b * V;
  const int slice = (V + kST - 1) / kST;
  const int k0 = min(V, tid * slice), k1 = min(V, k0 + slice);

  // ---- normaliser of the root distribution
  double mx = -INFINITY;
  for (int k = k0; k < k1; ++k) mx = fmax(mx, (double)root[k] * inv_t);
  const double M0 = block_reduce<true>(sh, mx);
  double s = 0.0;
  for (int k = k0; k < k1; ++k) s += exp((double)root[k] * inv_t - M0);
  const double lse_root = M0 + log(block_reduce<false>(sh, s));

  // ---- acceptance tests
  const bool open = (gate == nullptr) || gate[b] != 0;
  if (tid == 0) sh.flags = 0;
  for (int i = tid; i < W; i += kST) {
    int ln = open ? cand_len[(int64_t)b * W + i] : 0;
    ln = ln < 0 ? 0 : (ln > D ? D : ln);
    sh.lens[i] = ln;
    sh.a_len[i] = ln;
  }
  __syncthreads();
  for (int idx = tid; idx < M; idx += kST) {
    const int i = idx / D, o = idx % D;
    sh.tie[idx] = 0;
    if (o >= sh.lens[i]) continue;
    const int x = cand_tok[((int64_t)b * W + i) * D + o];
    double p = 0.0, Q = 1.0;
    if (x >= 0 && x < V) {
      double z, l;
      if (o == 0) {
        z = (double)root[x];
        l = lse_root;
      } else {
        const int64_t r = (int64_t)b * M + i * D + o - 1;
        z = (double)logits[r * V + x];
        l = row_lse[r];
      }
      p = exp(z * inv_t - l);
      if (q) Q = (double)q[((int64_t)b * M + idx) * V + x];
    } else {
      atomicOr(&sh.flags, FLAG_BAD_TOKEN);
    }
    const double lhs = u_acc[((int64_t)b * W + i) * D + o] * Q;
    if (fabs(lhs - p) < 1e-4 * fmax(p, lhs)) sh.tie[idx] = 1;
    if (!(lhs < p)) atomicMin(&sh.a_len[i], o);
  }
  __syncthreads();
  for (int idx = tid; idx < M; idx += kST) {
    const int i = idx / D, o = idx % D;
    if (o < sh.lens[i] && o <= sh.a_len[i] && sh.tie[idx]) atomicOr(&sh.flags, FLAG_ACCEPT_TIE);
  }
  __syncthreads();

  // ---- choose the candidate and the distribution of the extra token
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
      sh.u = u_res[(int64_t)b * W];
      sh.flags |= FLAG_NO_CANDIDATE;
    } else {
      const int ab = sh.a_len[best];
      sh.ab = ab;
      sh.u = u_res[(int64_t)b * W + best];
      sh.prow = (ab == 0) ? -1 : (int64_t)b * M + best * D + ab - 1;
      if (ab < sh.lens[best]) {
        sh.mode = MODE_RESID;
        if (q) sh.qrow = (int64_t)b * M + best * D + ab;
        else sh.xpt = cand_tok[((int64_t)b * W + best) * D + ab];
      } else {
        sh.mode = MODE_BONUS;
      }
    }
    sh.lse = (sh.prow < 0) ? lse_root : row_lse[sh.prow];
  }
  __syncthreads();
  const float *zrow = (sh.prow < 0) ? root : logits + sh.prow * V;
  const double lse = sh.lse;
  const float *qrow = (sh.qrow < 0) ? nullptr : q + sh.qrow * V;
  const int xpt = sh.xpt;
  bool resid = sh.mode == MODE_RESID;

  auto weight = [&](int k) -> double {
    const double pk = exp((double)zrow[k] * inv_t - lse);
    if (!resid) return pk;
    const double qk = qrow ? (double)qrow[k] : (k == xpt ? 1.0 : 0.0);
    return fmax(0.0, pk - qk);
  };

  double part = 0.0;
  for (int k = k0; k < k1; ++k) part += weight(k);
  double S = block_reduce<false>(sh, part);
  if (!(S > 0.0)) {
    resid = false;
    if (tid == 0) sh.flags |= FLAG_DEGENERATE;
    part = 0.0;
    for (int k = k0; k < k1; ++k) part += weight(k);
    S = block_reduce<false>(sh, part);
  }
  // slice sums in order -> owner slice of u*S
  sh.red[tid] = part;
  __syncthreads();
  const double xs = sh.u * S;
  if (tid == 0) {
    double run = 0.0;
    int owner = kST - 1;
    double excl = 0.0;
    for (int t = 0; t < kST; ++t) {
      const double nxt = run + sh.red[t];
      if (nxt > xs && sh.red[t] > 0.0) {
        owner = t;
        excl = run;
        break;
      }
      run = nxt;
      excl = run;
    }
    sh.owner = owner;
    sh.excl = excl;
    sh.S = S;
  }
  __syncthreads();
  {
    const int ok0 = min(V, sh.owner * slice), ok1 = min(V, ok0 + slice);
    for (int k = ok0 + tid; k < ok1; k += kST) sh.slice_val[k - ok0] = weight(k);
  }
  __syncthreads();
  if (tid == 0) {
    const int ok0 = min(V, sh.owner * slice), ok1 = min(V, ok0 + slice);
    double run = sh.excl, prev = sh.excl;
    int y = V - 1;
    bool found = false;
    for (int k = ok0; k < ok1; ++k) {
      prev = run;
      run += sh.slice_val[k - ok0];
      if (run > xs) {
        y = k;
        found = true;
        break;
      }
    }
    if (!found) prev = run;
    const double hi = found ? run : prev;
    const double lo = found ? prev : prev;
    int fl = sh.flags;
    if (fabs(xs - lo) < 1e-8 * S || fabs(hi - xs) < 1e-8 * S) fl |= FLAG_CDF_TIE;
    const int best = sh.best, ab = sh.ab;
    int32_t *ot = out_tok + (int64_t)b * (D + 1);
    for (int o = 0; o < ab; ++o) ot[o] = cand_tok[((int64_t)b * W + best) * D + o];
    ot[ab] = y;
    for (int o = ab + 1; o <= D; ++o) ot[o] = -1;
    n_acc[b] = ab;
    best_out[b] = best;
    n_out[b] = ab + 1;
    if (flags) {
      if (flags_accumulate) atomicOr(&flags[b], fl);
      else flags[b] = fl;
    }
  }
  for (int i = tid; i < W; i += kST)
    acc_per_cand[(int64_t)b * W + i] = (sh.lens[i] >= 1) ? sh.a_len[i] : 0;
}

}  // namespace

size_t sample_workspace_bytes(int B, int W, int D, int V) {
  (void)B;
  (void)W;
  (void)D;
  (void)V;
  return 0;
}

hipError_t launch_sampler(int B, int W, int D, int V, float temperature, const float *root_logits,
                          const float *logits, const double *row_lse, const float *q,
                          const int32_t *cand_tok, const int32_t *cand_len, const double *u_acc,
                          const double *u_res, const int32_t *gate, int32_t *n_acc, int32_t *best,
                          int32_t *out_tok, int32_t *n_out, int32_t *acc_per_cand,
                          int32_t *flags, int flags_accumulate, void *ws, hipStream_t st) {
  (void)ws;
  hipLaunchKernelGGL(sampler_kernel, dim3(B), dim3(kST), 0, st, W, D, V,
                     1.0 / (double)temperature, root_logits, logits, row_lse, q, cand_tok,
                     cand_len, u_acc, u_res, gate, n_acc, best, out_tok, n_out, acc_per_cand,
                     flags, flags_accumulate);
  return hipGetLastError();
}

}  // namespace vs
