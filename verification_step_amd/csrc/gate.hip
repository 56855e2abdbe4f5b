// Copy-candidate retrieval and probe gate.
//
// Retrieval follows the SwitchSD summary (onedev.kr/papers/87), "무엇과 다른가": the
// kappa-gram ending at the current token is looked up among earlier positions of the
// context; up to W occurrences, most recent first, each continued for D tokens.
// The probe is that page's bias-free linear probe sigma(w.h) ("어떻게 동작하나"), and
// the copy path opens only when the probe reaches tau AND an occurrence exists.
//
// One workgroup (1024 threads) per sequence.  The context is staged into LDS a
// segment at a time, from the end backwards, so the usual case -- an occurrence
// near the current token -- touches one segment.  Every end position j of the
// segment gets a polynomial hash of its kappa-window (wrapping 32-bit arithmetic),
// compared with the key's hash; hash hits are confirmed by comparing the kappa
// ids, so the result is exact.  Wave ballots turn the per-position match bits into
// ranks in descending-j order; the first W ranks are the candidates.

#include "vs_internal.hpp"

namespace vs {

namespace {

constexpr int kGateThreads = 1024;
constexpr int kSeg = 8192;        // context tokens staged per LDS segment
constexpr int kMaxKappa = 16;
constexpr uint32_t kHashMul = 0x9E3779B1u;

struct GateShared {
  int32_t tok[kSeg + kMaxKappa];
  int32_t wave_cnt[kGateThreads / kWave];
  int32_t found;
  float red[kGateThreads / kWave];
};

// Retrieval for sequence b; returns n_found (uniform over the workgroup).  The first
// segment staged is the top of the context including the current token t, so the
// key and (nearly always) the continuations are read from LDS, not global memory.
__device__ int copy_match_wg(GateShared &sh, const int32_t *ctx, int64_t ctx_total,
                             const int32_t *ctx_off, int b, int kappa, int W, int D,
                             int32_t *cand_tok, int32_t *cand_len, int32_t *cand_pos,
                             int *flag_out) {
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wv = tid / kWave;
  const int64_t lo = ctx_off[b];
  const int64_t hi = ctx_off[b + 1];
  const bool bad = !(lo >= 0 && lo <= hi && hi <= ctx_total);
  const int64_t L = bad ? 0 : hi - lo;
  const int64_t t = L - 1;
  const int32_t *c = ctx + (bad ? 0 : lo);
  if (tid == 0) sh.found = 0;

  if (L >= kappa + 1) {
    // end positions j run from t-1 down to kappa-1, a segment of kSeg at a time; the
    // segment [seg_lo, seg_hi] stages tokens base = seg_lo-kappa+1 .. top, where top
    // is t for the first segment (key and continuations) and seg_hi afterwards
    int32_t key[kMaxKappa];
    uint32_t key_hash = 0;
    int64_t seg_hi = t - 1;
    bool first = true;
    while (seg_hi >= kappa - 1) {
      const int64_t seg_lo = max((int64_t)(kappa - 1), seg_hi - kSeg + 1);
      const int n = (int)(seg_hi - seg_lo + 1);
      const int64_t base = seg_lo - kappa + 1;
      const int64_t top = first ? t : seg_hi;
      const int ns = (int)(top - base + 1);
      __syncthreads();          // the previous segment's readers are done
      for (int k = tid; k < ns; k += kGateThreads) sh.tok[k] = c[base + k];
      __syncthreads();
      if (first) {
#pragma unroll
        for (int m = 0; m < kMaxKappa; ++m) {
          key[m] = (m < kappa) ? sh.tok[(int)(t - kappa + 1 + m - base)] : 0;
          if (m < kappa) key_hash = key_hash * kHashMul + (uint32_t)key[m];
        }
      }
      // scan the segment from its top in steps of 1024 positions
      for (int s0 = 0; s0 < n; s0 += kGateThreads) {
        const int r = s0 + tid;                 // rank of the position inside the segment
        bool match = false;
        int64_t j = seg_hi - r;
        if (r < n) {
          const int e = (int)(j - base);        // index of token j in tok[]
          uint32_t hsh = 0;
          for (int m = 0; m < kappa; ++m) hsh = hsh * kHashMul + (uint32_t)sh.tok[e - kappa + 1 + m];
          if (hsh == key_hash) {
            match = true;
            for (int m = 0; m < kappa; ++m) match &= (sh.tok[e - kappa + 1 + m] == key[m]);
          }
        }
        const uint64_t bal = __ballot(match);
        if (lane == 0) sh.wave_cnt[wv] = __popcll(bal);
        __syncthreads();
        int before = sh.found;
        for (int w2 = 0; w2 < wv; ++w2) before += sh.wave_cnt[w2];
        const int rank = before + __popcll(bal & ((1ull << lane) - 1ull));
        if (match && rank < W) {
          const int ln = (int)min((int64_t)D, t - j);
          cand_pos[(int64_t)b * W + rank] = (int32_t)j;
          cand_len[(int64_t)b * W + rank] = ln;
          int32_t *dst = cand_tok + ((int64_t)b * W + rank) * D;
          for (int o = 0; o < D; ++o) {
            const int64_t pos = j + 1 + o;
            dst[o] = (o >= ln) ? -1 : (pos <= top ? sh.tok[(int)(pos - base)] : c[pos]);
          }
        }
        __syncthreads();
        if (tid == 0) {
          int tot = 0;
          for (int w2 = 0; w2 < kGateThreads / kWave; ++w2) tot += sh.wave_cnt[w2];
          sh.found = min(W, sh.found + tot);
        }
        __syncthreads();
        if (sh.found >= W) break;
      }
      if (sh.found >= W) break;
      seg_hi = seg_lo - 1;
      first = false;
    }
  }
  __syncthreads();
  const int nf = sh.found;
  // missing candidates
  for (int k = tid; k < (W - nf) * D; k += kGateThreads) {
    const int i = nf + k / D;
    cand_tok[((int64_t)b * W + i) * D + k % D] = -1;
  }
  for (int i = nf + tid; i < W; i += kGateThreads) {
    cand_len[(int64_t)b * W + i] = 0;
    cand_pos[(int64_t)b * W + i] = -1;
  }
  *flag_out = bad ? FLAG_BAD_CTX : 0;
  return nf;
}

// this thread's share of w . h.  The first kProbeRegs products' operands are loaded
// into registers before the retrieval and multiplied after it, so that their latency
// overlaps the retrieval; any remainder (d > kProbeRegs * threads) is read after.
constexpr int kProbeRegs = 8;
struct ProbeRegs {
  float w[kProbeRegs];
  uint32_t h[kProbeRegs];   // raw bits (bf16 in the low half, or fp32), decoded at use
};
__device__ __forceinline__ ProbeRegs probe_load(const void *h, int h_bf16, const float *w, int b,
                                                int d) {
  // branch-free: out-of-range slots read element d-1 and get weight 0, so every load
  // is issued before the first use (no wait between them)
  ProbeRegs r;
  const int tid = threadIdx.x;
  int kk[kProbeRegs];
#pragma unroll
  for (int i = 0; i < kProbeRegs; ++i) kk[i] = min(tid + i * kGateThreads, d - 1);
  if (h_bf16) {
    const bf16_t *hb = (const bf16_t *)h + (int64_t)b * d;
#pragma unroll
    for (int i = 0; i < kProbeRegs; ++i) r.h[i] = hb[kk[i]];
  } else {
    const float *hf = (const float *)h + (int64_t)b * d;
#pragma unroll
    for (int i = 0; i < kProbeRegs; ++i) r.h[i] = __float_as_uint(hf[kk[i]]);
  }
#pragma unroll
  for (int i = 0; i < kProbeRegs; ++i) r.w[i] = (tid + i * kGateThreads < d) ? w[kk[i]] : 0.f;
  return r;
}
__device__ float probe_partial(const ProbeRegs &r, const void *h, int h_bf16, const float *w,
                               int b, int d) {
  const int tid = threadIdx.x;
  float acc = 0.f;
#pragma unroll
  for (int i = 0; i < kProbeRegs; ++i)
    acc = fmaf(r.w[i], h_bf16 ? __uint_as_float(r.h[i] << 16) : __uint_as_float(r.h[i]), acc);
  for (int k = tid + kProbeRegs * kGateThreads; k < d; k += kGateThreads)
    acc = fmaf(w[k], h_bf16 ? bf16_to_f32(((const bf16_t *)h)[(int64_t)b * d + k])
                            : ((const float *)h)[(int64_t)b * d + k], acc);
  return acc;
}

// workgroup sum of the partials in a fixed tree order (every thread gets the total)
__device__ float probe_reduce(GateShared &sh, float acc) {
  const int tid = threadIdx.x;
  for (int off = kWave / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  __syncthreads();
  if ((tid & (kWave - 1)) == 0) sh.red[tid / kWave] = acc;
  __syncthreads();
  float x = 0.f;
  for (int w2 = 0; w2 < kGateThreads / kWave; ++w2) x += sh.red[w2];
  return x;
}

__global__ void __launch_bounds__(kGateThreads)
gate_kernel(const int32_t *ctx, int64_t ctx_total, const int32_t *ctx_off, int kappa, int W,
            int D, int32_t *cand_tok, int32_t *cand_len, int32_t *cand_pos, int32_t *n_found,
            int32_t *flags, const void *h, int h_bf16, const float *w, int d, float tau,
            float *score, int32_t *gate) {
  __shared__ GateShared sh;
  const int b = blockIdx.x;
  int fl = 0;
  ProbeRegs pr{};
  if (h != nullptr) pr = probe_load(h, h_bf16, w, b, d);
  const int nf = copy_match_wg(sh, ctx, ctx_total, ctx_off, b, kappa, W, D, cand_tok, cand_len,
                               cand_pos, &fl);
  float s = 0.f;
  int g = 0;
  if (h != nullptr) {
    const float x = probe_reduce(sh, probe_partial(pr, h, h_bf16, w, b, d));
    const double sd = 1.0 / (1.0 + exp(-(double)x));
    s = (float)sd;
    g = (sd >= (double)tau) && (nf >= 1);
    if (fabs(sd - (double)tau) < 1e-5) fl |= FLAG_PROBE_TIE;
  }
  if (threadIdx.x == 0) {
    n_found[b] = nf;
    if (flags) flags[b] = fl;
    if (h != nullptr) {
      score[b] = s;
      gate[b] = g;
    }
  }
}

__global__ void __launch_bounds__(kGateThreads)
probe_kernel(const void *h, int h_bf16, const float *w, int d, float tau, const int32_t *n_found,
             float *score, int32_t *gate, int32_t *flags) {
  __shared__ GateShared sh;
  const int b = blockIdx.x;
  const float x = probe_reduce(sh, probe_partial(probe_load(h, h_bf16, w, b, d), h, h_bf16, w, b, d));
  if (threadIdx.x == 0) {
    const double sd = 1.0 / (1.0 + exp(-(double)x));
    score[b] = (float)sd;
    gate[b] = (sd >= (double)tau) && (n_found == nullptr || n_found[b] >= 1);
    if (flags) flags[b] = (fabs(sd - (double)tau) < 1e-5) ? FLAG_PROBE_TIE : 0;
  }
}

}  // namespace

hipError_t launch_copy_match(const int32_t *ctx, int64_t ctx_total, const int32_t *ctx_off, int B,
                             int kappa, int W, int D, int32_t *cand_tok, int32_t *cand_len,
                             int32_t *cand_pos, int32_t *n_found, int32_t *flags, const void *h,
                             int h_bf16, const float *w, int d, float tau, float *score,
                             int32_t *gate, hipStream_t st) {
  hipLaunchKernelGGL(gate_kernel, dim3(B), dim3(kGateThreads), 0, st, ctx, ctx_total, ctx_off,
                     kappa, W, D, cand_tok, cand_len, cand_pos, n_found, flags, h, h_bf16, w, d,
                     tau, score, gate);
  return hipGetLastError();
}

hipError_t launch_probe_gate(const void *h, int h_bf16, const float *w, int B, int d, float tau,
                             const int32_t *n_found, float *score, int32_t *gate, int32_t *flags,
                             hipStream_t st) {
  hipLaunchKernelGGL(probe_kernel, dim3(B), dim3(kGateThreads), 0, st, h, h_bf16, w, d, tau,
                     n_found, score, gate, flags);
  return hipGetLastError();
}

}  // namespace vs
