// Copy-candidate retrieval and probe gate of one sequence, as the work of one
// workgroup of NT threads (NT a multiple of 64).  Used by the standalone launch
// (1024 threads) and by the verify attention launch, whose first workgroups run it
// beside the attention workgroups.
//
// Retrieval follows the SwitchSD summary (onedev.kr/papers/87), "무엇과 다른가": the
// kappa-gram ending at the current token is looked up among earlier positions of the
// context; up to W occurrences, most recent first, each continued for D tokens.
// The probe is that page's bias-free linear probe sigma(w.h) ("어떻게 동작하나"), and
// the copy path opens only when the probe reaches tau AND an occurrence exists.
//
// One workgroup per sequence.  The context is staged into LDS a
// segment at a time, from the end backwards, so the usual case -- an occurrence
// near the current token -- touches one segment.  Every end position j of the
// segment gets a polynomial hash of its kappa-window (wrapping 32-bit arithmetic),
// compared with the key's hash; hash hits are confirmed by comparing the kappa
// ids, so the result is exact.  Wave ballots turn the per-position match bits into
// ranks in descending-j order; the first W ranks are the candidates.

#pragma once

#include "vs_internal.hpp"

namespace vs {

constexpr int kMaxKappa = 16;
constexpr uint32_t kHashMul = 0x9E3779B1u;

template <int NT>
struct GateShared {
  static constexpr int kSeg = 8 * NT;        // context tokens staged per LDS segment
  int32_t tok[kSeg + kMaxKappa];
  int32_t wave_cnt[NT / kWave];
  int32_t found;
  float red[NT / kWave];
};

// Retrieval for sequence b; returns n_found (uniform over the workgroup).  The first
// segment staged is the top of the context including the current token t, so the
// key and (nearly always) the continuations are read from LDS, not global memory.
template <int NT>
__device__ int copy_match_wg(GateShared<NT> &sh, const int32_t *ctx, int64_t ctx_total,
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
    // end positions j run from t-1 down to kappa-1, one LDS segment at a time; the
    // segment [seg_lo, seg_hi] stages tokens base = seg_lo-kappa+1 .. top, where top
    // is t for the first segment (key and continuations) and seg_hi afterwards
    int32_t key[kMaxKappa];
    uint32_t key_hash = 0;
    int64_t seg_hi = t - 1;
    bool first = true;
    while (seg_hi >= kappa - 1) {
      const int64_t seg_lo = max((int64_t)(kappa - 1), seg_hi - GateShared<NT>::kSeg + 1);
      const int n = (int)(seg_hi - seg_lo + 1);
      const int64_t base = seg_lo - kappa + 1;
      const int64_t top = first ? t : seg_hi;
      const int ns = (int)(top - base + 1);
      __syncthreads();          // the previous segment's readers are done
      for (int k = tid; k < ns; k += NT) sh.tok[k] = c[base + k];
      __syncthreads();
      if (first) {
#pragma unroll
        for (int m = 0; m < kMaxKappa; ++m) {
          key[m] = (m < kappa) ? sh.tok[(int)(t - kappa + 1 + m - base)] : 0;
          if (m < kappa) key_hash = key_hash * kHashMul + (uint32_t)key[m];
        }
      }
      // scan the segment from its top in steps of NT positions
      for (int s0 = 0; s0 < n; s0 += NT) {
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
          for (int w2 = 0; w2 < NT / kWave; ++w2) tot += sh.wave_cnt[w2];
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
  for (int k = tid; k < (W - nf) * D; k += NT) {
    const int i = nf + k / D;
    cand_tok[((int64_t)b * W + i) * D + k % D] = -1;
  }
  for (int i = nf + tid; i < W; i += NT) {
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
template <int NT>
__device__ __forceinline__ ProbeRegs probe_load(const void *h, int h_bf16, const float *w, int b,
                                                int d) {
  // branch-free: out-of-range slots read element d-1 and get weight 0, so every load
  // is issued before the first use (no wait between them)
  ProbeRegs r;
  const int tid = threadIdx.x;
  int kk[kProbeRegs];
#pragma unroll
  for (int i = 0; i < kProbeRegs; ++i) kk[i] = min(tid + i * NT, d - 1);
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
  for (int i = 0; i < kProbeRegs; ++i) r.w[i] = (tid + i * NT < d) ? w[kk[i]] : 0.f;
  return r;
}
template <int NT>
__device__ float probe_partial(const ProbeRegs &r, const void *h, int h_bf16, const float *w,
                               int b, int d) {
  const int tid = threadIdx.x;
  float acc = 0.f;
#pragma unroll
  for (int i = 0; i < kProbeRegs; ++i)
    acc = fmaf(r.w[i], h_bf16 ? __uint_as_float(r.h[i] << 16) : __uint_as_float(r.h[i]), acc);
  for (int k = tid + kProbeRegs * NT; k < d; k += NT)
    acc = fmaf(w[k], h_bf16 ? bf16_to_f32(((const bf16_t *)h)[(int64_t)b * d + k])
                            : ((const float *)h)[(int64_t)b * d + k], acc);
  return acc;
}

// workgroup sum of the partials in a fixed tree order (every thread gets the total)
template <int NT>
__device__ float probe_reduce(GateShared<NT> &sh, float acc) {
  const int tid = threadIdx.x;
  for (int off = kWave / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  __syncthreads();
  if ((tid & (kWave - 1)) == 0) sh.red[tid / kWave] = acc;
  __syncthreads();
  float x = 0.f;
  for (int w2 = 0; w2 < NT / kWave; ++w2) x += sh.red[w2];
  return x;
}

// the whole gate of sequence b: retrieval, probe, outputs
template <int NT>
__device__ void gate_wg(const GateArgs &g, int b, GateShared<NT> &sh) {
  int fl = 0;
  ProbeRegs pr{};
  if (g.h != nullptr) pr = probe_load<NT>(g.h, g.h_bf16, g.w, b, g.d);
  const int nf = copy_match_wg<NT>(sh, g.ctx, g.ctx_total, g.ctx_off, b, g.kappa, g.W, g.D,
                                   g.cand_tok, g.cand_len, g.cand_pos, &fl);
  float s = 0.f;
  int gt = 0;
  if (g.h != nullptr) {
    const float x = probe_reduce<NT>(sh, probe_partial<NT>(pr, g.h, g.h_bf16, g.w, b, g.d));
    const double sd = 1.0 / (1.0 + exp(-(double)x));
    s = (float)sd;
    gt = (sd >= (double)g.tau) && (nf >= 1);
    if (fabs(sd - (double)g.tau) < 1e-5) fl |= FLAG_PROBE_TIE;
  }
  if (threadIdx.x == 0) {
    g.n_found[b] = nf;
    if (g.flags) g.flags[b] = fl;
    if (g.h != nullptr) {
      g.score[b] = s;
      g.gate[b] = gt;
    }
  }
}

}  // namespace vs
