// Copy-candidate retrieval and probe gate: the standalone launches (one 1024-thread
// workgroup per sequence).  The workgroup's work is in gate_wg.hpp.

#include "gate_wg.hpp"

namespace vs {

namespace {

constexpr int kGateThreads = 1024;

__global__ void __launch_bounds__(kGateThreads)
gate_kernel(GateArgs g) {
  __shared__ GateShared<kGateThreads> sh;
  gate_wg<kGateThreads>(g, blockIdx.x, sh);
}

__global__ void __launch_bounds__(kGateThreads)
probe_kernel(const void *h, int h_bf16, const float *w, int d, float tau, const int32_t *n_found,
             float *score, int32_t *gate, int32_t *flags) {
  __shared__ GateShared<kGateThreads> sh;
  const int b = blockIdx.x;
  const float x = probe_reduce<kGateThreads>(
      sh, probe_partial<kGateThreads>(probe_load<kGateThreads>(h, h_bf16, w, b, d), h, h_bf16, w,
                                      b, d));
  if (threadIdx.x == 0) {
    const double sd = 1.0 / (1.0 + exp(-(double)x));
    score[b] = (float)sd;
    gate[b] = (sd >= (double)tau) && (n_found == nullptr || n_found[b] >= 1);
    if (flags) flags[b] = (fabs(sd - (double)tau) < 1e-5) ? FLAG_PROBE_TIE : 0;
  }
}

}  // namespace

GateArgs gate_args(const int32_t *ctx, int64_t ctx_total, const int32_t *ctx_off, int kappa, int W,
                   int D, int32_t *cand_tok, int32_t *cand_len, int32_t *cand_pos,
                   int32_t *n_found, int32_t *flags, const void *h, int h_bf16, const float *w,
                   int d, float tau, float *score, int32_t *gate) {
  GateArgs g;
  g.ctx = ctx;
  g.ctx_total = ctx_total;
  g.ctx_off = ctx_off;
  g.kappa = kappa;
  g.W = W;
  g.D = D;
  g.cand_tok = cand_tok;
  g.cand_len = cand_len;
  g.cand_pos = cand_pos;
  g.n_found = n_found;
  g.flags = flags;
  g.h = h;
  g.h_bf16 = h_bf16;
  g.w = w;
  g.d = d;
  g.tau = tau;
  g.score = score;
  g.gate = gate;
  return g;
}

hipError_t launch_copy_match(const int32_t *ctx, int64_t ctx_total, const int32_t *ctx_off, int B,
                             int kappa, int W, int D, int32_t *cand_tok, int32_t *cand_len,
                             int32_t *cand_pos, int32_t *n_found, int32_t *flags, const void *h,
                             int h_bf16, const float *w, int d, float tau, float *score,
                             int32_t *gate, hipStream_t st) {
  const GateArgs g = gate_args(ctx, ctx_total, ctx_off, kappa, W, D, cand_tok, cand_len, cand_pos,
                               n_found, flags, h, h_bf16, w, d, tau, score, gate);
  hipLaunchKernelGGL(gate_kernel, dim3(B), dim3(kGateThreads), 0, st, g);
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
