// C ABI of libvstep: argument validation (before anything is enqueued), workspace
// sizing and the verify-step orchestration.  See include/vstep.h for the contract.

#include "../../include/vstep.h"
#include "../../include/vstep_measure.h"
#include "vs_internal.hpp"

#include <math.h>

#include <mutex>

namespace {

constexpr int kMaxRows = 1024;      // W*D per sequence
constexpr int kMaxVocabSampler = 1024 * 512;

inline hipStream_t S(void *s) { return (hipStream_t)s; }

inline int hip_status(hipError_t e) { return e == hipSuccess ? VS_OK : VS_ERR_HIP; }

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

constexpr int kMaxLayers = 1024;

// layers of a descriptor: 0 reads as one; negative is invalid (returned as 0)
inline int layers_of(int32_t n) { return n == 0 ? 1 : (n < 0 ? 0 : n); }

// attention workgroups of one launch (prefix splits of the bf16 plan, or one wave per
// row and head for fp32), for the grid-size limit
int64_t attn_launch_groups(int B, int W, int D, int Hq, int Hkv, int max_pages, int dtype,
                           int L) {
  if (dtype == VS_BF16) {
    const vs::AttnPlan p = vs::attn_plan(B, W, D, Hq, Hkv, max_pages, 16, L);
    return (int64_t)p.n_rb * (p.n_splits + 1) * B * Hkv * L;
  }
  return ((int64_t)L * B * W * D * Hq + 3) / 4;
}

int check_attn(const vs_attn_desc *d) {
  if (!d) return VS_ERR_INVALID_ARG;
  if (d->B <= 0 || d->W <= 0 || d->D <= 0 || d->Hq <= 0 || d->Hkv <= 0 || d->head_dim <= 0 ||
      d->max_pages < 0 || d->n_pool_pages < 0)
    return VS_ERR_INVALID_ARG;
  if ((int64_t)d->W * d->D > kMaxRows) return VS_ERR_INVALID_ARG;
  if (d->Hq % d->Hkv != 0) return VS_ERR_INVALID_ARG;
  // a paged prefix needs a non-empty pool: masked keys of bad pages are read from it
  if (d->max_pages > 0 && d->n_pool_pages < 1) return VS_ERR_INVALID_ARG;
  if (d->page_size != 16) return VS_ERR_UNSUPPORTED;
  if (d->dtype == VS_BF16) {
    if (d->head_dim != 128) return VS_ERR_UNSUPPORTED;
  } else if (d->dtype == VS_F32) {
    if (d->head_dim != 16 && d->head_dim != 32 && d->head_dim != 64) return VS_ERR_UNSUPPORTED;
  } else {
    return VS_ERR_UNSUPPORTED;
  }
  if ((int64_t)d->max_pages * 16 > (1 << 28)) return VS_ERR_UNSUPPORTED;
  const int L = layers_of(d->n_layers);
  if (L < 1) return VS_ERR_INVALID_ARG;
  if (L > kMaxLayers) return VS_ERR_UNSUPPORTED;
  if (attn_launch_groups(d->B, d->W, d->D, d->Hq, d->Hkv, d->max_pages, d->dtype, L) > (1 << 30))
    return VS_ERR_UNSUPPORTED;
  return VS_OK;
}

int check_head(const vs_head_desc *d) {
  if (!d) return VS_ERR_INVALID_ARG;
  if (d->M <= 0 || d->d <= 0 || d->V <= 0 || d->rank < 0) return VS_ERR_INVALID_ARG;
  if (!(d->temperature > 0.f) || !isfinite(d->temperature)) return VS_ERR_INVALID_ARG;
  if (d->dtype == VS_BF16) {
    if (d->d % 32 != 0 || d->rank % 32 != 0) return VS_ERR_UNSUPPORTED;
  } else if (d->dtype != VS_F32) {
    return VS_ERR_UNSUPPORTED;
  }
  return VS_OK;
}

int check_sample(const vs_sample_desc *d) {
  if (!d) return VS_ERR_INVALID_ARG;
  if (d->B <= 0 || d->W <= 0 || d->D <= 0 || d->V <= 0) return VS_ERR_INVALID_ARG;
  if ((int64_t)d->W * d->D > kMaxRows) return VS_ERR_INVALID_ARG;
  if (!(d->temperature > 0.f) || !isfinite(d->temperature)) return VS_ERR_INVALID_ARG;
  if (d->V > kMaxVocabSampler) return VS_ERR_UNSUPPORTED;
  if (d->accept_mode != VS_ACCEPT_LONGEST && d->accept_mode != VS_ACCEPT_MULTI &&
      d->accept_mode != VS_ACCEPT_GREEDY)
    return VS_ERR_INVALID_ARG;
  if (d->accept_mode == VS_ACCEPT_MULTI && d->W > 64) return VS_ERR_UNSUPPORTED;
  return VS_OK;
}

// the multi-candidate kernels run when there is more than one candidate (with one, the
// rule is the single-chain rule); they take copy drafts only
static bool sample_multi(int accept_mode, int W) { return accept_mode == VS_ACCEPT_MULTI && W > 1; }

// sampler rule: 0 longest run (also multi with one candidate), 1 multi, 2 greedy
static int sample_rule(int accept_mode, int W) {
  return accept_mode == VS_ACCEPT_GREEDY ? 2 : (sample_multi(accept_mode, W) ? 1 : 0);
}

float attn_scale(float scale, int hd) { return scale > 0.f ? scale : 1.0f / sqrtf((float)hd); }

struct StepLayout {
  size_t attn, head, sample, total;
};

StepLayout step_layout(const vs_step_desc *d) {
  StepLayout L;
  L.attn = 0;
  const size_t a = vs::attn_workspace_bytes(d->B, d->W, d->D, d->Hq, d->Hkv, d->head_dim,
                                            d->max_pages, 16, d->dtype, layers_of(d->n_layers));
  L.head = align256(a);
  const size_t h = vs::head_workspace_bytes(d->B * d->W * d->D, d->d, d->V, 0, d->dtype);
  L.sample = align256(L.head + h);
  const size_t s = vs::sample_workspace_bytes(d->B, d->W, d->D, d->V);
  L.total = align256(L.sample + s);
  return L;
}

// ---- fixed scratch area of vs_verify_step_noalloc (no allocation on the call path)
// One array per GPU, a file-scope device global: the HIP runtime places a copy on
// every device the library's code object is loaded on, and keeps it until the process
// ends.  Host code never passes `scratch` itself to a kernel (on the host that name is
// only a stand-in for the symbol): the device address of each GPU's copy is looked up
// once with hipGetSymbolAddress, with that GPU current, and kept in scratch_dev.
constexpr size_t kScratchBytes = VS_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxScratchDevices = 64;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
void *scratch_dev[kMaxScratchDevices];
std::mutex scratch_mu;

// The scratch address on the device of `stream` (which must be the current device).
int scratch_for_stream(hipStream_t stream, void **out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return VS_ERR_HIP;
  if (dev < 0 || dev >= kMaxScratchDevices) return VS_ERR_UNSUPPORTED;
  if (stream != nullptr) {
    int sdev = -1;
    if (hipStreamGetDevice(stream, &sdev) != hipSuccess) return VS_ERR_HIP;
    if (sdev != dev) return VS_ERR_INVALID_ARG;
  }
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (scratch_dev[dev] == nullptr) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return VS_ERR_HIP;
    scratch_dev[dev] = p;
  }
  *out = scratch_dev[dev];
  return VS_OK;
}

}  // namespace

extern "C" {

int vs_abi_version(void) { return VS_ABI_VERSION; }

const char *vs_status_str(int s) {
  switch (s) {
    case VS_OK: return "ok";
    case VS_ERR_INVALID_ARG: return "invalid argument";
    case VS_ERR_UNSUPPORTED: return "unsupported configuration";
    case VS_ERR_WORKSPACE: return "workspace missing or too small";
    case VS_ERR_HIP: return "HIP launch or runtime error";
    default: return "unknown status";
  }
}

int vs_copy_match(const int32_t *ctx, int64_t ctx_total, const int32_t *ctx_off, int B, int kappa,
                  int W, int D, int32_t *cand_tok, int32_t *cand_len, int32_t *cand_pos,
                  int32_t *n_found, int32_t *flags, void *stream) {
  if (!ctx_off || !cand_tok || !cand_len || !cand_pos || !n_found) return VS_ERR_INVALID_ARG;
  if (ctx_total < 0 || (ctx_total > 0 && !ctx)) return VS_ERR_INVALID_ARG;
  if (B <= 0 || W <= 0 || D <= 0 || (int64_t)W * D > kMaxRows) return VS_ERR_INVALID_ARG;
  if (kappa < 1 || kappa > 16) return VS_ERR_UNSUPPORTED;
  return hip_status(vs::launch_copy_match(ctx, ctx_total, ctx_off, B, kappa, W, D, cand_tok,
                                          cand_len, cand_pos, n_found, flags, nullptr, 0, nullptr,
                                          0, 0.f, nullptr, nullptr, S(stream)));
}

int vs_probe_gate(const void *h, int h_dtype, const float *w, int B, int d, float tau,
                  const int32_t *n_found, float *score, int32_t *gate, int32_t *flags,
                  void *stream) {
  if (!h || !w || !score || !gate) return VS_ERR_INVALID_ARG;
  if (B <= 0 || d <= 0 || !isfinite(tau)) return VS_ERR_INVALID_ARG;
  if (h_dtype != VS_F32 && h_dtype != VS_BF16) return VS_ERR_UNSUPPORTED;
  return hip_status(vs::launch_probe_gate(h, h_dtype == VS_BF16, w, B, d, tau, n_found, score,
                                          gate, flags, S(stream)));
}

size_t vs_attention_workspace_bytes(const vs_attn_desc *d) {
  if (check_attn(d) != VS_OK) return 0;
  return vs::attn_workspace_bytes(d->B, d->W, d->D, d->Hq, d->Hkv, d->head_dim, d->max_pages,
                                  d->page_size, d->dtype, layers_of(d->n_layers));
}

int vs_verify_attention(const vs_attn_desc *d, const void *q, const void *k_cand,
                        const void *v_cand, const void *k_pool, const void *v_pool,
                        const int32_t *page_table, const int32_t *prefix_len, void *out,
                        int32_t *flags, void *workspace, size_t ws_bytes, void *stream) {
  int st = check_attn(d);
  if (st != VS_OK) return st;
  if (!q || !k_cand || !v_cand || !prefix_len || !out) return VS_ERR_INVALID_ARG;
  if (d->max_pages > 0 && (!k_pool || !v_pool || !page_table)) return VS_ERR_INVALID_ARG;
  const size_t need = vs_attention_workspace_bytes(d);
  if (need > 0 && (!workspace || ws_bytes < need)) return VS_ERR_WORKSPACE;
  if (flags) {
    hipError_t e = vs::launch_zero_i32(flags, d->B, S(stream));
    if (e != hipSuccess) return VS_ERR_HIP;
  }
  return hip_status(vs::launch_attention(d->B, d->W, d->D, d->Hq, d->Hkv, d->head_dim,
                                         d->max_pages, d->n_pool_pages, d->dtype,
                                         attn_scale(d->scale, d->head_dim), q, k_cand, v_cand,
                                         k_pool, v_pool, page_table, prefix_len, out, flags,
                                         workspace, S(stream), nullptr, layers_of(d->n_layers)));
}

size_t vs_packed_weight_bytes(int N, int K) {
  if (N <= 0 || K <= 0 || K % 32 != 0) return 0;
  return vs::packed_weight_elems(N, K) * 2;
}

int vs_pack_weight(const void *src, void *dst, int N, int K, void *stream) {
  if (!src || !dst || N <= 0 || K <= 0) return VS_ERR_INVALID_ARG;
  if (K % 32 != 0) return VS_ERR_UNSUPPORTED;
  return hip_status(vs::launch_pack_weight(src, dst, N, K, S(stream)));
}

size_t vs_head_workspace_bytes(const vs_head_desc *d) {
  if (check_head(d) != VS_OK) return 0;
  return vs::head_workspace_bytes(d->M, d->d, d->V, d->rank, d->dtype);
}

int vs_lm_head(const vs_head_desc *d, const void *h, const void *w_full, const void *w_down,
               const void *w_up, float *logits, double *row_lse, float *probs, void *workspace,
               size_t ws_bytes, void *stream) {
  int st = check_head(d);
  if (st != VS_OK) return st;
  if (!h || !logits || !row_lse) return VS_ERR_INVALID_ARG;
  if (d->rank == 0 && !w_full) return VS_ERR_INVALID_ARG;
  if (d->rank > 0 && (!w_down || !w_up || w_full)) return VS_ERR_INVALID_ARG;
  if (d->write_probs && !probs) return VS_ERR_INVALID_ARG;
  if (!workspace || ws_bytes < vs_head_workspace_bytes(d)) return VS_ERR_WORKSPACE;
  const vs::HeadWs hw = vs::head_ws(workspace, d->M, d->V, d->rank);
  hipError_t e = vs::launch_head_gemm(d->M, d->d, d->V, d->rank, d->dtype, d->temperature, h,
                                      w_full, w_down, w_up, logits, hw, nullptr, 0, nullptr,
                                      S(stream));
  if (e != hipSuccess) return VS_ERR_HIP;
  return hip_status(vs::launch_head_finish(d->M, d->V, d->temperature, logits, row_lse,
                                           d->write_probs ? probs : nullptr, hw, S(stream)));
}

size_t vs_sample_workspace_bytes(const vs_sample_desc *d) {
  if (check_sample(d) != VS_OK) return 0;
  // greedy without a head before it: the tile statistics of the given logits
  return vs::sample_workspace_bytes(d->B, d->W, d->D, d->V, d->accept_mode == VS_ACCEPT_GREEDY);
}

int vs_reject_sample(const vs_sample_desc *d, const float *root_logits, const float *logits,
                     const double *row_lse, const float *q, const int32_t *cand_tok,
                     const int32_t *cand_len, const double *u_acc, const double *u_res,
                     const int32_t *gate, int32_t *n_acc, int32_t *best, int32_t *out_tok,
                     int32_t *n_out, int32_t *acc_per_cand, int32_t *flags, void *workspace,
                     size_t ws_bytes, void *stream) {
  int st = check_sample(d);
  if (st != VS_OK) return st;
  const int rule = sample_rule(d->accept_mode, d->W);
  const bool greedy = rule == 2;
  if (!root_logits || !logits || !row_lse || !cand_tok || !cand_len ||
      (!greedy && (!u_acc || !u_res)) || !n_acc || !best || !out_tok || !n_out || !acc_per_cand)
    return VS_ERR_INVALID_ARG;
  // copy drafts (point masses) walk the chain in LDS, within its bound
  if (rule == 1 && !q && !vs::sampler_multi_fits(d->W, d->D)) return VS_ERR_UNSUPPORTED;
  const size_t need = vs_sample_workspace_bytes(d);
  if (!workspace || ws_bytes < need) return VS_ERR_WORKSPACE;
  const vs::SampleWs sw = vs::sample_ws(workspace, d->B, d->W, d->D, d->V, greedy);
  hipError_t e = vs::launch_root_stats(root_logits, d->B, d->V, d->temperature, sw.root_stats,
                                       S(stream));
  if (e != hipSuccess) return VS_ERR_HIP;
  if (greedy) {
    e = vs::launch_row_stats(logits, d->B * d->W * d->D, d->V, d->temperature, sw.row_stats,
                             S(stream));
    if (e != hipSuccess) return VS_ERR_HIP;
  }
  // row_lse is an input here: only the root normalisers and the tests are computed
  e = vs::launch_lse_tests(d->B, d->W, d->D, d->V, d->temperature, nullptr,
                           const_cast<double *>(row_lse), root_logits, logits, q, cand_tok,
                           cand_len, gate, u_acc, sw, S(stream), rule, sw.row_stats);
  if (e != hipSuccess) return VS_ERR_HIP;
  return hip_status(vs::launch_sampler(d->B, d->W, d->D, d->V, d->temperature, root_logits, logits,
                                       row_lse, q, cand_tok, cand_len, u_res, gate, n_acc, best,
                                       out_tok, n_out, acc_per_cand, flags, 0, sw, S(stream),
                                       nullptr, rule, u_acc));
}

static int check_step(const vs_step_desc *d) {
  if (!d) return VS_ERR_INVALID_ARG;
  vs_attn_desc ad = {d->B, d->W, d->D, d->Hq, d->Hkv, d->head_dim, d->page_size, d->max_pages,
                     d->n_pool_pages, d->dtype, d->scale, d->n_layers};
  int st = check_attn(&ad);
  if (st != VS_OK) return st;
  vs_head_desc hd = {d->B * d->W * d->D, d->d, d->V, 0, d->dtype, d->temperature, 0};
  if ((st = check_head(&hd)) != VS_OK) return st;
  vs_sample_desc sd = {d->B, d->W, d->D, d->V, d->temperature, d->accept_mode};
  if ((st = check_sample(&sd)) != VS_OK) return st;
  if (d->d != d->Hq * d->head_dim) return VS_ERR_INVALID_ARG;
  if (!d->external_drafts) {
    if (d->kappa < 1 || d->kappa > 16) return VS_ERR_UNSUPPORTED;
    if (d->ctx_total < 0 || !isfinite(d->tau)) return VS_ERR_INVALID_ARG;
  }
  return VS_OK;
}

size_t vs_step_workspace_bytes(const vs_step_desc *d) {
  if (check_step(d) != VS_OK) return 0;
  return step_layout(d).total;
}

static int verify_step_impl(const vs_step_desc *d, const vs_step_io *io, void *workspace,
                            size_t ws_bytes, void *stream, bool clear_counters) {
  int st = check_step(d);
  if (st != VS_OK) return st;
  if (!io) return VS_ERR_INVALID_ARG;
  const int rule = sample_rule(d->accept_mode, d->W);
  if (!io->q || !io->k_cand || !io->v_cand || !io->prefix_len || !io->w_full ||
      !io->root_logits || (rule != 2 && (!io->u_acc || !io->u_res)) || !io->cand_tok ||
      !io->cand_len ||
      !io->attn_out || !io->logits || !io->row_lse || !io->n_acc || !io->best || !io->out_tok ||
      !io->n_out || !io->acc_per_cand || !io->flags)
    return VS_ERR_INVALID_ARG;
  if (d->max_pages > 0 && (!io->k_pool || !io->v_pool || !io->page_table))
    return VS_ERR_INVALID_ARG;
  if (!d->external_drafts) {
    if (!io->ctx_off || (d->ctx_total > 0 && !io->ctx) || !io->probe_h || !io->probe_w ||
        !io->cand_pos || !io->n_found || !io->score || !io->gate)
      return VS_ERR_INVALID_ARG;
  }
  if (io->aux_stream && (!io->fork_event || !io->join_event)) return VS_ERR_INVALID_ARG;
  if (rule == 1 && !io->q_draft && !vs::sampler_multi_fits(d->W, d->D)) return VS_ERR_UNSUPPORTED;
  const StepLayout L = step_layout(d);
  if (!workspace || ws_bytes < L.total) return VS_ERR_WORKSPACE;
  hipStream_t s = S(stream);
  hipEvent_t *ev = (hipEvent_t *)io->stage_events;
  auto mark = [&](int i) -> bool {
    return ev == nullptr || hipEventRecord(ev[i], s) == hipSuccess;
  };
  const int M = d->B * d->W * d->D;
  const int n_layers = layers_of(d->n_layers);
  char *ws = (char *)workspace;
  const vs::HeadWs hw = vs::head_ws(ws + L.head, M, d->V, 0);
  const vs::SampleWs sw = vs::sample_ws(ws + L.sample, d->B, d->W, d->D, d->V);
  hipError_t e;
  if (clear_counters) {
    // a shared scratch area holds whatever the last call left there: the words that
    // must start at zero (sampler counters, attention flags) are cleared by a kernel
    e = vs::launch_zero_i32((int32_t *)sw.counters, d->B, s);
    if (e == hipSuccess) e = vs::launch_zero_i32(sw.attn_flags, d->B, s);
    if (e != hipSuccess) return VS_ERR_HIP;
  }
  if (!mark(0)) return VS_ERR_HIP;
  // 1. copy retrieval + probe gate.  With fp32 attention, or bf16 attention whose row
  //    blocks have four or more waves, its B workgroups ride in the attention launch
  //    (step 2) and run beside the attention workgroups; otherwise one launch of its
  //    own, on the auxiliary stream when given.  It is the first writer of io->flags; attention reports
  //    into the workspace (sw.attn_flags), which the sampler folds in, so the two never
  //    race.
  const bool copy_path = !d->external_drafts;
  const bool fuse = copy_path && vs::attn_fuses_gate(d->B, d->W, d->D, d->Hq, d->Hkv,
                                                     d->max_pages, d->dtype);
  const vs::GateArgs ga = vs::gate_args(io->ctx, d->ctx_total, io->ctx_off, d->kappa, d->W, d->D,
                                        io->cand_tok, io->cand_len, io->cand_pos, io->n_found,
                                        io->flags, io->probe_h, d->dtype == VS_BF16, io->probe_w,
                                        d->d, d->tau, io->score, io->gate);
  const bool fork = io->aux_stream != nullptr && copy_path && !fuse;
  hipStream_t gs = s;
  if (fork) {
    gs = S(io->aux_stream);
    if (hipEventRecord((hipEvent_t)io->fork_event, s) != hipSuccess ||
        hipStreamWaitEvent(gs, (hipEvent_t)io->fork_event, 0) != hipSuccess)
      return VS_ERR_HIP;
  }
  if (copy_path && !fuse) {
    e = vs::launch_copy_match(io->ctx, d->ctx_total, io->ctx_off, d->B, d->kappa, d->W, d->D,
                              io->cand_tok, io->cand_len, io->cand_pos, io->n_found, io->flags,
                              io->probe_h, d->dtype == VS_BF16, io->probe_w, d->d, d->tau,
                              io->score, io->gate, gs);
    if (e != hipSuccess) return VS_ERR_HIP;
    if (fork && hipEventRecord((hipEvent_t)io->join_event, gs) != hipSuccess) return VS_ERR_HIP;
  }
  if (!mark(1)) return VS_ERR_HIP;
  // 2. verify attention (with the gate's workgroups in front when fused)
  e = vs::launch_attention(d->B, d->W, d->D, d->Hq, d->Hkv, d->head_dim, d->max_pages,
                           d->n_pool_pages, d->dtype, attn_scale(d->scale, d->head_dim), io->q,
                           io->k_cand, io->v_cand, io->k_pool, io->v_pool, io->page_table,
                           io->prefix_len, io->attn_out, sw.attn_flags, ws + L.attn, s,
                           fuse ? &ga : nullptr, n_layers);
  if (e != hipSuccess || !mark(2)) return VS_ERR_HIP;
  // 3. head: GEMM + tile statistics (verify rows and root rows) over the last layer's
  //    attention output
  const char *head_in = (const char *)io->attn_out +
                        (size_t)(n_layers - 1) * M * d->d * (d->dtype == VS_BF16 ? 2 : 4);
  e = vs::launch_head_gemm(M, d->d, d->V, 0, d->dtype, d->temperature, head_in, io->w_full,
                           nullptr, nullptr, io->logits, hw, io->root_logits, d->B,
                           sw.root_stats, s);
  if (e != hipSuccess || !mark(3)) return VS_ERR_HIP;
  if (fork && hipStreamWaitEvent(s, (hipEvent_t)io->join_event, 0) != hipSuccess)
    return VS_ERR_HIP;
  // 4. normalisers of every row and the acceptance test of every draft token
  const int32_t *gate = d->external_drafts ? nullptr : io->gate;
  e = vs::launch_lse_tests(d->B, d->W, d->D, d->V, d->temperature, hw.stats, io->row_lse,
                           io->root_logits, io->logits, io->q_draft, io->cand_tok, io->cand_len,
                           gate, io->u_acc, sw, s, rule, hw.stats);
  if (e != hipSuccess || !mark(4)) return VS_ERR_HIP;
  // 5. longest accepted run (or the multi-candidate chain) and the extra token (flags: accumulate onto the gate's,
  //    or written whole when there was no retrieval)
  e = vs::launch_sampler(d->B, d->W, d->D, d->V, d->temperature, io->root_logits, io->logits,
                         io->row_lse, io->q_draft, io->cand_tok, io->cand_len, io->u_res, gate,
                         io->n_acc, io->best, io->out_tok, io->n_out, io->acc_per_cand, io->flags,
                         d->external_drafts ? 0 : 1, sw, s, sw.attn_flags, rule, io->u_acc);
  if (e != hipSuccess || !mark(5)) return VS_ERR_HIP;
  return VS_OK;
}

int vs_verify_step(const vs_step_desc *d, const vs_step_io *io, void *workspace,
                   size_t ws_bytes, void *stream) {
  return verify_step_impl(d, io, workspace, ws_bytes, stream, false);
}

int vs_verify_step_noalloc(const vs_step_desc *d, const vs_step_io *io, void *stream) {
  const int st = check_step(d);
  if (st != VS_OK) return st;
  if (!io) return VS_ERR_INVALID_ARG;
  if (step_layout(d).total > kScratchBytes) return VS_ERR_UNSUPPORTED;
  void *ptr = nullptr;
  const int sst = scratch_for_stream(S(stream), &ptr);
  if (sst != VS_OK) return sst;
  return verify_step_impl(d, io, ptr, kScratchBytes, stream, true);
}

size_t vs_draft_sample_workspace_bytes(int rows, int V) {
  if (rows <= 0 || V <= 0 || V > kMaxVocabSampler) return 0;
  return vs::draft_workspace_bytes(rows, V);
}

int vs_draft_sample(const float *q, int rows, int V, const double *u, int32_t *tok,
                    int32_t *flags, void *workspace, size_t ws_bytes, void *stream) {
  if (!q || !u || !tok || rows <= 0 || V <= 0) return VS_ERR_INVALID_ARG;
  if (V > kMaxVocabSampler) return VS_ERR_UNSUPPORTED;
  if (!workspace || ws_bytes < vs::draft_workspace_bytes(rows, V)) return VS_ERR_WORKSPACE;
  return hip_status(vs::launch_draft_sample(q, rows, V, u, tok, flags, workspace, S(stream)));
}

size_t vs_copy_labels_workspace_bytes(int64_t ctx_total) {
  if (ctx_total < 0 || ctx_total >= INT32_MAX) return 0;
  return vs::labels_workspace_bytes(ctx_total);
}

int vs_copy_labels(const int32_t *ctx, int64_t ctx_total, const int32_t *ctx_off, int B,
                   int kappa, uint8_t *labels, int32_t *flags, void *workspace,
                   size_t ws_bytes, void *stream) {
  if (!ctx_off || (ctx_total > 0 && (!ctx || !labels)) || B <= 0 || ctx_total < 0)
    return VS_ERR_INVALID_ARG;
  if (kappa < 1 || kappa > 16 || ctx_total >= INT32_MAX) return VS_ERR_UNSUPPORTED;
  if (!workspace || ws_bytes < vs::labels_workspace_bytes(ctx_total)) return VS_ERR_WORKSPACE;
  return hip_status(vs::launch_copy_labels(ctx, ctx_total, ctx_off, B, kappa, labels, flags,
                                           workspace, S(stream)));
}

static int check_kv(const vs_kv_desc *d, bool commit) {
  if (!d) return VS_ERR_INVALID_ARG;
  if (d->B <= 0 || d->max_pages <= 0 || d->n_pool_pages <= 0) return VS_ERR_INVALID_ARG;
  if (d->page_size != 16) return VS_ERR_UNSUPPORTED;
  if (d->B > vs::kMaxSeqKv) return VS_ERR_UNSUPPORTED;
  if ((int64_t)d->max_pages * 16 > (1 << 28)) return VS_ERR_UNSUPPORTED;
  if (commit) {
    if (d->W <= 0 || d->D <= 0 || d->Hkv <= 0 || d->head_dim <= 0) return VS_ERR_INVALID_ARG;
    if ((int64_t)d->W * d->D > kMaxRows) return VS_ERR_INVALID_ARG;
    if (d->dtype != VS_BF16 && d->dtype != VS_F32) return VS_ERR_UNSUPPORTED;
    const int L = layers_of(d->n_layers);
    if (L < 1) return VS_ERR_INVALID_ARG;
    if (L > 65535) return VS_ERR_UNSUPPORTED;
  }
  return VS_OK;
}

size_t vs_kv_workspace_bytes(const vs_kv_desc *d) {
  if (check_kv(d, true) != VS_OK) return 0;
  return vs::kv_workspace_bytes(d->B);
}

int vs_kv_commit(const vs_kv_desc *d, const void *k_cand, const void *v_cand, const int32_t *best,
                 const int32_t *n_acc, void *k_pool, void *v_pool, int32_t *page_table,
                 int32_t *prefix_len, int32_t *free_list, int32_t *n_free, int32_t *flags,
                 void *workspace, size_t ws_bytes, void *stream) {
  const int st = check_kv(d, true);
  if (st != VS_OK) return st;
  if (!k_cand || !v_cand || !best || !n_acc || !k_pool || !v_pool || !page_table ||
      !prefix_len || !free_list || !n_free)
    return VS_ERR_INVALID_ARG;
  if (!workspace || ws_bytes < vs::kv_workspace_bytes(d->B)) return VS_ERR_WORKSPACE;
  return hip_status(vs::launch_kv_commit(d->B, d->W, d->D, d->Hkv, d->head_dim, d->max_pages,
                                         d->n_pool_pages, d->dtype == VS_BF16 ? 2 : 4, k_cand,
                                         v_cand, best, n_acc, k_pool, v_pool, page_table,
                                         prefix_len, free_list, n_free, flags, workspace,
                                         S(stream), layers_of(d->n_layers)));
}

int vs_measure_read(const void *buf, size_t bytes, uint32_t *sink, int n_wg, int pattern,
                    void *stream) {
  if (!buf || !sink || bytes < 16 || n_wg <= 0 || (pattern != 0 && pattern != 1))
    return VS_ERR_INVALID_ARG;
  if (pattern == 1 && bytes / 16 < (size_t)n_wg) return VS_ERR_INVALID_ARG;
  return hip_status(vs::launch_peak_read(buf, bytes, sink, n_wg, pattern, S(stream)));
}

int vs_measure_mfma(int n_wg, int iters, float *sink, void *stream) {
  if (!sink || n_wg <= 0 || iters <= 0) return VS_ERR_INVALID_ARG;
  return hip_status(vs::launch_peak_mfma(n_wg, iters, sink, S(stream)));
}

int vs_kv_pack_pages(const void *k_src, const void *v_src, int64_t n_tokens, int Hkv,
                     int head_dim, int dtype, void *k_pool, void *v_pool, void *stream) {
  if (!k_src || !v_src || !k_pool || !v_pool) return VS_ERR_INVALID_ARG;
  if (n_tokens <= 0 || Hkv <= 0 || head_dim <= 0) return VS_ERR_INVALID_ARG;
  if (dtype != VS_BF16 && dtype != VS_F32) return VS_ERR_UNSUPPORTED;
  if (head_dim > 256 || (n_tokens + 15) / 16 > INT32_MAX || Hkv > 65535) return VS_ERR_UNSUPPORTED;
  return hip_status(vs::launch_kv_pack(k_src, v_src, n_tokens, Hkv, head_dim,
                                       dtype == VS_BF16 ? 2 : 4, k_pool, v_pool, S(stream)));
}

int vs_kv_truncate(const vs_kv_desc *d, const int32_t *new_len, int32_t *page_table,
                   int32_t *prefix_len, int32_t *free_list, int32_t *n_free, int32_t *flags,
                   void *stream) {
  const int st = check_kv(d, false);
  if (st != VS_OK) return st;
  if (!new_len || !page_table || !prefix_len || !free_list || !n_free) return VS_ERR_INVALID_ARG;
  return hip_status(vs::launch_kv_truncate(d->B, d->max_pages, d->n_pool_pages, new_len,
                                           page_table, prefix_len, free_list, n_free, flags,
                                           S(stream)));
}

}  // extern "C"
