// Internal declarations shared by the HIP translation units of libvstep.
// Kernels are written for gfx950 (CDNA4): wave64, MFMA bf16 16x16x32.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vs {

typedef uint16_t bf16_t;  // raw bf16 bits
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;

constexpr int kWave = 64;
// vocabulary span of one head workgroup; softmax tile statistics come at this grain
constexpr int kHeadVocabTile = 256;

// flag bits (same values as the public header)
enum : int {
  FLAG_PROBE_TIE = 1, FLAG_ACCEPT_TIE = 2, FLAG_CDF_TIE = 4, FLAG_DEGENERATE = 8,
  FLAG_NO_CANDIDATE = 16, FLAG_BAD_PAGE = 32, FLAG_BAD_CTX = 64, FLAG_BAD_TOKEN = 128,
  FLAG_POOL_EMPTY = 256, FLAG_SYNC_TIMEOUT = 512
};

__device__ __forceinline__ float bf16_to_f32(bf16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;

// fp32 -> bf16 pair, round to nearest even (one v_cvt_pk_bf16_f32 on gfx950)
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2_t r = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(bf16_t, (__bf16)f);
}

// x = hi + lo with hi = bf16(x) and lo = bf16(x - hi), for a pair of values (x - hi
// is exact in fp32).  hi is converted once, in an opaque instruction, and read back
// from its packed bits (the compiler would otherwise convert each value again).
__device__ __forceinline__ void split_bf16x2(float x0, float x1, uint32_t &hi, uint32_t &lo) {
  asm("v_cvt_pk_bf16_f32 %0, %1, %2" : "=v"(hi) : "v"(x0), "v"(x1));
  const float h0 = __uint_as_float(hi << 16);
  const float h1 = __uint_as_float(hi & 0xffff0000u);
  lo = pack_bf16x2(x0 - h0, x1 - h1);
}

__device__ __forceinline__ f32x4 mfma16x16x32(const bf16x8 &a, const bf16x8 &b, const f32x4 &c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

template <typename T>
__device__ __forceinline__ T ceil_div(T a, T b) { return (a + b - 1) / b; }

// Bijection of a 1-D workgroup index so that consecutive logical tiles land on the
// same XCD (workgroups are dealt round-robin over the 8 XCDs of an MI355X), letting
// tiles that share operands share that XCD's L2.
__device__ __forceinline__ int xcd_remap(int bid, int nblocks) {
  const int q = nblocks / 8;
  if (bid >= 8 * q) return bid;
  return (bid % 8) * q + bid / 8;
}

// ---------------------------------------------------------------------------- launchers
struct AttnPlan {
  int rt;           // row tiles (16 rows) per wave
  int nw;           // waves per workgroup
  int rows_per_kv;  // g * M
  int n_rb;         // row blocks per (sequence, kv head)
  int rows_per_block;
  int split_keys;   // prefix keys per split (multiple of 32)
  int n_splits;     // prefix splits (a candidate split is added after them)
};

// L: layers covered by one launch (they share page table and prefix lengths)
AttnPlan attn_plan(int B, int W, int D, int Hq, int Hkv, int max_pages, int page, int L);
size_t attn_workspace_bytes(int B, int W, int D, int Hq, int Hkv, int hd, int max_pages, int page,
                            int dtype, int L);

// Retrieval + probe of the copy path, one sequence per workgroup (gate_wg.hpp).
struct GateArgs {
  const int32_t *ctx;
  int64_t ctx_total;
  const int32_t *ctx_off;
  int kappa, W, D;
  int32_t *cand_tok, *cand_len, *cand_pos, *n_found, *flags;
  const void *h;            // probe input [B, d] or null (retrieval only)
  int h_bf16;
  const float *w;
  int d;
  float tau;
  float *score;
  int32_t *gate;
};
GateArgs gate_args(const int32_t *ctx, int64_t ctx_total, const int32_t *ctx_off, int kappa, int W,
                   int D, int32_t *cand_tok, int32_t *cand_len, int32_t *cand_pos,
                   int32_t *n_found, int32_t *flags, const void *h, int h_bf16, const float *w,
                   int d, float tau, float *score, int32_t *gate);

hipError_t launch_copy_match(const int32_t *ctx, int64_t ctx_total, const int32_t *ctx_off, int B,
                             int kappa, int W, int D, int32_t *cand_tok, int32_t *cand_len,
                             int32_t *cand_pos, int32_t *n_found, int32_t *flags,
                             // fused probe (h == nullptr: retrieval only)
                             const void *h, int h_bf16, const float *w, int d, float tau,
                             float *score, int32_t *gate, hipStream_t st);

hipError_t launch_probe_gate(const void *h, int h_bf16, const float *w, int B, int d, float tau,
                             const int32_t *n_found, float *score, int32_t *gate, int32_t *flags,
                             hipStream_t st);

// Whether the attention launch of these shapes can carry the copy path's gate as extra
// workgroups (bf16 row blocks of at least four waves).
bool attn_fuses_gate(int B, int W, int D, int Hq, int Hkv, int max_pages, int dtype);
// gate != null: the B gate workgroups run first in the same launch (attn_fuses_gate
// must hold).
hipError_t launch_attention(int B, int W, int D, int Hq, int Hkv, int hd, int max_pages,
                            int n_pool_pages, int dtype, float scale, const void *q,
                            const void *k_cand, const void *v_cand, const void *k_pool,
                            const void *v_pool, const int32_t *page_table,
                            const int32_t *prefix_len, void *out, int32_t *flags, void *ws,
                            hipStream_t st, const GateArgs *gate = nullptr, int L = 1);

// Head workspace: per-tile (max, sumexp) statistics [rows][n_vt] and the low-rank
// intermediate.
struct HeadWs {
  float2 *stats;   // [M][n_vt]
  float *t;        // [M][rank]
  size_t bytes;
};
HeadWs head_ws(void *ws, int M, int V, int rank);
// bf16 weights [N, K] -> MFMA operand tiles (see head.hip); K % 32 == 0
size_t packed_weight_elems(int N, int K);
hipError_t launch_pack_weight(const void *src, void *dst, int N, int K, hipStream_t st);
size_t head_workspace_bytes(int M, int d, int V, int rank, int dtype);
// GEMM + tile statistics.  root_logits/root_stats (may be null): also compute the
// tile statistics of B root rows over the same vocabulary tiles.
hipError_t launch_head_gemm(int M, int d, int V, int rank, int dtype, float temperature,
                            const void *h, const void *w_full, const void *w_down,
                            const void *w_up, float *logits, const HeadWs &ws,
                            const float *root_logits, int B_root, float2 *root_stats,
                            hipStream_t st);
// Row normalisers (and optional probabilities) from the tile statistics.
hipError_t launch_head_finish(int M, int V, float temperature, const float *logits,
                              double *row_lse, float *probs, const HeadWs &ws, hipStream_t st);

struct SampleWs {
  uint32_t *counters;   // [B], zero between calls
  double2 *chunk_sums;  // [B][n_chunks]
  float2 *root_stats;   // [B][n_vt]
  double *root_lse;     // [B]
  uint8_t *code;        // [B][W][D] acceptance codes
  int32_t *attn_flags;  // [B] flags raised by attention inside the step, zero between calls
  double *pv;           // [B][W*D+1][W] multi-candidate acceptance: p of each candidate token
  int32_t *amax;        // [B*W*D + B] greedy: argmax of every verify row, then the root rows
  uint8_t *amax_tie;    // [B*W*D + B] greedy: near tie between the two largest logits
  double *resid;        // [B][2][V] multi-candidate acceptance with dense drafts: residual rows
  double *dpart;        // [B][2][128] and its published chunk sums
  float2 *row_stats;    // [B*W*D][n_vt] tile statistics of given logits (greedy, standalone)
  size_t bytes;
};
SampleWs sample_ws(void *ws, int B, int W, int D, int V, bool row_stats = false);
size_t sample_workspace_bytes(int B, int W, int D, int V, bool row_stats = false);
// whether the multi-candidate acceptance handles W candidates of D tokens
bool sampler_multi_fits(int W, int D);
hipError_t launch_root_stats(const float *root_logits, int B, int V, float temperature,
                             float2 *stats, hipStream_t st);
// tile statistics (max, sum exp) [rows][n_vt] of any fp32 rows
hipError_t launch_row_stats(const float *logits, int rows, int V, float temperature,
                            float2 *stats, hipStream_t st);
// fp64 row normalisers from tile statistics [rows][n_vt]
hipError_t launch_lse_from_stats(const float2 *stats, int rows, int V, double *lse,
                                 hipStream_t st);
// Normalisers of the verify rows (row_stats != null; else row_lse is an input) and of
// the root rows (ws.root_stats -> ws.root_lse), and the acceptance test of every draft
// position (-> ws.code), or with multi (rule 1) the p of every candidate token under
// every row (-> ws.pv), or with greedy (rule 2) the argmax of every row (-> ws.amax,
// from am_stats and ws.root_stats) and the argmax tests (-> ws.code).
hipError_t launch_lse_tests(int B, int W, int D, int V, float temperature,
                            const float2 *row_stats, double *row_lse, const float *root_logits,
                            const float *logits, const float *q, const int32_t *cand_tok,
                            const int32_t *cand_len, const int32_t *gate, const double *u_acc,
                            const SampleWs &ws, hipStream_t st, int rule = 0,
                            const float2 *am_stats = nullptr);
// Longest accepted run (or with multi the multi-candidate chain over ws.pv and u_acc),
// residual / bonus draw, outputs (reads ws.code, ws.root_lse).
hipError_t launch_sampler(int B, int W, int D, int V, float temperature, const float *root_logits,
                          const float *logits, const double *row_lse, const float *q,
                          const int32_t *cand_tok, const int32_t *cand_len, const double *u_res,
                          const int32_t *gate, int32_t *n_acc, int32_t *best, int32_t *out_tok,
                          int32_t *n_out, int32_t *acc_per_cand, int32_t *flags,
                          int flags_accumulate, const SampleWs &ws, hipStream_t st,
                          int32_t *attn_flags = nullptr, int rule = 0,
                          const double *u_acc = nullptr);

hipError_t launch_zero_i32(int32_t *p, int n, hipStream_t st);

// ---- draft tokens by inverse CDF of stored probability rows (sampler.hip)
size_t draft_workspace_bytes(int rows, int V);
hipError_t launch_draft_sample(const float *q, int rows, int V, const double *u, int32_t *tok,
                               int32_t *flags, void *ws, hipStream_t st);

// ---- copy-mode labels (labels.hip)
size_t labels_workspace_bytes(int64_t total);
hipError_t launch_copy_labels(const int32_t *ctx, int64_t total, const int32_t *ctx_off, int B,
                              int kappa, uint8_t *labels, int32_t *flags, void *ws,
                              hipStream_t st);

// ---- measured ceilings (peaks.hip)
hipError_t launch_peak_read(const void *buf, size_t bytes, uint32_t *sink, int n_wg,
                            int pattern, hipStream_t st);
hipError_t launch_peak_mfma(int n_wg, int iters, float *sink, hipStream_t st);

// ---- KV commit and rollback (kv.hip)
constexpr int kMaxSeqKv = 2048;   // sequences per call
size_t kv_workspace_bytes(int B);
hipError_t launch_kv_commit(int B, int W, int D, int Hkv, int hd, int max_pages, int n_pool_pages,
                            int esz, const void *k_cand, const void *v_cand, const int32_t *best,
                            const int32_t *n_acc, void *k_pool, void *v_pool, int32_t *page_table,
                            int32_t *prefix_len, int32_t *free_list, int32_t *n_free,
                            int32_t *flags, void *ws, hipStream_t st, int L = 1);
// token-major K/V [n_tokens][Hkv][hd] -> the verify step's pages (esz: 2 bf16, 4 fp32)
hipError_t launch_kv_pack(const void *k_src, const void *v_src, int64_t n_tokens, int Hkv, int hd,
                          int esz, void *k_pool, void *v_pool, hipStream_t st);
hipError_t launch_kv_truncate(int B, int max_pages, int n_pool_pages, const int32_t *new_len,
                              int32_t *page_table, int32_t *prefix_len, int32_t *free_list,
                              int32_t *n_free, int32_t *flags, hipStream_t st);

}  // namespace vs
