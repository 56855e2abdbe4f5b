// Vocabulary projection of the verify step.
//
// Full head: z = W_full h for every verify row (the GEMM that batching the
// candidates turns the decode GEMV into: rejection-sampling blog, blog.huny.dev,
// section 1).  Low-rank head: z = W_up (W_down h) ("SlimSpec: Low-Rank Draft
// LM-Head ...", gist.science, "방법론 / 아키텍처"), the rank-r intermediate kept in fp32.
//
// bf16 GEMM out[M,N] = H[M,K] . W[N,K]^T, MFMA 16x16x32 bf16, fp32 accumulation:
//   * a workgroup = 4 waves; each wave owns VT 16-row tiles of W (vocabulary) and
//     all MT 16-row tiles of the workgroup's H block;
//   * W is read exactly once, straight from HBM into registers in MFMA operand
//     layout (16-byte loads; each row segment of 256 B is fully used), with the
//     next K-chunk prefetched while the current one is multiplied;
//   * the H block is shared through LDS one K-chunk at a time (padded rows: no bank
//     conflicts on the 16-byte fragment reads);
//   * H may be fp32 (the low-rank intermediate): it is then split on the fly into
//     bf16 hi + lo parts and multiplied twice, keeping ~16 mantissa bits;
//   * the epilogue writes fp32 logits and, per (row, workgroup vocabulary tile),
//     the max and sum of exp(z/T - max): the sampler's normaliser needs no second
//     pass over the logits.

#include "vs_internal.hpp"

namespace vs {

namespace {

constexpr int kThreads = 256;
constexpr int kKC = 128;            // K per chunk
constexpr int kHStride = kKC + 8;   // staged H row (bf16 elements)
constexpr int kVT = 2;              // vocabulary tiles per wave
constexpr int kVocabPerWG = 4 * kVT * 16;

struct GemmArgs {
  const void *h;      // [M, K] bf16, or fp32 when SPLIT
  const bf16_t *w;    // [N, K]
  float *out;         // [M, N]
  float2 *stats;      // [n_vtiles, M] (max, sumexp) of out/T, or null
  int M, N, K;
  int n_mblocks;
  float inv_t;
};

template <int MT, bool SPLIT>
__global__ void __launch_bounds__(kThreads)
head_gemm_kernel(GemmArgs a) {
  __shared__ __attribute__((aligned(16))) bf16_t Hs[(SPLIT ? 2 : 1) * MT * 16 * kHStride];
  __shared__ float2 red[4][MT * 16];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int l16 = lane & 15;
  const int lg = lane >> 4;
  const int n_vtiles = (a.N + kVocabPerWG - 1) / kVocabPerWG;
  const int nblocks = n_vtiles * a.n_mblocks;
  const int bid = xcd_remap(blockIdx.x, nblocks);
  const int mb = bid % a.n_mblocks;   // M blocks of one vocabulary tile are neighbours
  const int vt = bid / a.n_mblocks;
  const int vbase = vt * kVocabPerWG;
  const int mbase = mb * MT * 16;
  const int nchunks = (a.K + kKC - 1) / kKC;

  // W operand pointers (rows clamped into range; masked in the epilogue)
  const bf16_t *wrow[kVT];
#pragma unroll
  for (int v = 0; v < kVT; ++v) {
    int n = vbase + (wv * kVT + v) * 16 + l16;
    n = n < a.N ? n : a.N - 1;
    wrow[v] = a.w + (int64_t)n * a.K + 8 * lg;
  }
  auto load_w = [&](bf16x8 (&dst)[kVT][kKC / 32], int c) {
    const int kc0 = c * kKC;
#pragma unroll
    for (int v = 0; v < kVT; ++v)
#pragma unroll
      for (int s = 0; s < kKC / 32; ++s)
        dst[v][s] = (kc0 + 32 * s < a.K) ? *(const bf16x8 *)(wrow[v] + kc0 + 32 * s) : bf16x8{};
  };

  // H staging: MT*16 rows x kKC columns, 8 elements per thread per pass
  constexpr int kHPass = (MT * 16 * (kKC / 8) + kThreads - 1) / kThreads;
  typedef __attribute__((__vector_size__(8 * sizeof(float)))) float f32x8;
  using HReg = typename std::conditional<SPLIT, f32x8, u32x4>::type;
  HReg hreg[kHPass];
  auto load_h = [&](int c) {
    const int kc0 = c * kKC;
#pragma unroll
    for (int p = 0; p < kHPass; ++p) {
      const int idx = tid + p * kThreads;
      const int r = idx / (kKC / 8);
      const int cc = (idx % (kKC / 8)) * 8;
      const int m = mbase + r;
      const bool ok = (r < MT * 16) && (m < a.M) && (kc0 + cc < a.K);
      if constexpr (SPLIT) {
        const float *src = (const float *)a.h + (int64_t)m * a.K + kc0 + cc;
        hreg[p] = ok ? *(const f32x8 *)src : f32x8{};
      } else {
        const bf16_t *src = (const bf16_t *)a.h + (int64_t)m * a.K + kc0 + cc;
        hreg[p] = ok ? *(const u32x4 *)src : u32x4{0u, 0u, 0u, 0u};
      }
    }
  };
  auto store_h = [&]() {
#pragma unroll
    for (int p = 0; p < kHPass; ++p) {
      const int idx = tid + p * kThreads;
      const int r = idx / (kKC / 8);
      const int cc = (idx % (kKC / 8)) * 8;
      if (r >= MT * 16) continue;
      if constexpr (SPLIT) {
        uint32_t hi[4], lo[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float x0 = hreg[p][2 * e], x1 = hreg[p][2 * e + 1];
          const bf16_t h0 = f32_to_bf16(x0), h1 = f32_to_bf16(x1);
          hi[e] = (uint32_t)h0 | ((uint32_t)h1 << 16);
          lo[e] = pack_bf16x2(x0 - bf16_to_f32(h0), x1 - bf16_to_f32(h1));
        }
        *(u32x4 *)&Hs[r * kHStride + cc] = u32x4{hi[0], hi[1], hi[2], hi[3]};
        *(u32x4 *)&Hs[(MT * 16 + r) * kHStride + cc] = u32x4{lo[0], lo[1], lo[2], lo[3]};
      } else {
        *(u32x4 *)&Hs[r * kHStride + cc] = hreg[p];
      }
    }
  };

  f32x4 acc[kVT][MT];
#pragma unroll
  for (int v = 0; v < kVT; ++v)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[v][mt] = f32x4{0.f, 0.f, 0.f, 0.f};

  bf16x8 wcur[kVT][kKC / 32], wnext[kVT][kKC / 32];
  load_h(0);
  load_w(wcur, 0);
  for (int c = 0; c < nchunks; ++c) {
    __syncthreads();
    store_h();
    __syncthreads();
    if (c + 1 < nchunks) {
      load_h(c + 1);
      load_w(wnext, c + 1);
    }
#pragma unroll
    for (int s = 0; s < kKC / 32; ++s) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const bf16x8 hf = *(const bf16x8 *)&Hs[(mt * 16 + l16) * kHStride + 32 * s + 8 * lg];
#pragma unroll
        for (int v = 0; v < kVT; ++v) acc[v][mt] = mfma16x16x32(wcur[v][s], hf, acc[v][mt]);
        if constexpr (SPLIT) {
          const bf16x8 hl =
              *(const bf16x8 *)&Hs[((MT + mt) * 16 + l16) * kHStride + 32 * s + 8 * lg];
#pragma unroll
          for (int v = 0; v < kVT; ++v) acc[v][mt] = mfma16x16x32(wcur[v][s], hl, acc[v][mt]);
        }
      }
    }
    if (c + 1 < nchunks) {
#pragma unroll
      for (int v = 0; v < kVT; ++v)
#pragma unroll
        for (int s = 0; s < kKC / 32; ++s) wcur[v][s] = wnext[v][s];
    }
  }

  // ---- epilogue: logits and per-tile softmax statistics
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int m = mbase + mt * 16 + l16;
    float vmax = -INFINITY;
#pragma unroll
    for (int v = 0; v < kVT; ++v) {
      const int n0 = vbase + (wv * kVT + v) * 16 + 4 * lg;
      if (m < a.M) {
        float *op = a.out + (int64_t)m * a.N + n0;
        if (n0 + 3 < a.N) {
          *(f32x4 *)op = acc[v][mt];
        } else {
          for (int j = 0; j < 4; ++j)
            if (n0 + j < a.N) op[j] = acc[v][mt][j];
        }
      }
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (n0 + j < a.N) vmax = fmaxf(vmax, acc[v][mt][j] * a.inv_t);
    }
    if (a.stats == nullptr) continue;
    vmax = fmaxf(vmax, __shfl_xor(vmax, 16));
    vmax = fmaxf(vmax, __shfl_xor(vmax, 32));
    float vs = 0.f;
#pragma unroll
    for (int v = 0; v < kVT; ++v) {
      const int n0 = vbase + (wv * kVT + v) * 16 + 4 * lg;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (n0 + j < a.N) vs += expf(acc[v][mt][j] * a.inv_t - vmax);
    }
    vs += __shfl_xor(vs, 16);
    vs += __shfl_xor(vs, 32);
    if (lg == 0) red[wv][mt * 16 + l16] = make_float2(vmax, vs);
  }
  if (a.stats == nullptr) return;
  __syncthreads();
  for (int r = tid; r < MT * 16; r += kThreads) {
    const int m = mbase + r;
    if (m >= a.M) continue;
    float mx = -INFINITY;
    for (int w2 = 0; w2 < 4; ++w2) mx = fmaxf(mx, red[w2][r].x);
    float sm = 0.f;
    for (int w2 = 0; w2 < 4; ++w2)
      if (red[w2][r].x != -INFINITY) sm += red[w2][r].y * expf(red[w2][r].x - mx);
    a.stats[(int64_t)vt * a.M + m] = make_float2(mx, sm);
  }
}

// fp32 GEMM on the vector ALU: out[m, n] = sum_k A[m,k] B[n,k]; optional tile stats
// over the same vocabulary tiles as the MFMA kernel.
__global__ void __launch_bounds__(kThreads)
gemm_f32_kernel(const float *A, const float *B, float *out, int M, int N, int K) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (int64_t)M * N) return;
  const int n = (int)(gid % N);
  const int m = (int)(gid / N);
  const float *ap = A + (int64_t)m * K;
  const float *bp = B + (int64_t)n * K;
  float s = 0.f;
  for (int k = 0; k < K; ++k) s = fmaf(ap[k], bp[k], s);
  out[gid] = s;
}

// Tile statistics from stored logits (used by the fp32 path).
__global__ void __launch_bounds__(kThreads)
tile_stats_kernel(const float *logits, float2 *stats, int M, int N, float inv_t) {
  const int vt = blockIdx.x;
  const int m = blockIdx.y;
  __shared__ float2 red[kThreads];
  const int n = vt * kVocabPerWG + threadIdx.x;
  const bool ok = threadIdx.x < kVocabPerWG && n < N;
  const float x = ok ? logits[(int64_t)m * N + n] * inv_t : -INFINITY;
  red[threadIdx.x] = make_float2(x, ok ? 1.f : 0.f);
  __syncthreads();
  if (threadIdx.x == 0) {
    float mx = -INFINITY;
    for (int i = 0; i < kVocabPerWG; ++i) mx = fmaxf(mx, red[i].x);
    float sm = 0.f;
    for (int i = 0; i < kVocabPerWG; ++i)
      if (red[i].y > 0.f) sm += expf(red[i].x - mx);
    stats[(int64_t)vt * M + m] = make_float2(mx, sm);
  }
}

// Row normaliser: lse[m] = max + log(sum_t s_t exp(m_t - max)) in fp64.
__global__ void __launch_bounds__(kThreads)
head_lse_kernel(const float2 *stats, double *row_lse, int M, int n_vtiles) {
  const int m = blockIdx.x;
  __shared__ double red[kThreads];
  double mx = -INFINITY;
  for (int t = threadIdx.x; t < n_vtiles; t += kThreads)
    mx = fmax(mx, (double)stats[(int64_t)t * M + m].x);
  red[threadIdx.x] = mx;
  __syncthreads();
  for (int off = kThreads / 2; off > 0; off >>= 1) {
    if (threadIdx.x < off) red[threadIdx.x] = fmax(red[threadIdx.x], red[threadIdx.x + off]);
    __syncthreads();
  }
  const double M0 = red[0];
  __syncthreads();
  double s = 0.0;
  for (int t = threadIdx.x; t < n_vtiles; t += kThreads) {
    const float2 st = stats[(int64_t)t * M + m];
    if (st.x != -INFINITY) s += (double)st.y * exp((double)st.x - M0);
  }
  red[threadIdx.x] = s;
  __syncthreads();
  for (int off = kThreads / 2; off > 0; off >>= 1) {
    if (threadIdx.x < off) red[threadIdx.x] += red[threadIdx.x + off];
    __syncthreads();
  }
  if (threadIdx.x == 0) row_lse[m] = M0 + log(red[0]);
}

__global__ void __launch_bounds__(kThreads)
head_probs_kernel(const float *logits, const double *row_lse, float *probs, int M, int N,
                  double inv_t) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (int64_t)M * N) return;
  const int m = (int)(gid / N);
  probs[gid] = (float)exp((double)logits[gid] * inv_t - row_lse[m]);
}

int pick_mt(int M, int *n_mblocks) {
  const int tiles = (M + 15) / 16;
  if (tiles <= 8) {
    *n_mblocks = 1;
    return tiles;
  }
  int best = 8, best_waste = 1 << 30;
  for (int mt = 8; mt >= 5; --mt) {
    const int nb = (tiles + mt - 1) / mt;
    const int waste = nb * mt - tiles;
    if (waste < best_waste) {
      best_waste = waste;
      best = mt;
    }
  }
  *n_mblocks = (tiles + best - 1) / best;
  return best;
}

hipError_t launch_gemm_bf16(const void *h, bool split, const bf16_t *w, float *out, float2 *stats,
                            int M, int N, int K, float inv_t, hipStream_t st) {
  GemmArgs a;
  a.h = h;
  a.w = w;
  a.out = out;
  a.stats = stats;
  a.M = M;
  a.N = N;
  a.K = K;
  a.inv_t = inv_t;
  const int mt = pick_mt(M, &a.n_mblocks);
  const int n_vtiles = (N + kVocabPerWG - 1) / kVocabPerWG;
  const dim3 grid(n_vtiles * a.n_mblocks);
#define VS_GEMM_CASE(MTV)                                                              \
  case MTV:                                                                            \
    if (split)                                                                         \
      hipLaunchKernelGGL((head_gemm_kernel<MTV, true>), grid, dim3(kThreads), 0, st, a); \
    else                                                                               \
      hipLaunchKernelGGL((head_gemm_kernel<MTV, false>), grid, dim3(kThreads), 0, st, a); \
    break;
  switch (mt) {
    VS_GEMM_CASE(1)
    VS_GEMM_CASE(2)
    VS_GEMM_CASE(3)
    VS_GEMM_CASE(4)
    VS_GEMM_CASE(5)
    VS_GEMM_CASE(6)
    VS_GEMM_CASE(7)
    VS_GEMM_CASE(8)
    default:
      return hipErrorInvalidValue;
  }
#undef VS_GEMM_CASE
  return hipGetLastError();
}

struct HeadWs {
  float2 *stats;
  float *t;  // low-rank intermediate [M, rank]
};

HeadWs head_ws(void *ws, int M, int V) {
  HeadWs w;
  const int n_vtiles = (V + kVocabPerWG - 1) / kVocabPerWG;
  w.stats = (float2 *)ws;
  size_t off = (size_t)n_vtiles * M * sizeof(float2);
  off = (off + 255) & ~(size_t)255;
  w.t = (float *)((char *)ws + off);
  return w;
}

}  // namespace

size_t head_workspace_bytes(int M, int d, int V, int rank, int dtype) {
  (void)d;
  (void)dtype;
  const int n_vtiles = (V + kVocabPerWG - 1) / kVocabPerWG;
  size_t off = (size_t)n_vtiles * M * sizeof(float2);
  off = (off + 255) & ~(size_t)255;
  return off + (size_t)M * (rank > 0 ? rank : 0) * sizeof(float) + 256;
}

hipError_t launch_head_gemm(int M, int d, int V, int rank, int dtype, float temperature,
                            const void *h, const void *w_full, const void *w_down,
                            const void *w_up, float *logits, void *ws, hipStream_t st) {
  const HeadWs w = head_ws(ws, M, V);
  const float inv_t = 1.0f / temperature;
  hipError_t e;
  if (dtype == 1) {
    if (rank == 0)
      return launch_gemm_bf16(h, false, (const bf16_t *)w_full, logits, w.stats, M, V, d, inv_t,
                              st);
    e = launch_gemm_bf16(h, false, (const bf16_t *)w_down, w.t, nullptr, M, rank, d, 1.f, st);
    if (e != hipSuccess) return e;
    return launch_gemm_bf16(w.t, true, (const bf16_t *)w_up, logits, w.stats, M, V, rank, inv_t,
                            st);
  }
  // fp32
  const float *A = (const float *)h;
  int K = d;
  if (rank > 0) {
    const int64_t n = (int64_t)M * rank;
    hipLaunchKernelGGL(gemm_f32_kernel, dim3((unsigned)((n + kThreads - 1) / kThreads)),
                       dim3(kThreads), 0, st, A, (const float *)w_down, w.t, M, rank, d);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    A = w.t;
    K = rank;
  }
  const float *Bm = (const float *)(rank > 0 ? w_up : w_full);
  const int64_t n = (int64_t)M * V;
  hipLaunchKernelGGL(gemm_f32_kernel, dim3((unsigned)((n + kThreads - 1) / kThreads)),
                     dim3(kThreads), 0, st, A, Bm, logits, M, V, K);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int n_vtiles = (V + kVocabPerWG - 1) / kVocabPerWG;
  hipLaunchKernelGGL(tile_stats_kernel, dim3(n_vtiles, M), dim3(kThreads), 0, st, logits,
                     w.stats, M, V, inv_t);
  return hipGetLastError();
}

hipError_t launch_head_finish(int M, int d, int V, int rank, int dtype, float temperature,
                              const float *logits, double *row_lse, float *probs, void *ws,
                              hipStream_t st) {
  (void)d;
  (void)rank;
  (void)dtype;
  const HeadWs w = head_ws(ws, M, V);
  const int n_vtiles = (V + kVocabPerWG - 1) / kVocabPerWG;
  hipLaunchKernelGGL(head_lse_kernel, dim3(M), dim3(kThreads), 0, st, w.stats, row_lse, M,
                     n_vtiles);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || probs == nullptr) return e;
  const int64_t n = (int64_t)M * V;
  hipLaunchKernelGGL(head_probs_kernel, dim3((unsigned)((n + kThreads - 1) / kThreads)),
                     dim3(kThreads), 0, st, logits, row_lse, probs, M, V,
                     1.0 / (double)temperature);
  return hipGetLastError();
}

}  // namespace vs
