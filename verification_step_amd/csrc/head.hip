// Vocabulary projection of the verify step.
//
// Full head: z = W_full h for every verify row -- the GEMM that batching the
// candidates turns the decode GEMV into (rejection-sampling blog, blog.huny.dev,
// section 1).  Low-rank head: z = W_up (W_down h) ("SlimSpec: Low-Rank Draft
// LM-Head ...", gist.science, "방법론 / 아키텍처"), the rank-r intermediate kept in fp32.
//
// bf16 GEMM out[M,N] = H[M,K] . W[N,K]^T on MFMA 16x16x32 bf16, fp32 accumulation.
// For the verify head (M = W*D rows, N = V >= 1e5) the product is bound by reading
// W once from HBM, so the kernel is built around keeping enough of W in flight:
//   * bf16 weights are prepacked once (vs_pack_weight) into MFMA operand tiles:
//     16 rows x 32 columns = 1 KB, lane l's 16 bytes at offset 16*l, tiles of one
//     16-row strip consecutive along K.  A wave's load of one tile is a single
//     contiguous 1 KB access and each strip streams sequentially through memory;
//   * a workgroup = 4 waves x 64 vocabulary rows; each wave streams its own strips
//     of W and the H fragments straight into registers, through a ring of register
//     buffers issued several K-steps ahead (W and H at the same distance, so the
//     in-order load counter never makes a wave wait for data it does not need yet);
//   * no LDS and no barrier in the K loop: waves progress independently; H (a few
//     hundred KB) stays in L2;
//   * fp32 H (the low-rank intermediate) is split on the fly into bf16 hi + lo and
//     multiplied twice (about 16 significant bits);
//   * the epilogue writes fp32 logits and, per row and 256-row vocabulary tile,
//     (max, sum exp(z/T - max)); the same tiles' statistics of the root logits
//     can be folded in, so the sampler's normalisers need no pass over the logits.
// Low-rank stage W_down (N = r = 512, K = d) splits K across workgroups and sums
// the partials in a fixed order.

#include "vs_internal.hpp"

#include <stdlib.h>
#include <type_traits>

namespace vs {

namespace {

constexpr int kThreads = 256;
constexpr int kVT = 4;             // 16-row vocabulary tiles per wave
constexpr int kPD = 2;             // K-steps (of 32) loaded ahead of use
constexpr int kRing = kPD + 1;
static_assert(kHeadVocabTile == 4 * kVT * 16, "workgroup vocabulary span");

typedef __attribute__((__vector_size__(8 * sizeof(float)))) float f32x8;

struct GemmArgs {
  const void *h;        // [M, K] bf16, or fp32 when SPLIT
  const bf16_t *w;      // packed [ceil(N/16)][K/32][64][8]
  float *out;           // [M, N] (or partial [ksplit][M][N])
  float2 *stats;        // [M][n_vt] or null
  const float *root;    // [B_root, N] or null
  float2 *root_stats;   // [B_root][n_vt]
  int M, N, K, B_root;
  int n_mblocks;
  int kspan;            // K per split (multiple of 32)
  float inv_t;
};

template <int MT, bool SPLIT>
__global__ void __launch_bounds__(kThreads)
head_stream_kernel(GemmArgs a) {
  __shared__ float2 red[4][MT * 16];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int l16 = lane & 15;
  const int lg = lane >> 4;
  const int n_vt = (a.N + kHeadVocabTile - 1) / kHeadVocabTile;
  const int nblocks = n_vt * a.n_mblocks;
  const int bid = xcd_remap(blockIdx.x, nblocks);
  const int mb = bid % a.n_mblocks;
  const int vt = bid / a.n_mblocks;
  const int ks = blockIdx.y;
  const int vbase = vt * kHeadVocabTile + wv * (kVT * 16);
  const int mbase = mb * MT * 16;
  const int k0 = ks * a.kspan;
  const int k1 = min(a.K, k0 + a.kspan);
  const int nsteps = (k1 - k0) / 32;

  // packed W: strip (16 rows) t, K-step s at element ((t * ksteps + s) * 64 + lane) * 8
  const int ksteps_all = a.K / 32;
  const int n_strips = (a.N + 15) / 16;
  const bf16_t *wp[kVT];
#pragma unroll
  for (int v = 0; v < kVT; ++v) {
    int t = vbase / 16 + v;
    t = t < n_strips ? t : n_strips - 1;
    wp[v] = a.w + (((int64_t)t * ksteps_all + k0 / 32) * 64 + lane) * 8;
  }
  using HElem = typename std::conditional<SPLIT, f32x8, bf16x8>::type;
  const HElem *hp[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    int m = mbase + mt * 16 + l16;
    m = m < a.M ? m : a.M - 1;
    if constexpr (SPLIT)
      hp[mt] = (const HElem *)((const float *)a.h + (int64_t)m * a.K + k0 + 8 * lg);
    else
      hp[mt] = (const HElem *)((const bf16_t *)a.h + (int64_t)m * a.K + k0 + 8 * lg);
  }

  bf16x8 wr[kRing][kVT];
  HElem hr[kRing][MT];
  auto load = [&](int slot, int s) {
#pragma unroll
    for (int v = 0; v < kVT; ++v) wr[slot][v] = *(const bf16x8 *)(wp[v] + 512 * s);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      if constexpr (SPLIT)
        hr[slot][mt] = *(const HElem *)((const float *)hp[mt] + 32 * s);
      else
        hr[slot][mt] = *(const HElem *)((const bf16_t *)hp[mt] + 32 * s);
    }
  };

  f32x4 acc[kVT][MT];
#pragma unroll
  for (int v = 0; v < kVT; ++v)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[v][mt] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int slot) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      if constexpr (SPLIT) {
        const f32x8 x = hr[slot][mt];
        uint32_t hk[4], lk[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) split_bf16x2(x[2 * e], x[2 * e + 1], hk[e], lk[e]);
        const bf16x8 hi = __builtin_bit_cast(bf16x8, *(const u32x4 *)hk);
        const bf16x8 lo = __builtin_bit_cast(bf16x8, *(const u32x4 *)lk);
#pragma unroll
        for (int v = 0; v < kVT; ++v) {
          acc[v][mt] = mfma16x16x32(wr[slot][v], hi, acc[v][mt]);
          acc[v][mt] = mfma16x16x32(wr[slot][v], lo, acc[v][mt]);
        }
      } else {
#pragma unroll
        for (int v = 0; v < kVT; ++v) acc[v][mt] = mfma16x16x32(wr[slot][v], hr[slot][mt], acc[v][mt]);
      }
    }
  };

#pragma unroll
  for (int p = 0; p < kPD; ++p)
    if (p < nsteps) load(p, p);
  for (int s = 0; s < nsteps; s += kRing) {
#pragma unroll
    for (int u = 0; u < kRing; ++u) {
      const int ss = s + u;
      if (ss + kPD < nsteps) load((u + kPD) % kRing, ss + kPD);
      if (ss < nsteps) compute(u);
    }
  }

  float *out = a.out + (int64_t)ks * a.M * a.N;
  // ---- epilogue: logits (+ tile statistics)
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int m = mbase + mt * 16 + l16;
    float vmax = -INFINITY;
#pragma unroll
    for (int v = 0; v < kVT; ++v) {
      const int n0 = vbase + v * 16 + 4 * lg;
      if (m < a.M) {
        float *op = out + (int64_t)m * a.N + n0;
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
      const int n0 = vbase + v * 16 + 4 * lg;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (n0 + j < a.N) vs += expf(acc[v][mt][j] * a.inv_t - vmax);
    }
    vs += __shfl_xor(vs, 16);
    vs += __shfl_xor(vs, 32);
    if (lg == 0) red[wv][mt * 16 + l16] = make_float2(vmax, vs);
  }
  if (a.stats == nullptr) return;

  // root rows over this workgroup's vocabulary tile (one wave per row)
  if (a.root != nullptr && mb == 0) {
    for (int b = wv; b < a.B_root; b += 4) {
      const float *row = a.root + (int64_t)b * a.N;
      float x[kHeadVocabTile / 64];
      float mx = -INFINITY;
#pragma unroll
      for (int j = 0; j < kHeadVocabTile / 64; ++j) {
        const int k = vt * kHeadVocabTile + j * 64 + lane;
        x[j] = (k < a.N) ? row[k] * a.inv_t : -INFINITY;
        mx = fmaxf(mx, x[j]);
      }
      for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
      float sm = 0.f;
#pragma unroll
      for (int j = 0; j < kHeadVocabTile / 64; ++j)
        if (x[j] != -INFINITY) sm += expf(x[j] - mx);
      for (int off = 32; off > 0; off >>= 1) sm += __shfl_xor(sm, off);
      if (lane == 0) a.root_stats[(int64_t)b * n_vt + vt] = make_float2(mx, sm);
    }
  }
  __syncthreads();
  for (int r = tid; r < MT * 16; r += kThreads) {
    const int m = mbase + r;
    if (m >= a.M) continue;
    float mx = -INFINITY;
    for (int w2 = 0; w2 < 4; ++w2) mx = fmaxf(mx, red[w2][r].x);
    float sm = 0.f;
    for (int w2 = 0; w2 < 4; ++w2)
      if (red[w2][r].x != -INFINITY) sm += red[w2][r].y * expf(red[w2][r].x - mx);
    a.stats[(int64_t)m * n_vt + vt] = make_float2(mx, sm);
  }
}

// Head GEMM with H shared through LDS (bf16 H, K % 128 == 0): the workgroup stages
// H in chunks of 128 columns with direct global->LDS transfers (double-buffered,
// 16-byte chunk c of row r at position c ^ (r & 15): conflict-free fragment reads),
// while each wave keeps streaming its packed W strips through its register ring.
constexpr int kHC = 128;                 // H columns per LDS chunk (4 K-steps)
typedef __attribute__((address_space(3))) void lds_void_t;

__device__ __forceinline__ void dma16_h(const void *g, bf16_t *lds_dst) {
  // opaque to the compiler's wait insertion (which would drain every transfer before
  // any LDS read); completion is waited for explicitly before the publishing barrier
  const uint32_t lds = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void_t *)lds_dst);
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(g), "s"(lds)
               : "memory", "m0");
}

// A workgroup of 4*NG waves shares one staging of H.  Each wave streams VT 16-row
// strips of W: with VT = 4 a vocabulary tile (256 rows of W) takes 4 waves and the
// workgroup holds NG tiles; with VT = 2 it takes 8 waves, which halves the register
// tile per row so that up to 12 row tiles (192 rows) fit in one row block and each
// strip of W is streamed once instead of once per row block.
template <int MT, int NG, int VT = kVT>
__global__ void __launch_bounds__(kThreads * NG, 2)
head_lds_kernel(GemmArgs a) {
  constexpr int kWPT = kHeadVocabTile / (VT * 16);   // waves per vocabulary tile
  constexpr int kTPW = 4 * NG / kWPT;                 // vocabulary tiles per workgroup
  static_assert(kTPW >= 1 && kTPW * kWPT == 4 * NG, "waves split evenly over tiles");
  // the H double buffer; after the K loop the same LDS stages each wave's logits tile
  // (16 rows x 16 VT columns, rows padded to kStRow floats) for whole-segment stores
  constexpr int kHsBuf = MT * 16 * kHC;
  constexpr int kStRow = 68;
  constexpr int kStageF = 4 * NG * 16 * kStRow;
  constexpr int kHsAll = (4 * kHsBuf >= 4 * kStageF) ? 2 * kHsBuf : 2 * kStageF;
  __shared__ __attribute__((aligned(1024))) bf16_t Hs_all[kHsAll];
  bf16_t(*Hs)[kHsBuf] = reinterpret_cast<bf16_t(*)[kHsBuf]>(Hs_all);
  __shared__ float2 red[4 * NG][MT * 16];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int grp = wv / kWPT;        // vocabulary tile of this wave within the workgroup
  const int wq = wv % kWPT;         // wave within the tile
  const int l16 = lane & 15;
  const int lg = lane >> 4;
  const int n_vt = (a.N + kHeadVocabTile - 1) / kHeadVocabTile;
  const int nblocks = ((n_vt + kTPW - 1) / kTPW) * a.n_mblocks;
  const int bid = xcd_remap(blockIdx.x, nblocks);
  const int mb = bid % a.n_mblocks;
  const int vt = (bid / a.n_mblocks) * kTPW + grp;
  const bool tile_ok = vt < n_vt;
  const int vbase = vt * kHeadVocabTile + wq * (VT * 16);
  const int mbase = mb * MT * 16;
  const int nsteps = a.K / 32;
  const int nchunks = a.K / kHC;

  const int n_strips = (a.N + 15) / 16;
  const bf16_t *wp[VT];
#pragma unroll
  for (int v = 0; v < VT; ++v) {
    int t = vbase / 16 + v;
    t = t < n_strips ? t : n_strips - 1;
    wp[v] = a.w + ((int64_t)t * nsteps * 64 + lane) * 8;
  }
  constexpr int kPDL = 3, kRingL = kPDL + 1;   // W steps in flight; one ring turn per chunk
  bf16x8 wr[kRingL][VT];
  auto load_w = [&](int slot, int s) {
#pragma unroll
    for (int v = 0; v < VT; ++v) wr[slot][v] = *(const bf16x8 *)(wp[v] + 512 * s);
  };
  // H chunk c: MT*16 rows x 128 columns = MT*4 transfers of 1 KB (4 rows each); wave
  // wv issues transfers wv, wv+4*NG, ...
  // (32-bit element offsets of each transfer, computed once: H has M*K < 2^31 elements)
  const bf16_t *hbase = (const bf16_t *)a.h;
  constexpr int kHT = (MT + NG - 1) / NG;   // transfers per wave per chunk
  uint32_t hofs[kHT];
#pragma unroll
  for (int ii = 0; ii < kHT; ++ii) {
    const int row = 4 * (wv + 4 * NG * ii) + (lane >> 4);
    const int ch = (lane & 15) ^ (row & 15);
    int m = mbase + row;
    m = m < a.M ? m : a.M - 1;
    hofs[ii] = (uint32_t)m * (uint32_t)a.K + 8 * ch;
  }
  auto issue_h = [&](int c, int buf) {
#pragma unroll
    for (int ii = 0; ii < kHT; ++ii) {
      const int i = wv + 4 * NG * ii;
      if (i >= MT * 4) break;
      dma16_h(hbase + hofs[ii] + c * kHC, &Hs[buf][i * 512]);
    }
  };

  f32x4 acc[VT][MT];
#pragma unroll
  for (int v = 0; v < VT; ++v)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[v][mt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // the root row this wave folds into the tile statistics, loaded before the K loop (at
  // most one root row per wave, and only where the accumulators leave registers free):
  // the epilogue then waits on no load
  constexpr bool kRootPre = MT * VT <= 24;
  const bool root_pre = kRootPre && a.root != nullptr && mb == 0 && tile_ok && a.B_root <= kWPT;
  float rx[kHeadVocabTile / 64];
#pragma unroll
  for (int j = 0; j < kHeadVocabTile / 64; ++j) {
    const int k = vt * kHeadVocabTile + j * 64 + lane;
    rx[j] = (root_pre && wq < a.B_root && k < a.N) ? a.root[(int64_t)wq * a.N + k] * a.inv_t : -INFINITY;
  }

  issue_h(0, 0);
#pragma unroll
  for (int p = 0; p < kPDL; ++p) load_w(p, p);
  __builtin_amdgcn_s_waitcnt(0);      // H chunk 0 (and the first W steps) have landed
  __syncthreads();
  for (int c = 0; c < nchunks; ++c) {
    const int buf = c & 1;
    if (c + 1 < nchunks) issue_h(c + 1, buf ^ 1);
#pragma unroll
    for (int u = 0; u < kHC / 32; ++u) {
      const int ss = c * (kHC / 32) + u;
      // ring slot of step ss is ss % kRingL; kHC/32 == kRingL keeps it static
      if (ss + kPDL < nsteps) load_w((u + kPDL) % kRingL, ss + kPDL);
      // all of this step's H fragments are read first, then the products: one LDS
      // latency per step instead of one per pair of row tiles
      bf16x8 hf[MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int row = mt * 16 + l16;
        const int pch = (4 * u + lg) ^ (row & 15);
        hf[mt] = *(const bf16x8 *)&Hs[buf][row * kHC + 8 * pch];
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int v = 0; v < VT; ++v) acc[v][mt] = mfma16x16x32(wr[u][v], hf[mt], acc[v][mt]);
      __builtin_amdgcn_sched_group_barrier(0x100, MT, 0);       // the LDS reads
      __builtin_amdgcn_sched_group_barrier(0x008, MT * VT, 0);  // then the products
    }
    if (c + 1 < nchunks) {
      // everything up to this chunk's H transfers: only the W loads issued after them
      // (kHC/32 steps x VT) may still be in flight
      __builtin_amdgcn_s_waitcnt(0x0F70 | ((kHC / 32) * VT & 15) | ((((kHC / 32) * VT) >> 4) << 14));
      __syncthreads();
    }
  }
  static_assert(kHC / 32 == kRingL, "one ring turn per H chunk");

  // ---- epilogue: logits + tile statistics.  With one or two row blocks (the weight
  // stream dominates) each row tile goes through LDS: a wave writes its 16 x (16 VT)
  // fragment, then stores it as whole rows of 64 VT contiguous bytes (4 rows per
  // instruction at VT = 4, 8 at VT = 2) -- whole cache lines, written non-temporally
  // (the sampler reads one of these rows back, later).  With more row blocks
  // (matrix-bound shapes) the fragments are stored directly.
  const bool staged = a.n_mblocks <= 2;
  float *stg = reinterpret_cast<float *>(Hs_all) + wv * 16 * kStRow;
  if (staged) __syncthreads();   // every wave is done reading H
  // WHOLE: the workgroup's rows and vocabulary columns all lie inside M x N (every
  // tile but the last vocabulary tile and the last row block), so no bounds are tested
  auto epilogue = [&](auto whole_tag) {
    constexpr bool WHOLE = decltype(whole_tag)::value;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      float vmax = -INFINITY;
#pragma unroll
      for (int v = 0; v < VT; ++v) {
        const int n0 = vbase + v * 16 + 4 * lg;
        if (staged) {
          *(f32x4 *)&stg[l16 * kStRow + v * 16 + 4 * lg] = acc[v][mt];
        } else {
          const int m = mbase + mt * 16 + l16;
          if (WHOLE || m < a.M) {
            float *op = a.out + (int64_t)m * a.N + n0;
            if (WHOLE || n0 + 3 < a.N) {
              *(f32x4 *)op = acc[v][mt];
            } else {
              for (int j = 0; j < 4; ++j)
                if (n0 + j < a.N) op[j] = acc[v][mt][j];
            }
          }
        }
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (WHOLE || n0 + j < a.N) vmax = fmaxf(vmax, acc[v][mt][j] * a.inv_t);
      }
      if (staged) {
        // each wave reads back only its own fragment: a wave-level sync suffices
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        constexpr int kLPR = 4 * VT;     // lanes per fragment row, 4 floats each
        constexpr int kRPI = 64 / kLPR;  // fragment rows per store instruction
#pragma unroll
        for (int i = 0; i < 16 / kRPI; ++i) {
          const int r = kRPI * i + lane / kLPR;
          const int c = 4 * (lane % kLPR);
          const int m = mbase + mt * 16 + r;
          const int n = vbase + c;
          if (WHOLE || (m < a.M && n < a.N)) {
            const f32x4 val = *(const f32x4 *)&stg[r * kStRow + c];
            float *op = a.out + (int64_t)m * a.N + n;
            if (WHOLE || (n + 3 < a.N && ((a.N & 3) == 0))) {
              __builtin_nontemporal_store(val, (f32x4 *)op);
            } else {
              for (int j = 0; j < 4; ++j)
                if (n + j < a.N) op[j] = val[j];
            }
          }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      }
      if (a.stats == nullptr) continue;
      vmax = fmaxf(vmax, __shfl_xor(vmax, 16));
      vmax = fmaxf(vmax, __shfl_xor(vmax, 32));
      float vs = 0.f;
#pragma unroll
      for (int v = 0; v < VT; ++v) {
        const int n0 = vbase + v * 16 + 4 * lg;
#pragma unroll
        for (int j = 0; j < 4; ++j)
          // the hardware exp2 of the log2(e)-scaled difference (one instruction where
          // expf takes a range-reduction sequence); within an ulp or two, far inside
          // the normaliser's tolerance
          if (WHOLE || n0 + j < a.N)
            vs += __builtin_amdgcn_exp2f((acc[v][mt][j] * a.inv_t - vmax) * 1.4426950408889634f);
      }
      vs += __shfl_xor(vs, 16);
      vs += __shfl_xor(vs, 32);
      if (lg == 0) red[wv][mt * 16 + l16] = make_float2(vmax, vs);
    }
  };
  // (a.N & 3) == 0 keeps the whole-tile stores 16-byte aligned
  const bool whole = mbase + MT * 16 <= a.M && (vt + 1) * kHeadVocabTile <= a.N && (a.N & 3) == 0;
  if (whole)
    epilogue(std::true_type{});
  else
    epilogue(std::false_type{});
  if (a.stats == nullptr) return;
  if (a.root != nullptr && mb == 0 && tile_ok) {
    for (int b = wq; b < a.B_root; b += kWPT) {
      const float *row = a.root + (int64_t)b * a.N;
      float x[kHeadVocabTile / 64];
      float mx = -INFINITY;
#pragma unroll
      for (int j = 0; j < kHeadVocabTile / 64; ++j) {
        const int k = vt * kHeadVocabTile + j * 64 + lane;
        x[j] = root_pre ? rx[j] : ((k < a.N) ? row[k] * a.inv_t : -INFINITY);
        mx = fmaxf(mx, x[j]);
      }
      for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
      float sm = 0.f;
#pragma unroll
      for (int j = 0; j < kHeadVocabTile / 64; ++j)
        if (x[j] != -INFINITY) sm += expf(x[j] - mx);
      for (int off = 32; off > 0; off >>= 1) sm += __shfl_xor(sm, off);
      if (lane == 0) a.root_stats[(int64_t)b * n_vt + vt] = make_float2(mx, sm);
    }
  }
  __syncthreads();
  if (!tile_ok) return;
  constexpr int kTT = 64 * kWPT;   // threads of one vocabulary tile (its waves)
  for (int r = tid % kTT; r < MT * 16; r += kTT) {
    const int m = mbase + r;
    if (m >= a.M) continue;
    const float2 *rw = &red[kWPT * grp][r];
    float mx = -INFINITY;
    for (int w2 = 0; w2 < kWPT; ++w2) mx = fmaxf(mx, rw[w2 * MT * 16].x);
    float sm = 0.f;
    for (int w2 = 0; w2 < kWPT; ++w2)
      if (rw[w2 * MT * 16].x != -INFINITY)
        sm += rw[w2 * MT * 16].y * expf(rw[w2 * MT * 16].x - mx);
    a.stats[(int64_t)m * n_vt + vt] = make_float2(mx, sm);
  }
}

// Row-major [N, K] bf16 -> MFMA operand tiles [ceil(N/16)][K/32][64 lanes][8]; rows
// past N are zero.  Pure data movement: one thread per 16-byte lane slot.
__global__ void __launch_bounds__(kThreads)
pack_weight_kernel(const bf16_t *src, bf16_t *dst, int N, int K) {
  const int64_t slot = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int64_t ks = K / 32;
  const int64_t n_slots = (int64_t)((N + 15) / 16) * ks * 64;
  if (slot >= n_slots) return;
  const int lane = (int)(slot % 64);
  const int64_t tile = slot / 64;
  const int64_t s = tile % ks;
  const int64_t t = tile / ks;
  const int64_t n = t * 16 + (lane & 15);
  const int64_t k = s * 32 + 8 * (lane >> 4);
  u32x4 v = {0u, 0u, 0u, 0u};
  if (n < N) v = *(const u32x4 *)(src + n * K + k);
  *(u32x4 *)(dst + slot * 8) = v;
}

// sum of K-split partials [ks][n] in split order; the loads of 16 splits are issued
// together so that one thread does not wait out ksplit memory latencies in a row
__global__ void __launch_bounds__(kThreads)
sum_splits_kernel(const float *part, int ksplit, int64_t n, float *out) {
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i >= n) return;
  float s = 0.f;
  int k = 0;
  for (; k + 16 <= ksplit; k += 16) {
    float x[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) x[j] = part[(int64_t)(k + j) * n + i];
#pragma unroll
    for (int j = 0; j < 16; ++j) s += x[j];
  }
  for (; k < ksplit; ++k) s += part[(int64_t)k * n + i];
  out[i] = s;
}

// fp32 GEMM on the vector ALU: out[m, n] = sum_k A[m,k] B[n,k]
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

// fp32 head in one launch: a workgroup takes one 256-wide vocabulary tile (one column
// per thread) for kF32Rows rows of H, staged through LDS in chunks of kF32KC columns.
// Each logit is a k-ordered fmaf chain; then the tile statistics of those rows (max,
// then sum exp(x - max), by wave shuffles and one LDS slot per wave), and, in row
// block 0, the same statistics of the root rows (one wave per row, four ids per lane).
constexpr int kF32Rows = 8;
constexpr int kF32KC = 256;

__global__ void __launch_bounds__(kThreads)
head_f32_kernel(const float *H, const float *W, float *out, float2 *stats, const float *root,
                float2 *root_stats, int M, int N, int K, int B_root, float inv_t) {
  static_assert(kThreads == 256 && kHeadVocabTile == 256, "one column per thread");
  __shared__ float hs[kF32Rows][kF32KC];
  __shared__ float wmax[kF32Rows][4], wsum[kF32Rows][4];
  const int vt = blockIdx.x;
  const int n_vt = gridDim.x;
  const int m0 = blockIdx.y * kF32Rows;
  const int tid = threadIdx.x;
  const int wv = tid >> 6;
  const int lane = tid & 63;
  const int n = vt * kHeadVocabTile + tid;
  const bool ok = n < N;
  const float *wrow = W + (int64_t)(ok ? n : N - 1) * K;
  const bool vec = ((K & 3) == 0) && ((reinterpret_cast<uintptr_t>(W) & 15) == 0);

  float acc[kF32Rows];
#pragma unroll
  for (int r = 0; r < kF32Rows; ++r) acc[r] = 0.f;
  for (int k0 = 0; k0 < K; k0 += kF32KC) {
    const int kc = min(kF32KC, K - k0);
    // the chunk's first 64 columns of the W row, issued before the H staging so that
    // the two loads overlap
    float4 w4[16];
    if (vec && kc >= 64) {
#pragma unroll
      for (int q = 0; q < 16; ++q) w4[q] = *reinterpret_cast<const float4 *>(wrow + k0 + 4 * q);
    }
    __syncthreads();   // the previous chunk has been consumed
    constexpr int kPerT = kF32Rows * kF32KC / kThreads;
    float hv[kPerT];
#pragma unroll
    for (int it = 0; it < kPerT; ++it) {   // all loads first, then the LDS writes
      const int r = (tid + it * kThreads) / kF32KC, k = (tid + it * kThreads) % kF32KC;
      hv[it] = (m0 + r < M && k < kc) ? H[(int64_t)(m0 + r) * K + k0 + k] : 0.f;
    }
#pragma unroll
    for (int it = 0; it < kPerT; ++it)
      hs[(tid + it * kThreads) / kF32KC][(tid + it * kThreads) % kF32KC] = hv[it];
    __syncthreads();
    int k = 0;
    if (vec) {
      // 64 columns of the W row in flight at once, then their products in k order
      for (; k + 64 <= kc; k += 64) {
        if (k > 0) {
#pragma unroll
          for (int q = 0; q < 16; ++q) w4[q] = *reinterpret_cast<const float4 *>(wrow + k0 + k + 4 * q);
        }
        __builtin_amdgcn_sched_barrier(0);   // keep the 16 loads ahead of their uses
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const float wk[4] = {w4[q].x, w4[q].y, w4[q].z, w4[q].w};
#pragma unroll
          for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < kF32Rows; ++r) acc[r] = fmaf(hs[r][k + 4 * q + j], wk[j], acc[r]);
        }
      }
      for (; k + 4 <= kc; k += 4) {
        const float4 w4 = *reinterpret_cast<const float4 *>(wrow + k0 + k);
        const float wk[4] = {w4.x, w4.y, w4.z, w4.w};
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int r = 0; r < kF32Rows; ++r) acc[r] = fmaf(hs[r][k + j], wk[j], acc[r]);
      }
    }
#pragma unroll 8
    for (; k < kc; ++k) {
      const float w = wrow[k0 + k];
#pragma unroll
      for (int r = 0; r < kF32Rows; ++r) acc[r] = fmaf(hs[r][k], w, acc[r]);
    }
  }
#pragma unroll
  for (int r = 0; r < kF32Rows; ++r)
    if (ok && m0 + r < M) out[(int64_t)(m0 + r) * N + n] = acc[r];

  if (stats != nullptr) {
    float x[kF32Rows];
#pragma unroll
    for (int r = 0; r < kF32Rows; ++r) {
      x[r] = ok ? acc[r] * inv_t : -INFINITY;
      float v = x[r];
      for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
      if (lane == 0) wmax[r][wv] = v;
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < kF32Rows; ++r) {
      const float mx = fmaxf(fmaxf(wmax[r][0], wmax[r][1]), fmaxf(wmax[r][2], wmax[r][3]));
      float e = ok ? expf(x[r] - mx) : 0.f;
      for (int o = 32; o > 0; o >>= 1) e += __shfl_xor(e, o);
      if (lane == 0) wsum[r][wv] = e;
    }
    __syncthreads();
    if (tid < kF32Rows && m0 + tid < M) {
      const float mx = fmaxf(fmaxf(wmax[tid][0], wmax[tid][1]), fmaxf(wmax[tid][2], wmax[tid][3]));
      stats[(int64_t)(m0 + tid) * n_vt + vt] =
          make_float2(mx, (wsum[tid][0] + wsum[tid][1]) + (wsum[tid][2] + wsum[tid][3]));
    }
  }
  if (root == nullptr || root_stats == nullptr || blockIdx.y != 0) return;
  for (int b = wv; b < B_root; b += 4) {
    const float *row = root + (int64_t)b * N;
    float x[kHeadVocabTile / 64];
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < kHeadVocabTile / 64; ++j) {
      const int k = vt * kHeadVocabTile + j * 64 + lane;
      x[j] = (k < N) ? row[k] * inv_t : -INFINITY;
      mx = fmaxf(mx, x[j]);
    }
    for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
    float sm = 0.f;
#pragma unroll
    for (int j = 0; j < kHeadVocabTile / 64; ++j)
      if (x[j] != -INFINITY) sm += expf(x[j] - mx);
    for (int off = 32; off > 0; off >>= 1) sm += __shfl_xor(sm, off);
    if (lane == 0) root_stats[(int64_t)b * n_vt + vt] = make_float2(mx, sm);
  }
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

constexpr int kLowrankSplit = 64;

hipError_t launch_stream(GemmArgs a, bool split, int ksplit, hipStream_t st) {
  const int mt = pick_mt(a.M, &a.n_mblocks);
  const int n_vt = (a.N + kHeadVocabTile - 1) / kHeadVocabTile;
  const dim3 grid(n_vt * a.n_mblocks, ksplit);
  // the LDS-staged kernels address H with 32-bit element offsets
  const bool h32 = (int64_t)a.M * a.K <= (int64_t)INT32_MAX;
  if (!split && ksplit == 1 && a.K % kHC == 0 && h32 && getenv("VSTEP_HEAD_STREAM") == nullptr) {
    // two vocabulary tiles per workgroup (one workgroup per CU): H is staged once per
    // CU instead of twice, which measured faster at every M tried (7, 32, 80)
    const char *ngv = getenv("VSTEP_HEAD_NG");
    const int ng = ngv ? atoi(ngv) : 2;
    // 9..12 row tiles: one row block of 8 waves x 2 strips per vocabulary tile, so W is
    // streamed once (two row blocks of 4 strips per wave would each stream it)
    const int tiles = (a.M + 15) / 16;
    const char *tallv = getenv("VSTEP_HEAD_TALL");
    if (ng == 2 && tiles > 8 && tiles <= 12 && !(tallv && atoi(tallv) == 0)) {
      a.n_mblocks = 1;
      switch (tiles) {
        case 9: hipLaunchKernelGGL((head_lds_kernel<9, 2, 2>), dim3(n_vt), dim3(2 * kThreads), 0, st, a); break;
        case 10: hipLaunchKernelGGL((head_lds_kernel<10, 2, 2>), dim3(n_vt), dim3(2 * kThreads), 0, st, a); break;
        case 11: hipLaunchKernelGGL((head_lds_kernel<11, 2, 2>), dim3(n_vt), dim3(2 * kThreads), 0, st, a); break;
        default: hipLaunchKernelGGL((head_lds_kernel<12, 2, 2>), dim3(n_vt), dim3(2 * kThreads), 0, st, a); break;
      }
      return hipGetLastError();
    }
#define VS_LDS_CASE(MTV)                                                                  \
  case MTV:                                                                               \
    if (ng == 2)                                                                          \
      hipLaunchKernelGGL((head_lds_kernel<MTV, 2>), dim3(((n_vt + 1) / 2) * a.n_mblocks),    \
                         dim3(2 * kThreads), 0, st, a);                                   \
    else                                                                                  \
      hipLaunchKernelGGL((head_lds_kernel<MTV, 1>), grid, dim3(kThreads), 0, st, a);      \
    break;
    switch (mt) {
      VS_LDS_CASE(1)
      VS_LDS_CASE(2)
      VS_LDS_CASE(3)
      VS_LDS_CASE(4)
      VS_LDS_CASE(5)
      VS_LDS_CASE(6)
      VS_LDS_CASE(7)
      VS_LDS_CASE(8)
      default:
        return hipErrorInvalidValue;
    }
#undef VS_LDS_CASE
    return hipGetLastError();
  }
#define VS_GEMM_CASE(MTV)                                                                   \
  case MTV:                                                                                 \
    if (split)                                                                              \
      hipLaunchKernelGGL((head_stream_kernel<MTV, true>), grid, dim3(kThreads), 0, st, a);  \
    else                                                                                    \
      hipLaunchKernelGGL((head_stream_kernel<MTV, false>), grid, dim3(kThreads), 0, st, a); \
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

}  // namespace

size_t packed_weight_elems(int N, int K) { return (size_t)((N + 15) / 16) * 16 * K; }

hipError_t launch_pack_weight(const void *src, void *dst, int N, int K, hipStream_t st) {
  const int64_t n_slots = (int64_t)((N + 15) / 16) * (K / 32) * 64;
  hipLaunchKernelGGL(pack_weight_kernel, dim3((unsigned)((n_slots + kThreads - 1) / kThreads)),
                     dim3(kThreads), 0, st, (const bf16_t *)src, (bf16_t *)dst, N, K);
  return hipGetLastError();
}

HeadWs head_ws(void *ws, int M, int V, int rank) {
  HeadWs w;
  const int n_vt = (V + kHeadVocabTile - 1) / kHeadVocabTile;
  char *p = (char *)ws;
  size_t off = 0;
  w.stats = (float2 *)(p + off);
  off += ((size_t)M * n_vt * sizeof(float2) + 255) & ~(size_t)255;
  w.t = (float *)(p + off);
  if (rank > 0) off += ((size_t)(kLowrankSplit + 1) * M * rank * sizeof(float) + 255) & ~(size_t)255;
  w.bytes = off;
  return w;
}

size_t head_workspace_bytes(int M, int d, int V, int rank, int dtype) {
  (void)d;
  (void)dtype;
  return head_ws(nullptr, M, V, rank).bytes;
}

hipError_t launch_head_gemm(int M, int d, int V, int rank, int dtype, float temperature,
                            const void *h, const void *w_full, const void *w_down,
                            const void *w_up, float *logits, const HeadWs &ws,
                            const float *root_logits, int B_root, float2 *root_stats,
                            hipStream_t st) {
  const float inv_t = 1.0f / temperature;
  hipError_t e;
  if (dtype == 1) {
    GemmArgs a{};
    a.inv_t = inv_t;
    a.root = root_logits;
    a.root_stats = root_stats;
    a.B_root = B_root;
    if (rank > 0) {
      // t = H W_down^T, K split over workgroups, partials summed in split order
      float *part = ws.t + (size_t)M * rank;
      const int kspan = ((d / kLowrankSplit + 31) / 32) * 32;
      const int ksplit = (d + kspan - 1) / kspan;
      a.h = h;
      a.w = (const bf16_t *)w_down;
      a.out = part;
      a.stats = nullptr;
      a.root = nullptr;
      a.M = M;
      a.N = rank;
      a.K = d;
      a.kspan = kspan;
      if ((e = launch_stream(a, false, ksplit, st)) != hipSuccess) return e;
      const int64_t n = (int64_t)M * rank;
      hipLaunchKernelGGL(sum_splits_kernel, dim3((unsigned)((n + kThreads - 1) / kThreads)),
                         dim3(kThreads), 0, st, part, ksplit, n, ws.t);
      if ((e = hipGetLastError()) != hipSuccess) return e;
      a.h = ws.t;
      a.w = (const bf16_t *)w_up;
      a.K = rank;
      a.root = root_logits;
    } else {
      a.h = h;
      a.w = (const bf16_t *)w_full;
      a.K = d;
    }
    a.out = logits;
    a.stats = ws.stats;
    a.M = M;
    a.N = V;
    a.kspan = a.K;
    return launch_stream(a, rank > 0, 1, st);
  }
  // fp32
  const float *A = (const float *)h;
  int K = d;
  if (rank > 0) {
    const int64_t n = (int64_t)M * rank;
    hipLaunchKernelGGL(gemm_f32_kernel, dim3((unsigned)((n + kThreads - 1) / kThreads)),
                       dim3(kThreads), 0, st, A, (const float *)w_down, ws.t, M, rank, d);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    A = ws.t;
    K = rank;
  }
  const float *Bm = (const float *)(rank > 0 ? w_up : w_full);
  const int n_vt = (V + kHeadVocabTile - 1) / kHeadVocabTile;
  const bool with_root = root_logits != nullptr && root_stats != nullptr;
  hipLaunchKernelGGL(head_f32_kernel, dim3(n_vt, (M + kF32Rows - 1) / kF32Rows), dim3(kThreads),
                     0, st, A, Bm, logits, ws.stats, with_root ? root_logits : nullptr,
                     with_root ? root_stats : nullptr, M, V, K, B_root, inv_t);
  return hipGetLastError();
}

hipError_t launch_head_finish(int M, int V, float temperature, const float *logits,
                              double *row_lse, float *probs, const HeadWs &ws, hipStream_t st) {
  hipError_t e = launch_lse_from_stats(ws.stats, M, V, row_lse, st);
  if (e != hipSuccess || probs == nullptr) return e;
  const int64_t n = (int64_t)M * V;
  hipLaunchKernelGGL(head_probs_kernel, dim3((unsigned)((n + kThreads - 1) / kThreads)),
                     dim3(kThreads), 0, st, logits, row_lse, probs, M, V,
                     1.0 / (double)temperature);
  return hipGetLastError();
}

}  // namespace vs
