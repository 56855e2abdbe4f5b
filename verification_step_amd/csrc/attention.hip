// Block-triangular verify attention (SwitchSD summary, onedev.kr/papers/87,
// "무엇과 다른가"): every candidate row attends to the whole prefix and to the rows
// of its own candidate up to itself; other candidates are masked out.  The mask is
// evaluated from (candidate, offset) indices, never materialised.
//
// bf16 path (head_dim 128), per workgroup = (sequence b, KV head, row block, key split):
//   * the g*M query rows that share a KV head (GQA) are ordered r = m*g + h_local
//     and cut into blocks of NW waves x RT tiles x 16 rows;
//   * prefix keys are split in ranges of `split_keys` (paged KV, 16-token pages);
//     the candidates' own keys form one extra split;
//   * the paged cache is head-major per page: K [page][kv head][16 tokens][hd] and
//     V transposed within a page, [page][kv head][hd][16 tokens], so a 32-key block
//     of either is a few contiguous 4 KB runs; the next block is loaded into
//     registers while the current one (double-buffered in LDS) is multiplied;
//   * K sits in LDS row-major and V key-contiguous, the A operand of the PV product;
//   * S^T = K Q^T with MFMA 16x16x32 bf16: a lane holds 4 keys x 1 query row, so
//     the row max needs two cross-lane exchanges and the probabilities P^T feed the
//     next MFMA (O^T += V^T P^T) straight from registers;
//   * online softmax in fp32 (exp2 domain); P enters the PV product as bf16 hi + lo
//     (two MFMAs), which keeps the output error at the bf16 rounding of O itself;
//   * partial (max, sum, O) per split go to the workspace and a combine kernel
//     merges them in a fixed order.
// fp32 path (head_dim 16/32/64): one thread per (query row, head), plain loops.

#include "vs_internal.hpp"

#include <stdio.h>
#include <stdlib.h>

namespace vs {

namespace {

constexpr int kHD = 128;
constexpr int kKB = 32;            // keys per block
constexpr int kPage = 16;

struct AttnArgs {
  const bf16_t *q, *k_cand, *v_cand, *k_pool, *v_pool;
  const int32_t *page_table, *prefix_len;
  bf16_t *out;
  float *part_o;   // [B*Hkv][n_rb][n_splits+1][rows_per_block][hd]
  float *part_ml;  // [B*Hkv][n_rb][n_splits+1][rows_per_block][2]
  int32_t *flags;
  int B, W, D, M, Hq, Hkv, g, max_pages, n_pool_pages;
  int rows_per_kv, n_rb, rows_per_block, split_keys, n_splits;
  float scale_log2;
};

__device__ __forceinline__ int clamp_prefix(int P, int max_keys, bool *bad) {
  if (P < 0 || P > max_keys) {
    *bad = true;
    return P < 0 ? 0 : max_keys;
  }
  return P;
}

// LDS images of one 32-key block (two pages), both without padding and XOR-swizzled
// so that the MFMA fragment reads are free of bank conflicts:
//   K:   32 keys x 128 hd; the 16-byte chunk c of key k sits at position c ^ (k & 15)
//   V^T: per page, 128 hd rows x 16 keys (32 bytes a row); the 16-byte half h (keys
//        8h..8h+7) of row r sits at position h ^ ((r >> 3) & 1)
// Each is 8 KB = 8 wave-wide 16-byte-per-lane transfers, which global_load_lds
// writes straight into LDS (lane l -> bytes 16l..16l+15 of the transfer); every
// transfer reads one contiguous 1 KB run of the paged cache (4 key rows of K, or 32
// head-dim rows of one V^T page).
constexpr int kBlkElems = kKB * kHD;      // bf16 elements per K (or V^T) block image
constexpr int kNBuf = 4;                  // blocks in flight per workgroup
constexpr int kMaxSplitPages = 512;       // split_keys <= 8192

typedef __attribute__((address_space(3))) void lds_void;

// 16 bytes per lane from global memory straight into LDS (lane l -> lds_dst + 16 l).
// Issued as an opaque instruction: the compiler's automatic waits would otherwise
// drain every in-flight transfer before any read of the ring; completion is tracked
// explicitly with s_waitcnt vmcnt before the barrier that publishes a block.
__device__ __forceinline__ void dma16(const void *g, bf16_t *lds_dst) {
  // the destination is wave-uniform by construction; make that explicit for the SGPR
  const uint32_t lds = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void *)lds_dst);
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(g), "s"(lds)
               : "memory", "m0");
}

template <int RT, int NW>
__global__ void __launch_bounds__(64 * NW)
attn_mfma_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(1024))) bf16_t Kb[kNBuf][kBlkElems];
  __shared__ __attribute__((aligned(1024))) bf16_t Vb[kNBuf][kBlkElems];
  __shared__ int pages[kMaxSplitPages];

  constexpr int kIPW = 16 / NW;           // 1 KB transfers per wave per block
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int l16 = lane & 15;
  const int lg = lane >> 4;

  const int n_sp = a.n_splits + 1;
  const int nblocks = a.n_rb * n_sp * a.B * a.Hkv;
  const int bid = xcd_remap(blockIdx.x, nblocks);
  const int rb = bid % a.n_rb;
  const int s = (bid / a.n_rb) % n_sp;
  const int z = bid / (a.n_rb * n_sp);
  const int b = z / a.Hkv;
  const int kvh = z % a.Hkv;

  bool badP = false;
  const int P = clamp_prefix(a.prefix_len[b], a.max_pages * kPage, &badP);
  const int n_pref = (P + a.split_keys - 1) / a.split_keys;
  const int n_active = n_pref + 1;
  const bool is_cand = (s == a.n_splits);
  if (!is_cand && s >= n_pref) return;
  if (badP && is_cand && rb == 0 && kvh == 0 && tid == 0 && a.flags)
    atomicOr(&a.flags[b], FLAG_BAD_PAGE);

  const int k_begin = is_cand ? 0 : s * a.split_keys;
  const int k_end = is_cand ? a.M : min(P, (s + 1) * a.split_keys);
  const int nblk = (k_end - k_begin + kKB - 1) / kKB;

  // ---- this lane's query rows and fragments
  int rr[RT], mrow[RT];
  bf16x8 qf[RT][4];
#pragma unroll
  for (int t = 0; t < RT; ++t) {
    rr[t] = rb * a.rows_per_block + (wv * RT + t) * 16 + l16;
    const bool ok = rr[t] < a.rows_per_kv;
    mrow[t] = ok ? rr[t] / a.g : a.M;   // a.M marks a padding row
    const int hq = kvh * a.g + (ok ? rr[t] % a.g : 0);
    const bf16_t *qp = a.q + (((int64_t)b * a.M + (ok ? mrow[t] : 0)) * a.Hq + hq) * kHD;
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) qf[t][s4] = ok ? *(const bf16x8 *)(qp + 32 * s4 + 8 * lg) : bf16x8{};
  }
  // all ordinary loads done before the ring starts: inside the loop the only vector
  // memory operations are the explicitly counted LDS transfers
  __builtin_amdgcn_s_waitcnt(0);

  f32x4 O[RT][8];
  float m_run[RT], l_part[RT];
#pragma unroll
  for (int t = 0; t < RT; ++t) {
    m_run[t] = -INFINITY;
    l_part[t] = 0.f;
#pragma unroll
    for (int tt = 0; tt < 8; ++tt) O[t][tt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // ---- the split's page indices, once (bad pages -> -1, flagged)
  if (!is_cand) {
    const int32_t *ptab = a.page_table + (int64_t)b * a.max_pages + k_begin / kPage;
    const int np = (k_end - k_begin + kPage - 1) / kPage;
    bool bad = false;
    for (int i = tid; i < np; i += 64 * NW) {
      const int v = ptab[i];
      const bool ok = v >= 0 && v < a.n_pool_pages;
      pages[i] = ok ? v : -1;
      bad |= !ok;
    }
    if (bad && a.flags) atomicOr(&a.flags[b], FLAG_BAD_PAGE);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  // issue this wave's share of block j (prefix) into ring slot `slot`
  auto issue_prefix = [&](int j, int slot) {
    const int kb = k_begin + j * kKB;
#pragma unroll
    for (int ii = 0; ii < kIPW; ++ii) {
      const int i = wv + ii * NW;           // transfer index 0..15
      if (i < 8) {
        const int key = 4 * i + (lane >> 4);
        const int c = (lane & 15) ^ (key & 15);
        const int pg = pages[(kb - k_begin) / kPage + (key >> 4)];
        const bf16_t *src = a.k_pool;
        if (pg >= 0 && kb + key < k_end)
          src = a.k_pool + (((int64_t)pg * a.Hkv + kvh) * kPage + (key & 15)) * kHD + 8 * c;
        dma16(src, &Kb[slot][i * 512]);
      } else {
        const int i2 = i - 8;
        const int pp = i2 >> 2;                        // page within the block
        const int r = 32 * (i2 & 3) + (lane >> 1);     // head-dim row
        const int h = (lane & 1) ^ ((r >> 3) & 1);     // key half stored at this slot
        const int pg = (kb + 16 * pp < k_end) ? pages[(kb - k_begin) / kPage + pp] : -1;
        const bf16_t *src = a.v_pool;
        if (pg >= 0)
          src = a.v_pool + (((int64_t)pg * a.Hkv + kvh) * kHD + r) * kPage + 8 * h;
        dma16(src, &Vb[slot][i2 * 512]);
      }
    }
  };
  // candidate keys (row-major [B*M, Hkv, hd]): staged through registers, V transposed
  auto stage_cand = [&](int slot, int kb) {
    for (int c = tid; c < kKB * 16; c += 64 * NW) {
      const int key = c >> 4, ch = c & 15;
      const int pos = kb + key;
      u32x4 kv = {0u, 0u, 0u, 0u}, vv = {0u, 0u, 0u, 0u};
      if (pos < k_end) {
        const int64_t off = (((int64_t)b * a.M + pos) * a.Hkv + kvh) * kHD + 8 * ch;
        kv = *(const u32x4 *)(a.k_cand + off);
        vv = *(const u32x4 *)(a.v_cand + off);
      }
      *(u32x4 *)&Kb[slot][key * kHD + 8 * (ch ^ (key & 15))] = kv;
      const bf16_t *ve = (const bf16_t *)&vv;
      const int pp = key >> 4, kk = key & 15;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int r = 8 * ch + e;
        const int h = (kk >> 3) ^ ((r >> 3) & 1);
        Vb[slot][pp * 2048 + r * 16 + 8 * h + (kk & 7)] = ve[e];
      }
    }
  };

  auto compute = [&](int slot, int kb) {
    bf16x8 ka[4], kb2[4], vf[8];
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      const int pch = (4 * s4 + lg) ^ l16;
      ka[s4] = *(const bf16x8 *)&Kb[slot][l16 * kHD + 8 * pch];
      kb2[s4] = *(const bf16x8 *)&Kb[slot][(16 + l16) * kHD + 8 * pch];
    }
    // keys 4lg..4lg+3 of page 0 and of page 1 (block keys 16+4lg..): half lg>>1
    const int hsw = ((lg >> 1) ^ ((l16 >> 3) & 1)) * 8 + 4 * (lg & 1);
#pragma unroll
    for (int tt = 0; tt < 8; ++tt) {
      const int r = 16 * tt + l16;
      typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
      const bf16x4 lo = *(const bf16x4 *)&Vb[slot][r * 16 + hsw];
      const bf16x4 hi = *(const bf16x4 *)&Vb[slot][2048 + r * 16 + hsw];
      vf[tt] = bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
    // block validity, uniform over the workgroup: two page lookups per block; a block
    // of 32 in-range keys on two valid pages needs no per-key mask
    int pv0 = 1, pv1 = 1;
    if (!is_cand) {
      const int pl = (kb - k_begin) >> 4;
      pv0 = pages[pl] >= 0;
      pv1 = (kb + 16 < k_end) ? (pages[pl + 1] >= 0) : 0;
    }
    const bool full = !is_cand && pv0 && pv1 && (kb + kKB <= k_end);
#pragma unroll
    for (int t = 0; t < RT; ++t) {
      f32x4 sa = {0.f, 0.f, 0.f, 0.f}, sb = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) {
        sa = mfma16x16x32(ka[s4], qf[t][s4], sa);
        sb = mfma16x16x32(kb2[s4], qf[t][s4], sb);
      }
      float xa[4], xb[4];
      if (full) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          xa[j] = sa[j] * a.scale_log2;
          xb[j] = sb[j] * a.scale_log2;
        }
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int ka_i = kb + 4 * lg + j, kb_i = kb + 16 + 4 * lg + j;
          bool va, vb;
          if (is_cand) {
            const int m = mrow[t];
            va = ka_i < k_end && m < a.M && ka_i / a.D == m / a.D && ka_i <= m;
            vb = kb_i < k_end && m < a.M && kb_i / a.D == m / a.D && kb_i <= m;
          } else {
            va = pv0 && ka_i < k_end;
            vb = pv1 && kb_i < k_end;
          }
          xa[j] = va ? sa[j] * a.scale_log2 : -INFINITY;
          xb[j] = vb ? sb[j] * a.scale_log2 : -INFINITY;
        }
      }
      float bmax = fmaxf(fmaxf(fmaxf(xa[0], xa[1]), fmaxf(xa[2], xa[3])),
                         fmaxf(fmaxf(xb[0], xb[1]), fmaxf(xb[2], xb[3])));
      bmax = fmaxf(bmax, __shfl_xor(bmax, 16));
      bmax = fmaxf(bmax, __shfl_xor(bmax, 32));
      // rescale the running sums only when some row's maximum grew
      const float mnew = fmaxf(m_run[t], bmax);
      const bool grow = mnew > m_run[t];
      if (__ballot(grow) != 0) {
        const float corr = grow ? exp2f(m_run[t] - mnew) : 1.f;
        l_part[t] *= corr;
#pragma unroll
        for (int tt = 0; tt < 8; ++tt) O[t][tt] *= corr;
        m_run[t] = mnew;
      }
      const float mref = (m_run[t] == -INFINITY) ? 0.f : m_run[t];
      float pa[4], pb[4], psum = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        pa[j] = exp2f(xa[j] - mref);
        pb[j] = exp2f(xb[j] - mref);
        psum += pa[j] + pb[j];
      }
      l_part[t] += psum;
      // P = hi + lo, both bf16: the PV product keeps ~16 significant bits of P
      uint32_t hk[4], lk[4];
      split_bf16x2(pa[0], pa[1], hk[0], lk[0]);
      split_bf16x2(pa[2], pa[3], hk[1], lk[1]);
      split_bf16x2(pb[0], pb[1], hk[2], lk[2]);
      split_bf16x2(pb[2], pb[3], hk[3], lk[3]);
      const bf16x8 phi = *(const bf16x8 *)hk;
      const bf16x8 plo = *(const bf16x8 *)lk;
#pragma unroll
      for (int tt = 0; tt < 8; ++tt) {
        O[t][tt] = mfma16x16x32(vf[tt], phi, O[t][tt]);
        O[t][tt] = mfma16x16x32(vf[tt], plo, O[t][tt]);
      }
    }
  };

  if (is_cand) {
    for (int j = 0; j < nblk; ++j) {
      const int slot = j & 1;
      stage_cand(slot, k_begin + j * kKB);
      __syncthreads();
      compute(slot, k_begin + j * kKB);
    }
  } else {
    // ring: blocks j+1..j+kNBuf-2 stay in flight while block j is multiplied
#pragma unroll
    for (int j = 0; j < kNBuf - 1; ++j)
      if (j < nblk) issue_prefix(j, j);
    for (int j = 0; j < nblk; ++j) {
      if (j + kNBuf - 2 < nblk)
        __builtin_amdgcn_s_waitcnt(0x0F70 | (((kNBuf - 2) * kIPW) & 15) |
                                   ((((kNBuf - 2) * kIPW) >> 4) << 14));
      else
        __builtin_amdgcn_s_waitcnt(0x0F70);   // tail: everything issued is needed
      __syncthreads();
      if (j + kNBuf - 1 < nblk) issue_prefix(j + kNBuf - 1, (j + kNBuf - 1) % kNBuf);
      compute(j % kNBuf, k_begin + j * kKB);
    }
  }

  // ---- finish: row sums over the 4 lane groups, then final output or partials
#pragma unroll
  for (int t = 0; t < RT; ++t) {
    float l = l_part[t];
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    const bool ok = rr[t] < a.rows_per_kv;
    if (!ok) continue;
    const int row_in_block = (wv * RT + t) * 16 + l16;
    if (n_active == 1) {
      const float inv = l > 0.f ? 1.f / l : 0.f;
      const int hq = kvh * a.g + rr[t] % a.g;
      bf16_t *op = a.out + (((int64_t)b * a.M + mrow[t]) * a.Hq + hq) * kHD;
#pragma unroll
      for (int tt = 0; tt < 8; ++tt) {
        uint32_t w0 = pack_bf16x2(O[t][tt][0] * inv, O[t][tt][1] * inv);
        uint32_t w1 = pack_bf16x2(O[t][tt][2] * inv, O[t][tt][3] * inv);
        *(uint2 *)(op + 16 * tt + 4 * lg) = make_uint2(w0, w1);
      }
    } else {
      const int64_t slot =
          (((int64_t)z * a.n_rb + rb) * n_sp + s) * a.rows_per_block + row_in_block;
      float *po = a.part_o + slot * kHD;
#pragma unroll
      for (int tt = 0; tt < 8; ++tt) *(f32x4 *)(po + 16 * tt + 4 * lg) = O[t][tt];
      if (lg == 0) {
        a.part_ml[slot * 2 + 0] = m_run[t];
        a.part_ml[slot * 2 + 1] = l;
      }
    }
  }
}

// Merge the split partials of every row in a fixed order (prefix splits ascending,
// then the candidate split).  One thread per (row, 4 head-dim values).
__global__ void __launch_bounds__(256)
attn_combine_kernel(AttnArgs a) {
  const int n_sp = a.n_splits + 1;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total_rows = (int64_t)a.B * a.Hkv * a.n_rb * a.rows_per_block;
  const int64_t row = gid / 32;
  const int c4 = (int)(gid % 32) * 4;
  if (row >= total_rows) return;
  const int row_in_block = (int)(row % a.rows_per_block);
  const int rb = (int)((row / a.rows_per_block) % a.n_rb);
  const int z = (int)(row / ((int64_t)a.rows_per_block * a.n_rb));
  const int b = z / a.Hkv, kvh = z % a.Hkv;
  const int rr = rb * a.rows_per_block + row_in_block;
  if (rr >= a.rows_per_kv) return;
  bool badP = false;
  const int P = clamp_prefix(a.prefix_len[b], a.max_pages * kPage, &badP);
  const int n_pref = (P + a.split_keys - 1) / a.split_keys;
  if (n_pref == 0) return;  // the candidate split alone wrote the output
  const int64_t base = ((int64_t)z * a.n_rb + rb) * n_sp;
  float mx = -INFINITY;
  for (int k = 0; k <= n_pref; ++k) {
    const int sp = (k == n_pref) ? a.n_splits : k;
    mx = fmaxf(mx, a.part_ml[((base + sp) * a.rows_per_block + row_in_block) * 2]);
  }
  const float mref = (mx == -INFINITY) ? 0.f : mx;
  float l = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int k = 0; k <= n_pref; ++k) {
    const int sp = (k == n_pref) ? a.n_splits : k;
    const int64_t slot = (base + sp) * a.rows_per_block + row_in_block;
    const float w = exp2f(a.part_ml[slot * 2] - mref);
    l += w * a.part_ml[slot * 2 + 1];
    const f32x4 o = *(const f32x4 *)(a.part_o + slot * kHD + c4);
    acc += w * o;
  }
  const float inv = l > 0.f ? 1.f / l : 0.f;
  const int m = rr / a.g;
  const int hq = kvh * a.g + rr % a.g;
  bf16_t *op = a.out + (((int64_t)b * a.M + m) * a.Hq + hq) * kHD + c4;
  *(uint2 *)op = make_uint2(pack_bf16x2(acc[0] * inv, acc[1] * inv),
                            pack_bf16x2(acc[2] * inv, acc[3] * inv));
}

// ---------------------------------------------------------------------------- fp32 path
template <int HD>
__global__ void __launch_bounds__(256)
attn_f32_kernel(const float *q, const float *k_cand, const float *v_cand, const float *k_pool,
                const float *v_pool, const int32_t *page_table, const int32_t *prefix_len,
                float *out, int32_t *flags, int B, int W, int D, int Hq, int Hkv, int max_pages,
                int n_pool_pages, float scale) {
  const int M = W * D;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (int64_t)B * M * Hq) return;
  const int hq = (int)(gid % Hq);
  const int r = (int)((gid / Hq) % M);
  const int b = (int)(gid / ((int64_t)Hq * M));
  const int kvh = hq / (Hq / Hkv);
  bool badP = false;
  const int P = clamp_prefix(prefix_len[b], max_pages * kPage, &badP);
  if (badP && flags && r == 0 && hq == 0) atomicOr(&flags[b], FLAG_BAD_PAGE);
  float qv[HD], acc[HD];
  const float *qp = q + (((int64_t)b * M + r) * Hq + hq) * HD;
  for (int e = 0; e < HD; ++e) {
    qv[e] = qp[e];
    acc[e] = 0.f;
  }
  float mx = -INFINITY, l = 0.f;
  const int i = r / D, o = r % D;
  const int nkeys = P + o + 1;
  for (int k = 0; k < nkeys; ++k) {
    const float *kp, *vp;
    int vstride = 1;
    if (k < P) {
      const int pg = page_table[(int64_t)b * max_pages + k / kPage];
      if (pg < 0 || pg >= n_pool_pages) {
        if (flags && (k % kPage) == 0 && hq == 0) atomicOr(&flags[b], FLAG_BAD_PAGE);
        continue;
      }
      kp = k_pool + (((int64_t)pg * Hkv + kvh) * kPage + k % kPage) * HD;
      vp = v_pool + ((int64_t)pg * Hkv + kvh) * HD * kPage + k % kPage;
      vstride = kPage;
    } else {
      const int64_t off = (((int64_t)b * M + i * D + (k - P)) * Hkv + kvh) * HD;
      kp = k_cand + off;
      vp = v_cand + off;
    }
    float sdot = 0.f;
    for (int e = 0; e < HD; ++e) sdot = fmaf(qv[e], kp[e], sdot);
    sdot *= scale;
    const float mnew = fmaxf(mx, sdot);
    const float corr = expf(mx - mnew);
    const float p = expf(sdot - mnew);
    l = l * corr + p;
    for (int e = 0; e < HD; ++e) acc[e] = acc[e] * corr + p * vp[e * vstride];
    mx = mnew;
  }
  float *op = out + (((int64_t)b * M + r) * Hq + hq) * HD;
  const float inv = l > 0.f ? 1.f / l : 0.f;
  for (int e = 0; e < HD; ++e) op[e] = acc[e] * inv;
}

__global__ void zero_i32_kernel(int32_t *p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

}  // namespace

AttnPlan attn_plan(int B, int W, int D, int Hq, int Hkv, int max_pages, int page) {
  AttnPlan p{};
  const int M = W * D;
  const int g = Hq / Hkv;
  p.rows_per_kv = g * M;
  const int tiles = (p.rows_per_kv + 15) / 16;
  // row block: fewest padded rows, then the largest block (fewer re-reads of K/V)
  int best_waste = 1 << 30, best_rows = 0;
  for (int rt = 1; rt <= 2; ++rt) {
    for (int nw = 2; nw <= (rt == 1 ? 8 : 4); nw *= 2) {
      const int tpb = rt * nw;
      const int nrb = (tiles + tpb - 1) / tpb;
      const int waste = nrb * tpb - tiles;
      const int rows = tpb * 16;
      if (waste < best_waste || (waste == best_waste && rows > best_rows)) {
        best_waste = waste;
        best_rows = rows;
        p.rt = rt;
        p.nw = nw;
      }
    }
  }
  // key splits: about 256 workgroups of prefix work for the longest sequence's share
  const int max_keys = max_pages * page;
  int split_keys = 0;
  // tuning override "rt,nw,split_keys" (values <= 0 keep the heuristic's choice)
  if (const char *ov = getenv("VSTEP_ATTN_PLAN")) {
    int rt = 0, nw = 0, sk = 0;
    if (sscanf(ov, "%d,%d,%d", &rt, &nw, &sk) == 3) {
      if ((rt == 1 && (nw == 2 || nw == 4 || nw == 8)) || (rt == 2 && (nw == 2 || nw == 4))) {
        p.rt = rt;
        p.nw = nw;
      }
      if (sk > 0) split_keys = ((sk + kKB - 1) / kKB) * kKB;
    }
  }
  p.rows_per_block = p.rt * p.nw * 16;
  p.n_rb = (tiles + p.rt * p.nw - 1) / (p.rt * p.nw);
  if (split_keys == 0) {
    const int groups = B * Hkv * p.n_rb;
    int want = (256 + groups - 1) / groups;
    if (want < 1) want = 1;
    int sk = (max_keys + want - 1) / want;
    sk = ((sk + kKB - 1) / kKB) * kKB;
    if (sk < 256) sk = 256;
    split_keys = sk;
  }
  if (split_keys > kMaxSplitPages * kPage) split_keys = kMaxSplitPages * kPage;
  p.split_keys = split_keys;
  p.n_splits = (max_keys + split_keys - 1) / split_keys;
  if (p.n_splits < 1) p.n_splits = 1;
  return p;
}

size_t attn_workspace_bytes(int B, int W, int D, int Hq, int Hkv, int hd, int max_pages, int page,
                            int dtype) {
  if (dtype != 1) return 0;
  const AttnPlan p = attn_plan(B, W, D, Hq, Hkv, max_pages, page);
  const size_t slots = (size_t)B * Hkv * p.n_rb * (p.n_splits + 1) * p.rows_per_block;
  return slots * (size_t)(kHD + 2) * sizeof(float) + 256;
}

hipError_t launch_attention(int B, int W, int D, int Hq, int Hkv, int hd, int max_pages,
                            int n_pool_pages, int dtype, float scale, const void *q,
                            const void *k_cand, const void *v_cand, const void *k_pool,
                            const void *v_pool, const int32_t *page_table,
                            const int32_t *prefix_len, void *out, int32_t *flags, void *ws,
                            hipStream_t st) {
  const int M = W * D;
  if (dtype == 0) {
    const int64_t n = (int64_t)B * M * Hq;
    const int blocks = (int)((n + 255) / 256);
#define VS_F32_ATTN(HDV)                                                                       \
  hipLaunchKernelGGL(attn_f32_kernel<HDV>, dim3(blocks), dim3(256), 0, st, (const float *)q,   \
                     (const float *)k_cand, (const float *)v_cand, (const float *)k_pool,      \
                     (const float *)v_pool, page_table, prefix_len, (float *)out, flags, B, W, \
                     D, Hq, Hkv, max_pages, n_pool_pages, scale)
    if (hd == 16) VS_F32_ATTN(16);
    else if (hd == 32) VS_F32_ATTN(32);
    else VS_F32_ATTN(64);
#undef VS_F32_ATTN
    return hipGetLastError();
  }
  const AttnPlan p = attn_plan(B, W, D, Hq, Hkv, max_pages, kPage);
  AttnArgs a;
  a.q = (const bf16_t *)q;
  a.k_cand = (const bf16_t *)k_cand;
  a.v_cand = (const bf16_t *)v_cand;
  a.k_pool = (const bf16_t *)k_pool;
  a.v_pool = (const bf16_t *)v_pool;
  a.page_table = page_table;
  a.prefix_len = prefix_len;
  a.out = (bf16_t *)out;
  const size_t slots = (size_t)B * Hkv * p.n_rb * (p.n_splits + 1) * p.rows_per_block;
  a.part_o = (float *)ws;
  a.part_ml = a.part_o + slots * kHD;
  a.flags = flags;
  a.B = B;
  a.W = W;
  a.D = D;
  a.M = M;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.g = Hq / Hkv;
  a.max_pages = max_pages;
  a.n_pool_pages = n_pool_pages;
  a.rows_per_kv = p.rows_per_kv;
  a.n_rb = p.n_rb;
  a.rows_per_block = p.rows_per_block;
  a.split_keys = p.split_keys;
  a.n_splits = p.n_splits;
  a.scale_log2 = scale * 1.4426950408889634f;
  const int nblocks = p.n_rb * (p.n_splits + 1) * B * Hkv;
  const dim3 grid(nblocks), block(64 * p.nw);
  if (p.rt == 1 && p.nw == 2) hipLaunchKernelGGL((attn_mfma_kernel<1, 2>), grid, block, 0, st, a);
  else if (p.rt == 1 && p.nw == 4) hipLaunchKernelGGL((attn_mfma_kernel<1, 4>), grid, block, 0, st, a);
  else if (p.rt == 1) hipLaunchKernelGGL((attn_mfma_kernel<1, 8>), grid, block, 0, st, a);
  else if (p.nw == 2) hipLaunchKernelGGL((attn_mfma_kernel<2, 2>), grid, block, 0, st, a);
  else hipLaunchKernelGGL((attn_mfma_kernel<2, 4>), grid, block, 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t threads = (int64_t)B * Hkv * p.n_rb * p.rows_per_block * 32;
  hipLaunchKernelGGL(attn_combine_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0,
                     st, a);
  return hipGetLastError();
}

hipError_t launch_zero_i32(int32_t *p, int n, hipStream_t st) {
  if (n <= 0 || p == nullptr) return hipSuccess;
  hipLaunchKernelGGL(zero_i32_kernel, dim3((n + 255) / 256), dim3(256), 0, st, p, n);
  return hipGetLastError();
}

}  // namespace vs
