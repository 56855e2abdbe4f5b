// Block-triangular verify attention (SwitchSD summary, onedev.kr/papers/87,
// "무엇과 다른가"): every candidate row attends to the whole prefix and to the rows
// of its own candidate up to itself; other candidates are masked out.  The mask is
// evaluated from (candidate, offset) indices, never materialised.
//
// bf16 path (head_dim 128), per workgroup = (sequence b, KV head, row block, key split):
//   * the g*M query rows that share a KV head (GQA) are ordered r = m*g + h_local
//     and cut into tiles of 32 rows, one per wave; NW waves form a row block and
//     share one stream of K/V blocks through LDS;
//   * prefix keys are split in ranges of `split_keys` (paged KV, 16-token pages);
//     the candidates' own keys form one extra split;
//   * the paged cache is head-major per page: K [page][kv head][16 tokens][hd] and
//     V transposed within a page, [page][kv head][hd][16 tokens], so a 32-key block
//     of either is a few contiguous 4 KB runs, moved by direct global->LDS transfers
//     into a ring of kNBuf blocks that runs ahead of the multiplication;
//   * S^T = K Q^T with MFMA 32x32x16 bf16: a lane holds 16 keys x 1 query row, the
//     other 16 keys of that row sit in lane l^32, so the row max is one cross-lane
//     swap; the probabilities P^T feed the PV product (O^T += V^T P^T) straight
//     from registers;
//   * online softmax in fp32 in the exp2 domain, with a lazy reference maximum: the
//     accumulators are rescaled only when a row's block maximum exceeds the
//     reference by more than kLazy (P stays below 2^kLazy, exact either way);
//   * P enters the PV product as bf16 hi + lo (two MFMAs), which keeps the output
//     error at the bf16 rounding of O itself;
//   * partial (max, sum, O) per split go to the workspace and a combine kernel
//     merges them in a fixed order.
// Layers: one launch may cover L layers that share the page table and prefix lengths
// (a page id names the same slot in every layer's pool); each layer has its own
// queries, candidate keys/values, pools and output at a fixed stride, and the
// workgroups of all layers form one grid.
// fp32 path (head_dim 16/32/64): one wave per (layer, query row, head), plain loops.

#include "gate_wg.hpp"
#include "vs_internal.hpp"

#include <stdio.h>
#include <stdlib.h>

namespace vs {

namespace {

constexpr int kHD = 128;
constexpr int kKB = 32;            // keys per block
constexpr int kPage = 16;
constexpr int kTileRows = 32;      // query rows per wave
constexpr float kLazy = 8.0f;      // log2 headroom of the lazy reference maximum

typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;

__device__ __forceinline__ f32x16 mfma32x32x16(const bf16x8 &a, const bf16x8 &b, const f32x16 &c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// max of x over lanes l and l^32
__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float sum_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

struct AttnArgs {
  const bf16_t *q, *k_cand, *v_cand, *k_pool, *v_pool;
  const int32_t *page_table, *prefix_len;
  bf16_t *out;
  float *part_o;   // [L*B*Hkv][n_rb][n_splits+1][rows_per_block][hd]
  float *part_ml;  // [L*B*Hkv][n_rb][n_splits+1][rows_per_block][2]
  int32_t *flags;
  int64_t q_ls, c_ls, p_ls;   // per-layer strides (elements) of q/out, k/v_cand, pools
  int B, W, D, M, Hq, Hkv, g, max_pages, n_pool_pages, L;
  int rows_per_kv, n_rb, rows_per_block, split_keys, n_splits;
  float scale_log2;
  int n_gate;        // leading workgroups that run the copy path's gate (0: none)
  GateArgs gate;
  int grp_map;
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

// 16 bytes per lane from global memory straight into LDS: lane l reads sbase + voff_l
// and writes LDS bytes lds + 16 l .. lds + 16 l + 15.  sbase and lds are wave-uniform
// (SGPRs).  Issued as an opaque instruction: the compiler's automatic waits would
// otherwise drain every in-flight transfer before any read of the ring; completion is
// tracked explicitly with s_waitcnt vmcnt before the barrier that publishes a block.
__device__ __forceinline__ void dma16(const void *sbase, uint32_t voff, uint32_t lds) {
  // both operands are uniform by construction; readfirstlane makes that visible
  // (readfirstlane returns int: each half goes through uint32_t so that the low word
  // is not sign-extended into the high one)
  const uint64_t sb = (uint64_t)(uintptr_t)sbase;
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)sb);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(sb >> 32));
  const uint64_t sbu = ((uint64_t)hi << 32) | (uint64_t)lo;
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"((const void *)(uintptr_t)sbu),
                 "s"(__builtin_amdgcn_readfirstlane(lds))
               : "memory", "m0");
}

__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(const lds_void *)p);
}

// Key order of the QK product inside a 16-key page: MFMA row i holds key perm16(i),
// bits 2 and 3 swapped, so that lane half h of the 32x32 result holds keys 8h..8h+7
// of each page -- eight consecutive keys, one 16-byte V^T read for the PV product.
__device__ __forceinline__ int perm16(int i) {
  return (i & ~12) | ((i & 4) << 1) | ((i & 8) >> 1);
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

template <int NW>
__global__ void __launch_bounds__(64 * NW, 2)
attn_mfma_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(1024))) bf16_t Kb[kNBuf][kBlkElems];
  __shared__ __attribute__((aligned(1024))) bf16_t Vb[kNBuf][kBlkElems];
  __shared__ int pages[kMaxSplitPages];

  // a block is 16 transfers of 1 KB (8 of K, 8 of V^T); wave wv issues wv, wv+NW, ...
  constexpr int kT = 16;
  constexpr int kIPW = (kT + NW - 1) / NW;
  constexpr bool kEven = (kT % NW) == 0;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int h = lane >> 5;
  const bool full_share = kEven || wv < kT % NW;   // this wave issues kIPW transfers

  // the first n_gate workgroups retrieve and gate one sequence each, in the LDS of the
  // K ring, while the attention workgroups after them start
  if constexpr (NW >= 4) {
    static_assert(sizeof(GateShared<64 * NW>) <= sizeof(Kb), "gate state fits the K ring");
    if ((int)blockIdx.x < a.n_gate) {
      gate_wg<64 * NW>(a.gate, blockIdx.x, *reinterpret_cast<GateShared<64 * NW> *>(&Kb[0][0]));
      return;
    }
  }
  // one prefix split: its workgroup also takes the candidates' keys (no partials)
  const bool fold = a.n_splits == 1;
  const int n_sp = fold ? 1 : a.n_splits + 1;
  // Workgroup -> (row block, split, (layer, sequence, kv head)).  Workgroups are dealt
  // round-robin over the 8 XCDs; the row blocks of one split (which read the same K/V)
  // sit on one XCD, and consecutive (split, group) pairs on consecutive XCDs, so that
  // splits of uneven length -- ragged prefixes -- spread over every XCD.  Workgroup j
  // (after the gate's) is row block (j/8) % n_rb of pair ((j/8) / n_rb) * 8 + j % 8;
  // pairs past the last return at once.  One sequence (grp_map 1): pairs split-major
  // (pair = z + groups * s), so that its short candidate splits are dispatched last,
  // behind the prefix splits, when the grid outgrows one round; batches (grp_map 2):
  // group-major (pair = s + splits * z); batches of up to 64 sequences (grp_map 3):
  // longest first -- every full-length split of every sequence, then the partial
  // splits by decreasing length, then the candidate splits, then the empty ones -- so
  // that the grid's last round holds short work (the batch's prefix lengths live on the
  // device: each wave ranks them itself, lane b holding sequence b).
  int rb, s, z;
  int P_ranked = -1;
  bool bad_ranked = false;
  if (a.grp_map) {
    const int n_z = a.B * a.Hkv * a.L;
    const int n_pairs = n_sp * n_z;
    const int j = (int)blockIdx.x - a.n_gate;
    const int r = j >> 3;
    const int pair = (r / a.n_rb) * 8 + (j & 7);
    if (pair >= n_pairs) return;
    rb = r % a.n_rb;
    if (a.grp_map == 3) {
      const int G = a.Hkv * a.L;                  // groups of one sequence
      bool bl = false;
      const int Pl = lane < a.B ? clamp_prefix(a.prefix_len[lane], a.max_pages * kPage, &bl) : 0;
      const int nfull = Pl / a.split_keys;        // its full-length splits
      const int rem = Pl - nfull * a.split_keys;  // keys of its partial split (0: none)
      int incl = nfull;                           // inclusive scan over the sequences
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int t = __shfl_up(incl, off);
        if (lane >= off) incl += t;
      }
      const int F = __builtin_amdgcn_readlane(incl, 63);
      const int Pn = __popcll(__ballot(rem > 0));
      const int u = pair / G, gi = pair % G;
      int bs;
      if (u < F) {
        bs = __builtin_ctzll(__ballot(incl > u));
        s = u - (__builtin_amdgcn_readlane(incl, bs) - __builtin_amdgcn_readlane(nfull, bs));
      } else if (u < F + Pn) {
        // rank among the partial splits: longer first, equal lengths by sequence
        int rank = 0;
#pragma unroll
        for (int o = 0; o < 64; ++o) {
          const int r2 = __builtin_amdgcn_readlane(rem, o);
          rank += (r2 > rem || (r2 == rem && o < lane)) ? 1 : 0;
        }
        bs = __builtin_ctzll(__ballot(rem > 0 && rank == u - F));
        s = __builtin_amdgcn_readlane(nfull, bs);
      } else if (u < F + Pn + a.B) {
        bs = u - F - Pn;
        s = a.n_splits;
      } else {
        return;
      }
      z = (gi / a.Hkv) * (a.B * a.Hkv) + bs * a.Hkv + gi % a.Hkv;
      P_ranked = __builtin_amdgcn_readlane(Pl, bs);
      bad_ranked = __builtin_amdgcn_readlane(bl ? 1 : 0, bs) != 0;
    } else if (a.grp_map == 1) {
      s = pair / n_z;
      z = pair % n_z;
    } else {
      s = pair % n_sp;
      z = pair / n_sp;
    }
  } else {
    const int nblocks = a.n_rb * n_sp * a.B * a.Hkv * a.L;
    const int bid = xcd_remap((int)blockIdx.x - a.n_gate, nblocks);
    rb = bid % a.n_rb;
    s = (bid / a.n_rb) % n_sp;
    z = bid / (a.n_rb * n_sp);        // (layer, sequence, kv head)
  }
  const int zs = z % (a.B * a.Hkv);
  const int layer = z / (a.B * a.Hkv);
  const int b = zs / a.Hkv;
  const int kvh = zs % a.Hkv;
  const bf16_t *q_l = a.q + layer * a.q_ls;
  const bf16_t *kc_l = a.k_cand + layer * a.c_ls;
  const bf16_t *vc_l = a.v_cand + layer * a.c_ls;
  const bf16_t *kp_l = a.k_pool + layer * a.p_ls;
  const bf16_t *vp_l = a.v_pool + layer * a.p_ls;

  bool badP = bad_ranked;
  const int P = P_ranked >= 0 ? P_ranked : clamp_prefix(a.prefix_len[b], a.max_pages * kPage, &badP);
  const int n_pref = (P + a.split_keys - 1) / a.split_keys;
  const int n_active = n_pref + 1;
  const bool is_cand = !fold && s == a.n_splits;
  if (!is_cand && !fold && s >= n_pref) return;
  if (badP && (is_cand || fold) && rb == 0 && kvh == 0 && layer == 0 && tid == 0 && a.flags)
    atomicOr(&a.flags[b], FLAG_BAD_PAGE);

  const int k_begin = is_cand ? 0 : s * a.split_keys;
  const int k_end = is_cand ? a.M : min(P, (s + 1) * a.split_keys);
  const int nblk = (k_end - k_begin + kKB - 1) / kKB;

  // ---- this lane's query row (one of the wave's 32) and its Q^T fragments
  const int rr = rb * a.rows_per_block + wv * kTileRows + l32;
  const bool rok = rr < a.rows_per_kv;
  const int mrow = rok ? rr / a.g : a.M;   // a.M marks a padding row
  const int hq = kvh * a.g + (rok ? rr % a.g : 0);
  bf16x8 qf[8];
  {
    const bf16_t *qp = q_l + (((int64_t)b * a.M + (rok ? mrow : 0)) * a.Hq + hq) * kHD + 8 * h;
#pragma unroll
    for (int s8 = 0; s8 < 8; ++s8) qf[s8] = rok ? *(const bf16x8 *)(qp + 16 * s8) : bf16x8{};
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
  // all ordinary loads done before the ring starts: inside the loop the only vector
  // memory operations are the explicitly counted LDS transfers
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  f32x16 O[4];
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int j = 0; j < 16; ++j) O[t][j] = 0.f;
  float m_run = -INFINITY, l_part = 0.f;
  const float c = a.scale_log2;

  // this wave's transfers of a block: byte offset of each lane's 16 bytes inside the
  // (page, KV head) run of the pool, and the transfer's place in the LDS block image
  //   K transfer i < 8: keys 4i..4i+3 (page i/4); chunk c of key k lands at c ^ (k & 15)
  //   V^T transfer i >= 8: page (i-8)/4, head-dim rows 32((i-8)%4) + l/2, key half
  //   hh = (l & 1) ^ ((r >> 3) & 1) lands at position l & 1 of row r
  uint32_t voff[kIPW];
#pragma unroll
  for (int ii = 0; ii < kIPW; ++ii) {
    const int i = min(wv + ii * NW, kT - 1);
    if (i < 8) {
      const int key = 4 * i + (lane >> 4);
      const int ch = (lane & 15) ^ (key & 15);
      voff[ii] = (uint32_t)(((key & 15) * kHD + 8 * ch) * 2);
    } else {
      const int r = 32 * ((i - 8) & 3) + (lane >> 1);
      const int hh = (lane & 1) ^ ((r >> 3) & 1);
      voff[ii] = (uint32_t)((r * kPage + 8 * hh) * 2);
    }
  }
  const uint32_t kb_lds = lds_addr(&Kb[0][0]);
  const uint32_t vb_lds = lds_addr(&Vb[0][0]);
  constexpr uint32_t kSlotBytes = kBlkElems * 2;

  // issue this wave's share of block j (prefix) into ring slot `slot`
  auto issue_prefix = [&](int j, int slot) {
    const int kb = k_begin + j * kKB;
    const int pl = 2 * j;
    const int pg0 = __builtin_amdgcn_readfirstlane(pages[pl]);
    const int pg1 = __builtin_amdgcn_readfirstlane((kb + kPage < k_end) ? pages[pl + 1] : -1);
    // a missing or bad page reads the pool's first run instead; its keys are masked
    const int64_t run0 = pg0 >= 0 ? ((int64_t)pg0 * a.Hkv + kvh) * (kPage * kHD) : 0;
    const int64_t run1 = pg1 >= 0 ? ((int64_t)pg1 * a.Hkv + kvh) * (kPage * kHD) : 0;
#pragma unroll
    for (int ii = 0; ii < kIPW; ++ii) {
      const int i = wv + ii * NW;           // transfer index 0..15
      if (i >= kT) break;
      const int64_t run = ((i & 7) >> 2) ? run1 : run0;
      if (i < 8)
        dma16(kp_l + run, voff[ii], kb_lds + slot * kSlotBytes + i * 1024);
      else
        dma16(vp_l + run, voff[ii], vb_lds + slot * kSlotBytes + (i - 8) * 1024);
    }
  };
  // candidate keys (row-major [B*M, Hkv, hd]): staged through registers, V transposed
  auto stage_cand = [&](int slot, int kb) {
    for (int cc = tid; cc < kKB * 16; cc += 64 * NW) {
      const int key = cc >> 4, ch = cc & 15;
      const int pos = kb + key;
      u32x4 kv = {0u, 0u, 0u, 0u}, vv = {0u, 0u, 0u, 0u};
      if (pos < a.M) {
        const int64_t off = (((int64_t)b * a.M + pos) * a.Hkv + kvh) * kHD + 8 * ch;
        kv = *(const u32x4 *)(kc_l + off);
        vv = *(const u32x4 *)(vc_l + off);
      }
      *(u32x4 *)&Kb[slot][key * kHD + 8 * (ch ^ (key & 15))] = kv;
      const bf16_t *ve = (const bf16_t *)&vv;
      const int pp = key >> 4, kk = key & 15;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int r = 8 * ch + e;
        const int hh = (kk >> 3) ^ ((r >> 3) & 1);
        Vb[slot][pp * 2048 + r * 16 + 8 * hh + (kk & 7)] = ve[e];
      }
    }
  };

  // MFMA row l32 of the QK product is key krow of the block; lane l, register j of
  // S^T then holds key 16*(j/8) + 8h + j%8, row l32
  const int krow = (l32 & 16) | perm16(l32 & 15);
  auto load_k = [&](int slot, bf16x8 *kf) {
#pragma unroll
    for (int s8 = 0; s8 < 8; ++s8) {
      const int pc = (2 * s8 + h) ^ (krow & 15);
      kf[s8] = *(const bf16x8 *)&Kb[slot][krow * kHD + 8 * pc];
    }
  };
  // V^T fragment (t, ks): head-dim row 32t + l32, keys 8h..8h+7 of page ks
  auto load_v = [&](int slot, bf16x8 *vf) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int r = 32 * t + l32;
      const int sw = (r >> 3) & 1;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
        vf[2 * t + ks] = *(const bf16x8 *)&Vb[slot][ks * 2048 + r * 16 + 8 * (h ^ sw)];
    }
  };
  auto qk_mma = [&](const bf16x8 *kf) -> f32x16 {
    f32x16 S;
#pragma unroll
    for (int j = 0; j < 16; ++j) S[j] = 0.f;
#pragma unroll
    for (int s8 = 0; s8 < 8; ++s8) S = mfma32x32x16(kf[s8], qf[s8], S);
    return S;
  };

  // V^T fragments of a prefix block that is not full: the values of keys past the
  // prefix or on a bad page set to zero.  Their probabilities are zero already, but a
  // page tail may hold anything (a NaN or an infinity times zero would reach O).
  auto mask_v = [&](bf16x8 *vf, int kb) {
    const int pl = (kb - k_begin) >> 4;
    const bool pv0 = pages[pl] >= 0;
    const bool pv1 = (kb + 16 < k_end) && pages[pl + 1] >= 0;
    if (pv0 && pv1 && kb + kKB <= k_end) return;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const bool pok = ks == 0 ? pv0 : pv1;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        u32x4 w = __builtin_bit_cast(u32x4, vf[2 * t + ks]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int k0 = kb + 16 * ks + 8 * h + 2 * e;   // keys of this word's two values
          w[e] &= ((pok && k0 < k_end) ? 0x0000ffffu : 0u) | ((pok && k0 + 1 < k_end) ? 0xffff0000u : 0u);
        }
        vf[2 * t + ks] = __builtin_bit_cast(bf16x8, w);
      }
    }
  };

  // masking and the running maximum of one block's scores (may rescale O and l);
  // cand: a block of the candidates' own keys, else of the prefix
  auto softmax_max = [&](f32x16 &S, int kb, bool cand) {
    // block validity, uniform over the workgroup: a block of 32 in-range keys on two
    // valid pages needs no per-key mask
    int pv0 = 1, pv1 = 1;
    if (!cand) {
      const int pl = (kb - k_begin) >> 4;
      pv0 = pages[pl] >= 0;
      pv1 = (kb + 16 < k_end) ? (pages[pl + 1] >= 0) : 0;
    }
    const bool full = !cand && pv0 && pv1 && (kb + kKB <= k_end);
    if (!full) {
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int kpos = kb + 16 * (j >> 3) + 8 * h + (j & 7);
        bool v;
        if (cand)
          v = kpos < a.M && mrow < a.M && kpos / a.D == mrow / a.D && kpos <= mrow;
        else
          v = (j < 8 ? pv0 : pv1) && kpos < k_end;
        S[j] = v ? S[j] : -INFINITY;
      }
    }
    float bm = fmaxf(fmaxf(fmaxf(S[0], S[1]), fmaxf(S[2], S[3])),
                     fmaxf(fmaxf(S[4], S[5]), fmaxf(S[6], S[7])));
    bm = fmaxf(bm, fmaxf(fmaxf(fmaxf(S[8], S[9]), fmaxf(S[10], S[11])),
                         fmaxf(fmaxf(S[12], S[13]), fmaxf(S[14], S[15]))));
    const float bms = max_xor32(bm) * c;
    // lazy reference maximum: rescale only when a row outgrows it by more than kLazy
    const bool grow = bms > m_run + kLazy;
    if (__ballot(grow) != 0) {
      const float mn = grow ? bms : m_run;
      const float alpha = grow ? __builtin_amdgcn_exp2f(m_run - mn) : 1.f;
      l_part *= alpha;
#pragma unroll
      for (int t = 0; t < 4; ++t) O[t] *= alpha;
      m_run = mn;
    }
  };

  // probabilities of one block (P = hi + lo, both bf16: the PV product keeps ~16
  // significant bits of P) and its PV product
  auto softmax_pv = [&](const f32x16 &S, const bf16x8 *vf) {
    const float mref = (m_run == -INFINITY) ? 0.f : m_run;
    float p[16];
    float psum = 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      p[j] = __builtin_amdgcn_exp2f(fmaf(S[j], c, -mref));
      psum += p[j];
    }
    l_part += psum;
    uint32_t hk[8], lk[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) split_bf16x2(p[2 * e], p[2 * e + 1], hk[e], lk[e]);
    const bf16x8 ph0 = __builtin_bit_cast(bf16x8, u32x4{hk[0], hk[1], hk[2], hk[3]});
    const bf16x8 ph1 = __builtin_bit_cast(bf16x8, u32x4{hk[4], hk[5], hk[6], hk[7]});
    const bf16x8 pl0 = __builtin_bit_cast(bf16x8, u32x4{lk[0], lk[1], lk[2], lk[3]});
    const bf16x8 pl1 = __builtin_bit_cast(bf16x8, u32x4{lk[4], lk[5], lk[6], lk[7]});
    // the four head-dim tiles are independent accumulation chains: interleave them
#pragma unroll
    for (int t = 0; t < 4; ++t) O[t] = mfma32x32x16(vf[2 * t], ph0, O[t]);
#pragma unroll
    for (int t = 0; t < 4; ++t) O[t] = mfma32x32x16(vf[2 * t], pl0, O[t]);
#pragma unroll
    for (int t = 0; t < 4; ++t) O[t] = mfma32x32x16(vf[2 * t + 1], ph1, O[t]);
#pragma unroll
    for (int t = 0; t < 4; ++t) O[t] = mfma32x32x16(vf[2 * t + 1], pl1, O[t]);
  };

  // ring waits: all of this wave's transfers except those of the last n blocks issued
  auto wait_blocks = [&](int n) {
    if (n >= 2) {
      if (full_share) wait_vmcnt<2 * kIPW>();
      else wait_vmcnt<2 * (kIPW - 1)>();
    } else if (n == 1) {
      if (full_share) wait_vmcnt<kIPW>();
      else wait_vmcnt<kIPW - 1>();
    } else {
      wait_vmcnt<0>();
    }
  };

  // a wave whose 32 rows all lie past the KV head's rows (the padding of the last row
  // block) only moves its share of the blocks and keeps the barriers
  const bool idle = rb * a.rows_per_block + wv * kTileRows >= a.rows_per_kv;
  if (!is_cand && nblk > 0 && idle) {
#pragma unroll
    for (int j = 0; j < 3; ++j)
      if (j < nblk) issue_prefix(j, j);
    wait_blocks(min(nblk - 1, 2));
    __syncthreads();
    for (int j = 0; j < nblk; ++j) {
      wait_blocks(min(nblk - 1, j + 2) - (j + 1));
      __syncthreads();
      if (j + 3 < nblk) issue_prefix(j + 3, (j + 3) & 3);
    }
  } else if (!is_cand && nblk > 0) {
    // software pipeline over the ring: in iteration j block j+1's QK product is
    // interleaved with block j's softmax and PV product, and block j+3 is in flight
    static_assert(kNBuf == 4, "ring of four blocks");
#pragma unroll
    for (int j = 0; j < 3; ++j)
      if (j < nblk) issue_prefix(j, j);
    wait_blocks(min(nblk - 1, 2));   // block 0
    __syncthreads();
    f32x16 S_cur;
    {
      bf16x8 kf[8];
      load_k(0, kf);
      S_cur = qk_mma(kf);
    }
    for (int j = 0; j < nblk; ++j) {
      const int kb = k_begin + j * kKB;
      // block j+1 must have landed; the blocks issued after it may still be in flight
      wait_blocks(min(nblk - 1, j + 2) - (j + 1));
      __syncthreads();
      if (j + 3 < nblk) issue_prefix(j + 3, (j + 3) & 3);
      const bool more = j + 1 < nblk;
      bf16x8 kf[8], vf[8];
      load_k(more ? (j + 1) & 3 : j & 3, kf);
      load_v(j & 3, vf);
      mask_v(vf, kb);
      softmax_max(S_cur, kb, false);
      f32x16 S_next = qk_mma(kf);     // harmless recomputation on the last block
      softmax_pv(S_cur, vf);
      // issue order: QK products between the exponentials, PV products as P is ready
#pragma unroll
      for (int g8 = 0; g8 < 8; ++g8) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);   // five VALU
      }
#pragma unroll
      for (int g16 = 0; g16 < 16; ++g16) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
      }
      S_cur = S_next;
    }
  }
  if (is_cand || fold) {
    // the candidates' keys (after the prefix when folded: every wave is done reading
    // the ring before it is restaged)
    if (fold) __syncthreads();
    const int nc = (a.M + kKB - 1) / kKB;
    for (int j = 0; j < nc; ++j) {
      const int slot = j & 1;
      const int kb = j * kKB;
      stage_cand(slot, kb);
      __syncthreads();
      if (idle) continue;
      bf16x8 kf[8], vf[8];
      load_k(slot, kf);
      load_v(slot, vf);
      f32x16 S = qk_mma(kf);
      softmax_max(S, kb, true);
      softmax_pv(S, vf);
    }
  }

  // ---- finish: the row's sum over both lane halves, then final output or partials
  const float l = sum_xor32(l_part);
  if (!rok) return;
  // O^T register j of tile t: head dim 32t + 8*(j/4) + 4h + j%4
  if (fold || n_active == 1) {
    const float inv = l > 0.f ? 1.f / l : 0.f;
    bf16_t *op = a.out + layer * a.q_ls + (((int64_t)b * a.M + mrow) * a.Hq + hq) * kHD + 4 * h;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const uint32_t w0 = pack_bf16x2(O[t][4 * q4] * inv, O[t][4 * q4 + 1] * inv);
        const uint32_t w1 = pack_bf16x2(O[t][4 * q4 + 2] * inv, O[t][4 * q4 + 3] * inv);
        *(uint2 *)(op + 32 * t + 8 * q4) = make_uint2(w0, w1);
      }
  } else {
    const int row_in_block = wv * kTileRows + l32;
    const int64_t slot =
        (((int64_t)z * a.n_rb + rb) * n_sp + s) * a.rows_per_block + row_in_block;
    float *po = a.part_o + slot * kHD + 4 * h;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
        *(f32x4 *)(po + 32 * t + 8 * q4) =
            f32x4{O[t][4 * q4], O[t][4 * q4 + 1], O[t][4 * q4 + 2], O[t][4 * q4 + 3]};
    if (h == 0) *(float2 *)(a.part_ml + slot * 2) = make_float2(m_run, l);
  }
}

// Merge the split partials of every row in a fixed order (prefix splits ascending,
// then the candidate split): one pass over groups of eight splits, whose loads are
// independent, with the running maximum rescaled between groups.  One thread per
// (row, 4 head-dim values).
__global__ void __launch_bounds__(256)
attn_combine_kernel(AttnArgs a) {
  const int n_sp = a.n_splits + 1;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total_rows = (int64_t)a.L * a.B * a.Hkv * a.n_rb * a.rows_per_block;
  const int64_t row = gid / 32;
  const int c4 = (int)(gid % 32) * 4;
  if (row >= total_rows) return;
  const int row_in_block = (int)(row % a.rows_per_block);
  const int rb = (int)((row / a.rows_per_block) % a.n_rb);
  const int z = (int)(row / ((int64_t)a.rows_per_block * a.n_rb));   // (layer, b, kv head)
  const int layer = z / (a.B * a.Hkv);
  const int b = (z / a.Hkv) % a.B, kvh = z % a.Hkv;
  const int rr = rb * a.rows_per_block + row_in_block;
  if (rr >= a.rows_per_kv) return;
  bool badP = false;
  const int P = clamp_prefix(a.prefix_len[b], a.max_pages * kPage, &badP);
  const int n_pref = (P + a.split_keys - 1) / a.split_keys;
  if (n_pref == 0) return;  // the candidate split alone wrote the output
  const int n = n_pref + 1;
  const int64_t base = ((int64_t)z * a.n_rb + rb) * n_sp;
  float mx = -INFINITY, l = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int k0 = 0; k0 < n; k0 += 8) {
    float2 ml[8];
    f32x4 o[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int k = k0 + u;
      ml[u] = make_float2(-INFINITY, 0.f);
      o[u] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (k < n) {
        const int sp = (k == n_pref) ? a.n_splits : k;
        const int64_t slot = (base + sp) * a.rows_per_block + row_in_block;
        ml[u] = *(const float2 *)(a.part_ml + slot * 2);
        o[u] = *(const f32x4 *)(a.part_o + slot * kHD + c4);
      }
    }
    float gm = ml[0].x;
#pragma unroll
    for (int u = 1; u < 8; ++u) gm = fmaxf(gm, ml[u].x);
    const float mnew = fmaxf(mx, gm);
    if (mnew == -INFINITY) continue;     // no visible key so far
    const float sc = exp2f(mx - mnew);   // 0 while mx is still -inf
    acc *= sc;
    l *= sc;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const float w = exp2f(ml[u].x - mnew);
      acc += w * o[u];
      l += w * ml[u].y;
    }
    mx = mnew;
  }
  const float inv = l > 0.f ? 1.f / l : 0.f;
  const int m = rr / a.g;
  const int hq = kvh * a.g + rr % a.g;
  bf16_t *op = a.out + layer * a.q_ls + (((int64_t)b * a.M + m) * a.Hq + hq) * kHD + c4;
  *(uint2 *)op = make_uint2(pack_bf16x2(acc[0] * inv, acc[1] * inv),
                            pack_bf16x2(acc[2] * inv, acc[3] * inv));
}

// ---------------------------------------------------------------------------- fp32 path
// One wave per (sequence, row, query head).  Lane l takes keys l, l+64, ... with its own
// running max, sum and output accumulator; the 64 partial softmaxes are then merged
// across the wave.  Keys are independent across lanes, so the dependent chain of one
// lane is ceil(keys/64) long instead of keys long.
__device__ __forceinline__ float wave_max_f32(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

__device__ __forceinline__ float wave_sum_f32(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// The copy path's gate can ride in front: the first n_gate workgroups retrieve and gate
// one sequence each.
template <int HD>
__global__ void __launch_bounds__(256)
attn_f32_kernel(const float *q, const float *k_cand, const float *v_cand, const float *k_pool,
                const float *v_pool, const int32_t *page_table, const int32_t *prefix_len,
                float *out, int32_t *flags, int B, int W, int D, int Hq, int Hkv, int max_pages,
                int n_pool_pages, float scale, int n_gate, GateArgs gate, int L) {
  static_assert(HD <= 64, "one output element per lane");
  if ((int)blockIdx.x < n_gate) {
    __shared__ GateShared<256> gsh;
    gate_wg<256>(gate, blockIdx.x, gsh);
    return;
  }
  const int M = W * D;
  const int lane = threadIdx.x & 63;
  const int64_t task = (int64_t)((int)blockIdx.x - n_gate) * 4 + (threadIdx.x >> 6);
  const int64_t per_layer = (int64_t)B * M * Hq;
  if (task >= per_layer * L) return;     // uniform per wave
  const int hq = (int)(task % Hq);
  const int r = (int)((task / Hq) % M);
  const int b = (int)((task / ((int64_t)Hq * M)) % B);
  const int layer = (int)(task / per_layer);
  {
    const int64_t qs = per_layer * HD, cs = (int64_t)B * M * Hkv * HD;
    const int64_t ps = (int64_t)n_pool_pages * Hkv * kPage * HD;
    q += layer * qs;
    out += layer * qs;
    k_cand += layer * cs;
    v_cand += layer * cs;
    if (k_pool) k_pool += layer * ps;
    if (v_pool) v_pool += layer * ps;
  }
  const int kvh = hq / (Hq / Hkv);
  bool badP = false;
  const int P = clamp_prefix(prefix_len[b], max_pages * kPage, &badP);
  if (badP && flags && r == 0 && hq == 0 && layer == 0 && lane == 0) atomicOr(&flags[b], FLAG_BAD_PAGE);
  float qv[HD], acc[HD];
  const float *qp = q + (((int64_t)b * M + r) * Hq + hq) * HD;
#pragma unroll
  for (int e = 0; e < HD; ++e) {
    qv[e] = qp[e];
    acc[e] = 0.f;
  }
  float mx = -INFINITY, l = 0.f;
  const int i = r / D, o = r % D;
  const int nkeys = P + o + 1;
  for (int k = lane; k < nkeys; k += 64) {
    const float *kp, *vp;
    int vstride = 1;
    if (k < P) {
      const int pg = page_table[(int64_t)b * max_pages + k / kPage];
      if (pg < 0 || pg >= n_pool_pages) {
        if (flags && (k % kPage) == 0 && hq == 0 && layer == 0) atomicOr(&flags[b], FLAG_BAD_PAGE);
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
#pragma unroll
    for (int e = 0; e < HD; ++e) sdot = fmaf(qv[e], kp[e], sdot);
    sdot *= scale;
    const float mnew = fmaxf(mx, sdot);
    const float corr = expf(mx - mnew);
    const float p = expf(sdot - mnew);
    l = l * corr + p;
#pragma unroll
    for (int e = 0; e < HD; ++e) acc[e] = acc[e] * corr + p * vp[e * vstride];
    mx = mnew;
  }
  // merge the lanes' partial softmaxes (a lane without keys carries weight 0)
  const float gmax = wave_max_f32(mx);
  const float c = (mx == -INFINITY) ? 0.f : expf(mx - gmax);
  l = wave_sum_f32(l * c);
  const float inv = l > 0.f ? 1.f / l : 0.f;
  float *op = out + (((int64_t)b * M + r) * Hq + hq) * HD;
#pragma unroll
  for (int e = 0; e < HD; ++e) {
    const float v = wave_sum_f32(acc[e] * c);
    if (lane == e) op[e] = v * inv;
  }
}

__global__ void zero_i32_kernel(int32_t *p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

}  // namespace

bool attn_fuses_gate(int B, int W, int D, int Hq, int Hkv, int max_pages, int dtype) {
  return dtype == 0 || (dtype == 1 && attn_plan(B, W, D, Hq, Hkv, max_pages, kPage, 1).nw >= 4);
}

AttnPlan attn_plan(int B, int W, int D, int Hq, int Hkv, int max_pages, int page, int L) {
  AttnPlan p{};
  const int M = W * D;
  const int g = Hq / Hkv;
  p.rows_per_kv = g * M;
  p.rt = 1;
  const int tiles = (p.rows_per_kv + kTileRows - 1) / kTileRows;
  // row block: four waves (measured best at the Llama-8B/70B and batched shapes), fewer
  // when the KV head has fewer row tiles
  static const int kNW[] = {1, 2, 4, 5, 8};
  p.nw = tiles >= 4 ? 4 : (tiles >= 2 ? 2 : 1);
  // key splits: about 512 workgroups, at least 256 keys per split (128 for one-wave
  // row blocks), at most 1,280 in a batch
  const int max_keys = max_pages * page;
  int split_keys = 0;
  // tuning override "nw,split_keys" (values <= 0 keep the heuristic's choice)
  if (const char *ov = getenv("VSTEP_ATTN_PLAN")) {
    int nw = 0, sk = 0;
    if (sscanf(ov, "%d,%d", &nw, &sk) == 2) {
      for (int v : kNW)
        if (nw == v) p.nw = nw;
      if (sk > 0) split_keys = ((sk + kKB - 1) / kKB) * kKB;
    }
  }
  p.rows_per_block = p.nw * kTileRows;
  p.n_rb = (tiles + p.nw - 1) / p.nw;
  if (split_keys == 0) {
    const int groups = L * B * Hkv * p.n_rb;
    // one-wave workgroups leave room for many more per CU: their splits may be as
    // short as the 4-block ring (128 keys)
    const int min_keys = p.nw == 1 ? 128 : 256;
    if (B == 1) {
      // one sequence: all its splits are equally long, so one round of about 512
      // equal workgroups (two per CU; the candidates' short splits fill in behind)
      const int want = groups < 512 ? 512 / groups : 1;
      int sk = (max_keys + want - 1) / want;
      sk = ((sk + kKB - 1) / kKB) * kKB;
      split_keys = sk < min_keys ? min_keys : sk;
    } else {
      // a batch may be ragged: short splits keep the workgroups even (taken longest
      // first, 1,280 keys packed the 32-sequence ragged batch best: 1,024 / 1,280 /
      // 1,536 / 2,048 keys gave 176 / 167 / 180 / 176 us with the merge)
      const int want = (512 + groups - 1) / groups;
      int sk = (max_keys + want - 1) / want;
      sk = ((sk + kKB - 1) / kKB) * kKB;
      split_keys = sk < min_keys ? min_keys : (sk > 1280 ? 1280 : sk);
    }
  }
  if (split_keys > kMaxSplitPages * kPage) split_keys = kMaxSplitPages * kPage;
  p.split_keys = split_keys;
  p.n_splits = (max_keys + split_keys - 1) / split_keys;
  if (p.n_splits < 1) p.n_splits = 1;
  return p;
}

// partial slots of the split-K form (none when the one prefix split takes the candidates)
static size_t attn_slots(const AttnPlan &p, int B, int Hkv, int L) {
  if (p.n_splits == 1) return 0;
  return (size_t)L * B * Hkv * p.n_rb * (p.n_splits + 1) * p.rows_per_block;
}

size_t attn_workspace_bytes(int B, int W, int D, int Hq, int Hkv, int hd, int max_pages, int page,
                            int dtype, int L) {
  if (dtype != 1) return 0;
  const AttnPlan p = attn_plan(B, W, D, Hq, Hkv, max_pages, page, L);
  return attn_slots(p, B, Hkv, L) * (size_t)(kHD + 2) * sizeof(float) + 256;
}

hipError_t launch_attention(int B, int W, int D, int Hq, int Hkv, int hd, int max_pages,
                            int n_pool_pages, int dtype, float scale, const void *q,
                            const void *k_cand, const void *v_cand, const void *k_pool,
                            const void *v_pool, const int32_t *page_table,
                            const int32_t *prefix_len, void *out, int32_t *flags, void *ws,
                            hipStream_t st, const GateArgs *gate, int L) {
  const int M = W * D;
  if (L < 1) return hipErrorInvalidValue;
  if (dtype == 0) {
    const int64_t n = (int64_t)L * B * M * Hq;    // one wave each, four per workgroup
    const int n_gate = gate != nullptr ? B : 0;
    const int blocks = (int)((n + 3) / 4) + n_gate;
    const GateArgs ga = gate != nullptr ? *gate : GateArgs{};
#define VS_F32_ATTN(HDV)                                                                       \
  hipLaunchKernelGGL(attn_f32_kernel<HDV>, dim3(blocks), dim3(256), 0, st, (const float *)q,   \
                     (const float *)k_cand, (const float *)v_cand, (const float *)k_pool,      \
                     (const float *)v_pool, page_table, prefix_len, (float *)out, flags, B, W, \
                     D, Hq, Hkv, max_pages, n_pool_pages, scale, n_gate, ga, L)
    if (hd == 16) VS_F32_ATTN(16);
    else if (hd == 32) VS_F32_ATTN(32);
    else VS_F32_ATTN(64);
#undef VS_F32_ATTN
    return hipGetLastError();
  }
  const AttnPlan p = attn_plan(B, W, D, Hq, Hkv, max_pages, kPage, L);
  const bool fold = p.n_splits == 1;
  AttnArgs a;
  a.q = (const bf16_t *)q;
  a.k_cand = (const bf16_t *)k_cand;
  a.v_cand = (const bf16_t *)v_cand;
  a.k_pool = (const bf16_t *)k_pool;
  a.v_pool = (const bf16_t *)v_pool;
  a.page_table = page_table;
  a.prefix_len = prefix_len;
  a.out = (bf16_t *)out;
  const size_t slots = attn_slots(p, B, Hkv, L);
  a.part_o = (float *)ws;
  a.part_ml = a.part_o + slots * kHD;
  a.flags = flags;
  a.L = L;
  a.q_ls = (int64_t)B * M * Hq * kHD;
  a.c_ls = (int64_t)B * M * Hkv * kHD;
  a.p_ls = (int64_t)n_pool_pages * Hkv * kPage * kHD;
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
  a.n_gate = 0;
  if (gate != nullptr) {
    if (p.nw < 4) return hipErrorInvalidValue;
    a.n_gate = B;
    a.gate = *gate;
  }
  const int n_pairs = (fold ? 1 : p.n_splits + 1) * B * Hkv * L;
  {
    const char *mv = getenv("VSTEP_ATTN_MAP");
    a.grp_map = mv ? atoi(mv) : (B == 1 ? 1 : 3);
    if (a.grp_map < 0 || a.grp_map > 3) a.grp_map = 2;
    // the longest-first order ranks the sequences inside one wave; one split has no
    // order to choose
    if (a.grp_map == 3 && (B > 64 || fold)) a.grp_map = 2;
  }
  const int nblocks = a.grp_map ? 8 * p.n_rb * ((n_pairs + 7) / 8) : p.n_rb * n_pairs;
  const dim3 grid(nblocks + a.n_gate), block(64 * p.nw);
  switch (p.nw) {
    case 1: hipLaunchKernelGGL((attn_mfma_kernel<1>), grid, block, 0, st, a); break;
    case 2: hipLaunchKernelGGL((attn_mfma_kernel<2>), grid, block, 0, st, a); break;
    case 4: hipLaunchKernelGGL((attn_mfma_kernel<4>), grid, block, 0, st, a); break;
    case 5: hipLaunchKernelGGL((attn_mfma_kernel<5>), grid, block, 0, st, a); break;
    case 8: hipLaunchKernelGGL((attn_mfma_kernel<8>), grid, block, 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || fold) return e;
  const int64_t threads = (int64_t)L * B * Hkv * p.n_rb * p.rows_per_block * 32;
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
