// KV commit and rollback over the paged cache.
//
// The rejection-sampling blog (blog.huny.dev), section 6: once a draft is verified,
// the KV blocks of the rejected tokens go back to the paged pool at once and none
// may leak.  Here the candidates' K/V live in their own buffers during the verify
// step, so the step itself leaves the cache untouched; afterwards
//   * commit appends each sequence's accepted rows (candidate `best`, rows 0..a-1)
//     to its cache, taking new pages off a free-page stack, and
//   * truncate rolls a sequence back to a shorter length, pushing the pages past it
//     back onto the stack.
// Pages are taken and returned in a fixed order (sequence order, then page order),
// so the page ids every sequence receives do not depend on scheduling.
//
// Layout (as the attention kernels read it): K pages [page][kv head][16][hd], V pages
// transposed [page][kv head][hd][16].
//
// Each call is a planning workgroup (the sequences' page needs, a serial pass that
// assigns stack positions, then the page-table updates, all in LDS) and, for commit,
// a copy kernel of one workgroup per (accepted row, sequence).

#include "vs_internal.hpp"

namespace vs {

namespace {

constexpr int kKT = 256;
constexpr int kPg = 16;
constexpr int kPreload = 4096;       // free-stack entries the planner holds in LDS

enum : int { ST_NONE = 0, ST_COMMIT = 1, ST_EMPTY = 2, ST_BAD = 3 };

struct KvShared {
  int st[kMaxSeqKv];     // state of each sequence
  int need[kMaxSeqKv];   // pages to take (commit) or to return (truncate)
  int off[kMaxSeqKv];    // stack position of its first page, relative to the call's start
  int top[kPreload];     // commit: free_list[n_free0 - 1 - k] (the pop order)
  int n_free0, n_free1;
};

__device__ __forceinline__ int pages_for(int n) { return (n + kPg - 1) / kPg; }

struct CommitArgs {
  int B, W, D, max_pages, n_pool_pages;
  const int32_t *best, *n_acc;
  int32_t *page_table, *prefix_len, *free_list, *n_free, *flags;
  int32_t *plan;         // [B][3]: (P, a, best) of a committed sequence; a = 0 otherwise
};

__global__ void __launch_bounds__(kKT)
kv_commit_plan_kernel(CommitArgs a) {
  __shared__ KvShared sh;
  const int tid = threadIdx.x;
  if (tid == 0) sh.n_free0 = *a.n_free;
  __syncthreads();
  // a stack count outside [0, n_pool_pages] is not read from: every request is refused
  const bool stack_ok = sh.n_free0 >= 0 && sh.n_free0 <= a.n_pool_pages;
  // ---- every sequence's request, in parallel
  for (int b = tid; b < a.B; b += kKT) {
    const int i = a.best[b];
    int n = a.n_acc[b];
    n = n < 0 ? 0 : (n > a.D ? a.D : n);
    int st = ST_NONE, need = 0;
    if (i >= 0 && i < a.W && n > 0) {
      const int P = a.prefix_len[b];
      if (P < 0 || P + n > a.max_pages * kPg) {
        st = ST_BAD;
      } else {
        const int have = pages_for(P);
        need = pages_for(P + n) - have;
        st = stack_ok ? ST_COMMIT : ST_BAD;
        if (P % kPg) {
          const int pg = a.page_table[(int64_t)b * a.max_pages + have - 1];
          if (pg < 0 || pg >= a.n_pool_pages) st = ST_BAD;
        }
      }
    }
    sh.st[b] = st;
    sh.need[b] = need;
  }
  __syncthreads();
  const int n0 = stack_ok ? sh.n_free0 : 0;
  for (int k = tid; k < kPreload && k < n0; k += kKT) sh.top[k] = a.free_list[n0 - 1 - k];
  __syncthreads();
  // ---- stack positions, in sequence order (one thread; every read is from LDS
  //      except pops past the preloaded part of the stack)
  if (tid == 0) {
    int taken = 0;
    for (int b = 0; b < a.B; ++b) {
      if (sh.st[b] != ST_COMMIT) continue;
      const int need = sh.need[b];
      if (need > n0 - taken) {
        sh.st[b] = ST_EMPTY;
        continue;
      }
      bool ok = true;
      for (int k = 0; k < need; ++k) {
        const int pos = taken + k;
        const int pg = pos < kPreload ? sh.top[pos] : a.free_list[n0 - 1 - pos];
        ok &= pg >= 0 && pg < a.n_pool_pages;
      }
      if (!ok) {
        sh.st[b] = ST_BAD;
        continue;
      }
      sh.off[b] = taken;
      taken += need;
    }
    sh.n_free1 = stack_ok ? n0 - taken : sh.n_free0;
  }
  __syncthreads();
  // ---- page tables, lengths, plan, flags
  for (int b = tid; b < a.B; b += kKT) {
    const int st = sh.st[b];
    int32_t *pl = a.plan + 3 * b;
    if (st == ST_COMMIT) {
      const int P = a.prefix_len[b];
      int n = a.n_acc[b];
      n = n > a.D ? a.D : n;
      const int have = pages_for(P);
      for (int k = 0; k < sh.need[b]; ++k) {
        const int pos = sh.off[b] + k;
        a.page_table[(int64_t)b * a.max_pages + have + k] =
            pos < kPreload ? sh.top[pos] : a.free_list[n0 - 1 - pos];
      }
      a.prefix_len[b] = P + n;
      pl[0] = P;
      pl[1] = n;
      pl[2] = a.best[b];
    } else {
      pl[0] = 0;
      pl[1] = 0;
      pl[2] = 0;
    }
    if (a.flags)
      a.flags[b] = st == ST_EMPTY ? FLAG_POOL_EMPTY : (st == ST_BAD ? FLAG_BAD_PAGE : 0);
  }
  if (tid == 0) *a.n_free = sh.n_free1;
}

// One workgroup per (row o, sequence b, layer): row (b, best, o) of the layer's
// candidate K/V goes to token P + o of the layer's pool (the page table is shared by
// every layer).  E = element type of the model tensors (bf16 bits or fp32).
template <typename E>
__global__ void __launch_bounds__(kKT)
kv_copy_kernel(const E *k_cand, const E *v_cand, E *k_pool, E *v_pool,
               const int32_t *page_table, const int32_t *plan, int W, int D, int Hkv, int hd,
               int max_pages, int64_t cand_ls, int64_t pool_ls) {
  const int o = blockIdx.x;
  const int b = blockIdx.y;
  const int64_t layer = blockIdx.z;
  k_cand += layer * cand_ls;
  v_cand += layer * cand_ls;
  k_pool += layer * pool_ls;
  v_pool += layer * pool_ls;
  const int32_t *pl = plan + 3 * b;
  if (o >= pl[1]) return;
  const int pos = pl[0] + o;
  const int pg = page_table[(int64_t)b * max_pages + pos / kPg];
  const int t = pos % kPg;
  const int64_t src = (((int64_t)b * W + pl[2]) * D + o) * Hkv * hd;
  for (int e = threadIdx.x; e < Hkv * hd; e += kKT) {
    const int kvh = e / hd, d = e % hd;
    k_pool[(((int64_t)pg * Hkv + kvh) * kPg + t) * hd + d] = k_cand[src + e];
    v_pool[(((int64_t)pg * Hkv + kvh) * hd + d) * kPg + t] = v_cand[src + e];
  }
}

struct TruncArgs {
  int B, max_pages, n_pool_pages;
  const int32_t *new_len;
  int32_t *page_table, *prefix_len, *free_list, *n_free, *flags;
};

__global__ void __launch_bounds__(kKT)
kv_truncate_kernel(TruncArgs a) {
  __shared__ KvShared sh;
  const int tid = threadIdx.x;
  if (tid == 0) sh.n_free0 = *a.n_free;
  __syncthreads();
  const bool stack_ok = sh.n_free0 >= 0 && sh.n_free0 <= a.n_pool_pages;
  for (int b = tid; b < a.B; b += kKT) {
    const int P = a.prefix_len[b], L = a.new_len[b];
    int st = ST_COMMIT, cnt = 0;
    if (!stack_ok || P < 0 || P > a.max_pages * kPg || L < 0 || L > P) {
      st = ST_BAD;
    } else {
      const int keep = pages_for(L), have = pages_for(P);
      cnt = have - keep;
      for (int j = keep; j < have; ++j) {
        const int pg = a.page_table[(int64_t)b * a.max_pages + j];
        if (pg < 0 || pg >= a.n_pool_pages) st = ST_BAD;
      }
    }
    sh.st[b] = st;
    sh.need[b] = cnt;
  }
  __syncthreads();
  if (tid == 0) {
    int pushed = 0;
    const int n0 = sh.n_free0;
    for (int b = 0; b < a.B; ++b) {
      if (sh.st[b] != ST_COMMIT) continue;
      if (n0 + pushed + sh.need[b] > a.n_pool_pages) {
        sh.st[b] = ST_BAD;
        continue;
      }
      sh.off[b] = pushed;
      pushed += sh.need[b];
    }
    sh.n_free1 = n0 + pushed;
  }
  __syncthreads();
  for (int b = tid; b < a.B; b += kKT) {
    const int st = sh.st[b];
    if (st == ST_COMMIT) {
      const int L = a.new_len[b];
      const int keep = pages_for(L);
      int32_t *pt = a.page_table + (int64_t)b * a.max_pages;
      for (int k = 0; k < sh.need[b]; ++k) {
        a.free_list[sh.n_free0 + sh.off[b] + k] = pt[keep + k];
        pt[keep + k] = -1;
      }
      a.prefix_len[b] = L;
    }
    if (a.flags) a.flags[b] = st == ST_BAD ? FLAG_BAD_PAGE : 0;
  }
  if (tid == 0) *a.n_free = sh.n_free1;
}

}  // namespace

size_t kv_workspace_bytes(int B) { return (((size_t)B * 3 * sizeof(int32_t)) + 255) & ~(size_t)255; }

hipError_t launch_kv_commit(int B, int W, int D, int Hkv, int hd, int max_pages, int n_pool_pages,
                            int esz, const void *k_cand, const void *v_cand, const int32_t *best,
                            const int32_t *n_acc, void *k_pool, void *v_pool, int32_t *page_table,
                            int32_t *prefix_len, int32_t *free_list, int32_t *n_free,
                            int32_t *flags, void *ws, hipStream_t st, int L) {
  if (L < 1 || L > 65535) return hipErrorInvalidValue;
  CommitArgs a;
  a.B = B;
  a.W = W;
  a.D = D;
  a.max_pages = max_pages;
  a.n_pool_pages = n_pool_pages;
  a.best = best;
  a.n_acc = n_acc;
  a.page_table = page_table;
  a.prefix_len = prefix_len;
  a.free_list = free_list;
  a.n_free = n_free;
  a.flags = flags;
  a.plan = (int32_t *)ws;
  hipLaunchKernelGGL(kv_commit_plan_kernel, dim3(1), dim3(kKT), 0, st, a);
  if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  const dim3 grid(D, B, L);
  const int64_t cand_ls = (int64_t)B * W * D * Hkv * hd;
  const int64_t pool_ls = (int64_t)n_pool_pages * Hkv * kPg * hd;
  if (esz == 2)
    hipLaunchKernelGGL(kv_copy_kernel<uint16_t>, grid, dim3(kKT), 0, st,
                       (const uint16_t *)k_cand, (const uint16_t *)v_cand, (uint16_t *)k_pool,
                       (uint16_t *)v_pool, page_table, a.plan, W, D, Hkv, hd, max_pages, cand_ls,
                       pool_ls);
  else
    hipLaunchKernelGGL(kv_copy_kernel<uint32_t>, grid, dim3(kKT), 0, st,
                       (const uint32_t *)k_cand, (const uint32_t *)v_cand, (uint32_t *)k_pool,
                       (uint32_t *)v_pool, page_table, a.plan, W, D, Hkv, hd, max_pages, cand_ls,
                       pool_ls);
  return hipGetLastError();
}

hipError_t launch_kv_truncate(int B, int max_pages, int n_pool_pages, const int32_t *new_len,
                              int32_t *page_table, int32_t *prefix_len, int32_t *free_list,
                              int32_t *n_free, int32_t *flags, hipStream_t st) {
  TruncArgs a;
  a.B = B;
  a.max_pages = max_pages;
  a.n_pool_pages = n_pool_pages;
  a.new_len = new_len;
  a.page_table = page_table;
  a.prefix_len = prefix_len;
  a.free_list = free_list;
  a.n_free = n_free;
  a.flags = flags;
  hipLaunchKernelGGL(kv_truncate_kernel, dim3(1), dim3(kKT), 0, st, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------
// Token-major K/V (the layout a cache written token by token has: [tokens][kv head][hd],
// pages of 16 tokens one after another) into the pages the verify step reads: K
// [page][kv head][16][hd] and V [page][kv head][hd][16].  One workgroup per (page, kv
// head); V goes through LDS to be transposed.  Positions at or past n_tokens in the last
// page are written as zero.
namespace {
template <typename T>
__global__ void __launch_bounds__(kKT)
kv_pack_kernel(const T *k_src, const T *v_src, int64_t n_tokens, int Hkv, int hd, T *k_pool,
               T *v_pool) {
  extern __shared__ unsigned char pack_lds[];
  T *tile = reinterpret_cast<T *>(pack_lds);   // [16][hd]
  const int64_t pg = blockIdx.x;
  const int kvh = blockIdx.y;
  const int tid = threadIdx.x;
  const int n = kPg * hd;
  T *kd = k_pool + (pg * Hkv + kvh) * (int64_t)n;
  for (int i = tid; i < n; i += kKT) {
    const int t = i / hd, e = i % hd;
    const int64_t tok = pg * kPg + t;
    const T kv = tok < n_tokens ? k_src[(tok * Hkv + kvh) * hd + e] : T(0);
    kd[i] = kv;                                   // K keeps the token-major order of a page
    tile[i] = tok < n_tokens ? v_src[(tok * Hkv + kvh) * hd + e] : T(0);
  }
  __syncthreads();
  T *vd = v_pool + (pg * Hkv + kvh) * (int64_t)n;
  for (int i = tid; i < n; i += kKT) {
    const int e = i / kPg, t = i % kPg;
    vd[i] = tile[t * hd + e];                     // V^T: the 16 tokens of one coordinate
  }
}

}  // namespace

hipError_t launch_kv_pack(const void *k_src, const void *v_src, int64_t n_tokens, int Hkv, int hd,
                          int esz, void *k_pool, void *v_pool, hipStream_t st) {
  const int64_t n_pages = (n_tokens + kPg - 1) / kPg;
  if (n_pages <= 0) return hipSuccess;
  const dim3 grid((unsigned)n_pages, (unsigned)Hkv);
  const size_t lds = (size_t)kPg * hd * esz;
  if (esz == 2)
    hipLaunchKernelGGL(kv_pack_kernel<uint16_t>, grid, dim3(kKT), lds, st, (const uint16_t *)k_src,
                       (const uint16_t *)v_src, n_tokens, Hkv, hd, (uint16_t *)k_pool,
                       (uint16_t *)v_pool);
  else
    hipLaunchKernelGGL(kv_pack_kernel<float>, grid, dim3(kKT), lds, st, (const float *)k_src,
                       (const float *)v_src, n_tokens, Hkv, hd, (float *)k_pool, (float *)v_pool);
  return hipGetLastError();
}

}  // namespace vs
