// Copy-mode labels (SwitchSD summary, onedev.kr/papers/87, "어떻게 동작하나"): a token
// position is labelled 1 when it lies inside a verbatim run of at least kappa tokens
// that already appeared earlier in the same context.  A run of length >= kappa holds a
// kappa-gram at each offset, each of which also occurs earlier, so a position is
// labelled iff a kappa-gram window covering it occurs at an earlier start (the earlier
// occurrence may overlap the later one).
//
// Four launches over the flattened contexts, one thread per position:
//   1. check the offsets (non-decreasing inside the buffer) and clear the hash table;
//   2. insert every kappa-gram start into an open-addressing table keyed by (sequence,
//      kappa tokens): a slot is claimed by a 64-bit compare-and-swap of (sequence,
//      representative start) and keeps the smallest start of its gram (atomicMin);
//   3. R[s] = 1 iff the smallest start of s's gram is smaller than s;
//   4. label[p] = OR of R over the windows covering p.
// The table has at least twice as many slots as positions, so every probe sequence
// meets an empty slot; gram equality is checked on the tokens, never on the hash.

#include "vs_internal.hpp"

#include <limits.h>

#include <algorithm>

namespace vs {

namespace {

constexpr int kLT = 256;
constexpr uint64_t kEmpty = ~(uint64_t)0;

struct LabelArgs {
  const int32_t *ctx;
  const int32_t *ctx_off;
  int64_t total;
  int B, kappa;
  uint8_t *labels;
  int32_t *flags;
  unsigned long long *key;   // [S]: (sequence << 32) | representative start, or kEmpty
  int32_t *first;            // [S]: smallest start of the slot's gram
  uint8_t *rep;              // [total]: R
  int32_t *valid;            // one word
  uint32_t mask;             // S - 1
};

// the sequence holding position p (largest b with off[b] <= p), or -1 when p lies
// outside [off[0], off[B]); offsets already known to be non-decreasing
__device__ __forceinline__ int seq_of(const LabelArgs &a, int p, int &lo, int &hi) {
  if (p < a.ctx_off[0] || p >= a.ctx_off[a.B]) return -1;
  int l = 0, h = a.B;                    // off[l] <= p < off[h]
  while (h - l > 1) {
    const int m = (l + h) >> 1;
    if (a.ctx_off[m] <= p) l = m;
    else h = m;
  }
  lo = a.ctx_off[l];
  hi = a.ctx_off[l + 1];
  return l;
}

__device__ __forceinline__ uint32_t gram_hash(const int32_t *g, int kappa, int b) {
  uint64_t h = 0x9E3779B97F4A7C15ull ^ (uint64_t)(uint32_t)b;
  for (int i = 0; i < kappa; ++i) {
    h ^= (uint64_t)(uint32_t)g[i];
    h *= 0xBF58476D1CE4E5B9ull;
    h ^= h >> 31;
  }
  return (uint32_t)(h ^ (h >> 32));
}

__device__ __forceinline__ bool same_gram(const int32_t *x, const int32_t *y, int kappa) {
  bool eq = true;
  for (int i = 0; i < kappa; ++i) eq &= x[i] == y[i];
  return eq;
}

__global__ void __launch_bounds__(kLT)
labels_init_kernel(LabelArgs a) {
  const int64_t gid = (int64_t)blockIdx.x * kLT + threadIdx.x;
  const int64_t nslots = (int64_t)a.mask + 1;
  for (int64_t i = gid; i < nslots; i += (int64_t)gridDim.x * kLT) {
    a.key[i] = kEmpty;
    a.first[i] = INT_MAX;
  }
  if (blockIdx.x != 0) return;
  __shared__ int bad;
  if (threadIdx.x == 0)
    bad = (a.ctx_off[0] < 0 || (int64_t)a.ctx_off[a.B] > a.total) ? 1 : 0;
  __syncthreads();
  for (int b = threadIdx.x; b < a.B; b += kLT)
    if (a.ctx_off[b + 1] < a.ctx_off[b]) bad = 1;
  __syncthreads();
  if (threadIdx.x == 0) *a.valid = !bad;
  if (a.flags)
    for (int b = threadIdx.x; b < a.B; b += kLT) a.flags[b] = bad ? FLAG_BAD_CTX : 0;
}

__global__ void __launch_bounds__(kLT)
labels_insert_kernel(LabelArgs a) {
  if (!*a.valid) return;
  const int64_t s = (int64_t)blockIdx.x * kLT + threadIdx.x;
  if (s >= a.total) return;
  int lo, hi;
  const int b = seq_of(a, (int)s, lo, hi);
  if (b < 0 || s + a.kappa > hi) return;
  const int32_t *g = a.ctx + s;
  const unsigned long long mine = ((unsigned long long)(uint32_t)b << 32) | (uint32_t)s;
  uint32_t slot = gram_hash(g, a.kappa, b) & a.mask;
  for (uint32_t n = 0; n <= a.mask; ++n, slot = (slot + 1) & a.mask) {
    unsigned long long k = a.key[slot];
    if (k == kEmpty) {
      k = atomicCAS(&a.key[slot], kEmpty, mine);
      if (k == kEmpty) {
        atomicMin(&a.first[slot], (int)s);
        return;
      }
    }
    if ((int)(k >> 32) == b && same_gram(a.ctx + (uint32_t)k, g, a.kappa)) {
      atomicMin(&a.first[slot], (int)s);
      return;
    }
  }
}

__global__ void __launch_bounds__(kLT)
labels_query_kernel(LabelArgs a) {
  if (!*a.valid) return;
  const int64_t s = (int64_t)blockIdx.x * kLT + threadIdx.x;
  if (s >= a.total) return;
  int lo, hi;
  const int b = seq_of(a, (int)s, lo, hi);
  if (b < 0) return;
  uint8_t r = 0;
  if (s + a.kappa <= hi) {
    const int32_t *g = a.ctx + s;
    uint32_t slot = gram_hash(g, a.kappa, b) & a.mask;
    for (uint32_t n = 0; n <= a.mask; ++n, slot = (slot + 1) & a.mask) {
      const unsigned long long k = a.key[slot];
      if (k == kEmpty) break;            // not reached: s itself was inserted
      if ((int)(k >> 32) == b && same_gram(a.ctx + (uint32_t)k, g, a.kappa)) {
        r = a.first[slot] < (int)s ? 1 : 0;
        break;
      }
    }
  }
  a.rep[s] = r;
}

__global__ void __launch_bounds__(kLT)
labels_mark_kernel(LabelArgs a) {
  if (!*a.valid) return;
  const int64_t p = (int64_t)blockIdx.x * kLT + threadIdx.x;
  if (p >= a.total) return;
  int lo, hi;
  const int b = seq_of(a, (int)p, lo, hi);
  if (b < 0) return;
  const int s0 = max(lo, (int)p - a.kappa + 1);
  const int s1 = min((int)p, hi - a.kappa);
  uint8_t y = 0;
  for (int s = s0; s <= s1; ++s) y |= a.rep[s];
  a.labels[p] = y;
}

uint32_t label_slots(int64_t total) {
  uint64_t s = 1024;
  while (s < 2 * (uint64_t)total) s <<= 1;
  return (uint32_t)s;
}

}  // namespace

size_t labels_workspace_bytes(int64_t total) {
  const uint64_t S = label_slots(total);
  size_t off = 0;
  off += (S * 8 + 255) & ~(size_t)255;
  off += (S * 4 + 255) & ~(size_t)255;
  off += ((size_t)total + 255) & ~(size_t)255;
  off += 256;
  return off;
}

hipError_t launch_copy_labels(const int32_t *ctx, int64_t total, const int32_t *ctx_off, int B,
                              int kappa, uint8_t *labels, int32_t *flags, void *ws,
                              hipStream_t st) {
  const uint64_t S = label_slots(total);
  char *p = (char *)ws;
  LabelArgs a;
  a.ctx = ctx;
  a.ctx_off = ctx_off;
  a.total = total;
  a.B = B;
  a.kappa = kappa;
  a.labels = labels;
  a.flags = flags;
  a.key = (unsigned long long *)p;
  p += (S * 8 + 255) & ~(size_t)255;
  a.first = (int32_t *)p;
  p += (S * 4 + 255) & ~(size_t)255;
  a.rep = (uint8_t *)p;
  p += ((size_t)total + 255) & ~(size_t)255;
  a.valid = (int32_t *)p;
  a.mask = (uint32_t)(S - 1);
  const int init_blocks = (int)std::min<uint64_t>((S + kLT - 1) / kLT, 2048);
  hipLaunchKernelGGL(labels_init_kernel, dim3(init_blocks), dim3(kLT), 0, st, a);
  if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  if (total == 0) return hipSuccess;
  const unsigned blocks = (unsigned)((total + kLT - 1) / kLT);
  hipLaunchKernelGGL(labels_insert_kernel, dim3(blocks), dim3(kLT), 0, st, a);
  if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  hipLaunchKernelGGL(labels_query_kernel, dim3(blocks), dim3(kLT), 0, st, a);
  if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  hipLaunchKernelGGL(labels_mark_kernel, dim3(blocks), dim3(kLT), 0, st, a);
  return hipGetLastError();
}

}  // namespace vs
