// Block-wide pieces of the top-k selection of the sparse attention step (DeepSeek V4.1 page,
// `Indexer.forward`: top-k by score, re-sorted into position order, unreachable -> -1, the rest
// shifted by `offset`) and the window part of an index row (`get_window_topk_idxs`), shared by
// the top-k kernels and the decode attention kernel that selects its own index rows.
#pragma once
#include <type_traits>

#include "dsa_internal.h"

namespace dsa {
namespace topk_dev {

__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;  // -0.0 == +0.0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive prefix sum over the block (blockDim.x threads, multiple of 64); returns the
// exclusive prefix of `v` and writes the block total to *total.
template <int NT>
__device__ __forceinline__ int block_exclusive_scan(int v, int* scratch /* NT/64 + 1 ints */, int* total) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(incl, o, 64);
    if (lane >= o) incl += u;
  }
  if (lane == 63) scratch[wave] = incl;
  __syncthreads();
  int wbase = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    const int s = scratch[i];
    wbase += (i < wave) ? s : 0;
    tot += s;
  }
  __syncthreads();
  *total = tot;
  return wbase + incl - v;
}

template <int NT>
__device__ __forceinline__ uint32_t block_reduce_and_or(uint32_t a, uint32_t o, uint32_t* scratch, uint32_t* out_or) {
  constexpr int NW = NT / 64;
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) {
    a &= __shfl_xor(a, m, 64);
    o |= __shfl_xor(o, m, 64);
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) {
    scratch[2 * wave] = a;
    scratch[2 * wave + 1] = o;
  }
  __syncthreads();
  uint32_t ra = 0xFFFFFFFFu, ro = 0u;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    ra &= scratch[2 * i];
    ro |= scratch[2 * i + 1];
  }
  __syncthreads();
  *out_or = ro;
  return ra;
}

// Entry s of query t's window row (`get_window_topk_idxs`): chunk positions in prefill
// (start_pos == 0), ring slots oldest first in decode; -1 past the query / for an unfilled slot.
__device__ __forceinline__ int window_entry(int t, int s, int start_pos, int W) {
  if (start_pos == 0) {
    const int first = t - W + 1 > 0 ? t - W + 1 : 0;
    const int pos = first + s;
    return pos <= t ? pos : -1;
  }
  const int oldest = start_pos % W + 1;
  const int slot = oldest + s < W ? oldest + s : oldest + s - W;
  return slot <= start_pos ? slot : -1;
}

template <int NT>
struct TopkSmem {
  int hist[256];
  int scan[NT / 64 + 2];
  uint32_t red[2 * (NT / 64)];
  int sel[3];
};

// The K best of the c visible scores srow[0..c) (c > K, c <= NT * KPT), ties to the lower
// position, emitted in ascending position order as put(slot, position + offset), slot 0..K-1.
// Every thread of the NT-thread block calls it.  Thread i keeps the scores of positions
// KPT*i .. KPT*i + KPT-1 in registers as order-preserving 32-bit keys (a larger float gives a
// larger key; -0.0 is folded onto +0.0).  A radix select finds the key of the K-th best score,
// 8 bits per pass, starting at the highest bit where the row's keys differ (so the first histogram
// already spreads the keys over many bins instead of piling onto one exponent).  Then one pass over
// the registers keeps every key above that threshold and, of the keys equal to it, the lowest
// positions; block prefix sums over the per-thread counts give each kept position its slot.  The
// select stops early once the chosen bin holds exactly the keys still to be taken.
template <int NT, int KPT, typename Put>
__device__ __forceinline__ void block_topk(const float* __restrict__ srow, int c, int K, int offset,
                                           TopkSmem<NT>& sm, Put put) {
  static_assert(KPT <= 64, "one keep bit per key in a 64-bit mask");
  using Bits = typename std::conditional<(KPT > 32), uint64_t, uint32_t>::type;
  const int tid = threadIdx.x;
  const int jbase = tid * KPT;
  uint32_t key[KPT];
  // loads first (clamped, always in bounds), then branch-free keys, so the loads overlap
#pragma unroll
  for (int i = 0; i < KPT; ++i) key[i] = __float_as_uint(srow[min(jbase + i, c - 1)]);
  uint32_t kand = 0xFFFFFFFFu, kor = 0u;
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    const bool vis = jbase + i < c;
    const uint32_t k = order_key(__uint_as_float(key[i]));
    key[i] = vis ? k : 0u;  // invisible: below every real key
    kand &= vis ? k : 0xFFFFFFFFu;
    kor |= vis ? k : 0u;
  }
  uint32_t all_or;
  const uint32_t all_and = block_reduce_and_or<NT>(kand, kor, sm.red, &all_or);
  const uint32_t diff = all_and ^ all_or;  // bits that differ among the visible keys

  uint32_t prefix = all_and & ~diff;  // bits shared by every visible key
  uint32_t mask = ~diff;              // bits already fixed
  int remaining = K;                  // how many of the keys matching `prefix` are still to be taken
  if (diff != 0u) {
    int hb = 31 - __builtin_clz(diff);  // highest differing bit
    while (true) {
      const int lo = hb >= 7 ? hb - 7 : 0;
      const int width = hb - lo + 1;
      const uint32_t dmask = ((width == 32) ? 0xFFFFFFFFu : ((1u << width) - 1u)) << lo;
      for (int i = tid; i < 256; i += NT) sm.hist[i] = 0;
      __syncthreads();
#pragma unroll
      for (int i = 0; i < KPT; ++i) {
        if (jbase + i < c && (key[i] & mask) == prefix) atomicAdd(&sm.hist[(key[i] & dmask) >> lo], 1);
      }
      __syncthreads();
      // suffix counts over the bins (largest digit first): thread i takes bin 255 - i
      const int bin = 255 - (tid & 255);
      const int cnt = tid < 256 ? sm.hist[bin] : 0;
      int tot;
      const int excl = block_exclusive_scan<NT>(cnt, sm.scan, &tot);  // keys in bins above `bin`
      if (tid < 256 && excl < remaining && excl + cnt >= remaining) {
        sm.sel[0] = bin;
        sm.sel[1] = excl;
        sm.sel[2] = cnt;
      }
      __syncthreads();
      const int sbin = sm.sel[0];
      remaining -= sm.sel[1];
      const int in_bin = sm.sel[2];
      prefix |= ((uint32_t)sbin << lo);
      mask |= dmask;
      __syncthreads();
      // every key of the chosen bin is taken: the bits fixed so far decide the whole selection
      if (lo == 0 || in_bin == remaining) break;
      hb = lo - 1;
    }
  }
  // Under `mask` (the bits fixed so far), `prefix` is the K-th best visible key: keep keys above it
  // and the first `remaining` keys equal to it in position order (all of them when the select
  // stopped early, as then exactly `remaining` keys are equal to it)
  const uint32_t tau = prefix;
  int n_eq = 0;
#pragma unroll
  for (int i = 0; i < KPT; ++i) n_eq += (jbase + i < c && (key[i] & mask) == tau) ? 1 : 0;
  int tot_eq;
  int eq_before = block_exclusive_scan<NT>(n_eq, sm.scan, &tot_eq);
  int n_keep = 0;
  Bits keep_bits = 0u;
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    const bool vis = jbase + i < c;
    const uint32_t mk = key[i] & mask;
    bool k = vis && mk > tau;
    if (vis && mk == tau) {
      k = eq_before < remaining;
      ++eq_before;
    }
    if (k) {
      keep_bits |= (Bits)1 << i;
      ++n_keep;
    }
  }
  int tot_keep;
  int pos = block_exclusive_scan<NT>(n_keep, sm.scan, &tot_keep);
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    if (((keep_bits >> i) & 1u) && pos < K) put(pos++, jbase + i + offset);
  }
}

}  // namespace topk_dev
}  // namespace dsa
