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

// Block scan of a 64-bit word that packs four 16-bit counters (no carries cross
// a field as long as every field's block total stays below 65536).  Returns the exclusive prefix of
// `v` and writes the block total to *total.  `scratch` (NT/64 words) is written once and read after
// the one barrier; the caller gives every scan of a kernel its own scratch.
template <int NT>
__device__ __forceinline__ uint64_t block_scan_packed(uint64_t v, uint64_t* scratch, uint64_t* total) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  uint64_t incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint64_t u = __shfl_up(incl, o, 64);
    if (lane >= o) incl += u;
  }
  if (lane == 63) scratch[wave] = incl;
  __syncthreads();
  uint64_t wbase = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    const uint64_t s = scratch[i];
    wbase += (i < wave) ? s : 0;
    tot += s;
  }
  *total = tot;
  return wbase + incl - v;
}

__device__ __forceinline__ int field16(uint64_t w, int j) { return (int)((w >> (16 * j)) & 0xFFFFu); }

// sum of fields 0 .. j-1
__device__ __forceinline__ int fields_below(uint64_t w, int j) {
  int s = 0;
#pragma unroll
  for (int i = 0; i < 3; ++i) s += i < j ? field16(w, i) : 0;
  return s;
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
  static constexpr int NW = NT / 64;
  static constexpr int R = NW;     // histogram copies: lane l counts into copy l % R
  static constexpr int RP = 257;   // copy stride in ints: the copies of one bin sit in different banks
  int hist[2][R * RP];             // two sets, used on alternate passes
  alignas(16) int cnt[2][256];     // per-pass bin totals
  uint32_t red[2 * NW];
  uint64_t scan[2][NW];
};

// The K best of the c visible scores srow[0..c) (c > K, c <= NT * KPT; the row holds T >= c
// scores), ties to the lower position, emitted in ascending position order as
// put(slot, position + offset), slot 0..K-1.  Every thread of the NT-thread block calls it.
//
// Thread t keeps KPT scores in registers as order-preserving 32-bit keys (a larger float gives a
// larger key; -0.0 is folded onto +0.0): J chunks of E consecutive positions, chunk j covering
// positions E*(NT*j + t) .. +E-1, so the loads of a wave are contiguous and vectorised.  A radix
// select finds the key of the K-th best score, 8 bits per pass, starting at the highest bit where
// the row's keys differ, and stops early once the chosen bin holds exactly the keys still to be
// taken.  Each pass counts into R copies of the histogram (lane l into copy l % R, so keys that
// share a bin, as whole exponent ranges do in the first pass, spread their atomics over R
// addresses) and costs two barriers.  Then one pass over the registers keeps every key above the
// threshold and, of the keys equal to it, the lowest positions (ranked by a packed block scan that
// is skipped when the select stopped early: then every equal key is kept); a second packed scan
// gives each kept position its slot.
template <int NT, int KPT, typename Put>
__device__ __forceinline__ void block_topk(const float* __restrict__ srow, int T, int c, int K, int offset,
                                           TopkSmem<NT>& sm, Put put) {
  constexpr int NW = NT / 64;
  constexpr int R = TopkSmem<NT>::R;
  constexpr int RP = TopkSmem<NT>::RP;
  constexpr int J = KPT < 4 ? KPT : 4;  // chunks per thread (one 16-bit field each in the scans)
  constexpr int E = KPT / J;            // consecutive positions per chunk
  static_assert(J * E == KPT && E <= 16, "KPT is 1, 2, 4 or a multiple of 4 up to 64");
  static_assert(E * NT < 65536, "a chunk's block total fits a 16-bit field");
  using Bits = typename std::conditional<(KPT > 32), uint64_t, uint32_t>::type;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  uint32_t key[KPT];
  // loads first, then branch-free keys, so the loads overlap.  Vector loads need whole chunks
  // inside the row (T a multiple of E) and an aligned row; a chunk past c reads chunk 0 instead.
  constexpr int VA = E >= 4 ? 16 : 4 * E;
  const bool vec = E > 1 && T % E == 0 && (reinterpret_cast<uintptr_t>(srow) & (VA - 1)) == 0;
  if (vec) {
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int p0 = E * (NT * j + tid);
      const float* src = srow + (p0 < c ? p0 : 0);
      if constexpr (E >= 4) {
#pragma unroll
        for (int q = 0; q < E / 4; ++q) {
          const float4 v = *reinterpret_cast<const float4*>(src + 4 * q);
          key[j * E + 4 * q + 0] = __float_as_uint(v.x);
          key[j * E + 4 * q + 1] = __float_as_uint(v.y);
          key[j * E + 4 * q + 2] = __float_as_uint(v.z);
          key[j * E + 4 * q + 3] = __float_as_uint(v.w);
        }
      } else {
        const float2 v = *reinterpret_cast<const float2*>(src);
        key[j * E + 0] = __float_as_uint(v.x);
        key[j * E + 1] = __float_as_uint(v.y);
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < J; ++j)
#pragma unroll
      for (int e = 0; e < E; ++e) key[j * E + e] = __float_as_uint(srow[min(E * (NT * j + tid) + e, c - 1)]);
  }
  // this pass's histogram set starts at zero (the other set is cleared during the first pass)
  for (int i = tid; i < R * RP; i += NT) sm.hist[0][i] = 0;
  uint32_t kand = 0xFFFFFFFFu, kor = 0u;
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    const bool vis = E * (NT * (i / E) + tid) + i % E < c;
    const uint32_t k = order_key(__uint_as_float(key[i]));
    key[i] = vis ? k : 0u;  // invisible: below every real key
    kand &= vis ? k : 0xFFFFFFFFu;
    kor |= vis ? k : 0u;
  }
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) {
    kand &= __shfl_xor(kand, m, 64);
    kor |= __shfl_xor(kor, m, 64);
  }
  if (lane == 0) {
    sm.red[2 * wave] = kand;
    sm.red[2 * wave + 1] = kor;
  }
  __syncthreads();
  uint32_t all_and = 0xFFFFFFFFu, all_or = 0u;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    all_and &= sm.red[2 * i];
    all_or |= sm.red[2 * i + 1];
  }
  const uint32_t diff = all_and ^ all_or;  // bits that differ among the visible keys

  uint32_t prefix = all_and & ~diff;  // bits shared by every visible key
  uint32_t mask = ~diff;              // bits already fixed
  int remaining = K;                  // how many of the keys matching `prefix` are still to be taken
  bool exact = false;                 // exactly `remaining` visible keys match `prefix` under `mask`
  if (diff != 0u) {
    int hb = 31 - __builtin_clz(diff);  // highest differing bit
    int set = 0;
    while (true) {
      const int lo = hb >= 7 ? hb - 7 : 0;
      const int width = hb - lo + 1;
      const uint32_t dmask = ((width == 32) ? 0xFFFFFFFFu : ((1u << width) - 1u)) << lo;
      int* h = sm.hist[set] + (lane & (R - 1)) * RP;
#pragma unroll
      for (int i = 0; i < KPT; ++i) {
        const bool vis = E * (NT * (i / E) + tid) + i % E < c;
        if (vis && (key[i] & mask) == prefix) atomicAdd(&h[(key[i] & dmask) >> lo], 1);
      }
      __syncthreads();
      // bin totals of this pass; the other set, last read before this pass's counting, is cleared
      // for the next pass
      if (tid < 256) {
        int s = 0;
#pragma unroll
        for (int r = 0; r < R; ++r) s += sm.hist[set][r * RP + tid];
        sm.cnt[set][tid] = s;
      }
      for (int i = tid; i < R * RP; i += NT) sm.hist[set ^ 1][i] = 0;
      __syncthreads();
      // every wave picks the digit: lane l scans digits 255-4l .. 252-4l (largest first)
      const int4 h4 = *reinterpret_cast<const int4*>(&sm.cnt[set][252 - 4 * lane]);
      const int c0 = h4.w, c1 = h4.z, c2 = h4.y, c3 = h4.x;
      const int mine = c0 + c1 + c2 + c3;
      int incl = mine;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int u = __shfl_up(incl, o, 64);
        if (lane >= o) incl += u;
      }
      const int excl = incl - mine;  // keys in digits above this lane's four
      const uint64_t hit = __builtin_amdgcn_ballot_w64(excl < remaining && incl >= remaining);
      const int src = __builtin_ctzll(hit);
      int digit = 0, above = 0, in_digit = 0;
      if (lane == src) {
        int a = excl;
        if (a + c0 >= remaining) {
          digit = 255 - 4 * lane;
          in_digit = c0;
        } else if ((a += c0) + c1 >= remaining) {
          digit = 254 - 4 * lane;
          in_digit = c1;
        } else if ((a += c1) + c2 >= remaining) {
          digit = 253 - 4 * lane;
          in_digit = c2;
        } else {
          a += c2;
          digit = 252 - 4 * lane;
          in_digit = c3;
        }
        above = a;
      }
      digit = __shfl(digit, src, 64);
      above = __shfl(above, src, 64);
      in_digit = __shfl(in_digit, src, 64);
      remaining -= above;
      prefix |= ((uint32_t)digit << lo);
      mask |= dmask;
      set ^= 1;
      if (in_digit == remaining) {
        exact = true;  // every key of the chosen digit is taken
        break;
      }
      if (lo == 0) break;
      hb = lo - 1;
    }
  }
  // Under `mask` (the bits fixed so far), `prefix` is the K-th best visible key: keep the keys above
  // it and the first `remaining` keys equal to it in position order
  const uint32_t tau = prefix;
  int eq_base[J];
#pragma unroll
  for (int j = 0; j < J; ++j) eq_base[j] = 0;
  if (!exact) {
    uint64_t eqw = 0;
#pragma unroll
    for (int j = 0; j < J; ++j) {
      int n = 0;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const int i = j * E + e;
        n += (E * (NT * j + tid) + e < c && (key[i] & mask) == tau) ? 1 : 0;
      }
      eqw |= (uint64_t)n << (16 * j);
    }
    uint64_t eq_tot;
    const uint64_t eq_before = block_scan_packed<NT>(eqw, sm.scan[0], &eq_tot);
#pragma unroll
    for (int j = 0; j < J; ++j) eq_base[j] = fields_below(eq_tot, j) + field16(eq_before, j);
  }
  Bits keep_bits = 0u;
  uint64_t kw = 0;
#pragma unroll
  for (int j = 0; j < J; ++j) {
    int rank = eq_base[j], n = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int i = j * E + e;
      const bool vis = E * (NT * j + tid) + e < c;
      const uint32_t mk = key[i] & mask;
      bool k = vis && mk > tau;
      if (vis && mk == tau) {
        k = exact || rank < remaining;
        ++rank;
      }
      if (k) {
        keep_bits |= (Bits)1 << i;
        ++n;
      }
    }
    kw |= (uint64_t)n << (16 * j);
  }
  uint64_t k_tot;
  const uint64_t k_before = block_scan_packed<NT>(kw, sm.scan[1], &k_tot);
#pragma unroll
  for (int j = 0; j < J; ++j) {
    int slot = fields_below(k_tot, j) + field16(k_before, j);
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int i = j * E + e;
      if (((keep_bits >> i) & 1u) && slot < K) put(slot++, E * (NT * j + tid) + e + offset);
    }
  }
}

}  // namespace topk_dev
}  // namespace dsa
