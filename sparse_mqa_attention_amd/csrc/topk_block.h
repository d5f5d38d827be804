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

// Inclusive prefix over the 64 lanes of a wave: DPP shifts within each row of 16 lanes, then the
// row broadcasts of lanes 15 and 31 carry the row totals up (rows the mask leaves out keep x).
__device__ __forceinline__ uint32_t wave_incl_sum(uint32_t x) {
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xf, 0xf, false);  // row_shr:1
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xf, 0xf, false);  // row_shr:2
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xf, 0xf, false);  // row_shr:4
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xf, 0xf, false);  // row_shr:8
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xa, 0xf, false);  // row_bcast:15
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return x;
}

// AND and OR of the wave's values (lane 63 of the inclusive prefix), uniform
__device__ __forceinline__ void wave_and_or(uint32_t& a, uint32_t& o) {
  a &= (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)a, 0x111, 0xf, 0xf, false);
  o |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)o, 0x111, 0xf, 0xf, false);
  a &= (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)a, 0x112, 0xf, 0xf, false);
  o |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)o, 0x112, 0xf, 0xf, false);
  a &= (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)a, 0x114, 0xf, 0xf, false);
  o |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)o, 0x114, 0xf, 0xf, false);
  a &= (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)a, 0x118, 0xf, 0xf, false);
  o |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)o, 0x118, 0xf, 0xf, false);
  a &= (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)a, 0x142, 0xa, 0xf, false);
  o |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)o, 0x142, 0xa, 0xf, false);
  a &= (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)a, 0x143, 0xc, 0xf, false);
  o |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)o, 0x143, 0xc, 0xf, false);
  a = (uint32_t)__builtin_amdgcn_readlane((int)a, 63);
  o = (uint32_t)__builtin_amdgcn_readlane((int)o, 63);
}

// Block scan of a 64-bit word that packs four 16-bit counters (no carry crosses a field as long as
// every field's block total stays below 65536, so the two 32-bit halves scan apart).  Returns the
// exclusive prefix of `v` and writes the block total to *total.  `scratch` (NT/64 words) is
// written once and read after the one barrier; each scan of a kernel gets its own scratch.
template <int NT>
__device__ __forceinline__ uint64_t block_scan_packed(uint64_t v, uint64_t* scratch, uint64_t* total) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const uint64_t incl = ((uint64_t)wave_incl_sum((uint32_t)(v >> 32)) << 32) | wave_incl_sum((uint32_t)v);
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
  alignas(16) int hist[2][R * RP]; // two sets, used on alternate passes
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
//
// CO = true reads the scores at device scope (past the CU's L1), for rows that other workgroups
// wrote during the same launch.
template <int NT, int KPT, bool CO = false, typename Put>
__device__ __forceinline__ void block_topk(const float* __restrict__ srow, int T, int c, int K, int offset,
                                           TopkSmem<NT>& sm, Put put) {
  constexpr int NW = NT / 64;
  constexpr int R = TopkSmem<NT>::R;
  constexpr int RP = TopkSmem<NT>::RP;
  constexpr int J = KPT < 4 ? KPT : 4;  // chunks per thread (one 16-bit field each in the scans)
  constexpr int E = KPT / J;            // consecutive positions per chunk
  static_assert(J * E == KPT && E <= 16, "KPT is 1, 2, 4 or a multiple of 4 up to 64");
  // one thread per histogram bin totals each pass: with fewer than 256 threads the upper bins
  // would keep stale counts, the select could keep more than K keys and put() would be handed
  // slots past K
  static_assert(NT >= 256 && NT % 64 == 0, "block_topk needs at least 256 threads");
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
      if constexpr (CO) {  // 8-byte device-scope loads
#pragma unroll
        for (int q = 0; q < E / 2; ++q) {
          const uint64_t v = __hip_atomic_load(reinterpret_cast<const uint64_t*>(src + 2 * q), __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT);
          key[j * E + 2 * q + 0] = (uint32_t)v;
          key[j * E + 2 * q + 1] = (uint32_t)(v >> 32);
        }
      } else if constexpr (E >= 4) {
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
      for (int e = 0; e < E; ++e) {
        const float* src = srow + min(E * (NT * j + tid) + e, c - 1);
        key[j * E + e] = CO ? __hip_atomic_load(reinterpret_cast<const uint32_t*>(src), __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT)
                            : __float_as_uint(*src);
      }
  }
  // this pass's histogram set starts at zero (the other set is cleared during the first pass)
  for (int i = tid; i < R * RP / 4; i += NT) reinterpret_cast<int4*>(sm.hist[0])[i] = int4{0, 0, 0, 0};
  uint32_t kand = 0xFFFFFFFFu, kor = 0u;
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    const bool vis = E * (NT * (i / E) + tid) + i % E < c;
    const uint32_t k = order_key(__uint_as_float(key[i]));
    key[i] = vis ? k : 0u;  // invisible: below every real key
    kand &= vis ? k : 0xFFFFFFFFu;
    kor |= vis ? k : 0u;
  }
  wave_and_or(kand, kor);
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
      for (int i = tid; i < R * RP / 4; i += NT) reinterpret_cast<int4*>(sm.hist[set ^ 1])[i] = int4{0, 0, 0, 0};
      __syncthreads();
      // every wave picks the digit: lane l scans digits 255-4l .. 252-4l (largest first)
      const int4 h4 = *reinterpret_cast<const int4*>(&sm.cnt[set][252 - 4 * lane]);
      const int c0 = h4.w, c1 = h4.z, c2 = h4.y, c3 = h4.x;
      const int mine = c0 + c1 + c2 + c3;
      const int incl = (int)wave_incl_sum((uint32_t)mine);
      const int excl = incl - mine;  // keys in digits above this lane's four
      // the one lane whose four digits hold the `remaining`-th key; every lane works out its own
      // candidate and the answer is read from that lane
      const int src = __builtin_ctzll(__builtin_amdgcn_ballot_w64(excl < remaining && incl >= remaining));
      const int a1 = excl + c0, a2 = a1 + c1, a3 = a2 + c2;
      const int sub = a1 >= remaining ? 0 : a2 >= remaining ? 1 : a3 >= remaining ? 2 : 3;
      const int above_l = sub == 0 ? excl : sub == 1 ? a1 : sub == 2 ? a2 : a3;
      const int in_l = sub == 0 ? c0 : sub == 1 ? c1 : sub == 2 ? c2 : c3;
      const int digit = __builtin_amdgcn_readlane(255 - 4 * lane - sub, src);
      const int above = __builtin_amdgcn_readlane(above_l, src);
      const int in_digit = __builtin_amdgcn_readlane(in_l, src);
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
  if (exact) {  // every key at or above the threshold is taken
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const bool vis = E * (NT * (i / E) + tid) + i % E < c;
      keep_bits |= (vis && (key[i] & mask) >= tau) ? (Bits)1 << i : (Bits)0;
    }
  } else {
#pragma unroll
    for (int j = 0; j < J; ++j) {
      int rank = eq_base[j];
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const int i = j * E + e;
        const bool vis = E * (NT * j + tid) + e < c;
        const uint32_t mk = key[i] & mask;
        bool k = vis && mk > tau;
        if (vis && mk == tau) {
          k = rank < remaining;
          ++rank;
        }
        keep_bits |= k ? (Bits)1 << i : (Bits)0;
      }
    }
  }
  constexpr uint32_t CM = (1u << E) - 1u;  // one chunk's bits
  uint64_t kw = 0;
#pragma unroll
  for (int j = 0; j < J; ++j) kw |= (uint64_t)__builtin_popcount((uint32_t)(keep_bits >> (j * E)) & CM) << (16 * j);
  uint64_t k_tot;
  const uint64_t k_before = block_scan_packed<NT>(kw, sm.scan[1], &k_tot);
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const uint32_t cb = (uint32_t)(keep_bits >> (j * E)) & CM;
    const int base = fields_below(k_tot, j) + field16(k_before, j);
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int slot = base + __builtin_popcount(cb & ((1u << e) - 1u));
      if (((cb >> e) & 1u) && slot < K) put(slot, E * (NT * j + tid) + e + offset);
    }
  }
}

}  // namespace topk_dev
}  // namespace dsa
