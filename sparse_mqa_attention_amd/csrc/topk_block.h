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

// Raw bits of the E consecutive scores of a chunk starting at p0 (a chunk past c reads the row's
// start instead, so every load stays inside the row).  Vector loads need whole chunks inside the
// row (T a multiple of E) and an aligned row.  CO: 8-byte device-scope loads (past the CU's L1).
template <int E, bool CO>
__device__ __forceinline__ void load_chunk(const float* __restrict__ srow, int p0, int c, bool vec,
                                           uint32_t (&k)[E]) {
  if (vec) {
    const float* src = srow + (p0 < c ? p0 : 0);
    if constexpr (CO) {
#pragma unroll
      for (int q = 0; q < E / 2; ++q) {
        const uint64_t v = __hip_atomic_load(reinterpret_cast<const uint64_t*>(src + 2 * q), __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT);
        k[2 * q + 0] = (uint32_t)v;
        k[2 * q + 1] = (uint32_t)(v >> 32);
      }
    } else if constexpr (E >= 4) {
#pragma unroll
      for (int q = 0; q < E / 4; ++q) {
        const float4 v = *reinterpret_cast<const float4*>(src + 4 * q);
        k[4 * q + 0] = __float_as_uint(v.x);
        k[4 * q + 1] = __float_as_uint(v.y);
        k[4 * q + 2] = __float_as_uint(v.z);
        k[4 * q + 3] = __float_as_uint(v.w);
      }
    } else if constexpr (E == 2) {
      const float2 v = *reinterpret_cast<const float2*>(src);
      k[0] = __float_as_uint(v.x);
      k[1] = __float_as_uint(v.y);
    } else {
      k[0] = __float_as_uint(src[0]);
    }
  } else {
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const float* src = srow + min(p0 + e, c - 1);
      k[e] = CO ? __hip_atomic_load(reinterpret_cast<const uint32_t*>(src), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                : __float_as_uint(*src);
    }
  }
}

// The K best of the c visible scores srow[0..c) (c > K, c <= NT * KPT; the row holds T >= c
// scores), ties to the lower position, emitted in ascending position order as
// put(slot, position + offset), slot 0..K-1.  Every thread of the NT-thread block calls it.
//
// Thread t holds KPT scores as order-preserving 32-bit keys (a larger float gives a larger key;
// -0.0 is folded onto +0.0): J chunks of E consecutive positions, chunk j covering positions
// E*(NT*j + t) .. +E-1, so the loads of a wave are contiguous and vectorised.  A radix select finds
// the key of the K-th best score, 8 bits per pass, starting at the highest bit where the row's keys
// differ, and stops early once the chosen bin holds exactly the keys still to be taken.  Each pass
// counts into R copies of the histogram (lane l into copy l % R, so keys that share a bin, as whole
// exponent ranges do in the first pass, spread their atomics over R addresses) and costs two
// barriers.  Then one pass over the keys keeps every key above the threshold and, of the keys equal
// to it, the lowest positions (ranked by a packed block scan that is skipped when the select stopped
// early: then every equal key is kept); a second packed scan gives each kept position its slot.
//
// Up to 32 keys per thread stay in registers for the whole select.  64 keys per thread (rows of up
// to 65536 scores at 1024 threads) would not fit the 128 registers a thread has at that block size,
// so then each pass re-reads its chunk's scores from the row (L2-resident after the first pass)
// and only one chunk's keys are live at a time.
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
  constexpr bool ST = KPT > 32;         // keys re-read per pass instead of held in registers
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
  constexpr int VA = E >= 4 ? 16 : 4 * E;
  const bool vec = E > 1 && T % E == 0 && (reinterpret_cast<uintptr_t>(srow) & (VA - 1)) == 0;
  // order keys of chunk j (0 for an invisible position, below every real key)
  auto to_keys = [&](int j, uint32_t (&k)[E]) {
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const bool vis = E * (NT * j + tid) + e < c;
      k[e] = vis ? order_key(__uint_as_float(k[e])) : 0u;
    }
  };
  uint32_t key[ST ? 1 : KPT];  // all keys (held mode)
  // the keys of chunk j in kc: from the registers, or re-read from the row
  auto chunk_keys = [&](int j, uint32_t (&kc)[E]) {
    if constexpr (ST) {
      // an offset the compiler cannot see through, so the re-reads stay in their pass instead of
      // being hoisted out of the pass loop (which would hold every key again)
      int z = 0;
      asm volatile("" : "+v"(z));
      load_chunk<E, CO>(srow + z, E * (NT * j + tid), c, vec, kc);
      to_keys(j, kc);
    } else {
#pragma unroll
      for (int e = 0; e < E; ++e) kc[e] = key[j * E + e];
    }
  };
  if constexpr (!ST) {
    // loads first, then branch-free keys, so the loads overlap
#pragma unroll
    for (int j = 0; j < J; ++j) {
      uint32_t kc[E];
      load_chunk<E, CO>(srow, E * (NT * j + tid), c, vec, kc);
#pragma unroll
      for (int e = 0; e < E; ++e) key[j * E + e] = kc[e];
    }
  }
  // this pass's histogram set starts at zero (the other set is cleared during the first pass)
  for (int i = tid; i < R * RP / 4; i += NT) reinterpret_cast<int4*>(sm.hist[0])[i] = int4{0, 0, 0, 0};
  uint32_t kand = 0xFFFFFFFFu, kor = 0u;
  auto and_or_chunk = [&](int j) {
    uint32_t kc[E];
    if constexpr (ST) {
      load_chunk<E, CO>(srow, E * (NT * j + tid), c, vec, kc);
    } else {
#pragma unroll
      for (int e = 0; e < E; ++e) kc[e] = key[j * E + e];
    }
    to_keys(j, kc);
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const bool vis = E * (NT * j + tid) + e < c;
      if constexpr (!ST) key[j * E + e] = kc[e];
      kand &= vis ? kc[e] : 0xFFFFFFFFu;
      kor |= vis ? kc[e] : 0u;
    }
  };
  if constexpr (ST) {
#pragma unroll 1
    for (int j = 0; j < J; ++j) and_or_chunk(j);
  } else {
#pragma unroll
    for (int j = 0; j < J; ++j) and_or_chunk(j);
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
      auto count_chunk = [&](int j) {
        uint32_t kc[E];
        chunk_keys(j, kc);
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const bool vis = E * (NT * j + tid) + e < c;
          if (vis && (kc[e] & mask) == prefix) atomicAdd(&h[(kc[e] & dmask) >> lo], 1);
        }
      };
      if constexpr (ST) {
#pragma unroll 1
        for (int j = 0; j < J; ++j) count_chunk(j);  // one chunk's loads in flight at a time
      } else {
#pragma unroll
        for (int j = 0; j < J; ++j) count_chunk(j);
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
  // rank of this thread's first key equal to tau in chunk j among all such keys (0 when exact:
  // then every equal key is kept and no ranks are needed)
  uint64_t eq_tot = 0, eq_before = 0;
  if (!exact) {
    uint64_t eqw = 0;
    auto eq_chunk = [&](int j) {
      uint32_t kc[E];
      chunk_keys(j, kc);
      int n = 0;
#pragma unroll
      for (int e = 0; e < E; ++e) n += (E * (NT * j + tid) + e < c && (kc[e] & mask) == tau) ? 1 : 0;
      eqw |= (uint64_t)n << (16 * j);
    };
    if constexpr (ST) {
#pragma unroll 1
      for (int j = 0; j < J; ++j) eq_chunk(j);
    } else {
#pragma unroll
      for (int j = 0; j < J; ++j) eq_chunk(j);
    }
    eq_before = block_scan_packed<NT>(eqw, sm.scan[0], &eq_tot);
  }
  Bits keep_bits = 0u;
  auto keep_chunk = [&](int j) {
    uint32_t kc[E];
    chunk_keys(j, kc);
    int rank = exact ? 0 : fields_below(eq_tot, j) + field16(eq_before, j);
    Bits kb = 0u;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const bool vis = E * (NT * j + tid) + e < c;
      const uint32_t mk = kc[e] & mask;
      bool k;
      if (exact) {  // every key at or above the threshold is taken
        k = vis && mk >= tau;
      } else {
        k = vis && mk > tau;
        if (vis && mk == tau) {
          k = rank < remaining;
          ++rank;
        }
      }
      kb |= k ? (Bits)1 << e : (Bits)0;
    }
    keep_bits |= kb << (j * E);
  };
  if constexpr (ST) {
#pragma unroll 1
    for (int j = 0; j < J; ++j) keep_chunk(j);
  } else {
#pragma unroll
    for (int j = 0; j < J; ++j) keep_chunk(j);
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
