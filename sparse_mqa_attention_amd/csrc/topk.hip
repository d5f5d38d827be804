// Top-k selection and window index rows of the sparse attention step.
//
// Top-k (DeepSeek V4.1 page, `Indexer.forward`: top-k by score, re-sorted into position order,
// unreachable -> -1, the rest shifted by `offset`): one workgroup per query row.  Each thread
// keeps KPT consecutive scores in registers as order-preserving 32-bit keys (a larger float gives
// a larger key; -0.0 is folded onto +0.0).  A radix select finds the key of the n-th best visible
// score, 8 bits per pass, starting at the highest bit where the row's keys differ (so the first
// histogram already spreads the keys over many bins instead of piling onto one exponent).  Then
// one pass over the registers keeps every key above that threshold and, of the keys equal to it,
// the lowest positions; block prefix sums over the per-thread counts give each kept position its
// output slot, so the row comes out in ascending position order without a sort.  Rows that see
// at most K positions need no scores at all: they are 0..c-1 followed by -1.
//
// Window rows (`get_window_topk_idxs`): a direct formula per entry.
#include "topk_block.h"

namespace dsa {

namespace {

using namespace topk_dev;

template <int NT, int KPT>
__global__ void __launch_bounds__(NT)
topk_kernel(const float* __restrict__ scores, int S, int T, int K, int start_pos, int ratio, int offset,
            int32_t* __restrict__ idx, int64_t ld_idx, int row0, int W, int Wc) {
  __shared__ TopkSmem<NT> sm;

  const int row = row0 + blockIdx.x;  // b*S + t
  const int t = row % S;
  const int tid = threadIdx.x;
  const int c = min(T, visible_rows(start_pos, t, ratio));
  for (int s = tid; s < Wc; s += NT) idx[(int64_t)row * ld_idx + s] = window_entry(t, s, start_pos, W);
  int32_t* out = idx + (int64_t)row * ld_idx + Wc;

  if (c <= K) {  // every visible position is kept
    for (int s = tid; s < K; s += NT) out[s] = s < c ? s + offset : -1;
    return;
  }
  // n = K here: exactly K positions are kept and no -1 is written
  block_topk<NT, KPT>(scores + (int64_t)row * T, T, c, K, offset, sm, [&](int slot, int v) { out[slot] = v; });
}

// Long rows of few queries (decode at long context): the select is split over the chunks of each
// row.  Stage 1: workgroup (g, row) keeps the K best visible scores of positions
// [g*kChunk, (g+1)*kChunk) as candidates (scores and positions, in ascending position order,
// padded with -inf / -1 to K), or all of them when the chunk has at most K visible positions.
// The K best of the row are among the chunks' K best (a position beaten by K others in its own
// chunk cannot be among the row's K best), so stage 2 selects the K best of the G*K candidates;
// chunks and each chunk's candidates are in position order, so ties between equal scores still
// go to the lower position.
constexpr int kChunk = 4096;  // positions per stage-1 workgroup: 256 threads x 16 keys

__global__ void __launch_bounds__(256)
topk_split_chunk_kernel(const float* __restrict__ scores, int S, int T, int K, int start_pos, int ratio, int G,
                        float* __restrict__ cand_s, int32_t* __restrict__ cand_p) {
  __shared__ TopkSmem<256> sm;
  const int g = blockIdx.x;
  const int row = blockIdx.y;  // b*S + t
  const int tid = threadIdx.x;
  const int c = min(T, visible_rows(start_pos, row % S, ratio));
  if (c <= K) return;  // the merge writes such rows without candidates
  const int p0 = g * kChunk;
  if (p0 >= c) return;  // chunks past the visible positions hold no candidates
  const int cg = min(kChunk, c - p0);
  float* cs = cand_s + ((int64_t)row * G + g) * K;
  int32_t* cp = cand_p + ((int64_t)row * G + g) * K;
  const float* srow = scores + (int64_t)row * T + p0;
  if (cg <= K) {
    for (int s = tid; s < K; s += 256) {
      cs[s] = s < cg ? srow[s] : -__builtin_inff();
      cp[s] = s < cg ? p0 + s : -1;
    }
    return;
  }
  block_topk<256, 16>(srow, T - p0, cg, K, 0, sm, [&](int slot, int v) {
    cs[slot] = srow[v];
    cp[slot] = p0 + v;
  });
}

// Stage 2: the row's window entries, then its K best candidates (their positions + offset) in
// ascending position order; rows with at most K visible positions as in topk_kernel.
template <int NT, int KPT>
__global__ void __launch_bounds__(NT)
topk_split_merge_kernel(const float* __restrict__ cand_s, const int32_t* __restrict__ cand_p, int G, int S, int T,
                        int K, int start_pos, int ratio, int offset, int32_t* __restrict__ idx, int64_t ld_idx, int W,
                        int Wc) {
  __shared__ TopkSmem<NT> sm;
  const int row = blockIdx.x;
  const int t = row % S;
  const int tid = threadIdx.x;
  const int c = min(T, visible_rows(start_pos, t, ratio));
  for (int s = tid; s < Wc; s += NT) idx[(int64_t)row * ld_idx + s] = window_entry(t, s, start_pos, W);
  int32_t* out = idx + (int64_t)row * ld_idx + Wc;
  if (c <= K) {
    for (int s = tid; s < K; s += NT) out[s] = s < c ? s + offset : -1;
    return;
  }
  const int n = (c + kChunk - 1) / kChunk * K;  // candidates of the chunks holding visible positions
  const int32_t* cp = cand_p + (int64_t)row * G * K;
  if (n <= K) {  // one chunk holds every visible position: its K candidates are the answer
    for (int s = tid; s < K; s += NT) out[s] = cp[s] + offset;
    return;
  }
  block_topk<NT, KPT>(cand_s + (int64_t)row * G * K, n, n, K, 0, sm,
                      [&](int slot, int i) { out[slot] = cp[i] + offset; });
}

// Candidate blocks of the two-level selection (`Indexer.forward` with a candidate source:
// `select_candidate_blocks` picks the source layer's best blocks of compressed positions; its body
// is not on the pages, so a block scores its largest visible score, a block is visible when its
// first position is, and the best n_sel visible blocks are kept, ties to the lower block).  One
// workgroup per query: block maxima into LDS, the block select of the top-k on them, and the chosen
// blocks as a bitmap row (bit i of word i/32).
constexpr int kCandMaxBlocks = 8192;

__global__ void __launch_bounds__(1024)
candidate_blocks_kernel(const float* __restrict__ scores, int S, int T, int start_pos, int ratio, int lbs, int n_sel,
                        uint32_t* __restrict__ bits, int64_t ld_bits) {
  __shared__ TopkSmem<1024> sm;
  __shared__ __attribute__((aligned(16))) float bmax[kCandMaxBlocks];
  __shared__ uint32_t bw[kCandMaxBlocks / 32];
  const int row = blockIdx.x;
  const int tid = threadIdx.x;
  const int bs = 1 << lbs;
  const int c = min(T, visible_rows(start_pos, row % S, ratio));
  const int nblk = (T + bs - 1) >> lbs;
  const int cb = (c + bs - 1) >> lbs;  // visible blocks
  const int nw = (nblk + 31) >> 5;
  for (int i = tid; i < nw; i += 1024) bw[i] = 0u;
  const float* srow = scores + (int64_t)row * T;
  // whole visible blocks of 4k positions in 16-byte loads (consecutive threads, consecutive blocks),
  // the rest one score at a time
  const bool vec = lbs >= 2 && (T & 3) == 0 && ((uintptr_t)srow & 15) == 0;
  const int full = vec ? c >> lbs : 0;  // blocks wholly visible
  for (int i = tid; i < full; i += 1024) {
    const float4* p = reinterpret_cast<const float4*>(srow + (i << lbs));
    float4 v = p[0];
    float m = fmaxf(fmaxf(v.x, v.y), fmaxf(v.z, v.w));
    for (int k = 1; k < (1 << (lbs - 2)); ++k) {
      v = p[k];
      m = fmaxf(m, fmaxf(fmaxf(v.x, v.y), fmaxf(v.z, v.w)));
    }
    bmax[i] = m;
  }
  for (int i = full + tid; i < cb; i += 1024) {
    const int e = min((i + 1) << lbs, c);
    float m = srow[i << lbs];
    for (int j = (i << lbs) + 1; j < e; ++j) m = fmaxf(m, srow[j]);
    bmax[i] = m;
  }
  __syncthreads();
  if (cb <= n_sel) {
    for (int i = tid; i < cb; i += 1024) atomicOr(&bw[i >> 5], 1u << (i & 31));
  } else {
    block_topk<1024, 8>(bmax, cb, cb, n_sel, 0, sm, [&](int slot, int i) { atomicOr(&bw[i >> 5], 1u << (i & 31)); });
  }
  __syncthreads();
  for (int i = tid; i < nw; i += 1024) bits[(int64_t)row * ld_bits + i] = bw[i];
}

// Many rows (prefill): one wave per row and no workgroup barriers.  Lane l holds the keys of
// positions 64g + l (g < KPL) in registers (invisible positions get key 0, below every real
// key).  The radix select takes 8-bit digits, from the highest bit where the row's keys differ,
// through a wave-private 256-bin LDS histogram kept in kWR copies (lane l counts into copy
// l % kWR, the copies kWP ints apart so one bin's copies sit in different banks: the first pass
// sees whole exponent ranges share a bin, and atomics to one address serialise).  It stops as
// soon as the chosen digit holds exactly the keys still to be taken.  The kept positions leave in
// ascending order through ballot/mbcnt prefix counts per group g, which also hand the ties at the
// threshold to the lowest positions.
constexpr int kWR = 4;    // histogram copies per wave
constexpr int kWP = 257;  // ints between copies

// Order-preserving key of a score for the one-wave kernel, in three VALU operations: a
// non-negative float u maps to u + 2^31, a negative one to -u (two's complement), which sends -0.0
// to the key of +0.0 with no compare.  Every float maps to a key >= 1, so 0 stays free to mark an
// invisible position.
__device__ __forceinline__ uint32_t wave_key(uint32_t u) {
  const uint32_t s = (uint32_t)((int32_t)u >> 31);
  return (u ^ (s | 0x80000000u)) - s;
}

// Three waves per SIMD (at most 168 VGPRs): with 8192 keys a row (128 per lane) a few values
// spill to scratch outside the per-key loops, and the third wave hides more of the score loads
// (15% faster than two).
template <int KPL>
__global__ void __launch_bounds__(256, 3)
topk_wave_kernel(const float* __restrict__ scores, int rows, int S, int T, int K, int start_pos, int ratio,
                 int offset, int32_t* __restrict__ idx, int64_t ld_idx, int W, int Wc) {
  static_assert(KPL % 16 == 0, "blocks of 16 groups");
  __shared__ int whist[4][kWR * kWP];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // b*S + t, the last rows (most visible positions) first; wave-uniform, no workgroup barrier below
  const int row = rows - 1 - (blockIdx.x * 4 + wave);
  if (row < 0) return;
  int* hist = whist[wave];
  const int t = row % S;
  const int c = min(T, visible_rows(start_pos, t, ratio));
  for (int s = lane; s < Wc; s += 64) idx[(int64_t)row * ld_idx + s] = window_entry(t, s, start_pos, W);
  int32_t* out = idx + (int64_t)row * ld_idx + Wc;

  if (c <= K) {  // every visible position is kept
    for (int s = lane; s < K; s += 64) out[s] = s < c ? s + offset : -1;
    return;
  }
  const float* srow = scores + (int64_t)row * T;
  uint32_t key[KPL];
  // all loads first, then branch-free keys (a branch per element would make the compiler wait
  // for each load before issuing the next).  The launcher keeps every read inside the scores
  // buffer (rows whose 64*KPL positions would run past its end go to the per-row workgroup
  // kernel).
  const float* lrow = srow + lane;
  const int ng = (c + 63) / 64;  // groups holding a visible position
  // groups past the last visible position are not read (one wave-uniform check per 16 groups;
  // their keys are masked to 0 below either way)
#pragma unroll
  for (int g0 = 0; g0 < KPL; g0 += 16) {
    if (g0 < ng) {
#pragma unroll
      for (int g = g0; g < g0 + 16 && g < KPL; ++g) key[g] = __float_as_uint(lrow[64 * g]);
    } else {
#pragma unroll
      for (int g = g0; g < g0 + 16 && g < KPL; ++g) key[g] = 0u;
    }
  }
  // keys, block by block of 16 groups: a block wholly visible needs no mask, the block holding
  // the last visible position masks each group, blocks past it stay 0
  uint32_t kand = 0xFFFFFFFFu, kor = 0u;
#pragma unroll
  for (int g0 = 0; g0 < KPL; g0 += 16) {
    if (64 * (g0 + 16) <= c) {
#pragma unroll
      for (int g = g0; g < g0 + 16; ++g) {
        const uint32_t k = wave_key(key[g]);
        key[g] = k;
        kand &= k;
        kor |= k;
      }
    } else if (g0 < ng) {
#pragma unroll
      for (int g = g0; g < g0 + 16; ++g) {
        const bool vis = 64 * g + lane < c;
        const uint32_t k = wave_key(key[g]);
        key[g] = vis ? k : 0u;
        kand &= vis ? k : 0xFFFFFFFFu;
        kor |= vis ? k : 0u;
      }
    }
  }
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) {
    kand &= __shfl_xor(kand, m, 64);
    kor |= __shfl_xor(kor, m, 64);
  }
  const uint32_t diff = kand ^ kor;  // bits that differ among the visible keys
  // prefix: the bits every visible key shares, then the digits chosen so far; the keys still in
  // the running are the visible ones equal to it under mask (the shared bits and those digits)
  uint32_t prefix = kand & ~diff;
  uint32_t mask = ~diff;
  int remaining = K;
  bool exact = false;  // exactly `remaining` visible keys agree with `prefix` down to bit lo_end
  int lo_end = 0;      // lowest bit of the last digit taken
  if (diff != 0u) {
    int hb = 31 - __builtin_clz(diff);
    // lane l owns digits 252-4l .. 255-4l in every copy: it clears them here and after each pass
#pragma unroll
    for (int r = 0; r < kWR; ++r)
#pragma unroll
      for (int j = 0; j < 4; ++j) hist[r * kWP + 252 - 4 * lane + j] = 0;
    int* hcopy = hist + (lane % kWR) * kWP;
    while (true) {
      const int lo = hb >= 7 ? hb - 7 : 0;
      const int width = hb - lo + 1;
      const uint32_t dmask = ((width == 32) ? 0xFFFFFFFFu : ((1u << width) - 1u)) << lo;
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      // constant trip counts (an early exit would stop the full unroll and push key[] out to
      // scratch memory); invisible keys are 0, which no score maps to; one wave-uniform check per
      // 16 groups skips the groups past the last visible position
#pragma unroll
      for (int g0 = 0; g0 < KPL; g0 += 16) {
        if (g0 < ng) {
#pragma unroll
          for (int g = g0; g < g0 + 16; ++g)
            if (key[g] != 0u && (key[g] & mask) == prefix) atomicAdd(&hcopy[(key[g] & dmask) >> lo], 1);
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
      __builtin_amdgcn_wave_barrier();
      // lane l takes digits 255-4l .. 252-4l (largest first), summed over the copies (and cleared
      // for the next pass); counts of keys in larger digits
      int hc[4] = {0, 0, 0, 0};
#pragma unroll
      for (int r = 0; r < kWR; ++r)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          int* hp = hist + r * kWP + 252 - 4 * lane + j;
          hc[j] += *hp;
          *hp = 0;
        }
      const int c0 = hc[3], c1 = hc[2], c2 = hc[1], c3 = hc[0];  // digits 255-4l, 254-4l, 253-4l, 252-4l
      const int mine = c0 + c1 + c2 + c3;
      int incl = mine;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int u = __shfl_up(incl, o, 64);
        if (lane >= o) incl += u;
      }
      const int excl = incl - mine;  // keys in digits above this lane's four
      const bool here = excl < remaining && incl >= remaining;
      const uint64_t hmask = __builtin_amdgcn_ballot_w64(here);
      const int src = __builtin_ctzll(hmask);
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
      if (in_digit == remaining) {
        exact = true;  // every key of the chosen digit is taken
        lo_end = lo;
        break;
      }
      if (lo == 0) break;
      hb = lo - 1;
    }
  }
  if (exact) {
    // keep every visible key at or above the chosen digit, in position order.  mask is every
    // bit from lo_end up plus bits all visible keys share (where key and prefix agree), so
    // (key & mask) >= prefix is key >= thr, thr being prefix cleared below lo_end; thr >= 1 also
    // drops the invisible keys (0).  Exactly K keys pass: stop once they are out.
    const uint32_t thr = max(prefix & (0xFFFFFFFFu << lo_end), 1u);
    int base = 0;
#pragma unroll
    for (int g0 = 0; g0 < KPL; g0 += 16) {
      if (g0 < ng && base < K) {
#pragma unroll
        for (int g = g0; g < g0 + 16; ++g) {
          const bool keep = key[g] >= thr;
          const uint64_t kb = __builtin_amdgcn_ballot_w64(keep);
          const int pos = base + __builtin_amdgcn_mbcnt_hi((uint32_t)(kb >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)kb, 0));
          if (keep && pos < K) *(int32_t*)((char*)out + (uint32_t)pos * 4u) = 64 * g + lane + offset;
          base += __builtin_popcountll(kb);
        }
      }
    }
    return;
  }
  const uint32_t tau = prefix;  // key of the K-th best visible score (a real key, so never 0)
  // keep keys > tau and the first `remaining` keys == tau, in position order (invisible keys are 0)
  int base = 0, eq_seen = 0;
#pragma unroll
  for (int g0 = 0; g0 < KPL; g0 += 16) {
    if (g0 < ng) {
#pragma unroll
      for (int g = g0; g < g0 + 16; ++g) {
        const uint64_t eqb = __builtin_amdgcn_ballot_w64(key[g] == tau);
        const int rank =
            eq_seen + __builtin_amdgcn_mbcnt_hi((uint32_t)(eqb >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)eqb, 0));
        eq_seen += __builtin_popcountll(eqb);
        const bool keep = key[g] > tau || (key[g] == tau && rank < remaining);
        const uint64_t kb = __builtin_amdgcn_ballot_w64(keep);
        const int pos = base + __builtin_amdgcn_mbcnt_hi((uint32_t)(kb >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)kb, 0));
        if (keep && pos < K) *(int32_t*)((char*)out + (uint32_t)pos * 4u) = 64 * g + lane + offset;
        base += __builtin_popcountll(kb);
      }
    }
  }
}

__global__ void window_idx_kernel(int S, int start_pos, int W, int Wc, int32_t* __restrict__ idx, int64_t ld_idx) {
  const int s = blockIdx.x * blockDim.x + threadIdx.x;
  const int row = blockIdx.y;  // b*S + t
  if (s >= Wc) return;
  idx[(int64_t)row * ld_idx + s] = window_entry(row % S, s, start_pos, W);
}

template <int NT, int KPT>
int launch_topk(const float* scores, int B, int S, int T, int K, int sp, int r, int off, int32_t* idx,
                int64_t ld, int W, int Wc, hipStream_t st) {
  hipLaunchKernelGGL((topk_kernel<NT, KPT>), dim3(B * S), dim3(NT), 0, st, scores, S, T, K, sp, r, off, idx, ld, 0, W,
                     Wc);
  return check_launch("topk_block");
}

}  // namespace

// Rows 0 .. head-1 on the one-wave kernel, whose reads of up to 64*KPL positions per row stay
// inside the buffer; the last `tail` rows on the per-row workgroup kernel (NT threads x KPT keys).
void topk_wave_split(int64_t rows, int T, int KPL, int64_t* head, int64_t* tail) {
  // row r reads positions r*T .. r*T + 64*KPL - 1, inside rows*T positions iff r <= rows - 64*KPL/T
  const int64_t over = ((int64_t)64 * KPL - T + T - 1) / T;  // rows whose read span would pass the end
  *tail = over < rows ? over : rows;
  *head = rows - *tail;
}

template <int KPL, int NT, int KPT>
int launch_topk_wave(const float* scores, int B, int S, int T, int K, int sp, int r, int off, int32_t* idx,
                     int64_t ld, int W, int Wc, hipStream_t st) {
  int64_t head64, tail64;
  topk_wave_split((int64_t)B * S, T, KPL, &head64, &tail64);
  const int head = (int)head64, tail = (int)tail64;
  int rc = DSA_OK;
  if (head > 0) {
    hipLaunchKernelGGL((topk_wave_kernel<KPL>), dim3((head + 3) / 4), dim3(256), 0, st, scores, head, S, T, K, sp, r,
                       off, idx, ld, W, Wc);
    rc = check_launch(KPL == 32 ? "topk_wave<32>" : KPL == 64 ? "topk_wave<64>" : "topk_wave<128>");
  }
  if (rc || tail == 0) return rc;
  hipLaunchKernelGGL((topk_kernel<NT, KPT>), dim3(tail), dim3(NT), 0, st, scores, S, T, K, sp, r, off, idx, ld,
                     head, W, Wc);
  return check_launch("topk_block");
}

// The split select applies to fewer than 1024 rows of more than 16384 scores whose G*K candidates
// a merge workgroup can hold; returns the workspace payload it needs (0 when it does not apply).
// Up to 16384 scores one workgroup per row is as fast (measured at 16 rows: 11.3 us against 14 us
// for the two split launches); from 32768 on the split wins (65536: ~20 us against ~177 us).
size_t topk_split_bytes(int B, int S, int T, int K) {
  const int64_t rows = (int64_t)B * S;
  if (rows <= 0 || rows >= 1024 || T <= 16384 || K <= 0) return 0;
  const int64_t G = (T + kChunk - 1) / kChunk;
  if (G * K > 32768) return 0;
  return (size_t)(rows * G * K) * (sizeof(float) + sizeof(int32_t));
}

int topk_split_launch(const float* scores, int B, int S, int T, int K, int sp, int r, int off, int32_t* idx,
                      int64_t ld, int W, int Wc, void* payload, hipStream_t st) {
  const int rows = B * S;
  const int G = (T + kChunk - 1) / kChunk;
  float* cand_s = (float*)payload;
  int32_t* cand_p = (int32_t*)(cand_s + (size_t)rows * G * K);
  hipLaunchKernelGGL(topk_split_chunk_kernel, dim3(G, rows), dim3(256), 0, st, scores, S, T, K, sp, r, G, cand_s,
                     cand_p);
  int rc = check_launch("topk_split_chunk");
  if (rc) return rc;
  const int n = G * K;
#define DSA_MERGE(NT_, KPT_)                                                                                      \
  hipLaunchKernelGGL((topk_split_merge_kernel<NT_, KPT_>), dim3(rows), dim3(NT_), 0, st, cand_s, cand_p, G, S, T, K, \
                     sp, r, off, idx, ld, W, Wc)
  if (n <= 2048) DSA_MERGE(256, 8);
  else if (n <= 4096) DSA_MERGE(512, 8);
  else if (n <= 8192) DSA_MERGE(1024, 8);
  else if (n <= 16384) DSA_MERGE(1024, 16);
  else DSA_MERGE(1024, 32);
#undef DSA_MERGE
  return check_launch("topk_split_merge");
}

int candidate_blocks_launch(const float* scores, int B, int S, int T, int start_pos, int ratio, int lbs, int n_sel,
                            uint32_t* bits, int64_t ld_bits, hipStream_t st) {
  if (((T + (1 << lbs) - 1) >> lbs) > kCandMaxBlocks)
    return fail(DSA_ERR_UNSUPPORTED, "dsa_candidate_blocks: more than %d blocks per row", kCandMaxBlocks);
  hipLaunchKernelGGL(candidate_blocks_kernel, dim3(B * S), dim3(1024), 0, st, scores, S, T, start_pos, ratio, lbs,
                     n_sel, bits, ld_bits);
  return check_launch("candidate_blocks");
}

// Rows of a top-k call on the one-wave kernel and on the per-row workgroup kernel.
void topk_plan(int B, int S, int T, int64_t* wave_rows, int64_t* block_rows) {  // rows without the split select
  const int64_t rows = (int64_t)B * S;
  *wave_rows = 0;
  *block_rows = rows;
  if (rows < 1024 || T > 8192 || T <= 0) return;
  topk_wave_split(rows, T, T <= 2048 ? 32 : T <= 4096 ? 64 : 128, wave_rows, block_rows);
}

// idx points at the row base; a row gets Wc window entries (W the window) then its K top-k entries.
// `payload` (may be null) is workspace past its header, of at least topk_split_bytes(B, S, T, K).
int topk_launch(const float* scores, int B, int S, int T, int K, int start_pos, int ratio, int offset,
                int32_t* idx, int64_t ld_idx, int W, int Wc, void* payload, hipStream_t st) {
  if (payload && topk_split_bytes(B, S, T, K) > 0)
    return topk_split_launch(scores, B, S, T, K, start_pos, ratio, offset, idx, ld_idx, W, Wc, payload, st);
  // many rows: one wave per row
  if ((int64_t)B * S >= 1024) {
    if (T <= 2048) return launch_topk_wave<32, 256, 8>(scores, B, S, T, K, start_pos, ratio, offset, idx, ld_idx, W, Wc, st);
    if (T <= 4096) return launch_topk_wave<64, 512, 8>(scores, B, S, T, K, start_pos, ratio, offset, idx, ld_idx, W, Wc, st);
    if (T <= 8192) return launch_topk_wave<128, 1024, 8>(scores, B, S, T, K, start_pos, ratio, offset, idx, ld_idx, W, Wc, st);
  }
  // T <= 256*KPT with KPT <= 8, then 1024 threads x up to 64 keys for the longest rows (64K context at ratio 1)
  if (T <= 256) return launch_topk<256, 1>(scores, B, S, T, K, start_pos, ratio, offset, idx, ld_idx, W, Wc, st);
  if (T <= 512) return launch_topk<256, 2>(scores, B, S, T, K, start_pos, ratio, offset, idx, ld_idx, W, Wc, st);
  if (T <= 1024) return launch_topk<256, 4>(scores, B, S, T, K, start_pos, ratio, offset, idx, ld_idx, W, Wc, st);
  if (T <= 2048) return launch_topk<256, 8>(scores, B, S, T, K, start_pos, ratio, offset, idx, ld_idx, W, Wc, st);
  if (T <= 4096) return launch_topk<512, 8>(scores, B, S, T, K, start_pos, ratio, offset, idx, ld_idx, W, Wc, st);
  if (T <= 8192) return launch_topk<1024, 8>(scores, B, S, T, K, start_pos, ratio, offset, idx, ld_idx, W, Wc, st);
  if (T <= 16384) return launch_topk<1024, 16>(scores, B, S, T, K, start_pos, ratio, offset, idx, ld_idx, W, Wc, st);
  if (T <= 32768) return launch_topk<1024, 32>(scores, B, S, T, K, start_pos, ratio, offset, idx, ld_idx, W, Wc, st);
  if (T <= 65536) return launch_topk<1024, 64>(scores, B, S, T, K, start_pos, ratio, offset, idx, ld_idx, W, Wc, st);
  return fail(DSA_ERR_UNSUPPORTED, "dsa_topk: T=%d exceeds the supported 65536 rows", T);
}

int window_idx_launch(int B, int S, int start_pos, int W, int Wc, int32_t* idx, int64_t ld_idx, hipStream_t st) {
  dim3 grid((Wc + 127) / 128, B * S);
  hipLaunchKernelGGL(window_idx_kernel, grid, dim3(128), 0, st, S, start_pos, W, Wc, idx, ld_idx);
  return check_launch("window_idx");
}

}  // namespace dsa
