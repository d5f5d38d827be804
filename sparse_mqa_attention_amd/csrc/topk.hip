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
#include "dsa_internal.h"

namespace dsa {

namespace {

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

template <int NT, int KPT>
__global__ void __launch_bounds__(NT)
topk_kernel(const float* __restrict__ scores, int S, int T, int K, int start_pos, int ratio, int offset,
            int32_t* __restrict__ idx, int64_t ld_idx) {
  __shared__ int hist[256];
  __shared__ int scan_scratch[NT / 64 + 2];
  __shared__ uint32_t red_scratch[2 * (NT / 64)];
  __shared__ int sel_info[2];

  const int row = blockIdx.x;  // b*S + t
  const int t = row % S;
  const int tid = threadIdx.x;
  const int c = min(T, visible_rows(start_pos, t, ratio));
  int32_t* out = idx + (int64_t)row * ld_idx;

  if (c <= K) {  // every visible position is kept
    for (int s = tid; s < K; s += NT) out[s] = s < c ? s + offset : -1;
    return;
  }
  // n = K here: exactly K positions are kept and no -1 is written
  const float* srow = scores + (int64_t)row * T;
  const int jbase = tid * KPT;
  uint32_t key[KPT];
  uint32_t kand = 0xFFFFFFFFu, kor = 0u;
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    const int j = jbase + i;
    key[i] = j < c ? order_key(srow[j]) : 0u;  // invisible: below every real key
    if (j < c) {
      kand &= key[i];
      kor |= key[i];
    }
  }
  uint32_t all_or;
  const uint32_t all_and = block_reduce_and_or<NT>(kand, kor, red_scratch, &all_or);
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
      for (int i = tid; i < 256; i += NT) hist[i] = 0;
      __syncthreads();
#pragma unroll
      for (int i = 0; i < KPT; ++i) {
        if (jbase + i < c && (key[i] & mask) == prefix) atomicAdd(&hist[(key[i] & dmask) >> lo], 1);
      }
      __syncthreads();
      // suffix counts over the bins (largest digit first): thread i takes bin 255 - i
      const int bin = 255 - (tid & 255);
      const int cnt = tid < 256 ? hist[bin] : 0;
      int tot;
      const int excl = block_exclusive_scan<NT>(cnt, scan_scratch, &tot);  // keys in bins above `bin`
      if (tid < 256 && excl < remaining && excl + cnt >= remaining) {
        sel_info[0] = bin;
        sel_info[1] = excl;
      }
      __syncthreads();
      const int sbin = sel_info[0];
      remaining -= sel_info[1];
      prefix |= ((uint32_t)sbin << lo);
      mask |= dmask;
      __syncthreads();
      if (lo == 0) break;
      hb = lo - 1;
    }
  }
  const uint32_t tau = prefix;  // key of the K-th best visible score
  // keep keys > tau, and the first `remaining` keys == tau in position order
  int n_eq = 0;
#pragma unroll
  for (int i = 0; i < KPT; ++i) n_eq += (jbase + i < c && key[i] == tau) ? 1 : 0;
  int tot_eq;
  int eq_before = block_exclusive_scan<NT>(n_eq, scan_scratch, &tot_eq);
  int n_keep = 0;
  uint32_t keep_bits = 0u;  // KPT <= 32
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    const bool vis = jbase + i < c;
    bool k = vis && key[i] > tau;
    if (vis && key[i] == tau) {
      k = eq_before < remaining;
      ++eq_before;
    }
    if (k) {
      keep_bits |= 1u << i;
      ++n_keep;
    }
  }
  int tot_keep;
  int pos = block_exclusive_scan<NT>(n_keep, scan_scratch, &tot_keep);
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    if ((keep_bits & (1u << i)) && pos < K) out[pos++] = jbase + i + offset;
  }
}

__global__ void window_idx_kernel(int S, int start_pos, int W, int Wc, int32_t* __restrict__ idx, int64_t ld_idx) {
  const int s = blockIdx.x * blockDim.x + threadIdx.x;
  const int row = blockIdx.y;  // b*S + t
  if (s >= Wc) return;
  const int t = row % S;
  int v;
  if (start_pos == 0) {
    const int first = t - W + 1 > 0 ? t - W + 1 : 0;
    const int pos = first + s;
    v = pos <= t ? pos : -1;
  } else {
    const int oldest = start_pos % W + 1;
    const int slot = oldest + s < W ? oldest + s : oldest + s - W;
    v = slot <= start_pos ? slot : -1;
  }
  idx[(int64_t)row * ld_idx + s] = v;
}

template <int NT, int KPT>
int launch_topk(const float* scores, int B, int S, int T, int K, int sp, int r, int off, int32_t* idx,
                int64_t ld, hipStream_t st) {
  hipLaunchKernelGGL((topk_kernel<NT, KPT>), dim3(B * S), dim3(NT), 0, st, scores, S, T, K, sp, r, off, idx, ld);
  return check_launch("topk");
}

}  // namespace

int topk_launch(const float* scores, int B, int S, int T, int K, int start_pos, int ratio, int offset,
                int32_t* idx, int64_t ld_idx, hipStream_t st) {
  // T <= 256*KPT with KPT <= 32, or 1024 threads x 64 keys for the longest rows
  if (T <= 256) return launch_topk<256, 1>(scores, B, S, T, K, start_pos, ratio, offset, idx, ld_idx, st);
  if (T <= 512) return launch_topk<256, 2>(scores, B, S, T, K, start_pos, ratio, offset, idx, ld_idx, st);
  if (T <= 1024) return launch_topk<256, 4>(scores, B, S, T, K, start_pos, ratio, offset, idx, ld_idx, st);
  if (T <= 2048) return launch_topk<256, 8>(scores, B, S, T, K, start_pos, ratio, offset, idx, ld_idx, st);
  if (T <= 4096) return launch_topk<512, 8>(scores, B, S, T, K, start_pos, ratio, offset, idx, ld_idx, st);
  if (T <= 8192) return launch_topk<1024, 8>(scores, B, S, T, K, start_pos, ratio, offset, idx, ld_idx, st);
  if (T <= 16384) return launch_topk<1024, 16>(scores, B, S, T, K, start_pos, ratio, offset, idx, ld_idx, st);
  if (T <= 32768) return launch_topk<1024, 32>(scores, B, S, T, K, start_pos, ratio, offset, idx, ld_idx, st);
  return fail(DSA_ERR_UNSUPPORTED, "dsa_topk: T=%d exceeds the supported 32768 rows", T);
}

int window_idx_launch(int B, int S, int start_pos, int W, int Wc, int32_t* idx, int64_t ld_idx, hipStream_t st) {
  dim3 grid((Wc + 127) / 128, B * S);
  hipLaunchKernelGGL(window_idx_kernel, grid, dim3(128), 0, st, S, start_pos, W, Wc, idx, ld_idx);
  return check_launch("window_idx");
}

}  // namespace dsa
