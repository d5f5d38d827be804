// Index scores for prefill (DeepSeek V4.1 page, `Indexer.forward`; many queries per batch):
//   scores[b,t,j] = w_scale * sum_h w[b,t,h] * relu(q_idx[b,t,h,:] . k_idx[b,j,:])  for j < c(t),
//   -inf for c(t) <= j < T, with c(t) = (start_pos + t + 1) / ratio.
//
// As a matrix product this is (query, head) rows x compressed-key columns with a short K (the
// index head dim, 128), reduced over heads in the epilogue.  With K that short, a tile loaded once
// must be reused across many tiles of the other operand, so:
//  * one workgroup owns 8 queries (2 per wave); their index heads stay in AGPRs as the MFMA A
//    operand for the whole kernel (32 heads x 128 dims per query = 8 k-steps of 16);
//  * the visible keys of the block stream through an LDS ring of 64-key tiles filled by direct
//    global->LDS copies (keys are contiguous rows, so a tile is one 16 KiB coalesced read); the
//    16-byte chunks of key row r are XOR-swizzled by r, so the B-operand reads (16 rows at one
//    chunk) touch every bank group once;
//  * v_mfma_f32_32x32x16_bf16 with heads as M and keys as N: the accumulator of lane (hf, c)
//    holds 16 heads of key c, so ReLU, head weights and the head sum stay in registers and one
//    cross-half shuffle finishes each key;
//  * keys past the block's last visible row are never loaded; the score row's invisible tail is
//    filled with -inf by plain stores; the blocks with the most visible keys are dispatched first.
#include "dsa_internal.h"

namespace dsa {

namespace {

constexpr int kXDI = 128;                // index head dim of this kernel
constexpr int kXKS = kXDI / 16;          // MFMA k-steps
constexpr int kXQ = 8;                   // queries per workgroup
constexpr int kXKT = 64;                 // keys per tile (two MFMA key blocks)
constexpr int kXRowB = kXDI * 2;         // bytes of one key row
constexpr int kXTileB = kXKT * kXRowB;   // 16 KiB
constexpr int kXNST = 4;                 // ring stages

// max(x, 0) in one instruction, as a signed integer max on the bits: a negative float (-0.0
// included) is a negative integer and becomes +0.0, a non-negative one is unchanged.  fmaxf on a
// value straight from an MFMA costs two (the compiler first quiets NaNs).
__device__ __forceinline__ float relu1(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

__global__ void __launch_bounds__(256, 2)
index_scores_prefill_kernel(const __bf16* __restrict__ q_idx, const __bf16* __restrict__ k_idx, int64_t k_bstride,
                            const __bf16* __restrict__ w, float w_scale, int S, int T, int H, int start_pos,
                            int ratio, int nqb, float* __restrict__ scores, CandMask cm) {
  __shared__ __attribute__((aligned(1024))) unsigned char ring[kXNST * kXTileB];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int hf = lane >> 5;
  const int c = lane & 31;

  // heaviest blocks (latest queries, most visible keys) first
  const int b = blockIdx.x / nqb;
  const int qb = nqb - 1 - blockIdx.x % nqb;
  const int t0 = qb * kXQ;
  const int nq = min(kXQ, S - t0);
  const int c_blk = min(T, visible_rows(start_pos, t0 + nq - 1, ratio));
  const int ntl = (c_blk + kXKT - 1) / kXKT;  // tiles holding a key visible to some query here

  const __bf16* kb = k_idx + (int64_t)b * k_bstride;

  // Copies of key tile i into ring slot i % NST: four wave instructions of 4 key rows each; lane l
  // fills physical chunk l & 15 of row 4 blk + l/16, which holds logical chunk (l & 15) ^ (row & 15).
  // Rows past T re-read row T-1 (in bounds; never scored).
  auto issue = [&](int i) {
    unsigned char* tile = ring + (i % kXNST) * kXTileB;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int blk = 4 * wave + u;
      const int r = 4 * blk + (lane >> 4);
      const int j = min(i * kXKT + r, T - 1);
      const int chunk = (lane & 15) ^ (r & 15);
      dma16_v(kb + (int64_t)j * kXDI + chunk * 8, (DSA_LDS void*)(tile + blk * 1024));
    }
  };

#pragma unroll
  for (int i = 0; i < kXNST - 1; ++i)
    if (i < ntl) issue(i);

  // this wave's two queries: index heads (A operand, AGPRs), head weights, visible counts
  bf16x8 qa[2][kXKS];
  float wv[2][16];
  int ct[2];
  bool live[2];
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const int t = t0 + 2 * wave + m;
    live[m] = t < S;
    ct[m] = live[m] ? min(T, visible_rows(start_pos, t, ratio)) : 0;
    const bool hv = live[m] && c < H;
    const __bf16* qp = q_idx + (((int64_t)b * S + min(t, S - 1)) * H + min(c, H - 1)) * kXDI + hf * 8;
#pragma unroll
    for (int s = 0; s < kXKS; ++s) qa[m][s] = hv ? *reinterpret_cast<const bf16x8*>(qp + 16 * s) : bf16x8{};
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int h = 8 * (e >> 2) + 4 * hf + (e & 3);
      const float wh = bf16_to_f32(w[((int64_t)b * S + min(t, S - 1)) * H + min(h, H - 1)]);
      wv[m][e] = (live[m] && h < H) ? wh : 0.f;
    }
#pragma unroll
    for (int s = 0; s < kXKS; ++s) asm volatile("" : "+a"(qa[m][s]));
  }
  wait_vmcnt<0>();  // the compiler's own loads above are done; only copies are counted below

  const float ninf = -__builtin_inff();
  // lane's B-operand base: key row c, chunk (2s + hf) ^ (c & 15)
  const int kop_row = c * kXRowB;
  const int kop_swz = c & 15;

  for (int i = 0; i < ntl; ++i) {
    const int later = min(kXNST - 2, ntl - 1 - i);
    if (later >= 2)
      wait_vmcnt<8>();
    else if (later == 1)
      wait_vmcnt<4>();
    else
      wait_vmcnt<0>();
    __syncthreads();  // tile i is complete; every wave is past tile i-1, whose slot is refilled
    if (i + kXNST - 1 < ntl) issue(i + kXNST - 1);

    const unsigned char* tile = ring + (i % kXNST) * kXTileB;
    // both 32-key blocks of the tile at once: four independent accumulator chains (query x key
    // block) over the eight k-steps, so the matrix core never waits on a dependent accumulator
    // and each chain ends holding its final logits (no partial sums to merge); a query that sees
    // nothing of the block (at most its last ones) is still multiplied and only its stores differ
    bf16x8 kop[2][kXKS];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int s = 0; s < kXKS; ++s)
        kop[kb][s] = *reinterpret_cast<const bf16x8*>(tile + kb * 32 * kXRowB + kop_row + (((2 * s + hf) ^ kop_swz) << 4));
    f32x16 acc[2][2];
#pragma unroll
    for (int s = 0; s < kXKS; ++s)
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) acc[m][kb] = mfma32(qa[m][s], kop[kb][s], s == 0 ? f32x16{} : acc[m][kb]);
    // keep the chains interleaved, operand reads two k-steps ahead of their MFMAs
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);  // LDS reads of k-steps 0, 1
#pragma unroll
    for (int s = 0; s < kXKS; ++s) {
      if (s + 2 < kXKS) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // reads of k-step s + 2
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);                    // MFMAs of k-step s
    }
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      float* out_row = scores + ((int64_t)b * S + t0 + 2 * wave + m) * T;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        float sum = 0.f;
#pragma unroll
        for (int e = 0; e < 16; ++e) sum += relu1(acc[m][kb][e]) * wv[m][e];
        // the two halves' sums, exchanged on the VALU (no LDS permute behind the operand reads):
        // v_permlane32_swap of sum with itself leaves {lower half's, upper half's} in every lane
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(sum), __float_as_uint(sum), false, false);
        sum = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
        const int j = i * kXKT + 32 * kb + c;
        if (live[m] && hf == 0 && j < T)
          out_row[j] = (j < ct[m] && cand_ok(cm, (int64_t)b * S + t0 + 2 * wave + m, j)) ? w_scale * sum : ninf;
      }
    }
  }

  // invisible tail of each score row: [ntl * 64, T)
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    if (!live[m]) continue;
    float* out_row = scores + ((int64_t)b * S + t0 + 2 * wave + m) * T;
    for (int j = ntl * kXKT + lane; j < T; j += 64) out_row[j] = ninf;
  }
}

}  // namespace

// Launches the prefill index kernel when it applies (bf16, index head dim 128, at most 32 index
// heads, enough queries, 16-byte aligned key rows); returns 1 if launched, 0 if not, <0 on error.
int index_scores_prefill_launch(const void* q_idx, const void* k_idx, int64_t kbs, const void* w, float w_scale,
                                int B, int S, int T, int H, int DI, int start_pos, int ratio, float* scores,
                                const CandMask& cm, hipStream_t st) {
  if (DI != kXDI || H > 32 || S < 64 || T < 1) return 0;
  if (((uintptr_t)k_idx & 15) != 0 || ((kbs * 2) & 15) != 0) return 0;
  const int nqb = (S + kXQ - 1) / kXQ;
  hipLaunchKernelGGL(index_scores_prefill_kernel, dim3(B * nqb), dim3(256), 0, st, (const __bf16*)q_idx,
                     (const __bf16*)k_idx, kbs, (const __bf16*)w, w_scale, S, T, H, start_pos, ratio, nqb, scores, cm);
  const int rc = check_launch("index_scores_prefill");
  return rc ? rc : 1;
}

}  // namespace dsa
