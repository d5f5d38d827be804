// One 32-row MFMA tile of index scores for one query (DeepSeek V4.1 page, `Indexer.forward`:
// the score of compressed row j is the head-weighted sum of relu(q_idx_h . k_idx_j)), shared by
// the index kernel and the decode attention kernel that scores its own rows, so both produce
// the same bits.
#pragma once
#include "dsa_internal.h"

namespace dsa {

// Physical 16-byte chunk of logical chunk `ch` in LDS row `r` (rows of NCH chunks).
template <int NCH>
__device__ __forceinline__ int qswz(int r, int ch) {
  constexpr int M = NCH < 16 ? NCH - 1 : 15;
  return ch ^ (r & M);
}

// The tile's rows are the N operand: lane (hf = lane/32, c = lane%32) holds row c's k-steps in
// kreg (elements 16s + 8hf .. +7 of the row in kreg[s]).  q_lds holds 32*MT heads of DI elements
// (chunk-swizzled rows, zero past the real heads) and w_lds their weights (zero past the real
// heads).  Returns sum_h w[h] * relu(q_h . k_c) for row c in both halves of the wave.
template <int DI, int MT>
__device__ __forceinline__ float index_tile_sum(const __bf16* q_lds, const float* w_lds,
                                                const bf16x8 (&kreg)[DI / 16], int hf, int c) {
  constexpr int NCH = DI / 8;
  constexpr int KS = DI / 16;
  float sum = 0.f;
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    f32x16 acc = {};
    const int h = 32 * m + c;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(&q_lds[h * DI + qswz<NCH>(h, 2 * s + hf) * 8]);
      acc = mfma32(a, kreg[s], acc);
    }
    // accumulator element e of lane (hf, c) is head 32m + 8(e/4) + 4hf + e%4 of row c
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int hh = 32 * m + 8 * (e >> 2) + 4 * hf + (e & 3);
      sum += fmaxf(acc[e], 0.f) * w_lds[hh];
    }
  }
  return sum + shfl_xor(sum, 32);
}

}  // namespace dsa
