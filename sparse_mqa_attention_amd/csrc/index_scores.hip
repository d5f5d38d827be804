// Index scores of the sparse attention step (DeepSeek V4.1 page, `Indexer.forward`):
//   scores[b,t,j] = w_scale * sum_h w[b,t,h] * relu(q_idx[b,t,h,:] . k_idx[b,j,:])  for j < c(t),
//   -inf for c(t) <= j < T, with c(t) = (start_pos + t + 1) / ratio (a compressed group is
//   visible once the query has passed its last token).
//
// bf16 path: one workgroup (4 waves) scores a block of QB queries against 256 compressed rows.
// Each wave owns 64 rows (two 32-row MFMA tiles) whose keys stay in registers as the B operand;
// the QB queries' index heads are staged once in LDS and read by all four waves as the A
// operand, so every key byte and every query byte crosses HBM/L2 once per block.  The MFMA is
// v_mfma_f32_32x32x16_bf16 with heads as M and rows as N: the accumulator of lane (hf, c) holds
// 16 heads of row c, so the ReLU, the head weights and the head sum happen in registers and one
// cross-half shuffle finishes each row.  Rows past c(t) are never multiplied: whole tiles past
// the visibility edge only store -inf.
#include "index_tile.h"

namespace dsa {

namespace {

constexpr int kIdxThreads = 256;  // 4 waves
constexpr int kRowsPerWave = 64;
constexpr int kRowsPerBlock = kIdxThreads / 64 * kRowsPerWave;  // 256

template <int DI, int MT, int QB>
__global__ void __launch_bounds__(kIdxThreads)
index_scores_bf16_kernel(const __bf16* __restrict__ q_idx, const __bf16* __restrict__ k_idx,
                         int64_t k_bstride, const __bf16* __restrict__ w, float w_scale, int S,
                         int T, int H, int start_pos, int ratio, float* __restrict__ scores, CandMask cm) {
  constexpr int NCH = DI / 8;   // 16-byte chunks per index row
  constexpr int KS = DI / 16;   // MFMA k-steps
  constexpr int HP = 32 * MT;   // padded heads
  __shared__ __attribute__((aligned(16))) __bf16 q_lds[QB * HP * DI];
  __shared__ float w_lds[QB * HP];

  const int b = blockIdx.z;
  const int t0 = blockIdx.y * QB;
  const int j0 = blockIdx.x * kRowsPerBlock;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int hf = lane >> 5;
  const int c = lane & 31;

  // ---- stage the block's index queries and head weights in LDS ----------------------
  const int nq = min(QB, S - t0);
  for (int e = tid; e < QB * HP * NCH; e += kIdxThreads) {
    const int ch = e % NCH;
    const int h = (e / NCH) % HP;
    const int q = e / (NCH * HP);
    u32x4 v = {0u, 0u, 0u, 0u};
    if (q < nq && h < H)
      v = *reinterpret_cast<const u32x4*>(q_idx + (((int64_t)b * S + t0 + q) * H + h) * DI + ch * 8);
    *reinterpret_cast<u32x4*>(&q_lds[(q * HP + h) * DI + qswz<NCH>(h, ch) * 8]) = v;
  }
  for (int e = tid; e < QB * HP; e += kIdxThreads) {
    const int h = e % HP, q = e / HP;
    w_lds[e] = (q < nq && h < H) ? bf16_to_f32(w[((int64_t)b * S + t0 + q) * H + h]) : 0.f;
  }

  // ---- this wave's keys: two 32-row tiles, B operand layout -------------------------
  const int jw = j0 + wave * kRowsPerWave;
  const int c_last = min(T, visible_rows(start_pos, t0 + nq - 1, ratio));
  bf16x8 kreg[2][KS];
  const bool wave_live = jw < c_last;
  // one query per block (decode): keys outside its candidate blocks are not read
  const int64_t row0 = (int64_t)b * S + t0;
  if (wave_live) {
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      const int j = jw + 32 * n + c;
      const __bf16* kp = k_idx + (int64_t)b * k_bstride + (int64_t)j * DI + hf * 8;
      const bool need = j < T && (QB > 1 || cand_ok(cm, row0, j));
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        if (need) {
          kreg[n][s] = *reinterpret_cast<const bf16x8*>(kp + s * 16);
        } else {
          kreg[n][s] = bf16x8{};
        }
      }
    }
  }
  __syncthreads();

  const float ninf = -__builtin_inff();
  for (int q = 0; q < nq; ++q) {
    const int t = t0 + q;
    const int ct = min(T, visible_rows(start_pos, t, ratio));
    float* out_row = scores + ((int64_t)b * S + t) * T;
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      const int jt = jw + 32 * n;
      if (jt >= T) break;
      const int j = jt + c;
      if (jt >= ct) {  // whole tile not visible yet: no multiply
        if (hf == 0 && j < T) out_row[j] = ninf;
        continue;
      }
      const bool ok = j < ct && cand_ok(cm, row0 + q, j);
      if (QB == 1 && __builtin_amdgcn_ballot_w64(ok) == 0ull) {  // no candidate in the tile: no multiply
        if (hf == 0 && j < T) out_row[j] = ninf;
        continue;
      }
      const float sum = index_tile_sum<DI, MT>(q_lds + q * HP * DI, w_lds + q * HP, kreg[n], hf, c);
      if (hf == 0 && j < T) out_row[j] = ok ? w_scale * sum : ninf;
    }
  }
  // rows of this wave never loaded (all invisible for the whole block): still write -inf
  (void)wave_live;
}

// fp32 path: one thread per (b, t, j); plain loops (small shapes only).
__global__ void index_scores_f32_kernel(const float* __restrict__ q_idx, const float* __restrict__ k_idx,
                                        int64_t k_bstride, const float* __restrict__ w, float w_scale,
                                        int S, int T, int H, int DI, int start_pos, int ratio,
                                        float* __restrict__ scores, CandMask cm) {
  const int j = blockIdx.x * blockDim.x + threadIdx.x;
  const int t = blockIdx.y;
  const int b = blockIdx.z;
  if (j >= T) return;
  const int ct = min(T, visible_rows(start_pos, t, ratio));
  float* out = scores + ((int64_t)b * S + t) * T + j;
  if (j >= ct || !cand_ok(cm, (int64_t)b * S + t, j)) {
    *out = -__builtin_inff();
    return;
  }
  const float* kp = k_idx + (int64_t)b * k_bstride + (int64_t)j * DI;
  float sum = 0.f;
  for (int h = 0; h < H; ++h) {
    const float* qp = q_idx + (((int64_t)b * S + t) * H + h) * DI;
    float dot = 0.f;
    for (int d = 0; d < DI; ++d) dot = fmaf(qp[d], kp[d], dot);
    sum = fmaf(fmaxf(dot, 0.f), w[((int64_t)b * S + t) * H + h], sum);
  }
  *out = w_scale * sum;
}

template <int DI, int MT, int QB>
int launch_bf16(const void* q, const void* k, int64_t kbs, const void* w, float ws, int B, int S, int T,
                int H, int sp, int r, float* scores, const CandMask& cm, hipStream_t st) {
  dim3 grid((T + kRowsPerBlock - 1) / kRowsPerBlock, (S + QB - 1) / QB, B);
  hipLaunchKernelGGL((index_scores_bf16_kernel<DI, MT, QB>), grid, dim3(kIdxThreads), 0, st,
                     (const __bf16*)q, (const __bf16*)k, kbs, (const __bf16*)w, ws, S, T, H, sp, r, scores, cm);
  return check_launch("index_scores_bf16");
}

// queries per block for prefill: keep the staged queries at 64 KiB of LDS
template <int DI, int MT>
constexpr int prefill_qb() {
  return (8 * 128 / (DI * MT)) < 1 ? 1 : (8 * 128 / (DI * MT)) > 16 ? 16 : (8 * 128 / (DI * MT));
}

template <int DI, int MT>
int launch_bf16_qb(const void* q, const void* k, int64_t kbs, const void* w, float ws, int B, int S, int T,
                   int H, int sp, int r, float* scores, const CandMask& cm, hipStream_t st) {
  if (S == 1) return launch_bf16<DI, MT, 1>(q, k, kbs, w, ws, B, S, T, H, sp, r, scores, cm, st);
  return launch_bf16<DI, MT, prefill_qb<DI, MT>()>(q, k, kbs, w, ws, B, S, T, H, sp, r, scores, cm, st);
}

template <int DI>
int launch_bf16_mt(const void* q, const void* k, int64_t kbs, const void* w, float ws, int B, int S, int T,
                   int H, int sp, int r, float* scores, const CandMask& cm, hipStream_t st) {
  if (H <= 32) return launch_bf16_qb<DI, 1>(q, k, kbs, w, ws, B, S, T, H, sp, r, scores, cm, st);
  return launch_bf16_qb<DI, 2>(q, k, kbs, w, ws, B, S, T, H, sp, r, scores, cm, st);
}

}  // namespace

int index_scores_prefill_launch(const void* q_idx, const void* k_idx, int64_t kbs, const void* w, float w_scale,
                                int B, int S, int T, int H, int DI, int start_pos, int ratio, float* scores,
                                const CandMask& cm, hipStream_t st);

int index_scores_launch(const void* q_idx, const void* k_idx, int64_t kbs, const void* w, float w_scale,
                        int dtype, int B, int S, int T, int H, int DI, int start_pos, int ratio,
                        float* scores, const CandMask& cm, hipStream_t st) {
  if (dtype == DSA_F32) {
    dim3 grid((T + 63) / 64, S, B);
    hipLaunchKernelGGL(index_scores_f32_kernel, grid, dim3(64), 0, st, (const float*)q_idx,
                       (const float*)k_idx, kbs, (const float*)w, w_scale, S, T, H, DI, start_pos, ratio,
                       scores, cm);
    return check_launch("index_scores_f32");
  }
  // prefill at index head dim 128: keys streamed past queries held in registers
  const int prc = index_scores_prefill_launch(q_idx, k_idx, kbs, w, w_scale, B, S, T, H, DI, start_pos, ratio,
                                              scores, cm, st);
  if (prc != 0) return prc < 0 ? prc : 0;
  switch (DI) {
    case 32: return launch_bf16_mt<32>(q_idx, k_idx, kbs, w, w_scale, B, S, T, H, start_pos, ratio, scores, cm, st);
    case 64: return launch_bf16_mt<64>(q_idx, k_idx, kbs, w, w_scale, B, S, T, H, start_pos, ratio, scores, cm, st);
    case 128: return launch_bf16_mt<128>(q_idx, k_idx, kbs, w, w_scale, B, S, T, H, start_pos, ratio, scores, cm, st);
    case 256: return launch_bf16_mt<256>(q_idx, k_idx, kbs, w, w_scale, B, S, T, H, start_pos, ratio, scores, cm, st);
    default: return fail(DSA_ERR_UNSUPPORTED, "dsa_index_scores: D_I=%d has no bf16 kernel (32, 64, 128, 256)", DI);
  }
}

}  // namespace dsa
