// Index scores with the indexer's fp4 operands (DeepSeek V4.1 pages: `Indexer.forward` quantises
// the index queries and keys to fp4, and `_compress_kv` gives the indexer's format: blocks of 32
// elements sharing one E8M0 power-of-two scale):
//   scores[b,t,j] = w_scale * sum_h w[b,t,h] * relu(q_idx[b,t,h,:] . k_idx[b,j,:])  for j < c(t),
//   -inf for c(t) <= j < T, with q_idx and k_idx the decoded fp4 values.
//
// The contraction runs on gfx950's block-scaled MFMA, v_mfma_scale_f32_32x32x64_f8f6f4 with both
// operands in e2m1: lane l supplies row l%32 of its operand over the 32 consecutive k-elements
// 32*(l/32) .. +31 (16 bytes, low nibble first) and the E8M0 byte of exactly that block, so a
// packed row is consumed as it lies in memory and each lane's scale is one byte of the row's scale
// bytes.  The products of e2m1 values and power-of-two scales are exact; sums are float32.
//
// Layout as the bf16 kernel: one workgroup (4 waves) scores QB queries against 256 compressed rows.
// Each wave holds the packed keys of its 64 rows (two 32-row tiles, 16 bytes per lane and k-step)
// and their scale bytes in registers as the B operand; the QB queries' packed index heads, their
// scale bytes and head weights are staged once in LDS as the A operand.  Heads are MFMA M and rows
// N, so the ReLU, head weights and head sum stay in registers.  A key row costs D_I/2 + D_I/32
// bytes of HBM (68 at D_I = 128, against 256 for bf16 keys).
#include "dsa_internal.h"

namespace dsa {

namespace {

constexpr int kMxThreads = 256;
constexpr int kMxRowsPerWave = 64;
constexpr int kMxRowsPerBlock = kMxThreads / 64 * kMxRowsPerWave;  // 256

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

// e2m1 x e2m1 block-scaled MFMA (format code 4 for both operands, scale byte 0 of each lane)
__device__ __forceinline__ v16f mfma_mxfp4(u32x4 a, u32x4 b, int sa, int sb, v16f c) {
  const v8i av = {(int)a[0], (int)a[1], (int)a[2], (int)a[3], 0, 0, 0, 0};
  const v8i bv = {(int)b[0], (int)b[1], (int)b[2], (int)b[3], 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, c, 4, 4, 0, sa, 0, sb);
}

// 16-byte chunk ch of LDS row r, XOR-swizzled over the row's NCH chunks so that 32 lanes reading one
// logical chunk of 32 consecutive rows spread over the banks
template <int NCH>
__device__ __forceinline__ int mx_swz(int r, int ch) {
  return ch ^ (r & (NCH - 1));
}

template <int DI, int MT, int QB>
__global__ void __launch_bounds__(kMxThreads)
index_scores_mxfp4_kernel(const uint8_t* __restrict__ q_idx, const uint8_t* __restrict__ q_scale,
                          const uint8_t* __restrict__ k_idx, const uint8_t* __restrict__ k_scale,
                          int64_t k_brows, const __bf16* __restrict__ w, float w_scale, int S, int T, int H,
                          int start_pos, int ratio, float* __restrict__ scores, CandMask cm) {
  constexpr int RB = DI / 2;     // packed bytes per row
  constexpr int NCH = RB / 16;   // 16-byte chunks per row
  constexpr int NB = DI / 32;    // scale bytes per row
  constexpr int KS = DI / 64;    // MFMA k-steps
  constexpr int HP = 32 * MT;    // heads padded to whole MFMA tiles
  static_assert(DI % 64 == 0 && NCH >= 2 && (NCH & (NCH - 1)) == 0, "index head dim 64, 128 or 256");
  __shared__ __attribute__((aligned(16))) uint8_t q_lds[QB * HP * RB];
  __shared__ uint8_t qs_lds[QB * HP * NB];
  __shared__ float w_lds[QB * HP];

  const int b = blockIdx.z;
  const int t0 = blockIdx.y * QB;
  const int j0 = blockIdx.x * kMxRowsPerBlock;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int hf = lane >> 5;
  const int c = lane & 31;

  // ---- stage the block's packed index queries, their scale bytes and head weights -----
  const int nq = min(QB, S - t0);
  for (int e = tid; e < QB * HP * NCH; e += kMxThreads) {
    const int ch = e % NCH;
    const int h = (e / NCH) % HP;
    const int q = e / (NCH * HP);
    u32x4 v = {0u, 0u, 0u, 0u};
    if (q < nq && h < H) v = *reinterpret_cast<const u32x4*>(q_idx + (((int64_t)b * S + t0 + q) * H + h) * RB + ch * 16);
    *reinterpret_cast<u32x4*>(&q_lds[(q * HP + h) * RB + mx_swz<NCH>(h, ch) * 16]) = v;
  }
  for (int e = tid; e < QB * HP * NB; e += kMxThreads) {
    const int k = e % NB;
    const int h = (e / NB) % HP;
    const int q = e / (NB * HP);
    // a padded head gets scale 2^-127 over zero nibbles: it contributes exactly 0
    qs_lds[e] = (q < nq && h < H) ? q_scale[(((int64_t)b * S + t0 + q) * H + h) * NB + k] : (uint8_t)0;
  }
  for (int e = tid; e < QB * HP; e += kMxThreads) {
    const int h = e % HP, q = e / HP;
    w_lds[e] = (q < nq && h < H) ? bf16_to_f32(w[((int64_t)b * S + t0 + q) * H + h]) : 0.f;
  }

  // ---- this wave's keys: two 32-row tiles, B operand layout ----------------------------
  const int jw = j0 + wave * kMxRowsPerWave;
  const int c_last = min(T, visible_rows(start_pos, t0 + nq - 1, ratio));
  u32x4 kreg[2][KS];
  int ksc[2][KS];
  // one query per block (decode): keys outside its candidate blocks are not read
  const int64_t row0 = (int64_t)b * S + t0;
#pragma unroll
  for (int n = 0; n < 2; ++n) {
    const int j = jw + 32 * n + c;
    const bool live = jw + 32 * n < c_last && j < T && (QB > 1 || cand_ok(cm, row0, j));
    const uint8_t* kp = k_idx + ((int64_t)b * k_brows + j) * RB + 16 * hf;
    const uint8_t* sp = k_scale + ((int64_t)b * k_brows + j) * NB + hf;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      kreg[n][s] = live ? *reinterpret_cast<const u32x4*>(kp + 32 * s) : u32x4{0u, 0u, 0u, 0u};
      ksc[n][s] = live ? (int)sp[2 * s] : 0;
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
      float sum = 0.f;
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const int h = 32 * m + c;
        const uint8_t* qrow = q_lds + (q * HP + h) * RB;
        const uint8_t* qsr = qs_lds + (q * HP + h) * NB + hf;
        v16f acc = {};
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          const u32x4 a = *reinterpret_cast<const u32x4*>(qrow + mx_swz<NCH>(h, 2 * s + hf) * 16);
          acc = mfma_mxfp4(a, kreg[n][s], (int)qsr[2 * s], ksc[n][s], acc);
        }
        // accumulator element e of lane (hf, c) is head 32m + 8(e/4) + 4hf + e%4 of row c
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int hh = 32 * m + 8 * (e >> 2) + 4 * hf + (e & 3);
          sum += fmaxf(acc[e], 0.f) * w_lds[q * HP + hh];
        }
      }
      sum += shfl_xor(sum, 32);
      if (hf == 0 && j < T) out_row[j] = ok ? w_scale * sum : ninf;
    }
  }
}

template <int DI, int MT, int QB>
int launch_mx(const uint8_t* q, const uint8_t* qs, const uint8_t* k, const uint8_t* ks, int64_t kbr, const void* w,
              float ws, int B, int S, int T, int H, int sp, int r, float* scores, const CandMask& cm, hipStream_t st) {
  dim3 grid((T + kMxRowsPerBlock - 1) / kMxRowsPerBlock, (S + QB - 1) / QB, B);
  hipLaunchKernelGGL((index_scores_mxfp4_kernel<DI, MT, QB>), grid, dim3(kMxThreads), 0, st, q, qs, k, ks, kbr,
                     (const __bf16*)w, ws, S, T, H, sp, r, scores, cm);
  return check_launch("index_scores_mxfp4");
}

template <int DI, int MT>
int launch_mx_qb(const uint8_t* q, const uint8_t* qs, const uint8_t* k, const uint8_t* ks, int64_t kbr,
                 const void* w, float ws, int B, int S, int T, int H, int sp, int r, float* scores, const CandMask& cm,
                 hipStream_t st) {
  if (S == 1) return launch_mx<DI, MT, 1>(q, qs, k, ks, kbr, w, ws, B, S, T, H, sp, r, scores, cm, st);
  return launch_mx<DI, MT, 16>(q, qs, k, ks, kbr, w, ws, B, S, T, H, sp, r, scores, cm, st);
}

template <int DI>
int launch_mx_mt(const uint8_t* q, const uint8_t* qs, const uint8_t* k, const uint8_t* ks, int64_t kbr,
                 const void* w, float ws, int B, int S, int T, int H, int sp, int r, float* scores, const CandMask& cm,
                 hipStream_t st) {
  if (H <= 32) return launch_mx_qb<DI, 1>(q, qs, k, ks, kbr, w, ws, B, S, T, H, sp, r, scores, cm, st);
  return launch_mx_qb<DI, 2>(q, qs, k, ks, kbr, w, ws, B, S, T, H, sp, r, scores, cm, st);
}

}  // namespace

int index_scores_mxfp4_launch(const uint8_t* q_idx, const uint8_t* q_scale, const uint8_t* k_idx,
                              const uint8_t* k_scale, int64_t k_brows, const void* w, float w_scale, int B, int S,
                              int T, int H, int DI, int start_pos, int ratio, float* scores, const CandMask& cm,
                              hipStream_t st) {
  switch (DI) {
    case 64: return launch_mx_mt<64>(q_idx, q_scale, k_idx, k_scale, k_brows, w, w_scale, B, S, T, H, start_pos, ratio, scores, cm, st);
    case 128: return launch_mx_mt<128>(q_idx, q_scale, k_idx, k_scale, k_brows, w, w_scale, B, S, T, H, start_pos, ratio, scores, cm, st);
    case 256: return launch_mx_mt<256>(q_idx, q_scale, k_idx, k_scale, k_brows, w, w_scale, B, S, T, H, start_pos, ratio, scores, cm, st);
    default: return fail(DSA_ERR_UNSUPPORTED, "dsa_index_scores_mxfp4: D_I=%d not in {64, 128, 256}", DI);
  }
}

}  // namespace dsa
