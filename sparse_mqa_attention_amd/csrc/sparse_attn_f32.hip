// fp32 sparse attention with a per-head sink (DeepSeek V4.1 page, `sparse_attn_kernel`), for
// small fp32 shapes: one workgroup per query, heads in sequence, logits staged in LDS.  The
// softmax uses the larger of the slot logits and the sink as its reference, so an all-empty row
// gives exactly 0 and a large sink cannot overflow.
#include "dsa_internal.h"

namespace dsa {

namespace {

constexpr int kF32Threads = 256;
constexpr int kF32MaxSlots = 8192;

__device__ float block_max(float v, float* red) {
  for (int m = 1; m < 64; m <<= 1) v = fmaxf(v, __shfl_xor(v, m, 64));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float r = red[0];
  for (int i = 1; i < kF32Threads / 64; ++i) r = fmaxf(r, red[i]);
  __syncthreads();
  return r;
}

__device__ float block_sum(float v, float* red) {
  for (int m = 1; m < 64; m <<= 1) v += __shfl_xor(v, m, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float r = 0.f;
  for (int i = 0; i < kF32Threads / 64; ++i) r += red[i];
  __syncthreads();
  return r;
}

__global__ void __launch_bounds__(kF32Threads)
sparse_attn_f32_kernel(const float* __restrict__ q, const float* __restrict__ win, int64_t win_n, int64_t win_bs,
                       int64_t win_rs, const float* __restrict__ comp, int64_t comp_bs, int64_t comp_rs,
                       const float* __restrict__ sink, const int32_t* __restrict__ idx, int L, float scale,
                       float* __restrict__ o, int S, int H, int D) {
  __shared__ float lg[kF32MaxSlots];
  __shared__ float red[kF32Threads / 64];
  const int t = blockIdx.x, b = blockIdx.y;
  const int64_t qrow = (int64_t)b * S + t;
  const int32_t* irow = idx + qrow * L;
  auto row_ptr = [&](int i) -> const float* {
    return i < win_n ? win + b * win_bs + (int64_t)i * win_rs : comp + b * comp_bs + (int64_t)(i - win_n) * comp_rs;
  };
  for (int h = 0; h < H; ++h) {
    const float* qh = q + (qrow * H + h) * D;
    float mx = -__builtin_inff();
    for (int s = threadIdx.x; s < L; s += kF32Threads) {
      const int i = irow[s];
      float v = -__builtin_inff();
      if (i >= 0) {
        const float* r = row_ptr(i);
        float dot = 0.f;
        for (int d = 0; d < D; ++d) dot = fmaf(qh[d], r[d], dot);
        v = dot * scale;
      }
      lg[s] = v;
      mx = fmaxf(mx, v);
    }
    const float M = fmaxf(block_max(mx, red), sink[h]);
    float part = 0.f;
    for (int s = threadIdx.x; s < L; s += kF32Threads) {
      const float e = expf(lg[s] - M);
      lg[s] = e;
      part += e;
    }
    const float den = block_sum(part, red) + expf(sink[h] - M);
    for (int d = threadIdx.x; d < D; d += kF32Threads) {
      float acc = 0.f;
      for (int s = 0; s < L; ++s) {
        const int i = irow[s];
        if (i >= 0) acc = fmaf(lg[s], row_ptr(i)[d], acc);
      }
      o[(qrow * H + h) * D + d] = acc / den;
    }
    __syncthreads();
  }
}

}  // namespace

int sparse_attn_f32_launch(const void* q, const dsa_kv_src* win, const dsa_kv_src* comp, const float* sink,
                           const int32_t* idx, int L, float scale, void* o, int B, int S, int H, int D,
                           hipStream_t st) {
  if (L > kF32MaxSlots) return fail(DSA_ERR_UNSUPPORTED, "dsa_sparse_attn: fp32 path takes at most %d slots", kF32MaxSlots);
  const bool has_comp = comp && comp->rows;
  hipLaunchKernelGGL(sparse_attn_f32_kernel, dim3(S, B), dim3(kF32Threads), 0, st, (const float*)q,
                     (const float*)win->rows, win->n_rows, win->batch_stride, win->row_stride,
                     has_comp ? (const float*)comp->rows : nullptr, has_comp ? comp->batch_stride : 0,
                     has_comp ? comp->row_stride : 0, sink, idx, L, scale, (float*)o, S, H, D);
  return check_launch("sparse_attn_f32");
}

}  // namespace dsa
