// The steps on either side of the sparse attention that `Attention.forward` and `_compress_kv`
// (DeepSeek V4.1 pages) run on the attention's own tensors:
//
//  * inverse rotary embedding of the output: `apply_rotary_emb(o[..., -rope_head_dim:], freqs_cis,
//    True)` right after `sparse_attn`.  The decode and prefill attention kernels apply it in their
//    epilogue before o is rounded to bf16; rope_inverse_kernel is the standalone pass for the
//    other attention kernels.
//  * the compressed-cache write: the compressor's latent rotated on its last rope_head_dim dims at
//    the group's position, quantised to fp4 e2m1 with one E4M3 scale per 16 elements, and stored
//    packed (element 2k in the low nibble of byte k) at the cache rows of this call.
//
// `apply_rotary_emb`'s body is not on the pages: dims 2i, 2i+1 of the rotated part are one complex
// number, multiplied by cos + i sin of its position (by the conjugate for the inverse).  The page
// rotates a bf16 tensor through float32, so the cache write takes exactly those steps: float32
// products and sums without fused multiply-adds, rounded to bf16.  The quantiser's body is not on
// the pages either: scale = E4M3(amax / 6) rounded to nearest-even and saturated at 448, code = the
// e2m1 value nearest x / scale (ties to the even code, at most 6), each step in float32, so that
// every code is decided as a float32 kernel decides it.
#include "dsa_internal.h"

namespace dsa {

namespace {

// One thread per (query row, head, pair) of the rotated part, in place.
template <typename T>
__global__ void rope_inverse_kernel(T* __restrict__ o, const float* __restrict__ freqs, int S, int H, int D, int P,
                                    int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const int p = (int)(i % P);
  const int64_t qh = i / P;  // (b*S + t) * H + h
  const int t = (int)((qh / H) % S);
  T* x = o + qh * D + (D - 2 * P) + 2 * p;
  float a = (float)x[0], b = (float)x[1];
  const float2 cs = *reinterpret_cast<const float2*>(freqs + ((int64_t)t * P + p) * 2);
  rope_rot_inv(a, b, cs.x, cs.y);
  x[0] = (T)a;
  x[1] = (T)b;
}

// float32 -> bf16 -> float32, round to nearest even
__device__ __forceinline__ float to_bf16(float x) { return (float)(__bf16)x; }

// nearest E4M3 value of v >= 0 (ties to even), saturated at 448; returns the value and its code
__device__ __forceinline__ float e4m3_rne(float v, uint32_t* code) {
  if (!(v > 0.f)) {
    *code = 0u;
    return 0.f;
  }
  int e;
  frexpf(v, &e);
  e -= 1;  // v in [2^e, 2^(e+1))
  e = e < -6 ? -6 : (e > 8 ? 8 : e);
  const float q = ldexpf(v, 3 - e);  // exact: a power-of-two scaling
  float val = ldexpf(rintf(q), e - 3);
  if (val > 448.f) val = 448.f;
  if (val == 0.f) {
    *code = 0u;
    return 0.f;
  }
  int ve;
  frexpf(val, &ve);
  ve -= 1;
  if (ve >= -6) {
    *code = (uint32_t)((ve + 7) << 3) | (uint32_t)rintf((ldexpf(val, -ve) - 1.f) * 8.f);
  } else {
    *code = (uint32_t)rintf(ldexpf(val, 9));  // subnormal: multiples of 2^-9
  }
  return val;
}

// e2m1 code of x / scale (ties to the even code, magnitude at most 6, sign in bit 3)
__device__ __forceinline__ uint32_t e2m1_code(float y) {
  const float m = fabsf(y);
  uint32_t c = (m > 0.25f) + (m >= 0.75f) + (m > 1.25f) + (m >= 1.75f) + (m > 2.5f) + (m >= 3.5f) + (m > 5.f);
  return c | (y < 0.f ? 8u : 0u);
}

// One thread per 16-element group of a latent row: rotate (rope part), round to bf16, quantise, store.
__global__ void compress_kv_write_kernel(const __bf16* __restrict__ latent, int64_t lat_bs, int n, int D, int P,
                                         const float* __restrict__ freqs, uint8_t* __restrict__ rows,
                                         int64_t rows_bs, uint8_t* __restrict__ scales, int64_t sc_bs, int64_t row0,
                                         int64_t total) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int G = D / 16;
  if (i >= total) return;
  const int gi = (int)(i % G);
  const int64_t br = i / G;  // b * n + r
  const int r = (int)(br % n);
  const int64_t b = br / n;
  const __bf16* src = latent + b * lat_bs + (int64_t)r * D + 16 * gi;
  float x[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) x[k] = (float)src[k];
  const int rope0 = D - 2 * P;  // first rotated dim (a multiple of 16)
  if (16 * gi >= rope0) {
    const float* f = freqs + ((int64_t)r * P + (16 * gi - rope0) / 2) * 2;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float c = f[2 * k], s = f[2 * k + 1];
      const float a = x[2 * k], bb = x[2 * k + 1];
      // the page's float32 complex product, without fused multiply-adds, rounded to bf16
      x[2 * k] = to_bf16(__fsub_rn(__fmul_rn(a, c), __fmul_rn(bb, s)));
      x[2 * k + 1] = to_bf16(__fadd_rn(__fmul_rn(a, s), __fmul_rn(bb, c)));
    }
  }
  float amax = 0.f;
#pragma unroll
  for (int k = 0; k < 16; ++k) amax = fmaxf(amax, fabsf(x[k]));
  uint32_t scode;
  const float scale = e4m3_rne(__fdiv_rn(amax, 6.f), &scode);
  uint32_t lo = 0u, hi = 0u;
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const uint32_t c = scale > 0.f ? e2m1_code(__fdiv_rn(x[k], scale)) : 0u;
    if (k < 8)
      lo |= c << (4 * k);
    else
      hi |= c << (4 * (k - 8));
  }
  uint8_t* dst = rows + b * rows_bs + (row0 + r) * (int64_t)(D / 2) + 8 * gi;
  *reinterpret_cast<uint2*>(dst) = make_uint2(lo, hi);
  scales[b * sc_bs + (row0 + r) * (int64_t)G + gi] = (uint8_t)scode;
}

}  // namespace

int rope_inverse_launch(void* o, int dtype, int B, int S, int H, int D, const float* freqs, int rope_dim,
                        hipStream_t st) {
  const int P = rope_dim / 2;
  const int64_t n = (int64_t)B * S * H * P;
  if (n == 0) return DSA_OK;
  const int64_t blocks = (n + 255) / 256;
  if (dtype == DSA_BF16)
    hipLaunchKernelGGL(rope_inverse_kernel<__bf16>, dim3((unsigned)blocks), dim3(256), 0, st, (__bf16*)o, freqs, S, H,
                       D, P, n);
  else
    hipLaunchKernelGGL(rope_inverse_kernel<float>, dim3((unsigned)blocks), dim3(256), 0, st, (float*)o, freqs, S, H, D,
                       P, n);
  return check_launch("rope_inverse");
}

int compress_kv_write_launch(const void* latent, int64_t lat_bs, int B, int n, int D, int rope_dim,
                             const float* freqs, uint8_t* rows, int64_t rows_bs, uint8_t* scales, int64_t sc_bs,
                             int64_t row0, hipStream_t st) {
  const int64_t total = (int64_t)B * n * (D / 16);
  if (total == 0) return DSA_OK;
  hipLaunchKernelGGL(compress_kv_write_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st,
                     (const __bf16*)latent, lat_bs, n, D, rope_dim / 2, freqs, rows, rows_bs, scales, sc_bs, row0,
                     total);
  return check_launch("compress_kv_write");
}

}  // namespace dsa
