// Sparse MQA attention for prefill (many queries) at head_dim 512 and up to 64 heads
// (DeepSeek V4.1 page, `sparse_attn_kernel`: gather the indexed rows of the one shared KV tensor,
// softmax with the per-head sink in the denominator, -1 slots ignored).
//
// One workgroup per query, 4 waves: wave (hg, dh) owns heads 32*hg..+31 over head_dim half dh.
// Each query gathers ~600 KiB of rows and every row is used by all 64 heads, so the kernel is built
// around keeping the gather going while the matrix cores work:
//  * rows are gathered with 16-byte direct global->LDS copies into a ring of NST 32-row tiles,
//    NST-1 tiles ahead of the MFMAs; each wave copies 8 rows per tile, one wave instruction per
//    row, with the row address formed in scalar registers from the index row (staged in LDS by
//    the same kind of copy); a -1 slot copies a zero row, so every tile costs the same number
//    of copies;
//  * fp4 compressed rows (e2m1 nibbles + E4M3 scale per 16) are gathered raw into a side ring and
//    decoded LDS->LDS just before use; every e2m1 x E4M3 product is exact in bf16;
//  * S^T = K . Q^T on v_mfma_f32_32x32x16_bf16 in two independent accumulator chains; the two
//    head_dim halves are summed through LDS, so both partner waves hold identical logits;
//  * the accumulator layout of S^T is the B-operand layout of P^T, so PV (O^T = V^T . P^T, V^T
//    via ds_read_b64_tr_b16) takes the probabilities straight from registers;
//  * online softmax in base 2 with a lazily raised running max (rescale only when a tile's max
//    passes the running max by more than 8).
//
// LDS tile layout: tile row r lives at slot P(r) = (r & 16) | 4*(r & 3) | ((r >> 2) & 3), rows are
// 1040 bytes apart (1024 + 16 of padding).  With that, the K operand read (16 lanes, 16 rows, one
// 16-byte chunk each) and the transposing V read (4 rows x 64 bytes per 32 lanes) both touch every
// LDS bank once, and every lane reads at a fixed base plus immediate offsets.
#include "dsa_internal.h"

namespace dsa {

namespace {

constexpr int kPD = 512;
constexpr int kPTile = 32;
constexpr int kPRow = 1040;       // LDS bytes per tile row
constexpr int kPMaxSlots = 1024;  // index slots staged in LDS
constexpr float kPLog2e = 1.4426950408889634f;
constexpr float kPRescale = 8.0f;
constexpr float kPMinit = -1.0e30f;

struct PreArgs {
  const __bf16* q;
  const unsigned char* win;
  int64_t win_n, win_bs, win_rs;  // bytes
  const unsigned char* comp;
  int64_t comp_bs, comp_rs;  // bytes
  const unsigned char* csc;
  int64_t csc_bs, csc_rs;
  const float* sink;
  const int32_t* idx;
  int L;
  float scale_log2;
  __bf16* o;
  int S, H, Q;
};

template <bool FP4>
struct PreCfg {
  static constexpr int NST = FP4 ? 3 : 4;       // ring stages
  static constexpr int TILE = kPTile * kPRow;   // bf16 rows of one tile
  static constexpr int RAW = kPTile * 288;      // fp4 rows: 256 nibble bytes + 32 scale bytes
  static constexpr int RING = NST * TILE;
  static constexpr int RAWS = FP4 ? NST * RAW : 0;
  static constexpr int XBUF = 4 * 4 * 64 * 16;  // one partial S^T tile per wave
  static constexpr int MASKS = 2 * NST * 4;     // per ring slot: valid rows, fp4 rows (one byte per wave)
  static constexpr int LDS = RING + RAWS + XBUF + MASKS + kPMaxSlots * 4;
  static_assert(LDS <= 160 * 1024, "LDS budget");
};

// Source of the copies for -1 slots: a zero row, so every slot costs exactly one copy.
__device__ __attribute__((aligned(1024))) unsigned char g_pre_zero_row[kPD * 2];

__device__ __forceinline__ int p_slot(int r) { return (r & 16) | ((r & 3) << 2) | ((r >> 2) & 3); }

__device__ __forceinline__ float p_e2m1(uint32_t nib) {
  const uint32_t m3 = nib & 7u;
  const uint32_t e = m3 >> 1;
  uint32_t bits = e ? (((e + 126u) << 23) | ((m3 & 1u) << 22)) : ((m3 & 1u) ? 0x3F000000u : 0u);
  bits |= (nib & 8u) << 28;
  return __uint_as_float(bits);
}

__device__ __forceinline__ float p_e4m3(uint32_t sc) {
  const uint32_t e = (sc >> 3) & 15u, m = sc & 7u;
  float v;
  if (e == 0u) {
    v = (float)m * 0.001953125f;
  } else if (e == 15u && m == 7u) {
    v = __uint_as_float(0x7FC00000u);
  } else {
    v = __uint_as_float(((e + 120u) << 23) | (m << 20));
  }
  return (sc & 0x80u) ? -v : v;
}

// 16-byte global -> LDS copies (lane l's 16 bytes land at lds_base + 16*l), written as inline asm
// so the compiler does not track them: it would otherwise wait for every outstanding copy before
// each LDS access.  The kernel waits for the copies itself (wait_vmcnt).  The s_nop gives the one
// wait state a copy needs after the M0 write that sets its LDS base.
__device__ __forceinline__ void dma16_s(const void* sbase, uint32_t voff, const DSA_LDS void* lds_base) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase),
               "{m0}"((uint32_t)(uintptr_t)lds_base)
               : "memory");
}
__device__ __forceinline__ void dma4_s(const void* sbase, uint32_t voff, const DSA_LDS void* lds_base) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dword %0, %1" ::"v"(voff), "s"(sbase), "{m0}"((uint32_t)(uintptr_t)lds_base)
               : "memory");
}
__device__ __forceinline__ void dma16_v(const void* gptr, const DSA_LDS void* lds_base) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gptr), "{m0}"((uint32_t)(uintptr_t)lds_base)
               : "memory");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  // gfx9 s_waitcnt: vmcnt in bits 3:0 and 15:14; expcnt (6:4) and lgkmcnt (11:8) left at "no wait"
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

template <bool FP4>
__global__ void __launch_bounds__(256) sparse_attn_prefill_kernel(PreArgs a) {
  using C = PreCfg<FP4>;
  __shared__ __attribute__((aligned(1024))) unsigned char smem[C::LDS];
  unsigned char* ring = smem;
  unsigned char* raw = smem + C::RING;
  float* xbuf = reinterpret_cast<float*>(smem + C::RING + C::RAWS);
  unsigned char* masks = smem + C::RING + C::RAWS + C::XBUF;  // [NST][2][4] bytes
  int* idx_lds = reinterpret_cast<int*>(smem + C::RING + C::RAWS + C::XBUF + C::MASKS);

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int hf = lane >> 5;
  const int c = lane & 31;
  const int j16 = lane & 15;
  const int hg = wave & 1, dh = wave >> 1;
  const int head = 32 * hg + c;

  const int qi = blockIdx.x;
  const int b = qi / a.S;
  const int L = a.L;
  const int ntiles = (L + kPTile - 1) / kPTile;

  const unsigned char* win_b = a.win + (int64_t)b * a.win_bs;
  const unsigned char* comp_b = a.comp + (int64_t)b * a.comp_bs;
  const unsigned char* csc_b = FP4 ? a.csc + (int64_t)b * a.csc_bs : nullptr;
  const int* irow = a.idx + (int64_t)qi * L;
  const int win_n = (int)a.win_n;
  // kept in scalar registers: left alone, the compiler re-reads the symbol's address for every row
  const unsigned char* zero_row = g_pre_zero_row;
  asm volatile("" : "+s"(zero_row));

  // Gather this wave's rows of tile ti into ring slot ti % NST: one copy per row (a -1 slot copies
  // the zero row), and record which rows are valid and which are fp4 rows still to decode.
  auto issue = [&](int ti) {
    const int slot = ti % C::NST;
    const int myidx = idx_lds[ti * kPTile + 8 * wave + (lane & 7)];
    unsigned char* tile = ring + slot * C::TILE;
    unsigned char* rtile = FP4 ? raw + slot * C::RAW : nullptr;
    uint32_t vbits = 0u, fbits = 0u;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int r = 8 * wave + k;
      const int iv = __builtin_amdgcn_readlane(myidx, k);
      vbits |= (iv >= 0 ? 1u : 0u) << k;
      if (FP4 && iv >= win_n) {
        // the raw row: 256 nibble bytes from lanes 0..15, then its 32 scale bytes from lanes 16..17
        const int64_t cr = iv - win_n;
        const unsigned char* src =
            lane < 16 ? comp_b + cr * a.comp_rs + lane * 16 : csc_b + cr * a.csc_rs + (lane - 16) * 16;
        if (lane < 18) dma16_v(src, (DSA_LDS void*)(rtile + r * 288));
        fbits |= 1u << k;
      } else {
        const unsigned char* src = iv < 0 ? zero_row
                                   : iv < win_n ? win_b + (int64_t)iv * a.win_rs
                                                : comp_b + (int64_t)(iv - win_n) * a.comp_rs;
        dma16_s(src, (uint32_t)lane * 16u, (DSA_LDS void*)(tile + p_slot(r) * kPRow));
      }
    }
    if (lane == 0) {
      masks[slot * 8 + wave] = (unsigned char)vbits;
      masks[slot * 8 + 4 + wave] = (unsigned char)fbits;
    }
  };

  // ---- prologue: the index row into LDS (copies, -1 past L), this wave's query heads (its half of
  // D), then the first tiles ----
  for (int i0 = 64 * wave; i0 < L; i0 += 256) {
    if (i0 + lane < L) dma4_s(irow + i0, (uint32_t)lane * 4u, (DSA_LDS void*)(idx_lds + i0));
  }
  for (int i = L + tid; i < ntiles * kPTile; i += 256) idx_lds[i] = -1;
  bf16x8 qreg[16];
  {
    const __bf16* qp = a.q + ((int64_t)qi * a.H + min(head, a.H - 1)) * kPD + 256 * dh + hf * 8;
#pragma unroll
    for (int s = 0; s < 16; ++s) qreg[s] = head < a.H ? *reinterpret_cast<const bf16x8*>(qp + 16 * s) : bf16x8{};
  }
  // the query operands live in AGPRs (MFMA reads them there), leaving the VGPRs to the
  // accumulators and to operands read ahead from LDS
#pragma unroll
  for (int s = 0; s < 16; ++s) asm volatile("" : "+a"(qreg[s]));
  const float sink2 = head < a.H ? a.sink[head] * kPLog2e : 0.f;
  wait_vmcnt<0>();
  __syncthreads();
#pragma unroll
  for (int j = 0; j < C::NST - 1; ++j)
    if (j < ntiles) issue(j);

  f32x16 acc[8];
#pragma unroll
  for (int m = 0; m < 8; ++m) acc[m] = f32x16{};
  float m_run = kPMinit;
  float l_run = 0.f;

  // lane bases: K operand (row c, chunks 32dh + hf + 2s) and transposed V operand
  const int k_base = p_slot(c) * kPRow + 16 * (32 * dh + hf);
  const int v_base = (4 * (j16 >> 2) + hf) * kPRow + 512 * dh + 32 * ((lane >> 4) & 1) + 8 * (j16 & 3);
  float* xmine = xbuf + wave * 4 * 64 * 4;
  const float* xpart = xbuf + (wave ^ 2) * 4 * 64 * 4;

  for (int ti = 0; ti < ntiles; ++ti) {
    // tile ti has landed once no more than the copies of the tiles issued after it are outstanding
    const int later = min(C::NST - 2, ntiles - 1 - ti);
    if (later >= 2)
      wait_vmcnt<16>();
    else if (later == 1)
      wait_vmcnt<8>();
    else
      wait_vmcnt<0>();
    __syncthreads();
    const int slot = ti % C::NST;
    const unsigned char* tile = ring + slot * C::TILE;
    const uint32_t vmask = *reinterpret_cast<const uint32_t*>(masks + slot * 8);
    if constexpr (FP4) {
      // decode this tile's fp4 rows into bf16: wave w takes rows w, w+4, ..., one chunk per lane
      const uint32_t fmask = *reinterpret_cast<const uint32_t*>(masks + slot * 8 + 4);
      const unsigned char* rtile = raw + slot * C::RAW;
      unsigned char* wtile = ring + slot * C::TILE;
      // fmask bit 8w+k marks row 8w+k
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int r = 4 * k + wave;
        if ((fmask >> r) & 1u) {
          const uint32_t word = *reinterpret_cast<const uint32_t*>(rtile + r * 288 + lane * 4);
          const float sc = p_e4m3(rtile[r * 288 + 256 + (lane >> 1)]);
          u32x4 v;
#pragma unroll
          for (int kk = 0; kk < 4; ++kk) {
            const bf16x2 pr = {(__bf16)(p_e2m1(word >> (8 * kk)) * sc), (__bf16)(p_e2m1(word >> (8 * kk + 4)) * sc)};
            v[kk] = __builtin_bit_cast(uint32_t, pr);
          }
          *reinterpret_cast<u32x4*>(wtile + p_slot(r) * kPRow + lane * 16) = v;
        }
      }
      __syncthreads();
    }
    // refill the slot used at ti-1 (every wave is past it)
    if (ti + C::NST - 1 < ntiles) issue(ti + C::NST - 1);

    // ---- partial S^T over this wave's half of D: two independent chains ----
    f32x16 s0 = {}, s1 = {};
    if (vmask != 0u) {
      const unsigned char* kp = tile + k_base;
#pragma unroll
      for (int s = 0; s < 16; s += 2) {
        const bf16x8 k0 = *reinterpret_cast<const bf16x8*>(kp + 32 * s);
        const bf16x8 k1 = *reinterpret_cast<const bf16x8*>(kp + 32 * s + 32);
        s0 = mfma32(k0, qreg[s], s0);
        s1 = mfma32(k1, qreg[s + 1], s1);
      }
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const f32x4 v = {s0[4 * g4] + s1[4 * g4], s0[4 * g4 + 1] + s1[4 * g4 + 1], s0[4 * g4 + 2] + s1[4 * g4 + 2],
                         s0[4 * g4 + 3] + s1[4 * g4 + 3]};
        *reinterpret_cast<f32x4*>(xmine + (g4 * 64 + lane) * 4) = v;
      }
    }
    __syncthreads();
    if (vmask != 0u) {
      float sv[16];
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const f32x4 mine = *reinterpret_cast<const f32x4*>(xmine + (g4 * 64 + lane) * 4);
        const f32x4 part = *reinterpret_cast<const f32x4*>(xpart + (g4 * 64 + lane) * 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float full = dh == 0 ? mine[i] + part[i] : part[i] + mine[i];  // same sum in both halves
          sv[4 * g4 + i] = full * a.scale_log2;
        }
      }
      if (vmask != 0xFFFFFFFFu) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int row = 8 * (e >> 2) + 4 * hf + (e & 3);
          if (!((vmask >> row) & 1u)) sv[e] = -__builtin_inff();
        }
      }
      float mloc = sv[0];
#pragma unroll
      for (int e = 1; e < 16; ++e) mloc = fmaxf(mloc, sv[e]);
      mloc = fmaxf(mloc, shfl_xor(mloc, 32));
      if (__builtin_amdgcn_ballot_w64(mloc > m_run + kPRescale) != 0ull) {
        const float m_new = fmaxf(m_run, mloc);
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int m = 0; m < 8; ++m)
#pragma unroll
          for (int e = 0; e < 16; ++e) acc[m][e] *= alpha;
      }
      bf16x8 pb[2];
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float p = __builtin_amdgcn_exp2f(sv[e] - m_run);
        l_run += p;
        pb[e >> 3][e & 7] = (__bf16)p;
      }
      // ---- O^T += V^T . P^T on this wave's half of D (8 independent chains) ----
      // k step ks, part pt reads tile rows 16ks + 8pt + 4hf + 0..3 = slots 16ks + 2pt + hf + 4*(0..3)
      const unsigned char* vp = tile + v_base;
#pragma unroll
      for (int m = 0; m < 8; ++m) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const bf16x4 lo = lds_read_tr16((const DSA_LDS __bf16*)(vp + (16 * ks) * kPRow + 64 * m));
          const bf16x4 hi = lds_read_tr16((const DSA_LDS __bf16*)(vp + (16 * ks + 2) * kPRow + 64 * m));
          const bf16x8 vf = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          acc[m] = mfma32(vf, pb[ks], acc[m]);
        }
      }
    }
  }

  if (head >= a.H) return;
  const float l_tot = l_run + shfl_xor(l_run, 32);
  const float mf = fmaxf(m_run, sink2);
  const float f = exp2f(m_run - mf);
  const float rn = f / (l_tot * f + exp2f(sink2 - mf));
  __bf16* op = a.o + ((int64_t)qi * a.H + head) * kPD + 256 * dh + 4 * hf;
#pragma unroll
  for (int m = 0; m < 8; ++m)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const bf16x4 v = {(__bf16)(acc[m][4 * g] * rn), (__bf16)(acc[m][4 * g + 1] * rn),
                        (__bf16)(acc[m][4 * g + 2] * rn), (__bf16)(acc[m][4 * g + 3] * rn)};
      *reinterpret_cast<bf16x4*>(op + 32 * m + 8 * g) = v;
    }
}

}  // namespace

// Launches the prefill kernel when it applies (head_dim 512, at most 64 heads, index rows of at
// most 1024 slots, enough queries to fill the GPU, 16-byte aligned rows); returns 1 if launched,
// 0 if not, <0 on error.
int sparse_attn_prefill_launch(const void* q, const dsa_kv_src* win, const dsa_kv_src* comp, const float* sink,
                               const int32_t* idx, int L, float scale, void* o, int B, int S, int H, int D,
                               hipStream_t st) {
  const int Q = B * S;
  if (D != kPD || H > 64 || L > kPMaxSlots || Q < 256) return 0;
  const bool fp4 = comp && comp->rows && comp->format == DSA_KV_FP4_E4M3_G16;
  PreArgs a{};
  a.q = (const __bf16*)q;
  a.win = (const unsigned char*)win->rows;
  a.win_n = win->n_rows;
  a.win_bs = win->batch_stride * 2;
  a.win_rs = win->row_stride * 2;
  if (comp && comp->rows) {
    a.comp = (const unsigned char*)comp->rows;
    a.comp_bs = fp4 ? comp->batch_stride : comp->batch_stride * 2;
    a.comp_rs = fp4 ? comp->row_stride : comp->row_stride * 2;
    a.csc = comp->scales;
    a.csc_bs = comp->scale_batch_stride;
    a.csc_rs = comp->scale_row_stride;
  }
  // the copies move 16-byte pieces: every row (and fp4 scale row) must start 16-byte aligned
  auto misaligned = [](const void* p, int64_t rs, int64_t bs) {
    return (((uintptr_t)p) & 15) != 0 || (rs & 15) != 0 || (bs & 15) != 0;
  };
  if (misaligned(a.win, a.win_rs, a.win_bs)) return 0;
  if (a.comp && misaligned(a.comp, a.comp_rs, a.comp_bs)) return 0;
  if (fp4 && misaligned(a.csc, a.csc_rs, a.csc_bs)) return 0;
  a.sink = sink;
  a.idx = idx;
  a.L = L;
  a.scale_log2 = scale * kPLog2e;
  a.o = (__bf16*)o;
  a.S = S;
  a.H = H;
  a.Q = Q;
  if (fp4)
    hipLaunchKernelGGL(sparse_attn_prefill_kernel<true>, dim3(Q), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(sparse_attn_prefill_kernel<false>, dim3(Q), dim3(256), 0, st, a);
  const int rc = check_launch("sparse_attn_prefill");
  return rc ? rc : 1;
}

}  // namespace dsa
