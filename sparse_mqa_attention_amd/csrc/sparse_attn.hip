// Sparse MQA attention with a per-head sink (DeepSeek V4.1 page, `sparse_attn_kernel` and
// `sparse_attn`; the two KV sources follow `Attention.forward`, which concatenates the window
// rows and the compressed rows and shifts compressed indices by the window row count):
//
//   o[b,t,h] = sum_s e^{l_s} kv[idx_s] / (sum_s e^{l_s} + e^{sink_h}),  l_s = scale * q[b,t,h] . kv[idx_s]
//
// over the slots s of the query's index row with idx_s != -1; the key and the value are the same
// row; a query with no valid slot gets 0.
//
// gfx950 design (bf16):
//  * One workgroup per (query, slot range).  Its waves form two halves that take alternate
//    32-row tiles; within a half each wave owns 32 heads, so every KV row staged in LDS feeds
//    32 heads per LDS read (64 heads per CU-wide read for H = 64).
//  * Rows are gathered with 16-byte direct global->LDS loads (no VGPR round trip), one wave
//    instruction per 1 KiB row, into a double-buffered tile per half.  The 16-byte chunks of a
//    row are XOR-swizzled by the row index so both MFMA operand reads below are bank-conflict
//    free.  fp4 compressed rows (e2m1 + one E4M3 scale per 16) go through registers and are
//    decoded to bf16 on the way into LDS; every e2m1 x E4M3 product is exact in bf16.
//  * QK^T runs as S^T = K . Q^T on v_mfma_f32_32x32x16_bf16: A = K rows from LDS (ds_read_b128),
//    B = the wave's 32 query heads, resident in registers for the whole workgroup.  The
//    accumulator then holds, per lane, 16 rows of one head, which is exactly the B-operand layout
//    P^T needs for PV (with the contraction index permuted consistently), so the probabilities go
//    from the softmax straight into the next MFMA without an LDS round trip.
//  * PV runs as O^T = V^T . P^T; V^T comes from the same LDS tile through the gfx950 transposing
//    read ds_read_b64_tr_b16.  O^T accumulates in registers (AGPRs) for the whole range.
//  * Online softmax in base 2 with a lazily raised running max: the accumulator is rescaled only
//    when a tile's max exceeds the running max by more than 8 (log2 units), which keeps every
//    exponent <= 2^8 while skipping almost all rescales after the first tiles.
//  * Decode has too few queries to fill 256 CUs, so the index row is split over several
//    workgroups that write unnormalised partials (running max, sum, O) to the workspace; a small
//    combine kernel folds them with the sink.  Prefill uses one workgroup per query and writes
//    o directly.
#include "dsa_internal.h"

namespace dsa {

namespace {

constexpr int kTile = 32;              // KV rows per tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kRescaleThresh = 8.0f;  // log2 units
constexpr float kMinit = -1.0e30f;      // finite start of the running max
constexpr int kSplitUnit = 32;          // slot granularity of a decode split (one tile)

struct AttnArgs {
  const __bf16* q;
  const unsigned char* win;  // bytes
  int64_t win_n, win_bs, win_rs;  // rows, batch stride, row stride (bytes)
  const unsigned char* comp;
  int64_t comp_bs, comp_rs;  // bytes
  const unsigned char* csc;  // fp4 scales
  int64_t csc_bs, csc_rs;
  const float* sink;
  const int32_t* idx;
  int L;
  float scale_log2;
  __bf16* o;
  float* part;  // split partials: acc [B,S,nsp,H,D] then (m, l) [B,S,nsp,H,2]
  int S, H, nsplit, split_slots;
};

__device__ __forceinline__ float e2m1_to_f32(uint32_t nib) {
  const uint32_t m3 = nib & 7u;
  const uint32_t e = m3 >> 1;
  uint32_t bits = e ? (((e + 126u) << 23) | ((m3 & 1u) << 22)) : ((m3 & 1u) ? 0x3F000000u : 0u);
  bits |= (nib & 8u) << 28;
  return __uint_as_float(bits);
}

__device__ __forceinline__ float e4m3_to_f32(uint32_t sc) {
  const uint32_t e = (sc >> 3) & 15u, m = sc & 7u;
  float v;
  if (e == 0u) {
    v = (float)m * 0.001953125f;  // m * 2^-9
  } else if (e == 15u && m == 7u) {
    v = __uint_as_float(0x7FC00000u);
  } else {
    v = __uint_as_float(((e + 120u) << 23) | (m << 20));
  }
  return (sc & 0x80u) ? -v : v;
}

// 8 consecutive elements of an fp4 row (one 32-bit word of nibbles) times their group scale.
__device__ __forceinline__ u32x4 fp4_chunk_to_bf16(uint32_t word, uint32_t scale_byte) {
  const float s = e4m3_to_f32(scale_byte);
  u32x4 r;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float lo = e2m1_to_f32(word >> (8 * k)) * s;
    const float hi = e2m1_to_f32(word >> (8 * k + 4)) * s;
    bf16x2 p = {(__bf16)lo, (__bf16)hi};
    r[k] = __builtin_bit_cast(uint32_t, p);
  }
  return r;
}

template <int D, int NHG, bool FP4>
struct AttnCfg {
  static constexpr int NW = 2 * NHG;            // waves: head groups x 2 halves of D
  static constexpr int NT = 64 * NW;
  static constexpr int DH = D / 2;              // head_dim half owned by one wave
  static constexpr int ROWB = D * 2;            // bytes of a bf16 row
  static constexpr int NCH = D / 8;             // 16-byte chunks per row
  static constexpr int RPI = 512 / D;           // rows per wave instruction (64 lanes x 16 B)
  static constexpr int LPR = 64 / RPI;          // lanes per row
  static constexpr int GROUPS = kTile / RPI;    // row groups per tile
  static constexpr int NK = (GROUPS + NW - 1) / NW;  // row groups per wave per tile (upper bound)
  static constexpr int TILE_BYTES = kTile * ROWB;
  static constexpr int XBUF_BYTES = NW * 64 * 16 * 4;  // one partial S^T tile per wave
  static constexpr int LDS_BYTES = 2 * TILE_BYTES + XBUF_BYTES;
  static constexpr int KSH = DH / 16;           // QK k-steps per wave
  static constexpr int NMT = DH / 32;           // PV M tiles per wave
};

template <int D, int NHG, bool FP4>
__global__ void __launch_bounds__(128 * NHG)
sparse_attn_bf16_kernel(AttnArgs a) {
  using C = AttnCfg<D, NHG, FP4>;
  __shared__ __attribute__((aligned(1024))) unsigned char smem[C::LDS_BYTES];
  float* xbuf = reinterpret_cast<float*>(smem + 2 * C::TILE_BYTES);

  const int sp = blockIdx.x;
  const int t = blockIdx.y;
  const int b = blockIdx.z;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int hg = wave >> 1;
  const int dh = wave & 1;
  const int hf = lane >> 5;
  const int c = lane & 31;
  const int head = 32 * hg + c;
  const int64_t qrow = (int64_t)b * a.S + t;

  const int s0 = sp * a.split_slots;
  const int s1 = min(a.L, s0 + a.split_slots);
  const int nslots = max(0, s1 - s0);
  const int ntiles = (nslots + kTile - 1) / kTile;
  const int32_t* irow = a.idx + qrow * a.L + s0;

  // index of tile slot `lane` (lanes 0..31), -1 past the range
  auto load_idx = [&](int ti) -> int {
    const int slot = ti * kTile + lane;
    return (lane < kTile && slot < nslots) ? irow[slot] : -1;
  };

  // query heads of this wave's half of D, B operand of S^T = K . Q^T
  bf16x8 qreg[C::KSH];
  {
    const __bf16* qp = a.q + (qrow * a.H + min(head, a.H - 1)) * D + C::DH * dh + hf * 8;
#pragma unroll
    for (int s = 0; s < C::KSH; ++s) qreg[s] = *reinterpret_cast<const bf16x8*>(qp + 16 * s);
    if (head >= a.H) {
#pragma unroll
      for (int s = 0; s < C::KSH; ++s) qreg[s] = bf16x8{};
    }
  }
  const float sink2 = head < a.H ? a.sink[head] * kLog2e : 0.f;

  f32x16 acc[C::NMT];
#pragma unroll
  for (int m = 0; m < C::NMT; ++m) acc[m] = f32x16{};
  float m_run = kMinit;
  float l_run = 0.f;

  uint32_t pend_word[FP4 ? C::NK : 1];
  uint32_t pend_scale[FP4 ? C::NK : 1];
  uint32_t pend_mask = 0u;

  const unsigned char* win_b = a.win + (int64_t)b * a.win_bs;
  const unsigned char* comp_b = a.comp + (int64_t)b * a.comp_bs;
  const unsigned char* csc_b = FP4 ? a.csc + (int64_t)b * a.csc_bs : nullptr;

  // Gather tile rows into stage `st`; `ivec` holds the tile's 32 indices in lanes 0..31.
  auto issue = [&](int st, int ivec) {
    unsigned char* tile = smem + st * C::TILE_BYTES;
    pend_mask = 0u;
#pragma unroll
    for (int k = 0; k < C::NK; ++k) {
      const int g = k * C::NW + wave;  // row group (uniform)
      if (g >= C::GROUPS) break;
      unsigned char* grp = tile + g * C::RPI * C::ROWB;
      const int r = g * C::RPI + lane / C::LPR;  // tile row of this lane
      const int p = lane % C::LPR;               // physical chunk this lane fills
      const int lchunk = p ^ row_swz<C::NCH>(r);
      int iv;
      if constexpr (C::RPI == 1) {
        iv = __builtin_amdgcn_readlane(ivec, g);  // one row per wave instruction: uniform
      } else {
        iv = __shfl(ivec, r, 64);
      }
      if (iv < 0) {
        *reinterpret_cast<u32x4*>(grp + lane * 16) = u32x4{0u, 0u, 0u, 0u};
      } else if (iv < a.win_n) {
        global_to_lds16(win_b + (int64_t)iv * a.win_rs + lchunk * 16, (DSA_LDS void*)grp);
      } else if constexpr (!FP4) {
        global_to_lds16(comp_b + (int64_t)(iv - a.win_n) * a.comp_rs + lchunk * 16, (DSA_LDS void*)grp);
      } else {
        const int64_t cr = iv - a.win_n;
        pend_word[k] = *reinterpret_cast<const uint32_t*>(comp_b + cr * a.comp_rs + lchunk * 4);
        pend_scale[k] = csc_b[cr * a.csc_rs + (lchunk >> 1)];
        pend_mask |= 1u << k;
      }
    }
  };
  auto finish = [&](int st) {
    if constexpr (FP4) {
      unsigned char* tile = smem + st * C::TILE_BYTES;
#pragma unroll
      for (int k = 0; k < C::NK; ++k) {
        const int g = k * C::NW + wave;
        if (g >= C::GROUPS) break;
        if (pend_mask & (1u << k))
          *reinterpret_cast<u32x4*>(tile + g * C::RPI * C::ROWB + lane * 16) =
              fp4_chunk_to_bf16(pend_word[k], pend_scale[k]);
      }
    }
  };

  int idx_cur = -1, idx_next = -1;
  if (ntiles > 0) {
    idx_cur = load_idx(0);
    idx_next = ntiles > 1 ? load_idx(1) : -1;
    issue(0, idx_cur);
    __builtin_amdgcn_s_waitcnt(0);
    finish(0);
  }
  __syncthreads();

  // lane-constant parts of the operand addresses
  const int qk_row_off = c * C::ROWB;
  const int qk_swz = row_swz<C::NCH>(c);
  const int qk_chunk0 = (C::DH / 8) * dh + hf;  // logical chunk of k-step 0
  const int j16 = lane & 15;
  const int colq = C::DH * dh + 16 * ((lane >> 4) & 1) + 4 * (j16 & 3);
  const int hoff = (j16 & 1) << 3;  // upper 4 columns of a 16-byte chunk
  int tr_row_off[2][2];
  int tr_swz[2][2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
#pragma unroll
    for (int pt = 0; pt < 2; ++pt) {
      const int R = 16 * ks + 8 * pt + 4 * hf + (j16 >> 2);
      tr_row_off[ks][pt] = R * C::ROWB + hoff;
      tr_swz[ks][pt] = row_swz<C::NCH>(R);
    }
  float* xmine = xbuf + (wave * 4) * 64 * 4;
  const float* xpart = xbuf + ((wave ^ 1) * 4) * 64 * 4;

  for (int ti = 0; ti < ntiles; ++ti) {
    const int st = ti & 1;
    int idx_after = -1;
    if (ti + 1 < ntiles) {
      issue(st ^ 1, idx_next);
      if (ti + 2 < ntiles) idx_after = load_idx(ti + 2);
    }
    const unsigned char* tile = smem + st * C::TILE_BYTES;
    const uint32_t vmask = (uint32_t)__builtin_amdgcn_ballot_w64(lane < kTile && idx_cur >= 0);
    // ---- partial S^T = K . Q^T over this wave's half of D ----
    f32x16 sacc = {};
    if (vmask != 0u) {
#pragma unroll
      for (int s = 0; s < C::KSH; ++s) {
        const bf16x8 kf =
            *reinterpret_cast<const bf16x8*>(tile + qk_row_off + (((qk_chunk0 + 2 * s) ^ qk_swz) << 4));
        sacc = mfma32(kf, qreg[s], sacc);
      }
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        f32x4 v = {sacc[4 * g4], sacc[4 * g4 + 1], sacc[4 * g4 + 2], sacc[4 * g4 + 3]};
        *reinterpret_cast<f32x4*>(xmine + (g4 * 64 + lane) * 4) = v;
      }
    }
    __syncthreads();
    if (vmask != 0u) {
      // full S^T = half(dh 0) + half(dh 1), the same sum in both partner waves
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const f32x4 o4 = *reinterpret_cast<const f32x4*>(xpart + (g4 * 64 + lane) * 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float mine = sacc[4 * g4 + i];
          sacc[4 * g4 + i] = dh == 0 ? mine + o4[i] : o4[i] + mine;
        }
      }
      // ---- online softmax (base 2) ----
      float sv[16];
      float mloc = -__builtin_inff();
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int row = 8 * (e >> 2) + 4 * hf + (e & 3);
        sv[e] = ((vmask >> row) & 1u) ? sacc[e] * a.scale_log2 : -__builtin_inff();
        mloc = fmaxf(mloc, sv[e]);
      }
      mloc = fmaxf(mloc, shfl_xor(mloc, 32));
      if (__builtin_amdgcn_ballot_w64(mloc > m_run + kRescaleThresh) != 0ull) {
        const float m_new = fmaxf(m_run, mloc);
        const float alpha = exp2f(m_run - m_new);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int m = 0; m < C::NMT; ++m)
#pragma unroll
          for (int e = 0; e < 16; ++e) acc[m][e] *= alpha;
      }
      bf16x8 pb[2];
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float p = exp2f(sv[e] - m_run);
        l_run += p;
        pb[e >> 3][e & 7] = (__bf16)p;
      }
      // ---- O^T += V^T . P^T on this wave's half of D ----
#pragma unroll
      for (int m = 0; m < C::NMT; ++m) {
        const int lch = (32 * m + colq) >> 3;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const bf16x4 lo = lds_read_tr16((const DSA_LDS __bf16*)(tile + tr_row_off[ks][0] + ((lch ^ tr_swz[ks][0]) << 4)));
          const bf16x4 hi = lds_read_tr16((const DSA_LDS __bf16*)(tile + tr_row_off[ks][1] + ((lch ^ tr_swz[ks][1]) << 4)));
          const bf16x8 vf = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          acc[m] = mfma32(vf, pb[ks], acc[m]);
        }
      }
    }
    if (ti + 1 < ntiles) {
      __builtin_amdgcn_s_waitcnt(0);
      finish(st ^ 1);
    }
    __syncthreads();
    idx_cur = idx_next;
    idx_next = idx_after;
  }

  if (head >= a.H) return;
  const float l_tot = l_run + shfl_xor(l_run, 32);
  if (a.nsplit == 1) {
    const float mf = fmaxf(m_run, sink2);
    const float f = exp2f(m_run - mf);
    const float r = f / (l_tot * f + exp2f(sink2 - mf));
    __bf16* op = a.o + (qrow * a.H + head) * D + C::DH * dh + 4 * hf;
#pragma unroll
    for (int m = 0; m < C::NMT; ++m)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x4 v = {(__bf16)(acc[m][4 * g] * r), (__bf16)(acc[m][4 * g + 1] * r), (__bf16)(acc[m][4 * g + 2] * r),
                    (__bf16)(acc[m][4 * g + 3] * r)};
        *reinterpret_cast<bf16x4*>(op + 32 * m + 8 * g) = v;
      }
  } else {
    const int64_t pidx = (qrow * a.nsplit + sp) * a.H + head;
    float* pp = a.part + pidx * D + C::DH * dh + 4 * hf;
#pragma unroll
    for (int m = 0; m < C::NMT; ++m)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4 v = {acc[m][4 * g], acc[m][4 * g + 1], acc[m][4 * g + 2], acc[m][4 * g + 3]};
        *reinterpret_cast<f32x4*>(pp + 32 * m + 8 * g) = v;
      }
    if (hf == 0 && dh == 0) {
      const int64_t nrow = (int64_t)gridDim.z * a.S * a.nsplit * a.H;
      float* ml = a.part + nrow * D + 2 * pidx;
      ml[0] = m_run;
      ml[1] = l_tot;
    }
  }
}

// Fold split partials: o = sum_s acc_s 2^{m_s - M} / (sum_s l_s 2^{m_s - M} + 2^{sink2 - M}).
template <typename OutT>
__global__ void combine_kernel(const float* __restrict__ part, const float* __restrict__ sink, int nsplit, int H,
                               int D, int64_t nrow, OutT* __restrict__ o) {
  const int64_t qh = (int64_t)blockIdx.x * H + blockIdx.y;  // (b*S + t)*H + h
  const int h = blockIdx.y;
  const float* ml = part + nrow * D;
  const float sink2 = sink[h] * kLog2e;
  float M = sink2;
  for (int s = 0; s < nsplit; ++s) M = fmaxf(M, ml[2 * ((blockIdx.x * (int64_t)nsplit + s) * H + h)]);
  float den = exp2f(sink2 - M);
  for (int s = 0; s < nsplit; ++s) {
    const int64_t pi = (blockIdx.x * (int64_t)nsplit + s) * H + h;
    den += ml[2 * pi + 1] * exp2f(ml[2 * pi] - M);
  }
  const float inv = 1.f / den;
  for (int d = threadIdx.x; d < D; d += blockDim.x) {
    float v = 0.f;
    for (int s = 0; s < nsplit; ++s) {
      const int64_t pi = (blockIdx.x * (int64_t)nsplit + s) * H + h;
      v += part[pi * D + d] * exp2f(ml[2 * pi] - M);
    }
    o[qh * D + d] = (OutT)(v * inv);
  }
}

template <int D, int NHG, bool FP4>
int launch_attn(const AttnArgs& a, int B, hipStream_t st) {
  using C = AttnCfg<D, NHG, FP4>;
  dim3 grid(a.nsplit, a.S, B);
  hipLaunchKernelGGL((sparse_attn_bf16_kernel<D, NHG, FP4>), grid, dim3(C::NT), 0, st, a);
  int rc = check_launch("sparse_attn_bf16");
  if (rc || a.nsplit == 1) return rc;
  hipLaunchKernelGGL(combine_kernel<__bf16>, dim3(B * a.S, a.H), dim3(128), 0, st, (const float*)a.part, a.sink,
                     a.nsplit, a.H, D, (int64_t)B * a.S * a.nsplit * a.H, a.o);
  return check_launch("sparse_attn_combine");
}

template <int D, bool FP4>
int launch_attn_h(const AttnArgs& a, int B, hipStream_t st) {
  const int nhg = (a.H + 31) / 32;
  if (nhg == 1) return launch_attn<D, 1, FP4>(a, B, st);
  if constexpr (D == 512) {
    return launch_attn<D, 2, FP4>(a, B, st);  // H <= 64 at head_dim 512
  } else {
    if (nhg == 2) return launch_attn<D, 2, FP4>(a, B, st);
    return launch_attn<D, 4, FP4>(a, B, st);
  }
}

}  // namespace

// Number of slot-range splits for a bf16 launch and the slots each covers.
void sparse_attn_split(int B, int S, int L, int* nsplit, int* split_slots) {
  const int queries = B * S;
  const int units = (L + kSplitUnit - 1) / kSplitUnit;
  int want = 1;
  if (queries < 256 && units > 1) want = (256 + queries - 1) / queries;
  if (want > units) want = units > 0 ? units : 1;
  const int per = units > 0 ? (units + want - 1) / want : 1;
  *split_slots = per * kSplitUnit;
  *nsplit = L > 0 ? (L + *split_slots - 1) / *split_slots : 1;
}

size_t sparse_attn_decode_workspace(int B, int S, int H, int D, int L, bool fp4);
int sparse_attn_decode_launch(const __bf16* q, const unsigned char* win, int64_t win_n, int64_t win_bs,
                              int64_t win_rs, const unsigned char* comp, int64_t comp_n, int64_t comp_bs,
                              int64_t comp_rs, const float* sink, const int32_t* idx, int L, float scale_log2,
                              __bf16* o, int B, int S, int H, int D, bool fp4, void* workspace,
                              const DecSelect* sel, const DecIndex* ix, const float* rope, int rope_dim,
                              hipStream_t st);

int sparse_attn_prefill_launch(const void* q, const dsa_kv_src* win, const dsa_kv_src* comp, const float* sink,
                               const int32_t* idx, int L, float scale, void* o, int B, int S, int H, int D,
                               const float* rope, int rope_dim, hipStream_t st);
int rope_inverse_launch(void* o, int dtype, int B, int S, int H, int D, const float* freqs, int rope_dim,
                        hipStream_t st);

// rope (may be null): the inverse rotary table [S][rope_dim/2][2] applied to o's last rope_dim dims,
// in the decode and prefill kernels' epilogue, otherwise as a pass after the attention
int sparse_attn_bf16_launch(const void* q, const dsa_kv_src* win, const dsa_kv_src* comp, const float* sink,
                            const int32_t* idx, int L, float scale, void* o, int B, int S, int H, int D,
                            void* workspace, const float* rope, int rope_dim, hipStream_t st) {
  AttnArgs a{};
  a.q = (const __bf16*)q;
  a.win = (const unsigned char*)win->rows;
  a.win_n = win->n_rows;
  a.win_bs = win->batch_stride * 2;
  a.win_rs = win->row_stride * 2;
  const bool fp4 = comp && comp->rows && comp->format == DSA_KV_FP4_E4M3_G16;
  if (comp && comp->rows) {
    a.comp = (const unsigned char*)comp->rows;
    a.comp_bs = fp4 ? comp->batch_stride : comp->batch_stride * 2;
    a.comp_rs = fp4 ? comp->row_stride : comp->row_stride * 2;
    a.csc = comp->scales;
    a.csc_bs = comp->scale_batch_stride;
    a.csc_rs = comp->scale_row_stride;
  }
  a.sink = sink;
  a.idx = idx;
  a.L = L;
  a.scale_log2 = scale * kLog2e;
  a.o = (__bf16*)o;
  a.part = workspace ? (float*)((char*)workspace + kWsHeaderBytes) : nullptr;  // after the header
  a.S = S;
  a.H = H;
  // decode batches: two-phase kernel without partial outputs when its shape and residency fit
  const int drc = sparse_attn_decode_launch(a.q, a.win, a.win_n, a.win_bs, a.win_rs, a.comp,
                                            comp && comp->rows ? comp->n_rows : 0, a.comp_bs, a.comp_rs, sink, idx,
                                            L, a.scale_log2, a.o, B, S, H, D, fp4, workspace, nullptr, nullptr,
                                            rope, rope_dim, st);
  if (drc != 0) return drc < 0 ? drc : 0;
  // prefill batches at head_dim 512 (bf16 or fp4 compressed rows): one workgroup per query
  const int prc = sparse_attn_prefill_launch(q, win, comp, sink, idx, L, scale, o, B, S, H, D, rope, rope_dim, st);
  if (prc != 0) return prc < 0 ? prc : 0;
  sparse_attn_split(B, S, L, &a.nsplit, &a.split_slots);
  int rc;
  switch (D) {
    case 64: rc = fp4 ? launch_attn_h<64, true>(a, B, st) : launch_attn_h<64, false>(a, B, st); break;
    case 128: rc = fp4 ? launch_attn_h<128, true>(a, B, st) : launch_attn_h<128, false>(a, B, st); break;
    case 256: rc = fp4 ? launch_attn_h<256, true>(a, B, st) : launch_attn_h<256, false>(a, B, st); break;
    case 512: rc = fp4 ? launch_attn_h<512, true>(a, B, st) : launch_attn_h<512, false>(a, B, st); break;
    default: return fail(DSA_ERR_UNSUPPORTED, "dsa_sparse_attn: bf16 head_dim %d not in {64,128,256,512}", D);
  }
  if (rc || !rope) return rc;
  return rope_inverse_launch(o, DSA_BF16, B, S, H, D, rope, rope_dim, st);
}

// Decode batches whose index rows the attention kernel can select itself (bf16 rows, the
// two-phase decode kernel applies, at most 2048 scores per row): one launch for top-k, window rows
// and attention.  Returns 1 if launched, 0 if not applicable, <0 on error.
int sparse_attn_bf16_select_launch(const void* q, const dsa_kv_src* win, const dsa_kv_src* comp, const float* sink,
                                   const DecSelect* sel, const DecIndex* ix, int L, float scale, void* o, int B, int S,
                                   int H, int D, void* workspace, hipStream_t st) {
  const bool fp4 = comp && comp->rows && comp->format == DSA_KV_FP4_E4M3_G16;
  if (fp4) return 0;
  const unsigned char* comp_rows = comp && comp->rows ? (const unsigned char*)comp->rows : nullptr;
  return sparse_attn_decode_launch((const __bf16*)q, (const unsigned char*)win->rows, win->n_rows,
                                   win->batch_stride * 2, win->row_stride * 2, comp_rows,
                                   comp_rows ? comp->n_rows : 0, comp_rows ? comp->batch_stride * 2 : 0,
                                   comp_rows ? comp->row_stride * 2 : 0, sink, nullptr, L, scale * kLog2e,
                                   (__bf16*)o, B, S, H, D, false, workspace, sel, ix, nullptr, 0, st);
}

size_t sparse_attn_bf16_workspace(int B, int S, int H, int D, int L, bool fp4) {
  int nsplit, per;
  sparse_attn_split(B, S, L, &nsplit, &per);
  const size_t rows = (size_t)B * S * nsplit * H;
  const size_t general = nsplit <= 1 ? 0 : rows * (size_t)D * 4 + rows * 2 * 4;
  const size_t decode = sparse_attn_decode_workspace(B, S, H, D, L, fp4);
  const size_t payload = general > decode ? general : decode;
  return payload ? kWsHeaderBytes + payload : 0;
}

}  // namespace dsa
