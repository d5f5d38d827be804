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
  static constexpr int MASKS = 2 * NST * 4 + 4;  // per ring slot: valid rows, fp4 rows (a byte per wave); tile set
  static constexpr int LDS = RING + RAWS + XBUF + MASKS + kPMaxSlots * 4;
  static_assert(LDS <= 160 * 1024, "LDS budget");
};

// Source of the copies for -1 slots: a zero row, so every slot costs exactly one copy.
__device__ __attribute__((aligned(1024))) unsigned char g_pre_zero_row[kPD * 2];

__device__ __forceinline__ int p_slot(int r) { return (r & 16) | ((r & 3) << 2) | ((r >> 2) & 3); }

// e2m1 code in bits 3:0 of n -> its value times 2^-126: the three magnitude bits placed at bit 22
// are the exponent field and top mantissa bit of the f32 (code 1, the e2m1 subnormal 0.5, lands on
// the f32 subnormal 2^-127); f32 subnormals are kept in this code.
__device__ __forceinline__ float p_e2m1_tiny(uint32_t n) {
  return __uint_as_float(((n & 7u) << 22) | ((n & 8u) << 28));
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

// x *= f in the register x already holds: a plain multiply inside the rare rescale branch makes
// the register allocator shuffle the whole accumulator set at the branch's merge.
__device__ __forceinline__ void scale_in_place(f32x16& v, float f) {
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    float x = v[e];
    asm volatile("v_mul_f32 %0, %0, %1" : "+v"(x) : "v"(f));
    v[e] = x;
  }
}

template <bool FP4>
__global__ void __launch_bounds__(256) sparse_attn_prefill_kernel(PreArgs a) {
  using C = PreCfg<FP4>;
  __shared__ __attribute__((aligned(1024))) unsigned char smem[C::LDS];
  unsigned char* ring = smem;
  unsigned char* raw = smem + C::RING;
  float* xbuf = reinterpret_cast<float*>(smem + C::RING + C::RAWS);
  unsigned char* masks = smem + C::RING + C::RAWS + C::XBUF;  // [NST][2][4] bytes
  uint32_t* tset = reinterpret_cast<uint32_t*>(masks + 2 * C::NST * 4);  // tiles with a valid slot
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
  const void* win_u = uniform_ptr(win_b);
  const void* comp_u = uniform_ptr(comp_b);
  const void* zero_u = uniform_ptr(zero_row);
  asm volatile("" : "+s"(zero_row));

  // Gather this wave's rows of tile ti into ring slot ti % NST: one copy per row (a -1 slot copies
  // the zero row), and record which rows are valid and which are fp4 rows still to decode.
  // The copies of a tile are issued in parts (rows k0..k1-1 of this wave's 8), spread over the
  // phases of the previous tile's work: a CU takes in copies at a bounded rate, and a copy issued
  // while the queue is full stalls its wave.  `myidx` holds the tile's slots in lanes 0..7.
  // slot codes (see the prologue): byte offset of the row from its base, bit 0 = compressed row,
  // bit 1 = empty slot (the zero row); for an fp4 compressed row the offset field holds its row
  auto tile_index = [&](int tile) { return idx_lds[tile * kPTile + 8 * wave + (lane & 7)]; };
  auto issue_masks = [&](int k, int myidx) {
    const int slot = k % C::NST;
    const uint32_t vbits = (uint32_t)__builtin_amdgcn_ballot_w64(lane < 8 && !(myidx & 2));
    const uint32_t fbits = FP4 ? (uint32_t)__builtin_amdgcn_ballot_w64(lane < 8 && (myidx & 1)) : 0u;
    if (lane == 0) {
      masks[slot * 8 + wave] = (unsigned char)vbits;
      masks[slot * 8 + 4 + wave] = (unsigned char)fbits;
    }
  };
  auto issue_rows = [&](int kpos, int myidx, int k0, int k1) {
    const int slot = kpos % C::NST;
    unsigned char* tile = ring + slot * C::TILE;
    unsigned char* rtile = FP4 ? raw + slot * C::RAW : nullptr;
#pragma unroll
    for (int k = k0; k < k1; ++k) {
      const int r = 8 * wave + k;
      const uint32_t x = (uint32_t)__builtin_amdgcn_readlane(myidx, k);
      if (FP4 && (x & 1u)) {
        // the raw row: 256 nibble bytes from lanes 0..15, then its 32 scale bytes from lanes 16..17
        const int64_t cr = x >> 4;
        const unsigned char* src =
            lane < 16 ? comp_b + cr * a.comp_rs + lane * 16 : csc_b + cr * a.csc_rs + (lane - 16) * 16;
        if (lane < 18) dma16_v(src, (DSA_LDS void*)(rtile + r * 288));
      } else {
        dma16_s(slot_base(x, win_u, comp_u, zero_u), (uint32_t)lane * 16u + (x & ~15u),
                (DSA_LDS void*)(tile + p_slot(r) * kPRow));
      }
    }
  };
  auto issue = [&](int k, int tile) {
    const int myidx = tile_index(tile);
    issue_masks(k, myidx);
    issue_rows(k, myidx, 0, 8);
  };

  // ---- prologue: the index row into LDS (copies, -1 past L), this wave's query heads (its half of
  // D), then the first tiles ----
  for (int i0 = 64 * wave; i0 < L; i0 += 256) {
    if (i0 + lane < L) dma4_s(irow + i0, (uint32_t)lane * 4u, (DSA_LDS void*)(idx_lds + i0));
  }
  for (int i = L + tid; i < ntiles * kPTile; i += 256) idx_lds[i] = -1;
  if (tid == 0) *tset = 0u;
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
  // index -> slot code: byte offset from the window or compressed base (bit 0 set for the
  // latter), or 2 for an empty slot; row offsets fit 32 bits (checked at launch)
  for (int i = tid; i < ntiles * kPTile; i += 256) {
    const int iv = idx_lds[i];
    uint32_t code;
    if (iv < 0)
      code = 2u;
    else if (iv < win_n)
      code = (uint32_t)iv * (uint32_t)a.win_rs;
    else
      code = FP4 ? ((uint32_t)(iv - win_n) << 4) | 1u : (uint32_t)(iv - win_n) * (uint32_t)a.comp_rs | 1u;
    idx_lds[i] = (int)code;
  }
  __syncthreads();
  // The loop runs over the tiles that hold at least one valid slot (a tile of -1 slots adds
  // nothing), in order; `pend` holds the tiles still to be issued.
  for (int i0 = 64 * wave; i0 < ntiles * kPTile; i0 += 256) {
    const uint64_t v = __builtin_amdgcn_ballot_w64(i0 + lane < ntiles * kPTile && !(idx_lds[i0 + lane] & 2));
    const uint32_t bits = (v & 0xFFFFFFFFull ? 1u : 0u) | (v >> 32 ? 2u : 0u);
    if (lane == 0 && bits) atomicOr(tset, bits << (i0 / kPTile));
  }
  __syncthreads();
  uint32_t pend = __builtin_amdgcn_readfirstlane(*tset);
  const int ntiles_live = __builtin_popcount(pend);
  auto next_tile = [&]() {
    const int tile = __builtin_ctz(pend);
    pend &= pend - 1u;
    return tile;
  };
#pragma unroll
  for (int j = 0; j < C::NST - 1; ++j)
    if (j < ntiles_live) issue(j, next_tile());

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

  auto tile_ptr = [&](int tj) -> const unsigned char* { return ring + (tj % C::NST) * C::TILE; };
  auto tile_vmask = [&](int tj) { return *reinterpret_cast<const uint32_t*>(masks + (tj % C::NST) * 8); };

  // decode tile tj's fp4 rows into bf16 (wave w takes rows w, w+4, ..., one 16-byte chunk per lane)
  auto decode = [&](int tj) {
    if constexpr (FP4) {
      const int slot = tj % C::NST;
      const uint32_t fmask = *reinterpret_cast<const uint32_t*>(masks + slot * 8 + 4);
      const unsigned char* rtile = raw + slot * C::RAW;
      unsigned char* wtile = ring + slot * C::TILE;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int r = 4 * k + wave;
        if ((fmask >> r) & 1u) {
          const uint32_t word = *reinterpret_cast<const uint32_t*>(rtile + r * 288 + lane * 4);
          const float sc = p_e4m3(rtile[r * 288 + 256 + (lane >> 1)]);
          u32x4 v;
#pragma unroll
          for (int kk = 0; kk < 4; ++kk) {
            // value = e2m1 * scale, exact in f32 and in bf16
            const float lo = __builtin_amdgcn_ldexpf(p_e2m1_tiny(word >> (8 * kk)), 126) * sc;
            const float hi = __builtin_amdgcn_ldexpf(p_e2m1_tiny(word >> (8 * kk + 4)), 126) * sc;
            const bf16x2 pr = {(__bf16)lo, (__bf16)hi};
            v[kk] = __builtin_bit_cast(uint32_t, pr);
          }
          *reinterpret_cast<u32x4*>(wtile + p_slot(r) * kPRow + lane * 16) = v;
        }
      }
    }
  };

  // partial S^T of tile tj over this wave's half of D, in two independent chains
  auto qk = [&](int tj, f32x16& s0, f32x16& s1) {
    const unsigned char* kp = tile_ptr(tj) + k_base;
    s0 = f32x16{};
    s1 = f32x16{};
#pragma unroll
    for (int s = 0; s < 16; s += 2) {
      const bf16x8 k0 = *reinterpret_cast<const bf16x8*>(kp + 32 * s);
      const bf16x8 k1 = *reinterpret_cast<const bf16x8*>(kp + 32 * s + 32);
      s0 = mfma32(k0, qreg[s], s0);
      s1 = mfma32(k1, qreg[s + 1], s1);
    }
  };
  auto xbuf_put = [&](const f32x16& s0, const f32x16& s1) {
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const f32x4 v = {s0[4 * g4] + s1[4 * g4], s0[4 * g4 + 1] + s1[4 * g4 + 1], s0[4 * g4 + 2] + s1[4 * g4 + 2],
                       s0[4 * g4 + 3] + s1[4 * g4 + 3]};
      *reinterpret_cast<f32x4*>(xmine + (g4 * 64 + lane) * 4) = v;
    }
  };
  // full q.k of the tile from both halves' partial sums; -inf where the slot is empty
  auto xbuf_get = [&](uint32_t vmask, float (&sv)[16]) {
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const f32x4 mine = *reinterpret_cast<const f32x4*>(xmine + (g4 * 64 + lane) * 4);
      const f32x4 part = *reinterpret_cast<const f32x4*>(xpart + (g4 * 64 + lane) * 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float full = dh == 0 ? mine[i] + part[i] : part[i] + mine[i];  // same sum in both halves
        sv[4 * g4 + i] = full;
      }
    }
    if (vmask != 0xFFFFFFFFu) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int row = 8 * (e >> 2) + 4 * hf + (e & 3);
        if (!((vmask >> row) & 1u)) sv[e] = -__builtin_inff();
      }
    }
  };

  // Software pipeline over the live tiles (position k is ring slot k % NST): iteration k runs QK of
  // tile k+1 on the matrix cores while the VALU does the softmax of tile k, then PV of tile k while
  // the partial logits of tile k+1 are exchanged; the copies of tile k+NST-1 are issued in parts
  // between those phases.  Before the loop: tile 0's logits.
  const int nt = ntiles_live;
  float sv[16];
  if (nt > 0) {
    const int later0 = min(C::NST - 2, nt - 1);
    if (later0 >= 2)
      wait_vmcnt<16>();
    else if (later0 == 1)
      wait_vmcnt<8>();
    else
      wait_vmcnt<0>();
    __syncthreads();
    if constexpr (FP4) {
      decode(0);
      __syncthreads();
    }
    f32x16 s0, s1;
    qk(0, s0, s1);
    xbuf_put(s0, s1);
    __syncthreads();
    xbuf_get(tile_vmask(0), sv);
  }

  for (int k = 0; k < nt; ++k) {
    const bool has_next = k + 1 < nt;
    // tile k+1 has landed once at most the copies of tile k+2 (issued one iteration ago) are out
    if (has_next) {
      if (k + 2 < nt && C::NST >= 4)
        wait_vmcnt<8>();
      else
        wait_vmcnt<0>();
    }
    __syncthreads();  // also: every wave is done with tile k-1, whose slot is refilled below
    if constexpr (FP4) {
      if (has_next) decode(k + 1);
      __syncthreads();
    }
    const int kn = k + C::NST - 1;
    const bool refill = kn < nt;
    int nidx = 0;
    if (refill) {
      nidx = tile_index(next_tile());
      issue_masks(kn, nidx);
      issue_rows(kn, nidx, 0, 2);
    }
    // ---- softmax of tile k, first part: its max, and the rare rescale of the accumulators ----
    // (ahead of QK of tile k+1, so the accumulators are the only large live set there)
    {
      float mloc = sv[0];
#pragma unroll
      for (int e = 1; e < 16; ++e) mloc = fmaxf(mloc, sv[e]);
      mloc = fmaxf(mloc, shfl_xor(mloc, 32)) * a.scale_log2;  // scale > 0
      if (__builtin_amdgcn_ballot_w64(mloc > m_run + kPRescale) != 0ull) {
        const float m_new = fmaxf(m_run, mloc);
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int m = 0; m < 8; ++m) scale_in_place(acc[m], alpha);
      }
    }
    // ---- matrix cores: QK of tile k+1 ----
    f32x16 s0, s1;
    if (has_next) qk(k + 1, s0, s1);
    if (refill) issue_rows(kn, nidx, 2, 4);

    // ---- VALU: probabilities of tile k (a -1 slot's logit is -inf: p = 0) ----
    bf16x8 pb[2];
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[e], a.scale_log2, -m_run));
      l_run += p;
      pb[e >> 3][e & 7] = (__bf16)p;
    }
    // tile k+1's partial logits out to LDS (waits for its QK), which frees their registers
    if (has_next) xbuf_put(s0, s1);
    if (refill) issue_rows(kn, nidx, 4, 6);
    // ---- matrix cores: O^T += V^T . P^T on this wave's half of D (8 independent chains); k step
    // ks, part pt reads tile rows 16ks + 8pt + 4hf + 0..3 = slots 16ks + 2pt + hf + 4*(0..3) ----
    {
      const unsigned char* vp = tile_ptr(k) + v_base;
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
    if (refill) issue_rows(kn, nidx, 6, 8);
    // ---- tile k+1's full logits from both halves ----
    if (has_next) {
      __syncthreads();
      xbuf_get(tile_vmask(k + 1), sv);
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
  // slot codes hold row byte offsets in 32 bits; the softmax folds a positive scale into exp2
  if (!(scale > 0.f) || (uint64_t)a.win_n * (uint64_t)a.win_rs >= (1ull << 31)) return 0;
  if (comp && comp->rows && (uint64_t)comp->n_rows * (uint64_t)(fp4 ? 16 : a.comp_rs) >= (1ull << 31)) return 0;
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
