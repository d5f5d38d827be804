// Sparse MQA attention for prefill (many queries) at head_dim 512 and up to 64 heads
// (DeepSeek V4.1 page, `sparse_attn_kernel`: gather the indexed rows of the one shared KV tensor,
// softmax with the per-head sink in the denominator, -1 slots ignored).
//
// One workgroup per query, 4 waves; wave w owns heads 16w..16w+15 over the whole head_dim, so a
// wave's logits are complete without any exchange between waves and the only workgroup barrier
// per tile is the one that hands a ring slot over.  Each query gathers ~600 KiB of rows, and every
// row is read by all four waves, twice (as K and as V), so the layout is built for LDS bandwidth:
//  * rows are gathered with 16-byte direct global->LDS copies into a ring of NST 32-row tiles,
//    NST-2 tiles ahead of the tile being multiplied; each wave copies 8 rows per tile, one wave
//    instruction per row, with the row address formed in scalar registers from the index row;
//  * tile rows are 1056 bytes apart: of the pitches measured, that one serves both the K operand
//    reads (16 rows x 16 bytes per 16 lanes) and the transposing V reads at ~150 B/clk per CU;
//  * S^T = K . Q^T on v_mfma_f32_16x16x32_bf16 (rows x 16 heads, K = 32 dims, 4 independent
//    chains); the accumulator of lane (g, c) holds rows 4g..4g+3 and 16+4g..16+4g+3 of head c,
//    which is exactly the B operand of O^T = V^T . P^T when the 32 tile rows are taken in the
//    order (4g+0..3, 16+4g+0..3) for k-group g, so the probabilities never leave their lane;
//  * V^T comes from two ds_read_b64_tr_b16 per operand (rows 4g.. and 16+4g.., one column per
//    lane); O^T is 32 accumulators of 16 dims x 16 heads;
//  * the QK of tile k+1 is issued before the softmax of tile k, so the matrix cores run while the
//    VALU computes the probabilities; online softmax in base 2 with a lazily raised running max
//    (the accumulators are rescaled only when a tile raises a head's max by more than 8).
#include "dsa_internal.h"

namespace dsa {

namespace {

constexpr int kHD = 512;
constexpr int kHTile = 32;
constexpr int kHPitch = 1056;
constexpr int kHTileB = kHTile * kHPitch;
constexpr int kHNST = 4;
constexpr int kHMaxSlots = 1024;
constexpr float kHLog2e = 1.4426950408889634f;
constexpr float kHRescale = 8.0f;
constexpr float kHMinit = -1.0e30f;

constexpr int kHRing = kHNST * kHTileB;
constexpr int kHMasks = kHNST * 8 + 4;  // per slot: valid rows, fp4 rows (a byte per wave each); tile set
constexpr int kHDummy = 1024;  // write target of the decode for rows that are not fp4
// per ring slot and wave: the fp4 scale bytes of the wave's 8 rows (the first 256 of 1024 bytes)
constexpr int kHStage = 1024;
constexpr int kHStageOff = kHRing + kHMasks + 12 + kHMaxSlots * 4 + kHDummy;
constexpr int kHLds = kHStageOff + kHNST * 4 * kHStage;
static_assert(kHStageOff % 16 == 0, "stage alignment");
static_assert(kHLds <= 160 * 1024, "LDS budget");

__device__ __forceinline__ int h_row(int r) { return kHPitch * r; }

typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2;

struct H16Args {
  const __bf16* q;
  const unsigned char* win;
  int64_t win_n, win_rs;  // rows, bytes
  int64_t win_bs;         // bytes
  const unsigned char* comp;
  int64_t comp_bs, comp_rs;  // bytes
  const unsigned char* csc;  // fp4 rows: E4M3 scales, one per 16 elements
  int64_t csc_bs, csc_rs;
  const float* sink;
  const int32_t* idx;
  int L;
  float scale_log2;
  __bf16* o;
  int S, H;
  const float* rope;  // inverse rotary table [S][rope_P][2] (cos, sin), or null
  int rope_P;         // rotated pairs at the end of each head's dims
};

// Source of the copies for -1 slots: a zero row, so every slot costs exactly one copy.
__device__ __attribute__((aligned(1024))) unsigned char g_h16_zero_row[kHD * 2];

// 16-byte global->LDS copy of one row piece per lane.  No memory clobber: the copies only ever
// target a ring slot that no wave reads until after the next wait and barrier (both of which are
// ordered against this statement), so LDS reads of the other slots may be scheduled across it.
__device__ __forceinline__ void h_dma16(const void* sbase, uint32_t voff, const DSA_LDS void* lds_base) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase),
               "{m0}"((uint32_t)(uintptr_t)lds_base));
}


__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// x *= f in the registers x already holds (a plain multiply inside the rare rescale branch makes
// the register allocator shuffle the accumulator set at the branch's merge)
__device__ __forceinline__ void h_scale(f32x4& v, float f) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    float x = v[e];
    asm volatile("v_mul_f32 %0, %0, %1" : "+v"(x) : "v"(f));
    v[e] = x;
  }
}

template <bool FP4>
__global__ void __launch_bounds__(256) sparse_attn_prefill_h16_kernel(H16Args a) {
  constexpr int kHCopies = FP4 ? 9 : 8;  // copy instructions per wave and tile
  __shared__ __attribute__((aligned(1024))) unsigned char smem[kHLds];
  unsigned char* ring = smem;
  unsigned char* masks = smem + kHRing;                                   // [NST][2][4] bytes
  uint32_t* tset = reinterpret_cast<uint32_t*>(masks + kHNST * 8);       // tiles with a valid slot
  int* idx_lds = reinterpret_cast<int*>(smem + kHRing + kHMasks + 12);  // 16-byte aligned
  unsigned char* dummy = smem + kHRing + kHMasks + 12 + kHMaxSlots * 4;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int g = lane >> 4;
  const int c = lane & 15;
  const int head = 16 * wave + c;

  const int qi = blockIdx.x;
  const int b = qi / a.S;
  const int L = a.L;
  const int ntiles = (L + kHTile - 1) / kHTile;

  const unsigned char* win_b = a.win + (int64_t)b * a.win_bs;
  const unsigned char* comp_b = a.comp + (int64_t)b * a.comp_bs;
  const unsigned char* csc_b = FP4 ? a.csc + (int64_t)b * a.csc_bs : nullptr;
  const int* irow = a.idx + (int64_t)qi * L;
  const int win_n = (int)a.win_n;
  const void* win_u = uniform_ptr(win_b);
  const void* comp_u = uniform_ptr(comp_b);
  const void* zero_u = uniform_ptr(g_h16_zero_row);
  const void* csc_u = FP4 ? uniform_ptr(csc_b) : zero_u;

  // ---- prologue: the index row into LDS (copies, -1 past L), this wave's query heads and the
  // sink, in that order, so that the index row can be used while the rest is still in flight ----
  for (int i0 = 64 * wave; i0 < L; i0 += 256) {
    if (i0 + lane < L) dma4_s(irow + i0, (uint32_t)lane * 4u, (DSA_LDS void*)(idx_lds + i0));
  }
  for (int i = L + tid; i < ntiles * kHTile; i += 256) idx_lds[i] = -1;
  if (tid == 0) *tset = 0u;
  // B operand of QK: lane (g, c) holds dims 32s + 8g .. 32s + 8g + 7 of head c.  Exactly 16 loads
  // and one sink load, unconditional (lanes of heads past H read head H-1: finite values whose
  // results are never stored), so that waiting for all but the last 17 vector memory operations
  // waits for the index row only; the sink is scaled where it is used, at the end.
  bf16x8 qreg[16];
  {
    const __bf16* qp = a.q + ((int64_t)qi * a.H + min(head, a.H - 1)) * kHD + 8 * g;
#pragma unroll
    for (int s = 0; s < 16; ++s) qreg[s] = *reinterpret_cast<const bf16x8*>(qp + 32 * s);
  }
  const float sink_raw = a.sink[min(head, a.H - 1)];
  wait_vmcnt<17>();
  __syncthreads();
  // index -> slot code: byte offset from the window or compressed base (bit 0 set for the
  // latter), or 2 for an empty slot; row offsets fit 32 bits (checked at launch).  Each wave
  // converts 64 consecutive slots at a time and marks the tiles among them that hold a valid slot.
  for (int i0 = 64 * wave; i0 < ntiles * kHTile; i0 += 256) {
    const int i = i0 + lane;
    const bool in = i < ntiles * kHTile;
    const int iv = in ? idx_lds[i] : -1;
    uint32_t code;
    if (iv < 0)
      code = 2u;
    else if (iv < win_n)
      code = (uint32_t)iv * (uint32_t)a.win_rs;
    else
      code = (uint32_t)(iv - win_n) * (uint32_t)a.comp_rs | 1u;
    if (in) idx_lds[i] = (int)code;
    const uint64_t v = __builtin_amdgcn_ballot_w64(in && iv >= 0);
    const uint32_t bits = (v & 0xFFFFFFFFull ? 1u : 0u) | (v >> 32 ? 2u : 0u);
    if (lane == 0 && bits) atomicOr(tset, bits << (i0 / kHTile));
  }
  __syncthreads();
  // The loop runs over the tiles that hold at least one valid slot, in order (a tile of -1 slots
  // adds nothing); position k of that list lives in ring slot k % NST.
  uint32_t pend = __builtin_amdgcn_readfirstlane(*tset);
  const int nt = __builtin_popcount(pend);

  // copies of this wave's 8 rows of position k and the tile's valid-row and fp4-row bytes.  Every
  // row is one wave instruction from a scalar base (slot codes: byte offset of the row from its
  // base, bit 0 = compressed row, bit 1 = empty slot, read from the zero row).  An fp4 row (256
  // nibble bytes) is read by lanes l and l+16, l+32, l+48 alike, so nothing past it is read; the
  // copies land in the first 1024 bytes of its pitch, where the decode writes the bf16 row.  One
  // more instruction per tile fetches the 32 scale bytes of each of the 8 rows into the wave's
  // stage of the slot (from the zero row when the tile has no fp4 row of this wave).
  // the slot codes of the next tile to copy (lane l: row 8*wave + l%8), read one issue ahead so
  // the read is off the path from the barrier to the copies
  int nidx = pend ? idx_lds[__builtin_ctz(pend) * kHTile + 8 * wave + (lane & 7)] : 0;
  // (fp4: lane l also holds the code of row (l mod 16)/2, for the scale copy)
  int nsc = (FP4 && pend) ? idx_lds[__builtin_ctz(pend) * kHTile + 8 * wave + ((lane & 15) >> 1)] : 0;
  auto issue = [&](int k) {
    pend &= pend - 1u;  // the tile being copied, whose codes are already in nidx (and nsc)
    const int myidx = nidx;
    const int slot = k % kHNST;
    const uint32_t vbits = (uint32_t)__builtin_amdgcn_ballot_w64(lane < 8 && !(myidx & 2));
    const uint32_t fbits = FP4 ? (uint32_t)__builtin_amdgcn_ballot_w64(lane < 8 && (myidx & 1)) : 0u;
    if (lane == 0) {
      masks[slot * 8 + wave] = (unsigned char)vbits;
      masks[slot * 8 + 4 + wave] = (unsigned char)fbits;
    }
    unsigned char* tb = ring + slot * kHTileB;
    const uint32_t fold = (uint32_t)(lane & 48) * 16u;  // lane*16 - fold = (lane mod 16)*16
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const uint32_t x = (uint32_t)__builtin_amdgcn_readlane(myidx, r);
      const uint32_t voff = (uint32_t)lane * 16u - (FP4 ? (x & 1u) * fold : 0u);
      h_dma16(slot_base(x, win_u, comp_u, zero_u), voff + (x & ~15u), (DSA_LDS void*)(tb + h_row(8 * wave + r)));
    }
    if constexpr (FP4) {
      // lane l (mod 16): 16 of the 32 scale bytes of row (l mod 16)/2 (scale rows are 32 bytes for
      // 256-byte nibble rows, so a row's byte offset / 8 is its scale row's); other rows re-read
      // scale row 0
      const uint32_t sc = (uint32_t)nsc;
      const uint32_t soff = ((sc & 1u) ? ((sc & ~15u) >> 3) : 0u) + (uint32_t)(lane & 1) * 16u;
      h_dma16(fbits ? csc_u : zero_u, fbits ? soff : 0u,
              (DSA_LDS void*)(smem + kHStageOff + (slot * 4 + wave) * kHStage));
    }
    if (pend) {
      nidx = idx_lds[__builtin_ctz(pend) * kHTile + 8 * wave + (lane & 7)];
      if constexpr (FP4) nsc = idx_lds[__builtin_ctz(pend) * kHTile + 8 * wave + ((lane & 15) >> 1)];
    }
  };
  // fp4 rows of position k that this wave copied, decoded in place (it has waited for its own
  // copies; the next barrier publishes them): lane l writes elements 8l..8l+7 from nibble bytes
  // 4l..4l+3 and scale byte l/2; a row's reads all complete before its write (one wave, in order).
  // All 8 rows go through the same instructions (a row that is not fp4 writes to a dummy area), so
  // the reads of every row are issued before the first conversion.
  auto decode = [&](int k) {
    if constexpr (FP4) {
      const int slot = k % kHNST;
      const uint32_t fb = __builtin_amdgcn_readfirstlane(masks[slot * 8 + 4 + wave]);
      if (fb != 0u) {
        unsigned char* tb = ring + slot * kHTileB + h_row(8 * wave);
        const unsigned char* stg = smem + kHStageOff + (slot * 4 + wave) * kHStage;
        uint32_t word[8], scb[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          word[r] = *reinterpret_cast<const uint32_t*>(tb + h_row(r) + 4 * lane);
          scb[r] = stg[32 * r + (lane >> 1)];
        }
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          const float sc = __builtin_amdgcn_cvt_f32_fp8((int)scb[r], 0);
          // e2m1 pairs at unit scale (exact), times the E4M3 scale: exact in f32 and in bf16
          const f32x2 e0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word[r], 1.0f, 0);
          const f32x2 e1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word[r], 1.0f, 1);
          const f32x2 e2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word[r], 1.0f, 2);
          const f32x2 e3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word[r], 1.0f, 3);
          auto pk = [&](f32x2 e) { return __builtin_bit_cast(uint32_t, bf16x2{(__bf16)(e[0] * sc), (__bf16)(e[1] * sc)}); };
          const u32x4 v = {pk(e0), pk(e1), pk(e2), pk(e3)};
          unsigned char* dst = ((fb >> r) & 1u) ? tb + h_row(r) : dummy;
          *reinterpret_cast<u32x4*>(dst + 16 * lane) = v;
        }
      }
    }
  };
#pragma unroll
  for (int j = 0; j < kHNST - 1; ++j)
    if (j < nt) issue(j);

  // lane bases: K operand (row c, 16-byte chunk 4s + g) and transposed V operand (rows 4g + c/4,
  // 32-byte column block, 8 bytes per lane)
  const int k_base = h_row(c) + 16 * g;
  const int k_hi = h_row(c + 16) - h_row(c);
  const int v_base = h_row(4 * g + (c >> 2)) + 8 * (c & 3);
  const int v_hi = h_row(16 + 4 * g + (c >> 2)) - h_row(4 * g + (c >> 2));

  // QK of position k: operand i (k-step i/2 of row block i%2) feeds chain 2(i%2) + (i/2)%2, so each
  // chain's MFMAs are four apart; the K reads run eight operands ahead of the MFMAs.
  auto kread = [&](const unsigned char* kp, int i) {
    return *reinterpret_cast<const bf16x8*>(kp + (i & 1) * k_hi + 64 * (i >> 1));
  };
  auto vread = [&](const unsigned char* vp, int d) {
    const bf16x4 lo = lds_read_tr16((const DSA_LDS __bf16*)(vp + 32 * d));
    const bf16x4 hi = lds_read_tr16((const DSA_LDS __bf16*)(vp + v_hi + 32 * d));
    return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  };

  f32x4 acc[32];
#pragma unroll
  for (int d = 0; d < 32; ++d) acc[d] = f32x4{};
  float m_run = kHMinit;
  float l_run = 0.f;
  auto tile_vmask = [&](int k) { return *reinterpret_cast<const uint32_t*>(masks + (k % kHNST) * 8); };

  // logits of the current position as four chains (summed when first used)
  f32x4 ch[4] = {};
  uint32_t vm = 0u;
  if (nt > 0) {
    if constexpr (FP4) {
      // positions 0 and 1 landed (own copies) and decoded before the first QK
      if (nt > 2)
        wait_vmcnt<kHCopies>();
      else
        wait_vmcnt<0>();
      decode(0);
      if (nt > 1) decode(1);
    } else {
      const int later0 = min(kHNST - 2, nt - 1);
      if (later0 >= 2)
        wait_vmcnt<2 * kHCopies>();
      else if (later0 == 1)
        wait_vmcnt<kHCopies>();
      else
        wait_vmcnt<0>();
    }
    __syncthreads();
#pragma unroll
    for (int s = 0; s < 16; ++s) asm volatile("" : "+a"(qreg[s]));
    const unsigned char* kp = ring + k_base;
#pragma unroll
    for (int i = 0; i < 32; ++i) ch[2 * (i & 1) + ((i >> 1) & 1)] = mfma16(kread(kp, i), qreg[i >> 1], ch[2 * (i & 1) + ((i >> 1) & 1)]);
    vm = tile_vmask(0);
  }

  for (int k = 0; k < nt; ++k) {
    // tile k+1 has landed once at most the copies of tile k+2 are out; the barrier also means every
    // wave is done with tile k-1, whose slot is refilled below
    if (k + 2 < nt)
      wait_vmcnt<kHCopies>();
    else
      wait_vmcnt<0>();
    __syncthreads();
    if (k + kHNST - 1 < nt) issue(k + kHNST - 1);
    const uint32_t vm_next = tile_vmask(k + 1);
    const unsigned char* kp = ring + ((k + 1) % kHNST) * kHTileB + k_base;
    const unsigned char* vp = ring + (k % kHNST) * kHTileB + v_base;

    // ---- one scheduling region: QK of tile k+1 on the matrix cores (a stale slot past the last
    // tile; never used), the softmax of tile k on the VALU against the running max as it stands,
    // and the first V operands of tile k ----
    const f32x4 sc0 = ch[0] + ch[1], sc1 = ch[2] + ch[3];
    f32x4 cn[4] = {};
    {
      bf16x8 kr[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) kr[i] = kread(kp, i);
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        const int sk = i >> 1, rb = i & 1;
        cn[2 * rb + (sk & 1)] = mfma16(kr[i & 7], qreg[sk], cn[2 * rb + (sk & 1)]);
        if (i + 8 < 32) kr[i & 7] = kread(kp, i + 8);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
      for (int i = 0; i < 24; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
    }
    // lane (g, c) holds rows 4g+v and 16+4g+v of head c
    float sv[8];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      sv[v] = (vm >> (4 * g + v)) & 1u ? sc0[v] : -__builtin_inff();
      sv[4 + v] = (vm >> (16 + 4 * g + v)) & 1u ? sc1[v] : -__builtin_inff();
    }
    float mloc = sv[0];
#pragma unroll
    for (int j = 1; j < 8; ++j) mloc = fmaxf(mloc, sv[j]);
    mloc = fmaxf(mloc, shfl_xor(mloc, 16));
    mloc = fmaxf(mloc, shfl_xor(mloc, 32)) * a.scale_log2;  // scale > 0
    float p[8];
    float lsum = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      p[j] = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[j], a.scale_log2, -m_run));
      lsum += p[j];
    }
    constexpr int kVPre = 4;
    bf16x8 vpre[kVPre];
#pragma unroll
    for (int d = 0; d < kVPre; ++d) vpre[d] = vread(vp, d);

    // rare: a tile raised some head's max by more than 8; rescale and redo the probabilities
    if (__builtin_amdgcn_ballot_w64(mloc > m_run + kHRescale) != 0ull) {
      const float m_new = fmaxf(m_run, mloc);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int d = 0; d < 32; ++d) h_scale(acc[d], alpha);
      lsum = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        p[j] = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[j], a.scale_log2, -m_run));
        lsum += p[j];
      }
    }
    l_run += lsum;
    bf16x8 pb;
#pragma unroll
    for (int j = 0; j < 8; ++j) pb[j] = (__bf16)p[j];

    // ---- matrix cores: O^T += V^T . P^T over the whole head_dim (32 independent chains), the
    // V reads eight operands ahead ----
#pragma unroll
    for (int d = 0; d < 32; ++d) acc[d] = mfma16(d < kVPre ? vpre[d] : vread(vp, d), pb, acc[d]);
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
    for (int i = 0; i < 24; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
#pragma unroll
    for (int j = 0; j < 4; ++j) ch[j] = cn[j];
    vm = vm_next;
    if constexpr (FP4) {
      // position k+2: its copies (own) landed once at most those of k+3 are out; decoded here so
      // the next iteration's barrier publishes it before its QK
      if (k + 2 < nt) {
        if (k + 3 < nt)
          wait_vmcnt<kHCopies>();
        else
          wait_vmcnt<0>();
        decode(k + 2);
      }
    }
  }
  wait_vmcnt<0>();

  if (head >= a.H) return;
  const float sink2 = sink_raw * kHLog2e;
  float l_tot = l_run + shfl_xor(l_run, 16);
  l_tot += shfl_xor(l_tot, 32);
  const float mf = fmaxf(m_run, sink2);
  const float f = exp2f(m_run - mf);
  const float rn = f / (l_tot * f + exp2f(sink2 - mf));
  // lane (g, c) holds dims 16d + 4g .. 16d + 4g + 3 of head c: two whole rotary pairs
  __bf16* op = a.o + ((int64_t)qi * a.H + head) * kHD + 4 * g;
  const int rope0 = kHD - 2 * a.rope_P;  // first rotated dim (a multiple of 16), kHD without a table
  const float* rrow = a.rope ? a.rope + (int64_t)(qi % a.S) * a.rope_P * 2 : nullptr;
#pragma unroll
  for (int d = 0; d < 32; ++d) {
    float v[4] = {acc[d][0] * rn, acc[d][1] * rn, acc[d][2] * rn, acc[d][3] * rn};
    if (rrow && 16 * d >= rope0) {
      const float4 cs = *reinterpret_cast<const float4*>(rrow + (16 * d + 4 * g - rope0));
      rope_rot_inv(v[0], v[1], cs.x, cs.y);
      rope_rot_inv(v[2], v[3], cs.z, cs.w);
    }
    const bf16x4 ov = {(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
    *reinterpret_cast<bf16x4*>(op + 16 * d) = ov;
  }
}

}  // namespace

// Launches the kernel when it applies (bf16 window rows, bf16 or fp4 compressed rows, head_dim 512,
// at most 64 heads, index rows of at most 1024 slots, enough queries to fill the GPU, 16-byte
// aligned rows and scale rows, row offsets within 32 bits, positive scale); returns 1 if
// launched, 0 if not, <0 on error.
int sparse_attn_prefill_h16_launch(const void* q, const dsa_kv_src* win, const dsa_kv_src* comp, const float* sink,
                                   const int32_t* idx, int L, float scale, void* o, int B, int S, int H, int D,
                                   const float* rope, int rope_dim, hipStream_t st) {
  const int Q = B * S;
  if (D != kHD || H > 64 || L > kHMaxSlots || Q < 256) return 0;
  const bool fp4 = comp && comp->rows && comp->format == DSA_KV_FP4_E4M3_G16;
  H16Args a{};
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
  // slot codes hold row byte offsets (fp4: row numbers) in 32 bits; the softmax folds a positive
  // scale into exp2
  if (!(scale > 0.f) || (uint64_t)a.win_n * (uint64_t)a.win_rs >= (1ull << 31)) return 0;
  if (a.comp && (uint64_t)comp->n_rows * (uint64_t)a.comp_rs >= (1ull << 31)) return 0;
  // fp4 rows: 256 nibble bytes and 32 scale bytes per row, densely strided (a row's byte offset
  // / 8 is then its scale row's)
  if (fp4 && (a.comp_rs != kHD / 2 || a.csc_rs != kHD / 16)) return 0;
  a.sink = sink;
  a.idx = idx;
  a.L = L;
  a.scale_log2 = scale * kHLog2e;
  a.o = (__bf16*)o;
  a.S = S;
  a.H = H;
  a.rope = rope;
  a.rope_P = rope ? rope_dim / 2 : 0;
  if (fp4)
    hipLaunchKernelGGL(sparse_attn_prefill_h16_kernel<true>, dim3(Q), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(sparse_attn_prefill_h16_kernel<false>, dim3(Q), dim3(256), 0, st, a);
  const int rc = check_launch("sparse_attn_prefill_h16");
  return rc ? rc : 1;
}

}  // namespace dsa
