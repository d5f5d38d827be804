// Sparse MQA attention for prefill (many queries) at head_dim 512 and up to 64 heads
// (DeepSeek V4.1 page, `sparse_attn_kernel`: gather the indexed rows of the one shared KV tensor,
// softmax with the per-head sink in the denominator, -1 slots ignored).
//
// One workgroup of two waves per query; wave w owns heads 32w..32w+31 over the whole head_dim, so
// a wave's logits are complete without any exchange and the only barrier per tile is the one that
// hands a ring slot over.  Each KV row staged in LDS is read by the two waves twice (as K and as
// V), and every read feeds 32 heads.  A workgroup takes under 80 KiB of LDS and one SIMD per wave,
// so two queries share a CU: one query's fixed costs (index row, q, the first copies, the output)
// overlap the other's tiles.
//  * rows are gathered with 16-byte direct global->LDS copies into a ring of two 32-row tiles; the
//    copies of tile k+1 go out as soon as tile k-1 has left the ring; each wave copies 16 rows per
//    tile, one wave instruction per row, with the row address formed in scalar registers from the
//    index row;
//  * tile rows are 1088 bytes apart with the chunks of each 64-byte block XOR-permuted per row
//    (p_swz), which keeps both operand reads below free of bank conflicts;
//  * S^T = K . Q^T as four v_mfma_f32_16x16x32_bf16 blocks per k-step (row half x head half, one
//    chain each): K from LDS (ds_read_b128), the wave's 32 query heads resident in VGPRs as the B
//    operand.  Lane (g, c) of the accumulators holds rows 4g..4g+3 (+16) of heads c and 16 + c;
//  * O^T = V^T . P^T on v_mfma_f32_32x32x16_bf16: one permlane16 swap per register pair between
//    16-lane groups turns the probabilities into its B operand (rows 8hf..8hf+7 of head lane%32 per
//    k-step), so they never go through LDS; V^T comes from two ds_read_b64_tr_b16 per operand; O^T
//    is 16 accumulators of 32 dims x 32 heads (the wave's AGPRs);
//  * online softmax in base 2 with a lazily raised running max (the accumulators are rescaled only
//    when a tile raises a head's max by more than 8);
//  * fp4 compressed rows (e2m1 nibbles + one E4M3 scale per 16) are copied as they lie (256 nibble
//    bytes and 32 scale bytes per row) and decoded to bf16 in place by the wave that copied them;
//    every e2m1 x E4M3 product is exact in bf16.
#include "dsa_internal.h"

namespace dsa {

namespace {

constexpr int kPD = 512;
constexpr int kPTile = 32;
constexpr int kPPitch = 1088;
constexpr int kPTileB = kPTile * kPPitch;
constexpr int kPNST = 2;
constexpr int kPMaxSlots = 1024;
constexpr int kPThreads = 128;
constexpr float kPLog2e = 1.4426950408889634f;
constexpr float kPRescale = 8.0f;
constexpr float kPMinit = -1.0e30f;

// LDS: the ring, per slot the valid-row and fp4-row words (16 bits per wave each), the tile set,
// the index row as slot codes; fp4 adds a write target for rows that are not fp4 and, per slot
// and wave, the scale bytes of the wave's 16 rows (512 bytes, staged by one 1 KiB copy)
constexpr int kPRing = kPNST * kPTileB;
constexpr int kPMaskOff = kPRing;
constexpr int kPTsetOff = kPMaskOff + kPNST * 8;
constexpr int kPIdxOff = kPTsetOff + 16;
constexpr int kPDummyOff = kPIdxOff + kPMaxSlots * 4;
constexpr int kPStage = 1024;
constexpr int kPStageOff = kPDummyOff + 1024;
constexpr int kPLdsBf16 = kPDummyOff;
constexpr int kPLdsFp4 = kPStageOff + kPNST * 2 * kPStage;
static_assert(kPIdxOff % 16 == 0 && kPStageOff % 16 == 0, "alignment");
static_assert(kPLdsFp4 <= 80 * 1024, "two workgroups per CU");

__device__ __forceinline__ int p_row(int r) { return kPPitch * r; }

// Tile rows are 1088 bytes apart (16 banks of 4 bytes further per row) and the four 16-byte chunks
// of each 64-byte block are XOR-permuted by p_swz(r) = (r / 4) % 4: logical chunk j of tile row r
// sits at physical chunk j ^ p_swz(r).  Then the K reads (16 rows at one logical chunk) and the
// transposing V reads (4 rows x 4 consecutive chunks per 32 lanes) each fall on 64 distinct banks,
// and every 64-byte block of a row is still copied by four consecutive lanes.
__device__ __forceinline__ uint32_t p_swz(int r) { return (uint32_t)((r >> 2) & 3); }

// The MFMAs are written as inline asm so that their operands sit where the loop needs them: the
// query heads (B of QK) and the logits in VGPRs, the output accumulators in AGPRs for the whole
// query.  The compiler inserts no wait states around inline asm, so the code provides them where
// an MFMA result or operand meets other instructions:
//  * a dependent MFMA reading its own accumulator as SrcC (same opcode, same registers) needs none;
//  * VALU reads of an MFMA result wait s_nop 15 (16 states, more than the 8-pass 16x16x32 MFMA
//    requires) or s_nop 15 + s_nop 3 (20 states, for the 16-pass 32x32x16);
//  * an MFMA reading a VGPR (or AGPR) written by a VALU instruction waits s_nop 1 (2 states): an
//    empty-bodied statement that emits it and takes the written registers as in-out operands
//    stands between the writes and every MFMA that reads them.
// Operands loaded from LDS or memory are covered by the s_waitcnt the compiler places before the
// statement that reads them.
__device__ __forceinline__ f32x4 qk_first(bf16x8 a, bf16x8 b) {
  f32x4 d;
  asm("v_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "v"(b));
  return d;
}
__device__ __forceinline__ void qk_next(f32x4& d, bf16x8 a, bf16x8 b) {
  asm("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "v"(b));
}
__device__ __forceinline__ void pv_mfma(f32x16& d, bf16x8 a, bf16x8 b) {
  asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(d) : "v"(a), "v"(b));
}

typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2;

struct PArgs {
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
__device__ __attribute__((aligned(1024))) unsigned char g_prefill_zero_row[kPD * 2];

// 16-byte global->LDS copy of one row piece per lane.  No memory clobber: the copies only ever
// target a ring slot (or stage) that no wave reads until after the next wait and barrier, both of
// which are ordered against this statement, so LDS reads of the other slot may be scheduled
// across it.
__device__ __forceinline__ void p_dma16(const void* sbase, uint32_t voff, const DSA_LDS void* lds_base) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase),
               "{m0}"((uint32_t)(uintptr_t)lds_base));
}

// Workgroup i runs on XCD i mod 8, and each XCD has its own L2.  Runs of 64 consecutive queries
// (whose window rows coincide, and whose top-k rows tend to overlap in real sequences) go to one
// XCD, and the runs are taken from the last query down: later queries see more rows, so the
// heaviest go first.
__device__ __forceinline__ int prefill_query(int bid, int Q) {
  constexpr int kRun = 64;
  const int full = Q / (8 * kRun) * (8 * kRun);
  int q = bid;
  if (bid < full) {
    const int x = bid & 7, n = bid >> 3;
    q = ((n / kRun) * 8 + x) * kRun + n % kRun;
  }
  return Q - 1 - q;
}

template <bool FP4>
__global__ void __launch_bounds__(kPThreads) sparse_attn_prefill_kernel(PArgs a) {
  constexpr int kCopies = FP4 ? 17 : 16;  // copy instructions per wave and tile
  __shared__ __attribute__((aligned(1024))) unsigned char smem[FP4 ? kPLdsFp4 : kPLdsBf16];
  unsigned char* ring = smem;
  unsigned char* masks = smem + kPMaskOff;  // per slot: valid rows (u32), fp4 rows (u32)
  uint32_t* tset = reinterpret_cast<uint32_t*>(smem + kPTsetOff);  // tiles with a valid slot
  int* idx_lds = reinterpret_cast<int*>(smem + kPIdxOff);

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int g = lane >> 4;   // QK layout: 16-lane group
  const int c = lane & 15;   //            lane in the group
  const int hf = lane >> 5;  // PV layout: half of the wave
  const int ho = lane & 31;  //            output head of this lane (in the wave's 32)

  const int Q = (int)gridDim.x;
  const int qi = prefill_query((int)blockIdx.x, Q);
  const int b = qi / a.S;
  const int L = a.L;
  const int ntiles = (L + kPTile - 1) / kPTile;

  const unsigned char* win_b = a.win + (int64_t)b * a.win_bs;
  const unsigned char* comp_b = a.comp + (int64_t)b * a.comp_bs;
  const unsigned char* csc_b = FP4 ? a.csc + (int64_t)b * a.csc_bs : nullptr;
  const int* irow = a.idx + (int64_t)qi * L;
  const int win_n = (int)a.win_n;
  const void* win_u = uniform_ptr(win_b);
  const void* comp_u = uniform_ptr(comp_b);
  const void* zero_u = uniform_ptr(g_prefill_zero_row);
  const void* csc_u = FP4 ? uniform_ptr(csc_b) : zero_u;

  // ---- prologue: the index row into LDS (copies, -1 past L), then this wave's query heads and
  // the sink, so that the index row can be used while the rest is still in flight ----
  for (int i0 = 64 * wave; i0 < L; i0 += kPThreads) {
    if (i0 + lane < L) dma4_s(irow + i0, (uint32_t)lane * 4u, (DSA_LDS void*)(idx_lds + i0));
  }
  for (int i = L + tid; i < ntiles * kPTile; i += kPThreads) idx_lds[i] = -1;
  if (tid == 0) *tset = 0u;
  // B operand of QK: lane (g, c) holds dims 32s + 8g .. 32s + 8g + 7 of heads 32w + c
  // (qreg[0][s]) and 32w + 16 + c (qreg[1][s]).  Exactly 32 loads and one sink load,
  // unconditional (lanes of heads past H read head H-1: finite values whose results are never
  // stored), so that waiting for all but the last 33 vector memory operations waits for the index
  // row only.
  bf16x8 qreg[2][16];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    const int qh = min(32 * wave + 16 * hh + c, a.H - 1);
    const __bf16* qp = a.q + ((int64_t)qi * a.H + qh) * kPD + 8 * g;
#pragma unroll
    for (int s = 0; s < 16; ++s) qreg[hh][s] = *reinterpret_cast<const bf16x8*>(qp + 32 * s);
  }
  const float sink_raw = a.sink[min(32 * wave + ho, a.H - 1)];
  wait_vmcnt<33>();
  __syncthreads();
  // index -> slot code: byte offset from the window or compressed base (bit 0 set for the
  // latter), or 2 for an empty slot; row offsets fit 32 bits (checked at launch).  Each wave
  // converts 64 consecutive slots at a time and marks the tiles among them that hold a valid slot.
  for (int i0 = 64 * wave; i0 < ntiles * kPTile; i0 += kPThreads) {
    const int i = i0 + lane;
    const bool in = i < ntiles * kPTile;
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
    if (lane == 0 && bits) atomicOr(tset, bits << (i0 / kPTile));
  }
  __syncthreads();
  // The loop runs over the tiles that hold at least one valid slot, in order (a tile of -1 slots
  // adds nothing); position k of that list lives in ring slot k % 2.
  uint32_t pend = __builtin_amdgcn_readfirstlane(*tset);
  const int nt = __builtin_popcount(pend);

  // copies of this wave's 16 rows of position k, and the position's valid-row and fp4-row bits.
  // Every row is one wave instruction from a scalar base (slot codes: byte offset of the row from
  // its base, bit 0 = compressed row, bit 1 = empty slot, read from the zero row).  An fp4 row
  // (256 nibble bytes) is read by lanes l, l+16, l+32, l+48 alike, so nothing past it is read; the
  // copies land in the first 1024 bytes of its pitch, where the decode writes the bf16 row.  One
  // more instruction per tile fetches the 32 scale bytes of each of the 16 rows into the wave's
  // stage of the slot (from the zero row when the wave has no fp4 row in the tile).
  // The slot codes of the next position to copy (lane l: row 16*wave + l%16; fp4: lane l also
  // holds the code of row (l%32)/2, for the scale copy) are read one issue ahead.
  int nidx = pend ? idx_lds[__builtin_ctz(pend) * kPTile + 16 * wave + (lane & 15)] : 0;
  int nsc = (FP4 && pend) ? idx_lds[__builtin_ctz(pend) * kPTile + 16 * wave + ((lane & 31) >> 1)] : 0;
  auto issue = [&](int k) {
    pend &= pend - 1u;  // the tile being copied, whose codes are already in nidx (and nsc)
    const int myidx = nidx;
    const int slot = k & 1;
    const uint32_t vbits = (uint32_t)__builtin_amdgcn_ballot_w64(lane < 16 && !(myidx & 2));
    const uint32_t fbits = FP4 ? (uint32_t)__builtin_amdgcn_ballot_w64(lane < 16 && (myidx & 1)) : 0u;
    if (lane == 0) {
      *reinterpret_cast<uint16_t*>(masks + slot * 8 + 2 * wave) = (uint16_t)vbits;
      *reinterpret_cast<uint16_t*>(masks + slot * 8 + 4 + 2 * wave) = (uint16_t)fbits;
    }
    unsigned char* tb = ring + slot * kPTileB;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const uint32_t x = (uint32_t)__builtin_amdgcn_readlane(myidx, r);
      // lane l lands at physical chunk l, so it reads logical chunk l ^ swz (fp4: nibble piece l%16)
      uint32_t voff = ((uint32_t)lane ^ p_swz(16 * wave + r)) * 16u;
      if (FP4 && (x & 1u)) voff = (uint32_t)(lane & 15) * 16u;
      p_dma16(slot_base(x, win_u, comp_u, zero_u), voff + (x & ~15u), (DSA_LDS void*)(tb + p_row(16 * wave + r)));
    }
    if constexpr (FP4) {
      // lane l (mod 32): 16 of the 32 scale bytes of row (l mod 32)/2 (scale rows are 32 bytes for
      // 256-byte nibble rows, so a row's byte offset / 8 is its scale row's); other rows re-read
      // scale row 0
      const uint32_t sc = (uint32_t)nsc;
      const uint32_t soff = ((sc & 1u) ? ((sc & ~15u) >> 3) : 0u) + (uint32_t)(lane & 1) * 16u;
      p_dma16(fbits ? csc_u : zero_u, fbits ? soff : 0u,
              (DSA_LDS void*)(smem + kPStageOff + (slot * 2 + wave) * kPStage));
    }
    if (pend) {
      nidx = idx_lds[__builtin_ctz(pend) * kPTile + 16 * wave + (lane & 15)];
      if constexpr (FP4) nsc = idx_lds[__builtin_ctz(pend) * kPTile + 16 * wave + ((lane & 31) >> 1)];
    }
  };
  // fp4 rows of position k that this wave copied, decoded in place (it has waited for its own
  // copies; the next barrier publishes them): lane l writes elements 8l..8l+7 from nibble bytes
  // 4l..4l+3 and scale byte l/2; a row's reads all complete before its write (one wave, in order).
  // Eight rows go through the same instructions at a time (a row that is not fp4 writes to a dummy
  // area), so the reads of all eight are issued before the first conversion.
  auto decode = [&](int k) {
    if constexpr (FP4) {
      const int slot = k & 1;
      const uint32_t fb = __builtin_amdgcn_readfirstlane(*reinterpret_cast<const uint16_t*>(masks + slot * 8 + 4 + 2 * wave));
      if (fb != 0u) {
        unsigned char* dummy = smem + kPDummyOff;
        const unsigned char* stg = smem + kPStageOff + (slot * 2 + wave) * kPStage;
#pragma unroll
        for (int h8 = 0; h8 < 2; ++h8) {
          if (((fb >> (8 * h8)) & 0xFFu) == 0u) continue;
          unsigned char* tb = ring + slot * kPTileB + p_row(16 * wave + 8 * h8);
          uint32_t word[8], scb[8];
#pragma unroll
          for (int r = 0; r < 8; ++r) {
            word[r] = *reinterpret_cast<const uint32_t*>(tb + p_row(r) + 4 * lane);
            scb[r] = stg[32 * (8 * h8 + r) + (lane >> 1)];
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
            unsigned char* dst = ((fb >> (8 * h8 + r)) & 1u) ? tb + p_row(r) : dummy;
            *reinterpret_cast<u32x4*>(dst + 16 * (lane ^ p_swz(16 * wave + 8 * h8 + r))) = v;
          }
        }
      }
    }
  };

  // lane offsets of the operand reads (the swizzle moves chunks only within their 64-byte block,
  // so the block comes in as an immediate offset).  K operand: row c of a 16-row half, logical chunk
  // 4s + g.  Transposed V operand: 16-lane group G = lane/16 (hf = G/2), lane i = c: rows 8hf + i/4
  // (lo) and 8hf + 4 + i/4 (hi), logical byte 64d + 32(G%2) + 8(i%4), i.e. chunk 4d + x with
  // x = 2(G%2) + (i%4)/2.
  const uint32_t koff = (uint32_t)p_row(c) + 16u * ((uint32_t)g ^ p_swz(c));
  uint32_t voff[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int row = 8 * hf + 4 * h + (c >> 2);
    const uint32_t x = (uint32_t)(2 * (g & 1) + ((c & 3) >> 1));
    voff[h] = (uint32_t)p_row(row) + 16u * (x ^ p_swz(row)) + 8u * (uint32_t)(c & 1);
  }
  auto kread = [&](const unsigned char* tb, int rh, int s) {
    return *reinterpret_cast<const bf16x8*>(tb + koff + p_row(16 * rh) + 64 * s);
  };
  // V^T operand of k-step ks for dims 32d .. 32d+31: rows 16ks + 8hf .. 16ks + 8hf + 7
  auto vread = [&](const unsigned char* tb, int ks, int d) {
    const unsigned char* p = tb + p_row(16 * ks) + 64 * d;
    const bf16x4 lo = lds_read_tr16((const DSA_LDS __bf16*)(p + voff[0]));
    const bf16x4 hi = lds_read_tr16((const DSA_LDS __bf16*)(p + voff[1]));
    return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  };
  // swap between 16-lane groups 2j and 2j+1 of the wave: x's odd groups take y's even groups
  auto swap16 = [](uint32_t& x, uint32_t& y) {
    const auto r = __builtin_amdgcn_permlane16_swap(x, y, false, false);
    x = r[0];
    y = r[1];
  };
  auto max16 = [](float v) {  // max over lanes l and l^16
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  };
  auto max32 = [](float v) {  // max over lanes l and l^32
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  };

  f32x16 acc[16];
#pragma unroll
  for (int d = 0; d < 16; ++d) acc[d] = f32x16{};
  // running max and sum of heads c and 16 + c of the QK layout (each the same in the four lanes
  // of that head); the output head ho of this lane is the first when g is even, else the second
  float m_run[2] = {kPMinit, kPMinit};
  float l_run[2] = {0.f, 0.f};
  const bool o_hi = (g & 1) != 0;

  if (nt > 0) issue(0);
  if (nt > 1) issue(1);
  for (int k = 0; k < nt; ++k) {
    // this wave's copies of position k have landed (position 1's, issued in the prologue, may
    // still be out at k = 0); the barrier publishes every wave's rows and means every wave is
    // done with position k-1, whose slot is refilled below
    if (k == 0 && nt > 1)
      wait_vmcnt<kCopies>();
    else
      wait_vmcnt<0>();
    decode(k);
    __syncthreads();
    if (k >= 1 && k + 1 < nt) issue(k + 1);
    const int slot = k & 1;
    const uint32_t vm = *reinterpret_cast<const uint32_t*>(masks + slot * 8);
    const unsigned char* kp = ring + slot * kPTileB;
    const unsigned char* vp = kp;

    // ---- S^T = K . Q^T as four 16x16 blocks (row half rh, head half hh), one chain each, over
    // 16 k-steps of 32 dims; each K operand feeds both head halves ----
    f32x4 sacc[2][2];
    {
      bf16x8 kr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) kr[i] = kread(kp, i & 1, i >> 1);
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        const int rh = i & 1, s = i >> 1;
        if (s == 0) {
          sacc[rh][0] = qk_first(kr[i & 3], qreg[0][s]);
          sacc[rh][1] = qk_first(kr[i & 3], qreg[1][s]);
        } else {
          qk_next(sacc[rh][0], kr[i & 3], qreg[0][s]);
          qk_next(sacc[rh][1], kr[i & 3], qreg[1][s]);
        }
        if (i + 4 < 32) kr[i & 3] = kread(kp, (i + 4) & 1, (i + 4) >> 1);
      }
      asm("s_nop 15" : "+v"(sacc[0][0]), "+v"(sacc[0][1]), "+v"(sacc[1][0]), "+v"(sacc[1][1]));
    }
    // the first V operands, read while the softmax runs
    constexpr int kVPre = 4;
    bf16x8 vpre[kVPre];
#pragma unroll
    for (int d = 0; d < kVPre; ++d) vpre[d] = vread(vp, 0, d);
    // ---- online softmax: sacc[rh][hh][j] is row 16rh + 4g + j of head 16hh + c ----
    float mloc[2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      float mx = -__builtin_inff();
#pragma unroll
      for (int rh = 0; rh < 2; ++rh)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int row = 16 * rh + 4 * g + j;
          sacc[rh][hh][j] = (vm >> row) & 1u ? sacc[rh][hh][j] : -__builtin_inff();
          mx = fmaxf(mx, sacc[rh][hh][j]);
        }
      mloc[hh] = max32(max16(mx)) * a.scale_log2;  // scale > 0
    }
    // rare after the first tile: a tile raised some head's max by more than 8
    if (__builtin_amdgcn_ballot_w64(mloc[0] > m_run[0] + kPRescale || mloc[1] > m_run[1] + kPRescale) != 0ull) {
      float alpha[2];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const float m_new = fmaxf(m_run[hh], mloc[hh]);
        alpha[hh] = __builtin_amdgcn_exp2f(m_run[hh] - m_new);
        m_run[hh] = m_new;
        l_run[hh] *= alpha[hh];
      }
      if (k > 0) {  // the accumulators are still zero before the first tile
        const float ao = o_hi ? alpha[1] : alpha[0];
#pragma unroll
        for (int d = 0; d < 16; ++d) asm volatile("s_nop 15\n\ts_nop 3" : "+a"(acc[d]));
        // one accumulator at a time through VGPRs (the ordered empty statements keep the compiler
        // from moving all of them out of the AGPRs at once)
#pragma unroll
        for (int d = 0; d < 16; ++d) {
          f32x16 t = acc[d];
          asm volatile("" : "+v"(t));
          t *= ao;
          asm volatile("" : "+v"(t));
          acc[d] = t;
          asm volatile("s_nop 1" : "+a"(acc[d]));
        }
      }
    }
    // probabilities in bf16, two per register: xs[rh] = head c, ys[rh] = head 16 + c
    uint32_t xs[2][2], ys[2][2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      float lsum = 0.f;
#pragma unroll
      for (int rh = 0; rh < 2; ++rh) {
        float p[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          p[j] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[rh][hh][j], a.scale_log2, -m_run[hh]));
          lsum += p[j];
        }
        const uint32_t w0 = __builtin_bit_cast(uint32_t, bf16x2{(__bf16)p[0], (__bf16)p[1]});
        const uint32_t w1 = __builtin_bit_cast(uint32_t, bf16x2{(__bf16)p[2], (__bf16)p[3]});
        if (hh == 0) {
          xs[rh][0] = w0;
          xs[rh][1] = w1;
        } else {
          ys[rh][0] = w0;
          ys[rh][1] = w1;
        }
      }
      l_run[hh] += lsum;
    }
    // B operand of PV k-step ks (rows 16ks + 8hf .. +7 of head ho): an even group keeps its head-c
    // rows 16ks + 4g .. +3 and takes the odd group's (the next four rows); an odd group takes the
    // even group's head-(16+c) rows and keeps its own
    bf16x8 pb[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      swap16(xs[ks][0], ys[ks][0]);
      swap16(xs[ks][1], ys[ks][1]);
      const u32x4 w = {xs[ks][0], xs[ks][1], ys[ks][0], ys[ks][1]};
      pb[ks] = __builtin_bit_cast(bf16x8, w);
      asm("s_nop 1" : "+v"(pb[ks]));  // VALU writes above, MFMA reads below
    }

    // ---- O^T += V^T . P^T over the whole head_dim: 16 chains ----
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
      for (int d = 0; d < 16; ++d) {
        pv_mfma(acc[d], (ks == 0 && d < kVPre) ? vpre[d] : vread(vp, ks, d), pb[ks]);
      }
    }
  }
  wait_vmcnt<0>();
#pragma unroll
  for (int d = 0; d < 16; ++d) asm volatile("s_nop 15\n\ts_nop 3" : "+a"(acc[d]));

  // per-head sums over the four lanes of each head (identical in all of them)
  float l_tot[2];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    const auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(l_run[hh]), __float_as_uint(l_run[hh]), false, false);
    const float s16 = __uint_as_float(r16[0]) + __uint_as_float(r16[1]);
    const auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(s16), __float_as_uint(s16), false, false);
    l_tot[hh] = __uint_as_float(r32[0]) + __uint_as_float(r32[1]);
  }
  const int head = 32 * wave + ho;
  if (head >= a.H) return;
  const float mo = o_hi ? m_run[1] : m_run[0];
  const float lo_ = o_hi ? l_tot[1] : l_tot[0];
  const float sink2 = sink_raw * kPLog2e;
  const float mf = fmaxf(mo, sink2);
  const float f = exp2f(mo - mf);
  const float rn = f / (lo_ * f + exp2f(sink2 - mf));
  // lane (hf, ho) holds dims 32d + 8j + 4hf .. +3 of head ho (j = 0..3): two whole rotary pairs
  __bf16* op = a.o + ((int64_t)qi * a.H + head) * kPD + 4 * hf;
  const int rope0 = kPD - 2 * a.rope_P;  // first rotated dim (a multiple of 16), kPD without a table
  const float* rrow = a.rope ? a.rope + (int64_t)(qi % a.S) * a.rope_P * 2 : nullptr;
#pragma unroll
  for (int d = 0; d < 16; ++d) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int dim = 32 * d + 8 * j;  // + 4hf
      float v[4] = {acc[d][4 * j] * rn, acc[d][4 * j + 1] * rn, acc[d][4 * j + 2] * rn, acc[d][4 * j + 3] * rn};
      if (rrow && dim + 4 * hf >= rope0) {
        const float4 cs = *reinterpret_cast<const float4*>(rrow + (dim + 4 * hf - rope0));
        rope_rot_inv(v[0], v[1], cs.x, cs.y);
        rope_rot_inv(v[2], v[3], cs.z, cs.w);
      }
      const bf16x4 ov = {(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
      *reinterpret_cast<bf16x4*>(op + dim) = ov;
    }
  }
}

}  // namespace

// Launches the kernel when it applies (bf16 window rows, bf16 or fp4 compressed rows, head_dim 512,
// at most 64 heads, index rows of at most 1024 slots, enough queries to fill the GPU, 16-byte
// aligned rows and scale rows, row offsets within 32 bits, positive scale); returns 1 if
// launched, 0 if not, <0 on error.
int sparse_attn_prefill_launch(const void* q, const dsa_kv_src* win, const dsa_kv_src* comp, const float* sink,
                               const int32_t* idx, int L, float scale, void* o, int B, int S, int H, int D,
                               const float* rope, int rope_dim, hipStream_t st) {
  const int Q = B * S;
  if (D != kPD || H > 64 || L > kPMaxSlots || Q < 256) return 0;
  const bool fp4 = comp && comp->rows && comp->format == DSA_KV_FP4_E4M3_G16;
  PArgs a{};
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
  // slot codes hold row byte offsets in 32 bits; the softmax folds a positive scale into exp2
  if (!(scale > 0.f) || (uint64_t)a.win_n * (uint64_t)a.win_rs >= (1ull << 31)) return 0;
  if (a.comp && (uint64_t)comp->n_rows * (uint64_t)a.comp_rs >= (1ull << 31)) return 0;
  // fp4 rows: 256 nibble bytes and 32 scale bytes per row, densely strided (a row's byte offset
  // / 8 is then its scale row's)
  if (fp4 && (a.comp_rs != kPD / 2 || a.csc_rs != kPD / 16)) return 0;
  a.sink = sink;
  a.idx = idx;
  a.L = L;
  a.scale_log2 = scale * kPLog2e;
  a.o = (__bf16*)o;
  a.S = S;
  a.H = H;
  a.rope = rope;
  a.rope_P = rope ? rope_dim / 2 : 0;
  if (fp4)
    hipLaunchKernelGGL(sparse_attn_prefill_kernel<true>, dim3(Q), dim3(kPThreads), 0, st, a);
  else
    hipLaunchKernelGGL(sparse_attn_prefill_kernel<false>, dim3(Q), dim3(kPThreads), 0, st, a);
  const int rc = check_launch("sparse_attn_prefill");
  return rc ? rc : 1;
}

}  // namespace dsa
