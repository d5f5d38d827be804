// Internal definitions shared by the HIP sources of libdsa (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/dsa.h"

namespace dsa {

// ---- vector types used as MFMA operands -----------------------------------
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

#define DSA_LDS __attribute__((address_space(3)))

// 32x32x16 bf16 MFMA.  Lane l (hf = l/32, c = l%32) supplies A[c][8hf..8hf+7] and
// B[8hf..8hf+7][c]; accumulator element j holds C[8(j/4) + 4hf + (j%4)][c].
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// LDS transposing read of four 16-bit elements.  Within each 16-lane group,
// lane c receives column c of a 4x16 block whose row r is the four elements at
// the addresses of lanes 4r .. 4r+3 of that group.
__device__ __forceinline__ bf16x4 lds_read_tr16(const DSA_LDS __bf16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((DSA_LDS bf16x4*)p);
}

// 16-byte global -> LDS copy without passing through registers.  The LDS
// destination is wave-uniform: lane l's 16 bytes land at lds_base + 16*l.
__device__ __forceinline__ void global_to_lds16(const void* gptr, DSA_LDS void* lds_base) {
  __builtin_amdgcn_global_load_lds(gptr, lds_base, 16, 0, 0);
}

// ---- global -> LDS copies tracked by the kernel itself ---------------------------------------
// The same 16-byte (4-byte) copies as global_to_lds16, written as inline asm so the compiler does
// not track them: it would otherwise wait for every outstanding copy before each LDS access.  A
// kernel using them waits with wait_vmcnt, counting its own copies (each is one vector memory
// instruction per wave).  The s_nop gives the one wait state a copy needs after the M0 write that
// sets its LDS base.  _s forms take the row base in scalar registers and a per-lane 32-bit offset.

// A wave-uniform pointer, placed in scalar registers.  The registers are written by a VALU
// instruction (v_readfirstlane): a vector memory instruction that takes them as its scalar address
// must come at least 5 wait states later, and the compiler does not count wait states for an
// address consumed inside inline asm.  The _s copy helpers below therefore take bases formed by
// scalar instructions (or computed well before), except dma4_s, which waits itself.
__device__ __forceinline__ const void* uniform_ptr(const void* p) {
  const uint64_t v = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const void*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ void dma16_s(const void* sbase, uint32_t voff, const DSA_LDS void* lds_base) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase),
               "{m0}"((uint32_t)(uintptr_t)lds_base)
               : "memory");
}
// (the base comes straight from v_readfirstlane: s_nop 4 gives the 5 wait states before the
// copy reads it, which also cover the one the M0 write needs)
__device__ __forceinline__ void dma4_s(const void* sbase, uint32_t voff, const DSA_LDS void* lds_base) {
  sbase = uniform_ptr(sbase);
  asm volatile("s_nop 4\n\tglobal_load_lds_dword %0, %1" ::"v"(voff), "s"(sbase), "{m0}"((uint32_t)(uintptr_t)lds_base)
               : "memory");
}
__device__ __forceinline__ void dma16_v(const void* gptr, const DSA_LDS void* lds_base) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gptr), "{m0}"((uint32_t)(uintptr_t)lds_base)
               : "memory");
}
// Base of a gathered row from its slot code (the row's byte offset from its base, with bit 1 set
// for an empty slot, read from a zero row, and bit 0 set for a compressed row; else a window row).  Written as scalar selects: as C++ the compiler turns the choice into a table in
// private memory.
__device__ __forceinline__ const void* slot_base(uint32_t code, const void* win, const void* comp, const void* zero) {
  const void* r;
  asm("s_bitcmp1_b32 %1, 0\n\ts_cselect_b64 %0, %3, %2\n\ts_bitcmp1_b32 %1, 1\n\ts_cselect_b64 %0, %4, %0"
      : "=&s"(r)
      : "s"(code), "s"(win), "s"(comp), "s"(zero)
      : "scc");
  return r;
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  // gfx9 s_waitcnt: vmcnt in bits 3:0 and 15:14; expcnt (6:4) and lgkmcnt (11:8) left at "no wait"
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// XOR pattern applied to the 16-byte chunks of LDS row r (rows of NCH chunks).  Bijective on
// 0..15, so 16 consecutive rows read at one logical chunk hit 16 different bank groups, and the
// 4-row x 32-byte blocks of a transposing read spread over all bank groups two at a time.
template <int NCH>
__device__ __forceinline__ int row_swz(int r) {
  const int s = ((r & 3) << 2) | ((r >> 2) & 3);
  return NCH >= 16 ? s : (s & (NCH - 1));
}

__device__ __forceinline__ float bf16_to_f32(__bf16 x) { return (float)x; }

__device__ __forceinline__ int lane_id() { return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0)); }

template <typename T>
__device__ __forceinline__ T shfl_xor(T v, int mask) {
  return __shfl_xor(v, mask, 64);
}

// Index rows selected inside the decode attention kernel: the queries' scores [Q][T], top-k size
// K, visibility (start_pos, ratio), window W with Wc columns and the top-k offset; idx_out (may
// be null) receives the rows, ld_out apart.
struct DecSelect {
  const float* scores;
  int T, K, start_pos, ratio, W, Wc, offset;
  int32_t* idx_out;
  int64_t ld_out;
};

// Index scores computed by the decode attention kernel itself (with a DecSelect): index queries
// q_idx [Q][H_I][128], keys k_idx [B][T][128] (batch stride k_bstride elements), head weights
// w [Q][H_I], all bf16; the scores go to scores_out [Q][T] (the DecSelect's scores), where the
// query's workgroups exchange them.
struct DecIndex {
  const __bf16* q_idx;
  const __bf16* k_idx;
  int64_t k_bstride;
  const __bf16* w;
  float w_scale;
  int H_I;
  float* scores_out;
};

// Inverse rotary embedding of the output pair (x, y) by (c, s) (`Attention.forward` rotates o's
// last rope_head_dim dims back after the attention): (x + iy)(c - is).
__device__ __forceinline__ void rope_rot_inv(float& x, float& y, float c, float s) {
  const float nx = x * c + y * s;
  const float ny = y * c - x * s;
  x = nx;
  y = ny;
}

__device__ __forceinline__ int visible_rows(int start_pos, int t, int ratio) {
  return (start_pos + t + 1) / ratio;
}

// Candidate blocks of the two-level selection as the scoring kernels read them: bit i of word
// i/32 of query row r (words ld apart) is set when block i of 2^lbs compressed positions is a
// candidate.  bits == nullptr: every position is a candidate.
struct CandMask {
  const uint32_t* bits;
  int64_t ld;
  int lbs;
};

__device__ __forceinline__ bool cand_ok(const CandMask& m, int64_t row, int j) {
  if (m.bits == nullptr) return true;
  const int blk = j >> m.lbs;
  return ((m.bits[row * m.ld + (blk >> 5)] >> (blk & 31)) & 1u) != 0u;
}

}  // namespace dsa

namespace dsa {
// ---- workspace header ------------------------------------------------------------------------
// Every workspace starts with a header of per-query rendezvous counters (4 words per query, for up
// to kWsSyncQueries queries) that only the decode kernels touch; they leave it zero when they end,
// so it only has to be zero before a workspace's first use.  All other scratch follows it.
constexpr int kWsSyncQueries = 256;
constexpr size_t kWsHeaderBytes = (size_t)kWsSyncQueries * 16;

// ---- host side: error reporting, launch record, per-device set-up (abi.cpp) ------------------
struct DeviceState {
  int ready;          // dsa_init has run on this device
  int xcd_rr;         // workgroup i runs on XCD i mod 8 (the decode kernels' rendezvous needs it)
  int resident[6];    // decode kernel variants: workgroups resident at once
  void* scratch;      // device address of the allocation-free entry point's scratch array
};

int fail(int code, const char* fmt, ...);
// After a launch: DSA_ERR_HIP if the runtime reports an error, else records `what` as launched.
int check_launch(const char* what);
// The current device's state, set up (dsa_init) if it is not yet; DSA_ERR_STATE when that would
// have to happen under stream capture.
int ensure_device_init(hipStream_t st, DeviceState** out);
int decode_device_init(int dev, DeviceState& ds);
int decode_read_errors(uint32_t* bits);
}  // namespace dsa
