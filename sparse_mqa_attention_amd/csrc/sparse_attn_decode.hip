// Sparse MQA attention for decode batches (DeepSeek V4.1 page, `sparse_attn_kernel`; one query
// per sequence attending its window ring plus its top-k compressed rows, with a per-head sink).
//
// A decode batch has far fewer queries than the GPU has CUs, so each query's work is spread over
// NS workgroups, and the split is arranged so that no workgroup ever writes a partial output:
//
//  phase A (rows)  workgroup s of query q gathers rows [s*RPS, (s+1)*RPS) of the index row into
//                  LDS (direct 16-byte global->LDS loads, all rows in flight at once), computes
//                  the logits of all 64 heads on MFMA (S^T = K . Q^T), and publishes the
//                  probabilities P = 2^(l - m_s) in bf16 plus its per-head max m_s and sum l_s.
//  rendezvous      the NS workgroups of the query count themselves in on an arrival counter (in
//                  the caller's workspace, so calls on different workspaces never meet); the host
//                  only takes this path when every workgroup of the grid is resident at once, and
//                  the wait is bounded (a timeout raises a sticky error flag and poisons the output).
//                  All NS workgroups of a query run on one XCD, so P and the stats travel through
//                  the L2 they share, with no cache-wide write-back or invalidate (those cost tens
//                  of microseconds).
//  phase B (dims)  workgroup s computes output columns [s*D/NS, (s+1)*D/NS) of all 64 heads over
//                  ALL rows of the query: it re-gathers just those columns of every row (hits in
//                  the XCD's L2, which phase A of the sibling workgroups filled) and reads P from
//                  L2; O^T = V^T . P^T on MFMA, one accumulator per phase-A split scaled by
//                  2^(m_s - M) before it is added, then divided by sum_s l_s 2^(m_s - M) + 2^(sink - M).
//
// Blocks are numbered so that all NS workgroups of a query land on one XCD (dispatch assigns
// consecutive workgroups to the 8 XCDs round-robin, which the library checks once per device; the
// grid is padded to a multiple of 8 queries), keeping the rendezvous and the re-gather in one L2.
// What crosses HBM is each valid row once, q, o, and the small P (Q x 64 x L bf16).
//
// Stale lines in a CU's L1: a workgroup reads its siblings' P and stats only after the rendezvous,
// and P rows ([Q][64][Lp] bf16, Lp a multiple of 16*NS) and stats ([Q][NS][64][2] fp32) of
// different queries never share a 128-byte line, so no CU can hold an early copy of a line it
// reads there.  Scores rows ([Q][T] fp32) do share lines between neighbouring queries, so the
// exchanged scores are written and read at device scope (past the L1).
#include "index_tile.h"
#include "topk_block.h"

namespace dsa {

namespace {

constexpr int kDD = 512;                 // head_dim of this path
constexpr int kDH = 64;                  // heads of this path
constexpr int kDecRowsMax = 96;          // rows of one phase-A split: 96 KiB of LDS
constexpr int kDecQueriesMax = kWsSyncQueries - 1;  // padded to a multiple of 8, the grid's queries
                                                    // still fit the workspace header
constexpr float kLog2eD = 1.4426950408889634f;
constexpr uint64_t kSpinTimeoutTicks = 20000000ull;  // 0.2 s of the 100 MHz constant-rate counter

// Sticky error bits of the decode kernels (bit 0: a rendezvous timed out and that query's output
// was set to NaN); read and cleared by dsa_device_errors.
__device__ uint32_t g_dec_error;

struct DecArgs {
  const __bf16* q;
  const unsigned char* win;
  int64_t win_n, win_bs, win_rs;  // bytes
  const unsigned char* comp;
  int64_t comp_bs, comp_rs;       // bytes
  const float* sink;
  const int32_t* idx;
  int L;
  float scale_log2;
  __bf16* o;
  __bf16* pbuf;    // [Q][64][Lp] phase-A probabilities
  float* stats;    // [Q][NS][64][2] phase-A (max, sum)
  uint32_t* sync;  // [Qp][4] per query: score-exchange arrivals, rendezvous arrivals, departures
  int S, Q, Qp, RPS, Lp;
  const float* rope;  // inverse rotary table of the output [S][rope_P][2] (cos, sin), or null
  int rope_P;
  // index rows selected in the kernel (instead of read from idx): the query's scores [T], the
  // top-k size K, visibility (start_pos, ratio), window W with Wc columns, top-k offset; s == 0
  // writes the row to idx_out when that is set
  const float* scores;
  int T, K, start_pos, ratio, W, Wc, offset;
  int32_t* idx_out;
  int64_t ld_out;
  // index scores computed in the kernel (see DecIndex): scores then points at scores_out
  const __bf16* q_idx;
  const __bf16* k_idx;
  int64_t k_bstride;
  const __bf16* w_idx;
  float w_scale;
  int H_I;
};

template <int NS>
struct DecCfg {
  static constexpr int DS = kDD / NS;      // output columns per workgroup in phase B
  static constexpr int SLICEB = DS * 2;    // bytes of one row's column slice
  static constexpr int LPRB = SLICEB / 16; // lanes per slice (8 or 4)
  static constexpr int RPIB = 64 / LPRB;   // slices per wave instruction (8 or 16)
  static constexpr int NMB = DS / 32;      // phase-B M tiles per wave
  static constexpr int ROWS_BYTES = kDecRowsMax * kDD * 2;
  static constexpr int MAX_L = ROWS_BYTES / SLICEB;  // slots whose slices fit the same LDS
  static constexpr int NSW = NS / 2;       // phase-A splits each phase-B wave folds in
  static constexpr int KPS = NS == 8 ? 6 : 3;  // most 16-row k-steps per split (RPS <= 16*KPS)
  static constexpr int TA = (16 * KPS + 31) / 32;  // 32-row MFMA tiles covering one split
};

// chunk XOR of phase-B slice rows: keeps the 4-row x 32-byte transposing reads conflict free
template <int NS>
__device__ __forceinline__ int slice_swz(int r) {
  return NS == 8 ? (((r >> 1) & 3) << 1) : 0;
}

// The arrival counter is polled with a device-scope load: on gfx950 only that scope skips the
// CU's L1, so a narrower poll could spin on a stale line.
__device__ __forceinline__ uint32_t poll_load(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Source of the copies for -1 slots (and rows past the index row): a zero row, so every row of a
// gather costs one copy and no branch.
__device__ __attribute__((aligned(1024))) unsigned char g_dec_zero_row[kDD * 2];

// Slot code: the row's byte offset from its base, bit 0 = compressed row, bit 1 = empty slot.
__device__ __forceinline__ uint32_t dec_slot_code(int iv, int win_n, uint32_t win_rs, uint32_t comp_rs) {
  return iv < 0 ? 2u : iv < win_n ? (uint32_t)iv * win_rs : ((uint32_t)(iv - win_n) * comp_rs) | 1u;
}

// Row base of a slot code, per lane (vector selects).
__device__ __forceinline__ const unsigned char* dec_lane_base(uint32_t code, const unsigned char* win,
                                                             const unsigned char* comp, const unsigned char* zero) {
  const unsigned char* b = (code & 1u) ? comp : win;
  return (code & 2u) ? zero : b;
}

__device__ __forceinline__ uint32_t xcc_id() {
  uint32_t v;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(v));
  return v & 0xFu;
}

// SKPT = 0: the index rows come from idx; SKPT > 0: each workgroup selects its query's index row
// from the scores (window part, then the top-k part, exactly as the top-k kernels do), SKPT scores
// per thread.  IX = 1 (with SKPT > 0): the query's workgroups first compute those scores, each
// for its share of the compressed rows, and exchange them through the scores buffer.
template <int NS, int SKPT, int IX>
__global__ void __launch_bounds__(256) sparse_attn_decode_kernel(DecArgs a) {
  using C = DecCfg<NS>;
  constexpr int XBUF_FLOATS = 4 * C::TA * 16 * 64;  // per wave, per tile: one partial S^T tile
  __shared__ __attribute__((aligned(1024))) unsigned char rows[C::ROWS_BYTES];
  __shared__ __attribute__((aligned(16))) float xbuf[XBUF_FLOATS];
  __shared__ int idx_lds[C::MAX_L];
  __shared__ float stats_lds[NS * kDH * 2];
  __shared__ int flags[1];  // the rendezvous timed out
  // the in-kernel top-k works in the row buffer, which phase A fills only after it
  static_assert(sizeof(topk_dev::TopkSmem<256>) <= C::ROWS_BYTES, "top-k scratch fits the row buffer");
  topk_dev::TopkSmem<256>& tsm = *reinterpret_cast<topk_dev::TopkSmem<256>*>(rows);

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int hf = lane >> 5;
  const int c = lane & 31;
  const int j16 = lane & 15;

  // workgroup lb runs on XCD lb % 8; the Qp/8 queries of an XCD take its workgroups NS at a time
  // (Qp = Q rounded up to a multiple of 8; the padding queries' workgroups leave at once)
  int q, s;
  {
    const int lb = blockIdx.x;
    const int xcd = lb & 7, k = lb >> 3;
    q = xcd * (a.Qp >> 3) + k / NS;
    s = k % NS;
  }
  if (q >= a.Q) return;
  uint32_t* const qsync = a.sync + 4 * q;
  const int L = a.L;
  const int bq = q / a.S;  // batch of the query's KV
  const int32_t* irow = a.idx + (int64_t)q * L;
  const unsigned char* win_b = a.win + (int64_t)bq * a.win_bs;
  const unsigned char* comp_b = a.comp + (int64_t)bq * a.comp_bs;

  // =============================== phase A: logits of rows [a0, a0 + nr) for all heads
  // wave (hg, dh): heads 32*hg .. +31 over head_dim half dh; partial logits are summed in LDS
  const int a0 = s * a.RPS;
  const int nr = max(0, min(L, a0 + a.RPS) - a0);
  const int hg = wave & 1, dh = wave >> 1;
  const int head = 32 * hg + c;
  // the whole index row, once: phase A gathers its part, phase B every slot
  const int win_n = (int)a.win_n;
  bf16x8 qreg[kDD / 32];
  if constexpr (SKPT == 0) {
    int iv_reg[C::MAX_L / 256];
#pragma unroll
    for (int k = 0; k < C::MAX_L / 256; ++k) {
      const int i = tid + 256 * k;
      iv_reg[k] = (int)dec_slot_code(i < L ? irow[i] : -1, win_n, (uint32_t)a.win_rs, (uint32_t)a.comp_rs);
    }
    {
      const __bf16* qp = a.q + ((int64_t)q * kDH + head) * kDD + (kDD / 2) * dh + hf * 8;
#pragma unroll
      for (int k = 0; k < kDD / 32; ++k) qreg[k] = *reinterpret_cast<const bf16x8*>(qp + 16 * k);
    }
#pragma unroll
    for (int k = 0; k < C::MAX_L / 256; ++k)
      if (tid + 256 * k < L) idx_lds[tid + 256 * k] = iv_reg[k];
    __syncthreads();
  } else {
    const int t = q % a.S;
    const int cvis = min(a.T, visible_rows(a.start_pos, t, a.ratio));
    const __bf16* qp = a.q + ((int64_t)q * kDH + head) * kDD + (kDD / 2) * dh + hf * 8;
    if constexpr (IX == 0) {  // the attention's query, in flight while the rows are selected
#pragma unroll
      for (int k = 0; k < kDD / 32; ++k) qreg[k] = *reinterpret_cast<const bf16x8*>(qp + 16 * k);
    }
    if constexpr (IX != 0) {
      // ============================= index scores of compressed rows [j0, j1) of this query, with
      // the index kernel's tile arithmetic; the query's workgroups exchange them through the
      // scores buffer, in the L2 of the XCD they share
      constexpr int DI = 128;
      constexpr int NCH = DI / 8;
      constexpr int KS = DI / 16;
      const int hp = a.H_I > 32 ? 64 : 32;  // heads padded to whole MFMA tiles
      const int tps = ((a.T + NS - 1) / NS + 31) & ~31;  // rows per workgroup, whole 32-row tiles
      const int j0 = s * tps;
      const int j1 = min(a.T, j0 + tps);
      const int jw = j0 + 64 * wave;  // this wave's two tiles
      const __bf16* kb = a.k_idx + (int64_t)bq * a.k_bstride;
      // the keys first, then the index queries straight into LDS, so both are in flight at once
      bf16x8 kreg[2][KS];
#pragma unroll
      for (int n = 0; n < 2; ++n) {
        const int j = jw + 32 * n + c;
        const bool live = jw + 32 * n < min(j1, cvis) && j < j1;
#pragma unroll
        for (int k = 0; k < KS; ++k)
          kreg[n][k] = live ? *reinterpret_cast<const bf16x8*>(kb + (int64_t)j * DI + hf * 8 + 16 * k) : bf16x8{};
      }
      // wave w copies LDS rows 4i .. 4i+3 for i = w, w+4, ...: lane l the 16 bytes that belong at
      // physical chunk l%16 of row 4i + l/16 (the zero row past the real heads)
      __bf16* qi_lds = reinterpret_cast<__bf16*>(rows);
      float* wi_lds = reinterpret_cast<float*>(rows + 64 * DI * 2);
      for (int i = wave; i < hp / 4; i += 4) {
        const int h = 4 * i + (lane >> 4);
        const int ch = qswz<NCH>(h, lane & 15);
        const void* src = h < a.H_I ? (const void*)(a.q_idx + ((int64_t)q * a.H_I + h) * DI + ch * 8)
                                    : (const void*)(g_dec_zero_row + ch * 16);
        dma16_v(src, (DSA_LDS void*)(rows + i * 4 * DI * 2));
      }
      if (tid < hp) wi_lds[tid] = tid < a.H_I ? bf16_to_f32(a.w_idx[(int64_t)q * a.H_I + tid]) : 0.f;
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      float* srow = const_cast<float*>(a.scores) + (int64_t)q * a.T;
#pragma unroll
      for (int n = 0; n < 2; ++n) {
        const int jt = jw + 32 * n;
        const int j = jt + c;
        if (jt < j1) {
          float v = -__builtin_inff();
          if (jt < cvis) {  // a tile wholly past the visible rows is not multiplied
            const float sum = hp == 32 ? index_tile_sum<DI, 1>(qi_lds, wi_lds, kreg[n], hf, c)
                                       : index_tile_sum<DI, 2>(qi_lds, wi_lds, kreg[n], hf, c);
            if (j < cvis) v = a.w_scale * sum;
          }
          // written at device scope: the row may share lines with a neighbouring query's row
          if (hf == 0 && j < j1) __hip_atomic_store(&srow[j], v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
      // every score of this workgroup has reached L2 before it counts itself in
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();  // also: the staged index queries are read no more
      // the attention's query, in flight during the exchange and the selection
#pragma unroll
      for (int k = 0; k < kDD / 32; ++k) qreg[k] = *reinterpret_cast<const bf16x8*>(qp + 16 * k);
      if (tid == 0) {
        uint32_t* arrive_ix = &qsync[0];
        __hip_atomic_fetch_add(arrive_ix, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const uint64_t t0 = wall_clock64();
        int to = 0;
        for (uint32_t it = 1; poll_load(arrive_ix) < (uint32_t)NS; ++it) {
          if ((it & 15u) == 0u && wall_clock64() - t0 > kSpinTimeoutTicks) {
            to = 1;
            atomicOr(&g_dec_error, 1u);
            break;
          }
        }
        flags[0] = to;
      }
      __syncthreads();
    }
    // this query's index row from its scores: Wc window entries, then the K top-k entries
    for (int i = tid; i < a.Wc; i += 256) idx_lds[i] = topk_dev::window_entry(t, i, a.start_pos, a.W);
    if (cvis <= a.K) {  // every visible position is kept
      for (int i = tid; i < a.K; i += 256) idx_lds[a.Wc + i] = i < cvis ? i + a.offset : -1;
    } else {
      int* top = idx_lds + a.Wc;
      // scores the siblings wrote in this launch are read at device scope (past the L1)
      topk_dev::block_topk<256, SKPT, IX != 0>(a.scores + (int64_t)q * a.T, a.T, cvis, a.K, a.offset, tsm,
                                               [&](int slot, int v) { top[slot] = v; });
    }
    __syncthreads();
    // the row as selected (one workgroup of the query), then its slot codes in place (each entry
    // by the thread that wrote it out)
    const bool wr = a.idx_out != nullptr && s == 0;
    for (int i = tid; i < L; i += 256) {
      const int iv = idx_lds[i];
      if (wr) a.idx_out[(int64_t)q * a.ld_out + i] = iv;
      idx_lds[i] = (int)dec_slot_code(iv, win_n, (uint32_t)a.win_rs, (uint32_t)a.comp_rs);
    }
    __syncthreads();
  }
  // valid rows of this split as two 64-bit masks (rows 0..63, 64..95 of the split)
  const uint64_t vm0 = __builtin_amdgcn_ballot_w64(lane < nr && !(idx_lds[a0 + lane] & 2));
  const uint64_t vm1 = __builtin_amdgcn_ballot_w64(64 + lane < nr && !(idx_lds[a0 + 64 + lane] & 2));
  {
    // rows wave, wave+4, ...: this wave's codes in lanes 0..(TA*8-1), one copy per row from the row's
    // scalar base (a row past the split copies the zero row)
    const void* win_u = uniform_ptr(win_b);
    const void* comp_u = uniform_ptr(comp_b);
    const void* zero_u = uniform_ptr(g_dec_zero_row);
    const int rl = wave + 4 * lane;
    const int mycode = rl < nr ? idx_lds[a0 + rl] : 2;
#pragma unroll
    for (int k = 0; k < C::TA * 8; ++k) {
      const int r = wave + 4 * k;
      const uint32_t x = (uint32_t)__builtin_amdgcn_readlane(mycode, k);
      const int lch = lane ^ row_swz<64>(r);
      dma16_s(slot_base(x, win_u, comp_u, zero_u), (uint32_t)lch * 16u + (x & ~15u),
              (DSA_LDS void*)(rows + r * (kDD * 2)));
    }
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  float* xmine = xbuf + wave * (C::TA * 16 * 64);
  const float* xpart = xbuf + (wave ^ 2) * (C::TA * 16 * 64);
  f32x16 sacc[C::TA];
  {
    // one MFMA chain per tile, interleaved; rows past the split are masked below
    const int sw = row_swz<64>(c);
    const int ch0 = (kDD / 16) * dh + hf;  // logical chunk of k-step 0 in this half of D
#pragma unroll
    for (int ti = 0; ti < C::TA; ++ti) sacc[ti] = f32x16{};
#pragma unroll
    for (int k = 0; k < kDD / 32; ++k) {
#pragma unroll
      for (int ti = 0; ti < C::TA; ++ti) {
        const bf16x8 kf =
            *reinterpret_cast<const bf16x8*>(rows + (ti * 32 + c) * (kDD * 2) + (((ch0 + 2 * k) ^ sw) << 4));
        sacc[ti] = mfma32(kf, qreg[k], sacc[ti]);
      }
    }
#pragma unroll
    for (int ti = 0; ti < C::TA; ++ti)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const f32x4 v = {sacc[ti][4 * g4], sacc[ti][4 * g4 + 1], sacc[ti][4 * g4 + 2], sacc[ti][4 * g4 + 3]};
        *reinterpret_cast<f32x4*>(xmine + ((ti * 4 + g4) * 64 + lane) * 4) = v;
      }
  }
  __syncthreads();
  float sv[C::TA][16];
  float mloc = -__builtin_inff();
#pragma unroll
  for (int ti = 0; ti < C::TA; ++ti) {
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const f32x4 o4 = *reinterpret_cast<const f32x4*>(xpart + ((ti * 4 + g4) * 64 + lane) * 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int e = 4 * g4 + i;
        const int row = ti * 32 + 8 * g4 + 4 * hf + i;
        const float full = dh == 0 ? sacc[ti][e] + o4[i] : o4[i] + sacc[ti][e];  // same sum in both halves
        const bool ok = ((row < 64 ? (vm0 >> row) : (vm1 >> (row - 64))) & 1ull) != 0ull;
        sv[ti][e] = ok ? full * a.scale_log2 : -__builtin_inff();
        mloc = fmaxf(mloc, sv[ti][e]);
      }
    }
  }
  mloc = fmaxf(mloc, shfl_xor(mloc, 32));  // max over the split's rows for this lane's head
  const float mref = mloc == -__builtin_inff() ? 0.f : mloc;
  float lsum = 0.f;
  __bf16* prow = a.pbuf + ((int64_t)q * kDH + head) * a.Lp + a0;
#pragma unroll
  for (int ti = 0; ti < C::TA; ++ti) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int rb = ti * 32 + 8 * g + 4 * hf;
      float p[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[i] = __builtin_amdgcn_exp2f(sv[ti][4 * g + i] - mref);
        lsum += rb < a.RPS ? p[i] : 0.f;
      }
      // each half of the pair writes half of the rows; rows past nr carry P = 0
      if (rb < a.RPS && (g >> 1) == dh) {
        const bf16x4 pv = {(__bf16)p[0], (__bf16)p[1], (__bf16)p[2], (__bf16)p[3]};
        *reinterpret_cast<bf16x4*>(prow + rb) = pv;
      }
    }
  }
  lsum += shfl_xor(lsum, 32);
  if (dh == 0 && hf == 0) {
    float* st = a.stats + (((int64_t)q * NS + s) * kDH + head) * 2;
    st[0] = mloc;
    st[1] = lsum;
  }

  // =============================== arrival at the query's rendezvous
  // P and the stats are in the L2 the query's workgroups share once each wave's stores have
  // completed (the wait below, before the barrier), so they are visible to every reader once the
  // count reaches NS.  No cache-wide write-back or invalidate.  Nothing else is in flight here.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();  // also: every wave is done with phase A's rows
  uint32_t* arrive = &qsync[1];
  uint32_t* depart = &qsync[2];
  if (tid == 0) __hip_atomic_fetch_add(arrive, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

  // =============================== phase B gather, independent of the other workgroups
  // Columns [d0, d0 + DS) of every row of the query go into the LDS the split's rows used,
  // issued before the wait for the siblings so its latency hides in it.
  const int d0 = s * C::DS;
  const int Lk = (L + 15) & ~15;  // rows the MFMA k-steps touch
  {
    // one copy per group of RPIB slices; each lane picks its row's base (the zero row past L)
    const int ngrp = Lk / C::RPIB;
    const unsigned char* win_d = win_b + d0 * 2;
    const unsigned char* comp_d = comp_b + d0 * 2;
#pragma unroll 4
    for (int g = wave; g < ngrp; g += 4) {
      const int r = g * C::RPIB + lane / C::LPRB;
      const int p = lane % C::LPRB;
      const int lch = p ^ slice_swz<NS>(r);
      const uint32_t x = r < L ? (uint32_t)idx_lds[r] : 2u;
      const unsigned char* src = (x & 2u) ? g_dec_zero_row + lch * 16
                                          : dec_lane_base(x, win_d, comp_d, g_dec_zero_row) + (x & ~15u) + lch * 16;
      dma16_v(src, (DSA_LDS void*)(rows + g * C::RPIB * C::SLICEB));
    }
  }

  // =============================== wait for the query's NS workgroups (bounded)
  if (tid == 0) {
    const uint64_t t0 = wall_clock64();
    int to = 0;
    for (uint32_t it = 1; poll_load(arrive) < (uint32_t)NS; ++it) {
      if ((it & 15u) == 0u && wall_clock64() - t0 > kSpinTimeoutTicks) {
        to = 1;
        atomicOr(&g_dec_error, 1u);
        break;
      }
    }
    flags[0] = IX != 0 ? (flags[0] | to) : to;
  }
  __builtin_amdgcn_s_waitcnt(0);  // the slices have landed
  __syncthreads();

  // =============================== phase B: columns [d0, d0 + DS) of every head over all rows
  const int hb = wave & 1, kh = wave >> 1;
  const int headB = 32 * hb + c;
  // this wave's P operands (B of O^T = V^T . P^T): every k-step of its splits, loaded at once
  const __bf16* pcol = a.pbuf + ((int64_t)q * kDH + headB) * a.Lp + 8 * hf;
  bf16x8 pre[C::NSW][C::KPS];
#pragma unroll
  for (int tl = 0; tl < C::NSW; ++tl)
#pragma unroll
    for (int k = 0; k < C::KPS; ++k) {
      const int r0 = (kh + 2 * tl) * a.RPS + 16 * k;
      const bool ok = 16 * k < a.RPS && r0 < Lk;
      pre[tl][k] = !ok ? bf16x8{} : *reinterpret_cast<const bf16x8*>(pcol + r0);
    }
  for (int i = tid; i < NS * kDH * 2; i += 256)
    stats_lds[i] = a.stats[(int64_t)q * NS * kDH * 2 + i];
  __syncthreads();
  const float sink2 = a.sink[headB] * kLog2eD;
  float M = sink2;
#pragma unroll
  for (int t = 0; t < NS; ++t) M = fmaxf(M, stats_lds[(t * kDH + headB) * 2]);
  float den = exp2f(sink2 - M);
#pragma unroll
  for (int t = 0; t < NS; ++t) den += stats_lds[(t * kDH + headB) * 2 + 1] * exp2f(stats_lds[(t * kDH + headB) * 2] - M);
  __builtin_amdgcn_s_waitcnt(0);

  // lane-constant parts of the transposing reads
  const int colq = 16 * ((lane >> 4) & 1) + 4 * (j16 & 3);
  const int hoff = (j16 & 1) << 3;
  f32x16 tot[C::NMB];
#pragma unroll
  for (int mb = 0; mb < C::NMB; ++mb) tot[mb] = f32x16{};
#pragma unroll
  for (int tl = 0; tl < C::NSW; ++tl) {
    const int t = kh + 2 * tl;
    const int rb = t * a.RPS;
    if (rb >= Lk) break;
    const float fs = exp2f(stats_lds[(t * kDH + headB) * 2] - M);
    f32x16 acc[C::NMB];
#pragma unroll
    for (int mb = 0; mb < C::NMB; ++mb) acc[mb] = f32x16{};
#pragma unroll
    for (int k = 0; k < C::KPS; ++k) {
      const int r0 = rb + 16 * k;
      if (16 * k >= a.RPS || r0 >= Lk) break;
#pragma unroll
      for (int mb = 0; mb < C::NMB; ++mb) {
        const int col = 32 * mb + colq;
        const int lch = col >> 3;
        const int R0 = r0 + 8 * hf + (j16 >> 2);
        const bf16x4 lo = lds_read_tr16((const DSA_LDS __bf16*)(rows + R0 * C::SLICEB + ((lch ^ slice_swz<NS>(R0)) << 4) + hoff));
        const int R1 = R0 + 4;
        const bf16x4 hi = lds_read_tr16((const DSA_LDS __bf16*)(rows + R1 * C::SLICEB + ((lch ^ slice_swz<NS>(R1)) << 4) + hoff));
        const bf16x8 vf = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        acc[mb] = mfma32(vf, pre[tl][k], acc[mb]);
      }
    }
#pragma unroll
    for (int mb = 0; mb < C::NMB; ++mb)
#pragma unroll
      for (int e = 0; e < 16; ++e) tot[mb][e] += fs * acc[mb][e];
  }
  __syncthreads();  // done with the slices: reuse the LDS for the row-half reduction
  float* red = reinterpret_cast<float*>(rows);
  if (kh == 1) {
#pragma unroll
    for (int mb = 0; mb < C::NMB; ++mb)
#pragma unroll
      for (int e = 0; e < 16; ++e) red[((hb * C::NMB + mb) * 16 + e) * 64 + lane] = tot[mb][e];
  }
  __syncthreads();
  if (kh == 0) {
    const float inv = flags[0] ? __builtin_nanf("") : 1.f / den;
    __bf16* op = a.o + ((int64_t)q * kDH + headB) * kDD + d0 + 4 * hf;
    const int rope0 = kDD - 2 * a.rope_P;  // first rotated dim, kDD without a table
    const float* rrow = a.rope ? a.rope + (int64_t)(q % a.S) * a.rope_P * 2 : nullptr;
#pragma unroll
    for (int mb = 0; mb < C::NMB; ++mb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        float v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int e = 4 * g + i;
          v[i] = (tot[mb][e] + red[((hb * C::NMB + mb) * 16 + e) * 64 + lane]) * inv;
        }
        // the lane's four dims d .. d+3 are two whole rotary pairs
        const int d = d0 + 32 * mb + 8 * g + 4 * hf;
        if (rrow && d >= rope0) {
          const float4 cs = *reinterpret_cast<const float4*>(rrow + (d - rope0));
          rope_rot_inv(v[0], v[1], cs.x, cs.y);
          rope_rot_inv(v[2], v[3], cs.z, cs.w);
        }
        const bf16x4 ov = {(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
        *reinterpret_cast<bf16x4*>(op + 32 * mb + 8 * g) = ov;
      }
  }
  // departure, off the critical path: every sibling is past its wait by the time the last one
  // leaves, and that one clears the pair for the next call
  if (tid == 0 &&
      __hip_atomic_fetch_add(depart, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == (uint32_t)(NS - 1)) {
    if (IX != 0) __hip_atomic_exchange(&qsync[0], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_exchange(arrive, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_exchange(depart, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// How workgroups land on XCDs: the XCD-local rendezvous needs every workgroup with the same
// blockIdx mod 8 on the same XCD.  Run once per device by dsa_init.
__device__ uint32_t g_xcc_probe[2048];

__global__ void xcc_probe_kernel() {
  if (threadIdx.x == 0) g_xcc_probe[blockIdx.x] = xcc_id();
}

struct DecPlan {
  int ns, rps, lp, ok;
};

constexpr int kDecVariants = 6;  // (NS 8 | 16) x (idx rows given | selected | scored and selected)

template <int NS, int SKPT, int IX>
int resident_blocks(int dev) {
  int per_cu = 0, cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, sparse_attn_decode_kernel<NS, SKPT, IX>, 256, 0) !=
      hipSuccess)
    return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  return per_cu * cus;
}

DecPlan plan_decode(int Q, int H, int D, int L, bool fp4) {
  DecPlan p{0, 0, 0, 0};
  if (D != kDD || H != kDH || fp4 || Q <= 0 || Q > kDecQueriesMax || L <= 0) return p;
  p.ns = Q > 16 ? 8 : 16;
  const int per = (L + p.ns - 1) / p.ns;
  p.rps = (per + 15) & ~15;
  p.lp = p.ns * p.rps;
  const int max_l = p.ns == 8 ? DecCfg<8>::MAX_L : DecCfg<16>::MAX_L;
  const int kps = p.ns == 8 ? DecCfg<8>::KPS : DecCfg<16>::KPS;
  if (p.rps > kDecRowsMax || p.rps > 16 * kps || ((L + 15) & ~15) > max_l) return p;
  p.ok = 1;
  return p;
}

const char* const kDecNames[kDecVariants] = {
    "sparse_attn_decode<NS=8>",         "sparse_attn_decode<NS=16>",
    "sparse_attn_decode<NS=8,select>",  "sparse_attn_decode<NS=16,select>",
    "sparse_attn_decode<NS=8,score+select>", "sparse_attn_decode<NS=16,score+select>"};

}  // namespace

// One-time set-up of the decode kernels on device `dev` (current): the XCD placement probe (one
// launch on a private stream, then a synchronisation) and the resident workgroup count of every
// variant.
int decode_device_init(int dev, DeviceState& ds) {
  hipStream_t st = nullptr;
  if (hipStreamCreateWithFlags(&st, hipStreamNonBlocking) != hipSuccess)
    return fail(DSA_ERR_HIP, "dsa_init: stream creation failed on device %d", dev);
  hipLaunchKernelGGL(xcc_probe_kernel, dim3(2048), dim3(64), 0, st);
  uint32_t ids[2048];
  int ok = 1;
  if (hipGetLastError() != hipSuccess || hipStreamSynchronize(st) != hipSuccess ||
      hipMemcpyFromSymbol(ids, HIP_SYMBOL(g_xcc_probe), sizeof(ids)) != hipSuccess) {
    hipStreamDestroy(st);
    return fail(DSA_ERR_HIP, "dsa_init: XCD placement probe failed on device %d", dev);
  }
  hipStreamDestroy(st);
  for (int i = 8; i < 2048; ++i) ok &= ids[i] == ids[i & 7];
  ds.xcd_rr = ok;
  ds.resident[0] = resident_blocks<8, 0, 0>(dev);
  ds.resident[1] = resident_blocks<16, 0, 0>(dev);
  ds.resident[2] = resident_blocks<8, 8, 0>(dev);
  ds.resident[3] = resident_blocks<16, 8, 0>(dev);
  ds.resident[4] = resident_blocks<8, 8, 1>(dev);
  ds.resident[5] = resident_blocks<16, 8, 1>(dev);
  return DSA_OK;
}

// Bytes after the workspace header: P, then the stats.
size_t sparse_attn_decode_workspace(int B, int S, int H, int D, int L, bool fp4) {
  const DecPlan p = plan_decode(B * S, H, D, L, fp4);
  if (!p.ok) return 0;
  const size_t Q = (size_t)B * S;
  return Q * kDH * p.lp * 2 + Q * p.ns * kDH * 2 * 4;
}

// Returns 1 and launches when the two-phase decode path applies, 0 when the caller should use
// the general kernel, or a negative error.  With sel set, the kernel selects the index rows itself
// (idx is not read); that needs at most 2048 scores per row.  With ix set too, it also computes
// those scores (index head dim 128, at most 64 index heads).  `workspace` is the whole caller
// workspace: its header holds the per-query counters, P and the stats follow.
int sparse_attn_decode_launch(const __bf16* q, const unsigned char* win, int64_t win_n, int64_t win_bs,
                              int64_t win_rs, const unsigned char* comp, int64_t comp_n, int64_t comp_bs,
                              int64_t comp_rs, const float* sink, const int32_t* idx, int L, float scale_log2,
                              __bf16* o, int B, int S, int H, int D, bool fp4, void* workspace,
                              const DecSelect* sel, const DecIndex* ix, const float* rope, int rope_dim,
                              hipStream_t st) {
  const DecPlan p = plan_decode(B * S, H, D, L, fp4);
  if (!p.ok) return 0;
  if (sel && (sel->T > 2048 || sel->T < 1 || sel->Wc + sel->K != L)) return 0;
  if (ix && (!sel || ix->H_I < 1 || ix->H_I > 64 || ix->scores_out != sel->scores)) return 0;
  // slot codes hold row byte offsets in 32 bits; the copies move 16-byte pieces of rows
  if ((uint64_t)win_n * (uint64_t)win_rs >= (1ull << 31) || (uint64_t)comp_n * (uint64_t)comp_rs >= (1ull << 31))
    return 0;
  if ((((uintptr_t)win | (uintptr_t)comp) & 15) || ((win_rs | win_bs | comp_rs | comp_bs) & 15)) return 0;
  DeviceState* ds = nullptr;
  const int irc = ensure_device_init(st, &ds);
  if (irc) return irc;
  if (!ds->xcd_rr) return 0;  // workgroups do not land on XCDs round-robin: no XCD-local rendezvous
  const int vi = (p.ns == 8 ? 0 : 1) + (sel ? 2 : 0) + (ix ? 2 : 0);
  const int Q = B * S;
  const int Qp = (Q + 7) & ~7;
  if (Qp * p.ns > ds->resident[vi]) return 0;  // the rendezvous needs every workgroup resident at once
  DecArgs a{};
  a.q = q;
  a.win = win;
  a.win_n = win_n;
  a.win_bs = win_bs;
  a.win_rs = win_rs;
  a.comp = comp;
  a.comp_bs = comp_bs;
  a.comp_rs = comp_rs;
  a.sink = sink;
  a.idx = idx;
  a.L = L;
  a.scale_log2 = scale_log2;
  a.o = o;
  a.sync = (uint32_t*)workspace;
  a.pbuf = (__bf16*)((char*)workspace + kWsHeaderBytes);
  a.stats = (float*)((char*)a.pbuf + (size_t)Q * kDH * p.lp * 2);
  a.S = S;
  a.Q = Q;
  a.Qp = Qp;
  a.RPS = p.rps;
  a.Lp = p.lp;
  a.rope = rope;
  a.rope_P = rope ? rope_dim / 2 : 0;
  if (sel) {
    a.scores = sel->scores;
    a.T = sel->T;
    a.K = sel->K;
    a.start_pos = sel->start_pos;
    a.ratio = sel->ratio;
    a.W = sel->W;
    a.Wc = sel->Wc;
    a.offset = sel->offset;
    a.idx_out = sel->idx_out;
    a.ld_out = sel->ld_out;
  }
  if (ix) {
    a.q_idx = ix->q_idx;
    a.k_idx = ix->k_idx;
    a.k_bstride = ix->k_bstride;
    a.w_idx = ix->w;
    a.w_scale = ix->w_scale;
    a.H_I = ix->H_I;
  }
  dim3 grid(Qp * p.ns);
  switch (vi) {
    case 0: hipLaunchKernelGGL((sparse_attn_decode_kernel<8, 0, 0>), grid, dim3(256), 0, st, a); break;
    case 1: hipLaunchKernelGGL((sparse_attn_decode_kernel<16, 0, 0>), grid, dim3(256), 0, st, a); break;
    case 2: hipLaunchKernelGGL((sparse_attn_decode_kernel<8, 8, 0>), grid, dim3(256), 0, st, a); break;
    case 3: hipLaunchKernelGGL((sparse_attn_decode_kernel<16, 8, 0>), grid, dim3(256), 0, st, a); break;
    case 4: hipLaunchKernelGGL((sparse_attn_decode_kernel<8, 8, 1>), grid, dim3(256), 0, st, a); break;
    default: hipLaunchKernelGGL((sparse_attn_decode_kernel<16, 8, 1>), grid, dim3(256), 0, st, a); break;
  }
  const int rc = check_launch(kDecNames[vi]);
  return rc ? rc : 1;
}

// Read and clear the sticky error bits of the decode kernels (device `dev` current, idle).
int decode_read_errors(uint32_t* bits) {
  uint32_t v = 0, z = 0;
  if (hipMemcpyFromSymbol(&v, HIP_SYMBOL(g_dec_error), sizeof(v)) != hipSuccess ||
      hipMemcpyToSymbol(HIP_SYMBOL(g_dec_error), &z, sizeof(z)) != hipSuccess)
    return fail(DSA_ERR_HIP, "dsa_device_errors: reading the error flags failed");
  *bits = v;
  return DSA_OK;
}

}  // namespace dsa
