/*
 * dsa.h -- C ABI of the sparse MQA attention step for AMD Instinct MI355X (gfx950).
 *
 * The step has three stages, each a call here (all asynchronous on the
 * caller's HIP stream, none allocating device memory):
 *
 *   dsa_index_scores  score every compressed KV row for every query
 *   dsa_candidate_blocks, dsa_index_scores_masked  the two-level selection's candidate blocks
 *   dsa_index_scores_mxfp4  the same with the indexer's fp4 (E8M0 per 32) query and key rows
 *   dsa_topk          keep the index_topk best visible rows per query
 *   dsa_window_idx    the sliding-window part of each query's index row
 *   dsa_select        window part and top-k part of the index rows in one launch
 *   dsa_sparse_attn   attend all heads over the rows an index row names
 *   dsa_sparse_attn_rope, dsa_rope_inverse  the output's inverse rotary embedding (fused)
 *   dsa_compress_kv_write  rotary embedding + fp4 quantisation of new compressed-cache rows
 *   dsa_sparse_attn_select  dsa_select then dsa_sparse_attn, one launch where the decode
 *                     attention kernel can select its own index rows
 *   dsa_sparse_attn_step  the whole step: dsa_index_scores then dsa_sparse_attn_select, one
 *                     launch where the decode attention kernel can also score the rows
 *
 * Citations refer to the DeepSeek V4.1 model pages ("attention/attend/selected",
 * "reindex-layer/read-weights") by the class or function that holds the step.
 *
 * Conventions shared by every call:
 *  - Device pointers are caller-owned memory on the current HIP device; the
 *    library never frees or retains them past the call.  Every call only
 *    enqueues kernels on `stream` (NULL = the legacy default stream) and
 *    returns without synchronising, with three exceptions, each stated where
 *    it applies: dsa_init (and the first decode call on a device dsa_init has
 *    not prepared, which runs it), dsa_device_errors, and DSA_DEBUG mode.
 *  - Tensors are dense, row-major, in the stated layout.  Where a batch stride
 *    is taken, it is in elements (rows * row length for a dense batch), so a
 *    cache slice [:B, :n] of a larger [max_B, max_n, D] buffer can be passed
 *    without a copy.
 *  - Return value: DSA_OK (0) on success, a negative DSA_ERR_* code otherwise.
 *    Invalid arguments are rejected before anything is enqueued; the reason
 *    is available from dsa_last_error() (thread-local text, valid until the
 *    next call on the same thread).  No C++ exception crosses the ABI.
 *  - Index values inside idx rows are not range-checked on the device (as on
 *    the pages, an out-of-range index is a caller error); -1 marks an empty
 *    slot.  With DSA_DEBUG=1 in the environment (or dsa_set_debug(1)),
 *    dsa_sparse_attn copies the caller's idx to the host and rejects any entry
 *    outside [-1, rows) with DSA_ERR_INDEX before launching (one
 *    synchronisation per call; not allowed under stream capture).
 *  - Workspace: a call that takes one uses it as scratch.  Its first
 *    DSA_WORKSPACE_HEADER_BYTES hold per-query rendezvous counters of the
 *    decode kernels, which must be zero before the workspace's first use (for
 *    example allocated zero-filled); every call leaves them zero again when
 *    its kernels end.  Calls in stream order may share a workspace; calls that
 *    can run at the same time (other streams, graphs replayed concurrently)
 *    need workspaces of their own.
 */
#ifndef DSA_H_
#define DSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DSA_ABI_VERSION 2
#define DSA_WORKSPACE_HEADER_BYTES 4096
#define DSA_NOALLOC_SCRATCH_BYTES (32u << 20) /* scratch of dsa_sparse_attn_step_noalloc */

typedef struct ihipStream_t* dsa_stream_t; /* a hipStream_t */

enum dsa_status {
  DSA_OK = 0,
  DSA_ERR_NULL = -1,        /* a required pointer is NULL */
  DSA_ERR_SHAPE = -2,       /* a size is negative, zero where it may not be, or inconsistent */
  DSA_ERR_DTYPE = -3,       /* unknown dtype or format code */
  DSA_ERR_UNSUPPORTED = -4, /* valid arguments with no instantiated kernel (e.g. head_dim 96) */
  DSA_ERR_HIP = -5,         /* the HIP runtime reported an error at launch */
  DSA_ERR_WORKSPACE = -6,   /* workspace NULL or smaller than the size the query returns */
  DSA_ERR_STATE = -7,       /* a synchronising step was needed under stream capture (see dsa_init) */
  DSA_ERR_INDEX = -8        /* DSA_DEBUG: an idx entry outside [-1, rows) */
};

enum dsa_dtype {
  DSA_F32 = 0,  /* IEEE binary32 */
  DSA_BF16 = 1  /* bfloat16 */
};

enum dsa_kv_format {
  DSA_KV_DENSE = 0,        /* rows of D elements in the call's dtype */
  DSA_KV_FP4_E4M3_G16 = 1  /* rows of D/2 bytes of e2m1 nibbles (element 2k in the low
                              nibble of byte k) plus D/16 E4M3 scale bytes, one per 16
                              consecutive elements (compressed KV of `_compress_kv`);
                              only with dtype DSA_BF16 */
};

/* Library identity. */
int dsa_abi_version(void);
const char* dsa_last_error(void);

/*
 * What the last call on this thread launched: the number of kernels it enqueued and their names
 * joined by '+' (for example "index_scores_bf16+topk<256,8>+sparse_attn_decode<NS=8>").  The
 * record is reset at the start of every call and is valid until the next call on the thread.
 */
int dsa_last_launch_count(void);
const char* dsa_last_launches(void);

/*
 * Per-device set-up (call once per device before the first decode call, and before capturing any
 * call into a graph): checks on which XCD each workgroup runs (the decode kernels keep all
 * workgroups of a query on one XCD and meet in its L2, which needs workgroup i on XCD i mod 8),
 * records how many workgroups of each decode kernel fit on the device at once, and reads
 * DSA_DEBUG.  Launches one small kernel on a private stream and synchronises with it.
 * Idempotent and thread-safe.  A call that needs a device dsa_init has not prepared runs it
 * itself (one synchronisation), or returns DSA_ERR_STATE under stream capture.  Where the XCD check
 * fails, the decode kernels are not used and the calls take their multi-launch paths.
 */
int dsa_init(int device);

/*
 * Reads and clears the device's sticky error bits (bit 0: a decode rendezvous timed out; that
 * query's output was set to NaN).  Synchronises the device first.
 */
int dsa_device_errors(int device, uint32_t* flags);

/* Turns the DSA_DEBUG index checks on (1) or off (0); returns the previous setting. */
int dsa_set_debug(int on);

/*
 * Host-side range check of index rows (what DSA_DEBUG runs on a copy of idx): DSA_OK when every
 * one of the `count` entries of the host array idx is -1 or in [0, n_rows); DSA_ERR_INDEX
 * otherwise, with the position of the first bad entry in *first_bad (may be NULL).
 */
int dsa_check_idx(const int32_t* idx, int64_t count, int64_t n_rows, int64_t* first_bad);

/*
 * Index scores (`Indexer.forward`: einsum of the index query heads with the
 * shared index key per compressed row, ReLU, weighted by `weights_proj`,
 * summed over heads; invisible groups masked to -inf):
 *
 *   scores[b,t,j] = w_scale * sum_h w[b,t,h] * max(0, sum_d q_idx[b,t,h,d] * k_idx[b,j,d])
 *                   for j <  c(t) = (start_pos + t + 1) / ratio  (integer division)
 *   scores[b,t,j] = -inf  for c(t) <= j < T
 *
 *   q_idx  [B, S, H_I, D_I]  dtype            contiguous
 *   k_idx  [B, T, D_I]       dtype            batch stride k_batch_stride (>= T*D_I)
 *   w      [B, S, H_I]       dtype            raw head weights (weights_proj output)
 *   scores [B, S, T]         float32          written in full
 *   w_scale: the page's index_head_dim**-0.5 * index_n_heads**-0.5 (or any positive factor)
 *
 * Products are exact, sums are float32.  Supported: D_I in {32, 64, 128, 256},
 * H_I in 1..64 (bf16: multiples of 8 run fastest), T >= 0 (T == 0 writes nothing).
 * Requires T <= (start_pos + S) / ratio and ratio >= 1.
 */
int dsa_index_scores(const void* q_idx, const void* k_idx, int64_t k_batch_stride, const void* w,
                     float w_scale, int dtype, int B, int S, int T, int H_I, int D_I, int start_pos,
                     int ratio, float* scores, dsa_stream_t stream);

/*
 * Candidate blocks of the two-level selection (`Indexer.forward` with a candidate source: the
 * source layer picks candidate_topk_blocks blocks of candidate_block_size compressed positions
 * from its scores, `select_candidate_blocks`; later indexers mask their scores outside them).
 * The pages do not show that function; this library's reading: block i covers positions
 * i*block_size .. +block_size-1 and is visible to query t when its first position is (i*block_size
 * < c(t)); its score is the largest of its visible scores; the min(n_blocks, visible blocks) best
 * visible blocks are chosen, equal scores going to the lower block.
 */
typedef struct dsa_candidates {
  const uint32_t* bits; /* [B, S, ld_bits] words: bit i%32 of word i/32 of query (b,t): block i chosen */
  int64_t ld_bits;      /* words per query row, >= ceil(ceil(T / block_size) / 32) */
  int block_size;       /* compressed positions per block, a power of two */
} dsa_candidates;

/*
 * The candidate blocks of every query from the source layer's scores [B, S, T] float32 (as
 * dsa_index_scores writes them; j >= c(t) is not read): bits [B, S, ld_bits] uint32, each row
 * written in full (words past the last block are zero).  Supported: T / block_size <= 8192.
 */
int dsa_candidate_blocks(const float* scores, int B, int S, int T, int start_pos, int ratio, int block_size,
                         int n_blocks, uint32_t* bits, int64_t ld_bits, dsa_stream_t stream);

/*
 * dsa_index_scores for a consumer of candidate blocks ("score with our own weights, but only inside
 * the source's candidate blocks"): the same scores at positions whose block is a candidate of that
 * query, -inf elsewhere.  For one query per batch (decode) the keys outside the candidate blocks are
 * not read.  cand may be NULL (no mask).  Errors: those of dsa_index_scores, and DSA_ERR_SHAPE for a
 * block size that is not a power of two or rows of too few words.
 */
int dsa_index_scores_masked(const void* q_idx, const void* k_idx, int64_t k_batch_stride, const void* w,
                            float w_scale, int dtype, int B, int S, int T, int H_I, int D_I, int start_pos, int ratio,
                            const dsa_candidates* cand, float* scores, dsa_stream_t stream);

/*
 * Index scores with the indexer's fp4 operands (`Indexer.forward` quantises the index queries and
 * keys to fp4; `_compress_kv` gives the indexer's blocks: 32 elements per E8M0 scale):
 * the same scores as dsa_index_scores over the decoded values
 *   value = e2m1(nibble) * 2^(scale byte - 127)   (scale byte 255 is NaN),
 * element 2k of a row in the low nibble of byte k, elements 32i .. 32i+31 scaled by scale byte i.
 *
 *   q_idx   [B, S, H_I, D_I/2] uint8 packed e2m1     q_scale [B, S, H_I, D_I/32] uint8 E8M0
 *   k_idx   [B, k_batch_rows, D_I/2] uint8           k_scale [B, k_batch_rows, D_I/32] uint8
 *           (rows 0 .. T-1 of each batch are read; k_batch_rows >= T, so a cache slice needs no copy)
 *   w       [B, S, H_I] bf16 raw head weights;  scores [B, S, T] float32, written in full
 *
 * Products are exact (block-scaled MFMA on e2m1 operands), sums float32.  Supported: D_I in
 * {64, 128, 256}, H_I in 1..64; q_idx and k_idx 16-byte aligned.  Same visibility rules and errors as
 * dsa_index_scores.  cand (may be NULL): candidate blocks, as for dsa_index_scores_masked.
 */
int dsa_index_scores_mxfp4(const uint8_t* q_idx, const uint8_t* q_scale, const uint8_t* k_idx,
                           const uint8_t* k_scale, int64_t k_batch_rows, const void* w, float w_scale, int B, int S,
                           int T, int H_I, int D_I, int start_pos, int ratio, const dsa_candidates* cand,
                           float* scores, dsa_stream_t stream);

/*
 * Top-k selection (`Indexer.forward`: top-k by score, re-sorted into position
 * order, unreachable -> -1, the rest shifted by `offset`):
 *
 *   K = min(index_topk, T).  For query t, with n = min(K, c(t)) and
 *   c(t) = (start_pos + t + 1) / ratio, the first n entries of the row are
 *   offset + j for the n visible positions j < c(t) with the largest scores
 *   (equal scores: the lower position wins; -0.0 equals +0.0), in ascending j;
 *   entries n..K-1 are -1.
 *
 *   scores [B, S, T] float32 (only j < c(t) is read)
 *   idx    int32, row (b,t) starts at idx + (b*S + t) * ld_idx; K entries are written,
 *          so a [B, S, Wc + K] buffer is filled at its tail by passing idx + Wc, ld_idx = Wc + K.
 *
 *   workspace: device memory of dsa_topk_workspace_size(B, S, T, index_topk) bytes (zero-filled
 *          header as for every workspace; may be NULL when that size is 0).  With it, rows of few
 *          queries and more than 16384 scores are selected in two launches over 4096-score chunks
 *          (the chunks' best K as candidates, then the best K of those); without it (NULL), by one
 *          workgroup per row.  Both give the same result.
 *
 * Supported: T <= 65536.  NaN scores are outside the contract.
 */
int dsa_topk(const float* scores, int B, int S, int T, int index_topk, int start_pos, int ratio,
             int offset, int32_t* idx, int64_t ld_idx, void* workspace, size_t workspace_bytes,
             dsa_stream_t stream);

/* Bytes of workspace dsa_topk and dsa_select use for this shape (0 when none). */
size_t dsa_topk_workspace_size(int B, int S, int T, int index_topk);

/*
 * How dsa_topk and dsa_select share the B*S rows between their two kernels: the first *wave_rows
 * rows go to the one-wave-per-row kernel (many rows, T <= 8192; its reads of a whole number of
 * 64-key groups must stay inside the scores buffer), the other *block_rows rows to the
 * one-workgroup-per-row kernel.  Host arithmetic only, nothing is launched.
 */
int dsa_topk_plan(int B, int S, int T, int64_t* wave_rows, int64_t* block_rows);

/*
 * Window index rows (`get_window_topk_idxs`):
 *   start_pos == 0 (prefill): Wc = min(S, W); row t holds chunk positions
 *     max(0, t-W+1) + s for s < Wc, with -1 where that exceeds t.
 *   start_pos > 0 (decode, S must be 1): Wc = W; the ring slots oldest first,
 *     (start_pos mod W) + 1 .. W-1, then 0 .. start_pos mod W, with -1 for a
 *     slot greater than start_pos (ring still filling).
 *   idx int32, row (b,t) starts at idx + (b*S + t) * ld_idx; Wc entries are written.
 * Other combinations (start_pos > 0 with S > 1) are not defined by the page
 * and return DSA_ERR_UNSUPPORTED.
 */
int dsa_window_idx(int B, int S, int start_pos, int W, int32_t* idx, int64_t ld_idx,
                   dsa_stream_t stream);

/* Window columns dsa_window_idx writes (min(S, W) in prefill, W in decode), or a negative error. */
int dsa_window_cols(int S, int start_pos, int W);

/*
 * A whole index row in one launch (`Indexer.forward` and `get_window_topk_idxs` as the attention
 * layer joins them): row (b,t) of idx gets its Wc = dsa_window_cols(S, start_pos, W) window
 * entries at columns [0, Wc), exactly as dsa_window_idx writes them, and its K = min(index_topk, T)
 * top-k entries at columns [Wc, Wc + K), exactly as dsa_topk writes them with the given offset
 * (the window-KV row count: S in prefill, W in decode).  Same as the two calls in sequence,
 * with one kernel instead of two.
 *
 *   scores [B, S, T] float32 (may be NULL when T == 0)
 *   idx    int32, row (b,t) starts at idx + (b*S + t) * ld_idx, ld_idx >= Wc + K.
 *   workspace: as for dsa_topk.
 *
 * Errors: those of dsa_window_idx and dsa_topk.
 */
int dsa_select(const float* scores, int B, int S, int T, int index_topk, int start_pos, int ratio, int W,
               int offset, int32_t* idx, int64_t ld_idx, void* workspace, size_t workspace_bytes,
               dsa_stream_t stream);

/*
 * One KV source of sparse attention.  Rows are D elements of the call's dtype
 * (DSA_KV_DENSE) or fp4 rows with E4M3 group scales (DSA_KV_FP4_E4M3_G16).
 *   rows:   row r of batch b at rows + b*batch_stride + r*row_stride (in elements
 *           for DENSE, in bytes for FP4, whose row is D/2 bytes)
 *   scales: FP4 only; row r of batch b at scales + b*scale_batch_stride + r*scale_row_stride
 *           (bytes; a row is D/16 bytes)
 */
typedef struct dsa_kv_src {
  const void* rows;
  int64_t n_rows;
  int64_t batch_stride;
  int64_t row_stride;
  int format; /* enum dsa_kv_format */
  const uint8_t* scales;
  int64_t scale_batch_stride;
  int64_t scale_row_stride;
} dsa_kv_src;

/*
 * Sparse attention with a per-head sink (`sparse_attn_kernel` / `sparse_attn`;
 * `Attention.forward` concatenates the window rows and the compressed rows
 * into one KV tensor and shifts compressed indices by the window row count):
 *
 *   the KV row named by index i of batch b is win row i when i < win->n_rows,
 *   otherwise comp row i - win->n_rows.  Key and value are the same row.
 *   For each (b, t, h), over the slots s with idx[b,t,s] != -1:
 *     l_s = scale * q[b,t,h,:] . row_s
 *     o[b,t,h,:] = sum_s e^{l_s} row_s / (sum_s e^{l_s} + e^{sink[h]})
 *   A query with no valid slot gets o = 0.  Duplicate indices count once each.
 *
 *   q    [B, S, H, D] dtype, contiguous
 *   sink [H] float32
 *   idx  [B, S, L] int32, contiguous (L >= 0)
 *   o    [B, S, H, D] dtype, contiguous, written in full
 *   comp may be NULL (or have n_rows 0) when no index reaches past the window.
 *   workspace: device memory of at least dsa_sparse_attn_workspace_size(...) bytes
 *     (may be NULL when that size is 0); zero-filled header, see the conventions above.
 *
 * Supported: dtype BF16 with D in {64, 128, 256, 512} and H in 1..128, or dtype
 * F32 with D <= 512 and H <= 64.  Accumulation is float32; the probabilities
 * multiplying the bf16 rows are rounded to bf16 (as the page's kernel does).
 */
int dsa_sparse_attn(const void* q, const dsa_kv_src* win, const dsa_kv_src* comp, const float* sink,
                    const int32_t* idx, int L, float scale, void* o, int dtype, int B, int S, int H,
                    int D, void* workspace, size_t workspace_bytes, dsa_stream_t stream);

/* Bytes of workspace dsa_sparse_attn needs for this shape (0 when none; otherwise at least
   DSA_WORKSPACE_HEADER_BYTES). */
size_t dsa_sparse_attn_workspace_size(int dtype, int B, int S, int H, int D, int L);

/* Bytes of workspace dsa_sparse_attn_select, dsa_sparse_attn_step and dsa_sparse_attn_step_mxfp4
   need: enough for the index-row selection and for the attention over rows of
   L = dsa_window_cols(S, start_pos, W) + min(index_topk, T) entries (0 when none). */
size_t dsa_step_workspace_size(int dtype, int B, int S, int H, int D, int T, int index_topk, int start_pos,
                               int W);

/*
 * Sparse attention followed by the inverse rotary embedding of its output (`Attention.forward`:
 * `apply_rotary_emb(o[..., -rope_head_dim:], freqs_cis, True)` right after `sparse_attn`): the
 * results of dsa_sparse_attn, then for each query t (positions of this call) and head, the pairs
 * (o[2i], o[2i+1]) of its last rope_dim dims replaced by (o[2i] + i o[2i+1]) (cos - i sin), with
 * (cos, sin) = freqs[t][i].  The decode and prefill kernels rotate in their epilogue (before the
 * output is rounded to bf16); other shapes run dsa_rope_inverse after the attention.
 *
 *   freqs [S, rope_dim/2, 2] float32 (cos, sin), 16-byte aligned; rope_dim a multiple of 16, <= D.
 *   Other arguments and errors: those of dsa_sparse_attn.
 */
int dsa_sparse_attn_rope(const void* q, const dsa_kv_src* win, const dsa_kv_src* comp, const float* sink,
                         const int32_t* idx, int L, float scale, void* o, int dtype, int B, int S, int H, int D,
                         const float* freqs, int rope_dim, void* workspace, size_t workspace_bytes,
                         dsa_stream_t stream);

/* The inverse rotary embedding alone, in place on o [B, S, H, D] (dtype), as dsa_sparse_attn_rope
   applies it. */
int dsa_rope_inverse(void* o, int dtype, int B, int S, int H, int D, const float* freqs, int rope_dim,
                     dsa_stream_t stream);

/*
 * The compressed-cache write of `_compress_kv`: the latent rows are rotated on their last rope_dim
 * dims (freqs of each row's group position), fp4-quantised with one E4M3 scale per 16 elements and
 * stored at rows row0 .. row0+n-1 of the fp4 cache (the layout DSA_KV_FP4_E4M3_G16 reads).  Each
 * step is taken in the precision of the page's bf16 tensors: float32 products and sums without
 * fused multiply-adds, rounded to bf16; scale = E4M3(amax / 6) to nearest-even, saturated at 448;
 * code = the e2m1 value nearest x / scale (ties to the even code, at most 6).
 *
 *   latent [B, n, D] bf16, batch stride latent_batch_stride (elements)
 *   freqs  [n, rope_dim/2, 2] float32 (cos, sin), 16-byte aligned; rope_dim a multiple of 16, <= D
 *   rows   [B, >= row0 + n, D/2] uint8 (batch stride in bytes, 8-byte aligned rows)
 *   scales [B, >= row0 + n, D/16] uint8 (batch stride in bytes)
 */
int dsa_compress_kv_write(const void* latent, int64_t latent_batch_stride, int B, int n, int D, const float* freqs,
                          int rope_dim, uint8_t* rows, int64_t rows_batch_stride, uint8_t* scales,
                          int64_t scales_batch_stride, int64_t row0, dsa_stream_t stream);

/*
 * The index rows and the attention over them (`Indexer.forward`, `get_window_topk_idxs` and
 * `sparse_attn` as `Attention.forward` chains them): the same results as
 *
 *   dsa_select(scores, B, S, T, index_topk, start_pos, ratio, W, win->n_rows, idx, L, workspace, ...)
 *   dsa_sparse_attn(q, win, comp, sink, idx, L, scale, o, dtype, B, S, H, D, workspace, ...)
 *
 * with L = dsa_window_cols(S, start_pos, W) + min(index_topk, T).  For decode batches that the
 * two-phase decode attention kernel takes (bf16, D = 512, H = 64, dense rows, fewer than 256
 * queries, all of its workgroups resident at once, T <= 2048, the device's XCD check passed in
 * dsa_init) it is one launch: every workgroup of a query selects that query's index row from its
 * scores in the kernel's prologue.  Otherwise it makes the two calls above.  dsa_last_launches()
 * tells which happened.
 *
 *   scores [B, S, T] float32; q, win, comp, sink, o, workspace as for dsa_sparse_attn, with the
 *   workspace sized by dsa_step_workspace_size(dtype, B, S, H, D, T, index_topk, start_pos, W).
 *   idx    [B, S, L] int32, contiguous: receives the index rows.  It may be NULL when the one-launch
 *          path applies (the rows are then not written out); DSA_ERR_NULL when it does not.
 *
 * Errors: those of dsa_select and dsa_sparse_attn.
 */
int dsa_sparse_attn_select(const float* scores, int T, int index_topk, int start_pos, int ratio, int W,
                           const void* q, const dsa_kv_src* win, const dsa_kv_src* comp, const float* sink,
                           float scale, void* o, int dtype, int B, int S, int H, int D, int32_t* idx,
                           void* workspace, size_t workspace_bytes, dsa_stream_t stream);

/*
 * The whole step (`Indexer.forward` for the scores and the index rows, `get_window_topk_idxs`,
 * `sparse_attn` as `Attention.forward` chains them): the same results as
 *
 *   dsa_index_scores(q_idx, k_idx, k_batch_stride, w, w_scale, dtype, B, S, T, H_I, D_I,
 *                    start_pos, ratio, scores, stream)
 *   dsa_sparse_attn_select(scores, T, index_topk, start_pos, ratio, W, q, win, comp, sink,
 *                          scale, o, dtype, B, S, H, D, idx, workspace, workspace_bytes, stream)
 *
 * For the decode batches whose index rows dsa_sparse_attn_select selects inside the decode
 * attention kernel, and with D_I = 128, H_I <= 64, 16-byte aligned q_idx and k_idx and
 * k_batch_stride a multiple of 8, it is one launch: the workgroups of a query each score a share
 * of the compressed rows into `scores`, meet, select the query's index row from all of its scores
 * and attend.  That needs the workgroups of a query to share one L2 (checked once per device by
 * dsa_init); where they do not, or the shape does not fit, it makes the two calls above.
 * dsa_last_launches() tells which happened.
 *
 *   q_idx, k_idx, w, w_scale, H_I, D_I, T, start_pos, ratio: as for dsa_index_scores
 *   scores [B, S, T] float32, required: always written in full (dsa_index_scores' contract)
 *   index_topk, W, q, win, comp, sink, scale, o, dtype, B, S, H, D, idx, workspace: as for
 *   dsa_sparse_attn_select (idx may be NULL where that call allows it)
 *
 * Errors: those of dsa_index_scores and dsa_sparse_attn_select.
 */
int dsa_sparse_attn_step(const void* q_idx, const void* k_idx, int64_t k_batch_stride, const void* w, float w_scale,
                         int H_I, int D_I, int T, int index_topk, int start_pos, int ratio, int W, const void* q,
                         const dsa_kv_src* win, const dsa_kv_src* comp, const float* sink, float scale, void* o,
                         int dtype, int B, int S, int H, int D, float* scores, int32_t* idx, void* workspace,
                         size_t workspace_bytes, dsa_stream_t stream);

/*
 * The whole step with the indexer's fp4 operands: the same results as
 *
 *   dsa_index_scores_mxfp4(q_idx, q_scale, k_idx, k_scale, k_batch_rows, w, w_scale, B, S, T, H_I, D_I,
 *                          start_pos, ratio, NULL, scores, stream)
 *   dsa_sparse_attn_select(scores, T, index_topk, start_pos, ratio, W, q, win, comp, sink, scale, o,
 *                          dtype, B, S, H, D, idx, workspace, workspace_bytes, stream)
 *
 * (dtype must be DSA_BF16).  Errors: those of the two calls.
 */
int dsa_sparse_attn_step_mxfp4(const uint8_t* q_idx, const uint8_t* q_scale, const uint8_t* k_idx,
                               const uint8_t* k_scale, int64_t k_batch_rows, const void* w, float w_scale, int H_I,
                               int D_I, int T, int index_topk, int start_pos, int ratio, int W, const void* q,
                               const dsa_kv_src* win, const dsa_kv_src* comp, const float* sink, float scale,
                               void* o, int dtype, int B, int S, int H, int D, float* scores, int32_t* idx,
                               void* workspace, size_t workspace_bytes, dsa_stream_t stream);

/*
 * The whole step without a workspace argument, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid allocation).  Same
 * arguments, results and launches as dsa_sparse_attn_step, minus workspace and workspace_bytes: the
 * scratch is a fixed array of DSA_NOALLOC_SCRATCH_BYTES (32 MiB) per device that the library
 * holds until the process ends.  The call allocates nothing.
 *
 *  - dsa_init(device) must have run on the current device (DSA_ERR_STATE otherwise); it looks up
 *    the array's device address.
 *  - Shapes whose dsa_step_workspace_size exceeds the array are refused with
 *    DSA_ERR_WORKSPACE before anything is launched (decode batches of up to 32 queries with
 *    H = 64, D = 512 and L <= 768 fit; prefill batches of 256 or more queries at D = 512 need no
 *    scratch).
 *  - Every call on a device shares that device's array, which keeps the last call's contents: the
 *    rendezvous counters at its start are zero when the library loads and every call leaves them
 *    zero.  Calls that can run at the same time on one device (other streams, concurrently
 *    replayed graphs) race on the array and must not overlap.
 */
int dsa_sparse_attn_step_noalloc(const void* q_idx, const void* k_idx, int64_t k_batch_stride, const void* w,
                                 float w_scale, int H_I, int D_I, int T, int index_topk, int start_pos, int ratio,
                                 int W, const void* q, const dsa_kv_src* win, const dsa_kv_src* comp,
                                 const float* sink, float scale, void* o, int dtype, int B, int S, int H, int D,
                                 float* scores, int32_t* idx, dsa_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* DSA_H_ */
