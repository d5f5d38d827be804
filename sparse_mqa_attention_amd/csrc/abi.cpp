// C ABI of libdsa: argument validation, error text, dispatch to the HIP launchers.
// Nothing here allocates device memory or synchronises the stream.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <vector>

#include "../../include/dsa.h"
#include "dsa_internal.h"

namespace dsa {

static thread_local char g_err[512] = "";
// kernels the last top-level call on this thread launched: count and '+'-joined names
static thread_local int g_nlaunch = 0;
static thread_local char g_launches[512] = "";
static thread_local int g_depth = 0;

// Marks a top-level entry point: clears the error text and the launch record once per call (the
// composite calls go through the simpler ones).
struct Entry {
  Entry() {
    if (g_depth++ == 0) {
      g_err[0] = 0;
      g_nlaunch = 0;
      g_launches[0] = 0;
    }
  }
  ~Entry() { --g_depth; }
};

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int check_launch(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(DSA_ERR_HIP, "%s: launch failed: %s", what, hipGetErrorString(e));
  ++g_nlaunch;
  const size_t n = strlen(g_launches);
  snprintf(g_launches + n, sizeof(g_launches) - n, "%s%s", n ? "+" : "", what);
  return DSA_OK;
}

// ---- per-device set-up -------------------------------------------------------------------------
constexpr int kMaxDevices = 64;
static DeviceState g_dev[kMaxDevices];
static std::mutex g_dev_mu;
static int g_debug = -1;  // -1: not read from DSA_DEBUG yet

int scratch_device_init(int dev, DeviceState& ds);
size_t scratch_bytes();

static bool debug_on() {
  if (g_debug < 0) {
    const char* e = getenv("DSA_DEBUG");
    g_debug = (e && e[0] && strcmp(e, "0") != 0) ? 1 : 0;
  }
  return g_debug > 0;
}

static int init_device(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return fail(DSA_ERR_SHAPE, "dsa_init: device %d out of range", dev);
  std::lock_guard<std::mutex> lk(g_dev_mu);
  DeviceState& ds = g_dev[dev];
  if (ds.ready) return DSA_OK;
  int prev = 0;
  if (hipGetDevice(&prev) != hipSuccess) return fail(DSA_ERR_HIP, "dsa_init: no current device");
  if (prev != dev && hipSetDevice(dev) != hipSuccess) return fail(DSA_ERR_HIP, "dsa_init: cannot select device %d", dev);
  int rc = decode_device_init(dev, ds);
  if (rc == DSA_OK) rc = scratch_device_init(dev, ds);
  if (prev != dev) hipSetDevice(prev);
  if (rc == DSA_OK) ds.ready = 1;
  debug_on();
  return rc;
}

int ensure_device_init(hipStream_t st, DeviceState** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return fail(DSA_ERR_HIP, "no usable current HIP device");
  DeviceState& ds = g_dev[dev];
  if (!ds.ready) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(st, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone)
      return fail(DSA_ERR_STATE, "device %d is not set up: call dsa_init(%d) before capturing a graph", dev, dev);
    const int rc = init_device(dev);
    if (rc) return rc;
  }
  *out = &ds;
  return DSA_OK;
}

// DSA_DEBUG: the caller's index rows are copied to the host and range-checked before the attention
// is launched (one synchronisation per call).
static int debug_check_idx(const int32_t* idx, int64_t count, int64_t n_rows, hipStream_t st) {
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(st, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone)
    return fail(DSA_ERR_STATE, "DSA_DEBUG index checks cannot run under stream capture");
  std::vector<int32_t> h((size_t)count);
  if (hipMemcpyAsync(h.data(), idx, (size_t)count * 4, hipMemcpyDeviceToHost, st) != hipSuccess ||
      hipStreamSynchronize(st) != hipSuccess)
    return fail(DSA_ERR_HIP, "DSA_DEBUG: copying idx to the host failed");
  int64_t bad = -1;
  if (dsa_check_idx(h.data(), count, n_rows, &bad) != DSA_OK)
    return fail(DSA_ERR_INDEX, "dsa_sparse_attn: idx entry %lld is %d, outside [-1, %lld)", (long long)bad,
                h[(size_t)bad], (long long)n_rows);
  return DSA_OK;
}

int index_scores_launch(const void*, const void*, int64_t, const void*, float, int, int, int, int, int, int, int, int,
                        float*, const CandMask&, hipStream_t);
int candidate_blocks_launch(const float*, int, int, int, int, int, int, int, uint32_t*, int64_t, hipStream_t);
int topk_launch(const float*, int, int, int, int, int, int, int, int32_t*, int64_t, int, int, void*, hipStream_t);
size_t topk_split_bytes(int, int, int, int);
int index_scores_mxfp4_launch(const uint8_t*, const uint8_t*, const uint8_t*, const uint8_t*, int64_t, const void*,
                              float, int, int, int, int, int, int, int, float*, const CandMask&, hipStream_t);
void topk_plan(int, int, int, int64_t*, int64_t*);
int window_idx_launch(int, int, int, int, int, int32_t*, int64_t, hipStream_t);
int sparse_attn_bf16_launch(const void*, const dsa_kv_src*, const dsa_kv_src*, const float*, const int32_t*, int,
                            float, void*, int, int, int, int, void*, const float*, int, hipStream_t);
int rope_inverse_launch(void*, int, int, int, int, int, const float*, int, hipStream_t);
int compress_kv_write_launch(const void*, int64_t, int, int, int, int, const float*, uint8_t*, int64_t, uint8_t*,
                             int64_t, int64_t, hipStream_t);
int sparse_attn_f32_launch(const void*, const dsa_kv_src*, const dsa_kv_src*, const float*, const int32_t*, int,
                           float, void*, int, int, int, int, hipStream_t);
size_t sparse_attn_bf16_workspace(int, int, int, int, int, bool);
int sparse_attn_bf16_select_launch(const void*, const dsa_kv_src*, const dsa_kv_src*, const float*, const DecSelect*,
                                   const DecIndex*, int, float, void*, int, int, int, int, void*, hipStream_t);

}  // namespace dsa

using dsa::fail;

extern "C" {

int dsa_abi_version(void) { return DSA_ABI_VERSION; }

const char* dsa_last_error(void) { return dsa::g_err; }

int dsa_last_launch_count(void) { return dsa::g_nlaunch; }

const char* dsa_last_launches(void) { return dsa::g_launches; }

int dsa_init(int device) {
  dsa::Entry e;
  return dsa::init_device(device);
}

int dsa_device_errors(int device, uint32_t* flags) {
  dsa::Entry e;
  if (!flags) return fail(DSA_ERR_NULL, "dsa_device_errors: NULL flags");
  *flags = 0;
  if (device < 0 || device >= dsa::kMaxDevices) return fail(DSA_ERR_SHAPE, "dsa_device_errors: device %d", device);
  int prev = 0;
  if (hipGetDevice(&prev) != hipSuccess) return fail(DSA_ERR_HIP, "dsa_device_errors: no current device");
  if (prev != device && hipSetDevice(device) != hipSuccess)
    return fail(DSA_ERR_HIP, "dsa_device_errors: cannot select device %d", device);
  int rc = hipDeviceSynchronize() == hipSuccess ? DSA_OK : fail(DSA_ERR_HIP, "dsa_device_errors: synchronise failed");
  if (rc == DSA_OK) rc = dsa::decode_read_errors(flags);
  if (prev != device) hipSetDevice(prev);
  return rc;
}

int dsa_set_debug(int on) {
  const int prev = dsa::debug_on() ? 1 : 0;
  dsa::g_debug = on ? 1 : 0;
  return prev;
}

int dsa_topk_plan(int B, int S, int T, int64_t* wave_rows, int64_t* block_rows) {
  if (B < 0 || S < 0 || T < 0 || !wave_rows || !block_rows) return DSA_ERR_SHAPE;
  dsa::topk_plan(B, S, T, wave_rows, block_rows);
  return DSA_OK;
}

int dsa_check_idx(const int32_t* idx, int64_t count, int64_t n_rows, int64_t* first_bad) {
  if (first_bad) *first_bad = -1;
  if (count < 0 || n_rows < 0) return DSA_ERR_SHAPE;
  if (count > 0 && !idx) return DSA_ERR_NULL;
  for (int64_t i = 0; i < count; ++i) {
    const int32_t v = idx[i];
    if (v < -1 || (int64_t)v >= n_rows) {
      if (first_bad) *first_bad = i;
      return DSA_ERR_INDEX;
    }
  }
  return DSA_OK;
}

// dsa_index_scores with an optional candidate mask: argument checks, then the launch
static int index_scores_impl(const char* who, const void* q_idx, const void* k_idx, int64_t k_batch_stride,
                             const void* w, float w_scale, int dtype, int B, int S, int T, int H_I, int D_I,
                             int start_pos, int ratio, float* scores, const dsa::CandMask& cm, hipStream_t st) {
  if (dtype != DSA_F32 && dtype != DSA_BF16) return fail(DSA_ERR_DTYPE, "%s: dtype %d", who, dtype);
  if (B < 0 || S < 0 || T < 0 || H_I <= 0 || D_I <= 0 || start_pos < 0 || ratio <= 0)
    return fail(DSA_ERR_SHAPE, "%s: bad sizes B=%d S=%d T=%d H_I=%d D_I=%d start_pos=%d ratio=%d", who, B, S, T, H_I,
                D_I, start_pos, ratio);
  if ((int64_t)T > ((int64_t)start_pos + S) / ratio)
    return fail(DSA_ERR_SHAPE, "%s: T=%d exceeds (start_pos+S)/ratio=%lld", who, T,
                (long long)(((int64_t)start_pos + S) / ratio));
  if (H_I > 64) return fail(DSA_ERR_UNSUPPORTED, "%s: H_I=%d > 64", who, H_I);
  if (B == 0 || S == 0 || T == 0) return DSA_OK;
  if (!q_idx || !k_idx || !w || !scores) return fail(DSA_ERR_NULL, "%s: NULL tensor pointer", who);
  if (k_batch_stride < (int64_t)T * D_I)
    return fail(DSA_ERR_SHAPE, "%s: k_batch_stride %lld < T*D_I", who, (long long)k_batch_stride);
  if (dtype == DSA_BF16 && (((uintptr_t)q_idx | (uintptr_t)k_idx) & 15))
    return fail(DSA_ERR_SHAPE, "%s: q_idx and k_idx must be 16-byte aligned", who);
  if (dtype == DSA_BF16 && (k_batch_stride % 8))
    return fail(DSA_ERR_SHAPE, "%s: k_batch_stride must be a multiple of 8 elements", who);
  return dsa::index_scores_launch(q_idx, k_idx, k_batch_stride, w, w_scale, dtype, B, S, T, H_I, D_I, start_pos,
                                  ratio, scores, cm, st);
}

int dsa_index_scores(const void* q_idx, const void* k_idx, int64_t k_batch_stride, const void* w, float w_scale,
                     int dtype, int B, int S, int T, int H_I, int D_I, int start_pos, int ratio, float* scores,
                     dsa_stream_t stream) {
  dsa::Entry entry_;
  return index_scores_impl("dsa_index_scores", q_idx, k_idx, k_batch_stride, w, w_scale, dtype, B, S, T, H_I, D_I,
                           start_pos, ratio, scores, dsa::CandMask{nullptr, 0, 0}, (hipStream_t)stream);
}

// the candidate mask of a call: checked, with the block size as its log2
static int cand_mask(const dsa_candidates* cand, int T, dsa::CandMask* out, const char* who) {
  *out = dsa::CandMask{nullptr, 0, 0};
  if (!cand) return DSA_OK;
  if (!cand->bits) return fail(DSA_ERR_NULL, "%s: candidate bits NULL", who);
  const int bs = cand->block_size;
  if (bs <= 0 || (bs & (bs - 1)))
    return fail(DSA_ERR_SHAPE, "%s: candidate block size %d is not a power of two", who, bs);
  const int64_t words = (((int64_t)T + bs - 1) / bs + 31) / 32;
  if (cand->ld_bits < words)
    return fail(DSA_ERR_SHAPE, "%s: candidate rows of %lld words, %lld needed", who, (long long)cand->ld_bits,
                (long long)words);
  *out = dsa::CandMask{cand->bits, cand->ld_bits, __builtin_ctz(bs)};
  return DSA_OK;
}

int dsa_index_scores_masked(const void* q_idx, const void* k_idx, int64_t k_batch_stride, const void* w,
                            float w_scale, int dtype, int B, int S, int T, int H_I, int D_I, int start_pos, int ratio,
                            const dsa_candidates* cand, float* scores, dsa_stream_t stream) {
  dsa::Entry entry_;
  dsa::CandMask cm;
  const int crc = cand_mask(cand, T, &cm, "dsa_index_scores_masked");
  if (crc) return crc;
  return index_scores_impl("dsa_index_scores_masked", q_idx, k_idx, k_batch_stride, w, w_scale, dtype, B, S, T, H_I,
                           D_I, start_pos, ratio, scores, cm, (hipStream_t)stream);
}

int dsa_candidate_blocks(const float* scores, int B, int S, int T, int start_pos, int ratio, int block_size,
                         int n_blocks, uint32_t* bits, int64_t ld_bits, dsa_stream_t stream) {
  dsa::Entry entry_;
  if (B < 0 || S < 0 || T < 0 || start_pos < 0 || ratio <= 0 || n_blocks <= 0)
    return fail(DSA_ERR_SHAPE, "dsa_candidate_blocks: bad sizes B=%d S=%d T=%d n_blocks=%d", B, S, T, n_blocks);
  if (block_size <= 0 || (block_size & (block_size - 1)))
    return fail(DSA_ERR_SHAPE, "dsa_candidate_blocks: block size %d is not a power of two", block_size);
  const int64_t words = (((int64_t)T + block_size - 1) / block_size + 31) / 32;
  if (ld_bits < words)
    return fail(DSA_ERR_SHAPE, "dsa_candidate_blocks: rows of %lld words, %lld needed", (long long)ld_bits,
                (long long)words);
  if (B == 0 || S == 0 || T == 0) return DSA_OK;
  if (!scores || !bits) return fail(DSA_ERR_NULL, "dsa_candidate_blocks: NULL pointer");
  return dsa::candidate_blocks_launch(scores, B, S, T, start_pos, ratio, __builtin_ctz(block_size), n_blocks, bits,
                                      ld_bits, (hipStream_t)stream);
}

int dsa_index_scores_mxfp4(const uint8_t* q_idx, const uint8_t* q_scale, const uint8_t* k_idx,
                           const uint8_t* k_scale, int64_t k_batch_rows, const void* w, float w_scale, int B, int S,
                           int T, int H_I, int D_I, int start_pos, int ratio, const dsa_candidates* cand,
                           float* scores, dsa_stream_t stream) {
  dsa::Entry entry_;
  dsa::CandMask cm;
  const int crc = cand_mask(cand, T, &cm, "dsa_index_scores_mxfp4");
  if (crc) return crc;
  if (B < 0 || S < 0 || T < 0 || H_I <= 0 || D_I <= 0 || start_pos < 0 || ratio <= 0)
    return fail(DSA_ERR_SHAPE, "dsa_index_scores_mxfp4: bad sizes B=%d S=%d T=%d H_I=%d D_I=%d start_pos=%d ratio=%d",
                B, S, T, H_I, D_I, start_pos, ratio);
  if ((int64_t)T > ((int64_t)start_pos + S) / ratio)
    return fail(DSA_ERR_SHAPE, "dsa_index_scores_mxfp4: T=%d exceeds (start_pos+S)/ratio=%lld", T,
                (long long)(((int64_t)start_pos + S) / ratio));
  if (H_I > 64) return fail(DSA_ERR_UNSUPPORTED, "dsa_index_scores_mxfp4: H_I=%d > 64", H_I);
  if (D_I != 64 && D_I != 128 && D_I != 256)
    return fail(DSA_ERR_UNSUPPORTED, "dsa_index_scores_mxfp4: D_I=%d not in {64, 128, 256}", D_I);
  if (B == 0 || S == 0 || T == 0) return DSA_OK;
  if (!q_idx || !q_scale || !k_idx || !k_scale || !w || !scores)
    return fail(DSA_ERR_NULL, "dsa_index_scores_mxfp4: NULL tensor pointer");
  if (k_batch_rows < T) return fail(DSA_ERR_SHAPE, "dsa_index_scores_mxfp4: k_batch_rows %lld < T", (long long)k_batch_rows);
  if (((uintptr_t)q_idx | (uintptr_t)k_idx) & 15)
    return fail(DSA_ERR_SHAPE, "dsa_index_scores_mxfp4: q_idx and k_idx must be 16-byte aligned");
  return dsa::index_scores_mxfp4_launch(q_idx, q_scale, k_idx, k_scale, k_batch_rows, w, w_scale, B, S, T, H_I, D_I,
                                        start_pos, ratio, scores, cm, (hipStream_t)stream);
}

size_t dsa_topk_workspace_size(int B, int S, int T, int index_topk) {
  if (B <= 0 || S <= 0 || T <= 0 || index_topk <= 0) return 0;
  const int K = index_topk < T ? index_topk : T;
  const size_t p = dsa::topk_split_bytes(B, S, T, K);
  return p ? dsa::kWsHeaderBytes + p : 0;
}

// the workspace past its header when it holds the split select's candidates, else null
static void* topk_payload(int B, int S, int T, int K, void* workspace, size_t workspace_bytes) {
  const size_t p = dsa::topk_split_bytes(B, S, T, K);
  if (!p || !workspace || workspace_bytes < dsa::kWsHeaderBytes + p) return nullptr;
  return (char*)workspace + dsa::kWsHeaderBytes;
}

int dsa_topk(const float* scores, int B, int S, int T, int index_topk, int start_pos, int ratio, int offset,
             int32_t* idx, int64_t ld_idx, void* workspace, size_t workspace_bytes, dsa_stream_t stream) {
  dsa::Entry entry_;
  if (B < 0 || S < 0 || T < 0 || index_topk < 0 || start_pos < 0 || ratio <= 0 || offset < 0)
    return fail(DSA_ERR_SHAPE, "dsa_topk: bad sizes B=%d S=%d T=%d index_topk=%d start_pos=%d ratio=%d offset=%d", B,
                S, T, index_topk, start_pos, ratio, offset);
  const int K = index_topk < T ? index_topk : T;
  if (ld_idx < K) return fail(DSA_ERR_SHAPE, "dsa_topk: ld_idx %lld < K=%d", (long long)ld_idx, K);
  if (B == 0 || S == 0 || K == 0) return DSA_OK;
  if (!scores || !idx) return fail(DSA_ERR_NULL, "dsa_topk: NULL pointer");
  return dsa::topk_launch(scores, B, S, T, K, start_pos, ratio, offset, idx, ld_idx, 0, 0,
                          topk_payload(B, S, T, K, workspace, workspace_bytes), (hipStream_t)stream);
}

int dsa_window_cols(int S, int start_pos, int W) {
  if (S < 0 || start_pos < 0 || W <= 0) return fail(DSA_ERR_SHAPE, "dsa_window_cols: S=%d start_pos=%d W=%d", S, start_pos, W);
  if (start_pos == 0) return S < W ? S : W;
  if (S != 1) return fail(DSA_ERR_UNSUPPORTED, "window rows with start_pos > 0 are defined for one query (S=%d)", S);
  return W;
}

int dsa_window_idx(int B, int S, int start_pos, int W, int32_t* idx, int64_t ld_idx, dsa_stream_t stream) {
  dsa::Entry entry_;
  if (B < 0) return fail(DSA_ERR_SHAPE, "dsa_window_idx: B=%d", B);
  const int Wc = dsa_window_cols(S, start_pos, W);
  if (Wc < 0) return Wc;
  if (ld_idx < Wc) return fail(DSA_ERR_SHAPE, "dsa_window_idx: ld_idx %lld < %d columns", (long long)ld_idx, Wc);
  if (B == 0 || S == 0 || Wc == 0) return DSA_OK;
  if (!idx) return fail(DSA_ERR_NULL, "dsa_window_idx: NULL idx");
  return dsa::window_idx_launch(B, S, start_pos, W, Wc, idx, ld_idx, (hipStream_t)stream);
}

int dsa_select(const float* scores, int B, int S, int T, int index_topk, int start_pos, int ratio, int W,
               int offset, int32_t* idx, int64_t ld_idx, void* workspace, size_t workspace_bytes,
               dsa_stream_t stream) {
  dsa::Entry entry_;
  if (B < 0 || S < 0 || T < 0 || index_topk < 0 || start_pos < 0 || ratio <= 0 || offset < 0)
    return fail(DSA_ERR_SHAPE, "dsa_select: bad sizes B=%d S=%d T=%d index_topk=%d start_pos=%d ratio=%d offset=%d",
                B, S, T, index_topk, start_pos, ratio, offset);
  const int Wc = dsa_window_cols(S, start_pos, W);
  if (Wc < 0) return Wc;
  const int K = index_topk < T ? index_topk : T;
  if (ld_idx < (int64_t)Wc + K)
    return fail(DSA_ERR_SHAPE, "dsa_select: ld_idx %lld < Wc + K = %d", (long long)ld_idx, Wc + K);
  if (B == 0 || S == 0 || Wc + K == 0) return DSA_OK;
  if (!idx || (K > 0 && !scores)) return fail(DSA_ERR_NULL, "dsa_select: NULL pointer");
  if (K == 0) return dsa::window_idx_launch(B, S, start_pos, W, Wc, idx, ld_idx, (hipStream_t)stream);
  return dsa::topk_launch(scores, B, S, T, K, start_pos, ratio, offset, idx, ld_idx, W, Wc,
                          topk_payload(B, S, T, K, workspace, workspace_bytes), (hipStream_t)stream);
}

size_t dsa_sparse_attn_workspace_size(int dtype, int B, int S, int H, int D, int L) {
  if (dtype != DSA_BF16 || B <= 0 || S <= 0 || H <= 0 || D <= 0 || L <= 0) return 0;
  // the size covers every kernel the call may pick for this shape (dense or fp4 compressed rows)
  const size_t a = dsa::sparse_attn_bf16_workspace(B, S, H, D, L, false);
  const size_t b = dsa::sparse_attn_bf16_workspace(B, S, H, D, L, true);
  return a > b ? a : b;
}

size_t dsa_step_workspace_size(int dtype, int B, int S, int H, int D, int T, int index_topk, int start_pos,
                               int W) {
  if (B <= 0 || S <= 0 || T < 0 || index_topk < 0) return 0;
  const int Wc = dsa_window_cols(S, start_pos, W);
  if (Wc < 0) return 0;
  const int K = index_topk < T ? index_topk : T;
  const size_t a = dsa_sparse_attn_workspace_size(dtype, B, S, H, D, Wc + K);
  const size_t t = dsa_topk_workspace_size(B, S, T, index_topk);
  return a > t ? a : t;
}

static int check_src(const dsa_kv_src* s, const char* name, int dtype, int D, int B, bool required) {
  if (!s) return required ? fail(DSA_ERR_NULL, "dsa_sparse_attn: %s source is NULL", name) : DSA_OK;
  if (s->n_rows < 0) return fail(DSA_ERR_SHAPE, "dsa_sparse_attn: %s n_rows %lld", name, (long long)s->n_rows);
  if (s->n_rows == 0) return DSA_OK;
  if (!s->rows) return fail(DSA_ERR_NULL, "dsa_sparse_attn: %s rows NULL with n_rows %lld", name, (long long)s->n_rows);
  if (s->format == DSA_KV_DENSE) {
    if (s->row_stride < D || (B > 1 && s->batch_stride < s->n_rows * s->row_stride - (s->row_stride - D)))
      return fail(DSA_ERR_SHAPE, "dsa_sparse_attn: %s strides too small for D=%d", name, D);
    if (dtype == DSA_BF16 && (((uintptr_t)s->rows & 15) || (s->row_stride % 8) || (s->batch_stride % 8)))
      return fail(DSA_ERR_SHAPE, "dsa_sparse_attn: bf16 %s rows need 16-byte alignment of every row", name);
  } else if (s->format == DSA_KV_FP4_E4M3_G16) {
    if (dtype != DSA_BF16) return fail(DSA_ERR_DTYPE, "dsa_sparse_attn: fp4 %s rows need dtype bf16", name);
    if (!s->scales) return fail(DSA_ERR_NULL, "dsa_sparse_attn: fp4 %s scales NULL", name);
    if (D % 16) return fail(DSA_ERR_SHAPE, "dsa_sparse_attn: fp4 rows need D %% 16 == 0");
    if (s->row_stride < D / 2 || s->scale_row_stride < D / 16)
      return fail(DSA_ERR_SHAPE, "dsa_sparse_attn: fp4 %s strides too small", name);
    if (((uintptr_t)s->rows & 3) || (s->row_stride & 3) || (s->batch_stride & 3))
      return fail(DSA_ERR_SHAPE, "dsa_sparse_attn: fp4 %s rows need 4-byte alignment", name);
  } else {
    return fail(DSA_ERR_DTYPE, "dsa_sparse_attn: %s format %d", name, s->format);
  }
  return DSA_OK;
}

// dsa_sparse_attn, with the output's inverse rotary embedding when rope is set
static int sparse_attn_impl(const void* q, const dsa_kv_src* win, const dsa_kv_src* comp, const float* sink,
                            const int32_t* idx, int L, float scale, void* o, int dtype, int B, int S, int H, int D,
                            void* workspace, size_t workspace_bytes, const float* rope, int rope_dim,
                            dsa_stream_t stream) {
  if (dtype != DSA_F32 && dtype != DSA_BF16) return fail(DSA_ERR_DTYPE, "dsa_sparse_attn: dtype %d", dtype);
  if (B < 0 || S < 0 || H <= 0 || D <= 0 || L < 0)
    return fail(DSA_ERR_SHAPE, "dsa_sparse_attn: bad sizes B=%d S=%d H=%d D=%d L=%d", B, S, H, D, L);
  int rc = check_src(win, "window", dtype, D, B, true);
  if (rc) return rc;
  rc = check_src(comp, "compressed", dtype, D, B, false);
  if (rc) return rc;
  if (win->format != DSA_KV_DENSE) return fail(DSA_ERR_DTYPE, "dsa_sparse_attn: window rows must be dense");
  if (dtype == DSA_BF16) {
    if (D != 64 && D != 128 && D != 256 && D != 512)
      return fail(DSA_ERR_UNSUPPORTED, "dsa_sparse_attn: bf16 head_dim %d not in {64,128,256,512}", D);
    if (H > (D == 512 ? 64 : 128)) return fail(DSA_ERR_UNSUPPORTED, "dsa_sparse_attn: H=%d too large for D=%d", H, D);
  } else {
    if (D > 512 || H > 64) return fail(DSA_ERR_UNSUPPORTED, "dsa_sparse_attn: fp32 path takes D<=512, H<=64");
    if (comp && comp->n_rows > 0 && comp->format != DSA_KV_DENSE)
      return fail(DSA_ERR_DTYPE, "dsa_sparse_attn: fp32 path takes dense rows only");
  }
  if (B == 0 || S == 0) return DSA_OK;
  if (!q || !sink || !o || (L > 0 && !idx)) return fail(DSA_ERR_NULL, "dsa_sparse_attn: NULL tensor pointer");
  if (dtype == DSA_BF16 && (((uintptr_t)q | (uintptr_t)o) & 15))
    return fail(DSA_ERR_SHAPE, "dsa_sparse_attn: q and o must be 16-byte aligned");
  const size_t need = dsa_sparse_attn_workspace_size(dtype, B, S, H, D, L);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(DSA_ERR_WORKSPACE, "dsa_sparse_attn: workspace of %zu bytes needed, %zu given", need, workspace_bytes);
  if (L > 0 && dsa::debug_on()) {
    const int64_t n_total = win->n_rows + ((comp && comp->n_rows > 0) ? comp->n_rows : 0);
    const int rc = dsa::debug_check_idx(idx, (int64_t)B * S * L, n_total, (hipStream_t)stream);
    if (rc) return rc;
  }
  dsa_kv_src empty{};
  const dsa_kv_src* cs = (comp && comp->n_rows > 0) ? comp : &empty;
  if (dtype == DSA_BF16)
    return dsa::sparse_attn_bf16_launch(q, win, cs, sink, idx, L, scale, o, B, S, H, D, workspace, rope, rope_dim,
                                        (hipStream_t)stream);
  rc = dsa::sparse_attn_f32_launch(q, win, cs, sink, idx, L, scale, o, B, S, H, D, (hipStream_t)stream);
  if (rc || !rope) return rc;
  return dsa::rope_inverse_launch(o, DSA_F32, B, S, H, D, rope, rope_dim, (hipStream_t)stream);
}

int dsa_sparse_attn(const void* q, const dsa_kv_src* win, const dsa_kv_src* comp, const float* sink,
                    const int32_t* idx, int L, float scale, void* o, int dtype, int B, int S, int H, int D,
                    void* workspace, size_t workspace_bytes, dsa_stream_t stream) {
  dsa::Entry entry_;
  return sparse_attn_impl(q, win, comp, sink, idx, L, scale, o, dtype, B, S, H, D, workspace, workspace_bytes,
                          nullptr, 0, stream);
}

static int check_rope(const float* freqs, int rope_dim, int D, const char* who) {
  if (!freqs) return fail(DSA_ERR_NULL, "%s: NULL rotary table", who);
  if (rope_dim <= 0 || rope_dim > D || rope_dim % 16)
    return fail(DSA_ERR_SHAPE, "%s: rope_dim %d must be a multiple of 16 in (0, D=%d]", who, rope_dim, D);
  if ((uintptr_t)freqs & 15) return fail(DSA_ERR_SHAPE, "%s: the rotary table must be 16-byte aligned", who);
  return DSA_OK;
}

int dsa_sparse_attn_rope(const void* q, const dsa_kv_src* win, const dsa_kv_src* comp, const float* sink,
                         const int32_t* idx, int L, float scale, void* o, int dtype, int B, int S, int H, int D,
                         const float* freqs, int rope_dim, void* workspace, size_t workspace_bytes,
                         dsa_stream_t stream) {
  dsa::Entry entry_;
  if (B > 0 && S > 0) {
    const int rc = check_rope(freqs, rope_dim, D, "dsa_sparse_attn_rope");
    if (rc) return rc;
  }
  return sparse_attn_impl(q, win, comp, sink, idx, L, scale, o, dtype, B, S, H, D, workspace, workspace_bytes, freqs,
                          rope_dim, stream);
}

int dsa_rope_inverse(void* o, int dtype, int B, int S, int H, int D, const float* freqs, int rope_dim,
                     dsa_stream_t stream) {
  dsa::Entry entry_;
  if (dtype != DSA_F32 && dtype != DSA_BF16) return fail(DSA_ERR_DTYPE, "dsa_rope_inverse: dtype %d", dtype);
  if (B < 0 || S < 0 || H <= 0 || D <= 0) return fail(DSA_ERR_SHAPE, "dsa_rope_inverse: bad sizes");
  if (B == 0 || S == 0) return DSA_OK;
  int rc = check_rope(freqs, rope_dim, D, "dsa_rope_inverse");
  if (rc) return rc;
  if (!o) return fail(DSA_ERR_NULL, "dsa_rope_inverse: NULL output");
  return dsa::rope_inverse_launch(o, dtype, B, S, H, D, freqs, rope_dim, (hipStream_t)stream);
}

int dsa_compress_kv_write(const void* latent, int64_t latent_batch_stride, int B, int n, int D, const float* freqs,
                          int rope_dim, uint8_t* rows, int64_t rows_batch_stride, uint8_t* scales,
                          int64_t scales_batch_stride, int64_t row0, dsa_stream_t stream) {
  dsa::Entry entry_;
  if (B < 0 || n < 0 || D <= 0 || row0 < 0) return fail(DSA_ERR_SHAPE, "dsa_compress_kv_write: bad sizes");
  if (D % 16) return fail(DSA_ERR_SHAPE, "dsa_compress_kv_write: D=%d is not a multiple of 16", D);
  if (B == 0 || n == 0) return DSA_OK;
  int rc = check_rope(freqs, rope_dim, D, "dsa_compress_kv_write");
  if (rc) return rc;
  if (!latent || !rows || !scales) return fail(DSA_ERR_NULL, "dsa_compress_kv_write: NULL pointer");
  if (latent_batch_stride < (int64_t)n * D || rows_batch_stride < (row0 + n) * (int64_t)(D / 2) ||
      scales_batch_stride < (row0 + n) * (int64_t)(D / 16))
    return fail(DSA_ERR_SHAPE, "dsa_compress_kv_write: a batch stride is smaller than the rows it must hold");
  if (((uintptr_t)rows & 7) || (rows_batch_stride & 7))
    return fail(DSA_ERR_SHAPE, "dsa_compress_kv_write: cache rows must be 8-byte aligned");
  return dsa::compress_kv_write_launch(latent, latent_batch_stride, B, n, D, rope_dim, freqs, rows, rows_batch_stride,
                                       scales, scales_batch_stride, row0, (hipStream_t)stream);
}

int dsa_sparse_attn_select(const float* scores, int T, int index_topk, int start_pos, int ratio, int W,
                           const void* q, const dsa_kv_src* win, const dsa_kv_src* comp, const float* sink,
                           float scale, void* o, int dtype, int B, int S, int H, int D, int32_t* idx,
                           void* workspace, size_t workspace_bytes, dsa_stream_t stream) {
  dsa::Entry entry_;
  if (B < 0 || S < 0 || T < 0 || index_topk < 0 || start_pos < 0 || ratio <= 0)
    return fail(DSA_ERR_SHAPE, "dsa_sparse_attn_select: bad sizes B=%d S=%d T=%d index_topk=%d start_pos=%d ratio=%d",
                B, S, T, index_topk, start_pos, ratio);
  if (!win) return fail(DSA_ERR_NULL, "dsa_sparse_attn_select: window source missing");
  const int Wc = dsa_window_cols(S, start_pos, W);
  if (Wc < 0) return Wc;
  const int K = index_topk < T ? index_topk : T;
  const int L = Wc + K;
  if (B == 0 || S == 0) return DSA_OK;
  if (win->n_rows > 0x7FFFFFFF) return fail(DSA_ERR_SHAPE, "dsa_sparse_attn_select: window rows beyond 32-bit indices");
  const int offset = (int)win->n_rows;
  if (K > 0 && !scores) return fail(DSA_ERR_NULL, "dsa_sparse_attn_select: NULL scores");
  // one launch when the decode attention kernel can select the rows itself
  if (dtype == DSA_BF16 && K > 0 && T <= 2048 && q && sink && o && (((uintptr_t)q | (uintptr_t)o) & 15) == 0 &&
      win->rows && win->format == DSA_KV_DENSE) {
    int rc = check_src(win, "window", dtype, D, B, true);
    if (rc) return rc;
    rc = check_src(comp, "compressed", dtype, D, B, false);
    if (rc) return rc;
    const size_t need = dsa_step_workspace_size(dtype, B, S, H, D, T, index_topk, start_pos, W);
    if (need > 0 && (!workspace || workspace_bytes < need))
      return fail(DSA_ERR_WORKSPACE, "dsa_sparse_attn_select: workspace of %zu bytes needed, %zu given", need,
                  workspace_bytes);
    dsa::DecSelect sel{scores, T, K, start_pos, ratio, W, Wc, offset, idx, (int64_t)L};
    dsa_kv_src empty{};
    const dsa_kv_src* cs = (comp && comp->n_rows > 0) ? comp : &empty;
    rc = dsa::sparse_attn_bf16_select_launch(q, win, cs, sink, &sel, nullptr, L, scale, o, B, S, H, D, workspace,
                                             (hipStream_t)stream);
    if (rc != 0) return rc < 0 ? rc : DSA_OK;
  }
  // otherwise: the index rows into idx, then the attention over them
  if (!idx) return fail(DSA_ERR_NULL, "dsa_sparse_attn_select: idx needed for this shape");
  const size_t need = dsa_step_workspace_size(dtype, B, S, H, D, T, index_topk, start_pos, W);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(DSA_ERR_WORKSPACE, "dsa_sparse_attn_select: workspace of %zu bytes needed, %zu given", need,
                workspace_bytes);
  int rc = dsa_select(scores, B, S, T, index_topk, start_pos, ratio, W, offset, idx, L, workspace, workspace_bytes,
                      stream);
  if (rc) return rc;
  return dsa_sparse_attn(q, win, comp, sink, idx, L, scale, o, dtype, B, S, H, D, workspace, workspace_bytes, stream);
}

int dsa_sparse_attn_step(const void* q_idx, const void* k_idx, int64_t k_batch_stride, const void* w, float w_scale,
                         int H_I, int D_I, int T, int index_topk, int start_pos, int ratio, int W, const void* q,
                         const dsa_kv_src* win, const dsa_kv_src* comp, const float* sink, float scale, void* o,
                         int dtype, int B, int S, int H, int D, float* scores, int32_t* idx, void* workspace,
                         size_t workspace_bytes, dsa_stream_t stream) {
  dsa::Entry entry_;
  if (dtype != DSA_F32 && dtype != DSA_BF16) return fail(DSA_ERR_DTYPE, "dsa_sparse_attn_step: dtype %d", dtype);
  if (B < 0 || S < 0 || T < 0 || H_I <= 0 || D_I <= 0 || index_topk < 0 || start_pos < 0 || ratio <= 0)
    return fail(DSA_ERR_SHAPE,
                "dsa_sparse_attn_step: bad sizes B=%d S=%d T=%d H_I=%d D_I=%d index_topk=%d start_pos=%d ratio=%d", B,
                S, T, H_I, D_I, index_topk, start_pos, ratio);
  if (!win) return fail(DSA_ERR_NULL, "dsa_sparse_attn_step: window source missing");
  const int Wc = dsa_window_cols(S, start_pos, W);
  if (Wc < 0) return Wc;
  if (B == 0 || S == 0) return DSA_OK;
  const int K = index_topk < T ? index_topk : T;
  const int L = Wc + K;
  // one launch: the decode attention kernel scores, selects and attends (index head dim 128)
  if (dtype == DSA_BF16 && K > 0 && T <= 2048 && D_I == 128 && H_I <= 64 && q_idx && k_idx && w && scores && q &&
      sink && o && (((uintptr_t)q | (uintptr_t)o | (uintptr_t)q_idx | (uintptr_t)k_idx) & 15) == 0 &&
      k_batch_stride >= (int64_t)T * D_I && k_batch_stride % 8 == 0 &&
      (int64_t)T <= ((int64_t)start_pos + S) / ratio && win->rows && win->format == DSA_KV_DENSE &&
      win->n_rows <= 0x7FFFFFFF) {
    int rc = check_src(win, "window", dtype, D, B, true);
    if (rc) return rc;
    rc = check_src(comp, "compressed", dtype, D, B, false);
    if (rc) return rc;
    const size_t need = dsa_step_workspace_size(dtype, B, S, H, D, T, index_topk, start_pos, W);
    if (need > 0 && (!workspace || workspace_bytes < need))
      return fail(DSA_ERR_WORKSPACE, "dsa_sparse_attn_step: workspace of %zu bytes needed, %zu given", need,
                  workspace_bytes);
    dsa::DecSelect sel{scores, T, K, start_pos, ratio, W, Wc, (int)win->n_rows, idx, (int64_t)L};
    dsa::DecIndex ix{(const __bf16*)q_idx, (const __bf16*)k_idx, k_batch_stride, (const __bf16*)w, w_scale, H_I,
                     scores};
    dsa_kv_src empty{};
    const dsa_kv_src* cs = (comp && comp->n_rows > 0) ? comp : &empty;
    rc = dsa::sparse_attn_bf16_select_launch(q, win, cs, sink, &sel, &ix, L, scale, o, B, S, H, D, workspace,
                                             (hipStream_t)stream);
    if (rc != 0) return rc < 0 ? rc : DSA_OK;
  }
  // otherwise: the index scores, then the index rows and the attention (the workspace is checked
  // before anything is launched)
  const size_t need = dsa_step_workspace_size(dtype, B, S, H, D, T, index_topk, start_pos, W);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(DSA_ERR_WORKSPACE, "dsa_sparse_attn_step: workspace of %zu bytes needed, %zu given", need,
                workspace_bytes);
  int rc = dsa_index_scores(q_idx, k_idx, k_batch_stride, w, w_scale, dtype, B, S, T, H_I, D_I, start_pos, ratio,
                            scores, stream);
  if (rc) return rc;
  return dsa_sparse_attn_select(scores, T, index_topk, start_pos, ratio, W, q, win, comp, sink, scale, o, dtype, B, S,
                                H, D, idx, workspace, workspace_bytes, stream);
}

int dsa_sparse_attn_step_noalloc(const void* q_idx, const void* k_idx, int64_t k_batch_stride, const void* w,
                                 float w_scale, int H_I, int D_I, int T, int index_topk, int start_pos, int ratio,
                                 int W, const void* q, const dsa_kv_src* win, const dsa_kv_src* comp,
                                 const float* sink, float scale, void* o, int dtype, int B, int S, int H, int D,
                                 float* scores, int32_t* idx, dsa_stream_t stream) {
  dsa::Entry entry_;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= dsa::kMaxDevices)
    return fail(DSA_ERR_HIP, "dsa_sparse_attn_step_noalloc: no usable current HIP device");
  const dsa::DeviceState& ds = dsa::g_dev[dev];
  if (!ds.ready || !ds.scratch)
    return fail(DSA_ERR_STATE, "dsa_sparse_attn_step_noalloc: call dsa_init(%d) first", dev);
  if (B < 0 || S < 0 || T < 0 || index_topk < 0 || start_pos < 0 || W <= 0)
    return fail(DSA_ERR_SHAPE, "dsa_sparse_attn_step_noalloc: bad sizes B=%d S=%d T=%d index_topk=%d", B, S, T,
                index_topk);
  const int Wc = dsa_window_cols(S, start_pos, W);
  if (Wc < 0) return Wc;
  const size_t need = dsa_step_workspace_size(dtype, B, S, H, D, T, index_topk, start_pos, W);
  const size_t have = dsa::scratch_bytes();
  if (need > have)
    return fail(DSA_ERR_WORKSPACE,
                "dsa_sparse_attn_step_noalloc: this shape needs %zu bytes of scratch, the fixed array holds %zu "
                "(use dsa_sparse_attn_step with a workspace)",
                need, have);
  return dsa_sparse_attn_step(q_idx, k_idx, k_batch_stride, w, w_scale, H_I, D_I, T, index_topk, start_pos, ratio, W,
                              q, win, comp, sink, scale, o, dtype, B, S, H, D, scores, idx, ds.scratch, have, stream);
}

int dsa_sparse_attn_step_mxfp4(const uint8_t* q_idx, const uint8_t* q_scale, const uint8_t* k_idx,
                               const uint8_t* k_scale, int64_t k_batch_rows, const void* w, float w_scale, int H_I,
                               int D_I, int T, int index_topk, int start_pos, int ratio, int W, const void* q,
                               const dsa_kv_src* win, const dsa_kv_src* comp, const float* sink, float scale,
                               void* o, int dtype, int B, int S, int H, int D, float* scores, int32_t* idx,
                               void* workspace, size_t workspace_bytes, dsa_stream_t stream) {
  dsa::Entry entry_;
  if (dtype != DSA_BF16) return fail(DSA_ERR_DTYPE, "dsa_sparse_attn_step_mxfp4: the attention dtype must be bf16");
  if (!win) return fail(DSA_ERR_NULL, "dsa_sparse_attn_step_mxfp4: window source missing");
  const int Wc = dsa_window_cols(S, start_pos, W);
  if (Wc < 0) return Wc;
  // validate the attention half before anything is launched
  if (B < 0 || S < 0 || T < 0 || index_topk < 0 || start_pos < 0 || ratio <= 0)
    return fail(DSA_ERR_SHAPE, "dsa_sparse_attn_step_mxfp4: bad sizes B=%d S=%d T=%d index_topk=%d", B, S, T,
                index_topk);
  if (B == 0 || S == 0) return DSA_OK;
  const size_t need = dsa_step_workspace_size(dtype, B, S, H, D, T, index_topk, start_pos, W);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(DSA_ERR_WORKSPACE, "dsa_sparse_attn_step_mxfp4: workspace of %zu bytes needed, %zu given", need,
                workspace_bytes);
  int rc = dsa_index_scores_mxfp4(q_idx, q_scale, k_idx, k_scale, k_batch_rows, w, w_scale, B, S, T, H_I, D_I,
                                  start_pos, ratio, nullptr, scores, stream);
  if (rc) return rc;
  return dsa_sparse_attn_select(scores, T, index_topk, start_pos, ratio, W, q, win, comp, sink, scale, o, dtype, B, S,
                                H, D, idx, workspace, workspace_bytes, stream);
}

}  // extern "C"
