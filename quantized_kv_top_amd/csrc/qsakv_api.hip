// C ABI layer: host-side validation and dispatch.  Every check runs before
// any HIP call; kernels are enqueued on the caller's stream and nothing here
// synchronizes or allocates.
#include <cmath>
#include <cstdint>
#include <cstring>
#include <limits>
#include <mutex>

#include "qsakv.h"
#include "qsakv_internal.h"

// Split-K scratch of qsa_sparse_attn_decode_noalloc.  Every GPU the library
// runs on holds its own copy until the process ends.  In host code the name
// is only a stand-in for the symbol: kernels and copies use the device
// address that hipGetSymbolAddress returns for the current GPU.
static __device__ __align__(256) unsigned char scratch[QSA_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local int32_t g_last_hip_error = 0;

// Device address of `scratch` on each GPU, looked up once per device (with
// that device current) on the first no-alloc call that runs there.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

hipError_t scratch_ptr(hipStream_t stream, void** out) {
  int dev = 0;
  hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    int cur = 0;
    e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    const hipError_t back = cur != dev ? hipSetDevice(cur) : hipSuccess;
    if (e != hipSuccess) return e;
    if (back != hipSuccess) return back;
    if (!ptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

constexpr int64_t kI64Max = std::numeric_limits<int64_t>::max();

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool is_pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }

int log2i(int64_t x) {
  int l = 0;
  while ((int64_t(1) << l) < x) ++l;
  return l;
}

// a * b without signed overflow; false if it would exceed kI64Max
bool mul_ok(int64_t a, int64_t b, int64_t* out) {
  if (a < 0 || b < 0) return false;
  if (a != 0 && b > kI64Max / a) return false;
  *out = a * b;
  return true;
}

bool scale_ok(float s) { return std::isfinite(s) && s >= std::numeric_limits<float>::min(); }

// The E4M3 converter's float32 quotient, on the host (IEEE binary32).
float div_f32(float a, float b) {
  volatile float q = a / b;
  return q;
}

// Smallest non-negative float32 bit pattern u (as |x|) whose quotient
// y = fl32(|x| / scale) satisfies the predicate; y is non-decreasing in u
// (division by a positive number and round-to-nearest are monotone), and
// u = +inf satisfies every predicate, so a binary search is exact.
enum CalibPred { kCalibSat, kCalibSub, kCalibNorm };
uint32_t calib_threshold(float scale, CalibPred pred) {
  uint32_t lo = 0, hi = 0x7F800000u;
  while (lo < hi) {
    const uint32_t mid = lo + (hi - lo) / 2;
    float v;
    std::memcpy(&v, &mid, 4);
    const float y = div_f32(v, scale);
    const bool ok = pred == kCalibSat ? y > 448.0f
                    : pred == kCalibSub ? y >= 0x1p-9f
                                        : y >= 0x1p-6f;
    if (ok)
      hi = mid;
    else
      lo = mid + 1;
  }
  return lo;
}

int64_t row_bytes(int kind, int64_t d) {
  switch (kind) {
    case QKV_CACHE_INT8: return d;
    case QKV_CACHE_INT8_INLINE: return d + 4;
    case QKV_CACHE_E4M3: return d;
    case QKV_CACHE_NVFP4: return d / 2;
    default: return 2 * d;
  }
}

// Checks shared by every call that touches a cache.
qkv_status check_cache(const qkv_cache* c, bool need_data) {
  if (!c) return QKV_ERR_NULL;
  if (c->kind < QKV_CACHE_INT8 || c->kind > QKV_CACHE_NVFP4) return QKV_ERR_UNSUPPORTED;
  if (c->num_blocks <= 0 || c->num_kv_heads <= 0 || c->reserved != 0) return QKV_ERR_BAD_SHAPE;
  if (!is_pow2(c->block_size) || c->block_size > 1024) return QKV_ERR_BAD_SHAPE;
  if (c->head_dim != 128 && c->head_dim != 256) return QKV_ERR_UNSUPPORTED;
  int64_t slots, t;
  if (!mul_ok(c->num_blocks, c->block_size, &slots) || slots > INT32_MAX) return QKV_ERR_BAD_SHAPE;
  if (!mul_ok(slots, c->num_kv_heads, &t) || !mul_ok(t, row_bytes(c->kind, c->head_dim), &t))
    return QKV_ERR_BAD_SHAPE;
  if (need_data) {
    if (!c->k || !c->v) return QKV_ERR_NULL;
    const bool side = c->kind == QKV_CACHE_INT8 || c->kind == QKV_CACHE_NVFP4;
    if (side && !c->kv_scale) return QKV_ERR_NULL;
    const uintptr_t a = c->kind == QKV_CACHE_INT8_INLINE ? 4 : 16;
    if (!aligned(c->k, a) || !aligned(c->v, a)) return QKV_ERR_ALIGNMENT;
    if (side && !aligned(c->kv_scale, c->kind == QKV_CACHE_INT8 ? 8 : 16)) return QKV_ERR_ALIGNMENT;
  }
  if ((c->kind == QKV_CACHE_E4M3 || c->kind == QKV_CACHE_NVFP4) &&
      (!scale_ok(c->k_scale) || !scale_ok(c->v_scale)))
    return QKV_ERR_BAD_SCALE;
  return QKV_OK;
}

qkv_status finish(hipError_t e) {
  if (e != hipSuccess) {
    g_last_hip_error = (int32_t)e;
    return QKV_ERR_HIP;
  }
  return QKV_OK;
}

qkv_status check_args(const qkv_cache* c, const qsa_args* a) {
  if (!a) return QKV_ERR_NULL;
  // topk <= 2^30 keeps ceil(topk / P) * P and every partition's end within int32
  if (a->num_rows < 0 || a->num_q_heads <= 0 || a->num_seqs <= 0 || a->block_table_stride <= 0 ||
      a->topk <= 0 || a->topk > (1 << 30))
    return QKV_ERR_BAD_SHAPE;
  if (a->num_q_heads % c->num_kv_heads != 0) return QKV_ERR_BAD_SHAPE;
  const int group = a->num_q_heads / c->num_kv_heads;
  if (group > 16) return QKV_ERR_UNSUPPORTED;
  if (a->q_dtype != QKV_BF16 && a->q_dtype != QKV_FP16) return QKV_ERR_UNSUPPORTED;
  if (c->kind == QKV_CACHE_BF16 && a->q_dtype != QKV_BF16) return QKV_ERR_UNSUPPORTED;
  if (a->out_dtype != QKV_BF16 && a->out_dtype != QKV_FP16 && a->out_dtype != QKV_FP32)
    return QKV_ERR_UNSUPPORTED;
  // the softmax scale must be finite and positive (as the header states)
  if (!std::isfinite(a->sm_scale) || !(a->sm_scale > 0.f)) return QKV_ERR_BAD_SCALE;
  int64_t t;
  if (!mul_ok(a->num_rows, a->num_q_heads, &t) || t > INT32_MAX) return QKV_ERR_BAD_SHAPE;
  if (!mul_ok(a->num_rows, a->topk, &t) || t > INT32_MAX) return QKV_ERR_BAD_SHAPE;
  if (!mul_ok(a->num_seqs, a->block_table_stride, &t) || t > INT32_MAX) return QKV_ERR_BAD_SHAPE;
  if (a->num_rows == 0) return QKV_OK;
  if (!a->q || !a->out || !a->row_seq || !a->block_table || !a->topk_idx) return QKV_ERR_NULL;
  if (!aligned(a->q, 16) || !aligned(a->out, 16) || !aligned(a->row_seq, 4) ||
      !aligned(a->block_table, 4) || !aligned(a->topk_idx, 4) ||
      (a->lse && !aligned(a->lse, 4)))
    return QKV_ERR_ALIGNMENT;
  return QKV_OK;
}

qsakv::AttnParams make_params(const qkv_cache* c, const qsa_args* a, int32_t splits) {
  qsakv::AttnParams p{};
  p.q = a->q;
  p.row_seq = a->row_seq;
  p.block_table = a->block_table;
  p.topk_idx = a->topk_idx;
  p.out = a->out;
  p.lse = a->lse;
  p.k = static_cast<const uint8_t*>(c->k);
  p.v = static_cast<const uint8_t*>(c->v);
  p.kv_scale = c->kv_scale;
  p.sm_log2e = (float)((double)a->sm_scale * 1.4426950408889634);
  const bool layer_scales = c->kind == QKV_CACHE_E4M3 || c->kind == QKV_CACHE_NVFP4;
  p.k_scale = layer_scales ? c->k_scale : 1.f;
  p.v_scale = layer_scales ? c->v_scale : 1.f;
  p.q_dtype = a->q_dtype;
  p.out_dtype = a->out_dtype;
  p.num_rows = a->num_rows;
  p.num_q_heads = a->num_q_heads;
  p.num_kv_heads = c->num_kv_heads;
  p.group = a->num_q_heads / c->num_kv_heads;
  p.num_seqs = a->num_seqs;
  p.bt_stride = a->block_table_stride;
  p.topk = a->topk;
  p.num_blocks = c->num_blocks;
  p.log2_bs = log2i(c->block_size);
  p.num_splits = splits;
  p.chunk = (a->topk + splits - 1) / splits;
  return p;
}

// Workspace layout: [R*Hq*P*D fp32 partials | pad to 256 B]
// [R*Hq*P*2 fp32 (max, sum)].
struct WsLayout {
  int64_t o_bytes, ml_bytes;
};

bool ws_layout(int64_t rows, int64_t heads, int64_t d, int64_t splits, WsLayout* l) {
  if (rows < 0 || heads <= 0 || (d != 128 && d != 256) || splits < 1 || splits > 64) return false;
  int64_t n, rh;
  if (!mul_ok(rows, heads, &rh) || !mul_ok(rh, splits, &n)) return false;
  if (!mul_ok(n, d * 4, &l->o_bytes) || !mul_ok(n, 8, &l->ml_bytes)) return false;
  l->o_bytes = (l->o_bytes + 255) / 256 * 256;
  return l->o_bytes <= kI64Max - l->ml_bytes;
}

size_t ws_bytes(int64_t rows, int64_t heads, int64_t d, int64_t splits) {
  WsLayout l;
  if (!ws_layout(rows, heads, d, splits, &l) || splits == 1) return 0;
  return (size_t)(l.o_bytes + l.ml_bytes);
}

// Workspace of qsa_topk_select: segment lists' keys, then positions, each
// [num_rows][row_slots] and 256-B aligned.
struct TopkWs {
  int seg_len = 0;
  int64_t row_slots = 0, key_bytes = 0, bytes = 0;
};

bool topk_ws(int64_t rows, int64_t stride, int64_t k, TopkWs* w) {
  *w = TopkWs{};
  if (rows < 0 || stride < 0 || stride > (1 << 30) || k < 1 || k > INT32_MAX) return false;
  w->seg_len = qsakv::topk_segment_len(stride, (int32_t)k);
  if (w->seg_len == 0) return true;
  const int64_t segs = (stride + w->seg_len - 1) / w->seg_len;
  w->row_slots = (segs * k + 3) / 4 * 4;
  int64_t n;
  if (!mul_ok(rows, w->row_slots, &n) || !mul_ok(n, 4, &w->key_bytes)) return false;
  w->key_bytes = (w->key_bytes + 255) / 256 * 256;
  if (w->key_bytes > kI64Max / 2) return false;
  w->bytes = 2 * w->key_bytes;
  return true;
}

// Checks shared by the two split-K entry points (nothing launched).
qkv_status check_decode(const qkv_cache* cache, const qsa_args* args, int32_t num_splits) {
  qkv_status st = check_cache(cache, true);
  if (st != QKV_OK) return st;
  st = check_args(cache, args);
  if (st != QKV_OK) return st;
  if (num_splits < 1 || num_splits > 64) return QKV_ERR_UNSUPPORTED;
  int64_t items;
  if (!mul_ok((int64_t)args->num_rows * cache->num_kv_heads, num_splits, &items) ||
      items > INT32_MAX)
    return QKV_ERR_BAD_SHAPE;
  return QKV_OK;
}

// The split-K launches on a checked call: the partitions (into the
// workspace `ws`, unused when num_splits == 1), then the merge.
qkv_status run_decode(const qkv_cache* cache, const qsa_args* args, int32_t num_splits, char* ws,
                      hipStream_t s) {
  qsakv::AttnParams p = make_params(cache, args, num_splits);
  if (num_splits == 1)
    return finish(qsakv::launch_attn(cache->kind, cache->head_dim, p, s));
  WsLayout l;
  ws_layout(args->num_rows, args->num_q_heads, cache->head_dim, num_splits, &l);
  p.ws_o = reinterpret_cast<float*>(ws);
  p.ws_ml = reinterpret_cast<float*>(ws + l.o_bytes);
  const hipError_t e = qsakv::launch_attn(cache->kind, cache->head_dim, p, s);
  if (e != hipSuccess) return finish(e);
  return finish(qsakv::launch_merge(cache->head_dim, p, s));
}

}  // namespace

extern "C" {

qkv_status kv_quant_write(const qkv_cache* cache, const void* k_src, const void* v_src,
                          int32_t src_dtype, int64_t num_tokens, const int64_t* slot_mapping,
                          void* stream) {
  qkv_status st = check_cache(cache, true);
  if (st != QKV_OK) return st;
  if (num_tokens < 0) return QKV_ERR_BAD_SHAPE;
  if (src_dtype != QKV_FP32 && src_dtype != QKV_BF16 && src_dtype != QKV_FP16)
    return QKV_ERR_UNSUPPORTED;
  int64_t t;
  if (!mul_ok(num_tokens, (int64_t)cache->num_kv_heads * cache->head_dim * 4, &t))
    return QKV_ERR_BAD_SHAPE;
  if (num_tokens == 0) return QKV_OK;
  if (!k_src || !v_src || !slot_mapping) return QKV_ERR_NULL;
  if (!aligned(k_src, 16) || !aligned(v_src, 16) || !aligned(slot_mapping, 8))
    return QKV_ERR_ALIGNMENT;
  qsakv::WriteParams p{};
  p.k_src = k_src;
  p.v_src = v_src;
  p.slot_mapping = slot_mapping;
  p.k = static_cast<uint8_t*>(cache->k);
  p.v = static_cast<uint8_t*>(cache->v);
  p.kv_scale = cache->kv_scale;
  p.k_scale = cache->k_scale;
  p.v_scale = cache->v_scale;
  p.num_tokens = num_tokens;
  p.num_slots = (int64_t)cache->num_blocks * cache->block_size;
  p.num_kv_heads = cache->num_kv_heads;
  p.src_dtype = src_dtype;
  return finish(qsakv::launch_kv_write(cache->kind, cache->head_dim, p,
                                       static_cast<hipStream_t>(stream)));
}

qkv_status qsa_sparse_attn_prefill(const qkv_cache* cache, const qsa_args* args, void* stream) {
  qkv_status st = check_cache(cache, true);
  if (st != QKV_OK) return st;
  st = check_args(cache, args);
  if (st != QKV_OK || args->num_rows == 0) return st;
  const qsakv::AttnParams p = make_params(cache, args, 1);
  return finish(qsakv::launch_attn(cache->kind, cache->head_dim, p,
                                   static_cast<hipStream_t>(stream)));
}

size_t qsa_decode_workspace_bytes(int32_t num_rows, int32_t num_q_heads, int32_t head_dim,
                                  int32_t num_splits) {
  return ws_bytes(num_rows, num_q_heads, head_dim, num_splits);
}

qkv_status qsa_sparse_attn_decode(const qkv_cache* cache, const qsa_args* args, int32_t num_splits,
                                  void* workspace, size_t workspace_bytes, void* stream) {
  const qkv_status st = check_decode(cache, args, num_splits);
  if (st != QKV_OK || args->num_rows == 0) return st;
  if (num_splits > 1) {
    const size_t need = ws_bytes(args->num_rows, args->num_q_heads, cache->head_dim, num_splits);
    if (!workspace || workspace_bytes < need || !aligned(workspace, 256))
      return QKV_ERR_WORKSPACE;
  }
  return run_decode(cache, args, num_splits, static_cast<char*>(workspace),
                    static_cast<hipStream_t>(stream));
}

qkv_status qsa_sparse_attn_decode_noalloc(const qkv_cache* cache, const qsa_args* args,
                                          int32_t num_splits, void* stream) {
  const qkv_status st = check_decode(cache, args, num_splits);
  if (st != QKV_OK || args->num_rows == 0) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (num_splits == 1) return run_decode(cache, args, 1, nullptr, s);
  const size_t need = ws_bytes(args->num_rows, args->num_q_heads, cache->head_dim, num_splits);
  if (need > QSA_NOALLOC_SCRATCH_BYTES) return QKV_ERR_SCRATCH;
  void* ws = nullptr;
  const hipError_t e = scratch_ptr(s, &ws);
  if (e != hipSuccess) return finish(e);
  return run_decode(cache, args, num_splits, static_cast<char*>(ws), s);
}


size_t qkv_calib_workspace_bytes(void) { return qsakv::calib_workspace_bytes(); }

qkv_status kv_calib_stats(const void* x, int32_t src_dtype, int64_t n, float scale,
                          qkv_calib_result* out, void* workspace, size_t workspace_bytes,
                          void* stream) {
  if (src_dtype < QKV_BF16 || src_dtype > QKV_FP32) return QKV_ERR_UNSUPPORTED;
  if (n < 0) return QKV_ERR_BAD_SHAPE;
  if (!out || (n > 0 && !x)) return QKV_ERR_NULL;
  if (!scale_ok(scale)) return QKV_ERR_BAD_SCALE;
  if (!aligned(out, 8) || (x && !aligned(x, 16))) return QKV_ERR_ALIGNMENT;
  if (!workspace || workspace_bytes < qsakv::calib_workspace_bytes() || !aligned(workspace, 256))
    return QKV_ERR_WORKSPACE;
  qsakv::CalibParams p;
  p.x = x;
  p.n = n;
  p.src_dtype = src_dtype;
  p.t_sat = calib_threshold(scale, kCalibSat);
  p.t_sub = calib_threshold(scale, kCalibSub);
  p.t_norm = calib_threshold(scale, kCalibNorm);
  p.workspace = workspace;
  p.out = out;
  return finish(qsakv::launch_calib(p, static_cast<hipStream_t>(stream)));
}

size_t qsa_topk_workspace_bytes(int32_t num_rows, int32_t row_stride, int32_t topk) {
  TopkWs w;
  return topk_ws(num_rows, row_stride, topk, &w) ? (size_t)w.bytes : 0;
}

qkv_status qsa_topk_select(const void* scores, int32_t score_dtype, int32_t num_rows,
                           int32_t row_stride, const int32_t* row_len, int32_t topk,
                           int32_t* topk_idx, void* workspace, size_t workspace_bytes,
                           void* stream) {
  if (score_dtype < QKV_BF16 || score_dtype > QKV_FP32) return QKV_ERR_UNSUPPORTED;
  if (num_rows < 0 || row_stride < 0 || row_stride > (1 << 30) || topk < 1)
    return QKV_ERR_BAD_SHAPE;
  int64_t outs;
  if (!mul_ok(num_rows, topk, &outs) || outs > INT32_MAX) return QKV_ERR_BAD_SHAPE;
  TopkWs w;
  if (!topk_ws(num_rows, row_stride, topk, &w)) return QKV_ERR_BAD_SHAPE;
  if (num_rows == 0) return QKV_OK;
  if (!scores || !row_len || !topk_idx) return QKV_ERR_NULL;
  const int64_t esize = score_dtype == QKV_FP32 ? 4 : 2;
  if (!aligned(scores, 16) || (row_stride * esize) % 16 != 0 || !aligned(row_len, 4) ||
      !aligned(topk_idx, 4))
    return QKV_ERR_ALIGNMENT;
  if (w.bytes > 0 && (!workspace || workspace_bytes < (size_t)w.bytes || !aligned(workspace, 256)))
    return QKV_ERR_WORKSPACE;
  qsakv::TopkParams p{};
  p.scores = scores;
  p.row_len = row_len;
  p.out = topk_idx;
  p.num_rows = num_rows;
  p.row_stride = row_stride;
  p.topk = topk;
  p.seg_len = w.seg_len;
  p.row_slots = (int32_t)w.row_slots;
  if (w.bytes > 0) {
    p.ws_key = static_cast<uint32_t*>(workspace);
    p.ws_pos = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + w.key_bytes);
  }
  return finish(qsakv::launch_topk(score_dtype, p, static_cast<hipStream_t>(stream)));
}

qkv_status qkv_cache_bytes(int32_t kind, int32_t num_blocks, int32_t block_size,
                           int32_t num_kv_heads, int32_t head_dim, size_t* k_bytes,
                           size_t* v_bytes, size_t* scale_bytes) {
  if (kind < QKV_CACHE_INT8 || kind > QKV_CACHE_NVFP4) return QKV_ERR_UNSUPPORTED;
  if (head_dim != 128 && head_dim != 256) return QKV_ERR_UNSUPPORTED;
  if (num_blocks <= 0 || num_kv_heads <= 0 || !is_pow2(block_size) || block_size > 1024)
    return QKV_ERR_BAD_SHAPE;
  int64_t rows, kb, sb = 0;
  if (!mul_ok((int64_t)num_blocks * block_size, num_kv_heads, &rows) ||
      !mul_ok(rows, row_bytes(kind, head_dim), &kb))
    return QKV_ERR_BAD_SHAPE;
  if (kind == QKV_CACHE_INT8 && !mul_ok(rows, 8, &sb)) return QKV_ERR_BAD_SHAPE;
  if (kind == QKV_CACHE_NVFP4 && !mul_ok(rows, 2 * (head_dim / 16), &sb)) return QKV_ERR_BAD_SHAPE;
  if (k_bytes) *k_bytes = (size_t)kb;
  if (v_bytes) *v_bytes = (size_t)kb;
  if (scale_bytes) *scale_bytes = (size_t)sb;
  return QKV_OK;
}

const char* qkv_status_str(int32_t status) {
  switch (status) {
    case QKV_OK: return "QKV_OK";
    case QKV_ERR_NULL: return "QKV_ERR_NULL: a required pointer is NULL";
    case QKV_ERR_BAD_SHAPE: return "QKV_ERR_BAD_SHAPE: invalid or inconsistent size";
    case QKV_ERR_UNSUPPORTED: return "QKV_ERR_UNSUPPORTED: configuration outside the supported set";
    case QKV_ERR_BAD_SCALE: return "QKV_ERR_BAD_SCALE: scale missing, non-finite or not positive";
    case QKV_ERR_WORKSPACE: return "QKV_ERR_WORKSPACE: split-K workspace missing, small or misaligned";
    case QKV_ERR_HIP: return "QKV_ERR_HIP: the HIP runtime reported an error";
    case QKV_ERR_ALIGNMENT: return "QKV_ERR_ALIGNMENT: device pointer misaligned";
    case QKV_ERR_SCRATCH:
      return "QKV_ERR_SCRATCH: the call needs more split-K scratch than the no-alloc entry "
             "point's static buffer holds (QSA_NOALLOC_SCRATCH_BYTES); use "
             "qsa_sparse_attn_decode with a workspace";
    default: return "unknown qkv_status";
  }
}

int32_t qkv_last_hip_error(void) { return g_last_hip_error; }

int32_t qkv_abi_version(void) { return QSAKV_ABI_VERSION; }

}  // extern "C"
