// Top-k selection of each query row's positions from indexer scores (gfx950).
//
// What is computed: row r has n = clamp(row_len[r], 0, row_stride) candidate
// positions 0 .. n-1 with one score each; its list is the k positions with
// the largest scores (compared as numbers: -0 == +0, NaN below -inf), equal
// scores taken in increasing position order, written in increasing position
// order and padded with -1 when n < k.  This is the selection ahead of the
// sparse attention on page "[Model][SM70][FP8] Add calibrated E4M3 QSA KV
// cache" (validated contract: FP16 indexer caches score the candidates and
// each row's list is selected from them), on scores that are inputs here.
//
// Method: radix selection on order-preserving integer keys.  A score maps to
// an unsigned key whose integer order is the ranking (sign-magnitude flip,
// -0 folded onto +0, NaN to 0).  One workgroup of 1024 threads per row builds
// an LDS histogram of the top 11 key bits over the row, finds the digit of
// the k-th largest key with a block scan over the bins, and repeats on the
// next bits of the keys that share the digits found so far (11 + 11 + 10
// bits for fp32 scores, 11 + 5 for fp16 / bf16), which leaves the exact k-th
// key T and the number of ties at T to take.  A last pass in position order
// writes every position with key > T and the first such ties: one block
// scan per tile gives each thread how many of both lie before it.  Each pass
// streams the row (the later ones mostly from L2 / MALL); the bound is the
// read of the scores.
#include "qsakv_device.h"
#include "qsakv_internal.h"

namespace qsakv {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / kWave;
constexpr int kBins = 2048;      // 11-bit digits

// Order-preserving keys.  fp32: the larger the score, the larger the key;
// -0 and +0 share a key; every NaN maps to 0, below -inf's key.
__device__ __forceinline__ uint32_t key_f32(uint32_t u) {
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0u;
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
// 16-bit patterns (fp16: NaN above 0x7c00; bf16: above 0x7f80).
template <uint32_t kInfBits>
__device__ __forceinline__ uint32_t key_h(uint32_t h) {
  if ((h & 0x7fffu) > kInfBits) return 0u;
  if (h == 0x8000u) h = 0u;
  return (h & 0x8000u) ? (~h & 0xffffu) : (h | 0x8000u);
}

template <int SRC>
struct Keys;
template <>
struct Keys<kDtFP32> {
  static constexpr int kVec = 4;                 // scores per 16-byte load
  static constexpr int kPasses = 3;
  static constexpr int kShift[3] = {21, 10, 0};
  static constexpr int kWidth[3] = {11, 11, 10};
  __device__ static uint32_t key(const u32x4& v, int e) { return key_f32(v[e]); }
};
template <>
struct Keys<kDtFP16> {
  static constexpr int kVec = 8;
  static constexpr int kPasses = 2;
  static constexpr int kShift[3] = {5, 0, 0};
  static constexpr int kWidth[3] = {11, 5, 0};
  __device__ static uint32_t key(const u32x4& v, int e) {
    return key_h<0x7c00u>((v[e >> 1] >> (16 * (e & 1))) & 0xffffu);
  }
};
template <>
struct Keys<kDtBF16> {
  static constexpr int kVec = 8;
  static constexpr int kPasses = 2;
  static constexpr int kShift[3] = {5, 0, 0};
  static constexpr int kWidth[3] = {11, 5, 0};
  __device__ static uint32_t key(const u32x4& v, int e) {
    return key_h<0x7f80u>((v[e >> 1] >> (16 * (e & 1))) & 0xffffu);
  }
};

// Exclusive prefix sum of v over the workgroup's threads (in thread order);
// *total gets the sum over all threads.  s_tmp: kWaves words of LDS.
__device__ __forceinline__ uint32_t block_exscan(uint32_t v, uint32_t* s_tmp, uint32_t* total) {
  const int lane = lane_id(), w = threadIdx.x / kWave;
  uint32_t x = v;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const uint32_t y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == kWave - 1) s_tmp[w] = x;
  __syncthreads();
  uint32_t off = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) {
    const uint32_t t = s_tmp[i];
    off += i < w ? t : 0u;
    tot += t;
  }
  __syncthreads();    // s_tmp may be reused
  *total = tot;
  return off + x - v;
}

template <int SRC>
__global__ __launch_bounds__(kThreads) void topk_select_kernel(TopkParams p) {
  using K = Keys<SRC>;
  constexpr int kVec = K::kVec;
  __shared__ uint32_t s_hist[kBins];
  __shared__ uint32_t s_tmp[kWaves];
  __shared__ uint32_t s_sel[2];

  const int r = blockIdx.x;
  const int tid = threadIdx.x;
  const int k = p.topk;
  int32_t* out = p.out + (int64_t)r * k;
  const int n = min(max(p.row_len[r], 0), p.row_stride);

  if (n <= k) {          // every candidate is listed
    for (int i = tid; i < k; i += kThreads) out[i] = i < n ? i : -1;
    return;
  }

  const u32x4* row = reinterpret_cast<const u32x4*>(
      static_cast<const uint8_t*>(p.scores) + (int64_t)r * p.row_stride * (SRC == kDtFP32 ? 4 : 2));
  const int nvec = (n + kVec - 1) / kVec;   // 16-byte groups holding the candidates

  // ---- radix selection of the k-th largest key ------------------------------
  uint32_t pmask = 0, pval = 0, need = (uint32_t)k;
#pragma unroll
  for (int pass = 0; pass < K::kPasses; ++pass) {
    const int shift = K::kShift[pass];
    const uint32_t dmask = (1u << K::kWidth[pass]) - 1u;
    for (int b = tid; b < kBins; b += kThreads) s_hist[b] = 0u;
    __syncthreads();
    for (int g = tid; g < nvec; g += kThreads) {
      const u32x4 v = row[g];
#pragma unroll
      for (int e = 0; e < kVec; ++e) {
        const uint32_t key = K::key(v, e);
        if (g * kVec + e < n && (key & pmask) == pval)
          atomicAdd(&s_hist[(key >> shift) & dmask], 1u);
      }
    }
    __syncthreads();
    // thread t holds bins 2047 - 2t (upper) and 2046 - 2t; the scan in thread
    // order counts the keys in all higher bins
    const int bhi = kBins - 1 - 2 * tid, blo = bhi - 1;
    const uint32_t chi = s_hist[bhi], clo = s_hist[blo];
    uint32_t tot;
    const uint32_t above = block_exscan(chi + clo, s_tmp, &tot);
    if (above < need && need <= above + chi + clo) {
      const bool hi = need <= above + chi;
      s_sel[0] = (uint32_t)(hi ? bhi : blo);
      s_sel[1] = need - above - (hi ? 0u : chi);
    }
    __syncthreads();
    pval |= s_sel[0] << shift;
    pmask |= dmask << shift;
    need = s_sel[1];
    __syncthreads();   // s_sel and s_hist are rewritten by the next pass
  }
  const uint32_t T = pval;       // the k-th largest key
  const uint32_t ties = need;    // keys equal to T that are listed (>= 1)
  const uint32_t n_gt = (uint32_t)k - ties;

  // ---- positions in order: key > T, and the first `ties` keys == T ----------
  uint32_t gt_base = 0, eq_base = 0;
  for (int g0 = 0; g0 < nvec; g0 += kThreads) {
    const int g = g0 + tid;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (g < nvec) v = row[g];
    uint32_t cg = 0, ce = 0;
    uint32_t keys[kVec];
#pragma unroll
    for (int e = 0; e < kVec; ++e) {
      keys[e] = (g < nvec && g * kVec + e < n) ? K::key(v, e) : 0u;
      const bool valid = g < nvec && g * kVec + e < n;
      cg += (valid && keys[e] > T) ? 1u : 0u;
      ce += (valid && keys[e] == T) ? 1u : 0u;
    }
    uint32_t tot;
    const uint32_t before = block_exscan(cg | (ce << 16), s_tmp, &tot);
    uint32_t gb = gt_base + (before & 0xffffu), eb = eq_base + (before >> 16);
#pragma unroll
    for (int e = 0; e < kVec; ++e) {
      const bool valid = g < nvec && g * kVec + e < n;
      if (!valid) continue;
      const int pos = g * kVec + e;
      if (keys[e] > T) {
        out[gb + min(eb, ties)] = pos;
        ++gb;
      } else if (keys[e] == T) {
        if (eb < ties) out[gb + eb] = pos;
        ++eb;
      }
    }
    gt_base += tot & 0xffffu;
    eq_base += tot >> 16;
    if (gt_base == n_gt && eq_base >= ties) break;   // the list is complete
  }
}

}  // namespace

hipError_t launch_topk(int src_dtype, const TopkParams& p, hipStream_t s) {
  const dim3 grid((unsigned)p.num_rows), block(kThreads);
  if (src_dtype == kDtFP32)
    topk_select_kernel<kDtFP32><<<grid, block, 0, s>>>(p);
  else if (src_dtype == kDtFP16)
    topk_select_kernel<kDtFP16><<<grid, block, 0, s>>>(p);
  else
    topk_select_kernel<kDtBF16><<<grid, block, 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace qsakv
