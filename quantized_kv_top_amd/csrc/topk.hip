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
// Method: radix selection on order-preserving integer keys.  Every score is
// widened to float32 (exact for fp16 / bf16) and mapped to an unsigned key
// whose integer order is the ranking (-0 folded onto +0, sign-magnitude
// flip, NaN to 0).  One workgroup of 1024 threads per row, two per CU:
//   * the row is read once into registers and turned into keys;
//   * an LDS histogram of the top 11 key bits gives the digit d0 of the k-th
//     largest key (the bins are summed in 16 slices, one barrier, then every
//     wave locates the digit by itself);
//   * the keys whose top digit is at least d0 -- the sure ones above d0's bin
//     and that whole bin, typically little more than k -- go to LDS in
//     position order (per-wave scans of per-group counts, one barrier);
//   * the remaining 11 + 10 bits are selected over those candidates only,
//     which leaves the exact k-th key T and the number of ties at T to take;
//   * a pass over the candidates in position order writes every position
//     with key > T and the first such ties (one block scan per 1024
//     candidates gives each thread how many of both lie before it).
// When d0's bin overflows LDS (heavily tied scores) the remaining passes
// re-read the row (L2-resident by then); rows longer than the register
// capacity (32768 scores) stream every pass from memory.  The bound is the
// single read of the scores from HBM.
#include "qsakv_device.h"
#include "qsakv_internal.h"

namespace qsakv {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / kWave;
constexpr int kBins = 2048;      // 11-bit digits
constexpr int kCand = 4096;      // candidates kept in LDS after the first digit
constexpr int kMaxKPT = 32;      // scores per thread held in registers (rows <= 32768)

// Order-preserving keys, one 32-bit key per score whatever its type (fp16
// and bf16 scores are widened to float32 exactly): the larger the score, the
// larger the key.  x + 0 turns -0 into +0 and leaves every other value,
// denormals included, as it is, so -0 and +0 share a key; the sign-magnitude
// flip orders the rest; every NaN maps to 0, below -inf's key 0x007fffff.
__device__ __forceinline__ uint32_t score_key(float x) {
  const float z = x + 0.0f;
  const uint32_t u = __float_as_uint(z);
  const uint32_t k = u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
  return z != z ? 0u : k;
}

// Radix digits of the keys: 11 + 11 + 10 bits from the top.
constexpr int kPasses = 3;
constexpr int kShift[kPasses] = {21, 10, 0};
constexpr int kWidth[kPasses] = {11, 11, 10};

// Scores of a 16-byte group: kVec of them.
template <int SRC>
struct Src;
template <>
struct Src<kDtFP32> {
  static constexpr int kVec = 4;
  __device__ static float at(const u32x4& v, int e) { return __uint_as_float(v[e]); }
};
template <>
struct Src<kDtFP16> {
  static constexpr int kVec = 8;
  __device__ static float at(const u32x4& v, int e) {
    return (float)bitcast<_Float16>((uint16_t)(v[e >> 1] >> (16 * (e & 1))));
  }
};
template <>
struct Src<kDtBF16> {
  static constexpr int kVec = 8;
  __device__ static float at(const u32x4& v, int e) {
    const uint32_t w = v[e >> 1];
    return __uint_as_float((e & 1) ? (w & 0xffff0000u) : (w << 16));
  }
};

// A value every thread of the workgroup holds alike (read from LDS after a
// barrier, or a wave reduction): kept in a scalar register.
__device__ __forceinline__ uint32_t uniform(uint32_t x) { return __builtin_amdgcn_readfirstlane(x); }

// Inclusive prefix sum over the wave's lanes in the VALU: DPP shifts of 1, 2,
// 4 and 8 lanes within each 16-lane row, then the broadcasts of lane 15 into
// rows 1 and 3 and of lane 31 into rows 2 and 3.  Lanes a shift leaves
// without a source add 0.
__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t v) {
  int x = (int)v;
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);   // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);   // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);   // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);   // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);   // row_bcast:15
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);   // row_bcast:31
  return (uint32_t)x;
}

struct __align__(16) Smem {
  uint32_t hist[3][kBins];          // one histogram per radix pass, cleared once
  uint32_t tmp[2][kWaves];          // wave totals of the block scans, alternating
  uint32_t seg[kMaxKPT / 4 * kWaves];  // candidates per (register group, wave)
  uint32_t slice[kWaves];           // histogram slice sums of a digit pick
};

// Workgroup-wide exclusive prefix sums in thread order, one barrier each: the
// wave totals alternate between two LDS buffers, so a buffer is rewritten
// only after the barrier of the scan in between (every thread calls the
// scans in the same order).
struct BlockScan {
  Smem& s;
  uint32_t phase = 0;
  __device__ uint32_t exscan(uint32_t v, uint32_t* total) {
    const int lane = lane_id();
    const int w = (int)uniform(threadIdx.x / kWave);
    uint32_t* tmp = s.tmp[phase];
    phase ^= 1u;
    const uint32_t x = wave_inclusive_scan(v);
    if (lane == kWave - 1) tmp[w] = x;
    __syncthreads();
    const uint32_t ts = wave_inclusive_scan(lane < kWaves ? tmp[lane] : 0u);
    *total = __builtin_amdgcn_readlane(ts, kWaves - 1);
    const uint32_t below = w > 0 ? __builtin_amdgcn_readlane(ts, w - 1) : 0u;
    return below + x - v;
  }
};

// Keys with (key & pmask) == pval are still in play; `need` of them go into
// the list.
struct Sel {
  uint32_t pmask, pval, need;
};

__device__ __forceinline__ void clear_hists(Smem& s) {
  for (int b = threadIdx.x; b < 3 * kBins; b += kThreads) (&s.hist[0][0])[b] = 0u;
}

__device__ __forceinline__ void count_key(uint32_t* h, uint32_t key, const Sel& st, int shift,
                                          uint32_t dmask) {
  if ((key & st.pmask) == st.pval) atomicAdd(&h[(key >> shift) & dmask], 1u);
}

// h holds the histogram (complete: after a barrier) of the digit at `shift`
// of the keys in play: find the digit of the need-th largest of them,
// narrow the state to it and return the count of its bin.  Bins are taken
// from the top in 16 slices of 128: wave w sums slice w (two bins per lane,
// conflict-free), one barrier publishes the slice sums, then every wave on
// its own finds the slice where the count from the top reaches `need` and,
// scanning that slice's bins, the bin.  h is only read.
__device__ __forceinline__ uint32_t pick_digit(Smem& s, const uint32_t* h, int shift, int width,
                                               Sel& st) {
  constexpr int kSlice = kBins / kWaves;                 // 128
  const int lane = lane_id();
  const int w = (int)uniform(threadIdx.x / kWave);
  {
    const int top = kBins - 1 - kSlice * w;
    const uint32_t sum = wave_inclusive_scan(h[top - lane] + h[top - kWave - lane]);
    if (lane == kWave - 1) s.slice[w] = sum;
  }
  __syncthreads();
  const uint32_t t = lane < kWaves ? s.slice[lane] : 0u;
  const uint32_t ti = wave_inclusive_scan(t);
  const int q = __builtin_ctzll(__ballot(ti >= st.need));
  const uint32_t above = __builtin_amdgcn_readlane(ti, q) - __builtin_amdgcn_readlane(t, q);
  const int top = kBins - 1 - kSlice * q;
  const uint32_t c0 = h[top - lane], c1 = h[top - kWave - lane];
  const uint32_t i0 = above + wave_inclusive_scan(c0);
  const uint64_t m0 = __ballot(i0 >= st.need);
  int bin;
  uint32_t cnt, incl;
  if (m0) {
    const int l = __builtin_ctzll(m0);
    bin = top - l;
    cnt = __builtin_amdgcn_readlane(c0, l);
    incl = __builtin_amdgcn_readlane(i0, l);
  } else {
    const uint32_t i1 = __builtin_amdgcn_readlane(i0, kWave - 1) + wave_inclusive_scan(c1);
    const int l = __builtin_ctzll(__ballot(i1 >= st.need));
    bin = top - kWave - l;
    cnt = __builtin_amdgcn_readlane(c1, l);
    incl = __builtin_amdgcn_readlane(i1, l);
  }
  st.need -= incl - cnt;
  st.pval |= (uint32_t)bin << shift;
  st.pmask |= ((1u << width) - 1u) << shift;
  return cnt;
}

// One tile of the list, in position order: V elements per thread (pos < 0:
// none); with T the k-th largest key and `ties` the number of keys == T to
// list, an element goes to slot (#keys > T before it) + min(#keys == T
// before it, ties) if its key is > T, or if it is one of the first `ties`
// keys == T.
template <int V>
__device__ __forceinline__ void emit_tile(BlockScan& bs, const uint32_t (&key)[V],
                                          const int (&pos)[V], uint32_t T, uint32_t ties,
                                          uint32_t& gt_base, uint32_t& eq_base, int32_t* out) {
  uint32_t cg = 0, ce = 0;
#pragma unroll
  for (int e = 0; e < V; ++e) {
    cg += (pos[e] >= 0 && key[e] > T) ? 1u : 0u;
    ce += (pos[e] >= 0 && key[e] == T) ? 1u : 0u;
  }
  uint32_t tot;
  const uint32_t before = bs.exscan(cg | (ce << 16), &tot);   // < 2^16 per tile
  uint32_t gb = gt_base + (before & 0xffffu), eb = eq_base + (before >> 16);
#pragma unroll
  for (int e = 0; e < V; ++e) {
    if (pos[e] < 0) continue;
    if (key[e] > T) {
      out[gb + min(eb, ties)] = pos[e];
      ++gb;
    } else if (key[e] == T) {
      if (eb < ties) out[gb + eb] = pos[e];
      ++eb;
    }
  }
  gt_base += tot & 0xffffu;
  eq_base += tot >> 16;
}

// ---- passes that stream the row from memory ---------------------------------
// (the histograms are clear and published by a barrier before the first)
template <int SRC>
__device__ void stream_passes(Smem& s, const u32x4* row, int n, int first, Sel& st) {
  constexpr int kVec = Src<SRC>::kVec;
  const int nvec = (n + kVec - 1) / kVec;
#pragma unroll
  for (int pass = 0; pass < kPasses; ++pass) {
    if (pass < first) continue;
    const uint32_t dmask = (1u << kWidth[pass]) - 1u;
    for (int g = threadIdx.x; g < nvec; g += kThreads) {
      const u32x4 v = row[g];
#pragma unroll
      for (int e = 0; e < kVec; ++e)
        if (g * kVec + e < n)
          count_key(s.hist[pass], score_key(Src<SRC>::at(v, e)), st, kShift[pass], dmask);
    }
    __syncthreads();
    pick_digit(s, s.hist[pass], kShift[pass], kWidth[pass], st);
  }
}

template <int SRC>
__device__ void stream_emit(BlockScan& bs, const u32x4* row, int n, const Sel& st, int k,
                            int32_t* out) {
  constexpr int kVec = Src<SRC>::kVec;
  const int nvec = (n + kVec - 1) / kVec;
  const uint32_t T = st.pval, ties = st.need, n_gt = (uint32_t)k - ties;
  uint32_t gt_base = 0, eq_base = 0;
  for (int g0 = 0; g0 < nvec; g0 += kThreads) {
    const int g = g0 + (int)threadIdx.x;
    const u32x4 v = g < nvec ? row[g] : u32x4{0u, 0u, 0u, 0u};
    uint32_t key[kVec];
    int pos[kVec];
#pragma unroll
    for (int e = 0; e < kVec; ++e) {
      key[e] = score_key(Src<SRC>::at(v, e));
      pos[e] = (g < nvec && g * kVec + e < n) ? g * kVec + e : -1;
    }
    emit_tile<kVec>(bs, key, pos, T, ties, gt_base, eq_base, out);
    if (gt_base == n_gt && eq_base >= ties) break;   // uniform: the list is complete
  }
}

// rows with at most k candidates list all of them
__device__ __forceinline__ bool list_all(int n, int k, int32_t* out) {
  if (n > k) return false;
  for (int i = threadIdx.x; i < k; i += kThreads) out[i] = i < n ? i : -1;
  return true;
}

template <int SRC>
__device__ __forceinline__ const u32x4* row_ptr(const TopkParams& p, int r) {
  return reinterpret_cast<const u32x4*>(static_cast<const uint8_t*>(p.scores) +
                                        (int64_t)r * p.row_stride * (SRC == kDtFP32 ? 4 : 2));
}

// Rows beyond the register capacity: every pass streams the row.
template <int SRC>
__global__ __launch_bounds__(kThreads) void topk_stream_kernel(TopkParams p) {
  __shared__ Smem s;
  const int r = blockIdx.x, k = p.topk;
  int32_t* out = p.out + (int64_t)r * k;
  const int n = min(max(p.row_len[r], 0), p.row_stride);
  if (list_all(n, k, out)) return;
  const u32x4* row = row_ptr<SRC>(p, r);
  BlockScan bs{s};
  Sel st{0u, 0u, (uint32_t)k};
  clear_hists(s);
  __syncthreads();
  stream_passes<SRC>(s, row, n, 0, st);
  stream_emit<SRC>(bs, row, n, st, k, out);
}

// One row whose keys a thread holds in registers (group j of thread t: the
// kVec scores at positions (t + 1024 j) kVec ..; positions beyond the row's
// n carry key 0, the lowest, which never reaches the list of a row with more
// than k candidates): the first digit from registers, then the keys of its
// bin and above (the candidates) to LDS in position order and the remaining
// digits over them -- or, when the candidates overflow LDS (heavy ties), the
// remaining passes re-read the row.
template <int SRC, int KPT>
__device__ __forceinline__ void select_row(Smem& s, uint32_t* s_key, int32_t* s_pos,
                                           const uint32_t (&key)[KPT / Src<SRC>::kVec]
                                                                [Src<SRC>::kVec],
                                           const u32x4* row, int n, int k, int32_t* out) {
  constexpr int kVec = Src<SRC>::kVec;
  constexpr int kGroups = KPT / kVec;
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int w = (int)uniform(tid / kWave);
  BlockScan bs{s};
  clear_hists(s);
  __syncthreads();

  // ---- first digit, from registers -------------------------------------------
  Sel st{0u, 0u, (uint32_t)k};
#pragma unroll
  for (int j = 0; j < kGroups; ++j)
#pragma unroll
    for (int e = 0; e < kVec; ++e) atomicAdd(&s.hist[0][key[j][e] >> kShift[0]], 1u);
  __syncthreads();
  const uint32_t bin0 = pick_digit(s, s.hist[0], kShift[0], kWidth[0], st);
  // keys with a top digit above d0 are all listed; d0's bin holds the rest
  const uint32_t lo = st.pval;                           // d0 << kShift[0]
  const uint32_t ncand = (uint32_t)k - st.need + bin0;
  if (ncand > (uint32_t)kCand) {                         // uniform
    stream_passes<SRC>(s, row, n, 1, st);
    stream_emit<SRC>(bs, row, n, st, k, out);
    return;
  }

  // ---- candidates (top digit >= d0) to LDS, in position order ---------------
  // Position order is (register group j, wave, lane, element).  Each wave
  // scans its per-group counts (three groups per 32-bit word, 10-bit
  // fields), one barrier publishes the (group, wave) counts, and every wave
  // scans those to place its shares.
  {
    constexpr int kWords = (kGroups + 2) / 3;
    uint32_t cnt[kGroups], wincl[kWords];
#pragma unroll
    for (int j = 0; j < kGroups; ++j) {
      cnt[j] = 0;
#pragma unroll
      for (int e = 0; e < kVec; ++e) cnt[j] += key[j][e] >= lo ? 1u : 0u;
    }
#pragma unroll
    for (int q = 0; q < kWords; ++q) {
      uint32_t v = 0;
#pragma unroll
      for (int i = 0; i < 3; ++i)
        if (3 * q + i < kGroups) v |= cnt[3 * q + i] << (10 * i);
      wincl[q] = wave_inclusive_scan(v);
      if (lane == kWave - 1) {
#pragma unroll
        for (int i = 0; i < 3; ++i)
          if (3 * q + i < kGroups) s.seg[(3 * q + i) * kWaves + w] = (wincl[q] >> (10 * i)) & 0x3ffu;
      }
    }
    __syncthreads();
    constexpr int kSeg = kGroups * kWaves;               // <= 128: two values per lane
    const uint32_t c0 = lane < kSeg ? s.seg[lane] : 0u;
    const uint32_t c1 = lane + kWave < kSeg ? s.seg[lane + kWave] : 0u;
    const uint32_t i0 = wave_inclusive_scan(c0);
    const uint32_t i1 = wave_inclusive_scan(c1) + __builtin_amdgcn_readlane(i0, kWave - 1);
#pragma unroll
    for (int j = 0; j < kGroups; ++j) {
      const int sg = j * kWaves + w;                     // this wave's share of group j
      const uint32_t start = sg < kWave
          ? __builtin_amdgcn_readlane(i0, sg) - __builtin_amdgcn_readlane(c0, sg)
          : __builtin_amdgcn_readlane(i1, sg - kWave) - __builtin_amdgcn_readlane(c1, sg - kWave);
      uint32_t o = start + ((wincl[j / 3] >> (10 * (j % 3))) & 0x3ffu) - cnt[j];
      const int base = (tid + j * kThreads) * kVec;
#pragma unroll
      for (int e = 0; e < kVec; ++e) {
        if (key[j][e] >= lo) {
          s_key[o] = key[j][e];
          s_pos[o] = base + e;
          ++o;
        }
      }
    }
    __syncthreads();
  }

  // ---- remaining digits over the candidates ----------------------------------
#pragma unroll
  for (int pass = 1; pass < kPasses; ++pass) {
    const uint32_t dmask = (1u << kWidth[pass]) - 1u;
    for (int i = tid; i < (int)ncand; i += kThreads)
      count_key(s.hist[pass], s_key[i], st, kShift[pass], dmask);
    __syncthreads();
    pick_digit(s, s.hist[pass], kShift[pass], kWidth[pass], st);
  }

  // ---- the list ---------------------------------------------------------------
  const uint32_t T = st.pval, ties = st.need, n_gt = (uint32_t)k - ties;
  uint32_t gt_base = 0, eq_base = 0;
  for (int c0 = 0; c0 < (int)ncand; c0 += kThreads) {
    const int i = c0 + tid;
    const uint32_t kk[1] = {i < (int)ncand ? s_key[i] : 0u};
    const int pos[1] = {i < (int)ncand ? s_pos[i] : -1};
    emit_tile<1>(bs, kk, pos, T, ties, gt_base, eq_base, out);
    if (gt_base == n_gt && eq_base >= ties) break;       // uniform
  }
}

// Rows of up to KPT * 1024 scores, one workgroup each, two per CU (8 waves
// per SIMD, <= 64 registers): the row's 16-byte groups are loaded at once
// (addresses clamped to the row's last group) and turned into keys.
template <int SRC, int KPT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(8, 8)))
void topk_cand_kernel(TopkParams p) {
  constexpr int kVec = Src<SRC>::kVec;
  constexpr int kGroups = KPT / kVec;                   // 16-byte groups per thread
  __shared__ Smem s;
  __shared__ uint32_t s_key[kCand];
  __shared__ int32_t s_pos[kCand];
  const int tid = threadIdx.x, k = p.topk, r = blockIdx.x;
  int32_t* out = p.out + (int64_t)r * k;
  const int n = min(max(p.row_len[r], 0), p.row_stride);
  if (list_all(n, k, out)) return;
  const u32x4* row = row_ptr<SRC>(p, r);
  const int last = (n + kVec - 1) / kVec - 1;
  uint32_t key[kGroups][kVec];
  {
    u32x4 raw[kGroups];
#pragma unroll
    for (int j = 0; j < kGroups; ++j) raw[j] = row[min(tid + j * kThreads, last)];
#pragma unroll
    for (int j = 0; j < kGroups; ++j)
#pragma unroll
      for (int e = 0; e < kVec; ++e)
        key[j][e] = (tid + j * kThreads) * kVec + e < n ? score_key(Src<SRC>::at(raw[j], e)) : 0u;
  }
  select_row<SRC, KPT>(s, s_key, s_pos, key, row, n, k, out);
}

template <int SRC>
hipError_t launch_src(const TopkParams& p, hipStream_t s) {
  const dim3 grid((unsigned)p.num_rows), block(kThreads);
  const int64_t per_thread = ((int64_t)p.row_stride + kThreads - 1) / kThreads;
  if (per_thread <= 8)
    topk_cand_kernel<SRC, 8><<<grid, block, 0, s>>>(p);
  else if (per_thread <= 16)
    topk_cand_kernel<SRC, 16><<<grid, block, 0, s>>>(p);
  else if (per_thread <= kMaxKPT)
    topk_cand_kernel<SRC, kMaxKPT><<<grid, block, 0, s>>>(p);
  else
    topk_stream_kernel<SRC><<<grid, block, 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_topk(int src_dtype, const TopkParams& p, hipStream_t s) {
  if (src_dtype == kDtFP32) return launch_src<kDtFP32>(p, s);
  if (src_dtype == kDtFP16) return launch_src<kDtFP16>(p, s);
  return launch_src<kDtBF16>(p, s);
}

}  // namespace qsakv
