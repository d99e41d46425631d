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
//   * an LDS histogram of the top 11 key bits (counted into four copies with
//     bins XOR-swizzled by copy, then summed) gives the digit d0 of the k-th
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

// ---- where a row's keys come from and where its list goes ----------------------
// Scores of one row (or of one segment of it): element idx is the score at
// position pos0 + idx.
template <int SRC>
struct ScoreRow {
  static constexpr int kVec = Src<SRC>::kVec;
  const u32x4* data;      // 16-byte groups of the row (segment)
  int n;                  // elements in play
  int pos0;
  __device__ uint32_t key(const u32x4& v, int e) const { return score_key(Src<SRC>::at(v, e)); }
  __device__ int pos(int idx) const { return pos0 + idx; }
};
// The segments' lists of one row, concatenated: keys already mapped, the
// positions beside them.
struct KeyRow {
  static constexpr int kVec = 4;
  const u32x4* data;
  int n;
  const int32_t* posv;
  __device__ uint32_t key(const u32x4& v, int e) const { return v[e]; }
  __device__ int pos(int idx) const { return posv[idx]; }
};
// The final list: positions.
struct ListOut {
  int32_t* out;
  __device__ void put(uint32_t slot, uint32_t, int pos) const { out[slot] = pos; }
};
// A segment's list: keys and positions, for the merge.
struct PairOut {
  uint32_t* key;
  int32_t* pos;
  __device__ void put(uint32_t slot, uint32_t k, int p) const {
    key[slot] = k;
    pos[slot] = p;
  }
};

// One tile of the list, in position order: V elements per thread (idx < 0:
// none); with T the k-th largest key and `ties` the number of keys == T to
// list, an element goes to slot (#keys > T before it) + min(#keys == T
// before it, ties) if its key is > T, or if it is one of the first `ties`
// keys == T.
template <int V, typename R, typename O>
__device__ __forceinline__ void emit_tile(BlockScan& bs, const R& row, const O& o,
                                          const uint32_t (&key)[V], const int (&idx)[V],
                                          uint32_t T, uint32_t ties, uint32_t& gt_base,
                                          uint32_t& eq_base) {
  uint32_t cg = 0, ce = 0;
#pragma unroll
  for (int e = 0; e < V; ++e) {
    cg += (idx[e] >= 0 && key[e] > T) ? 1u : 0u;
    ce += (idx[e] >= 0 && key[e] == T) ? 1u : 0u;
  }
  uint32_t tot;
  const uint32_t before = bs.exscan(cg | (ce << 16), &tot);   // < 2^16 per tile
  uint32_t gb = gt_base + (before & 0xffffu), eb = eq_base + (before >> 16);
#pragma unroll
  for (int e = 0; e < V; ++e) {
    if (idx[e] < 0) continue;
    if (key[e] > T) {
      o.put(gb + min(eb, ties), key[e], row.pos(idx[e]));
      ++gb;
    } else if (key[e] == T) {
      if (eb < ties) o.put(gb + eb, key[e], row.pos(idx[e]));
      ++eb;
    }
  }
  gt_base += tot & 0xffffu;
  eq_base += tot >> 16;
}

// ---- passes that stream the row from memory ---------------------------------
// (the histograms are clear and published by a barrier before the first)
template <typename R>
__device__ void stream_passes(Smem& s, const R& row, int first, Sel& st) {
  constexpr int kVec = R::kVec;
  const int nvec = (row.n + kVec - 1) / kVec;
#pragma unroll
  for (int pass = 0; pass < kPasses; ++pass) {
    if (pass < first) continue;
    const uint32_t dmask = (1u << kWidth[pass]) - 1u;
    for (int g = threadIdx.x; g < nvec; g += kThreads) {
      const u32x4 v = row.data[g];
#pragma unroll
      for (int e = 0; e < kVec; ++e)
        if (g * kVec + e < row.n) count_key(s.hist[pass], row.key(v, e), st, kShift[pass], dmask);
    }
    __syncthreads();
    pick_digit(s, s.hist[pass], kShift[pass], kWidth[pass], st);
  }
}

template <typename R, typename O>
__device__ void stream_emit(BlockScan& bs, const R& row, const O& o, const Sel& st, int k) {
  constexpr int kVec = R::kVec;
  const int nvec = (row.n + kVec - 1) / kVec;
  const uint32_t T = st.pval, ties = st.need, n_gt = (uint32_t)k - ties;
  uint32_t gt_base = 0, eq_base = 0;
  for (int g0 = 0; g0 < nvec; g0 += kThreads) {
    const int g = g0 + (int)threadIdx.x;
    const u32x4 v = g < nvec ? row.data[g] : u32x4{0u, 0u, 0u, 0u};
    uint32_t key[kVec];
    int idx[kVec];
#pragma unroll
    for (int e = 0; e < kVec; ++e) {
      key[e] = row.key(v, e);
      idx[e] = (g < nvec && g * kVec + e < row.n) ? g * kVec + e : -1;
    }
    emit_tile<kVec>(bs, row, o, key, idx, T, ties, gt_base, eq_base);
    if (gt_base == n_gt && eq_base >= ties) break;   // uniform: the list is complete
  }
}

// The whole row streamed (rows beyond the register capacity).
template <typename R, typename O>
__device__ void stream_select(Smem& s, const R& row, const O& o, int k) {
  BlockScan bs{s};
  Sel st{0u, 0u, (uint32_t)k};
  clear_hists(s);
  __syncthreads();
  stream_passes(s, row, 0, st);
  stream_emit(bs, row, o, st, k);
}

template <int SRC>
__device__ __forceinline__ const u32x4* row_ptr(const TopkParams& p, int r) {
  return reinterpret_cast<const u32x4*>(static_cast<const uint8_t*>(p.scores) +
                                        (int64_t)r * p.row_stride * (SRC == kDtFP32 ? 4 : 2));
}

// Registers of a thread for rows of up to KPT * 1024 elements: group j holds
// the kVec elements at (t + 1024 j) kVec ..; elements at and beyond row.n
// carry key 0, the lowest, which never reaches the list of a row with more
// than k elements.
template <typename R, int KPT>
struct RegKeys {
  static constexpr int kVec = R::kVec;
  static constexpr int kGroups = KPT / kVec;
  uint32_t key[kGroups][kVec];
  __device__ void load(const R& row) {
    const int last = max((row.n + kVec - 1) / kVec, 1) - 1;   // loads clamped to the last group
    u32x4 raw[kGroups];
#pragma unroll
    for (int j = 0; j < kGroups; ++j) raw[j] = row.data[min((int)threadIdx.x + j * kThreads, last)];
#pragma unroll
    for (int j = 0; j < kGroups; ++j)
#pragma unroll
      for (int e = 0; e < kVec; ++e)
        key[j][e] = ((int)threadIdx.x + j * kThreads) * kVec + e < row.n ? row.key(raw[j], e) : 0u;
  }
};

// One row held in registers, more than k elements: the first digit from
// registers, then the keys of its bin and above (the candidates) to LDS in
// position order and the remaining digits over them -- or, when the
// candidates overflow LDS (heavy ties), the remaining passes re-read the row.
template <typename R, int KPT, typename O>
__device__ __forceinline__ void select_row(Smem& s, uint32_t* s_cand, const RegKeys<R, KPT>& rk,
                                           const R& row, const O& o, int k) {
  uint32_t* s_key = s_cand;                              // candidates: keys, then indices
  int32_t* s_idx = reinterpret_cast<int32_t*>(s_cand + kCand);
  constexpr int kVec = R::kVec;
  constexpr int kGroups = KPT / kVec;
  const auto& key = rk.key;
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int w = (int)uniform(tid / kWave);
  BlockScan bs{s};
  clear_hists(s);
  for (int i = tid; i < 2 * kCand; i += kThreads) s_cand[i] = 0u;
  __syncthreads();

  // ---- first digit, from registers -------------------------------------------
  // Four histogram copies in the (not yet used) candidate buffer, lane l
  // counting into copy l mod 4 with its bins XOR-swizzled by the copy index:
  // lanes of one instruction that hit a hot bin land on different
  // addresses and banks.  The copies are summed into s.hist[0].
  Sel st{0u, 0u, (uint32_t)k};
  {
    const uint32_t cp = (uint32_t)lane & 3u;
    uint32_t* h4 = s_cand + cp * kBins;
#pragma unroll
    for (int j = 0; j < kGroups; ++j)
#pragma unroll
      for (int e = 0; e < kVec; ++e) atomicAdd(&h4[(key[j][e] >> kShift[0]) ^ cp], 1u);
  }
  __syncthreads();
  for (int b = tid; b < kBins; b += kThreads)
    s.hist[0][b] = s_cand[b] + s_cand[kBins + (b ^ 1)] + s_cand[2 * kBins + (b ^ 2)] +
                   s_cand[3 * kBins + (b ^ 3)];
  __syncthreads();
  const uint32_t bin0 = pick_digit(s, s.hist[0], kShift[0], kWidth[0], st);
  // keys with a top digit above d0 are all listed; d0's bin holds the rest
  const uint32_t lo = st.pval;                           // d0 << kShift[0]
  const uint32_t ncand = (uint32_t)k - st.need + bin0;
  if (ncand > (uint32_t)kCand) {                         // uniform
    stream_passes(s, row, 1, st);
    stream_emit(bs, row, o, st, k);
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
      uint32_t oo = start + ((wincl[j / 3] >> (10 * (j % 3))) & 0x3ffu) - cnt[j];
      const int base = (tid + j * kThreads) * kVec;
#pragma unroll
      for (int e = 0; e < kVec; ++e) {
        if (key[j][e] >= lo) {
          s_key[oo] = key[j][e];
          s_idx[oo] = base + e;
          ++oo;
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
  // four consecutive candidates per thread: one block scan covers the whole
  // candidate buffer (position order is thread order, then element order)
  const uint32_t T = st.pval, ties = st.need, n_gt = (uint32_t)k - ties;
  uint32_t gt_base = 0, eq_base = 0;
  constexpr int kPerThread = 4;
  for (int c0 = 0; c0 < (int)ncand; c0 += kPerThread * kThreads) {
    uint32_t kk[kPerThread];
    int ix[kPerThread];
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) {
      const int i = c0 + kPerThread * tid + e;
      kk[e] = i < (int)ncand ? s_key[i] : 0u;
      ix[e] = i < (int)ncand ? s_idx[i] : -1;
    }
    emit_tile<kPerThread>(bs, row, o, kk, ix, T, ties, gt_base, eq_base);
    if (gt_base == n_gt && eq_base >= ties) break;       // uniform
  }
}

// ---- kernels --------------------------------------------------------------------

// Rows beyond the register capacity, one workgroup each: every pass streams
// the row.
template <int SRC>
__global__ __launch_bounds__(kThreads) void topk_stream_kernel(TopkParams p) {
  __shared__ Smem s;
  const int r = blockIdx.x, k = p.topk;
  int32_t* out = p.out + (int64_t)r * k;
  const int n = min(max(p.row_len[r], 0), p.row_stride);
  if (n <= k) {
    for (int i = threadIdx.x; i < k; i += kThreads) out[i] = i < n ? i : -1;
    return;
  }
  stream_select(s, ScoreRow<SRC>{row_ptr<SRC>(p, r), n, 0}, ListOut{out}, k);
}

// Rows of up to KPT * 1024 scores, one workgroup each, two per CU (8 waves
// per SIMD, <= 64 registers).
template <int SRC, int KPT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(8, 8)))
void topk_cand_kernel(TopkParams p) {
  __shared__ Smem s;
  __shared__ uint32_t s_cand[2 * kCand];
  const int r = blockIdx.x, k = p.topk;
  int32_t* out = p.out + (int64_t)r * k;
  const int n = min(max(p.row_len[r], 0), p.row_stride);
  if (n <= k) {
    for (int i = threadIdx.x; i < k; i += kThreads) out[i] = i < n ? i : -1;
    return;
  }
  const ScoreRow<SRC> row{row_ptr<SRC>(p, r), n, 0};
  RegKeys<ScoreRow<SRC>, KPT> rk;
  rk.load(row);
  select_row(s, s_cand, rk, row, ListOut{out}, k);
}

// Long rows, stage 1: segment s (positions [s L, (s + 1) L)) of row r
// selects its own top k into the workspace -- keys and positions, in
// position order; a segment with at most k elements in play lists them all.
// The row's top k is among its segments' lists: an element that fewer than
// k elements of the row rank ahead of has fewer than k ahead of it in its
// segment too.
template <int SRC, int KPT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(8, 8)))
void topk_seg_kernel(TopkParams p) {
  __shared__ Smem s;
  __shared__ uint32_t s_cand[2 * kCand];
  const int seg = blockIdx.x, r = blockIdx.y, k = p.topk, L = p.seg_len;
  const int n = min(max(p.row_len[r], 0), p.row_stride);
  const int ns = min(max(n - seg * L, 0), L);
  if (ns == 0) return;
  const int64_t slot0 = (int64_t)r * p.row_slots + (int64_t)seg * k;
  const PairOut o{p.ws_key + slot0, p.ws_pos + slot0};
  const ScoreRow<SRC> row{row_ptr<SRC>(p, r) + (int64_t)seg * L / Src<SRC>::kVec, ns, seg * L};
  RegKeys<ScoreRow<SRC>, KPT> rk;
  rk.load(row);
  if (ns <= k) {                                         // the whole segment, in order
    constexpr int kVec = Src<SRC>::kVec;
#pragma unroll
    for (int j = 0; j < KPT / kVec; ++j)
#pragma unroll
      for (int e = 0; e < kVec; ++e) {
        const int idx = ((int)threadIdx.x + j * kThreads) * kVec + e;
        if (idx < ns) o.put(idx, rk.key[j][e], row.pos(idx));
      }
    return;
  }
  select_row(s, s_cand, rk, row, o, k);
}

// Long rows, stage 2: the segments' lists of row r, concatenated (every
// segment before the row's last non-empty one lists exactly k, so the
// concatenation is dense and in position order), hold the row's top k.
template <int KPT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(8, 8)))
void topk_merge_kernel(TopkParams p) {
  __shared__ Smem s;
  __shared__ uint32_t s_cand[2 * kCand];
  const int r = blockIdx.x, k = p.topk, L = p.seg_len;
  int32_t* out = p.out + (int64_t)r * k;
  const int n = min(max(p.row_len[r], 0), p.row_stride);
  const int full = n / L, tail = n - full * L;           // full segments, rest of the last
  const int m = full * k + min(tail, k);                 // listed elements (full * L >= full * k)
  const int64_t slot0 = (int64_t)r * p.row_slots;      // 16-byte aligned
  const KeyRow row{reinterpret_cast<const u32x4*>(p.ws_key + slot0), m, p.ws_pos + slot0};
  if (m <= k) {
    for (int i = threadIdx.x; i < k; i += kThreads) out[i] = i < m ? row.pos(i) : -1;
    return;
  }
  RegKeys<KeyRow, KPT> rk;
  rk.load(row);
  select_row(s, s_cand, rk, row, ListOut{out}, k);
}

}  // namespace

// Segment length for split selection of long rows (0: no split): the
// largest of 32768, 16384, 8192 that is at least 4 k and keeps the merged
// lists (segments x k) within the 32768 keys one workgroup holds (fewer,
// longer segments: a smaller merge; 40 decode rows of 131072 scores, top
// 2048: 34 us with 32K segments, 38 with 16K, 44 with 8K).
int topk_segment_len(int64_t row_stride, int32_t topk) {
  if (row_stride <= (int64_t)kMaxKPT * kThreads) return 0;
  for (int L = kMaxKPT * kThreads; L >= 8192; L /= 2) {
    const int64_t segs = (row_stride + L - 1) / L;
    if (L >= 4 * (int64_t)topk && segs * topk <= (int64_t)kMaxKPT * kThreads) return L;
  }
  return 0;
}

namespace {

template <int SRC>
hipError_t launch_src(const TopkParams& p, hipStream_t s) {
  const dim3 block(kThreads);
  const int64_t per_thread = ((int64_t)p.row_stride + kThreads - 1) / kThreads;
  if (p.seg_len > 0) {
    const int nseg = (int)((p.row_stride + p.seg_len - 1) / p.seg_len);
    const int kpt = p.seg_len / kThreads;
    const dim3 g1((unsigned)nseg, (unsigned)p.num_rows);
    if (kpt <= 8)
      topk_seg_kernel<SRC, 8><<<g1, block, 0, s>>>(p);
    else if (kpt <= 16)
      topk_seg_kernel<SRC, 16><<<g1, block, 0, s>>>(p);
    else
      topk_seg_kernel<SRC, kMaxKPT><<<g1, block, 0, s>>>(p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t merged = (int64_t)nseg * p.topk;
    const dim3 g2((unsigned)p.num_rows);
    if (merged <= 8 * kThreads)
      topk_merge_kernel<8><<<g2, block, 0, s>>>(p);
    else if (merged <= 16 * kThreads)
      topk_merge_kernel<16><<<g2, block, 0, s>>>(p);
    else
      topk_merge_kernel<kMaxKPT><<<g2, block, 0, s>>>(p);
    return hipGetLastError();
  }
  const dim3 grid((unsigned)p.num_rows);
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
