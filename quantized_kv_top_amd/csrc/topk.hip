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
// -0 folded onto +0, NaN to 0).  One workgroup of 1024 threads per row:
//   * the row is read once into registers and turned into keys;
//   * an LDS histogram of the top 11 key bits and a block scan over its bins
//     give the digit d0 of the k-th largest key;
//   * the keys whose top digit is at least d0 -- the k - (ties in d0) sure
//     ones and d0's whole bin, typically little more than k -- are copied to
//     LDS in position order;
//   * the remaining digits (11 + 10 bits for fp32 scores, 5 for fp16 / bf16)
//     are selected over those candidates only, which leaves the exact k-th
//     key T and the number of ties at T to take;
//   * a pass over the candidates in position order writes every position
//     with key > T and the first such ties (one block scan per 1024
//     candidates gives each thread how many of both lie before it).
// When d0's bin is too large for LDS (heavily tied scores) the remaining
// passes re-read the row instead (L2-resident by then); rows longer than the
// register capacity (32768 fp32 / 65536 fp16 or bf16 scores) stream every
// pass from memory.  The bound is the single read of the scores from HBM.
#include "qsakv_device.h"
#include "qsakv_internal.h"

namespace qsakv {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / kWave;
constexpr int kBins = 2048;      // 11-bit digits
constexpr int kCand = 4096;      // candidates kept in LDS after the first digit
constexpr int kMaxEPT = 8;       // 16-byte groups of the row per thread in registers

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

struct Smem {
  uint32_t hist[kBins];
  uint32_t tmp[2][kWaves];   // wave totals of the block scans, alternating
  uint32_t sel[3];           // the picked digit, the keys still needed, its bin's count
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

__device__ __forceinline__ void clear_hist(Smem& s) {
  for (int b = threadIdx.x; b < kBins; b += kThreads) s.hist[b] = 0u;
  __syncthreads();
}

__device__ __forceinline__ void count_key(Smem& s, uint32_t key, const Sel& st, int shift,
                                          uint32_t dmask) {
  if ((key & st.pmask) == st.pval) atomicAdd(&s.hist[(key >> shift) & dmask], 1u);
}

// s.hist holds the histogram of the digit at `shift` of the keys in play:
// find the digit of the need-th largest of them and narrow the state to it;
// returns the count of the picked digit's bin.  Thread t scans bins
// 2047 - 2t (upper) and 2046 - 2t, so the exclusive scan in thread order
// counts the keys in all higher bins.  s.hist is left as is.
__device__ __forceinline__ uint32_t pick_digit(Smem& s, BlockScan& bs, int shift, int width,
                                               Sel& st) {
  const int bhi = kBins - 1 - 2 * (int)threadIdx.x, blo = bhi - 1;
  const uint32_t chi = s.hist[bhi], clo = s.hist[blo];
  uint32_t tot;
  const uint32_t above = bs.exscan(chi + clo, &tot);
  if (above < st.need && st.need <= above + chi + clo) {
    const bool hi = st.need <= above + chi;
    s.sel[0] = (uint32_t)(hi ? bhi : blo);
    s.sel[1] = st.need - above - (hi ? 0u : chi);
    s.sel[2] = hi ? chi : clo;
  }
  __syncthreads();
  st.pval |= uniform(s.sel[0]) << shift;
  st.pmask |= ((1u << width) - 1u) << shift;
  st.need = uniform(s.sel[1]);
  // s.sel is next written after at least one more barrier (the next pick's
  // scan), when every thread has read it
  return uniform(s.sel[2]);
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
template <int SRC>
__device__ void stream_passes(Smem& s, BlockScan& bs, const u32x4* row, int n, int first,
                              Sel& st) {
  using K = Keys<SRC>;
  constexpr int kVec = K::kVec;
  const int nvec = (n + kVec - 1) / kVec;
#pragma unroll
  for (int pass = 0; pass < K::kPasses; ++pass) {
    if (pass < first) continue;
    const int shift = K::kShift[pass];
    const uint32_t dmask = (1u << K::kWidth[pass]) - 1u;
    clear_hist(s);
    for (int g = threadIdx.x; g < nvec; g += kThreads) {
      const u32x4 v = row[g];
#pragma unroll
      for (int e = 0; e < kVec; ++e)
        if (g * kVec + e < n) count_key(s, K::key(v, e), st, shift, dmask);
    }
    __syncthreads();
    pick_digit(s, bs, shift, K::kWidth[pass], st);
  }
}

template <int SRC>
__device__ void stream_emit(BlockScan& bs, const u32x4* row, int n, const Sel& st, int k,
                            int32_t* out) {
  using K = Keys<SRC>;
  constexpr int kVec = K::kVec;
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
      key[e] = K::key(v, e);
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
  stream_passes<SRC>(s, bs, row, n, 0, st);
  stream_emit<SRC>(bs, row, n, st, k, out);
}

// Two workgroups per CU (8 waves per SIMD, <= 64 registers) while the keys
// leave room: every fp32 row and 16-bit rows of up to 32768 scores; longer
// 16-bit rows run one workgroup per CU.
template <int SRC, int EPT>
constexpr int cand_waves() { return (SRC == kDtFP32 || EPT <= 4) ? 8 : 4; }

// Rows of up to EPT * 1024 16-byte groups: read once into registers (thread
// t holds groups t, t + 1024, ...), first digit from registers, then the
// candidates in LDS.
template <int SRC, int EPT>
__global__ __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(cand_waves<SRC, EPT>(), cand_waves<SRC, EPT>())))
void topk_cand_kernel(TopkParams p) {
  using K = Keys<SRC>;
  constexpr int kVec = K::kVec;
  constexpr bool kWide = SRC == kDtFP32;
  __shared__ Smem s;
  __shared__ uint32_t s_key[kCand];
  __shared__ int32_t s_pos[kCand];

  const int r = blockIdx.x, k = p.topk;
  const int tid = threadIdx.x;
  int32_t* out = p.out + (int64_t)r * k;
  const int n = min(max(p.row_len[r], 0), p.row_stride);
  if (list_all(n, k, out)) return;
  const u32x4* row = row_ptr<SRC>(p, r);
  const int nvec = (n + kVec - 1) / kVec;

  // keys: fp32 one per word; 16-bit two per word (element e of a group in
  // half e & 1 of word e >> 1)
  u32x4 kv[EPT];
#pragma unroll
  for (int j = 0; j < EPT; ++j) {
    const int g = tid + j * kThreads;
    kv[j] = g < nvec ? row[g] : u32x4{0u, 0u, 0u, 0u};
  }
#pragma unroll
  for (int j = 0; j < EPT; ++j)
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      if constexpr (kWide) {
        kv[j][w] = key_f32(kv[j][w]);
      } else {
        const uint32_t lo = K::key(kv[j], 2 * w), hi = K::key(kv[j], 2 * w + 1);
        kv[j][w] = lo | (hi << 16);
      }
    }
  auto key_at = [&](int j, int e) -> uint32_t {
    if constexpr (kWide) return kv[j][e];
    else return (kv[j][e >> 1] >> (16 * (e & 1))) & 0xffffu;
  };

  // ---- first digit, from registers -------------------------------------------
  BlockScan bs{s};
  Sel st{0u, 0u, (uint32_t)k};
  constexpr int kShift0 = K::kShift[0];
  clear_hist(s);
#pragma unroll
  for (int j = 0; j < EPT; ++j)
#pragma unroll
    for (int e = 0; e < kVec; ++e)
      if ((tid + j * kThreads) * kVec + e < n)
        count_key(s, key_at(j, e), st, kShift0, (1u << K::kWidth[0]) - 1u);
  __syncthreads();
  const uint32_t bin0 = pick_digit(s, bs, kShift0, K::kWidth[0], st);
  // keys with a top digit above d0 are all listed; d0's bin holds the rest
  const uint32_t lo = st.pval;                           // d0 << kShift0
  const uint32_t ncand = (uint32_t)k - st.need + bin0;
  if (ncand > (uint32_t)kCand) {                         // uniform
    stream_passes<SRC>(s, bs, row, n, 1, st);
    stream_emit<SRC>(bs, row, n, st, k, out);
    return;
  }

  // ---- candidates (top digit >= d0) to LDS, in position order ---------------
  uint32_t cbase = 0;
#pragma unroll
  for (int j = 0; j < EPT; ++j) {
    if (j * kThreads >= nvec) break;                     // uniform
    const int base = (tid + j * kThreads) * kVec;
    uint32_t c = 0;
#pragma unroll
    for (int e = 0; e < kVec; ++e) c += (base + e < n && key_at(j, e) >= lo) ? 1u : 0u;
    uint32_t tot;
    uint32_t o = cbase + bs.exscan(c, &tot);
#pragma unroll
    for (int e = 0; e < kVec; ++e) {
      const uint32_t key = key_at(j, e);
      if (base + e < n && key >= lo) {
        s_key[o] = key;
        s_pos[o] = base + e;
        ++o;
      }
    }
    cbase += tot;
  }
  __syncthreads();

  // ---- remaining digits over the candidates ----------------------------------
#pragma unroll
  for (int pass = 1; pass < K::kPasses; ++pass) {
    const int shift = K::kShift[pass];
    const uint32_t dmask = (1u << K::kWidth[pass]) - 1u;
    clear_hist(s);
    for (int i = tid; i < (int)ncand; i += kThreads) count_key(s, s_key[i], st, shift, dmask);
    __syncthreads();
    pick_digit(s, bs, shift, K::kWidth[pass], st);
  }

  // ---- the list ---------------------------------------------------------------
  const uint32_t T = st.pval, ties = st.need, n_gt = (uint32_t)k - ties;
  uint32_t gt_base = 0, eq_base = 0;
  for (int c0 = 0; c0 < (int)ncand; c0 += kThreads) {
    const int i = c0 + tid;
    const uint32_t key[1] = {i < (int)ncand ? s_key[i] : 0u};
    const int pos[1] = {i < (int)ncand ? s_pos[i] : -1};
    emit_tile<1>(bs, key, pos, T, ties, gt_base, eq_base, out);
    if (gt_base == n_gt && eq_base >= ties) break;       // uniform
  }
}

template <int SRC>
hipError_t launch_src(const TopkParams& p, hipStream_t s) {
  constexpr int kVec = Keys<SRC>::kVec;
  const dim3 grid((unsigned)p.num_rows), block(kThreads);
  const int64_t groups = ((int64_t)p.row_stride + kVec - 1) / kVec;
  if (groups <= 2 * kThreads)
    topk_cand_kernel<SRC, 2><<<grid, block, 0, s>>>(p);
  else if (groups <= 4 * kThreads)
    topk_cand_kernel<SRC, 4><<<grid, block, 0, s>>>(p);
  else if (groups <= kMaxEPT * kThreads)
    topk_cand_kernel<SRC, kMaxEPT><<<grid, block, 0, s>>>(p);
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
