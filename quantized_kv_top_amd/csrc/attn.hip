// Top-k sparse attention over a paged, quantized KV cache (gfx950).
//
// What is computed (per query row r, query head h, KV head g = h / G):
//   softmax attention of q[r][h] over the K/V rows of the positions listed in
//   topk_idx[r], gathered through the block table and dequantized exactly.
// This is the QSA read path of page "int8 per-(token,head) KV cache for the
// Qwen3.8-Flash-Next QSA path" (section "The finding worth upstreaming":
// scattered token rows are gathered per query row), with the E4M3 scale
// placement of page "[Perf][SM70][FP8] Hoist QSA E4M3 KV scales" (section
// "Changes": the K scale folds into the post-dot softmax factor, the V scale
// is applied once after normalization or after the split-K merge).
//
// Work decomposition
//   One workgroup (4 waves) per (row, KV head, split partition).  The
//   partition's list positions are cut into super-tiles of 64 positions,
//   dealt round-robin to the waves; each lane resolves one position to a
//   slot (index -> block table -> slot).  A super-tile is two 32-token
//   tiles; the K/V rows of the next tile are in flight (in registers) while
//   the current one is computed.
//
// Per 32-token tile, in MFMA 16x16x32 terms (GQA heads on the N side):
//   S^T[t][h] = K[t][:] . Q[h][:]          A = K rows (M = 16 tokens), B = Q^T
//   online softmax over the tile (log2 domain, running max per head)
//   O^T[d][h] += V^T[d][t] . W[t][h]       A = V^T (M = 16 d's), B = W
// so the row's G <= 16 query heads share every gathered K/V tile.  The int8
// and E4M3 codes become exact fp16 operands in registers; Q is rounded to
// fp16 after an exact power-of-two prescale; bf16 caches run bf16 MFMA.
// The int8 per-token K scale multiplies the logit after the dot product; the
// per-token V scale is folded into the softmax weight W = p * s_v / sigma,
// with sigma the running maximum V scale of the wave (kept exact by
// rescaling the accumulator by a power-free ratio when it grows).
#include "qsakv_device.h"
#include "qsakv_internal.h"

namespace qsakv {
namespace {

constexpr int kWaves = 4;
constexpr int kSuper = 64;   // list positions per super-tile (one per lane)
constexpr float kNegInf = -__builtin_inff();

template <int KIND, int D>
struct Geo {
  static constexpr bool kOneByte = KIND != kBF16;
  static constexpr int kDataBytes = kOneByte ? D : 2 * D;              // K or V row payload
  static constexpr int kRowBytes = KIND == kInt8Inline ? D + 4 : kDataBytes;
  static constexpr int kKChunks = kDataBytes / 64;                      // 16-B chunks / lane / token
  static constexpr int kVBytes = kDataBytes / 16;                       // bytes / lane / token
  static constexpr int kVWords = kVBytes / 4;
  static constexpr int kQK = D / 32;                                    // MFMAs per 16 tokens
  static constexpr int kPV = D / 16;                                    // MFMAs per tile
  static constexpr int kOut = D / 4;                                    // outputs per lane
};

// Raw gathered data of one 32-token tile, as held by one lane.
template <int KIND, int D>
struct TileRaw {
  using G = Geo<KIND, D>;
  u32x4 k[2][G::kKChunks];          // tokens ln16 and 16 + ln16
  uint32_t v[8][G::kVWords];        // tokens tok(grp, e), e = 0..7
  float sk[8], sv[8];               // int8 scales of tokens tok(grp, e)
  uint32_t valid;                   // bit e: token tok(grp, e) is attended
};

// Token (0..31 within the tile) held in k-slot e of lane group grp: the
// order in which the QK^T output of the two 16-token halves lands in a lane.
__device__ __forceinline__ int tok_of(int grp, int e) {
  return e < 4 ? 4 * grp + e : 16 + 4 * grp + (e - 4);
}

template <typename T>
__device__ __forceinline__ T ld(const uint8_t* p) { return *reinterpret_cast<const T*>(p); }

// Issue the loads of one tile.  `slot` is this lane's resolved slot of list
// position (super-tile base + lane); `half` selects positions 0..31 or 32..63.
template <int KIND, int D>
__device__ __forceinline__ void issue_tile(TileRaw<KIND, D>& t, const AttnParams& p, int g,
                                           int slot, int half) {
  using G = Geo<KIND, D>;
  const int lane = lane_id(), ln16 = lane & 15, grp = lane >> 4;
  const int hkv = p.num_kv_heads;
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int s = __shfl(slot, half * 32 + b * 16 + ln16);
    const int64_t row = ((int64_t)(s < 0 ? 0 : s) * hkv + g) * G::kRowBytes;
    const uint8_t* kr = p.k + row + 16 * grp;
#pragma unroll
    for (int c = 0; c < G::kKChunks; ++c) {
      if constexpr (KIND == kInt8Inline) {
        const uint32_t* w = reinterpret_cast<const uint32_t*>(kr + 64 * c);
        t.k[b][c] = u32x4{w[0], w[1], w[2], w[3]};
      } else {
        t.k[b][c] = ld<u32x4>(kr + 64 * c);
      }
    }
  }
  uint32_t valid = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int s = __shfl(slot, half * 32 + tok_of(grp, e));
    valid |= (s >= 0 ? 1u : 0u) << e;
    const int64_t rowi = (int64_t)(s < 0 ? 0 : s) * hkv + g;
    const uint8_t* vr = p.v + rowi * G::kRowBytes + ln16 * G::kVBytes;
    if constexpr (KIND == kInt8Inline) {  // 4-byte aligned rows: dword loads
      const uint32_t* wv = reinterpret_cast<const uint32_t*>(vr);
#pragma unroll
      for (int i = 0; i < G::kVWords; ++i) t.v[e][i] = wv[i];
    } else if constexpr (G::kVWords == 4) {
      const u32x4 w = ld<u32x4>(vr);
#pragma unroll
      for (int i = 0; i < 4; ++i) t.v[e][i] = w[i];
    } else if constexpr (G::kVWords == 2) {
      const u32x2 w = ld<u32x2>(vr);
      t.v[e][0] = w[0];
      t.v[e][1] = w[1];
    } else {  // 8 words (bf16, D = 256)
      const u32x4 w0 = ld<u32x4>(vr), w1 = ld<u32x4>(vr + 16);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        t.v[e][i] = w0[i];
        t.v[e][4 + i] = w1[i];
      }
    }
    if constexpr (KIND == kE4M3 || KIND == kBF16) {
      // a padding token reads row 0; clear its codes so that a NaN stored
      // there cannot reach the weighted sum (its weight is exactly 0)
#pragma unroll
      for (int i = 0; i < G::kVWords; ++i) t.v[e][i] = s < 0 ? 0u : t.v[e][i];
    }
    if constexpr (KIND == kInt8) {
      const float2 sc = *reinterpret_cast<const float2*>(p.kv_scale + rowi * 2);
      t.sk[e] = sc.x;
      t.sv[e] = sc.y;
    } else if constexpr (KIND == kInt8Inline) {
      t.sk[e] = *reinterpret_cast<const float*>(p.k + rowi * G::kRowBytes + D);
      t.sv[e] = *reinterpret_cast<const float*>(p.v + rowi * G::kRowBytes + D);
    }
  }
  t.valid = valid;
}

struct WaveState {
  float m;     // running max of the logits (log2 domain), per head
  float l;     // this lane's partial sum of exp2(logit - m)
  float sig;   // running max V scale (int8 kinds), wave-uniform
};

template <int KIND, int D>
using QOp = std::conditional_t<KIND == kBF16, bf16x8, f16x8>;

template <int KIND, int D>
__device__ __forceinline__ void compute_tile(const TileRaw<KIND, D>& t,
                                             const QOp<KIND, D> (&q)[Geo<KIND, D>::kQK],
                                             float kfac, WaveState& st,
                                             f32x4 (&o)[Geo<KIND, D>::kPV]) {
  using G = Geo<KIND, D>;
  // ---- S^T = K Q^T for the two 16-token halves --------------------------
  f32x4 s[2];
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    s[b] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < G::kQK; ++i) {
      if constexpr (KIND == kBF16) {
        s[b] = mfma16(bitcast<bf16x8>(t.k[b][i]), q[i], s[b]);
      } else {
        const u32x4& c = t.k[b][i >> 1];
        const uint32_t w0 = c[2 * (i & 1)], w1 = c[2 * (i & 1) + 1];
        const f16x8 a = (KIND == kE4M3) ? e4m3x8_to_f16(w0, w1) : i8x8_to_f16(w0, w1);
        s[b] = mfma16(a, q[i], s[b]);
      }
    }
  }
  // ---- online softmax in the log2 domain --------------------------------
  float y[8];
  float mx = kNegInf;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float raw = e < 4 ? s[0][e] : s[1][e - 4];
    float f = kfac;
    if constexpr (KIND == kInt8 || KIND == kInt8Inline) f *= t.sk[e];
    y[e] = ((t.valid >> e) & 1u) ? raw * f : kNegInf;
    mx = fmaxf(mx, y[e]);
  }
  mx = group4_max(mx);
  const float m_new = fmaxf(st.m, mx);
  const float m_use = m_new == kNegInf ? 0.f : m_new;
  const float alpha = __builtin_amdgcn_exp2f(st.m - m_use);
  float pr[8], psum = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    pr[e] = __builtin_amdgcn_exp2f(y[e] - m_use);
    psum += pr[e];
  }
  st.l = st.l * alpha + psum;
  st.m = m_new;

  float beta = alpha;
  float w[8];
  if constexpr (KIND == kInt8 || KIND == kInt8Inline) {
    float smax = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) smax = fmaxf(smax, ((t.valid >> e) & 1u) ? t.sv[e] : 0.f);
    smax = group4_max(smax);
    const float sig_new = fmaxf(st.sig, smax);
    const float rs = sig_new > 0.f ? 1.f / sig_new : 0.f;
    beta = alpha * (st.sig * rs);
    st.sig = sig_new;
#pragma unroll
    for (int e = 0; e < 8; ++e) w[e] = pr[e] * (t.sv[e] * rs);
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) w[e] = pr[e];
  }
  if (__any(beta != 1.f)) {
#pragma unroll
    for (int j = 0; j < G::kPV; ++j) o[j] *= beta;
  }
  // ---- O^T += V^T W -------------------------------------------------------
  if constexpr (KIND == kBF16) {
    bf16x8 bw;
#pragma unroll
    for (int e = 0; e < 8; ++e) bw[e] = (__bf16)w[e];
#pragma unroll
    for (int c = 0; c < G::kVWords; ++c) {
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        u32x4 a;
#pragma unroll
        for (int k = 0; k < 4; ++k)
          a[k] = perm(t.v[2 * k + 1][c], t.v[2 * k][c], hb ? 0x07060302u : 0x05040100u);
        o[2 * c + hb] = mfma16(bitcast<bf16x8>(a), bw, o[2 * c + hb]);
      }
    }
  } else {
    f16x8 bw;
#pragma unroll
    for (int e = 0; e < 8; ++e) bw[e] = (_Float16)w[e];
#pragma unroll
    for (int c = 0; c < G::kVWords; ++c) {
      // interleave the byte lanes of token pairs: tk[k][0] = (x0 y0 x1 y1),
      // tk[k][1] = (x2 y2 x3 y3) for x = token 2k, y = token 2k+1
      uint32_t tk[4][2];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        uint32_t x = t.v[2 * k][c], yv = t.v[2 * k + 1][c];
        if constexpr (KIND != kE4M3) {
          x ^= 0x80808080u;
          yv ^= 0x80808080u;
        }
        tk[k][0] = perm(yv, x, 0x05010400u);
        tk[k][1] = perm(yv, x, 0x07030602u);
      }
#pragma unroll
      for (int bb = 0; bb < 4; ++bb) {
        const int half = bb >> 1, hi = bb & 1;
        f16x8 a;
        if constexpr (KIND == kE4M3) {
          u32x4 r;
#pragma unroll
          for (int k = 0; k < 4; ++k)
            r[k] = hi ? e4m3pair_to_f16x2<true>(tk[k][half])
                      : e4m3pair_to_f16x2<false>(tk[k][half]);
          a = bitcast<f16x8>(r);
        } else {
          u32x4 r;
#pragma unroll
          for (int k = 0; k < 4; ++k) r[k] = i8pair_to_f16x2(tk[k][half], hi ? kSelB23 : kSelB01);
          a = sub1152(r);
        }
        o[4 * c + bb] = mfma16(a, bw, o[4 * c + bb]);
      }
    }
  }
}

template <int KIND, int D>
__global__ __launch_bounds__(kWaves * kWave) void qsa_attn_kernel(AttnParams p) {
  using G = Geo<KIND, D>;
  __shared__ float s_obuf[G::kOut * kWave];
  __shared__ float s_m[kWaves][16], s_l[kWaves][16], s_sig[kWaves];

  const int lane = lane_id(), ln16 = lane & 15, grp = lane >> 4;
  const int w = threadIdx.x >> 6;

  // ---- item: (row, KV head, partition); consecutive items share an XCD ----
  const int nitems = p.num_rows * p.num_kv_heads * p.num_splits;
  int item;
  {
    const int b = blockIdx.x, x = b & 7, k = b >> 3;
    const int q8 = nitems >> 3, rem = nitems & 7;
    item = x * q8 + (x < rem ? x : rem) + k;
  }
  const int part = item % p.num_splits;
  const int rg = item / p.num_splits;
  const int g = rg % p.num_kv_heads;
  const int r = rg / p.num_kv_heads;
  const int pbeg = min(part * p.chunk, p.topk);
  const int pend = min(pbeg + p.chunk, p.topk);
  const int seq = p.row_seq[r];
  const bool seq_ok = seq >= 0 && seq < p.num_seqs;
  const int npos = seq_ok ? pend - pbeg : 0;
  const int32_t* idx_row = p.topk_idx + (int64_t)r * p.topk + pbeg;
  const int32_t* bt_row = p.block_table + (int64_t)(seq_ok ? seq : 0) * p.bt_stride;
  const int bs_mask = (1 << p.log2_bs) - 1;

  // ---- Q operand (B of QK^T) and the logit factor -------------------------
  const bool head_ok = ln16 < p.group;
  const int hq = g * p.group + ln16;
  QOp<KIND, D> qop[G::kQK];
  float kfac;
  {
    const int64_t qoff = ((int64_t)r * p.num_q_heads + (head_ok ? hq : 0)) * D;
    const uint16_t* qrow = static_cast<const uint16_t*>(p.q) + qoff;
    u32x4 raw[G::kQK];
#pragma unroll
    for (int i = 0; i < G::kQK; ++i) {
      const int d0 = G::kOneByte ? 64 * (i >> 1) + 16 * grp + 8 * (i & 1) : 32 * i + 8 * grp;
      raw[i] = head_ok ? *reinterpret_cast<const u32x4*>(qrow + d0) : u32x4{0, 0, 0, 0};
    }
    if constexpr (KIND == kBF16) {
#pragma unroll
      for (int i = 0; i < G::kQK; ++i) qop[i] = bitcast<bf16x8>(raw[i]);
      kfac = p.sm_log2e;
    } else if (p.q_dtype == kDtFP16) {
#pragma unroll
      for (int i = 0; i < G::kQK; ++i) qop[i] = bitcast<f16x8>(raw[i]);
      kfac = p.sm_log2e * p.k_scale;
    } else {
      // bf16 queries: exact power-of-two prescale so max|q| lands in
      // [2^14, 2^15), then round to fp16 (exact for every element >= 2^-14
      // after scaling; smaller ones keep an absolute error <= 2^-25).
      float amax = 0.f;
#pragma unroll
      for (int i = 0; i < G::kQK; ++i)
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          amax = fmaxf(amax, fabsf(__uint_as_float(raw[i][k] << 16)));
          amax = fmaxf(amax, fabsf(__uint_as_float(raw[i][k] & 0xFFFF0000u)));
        }
      amax = group4_max(amax);
      int ex = 0;
      if (amax > 0.f) frexpf(amax, &ex);
      int e = amax > 0.f ? 15 - ex : 0;
      e = e > 127 ? 127 : (e < -126 ? -126 : e);
      const float sc = ldexpf(1.f, e);
#pragma unroll
      for (int i = 0; i < G::kQK; ++i) {
        f16x8 h;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          h[2 * k] = (_Float16)(__uint_as_float(raw[i][k] << 16) * sc);
          h[2 * k + 1] = (_Float16)(__uint_as_float(raw[i][k] & 0xFFFF0000u) * sc);
        }
        qop[i] = h;
      }
      kfac = p.sm_log2e * p.k_scale * ldexpf(1.f, -e);
    }
  }

  // ---- the wave's super-tiles ---------------------------------------------
  const int nsuper = (npos + kSuper - 1) / kSuper;
  const int my_n = nsuper > w ? (nsuper - w + kWaves - 1) / kWaves : 0;
  auto load_pos = [&](int k) -> int {
    if (k >= my_n) return -1;
    const int j = (w + kWaves * k) * kSuper + lane;
    return j < npos ? idx_row[j] : -1;
  };
  auto load_blk = [&](int pos) -> int {
    if (pos < 0) return -1;
    const int lb = pos >> p.log2_bs;
    return lb < p.bt_stride ? bt_row[lb] : -1;
  };
  auto make_slot = [&](int pos, int blk) -> int {
    return (blk >= 0 && blk < p.num_blocks) ? (blk << p.log2_bs) + (pos & bs_mask) : -1;
  };

  WaveState st{kNegInf, 0.f, 0.f};
  f32x4 o[G::kPV];
#pragma unroll
  for (int j = 0; j < G::kPV; ++j) o[j] = f32x4{0.f, 0.f, 0.f, 0.f};

  if (my_n > 0) {
    TileRaw<KIND, D> ta, tb;
    int pos1 = load_pos(1);
    int pos0 = load_pos(0);
    int slot = make_slot(pos0, load_blk(pos0));
    issue_tile<KIND, D>(ta, p, g, slot, 0);
    int blk1 = load_blk(pos1);
    int pos2 = load_pos(2);
    issue_tile<KIND, D>(tb, p, g, slot, 1);
    for (int k = 0; k < my_n; ++k) {
      compute_tile<KIND, D>(ta, qop, kfac, st, o);
      const bool more = k + 1 < my_n;
      if (more) {
        slot = make_slot(pos1, blk1);
        issue_tile<KIND, D>(ta, p, g, slot, 0);
      }
      const int blk2 = load_blk(pos2);
      const int pos3 = load_pos(k + 3);
      compute_tile<KIND, D>(tb, qop, kfac, st, o);
      if (more) issue_tile<KIND, D>(tb, p, g, slot, 1);
      pos1 = pos2;
      blk1 = blk2;
      pos2 = pos3;
    }
  }

  // ---- merge the waves' partial results -----------------------------------
  const float l_h = group4_sum(st.l);
  if (grp == 0) {
    s_m[w][ln16] = st.m;
    s_l[w][ln16] = l_h;
  }
  if (lane == 0) s_sig[w] = st.sig;
  __syncthreads();
  float M = kNegInf;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) M = fmaxf(M, s_m[i][ln16]);
  float L = 0.f, myf = 0.f;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) {
    const float mi = s_m[i][ln16];
    const float f = mi == kNegInf ? 0.f : __builtin_amdgcn_exp2f(mi - M);
    L += f * s_l[i][ln16];
    if (i == w) myf = f;
  }
  if constexpr (KIND == kInt8 || KIND == kInt8Inline) myf *= st.sig;
  for (int i = 0; i < kWaves - 1; ++i) {
    if (w == i) {
#pragma unroll
      for (int j = 0; j < G::kPV; ++j)
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int idx = (j * 4 + k) * kWave + lane;
          const float v = myf * o[j][k];
          s_obuf[idx] = i == 0 ? v : s_obuf[idx] + v;
        }
    }
    __syncthreads();
  }
  if (w != kWaves - 1) return;
#pragma unroll
  for (int j = 0; j < G::kPV; ++j)
#pragma unroll
    for (int k = 0; k < 4; ++k) o[j][k] = s_obuf[(j * 4 + k) * kWave + lane] + myf * o[j][k];

  // lane (ln16, grp) holds d = (D/16) * (4*grp + k) + j for k < 4, j < D/16:
  // D/4 contiguous outputs starting at (D/4) * grp.
  const int64_t orow = (int64_t)r * p.num_q_heads + hq;
  if (p.num_splits == 1) {
    if (!head_ok) return;
    const bool any = L > 0.f;
    const float inv = any ? p.v_scale / L : 0.f;
    if (p.lse && grp == 0) p.lse[orow] = any ? (M + __log2f(L)) * kLn2 : kNegInf;
    float vals[G::kOut];
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
      for (int j = 0; j < G::kPV; ++j) vals[k * G::kPV + j] = o[j][k] * inv;
    const int64_t ob = orow * D + G::kOut * grp;
    if (p.out_dtype == kDtFP32) {
      float4* dst = reinterpret_cast<float4*>(static_cast<float*>(p.out) + ob);
#pragma unroll
      for (int i = 0; i < G::kOut / 4; ++i)
        dst[i] = float4{vals[4 * i], vals[4 * i + 1], vals[4 * i + 2], vals[4 * i + 3]};
    } else if (p.out_dtype == kDtBF16) {
      u32x4* dst = reinterpret_cast<u32x4*>(static_cast<uint16_t*>(p.out) + ob);
#pragma unroll
      for (int i = 0; i < G::kOut / 8; ++i) {
        u32x4 v;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          bf16x2 b;
          b[0] = (__bf16)vals[8 * i + 2 * k];
          b[1] = (__bf16)vals[8 * i + 2 * k + 1];
          v[k] = bitcast<uint32_t>(b);
        }
        dst[i] = v;
      }
    } else {
      u32x4* dst = reinterpret_cast<u32x4*>(static_cast<uint16_t*>(p.out) + ob);
#pragma unroll
      for (int i = 0; i < G::kOut / 8; ++i) {
        u32x4 v;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          f16x2 h;
          h[0] = (_Float16)vals[8 * i + 2 * k];
          h[1] = (_Float16)vals[8 * i + 2 * k + 1];
          v[k] = bitcast<uint32_t>(h);
        }
        dst[i] = v;
      }
    }
  } else {
    if (!head_ok) return;
    const int64_t pi = orow * p.num_splits + part;
    if (grp == 0) {
      p.ws_ml[2 * pi] = M;
      p.ws_ml[2 * pi + 1] = L;
    }
    float4* dst = reinterpret_cast<float4*>(p.ws_o + pi * D + G::kOut * grp);
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
      for (int j4 = 0; j4 < G::kPV / 4; ++j4)
        dst[(k * G::kPV) / 4 + j4] =
            float4{o[4 * j4][k], o[4 * j4 + 1][k], o[4 * j4 + 2][k], o[4 * j4 + 3][k]};
  }
}

// Log-sum-exp merge of the split-K partials of one (row, head) per wave:
// M = max M_p, L = sum L_p 2^(M_p - M), out = sum o_p 2^(M_p - M) / L, times
// the E4M3 V scale (applied once, after the merge).
template <int D>
__global__ __launch_bounds__(kWave) void qsa_merge_kernel(AttnParams p) {
  constexpr int E = D / kWave;
  const int lane = lane_id();
  const int64_t rh = blockIdx.x;   // r * Hq + h
  const int P = p.num_splits;
  const int64_t base = rh * P;
  float mp = kNegInf, lp = 0.f;
  if (lane < P) {
    mp = p.ws_ml[2 * (base + lane)];
    lp = p.ws_ml[2 * (base + lane) + 1];
  }
  const float M = wave_max(mp);
  const float f = (mp == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(mp - M);
  const float L = wave_sum(f * lp);
  float acc[E];
#pragma unroll
  for (int i = 0; i < E; ++i) acc[i] = 0.f;
  for (int q = 0; q < P; ++q) {
    const float fq = __shfl(f, q);
    const float* src = p.ws_o + (base + q) * D + lane * E;
    if constexpr (E == 4) {
      const float4 v = *reinterpret_cast<const float4*>(src);
      acc[0] += fq * v.x; acc[1] += fq * v.y; acc[2] += fq * v.z; acc[3] += fq * v.w;
    } else {
      const float2 v = *reinterpret_cast<const float2*>(src);
      acc[0] += fq * v.x; acc[1] += fq * v.y;
    }
  }
  const bool any = L > 0.f;
  const float inv = any ? p.v_scale / L : 0.f;
  if (p.lse && lane == 0) p.lse[rh] = any ? (M + __log2f(L)) * kLn2 : kNegInf;
  const int64_t ob = rh * D + lane * E;
  if (p.out_dtype == kDtFP32) {
    float* dst = static_cast<float*>(p.out) + ob;
#pragma unroll
    for (int i = 0; i < E; ++i) dst[i] = acc[i] * inv;
  } else if (p.out_dtype == kDtBF16) {
    __bf16* dst = static_cast<__bf16*>(p.out) + ob;
#pragma unroll
    for (int i = 0; i < E; ++i) dst[i] = (__bf16)(acc[i] * inv);
  } else {
    _Float16* dst = static_cast<_Float16*>(p.out) + ob;
#pragma unroll
    for (int i = 0; i < E; ++i) dst[i] = (_Float16)(acc[i] * inv);
  }
}

template <int KIND>
hipError_t launch_kind(int head_dim, const AttnParams& p, hipStream_t s) {
  const unsigned grid = (unsigned)(p.num_rows * p.num_kv_heads * p.num_splits);
  const dim3 block(kWaves * kWave);
  if (head_dim == 256)
    qsa_attn_kernel<KIND, 256><<<grid, block, 0, s>>>(p);
  else
    qsa_attn_kernel<KIND, 128><<<grid, block, 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn(int kind, int head_dim, const AttnParams& p, hipStream_t s) {
  switch (kind) {
    case kInt8: return launch_kind<kInt8>(head_dim, p, s);
    case kInt8Inline: return launch_kind<kInt8Inline>(head_dim, p, s);
    case kE4M3: return launch_kind<kE4M3>(head_dim, p, s);
    default: return launch_kind<kBF16>(head_dim, p, s);
  }
}

hipError_t launch_merge(int head_dim, const AttnParams& p, hipStream_t s) {
  const unsigned grid = (unsigned)(p.num_rows * p.num_q_heads);
  if (head_dim == 256)
    qsa_merge_kernel<256><<<grid, dim3(kWave), 0, s>>>(p);
  else
    qsa_merge_kernel<128><<<grid, dim3(kWave), 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace qsakv
