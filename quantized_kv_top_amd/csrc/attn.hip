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
//   One workgroup per (row, KV head, split partition), of 1, 2, 4 or 8
//   waves by launch size (see launch_kd).  The
//   workgroup first resolves the partition's positions to slots (index ->
//   block table -> slot) into LDS, then its waves take the partition's
//   tiles of 16 tokens round-robin, keeping kDepth tiles of gathered rows in
//   registers: kDepth - 1 in flight while one is computed.  Waves merge in
//   LDS in a fixed order (bitwise reproducible).  With several partitions,
//   each writes an unnormalized partial and a second, small launch merges
//   them (log-sum-exp).
//
// Per tile, in MFMA 16x16 terms with the row's G <= 16 query heads on N:
//   S^T[t][h] = K[t][:] . Q[h][:]          A = K rows (M = 16 tokens), B = Q^T
//   online softmax over the tile (log2 domain, running max per head)
//   O^T[d][h] += V^T[d][t] . W[t][h]       A = V^T (M = 16 d's), B = W
// so the G query heads share every gathered K/V tile.  The QK^T output of a
// 16-token tile gives each lane 4 tokens of one head, which is exactly the
// B operand of the K = 16 PV MFMA.
//
// Exact operands.  E4M3 codes become fp16 through gfx950's OCP-FP8 convert.
// An int8 code q becomes the fp16 value 1152 + q (0x64 in the high byte and
// q + 128 in the low byte -- exact, one byte permute per pair), then q itself
// by a packed fp16 subtract of 1152 (exact).  With the offset left in, the
// fp32 accumulators would carry 1152 * sum(Q) (logits) and 1152 * sum(W)
// (outputs) -- terms that can dwarf the signal (outlier keys with
// nonzero-mean queries; concentrated weights over small outputs) and whose
// rounding would land on it.  Queries are rounded to fp16 after an exact
// power-of-two prescale; bf16 caches run bf16 MFMA directly (their query
// operand staged in LDS at D = 256, where the registers go to the tiles in
// flight).
//
// Scales.  The int8 per-token K scale multiplies the logit after the dot
// product; the per-token V scale enters the softmax weight
// W = p * s_v / sigma (sigma a running reference V scale).  The running max
// m and sigma are only moved when a tile exceeds them by 2^8 (m) or 16x
// (sigma): weights stay below 2^12, far inside fp16, and the accumulator is
// rescaled only on those rare moves.
#include "qsakv_device.h"
#include "qsakv_internal.h"

namespace qsakv {
namespace {

// list positions each thread resolves per LDS batch: 1024 per batch, at
// most 4 per thread (more would cost registers at one wave per workgroup)
template <int NW>
constexpr int pos_per_thread() { return 1024 / (NW * 64) < 4 ? 1024 / (NW * 64) : 4; }

constexpr float kNegInf = -__builtin_inff();
constexpr float kMaxSlack = 8.f;      // log2 units the running max may lag behind
constexpr float kSigSlack = 16.f;     // factor sigma may lag behind a tile's V scale

typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

template <int KIND, int D, int TT>
struct Geo {
  static_assert(TT == 16, "tiles are 16 tokens: one MFMA block of K rows");
  static constexpr bool kOneByte = KIND == kInt8 || KIND == kInt8Inline || KIND == kE4M3;
  static constexpr bool kFp4 = KIND == kNvfp4;                          // two codes per byte
  static constexpr bool kInt = KIND == kInt8 || KIND == kInt8Inline;
  static constexpr int kDataBytes = kFp4 ? D / 2 : kOneByte ? D : 2 * D;   // K or V row payload
  static constexpr int kRowBytes = KIND == kInt8Inline ? D + 4 : kDataBytes;
  static constexpr int kKChunks = kDataBytes / 64;                      // 16-B chunks / lane / token
  static constexpr int kVBytes = kDataBytes / 16;                       // bytes / lane / token
  static constexpr int kVWords = kVBytes / 4;
  static constexpr int kBlkScales = D / 16;                             // NVFP4 block scales / row
  static constexpr int kQK = D / 32;                                    // MFMAs per 16 tokens
  static constexpr int kPV = D / 16;                                    // PV MFMAs per tile
  static constexpr int kOut = D / 4;                                    // outputs per lane
  static constexpr int kBlk = TT / 16;                                  // 16-token blocks
  // bf16 at D = 256: the query operand (32 registers) lives in LDS so that
  // 16-token tiles fit two waves per SIMD
  static constexpr bool kQLds = KIND == kBF16 && D == 256;
  static constexpr int kTok = TT / 4;                                   // V tokens per lane
  // tiles held in registers per wave: one in flight while one is computed
  static constexpr int kDepth = 2;
};

// Raw gathered data of one tile, as held by one lane.
template <int KIND, int D, int TT>
struct TileRaw {
  using G = Geo<KIND, D, TT>;
  u32x4 k[G::kBlk][G::kKChunks];    // tokens 16 b + ln16
  uint32_t v[G::kTok][G::kVWords];  // tokens tok(grp, e)
  float sk[G::kTok], sv[G::kTok];   // int8 scales of tokens tok(grp, e)
  // NVFP4: K block-scale codes of token 16 b + ln16, chunk c's pair in the
  // low 16 bits (byte i = block 2 grp + 8 c + i); the V block-scale code of
  // token tok(grp, e).  Held as loaded: no arithmetic touches a load result
  // before the tile is computed, so issuing a tile never waits for it.
  uint32_t ksc[G::kBlk][G::kFp4 ? G::kKChunks : 1];
  uint32_t vsc[G::kFp4 ? G::kTok : 1];
  uint32_t valid;                   // bit e: token tok(grp, e) is attended
};

template <typename T>
__device__ __forceinline__ T ld(const uint8_t* p) { return *reinterpret_cast<const T*>(p); }

// Issue the loads of one tile whose resolved slots (-1 = padding) are
// ts[0..TT) in LDS.  Lane (ln16, grp) gathers the K rows of tokens 16 b +
// ln16 (16 bytes per 64-byte chunk) and the V rows and scales of tokens
// 4 grp .. 4 grp + 3 (+16): the k-slot order in which the QK^T output of a
// 16-token block lands in a lane.
template <int KIND, int D, int TT>
__device__ __forceinline__ void issue_tile(TileRaw<KIND, D, TT>& t, const AttnParams& p, int g,
                                           const int* ts) {
  using G = Geo<KIND, D, TT>;
  const int lane = lane_id(), ln16 = lane & 15, grp = lane >> 4;
  const int hkv = p.num_kv_heads;
#pragma unroll
  for (int b = 0; b < G::kBlk; ++b) {
    const int s = ts[b * 16 + ln16];
    const int64_t row = ((int64_t)(s < 0 ? 0 : s) * hkv + g) * G::kRowBytes;
    const uint8_t* kr = p.k + row + 16 * grp;
#pragma unroll
    for (int c = 0; c < G::kKChunks; ++c) {
      if constexpr (KIND == kInt8Inline) {   // 4-byte aligned rows: dword loads
        const uint32_t* w = reinterpret_cast<const uint32_t*>(kr + 64 * c);
        t.k[b][c] = u32x4{w[0], w[1], w[2], w[3]};
      } else {
        t.k[b][c] = ld<u32x4>(kr + 64 * c);
      }
    }
    if constexpr (G::kFp4) {
      // chunk c of this lane holds the codes of blocks 2 grp + 8 c and + 1
      const uint8_t* sr = reinterpret_cast<const uint8_t*>(p.kv_scale) +
                          ((int64_t)(s < 0 ? 0 : s) * hkv + g) * 2 * G::kBlkScales + 2 * grp;
#pragma unroll
      for (int c = 0; c < G::kKChunks; ++c) t.ksc[b][c] = ld<uint16_t>(sr + 8 * c);
    }
  }
  int vs[G::kTok];
  {
    const int4 s0 = *reinterpret_cast<const int4*>(ts + 4 * grp);
    vs[0] = s0.x; vs[1] = s0.y; vs[2] = s0.z; vs[3] = s0.w;
  }
  uint32_t valid = 0;
#pragma unroll
  for (int e = 0; e < G::kTok; ++e) {
    const int s = vs[e];
    valid |= (s >= 0 ? 1u : 0u) << e;
    const int64_t rowi = (int64_t)(s < 0 ? 0 : s) * hkv + g;
    const uint8_t* vr = p.v + rowi * G::kRowBytes + ln16 * G::kVBytes;
    if constexpr (KIND == kInt8Inline) {
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
    } else if constexpr (G::kVWords == 1) {  // NVFP4, D = 128
      t.v[e][0] = ld<uint32_t>(vr);
    } else {  // 8 words (bf16, D = 256)
      const u32x4 w0 = ld<u32x4>(vr), w1 = ld<u32x4>(vr + 16);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        t.v[e][i] = w0[i];
        t.v[e][4 + i] = w1[i];
      }
    }
    if constexpr (G::kFp4) {
      // the lane's D/16 values of the row form block ln16 * kVBytes / 8
      // (a padding token reads row 0's; cleared where the tile is computed)
      t.vsc[e] = reinterpret_cast<const uint8_t*>(p.kv_scale)[(rowi * 2 + 1) * G::kBlkScales +
                                                               ln16 * G::kVBytes / 8];
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
  float m;     // running max in use (log2 domain), per head
  float l;     // this lane's partial sum of exp2(logit - m)
  float sig;   // reference V scale (int8 kinds), wave-uniform
  float rsig;  // 1 / sig (0 while sig is 0)
};

template <int KIND>
using QOp = std::conditional_t<KIND == kBF16, bf16x8, f16x8>;

// Where a tile reads the query operand (B of QK^T) from: the wave's
// registers, or -- where the registers are needed for the tiles in flight
// -- the workgroup's copy in LDS.
template <int KIND, int N>
struct QRegs {
  QOp<KIND> v[N];
  __device__ __forceinline__ QOp<KIND> operator[](int i) const { return v[i]; }
};
template <int KIND>
struct QLds {
  const QOp<KIND>* p;   // this lane's first vector; vectors are kWave apart
  __device__ __forceinline__ QOp<KIND> operator[](int i) const { return p[i * kWave]; }
};

// Byte lanes of the token pair (x, y) interleaved: tk[0] = (x0 y0 x1 y1),
// tk[1] = (x2 y2 x3 y3); int8 codes are biased to q + 128 on the way.
template <int KIND>
__device__ __forceinline__ void interleave_pair(uint32_t x, uint32_t y, uint32_t (&tk)[2]) {
  tk[0] = perm(y, x, 0x05010400u);
  tk[1] = perm(y, x, 0x07030602u);
  if constexpr (KIND != kE4M3) {
    tk[0] ^= 0x80808080u;
    tk[1] ^= 0x80808080u;
  }
}
// The fp16 pair (x_j, y_j) for byte j = bb of the interleaved words.
template <int KIND>
__device__ __forceinline__ uint32_t v_pair_f16(const uint32_t (&tk)[2], int bb) {
  const int half = bb >> 1, hi = bb & 1;
  if constexpr (KIND == kE4M3)
    return hi ? e4m3pair_to_f16x2<true>(tk[half]) : e4m3pair_to_f16x2<false>(tk[half]);
  else
    return i8pair_unbias(i8pair_to_f16x2(tk[half], hi ? kSelB23 : kSelB01));
}

template <int KIND, int D, int TT, typename QS>
__device__ __forceinline__ void compute_tile(const TileRaw<KIND, D, TT>& t, const QS& q,
                                             float kfac, WaveState& st,
                                             f32x4 (&o)[Geo<KIND, D, TT>::kPV]) {
  using G = Geo<KIND, D, TT>;
  constexpr int NT = G::kTok;
  // an LDS-resident query is read again for every tile (not kept live in
  // registers across the loop)
  if constexpr (G::kQLds) __asm__ volatile("" ::: "memory");
  // ---- S^T = K Q^T for the 16-token blocks -------------------------------
  f32x4 s[G::kBlk];
#pragma unroll
  for (int b = 0; b < G::kBlk; ++b) {
    s[b] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < G::kQK; ++i) {
      if constexpr (KIND == kBF16) {
        s[b] = mfma16(bitcast<bf16x8>(t.k[b][i]), q[i], s[b]);
      } else if constexpr (G::kFp4) {
        // step i: word i & 3 of chunk i >> 2 (8 codes), block 2 grp + 8 (i >> 2)
        // + ((i & 3) >> 1); operand = E2M1 value x block scale, exact in fp16
        const uint32_t w = t.k[b][i >> 2][i & 3];
        const uint32_t scb = (t.ksc[b][i >> 2] >> (8 * ((i & 3) >> 1))) & 0xFFu;
        const f16x2 sc2 = bitcast<f16x2>(e4m3pair_to_f16x2<false>(scb | (scb << 8)));
        u32x4 a;
        a[0] = bitcast<uint32_t>(bitcast<f16x2>(e2m1pair_to_f16x2<0>(w)) * sc2);
        a[1] = bitcast<uint32_t>(bitcast<f16x2>(e2m1pair_to_f16x2<1>(w)) * sc2);
        a[2] = bitcast<uint32_t>(bitcast<f16x2>(e2m1pair_to_f16x2<2>(w)) * sc2);
        a[3] = bitcast<uint32_t>(bitcast<f16x2>(e2m1pair_to_f16x2<3>(w)) * sc2);
        s[b] = mfma16(bitcast<f16x8>(a), q[i], s[b]);
      } else {
        const u32x4& c = t.k[b][i >> 1];
        const uint32_t w0 = c[2 * (i & 1)], w1 = c[2 * (i & 1) + 1];
        u32x4 a;
        if constexpr (KIND == kE4M3) {
          a[0] = e4m3pair_to_f16x2<false>(w0);
          a[1] = e4m3pair_to_f16x2<true>(w0);
          a[2] = e4m3pair_to_f16x2<false>(w1);
          a[3] = e4m3pair_to_f16x2<true>(w1);
        } else {
          // 1152 + q by byte permute, then the 1152 taken off in fp16 (exact
          // for every code): the operand is q itself, so each logit's
          // accumulation error scales with its own products and not with
          // 1152 times the query's sum over the head dimension
          const uint32_t x0 = w0 ^ 0x80808080u, x1 = w1 ^ 0x80808080u;
          a[0] = i8pair_unbias(i8pair_to_f16x2(x0, kSelB01));
          a[1] = i8pair_unbias(i8pair_to_f16x2(x0, kSelB23));
          a[2] = i8pair_unbias(i8pair_to_f16x2(x1, kSelB01));
          a[3] = i8pair_unbias(i8pair_to_f16x2(x1, kSelB23));
        }
        s[b] = mfma16(bitcast<f16x8>(a), q[i], s[b]);
      }
    }
  }
  // ---- online softmax in the log2 domain --------------------------------
  float y[NT];
  float mx = kNegInf;
#pragma unroll
  for (int e = 0; e < NT; ++e) {
    const float raw = s[e >> 2][e & 3];
    float f = kfac;
    if constexpr (G::kInt) f *= t.sk[e];
    y[e] = ((t.valid >> e) & 1u) ? raw * f : kNegInf;
    mx = fmaxf(mx, y[e]);
  }
  mx = group4_max(mx);
  float alpha = 1.f;
  if (mx > st.m + kMaxSlack) {           // the running max moves (rare)
    alpha = __builtin_amdgcn_exp2f(st.m - mx);
    st.m = mx;
  }
  const float m_use = st.m == kNegInf ? 0.f : st.m;
  float pr[NT], psum = 0.f;
#pragma unroll
  for (int e = 0; e < NT; ++e) {
    pr[e] = __builtin_amdgcn_exp2f(y[e] - m_use);
    psum += pr[e];
  }
  st.l = st.l * alpha + psum;

  float beta = alpha;
  float w[NT];
  if constexpr (G::kInt) {
    float smax = 0.f;
#pragma unroll
    for (int e = 0; e < NT; ++e) smax = fmaxf(smax, ((t.valid >> e) & 1u) ? t.sv[e] : 0.f);
    smax = group4_max(smax);
    if (smax > st.sig * kSigSlack) {     // the reference V scale moves (rare)
      beta *= st.sig / smax;
      st.sig = smax;
      st.rsig = 1.f / smax;
    }
    const float rs = st.rsig;
#pragma unroll
    for (int e = 0; e < NT; ++e) {
      // A padding token reads row 0's scale: it is replaced by 0 (a NaN or
      // inf stored there would otherwise turn the zero weight into NaN).
      const float sv = ((t.valid >> e) & 1u) ? t.sv[e] : 0.f;
      w[e] = pr[e] * (sv * rs);
    }
  } else {
#pragma unroll
    for (int e = 0; e < NT; ++e) w[e] = pr[e];
  }
  if (__any(beta != 1.f)) {
#pragma unroll
    for (int j = 0; j < G::kPV; ++j) o[j] *= beta;
  }
  // ---- O^T += V^T W -------------------------------------------------------
  // A padding token reads row 0: its codes (E4M3, bf16) or its block scale
  // (NVFP4) are cleared here, so that a NaN stored there cannot reach the
  // weighted sum (its weight is exactly 0).
  uint32_t vm[G::kTok][G::kVWords];
#pragma unroll
  for (int e = 0; e < G::kTok; ++e)
#pragma unroll
    for (int i = 0; i < G::kVWords; ++i)
      vm[e][i] = (KIND == kE4M3 || KIND == kBF16) && !((t.valid >> e) & 1u) ? 0u : t.v[e][i];
  if constexpr (KIND == kBF16) {
#pragma unroll
    for (int c = 0; c < G::kVWords; ++c) {
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        const uint32_t sel = hb ? 0x07060302u : 0x05040100u;
        bf16x4 bw;
#pragma unroll
        for (int e = 0; e < 4; ++e) bw[e] = (__bf16)w[e];
        u32x2 a;
        a[0] = perm(vm[1][c], vm[0][c], sel);
        a[1] = perm(vm[3][c], vm[2][c], sel);
        o[2 * c + hb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(bitcast<bf16x4>(a), bw,
                                                                   o[2 * c + hb], 0, 0, 0);
      }
    }
  } else if constexpr (G::kFp4) {
    // token e's word c: 8 codes = the lane's d-values 8 c .. 8 c + 7.  The
    // words of token pairs (0, 1) and (2, 3) are nibble-interleaved: byte j
    // of x01 holds token 0's and token 1's codes of one d-value, so its FP4
    // conversion is the (token 0, token 1) half of the A operand; times the
    // pair's block scales, exact in fp16.
    f16x4 bw;
#pragma unroll
    for (int e = 0; e < 4; ++e) bw[e] = (_Float16)w[e];
    uint32_t vs[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) vs[e] = ((t.valid >> e) & 1u) ? t.vsc[e] : 0u;
    const f16x2 sc01 = bitcast<f16x2>(e4m3pair_to_f16x2<false>(perm(vs[1], vs[0], 0x0C0C0400u)));
    const f16x2 sc23 = bitcast<f16x2>(e4m3pair_to_f16x2<false>(perm(vs[3], vs[2], 0x0C0C0400u)));
#pragma unroll
    for (int c = 0; c < G::kVWords; ++c) {
      const uint32_t w0 = vm[0][c], w1 = vm[1][c], w2 = vm[2][c], w3 = vm[3][c];
      const uint32_t x01[2] = {(w0 & 0x0F0F0F0Fu) | ((w1 << 4) & 0xF0F0F0F0u),    // low nibbles
                               ((w0 >> 4) & 0x0F0F0F0Fu) | (w1 & 0xF0F0F0F0u)};  // high nibbles
      const uint32_t x23[2] = {(w2 & 0x0F0F0F0Fu) | ((w3 << 4) & 0xF0F0F0F0u),
                               ((w2 >> 4) & 0x0F0F0F0Fu) | (w3 & 0xF0F0F0F0u)};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          uint32_t p01, p23;
          if (j == 0) { p01 = e2m1pair_to_f16x2<0>(x01[h]); p23 = e2m1pair_to_f16x2<0>(x23[h]); }
          else if (j == 1) { p01 = e2m1pair_to_f16x2<1>(x01[h]); p23 = e2m1pair_to_f16x2<1>(x23[h]); }
          else if (j == 2) { p01 = e2m1pair_to_f16x2<2>(x01[h]); p23 = e2m1pair_to_f16x2<2>(x23[h]); }
          else { p01 = e2m1pair_to_f16x2<3>(x01[h]); p23 = e2m1pair_to_f16x2<3>(x23[h]); }
          u32x2 a;
          a[0] = bitcast<uint32_t>(bitcast<f16x2>(p01) * sc01);
          a[1] = bitcast<uint32_t>(bitcast<f16x2>(p23) * sc23);
          o[8 * c + 2 * j + h] = __builtin_amdgcn_mfma_f32_16x16x16f16(bitcast<f16x4>(a), bw,
                                                                      o[8 * c + 2 * j + h], 0, 0, 0);
        }
      }
    }
  } else {
#pragma unroll
    for (int c = 0; c < G::kVWords; ++c) {
      uint32_t tk[NT / 2][2];
#pragma unroll
      for (int k = 0; k < NT / 2; ++k) interleave_pair<KIND>(vm[2 * k][c], vm[2 * k + 1][c], tk[k]);
#pragma unroll
      for (int bb = 0; bb < 4; ++bb) {
        f16x4 bw;
#pragma unroll
        for (int e = 0; e < 4; ++e) bw[e] = (_Float16)w[e];
        u32x2 r;
        r[0] = v_pair_f16<KIND>(tk[0], bb);
        r[1] = v_pair_f16<KIND>(tk[1], bb);
        o[4 * c + bb] = __builtin_amdgcn_mfma_f32_16x16x16f16(bitcast<f16x4>(r), bw,
                                                               o[4 * c + bb], 0, 0, 0);
      }
    }
  }
}

// Store D/4 contiguous floats (a lane's share of one head's output row).
template <int N>
__device__ __forceinline__ void store_row(void* out, int out_dtype, int64_t off, const float* v) {
  if (out_dtype == kDtFP32) {
    float4* dst = reinterpret_cast<float4*>(static_cast<float*>(out) + off);
#pragma unroll
    for (int i = 0; i < N / 4; ++i) dst[i] = float4{v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]};
  } else {
    u32x4* dst = reinterpret_cast<u32x4*>(static_cast<uint16_t*>(out) + off);
#pragma unroll
    for (int i = 0; i < N / 8; ++i) {
      u32x4 q;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        if (out_dtype == kDtBF16) {
          bf16x2 b;
          b[0] = (__bf16)v[8 * i + 2 * k];
          b[1] = (__bf16)v[8 * i + 2 * k + 1];
          q[k] = bitcast<uint32_t>(b);
        } else {
          f16x2 h;
          h[0] = (_Float16)v[8 * i + 2 * k];
          h[1] = (_Float16)v[8 * i + 2 * k + 1];
          q[k] = bitcast<uint32_t>(h);
        }
      }
      dst[i] = q;
    }
  }
}

template <int KIND, int D, int TT, int NW, bool kMulti>
__device__ __forceinline__ void attn_body(const AttnParams& p) {
  using G = Geo<KIND, D, TT>;
  constexpr int kThreads = NW * kWave;
  constexpr int kPer = pos_per_thread<NW>();
  constexpr int kChunk = kPer * kThreads;   // list positions resolved per LDS batch
  __shared__ __align__(16) int s_slot[kChunk];
  __shared__ float s_m[NW][16], s_l[NW][16];
  // cross-wave merge: two waves pair up (one buffer); four or eight waves
  // each park their accumulator (one buffer per wave)
  constexpr int kObufs = NW >= 4 ? NW : 1;
  __shared__ f32x4 s_obuf[kObufs][G::kPV * kWave];
  __shared__ float s_sig[NW];
  __shared__ QOp<KIND> s_q[G::kQLds ? G::kQK * kWave : 1];

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
  const int nlist = min(pbeg + p.chunk, p.topk) - pbeg;
  const int32_t* idx_row = p.topk_idx + (int64_t)r * p.topk + pbeg;
  const int bs_mask = (1 << p.log2_bs) - 1;

  // ---- the independent loads go out together: the row's sequence, the
  // first chunk of list positions and the query --------------------------------
  const int seq = p.row_seq[r];
  int cpos[kPer];
  auto chunk_start = [&](int c0) {
    const int cn = min(kChunk, nlist - c0);
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int i = threadIdx.x + u * kThreads;
      cpos[u] = i < cn ? idx_row[c0 + i] : -1;
    }
  };
  if (nlist > 0) chunk_start(0);

  const bool head_ok = ln16 < p.group;
  const int hq = g * p.group + ln16;
  u32x4 qraw[G::kQK];
  {
    const int64_t qoff = ((int64_t)r * p.num_q_heads + (head_ok ? hq : 0)) * D;
    const uint16_t* qrow = static_cast<const uint16_t*>(p.q) + qoff;
#pragma unroll
    for (int i = 0; i < G::kQK; ++i) {
      const int d0 = G::kFp4 ? 128 * (i >> 2) + 32 * grp + 8 * (i & 3)
                   : G::kOneByte ? 64 * (i >> 1) + 16 * grp + 8 * (i & 1) : 32 * i + 8 * grp;
      qraw[i] = head_ok ? *reinterpret_cast<const u32x4*>(qrow + d0) : u32x4{0, 0, 0, 0};
    }
  }

  // ---- slots of the partition, resolved into LDS a chunk at a time --------
  // (position -> block table -> slot; -1 for padding and for anything out of
  // range).
  const bool seq_ok = seq >= 0 && seq < p.num_seqs;
  const int npos = seq_ok ? nlist : 0;
  const int32_t* bt_row = p.block_table + (int64_t)(seq_ok ? seq : 0) * p.bt_stride;
  auto chunk_finish = [&](int c0) {
    const int cn = min(kChunk, npos - c0);
    const int rounded = (cn + TT - 1) / TT * TT;
    int blk[kPer];
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int pos = cpos[u];
      const int lb = pos >> p.log2_bs;
      blk[u] = (pos >= 0 && lb < p.bt_stride) ? bt_row[lb] : -1;
    }
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int i = threadIdx.x + u * kThreads;
      const int pos = cpos[u];
      if (i < rounded)
        s_slot[i] = (blk[u] >= 0 && blk[u] < p.num_blocks) ? (blk[u] << p.log2_bs) + (pos & bs_mask)
                                                            : -1;
    }
  };
  if (npos > 0) chunk_finish(0);

  // ---- the wave's first two tiles go out before the query setup ------------
  // tiles w, w + NW, w + 2 NW, ... of a chunk, kDepth of them in registers:
  // kDepth - 1 in flight while one is computed
  __syncthreads();                   // the first chunk's slots are published
  auto ts = [&](int k) { return s_slot + (w + NW * k) * TT; };
  auto wave_tiles = [&](int c0) {
    const int ntiles = (min(kChunk, npos - c0) + TT - 1) / TT;
    return ntiles > w ? (ntiles - w + NW - 1) / NW : 0;
  };
  int my_n = npos > 0 ? wave_tiles(0) : 0;
  TileRaw<KIND, D, TT> ta, tb;
  if (my_n > 0) issue_tile<KIND, D, TT>(ta, p, g, ts(0));
  if (my_n > 1) issue_tile<KIND, D, TT>(tb, p, g, ts(1));

  // ---- Q operand (B of QK^T) and the logit factor --------------------------
  QOp<KIND> qop[G::kQK];
  float kfac;
  if constexpr (KIND == kBF16) {
#pragma unroll
    for (int i = 0; i < G::kQK; ++i) qop[i] = bitcast<bf16x8>(qraw[i]);
    kfac = p.sm_log2e;
  } else {
    int e = 0;
    if (p.q_dtype == kDtFP16) {
#pragma unroll
      for (int i = 0; i < G::kQK; ++i) qop[i] = bitcast<f16x8>(qraw[i]);
    } else {
      // bf16 queries: exact power-of-two prescale so max|q| lands in
      // [2^14, 2^15), then round to fp16 (exact for every element >= 2^-14
      // after scaling; smaller ones keep an absolute error <= 2^-25).
      float amax = 0.f;
#pragma unroll
      for (int i = 0; i < G::kQK; ++i)
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          amax = fmaxf(amax, fabsf(__uint_as_float(qraw[i][k] << 16)));
          amax = fmaxf(amax, fabsf(__uint_as_float(qraw[i][k] & 0xFFFF0000u)));
        }
      amax = group4_max(amax);
      int ex = 0;
      if (amax > 0.f) frexpf(amax, &ex);
      e = amax > 0.f ? 15 - ex : 0;
      e = e > 127 ? 127 : (e < -126 ? -126 : e);
      const float sc = ldexpf(1.f, e);
#pragma unroll
      for (int i = 0; i < G::kQK; ++i) {
        f16x8 h;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          h[2 * k] = (_Float16)(__uint_as_float(qraw[i][k] << 16) * sc);
          h[2 * k + 1] = (_Float16)(__uint_as_float(qraw[i][k] & 0xFFFF0000u) * sc);
        }
        qop[i] = h;
      }
    }
    kfac = p.sm_log2e * p.k_scale * ldexpf(1.f, -e);
  }

  using QS = std::conditional_t<G::kQLds, QLds<KIND>, QRegs<KIND, G::kQK>>;
  QS qs;
  if constexpr (G::kQLds) {
    if (w == 0) {          // published by the barrier below
#pragma unroll
      for (int i = 0; i < G::kQK; ++i) s_q[i * kWave + lane] = qop[i];
    }
    qs.p = s_q + lane;
    __syncthreads();
  } else {
#pragma unroll
    for (int i = 0; i < G::kQK; ++i) qs.v[i] = qop[i];
  }

  // ---- the wave's tiles -----------------------------------------------------
  WaveState st{kNegInf, 0.f, 0.f, 0.f};
  f32x4 o[G::kPV];
#pragma unroll
  for (int j = 0; j < G::kPV; ++j) o[j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Tiles k (in ta) and k + 1 (in tb) are in flight at the top of each
  // pass.  The steady passes issue both successors unconditionally, so a
  // tile's loads land straight in the registers the next pass reads; the
  // last one to three tiles are finished after the loop.
  auto tile_loop = [&]() {
    int k = 0;
    for (; k + 3 < my_n; k += 2) {
      compute_tile<KIND, D, TT, QS>(ta, qs, kfac, st, o);
      issue_tile<KIND, D, TT>(ta, p, g, ts(k + 2));
      compute_tile<KIND, D, TT, QS>(tb, qs, kfac, st, o);
      issue_tile<KIND, D, TT>(tb, p, g, ts(k + 3));
    }
    const int r = my_n - k;                                 // 0 .. 3 tiles left
    if (r > 0) {
      compute_tile<KIND, D, TT, QS>(ta, qs, kfac, st, o);
      if (r > 2) issue_tile<KIND, D, TT>(ta, p, g, ts(k + 2));
    }
    if (r > 1) compute_tile<KIND, D, TT, QS>(tb, qs, kfac, st, o);
    if (r > 2) compute_tile<KIND, D, TT, QS>(ta, qs, kfac, st, o);
  };
  // Partitions that fit one LDS chunk of slots (kMulti false: chosen by the
  // host from the partition size) run the tile loop alone; with no chunk
  // loop around it the compiler follows the two tiles in flight across its
  // back edge and waits for each tile's loads as they are used rather than
  // for all loads outstanding.
  if constexpr (!kMulti) {
    tile_loop();
  } else {
    for (int c0 = 0; c0 < npos; c0 += kChunk) {
      if (c0 > 0) {
        __syncthreads();               // the previous chunk's slots are consumed
        chunk_start(c0);
        chunk_finish(c0);
        __syncthreads();
        my_n = wave_tiles(c0);
        if (my_n > 0) issue_tile<KIND, D, TT>(ta, p, g, ts(0));
        if (my_n > 1) issue_tile<KIND, D, TT>(tb, p, g, ts(1));
      }
      tile_loop();
    }
  }

  // ---- merge the waves' partial results -----------------------------------
  // Each wave's accumulator is weighted by exp2(m_w - M) (and, for int8, its
  // reference V scale) toward the common max M.  Two waves: the upper one
  // parks its weighted accumulator in LDS and the lower one adds it.  Four or
  // eight waves: every wave parks its raw accumulator, then wave w sums
  // slices j = w, w + NW, ... over the waves in wave order and leaves them in
  // wave 0's buffer -- two barriers in all, a fixed order (bitwise
  // reproducible); the total ends in wave 0.
  const float l_h = group4_sum(st.l);
  if (grp == 0) {
    s_m[w][ln16] = st.m;
    s_l[w][ln16] = l_h;
  }
  if constexpr (NW >= 4) {
    if (lane == 0) s_sig[w] = G::kInt ? st.sig : 1.f;
#pragma unroll
    for (int j = 0; j < G::kPV; ++j) s_obuf[w][j * kWave + lane] = o[j];
  }
  __syncthreads();
  float M = kNegInf;
#pragma unroll
  for (int i = 0; i < NW; ++i) M = fmaxf(M, s_m[i][ln16]);
  float L = 0.f, f[NW];
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    const float mi = s_m[i][ln16];
    f[i] = mi == kNegInf ? 0.f : __builtin_amdgcn_exp2f(mi - M);
    L += f[i] * s_l[i][ln16];
  }
  if constexpr (NW >= 4) {
#pragma unroll
    for (int i = 0; i < NW; ++i) f[i] *= s_sig[i];
    for (int j = w; j < G::kPV; j += NW) {
      f32x4 acc = s_obuf[0][j * kWave + lane] * f[0];
#pragma unroll
      for (int i = 1; i < NW; ++i) acc += s_obuf[i][j * kWave + lane] * f[i];
      s_obuf[0][j * kWave + lane] = acc;
    }
    __syncthreads();
    if (w == 0) {
#pragma unroll
      for (int j = 0; j < G::kPV; ++j) o[j] = s_obuf[0][j * kWave + lane];
    }
  } else if constexpr (NW == 2) {
    float myf = f[w];
    if constexpr (G::kInt) myf *= st.sig;
#pragma unroll
    for (int j = 0; j < G::kPV; ++j) o[j] *= myf;
    if (w == 1) {
#pragma unroll
      for (int j = 0; j < G::kPV; ++j) s_obuf[0][j * kWave + lane] = o[j];
    }
    __syncthreads();
    if (w == 0) {
#pragma unroll
      for (int j = 0; j < G::kPV; ++j) o[j] += s_obuf[0][j * kWave + lane];
    }
  } else {
    float myf = f[0];
    if constexpr (G::kInt) myf *= st.sig;
#pragma unroll
    for (int j = 0; j < G::kPV; ++j) o[j] *= myf;
  }
  if (w != 0 || !head_ok) return;

  // lane (ln16, grp) holds d = (D/16) * (4*grp + k) + j for k < 4, j < D/16:
  // D/4 contiguous outputs starting at (D/4) * grp.
  const int64_t orow = (int64_t)r * p.num_q_heads + hq;
  if (p.num_splits == 1) {
    const bool any = L > 0.f;
    const float inv = any ? p.v_scale / L : 0.f;
    if (p.lse && grp == 0) p.lse[orow] = any ? (M + __log2f(L)) * kLn2 : kNegInf;
    float vals[G::kOut];
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
      for (int j = 0; j < G::kPV; ++j) vals[k * G::kPV + j] = o[j][k] * inv;
    store_row<G::kOut>(p.out, p.out_dtype, orow * D + G::kOut * grp, vals);
  } else {
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

// 16-token tiles at two waves per SIMD (<= 256 registers per wave).
template <int KIND, int D, int NW, bool kMulti>
__global__ __launch_bounds__(NW * kWave) __attribute__((amdgpu_waves_per_eu(2, 2)))
void qsa_attn16_kernel(AttnParams p) {
  attn_body<KIND, D, 16, NW, kMulti>(p);
}

// Log-sum-exp merge of the split-K partials of one (row, head) per wave:
// M = max_p m_p, L = sum_p L_p 2^(m_p - M), out = sum_p o_p 2^(m_p - M) / L,
// times the E4M3 V scale (applied once, after the merge).  Each lane owns
// D/64 outputs; the first kPre partials (every one, for P <= kPre: the host
// picks kPre = 8 or 16 by P) are loaded together with the (max, sum) pairs,
// so the call costs about one memory round trip.
template <int D, int kPre>
__global__ __launch_bounds__(kWave) void qsa_merge_kernel(AttnParams p) {
  constexpr int E = D / kWave;
  const int lane = lane_id();
  // (row, query head) r * Hq + h; consecutive ones share an XCD, in the same
  // split as the attention launch's items, so that a head's partials are
  // mostly read on the XCD whose L2 holds them
  int64_t rh;
  {
    const int n = p.num_rows * p.num_q_heads;
    const int b = blockIdx.x, x = b & 7, k = b >> 3;
    const int q8 = n >> 3, rem = n & 7;
    rh = x * q8 + (x < rem ? x : rem) + k;
  }
  const int P = p.num_splits;
  const int64_t base = rh * P;
  const float* src = p.ws_o + base * D + lane * E;
  // every load is issued, with no branch between them (a conditional load
  // makes the compiler copy its register and wait for it): slots past P
  // re-read the last partial and get weight 0 below (P >= 2 here)
  float pre[kPre][E];
#pragma unroll
  for (int q = 0; q < kPre; ++q) {
    const int64_t qq = q < P ? q : P - 1;
    if constexpr (E == 4) {
      const float4 v = *reinterpret_cast<const float4*>(src + qq * D);
      pre[q][0] = v.x; pre[q][1] = v.y; pre[q][2] = v.z; pre[q][3] = v.w;
    } else {
      const float2 v = *reinterpret_cast<const float2*>(src + qq * D);
      pre[q][0] = v.x; pre[q][1] = v.y;
    }
  }
  // the partitions' (max, sum) pairs: lane q loads pair q with the partials
  // (one vector load, the same round trip), then every lane reads them
  // across lanes -- no reductions, and no scalar loads (more than 15 of
  // those in flight would be split into two round trips)
  const float* ml = p.ws_ml + 2 * base;
  const int lq_idx = (lane & (kPre - 1)) < P ? (lane & (kPre - 1)) : P - 1;
  const float2 mlv = *reinterpret_cast<const float2*>(ml + 2 * lq_idx);
  float mq[kPre], lq[kPre];
#pragma unroll
  for (int q = 0; q < kPre; ++q) {
    const float m = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mlv.x), q));
    const float l = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mlv.y), q));
    mq[q] = q < P ? m : kNegInf;
    lq[q] = q < P ? l : 0.f;
  }
  float M = kNegInf;
#pragma unroll
  for (int q = 0; q < kPre; ++q) M = fmaxf(M, mq[q]);
  for (int q = kPre; q < P; ++q) M = fmaxf(M, ml[2 * q]);
  float L = 0.f;
  float acc[E];
#pragma unroll
  for (int i = 0; i < E; ++i) acc[i] = 0.f;
#pragma unroll
  for (int q = 0; q < kPre; ++q) {
    const float fq = mq[q] == kNegInf ? 0.f : __builtin_amdgcn_exp2f(mq[q] - M);
    L += fq * lq[q];
#pragma unroll
    for (int i = 0; i < E; ++i) acc[i] += fq * pre[q][i];
  }
  for (int q = kPre; q < P; ++q) {
    const float mq = ml[2 * q];
    const float fq = mq == kNegInf ? 0.f : __builtin_amdgcn_exp2f(mq - M);
    L += fq * ml[2 * q + 1];
#pragma unroll
    for (int i = 0; i < E; ++i) acc[i] += fq * src[(int64_t)q * D + i];
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

// Waves per workgroup.  A workgroup's fixed cost is a chain of dependent
// memory round trips (list positions, block table, first tile, partial
// store), so launches with few items spread each item over more waves and
// run in one wave of workgroups where they can: at two waves per SIMD the
// chip holds 2048 waves (8 per item up to 256 items, 4 up to 512, 2 up to
// 1024, 1 up to 2048).  Large launches (prefill) keep 4 waves per item.
template <int KIND, int D, int NW>
hipError_t launch_knw(const AttnParams& p, unsigned grid, hipStream_t s) {
  // slots resolved per LDS batch by an NW-wave workgroup (attn_body's kChunk)
  constexpr int kChunk = pos_per_thread<NW>() * NW * kWave;
  if (p.chunk <= kChunk)
    qsa_attn16_kernel<KIND, D, NW, false><<<grid, dim3(NW * kWave), 0, s>>>(p);
  else
    qsa_attn16_kernel<KIND, D, NW, true><<<grid, dim3(NW * kWave), 0, s>>>(p);
  return hipGetLastError();
}

template <int KIND, int D>
hipError_t launch_kd(const AttnParams& p, hipStream_t s) {
  const int64_t items = (int64_t)p.num_rows * p.num_kv_heads * p.num_splits;
  const unsigned grid = (unsigned)items;
  if (items <= 256) return launch_knw<KIND, D, 8>(p, grid, s);
  if (items > 512 && items <= 1024) return launch_knw<KIND, D, 2>(p, grid, s);
  if (items > 1024 && items <= 2048) return launch_knw<KIND, D, 1>(p, grid, s);
  return launch_knw<KIND, D, 4>(p, grid, s);
}

template <int KIND>
hipError_t launch_kind(int head_dim, const AttnParams& p, hipStream_t s) {
  return head_dim == 256 ? launch_kd<KIND, 256>(p, s) : launch_kd<KIND, 128>(p, s);
}

}  // namespace

hipError_t launch_attn(int kind, int head_dim, const AttnParams& p, hipStream_t s) {
  switch (kind) {
    case kInt8: return launch_kind<kInt8>(head_dim, p, s);
    case kInt8Inline: return launch_kind<kInt8Inline>(head_dim, p, s);
    case kE4M3: return launch_kind<kE4M3>(head_dim, p, s);
    case kNvfp4: return launch_kind<kNvfp4>(head_dim, p, s);
    default: return launch_kind<kBF16>(head_dim, p, s);
  }
}

template <int D>
void launch_merge_d(const AttnParams& p, unsigned grid, hipStream_t s) {
  if (p.num_splits <= 8)
    qsa_merge_kernel<D, 8><<<grid, dim3(kWave), 0, s>>>(p);
  else
    qsa_merge_kernel<D, 16><<<grid, dim3(kWave), 0, s>>>(p);
}

hipError_t launch_merge(int head_dim, const AttnParams& p, hipStream_t s) {
  const unsigned grid = (unsigned)(p.num_rows * p.num_q_heads);
  if (head_dim == 256)
    launch_merge_d<256>(p, grid, s);
  else
    launch_merge_d<128>(p, grid, s);
  return hipGetLastError();
}

}  // namespace qsakv
