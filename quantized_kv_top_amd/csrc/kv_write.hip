// Quantize-on-write of K/V rows into a paged cache.
//
// Several (token, KV head) rows of K or of V per wave, 16 consecutive
// elements per lane.  The int8 arithmetic is the per-(token, head) symmetric rule of
// page "int8 per-(token,head) KV cache for the Qwen3.8-Flash-Next QSA path"
// (section "Headline result"): a = max|x|, s = fl32(a / 127),
// q = clamp(rne(fl32(x / s)), -127, 127), a zero row stores s = 0, q = 0.
// The E4M3 rule is the converter contract of page "Qwen3.8 Flash Next NVFP4
// QSA FP8 E4M3 KV Scales" (section "Calibration"):
// code = e4m3fn(fl32(x / scale)) with saturation.  NVFP4 (a reading: the
// pages name it only as a KV variant outside that contract): per block of
// 16 elements -- exactly a lane's share -- a = max|x|, block scale code
// sc = e4m3fn(fl32(fl32(a / 6) / g)) with the layer's scale g, and element
// codes e2m1(fl32(x / fl32(S g))), S the value of sc.  All quotients are IEEE
// correctly rounded fp32 divisions (hipcc's default '/'), so every stored
// byte is determined by its source row alone and is bit-exact.
#include "qsakv_device.h"
#include "qsakv_internal.h"

namespace qsakv {
namespace {

// Work decomposition: K and V are two streams of rows (row = token * Hkv +
// head, D elements each).  A wave takes kRPW consecutive rows of one stream
// -- a contiguous span of the source -- with 16 elements per lane, kLPR lanes
// per row; the row's max is reduced over its kLPR lanes.  The source and the
// rows' slots are loaded together; stores are 16-byte (or dword, for the
// 4-byte-aligned inline rows) per lane.
constexpr int kEPL = 16;          // elements per lane
constexpr int kWavesPerBlock = 4;

template <int SRC>
__device__ __forceinline__ void load_src16(const void* base, int64_t elem_off, float (&x)[kEPL]) {
  if constexpr (SRC == kDtFP32) {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(base) + elem_off);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float4 v = p[i];
      x[4 * i] = v.x; x[4 * i + 1] = v.y; x[4 * i + 2] = v.z; x[4 * i + 3] = v.w;
    }
  } else {
    const u32x4* p = reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(base) + elem_off);
    const u32x4 w0 = p[0], w1 = p[1];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t w = i < 4 ? w0[i] : w1[i - 4];
      if constexpr (SRC == kDtBF16) {
        x[2 * i] = __uint_as_float(w << 16);
        x[2 * i + 1] = __uint_as_float(w & 0xFFFF0000u);
      } else {
        const f16x2 h = bitcast<f16x2>(w);
        x[2 * i] = (float)h[0];
        x[2 * i + 1] = (float)h[1];
      }
    }
  }
}

// max over the kLPR lanes of a row (aligned groups of kLPR lanes)
template <int kLPR>
__device__ __forceinline__ float row_max(float a) {
#pragma unroll
  for (int o = kLPR / 2; o >= 1; o >>= 1) a = fmaxf(a, __shfl_xor(a, o));
  return a;
}

// OCP E4M3FN encode of an fp32 value: round to nearest even, saturate to
// +-448, NaN -> S.1111.111, sign of zero kept.  Integer form of the
// definition: the top 3 mantissa bits are rounded half-to-even at bit 20
// (carry may bump the exponent); below 2^-6 the quantum is 2^-9.
__device__ __forceinline__ uint32_t e4m3_encode(float y) {
  const uint32_t u = __float_as_uint(y);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7FFFFFFFu;
  uint32_t code;
  if (a > 0x7F800000u) {
    code = 0x7Fu;                                     // NaN
  } else if (a >= 0x43E00000u) {
    code = 0x7Eu;                                     // >= 448 or inf: saturate
  } else if (a < 0x3C800000u) {                       // < 2^-6: subnormal step 2^-9
    code = (uint32_t)rintf(__uint_as_float(a) * 512.0f);
  } else {
    const uint32_t r = a + 0x7FFFFu + ((a >> 20) & 1u);
    code = (r >> 20) - 960u;                          // ((e - 120) << 3) | m3
  }
  return sign | code;
}

// E4M3FN code (0 .. 0x7E, sign clear) -> its value, exactly.
__device__ __forceinline__ float e4m3_value(uint32_t c) {
  const int e = (int)((c >> 3) & 0xFu), m = (int)(c & 7u);
  return e ? ldexpf((float)(8 + m), e - 10) : ldexpf((float)m, -9);
}

// FP4 E2M1 code of an fp32 value: the nearest of 0, 0.5, 1, 1.5, 2, 3, 4, 6
// with ties to the even code (the midpoints 0.25, 0.75, 1.25, 1.75, 2.5,
// 3.5, 5 go to codes 0, 2, 2, 4, 4, 6, 6), saturating at 6; sign bit from
// y; NaN -> +0.
__device__ __forceinline__ uint32_t e2m1_encode(float y) {
  const float a = fabsf(y);
  if (!(a == a)) return 0u;
  const uint32_t c = a <= 0.25f ? 0u : a < 0.75f ? 1u : a <= 1.25f ? 2u : a < 1.75f ? 3u
                   : a <= 2.5f ? 4u : a < 3.5f ? 5u : a <= 5.0f ? 6u : 7u;
  return ((__float_as_uint(y) >> 28) & 8u) | c;
}

// Quantize this lane's kEPL elements of one K or V row (lanes part = 0 ..
// kLPR-1 of the row together) and store the codes at cache row `row` of
// `base`.  Returns the bits of what the caller stores beside them: the
// int8 scale s (side layout), or this lane's NVFP4 block-scale code; the
// inline int8 layout stores its scale itself.
template <int KIND, int D>
__device__ __forceinline__ uint32_t quantize_row(const WriteParams& p, uint8_t* base, int64_t row,
                                              int part, int which, const float (&x)[kEPL]) {
  constexpr int kLPR = D / kEPL;
  if constexpr (KIND == kInt8 || KIND == kInt8Inline) {
    float a = 0.f;
#pragma unroll
    for (int i = 0; i < kEPL; ++i) a = fmaxf(a, fabsf(x[i]));
    a = row_max<kLPR>(a);
    const float s = a / 127.0f;
    // x / s is taken as x * RN(1/s).  |x / s| <= 127 (1 + 2^-24), and the
    // product is within |x / s| 2^-23 (1 + 2^-25) of the exact quotient, so
    // within 2^-16 + 2^-18 (its half ulp) of the correctly rounded one: both
    // round to the same integer unless the product lies within 2^-14 of a
    // half-integer.  There (and when 1/s overflows) x / s is divided out
    // exactly.  NaN and +-inf take the same course either way.
    const float r = 1.0f / s;
    const bool fast = r <= 3.4028234663852886e38f;
    uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < kEPL; ++i) {
      float q = 0.f;
      if (s != 0.f) {
        float y = x[i] * r;
        const float ay = fabsf(y);
        if (!fast || fabsf((ay - floorf(ay)) - 0.5f) <= 0x1p-14f) y = x[i] / s;
        q = fminf(fmaxf(rintf(y), -127.f), 127.f);
      }
      w[i >> 2] |= ((uint32_t)(int32_t)q & 0xFFu) << (8 * (i & 3));
    }
    if constexpr (KIND == kInt8) {
      *reinterpret_cast<u32x4*>(base + row * D + part * kEPL) = u32x4{w[0], w[1], w[2], w[3]};
    } else {  // 4-byte-aligned rows of D + 4 bytes
      uint32_t* dst = reinterpret_cast<uint32_t*>(base + row * (D + 4) + part * kEPL);
#pragma unroll
      for (int i = 0; i < 4; ++i) dst[i] = w[i];
      if (part == 0) *reinterpret_cast<float*>(base + row * (D + 4) + D) = s;
    }
    return __float_as_uint(s);
  } else if constexpr (KIND == kE4M3) {
    const float scale = which ? p.v_scale : p.k_scale;
    uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < kEPL; ++i) w[i >> 2] |= e4m3_encode(x[i] / scale) << (8 * (i & 3));
    *reinterpret_cast<u32x4*>(base + row * D + part * kEPL) = u32x4{w[0], w[1], w[2], w[3]};
    return 0u;
  } else if constexpr (KIND == kNvfp4) {
    const float g = which ? p.v_scale : p.k_scale;
    float a = 0.f;
#pragma unroll
    for (int i = 0; i < kEPL; ++i) {   // NaN ignored: a comparison with NaN is false
      const float v = fabsf(x[i]);     // (a NaN-quieting max could pass a NaN on)
      a = v > a ? v : a;
    }
    const float sb = a / 6.0f;
    const uint32_t sc = e4m3_encode(sb / g);
    const float eff = e4m3_value(sc) * g;
    uint32_t w[2] = {0u, 0u};
#pragma unroll
    for (int i = 0; i < kEPL; ++i)
      w[i >> 3] |= (eff > 0.f ? e2m1_encode(x[i] / eff) : 0u) << (4 * (i & 7));
    *reinterpret_cast<u32x2*>(base + row * (D / 2) + part * 8) = u32x2{w[0], w[1]};
    return sc;
  } else {  // kBF16: round to nearest even (identity for bf16 sources)
    uint32_t w[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      bf16x2 b;
      b[0] = (__bf16)x[2 * i];
      b[1] = (__bf16)x[2 * i + 1];
      w[i] = bitcast<uint32_t>(b);
    }
    u32x4* dst = reinterpret_cast<u32x4*>(base + row * (2 * D) + part * (2 * kEPL));
    dst[0] = u32x4{w[0], w[1], w[2], w[3]};
    dst[1] = u32x4{w[4], w[5], w[6], w[7]};
    return 0u;
  }
}

// One wave takes kRPW source rows (token, KV head), K and V both: the two
// rows' sources are loaded together, and the row's K and V scales leave as
// one store (int8: the fp32 pair; NVFP4: each lane's two block-scale codes,
// 16-byte K and V runs side by side).
template <int KIND, int D, int SRC>
__global__ __launch_bounds__(kWavesPerBlock * kWave) void kv_write_kernel(WriteParams p) {
  constexpr int kLPR = D / kEPL;         // lanes per row
  constexpr int kRPW = kWave / kLPR;     // rows per wave
  const int lane = lane_id();
  const int sub = lane / kLPR, part = lane % kLPR;
  const int hkv = p.num_kv_heads;
  const int64_t nrow = p.num_tokens * hkv;                  // source rows
  const int64_t groups = (nrow + kRPW - 1) / kRPW;          // wave groups
  const int64_t stride = (int64_t)gridDim.x * kWavesPerBlock;
  for (int64_t gi = (int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6); gi < groups;
       gi += stride) {
    const int64_t r = gi * kRPW + sub;
    if (r >= nrow) continue;                                // whole rows drop out together
    const int64_t t = r / hkv;
    const int h = (int)(r - t * hkv);
    const int64_t slot = p.slot_mapping[t];
    float xk[kEPL], xv[kEPL];
    load_src16<SRC>(p.k_src, r * D + part * kEPL, xk);
    load_src16<SRC>(p.v_src, r * D + part * kEPL, xv);
    if (slot < 0 || slot >= p.num_slots) continue;
    const int64_t row = slot * hkv + h;
    const uint32_t sk = quantize_row<KIND, D>(p, p.k, row, part, 0, xk);
    const uint32_t sv = quantize_row<KIND, D>(p, p.v, row, part, 1, xv);
    if constexpr (KIND == kInt8) {
      if (part == 0) *reinterpret_cast<u32x2*>(p.kv_scale + row * 2) = u32x2{sk, sv};
    } else if constexpr (KIND == kNvfp4) {
      uint8_t* sc = reinterpret_cast<uint8_t*>(p.kv_scale) + row * 2 * (D / 16) + part;
      sc[0] = (uint8_t)sk;
      sc[D / 16] = (uint8_t)sv;
    }
  }
}

template <int KIND, int D>
hipError_t launch_src(const WriteParams& p, hipStream_t s) {
  constexpr int kRPW = kWave / (D / kEPL);
  const int64_t groups = (p.num_tokens * p.num_kv_heads + kRPW - 1) / kRPW;
  const int64_t want = (groups + kWavesPerBlock - 1) / kWavesPerBlock;
  const unsigned grid = (unsigned)(want < (1 << 20) ? want : (1 << 20));
  const dim3 block(kWavesPerBlock * kWave);
  switch (p.src_dtype) {
    case kDtFP32: kv_write_kernel<KIND, D, kDtFP32><<<grid, block, 0, s>>>(p); break;
    case kDtBF16: kv_write_kernel<KIND, D, kDtBF16><<<grid, block, 0, s>>>(p); break;
    default: kv_write_kernel<KIND, D, kDtFP16><<<grid, block, 0, s>>>(p); break;
  }
  return hipGetLastError();
}

template <int KIND>
hipError_t launch_d(int head_dim, const WriteParams& p, hipStream_t s) {
  return head_dim == 256 ? launch_src<KIND, 256>(p, s) : launch_src<KIND, 128>(p, s);
}

}  // namespace

hipError_t launch_kv_write(int kind, int head_dim, const WriteParams& p, hipStream_t s) {
  switch (kind) {
    case kInt8: return launch_d<kInt8>(head_dim, p, s);
    case kInt8Inline: return launch_d<kInt8Inline>(head_dim, p, s);
    case kE4M3: return launch_d<kE4M3>(head_dim, p, s);
    case kNvfp4: return launch_d<kNvfp4>(head_dim, p, s);
    default: return launch_d<kBF16>(head_dim, p, s);
  }
}

}  // namespace qsakv
