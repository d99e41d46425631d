// Quantize-on-write of K/V rows into a paged cache.
//
// One wave per (token, KV head, K|V) row; each lane holds D/64 consecutive
// elements.  The int8 arithmetic is the per-(token, head) symmetric rule of
// page "int8 per-(token,head) KV cache for the Qwen3.8-Flash-Next QSA path"
// (section "Headline result"): a = max|x|, s = fl32(a / 127),
// q = clamp(rne(fl32(x / s)), -127, 127), a zero row stores s = 0, q = 0.
// The E4M3 rule is the converter contract of page "Qwen3.8 Flash Next NVFP4
// QSA FP8 E4M3 KV Scales" (section "Calibration"):
// code = e4m3fn(fl32(x / scale)) with saturation.  Both quotients are IEEE
// correctly rounded fp32 divisions (hipcc's default '/'), so every stored
// byte is determined by its source row alone and is bit-exact.
#include "qsakv_device.h"
#include "qsakv_internal.h"

namespace qsakv {
namespace {

constexpr int kRowsPerBlock = 4;  // waves per workgroup

template <int SRC, int E>
__device__ __forceinline__ void load_src(const void* base, int64_t elem_off, float (&x)[E]) {
  if constexpr (SRC == kDtFP32) {
    const float* p = static_cast<const float*>(base) + elem_off;
    if constexpr (E == 4) {
      const float4 v = *reinterpret_cast<const float4*>(p);
      x[0] = v.x; x[1] = v.y; x[2] = v.z; x[3] = v.w;
    } else {
      const float2 v = *reinterpret_cast<const float2*>(p);
      x[0] = v.x; x[1] = v.y;
    }
  } else {
    const uint16_t* p = static_cast<const uint16_t*>(base) + elem_off;
    uint32_t w[E / 2];
    if constexpr (E == 4) {
      const u32x2 v = *reinterpret_cast<const u32x2*>(p);
      w[0] = v[0]; w[1] = v[1];
    } else {
      w[0] = *reinterpret_cast<const uint32_t*>(p);
    }
#pragma unroll
    for (int i = 0; i < E / 2; ++i) {
      if constexpr (SRC == kDtBF16) {
        x[2 * i] = __uint_as_float(w[i] << 16);
        x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
      } else {
        const f16x2 h = bitcast<f16x2>(w[i]);
        x[2 * i] = (float)h[0];
        x[2 * i + 1] = (float)h[1];
      }
    }
  }
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

template <int KIND, int D, int SRC>
__global__ __launch_bounds__(kRowsPerBlock * kWave) void kv_write_kernel(WriteParams p) {
  constexpr int E = D / kWave;
  const int lane = lane_id();
  const int64_t rows = p.num_tokens * p.num_kv_heads * 2;
  const int64_t stride = (int64_t)gridDim.x * kRowsPerBlock;
  for (int64_t rw = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6); rw < rows;
       rw += stride) {
    const int64_t t = rw / (2 * p.num_kv_heads);
    const int rem = (int)(rw - t * 2 * p.num_kv_heads);
    const int h = rem >> 1;
    const int which = rem & 1;  // 0 = K, 1 = V
    const int64_t slot = p.slot_mapping[t];
    if (slot < 0 || slot >= p.num_slots) continue;  // wave-uniform

    float x[E];
    const int64_t src_off = (t * p.num_kv_heads + h) * D + lane * E;
    load_src<SRC, E>(which ? p.v_src : p.k_src, src_off, x);
    uint8_t* base = which ? p.v : p.k;
    const int64_t row = slot * p.num_kv_heads + h;

    if constexpr (KIND == kInt8 || KIND == kInt8Inline) {
      float a = 0.f;
#pragma unroll
      for (int i = 0; i < E; ++i) a = fmaxf(a, fabsf(x[i]));
      a = wave_max(a);
      const float s = a / 127.0f;
      uint32_t packed = 0;
#pragma unroll
      for (int i = 0; i < E; ++i) {
        float q = 0.f;
        if (s != 0.f) q = fminf(fmaxf(rintf(x[i] / s), -127.f), 127.f);
        packed |= ((uint32_t)(int32_t)q & 0xFFu) << (8 * i);
      }
      constexpr int kRowBytes = (KIND == kInt8) ? D : D + 4;
      uint8_t* dst = base + row * kRowBytes;
      if constexpr (E == 4) {
        *reinterpret_cast<uint32_t*>(dst + lane * 4) = packed;
      } else {
        *reinterpret_cast<uint16_t*>(dst + lane * 2) = (uint16_t)packed;
      }
      if (lane == 0) {
        if constexpr (KIND == kInt8) {
          p.kv_scale[row * 2 + which] = s;
        } else {
          *reinterpret_cast<float*>(dst + D) = s;
        }
      }
    } else if constexpr (KIND == kE4M3) {
      const float scale = which ? p.v_scale : p.k_scale;
      uint32_t packed = 0;
#pragma unroll
      for (int i = 0; i < E; ++i) packed |= e4m3_encode(x[i] / scale) << (8 * i);
      uint8_t* dst = base + row * D;
      if constexpr (E == 4) {
        *reinterpret_cast<uint32_t*>(dst + lane * 4) = packed;
      } else {
        *reinterpret_cast<uint16_t*>(dst + lane * 2) = (uint16_t)packed;
      }
    } else {  // kBF16: round to nearest even (identity for bf16 sources)
      uint32_t w[E / 2];
#pragma unroll
      for (int i = 0; i < E / 2; ++i) {
        bf16x2 b;
        b[0] = (__bf16)x[2 * i];
        b[1] = (__bf16)x[2 * i + 1];
        w[i] = bitcast<uint32_t>(b);
      }
      uint8_t* dst = base + row * (2 * D) + lane * (2 * E);
      if constexpr (E == 4) {
        u32x2 v;
        v[0] = w[0];
        v[1] = w[1];
        *reinterpret_cast<u32x2*>(dst) = v;
      } else {
        *reinterpret_cast<uint32_t*>(dst) = w[0];
      }
    }
  }
}

template <int KIND, int D>
hipError_t launch_src(const WriteParams& p, hipStream_t s) {
  const int64_t rows = p.num_tokens * p.num_kv_heads * 2;
  const int64_t want = (rows + kRowsPerBlock - 1) / kRowsPerBlock;
  const unsigned grid = (unsigned)(want < (1 << 20) ? want : (1 << 20));
  const dim3 block(kRowsPerBlock * kWave);
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
    default: return launch_d<kBF16>(head_dim, p, s);
  }
}

}  // namespace qsakv
