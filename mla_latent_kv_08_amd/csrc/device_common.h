// Device-side helpers shared by the MLA decode kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef _Float16 half8 __attribute__((ext_vector_type(8)));

// ---------------------------------------------------------------------------
// bf16 <-> fp32
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b16) {
  return __uint_as_float(b16 << 16);
}

// Round-to-nearest-even fp32 -> bf16 bit pattern (NaN stays a quiet NaN).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

// fp32 <-> fp16 (round to nearest even; NaN and infinities carried over).
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)lo) |
         ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)hi) << 16);
}
__device__ __forceinline__ float f16_lo(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
}
__device__ __forceinline__ float f16_hi(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}

// ---------------------------------------------------------------------------
// FP4 latent codec: E2M1 codes with one E4M3 ("FN") scale per 16 channels.
// ---------------------------------------------------------------------------

// E4M3 code nearest to r >= 0 (fp32), ties to the even code, saturating to 448.
__device__ __forceinline__ uint32_t e4m3_encode_rne(float r) {
  if (!(r < 448.0f)) return 0x7eu;  // also catches +inf
  const uint32_t bits = __float_as_uint(r);
  const int e = (int)((bits >> 23) & 0xffu) - 127;
  if (e < -6) {
    // Subnormal E4M3 range: multiples of 2^-9; 8 * 2^-9 is the smallest normal.
    return (uint32_t)__builtin_rintf(r * 512.0f);
  }
  uint32_t keep = (bits >> 20) & 7u;
  const uint32_t rem = bits & 0xfffffu;
  if (rem > 0x80000u || (rem == 0x80000u && (keep & 1u))) keep += 1u;
  uint32_t E = (uint32_t)(e + 7);
  if (keep == 8u) {
    keep = 0u;
    E += 1u;
  }
  uint32_t code = (E << 3) | keep;
  return code > 0x7eu ? 0x7eu : code;
}

// E2M1 code of x under scale s > 0: nearest magnitude to |x|/s with ties to
// the even code. Thresholds s*midpoint are exact in fp32, so comparing |x|
// with them decides the real-valued rounding exactly.
__device__ __forceinline__ uint32_t e2m1_encode(float x, float s) {
  const float ax = fabsf(x);
  const float mids[7] = {0.25f, 0.75f, 1.25f, 1.75f, 2.5f, 3.5f, 5.0f};
  uint32_t k = 0;
#pragma unroll
  for (int j = 0; j < 7; ++j) {
    const float t = s * mids[j];
    k += (ax > t) ? 1u : 0u;
  }
  // A tie sits exactly on midpoint k (between codes k and k+1): choose the even one.
  if (k < 7u) {
    const float t = s * (k == 0 ? 0.25f : k == 1 ? 0.75f : k == 2 ? 1.25f : k == 3 ? 1.75f
                          : k == 4 ? 2.5f : k == 5 ? 3.5f : 5.0f);
    if (ax == t && (k & 1u)) k += 1u;
  }
  if (k == 0u) return 0u;
  return k | ((x < 0.0f) ? 8u : 0u);
}

// Two codes (byte e of w) times scale s as two bf16. The hardware conversion
// takes only the exponent of its scale, so it runs at scale 1 (exact E2M1
// values, straight to fp32) and the E4M3 scale is applied in fp32; every
// product of an E2M1 value and an E4M3 scale fits in bf16, so taking the high
// halves is exact.
template <int e>
__device__ __forceinline__ uint32_t fp4_pair(uint32_t w, float s) {
  const auto r = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, e);
  const float lo = r[0] * s;
  const float hi = r[1] * s;
  return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
}

// Two codes (byte e of w) times scale s as two fp16 (s2 = {s, s} in fp16):
// E2M1 values at scale 1 straight to fp16, then one packed fp16 multiply.
// Every E4M3 value is an fp16 number, and every product of an E2M1 value
// (2 significant bits, |v| <= 6) and an E4M3 scale (4 bits, 2^-9 .. 448)
// has at most 5 significant bits and lies in [2^-10, 2688], inside fp16's
// normal range: the product is exact.
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
template <int e>
__device__ __forceinline__ uint32_t fp4_pair_f16(uint32_t w, half2v s2) {
  const half2v v = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, e) * s2;
  return __builtin_bit_cast(uint32_t, v);
}

// Values of E4M3 ("FN") scale bytes: subnormal m * 2^-9, normal
// (1 + m/8) * 2^(e-7), NaN for e=15, m=7. The hardware FP8 conversion at
// scale 1 (whose scale only adds to the exponent) gives them exactly: one
// instruction for the two bytes of the low half of w.
__device__ __forceinline__ float2 e4m3_pair(uint32_t w) {
  const auto r = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w, 1.0f, false);
  return make_float2(r[0], r[1]);
}
__device__ __forceinline__ float e4m3_value(uint32_t byte) { return e4m3_pair(byte).x; }

// ---------------------------------------------------------------------------
// Cache addressing
// ---------------------------------------------------------------------------
struct CacheView {
  const uint8_t* latent;
  const uint8_t* scale;
  const uint8_t* rope;
  int64_t latent_stride;
  int64_t scale_stride;
  int64_t rope_stride;
  int64_t num_rows;
  const int32_t* page_table;
  int32_t page_size;  // 0 or 64
  int32_t capacity;
  int32_t pt_stride;
};

// Sequence length clamped to what the cache can hold.
__device__ __forceinline__ int clamp_len(int len, int capacity) {
  return len < 0 ? 0 : (len > capacity ? capacity : len);
}

// Physical row of logical token t of sequence b; sets bad (and returns 0)
// when a page index points outside the cache.
__device__ __forceinline__ int64_t phys_row(const CacheView& c, int b, int t, bool& bad) {
  if (c.page_size == 0) return (int64_t)b * c.capacity + t;
  const int page = c.page_table[(int64_t)b * c.pt_stride + (t >> 6)];
  const int64_t r = (int64_t)page * 64 + (t & 63);
  if (page < 0 || r >= c.num_rows) {
    bad = true;
    return 0;
  }
  return r;
}

}  // namespace mla
