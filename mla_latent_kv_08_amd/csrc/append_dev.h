// Cache append of one new token by one wave, shared by the append kernel and
// the fused append + absorb kernel.
//
// The Q new tokens of each sequence go to logical positions len-Q .. len-1,
// through the page table when the cache is paged (DeepSeek-V3 deep-dive page:
// compress the current token, store it in the latent/RoPE slot pool at
// token_pos times the row width; here with bounds checks). An FP4 latent cache
// is quantised on the way in: per 16 channels an E4M3 scale =
// RNE(fp32(amax / 6)), each channel the nearest E2M1 value of x/scale with
// ties to the even code (DeepSeek-V4.1-Flash course page, block 4A: FP4 latent
// with an E4M3 scale per 16 channels).
#pragma once

#include "internal.h"
#include "mla.h"

namespace mla {

__device__ __forceinline__ float load_src(const void* base, int64_t idx, int dtype) {
  if (dtype == MLA_F32) return reinterpret_cast<const float*>(base)[idx];
  return bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(base)[idx]);
}

// One 64-lane wave stores new token `token` (= b * Qn + j). The source row is
// read into registers before the length (and the page table) is looked at, so
// the row's load and the position lookup overlap instead of following each
// other.
constexpr int kAppendWords = 8;  // 4-byte words per lane and pass (2 KiB per wave)
__device__ __forceinline__ void append_token(const AppendParams& p, int token, int lane) {
  const int b = token / p.Qn;
  const int j = token % p.Qn;
  const int64_t src_row = (int64_t)b * p.Qn + j;
  const CacheView& c = p.cache;
  const int rope_words = p.Dr * (p.rope_dtype == MLA_F32 ? 4 : 2) / 4;
  const bool fp4 = p.latent_dtype == MLA_FP4_E2M1_E4M3X16;
  const int lat_words = fp4 ? 0 : p.Ckv * (p.latent_dtype == MLA_F32 ? 4 : 2) / 4;
  const uint32_t* __restrict__ src_pe = reinterpret_cast<const uint32_t*>(p.k_pe) + src_row * rope_words;
  const uint32_t* __restrict__ src_lat = reinterpret_cast<const uint32_t*>(p.c_kv) + src_row * lat_words;

  // First pass of the row (RoPE words, then latent words) into registers.
  const int total = rope_words + lat_words;
  uint32_t v[kAppendWords];
#pragma unroll
  for (int k = 0; k < kAppendWords; ++k) {
    const int i = lane + 64 * k;
    v[k] = i < rope_words ? src_pe[i] : (i < total ? src_lat[i - rope_words] : 0u);
  }
  const int len = p.seq_lens[b];
  const int pos = len - p.Qn + j;
  if (pos < 0 || pos >= c.capacity) return;
  bool bad = false;
  const int64_t r = phys_row(c, b, pos, bad);
  if (bad) return;
  uint32_t* dst_pe = reinterpret_cast<uint32_t*>(const_cast<uint8_t*>(c.rope) + r * c.rope_stride);
  uint8_t* lat = const_cast<uint8_t*>(c.latent) + r * c.latent_stride;
  uint32_t* dst_lat = reinterpret_cast<uint32_t*>(lat);
  for (int base = 0; base < total; base += 64 * kAppendWords) {
    if (base > 0) {
#pragma unroll
      for (int k = 0; k < kAppendWords; ++k) {
        const int i = base + lane + 64 * k;
        v[k] = i < rope_words ? src_pe[i] : (i < total ? src_lat[i - rope_words] : 0u);
      }
    }
#pragma unroll
    for (int k = 0; k < kAppendWords; ++k) {
      const int i = base + lane + 64 * k;
      if (i < rope_words) dst_pe[i] = v[k];
      else if (i < total) dst_lat[i - rope_words] = v[k];
    }
  }
  if (!fp4) return;

  // FP4: a pair of lanes per 16-channel group, 8 channels per lane.
  uint8_t* scl = const_cast<uint8_t*>(c.scale) + r * c.scale_stride;
  for (int c0 = lane * 8; c0 < p.Ckv; c0 += 64 * 8) {
    float v[8];
    float amax = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      v[e] = load_src(p.c_kv, src_row * p.Ckv + c0 + e, p.src_dtype);
      amax = fmaxf(amax, fabsf(v[e]));
    }
    amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
    const uint32_t sc = e4m3_encode_rne(__fdiv_rn(amax, 6.0f));  // correctly rounded fp32 division
    const float s = e4m3_to_f32(sc);
    uint32_t word = 0;
    if (s > 0.0f) {
#pragma unroll
      for (int e = 0; e < 8; ++e) word |= e2m1_encode(v[e], s) << (4 * e);
    }
    *reinterpret_cast<uint32_t*>(lat + c0 / 2) = word;
    if ((lane & 1) == 0) scl[c0 / 16] = (uint8_t)sc;
  }
}

}  // namespace mla
