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
//
// With a cosine/sine table the RoPE key is turned to its position before it is
// stored, and the step's queries (q_pe, the same positions) are turned in
// place (deep-dive page, forward_inference: the new token's RoPE key is the
// rotated projection; course page, block 4A: rotation by the cosine and sine
// of the position's angle). Pair i of the Dr/2 pairs, (2i, 2i+1) interleaved
// or (i, i + Dr/2) in halves, turns by angle a_i of the position's table row:
// (x, y) -> (x cos a_i - y sin a_i, x sin a_i + y cos a_i) in fp32, rounded
// once to the stored dtype. A position outside the table gives NaN.
//
// Latent-tail mode (DeepSeek-V4.1-Flash course page, block 4A: the rotary
// position sits on the tail of the latent, which serves as key and value):
// the last Dr dims of the new latent are turned instead of a separate key,
// before an FP4 latent is quantised; the row's RoPE slot is filled with zeros;
// the query rows are [B, H, Qn, Ckv] with their last Dr dims turned.
#pragma once

#include "internal.h"
#include "mla.h"

namespace mla {

__device__ __forceinline__ float load_src(const void* base, int64_t idx, int dtype) {
  if (dtype == MLA_F32) return reinterpret_cast<const float*>(base)[idx];
  return bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(base)[idx]);
}

__device__ __forceinline__ void store_dst(void* base, int64_t idx, int dtype, float v) {
  if (dtype == MLA_F32) {
    reinterpret_cast<float*>(base)[idx] = v;
  } else {
    reinterpret_cast<uint16_t*>(base)[idx] = (uint16_t)f32_to_bf16_bits(v);
  }
}

// Elements of rotated pair i of a Dr-wide vector.
__device__ __forceinline__ void rope_pair(const AppendParams& p, int i, int& i0, int& i1) {
  if (p.rope_style == MLA_ROPE_INTERLEAVED) {
    i0 = 2 * i;
    i1 = 2 * i + 1;
  } else {
    i0 = i;
    i1 = i + p.Dr / 2;
  }
}

// Element u (< Dr) of the turned tail of the new latent row `src_row`: the
// first or second output of its pair, from the source row (the pair's partner
// may belong to another lane).
__device__ __forceinline__ float tail_value(const AppendParams& p, int64_t src_row, int u, int pos) {
  const int half = p.Dr / 2;
  int i, first, second;
  bool is_second;
  if (p.rope_style == MLA_ROPE_INTERLEAVED) {
    i = u >> 1;
    is_second = u & 1;
    first = 2 * i;
    second = 2 * i + 1;
  } else {
    is_second = u >= half;
    i = is_second ? u - half : u;
    first = i;
    second = i + half;
  }
  const int64_t base = src_row * p.Ckv + (p.Ckv - p.Dr);
  const float x = load_src(p.c_kv, base + first, p.src_dtype);
  const float y = load_src(p.c_kv, base + second, p.src_dtype);
  float c = __uint_as_float(0x7fc00000u), s = c;
  if (pos >= 0 && pos < p.n_pos) {
    const float* row = p.cos_sin + (int64_t)pos * p.Dr;
    c = row[i];
    s = row[half + i];
  }
  return is_second ? __builtin_fmaf(x, s, y * c) : __builtin_fmaf(x, c, -(y * s));
}

// Pair i of src (element offset `so`, dtype `sd`) turned to position `pos`,
// stored to dst (offset `dof`, dtype `dd`); NaN outside the table.
__device__ __forceinline__ void rope_rotate_pair(const AppendParams& p, int pos, int i, const void* src, int64_t so,
                                                 int sd, void* dst, int64_t dof, int dd) {
  int i0, i1;
  rope_pair(p, i, i0, i1);
  const float x = load_src(src, so + i0, sd);
  const float y = load_src(src, so + i1, sd);
  float c = __uint_as_float(0x7fc00000u), s = c;
  if (pos >= 0 && pos < p.n_pos) {
    const float* row = p.cos_sin + (int64_t)pos * p.Dr;
    c = row[i];
    s = row[p.Dr / 2 + i];
  }
  store_dst(dst, dof + i0, dd, __builtin_fmaf(x, c, -(y * s)));
  store_dst(dst, dof + i1, dd, __builtin_fmaf(x, s, y * c));
}

// The step's queries q_pe [B, H, Qn, Dr], turned in place: one 64-lane wave
// takes pairs 512 * chunk .. +511 of all B*H*Qn*Dr/2 pairs (row (b, h, j),
// pair i), reads all of them before it writes any (the rotation is in place,
// so loads could not otherwise move above earlier stores), whatever the cache
// does with the token. Query j of sequence b has the position of new token j.
constexpr int kRopePairsPerLane = 8;
constexpr int kRopePairsPerChunk = 64 * kRopePairsPerLane;
__device__ __forceinline__ void rope_queries(const AppendParams& p, int64_t chunk, int lane) {
  const int half = p.Dr / 2;
  const int64_t total = (int64_t)p.B * p.H * p.Qn * half;
  float x[kRopePairsPerLane], y[kRopePairsPerLane], cs[kRopePairsPerLane], sn[kRopePairsPerLane];
  int64_t o0[kRopePairsPerLane], o1[kRopePairsPerLane];
  bool on[kRopePairsPerLane];
#pragma unroll
  for (int k = 0; k < kRopePairsPerLane; ++k) {
    const int64_t t = chunk * kRopePairsPerChunk + lane + 64 * k;
    on[k] = t < total;
    const int64_t row = on[k] ? t / half : 0;
    const int i = (int)(t - row * half);
    int i0, i1;
    rope_pair(p, on[k] ? i : 0, i0, i1);
    o0[k] = row * p.q_stride + p.q_off + i0;
    o1[k] = row * p.q_stride + p.q_off + i1;
    const int b = (int)(row / ((int64_t)p.H * p.Qn));
    const int j = (int)(row % p.Qn);
    const int pos = p.seq_lens[b] - p.Qn + j;
    x[k] = load_src(p.q_pe, o0[k], p.rope_dtype);
    y[k] = load_src(p.q_pe, o1[k], p.rope_dtype);
    cs[k] = __uint_as_float(0x7fc00000u);
    sn[k] = cs[k];
    if (pos >= 0 && pos < p.n_pos) {
      const float* r = p.cos_sin + (int64_t)pos * p.Dr;
      cs[k] = r[on[k] ? i : 0];
      sn[k] = r[half + (on[k] ? i : 0)];
    }
  }
#pragma unroll
  for (int k = 0; k < kRopePairsPerLane; ++k) {
    if (!on[k]) continue;
    store_dst(p.q_pe, o0[k], p.rope_dtype, __builtin_fmaf(x[k], cs[k], -(y[k] * sn[k])));
    store_dst(p.q_pe, o1[k], p.rope_dtype, __builtin_fmaf(x[k], sn[k], y[k] * cs[k]));
  }
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
  const bool rotate = p.cos_sin != nullptr;
  const bool tail = rotate && p.rope_tail;
  const bool has_rope = c.rope != nullptr;  // no RoPE section: the rotation lives in the latent's tail
  // Words copied as they are: the RoPE key only when it is not rotated; the
  // latent, without its tail in latent-tail mode.
  const int rope_words = rotate || !has_rope ? 0 : p.Dr * (p.rope_dtype == MLA_F32 ? 4 : 2) / 4;
  const bool fp4 = p.latent_dtype == MLA_FP4_E2M1_E4M3X16;
  const int lat_words = fp4 ? 0 : (tail ? p.Ckv - p.Dr : p.Ckv) * (p.latent_dtype == MLA_F32 ? 4 : 2) / 4;
  const int64_t lat_src_words = fp4 ? 0 : p.Ckv * (p.latent_dtype == MLA_F32 ? 4 : 2) / 4;
  const uint32_t* __restrict__ src_pe = reinterpret_cast<const uint32_t*>(p.k_pe) + src_row * rope_words;
  const uint32_t* __restrict__ src_lat = reinterpret_cast<const uint32_t*>(p.c_kv) + src_row * lat_src_words;

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
  if (rotate && !tail) {
    for (int i = lane; i < p.Dr / 2; i += 64) {
      rope_rotate_pair(p, pos, i, p.k_pe, src_row * p.Dr, p.rope_dtype, const_cast<uint8_t*>(c.rope) + r * c.rope_stride,
                       0, p.rope_dtype);
    }
  }
  if (tail) {
    for (int u = lane; u < p.Dr; u += 64) {
      if (has_rope) store_dst(const_cast<uint8_t*>(c.rope) + r * c.rope_stride, u, p.rope_dtype, 0.0f);
      if (!fp4) store_dst(lat, (p.Ckv - p.Dr) + u, p.latent_dtype, tail_value(p, src_row, u, pos));
    }
  }
  if (!fp4) return;

  // FP4: a pair of lanes per 16-channel group, 8 channels per lane.
  uint8_t* scl = const_cast<uint8_t*>(c.scale) + r * c.scale_stride;
  for (int c0 = lane * 8; c0 < p.Ckv; c0 += 64 * 8) {
    float v[8];
    float amax = 0.0f;
    int nan = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int ch = c0 + e;
      v[e] = tail && ch >= p.Ckv - p.Dr ? tail_value(p, src_row, ch - (p.Ckv - p.Dr), pos)
                                        : load_src(p.c_kv, src_row * p.Ckv + ch, p.src_dtype);
      amax = fmaxf(amax, fabsf(v[e]));
      nan |= v[e] != v[e] ? 1 : 0;
    }
    amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
    nan |= __shfl_xor(nan, 1, 64);
    // (A NaN element, from a position outside the RoPE table, gives the
    // group the E4M3 NaN scale, so the group decodes as NaN.)
    const uint32_t sc = nan ? 0x7fu : e4m3_encode_rne(__fdiv_rn(amax, 6.0f));  // correctly rounded fp32 division
    const float s = e4m3_value(sc);
    uint32_t word = 0;
    if (!nan && s > 0.0f) {
#pragma unroll
      for (int e = 0; e < 8; ++e) word |= e2m1_encode(v[e], s) << (4 * e);
    }
    *reinterpret_cast<uint32_t*>(lat + c0 / 2) = word;
    if ((lane & 1) == 0) scl[c0 / 16] = (uint8_t)sc;
  }
}

}  // namespace mla
