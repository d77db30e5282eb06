// Absorbed MLA decode attention on gfx950 matrix cores (bf16 or FP4 latent).
//
// All heads of a sequence share one latent row per token (DeepSeek-V3 deep-dive
// page: absorption on the query side; exercise page: scores against kv_cache
// and pe_cache, weighted sum over kv_cache). So one workgroup takes 128 query
// rows (h, q) of one sequence and streams that sequence's cache through LDS
// once for all of them:
//
//   S^T[t, r] = sum_c  K[t, c] * Qcat[r, c]      c over 512 latent + 64 RoPE
//   online softmax over t per row r (scaled, causal limit per row)
//   O^T[c, r] += sum_t C^T[c, t] * P^T[t, r]     c over the 512 latent
//
// Both contractions are v_mfma_f32_32x32x16_bf16 with fp32 accumulation. A
// wave owns 32 query rows; its Q fragments stay in registers for the whole
// sequence and its O^T accumulator is 512 x 32 fp32.
//
// Tokens are split across workgroups (flash-decoding): the 64-token tiles of
// all sequences, laid end to end, are dealt in equal contiguous runs to the W
// workgroups of a row block. A workgroup whose run covers a whole sequence
// writes x and lse directly; a piece of a sequence is written as a partial
// (x_s normalised, lse_s) and merged afterwards by the combine kernel:
//   lse = log sum_s exp(lse_s),  x = sum_s exp(lse_s - lse) x_s.
#include "internal.h"

namespace mla {
namespace {

constexpr int kThreads = 256;
constexpr int kChunks = 72;     // 16-byte chunks per token: 64 latent + 8 RoPE
constexpr int kRowBytes = 1168;  // LDS bytes per token row: 72 chunks + 16 bytes of padding
constexpr int kTileBytes = kTileTokens * kRowBytes;
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kRescaleLog2 = 8.0f;

// LDS byte offset of 16-byte chunk lc of tile token t. Rows are padded by 16
// bytes (292 dwords) so that the same chunk of 8 consecutive tokens falls in 8
// different bank groups, and every operand address is a per-lane base plus a
// compile-time offset.
__device__ __forceinline__ uint32_t chunk_off(int t, int lc) {
  return (uint32_t)(t * kRowBytes + lc * 16);
}

__device__ __forceinline__ uint4 ld16(const uint8_t* p) {
  return *reinterpret_cast<const uint4*>(p);
}

// Tiles of sequence b (64-token granularity).
__device__ __forceinline__ int seq_tiles(const AttnParams& p, int b) {
  return (clamp_len(p.seq_lens[b], p.cache.capacity) + kTileTokens - 1) / kTileTokens;
}

// Block-wide exclusive scan of one int per thread (256 threads). Returns the
// exclusive prefix; *total receives the sum over the block.
__device__ int block_exclusive_scan(int v, int* s_tmp, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int inc = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int u = __shfl_up(inc, d, 64);
    if (lane >= d) inc += u;
  }
  if (lane == 63) s_tmp[wave] = inc;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kThreads / 64; ++w) {
    const int x = s_tmp[w];
    base += (w < wave) ? x : 0;
    tot += x;
  }
  __syncthreads();
  *total = tot;
  return base + inc - v;
}

// Fill the LDS tile with tokens [tile*64, tile*64+64) of sequence b. Tokens at
// or beyond L are zero so they add nothing to either product.
template <bool kFp4>
__device__ __forceinline__ void stage_tile(const AttnParams& p, int b, int tile, int L,
                                           uint8_t* s_tile, bool& bad) {
  const int tid = threadIdx.x;
  const CacheView& c = p.cache;
  if constexpr (!kFp4) {
    // 18 chunks per thread, issued 3 at a time to bound live registers.
#pragma unroll 1
    for (int k0 = 0; k0 < kTileTokens * kChunks / kThreads; k0 += 3) {
#pragma unroll
    for (int k = k0; k < k0 + 3; ++k) {
      const int s = tid + kThreads * k;
      const int t = s / kChunks;
      const int lc = s - t * kChunks;
      const int tok = tile * kTileTokens + t;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (tok < L) {
        const int64_t r = phys_row(c, b, tok, bad);
        v = lc < 64 ? ld16(c.latent + r * c.latent_stride + lc * 16)
                    : ld16(c.rope + r * c.rope_stride + (lc - 64) * 16);
      }
      *reinterpret_cast<uint4*>(s_tile + chunk_off(t, lc)) = v;
    }
    }
  } else {
    // 16 code chunks (32 channels each) per token: 1024 per tile.
#pragma unroll
    for (int k = 0; k < kTileTokens * 16 / kThreads; ++k) {
      const int s = tid + kThreads * k;
      const int t = s >> 4;
      const int j = s & 15;
      const int tok = tile * kTileTokens + t;
      uint4 codes = make_uint4(0, 0, 0, 0);
      uint32_t sc = 0;
      if (tok < L) {
        const int64_t r = phys_row(c, b, tok, bad);
        codes = ld16(c.latent + r * c.latent_stride + j * 16);
        sc = *reinterpret_cast<const uint16_t*>(c.scale + r * c.scale_stride + j * 2);
      }
      const float s0 = e4m3_to_f32(sc & 0xffu);
      const float s1 = e4m3_to_f32(sc >> 8);
      const uint32_t words[4] = {codes.x, codes.y, codes.z, codes.w};
#pragma unroll
      for (int qd = 0; qd < 4; ++qd) {
        const float sv = qd < 2 ? s0 : s1;
        uint32_t outw[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t n0 = (words[qd] >> (8 * e)) & 0xfu;
          const uint32_t n1 = (words[qd] >> (8 * e + 4)) & 0xfu;
          const float v0 = __uint_as_float(e2m1_f32_bits(n0)) * sv;
          const float v1 = __uint_as_float(e2m1_f32_bits(n1)) * sv;
          // Products are exact in bf16: keep the upper half of the fp32 bits.
          outw[e] = (__float_as_uint(v0) >> 16) | (__float_as_uint(v1) & 0xffff0000u);
        }
        *reinterpret_cast<uint4*>(s_tile + chunk_off(t, 4 * j + qd)) =
            make_uint4(outw[0], outw[1], outw[2], outw[3]);
      }
    }
#pragma unroll
    for (int k = 0; k < kTileTokens * 8 / kThreads; ++k) {
      const int s = tid + kThreads * k;
      const int t = s >> 3;
      const int j = s & 7;
      const int tok = tile * kTileTokens + t;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (tok < L) {
        const int64_t r = phys_row(c, b, tok, bad);
        v = ld16(c.rope + r * c.rope_stride + j * 16);
      }
      *reinterpret_cast<uint4*>(s_tile + chunk_off(t, 64 + j)) = v;
    }
  }
}

template <bool kFp4>
__global__ void __launch_bounds__(kThreads, 1) attn_bf16_kernel(AttnParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t s_tile[kTileBytes];
  __shared__ int s_tmp[8];
  __shared__ int s_start[2];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int hi = lane >> 5;
  const int g = blockIdx.y;
  const int wg = blockIdx.x;

  // ---- work range: tiles [start, end) of the concatenated sequences ----
  const int per_thread = (p.B + kThreads - 1) / kThreads;
  const int b_lo = min(p.B, tid * per_thread);
  const int b_hi = min(p.B, b_lo + per_thread);
  int my_tiles = 0;
  for (int b = b_lo; b < b_hi; ++b) my_tiles += seq_tiles(p, b);
  int total = 0;
  const int base = block_exclusive_scan(my_tiles, s_tmp, &total);
  const int per = (total + p.workgroups - 1) / p.workgroups;
  const int start = wg * per;
  const int end = min(total, start + per);
  if (start >= end) return;  // uniform over the block
  if (start >= base && start < base + my_tiles) {
    int acc = base;
    for (int b = b_lo; b < b_hi; ++b) {
      const int n = seq_tiles(p, b);
      if (start < acc + n) {
        s_start[0] = b;
        s_start[1] = start - acc;
        break;
      }
      acc += n;
    }
  }
  __syncthreads();

  const int row_local = wave * 32 + (lane & 31);
  const int row = g * kRowsPerGroup + row_local;
  const bool row_ok = row < p.HQ;
  const int qi = row_ok ? row % p.Q : 0;
  const int slots = 2 * p.workgroups;

  int b = s_start[0];
  int tile = s_start[1];
  int remaining = end - start;
  bool first_segment = true;
  while (remaining > 0) {
    const int L = clamp_len(p.seq_lens[b], p.cache.capacity);
    const int nt = (L + kTileTokens - 1) / kTileTokens;
    const int seg_lo = tile;
    const int seg_hi = min(nt, tile + remaining);
    const int vis = L - p.Q + qi + 1;  // this lane's row sees tokens t < vis

    // Q fragments (B operand of S^T = K . Qcat^T): row `row`, channels
    // 16*ks + 8*hi .. +7 of [q_lat | q_pe].
    bf16x8 qf[36];
    {
      const int64_t grow = (int64_t)b * p.HQ + (row_ok ? row : 0);
      const uint16_t* ql = reinterpret_cast<const uint16_t*>(p.q_lat) + grow * 512;
      const uint16_t* qp = reinterpret_cast<const uint16_t*>(p.q_pe) + grow * 64;
#pragma unroll
      for (int ks = 0; ks < 32; ++ks) {
        qf[ks] = row_ok ? *reinterpret_cast<const bf16x8*>(ql + 16 * ks + 8 * hi) : bf16x8{};
      }
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        qf[32 + ks] = row_ok ? *reinterpret_cast<const bf16x8*>(qp + 16 * ks + 8 * hi) : bf16x8{};
      }
    }

    floatx16 o[16];
#pragma unroll
    for (int cb = 0; cb < 16; ++cb) o[cb] = floatx16{};
    float m = -INFINITY;
    float l = 0.0f;
    int seg_bad = 0;

    for (tile = seg_lo; tile < seg_hi; ++tile) {
      __syncthreads();  // previous tile fully consumed
      bool bad = false;
      stage_tile<kFp4>(p, b, tile, L, s_tile, bad);
      seg_bad |= __syncthreads_or(bad ? 1 : 0);

      // ---- S^T = K . Qcat^T for two 32-token blocks ----
      floatx16 s[2];
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
        floatx16 acc = floatx16{};
        const int t = tb * 32 + (lane & 31);
#pragma unroll
        for (int ks = 0; ks < 36; ++ks) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(s_tile + chunk_off(t, 2 * ks + hi));
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], acc, 0, 0, 0);
          if ((ks & 3) == 3) __builtin_amdgcn_sched_barrier(0);
        }
        s[tb] = acc;
      }

      // ---- online softmax (log2 domain); lane holds row `row`, 32 tokens ----
      float mx = -INFINITY;
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int tok = tile * kTileTokens + tb * 32 + 8 * (i >> 2) + 4 * hi + (i & 3);
          const float v = tok < vis ? s[tb][i] * p.scale_log2 : -INFINITY;
          s[tb][i] = v;
          mx = fmaxf(mx, v);
        }
      }
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      // Lazy rescaling: the exponent reference m moves only when the tile
      // maximum exceeds it by more than kRescaleLog2, so probabilities stay
      // <= 2^kRescaleLog2 and O is rarely touched outside the matrix cores.
      const bool upd = mx > m + kRescaleLog2;
      const float m_new = upd ? mx : m;
      const float alpha = upd ? exp2f(m - m_new) : 1.0f;
      const float m_use = m_new == -INFINITY ? 0.0f : m_new;
      float sum = 0.0f;
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float e = exp2f(s[tb][i] - m_use);
          s[tb][i] = e;
          sum += e;
        }
      }
      sum += __shfl_xor(sum, 32, 64);
      l = l * alpha + sum;
      if (__any(upd && m != -INFINITY)) {
#pragma unroll
        for (int cb = 0; cb < 16; ++cb) o[cb] *= alpha;
      }
      m = m_new;

      // P^T fragments: k-step kk = (tb, ss) uses registers 8*ss .. 8*ss+7 of block tb.
      bf16x8 pf[4];
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int tb = kk >> 1, ss = kk & 1;
        bf16x8 f;
#pragma unroll
        for (int j = 0; j < 8; ++j) f[j] = (__bf16)s[tb][8 * ss + j];
        pf[kk] = f;
      }

      // ---- O^T += C^T . P^T ----
      // A operand: channel cb*32 + lane%32, tokens of k-step kk in the order
      // the P^T registers hold them: 16*kk + 4*hi + {0,1,2,3,8,9,10,11}.
#pragma unroll
      for (int cb = 0; cb < 16; ++cb) {
        const int ch = cb * 32 + (lane & 31);
        const int lc = ch >> 3;
        const uint32_t cofs = (uint32_t)(ch & 7) * 2u;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          bf16x8 a;
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const int tok = 16 * kk + 4 * hi + (j & 3) + 8 * (j >> 2);
            a[j] = *reinterpret_cast<const __bf16*>(s_tile + chunk_off(tok, lc) + cofs);
          }
          o[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[kk], o[cb], 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }

    // ---- finish the segment ----
    const bool whole = seg_lo == 0 && seg_hi == nt;
    const float inv_l = l > 0.0f ? 1.0f / l : 0.0f;
    float lse_v = l > 0.0f ? (m + log2f(l)) * kLn2 : -INFINITY;
    if (seg_bad) lse_v = __uint_as_float(0x7fc00000u);
    const float nanv = __uint_as_float(0x7fc00000u);
    if (row_ok) {
      if (whole) {
        uint16_t* xo = reinterpret_cast<uint16_t*>(p.x_lat) + ((int64_t)b * p.HQ + row) * 512;
#pragma unroll
        for (int cb = 0; cb < 16; ++cb) {
#pragma unroll
          for (int i4 = 0; i4 < 4; ++i4) {
            const int ch = cb * 32 + 8 * i4 + 4 * hi;
            float v[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = seg_bad ? nanv : o[cb][4 * i4 + e] * inv_l;
            *reinterpret_cast<uint2*>(xo + ch) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
          }
        }
        if (p.lse != nullptr && hi == 0) p.lse[(int64_t)b * p.HQ + row] = lse_v;
      } else {
        const int slot = 2 * wg + (first_segment ? 0 : 1);
        const int64_t prow = ((int64_t)g * slots + slot) * kRowsPerGroup + row_local;
        float* xo = p.part_x + prow * 512;
#pragma unroll
        for (int cb = 0; cb < 16; ++cb) {
#pragma unroll
          for (int i4 = 0; i4 < 4; ++i4) {
            const int ch = cb * 32 + 8 * i4 + 4 * hi;
            float4 v;
            v.x = o[cb][4 * i4 + 0] * inv_l;
            v.y = o[cb][4 * i4 + 1] * inv_l;
            v.z = o[cb][4 * i4 + 2] * inv_l;
            v.w = o[cb][4 * i4 + 3] * inv_l;
            *reinterpret_cast<float4*>(xo + ch) = v;
          }
        }
        if (hi == 0) p.part_lse[prow] = lse_v;
      }
    }

    remaining -= seg_hi - seg_lo;
    first_segment = false;
    ++b;
    tile = 0;
    // Skip sequences without tiles (they own no part of the range).
    while (remaining > 0 && b < p.B && seq_tiles(p, b) == 0) ++b;
  }
}

// Merge partial results of sequences whose tiles were split over workgroups,
// and write x = 0 / lse = -inf for sequences without any cache rows.
// Grid: (B, groups * 8); each block handles 16 query rows of one sequence.
__global__ void __launch_bounds__(kThreads) attn_combine_kernel(AttnParams p) {
  __shared__ int s_tmp[8];
  const int tid = threadIdx.x;
  const int b = blockIdx.x;
  const int g = blockIdx.y >> 3;
  const int rb = blockIdx.y & 7;

  const int per_thread = (p.B + kThreads - 1) / kThreads;
  const int b_lo = min(p.B, tid * per_thread);
  const int b_hi = min(p.B, b_lo + per_thread);
  int my_tiles = 0;
  int before = 0;  // tiles of sequences < b in this thread's range
  for (int j = b_lo; j < b_hi; ++j) {
    const int n = seq_tiles(p, j);
    my_tiles += n;
    if (j < b) before += n;
  }
  int total = 0;
  const int base = block_exclusive_scan(before, s_tmp, &total);  // sum over threads -> cum_b
  (void)base;
  const int cum_b = total;
  int total_tiles = 0;
  block_exclusive_scan(my_tiles, s_tmp, &total_tiles);
  const int nb = seq_tiles(p, b);

  const int row_local = rb * 16 + (tid >> 4);
  const int row = g * kRowsPerGroup + row_local;
  const int c0 = (tid & 15) * 32;
  if (row >= p.HQ) return;
  const int64_t grow = (int64_t)b * p.HQ + row;
  uint16_t* xo = reinterpret_cast<uint16_t*>(p.x_lat) + grow * p.Ckv;

  if (nb == 0) {
#pragma unroll
    for (int k = 0; k < 8; ++k) *reinterpret_cast<uint2*>(xo + c0 + 4 * k) = make_uint2(0, 0);
    if (p.lse != nullptr && (tid & 15) == 0) p.lse[grow] = -INFINITY;
    return;
  }
  const int per = (total_tiles + p.workgroups - 1) / p.workgroups;
  const int i_first = cum_b / per;
  const int i_last = (cum_b + nb - 1) / per;
  if (i_first == i_last) return;  // the attention kernel wrote this sequence directly

  const int slots = 2 * p.workgroups;
  auto slot_of = [&](int i) { return 2 * i + ((i == i_first && cum_b != i_first * per) ? 1 : 0); };
  float mx = -INFINITY;
  bool any_nan = false;
  for (int i = i_first; i <= i_last; ++i) {
    const float v = p.part_lse[((int64_t)g * slots + slot_of(i)) * kRowsPerGroup + row_local];
    any_nan |= v != v;
    mx = fmaxf(mx, v);
  }
  float acc[32];
#pragma unroll
  for (int k = 0; k < 32; ++k) acc[k] = 0.0f;
  float lse_v;
  if (any_nan) {
    lse_v = __uint_as_float(0x7fc00000u);
#pragma unroll
    for (int k = 0; k < 32; ++k) acc[k] = lse_v;
  } else if (mx == -INFINITY) {
    lse_v = -INFINITY;
  } else {
    float tot = 0.0f;
    for (int i = i_first; i <= i_last; ++i) {
      tot += __expf(p.part_lse[((int64_t)g * slots + slot_of(i)) * kRowsPerGroup + row_local] - mx);
    }
    lse_v = mx + __logf(tot);
    for (int i = i_first; i <= i_last; ++i) {
      const int64_t prow = ((int64_t)g * slots + slot_of(i)) * kRowsPerGroup + row_local;
      const float w = __expf(p.part_lse[prow] - lse_v);
      if (w == 0.0f) continue;
      const float4* src = reinterpret_cast<const float4*>(p.part_x + prow * 512 + c0);
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const float4 v = src[k];
        acc[4 * k + 0] += w * v.x;
        acc[4 * k + 1] += w * v.y;
        acc[4 * k + 2] += w * v.z;
        acc[4 * k + 3] += w * v.w;
      }
    }
  }
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    *reinterpret_cast<uint2*>(xo + c0 + 4 * k) =
        make_uint2(pack_bf16x2(acc[4 * k], acc[4 * k + 1]), pack_bf16x2(acc[4 * k + 2], acc[4 * k + 3]));
  }
  if (p.lse != nullptr && (tid & 15) == 0) p.lse[grow] = lse_v;
}

}  // namespace

hipError_t launch_attn_bf16(const AttnParams& p, bool fp4_latent, hipStream_t s) {
  const dim3 grid(p.workgroups, p.groups);
  if (fp4_latent) {
    hipLaunchKernelGGL(attn_bf16_kernel<true>, grid, dim3(kThreads), 0, s, p);
  } else {
    hipLaunchKernelGGL(attn_bf16_kernel<false>, grid, dim3(kThreads), 0, s, p);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(attn_combine_kernel, dim3(p.B, p.groups * 8), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace mla
