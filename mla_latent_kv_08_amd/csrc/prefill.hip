// Attention for many new tokens per sequence (prefill, large Q) in the
// non-absorbed form the CANN fused-operator page describes: per chunk of cached
// tokens, the per-head key and value are decompressed from the latent in
// on-chip memory (K = C W_UK^T, V = C W_UV^T) and never written back, then used
// by an online-softmax attention. (CANN page, section 2: the chunk loop with
// the up-projection of K kept in local memory; exercise page: the scores
// q_nope.K_nope + q_pe.k_pe, scaled and causally masked, softmax, P.V.)
//
// Block (query tile of 64, head h, sequence b), 512 threads. Wave w holds, in
// registers for the whole block, the matrix-op fragments of one 32-row slice
// of the head's weights: W_UK rows 32w .. 32w+31 for w < 4, W_UV rows
// 32(w-4) .. for w >= 4, all 512 latent channels (128 VGPRs). For each tile
// of 32 cached tokens:
//   1. the latent rows go to LDS; the RoPE keys go straight to the key tile;
//   2. every wave forms its 32 x 32 slice of K (token-major) or V (stored
//      transposed, value-major) with v_mfma_f32_32x32x16_bf16, A = the latent
//      rows from LDS, B = its weight fragments;
//   3. waves 0..3 each take 16 queries: S = [q_nope | q_pe] . [K | k_pe]^T over
//      192 dims (v_mfma_f32_16x16x32_bf16), scale, causal limit, online softmax
//      (fp32 running max and sum per query), P in bf16 through LDS, O += P V.
// Query j of a sequence with `len` cached tokens (the Q new ones included) sees
// positions 0 .. len - Q + j. A query that sees nothing gets out = 0 and
// lse = -inf; a page index outside the cache makes the block's outputs NaN.
#include "prefill.h"

namespace mla {
namespace {

constexpr int kPfThreads = 512;
constexpr int kPfQ = 64;        // queries per block
constexpr int kPfT = 32;        // tokens per tile
static_assert(kPageTokens % kPfT == 0, "a tile never crosses a page");
constexpr int kCPitch = 520;    // latent row pitch in LDS (bf16)
constexpr int kKPitch = 200;    // key row pitch: 128 decompressed + 64 RoPE + pad
constexpr int kVPitch = 40;     // transposed value row pitch: 32 tokens + pad
constexpr int kPPitch = 40;     // probability row pitch: 32 tokens + pad
constexpr float kLn2 = 0.69314718055994530942f;

struct PrefillLds {
  uint16_t q[kPfQ * kKPitch];
  uint16_t c[2][kPfT * kCPitch];
  uint16_t k[2][kPfT * kKPitch];
  uint16_t vt[128 * kVPitch];
  uint16_t p[4][16 * kPPitch];
  int bad;
};

__device__ __forceinline__ uint16_t to_bf16(float v) { return (uint16_t)f32_to_bf16_bits(v); }

__global__ void __launch_bounds__(kPfThreads) prefill_kernel(PrefillParams p) {
  __shared__ __attribute__((aligned(16))) PrefillLds s;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, hi = lane >> 5;
  const int q0 = blockIdx.x * kPfQ;
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const int H = p.H, Q = p.Q;
  const CacheView& c = p.cache;
  const int len = clamp_len(p.seq_lens[b], c.capacity);
  const uint16_t* wkv = reinterpret_cast<const uint16_t*>(p.wkv_b) + (int64_t)h * 256 * 512;

  // This wave's weight slice: B lane l = weight row 32(w%4) + l%32 (of W_UK or
  // W_UV), channels 16ks + 8(l/32) .. +7.
  bf16x8 wf[32];
  {
    const uint16_t* wr = wkv + (int64_t)((wave >= 4 ? 128 : 0) + 32 * (wave & 3) + (lane & 31)) * 512 + 8 * hi;
#pragma unroll
    for (int ks = 0; ks < 32; ++ks) wf[ks] = *reinterpret_cast<const bf16x8*>(wr + 16 * ks);
  }
  // The block's query rows [q_nope (128) | q_pe (64)] to LDS (rows past Q
  // repeat the last one; their scores are masked out).
  for (int sidx = tid; sidx < kPfQ * 24; sidx += kPfThreads) {
    const int r = sidx / 24, ch = sidx - 24 * r;
    const int qi = min(q0 + r, Q - 1);
    const int64_t row = ((int64_t)b * H + h) * Q + qi;
    const uint16_t* src = ch < 16 ? reinterpret_cast<const uint16_t*>(p.q_nope) + row * 128 + 8 * ch
                                  : reinterpret_cast<const uint16_t*>(p.q_pe) + row * 64 + 8 * (ch - 16);
    *reinterpret_cast<uint4*>(&s.q[r * kKPitch + 8 * ch]) = *reinterpret_cast<const uint4*>(src);
  }
  const int l16 = lane & 15, g4 = lane >> 4;
  if (tid == 0) s.bad = 0;
  // Rows of this lane in the 16 x 16 result layouts: queries 4*(l/16) + i.
  float m[4], l[4];
  floatx4 o[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    m[i] = -INFINITY;
    l[i] = 0.0f;
  }
#pragma unroll
  for (int vb = 0; vb < 8; ++vb) o[vb] = floatx4{};

  // Tiles up to the last position any query of the block sees.
  const int pos_max = len - Q + min(q0 + kPfQ - 1, Q - 1);
  const int n_tiles = pos_max < 0 ? 0 : min(pos_max / kPfT + 1, (len + kPfT - 1) / kPfT);
  // Tile i uses buffers i % 2 of the latent rows and the keys. Waves 4..7
  // fetch tile i+1 into the other buffers while waves 0..3 run tile i's
  // attention: chunk j < 8 of thread u = tid - 256 is latent row
  // u / 64 + 4j, 16-byte chunk u % 64; chunk 8 is RoPE row u / 8, chunk u % 8.
  const int u = tid - 256;
  auto fetch = [&](int t0, int buf) {
    // A 32-token tile lies inside one 64-token page: one page lookup and one
    // bounds check per tile (the same for every thread). Rows past len are
    // read at the last row (always in bounds) and replaced by zeros, so the
    // nine loads carry no branches and are in flight together.
    const int last = min(kPfT - 1, len - 1 - t0);
    int64_t base;
    bool bad = false;
    if (c.page_size == 0) {
      base = (int64_t)b * c.capacity + t0;
    } else {
      // The same rule as the decode kernel: the whole page must exist (a
      // paged pool's num_rows is a multiple of the page size).
      const int page = c.page_table[(int64_t)b * c.pt_stride + t0 / kPageTokens];
      const int64_t p0 = (int64_t)page * kPageTokens;
      base = p0 + t0 % kPageTokens;
      bad = page < 0 || p0 + kPageTokens > c.num_rows;
    }
    bf16x8 pf[9];
    if (bad) {
      s.bad = 1;
#pragma unroll
      for (int j = 0; j < 9; ++j) pf[j] = bf16x8{};
    } else {
      const uint8_t* lat = c.latent + (u & 63) * 16;
      const int r0 = u >> 6;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        pf[j] = *reinterpret_cast<const bf16x8*>(lat + (base + min(r0 + 4 * j, last)) * c.latent_stride);
      }
      pf[8] = *reinterpret_cast<const bf16x8*>(c.rope + (base + min(u >> 3, last)) * c.rope_stride + (u & 7) * 16);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (r0 + 4 * j > last) pf[j] = bf16x8{};
      }
      if ((u >> 3) > last) pf[8] = bf16x8{};
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int sidx = u + 256 * j;
      *reinterpret_cast<bf16x8*>(&s.c[buf][(sidx >> 6) * kCPitch + (sidx & 63) * 8]) = pf[j];
    }
    *reinterpret_cast<bf16x8*>(&s.k[buf][(u >> 3) * kKPitch + 128 + (u & 7) * 8]) = pf[8];
  };
  __syncthreads();  // the flag is cleared before any fetch can set it
  if (wave >= 4 && n_tiles > 0) fetch(0, 0);
  for (int tile = 0; tile < n_tiles; ++tile) {
    const int t0 = tile * kPfT;
    const int buf = tile & 1;
    // Tile `tile` is in buffers `buf`; the previous tile's attention is done
    // with the transposed values.
    __syncthreads();
    // ---- 2. decompress: D[token][n] = sum_k C[token][k] W[n][k] for this wave's 32 rows n ----
    {
      floatx16 acc = floatx16{};
      const uint16_t* a = &s.c[buf][(lane & 31) * kCPitch + 8 * hi];
#pragma unroll
      for (int ks = 0; ks < 32; ++ks) {
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8*>(a + 16 * ks), wf[ks], acc, 0,
                                                      0, 0);
        // Keep the LDS reads within groups of 8 k-steps: hoisting all of them
        // would need another 128 registers.
        if ((ks & 7) == 7) __builtin_amdgcn_sched_barrier(0);
      }
      // D lane l: column n = 32(w%4) + l%32, tokens 8(i/4) + 4(l/32) + i%4.
      const int n = 32 * (wave & 3) + (lane & 31);
      if (wave < 4) {
#pragma unroll
        for (int i = 0; i < 16; ++i) s.k[buf][(8 * (i >> 2) + 4 * hi + (i & 3)) * kKPitch + n] = to_bf16(acc[i]);
      } else {
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          *reinterpret_cast<uint2*>(&s.vt[n * kVPitch + 8 * i4 + 4 * hi]) =
              make_uint2(pack_bf16x2(acc[4 * i4], acc[4 * i4 + 1]), pack_bf16x2(acc[4 * i4 + 2], acc[4 * i4 + 3]));
        }
      }
    }
    __syncthreads();
    // ---- 3. attention for 16 queries per wave (waves 0..3); the next tile's fetch (4..7) ----
    if (wave >= 4) {
      if (tile + 1 < n_tiles) fetch(t0 + kPfT, buf ^ 1);
    } else {
      floatx4 sc[2] = {floatx4{}, floatx4{}};
      // A lane l: query q0 + 16w + l%16, dims 32ks + 8(l/16) .. +7.
      const uint16_t* qr = &s.q[(16 * wave + l16) * kKPitch + 8 * g4];
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
        const uint16_t* kr = &s.k[buf][(16 * tb + l16) * kKPitch + 8 * g4];
#pragma unroll
        for (int ks = 0; ks < 6; ++ks) {
          sc[tb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*reinterpret_cast<const bf16x8*>(qr + 32 * ks),
                                                           *reinterpret_cast<const bf16x8*>(kr + 32 * ks), sc[tb], 0,
                                                           0, 0);
        }
      }
      // S lane l: token t0 + 16tb + l%16, queries q0 + 16w + 4(l/16) + i.
      float pr[2][4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int qg = q0 + 16 * wave + 4 * g4 + i;
        const int pos = len - Q + qg;
        float x[2];
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
          const int t = t0 + 16 * tb + l16;
          x[tb] = (qg < Q && t <= pos && t < len) ? sc[tb][i] * p.scale_log2 : -INFINITY;
        }
        float mx = fmaxf(x[0], x[1]);
#pragma unroll
        for (int d = 1; d < 16; d <<= 1) mx = fmaxf(mx, __shfl_xor(mx, d, 16));
        const float m_new = fmaxf(m[i], mx);
        const float alpha = m_new == m[i] ? 1.0f : __builtin_amdgcn_exp2f(m[i] - m_new);
        const float mu = m_new == -INFINITY ? 0.0f : m_new;
        float rs = 0.0f;
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
          pr[tb][i] = __builtin_amdgcn_exp2f(x[tb] - mu);
          rs += pr[tb][i];
        }
#pragma unroll
        for (int d = 1; d < 16; d <<= 1) rs += __shfl_xor(rs, d, 16);
        l[i] = l[i] * alpha + rs;
        m[i] = m_new;
#pragma unroll
        for (int vb = 0; vb < 8; ++vb) o[vb][i] *= alpha;
      }
      // P to this wave's LDS rows [query 4(l/16)+i][token 16tb + l%16], then
      // read back as the A operand (query l%16, tokens 8(l/16) .. +7).
      uint16_t* pw = s.p[wave];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) pw[(4 * g4 + i) * kPPitch + 16 * tb + l16] = to_bf16(pr[tb][i]);
      }
      const bf16x8 pa = *reinterpret_cast<const bf16x8*>(&pw[l16 * kPPitch + 8 * g4]);
#pragma unroll
      for (int vb = 0; vb < 8; ++vb) {
        const bf16x8 vbk = *reinterpret_cast<const bf16x8*>(&s.vt[(16 * vb + l16) * kVPitch + 8 * g4]);
        o[vb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, vbk, o[vb], 0, 0, 0);
      }
    }
  }
  __syncthreads();
  if (wave < 4) {
    const bool bad = s.bad != 0;
    const float nanv = __uint_as_float(0x7fc00000u);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int qg = q0 + 16 * wave + 4 * g4 + i;
      if (qg >= Q) continue;
      const int64_t row = ((int64_t)b * H + h) * Q + qg;
      const float inv = l[i] > 0.0f ? 1.0f / l[i] : 0.0f;
      uint16_t* orow = reinterpret_cast<uint16_t*>(p.out) + row * 128;
#pragma unroll
      for (int vb = 0; vb < 8; ++vb) orow[16 * vb + l16] = to_bf16(bad ? nanv : o[vb][i] * inv);
      if (p.lse != nullptr && l16 == 0) {
        p.lse[row] = bad ? nanv : (l[i] > 0.0f ? (m[i] + __log2f(l[i])) * kLn2 : -INFINITY);
      }
    }
  }
}

}  // namespace

hipError_t launch_prefill(const PrefillParams& p, hipStream_t s) {
  if (p.B == 0 || p.Q == 0) return hipSuccess;
  const int qt = (p.Q + kPfQ - 1) / kPfQ;
  if (p.H > 65535 || p.B > 65535) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(prefill_kernel, dim3(qt, p.H, p.B), dim3(kPfThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace mla
