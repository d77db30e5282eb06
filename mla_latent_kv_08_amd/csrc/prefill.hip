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
//      transposed, value-major) with v_mfma_f32_32x32x16_bf16 from the latent
//      rows in LDS and its weight fragments (K as W C^T, so that a lane holds
//      runs of dims of one token; V as C W^T, runs of tokens of one dim);
//   3. waves 0..3 each take 16 queries: S^T = [K | k_pe] . [q_nope | q_pe]^T
//      over 192 dims (v_mfma_f32_16x16x32_bf16), scale, causal limit, online
//      softmax (fp32 reference max per query, moved only on a jump past 2^8;
//      sums per lane), and O^T += V^T P^T with P^T in bf16 straight from the
//      score registers (V^T's columns are stored in their token order).
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
constexpr float kLn2 = 0.69314718055994530942f;
// The reference maximum of a query moves only when a tile's maximum passes it
// by more than this many binary orders of magnitude, so P <= 2^8.
constexpr float kLazyRescaleLog2 = 8.0f;
// s_waitcnt immediate: no vector-memory operation outstanding (lgkm and exp
// counters left alone).
constexpr int kVmcntZero = (7 << 4) | (15 << 8);

struct PrefillLds {
  uint16_t q[kPfQ * kKPitch];
  uint16_t c[2][kPfT * kCPitch];
  uint16_t k[2][kPfT * kKPitch];
  uint16_t vt[128 * kVPitch];
  int bad;
};

__device__ __forceinline__ uint16_t to_bf16(float v) { return (uint16_t)f32_to_bf16_bits(v); }
// Two values to a bf16 pair by the hardware conversion (round to nearest even,
// as f32_to_bf16_bits for every finite value).
__device__ __forceinline__ uint32_t bf16_pair(float lo, float hi) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)lo) | ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)hi) << 16);
}

// Lanes l and l ^ 16 (or l ^ 32) combine a value; both get the same result,
// operands in the same order (v_permlane16_swap / v_permlane32_swap instead
// of an LDS permute). Two of them combine the four lanes l % 16 + 16g of a
// column of the 16 x 16 result layouts.
__device__ __forceinline__ float xor16_max(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor16_sum(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor32_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

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
  // Attention waves 0..3: lane l takes query qg = q0 + 16w + l%16 (in every
  // 16 x 16 result layout below the query is the column), which sees
  // positions 0 .. lim (lim = -1: none). Its reference maximum, its sum (per
  // lane; the four lanes of a query are added at the end) and O^T columns.
  const int qg = q0 + 16 * wave + l16;
  const int lim = qg < Q ? len - Q + qg : -1;
  float m = -INFINITY, lsum = 0.0f;
  floatx4 o[8];
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
      // K (waves 0..3) is formed transposed, D = W C^T, so that a lane holds
      // runs of 4 dims of one token (8-byte stores into the token-major key
      // rows); V (waves 4..7) as D = C W^T, runs of 4 tokens of one dim for
      // the value-major V^T. The operand layouts are the same either way.
      floatx16 acc = floatx16{};
      const uint16_t* a = &s.c[buf][(lane & 31) * kCPitch + 8 * hi];
      if (wave < 4) {
#pragma unroll
        for (int ks = 0; ks < 32; ++ks) {
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[ks], *reinterpret_cast<const bf16x8*>(a + 16 * ks), acc, 0,
                                                        0, 0);
          // Keep the LDS reads within groups of 8 k-steps: hoisting all of
          // them would need another 128 registers.
          if ((ks & 7) == 7) __builtin_amdgcn_sched_barrier(0);
        }
        // D lane l: token l%32, dims 32w + 8(i/4) + 4(l/32) + i%4.
        uint16_t* kd = &s.k[buf][(lane & 31) * kKPitch + 32 * wave + 4 * hi];
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4) {
          *reinterpret_cast<uint2*>(kd + 8 * a4) =
              make_uint2(bf16_pair(acc[4 * a4], acc[4 * a4 + 1]), bf16_pair(acc[4 * a4 + 2], acc[4 * a4 + 3]));
        }
      } else {
#pragma unroll
        for (int ks = 0; ks < 32; ++ks) {
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8*>(a + 16 * ks), wf[ks], acc, 0,
                                                        0, 0);
          if ((ks & 7) == 7) __builtin_amdgcn_sched_barrier(0);
        }
        // D lane l: dim n = 32(w-4) + l%32, tokens 8(i/4) + 4(l/32) + i%4.
        // V^T's columns run in the order the attention waves hold their
        // probabilities: column 8g + j is token 4g + j for j < 4 and token
        // 16 + 4g + j - 4 otherwise, so tokens 8 i4 + 4 hi .. +3 go to column
        // 8 (2 (i4 % 2) + hi) + 4 (i4 / 2).
        const int n = 32 * (wave & 3) + (lane & 31);
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          *reinterpret_cast<uint2*>(&s.vt[n * kVPitch + 8 * (2 * (i4 & 1) + hi) + 4 * (i4 >> 1)]) =
              make_uint2(bf16_pair(acc[4 * i4], acc[4 * i4 + 1]), bf16_pair(acc[4 * i4 + 2], acc[4 * i4 + 3]));
        }
      }
    }
    __syncthreads();
    // ---- 3. attention for 16 queries per wave (waves 0..3); the next tile's fetch (4..7) ----
    if (wave >= 4) {
      if (tile + 1 < n_tiles) fetch(t0 + kPfT, buf ^ 1);
    } else {
      // S^T = [K | k_pe] . [q_nope | q_pe]^T for the tile's two 16-token
      // halves tb (A = key rows, B = query rows, both from LDS: token or
      // query l%16, dims 32ks + 8(l/16) .. +7).
      floatx4 sc[2] = {floatx4{}, floatx4{}};
      const uint16_t* qr = &s.q[(16 * wave + l16) * kKPitch + 8 * g4];
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
        const uint16_t* kr = &s.k[buf][(16 * tb + l16) * kKPitch + 8 * g4];
#pragma unroll
        for (int ks = 0; ks < 6; ++ks) {
          sc[tb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*reinterpret_cast<const bf16x8*>(kr + 32 * ks),
                                                           *reinterpret_cast<const bf16x8*>(qr + 32 * ks), sc[tb], 0,
                                                           0, 0);
        }
      }
      // sc[tb][i]: token t0 + 16tb + 4(l/16) + i for query qg. Online softmax
      // with a lazy rescale: the reference maximum moves only when the tile's
      // maximum passes it by more than 2^8, so P <= 2^8, and O is rescaled
      // (wave-wide) only then. The query's maximum over its four lanes by two
      // lane swaps.
      float x[2][4];
      float mx = -INFINITY;
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          x[tb][i] = t0 + 16 * tb + 4 * g4 + i <= lim ? sc[tb][i] * p.scale_log2 : -INFINITY;
          mx = fmaxf(mx, x[tb][i]);
        }
      }
      mx = xor32_max(xor16_max(mx));
      const float m_new = mx > m + kLazyRescaleLog2 ? mx : m;
      if (__any(m_new != m)) {
        const float alpha = m_new == m ? 1.0f : __builtin_amdgcn_exp2f(m - m_new);
#pragma unroll
        for (int vb = 0; vb < 8; ++vb) o[vb] *= alpha;
        lsum *= alpha;
      }
      m = m_new;
      const float mu = m == -INFINITY ? 0.0f : m;
      // P^T is the B operand of O^T += V^T P^T as it stands: lane l holds
      // k-steps 8(l/16) .. +7 = tokens 4(l/16) + 0..3 and 16 + 4(l/16) + 0..3,
      // the order of V^T's columns.
      bf16x8 pb;
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float pv = __builtin_amdgcn_exp2f(x[tb][i] - mu);
          lsum += pv;
          pb[4 * tb + i] = (__bf16)pv;
        }
      }
#pragma unroll
      for (int vb = 0; vb < 8; ++vb) {
        const bf16x8 va = *reinterpret_cast<const bf16x8*>(&s.vt[(16 * vb + l16) * kVPitch + 8 * g4]);
        o[vb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb, o[vb], 0, 0, 0);
      }
    }
  }
  __syncthreads();
  if (wave < 4) {
    const bool bad = s.bad != 0;
    const float nanv = __uint_as_float(0x7fc00000u);
    const float lt = xor32_sum(xor16_sum(lsum));
    if (qg < Q) {
      const int64_t row = ((int64_t)b * H + h) * Q + qg;
      const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
      // o[vb][i]: value dim 16vb + 4(l/16) + i of query qg.
      uint16_t* orow = reinterpret_cast<uint16_t*>(p.out) + row * 128 + 4 * g4;
#pragma unroll
      for (int vb = 0; vb < 8; ++vb) {
        float v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = bad ? nanv : o[vb][i] * inv;
        *reinterpret_cast<uint2*>(orow + 16 * vb) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
      }
      if (p.lse != nullptr && g4 == 0) {
        p.lse[row] = bad ? nanv : (lt > 0.0f ? (m + __log2f(lt)) * kLn2 : -INFINITY);
      }
    }
  }
}


// ---------------------------------------------------------------------------
// Long prefill in two kernels: the per-head keys and values are decompressed
// once per (token, head) into a workspace, then a flash-attention kernel
// streams them for every query tile. (CANN page, section 2: each chunk of
// the latent is decompressed once; the fused kernel above repeats that for
// every 64-query tile, which at Q = Lk is Q / 64 times the work.)
//
// Workspace: per (b, h) Lt = ceil(capacity / 32) tiles of 16 KiB each, tile
// j holding K[32 tokens][128] (token-major) then V^T[128][32] (value-major),
// bf16, tokens 32j .. 32j+31; rows past the sequence's length are zero. The
// columns of V^T run in the order the score fragments of the flash-attention
// kernel hold their tokens: within each group of 16, tokens 4..7 and 8..11
// trade places (column 16g + 8a + 4b + c holds token 16g + 8b + 4a + c).
// ---------------------------------------------------------------------------
constexpr int kKvTilesPerBlock = 8;  // tiles (of 32 tokens) per block of the decompression
constexpr int kWsTileBytes = 2 * kPfT * 128 * 2;
constexpr int kKsPitch = 136;        // K staging row pitch (bf16): 128 + 8

struct KvLds {
  uint16_t c[kPfT * kCPitch];
  uint16_t k[kPfT * kKsPitch];
  uint16_t vt[128 * kVPitch];
};

// First physical row of tile `t0 / 32` of sequence b, or -1 for a page index
// outside the cache (the same whole-page rule as the fused kernel).
// The page index is read through the constant address space (a scalar load:
// the index is uniform), so it does not wait behind the block's outstanding
// vector loads.
__device__ __forceinline__ int64_t pf_tile_base(const CacheView& c, int b, int t0) {
  if (c.page_size == 0) return (int64_t)b * c.capacity + t0;
  const int page = reinterpret_cast<const __attribute__((address_space(4))) int32_t*>(
      reinterpret_cast<uintptr_t>(c.page_table))[(int64_t)b * c.pt_stride + t0 / kPageTokens];
  const int64_t p0 = (int64_t)page * kPageTokens;
  if (page < 0 || p0 + kPageTokens > c.num_rows) return -1;
  return p0 + t0 % kPageTokens;
}

// Block (chunk of kKvTilesPerBlock tiles, head h, sequence b), 512 threads:
// wave w holds weight rows as in the fused kernel and forms its 32 x 32
// slice of K or V per tile; the tile leaves through LDS as whole rows.
__global__ void __launch_bounds__(kPfThreads) prefill_kv_kernel(PrefillParams p) {
  __shared__ __attribute__((aligned(16))) KvLds s;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, hi = lane >> 5;
  const int h = blockIdx.y, b = blockIdx.z;
  const CacheView& c = p.cache;
  const int len = clamp_len(p.seq_lens[b], c.capacity);
  const int n_tiles = (len + kPfT - 1) / kPfT;
  const int tile0 = blockIdx.x * kKvTilesPerBlock;
  if (tile0 >= n_tiles) return;
  const int tile1 = min(n_tiles, tile0 + kKvTilesPerBlock);
  const uint16_t* wkv = reinterpret_cast<const uint16_t*>(p.wkv_b) + (int64_t)h * 256 * 512;
  bf16x8 wf[32];
  {
    const uint16_t* wr = wkv + (int64_t)((wave >= 4 ? 128 : 0) + 32 * (wave & 3) + (lane & 31)) * 512 + 8 * hi;
#pragma unroll
    for (int ks = 0; ks < 32; ++ks) wf[ks] = *reinterpret_cast<const bf16x8*>(wr + 16 * ks);
  }
  uint8_t* ws = reinterpret_cast<uint8_t*>(p.kv_ws) + ((int64_t)b * p.H + h) * p.Lt * kWsTileBytes;
  // Thread tid moves 16-byte chunk tid % 64 of latent rows tid / 64 + 8j.
  const int cc = tid & 63, r0 = tid >> 6;
  auto load = [&](int tile, bf16x8* v) {
    const int t0 = tile * kPfT;
    const int last = min(kPfT - 1, len - 1 - t0);
    const int64_t base = pf_tile_base(c, b, t0);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = r0 + 8 * j;
      v[j] = bf16x8{};
      if (base >= 0 && r <= last) {
        v[j] = *reinterpret_cast<const bf16x8*>(c.latent + (base + r) * c.latent_stride + cc * 16);
      }
    }
  };
  bf16x8 v[4];
  load(tile0, v);
  // The weight fragments and the first tile have arrived: without this the
  // compiler carries their pending state into the loop and, at the top of
  // each step, waits for the previous step's stores along with the tile.
  __builtin_amdgcn_s_waitcnt(kVmcntZero);
  for (int tile = tile0; tile < tile1; ++tile) {
    __syncthreads();  // the previous tile's readers and copies are done
#pragma unroll
    for (int j = 0; j < 4; ++j) *reinterpret_cast<bf16x8*>(&s.c[(r0 + 8 * j) * kCPitch + cc * 8]) = v[j];
    if (tile + 1 < tile1) load(tile + 1, v);
    __syncthreads();
    // K transposed (D = W C^T: runs of 4 dims of one token per lane), V as
    // D = C W^T (runs of 4 tokens of one dim), as in the fused kernel.
    floatx16 acc = floatx16{};
    const uint16_t* a = &s.c[(lane & 31) * kCPitch + 8 * hi];
    if (wave < 4) {
#pragma unroll
      for (int ks = 0; ks < 32; ++ks) {
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[ks], *reinterpret_cast<const bf16x8*>(a + 16 * ks), acc, 0, 0,
                                                      0);
        if ((ks & 7) == 7) __builtin_amdgcn_sched_barrier(0);
      }
      // D lane l: token l%32, dims 32w + 8(i/4) + 4(l/32) + i%4.
      uint16_t* kd = &s.k[(lane & 31) * kKsPitch + 32 * wave + 4 * hi];
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        *reinterpret_cast<uint2*>(kd + 8 * a4) =
            make_uint2(bf16_pair(acc[4 * a4], acc[4 * a4 + 1]), bf16_pair(acc[4 * a4 + 2], acc[4 * a4 + 3]));
      }
    } else {
#pragma unroll
      for (int ks = 0; ks < 32; ++ks) {
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8*>(a + 16 * ks), wf[ks], acc, 0, 0,
                                                      0);
        if ((ks & 7) == 7) __builtin_amdgcn_sched_barrier(0);
      }
      // D lane l: dim n = 32(w-4) + l%32, tokens 8(i/4) + 4(l/32) + i%4.
      const int n = 32 * (wave & 3) + (lane & 31);
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {  // tokens 8 i4 + 4 hi .. +3, at their permuted columns
        *reinterpret_cast<uint2*>(&s.vt[n * kVPitch + 16 * (i4 >> 1) + 8 * hi + 4 * (i4 & 1)]) =
            make_uint2(bf16_pair(acc[4 * i4], acc[4 * i4 + 1]), bf16_pair(acc[4 * i4 + 2], acc[4 * i4 + 3]));
      }
    }
    __syncthreads();
    uint8_t* wt = ws + (int64_t)tile * kWsTileBytes;
    *reinterpret_cast<uint4*>(wt + (tid >> 4) * 256 + (tid & 15) * 16) =
        *reinterpret_cast<const uint4*>(&s.k[(tid >> 4) * kKsPitch + (tid & 15) * 8]);
    *reinterpret_cast<uint4*>(wt + kPfT * 256 + (tid >> 2) * 64 + (tid & 3) * 16) =
        *reinterpret_cast<const uint4*>(&s.vt[(tid >> 2) * kVPitch + (tid & 3) * 8]);
  }
}

constexpr int kFaWaves = 4;                 // waves per flash-attention block
constexpr int kFaQ = 32 * kFaWaves;         // queries per block (32 per wave)
constexpr int kFaThreads = 64 * kFaWaves;
static_assert(kFaThreads == 256 && kPfT == 32, "a tile is two K, two V^T and one RoPE piece per thread");

struct FaLds {
  uint16_t k[3][kPfT * kKPitch];   // [token][128 decompressed | 64 RoPE | pad]
  uint16_t vt[3][128 * kVPitch];   // [value dim][token, in the stored column order]
  int bad;
};

// Block of kFaQ queries of one (b, h); wave w takes queries q0 + 32w .. +31,
// lanes l and l + 32 both holding query l % 32.
//   S^T = [K | k_pe] . [q_nope | q_pe]^T for 32 tokens x 32 queries with
//   v_mfma_f32_32x32x16_bf16: A = key rows from LDS, B = the wave's query
//   fragments, held in registers. Lane l gets 16 of the tile's tokens for its
//   query and lane l ^ 32 the other 16, so a query's maximum is 15 maxima and
//   one lane swap, and its running sum stays per lane until the end.
//   Online softmax (log2 domain, c = softmax scale * log2 e) with a lazy
//   rescale: the reference maximum m moves only when a tile's maximum passes
//   it by more than 8 / c, so P = 2^(c s - c m) <= 256, and O and the sums are
//   rescaled (wave-wide) only then.
//   O^T += V^T P^T (v_mfma_f32_32x32x16_bf16, A = V^T rows from LDS): P^T in
//   bf16 is the B operand as it stands in the score registers, V^T's columns
//   being stored in that token order.
// Tiles pass through a ring of three LDS buffers, moved by all threads
// (prefetched into registers a tile ahead), with one barrier per tile: the
// matrix ops of S^T for the next tile are issued next to the exponentials of
// the current one. A wave whose queries see none of a tile skips its
// arithmetic. Blocks are dealt so that the query tiles of a (b, h) run on one
// XCD and share its L2, heaviest (last) query tiles first.
__global__ void __launch_bounds__(kFaThreads) prefill_fa_kernel(PrefillParams p) {
  __shared__ __attribute__((aligned(16))) FaLds s;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, hi = lane >> 5, l32 = lane & 31;
  const int nqt = (p.Q + kFaQ - 1) / kFaQ;
  const int xcd = blockIdx.x % 8, r = blockIdx.x / 8;
  const int unit = xcd + 8 * (r / nqt);
  if (unit >= p.B * p.H) return;
  const int qt = nqt - 1 - r % nqt;
  const int b = unit / p.H, h = unit % p.H;
  const int H = p.H, Q = p.Q;
  const CacheView& c = p.cache;
  const int len = clamp_len(p.seq_lens[b], c.capacity);
  const int q0 = qt * kFaQ;
  const int pos_max = len - Q + min(q0 + kFaQ - 1, Q - 1);
  const int n_tiles = pos_max < 0 ? 0 : min(pos_max / kPfT + 1, (len + kPfT - 1) / kPfT);
  const uint8_t* ws = reinterpret_cast<const uint8_t*>(p.kv_ws) + ((int64_t)b * H + h) * p.Lt * kWsTileBytes;

  // This lane's query sees positions 0 .. lim (lim = -1: none). The wave needs
  // tiles 0 .. w_tiles - 1, and a tile ending at or before full_lim needs no
  // mask (every query of the wave exists and sees all of it).
  const int qw = q0 + 32 * wave;
  const int qi = qw + l32;
  const int lim = qi < Q ? len - Q + qi : -1;
  const int w_last = len - Q + min(qw + 31, Q - 1);
  const int w_tiles = (qw >= Q || w_last < 0) ? 0 : min(w_last / kPfT + 1, n_tiles);
  const int full_lim = qw + 31 < Q ? len - Q + qw : -1;

  // Query fragments (B operand): query qi, dims 16ks + 8(l/32) .. +7 of
  // [q_nope | q_pe].
  bf16x8 qb[12];
  {
    const int64_t row = ((int64_t)b * H + h) * Q + min(qi, Q - 1);
    const uint16_t* qn = reinterpret_cast<const uint16_t*>(p.q_nope) + row * 128 + 8 * hi;
    const uint16_t* qp = reinterpret_cast<const uint16_t*>(p.q_pe) + row * 64 + 8 * hi;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qb[ks] = *reinterpret_cast<const bf16x8*>(qn + 16 * ks);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qb[8 + ks] = *reinterpret_cast<const bf16x8*>(qp + 16 * ks);
  }
  if (tid == 0) s.bad = 0;

  // Tile moves, prefetched into registers: thread tid carries K rows tid / 16
  // and 16 + tid / 16 (chunk tid % 16), V^T rows tid / 4 and 64 + tid / 4
  // (chunk tid % 4) and RoPE row tid / 8 (chunk tid % 8).
  uint4 nk0, nk1, nv0, nv1, nr;
  int nbad = 0;
  const int kof = (tid >> 4) * 256 + (tid & 15) * 16, vof = kPfT * 256 + (tid >> 2) * 64 + (tid & 3) * 16;
  auto load = [&](int tile) {
    const int t0 = tile * kPfT;
    const int64_t base = pf_tile_base(c, b, t0);
    const uint8_t* wt = ws + (int64_t)tile * kWsTileBytes;
    nk0 = *reinterpret_cast<const uint4*>(wt + kof);
    nk1 = *reinterpret_cast<const uint4*>(wt + kof + 16 * 256);
    nv0 = *reinterpret_cast<const uint4*>(wt + vof);
    nv1 = *reinterpret_cast<const uint4*>(wt + vof + 64 * 64);
    nbad = base < 0 ? 1 : 0;
    nr = make_uint4(0, 0, 0, 0);
    if (base >= 0 && t0 + (tid >> 3) < len) {
      nr = *reinterpret_cast<const uint4*>(c.rope + (base + (tid >> 3)) * c.rope_stride + (tid & 7) * 16);
    }
  };
  uint16_t* const ks0 = &s.k[0][(tid >> 4) * kKPitch + (tid & 15) * 8];
  uint16_t* const vs0 = &s.vt[0][(tid >> 2) * kVPitch + (tid & 3) * 8];
  uint16_t* const rs0 = &s.k[0][(tid >> 3) * kKPitch + 128 + (tid & 7) * 8];
  auto store = [&](int buf) {
    *reinterpret_cast<uint4*>(ks0 + buf * kPfT * kKPitch) = nk0;
    *reinterpret_cast<uint4*>(ks0 + buf * kPfT * kKPitch + 16 * kKPitch) = nk1;
    *reinterpret_cast<uint4*>(vs0 + buf * 128 * kVPitch) = nv0;
    *reinterpret_cast<uint4*>(vs0 + buf * 128 * kVPitch + 64 * kVPitch) = nv1;
    *reinterpret_cast<uint4*>(rs0 + buf * kPfT * kKPitch) = nr;
    if (nbad) s.bad = 1;
  };

  const float cs = p.scale_log2;
  const float thr = kLazyRescaleLog2 / cs;
  float m = -INFINITY, mc = 0.0f, lsum = 0.0f;  // reference maximum, c m (0 while m = -inf), sum
  floatx16 o[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) o[db] = floatx16{};
  // S^T of the tile in LDS buffer bi: st[i] is token t0 + 8(i/4) + 4(l/32) + i%4
  // of that tile for query qi.
  auto score = [&](int bi) {
    floatx16 acc = floatx16{};
    const uint16_t* kr = &s.k[bi][l32 * kKPitch + 8 * hi];
#pragma unroll
    for (int ks = 0; ks < 12; ++ks) {
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8*>(kr + 16 * ks), qb[ks], acc, 0, 0,
                                                    0);
    }
    return acc;
  };
  // Probabilities of st (bf16 P^T fragments) and their sum; then O^T += V^T P^T
  // from LDS buffer bi.
  auto prob_pv = [&](const floatx16& st, int bi) {
    bf16x8 pb[2];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(st[i], cs, -mc));
      lsum += pv;
      pb[i >> 3][i & 7] = (__bf16)pv;
    }
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const bf16x8 va = *reinterpret_cast<const bf16x8*>(&s.vt[bi][(32 * db + l32) * kVPitch + 16 * kk + 8 * hi]);
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[kk], o[db], 0, 0, 0);
      }
    }
  };

  // Software pipeline over a ring of three tile buffers: step k applies the
  // mask, maximum and rescale to S^T(k) (formed in step k-1), moves tile k+1
  // into the buffer tile k-2 left and requests tile k+2, passes the step's
  // one barrier, then issues the matrix ops of S^T(k+1) next to the
  // exponentials of tile k, and O^T += V^T P^T(k).
  floatx16 st = floatx16{};
  __syncthreads();  // the flag is cleared before any store can set it
  if (n_tiles > 0) {
    load(0);
    store(0);
  }
  // The query fragments have arrived (they did on the path above): without
  // this the compiler would wait for them inside the tile loop, behind the
  // prefetch of the tile after next.
  __builtin_amdgcn_s_waitcnt(kVmcntZero);
  if (n_tiles > 1) load(1);
  __syncthreads();
  if (w_tiles > 0) st = score(0);
  int bc = 0;  // buffer of tile k
  for (int tile = 0; tile < n_tiles; ++tile) {
    const int t0 = tile * kPfT;
    const int bn = bc == 2 ? 0 : bc + 1;  // buffer of tile k+1 (held tile k-2)
    if (tile < w_tiles) {
      if (t0 + kPfT - 1 > full_lim) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          if (t0 + 8 * (i >> 2) + 4 * hi + (i & 3) > lim) st[i] = -INFINITY;
        }
      }
      float mx = st[0];
#pragma unroll
      for (int i = 1; i < 16; ++i) mx = fmaxf(mx, st[i]);
      mx = xor32_max(mx);
      const bool need = mx > m + thr;
      if (__any(need)) {
        const float m_new = need ? mx : m;
        const float alpha = need ? __builtin_amdgcn_exp2f((m - m_new) * cs) : 1.0f;
#pragma unroll
        for (int db = 0; db < 4; ++db) {
#pragma unroll
          for (int i = 0; i < 16; ++i) o[db][i] *= alpha;
        }
        lsum *= alpha;
        m = m_new;
        mc = m == -INFINITY ? 0.0f : m * cs;
      }
    }
    if (tile + 1 < n_tiles) store(bn);
    if (tile + 2 < n_tiles) load(tile + 2);
    __syncthreads();
    if (tile + 1 < w_tiles) {
      const floatx16 sn = score(bn);
      prob_pv(st, bc);
      st = sn;
    } else if (tile < w_tiles) {
      prob_pv(st, bc);
    }
    bc = bn;
  }
  const bool bad = s.bad != 0;
  const float nanv = __uint_as_float(0x7fc00000u);
  const float lt = xor32_sum(lsum);
  if (qi < Q) {
    const int64_t row = ((int64_t)b * H + h) * Q + qi;
    const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
    uint16_t* orow = reinterpret_cast<uint16_t*>(p.out) + row * 128 + 4 * hi;
    // o[db][4a + e]: value dim 32db + 8a + 4(l/32) + e.
#pragma unroll
    for (int db = 0; db < 4; ++db) {
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = bad ? nanv : o[db][4 * a + e] * inv;
        *reinterpret_cast<uint2*>(orow + 32 * db + 8 * a) =
            make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
      }
    }
    if (p.lse != nullptr && hi == 0) {
      p.lse[row] = bad ? nanv : (lt > 0.0f ? (mc + __log2f(lt)) * kLn2 : -INFINITY);
    }
  }
}

}  // namespace

int64_t prefill_workspace_bytes(int B, int H, int Q, int capacity) {
  if (Q < kPrefillTwoKernelMinQ || B <= 0 || H <= 0) return 0;
  return (int64_t)B * H * ((capacity + kPfT - 1) / kPfT) * kWsTileBytes;
}

hipError_t launch_prefill(const PrefillParams& p, hipStream_t s) {
  if (p.B == 0 || p.Q == 0) return hipSuccess;
  if (p.H > 65535 || p.B > 65535) return hipErrorInvalidConfiguration;
  if (p.kv_ws != nullptr) {
    const int chunks = (p.Lt + kKvTilesPerBlock - 1) / kKvTilesPerBlock;
    if (chunks > 0) hipLaunchKernelGGL(prefill_kv_kernel, dim3(chunks, p.H, p.B), dim3(kPfThreads), 0, s, p);
    const int64_t units = ((int64_t)p.B * p.H + 7) / 8 * 8;
    const int64_t blocks = units * ((p.Q + kFaQ - 1) / kFaQ);
    if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(prefill_fa_kernel, dim3((unsigned)blocks), dim3(kFaThreads), 0, s, p);
    return hipGetLastError();
  }
  const int qt = (p.Q + kPfQ - 1) / kPfQ;
  hipLaunchKernelGGL(prefill_kernel, dim3(qt, p.H, p.B), dim3(kPfThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace mla
