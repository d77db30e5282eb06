// Absorbed MLA decode attention on gfx950 matrix cores (bf16 or FP4 latent).
//
// All heads of a sequence share one latent row per token (DeepSeek-V3 deep-dive
// page: W_UK absorbed on the query side; exercise page: scores against
// kv_cache and pe_cache, weighted sum over kv_cache). A workgroup takes 64
// query rows (h, q) of one sequence and streams that sequence's cache through
// LDS once for all of them:
//
//   S^T[t, r]  = sum_c K[t, c] Qcat[r, c]        c over 512 latent + 64 RoPE
//   online softmax over t per row r (scaled, causal limit per row)
//   O^T[c, r] += sum_t C^T[c, t] P^T[t, r]        c over the 512 latent
//
// Both contractions are v_mfma_f32_32x32x16_bf16 with fp32 accumulation.
// Wave w = (rh, ch): rows 32*rh..+31 of the block; it scores tokens 32*ch..+31
// of each 64-token tile and accumulates latent channels 256*ch..+255. The two
// waves of a row half swap their bf16 probabilities (and row max / sum)
// through LDS, so each accumulates P.V over all 64 tokens for its channels.
// Per wave: Q fragments 144 VGPRs, O^T 8 x 16 fp32 accumulators.
//
// Tiles of 64 tokens (one cache page) are double buffered in LDS: the loads
// of tile i+1 are issued into registers when tile i starts and written to
// the other buffer after tile i's P.V (an FP4 tile is decoded to bf16 on that
// write). The P.V operand (tokens along the contraction) is read with
// ds_read_b64_tr_b16 from the same row-major tile the score contraction reads.
//
// Tokens are split across workgroups (flash-decoding): the tiles of all
// sequences, end to end, are dealt in equal contiguous runs to the W
// workgroups of each row block. A run that covers a whole sequence writes x
// and lse directly; a piece of a sequence is written as a partial (x_s
// normalised, lse_s) and merged by the combine kernel:
//   lse = log sum_s exp(lse_s),  x = sum_s exp(lse_s - lse) x_s.
#include <type_traits>

#include "internal.h"

namespace mla {
namespace {

constexpr int kThreads = 256;
constexpr int kRowBytes = 1168;     // LDS bytes per token: 72 chunks of 16 B + 16 B padding
constexpr int kSlotsPerRow = kRowBytes / 16;  // 73
constexpr int kTileBytes = kTileTokens * kRowBytes;  // 74752
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kRescaleLog2 = 8.0f;  // p = 2^(s - m) stays <= 2^8

struct Xchg {
  uint4 p[4][64][2];  // bf16 probability fragments of each wave
  float mx[4][32];    // per-row max of each wave's 32 tokens
  float sum[4][32];   // per-row sum of each wave's probabilities
  int flag[4];        // a wave saw a row whose max exceeds the reference by > kRescaleLog2
};

constexpr int kSmemBytes = 2 * kTileBytes + (int)sizeof(Xchg);

typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) shortx4 lds_shortx4;

__device__ __forceinline__ shortx4 tr_read(const uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4*)(p));
}

__device__ __forceinline__ bf16x8 join(shortx4 a, shortx4 b) {
  const auto v = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ int seq_len(const AttnParams& p, int b) {
  return clamp_len(p.seq_lens[b], p.cache.capacity);
}

__device__ __forceinline__ int tiles_of(int L) { return (L + kTileTokens - 1) / kTileTokens; }

// Block-wide exclusive scan of one int per thread. *total gets the block sum.
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

// First physical row of tile `tile` of sequence b (a tile is one 64-row page).
__device__ __forceinline__ int64_t tile_row0(const CacheView& c, int b, int tile, bool& bad) {
  if (c.page_size == 0) return (int64_t)b * c.capacity + (int64_t)tile * kTileTokens;
  const int page = c.page_table[(int64_t)b * c.pt_stride + tile];
  const int64_t r0 = (int64_t)page * kTileTokens;
  if (page < 0 || r0 + kTileTokens > c.num_rows) {
    bad = true;
    return 0;
  }
  return r0;
}

// 64-bit select without control flow.
__device__ __forceinline__ const uint8_t* pick(bool c, const uint8_t* a, const uint8_t* b) {
  const uint64_t m = 0ull - (uint64_t)c;
  return reinterpret_cast<const uint8_t*>((reinterpret_cast<uint64_t>(a) & m) |
                                          (reinterpret_cast<uint64_t>(b) & ~m));
}

// Tile staging through registers: the loads of tile i+1 are issued right
// after the barrier that opens tile i and are written to LDS after tile i's
// P.V, so they stay in flight for a whole tile of compute.
//
// bf16 tiles: 64 tokens x 72 chunks of 16 B = 18 chunks per thread; thread
// tid takes chunks s = tid + 256*n, i.e. token s / 72, chunk s % 72 (0..63
// latent, 64..71 RoPE), advancing by (3, 40) per step. Tokens at or past
// `valid` re-read the last valid row: they are masked out of the softmax and
// their (finite) values meet zero probabilities.
constexpr int kBf16Regs = kTileTokens * 72 / kThreads;  // 18

struct Bf16Stage {
  uint4 v[kBf16Regs];
};

__device__ __forceinline__ void load_tile_bf16(const CacheView& c, int64_t row0, int valid, int tid,
                                               Bf16Stage& st) {
  // Opaque thread id: keeps the compiler from hoisting all 18 addresses out
  // of the tile loop (they would not fit in registers).
  asm volatile("" : "+v"(tid));
  const uint8_t* lat0 = c.latent + row0 * c.latent_stride;
  const uint8_t* rope0 = c.rope + row0 * c.rope_stride;
  const uint32_t ls = (uint32_t)c.latent_stride, rs = (uint32_t)c.rope_stride;
  int t = tid / 72;
  int cc = tid - t * 72;
#pragma unroll
  for (int n = 0; n < kBf16Regs; ++n) {
    const uint32_t tt = (uint32_t)min(t, valid - 1);
    const bool lat = cc < 64;
    const uint32_t off = tt * (lat ? ls : rs) + (uint32_t)(lat ? cc : cc - 64) * 16u;
    st.v[n] = *reinterpret_cast<const uint4*>(pick(lat, lat0, rope0) + off);
    cc += 40;
    t += 3;
    if (cc >= 72) {
      cc -= 72;
      t += 1;
    }
  }
}

__device__ __forceinline__ void store_tile_bf16(uint8_t* dst, int tid, const Bf16Stage& st) {
  asm volatile("" : "+v"(tid));
  int t = tid / 72;
  int cc = tid - t * 72;
#pragma unroll
  for (int n = 0; n < kBf16Regs; ++n) {
    *reinterpret_cast<uint4*>(dst + t * kRowBytes + cc * 16) = st.v[n];
    cc += 40;
    t += 3;
    if (cc >= 72) {
      cc -= 72;
      t += 1;
    }
  }
}

// FP4 tiles: per token 16 code chunks (32 channels each) with their 2 scale
// bytes, and 8 RoPE chunks. Thread tid takes code chunks s = tid + 256*k
// (token s >> 4, chunk s & 15) and RoPE chunks s = tid + 256*k (token s >> 3,
// chunk s & 7); it decodes its codes (E2M1 value times E4M3 scale, exact in
// bf16) when writing them to the bf16 tile.
struct Fp4Stage {
  uint4 codes[4];
  uint32_t scales[4];
  uint4 rope[2];
};

__device__ __forceinline__ void load_tile_fp4(const CacheView& c, int64_t row0, int valid, int tid,
                                              Fp4Stage& st) {
  asm volatile("" : "+v"(tid));
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int s = tid + kThreads * k;
    const int64_t r = row0 + min(s >> 4, valid - 1);
    const int j = s & 15;
    st.codes[k] = *reinterpret_cast<const uint4*>(c.latent + r * c.latent_stride + j * 16);
    st.scales[k] = *reinterpret_cast<const uint16_t*>(c.scale + r * c.scale_stride + j * 2);
  }
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int s = tid + kThreads * k;
    const int64_t r = row0 + min(s >> 3, valid - 1);
    st.rope[k] = *reinterpret_cast<const uint4*>(c.rope + r * c.rope_stride + (s & 7) * 16);
  }
}

__device__ __forceinline__ void store_tile_fp4(uint8_t* dst, int tid, const Fp4Stage& st) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int s = tid + kThreads * k;
    const int t = s >> 4;
    const int j = s & 15;
    const float s0 = e4m3_to_f32(st.scales[k] & 0xffu);
    const float s1 = e4m3_to_f32(st.scales[k] >> 8);
    const uint32_t words[4] = {st.codes[k].x, st.codes[k].y, st.codes[k].z, st.codes[k].w};
#pragma unroll
    for (int qd = 0; qd < 4; ++qd) {
      const float sv = qd < 2 ? s0 : s1;
      uint32_t outw[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float v0 = __uint_as_float(e2m1_f32_bits((words[qd] >> (8 * e)) & 0xfu)) * sv;
        const float v1 = __uint_as_float(e2m1_f32_bits((words[qd] >> (8 * e + 4)) & 0xfu)) * sv;
        outw[e] = (__float_as_uint(v0) >> 16) | (__float_as_uint(v1) & 0xffff0000u);
      }
      *reinterpret_cast<uint4*>(dst + t * kRowBytes + (4 * j + qd) * 16) =
          make_uint4(outw[0], outw[1], outw[2], outw[3]);
    }
  }
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int s = tid + kThreads * k;
    *reinterpret_cast<uint4*>(dst + (s >> 3) * kRowBytes + (64 + (s & 7)) * 16) = st.rope[k];
  }
}

template <bool kFp4>
__global__ void __launch_bounds__(kThreads, 1) attn_mfma_kernel(AttnParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[kSmemBytes];
  __shared__ int s_tmp[8];
  __shared__ int s_start[2];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int hi = lane >> 5;
  const int rh = wave & 1;
  const int ch = wave >> 1;

  // Block -> (run wg, row block g). Consecutive block ids go to the 8 XCDs in
  // turn; the G row blocks of one run share an XCD (and its L2), and are
  // dispatched next to each other, so the cache tiles they both read come
  // from HBM once.
  const int G = p.groups;
  const int bid = blockIdx.x;
  const int xcd = bid & 7;
  const int q8 = bid >> 3;
  const int g = q8 % G;
  const int wg = (q8 / G) * 8 + xcd;
  if (wg >= p.workgroups) return;

  // ---- this workgroup's run: tiles [start, end) of all sequences end to end ----
  const int per_thread = (p.B + kThreads - 1) / kThreads;
  const int b_lo = min(p.B, tid * per_thread);
  const int b_hi = min(p.B, b_lo + per_thread);
  int my_tiles = 0;
  for (int b = b_lo; b < b_hi; ++b) my_tiles += tiles_of(seq_len(p, b));
  int total = 0;
  const int base = block_exclusive_scan(my_tiles, s_tmp, &total);
  const int per = (total + p.workgroups - 1) / p.workgroups;
  const int start = wg * per;
  const int end = min(total, start + per);
  if (start >= end) return;
  if (start >= base && start < base + my_tiles) {
    int acc = base;
    for (int b = b_lo; b < b_hi; ++b) {
      const int n = tiles_of(seq_len(p, b));
      if (start < acc + n) {
        s_start[0] = b;
        s_start[1] = start - acc;
        break;
      }
      acc += n;
    }
  }
  __syncthreads();

  uint8_t* tiles = smem;  // two bf16 tiles: tile i lives in buffer i & 1
  Xchg* xc = reinterpret_cast<Xchg*>(smem + 2 * kTileBytes);

  const int row_local = rh * 32 + (lane & 31);
  const int row = g * 64 + row_local;
  const bool row_ok = row < p.HQ;
  const int qi = row_ok ? row % p.Q : 0;
  const int slots = 2 * p.workgroups;
  const int count = end - start;

  // Current tile (b, tile) and the next one to prefetch (nb, ntile).
  int b = s_start[0];
  int tile = s_start[1];
  int L = seq_len(p, b);
  int nb = b, ntile = tile, nL = L;
  auto advance = [&](int& bb, int& tt, int& LL) {
    ++tt;
    if (tt >= tiles_of(LL)) {
      tt = 0;
      do {
        ++bb;
      } while (bb < p.B && seq_len(p, bb) == 0);
      LL = bb < p.B ? seq_len(p, bb) : 0;
    }
  };

  // Stage tile 0 of the run into buffer 0 (visible after the first barrier).
  bool bad_cur = false;
  {
    const int64_t r0 = tile_row0(p.cache, b, tile, bad_cur);
    const int valid = bad_cur ? 1 : min(kTileTokens, L - tile * kTileTokens);
    if constexpr (kFp4) {
      Fp4Stage st;
      load_tile_fp4(p.cache, r0, valid, tid, st);
      store_tile_fp4(tiles, tid, st);
    } else {
      Bf16Stage st;
      load_tile_bf16(p.cache, r0, valid, tid, st);
      store_tile_bf16(tiles, tid, st);
    }
  }

  bf16x8 qf[36];
  floatx16 o[8];
  float m = -INFINITY, l = 0.0f;
  int seg_bad = 0;
  int seg_lo = tile;
  bool first_seg = true;

  for (int it = 0; it < count; ++it) {
    const int nt = tiles_of(L);
    if (it == 0 || tile == 0) {
      // New segment: Q fragments of this sequence (B operand of S^T = K Qcat^T):
      // row `row`, channels 16*ks + 8*hi .. +7 of [q_lat | q_pe].
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
#pragma unroll
      for (int cb = 0; cb < 8; ++cb) o[cb] = floatx16{};
      m = -INFINITY;
      l = 0.0f;
      seg_bad = 0;
      seg_lo = tile;
    }
    seg_bad |= bad_cur ? 1 : 0;

    // Tile `it` is in LDS for every wave, and every wave is done with tile
    // it-1, whose buffer receives tile it+1 below.
    __syncthreads();

    // Prefetch the next tile of the run into registers.
    bool bad_nxt = false;
    const bool has_next = it + 1 < count;
    using Stage = typename std::conditional<kFp4, Fp4Stage, Bf16Stage>::type;
    Stage st;
    if (has_next) {
      advance(nb, ntile, nL);
      const int64_t r0 = tile_row0(p.cache, nb, ntile, bad_nxt);
      const int valid = bad_nxt ? 1 : min(kTileTokens, nL - ntile * kTileTokens);
      if constexpr (kFp4) {
        load_tile_fp4(p.cache, r0, valid, tid, st);
      } else {
        load_tile_bf16(p.cache, r0, valid, tid, st);
      }
    }
    const uint8_t* tb = tiles + (it & 1) * kTileBytes;

    // ---- S^T block: tokens 32*ch .. +31 of the tile x rows 32*rh .. +31 ----
    floatx16 s = floatx16{};
    {
      const uint8_t* kb = tb + (32 * ch + (lane & 31)) * kRowBytes + hi * 16;
#pragma unroll
      for (int ks = 0; ks < 36; ++ks) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(kb + ks * 32);
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], s, 0, 0, 0);
        if ((ks & 3) == 3) __builtin_amdgcn_sched_barrier(0);
      }
    }

    // ---- online softmax in the log2 domain; lane holds row `row` ----
    const int vis = L - p.Q + qi + 1;  // this row sees tokens t < vis
    const int tok0 = tile * kTileTokens + 32 * ch + 4 * hi;
    float own_mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int tok = tok0 + 8 * (i >> 2) + (i & 3);
      const float v = tok < vis ? s[i] * p.scale_log2 : -INFINITY;
      s[i] = v;
      own_mx = fmaxf(own_mx, v);
    }
    own_mx = fmaxf(own_mx, __shfl_xor(own_mx, 32, 64));
    // The reference m moves only when a row max exceeds it by > kRescaleLog2,
    // so O is rarely rescaled and every probability stays <= 2^kRescaleLog2.
    const bool ovf = own_mx > m + kRescaleLog2;
    float m_use = m == -INFINITY ? 0.0f : m;
    float own_sum = 0.0f;
    bf16x8 pf[2];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float e = exp2f(s[i] - m_use);
      own_sum += e;
      pf[i >> 3][i & 7] = (__bf16)e;
    }
    own_sum += __shfl_xor(own_sum, 32, 64);
    const int pw = wave ^ 2;  // the other token half of this row half
    *reinterpret_cast<bf16x8*>(&xc->p[wave][lane][0]) = pf[0];
    *reinterpret_cast<bf16x8*>(&xc->p[wave][lane][1]) = pf[1];
    if (hi == 0) {
      xc->mx[wave][lane] = own_mx;
      xc->sum[wave][lane] = own_sum;
    }
    const bool wave_ovf = __any(ovf);
    if (lane == 0) xc->flag[wave] = wave_ovf ? 1 : 0;
    __syncthreads();
    const int any_ovf = xc->flag[0] | xc->flag[1] | xc->flag[2] | xc->flag[3];
    if (any_ovf) {
      // A row max rose: move the reference to the new max (both token halves
      // agree on it), recompute this wave's probabilities, rescale O and l.
      const float mx = fmaxf(own_mx, xc->mx[pw][lane & 31]);
      const bool upd = mx > m + kRescaleLog2;
      const float m_new = upd ? mx : m;
      const float alpha = upd ? exp2f(m - m_new) : 1.0f;
      m_use = m_new == -INFINITY ? 0.0f : m_new;
      own_sum = 0.0f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float e = exp2f(s[i] - m_use);
        own_sum += e;
        pf[i >> 3][i & 7] = (__bf16)e;
      }
      own_sum += __shfl_xor(own_sum, 32, 64);
      __syncthreads();  // every wave has read the old max and flags
      *reinterpret_cast<bf16x8*>(&xc->p[wave][lane][0]) = pf[0];
      *reinterpret_cast<bf16x8*>(&xc->p[wave][lane][1]) = pf[1];
      if (hi == 0) xc->sum[wave][lane] = own_sum;
      if (__any(upd && m != -INFINITY)) {
#pragma unroll
        for (int cb = 0; cb < 8; ++cb) o[cb] *= alpha;
      }
      l *= alpha;
      m = m_new;
      __syncthreads();
    }
    const float psum = xc->sum[pw][lane & 31];
    l += ch == 0 ? own_sum + psum : psum + own_sum;
    bf16x8 pp[2];
    pp[0] = *reinterpret_cast<const bf16x8*>(&xc->p[pw][lane][0]);
    pp[1] = *reinterpret_cast<const bf16x8*>(&xc->p[pw][lane][1]);
    // Token half 0 probabilities come from the ch = 0 wave, half 1 from ch = 1.
    const bf16x8 p0 = ch == 0 ? pf[0] : pp[0];
    const bf16x8 p1 = ch == 0 ? pf[1] : pp[1];
    const bf16x8 p2 = ch == 0 ? pp[0] : pf[0];
    const bf16x8 p3 = ch == 0 ? pp[1] : pf[1];

    // ---- O^T[c, r] += C^T[c, t] P^T[t, r] for this wave's 256 channels ----
    // A operand (k-step kk): channel lane%32 of the block, tokens
    // 16*kk + 4*hi + {0..3} and +8 + {0..3}, by two transposed LDS reads of
    // a 4 x 16 block each (16-lane groups: lane j -> row j/4, cols 4*(j%4)).
    {
      const int j = lane & 15;
      const uint8_t* vb = tb + (4 * hi + (j >> 2)) * kRowBytes +
                          (256 * ch + 16 * ((lane >> 4) & 1) + 4 * (j & 3)) * 2;
#pragma unroll
      for (int cb = 0; cb < 8; ++cb) {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const uint8_t* a0 = vb + 16 * kk * kRowBytes + cb * 64;
          const bf16x8 a = join(tr_read(a0), tr_read(a0 + 8 * kRowBytes));
          const bf16x8 bp = kk == 0 ? p0 : kk == 1 ? p1 : kk == 2 ? p2 : p3;
          o[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bp, o[cb], 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }

    // The prefetched tile goes to the other buffer.
    if (has_next) {
      if constexpr (kFp4) {
        store_tile_fp4(tiles + ((it + 1) & 1) * kTileBytes, tid, st);
      } else {
        store_tile_bf16(tiles + ((it + 1) & 1) * kTileBytes, tid, st);
      }
    }

    // ---- end of a segment: write x / lse, or a partial for the combine ----
    if (it == count - 1 || tile == nt - 1) {
      const bool whole = seg_lo == 0 && tile == nt - 1;
      const float inv_l = l > 0.0f ? 1.0f / l : 0.0f;
      const float nanv = __uint_as_float(0x7fc00000u);
      float lse_v = l > 0.0f ? (m + log2f(l)) * kLn2 : -INFINITY;
      if (seg_bad) lse_v = nanv;
      if (row_ok) {
        if (whole) {
          uint16_t* xo = reinterpret_cast<uint16_t*>(p.x_lat) + ((int64_t)b * p.HQ + row) * 512;
#pragma unroll
          for (int cb = 0; cb < 8; ++cb) {
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
              const int c = 256 * ch + 32 * cb + 8 * i4 + 4 * hi;
              float v[4];
#pragma unroll
              for (int e = 0; e < 4; ++e) v[e] = seg_bad ? nanv : o[cb][4 * i4 + e] * inv_l;
              *reinterpret_cast<uint2*>(xo + c) =
                  make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
            }
          }
          if (p.lse != nullptr && hi == 0 && ch == 0) p.lse[(int64_t)b * p.HQ + row] = lse_v;
        } else {
          const int slot = 2 * wg + (first_seg ? 0 : 1);
          const int64_t prow = ((int64_t)g * slots + slot) * 64 + row_local;
          float* xo = p.part_x + prow * 512;
#pragma unroll
          for (int cb = 0; cb < 8; ++cb) {
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
              const int c = 256 * ch + 32 * cb + 8 * i4 + 4 * hi;
              float4 v;
              v.x = o[cb][4 * i4 + 0] * inv_l;
              v.y = o[cb][4 * i4 + 1] * inv_l;
              v.z = o[cb][4 * i4 + 2] * inv_l;
              v.w = o[cb][4 * i4 + 3] * inv_l;
              *reinterpret_cast<float4*>(xo + c) = v;
            }
          }
          if (hi == 0 && ch == 0) p.part_lse[prow] = lse_v;
        }
      }
      first_seg = false;
    }

    // Move to the next tile of the run.
    if (it + 1 < count) {
      const bool new_seq = tile == nt - 1;
      b = nb;
      tile = ntile;
      L = nL;
      (void)new_seq;
    }
    bad_cur = bad_nxt;
  }
}

// Merge partial results of sequences whose tiles were split over workgroups,
// and write x = 0 / lse = -inf for sequences without any cache rows.
// Grid: (B, groups * 4); each block handles 16 query rows of one sequence.
__global__ void __launch_bounds__(kThreads) attn_combine_kernel(AttnParams p) {
  __shared__ int s_tmp[8];
  const int tid = threadIdx.x;
  const int b = blockIdx.x;
  const int g = blockIdx.y >> 2;
  const int rb = blockIdx.y & 3;

  const int per_thread = (p.B + kThreads - 1) / kThreads;
  const int b_lo = min(p.B, tid * per_thread);
  const int b_hi = min(p.B, b_lo + per_thread);
  int my_tiles = 0;
  int before = 0;
  for (int j = b_lo; j < b_hi; ++j) {
    const int n = tiles_of(seq_len(p, j));
    my_tiles += n;
    if (j < b) before += n;
  }
  int cum_b = 0;
  block_exclusive_scan(before, s_tmp, &cum_b);
  int total_tiles = 0;
  block_exclusive_scan(my_tiles, s_tmp, &total_tiles);
  const int nb = tiles_of(seq_len(p, b));

  const int row_local = rb * 16 + (tid >> 4);
  const int row = g * 64 + row_local;
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
    const float v = p.part_lse[((int64_t)g * slots + slot_of(i)) * 64 + row_local];
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
      tot += __expf(p.part_lse[((int64_t)g * slots + slot_of(i)) * 64 + row_local] - mx);
    }
    lse_v = mx + __logf(tot);
    for (int i = i_first; i <= i_last; ++i) {
      const int64_t prow = ((int64_t)g * slots + slot_of(i)) * 64 + row_local;
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
  const int blocks = ((p.workgroups + 7) / 8) * 8 * p.groups;
  if (fp4_latent) {
    hipLaunchKernelGGL(attn_mfma_kernel<true>, dim3(blocks), dim3(kThreads), 0, s, p);
  } else {
    hipLaunchKernelGGL(attn_mfma_kernel<false>, dim3(blocks), dim3(kThreads), 0, s, p);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(attn_combine_kernel, dim3(p.B, p.groups * 4), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace mla
